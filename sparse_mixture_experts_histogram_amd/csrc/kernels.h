// Launch wrappers of the gfx950 kernels (host side).  Each returns the
// hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>

#include "plan.h"

namespace moe {

// Outputs of the dispatch when the router runs it in the same launch.
struct DispatchOut {
  int32_t *counts, *offsets, *sorted_token, *slot_row;
  Tile *tiles_up, *tiles_down;
};

// Router logits + softmax + top-k + renormalise; also writes the per-block
// histogram and in-block stable ranks of the (token, slot) pairs.  `part`
// holds the split-K partial logits when P.rsplit > 1.  With a split router
// and a single token block, a non-null `dout` also makes the router run the
// dispatch (see router.hip); launch_dispatch must then not be called.
hipError_t launch_router(const Plan& P, const void* x, const void* w_router, const float* bias,
                         int32_t* idx, float* w, int32_t* blk_hist, int32_t* blk_rank,
                         float* part, const DispatchOut* dout, hipStream_t s);

// Per-block histogram and ranks from given top-k indices.
hipError_t launch_block_hist(const Plan& P, const int32_t* idx, int32_t* blk_hist,
                             int32_t* blk_rank, hipStream_t s);

// Scan + permute + tile schedules (one workgroup).  blk_hist is turned into
// per-block exclusive offsets in place.
hipError_t launch_dispatch(const Plan& P, const int32_t* idx, int32_t* blk_hist,
                           const int32_t* blk_rank, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_token, int32_t* slot_row, Tile* tiles_up,
                           Tile* tiles_down, hipStream_t s);

// Tile schedules from given group offsets (one workgroup).
hipError_t launch_tiles(const Plan& P, const int32_t* offsets, Tile* tiles_up, Tile* tiles_down,
                        hipStream_t s);

// E8M0 scale arrays of MXFP4 or MXFP8 expert weights (all null for dense weights).
struct MxScales {
  const uint8_t *up, *gate, *down, *s_up, *s_gate, *s_down;
};

struct ExpertArgs {
  const void* x;
  const void *w_up, *w_gate, *w_down, *ws_up, *ws_gate, *ws_down;
  const int32_t* sorted_token;
  const Tile* tiles_up;
  const Tile* tiles_down;
  void* h;
  float* out;     // expert outputs; with ksplit > 1, ksplit partial buffers of
                  // (R + kRowSlack) rows each, summed by the combine
  int ksplit;     // K ranges of the down GEMM (1 = direct result)
  MxScales mx;    // MX-format expert weights: their scales
  float* part;    // K-piece accumulators of a last-round split (see plan.h GemmShape::sk_cus)
};

// Grouped up/gate GEMM + SwiGLU (writes h).
hipError_t launch_expert_up(const Plan& P, const ExpertArgs& a, hipStream_t s);
// Grouped down GEMM (reads h, writes out).
hipError_t launch_expert_down(const Plan& P, const ExpertArgs& a, hipStream_t s);

// y[t] = sum_j w[t,j] out[slot_row[t,j]] + sum_s out[offsets[E+s]+t], where
// out[r] is the sum of `nparts` partial buffers `part_stride` floats apart.
hipError_t launch_combine(const Plan& P, const float* out, int nparts, int64_t part_stride,
                          const float* w, const int32_t* slot_row, const int32_t* offsets,
                          void* y, hipStream_t s);

}  // namespace moe
