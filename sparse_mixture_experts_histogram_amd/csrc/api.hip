// The extern "C" entry points of include/moe.h that launch work: host-side
// checks, workspace carving and the launch sequence on the caller's stream.
#include <hip/hip_runtime.h>

#include <initializer_list>
#include <mutex>

#include "kernels.h"
#include "plan.h"

namespace moe {
namespace {

struct Ws {
  char* base;
  template <typename T>
  T* at(size_t off) const {
    return (T*)(base + off);
  }
};

// MOE_OK with *empty set when the call has nothing to do (T == 0).
int prepare(const moe_desc* d, void* workspace, size_t ws_bytes, Plan* P, bool* empty) {
  int st = make_plan(d, P);
  if (st != MOE_OK) return st;
  *empty = d->T == 0;
  if (*empty) return MOE_OK;
  if (!workspace || ws_bytes < P->total) return MOE_ERR_WORKSPACE;
  if (((uintptr_t)workspace) & 255) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

inline int hip_ok(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)               \
  do {                              \
    int _st = hip_ok(expr);         \
    if (_st != MOE_OK) return _st;  \
  } while (0)

bool shared_ok(const moe_desc* d, const void* a, const void* b, const void* c) {
  return d->n_shared == 0 || (a && b && c);
}

// Token, weight and scale arrays are read in 16-byte chunks.
bool a16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if ((uintptr_t)p & 15) return false;
  return true;
}

}  // namespace
}  // namespace moe

namespace moe {
namespace {

// moe_forward's launch sequence; events[i] (when non-null) is recorded on the
// stream before launch i (router, dispatch, up/gate, down, combine) and
// events[5] after the last one.
// `mx` is the scale set of MXFP4 or MXFP8 expert weights (null for dense weights).
int forward_impl(const moe_desc* d, const void* x, const void* w_router,
                 const float* router_bias, const void* w_up, const void* w_gate,
                 const void* w_down, const void* ws_up, const void* ws_gate, const void* ws_down,
                 const moe_mx_scales* mx, void* y, int32_t* topk_idx, float* topk_w,
                 int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                 moe_stream stream, void* const* events) {
  if (d && (d->expert_format != MOE_EXPERTS_DENSE) != (mx != nullptr)) return MOE_ERR_INVALID_ARG;
  Plan P;
  bool empty = false;
  int st = prepare(d, workspace, workspace_bytes, &P, &empty);
  if (st != MOE_OK || empty) return st;
  if (!x || !w_router || !w_up || !w_gate || !w_down || !y) return MOE_ERR_INVALID_ARG;
  if (!shared_ok(d, ws_up, ws_gate, ws_down)) return MOE_ERR_INVALID_ARG;
  if (mx && (!mx->up || !mx->gate || !mx->down || !shared_ok(d, mx->s_up, mx->s_gate, mx->s_down)))
    return MOE_ERR_INVALID_ARG;
  if (!a16({x, w_router, w_up, w_gate, w_down, ws_up, ws_gate, ws_down}) ||
      (mx && !a16({mx->up, mx->gate, mx->down, mx->s_up, mx->s_gate, mx->s_down})))
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  auto mark = [&](int i) -> hipError_t {
    if (events && events[i]) return hipEventRecord((hipEvent_t)events[i], s);
    return hipSuccess;
  };
  Ws W{(char*)workspace};
  int32_t* idx = topk_idx ? topk_idx : W.at<int32_t>(P.o_idx);
  float* w = topk_w ? topk_w : W.at<float>(P.o_w);
  int32_t* counts = expert_counts ? expert_counts : W.at<int32_t>(P.o_counts);
  int32_t* blk_hist = W.at<int32_t>(P.o_blk_hist);
  int32_t* blk_rank = W.at<int32_t>(P.o_blk_rank);
  int32_t* offsets = W.at<int32_t>(P.o_offsets);
  int32_t* sorted = W.at<int32_t>(P.o_sorted);
  int32_t* slot = W.at<int32_t>(P.o_slot);
  Tile* tu = W.at<Tile>(P.o_tiles_up);
  Tile* td = W.at<Tile>(P.o_tiles_down);
  float* out = W.at<float>(P.o_out);
  MxScales sc{};
  if (mx)
    sc = MxScales{(const uint8_t*)mx->up,   (const uint8_t*)mx->gate,
                  (const uint8_t*)mx->down, (const uint8_t*)mx->s_up,
                  (const uint8_t*)mx->s_gate, (const uint8_t*)mx->s_down};
  ExpertArgs a{x, w_up, w_gate, w_down, ws_up, ws_gate, ws_down, sorted, tu, td,
               W.at<void>(P.o_h), out, P.down.ksplit, sc, W.at<float>(P.o_part)};
  const int64_t part_stride = ((int64_t)P.R + kRowSlack) * d->d;
  // With a split router and one token block (at most 16 tokens) the router
  // also runs the dispatch, and events 1 and 2 mark the same point.
  const bool fused = P.rsplit > 1 && P.nblk == 1;
  const DispatchOut dout{counts, offsets, sorted, slot, tu, td};
  MOE_TRY(mark(0));
  MOE_TRY(launch_router(P, x, w_router, router_bias, idx, w, blk_hist, blk_rank,
                        W.at<float>(P.o_router_part), fused ? &dout : nullptr, s));
  MOE_TRY(mark(1));
  if (!fused)
    MOE_TRY(launch_dispatch(P, idx, blk_hist, blk_rank, counts, offsets, sorted, slot, tu, td, s));
  MOE_TRY(mark(2));
  MOE_TRY(launch_expert_up(P, a, s));
  MOE_TRY(mark(3));
  MOE_TRY(launch_expert_down(P, a, s));
  MOE_TRY(mark(4));
  MOE_TRY(launch_combine(P, out, P.down.ksplit, part_stride, w, slot, offsets, y, s));
  MOE_TRY(mark(5));
  return MOE_OK;
}

}  // namespace
}  // namespace moe

namespace moe {
namespace {

// Scratch of moe_forward_noalloc.  Each GPU the library runs on holds its own
// copy (loaded with the code object) until the process ends.  Host code never
// passes this name to a kernel or a copy: it is a host-side stand-in; the
// device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_forward_noalloc(const moe_desc* d, const void* x, const void* w_router,
                        const float* router_bias, const void* w_up, const void* w_gate,
                        const void* w_down, const void* ws_up, const void* ws_gate,
                        const void* ws_down, void* y, int32_t* topk_idx, float* topk_w,
                        int32_t* expert_counts, moe_stream stream) {
  Plan P;
  int st = make_plan(d, &P);
  if (st != MOE_OK) return st;
  if (d->T == 0) return MOE_OK;
  if (P.total > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  void* ws = nullptr;
  st = device_scratch(&ws);
  if (st != MOE_OK) return st;
  return forward_impl(d, x, w_router, router_bias, w_up, w_gate, w_down, ws_up, ws_gate,
                      ws_down, nullptr, y, topk_idx, topk_w, expert_counts, ws,
                      MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int moe_forward(const moe_desc* d, const void* x, const void* w_router, const float* router_bias,
                const void* w_up, const void* w_gate, const void* w_down, const void* ws_up,
                const void* ws_gate, const void* ws_down, void* y, int32_t* topk_idx,
                float* topk_w, int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                moe_stream stream) {
  return forward_impl(d, x, w_router, router_bias, w_up, w_gate, w_down, ws_up, ws_gate,
                      ws_down, nullptr, y, topk_idx, topk_w, expert_counts, workspace,
                      workspace_bytes, stream, nullptr);
}

int moe_forward_mx(const moe_desc* d, const void* x, const void* w_router,
                   const float* router_bias, const void* w_up, const void* w_gate,
                   const void* w_down, const void* ws_up, const void* ws_gate,
                   const void* ws_down, const moe_mx_scales* scales, void* y,
                   int32_t* topk_idx, float* topk_w, int32_t* expert_counts, void* workspace,
                   size_t workspace_bytes, moe_stream stream, void* const* events) {
  if (!scales) return MOE_ERR_INVALID_ARG;
  return forward_impl(d, x, w_router, router_bias, w_up, w_gate, w_down, ws_up, ws_gate,
                      ws_down, scales, y, topk_idx, topk_w, expert_counts, workspace,
                      workspace_bytes, stream, events);
}

int moe_forward_timed(const moe_desc* d, const void* x, const void* w_router,
                      const float* router_bias, const void* w_up, const void* w_gate,
                      const void* w_down, const void* ws_up, const void* ws_gate,
                      const void* ws_down, void* y, int32_t* topk_idx, float* topk_w,
                      int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                      moe_stream stream, void* const* events) {
  return forward_impl(d, x, w_router, router_bias, w_up, w_gate, w_down, ws_up, ws_gate,
                      ws_down, nullptr, y, topk_idx, topk_w, expert_counts, workspace,
                      workspace_bytes, stream, events);
}

int moe_route(const moe_desc* d, const void* x, const void* w_router, const float* router_bias,
              int32_t* topk_idx, float* topk_w, void* workspace, size_t workspace_bytes,
              moe_stream stream) {
  Plan P;
  bool empty = false;
  int st = prepare(d, workspace, workspace_bytes, &P, &empty);
  if (st != MOE_OK || empty) return st;
  if (!x || !w_router || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if (!a16({x, w_router})) return MOE_ERR_INVALID_ARG;
  Ws W{(char*)workspace};
  MOE_TRY(launch_router(P, x, w_router, router_bias, topk_idx, topk_w,
                        W.at<int32_t>(P.o_blk_hist), W.at<int32_t>(P.o_blk_rank),
                        W.at<float>(P.o_router_part), nullptr, (hipStream_t)stream));
  return MOE_OK;
}

int moe_dispatch(const moe_desc* d, const int32_t* topk_idx, int32_t* expert_counts,
                 int32_t* group_offsets, int32_t* sorted_token, int32_t* slot_row,
                 void* workspace, size_t workspace_bytes, moe_stream stream) {
  Plan P;
  bool empty = false;
  int st = prepare(d, workspace, workspace_bytes, &P, &empty);
  if (st != MOE_OK || empty) return st;
  if (!topk_idx || !expert_counts || !group_offsets || !sorted_token || !slot_row)
    return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  Ws W{(char*)workspace};
  int32_t* blk_hist = W.at<int32_t>(P.o_blk_hist);
  int32_t* blk_rank = W.at<int32_t>(P.o_blk_rank);
  MOE_TRY(launch_block_hist(P, topk_idx, blk_hist, blk_rank, s));
  MOE_TRY(launch_dispatch(P, topk_idx, blk_hist, blk_rank, expert_counts, group_offsets,
                          sorted_token, slot_row, W.at<Tile>(P.o_tiles_up),
                          W.at<Tile>(P.o_tiles_down), s));
  return MOE_OK;
}

int moe_experts(const moe_desc* d, const void* x, const void* w_up, const void* w_gate,
                const void* w_down, const void* ws_up, const void* ws_gate, const void* ws_down,
                const int32_t* group_offsets, const int32_t* sorted_token, float* expert_out,
                void* workspace, size_t workspace_bytes, moe_stream stream) {
  if (d && d->expert_format != MOE_EXPERTS_DENSE) return MOE_ERR_INVALID_ARG;
  Plan P;
  bool empty = false;
  int st = prepare(d, workspace, workspace_bytes, &P, &empty);
  if (st != MOE_OK || empty) return st;
  if (!x || !w_up || !w_gate || !w_down || !group_offsets || !sorted_token || !expert_out)
    return MOE_ERR_INVALID_ARG;
  if (!shared_ok(d, ws_up, ws_gate, ws_down)) return MOE_ERR_INVALID_ARG;
  if (!a16({x, w_up, w_gate, w_down, ws_up, ws_gate, ws_down})) return MOE_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  Ws W{(char*)workspace};
  Tile* tu = W.at<Tile>(P.o_tiles_up);
  Tile* td = W.at<Tile>(P.o_tiles_down);
  MOE_TRY(launch_tiles(P, group_offsets, tu, td, s));
  ExpertArgs a{x, w_up, w_gate, w_down, ws_up, ws_gate, ws_down, sorted_token, tu, td,
               W.at<void>(P.o_h), expert_out, 1, MxScales{}, W.at<float>(P.o_part)};
  MOE_TRY(launch_expert_up(P, a, s));
  MOE_TRY(launch_expert_down(P, a, s));
  return MOE_OK;
}

int moe_combine(const moe_desc* d, const float* expert_out, const float* topk_w,
                const int32_t* slot_row, const int32_t* group_offsets, void* y,
                moe_stream stream) {
  Plan P;
  int st = make_plan(d, &P);
  if (st != MOE_OK || d->T == 0) return st;
  if (!expert_out || !topk_w || !slot_row || !group_offsets || !y) return MOE_ERR_INVALID_ARG;
  MOE_TRY(launch_combine(P, expert_out, 1, 0, topk_w, slot_row, group_offsets, y,
                         (hipStream_t)stream));
  return MOE_OK;
}

}  // extern "C"
