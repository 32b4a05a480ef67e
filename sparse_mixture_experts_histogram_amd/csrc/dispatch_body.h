// Dispatch: group the (token, slot) pairs by expert.
//
// Pages: "Mixture of experts: how MoE works and what it costs", section "What
// mixture of experts costs in compute" (tokens are grouped by expert before
// each feed-forward multiply); "Mixture of Experts: why a model with 671
// billion parameters uses only 37", the router section's per-expert loop and
// the fused-MoE remark (all expert multiplies in one launch over stacked
// weights); the per-expert token count printed in "Mixture of Experts
// Explained: Routers, Active Parameters and VRAM".
//
// Input: per-block expert histograms and in-block stable ranks (written by
// the router).  One workgroup of 1024 threads then
//   1. scans each expert's column of block counts -> expert totals and
//      per-block exclusive offsets (in place);
//   2. scans group sizes (routed experts, then shared experts with T rows
//      each) -> group row offsets;
//   3. writes the two GEMM tile schedules (see build_tiles);
//   4. places each pair at offsets[e] + block_offset[b][e] + rank, which is a
//      stable grouping (pairs of one expert keep increasing t*k+j order);
//      with an expert capacity `cap` (page "Mixture of Experts: why a model
//      with 671 billion parameters uses only 37", "Capacity factor: when
//      tokens don't fit") a pair whose position in its expert's run,
//      block_offset + rank, is cap or more is dropped (slot_row -1), and the
//      expert's group holds min(count, cap) rows;
//   5. fills the shared groups' rows with tokens 0..T-1.
// Everything is integer work and deterministic.  The body is a device
// function so that the router's finish kernel can run it when there is a
// single token block (the router and the dispatch then share one launch).
#pragma once
#include "device.h"
#include "kernels.h"

namespace moe {

constexpr int kDispatchThreads = 1024;
constexpr int kMaxGroups = kMaxExperts + kMaxShared;

struct TileCfg {
  int bm, bn, n_tiles, row_list, n_fastest;
};

// Exclusive scan of v over the block (kDispatchThreads entries, one per
// thread, in thread order); *total receives the sum.  A shuffle scan inside
// each wave, then every thread adds the totals of the waves before it: two
// barriers instead of one per doubling step.  buf holds at least
// kDispatchThreads / 64 ints.
__device__ __forceinline__ int block_excl_scan(int v, int* buf, int* total) {
  constexpr int NWV = kDispatchThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) buf[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const int t = buf[w];
    before += w < wave ? t : 0;
    all += t;
  }
  *total = all;
  __syncthreads();  // buf is free again
  return before + x - v;
}

// block_excl_scan of three values at once (one pair of barriers for all
// three); buf holds at least 3 * kDispatchThreads / 64 ints.
__device__ __forceinline__ void block_excl_scan3(const int (&v)[3], int* buf, int (&ex)[3],
                                                 int (&total)[3]) {
  constexpr int NWV = kDispatchThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x[3] = {v[0], v[1], v[2]};
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      const int y = __shfl_up(x[c], off);
      if (lane >= off) x[c] += y;
    }
  }
  if (lane == 63) {
#pragma unroll
    for (int c = 0; c < 3; ++c) buf[c * NWV + wave] = x[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const int t = buf[c * NWV + w];
      before += w < wave ? t : 0;
      all += t;
    }
    total[c] = all;
    ex[c] = before + x[c] - v[c];
  }
  __syncthreads();  // buf is free again
}

// Tile schedule of one grouped GEMM.  Group g has mt_g = ceil(size_g / bm)
// row tiles and n_tiles column tiles; its entries are laid out in chunks of
// about 32 tiles that hold every row tile of a few consecutive column tiles
// (row tile fastest), so the workgroups that run together on one XCD share
// both the weight tiles and the token tiles through that XCD's L2.
// tiles[0] = {entry count, row tiles, column tiles, 0}.
// The group of each row-tile slot is found once per slot (binary search over
// the group bases) into the LDS table rt_tab when there are at most
// kRowTileTable slots; entries then look it up.  (A search per entry was the
// largest part of the dispatch for layers with many experts and tiles.)
constexpr int kRowTileTable = 4096;
__device__ __forceinline__ int group_of_slot(const int* mbase, int G, int mL) {
  int lo = 0, hi = G - 1;  // largest g with mbase[g] <= mL (a non-empty group)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (mbase[mid] <= mL) lo = mid; else hi = mid - 1;
  }
  return lo;
}
// Entries first, first + stride, ... of the schedule are written by the
// calling thread (first = thread index and stride = block size for one
// workgroup; a global thread index and the grid's thread count when several
// workgroups share the work); the thread with first == 0 writes the header.
// Every workgroup builds the whole row-tile table in its own LDS.
// RL: the schedule is known to be a row-tile list (c.row_list set), so the
// code of the other layout is left out of the kernel.
template <bool RL = false>
__device__ __forceinline__ void build_tiles(const int* goff, const int* gsize, const int* mbase, int G, int mtot,
                            TileCfg c, Tile* tiles, int* rt_tab, int first, int stride) {
  const int total = mtot * c.n_tiles;
  if (first == 0) tiles[0] = Tile{total, mtot, c.n_tiles, 0};
  const bool tab = mtot <= kRowTileTable;
  if (tab) {
    for (int m = threadIdx.x; m < mtot; m += blockDim.x) rt_tab[m] = group_of_slot(mbase, G, m);
    __syncthreads();
  }
  // Row-tile list only: entry 1 + i is row tile i (in group order); a kernel
  // reads entry L as column tile L % n_tiles of row tile L / n_tiles.
  const bool rl = RL || c.row_list;
  const int entries = rl ? mtot : total;
  for (int L = first; L < entries; L += stride) {
    const int mL = rl ? L : L / c.n_tiles;  // row tile "slot"
    const int g = tab ? rt_tab[mL] : group_of_slot(mbase, G, mL);
    if (rl) {
      const int m0 = goff[g] + (mL - mbase[g]) * c.bm;
      tiles[1 + L] = Tile{g, m0, min(m0 + c.bm, goff[g] + gsize[g]), 0};
      continue;
    }
    if constexpr (RL) continue;
    const int Mg = (gsize[g] + c.bm - 1) / c.bm;
    const int local = L - mbase[g] * c.n_tiles;
    const int sn = Mg >= 32 ? 1 : 32 / Mg;
    const int chunk = local / (Mg * sn);
    const int within = local - chunk * Mg * sn;
    const int nin = min(sn, c.n_tiles - chunk * sn);  // column tiles in this chunk
    const int mt = c.n_fastest ? within / nin : within % Mg;
    const int nt = chunk * sn + (c.n_fastest ? within % nin : within / Mg);
    const int m0 = goff[g] + mt * c.bm;
    const int mend = min(m0 + c.bm, goff[g] + gsize[g]);
    tiles[1 + L] = Tile{g, m0, mend, nt * c.bn};
  }
  if (tab) __syncthreads();  // the table is free again
}

// Step 1 for experts [e0, e0 + nE) (nE <= kDispatchThreads), by one
// workgroup: each expert's column of block counts is split into S segments
// of about kBatch blocks (at most kDispatchThreads / Ep), one thread each; a
// thread per expert then walks the S segment sums in order.  Writes the
// expert totals to counts[] and to gsize[] (LDS, capped at cap; indexed from
// e0), and each block's exclusive offset over the column in place.  (S is
// not simply kDispatchThreads / Ep: with few blocks that serial walk over
// mostly empty segments was most of the dispatch time.  Loads go in batches
// of kBatch independent loads: one memory round trip per block was most of
// the dispatch time for many blocks and experts.)
__device__ __forceinline__ void column_scan(int32_t* blk_hist, int nblk, int E, int e0, int nE,
                                            int cap, int32_t* counts, int* gsize, int* part) {
  constexpr int kBatch = 32;
  const int tid = threadIdx.x;
  int Ep = 1;
  while (Ep < nE) Ep <<= 1;
  const int S = min(kDispatchThreads / Ep, max(1, (nblk + kBatch - 1) / kBatch));
  const int el = tid % Ep, seg = tid / Ep, e = e0 + el;
  const int b0 = seg < S ? (int)((int64_t)seg * nblk / S) : 0;
  const int b1 = seg < S ? (int)((int64_t)(seg + 1) * nblk / S) : 0;
  if (el < nE && seg < S) {
    int s = 0;
    for (int b = b0; b < b1; b += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = b + i < b1 ? blk_hist[(int64_t)(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) s += v[i];
    }
    part[seg * Ep + el] = s;
  }
  __syncthreads();
  if (tid < nE) {
    int run = 0;
    for (int q = 0; q < S; ++q) {
      const int v = part[q * Ep + tid];
      part[q * Ep + tid] = run;
      run += v;
    }
    gsize[tid] = min(run, cap);
    counts[e0 + tid] = run;
  }
  __syncthreads();
  if (el < nE && seg < S) {
    int run = part[seg * Ep + el];
    for (int b = b0; b < b1; b += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = b + i < b1 ? blk_hist[(int64_t)(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (b + i < b1) blk_hist[(int64_t)(b + i) * E + e] = run;
        run += v[i];
      }
    }
  }
}

// Steps 2-5 given the group sizes gsize[G] in LDS (routed experts capped at
// the capacity, then the shared groups): group offsets and row-tile bases in
// LDS, then the schedules, the placement of the pairs and the shared rows,
// over thread range (first, stride) as in build_tiles.  ONE_BLOCK: the
// block offsets are zero (a single token block), so blk_hist is not read.
// RL: both schedules are row-tile lists (see build_tiles).
template <bool ONE_BLOCK, bool RL = false>
__device__ __forceinline__ void layout_and_place(
    const int32_t* idx, const int32_t* blk_hist, const int32_t* blk_rank, int T, int k, int E,
    int n_sh, int cap, const int* gsize, int32_t* offsets, int32_t* sorted_token,
    int32_t* slot_row, Tile* tiles_up, TileCfg cu, Tile* tiles_down, TileCfg cd, int first,
    int stride) {
  __shared__ int scan_buf[3 * (kDispatchThreads / 64)];
  __shared__ int goff[kMaxGroups + 1];
  __shared__ int mb_up[kMaxGroups + 1];
  __shared__ int mb_dn[kMaxGroups + 1];
  __shared__ int rt_tab[kRowTileTable];
  const int tid = threadIdx.x;
  const int G = E + n_sh;
  // 2. group offsets; 3. row-tile bases of both schedules
  const int sz = tid < G ? gsize[tid] : 0;
  const int vals[3] = {sz, tid < G ? (sz + cu.bm - 1) / cu.bm : 0,
                       tid < G ? (sz + cd.bm - 1) / cd.bm : 0};
  int ex[3], tot[3];
  block_excl_scan3(vals, scan_buf, ex, tot);
  const int mtot_u = tot[1], mtot_d = tot[2];
  if (tid < G) goff[tid] = ex[0];
  if (tid == 0) goff[G] = tot[0];
  if (tid <= G) mb_up[tid] = tid < G ? ex[1] : mtot_u;
  if (tid <= G) mb_dn[tid] = tid < G ? ex[2] : mtot_d;
  __syncthreads();
  for (int g = first; g <= G; g += stride) offsets[g] = goff[g];
  if (RL && cu.bm == cd.bm) {
    // Two row-tile lists of the same row tiles: each group writes its own
    // entries of both (no group lookup per entry).
    for (int g = first; g < G; g += stride) {
      const int end = goff[g] + gsize[g];
      for (int m = mb_up[g]; m < mb_up[g + 1]; ++m) {
        const int m0 = goff[g] + (m - mb_up[g]) * cu.bm;
        const Tile t{g, m0, min(m0 + cu.bm, end), 0};
        tiles_up[1 + m] = t;
        tiles_down[1 + m] = t;
      }
    }
    if (first == 0) {
      tiles_up[0] = Tile{mtot_u * cu.n_tiles, mtot_u, cu.n_tiles, 0};
      tiles_down[0] = Tile{mtot_d * cd.n_tiles, mtot_d, cd.n_tiles, 0};
    }
  } else {
    build_tiles<RL>(goff, gsize, mb_up, G, mtot_u, cu, tiles_up, rt_tab, first, stride);
    build_tiles<RL>(goff, gsize, mb_dn, G, mtot_d, cd, tiles_down, rt_tab, first, stride);
  }

  // 4. stable placement of the routed pairs, kPlace pairs per thread at a
  // time (their index and rank loads, then their block-offset loads, are
  // each one batch)
  const int pairs = T * k;
  if constexpr (ONE_BLOCK) {
    for (int p = first; p < pairs; p += stride) {
      const int e = idx[p], r = blk_rank[p];
      if (r < cap) {
        slot_row[p] = goff[e] + r;
        sorted_token[goff[e] + r] = p / k;
      } else {
        slot_row[p] = -1;
      }
    }
  } else {
    constexpr int kPlace = 8;
    const uint32_t uk = (uint32_t)k;
    for (int p0 = first; p0 < pairs; p0 += kPlace * stride) {
      int ee[kPlace], rk[kPlace], off[kPlace];
#pragma unroll
      for (int i = 0; i < kPlace; ++i) {
        const int p = p0 + i * stride;
        ee[i] = p < pairs ? idx[p] : 0;
        rk[i] = p < pairs ? blk_rank[p] : 0;
      }
#pragma unroll
      for (int i = 0; i < kPlace; ++i) {
        const int p = p0 + i * stride;
        const int b = (int)((uint32_t)p / uk) / kRouterTokens;
        off[i] = p < pairs ? blk_hist[(int64_t)b * E + ee[i]] : 0;
      }
#pragma unroll
      for (int i = 0; i < kPlace; ++i) {
        const int p = p0 + i * stride;
        if (p >= pairs) continue;
        const int t = (int)((uint32_t)p / uk);
        const int r = off[i] + rk[i];  // position in the expert's run
        if (r < cap) {
          slot_row[p] = goff[ee[i]] + r;
          sorted_token[goff[ee[i]] + r] = t;
        } else {
          slot_row[p] = -1;
        }
      }
    }
  }
  // 5. shared groups: identity rows
  for (int s = 0; s < n_sh; ++s)
    for (int t = first; t < T; t += stride) sorted_token[goff[E + s] + t] = t;
}

// The whole dispatch, run by one workgroup of kDispatchThreads threads.
// ONE_BLOCK: a single token block whose histogram and ranks the same
// workgroup has just computed (the router's fused form: idx, blk_hist and
// blk_rank are LDS arrays, hence no __restrict__); the block's exclusive
// offsets are then all zero and there is no column scan.  Pair indices fit
// in 32 bits (the descriptor check bounds T * (k + n_shared) below 2^31).
// RL: both schedules are row-tile lists.
template <bool ONE_BLOCK, bool RL = false>
__device__ __forceinline__ void dispatch_body(
    const int32_t* idx, int32_t* blk_hist, const int32_t* blk_rank,
    int T, int k, int E, int n_sh, int nblk, int cap, int32_t* counts, int32_t* offsets,
    int32_t* sorted_token, int32_t* slot_row, Tile* tiles_up, TileCfg cu, Tile* tiles_down,
    TileCfg cd) {
  __shared__ int part[kDispatchThreads];
  __shared__ int gsize[kMaxGroups];
  const int tid = threadIdx.x;
  const int G = E + n_sh;
  if constexpr (ONE_BLOCK) {
    if (tid < E) {
      const int run = blk_hist[tid];
      gsize[tid] = min(run, cap);
      counts[tid] = run;
    }
  } else {
    column_scan(blk_hist, nblk, E, 0, E, cap, counts, gsize, part);
  }
  if (tid >= E && tid < G) gsize[tid] = T;
  __syncthreads();
  layout_and_place<ONE_BLOCK, RL>(idx, blk_hist, blk_rank, T, k, E, n_sh, cap, gsize, offsets,
                              sorted_token, slot_row, tiles_up, cu, tiles_down, cd, tid,
                              kDispatchThreads);
}

static inline TileCfg tile_cfg(const GemmShape& s) {
  return TileCfg{s.bm, s.bn, s.n_tiles, s.row_list ? 1 : 0, s.n_fastest};
}

}  // namespace moe
