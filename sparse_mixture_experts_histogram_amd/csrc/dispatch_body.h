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
__device__ __forceinline__ void build_tiles(const int* goff, const int* gsize, const int* mbase, int G, int mtot,
                            TileCfg c, Tile* tiles, int* rt_tab) {
  const int total = mtot * c.n_tiles;
  if (threadIdx.x == 0) tiles[0] = Tile{total, mtot, c.n_tiles, 0};
  const bool tab = mtot <= kRowTileTable;
  if (tab) {
    for (int m = threadIdx.x; m < mtot; m += blockDim.x) rt_tab[m] = group_of_slot(mbase, G, m);
    __syncthreads();
  }
  // Row-tile list only: entry 1 + i is row tile i (in group order); a kernel
  // reads entry L as row tile L % mtot of column tile L / mtot.
  const int entries = c.row_list ? mtot : total;
  for (int L = threadIdx.x; L < entries; L += blockDim.x) {
    const int mL = c.row_list ? L : L / c.n_tiles;  // row tile "slot"
    const int g = tab ? rt_tab[mL] : group_of_slot(mbase, G, mL);
    if (c.row_list) {
      const int m0 = goff[g] + (mL - mbase[g]) * c.bm;
      tiles[1 + L] = Tile{g, m0, min(m0 + c.bm, goff[g] + gsize[g]), 0};
      continue;
    }
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

// The whole dispatch, run by one workgroup of kDispatchThreads threads.
// (No __restrict__: in the router's fused form idx, blk_hist and blk_rank
// are LDS arrays the same workgroup has just written.)
__device__ __forceinline__ void dispatch_body(
    const int32_t* idx, int32_t* blk_hist, const int32_t* blk_rank,
    int T, int k, int E, int n_sh, int nblk, int cap, int32_t* counts, int32_t* offsets,
    int32_t* sorted_token, int32_t* slot_row, Tile* tiles_up, TileCfg cu, Tile* tiles_down,
    TileCfg cd) {
  __shared__ int part[kDispatchThreads];
  __shared__ int scan_buf[kDispatchThreads / 64];
  __shared__ int goff[kMaxGroups + 1];
  __shared__ int gsize[kMaxGroups];
  __shared__ int mb_up[kMaxGroups + 1];
  __shared__ int mb_dn[kMaxGroups + 1];
  __shared__ int rt_tab[kRowTileTable];
  const int tid = threadIdx.x;
  const int G = E + n_sh;

  // 1. column scans of the block histogram: expert e's column is split into
  // S segments of about kBatch blocks (at most kDispatchThreads / Ep), one
  // thread each; a thread per expert then walks the S segment sums in order.
  // (S is not simply kDispatchThreads / Ep: with few blocks that serial walk
  // over mostly empty segments was most of the dispatch time.)
  constexpr int kBatch = 32;
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int S = min(kDispatchThreads / Ep, max(1, (nblk + kBatch - 1) / kBatch));
  const int e = tid % Ep, seg = tid / Ep;
  const int b0 = seg < S ? (int)((int64_t)seg * nblk / S) : 0;
  const int b1 = seg < S ? (int)((int64_t)(seg + 1) * nblk / S) : 0;
  // (Loads go in batches of kBatch independent loads: a thread walks up to
  // nblk / S blocks, and one memory round trip per block was most of the
  // dispatch time for many blocks and experts.)
  if (e < E && seg < S) {
    int s = 0;
    for (int b = b0; b < b1; b += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = b + i < b1 ? blk_hist[(int64_t)(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) s += v[i];
    }
    part[seg * Ep + e] = s;
  }
  __syncthreads();
  if (tid < E) {
    int run = 0;
    for (int q = 0; q < S; ++q) {
      const int v = part[q * Ep + tid];
      part[q * Ep + tid] = run;
      run += v;
    }
    gsize[tid] = min(run, cap);
    counts[tid] = run;
  }
  __syncthreads();
  if (e < E && seg < S) {
    int run = part[seg * Ep + e];
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
  if (tid >= E && tid < G) gsize[tid] = T;
  __syncthreads();

  // 2. group offsets; 3. row-tile bases of both schedules
  int total;
  const int sz = tid < G ? gsize[tid] : 0;
  const int ex = block_excl_scan(sz, scan_buf, &total);
  if (tid < G) goff[tid] = ex;
  if (tid == 0) goff[G] = total;
  const int mu = tid < G ? (sz + cu.bm - 1) / cu.bm : 0;
  int mtot_u;
  const int exu = block_excl_scan(mu, scan_buf, &mtot_u);
  if (tid <= G) mb_up[tid] = tid < G ? exu : mtot_u;
  const int md = tid < G ? (sz + cd.bm - 1) / cd.bm : 0;
  int mtot_d;
  const int exd = block_excl_scan(md, scan_buf, &mtot_d);
  if (tid <= G) mb_dn[tid] = tid < G ? exd : mtot_d;
  __syncthreads();
  for (int g = tid; g <= G; g += blockDim.x) offsets[g] = goff[g];
  build_tiles(goff, gsize, mb_up, G, mtot_u, cu, tiles_up, rt_tab);
  build_tiles(goff, gsize, mb_dn, G, mtot_d, cd, tiles_down, rt_tab);

  // 4. stable placement of the routed pairs, kPlace pairs per thread at a
  // time (their index and rank loads, then their block-offset loads, are
  // each one batch)
  constexpr int kPlace = 8;
  const int64_t pairs = (int64_t)T * k;
  for (int64_t p0 = tid; p0 < pairs; p0 += (int64_t)kPlace * blockDim.x) {
    int ee[kPlace], rk[kPlace], off[kPlace];
#pragma unroll
    for (int i = 0; i < kPlace; ++i) {
      const int64_t p = p0 + (int64_t)i * blockDim.x;
      ee[i] = p < pairs ? idx[p] : 0;
      rk[i] = p < pairs ? blk_rank[p] : 0;
    }
#pragma unroll
    for (int i = 0; i < kPlace; ++i) {
      const int64_t p = p0 + (int64_t)i * blockDim.x;
      const int b = (int)(p / k) / kRouterTokens;
      off[i] = p < pairs ? blk_hist[(int64_t)b * E + ee[i]] : 0;
    }
#pragma unroll
    for (int i = 0; i < kPlace; ++i) {
      const int64_t p = p0 + (int64_t)i * blockDim.x;
      if (p >= pairs) continue;
      const int t = (int)(p / k);
      const int r = off[i] + rk[i];  // position in the expert's run
      if (r < cap) {
        slot_row[p] = goff[ee[i]] + r;
        sorted_token[goff[ee[i]] + r] = t;
      } else {
        slot_row[p] = -1;
      }
    }
  }
  // 5. shared groups: identity rows
  for (int s = 0; s < n_sh; ++s)
    for (int t = tid; t < T; t += blockDim.x) sorted_token[goff[E + s] + t] = t;
}

static inline TileCfg tile_cfg(const GemmShape& s) {
  return TileCfg{s.bm, s.bn, s.n_tiles, s.row_list ? 1 : 0, s.n_fastest};
}

}  // namespace moe
