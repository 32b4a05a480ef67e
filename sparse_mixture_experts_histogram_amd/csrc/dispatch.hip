// Dispatch kernel: see dispatch_body.h.
#include <algorithm>

#include "dispatch_body.h"

namespace moe {

// Token blocks up to which the single-workgroup dispatch runs; experts per
// workgroup of the column scan; most workgroups of the placement kernel.
constexpr int kDispatchOneGroupBlocks = 8;
constexpr int kDispatchScanExperts = 64;
constexpr int kDispatchMaxGroups = 64;

__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(
    const int32_t* __restrict__ idx, int32_t* blk_hist, const int32_t* __restrict__ blk_rank,
    int T, int k, int E, int n_sh, int nblk, int cap, int32_t* counts, int32_t* offsets,
    int32_t* sorted_token, int32_t* slot_row, Tile* tiles_up, TileCfg cu, Tile* tiles_down,
    TileCfg cd) {
  dispatch_body<false>(idx, blk_hist, blk_rank, T, k, E, n_sh, nblk, cap, counts, offsets,
                       sorted_token, slot_row, tiles_up, cu, tiles_down, cd);
}

// With many token blocks the dispatch runs as two multi-workgroup kernels
// instead of dispatch_kernel's one workgroup (whose time grew with the block
// count: 22 us at 32 blocks, 80 us at 256 blocks and 256 experts).
// 1. dispatch_scan_kernel: workgroup x runs the column scan of experts
//    [64 x, 64 x + 64): expert totals to counts[], block offsets in place.
__global__ __launch_bounds__(kDispatchThreads) void dispatch_scan_kernel(int32_t* blk_hist,
                                                                         int nblk, int E,
                                                                         int32_t* counts) {
  __shared__ int part[kDispatchThreads];
  __shared__ int gsize[kDispatchScanExperts];
  const int e0 = blockIdx.x * kDispatchScanExperts;
  column_scan(blk_hist, nblk, E, e0, min(kDispatchScanExperts, E - e0), 0x7fffffff, counts,
              gsize, part);
}

// 2. dispatch_place_kernel: every workgroup rebuilds the group sizes from
//    counts[] and the group offsets in its LDS, then the grid shares the
//    schedule entries, the placement of the pairs and the shared rows.
__global__ __launch_bounds__(kDispatchThreads) void dispatch_place_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ blk_hist,
    const int32_t* __restrict__ blk_rank, int T, int k, int E, int n_sh, int cap,
    const int32_t* __restrict__ counts, int32_t* offsets, int32_t* sorted_token,
    int32_t* slot_row, Tile* tiles_up, TileCfg cu, Tile* tiles_down, TileCfg cd) {
  __shared__ int gsize[kMaxGroups];
  const int tid = threadIdx.x, G = E + n_sh;
  if (tid < G) gsize[tid] = tid < E ? min(counts[tid], cap) : T;
  __syncthreads();
  layout_and_place<false>(idx, blk_hist, blk_rank, T, k, E, n_sh, cap, gsize, offsets,
                          sorted_token, slot_row, tiles_up, cu, tiles_down, cd,
                          blockIdx.x * kDispatchThreads + tid, gridDim.x * kDispatchThreads);
}

// Tile schedules from existing group offsets (used when the expert step is
// called on its own).
__global__ __launch_bounds__(kDispatchThreads) void tiles_kernel(const int32_t* __restrict__ offsets,
                                                                 int G, Tile* tiles_up, TileCfg cu,
                                                                 Tile* tiles_down, TileCfg cd) {
  __shared__ int scan_buf[kDispatchThreads / 64];
  __shared__ int goff[kMaxGroups + 1];
  __shared__ int gsize[kMaxGroups];
  __shared__ int mb_up[kMaxGroups + 1];
  __shared__ int mb_dn[kMaxGroups + 1];
  __shared__ int rt_tab[kRowTileTable];
  const int tid = threadIdx.x;
  if (tid <= G) goff[tid] = offsets[tid];
  __syncthreads();
  const int sz = tid < G ? goff[tid + 1] - goff[tid] : 0;
  if (tid < G) gsize[tid] = sz;
  int mtot_u, mtot_d;
  const int exu = block_excl_scan(tid < G ? (sz + cu.bm - 1) / cu.bm : 0, scan_buf, &mtot_u);
  if (tid <= G) mb_up[tid] = tid < G ? exu : mtot_u;
  const int exd = block_excl_scan(tid < G ? (sz + cd.bm - 1) / cd.bm : 0, scan_buf, &mtot_d);
  if (tid <= G) mb_dn[tid] = tid < G ? exd : mtot_d;
  __syncthreads();
  build_tiles(goff, gsize, mb_up, G, mtot_u, cu, tiles_up, rt_tab, tid, kDispatchThreads);
  build_tiles(goff, gsize, mb_dn, G, mtot_d, cd, tiles_down, rt_tab, tid, kDispatchThreads);
}

hipError_t launch_dispatch(const Plan& P, const int32_t* idx, int32_t* blk_hist,
                           const int32_t* blk_rank, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_token, int32_t* slot_row, Tile* tiles_up,
                           Tile* tiles_down, hipStream_t s) {
  const moe_desc& D = P.desc;
  if (P.nblk <= kDispatchOneGroupBlocks) {
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kDispatchThreads), 0, s, idx, blk_hist,
                       blk_rank, (int)D.T, D.k, D.E, D.n_shared, (int)P.nblk, P.cap, counts,
                       offsets, sorted_token, slot_row, tiles_up, tile_cfg(P.up), tiles_down,
                       tile_cfg(P.down));
    return hipGetLastError();
  }
  hipLaunchKernelGGL(dispatch_scan_kernel,
                     dim3((unsigned)((D.E + kDispatchScanExperts - 1) / kDispatchScanExperts)),
                     dim3(kDispatchThreads), 0, s, blk_hist, (int)P.nblk, D.E, counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // about 8 items (pairs, schedule entries, shared rows) per thread
  const int64_t work = P.pairs + P.up.max_tiles + P.down.max_tiles + (int64_t)D.n_shared * D.T;
  const int64_t per = 8LL * kDispatchThreads;
  const unsigned grid = (unsigned)std::min<int64_t>(kDispatchMaxGroups, (work + per - 1) / per);
  hipLaunchKernelGGL(dispatch_place_kernel, dim3(grid), dim3(kDispatchThreads), 0, s, idx,
                     blk_hist, blk_rank, (int)D.T, D.k, D.E, D.n_shared, P.cap, counts, offsets,
                     sorted_token, slot_row, tiles_up, tile_cfg(P.up), tiles_down,
                     tile_cfg(P.down));
  return hipGetLastError();
}

hipError_t launch_tiles(const Plan& P, const int32_t* offsets, Tile* tiles_up, Tile* tiles_down,
                        hipStream_t s) {
  hipLaunchKernelGGL(tiles_kernel, dim3(1), dim3(kDispatchThreads), 0, s, offsets, P.G, tiles_up,
                     tile_cfg(P.up), tiles_down, tile_cfg(P.down));
  return hipGetLastError();
}

}  // namespace moe
