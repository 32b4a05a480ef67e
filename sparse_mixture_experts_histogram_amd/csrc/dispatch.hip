// Dispatch kernel: see dispatch_body.h.
#include "dispatch_body.h"

namespace moe {

__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(
    const int32_t* __restrict__ idx, int32_t* blk_hist, const int32_t* __restrict__ blk_rank,
    int T, int k, int E, int n_sh, int nblk, int cap, int32_t* counts, int32_t* offsets,
    int32_t* sorted_token, int32_t* slot_row, Tile* tiles_up, TileCfg cu, Tile* tiles_down,
    TileCfg cd) {
  dispatch_body<false>(idx, blk_hist, blk_rank, T, k, E, n_sh, nblk, cap, counts, offsets,
                       sorted_token, slot_row, tiles_up, cu, tiles_down, cd);
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
  build_tiles(goff, gsize, mb_up, G, mtot_u, cu, tiles_up, rt_tab);
  build_tiles(goff, gsize, mb_dn, G, mtot_d, cd, tiles_down, rt_tab);
}

hipError_t launch_dispatch(const Plan& P, const int32_t* idx, int32_t* blk_hist,
                           const int32_t* blk_rank, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_token, int32_t* slot_row, Tile* tiles_up,
                           Tile* tiles_down, hipStream_t s) {
  const moe_desc& D = P.desc;
  hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kDispatchThreads), 0, s, idx, blk_hist,
                     blk_rank, (int)D.T, D.k, D.E, D.n_shared, (int)P.nblk, P.cap, counts, offsets,
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
