// Router: logits (x times the E x d router matrix, plus an optional per-expert
// bias), softmax, top-k with lowest-index ties, renormalisation of the kept
// probabilities, and the per-block expert histogram of the chosen pairs.
//
// Steps "Score", "Normalise", "Keep the top k" and "Renormalise" of page
// "Mixture of Experts Explained: Routers, Active Parameters and VRAM"; the
// router as one bias-free linear layer per page "Mixture of Experts: why a
// model with 671 billion parameters uses only 37", section "The router".
//
// One workgroup (4 waves) owns kRouterTokens tokens and every expert (with
// few tokens, several workgroups share a block's K range; see below).  The
// bf16 variant computes the logit tile with 16x16x32 bf16 MFMAs (exact bf16
// products, fp32 accumulation); the K range is split across waves when E
// leaves room for it and the partial tiles are summed in a fixed order.  Selection runs one
// wave per token on order-preserving uint32 keys of the fp32 scores: a
// wave-wide max picks the largest score, and a ballot of the experts holding
// it the lowest expert index among exact ties.  Only the kept logits are needed for the weights:
// w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), which equals renormalising the
// full softmax (page "Mixture of Experts Explained...", section "Softmax
// before or after the top-k step").
//
// Router options (bits of `mode`): kRouteSigmoid ranks sigmoid(l) + bias and
// weights the kept sigmoid(l) (the bias steers the choice only: page
// "Mixture of Experts: why a model with 671 billion parameters uses only 37",
// "How many experts to pick and how to score them"); kRouteRaw leaves the
// kept scores unnormalised (page "Mixture of Experts Explained...", "Why
// top-1 routing cannot renormalise"), so softmax weights then divide by the
// sum over all E experts, one more pass over the token's logits.
#include "device.h"
#include "dispatch_body.h"
#include "kernels.h"

namespace moe {

// Histogram of one block's pairs and each pair's rank among earlier pairs of
// the same expert (sel holds the block's n_pairs expert ids in pair order).
// The pairs are compared in batches of 16 independent LDS reads (a loop of
// one dependent read per pair was most of the router's tail time).
__device__ __forceinline__ void block_hist_rank(const int32_t* sel, int n_pairs, int E, int32_t* hist_out,
                                int32_t* rank_out) {
  constexpr int B = 16;
  for (int p = threadIdx.x; p < n_pairs; p += blockDim.x) {
    const int e = sel[p];
    int r = 0;
    for (int q0 = 0; q0 < p; q0 += B) {
      int v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) v[i] = q0 + i < p ? sel[q0 + i] : -1;
#pragma unroll
      for (int i = 0; i < B; ++i) r += (v[i] == e);
    }
    rank_out[p] = r;
  }
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
    for (int q0 = 0; q0 < n_pairs; q0 += B) {
      int v[B];
#pragma unroll
      for (int i = 0; i < B; ++i) v[i] = q0 + i < n_pairs ? sel[q0 + i] : -1;
#pragma unroll
      for (int i = 0; i < B; ++i) c += (v[i] == e);
    }
    hist_out[e] = c;
  }
}

// Top-k of the tokens of one block from LDS logits lg[tl*ld + e].
template <int EPL>
__device__ __forceinline__ void topk_block(const float* lg, int ld, const float* __restrict__ bias, int mode,
                           int t0, int T, int E, int k, int32_t* __restrict__ idx_out,
                           float* __restrict__ w_out, int32_t* sel) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  const bool sig = mode & kRouteSigmoid, raw = mode & kRouteRaw;
  for (int tl = wave; tl < kRouterTokens; tl += nwaves) {
    const int t = t0 + tl;
    if (t >= T) break;
    const float* lt = lg + tl * ld;
    // Selection key of expert e = lane + 64 i: the order-preserving uint32 of
    // its score; bit i of `live` marks an expert that exists and is not yet
    // chosen.  Each pick takes the wave's largest live key and, among live
    // keys equal to it, the lowest expert index (one ballot per i, lowest i
    // first, then the lowest lane).
    uint32_t key[EPL];
    uint32_t live = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + 64 * i;
      key[i] = 0;
      if (e < E) {
        const float b = bias ? bias[e] : 0.0f;
        const float v = sig ? sigmoid_f32(lt[e]) + b : lt[e] + b;
        key[i] = order_key(v);
        live |= 1u << i;
      }
    }
    // kept score of slot j: exp(v_j - v_0) (softmax numerator relative to
    // the largest key) or sigmoid(l_j)
    float v0 = 0.f, wsum = 0.f, my_w = 0.f;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (((live >> i) & 1u) && key[i] > m) m = key[i];
      m = wave_max_u32(m);
      int e = -1;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const uint64_t hit = __ballot(((live >> i) & 1u) && key[i] == m);
        if (e < 0 && hit) e = 64 * i + __builtin_ctzll(hit);
      }
      if (lane == (e & 63)) live &= ~(1u << (e >> 6));
      const float v = order_key_inv(m);
      if (j == 0) v0 = v;
      const float sc = sig ? sigmoid_f32(lt[e]) : expf(v - v0);
      wsum += sc;
      if (lane == j) {
        my_w = sc;
        my_e = e;
      }
    }
    float denom = wsum;
    if (raw) {
      if (sig) {
        denom = 1.0f;
      } else {  // softmax over all E experts
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
          const int e = lane + 64 * i;
          if (e < E) s += expf(lt[e] + (bias ? bias[e] : 0.0f) - v0);
        }
        denom = wave_sum_f32(s);
      }
    }
    if (lane < k) {
      idx_out[(int64_t)t * k + lane] = my_e;
      w_out[(int64_t)t * k + lane] = my_w / denom;
      sel[tl * k + lane] = my_e;
    }
  }
}

// Top-k, then this block's histogram and ranks into hist_out[E] and
// rank_out[pairs of the block] (global memory, or LDS in the fused dispatch).
template <int EPL>
__device__ __forceinline__ void router_tail(float* lg, int ld, int32_t* sel, const float* bias, int mode, int t0,
                            int T, int E, int k, int32_t* idx_out, float* w_out,
                            int32_t* hist_out, int32_t* rank_out) {
  topk_block<EPL>(lg, ld, bias, mode, t0, T, E, k, idx_out, w_out, sel);
  __syncthreads();
  const int nt = min(kRouterTokens, T - t0);
  block_hist_rank(sel, nt * k, E, hist_out, rank_out);
}

__device__ __forceinline__ void router_tail_to(float* lg, int ld, int32_t* sel, const float* bias, int mode,
                               int t0, int T, int E, int k, int32_t* idx_out, float* w_out,
                               int32_t* hist_out, int32_t* rank_out) {
  if (E <= 64)
    router_tail<1>(lg, ld, sel, bias, mode, t0, T, E, k, idx_out, w_out, hist_out, rank_out);
  else if (E <= 128)
    router_tail<2>(lg, ld, sel, bias, mode, t0, T, E, k, idx_out, w_out, hist_out, rank_out);
  else if (E <= 256)
    router_tail<4>(lg, ld, sel, bias, mode, t0, T, E, k, idx_out, w_out, hist_out, rank_out);
  else
    router_tail<8>(lg, ld, sel, bias, mode, t0, T, E, k, idx_out, w_out, hist_out, rank_out);
}

// The usual tail: the block's histogram and ranks go to global memory for
// the dispatch kernel.
__device__ __forceinline__ void router_tail_dispatch(float* lg, int ld, int32_t* sel, const float* bias, int mode,
                                     int t0, int T, int E, int k, int32_t* idx_out, float* w_out,
                                     int32_t* blk_hist, int32_t* blk_rank) {
  router_tail_to(lg, ld, sel, bias, mode, t0, T, E, k, idx_out, w_out,
                 blk_hist + (int64_t)blockIdx.x * E, blk_rank + (int64_t)t0 * k);
}

// Logits of the kRouterTokens tokens from t0 over k-steps [kb0, kb1) (32 k
// each) for every expert, into lg[16][ld] (LDS, which must hold KS partial
// tiles [KS][16][ld]).  NW waves: wave w sums K part w % KS of the expert
// tiles w / KS + i NW / KS; the KS partial tiles are then added in order.
template <int NT, int NW>
__device__ __forceinline__ void block_logits(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                             int T, int d, int E, int KS, int t0, int kb0, int kb1, float* lg,
                             int ld) {
  const int etiles = (E + 15) >> 4;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ks = wave % KS, tg = wave / KS, tstep = NW / KS;

  int row = t0 + (lane & 15);
  row = row < T ? row : T - 1;
  const uint16_t* xp = x + (int64_t)row * d + (lane >> 4) * 8;
  const uint16_t* wp[NT];
  f32x4 acc[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    int e = (tg + i * tstep) * 16 + (lane & 15);
    e = e < E ? e : E - 1;
    wp[i] = wr + (int64_t)e * d + (lane >> 4) * 8;
    acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // K loop in batches of U k-steps: all loads of a batch are issued before
  // its MFMAs, so each wave keeps U*(NT+1) 16-byte loads per lane in flight.
  // The last batch re-reads the last k-step for its slots past the range and
  // zeroes their token fragment, so every batch is one round of loads.
  // Tiles past the last expert read a clamped row and are not stored.
  constexpr int U = NT <= 2 ? 8 : 4;
  const int c0 = kb0 + ks * (kb1 - kb0) / KS, c1 = kb0 + (ks + 1) * (kb1 - kb0) / KS;
  for (int c = c0; c < c1; c += U) {
    u32x4 a[U], b[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int cu = min(c + u, c1 - 1);
      a[u] = *(const u32x4*)(xp + cu * 32);
#pragma unroll
      for (int i = 0; i < NT; ++i) b[u][i] = *(const u32x4*)(wp[i] + cu * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c + u >= c1) a[u] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < NT; ++i) acc[i] = mfma16(a[u], b[u][i], acc[i]);
    }
    __builtin_amdgcn_sched_group_barrier(0x020, U * (NT + 1), 0);  // every load first
    __builtin_amdgcn_sched_group_barrier(0x008, U * NT, 0);        // then the MFMAs
  }
  // D[m = token][n = expert]: lane holds expert (lane & 15), tokens 4*(lane>>4)+r
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int tile = tg + i * tstep;
    if (tile < etiles) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lg[(ks * kRouterTokens + 4 * (lane >> 4) + r) * ld + tile * 16 + (lane & 15)] = acc[i][r];
    }
  }
  __syncthreads();
  if (KS > 1) {
    for (int i = threadIdx.x; i < kRouterTokens * ld; i += blockDim.x) {
      float s = lg[i];
      for (int q = 1; q < KS; ++q) s += lg[q * kRouterTokens * ld + i];
      lg[i] = s;
    }
    __syncthreads();
  }
}

// One token block per workgroup, whole K.  Dynamic LDS: KS partial logit
// tiles [KS][16][ld] floats, then sel[16*k].
template <int NT, int NW>
__global__ __launch_bounds__(64 * NW) void router_bf16_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
    const float* __restrict__ bias, int mode, int T, int d, int E, int k, int KS,
    int32_t* idx_out, float* w_out, int32_t* blk_hist, int32_t* blk_rank) {
  extern __shared__ float lds[];
  const int ld = ((E + 15) >> 4) * 16 + 4;
  int32_t* sel = (int32_t*)(lds + KS * kRouterTokens * ld);
  const int t0 = blockIdx.x * kRouterTokens;
  block_logits<NT, NW>(x, wr, T, d, E, KS, t0, 0, d >> 5, lds, ld);
  router_tail_dispatch(lds, ld, sel, bias, mode, t0, T, E, k, idx_out, w_out, blk_hist,
                       blk_rank);
}

// Few token blocks: workgroup b computes the logits of token block
// b % nblk over K part b / nblk of nsplit and writes them to
// part[split][token][e] (rows of ep = 16 * expert tiles floats).
template <int NT, int NW>
__global__ __launch_bounds__(64 * NW) void router_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E, int KS,
    int nblk, int nsplit, float* __restrict__ part) {
  extern __shared__ float lds[];
  const int ep = ((E + 15) >> 4) * 16, ld = ep + 4;
  const int blk = blockIdx.x % nblk, split = blockIdx.x / nblk;
  const int t0 = blk * kRouterTokens, nk = d >> 5;
  block_logits<NT, NW>(x, wr, T, d, E, KS, t0, split * nk / nsplit, (split + 1) * nk / nsplit,
                       lds, ld);
  float* dst = part + ((int64_t)split * nblk * kRouterTokens + t0) * ep;
  for (int i = threadIdx.x; i < kRouterTokens * ep; i += blockDim.x)
    dst[i] = lds[(i / ep) * ld + i % ep];
}

// Many tokens and a large router matrix: each workgroup of the one-kernel
// router would stream the whole matrix for its 16 tokens (the DeepSeek-V3-
// shaped router, 3.67 MB, 256 times over).  Here a workgroup takes 64 tokens
// (four 16-token tiles, each weight fragment used for all four) over K part
// blockIdx.x / ngroups of nsplit, and writes part[split][token][e] for the
// finish kernel.  Wave w owns expert tiles w, w + 4, ... (NT of them); the K
// loop issues U k-steps of loads per batch before their MFMAs.
template <int NT>
__global__ __launch_bounds__(256) void router_wide_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E,
    int ngroups, int nsplit, float* __restrict__ part) {
  constexpr int TT = 4, U = 4;
  const int ep = ((E + 15) >> 4) * 16, etiles = ep >> 4;
  // split fastest: with 8 (or 4) K parts, each XCD (workgroup i runs on XCD
  // i % 8) reads one part of the router matrix, which stays in its L2
  const int split = blockIdx.x % nsplit, grp = blockIdx.x / nsplit;
  const int t0 = grp * (16 * TT);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint16_t* xp[TT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    int row = t0 + 16 * tt + (lane & 15);
    row = row < T ? row : T - 1;
    xp[tt] = x + (int64_t)row * d + (lane >> 4) * 8;
  }
  const uint16_t* wp[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    int e = (wave + 4 * i) * 16 + (lane & 15);
    e = e < E ? e : E - 1;
    wp[i] = wr + (int64_t)e * d + (lane >> 4) * 8;
  }
  f32x4 acc[TT][NT];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[tt][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nk = d >> 5;
  const int c0 = split * nk / nsplit, c1 = (split + 1) * nk / nsplit;
  for (int c = c0; c < c1; c += U) {
    u32x4 a[U][TT], b[U][NT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int cu = min(c + u, c1 - 1);
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) a[u][tt] = *(const u32x4*)(xp[tt] + cu * 32);
#pragma unroll
      for (int i = 0; i < NT; ++i) b[u][i] = *(const u32x4*)(wp[i] + cu * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (c + u >= c1) continue;
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[tt][i] = mfma16(a[u][tt], b[u][i], acc[tt][i]);
    }
  }
  // D[m = token][n = expert]: lane holds expert (lane & 15), tokens 4*(lane>>4)+r
  float* dst = part + ((int64_t)split * ngroups * (16 * TT) + t0) * ep;
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    const int tile = wave + 4 * i;
    if (tile >= etiles) continue;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dst[(int64_t)(16 * tt + 4 * (lane >> 4) + r) * ep + tile * 16 + (lane & 15)] = acc[tt][i][r];
  }
}

// Where the finish kernel runs the dispatch (null counts: it does not).
struct FusedDispatch {
  int32_t *counts, *offsets, *sorted_token, *slot_row;
  Tile *tiles_up, *tiles_down;
  TileCfg cu, cd;
  int n_sh, cap;
};

// Adds the nsplit (<= kMaxRouterSplit) partial logits of a token block in
// split order (partial q of token t at part[q * plane + t * ep + e]), then
// the same selection as the one-kernel router.  All
// partial loads of an element are issued before the first add, so the sum
// costs one memory round trip.  With a single token block and fd.counts
// set, the one workgroup then runs the whole dispatch (dispatch_body.h) on
// the indices, histogram and ranks it has just computed (kept in LDS), which
// saves the dispatch launch.  (With several blocks that would take a device-scope
// fence, which writes back and invalidates L2 and measured slower than the
// separate launch.)  kDispatchThreads threads; dynamic LDS: [16][ld] floats,
// then sel[16*k].
// EPL = experts per lane of the selection (E <= 64 EPL); FUSED: the single
// token block's workgroup also runs the dispatch.  Each (EPL, FUSED) pair is
// its own kernel so that a launch carries only the code it runs: these
// kernels run once per layer on one or a few workgroups, and a kernel holding
// every selection width and both tails was large enough for instruction
// fetch to dominate its time.
// FUSED: 0 no dispatch, 1 the dispatch, 2 the dispatch of two row-tile-list
// schedules (the decode kernels' layout; the other layout's code left out).
template <int EPL, int FUSED>
__global__ __launch_bounds__(kDispatchThreads) void router_finish_kernel(
    const float* __restrict__ part, int64_t plane, const float* __restrict__ bias, int mode, int T,
    int E, int k, int nblk, int nsplit, int32_t* idx_out, float* w_out, int32_t* blk_hist,
    int32_t* blk_rank, FusedDispatch fd) {
  extern __shared__ float lds[];
  const int ep = ((E + 15) >> 4) * 16, ld = ep + 4;
  int32_t* sel = (int32_t*)(lds + kRouterTokens * ld);
  const int t0 = blockIdx.x * kRouterTokens;
  const float* src = part + (int64_t)t0 * ep;
  // rows of the block's tokens only (the selection reads no others): with a
  // few tokens, one batch of loads per thread
  const int nt = min(kRouterTokens, T - t0);
  for (int i = threadIdx.x; i < nt * ep; i += blockDim.x) {
    float v[kMaxRouterSplit];
#pragma unroll
    for (int q = 0; q < kMaxRouterSplit; ++q) v[q] = src[(q < nsplit ? q : 0) * plane + i];
    float s = v[0];
#pragma unroll
    for (int q = 1; q < kMaxRouterSplit; ++q)
      if (q < nsplit) s += v[q];
    lds[(i / ep) * ld + i % ep] = s;
  }
  __syncthreads();
  if constexpr (!FUSED) {
    router_tail<EPL>(lds, ld, sel, bias, mode, t0, T, E, k, idx_out, w_out,
                     blk_hist + (int64_t)blockIdx.x * E, blk_rank + (int64_t)t0 * k);
  } else {
    // Fused dispatch (one token block, t0 = 0): the block's expert ids (sel,
    // in pair order), histogram and ranks stay in LDS for the dispatch
    // instead of a round trip through global memory.
    __shared__ int32_t f_hist[kMaxExperts];
    __shared__ int32_t f_rank[kRouterTokens * kMaxTopK];
    router_tail<EPL>(lds, ld, sel, bias, mode, t0, T, E, k, idx_out, w_out, f_hist, f_rank);
    __syncthreads();
    dispatch_body<true, FUSED == 2>(sel, f_hist, f_rank, T, k, E, fd.n_sh, nblk, fd.cap,
                                    fd.counts, fd.offsets, fd.sorted_token, fd.slot_row,
                                    fd.tiles_up, fd.cu, fd.tiles_down, fd.cd);
  }
}

// The finish kernel for E experts (and the fused dispatch or not).
template <int FUSED>
hipError_t launch_finish(dim3 grid, size_t lds, hipStream_t s, const float* part, int64_t plane,
                         const float* bias, int mode, int T, int E, int k, int nblk, int nsplit,
                         int32_t* idx, float* w, int32_t* blk_hist, int32_t* blk_rank,
                         FusedDispatch fd) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kDispatchThreads), lds, s, part, plane, bias, mode, T, E,
                       k, nblk, nsplit, idx, w, blk_hist, blk_rank, fd);
  };
  if (E <= 64)
    go(router_finish_kernel<1, FUSED>);
  else if (E <= 128)
    go(router_finish_kernel<2, FUSED>);
  else if (E <= 256)
    go(router_finish_kernel<4, FUSED>);
  else
    go(router_finish_kernel<8, FUSED>);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void router_f32_kernel(
    const float* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ bias,
    int mode, int T, int d, int E, int k, int32_t* idx_out, float* w_out, int32_t* blk_hist,
    int32_t* blk_rank) {
  extern __shared__ float lds[];
  const int ld = E + 1;
  float* lg = lds;
  int32_t* sel = (int32_t*)(lds + kRouterTokens * ld);
  const int t0 = blockIdx.x * kRouterTokens;
  for (int p = threadIdx.x; p < kRouterTokens * E; p += blockDim.x) {
    const int tl = p / E, e = p % E;
    const int t = t0 + tl;
    float acc = 0.f;
    if (t < T) {
      const float4* xr = (const float4*)(x + (int64_t)t * d);
      const float4* wrow = (const float4*)(wr + (int64_t)e * d);
      for (int c = 0; c < (d >> 2); ++c) {
        const float4 a = xr[c], b = wrow[c];
        acc = fmaf(a.x, b.x, acc);
        acc = fmaf(a.y, b.y, acc);
        acc = fmaf(a.z, b.z, acc);
        acc = fmaf(a.w, b.w, acc);
      }
    }
    lg[tl * ld + e] = acc;
  }
  __syncthreads();
  router_tail_dispatch(lg, ld, sel, bias, mode, t0, T, E, k, idx_out, w_out, blk_hist, blk_rank);
}

__global__ __launch_bounds__(256) void block_hist_kernel(const int32_t* __restrict__ idx, int T,
                                                         int E, int k, int32_t* blk_hist,
                                                         int32_t* blk_rank) {
  extern __shared__ int32_t sel_lds[];
  const int t0 = blockIdx.x * kRouterTokens;
  const int n = min(kRouterTokens, T - t0) * k;
  for (int p = threadIdx.x; p < n; p += blockDim.x) sel_lds[p] = idx[(int64_t)t0 * k + p];
  __syncthreads();
  block_hist_rank(sel_lds, n, E, blk_hist + (int64_t)blockIdx.x * E, blk_rank + (int64_t)t0 * k);
}

hipError_t launch_router(const Plan& P, const void* x, const void* w_router, const float* bias,
                         int32_t* idx, float* w, int32_t* blk_hist, int32_t* blk_rank,
                         float* part, const DispatchOut* dout, hipStream_t s) {
  const moe_desc& D = P.desc;
  const dim3 grid((unsigned)P.nblk);
  const size_t sel_bytes = (size_t)kRouterTokens * D.k * 4;
  if (D.dtype == MOE_F32) {
    const size_t lds = (size_t)kRouterTokens * (D.E + 1) * 4 + sel_bytes;
    hipLaunchKernelGGL(router_f32_kernel, grid, dim3(256), lds, s, (const float*)x,
                       (const float*)w_router, bias, P.route_mode, (int)D.T, D.d, D.E, D.k, idx,
                       w, blk_hist, blk_rank);
    return hipGetLastError();
  }
  // 4 waves; K is split over as many of them as the expert tiles leave free
  // (KS = 4 / tiles, a power of two).  With few token blocks, K is also
  // split over P.rsplit workgroups per block and a second kernel adds the
  // partial logits: one workgroup streaming the whole router matrix pays
  // one ~2 us memory round trip per batch of loads (measured on MI355X:
  // gpt-oss-shaped T=1, E=128, d=2880: 28 us in one kernel).
  constexpr int NW = 4;
  const int etiles = (D.E + 15) / 16;
  int KS = NW;
  while (KS > 1 && KS * etiles > NW) KS >>= 1;
  const int nt = (etiles + (NW / KS) - 1) / (NW / KS);
  const int ld = etiles * 16 + 4;
  const size_t lds = (size_t)KS * kRouterTokens * ld * 4 + sel_bytes;
  const uint16_t* xb = (const uint16_t*)x;
  const uint16_t* wb = (const uint16_t*)w_router;
  const int64_t ep = etiles * 16;
  if (P.rwide) {
    const int ngroups = (int)((D.T + P.rwide - 1) / P.rwide);
    const dim3 pgrid((unsigned)(ngroups * P.rsplit));
    auto partial = [&](auto kern) {
      hipLaunchKernelGGL(kern, pgrid, dim3(256), 0, s, xb, wb, (int)D.T, D.d, D.E, ngroups,
                         P.rsplit, part);
    };
    const int ntw = (etiles + 3) / 4;
    if (ntw <= 1)
      partial(router_wide_partial_kernel<1>);
    else if (ntw <= 2)
      partial(router_wide_partial_kernel<2>);
    else if (ntw <= 4)
      partial(router_wide_partial_kernel<4>);
    else
      partial(router_wide_partial_kernel<8>);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_finish<0>(grid, (size_t)kRouterTokens * ld * 4 + sel_bytes, s, part,
                                (int64_t)ngroups * P.rwide * ep, bias, P.route_mode, (int)D.T, D.E,
                                D.k, (int)P.nblk, P.rsplit, idx, w, blk_hist, blk_rank,
                                FusedDispatch{});
  }
  if (P.rsplit > 1) {
    FusedDispatch fd{};
    if (dout && P.nblk == 1) {
      fd = FusedDispatch{dout->counts, dout->offsets, dout->sorted_token, dout->slot_row,
                         dout->tiles_up, dout->tiles_down, tile_cfg(P.up), tile_cfg(P.down),
                         D.n_shared, P.cap};
    }
    const dim3 pgrid((unsigned)(P.nblk * P.rsplit));
    auto partial = [&](auto kern) {
      hipLaunchKernelGGL(kern, pgrid, dim3(64 * NW), lds, s, xb, wb, (int)D.T, D.d, D.E, KS,
                         (int)P.nblk, P.rsplit, part);
    };
    if (nt <= 1)
      partial(router_partial_kernel<1, NW>);
    else if (nt <= 2)
      partial(router_partial_kernel<2, NW>);
    else if (nt <= 4)
      partial(router_partial_kernel<4, NW>);
    else
      partial(router_partial_kernel<8, NW>);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t flds = (size_t)kRouterTokens * ld * 4 + sel_bytes;
    const int64_t plane = (int64_t)P.nblk * kRouterTokens * ep;
    if (fd.counts && fd.cu.row_list && fd.cd.row_list)
      return launch_finish<2>(grid, flds, s, part, plane, bias, P.route_mode, (int)D.T, D.E,
                              D.k, (int)P.nblk, P.rsplit, idx, w, blk_hist, blk_rank, fd);
    if (fd.counts)
      return launch_finish<1>(grid, flds, s, part, plane, bias, P.route_mode, (int)D.T, D.E,
                              D.k, (int)P.nblk, P.rsplit, idx, w, blk_hist, blk_rank, fd);
    return launch_finish<0>(grid, flds, s, part, plane, bias, P.route_mode, (int)D.T, D.E,
                                D.k, (int)P.nblk, P.rsplit, idx, w, blk_hist, blk_rank, fd);
  }
  auto args = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(64 * NW), lds, s, xb, wb, bias, P.route_mode, (int)D.T,
                       D.d, D.E, D.k, KS, idx, w, blk_hist, blk_rank);
  };
  if (nt <= 1)
    args(router_bf16_kernel<1, NW>);
  else if (nt <= 2)
    args(router_bf16_kernel<2, NW>);
  else if (nt <= 4)
    args(router_bf16_kernel<4, NW>);
  else
    args(router_bf16_kernel<8, NW>);
  return hipGetLastError();
}

hipError_t launch_block_hist(const Plan& P, const int32_t* idx, int32_t* blk_hist,
                             int32_t* blk_rank, hipStream_t s) {
  const moe_desc& D = P.desc;
  hipLaunchKernelGGL(block_hist_kernel, dim3((unsigned)P.nblk), dim3(256),
                     (size_t)kRouterTokens * D.k * 4, s, idx, (int)D.T, D.E, D.k, blk_hist,
                     blk_rank);
  return hipGetLastError();
}

}  // namespace moe
