// Weighted combine: y[t] = sum_{j<k} w[t,j] * out[slot_row[t,j]] + sum_s
// out[offsets[E+s] + t], summed in that order in float32 (step "Run and
// combine" of page "Mixture of Experts Explained: Routers, Active Parameters
// and VRAM"; shared experts added with weight one per page "Mixture of Experts
// (MoE): routing, expert parallelism, and memory", section "Shared
// experts").  A pair dropped by an expert capacity (slot_row -1) adds
// nothing.  A gather per token, no atomics, so the result is deterministic.
// When the down GEMM split K (into 2 to 4 ranges), each expert output row is
// the sum of its partial rows, added here in range order.
// HBM-bound: it reads (k + n_shared) float32 rows (per K range) and writes one
// row per token, with 16-byte accesses.
#include "device.h"
#include "kernels.h"

namespace moe {

// Workgroup (t, q) handles columns [1024 q, 1024 q + 1024) of token t, one
// float4 per thread.  The rows of a token are loaded in batches of
// kCombineBatch (all loads of a batch issued before the first add), so a
// token costs about ceil((k + n_shared) / kCombineBatch) memory round trips
// rather than one per row; the adds keep the order above.
constexpr int kCombineBatch = 8;
template <bool Y_BF16, int NP>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ out,
                                                      int64_t part_stride,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ slot_row,
                                                      const int32_t* __restrict__ offsets, int d,
                                                      int k, int E, int n_sh, void* y) {
  const int t = blockIdx.x;
  __shared__ int rows[kMaxTopK + kMaxShared];
  __shared__ float wts[kMaxTopK];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = slot_row[(int64_t)t * k + threadIdx.x];
    wts[threadIdx.x] = w[(int64_t)t * k + threadIdx.x];
  } else if (threadIdx.x < k + n_sh) {
    rows[threadIdx.x] = offsets[E + threadIdx.x - k] + t;
  }
  __syncthreads();
  const int c = blockIdx.y * blockDim.x + threadIdx.x;
  if (c >= (d >> 2)) return;
  // expert output row r: its NP partial K-range sums, added in order
  auto row4 = [&](int r) {
    float4 v[NP];
#pragma unroll
    for (int q = 0; q < NP; ++q)
      v[q] = ((const float4*)(out + q * part_stride + (int64_t)r * d))[c];
#pragma unroll
    for (int q = 1; q < NP; ++q) {
      v[0].x += v[q].x;
      v[0].y += v[q].y;
      v[0].z += v[q].z;
      v[0].w += v[q].w;
    }
    return v[0];
  };
  const int n = k + n_sh;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < n; j0 += kCombineBatch) {
    float4 v[kCombineBatch];
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const int j = j0 + i;
      const int r = j < n ? rows[j] : -1;  // -1: past the end, or dropped by a capacity
      v[i] = r >= 0 ? row4(r) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < kCombineBatch; ++i) {
      const int j = j0 + i;
      if (j >= n) break;
      if (j < k) {
        if (rows[j] < 0) continue;  // pair dropped by an expert capacity
        const float wj = wts[j];
        acc.x = fmaf(wj, v[i].x, acc.x);
        acc.y = fmaf(wj, v[i].y, acc.y);
        acc.z = fmaf(wj, v[i].z, acc.z);
        acc.w = fmaf(wj, v[i].w, acc.w);
      } else {  // shared experts, weight one
        acc.x += v[i].x;
        acc.y += v[i].y;
        acc.z += v[i].z;
        acc.w += v[i].w;
      }
    }
  }
  if (Y_BF16) {
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
    pk.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
    ((uint2*)((uint16_t*)y + (int64_t)t * d))[c] = pk;
  } else {
    ((float4*)((float*)y + (int64_t)t * d))[c] = acc;
  }
}

hipError_t launch_combine(const Plan& P, const float* out, int nparts, int64_t part_stride,
                          const float* w, const int32_t* slot_row, const int32_t* offsets,
                          void* y, hipStream_t s) {
  const moe_desc& D = P.desc;
  const dim3 grid((unsigned)D.T, (unsigned)((D.d / 4 + 255) / 256)), block(256);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, out, part_stride, w, slot_row, offsets, D.d, D.k,
                       D.E, D.n_shared, y);
  };
  const bool bf = D.y_dtype == MOE_BF16;
  switch (nparts) {
    case 1: bf ? go(combine_kernel<true, 1>) : go(combine_kernel<false, 1>); break;
    case 2: bf ? go(combine_kernel<true, 2>) : go(combine_kernel<false, 2>); break;
    case 3: bf ? go(combine_kernel<true, 3>) : go(combine_kernel<false, 3>); break;
    case 4: bf ? go(combine_kernel<true, 4>) : go(combine_kernel<false, 4>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
