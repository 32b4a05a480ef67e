// Grouped expert FFNs: for every group (routed expert or shared expert) the
// rows grouped for it by dispatch go through
//   up/gate:  h = SiLU(X W_gate^T) * (X W_up^T)      (X gathered by token)
//   down:     out = h W_down^T                        (float32)
// Pages: "Mixture of Experts: why a model with 671 billion parameters uses
// only 37" (an expert computes only the tokens assigned to it; experts are
// two linear layers with an activation; stacked per-projection expert
// tensors), "Mixture of Experts Explained: Routers, Active Parameters and
// VRAM" (gated three-matrix feed-forward block).
//
// bf16 kernel: one workgroup (4 waves) computes a tile of BN output columns
// by BM grouped rows with 32x32x16 bf16 MFMAs and fp32 accumulation.  The
// MFMA "A" operand is the weight tile (rows = output features) and "B" is the
// token tile, so each lane ends with 4 consecutive output features of one
// token, which it stores as one 8-byte (bf16 h) or 16-byte (fp32 out) write.
// Both operands are K-contiguous in memory and staged through LDS in 64-wide
// K slabs, double-buffered, with the 16-byte chunks of a row XOR-swizzled by
// (row/2)%8 so that the 16 lanes of each ds_read_b128 phase hit distinct banks.
// The up/gate tile holds the up and the gate rows of the same features, so
// SwiGLU is applied in registers before h is written.
//
// Workgroups walk a device-side tile list written by dispatch (no host
// readback).  Consecutive list entries share weight and token tiles; the
// workgroup index is remapped so that consecutive entries run on the same
// XCD (dispatch places workgroup i on XCD i % 8).
#include "device.h"
#include "kernels.h"

namespace moe {

struct GemmArgs {
  const uint16_t* tok;        // x [T, K] (gather) or h [rows, ldt] (direct)
  const int32_t* sorted;      // row -> token for the gather; null for direct rows
  int ldt;                    // row stride of tok, elements
  const uint16_t* w0;         // routed: up (or down) [E, N, K]
  const uint16_t* w1;         // routed: gate [E, N, K] (up/gate only)
  const uint16_t* s0;         // shared counterparts
  const uint16_t* s1;
  int E, N_r, N_s, K_r, K_s;  // routed / shared output columns and reduction length
  void* out;                  // h (bf16, up/gate) or out (fp32, down)
  int ldo;                    // row stride of out, elements
  const Tile* tiles;
};

constexpr int BK = 64;  // K slab (8 chunks of 8 bf16 per row)

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// Remap the workgroup index so consecutive tile-list entries share an XCD.
__device__ __forceinline__ int tile_of_block(const Tile* tiles) {
  const int count = tiles[0].g;
  const int per = (count + 7) >> 3;
  const int bid = blockIdx.x;
  if (bid >= per * 8) return -1;
  const int L = (bid & 7) * per + (bid >> 3);
  return L < count ? L : -1;
}

template <int BM, int BN, int WM, int WN, bool UPGATE>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WROWS = UPGATE ? 2 * BN : BN;        // weight rows in the tile
  constexpr int NWN = BN / WN, NWM = BM / WM;
  static_assert(NWN * NWM == 4, "4 waves");
  constexpr int TN = WN / 32, TM = WM / 32;           // 32x32 sub-tiles per wave
  constexpr int NS = UPGATE ? 2 : 1;                  // up and gate, or down
  constexpr int WCH = WROWS * 8 / 256;                // 16-byte chunks per thread
  constexpr int XCH = BM * 8 / 256;
  static_assert(WCH >= 1 && XCH >= 1, "tile too small");

  const int L = tile_of_block(a.tiles);
  if (L < 0) return;
  const Tile tl = a.tiles[1 + L];
  const bool sh = tl.g >= a.E;
  const int N = sh ? a.N_s : a.N_r;
  const int K = sh ? a.K_s : a.K_r;
  if (tl.n0 >= N) return;
  const int64_t wstride = (int64_t)N * K;
  const uint16_t* W0 = sh ? a.s0 + (tl.g - a.E) * wstride : a.w0 + tl.g * wstride;
  const uint16_t* W1 = UPGATE ? (sh ? a.s1 + (tl.g - a.E) * wstride : a.w1 + tl.g * wstride)
                              : nullptr;

  __shared__ __attribute__((aligned(16))) uint16_t lw[2][WROWS * BK];
  __shared__ __attribute__((aligned(16))) uint16_t lx[2][BM * BK];

  const int tid = threadIdx.x;
  // global source of each of this thread's chunks (row pointer + chunk)
  const uint16_t* wsrc[WCH];
  int wdst[WCH];
#pragma unroll
  for (int i = 0; i < WCH; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, ch = c & 7;
    int n, half;
    if (UPGATE) {
      half = r >= BN;
      n = tl.n0 + (half ? r - BN : r);
    } else {
      half = 0;
      n = tl.n0 + r;
    }
    n = n < N ? n : N - 1;
    wsrc[i] = (UPGATE && half ? W1 : W0) + (int64_t)n * K + ch * 8;
    wdst[i] = swz(r, ch);
  }
  const uint16_t* xsrc[XCH];
  int xdst[XCH];
#pragma unroll
  for (int i = 0; i < XCH; ++i) {
    const int c = tid + 256 * i;
    const int r = c >> 3, ch = c & 7;
    int row = tl.m0 + r;
    row = row < tl.m_end ? row : tl.m_end - 1;
    const int64_t src_row = a.sorted ? (int64_t)a.sorted[row] : (int64_t)row;
    xsrc[i] = a.tok + src_row * a.ldt + ch * 8;
    xdst[i] = swz(r, ch);
  }

  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % NWN, wm = wave / NWN;
  f32x16 acc[NS][TN][TM];
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[s][i][j][r] = 0.f;

  u32x4 rw[WCH], rx[XCH];
  auto gload = [&](int kt) {
    const int ko = kt * BK;
#pragma unroll
    for (int i = 0; i < WCH; ++i) rw[i] = *(const u32x4*)(wsrc[i] + ko);
#pragma unroll
    for (int i = 0; i < XCH; ++i) rx[i] = *(const u32x4*)(xsrc[i] + ko);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < WCH; ++i) *(u32x4*)(&lw[buf][wdst[i]]) = rw[i];
#pragma unroll
    for (int i = 0; i < XCH; ++i) *(u32x4*)(&lx[buf][xdst[i]]) = rx[i];
  };

  const int nk = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int ch = kk * 2 + (lane >> 5);
      u32x4 fx[TM];
#pragma unroll
      for (int j = 0; j < TM; ++j)
        fx[j] = *(const u32x4*)(&lx[buf][swz(wm * WM + j * 32 + (lane & 31), ch)]);
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          const u32x4 fw =
              *(const u32x4*)(&lw[buf][swz(s * BN + wn * WN + i * 32 + (lane & 31), ch)]);
#pragma unroll
          for (int j = 0; j < TM; ++j) acc[s][i][j] = mfma32(fw, fx[j], acc[s][i][j]);
        }
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // D[n = feature][m = row]: lane holds row (lane & 31) and, for q = 0..3,
  // features 8q + 4*(lane>>5) + 0..3 of each 32x32 sub-tile.
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int row = tl.m0 + wm * WM + j * 32 + (lane & 31);
    if (row >= tl.m_end) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = tl.n0 + wn * WN + i * 32 + 8 * q + 4 * (lane >> 5);
        if (n >= N) continue;
        if (UPGATE) {
          uint16_t hv[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            hv[r] = f32_to_bf16(silu_mul(acc[1][i][j][4 * q + r], acc[0][i][j][4 * q + r]));
          uint2 pk;
          pk.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
          pk.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
          *(uint2*)((uint16_t*)a.out + (int64_t)row * a.ldo + n) = pk;
        } else {
          float4 v;
          v.x = acc[0][i][j][4 * q + 0];
          v.y = acc[0][i][j][4 * q + 1];
          v.z = acc[0][i][j][4 * q + 2];
          v.w = acc[0][i][j][4 * q + 3];
          *(float4*)((float*)a.out + (int64_t)row * a.ldo + n) = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- float32
// Plain VALU tiles (32 rows x 32 features, K slabs of 16, the last one
// zero-padded) in float32.
struct GemmArgsF32 {
  const float* tok;
  const int32_t* sorted;
  int ldt;
  const float *w0, *w1, *s0, *s1;
  int E, N_r, N_s, K_r, K_s;
  float* out;
  int ldo;
  const Tile* tiles;
};

template <bool UPGATE>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgsF32 a) {
  constexpr int BM = 32, BN = 32, BKF = 16;
  constexpr int WROWS = UPGATE ? 2 * BN : BN;
  const int L = tile_of_block(a.tiles);
  if (L < 0) return;
  const Tile tl = a.tiles[1 + L];
  const bool sh = tl.g >= a.E;
  const int N = sh ? a.N_s : a.N_r;
  const int K = sh ? a.K_s : a.K_r;
  if (tl.n0 >= N) return;
  const int64_t wstride = (int64_t)N * K;
  const float* W0 = sh ? a.s0 + (tl.g - a.E) * wstride : a.w0 + tl.g * wstride;
  const float* W1 = UPGATE ? (sh ? a.s1 + (tl.g - a.E) * wstride : a.w1 + tl.g * wstride) : nullptr;

  __shared__ float lw[WROWS][BKF + 1];
  __shared__ float lx[BM][BKF + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;  // features 2tx..2tx+1, rows 2ty..2ty+1
  float acc[2][2][2] = {};
  for (int k0 = 0; k0 < K; k0 += BKF) {
    for (int c = tid; c < WROWS * BKF; c += 256) {
      const int r = c / BKF, kk = c % BKF;
      const int half = UPGATE && r >= BN;
      int n = tl.n0 + (half ? r - BN : r);
      n = n < N ? n : N - 1;
      lw[r][kk] = k0 + kk < K ? (half ? W1 : W0)[(int64_t)n * K + k0 + kk] : 0.f;
    }
    for (int c = tid; c < BM * BKF; c += 256) {
      const int r = c / BKF, kk = c % BKF;
      int row = tl.m0 + r;
      row = row < tl.m_end ? row : tl.m_end - 1;
      const int64_t src = a.sorted ? (int64_t)a.sorted[row] : (int64_t)row;
      lx[r][kk] = k0 + kk < K ? a.tok[src * a.ldt + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; ++kk) {
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const float xv = lx[2 * ty + mi][kk];
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          acc[0][mi][ni] = fmaf(xv, lw[2 * tx + ni][kk], acc[0][mi][ni]);
          if (UPGATE) acc[1][mi][ni] = fmaf(xv, lw[BN + 2 * tx + ni][kk], acc[1][mi][ni]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int row = tl.m0 + 2 * ty + mi;
    if (row >= tl.m_end) continue;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int n = tl.n0 + 2 * tx + ni;
      if (n >= N) continue;
      const float v = UPGATE ? silu_mul(acc[1][mi][ni], acc[0][mi][ni]) : acc[0][mi][ni];
      a.out[(int64_t)row * a.ldo + n] = v;
    }
  }
}

// ---------------------------------------------------------------- launch
static GemmArgs up_args(const Plan& P, const ExpertArgs& x) {
  const moe_desc& D = P.desc;
  const int ffn_s = D.n_shared ? D.ffn_shared : D.ffn;
  return GemmArgs{(const uint16_t*)x.x, x.sorted_token, D.d, (const uint16_t*)x.w_up,
                  (const uint16_t*)x.w_gate, (const uint16_t*)x.ws_up,
                  (const uint16_t*)x.ws_gate, D.E, D.ffn, ffn_s, D.d, D.d, x.h, P.ffn_max,
                  x.tiles_up};
}
static GemmArgs down_args(const Plan& P, const ExpertArgs& x) {
  const moe_desc& D = P.desc;
  const int ffn_s = D.n_shared ? D.ffn_shared : D.ffn;
  return GemmArgs{(const uint16_t*)x.h, nullptr, P.ffn_max, (const uint16_t*)x.w_down, nullptr,
                  (const uint16_t*)x.ws_down, nullptr, D.E, D.d, D.d, D.ffn, ffn_s, x.out, D.d,
                  x.tiles_down};
}

hipError_t launch_expert_up(const Plan& P, const ExpertArgs& x, hipStream_t s) {
  const moe_desc& D = P.desc;
  const dim3 block(256);
  const dim3 grid((unsigned)(((P.up.max_tiles + 7) / 8) * 8));
  if (P.kind == KIND_F32) {
    const int ffn_s = D.n_shared ? D.ffn_shared : D.ffn;
    GemmArgsF32 u{(const float*)x.x, x.sorted_token, D.d, (const float*)x.w_up,
                  (const float*)x.w_gate, (const float*)x.ws_up, (const float*)x.ws_gate,
                  D.E, D.ffn, ffn_s, D.d, D.d, (float*)x.h, P.ffn_max, x.tiles_up};
    hipLaunchKernelGGL(gemm_f32_kernel<true>, grid, block, 0, s, u);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<128, 64, 64, 32, true>), grid, block, 0, s,
                     up_args(P, x));
  return hipGetLastError();
}

hipError_t launch_expert_down(const Plan& P, const ExpertArgs& x, hipStream_t s) {
  const moe_desc& D = P.desc;
  const dim3 block(256);
  const dim3 grid((unsigned)(((P.down.max_tiles + 7) / 8) * 8));
  if (P.kind == KIND_F32) {
    const int ffn_s = D.n_shared ? D.ffn_shared : D.ffn;
    GemmArgsF32 dn{(const float*)x.h, nullptr, P.ffn_max, (const float*)x.w_down, nullptr,
                   (const float*)x.ws_down, nullptr, D.E, D.d, D.d, D.ffn, ffn_s, x.out, D.d,
                   x.tiles_down};
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, block, 0, s, dn);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 64, 64, false>), grid, block, 0, s,
                     down_args(P, x));
  return hipGetLastError();
}

}  // namespace moe
