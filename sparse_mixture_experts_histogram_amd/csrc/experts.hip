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
// Kernel families (the plan picks one per layer):
// - gemm_bf16_kernel (prefill): one workgroup (4 waves) computes a tile of
//   BN output columns by BM = 64, 128 or 256 grouped rows with 32x32x16 bf16
//   MFMAs and fp32 accumulation.  The MFMA "A" operand is the weight tile
//   (rows = output features) and "B" the token tile.  Both operands are
//   K-contiguous in memory and staged through LDS in 64-wide K slabs (one
//   128-byte line per tile row), copied by buffer_load_dwordx4 ... lds in
//   1 KB bursts of 8 whole rows into separate weight and token rings, with
//   the 16-byte chunks of a row XOR-swizzled so that the lanes of each
//   ds_read_b128 phase hit distinct banks.  Fragments of the next k-step are
//   read from LDS while the current MFMAs run.  When every wave spans all
//   rows of the tile, the tile runs the compiled form for its count of live
//   32-row groups.  A down GEMM with a long reduction splits its last,
//   partly filled round of tiles along K (gemm_fixup_kernel adds the pieces).
// - gemm_bf16_stream_kernel (decode): 16 x 16 tiles streaming the touched
//   experts' weights, the four waves splitting K.
// - gemm_mx_stream_kernel / gemm_mx_lds_kernel: MXFP4 and MXFP8 expert
//   weights widened to bf16 in registers.
// - gemm_f32_kernel: the float32 layer.
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
  int xcd_remap;              // 1: consecutive schedule entries run on one XCD
  int ksplit;                 // K ranges per tile (partial sums to separate outputs)
  int64_t split_stride;       // elements between the outputs of consecutive K ranges
  uint32_t tok_bytes;         // bytes of tok (the buffer range of its DMA)
  // MX-format experts: w0/w1/s0/s1 hold E2M1 codes [., N, K/2] (MXFP4) or
  // E4M3 codes [., N, K] (MXFP8) and these their E8M0 scales [., N, K/32]
  const uint8_t *sw0, *sw1, *ss0, *ss1;
  // Last-round split (prefill kernels): with sk_cus > 0 the tiles of a last,
  // partly filled round of sk_cus workgroups are cut along K into pieces
  // whose float32 accumulators go to `part` and are added by the fixup
  // kernel (see sk_layout).
  float* part;
  int sk_cus;
  int mx_line;  // MX code rows padded to whole 128-byte lines (MOE_FLAG_MX_LINE_ROWS)
};

// Schedule of the last-round split.  `count` tiles on C workgroup slots run
// count / C whole rounds and r = count % C tiles in a last round that leaves
// C - r slots idle.  Those r tiles are cut into s = C / r pieces along K (at
// least kSkMinSlabs slabs each), so the last round runs r * s pieces of
// about 1 / s of a tile.  Entries [0, dp) are whole tiles; entry dp + t * s +
// j is piece j of tile dp + t.  No split (r = 0, s = 1) when the last round
// is full or a piece would be too short.
constexpr int kSkMinSlabs = 8;
struct SkLayout {
  int dp, r, s;
};
__device__ __forceinline__ SkLayout sk_layout(int count, int C, int nk) {
  SkLayout L{count, 0, 1};
  if (C <= 0) return L;
  const int r = count % C;
  if (r == 0) return L;
  const int s = min(C / r, nk / kSkMinSlabs);
  if (s < 2) return L;
  return SkLayout{count - r, r, s};
}

constexpr int BK = 64;  // K slab: 8 chunks of 8 bf16 per tile row (one 128-byte line)

// LDS element offset of 16-byte chunk `chunk` of tile row `row` (rows of 128
// bytes).  A ds_read_b128 phase serves 16 lanes that read one chunk of 16
// consecutive rows; XOR-ing the chunk with (row / 2) % 8 spreads them over
// all 64 banks.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

// A tile entry read by every lane, made wave-uniform (scalar registers).
__device__ __forceinline__ Tile uniform_tile(const Tile& t) {
  return Tile{__builtin_amdgcn_readfirstlane(t.g), __builtin_amdgcn_readfirstlane(t.m0),
              __builtin_amdgcn_readfirstlane(t.m_end), __builtin_amdgcn_readfirstlane(t.n0)};
}

// Schedule entry of this workgroup.  With `remap`, consecutive entries run on
// one XCD (the dispatcher deals workgroup i to XCD i % 8), so the workgroups
// that share weight and token tiles share that XCD's L2; without it, entries
// are spread over all XCDs.
__device__ __forceinline__ int entry_of_block(int count, int remap) {
  const int bid = blockIdx.x;
  if (!remap) return bid < count ? bid : -1;
  const int per = (count + 7) >> 3;
  if (bid >= per * 8) return -1;
  const int L = (bid & 7) * per + (bid >> 3);
  return L < count ? L : -1;
}

__device__ __forceinline__ int tile_of_block(const Tile* tiles, int remap = 1) {
  return entry_of_block(tiles[0].g, remap);
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// s_waitcnt immediate that waits for at most `n` outstanding vector-memory
// operations and nothing else (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkm0 = ~(15 << 8);  // AND into an immediate to also wait lgkmcnt(0)

// One stage of a tile operand: 1 KB blocks of 8 rows, block b = wave + NW i.
// global_load_lds_dwordx4 fills bytes [16 l, 16 l + 16) of a block from lane
// l, so lane l fetches row 8 b + l / 8 at the chunk whose swizzled slot is
// l % 8: the 8 lanes of a row read its whole 128-byte line.
// The copies are buffer loads: the operand's base and size sit in a
// descriptor in scalar registers, each lane adds a 32-bit byte offset (its
// row and chunk), and the slab's K offset is the scalar offset, so no
// per-copy address arithmetic or 64-bit address registers are needed.
template <int NBLK, int NW, int AUX = 0>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rsrc, uint32_t soff,
                                         const uint32_t* off, uint16_t* lds, int wave) {
#pragma unroll
  for (int i = 0; i < NBLK; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(lds + (wave + NW * i) * 512), 16,
                                             off[i], soff, 0, AUX);
}

// dma_tile where block i reads through `dead` (a size-0 descriptor: zeros, no
// memory traffic) unless bit i of `live` is set.
template <int NBLK, int NW, int AUX = 0>
__device__ __forceinline__ void dma_tile_live(__amdgpu_buffer_rsrc_t rsrc,
                                              __amdgpu_buffer_rsrc_t dead, uint32_t live,
                                              uint32_t soff, const uint32_t* off, uint16_t* lds,
                                              int wave) {
#pragma unroll
  for (int i = 0; i < NBLK; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(((live >> i) & 1u) ? rsrc : dead,
                                             LDS_PTR(lds + (wave + NW * i) * 512), 16, off[i],
                                             soff, 0, AUX);
}

// Buffer descriptor of `bytes` bytes at p (raw buffer: no stride, no format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Float32 accumulators of one wave in register order: accumulator c of the
// wave at ((wave * NACC + c) * 64 + lane) * 16 floats (16-byte accesses,
// consecutive lanes contiguous).
template <int NS, int TN, int TM>
__device__ __forceinline__ void store_partial(f32x16 (&acc)[NS][TN][TM], float* dst, int wave,
                                              int lane) {
  constexpr int NACC = NS * TN * TM;
#pragma unroll
  for (int s = 0; s < NS; ++s)
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        float4* d = (float4*)(dst + ((wave * NACC + (s * TN + i) * TM + j) * 64 + lane) * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          d[q] = make_float4(acc[s][i][j][4 * q], acc[s][i][j][4 * q + 1], acc[s][i][j][4 * q + 2],
                             acc[s][i][j][4 * q + 3]);
      }
}
// D[n = feature][m = row]: lane holds row (lane & 31) and, for q = 0..3,
// features 8q + 4*(lane>>5) + 0..3 of each 32x32 sub-tile.  Outputs are
// written through LDS so that every store is a 16-byte piece of a whole
// row: a wave stages 32 rows x WN features at a time in a stage buffer of
// its own (row pitch padded by 16 bytes against bank conflicts), then stores
// them as 16-byte pieces, consecutive lanes along a row.
// store_rows32 writes one such 32-row group starting at row0 (rows at or
// past m_end and columns at or past N are not written); get(s, i, r) is
// element r of the accumulator of operand s (up/gate: 0 up, 1 gate) and
// 32-column sub-tile i.
template <int WN, int TN, bool UPGATE, class Get>
__device__ __forceinline__ void store_rows32(Get get, int row0, int col0, int m_end, int N,
                                             const GemmArgs& a, int split, char* st, int lane) {
  constexpr int ES = UPGATE ? 2 : 4;                  // output element bytes
  constexpr int RB = WN * ES, PITCH = RB + 16;        // staged row bytes, LDS pitch
  constexpr int LPR = RB / 16;                         // 16-byte pieces per staged row
  static_assert(RB % 16 == 0, "epilogue shape");
  char* outb = (char*)a.out + (int64_t)split * a.split_stride * ES;
#pragma unroll
  for (int i = 0; i < TN; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      char* dst = st + (lane & 31) * PITCH + (i * 32 + 8 * q + 4 * (lane >> 5)) * ES;
      if (UPGATE) {
        uint16_t hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          hv[r] = f32_to_bf16(silu_mul(get(1, i, 4 * q + r), get(0, i, 4 * q + r)));
        uint2 pk;
        pk.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16);
        pk.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
        *(uint2*)dst = pk;
      } else {
        *(float4*)dst = make_float4(get(0, i, 4 * q + 0), get(0, i, 4 * q + 1),
                                    get(0, i, 4 * q + 2), get(0, i, 4 * q + 3));
      }
    }
  }
#pragma unroll
  for (int id0 = 0; id0 < 32 * LPR; id0 += 64) {
    const int id = id0 + lane, r = id / LPR, cb = (id % LPR) * 16;
    if (id < 32 * LPR) {
      const u32x4 v = *(const u32x4*)(st + r * PITCH + cb);
      const int row = row0 + r, col = col0 + cb / ES;
      if (row < m_end && col < N) *(u32x4*)(outb + ((int64_t)row * a.ldo + col) * ES) = v;
    }
  }
}

// The wave's whole WM x WN tile, 32-row group by 32-row group (groups at or
// past the tile's last row are skipped).
template <int WM, int WN, int TN, int TM, bool UPGATE>
__device__ __forceinline__ void tile_epilogue(f32x16 (&acc)[UPGATE ? 2 : 1][TN][TM], const Tile& tl,
                                              int N, const GemmArgs& a, int split, char* st,
                                              int wm, int wn, int lane) {
  const int row0 = tl.m0 + wm * WM, col0 = tl.n0 + wn * WN;
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    if (row0 + 32 * j >= tl.m_end) break;  // row groups past the tile's last row
    store_rows32<WN, TN, UPGATE>([&](int s, int i, int r) { return acc[s][i][j][r]; },
                                 row0 + 32 * j, col0, tl.m_end, N, a, split, st, lane);
  }
}

constexpr int kPolX = 0;  // cache policy bits of the token bursts
// POLW: cache policy bits of the weight bursts (0, or non-temporal when each
// weight tile is read by a single row tile).
template <int BM, int BN, int WM, int WN, bool UPGATE, int NSW, int NSX, int POLW>
__global__ __launch_bounds__(64 * (BN / WN) * (BM / WM)) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WROWS = UPGATE ? 2 * BN : BN;        // weight rows in the tile
  constexpr int NWN = BN / WN, NWM = BM / WM;
  constexpr int NW = NWN * NWM;                       // waves
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int TN = WN / 32, TM = WM / 32;           // 32x32 sub-tiles per wave
  constexpr int NS = UPGATE ? 2 : 1;                  // up and gate, or down
  constexpr int WB = WROWS / (8 * NW);                // 1 KB blocks per wave and stage
  constexpr int XB = BM / (8 * NW);
  static_assert(WB >= 1 && XB >= 1 && (!UPGATE || WB % 2 == 0), "tile shape");
  static_assert(NSW >= 2 && NSW <= 4 && NSX >= 2 && NSX <= 3, "stages");

  // With a K split, entries [q*count, (q+1)*count) run K range q of every
  // tile and write their partial sums to output q.  With the last-round
  // split (never together with a K split) an entry past the whole tiles is
  // one K piece of a last-round tile, whose accumulators go to a.part.
  // The whole tiles take the first dpb workgroups (remapped per XCD); the
  // pieces take one workgroup each after them, in order, so consecutive
  // pieces land on different XCDs and are dispatched last.  (Remapping
  // them with the whole tiles gave some XCDs only whole tiles.)
  const int count = a.tiles[0].g;
  const SkLayout sk = sk_layout(count, a.sk_cus, min(a.K_r, a.K_s) / BK);
  const int dpb = ((sk.dp * a.ksplit + 7) >> 3) << 3;
  int split, nsplit, L, piece = -1;
  if ((int)blockIdx.x >= dpb) {
    piece = blockIdx.x - dpb;
    if (piece >= sk.r * sk.s) return;
    L = sk.dp + piece / sk.s;
    split = piece % sk.s;
    nsplit = sk.s;
  } else {
    const int idx = entry_of_block(sk.dp * a.ksplit, a.xcd_remap);
    if (idx < 0) return;
    split = idx / count;
    L = idx - split * count;
    nsplit = a.ksplit;
  }
  const Tile tl = uniform_tile(a.tiles[1 + L]);
  const bool sh = tl.g >= a.E;
  const int N = sh ? a.N_s : a.N_r;
  const int K = sh ? a.K_s : a.K_r;
  if (tl.n0 >= N) return;
  const int64_t wstride = (int64_t)N * K;
  const uint16_t* W0 = sh ? a.s0 + (tl.g - a.E) * wstride : a.w0 + tl.g * wstride;
  const uint16_t* W1 = UPGATE ? (sh ? a.s1 + (tl.g - a.E) * wstride : a.w1 + tl.g * wstride)
                              : nullptr;

  // NSW weight and NSX token stage buffers, as separate arrays so the
  // compiler can tell reads of one buffer from DMA still landing in another
  // (with one array per operand it waits for every copy before each read).
  // Stages past NSW / NSX point at a used buffer, chosen at compile time, so
  // their arrays are never referenced and take no LDS.
  constexpr int SW = WROWS * BK, SX = BM * BK;
  __shared__ __attribute__((aligned(1024))) uint16_t lw0[SW], lw1[SW];
  __shared__ __attribute__((aligned(1024))) uint16_t lw2_[NSW > 2 ? SW : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lw3_[NSW > 3 ? SW : 8];
  __shared__ __attribute__((aligned(1024))) uint16_t lx0[SX], lx1[SX];
  __shared__ __attribute__((aligned(1024))) uint16_t lx2_[NSX > 2 ? SX : 8];
  uint16_t* const lw2 = NSW > 2 ? lw2_ : lw0;
  uint16_t* const lw3 = NSW > 3 ? lw3_ : lw0;
  uint16_t* const lx2 = NSX > 2 ? lx2_ : lx0;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Source byte offsets: block b = wave + NW i holds tile rows 8 b .. 8 b + 7;
  // lane l reads row 8 b + l / 8 at chunk (l % 8) ^ ((row / 2) % 8), where
  // (row / 2) % 8 = 4 (wave % 2) + (l / 16) does not depend on i.  The gate
  // rows of an up/gate tile sit BN rows below the up rows of the same
  // features, so both halves share the offsets.
  const int rr = lane >> 3;
  const int gch = (lane & 7) ^ (((wave & 1) << 2) + (lane >> 4));
  constexpr int WOFF = UPGATE ? WB / 2 : WB;
  uint32_t woff[WOFF];
#pragma unroll
  for (int i = 0; i < WOFF; ++i) {
    int n = tl.n0 + 8 * (wave + NW * i) + rr;
    n = n < N ? n : N - 1;
    woff[i] = ((uint32_t)n * (uint32_t)K + gch * 8) * 2;
  }
  uint32_t xoff[XB];
#pragma unroll
  for (int i = 0; i < XB; ++i) {
    int row = tl.m0 + 8 * (wave + NW * i) + rr;
    row = row < tl.m_end ? row : tl.m_end - 1;
    const uint32_t src_row = a.sorted ? (uint32_t)a.sorted[row] : (uint32_t)row;
    xoff[i] = (src_row * (uint32_t)a.ldt + gch * 8) * 2;
  }
  const int nk_all = K / BK;
  const int kb = split * nk_all / nsplit;  // first slab of this K range
  const uint32_t wbytes = (uint32_t)(wstride * 2);
  const __amdgpu_buffer_rsrc_t rw0 = buffer_of(W0, wbytes);
  const __amdgpu_buffer_rsrc_t rw1 = buffer_of(UPGATE ? W1 : W0, wbytes);
  const __amdgpu_buffer_rsrc_t rx = buffer_of(a.tok, a.tok_bytes);
  // Ring turns and leading zero slabs.  A turn is lcm(NSW, NSX) slabs.  The
  // 3 + 3 ring prepends zero slabs up to a whole number of turns: their
  // copies go through a descriptor of size 0, which reads as zeros, so they
  // add nothing.  (A separate code path for a partial turn made the compiler
  // add a full drain at the top of its loop.)  The other rings run the
  // slabs left over after whole turns as straight-line code.
  constexpr int P = NSW == NSX ? NSW : NSW % NSX == 0 ? NSW : NSW * NSX;  // lcm for 2..4
  static_assert(P == 2 || P == 3 || P == 4 || P == 6, "ring turn");
  constexpr bool kPadTurns = NSW == 3 && NSX == 3;
  const int nk = (split + 1) * nk_all / nsplit - kb;  // slabs of this K range
  const int pad = kPadTurns ? (P - nk % P) % P : 0;
  const __amdgpu_buffer_rsrc_t rzero = buffer_of(W0, 0);
  auto dma_w = [&](int kt_local, uint16_t* lw) {
    const int s = kt_local - pad;
    const uint32_t koff = s < 0 ? 0u : (uint32_t)(kb + s) * (BK * 2);
    dma_tile<WOFF, NW, POLW>(s < 0 ? rzero : rw0, koff, woff, lw, wave);
    if (UPGATE) dma_tile<WOFF, NW, POLW>(s < 0 ? rzero : rw1, koff, woff, lw + BN * BK, wave);
  };
  // Token copy blocks whose 8 rows all lie past the tile's last row (a
  // group's short last tile) read through the size-0 descriptor: zeros, no
  // memory traffic, and the same instruction count, so every vmcnt wait
  // below still counts the same copies.  The rows they fill are never stored.
  uint32_t xlive = 0;
#pragma unroll
  for (int i = 0; i < XB; ++i)
    if (tl.m0 + 8 * (wave + NW * i) < tl.m_end) xlive |= 1u << i;
  // Token copies of the first XBL blocks per wave (XBL < XB: the blocks of
  // 32-row groups past the tile's last row are not copied at all).
  auto dma_x = [&](auto xblc, int kt_local, uint16_t* lx) {
    constexpr int XBL = decltype(xblc)::value;
    const int s = kt_local - pad;
    const uint32_t koff = s < 0 ? 0u : (uint32_t)(kb + s) * (BK * 2);
    dma_tile_live<XBL, NW, kPolX>(s < 0 ? rzero : rx, rzero, xlive, koff, xoff, lx, wave);
  };

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

  // The main loop for LB live 32-row groups of the wave tile: MFMAs,
  // fragment reads and token copies of the groups past the tile's last row
  // are left out (their accumulators stay zero and are never stored).  When
  // every wave spans all BM rows (WM == BM) all waves share one LB, chosen
  // per tile below among TM compiled forms, so no branch enters the
  // scheduled slab code; otherwise LB = TM.
  auto main_loop = [&](auto lbc) {
  constexpr int LB = decltype(lbc)::value;
  static_assert(LB >= 1 && LB <= TM, "live row groups");
  constexpr int XBL = XB * LB / TM;                 // token copy blocks per wave
  static_assert(LB == TM || XB == TM, "token blocks follow the 32-row groups");
  constexpr int NDL = WB + XBL;                     // DMA instructions per wave and stage

  // Fragment read offsets (elements) of k-step 0 of a slab: lane l reads row
  // (l % 32) of sub-tile 0 at chunk l / 32; the other sub-tiles are whole
  // 32-row blocks further.  Chunk 2 kk + c of a row sits at the slot of chunk
  // c XOR 2 kk, so k-step kk is k-step 0's offset XOR 16 kk.
  const int fxo = swz(wm * WM + (lane & 31), lane >> 5);
  const int fwo = swz(wn * WN + (lane & 31), lane >> 5);
  u32x4 fxA[TM], fwA[NS][TN], fxB[TM], fwB[NS][TN];  // fragments of even / odd k-steps
  auto fload = [&](const uint16_t* lw, const uint16_t* lx, int kk, u32x4* fx, u32x4 (*fw)[TN]) {
    const int ox = fxo ^ (kk << 4), ow = fwo ^ (kk << 4);
#pragma unroll
    for (int j = 0; j < LB; ++j) fx[j] = *(const u32x4*)(&lx[ox + j * 32 * BK]);
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < TN; ++i)
        fw[s][i] = *(const u32x4*)(&lw[ow + (s * BN + i * 32) * BK]);
  };
  auto mfmas = [&](const u32x4* fx, u32x4 (*fw)[TN]) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < LB; ++j) acc[s][i][j] = mfma32(fw[s][i], fx[j], acc[s][i][j]);
  };
  constexpr int NF = LB + NS * TN;   // fragment reads per k-step
  constexpr int NMF = NS * TN * LB;  // MFMAs per k-step
  // DMAs issued during k-steps 0, 1 and 2 of a slab: over kSpread k-steps
  // (at most three), about one per MFMA of a k-step where they fit
  constexpr int kSpreadRaw = (NDL + NMF - 1) / NMF;
  constexpr int kSpread = kSpreadRaw < 2 ? 2 : kSpreadRaw > 3 ? 3 : kSpreadRaw;
  constexpr int ND0 = (NDL + kSpread - 1) / kSpread;
  constexpr int ND1 = kSpread >= 2 ? (NDL - ND0 + kSpread - 2) / (kSpread - 1) : 0;
  constexpr int ND2 = NDL - ND0 - ND1;
  static_assert(LB < TM || (NMF >= NF && NMF >= ND0 && NMF >= ND1 && NMF >= ND2),
                "pipeline shape of a whole tile");
  // Issue order for one k-step: MFMAs one by one, each followed by its
  // share of the fragment reads and DMAs (with at least as many MFMAs as
  // either: one each after the first NF and nd MFMAs).
  auto pipeline = [&](int nd) {
#pragma unroll
    for (int r = 0; r < NMF; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int nr = NF / NMF + (r < NF % NMF ? 1 : 0);
#pragma unroll
      for (int q = 0; q < nr; ++q) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      const int ndr = nd / NMF + (r < nd % NMF ? 1 : 0);
#pragma unroll
      for (int q = 0; q < ndr; ++q) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Every slab issues the weight DMA of slab J + NSW - 1 and the token DMA
  // of slab J + NSX - 1 (clamped to the last slab: near the end it
  // re-fetches into a buffer nothing reads any more), the operand with the
  // shorter ring first.  Before reading slab J + 1 a wave waits until that
  // slab's copies have landed; the copies issued after the later of the two
  // may stay in flight.
  static_assert(NSX <= NSW, "the token ring is never the longer one");
  constexpr int NWI = (UPGATE ? 2 : 1) * WOFF;  // weight copies per slab
  // Copies issued after the last one slab J + 1 needs: with equal rings the
  // weights of J + 1 (issued in slab J + 2 - NSW, last in that slab), then
  // NSW - 2 whole slabs; with a longer weight ring the tokens of J + 1
  // (issued in slab J + 2 - NSX, before that slab's weight copies), then
  // NSX - 2 whole slabs.
  constexpr int WAIT = NSX == NSW ? (NSW - 2) * NDL : NWI + (NSX - 2) * NDL;
  static_assert(WAIT <= 63, "vmcnt range");
  auto dma = [&](int kt_w, uint16_t* lw, int kt_x, uint16_t* lx) {
    if constexpr (NSX < NSW) {
      dma_x(std::integral_constant<int, XBL>{}, kt_x, lx);
      dma_w(kt_w, lw);
    } else {
      dma_w(kt_w, lw);
      dma_x(std::integral_constant<int, XBL>{}, kt_x, lx);
    }
  };
  // Wait until this wave's copies of the next slab have landed (and every
  // fragment read is done), then for all waves.
  auto wait_next = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(WAIT) & kLgkm0);
    barrier();
  };

  const int m = nk + pad;  // slabs to run
  // Ring buffer i of each operand (i a constant, so the named array is used
  // directly and the compiler keeps telling the stages apart).
#define MOE_WB(i) ((i) == 0 ? lw0 : (i) == 1 ? lw1 : (i) == 2 ? lw2 : lw3)
#define MOE_XB(i) ((i) == 0 ? lx0 : (i) == 1 ? lx1 : lx2)
  if (m > 0) {
    // Copies of the slabs before 0, in the order a slab issues them: slab
    // q < 0 copies the tokens of q + NSX - 1 and the weights of q + NSW - 1
    // where those are >= 0.
    if constexpr (NSW == 4 && NSX == 2) {
      dma_w(0, lw0);
      dma_w(min(1, m - 1), lw1);
      dma(min(2, m - 1), lw2, 0, lx0);
    } else if constexpr (NSW == 3 && NSX == 2) {
      dma_w(0, lw0);
      dma(min(1, m - 1), lw1, 0, lx0);
    } else if constexpr (NSW == 3) {
      dma(0, lw0, 0, lx0);
      dma(min(1, m - 1), lw1, min(1, m - 1), lx1);
    } else {
      dma(0, lw0, 0, lx0);
    }
    wait_next();
    fload(lw0, lx0, 0, fxA, fwA);
    // One slab of four k-steps in ring position Q (weights in wr[Q % NSW],
    // tokens in xr[Q % NSX]): issue the copies ahead; each k-step's MFMAs run
    // while the next k-step's fragments are read; before the last k-step's
    // MFMAs, wait until the next slab has landed and read its first
    // fragments.  No branches inside, so each stretch between barriers is one
    // scheduling region; the final next-slab read of the layer is unused.
#define MOE_SLAB(J, Q)                                                    \
    {                                                                       \
      dma(min((J) + NSW - 1, m - 1), MOE_WB(((Q) + NSW - 1) % NSW),         \
          min((J) + NSX - 1, m - 1), MOE_XB(((Q) + NSX - 1) % NSX));        \
      fload(MOE_WB((Q) % NSW), MOE_XB((Q) % NSX), 1, fxB, fwB);             \
      mfmas(fxA, fwA);                                                      \
      pipeline(ND0);                                                        \
      fload(MOE_WB((Q) % NSW), MOE_XB((Q) % NSX), 2, fxA, fwA);             \
      mfmas(fxB, fwB);                                                      \
      pipeline(ND1);                                                        \
      fload(MOE_WB((Q) % NSW), MOE_XB((Q) % NSX), 3, fxB, fwB);             \
      mfmas(fxA, fwA);                                                      \
      pipeline(ND2);                                                        \
      wait_next();                                                          \
      fload(MOE_WB(((Q) + 1) % NSW), MOE_XB(((Q) + 1) % NSX), 0, fxA, fwA); \
      mfmas(fxB, fwB);                                                      \
      pipeline(0);                                                          \
    }
    // Whole turns of both rings, then the m % P slabs left over as the first
    // positions of one more turn.  Each remainder gets its own straight-line
    // copy: a shared tail with a branch after every slab made the compiler
    // spill the accumulators.  (Always whole turns with leading zero slabs.)
#define MOE_TURNS                                     \
    for (int j = 0; j < mt; j += P) {                   \
      MOE_SLAB(j, 0)                                    \
      MOE_SLAB(j + 1, 1)                                \
      if constexpr (P >= 3) MOE_SLAB(j + 2, 2)          \
      if constexpr (P == 4) MOE_SLAB(j + 3, 3)          \
      if constexpr (P == 6) {                           \
        MOE_SLAB(j + 3, 3)                              \
        MOE_SLAB(j + 4, 4)                              \
        MOE_SLAB(j + 5, 5)                              \
      }                                                 \
    }
    const int mr = kPadTurns ? 0 : m % P, mt = m - mr;
    switch (mr) {
      case 0:
        MOE_TURNS
        break;
      case 1:
        MOE_TURNS
        MOE_SLAB(mt, 0)
        break;
      case 2:
        if constexpr (P > 2) {
          MOE_TURNS
          MOE_SLAB(mt, 0)
          MOE_SLAB(mt + 1, 1)
        }
        break;
      case 3:
        if constexpr (P > 3) {
          MOE_TURNS
          MOE_SLAB(mt, 0)
          MOE_SLAB(mt + 1, 1)
          MOE_SLAB(mt + 2, 2)
        }
        break;
      case 4:
        if constexpr (P > 4) {
          MOE_TURNS
          MOE_SLAB(mt, 0)
          MOE_SLAB(mt + 1, 1)
          MOE_SLAB(mt + 2, 2)
          MOE_SLAB(mt + 3, 3)
        }
        break;
      default:
        if constexpr (P > 5) {
          MOE_TURNS
          MOE_SLAB(mt, 0)
          MOE_SLAB(mt + 1, 1)
          MOE_SLAB(mt + 2, 2)
          MOE_SLAB(mt + 3, 3)
          MOE_SLAB(mt + 4, 4)
        }
        break;
    }
#undef MOE_TURNS
#undef MOE_SLAB
#undef MOE_WB
#undef MOE_XB
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // drain the re-fetches
  }
  };  // main_loop
  if constexpr (WM == BM) {
    const int lb = (min(BM, tl.m_end - tl.m0) + 31) >> 5;
    if constexpr (TM == 4) {
      switch (lb) {
        case 1: main_loop(std::integral_constant<int, 1>{}); break;
        case 2: main_loop(std::integral_constant<int, 2>{}); break;
        case 3: main_loop(std::integral_constant<int, 3>{}); break;
        default: main_loop(std::integral_constant<int, 4>{}); break;
      }
    } else if constexpr (TM == 2) {
      if (lb == 1)
        main_loop(std::integral_constant<int, 1>{});
      else
        main_loop(std::integral_constant<int, 2>{});
    } else if constexpr (TM == 8) {
      switch (lb) {
        case 1: main_loop(std::integral_constant<int, 1>{}); break;
        case 2: main_loop(std::integral_constant<int, 2>{}); break;
        case 3: main_loop(std::integral_constant<int, 3>{}); break;
        case 4: main_loop(std::integral_constant<int, 4>{}); break;
        case 5: main_loop(std::integral_constant<int, 5>{}); break;
        case 6: main_loop(std::integral_constant<int, 6>{}); break;
        case 7: main_loop(std::integral_constant<int, 7>{}); break;
        default: main_loop(std::integral_constant<int, 8>{}); break;
      }
    } else {
      main_loop(std::integral_constant<int, TM>{});
    }
  } else {
    main_loop(std::integral_constant<int, TM>{});
  }

  if (piece >= 0) {  // a K piece of a last-round tile: accumulators to a.part
    store_partial<NS, TN, TM>(acc, a.part + (size_t)piece * (NW * NS * TN * TM * 1024), wave,
                              lane);
    return;
  }
  constexpr int PITCH = WN * (UPGATE ? 2 : 4) + 16;
  constexpr int STG = 32 * PITCH;  // staging bytes per wave
  static_assert(NW == 4, "epilogue shape");
  __syncthreads();  // every wave is done reading the stage buffers
  char* st;
  if constexpr (STG <= 2 * (SX < SW ? SX : SW)) {  // one stage buffer per wave
    st = (char*)(wave == 0 ? lw0 : wave == 1 ? lw1 : wave == 2 ? lx0 : lx1);
  } else {  // small token stages: two waves per weight stage
    static_assert(2 * STG <= 2 * SW, "staging fits the weight stages");
    st = (char*)(wave & 1 ? lw1 : lw0) + (wave >> 1) * STG;
  }
  tile_epilogue<WM, WN, TN, TM, UPGATE>(acc, tl, N, a, split, st, wm, wn, lane);
}

// Adds the K pieces of each last-round tile of a split GEMM launch (see
// sk_layout), in piece order, and writes the tile as the GEMM epilogue does
// (SwiGLU and bf16 h for up/gate, float32 for down).  The piece
// accumulators use the GEMM's register layout.  Workgroup b handles GEMM
// wave b % NW of split tile dp + b / NW; its wave j takes that GEMM wave's
// 32-row group j, so a tile is spread over NW * TM waves on several CUs (one
// workgroup per tile, walking its row groups in turn, left most CUs idle
// while the few last-round tiles were summed).
template <int BM, int BN, int WM, int WN, bool UPGATE>
__global__ __launch_bounds__(64 * (WM / 32)) void gemm_fixup_kernel(GemmArgs a) {
  constexpr int NWN = BN / WN, NWM = BM / WM, NW = NWN * NWM;
  constexpr int TN = WN / 32, TM = WM / 32, NS = UPGATE ? 2 : 1;
  constexpr int NACC = NS * TN * TM;
  constexpr int PITCH = WN * (UPGATE ? 2 : 4) + 16;
  constexpr size_t PIECE = (size_t)NW * NACC * 1024;  // floats per piece
  __shared__ __attribute__((aligned(16))) char stage[TM][32 * PITCH];
  const SkLayout sk = sk_layout(a.tiles[0].g, a.sk_cus, min(a.K_r, a.K_s) / BK);
  const int t = blockIdx.x / NW, gw = blockIdx.x % NW;  // tile, GEMM wave
  if (t >= sk.r) return;
  const Tile tl = uniform_tile(a.tiles[1 + sk.dp + t]);
  const int N = tl.g >= a.E ? a.N_s : a.N_r;
  if (tl.n0 >= N) return;  // the GEMM wrote no pieces for it either
  const int lane = threadIdx.x & 63, j = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = gw / NWN, wn = gw % NWN;
  const int row0 = tl.m0 + wm * WM + 32 * j;
  if (row0 >= tl.m_end) return;
  f32x16 acc[NS][TN];
  const float* base = a.part + (size_t)t * sk.s * PIECE;
  for (int p = 0; p < sk.s; ++p) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const float4* src = (const float4*)(base + p * PIECE +
                                            ((gw * NACC + (s * TN + i) * TM + j) * 64 + lane) * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 u = src[q];
          if (p == 0) {
            acc[s][i][4 * q] = u.x;
            acc[s][i][4 * q + 1] = u.y;
            acc[s][i][4 * q + 2] = u.z;
            acc[s][i][4 * q + 3] = u.w;
          } else {
            acc[s][i][4 * q] += u.x;
            acc[s][i][4 * q + 1] += u.y;
            acc[s][i][4 * q + 2] += u.z;
            acc[s][i][4 * q + 3] += u.w;
          }
        }
      }
  }
  store_rows32<WN, TN, UPGATE>([&](int s, int i, int r) { return acc[s][i][r]; }, row0,
                               tl.n0 + wn * WN, tl.m_end, N, a, 0, stage[j], lane);
}

// ---------------------------------------------------------------- decode
// Streaming kernel for a few rows per group (decode-sized batches), where the
// layer is bound by reading the touched experts' weights once from HBM.  A
// tile is 16 output features (up/gate: 16 up rows and 16 gate rows) by 16
// grouped rows.  The four waves split K; each copies its K range in 1 KB
// bursts (8 rows x 64 k: whole 128-byte lines) with global_load_lds_dwordx4
// into a ring of D LDS stages of its own, D - 1 slabs of 64 k ahead, and reads
// MFMA fragments from there.  A wave only reads what it fetched itself, so no
// workgroup barrier is needed until the cross-wave sum, which is added in
// wave order (deterministic).  Weight bursts are non-temporal (each weight is
// used by one tile only; the token rows, shared by all column tiles of a
// group, stay cached).  Measured on MI355X with a 2-stage ring: the Mixtral-
// shaped 16-token layer's expert GEMMs stream 6.6 TB/s; deeper rings were
// slower (fewer workgroups per CU), cached weight bursts ~20% slower.
// Rows of a 1 KB block are 128 bytes; the 16-byte chunk c of row r sits at
// slot c ^ ((r / 2) % 8), so the 16 lanes of a ds_read_b128 phase (16 rows,
// one chunk) hit distinct banks.  16x16x32 bf16 MFMAs take the weight rows as
// the A operand, so a lane ends with 4 consecutive features of one row.
constexpr int kWeightPolicy = 2;  // cache policy of the weight bursts: nt
template <bool UPGATE, int D>
__global__ __launch_bounds__(256) void gemm_bf16_stream_kernel(GemmArgs a) {
  constexpr int BN = 16, NS = UPGATE ? 2 : 1;
  constexpr int WBLK = NS * 2, XBLK = 2;         // 1 KB blocks per slab
  constexpr int NDMA = WBLK + XBLK;
  constexpr int SLAB = NDMA * 512;               // bf16 elements per slab
  static_assert((D - 1) * NDMA <= 63, "vmcnt range");
  const int L = tile_of_block(a.tiles);
  if (L < 0) return;
  const int ncol = __builtin_amdgcn_readfirstlane(a.tiles[0].m_end);  // column tile fastest
  Tile tl = uniform_tile(a.tiles[1 + L / ncol]);
  tl.n0 = (L % ncol) * BN;
  const bool sh = tl.g >= a.E;
  const int N = sh ? a.N_s : a.N_r;
  const int K = sh ? a.K_s : a.K_r;
  if (tl.n0 >= N) return;
  const int64_t wstride = (int64_t)N * K;
  const uint16_t* W0 = sh ? a.s0 + (tl.g - a.E) * wstride : a.w0 + tl.g * wstride;
  const uint16_t* W1 = UPGATE ? (sh ? a.s1 + (tl.g - a.E) * wstride : a.w1 + tl.g * wstride)
                              : W0;
  __shared__ __attribute__((aligned(1024))) uint16_t ring[4][D][SLAB];
  static_assert(NS * 64 * sizeof(f32x4) <= SLAB * sizeof(uint16_t), "partial sums fit a stage");

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this lane's source in each 1 KB block: row 8 b + lane / 8 of the tile, at
  // the global chunk that lands in slot lane % 8
  const uint16_t* src[NDMA];
#pragma unroll
  for (int b = 0; b < NDMA; ++b) {
    const int r = 8 * b + (lane >> 3);
    const int gch = (lane & 7) ^ ((r >> 1) & 7);
    if (b < WBLK) {
      int n = tl.n0 + (r & 15);
      n = n < N ? n : N - 1;
      src[b] = (UPGATE && b >= 2 ? W1 : W0) + (int64_t)n * K + gch * 8;
    } else {
      int row = tl.m0 + (r & 15);
      row = row < tl.m_end ? row : tl.m_end - 1;
      const int64_t t = a.sorted ? (int64_t)a.sorted[row] : (int64_t)row;
      src[b] = a.tok + t * a.ldt + gch * 8;
    }
  }
  const int nsl = K >> 6;
  const int s0 = wave * nsl / 4, s1 = (wave + 1) * nsl / 4, n = s1 - s0;
  auto dma = [&](int sl, uint16_t* dst) {
    sl = min(sl, s1 - 1);  // past the end: re-fetch the last slab into a dead stage
#pragma unroll
    for (int b = 0; b < WBLK; ++b)
      __builtin_amdgcn_global_load_lds((const void*)(src[b] + sl * 64), LDS_PTR(dst + b * 512),
                                       16, 0, kWeightPolicy);
#pragma unroll
    for (int b = WBLK; b < NDMA; ++b)
      __builtin_amdgcn_global_load_lds((const void*)(src[b] + sl * 64), LDS_PTR(dst + b * 512),
                                       16, 0, 0);
  };
  auto slot = [](int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 7)) << 3); };
  f32x4 acc[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (n > 0) {
#pragma unroll
    for (int i = 0; i < D - 1; ++i) dma(s0 + i, ring[wave][i]);
    for (int i = 0; i < n; ++i) {
      // the stage refilled now was read in the previous iteration: its reads are done
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(63) & kLgkm0);
      asm volatile("" ::: "memory");
      dma(s0 + i + D - 1, ring[wave][(i + D - 1) % D]);
      __builtin_amdgcn_s_waitcnt(vmcnt_imm((D - 1) * NDMA));  // slab i has landed
      asm volatile("" ::: "memory");
      const uint16_t* cur = ring[wave][i % D];
#pragma unroll
      for (int j = 0; j < 2; ++j) {  // two 32-k MFMA steps per slab
        const int c = j * 4 + (lane >> 4);
        const u32x4 fx = *(const u32x4*)(cur + WBLK * 512 + slot(lane & 15, c));
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          const u32x4 fw = *(const u32x4*)(cur + slot(16 * q + (lane & 15), c));
          acc[q] = mfma16(fw, fx, acc[q]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // drain the re-fetches
  }
  // partial sums go to the wave's own (drained) first stage
  if (wave > 0) {
    f32x4* red = (f32x4*)ring[wave][0];
#pragma unroll
    for (int q = 0; q < NS; ++q) red[q * 64 + lane] = acc[q];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    const f32x4* red = (const f32x4*)ring[w][0];
#pragma unroll
    for (int q = 0; q < NS; ++q) acc[q] += red[q * 64 + lane];
  }
  // D[n = feature][m = row]: lane holds row (lane & 15), features 4*(lane>>4)+0..3
  const int nn = tl.n0 + 4 * (lane >> 4);
  const int row = tl.m0 + (lane & 15);
  if (nn >= N || row >= tl.m_end) return;
  if (UPGATE) {
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(silu_mul(acc[1][0], acc[0][0])) |
           ((uint32_t)f32_to_bf16(silu_mul(acc[1][1], acc[0][1])) << 16);
    pk.y = (uint32_t)f32_to_bf16(silu_mul(acc[1][2], acc[0][2])) |
           ((uint32_t)f32_to_bf16(silu_mul(acc[1][3], acc[0][3])) << 16);
    *(uint2*)((uint16_t*)a.out + (int64_t)row * a.ldo + nn) = pk;
  } else {
    *(float4*)((float*)a.out + (int64_t)row * a.ldo + nn) =
        make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
  }
}

// ---------------------------------------------------------------- MXFP4
// Streaming kernel for MXFP4 expert weights.  A tile is 32 output features
// (two groups of 16) by 16 grouped rows; the four waves split K.  Weights
// are read as packed E2M1 codes plus one E8M0 scale per 32 of K (a quarter
// of the bf16 bytes, plus 1/32) and widened to bf16 in registers by
// v_cvt_scalef32_pk_bf16_fp4 (exact: an E2M1 value times a power of two is a
// bf16 value), then bf16 MFMAs with fp32 accumulation.
// Loads go straight into registers, no LDS.  Per 128-k unit, lane
// (r = lane % 16, g = lane / 16) takes, for each feature group, feature row
// r's codes of k [128u + 32g, 128u + 32g + 32): 16 bytes, one scale byte;
// and token row r's x of the same 32 k (64 bytes), shared by the two
// feature groups.  MFMA step s of the unit feeds k 128u + 32g + 8s + (0..7)
// from lane group g on both operands; the order of k inside a dot product is
// free, so this is the full sum.  A block past K (the last unit of a K that
// is an odd multiple of 64) reads a clamped address and its codes are
// zeroed.  Loads go in batches of U units, all issued before the batch's
// conversions and MFMAs.  Measured on MI355X (gpt-oss-shaped layer, T=128):
// 32 features per tile 0.55 ms, 64 features 0.66 ms (more registers, fewer
// waves in flight), 16 features with 16 k per lane 0.65 ms; batches of 1 or
// 2 units alike, 4 slower.
template <bool UPGATE>
__global__ __launch_bounds__(256) void gemm_mx_stream_kernel(GemmArgs a) {
  constexpr int NS = UPGATE ? 2 : 1;
  constexpr int FG = 2;   // 16-feature groups per tile
  constexpr int U = 2;    // 128-k units per batch of loads
  const int L = tile_of_block(a.tiles);
  if (L < 0) return;
  const int ncol = __builtin_amdgcn_readfirstlane(a.tiles[0].m_end);  // column tile fastest
  Tile tl = uniform_tile(a.tiles[1 + L / ncol]);
  tl.n0 = (L % ncol) * (16 * FG);
  const bool sh = tl.g >= a.E;
  const int N = sh ? a.N_s : a.N_r;
  const int K = sh ? a.K_s : a.K_r;
  if (tl.n0 >= N) return;
  const int ge = sh ? tl.g - a.E : tl.g;
  const int rstr = a.mx_line ? (K / 2 + 127) & ~127 : K / 2;  // code row pitch, bytes
  const int64_t cstride = (int64_t)N * rstr, sstride = (int64_t)N * (K / 32);
  const uint8_t* C[NS];
  const uint8_t* S[NS];
  C[0] = (const uint8_t*)(sh ? a.s0 : a.w0) + ge * cstride;
  S[0] = (sh ? a.ss0 : a.sw0) + ge * sstride;
  if (UPGATE) {
    C[NS - 1] = (const uint8_t*)(sh ? a.s1 : a.w1) + ge * cstride;
    S[NS - 1] = (sh ? a.ss1 : a.sw1) + ge * sstride;
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const uint8_t* cp[FG][NS];
  const uint8_t* sp[FG][NS];
#pragma unroll
  for (int f = 0; f < FG; ++f) {
    int n = tl.n0 + 16 * f + r;
    n = n < N ? n : N - 1;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      cp[f][q] = C[q] + (int64_t)n * rstr + g * 16;
      sp[f][q] = S[q] + (int64_t)n * (K / 32) + g;
    }
  }
  int row = tl.m0 + r;
  row = row < tl.m_end ? row : tl.m_end - 1;
  const int64_t tok = a.sorted ? (int64_t)a.sorted[row] : (int64_t)row;
  const uint16_t* xp = a.tok + tok * a.ldt + g * 32;
  const int nb = K >> 5;               // 32-k blocks
  const int nu = (nb + 3) >> 2;        // 128-k units (the last may hold 2 blocks)
  const int u0 = wave * nu / 4, u1 = (wave + 1) * nu / 4;
  f32x4 acc[FG][NS];
#pragma unroll
  for (int f = 0; f < FG; ++f)
#pragma unroll
    for (int q = 0; q < NS; ++q) acc[f][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int ub = u0; ub < u1; ub += U) {
    u32x4 cw[U][FG][NS];
    uint32_t sb[U][FG][NS];
    u32x4 xv[U][4];
    bool live[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int u = min(ub + i, u1 - 1);
      const int blk = 4 * u + g;
      live[i] = ub + i < u1 && blk < nb;
      const int bc = blk < nb ? blk : nb - 1;  // clamped block of the loads
      const int ofs = (bc - g) * 16;           // codes: 16 bytes per block
#pragma unroll
      for (int f = 0; f < FG; ++f)
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          cw[i][f][q] = *(const u32x4*)(cp[f][q] + ofs);
          sb[i][f][q] = sp[f][q][bc - g];
        }
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) xv[i][s2] = *(const u32x4*)(xp + (bc - g) * 32 + s2 * 8);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
#pragma unroll
      for (int f = 0; f < FG; ++f)
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          // E8M0 byte -> float32 2^(S-127): the exponent field, except 0
          // (2^-127, a float32 subnormal) and 255 (NaN)
          const uint32_t b = sb[i][f][q];
          const float scale =
              __uint_as_float(b == 0 ? 0x00400000u : b == 255 ? 0x7FC00000u : b << 23);
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const uint32_t w = live[i] ? cw[i][f][q][s2] : 0u;
            u32x4 fa;
            fa[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
            fa[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
            fa[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
            fa[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
            acc[f][q] = mfma16(fa, xv[i][s2], acc[f][q]);
          }
        }
    }
  }
  // partial sums of waves 1..3 through LDS, added to wave 0's in wave order
  __shared__ f32x4 red[3][FG * NS][64];
  if (wave > 0) {
#pragma unroll
    for (int f = 0; f < FG; ++f)
#pragma unroll
      for (int q = 0; q < NS; ++q) red[wave - 1][f * NS + q][lane] = acc[f][q];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int f = 0; f < FG; ++f)
#pragma unroll
      for (int q = 0; q < NS; ++q) acc[f][q] += red[w][f * NS + q][lane];
  // D[n = feature][m = row]: lane holds row (lane & 15) and, in group f,
  // features 16 f + 4 (lane >> 4) + 0..3
  const int orow = tl.m0 + (lane & 15);
  if (orow >= tl.m_end) return;
#pragma unroll
  for (int f = 0; f < FG; ++f) {
    const int nn = tl.n0 + 16 * f + 4 * (lane >> 4);
    if (nn >= N) continue;
    if (UPGATE) {
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(silu_mul(acc[f][1][0], acc[f][0][0])) |
             ((uint32_t)f32_to_bf16(silu_mul(acc[f][1][1], acc[f][0][1])) << 16);
      pk.y = (uint32_t)f32_to_bf16(silu_mul(acc[f][1][2], acc[f][0][2])) |
             ((uint32_t)f32_to_bf16(silu_mul(acc[f][1][3], acc[f][0][3])) << 16);
      *(uint2*)((uint16_t*)a.out + (int64_t)orow * a.ldo + nn) = pk;
    } else {
      *(float4*)((float*)a.out + (int64_t)orow * a.ldo + nn) =
          make_float4(acc[f][0][0], acc[f][0][1], acc[f][0][2], acc[f][0][3]);
    }
  }
}

// MXFP4 (EB = 4) or MXFP8 (EB = 8) weights through LDS, for batches with
// about one (token, expert) pair per expert and more: a tile is 16 rows x
// 16 NW features, one wave per 16 features over the whole of K, so the
// token slab in LDS is shared by NW waves (the direct-load kernel above
// re-reads it per wave).  K streams in
// stages of 256 (eight 32-k blocks) through a 3-stage ring of LDS copies: a
// stage holds the 16 x 256 token slab (8 KB, every wave copies 8 KB / NW
// of it) and, per wave and weight matrix, 16 feature rows x 128 code bytes
// (a copy instruction moves 128 contiguous bytes of 8 rows).  The tile's
// E8M0 scales (16 NW rows x K/32 bytes, one contiguous block in HBM) are
// copied to LDS once, before the ring starts, so no load into registers
// sits between the copies in flight (the compiler would then wait for all
// of them).  Lane (r, g) feeds k 32 j + 8 g + (0..7) of block j: codes dword
// g of feature row r's block j, widened with the row's block scale, and
// token row r.  16-byte chunks sit XOR-swizzled in LDS (codes: chunk c of
// row r at c ^ (r / 2) % 8; tokens: chunk c at c ^ r % 16) so fragment
// reads spread over the banks.  Blocks past K copy a clamped chunk of
// codes and zeros for the tokens, so they add nothing (a zero token times a
// finite code; a NaN code or scale there is one of the last live block's,
// which makes the sum NaN anyway); waves past N (a partial tile) re-read
// the last row and store nothing.  Needs K a multiple of 64 and at most kMxLdsMaxK.
// EB = 8 is the MXFP8 form: E4M3 codes, one per byte, so a row's stage is
// 256 bytes (a copy moves 4 rows, chunk c of row r at slot c ^ r % 16), a
// lane reads 8 bytes of its block and widens them with
// v_cvt_scalef32_pk_bf16_fp8; K up to kMx8MaxK.
// Code copies use the default cache policy, not the non-temporal one of the
// bf16 weight bursts: MX code rows (1440 bytes for the gpt-oss-shaped FP4
// layer, 2880 for FP8) start off 128-byte lines, so a row's 128-byte stage
// spans two lines, the second of which the next stage reads again; streamed
// non-temporally it was fetched twice.  Measured on MI355X, gpt-oss-shaped
// FP4 layer, T=128: L2 fetch of the up/gate GEMM 1.66x -> 1.11x the code and
// scale bytes, layer 0.487 -> 0.432 ms (T=32 and T=512 also -10%; FP8 -1%).
// CPOL is that policy: 0, or non-temporal (kWeightPolicy) for code rows on
// whole lines (MOE_FLAG_MX_LINE_ROWS) when about one row tile reads each
// weight tile (measured, gpt-oss-shaped line-row layer: T = 8 ... 128 -3 to
// -5% for both formats; T=512, where experts of more than 16 rows read
// their codes twice, +5 to +9%, so it keeps the default there).
template <bool UPGATE, int NW, int EB, int CPOL = 0>
__global__ __launch_bounds__(64 * NW) void gemm_mx_lds_kernel(GemmArgs a) {
  constexpr int NS = UPGATE ? 2 : 1;
  constexpr int XS = 16 * 256;               // token stage, bf16 elements (8 KB)
  constexpr int XI = 8 / NW;                 // token copies per wave and stage
  constexpr int RB = 32 * EB;                // code bytes of a row per stage (128 / 256)
  constexpr int CS = NW * NS * 16 * RB;      // code stage, bytes
  constexpr int NCC = 16 * RB / 1024;        // code copies per wave, matrix and stage
  constexpr int RPC = 1024 / RB, LPR = RB / 16;  // rows per copy, lanes per row
  constexpr int KMAX = EB == 8 ? kMx8MaxK : kMxLdsMaxK;
  constexpr int SCS = 16 * NW * (KMAX / 32);  // scales of one matrix, bytes
  constexpr int NLD = XI + NCC * NS;         // copies per wave and stage
  static_assert(NW == 4 || NW == 8, "the token slab splits into 1 KB copies per wave");
  static_assert(EB == 4 || EB == 8, "FP4 or FP8 elements");
  const int L = tile_of_block(a.tiles);
  if (L < 0) return;
  const int ncol = __builtin_amdgcn_readfirstlane(a.tiles[0].m_end);  // column tile fastest
  Tile tl = uniform_tile(a.tiles[1 + L / ncol]);
  tl.n0 = (L % ncol) * (16 * NW);
  const bool sh = tl.g >= a.E;
  const int N = sh ? a.N_s : a.N_r;
  const int K = sh ? a.K_s : a.K_r;
  if (tl.n0 >= N) return;
  const int ge = sh ? tl.g - a.E : tl.g;
  const int nb = K >> 5;                 // 32-k blocks
  const int nst = (nb + 7) >> 3;         // 256-k stages
  const int rowb = K * EB / 8;           // code bytes per weight row
  const int rstr = a.mx_line ? (rowb + 127) & ~127 : rowb;  // row pitch in the code array
  const int64_t cstride = (int64_t)N * rstr, sstride = (int64_t)N * nb;
  // one named array per stage, so the compiler tells reads of one stage
  // from copies still landing in another
  __shared__ __attribute__((aligned(1024))) uint16_t lx0[XS], lx1[XS], lx2[XS];
  __shared__ __attribute__((aligned(1024))) uint8_t lc0[CS], lc1[CS], lc2[CS];
  __shared__ __attribute__((aligned(1024))) uint8_t lsc[NS * SCS];
  // E8M0 byte -> float32 scale 2^(byte - 127) (byte 0: 2^-127, a float32
  // subnormal; byte 255: NaN), so a scale costs one LDS read instead of a
  // shift, two compares and two selects per block
  __shared__ float e8m0[256];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int b = threadIdx.x; b < 256; b += 64 * NW)
    e8m0[b] = __uint_as_float(b == 0 ? 0x00400000u : b == 255 ? 0x7FC00000u : (uint32_t)b << 23);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(63) & kLgkm0);  // written before the first barrier

  // token copy: instruction i of wave w fills 1 KB block b = w + NW i, rows
  // 2 b + l / 32; lane l takes LDS slot l % 32 of its row, global chunk
  // slot ^ row % 16.  The copies are buffer loads, and a chunk past K reads
  // at offset tok_bytes (out of range): zeros, so the 32-k blocks past K add
  // nothing whatever their (clamped) codes hold.
  uint32_t xoffb[XI];
  int xchunk[XI];
#pragma unroll
  for (int i = 0; i < XI; ++i) {
    const int xr = 2 * (wave + NW * i) + (lane >> 5);
    int xrow = tl.m0 + xr;
    xrow = xrow < tl.m_end ? xrow : tl.m_end - 1;
    const uint32_t xtok = a.sorted ? (uint32_t)a.sorted[xrow] : (uint32_t)xrow;
    xoffb[i] = xtok * (uint32_t)a.ldt * 2;
    xchunk[i] = (lane & 31) ^ (xr & 15);
  }
  const __amdgpu_buffer_rsrc_t rx = buffer_of(a.tok, a.tok_bytes);
  // code copy: instruction i of a matrix holds feature rows 16 w + RPC i +
  // l / LPR; lane l takes slot l % LPR, the row's 16-byte chunk of the stage
  // slot ^ (row / 2) % 8 (FP4) or slot ^ row % 16 (FP8)
  const uint8_t* csrc[NS][NCC];
  int cchunk[NCC];
#pragma unroll
  for (int i = 0; i < NCC; ++i) {
    const int cr = RPC * i + lane / LPR;
    cchunk[i] = (lane % LPR) ^ (EB == 4 ? ((cr >> 1) & 7) : (cr & 15));
    int64_t cn = tl.n0 + 16 * wave + cr;
    cn = cn < N ? cn : N - 1;
#pragma unroll
    for (int q = 0; q < NS; ++q)
      csrc[q][i] = (const uint8_t*)(q == 0 ? (sh ? a.s0 : a.w0) : (sh ? a.s1 : a.w1)) +
                   ge * cstride + cn * rstr;
  }
  // the row lookups above have landed before any copy is issued (a load
  // into registers behind copies in flight would wait for all of them)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_sched_barrier(0);
  // scales: the tile's rows x nb bytes of each matrix, 1 KB per copy
  // instruction, instruction i by wave i % NW (chunks past the end clamped)
  {
    const int rows = min(16 * NW, N - tl.n0);  // a multiple of 64, as N is
    const int nch = rows * nb / 16, ni = (nch + 63) >> 6;
#pragma unroll
    for (int q = 0; q < NS; ++q) {
      const uint8_t* src =
          (q == 0 ? (sh ? a.ss0 : a.sw0) : (sh ? a.ss1 : a.sw1)) + ge * sstride + (int64_t)tl.n0 * nb;
      for (int i = wave; i < ni; i += NW) {
        int c = 64 * i + lane;
        c = c < nch ? c : nch - 1;
        __builtin_amdgcn_global_load_lds((const void*)(src + 16 * c),
                                         LDS_PTR(lsc + q * SCS + i * 1024), 16, 0, 0);
      }
    }
  }
  // all copies of stage st (clamped past the end: a re-fetch into a dead stage)
  auto issue = [&](int st, uint16_t* lx, uint8_t* lc) {
    st = st < nst ? st : nst - 1;
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int c = 32 * st + xchunk[i];     // 8-k chunk along the token row
      const uint32_t off = c < (K >> 3) ? xoffb[i] + (uint32_t)c * 16 : a.tok_bytes;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, LDS_PTR(lx + (wave + NW * i) * 512), 16, off,
                                               0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
      for (int i = 0; i < NCC; ++i) {
        int b = LPR * st + cchunk[i];        // 16-byte code chunk along the row
        b = b < rowb / 16 ? b : rowb / 16 - 1;
        __builtin_amdgcn_global_load_lds((const void*)(csrc[q][i] + b * 16),
                                         LDS_PTR(lc + (wave * NS + q) * 16 * RB + i * 1024), 16,
                                         0, CPOL);
      }
  };
  f32x4 acc[NS];
#pragma unroll
  for (int q = 0; q < NS; ++q) acc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r = lane & 15, g = lane >> 4;
  const int srow = (16 * wave + r) * nb;     // this lane's scale row in LDS
  auto compute = [&](int st, const uint16_t* xs, const uint8_t* lc) {
    // the stage's 8 block scales of each matrix first: independent reads,
    // then their table entries, instead of a two-read chain per block
    uint32_t sbyte[NS][8];
    float scl[NS][8];
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        sbyte[q][j] = lsc[q * SCS + srow + min(8 * st + j, nb - 1)];
        asm volatile("" ::: "memory");  // no merged reads (they carry no alias information)
      }
#pragma unroll
    for (int q = 0; q < NS; ++q)
#pragma unroll
      for (int j = 0; j < 8; ++j) scl[q][j] = e8m0[sbyte[q][j]];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int xoff = r * 256 + (((4 * j + g) ^ r) << 3);
      const u32x4 fx = *(const u32x4*)(xs + xoff);
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        // FP4: dword g of block j (8 codes); FP8: bytes 8 g .. 8 g + 7 of
        // block j, which is chunks 2 j and 2 j + 1 of the row
        const int base = (wave * NS + q) * 16 * RB + r * RB;
        u32x2 w;
        if (EB == 4) {
          w[0] = *(const uint32_t*)(lc + base + ((j ^ ((r >> 1) & 7)) << 4) + 4 * g);
          w[1] = 0u;
        } else {
          w = *(const u32x2*)(lc + base + (((2 * j + (g >> 1)) ^ r) << 4) + 8 * (g & 1));
        }
        asm volatile("" ::: "memory");  // keep reads of different arrays apart (a
                                        // merged read carries no alias information)
        const float scale = scl[q][j];
        u32x4 fa;
        if (EB == 4) {
          fa[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[0], scale, 0));
          fa[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[0], scale, 1));
          fa[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[0], scale, 2));
          fa[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[0], scale, 3));
        } else {
          fa[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], scale, false));
          fa[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], scale, true));
          fa[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], scale, false));
          fa[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], scale, true));
        }
        acc[q] = mfma16(fa, fx, acc[q]);
      }
    }
  };
  // this wave's copies of the stage to read (and every older copy, the
  // scales included) have landed, then all waves'; a plain barrier (a
  // fenced one would wait for every copy in flight)
  auto wait_stage = [&]() {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(NLD));
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  issue(0, lx0, lc0);
  issue(1, lx1, lc1);
  int st = 0;
  for (; st + 3 <= nst; st += 3) {
    wait_stage();
    issue(st + 2, lx2, lc2);
    compute(st, lx0, lc0);
    wait_stage();
    issue(st + 3, lx0, lc0);
    compute(st + 1, lx1, lc1);
    wait_stage();
    issue(st + 4, lx1, lc1);
    compute(st + 2, lx2, lc2);
  }
  if (st < nst) {
    wait_stage();
    issue(st + 2, lx2, lc2);
    compute(st, lx0, lc0);
    if (st + 1 < nst) {
      wait_stage();
      compute(st + 1, lx1, lc1);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // drain the re-fetches
  // D[n = feature][m = row]: lane holds row (lane & 15), features 4*(lane>>4)+0..3
  const int nn = tl.n0 + 16 * wave + 4 * (lane >> 4);
  const int orow = tl.m0 + (lane & 15);
  if (orow >= tl.m_end || nn >= N) return;
  if (UPGATE) {
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(silu_mul(acc[1][0], acc[0][0])) |
           ((uint32_t)f32_to_bf16(silu_mul(acc[1][1], acc[0][1])) << 16);
    pk.y = (uint32_t)f32_to_bf16(silu_mul(acc[1][2], acc[0][2])) |
           ((uint32_t)f32_to_bf16(silu_mul(acc[1][3], acc[0][3])) << 16);
    *(uint2*)((uint16_t*)a.out + (int64_t)orow * a.ldo + nn) = pk;
  } else {
    *(float4*)((float*)a.out + (int64_t)orow * a.ldo + nn) =
        make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
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
                  x.tiles_up, P.up.xcd_remap, 1, 0, (uint32_t)(D.T * D.d * 2),
                  x.mx.up, x.mx.gate, x.mx.s_up, x.mx.s_gate, x.part, P.up.sk_cus,
                  (D.flags & MOE_FLAG_MX_LINE_ROWS) ? 1 : 0};
}
static GemmArgs down_args(const Plan& P, const ExpertArgs& x) {
  const moe_desc& D = P.desc;
  const int ffn_s = D.n_shared ? D.ffn_shared : D.ffn;
  return GemmArgs{(const uint16_t*)x.h, nullptr, P.ffn_max, (const uint16_t*)x.w_down, nullptr,
                  (const uint16_t*)x.ws_down, nullptr, D.E, D.d, D.d, D.ffn, ffn_s, x.out, D.d,
                  x.tiles_down, P.down.xcd_remap, x.ksplit,
                  (int64_t)((size_t)P.R + kRowSlack) * D.d,
                  (uint32_t)(((size_t)P.R + kRowSlack) * P.ffn_max * 2), x.mx.down, nullptr,
                  x.mx.s_down, nullptr, x.part, P.down.sk_cus,
                  (D.flags & MOE_FLAG_MX_LINE_ROWS) ? 1 : 0};
}

// LDS stages (weights, tokens) of the prefill GEMM instantiations, at most
// 160 KB: 256-row tiles hold 3 x 32 KB of weight slabs and 2 x 32 KB of
// token slabs, 128-row tiles 3 x (32 + 16) KB, 64-row tiles 2 x (32 + 8) KB
// (two workgroups per CU).  Measured on MI355X against
// 2 + 2 stages for 256-row tiles: Mixtral-shaped T=4096 layer 2.93 -> 2.62
// ms; a 16-slab down GEMM 0.116 -> 0.109 ms.
constexpr int kWStages256 = 3, kXStages256 = 2, kWStages128 = 3, kXStages128 = 3;
// Per-wave tile (rows x output columns) of the 256-row instantiations; the
// wave count is (BM / WM) * (BN / WN).
constexpr int kUp256WM = 128, kUp256WN = 64, kDown256WM = 128, kDown256WN = 128;

template <int BM, int BN, int WM, int WN, bool UPGATE, int NSW, int NSX>
static void launch_gemm(dim3 grid, hipStream_t s, const GemmArgs& a, bool stream_w) {
  constexpr int nw = (BM / WM) * (BN / WN);
  if (a.sk_cus > 0) {
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, UPGATE, NSW, NSX, 0>),
                       dim3(grid.x + 8 + (unsigned)a.sk_cus), dim3(64 * nw), 0, s, a);
    hipLaunchKernelGGL((gemm_fixup_kernel<BM, BN, WM, WN, UPGATE>),
                       dim3((unsigned)a.sk_cus * nw), dim3(64 * (WM / 32)), 0, s, a);
    return;
  }
  if (stream_w)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, UPGATE, NSW, NSX, kWeightPolicy>), grid,
                       dim3(64 * nw), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, UPGATE, NSW, NSX, 0>), grid,
                       dim3(64 * nw), 0, s, a);
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
  if (P.kind == KIND_MXFP8 && P.up.stream_w)
    hipLaunchKernelGGL((gemm_mx_lds_kernel<true, kMx8Waves, 8, kWeightPolicy>), grid,
                       dim3(64 * kMx8Waves), 0, s, up_args(P, x));
  else if (P.kind == KIND_MXFP8)
    hipLaunchKernelGGL((gemm_mx_lds_kernel<true, kMx8Waves, 8>), grid, dim3(64 * kMx8Waves), 0, s,
                       up_args(P, x));
  else if (P.kind == KIND_MXFP4 && P.up.bn == 16 * kMxUpWaves && P.up.stream_w)
    hipLaunchKernelGGL((gemm_mx_lds_kernel<true, kMxUpWaves, 4, kWeightPolicy>), grid,
                       dim3(64 * kMxUpWaves), 0, s, up_args(P, x));
  else if (P.kind == KIND_MXFP4 && P.up.bn == 16 * kMxUpWaves)
    hipLaunchKernelGGL((gemm_mx_lds_kernel<true, kMxUpWaves, 4>), grid, dim3(64 * kMxUpWaves), 0,
                       s, up_args(P, x));
  else if (P.kind == KIND_MXFP4)
    hipLaunchKernelGGL(gemm_mx_stream_kernel<true>, grid, block, 0, s, up_args(P, x));
  else if (P.kind == KIND_BF16_DECODE)
    hipLaunchKernelGGL((gemm_bf16_stream_kernel<true, 2>), grid, block, 0, s, up_args(P, x));
  else if (P.up.bm == 128)
    launch_gemm<128, 128, 128, 32, true, kWStages128, kXStages128>(grid, s, up_args(P, x),
                                                                   P.up.stream_w);
  else if (P.up.bm == 64)
    launch_gemm<64, 128, 64, 32, true, 2, 2>(grid, s, up_args(P, x), P.up.stream_w);
  else
    launch_gemm<256, 128, kUp256WM, kUp256WN, true, kWStages256, kXStages256>(grid, s, up_args(P, x),
                                                                             false);
  return hipGetLastError();
}

hipError_t launch_expert_down(const Plan& P, const ExpertArgs& x, hipStream_t s) {
  const moe_desc& D = P.desc;
  const dim3 block(256);
  const dim3 grid((unsigned)(((P.down.max_tiles * x.ksplit + 7) / 8) * 8));
  if (P.kind == KIND_F32) {
    const int ffn_s = D.n_shared ? D.ffn_shared : D.ffn;
    GemmArgsF32 dn{(const float*)x.h, nullptr, P.ffn_max, (const float*)x.w_down, nullptr,
                   (const float*)x.ws_down, nullptr, D.E, D.d, D.d, D.ffn, ffn_s, x.out, D.d,
                   x.tiles_down};
    hipLaunchKernelGGL(gemm_f32_kernel<false>, grid, block, 0, s, dn);
    return hipGetLastError();
  }
  if (P.kind == KIND_MXFP8 && P.down.stream_w)
    hipLaunchKernelGGL((gemm_mx_lds_kernel<false, kMx8Waves, 8, kWeightPolicy>), grid,
                       dim3(64 * kMx8Waves), 0, s, down_args(P, x));
  else if (P.kind == KIND_MXFP8)
    hipLaunchKernelGGL((gemm_mx_lds_kernel<false, kMx8Waves, 8>), grid, dim3(64 * kMx8Waves), 0, s,
                       down_args(P, x));
  else if (P.kind == KIND_MXFP4 && P.down.bn == 16 * kMxDownWaves && P.down.stream_w)
    hipLaunchKernelGGL((gemm_mx_lds_kernel<false, kMxDownWaves, 4, kWeightPolicy>), grid,
                       dim3(64 * kMxDownWaves), 0, s, down_args(P, x));
  else if (P.kind == KIND_MXFP4 && P.down.bn == 16 * kMxDownWaves)
    hipLaunchKernelGGL((gemm_mx_lds_kernel<false, kMxDownWaves, 4>), grid, dim3(64 * kMxDownWaves),
                       0, s, down_args(P, x));
  else if (P.kind == KIND_MXFP4)
    hipLaunchKernelGGL(gemm_mx_stream_kernel<false>, grid, block, 0, s, down_args(P, x));
  else if (P.kind == KIND_BF16_DECODE)
    hipLaunchKernelGGL((gemm_bf16_stream_kernel<false, 2>), grid, block, 0, s, down_args(P, x));
  else if (P.down.bm == 128)
    launch_gemm<128, 256, 128, 64, false, kWStages128, kXStages128>(grid, s, down_args(P, x),
                                                                    P.down.stream_w);
  else if (P.down.bm == 64)
    launch_gemm<64, 256, 64, 64, false, 2, 2>(grid, s, down_args(P, x), P.down.stream_w);
  else if (P.down.all_rows)
    launch_gemm<256, 256, 256, 64, false, kWStages256, kXStages256>(grid, s, down_args(P, x),
                                                                   P.down.stream_w);
  else
    launch_gemm<256, 256, kDown256WM, kDown256WN, false, kWStages256, kXStages256>(
        grid, s, down_args(P, x), false);
  return hipGetLastError();
}

}  // namespace moe
