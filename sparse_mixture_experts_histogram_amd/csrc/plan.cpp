// Host-side validation, path choice and workspace layout (no HIP calls).
#include "plan.h"

#include <algorithm>
#include <climits>
#include <cmath>

namespace moe {

// Tile shapes (rows per tile, output columns per tile) of the two grouped
// GEMMs for each kernel family; they must match the kernel instantiations
// launched in experts.hip.  Prefill uses 256-row tiles when experts average
// at least 384 rows (less padding is then worth the larger reuse), 64-row
// tiles when they average at most 32 (80 KB of LDS, two workgroups per CU,
// so twice the copies in flight for these weight-streaming layers; measured
// on MI355X: gpt-oss-shaped T=512, 16 rows per expert, 1.125 -> 1.093 ms;
// the DeepSeek-V3-shaped layer, 128 rows per expert, was 9% slower on them),
// else 128.
static int prefill_rows(const moe_desc* d) {
  const int64_t pairs = d->T * d->k;
  return pairs >= 384LL * d->E ? 256 : pairs <= 32LL * d->E ? 64 : 128;
}
// The down GEMM of layers averaging 128 to 384 rows per expert runs 256-row
// tiles whose waves each span all 256 rows, so a tile leaves out the MFMAs
// and token copies of its 32-row groups past the last row, and an expert of
// up to 256 rows streams its weights once (with 128-row tiles, one pass per
// row tile).  Measured on MI355X, DeepSeek-V3-shaped T=4096 (E=256, 128
// rows per expert on average, skewed): down GEMM 2.06 -> 1.95 ms.  The
// up/gate GEMM in that form was no faster than its 128-row tiles (3.57 ms
// against 3.58) and its kernel spilled registers, so it keeps them.
static bool down_all_rows(const moe_desc* d) {
  const int64_t pairs = d->T * d->k;
  return pairs >= 128LL * d->E && pairs < 384LL * d->E;
}
// The streaming kernels use 16-row tiles of 16 (bf16) or 32 (MXFP4) columns;
// MXFP4 layers with at least one (token, expert) pair per four experts and a
// reduction of at most kMxLdsMaxK use the LDS-staged kernel's wider tiles
// (measured on the gpt-oss-shaped layer, with the LDS kernel's cached code
// copies: T=8 0.140 -> 0.128 ms, T=16 0.212 -> 0.187 ms, T=32 alike; T=1
// slower, 0.050 -> 0.056 ms).
static bool streaming(int kind) {
  return kind == KIND_BF16_DECODE || kind == KIND_MXFP4 || kind == KIND_MXFP8;
}
static bool mx_lds(const moe_desc* d, int K) {
  return 4 * (int64_t)d->T * d->k >= d->E && K <= kMxLdsMaxK;
}
static int down_k(const moe_desc* d) {
  return d->n_shared && d->ffn_shared > d->ffn ? d->ffn_shared : d->ffn;
}
int up_row_tile(int kind, const moe_desc* d) {
  return kind == KIND_BF16_PREFILL ? prefill_rows(d) : streaming(kind) ? 16 : 32;
}
int up_col_tile(int kind, const moe_desc* d) {
  if (kind == KIND_MXFP4) return mx_lds(d, d->d) ? 16 * kMxUpWaves : 32;
  if (kind == KIND_MXFP8) return 16 * kMx8Waves;
  return kind == KIND_BF16_PREFILL ? 128 : streaming(kind) ? 16 : 32;
}
int down_row_tile(int kind, const moe_desc* d) {
  if (kind == KIND_BF16_PREFILL) return down_all_rows(d) ? 256 : prefill_rows(d);
  return streaming(kind) ? 16 : 32;
}
int down_col_tile(int kind, const moe_desc* d) {
  if (kind == KIND_MXFP4) return mx_lds(d, down_k(d)) ? 16 * kMxDownWaves : 32;
  if (kind == KIND_MXFP8) return 16 * kMx8Waves;
  return kind == KIND_BF16_PREFILL ? 256 : streaming(kind) ? 16 : 32;
}

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

static int validate(const moe_desc* d) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->T < 0 || d->d < 1 || d->E < 1 || d->k < 1 || d->ffn < 1) return MOE_ERR_INVALID_ARG;
  if (d->E > kMaxExperts || d->k > kMaxTopK || d->k > d->E) return MOE_ERR_INVALID_ARG;
  if (d->n_shared < 0 || d->n_shared > kMaxShared) return MOE_ERR_INVALID_ARG;
  if (d->n_shared > 0 && d->ffn_shared < 1) return MOE_ERR_INVALID_ARG;
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->y_dtype != MOE_F32 && d->y_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->path < MOE_PATH_AUTO || d->path > MOE_PATH_DECODE) return MOE_ERR_INVALID_ARG;
  if (d->scoring != MOE_SCORING_SOFTMAX && d->scoring != MOE_SCORING_SIGMOID)
    return MOE_ERR_INVALID_ARG;
  if (d->weighting != MOE_WEIGHTS_RENORM && d->weighting != MOE_WEIGHTS_RAW)
    return MOE_ERR_INVALID_ARG;
  if (d->expert_format != MOE_EXPERTS_DENSE && d->expert_format != MOE_EXPERTS_MXFP4 &&
      d->expert_format != MOE_EXPERTS_MXFP8)
    return MOE_ERR_INVALID_ARG;
  if (d->expert_format != MOE_EXPERTS_DENSE && d->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (d->flags & ~MOE_FLAG_MX_LINE_ROWS) return MOE_ERR_INVALID_ARG;
  if ((d->flags & MOE_FLAG_MX_LINE_ROWS) && d->expert_format == MOE_EXPERTS_DENSE)
    return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(d->capacity_factor) || d->capacity_factor < 0) return MOE_ERR_INVALID_ARG;
  const int64_t rows = d->T * (int64_t)(d->k + d->n_shared);
  if (rows + kRowSlack >= (int64_t(1) << 31)) return MOE_ERR_INVALID_ARG;
  const int q = d->dtype == MOE_BF16 ? 64 : 4;
  if (d->d % q || d->ffn % q) return MOE_ERR_UNSUPPORTED;
  if (d->n_shared > 0 && d->ffn_shared % q) return MOE_ERR_UNSUPPORTED;
  if (d->expert_format == MOE_EXPERTS_MXFP8 &&
      (d->d > kMx8MaxK || d->ffn > kMx8MaxK || (d->n_shared > 0 && d->ffn_shared > kMx8MaxK)))
    return MOE_ERR_UNSUPPORTED;
  // The bf16 GEMMs address x, h and each expert's weight matrix with 32-bit
  // byte offsets.
  if (d->dtype == MOE_BF16) {
    const int64_t ffn_max = d->n_shared > 0 ? std::max(d->ffn, d->ffn_shared) : d->ffn;
    const int64_t lim = int64_t(1) << 32;
    if (d->T * d->d * 2 >= lim || (rows + kRowSlack) * ffn_max * 2 >= lim ||
        ffn_max * d->d * 2 >= lim)
      return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int make_plan(const moe_desc* d, Plan* p) {
  int st = validate(d);
  if (st != MOE_OK) return st;
  Plan P{};
  P.desc = *d;
  const int64_t T = d->T;
  P.G = d->E + d->n_shared;
  P.pairs = T * d->k;
  P.R = T * (int64_t)(d->k + d->n_shared);
  P.nblk = cdiv(T, kRouterTokens);
  P.route_mode = (d->scoring == MOE_SCORING_SIGMOID ? kRouteSigmoid : 0) |
                 (d->weighting == MOE_WEIGHTS_RAW ? kRouteRaw : 0);
  // Expert capacity ceil(T*k/E * factor), in IEEE double in that order; no
  // expert receives more than T pairs, so larger capacities cut nothing.
  P.cap = INT_MAX;
  if (d->capacity_factor > 0) {
    const double c = std::ceil((double)(T * d->k) / (double)d->E * d->capacity_factor);
    P.cap = c < (double)T ? (int)c : INT_MAX;
  }
  // With few token blocks the router's K range is split over up to
  // kMaxRouterSplit workgroups per block (at least four 32-wide k-steps
  // each), up to about 256 workgroups.
  P.rsplit = 1;
  P.rwide = 0;
  if (d->dtype == MOE_BF16) {
    const int64_t nk = d->d / 32;
    if (kRouterWide > 0 && d->T >= 4 * kRouterWide && (int64_t)d->E * d->d >= kRouterWideMinWeights) {
      // many tokens, large router matrix: 64-token workgroups over K parts,
      // up to about 512 workgroups with at least 16 k-steps each
      P.rwide = kRouterWide;
      const int64_t groups = cdiv(d->T, kRouterWide);
      while (P.rsplit < kMaxRouterSplit && groups * P.rsplit * 2 <= 512 &&
             nk / (P.rsplit * 2) >= 16)
        P.rsplit *= 2;
    } else {
      while (P.rsplit < kMaxRouterSplit && P.nblk * P.rsplit * 2 <= 256 &&
             nk / (P.rsplit * 2) >= 4)
        P.rsplit *= 2;
    }
  }
  P.ffn_max = d->n_shared > 0 ? std::max(d->ffn, d->ffn_shared) : d->ffn;
  if (d->path == MOE_PATH_AUTO)
    P.path = (T * d->k <= 8LL * d->E) ? MOE_PATH_DECODE : MOE_PATH_PREFILL;
  else
    P.path = d->path;
  if (d->expert_format != MOE_EXPERTS_DENSE) P.path = MOE_PATH_DECODE;
  if (d->dtype == MOE_F32)
    P.kind = KIND_F32;
  else if (d->expert_format == MOE_EXPERTS_MXFP4)
    P.kind = KIND_MXFP4;
  else if (d->expert_format == MOE_EXPERTS_MXFP8)
    P.kind = KIND_MXFP8;
  else
    P.kind = P.path == MOE_PATH_DECODE ? KIND_BF16_DECODE : KIND_BF16_PREFILL;

  const int64_t nz = std::min<int64_t>(d->E, P.pairs);
  auto shape = [&](int bm, int bn, int ncols, int ncols_sh) {
    GemmShape s{};
    s.bm = bm;
    s.bn = bn;
    s.n_cols = ncols;
    s.n_cols_shared = d->n_shared > 0 ? ncols_sh : ncols;
    s.n_tiles = (int)cdiv(std::max(s.n_cols, s.n_cols_shared), bn);
    s.max_row_tiles = (P.pairs + nz * (bm - 1)) / bm + d->n_shared * cdiv(T, bm);
    s.max_tiles = s.max_row_tiles * s.n_tiles;
    return s;
  };
  P.up = shape(up_row_tile(P.kind, d), up_col_tile(P.kind, d), d->ffn, d->ffn_shared);
  P.down = shape(down_row_tile(P.kind, d), down_col_tile(P.kind, d), d->d, d->d);
  // The decode kernels walk a compact list of row tiles (see dispatch.hip),
  // column tile fastest: the workgroups that run together on one XCD share
  // the row tile's tokens through its L2 (each weight tile is read by one
  // workgroup only).  Measured on MI355X against row tile fastest:
  // gpt-oss-shaped bf16 layer T=128 1.049 -> 0.996 ms, T=32 -3%, T=8 -2%;
  // MX-format layers -1 to -3%.
  P.up.row_list = P.down.row_list = streaming(P.kind);
  P.up.all_rows = 0;
  P.down.all_rows = P.kind == KIND_BF16_PREFILL && down_all_rows(d);
  // Schedule order (measured on MI355X): both GEMMs run chunks of
  // consecutive entries per XCD; the up/gate GEMM with row tile fastest, the
  // down GEMM (long K, few column tiles) with column tile fastest.
  P.up.n_fastest = 0;
  P.up.xcd_remap = 1;
  P.down.n_fastest = 1;
  P.down.xcd_remap = 1;
  // A down GEMM of 128-row tiles with under three tiles per CU loses much of
  // its last round to idle CUs; when its K is long (>= 8192) splitting K in
  // two doubles the tiles at little per-tile cost (the combine adds the two
  // partial outputs in a fixed order).  Measured (on 256-row tiles, before
  // the last-round split below replaced it there): Mixtral-shaped T=4096
  // down 1.13 -> 1.08 ms; short-K layers got slower, so they keep one range.
  P.up.ksplit = 1;
  P.down.ksplit = 1;
  // A down GEMM of 256-row tiles with a long K (>= 8192) splits the tiles
  // of its last, partly filled round along K into pieces added by a fixup
  // kernel (sk_layout in experts.hip).  Measured on MI355X, Mixtral-shaped
  // T=4096: 560 whole tiles of 224 slabs (371 us each) in two full rounds,
  // then 48 tiles as 240 pieces of 45 slabs (88 us each); down GEMM plus
  // combine 0.961 -> 0.915 ms against the two-way K split of every tile
  // (whose combine added two partial buffers).  Each piece carries about
  // 20 us of fixed cost (prologue, a 256 KB float32 partial write and its
  // fixup read), so shorter reductions lost: the mid-size layer's 32- and
  // 16-slab tiles ran 14% and 29% slower split, and the up/gate GEMM gained
  // nothing.
  P.up.sk_cus = P.down.sk_cus = 0;
  const int k_down_max = std::max(d->ffn, d->n_shared ? d->ffn_shared : 0);
  if (P.kind == KIND_BF16_PREFILL && P.down.bm == 256 && k_down_max >= 8192)
    P.down.sk_cus = kCUs;
  if (P.kind == KIND_BF16_PREFILL && !P.down.sk_cus) {
    const int64_t est_tiles =
        (cdiv(P.pairs, P.down.bm) + std::min<int64_t>(d->E, P.pairs) / 2) * P.down.n_tiles;
    const int k_down = std::max(d->ffn, d->n_shared ? d->ffn_shared : 0);
    if (est_tiles < 3 * 256 && k_down >= 8192) P.down.ksplit = 2;
  }
  // Weight bursts of the 64- and 128-row prefill tiles skip the caches'
  // normal retention when experts average at most a quarter tile of rows:
  // nearly every weight tile is then read by one row tile only.  Measured on MI355X:
  // gpt-oss-shaped layer at T=512 (16 rows per expert) 1.175 -> 1.121 ms;
  // with many rows per expert (several row tiles re-reading each weight
  // tile, DeepSeek-V3-shaped T=4096) the same policy was 6% slower.
  P.up.stream_w = P.down.stream_w = 0;
  if (P.kind == KIND_BF16_PREFILL && P.up.bm <= 128 && P.pairs * 4 <= (int64_t)P.up.bm * d->E)
    P.up.stream_w = P.down.stream_w = 1;
  // MX code copies of the LDS-staged kernel go non-temporal for code rows on
  // whole lines with at most 8 (token, expert) pairs per expert on average
  // (each weight tile then read by about one 16-row tile; see experts.hip).
  if ((P.kind == KIND_MXFP4 || P.kind == KIND_MXFP8) && (d->flags & MOE_FLAG_MX_LINE_ROWS) &&
      P.pairs <= 8LL * d->E)
    P.up.stream_w = P.down.stream_w = 1;
  // A split down GEMM measured faster with its entries spread over all XCDs.
  if (P.down.ksplit > 1) P.down.xcd_remap = 0;

  const size_t A = 256;
  const size_t eb = d->dtype == MOE_BF16 ? 2 : 4;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + std::max<size_t>(bytes, 1), A);
    return at;
  };
  const size_t rows_ws = (size_t)P.R + kRowSlack;
  const size_t e_pad = (size_t)(d->E + 15) / 16 * 16;
  const size_t part_rows =
      P.rwide ? (size_t)cdiv(T, P.rwide) * P.rwide : (size_t)P.nblk * kRouterTokens;
  P.o_router_part = take(P.rsplit > 1 || P.rwide ? (size_t)P.rsplit * part_rows * e_pad * 4 : 0);
  P.o_blk_hist = take((size_t)P.nblk * d->E * 4);
  P.o_blk_rank = take((size_t)P.pairs * 4);
  P.o_counts = take((size_t)d->E * 4);
  P.o_offsets = take((size_t)(P.G + 1) * 4);
  P.o_tiles_up = take((size_t)(P.up.max_tiles + 1) * sizeof(Tile));
  P.o_tiles_down = take((size_t)(P.down.max_tiles + 1) * sizeof(Tile));
  P.o_sorted = take(rows_ws * 4);
  P.o_slot = take((size_t)P.pairs * 4);
  P.o_idx = take((size_t)P.pairs * 4);
  P.o_w = take((size_t)P.pairs * 4);
  P.o_h = take(rows_ws * (size_t)P.ffn_max * eb);
  P.o_out = take(rows_ws * (size_t)d->d * 4 * P.down.ksplit);
  // K-piece accumulators: at most kCUs pieces of one tile (BM x weight rows
  // of up/gate, BM x BN of down) in float32
  const size_t piece_up = (size_t)P.up.bm * 2 * P.up.bn * 4;
  const size_t piece_dn = (size_t)P.down.bm * P.down.bn * 4;
  P.o_part = take(P.up.sk_cus || P.down.sk_cus
                      ? (size_t)kCUs * std::max(P.up.sk_cus ? piece_up : 0, P.down.sk_cus ? piece_dn : 0)
                      : 0);
  P.total = o;
  *p = P;
  return MOE_OK;
}

}  // namespace moe

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: argument out of range";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape not supported by the kernels";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP runtime or launch error";
    case MOE_ERR_TOO_LARGE:
      return "MOE_ERR_TOO_LARGE: the layer needs more scratch than moe_forward_noalloc holds "
             "(MOE_NOALLOC_SCRATCH_BYTES); use moe_forward with a workspace";
    default: return "unknown moe_status";
  }
}

int moe_validate(const moe_desc* d) { return moe::validate(d); }

int moe_workspace_size(const moe_desc* d, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe::Plan p;
  int st = moe::make_plan(d, &p);
  if (st != MOE_OK) return st;
  *bytes = p.total;
  return MOE_OK;
}

int moe_resolve_path(const moe_desc* d) {
  moe::Plan p;
  int st = moe::make_plan(d, &p);
  return st != MOE_OK ? st : p.path;
}

int64_t moe_grouped_rows(const moe_desc* d) {
  moe::Plan p;
  int st = moe::make_plan(d, &p);
  return st != MOE_OK ? st : p.R;
}

}  // extern "C"
