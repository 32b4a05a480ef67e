// Host-side plan of one layer call: validation, path choice, tile shapes and
// the workspace layout.  Plain C++ (no HIP) so it can be built and checked on
// a machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "moe.h"

namespace moe {

// Tokens per router workgroup (one block of the per-block histogram).
constexpr int kRouterTokens = 16;
// Most workgroups sharing one router block's K range.
constexpr int kMaxRouterSplit = 16;
// Wide router form (tokens per workgroup; 0 disables it), used from 4 such
// groups of tokens and this many router weights (E * d) up.
constexpr int kRouterWide = 64;
constexpr int64_t kRouterWideMinWeights = 1 << 19;
// Largest supported expert count / top-k / shared experts.
constexpr int kMaxExperts = 512;
constexpr int kMaxTopK = 32;
constexpr int kMaxShared = 8;
// Compute units of an MI355X (gfx950): the workgroup slots of one round of
// one-workgroup-per-CU GEMM tiles.
constexpr int kCUs = 256;
// Rows of slack after the grouped rows so tile loads past the end stay in bounds.
constexpr int kRowSlack = 256;
// Router option bits: sigmoid scores with a selection-only bias; raw weights.
constexpr int kRouteSigmoid = 1, kRouteRaw = 2;
// MXFP4 experts: the LDS-staged kernel takes reductions up to this long, in
// tiles of 16 x 16 W features (W waves: kMxUpWaves for up/gate,
// kMxDownWaves for down); the direct-load kernel takes 16 x 32 tiles.
constexpr int kMxLdsMaxK = 3072;
constexpr int kMxUpWaves = 8, kMxDownWaves = 4;
// MXFP8 experts: always the LDS-staged kernel, 4 waves (16 x 64 tiles), K
// up to kMx8MaxK.
constexpr int kMx8Waves = 4, kMx8MaxK = 8192;

// One GEMM tile: rows [m0, m_end) of group g, output columns [n0, n0 + BN).
// Entry 0 of a schedule is a header: {entries, row tiles, column tiles, 0}.
struct Tile {
  int32_t g, m0, m_end, n0;
};

// Shape of one grouped-GEMM launch.
struct GemmShape {
  int bm;      // rows (tokens) per tile
  int bn;      // output columns per tile
  int n_cols;  // output columns of a routed group (ffn for up/gate, d for down)
  int n_cols_shared;
  int n_tiles;            // column tiles of the widest group
  int64_t max_row_tiles;  // upper bound of row tiles over all groups
  int64_t max_tiles;      // upper bound of (row tile, column tile) pairs
  bool row_list;          // schedule lists row tiles only (column tile = L % column tiles)
  int n_fastest;          // within a schedule chunk: 0 = row tile fastest, 1 = column
  int xcd_remap;          // consecutive schedule entries on one XCD (1) or spread (0)
  int ksplit;             // K ranges per tile in moe_forward (down GEMM only)
  int stream_w;           // weight bursts non-temporal (prefill kernels, 64- and 128-row
                          // tiles; MX LDS-staged kernel with line-row codes)
  int sk_cus;             // last-round split over this many workgroup slots (0: off)
  int all_rows;           // 256-row tiles whose waves each span all rows (prefill)
};

struct Plan {
  moe_desc desc;
  int path;          // resolved moe_path
  int G;             // groups = E + n_shared
  int64_t R;         // grouped rows = T*(k+n_shared)
  int64_t pairs;     // T*k
  int64_t nblk;      // router blocks
  int rsplit;        // router workgroups per block (split K; 1 = one kernel)
  int rwide;         // tokens per router workgroup of the wide split form (0: not used)
  int route_mode;    // kRouteSigmoid / kRouteRaw bits of the router options
  int cap;           // expert capacity in pairs (INT_MAX: no cut)
  int ffn_max;       // max(ffn, ffn_shared)
  int kind;          // kernel family, see KernelKind
  GemmShape up, down;
  // workspace byte offsets
  size_t o_router_part, o_blk_hist, o_blk_rank, o_counts, o_offsets, o_tiles_up, o_tiles_down, o_sorted,
      o_slot, o_idx, o_w, o_h, o_out, o_part, total;
};

enum KernelKind {
  KIND_F32 = 0,
  KIND_BF16_PREFILL = 1,
  KIND_BF16_DECODE = 2,
  KIND_MXFP4 = 3,
  KIND_MXFP8 = 4
};

// Fill `p` for `d`; returns a moe_status.
int make_plan(const moe_desc* d, Plan* p);

// Tile shapes of the grouped GEMMs per kernel family.
int up_row_tile(int kind, const moe_desc* d);
int up_col_tile(int kind, const moe_desc* d);
int down_row_tile(int kind, const moe_desc* d);
int down_col_tile(int kind, const moe_desc* d);

}  // namespace moe
