/*
 * moe.h -- C ABI of a single-GPU (MI355X, gfx950) sparse top-k Mixture-of-Experts
 * layer forward pass.
 *
 * The layer (page "Mixture of Experts Explained: Routers, Active Parameters and
 * VRAM", the five numbered routing steps; page "Mixture of Experts (MoE):
 * routing, expert parallelism, and memory", sections "How does MoE routing
 * work" and "Shared experts"):
 *
 *   logits[t,e] = sum_c x[t,c] * w_router[e,c] + router_bias[e]
 *   p[t,:]      = softmax(logits[t,:])                 over all E experts
 *   idx[t,0..k) = the k largest logits, descending, exact ties -> lower e
 *   w[t,j]      = p[t,idx[t,j]] / sum_j' p[t,idx[t,j']]   (renormalised)
 *   FFN_e(v)    = (SiLU(v W_gate[e]^T) * (v W_up[e]^T)) W_down[e]^T   (SwiGLU)
 *   y[t]        = sum_{j<k} w[t,j] * FFN_{idx[t,j]}(x[t]) + sum_s FFN_shared_s(x[t])
 *
 * Tokens are grouped by expert before the expert multiplies (page "Mixture of
 * experts: how MoE works and what it costs", section "What mixture of experts
 * costs in compute"; page "Mixture of Experts: why a model with 671 billion
 * parameters uses only 37", the router section's per-expert loop); by
 * default every (token, slot) pair is computed, none is dropped.
 *
 * Router options of the descriptor (the defaults, all zero, give the layer
 * above):
 *  - scoring = MOE_SCORING_SIGMOID (page "Mixture of Experts: why a model
 *    with 671 billion parameters uses only 37", sections "How many experts to
 *    pick and how to score them: top-k, softmax, sigmoid" and "The problem
 *    learned routing brings: load balancing"; page "Mixture of experts: how
 *    MoE works and what it costs", "Why load balancing is the hard part of
 *    MoE"): s[t,e] = sigmoid(x[t] . w_router[e]) per expert; the router bias
 *    only steers the choice, idx = the k largest s[t,e] + router_bias[e]
 *    (ties -> lower e), and w[t,j] = s[t,idx[t,j]] / sum_j' s[t,idx[t,j']].
 *  - weighting = MOE_WEIGHTS_RAW (page "Mixture of Experts Explained...",
 *    "Why top-1 routing cannot renormalise"): w[t,j] is the kept score as it
 *    is, p[t,idx[t,j]] (softmax over all E) or s[t,idx[t,j]], not divided by
 *    the kept sum.
 *  - capacity_factor > 0 (page "Mixture of Experts: why a model with 671
 *    billion parameters uses only 37", "Capacity factor: when tokens don't
 *    fit"; page "Mixture of Experts Explained...", the capacity passage in
 *    "Noise and the second expert"): each expert takes at most
 *    C = ceil(T*k/E * capacity_factor) pairs (evaluated in that order in IEEE
 *    double), the first C that chose it in pair order t*k+j.  A later pair is
 *    dropped: its term is missing from y and its slot_row is -1.
 *  - expert_format = MOE_EXPERTS_MXFP4 (page "Mixture of Experts: why a model
 *    with 671 billion parameters uses only 37", "What to do about it in
 *    practice"; page "Mixture of experts: how MoE works and what it costs",
 *    "What mixture of experts costs in memory"): the routed and shared expert
 *    weights are MXFP4 (the OCP Microscaling format: blocks of 32 elements
 *    along K share an E8M0 scale 2^(S-127); elements are FP4 E2M1 codes, two
 *    per byte, element 2i in the low nibble).  x, the router and y keep their
 *    types; products use the exactly dequantised weights.  Such a layer is
 *    run with moe_forward_mx, which also takes the scale arrays; it always
 *    uses the streaming (decode) expert kernels, whatever `path` says.
 *  - expert_format = MOE_EXPERTS_MXFP8 (page "Mixture of experts: how MoE
 *    works and what it costs", "What mixture of experts costs in memory":
 *    8-bit expert weights): the same MX blocking with FP8 E4M3 elements
 *    (bias 7, no infinity, 0x7F/0xFF NaN), one per byte.  d and ffn (and
 *    ffn_shared) at most 8192 (MOE_ERR_UNSUPPORTED otherwise).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller, row-major
 *    and contiguous, 16-byte aligned.  The library never allocates or frees
 *    memory; scratch comes from the caller's workspace.
 *  - Storage types: `dtype` of the descriptor applies to x and every weight
 *    (MOE_BF16: bfloat16 bit patterns; MOE_F32: IEEE float).  Router bias,
 *    routing weights and expert outputs are float32.  MOE_BF16 computes with
 *    bf16 products and float32 accumulation; MOE_F32 computes in float32.
 *  - Arguments are validated on the host, synchronously, before any launch;
 *    a failed check returns a negative moe_status and launches nothing.
 *  - GPU work is enqueued asynchronously on `stream` (a hipStream_t; NULL is
 *    the default stream); outputs are valid once the stream has reached it.
 *    A launch error returns MOE_ERR_HIP.
 *  - T == 0 returns MOE_OK once the descriptor is valid, without reading any
 *    pointer (workspace included) or launching anything.
 *  - Calls that share a workspace must be ordered on one stream.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 5

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a size, pointer or enum is out of range        */
  MOE_ERR_UNSUPPORTED = -2, /* valid layer, but a shape the kernels reject    */
  MOE_ERR_WORKSPACE = -3,   /* workspace pointer NULL or smaller than needed  */
  MOE_ERR_HIP = -4,         /* a HIP call or kernel launch failed             */
  MOE_ERR_TOO_LARGE = -5    /* moe_forward_noalloc: the layer needs more
                               scratch than MOE_NOALLOC_SCRATCH_BYTES         */
} moe_status;

/* Which expert-GEMM kernels run.  AUTO picks DECODE when the mean number of
 * rows per routed expert, T*k/E, is at most 8, else PREFILL.  MOE_F32 layers
 * always use their float32 kernels. */
typedef enum moe_path { MOE_PATH_AUTO = 0, MOE_PATH_PREFILL = 1, MOE_PATH_DECODE = 2 } moe_path;

/* Router scores (see the options above). */
typedef enum moe_scoring { MOE_SCORING_SOFTMAX = 0, MOE_SCORING_SIGMOID = 1 } moe_scoring;

/* Routing weights: kept scores renormalised over the kept set, or raw. */
typedef enum moe_weighting { MOE_WEIGHTS_RENORM = 0, MOE_WEIGHTS_RAW = 1 } moe_weighting;

/* Storage of the expert weights: `dtype`, MXFP4 or MXFP8 (see the options above). */
typedef enum moe_expert_format {
  MOE_EXPERTS_DENSE = 0,
  MOE_EXPERTS_MXFP4 = 1,
  MOE_EXPERTS_MXFP8 = 2
} moe_expert_format;

/*
 * moe_desc.flags bits.
 * MOE_FLAG_MX_LINE_ROWS (MXFP4 or MXFP8 experts only; MOE_ERR_INVALID_ARG
 * with dense experts): every row of every code array (one weight row of K
 * codes) starts on a 128-byte line, i.e. occupies ceil(K*bits/8 / 128) * 128
 * bytes, its codes first; the bytes after them are never read.  Scale arrays
 * keep their packed layout.  Results are identical to the packed layout's.
 * It serves callers that can store the weights that way: whole-line rows
 * let the expert kernels copy each row's codes without the second, partly
 * used line that a row starting mid-line costs (the gpt-oss-shaped layer's
 * 1440-byte MXFP4 rows: 4.5-7% faster).
 */
#define MOE_FLAG_MX_LINE_ROWS 1

typedef struct moe_desc {
  int64_t T;          /* tokens, >= 0                                        */
  int32_t d;          /* hidden size                                         */
  int32_t E;          /* routed experts, 1..512                              */
  int32_t k;          /* experts per token, 1..min(E,32)                     */
  int32_t ffn;        /* routed expert FFN width                             */
  int32_t n_shared;   /* always-on shared experts, 0..8                      */
  int32_t ffn_shared; /* their FFN width (ignored when n_shared == 0)        */
  int32_t dtype;      /* moe_dtype of x and all weights                      */
  int32_t y_dtype;    /* moe_dtype of y                                      */
  int32_t path;       /* moe_path                                            */
  int32_t scoring;    /* moe_scoring                                         */
  int32_t weighting;  /* moe_weighting                                       */
  int32_t expert_format; /* moe_expert_format                                */
  int32_t flags;      /* MOE_FLAG_* bits (0: none)                           */
  double capacity_factor; /* 0: dropless; > 0: expert capacity (see above)   */
} moe_desc;

/* Stream handle: a hipStream_t passed as an opaque pointer. */
typedef void* moe_stream;

/* ABI version of the loaded library (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static text for a moe_status value. */
const char* moe_status_str(int status);

/* Host-only check of a descriptor: MOE_OK, MOE_ERR_INVALID_ARG (T<0, d/E/k/
 * ffn < 1, k > E, E > 512, k > 32, n_shared outside 0..8, ffn_shared < 1 with
 * n_shared > 0, bad enum, unknown flags or MOE_FLAG_MX_LINE_ROWS with dense
 * experts, capacity_factor negative or not finite,
 * MXFP4 or MXFP8 experts with dtype MOE_F32, T*(k+n_shared) >= 2^31) or
 * MOE_ERR_UNSUPPORTED (MOE_BF16 with d, ffn or ffn_shared not a multiple of
 * 64, or with x (T*d), h ((T*(k+n_shared)+256)*max ffn) or one expert's
 * weight matrix (max ffn * d) reaching 4 GiB, as the bf16 kernels address
 * them with 32-bit byte offsets; MOE_F32 with d, ffn or ffn_shared not a
 * multiple of 4). */
int moe_validate(const moe_desc* desc);

/* Bytes of workspace every entry point below needs for `desc` (host only). */
int moe_workspace_size(const moe_desc* desc, size_t* bytes);

/* The path AUTO resolves to for `desc` (host only; returns a moe_path, or a
 * negative moe_status if the descriptor is invalid). */
int moe_resolve_path(const moe_desc* desc);

/* Rows of the grouped (permuted) layout: T*k routed rows followed by
 * T*n_shared shared rows (host only; negative moe_status if invalid). */
int64_t moe_grouped_rows(const moe_desc* desc);

/*
 * Whole layer forward (all steps below, in order, on one stream).
 *   x            [T,d]            dtype
 *   w_router     [E,d]            dtype
 *   router_bias  [E]              float32, or NULL for none
 *   w_up, w_gate [E,ffn,d]        dtype  (stacked per expert, K-contiguous)
 *   w_down       [E,d,ffn]        dtype
 *   ws_up, ws_gate [n_shared,ffn_shared,d], ws_down [n_shared,d,ffn_shared];
 *                NULL when n_shared == 0 (required otherwise)
 *   y            [T,d]            y_dtype (output)
 *   topk_idx     [T,k] int32      optional output (NULL: kept in workspace)
 *   topk_w       [T,k] float32    optional output
 *   expert_counts [E] int32       optional output: (token, slot) pairs routed to
 *                                 each expert (before any capacity cut)
 *   workspace    >= moe_workspace_size(desc) bytes, 256-byte aligned
 * x, w_router and the expert weight arrays are 16-byte aligned (the kernels
 * read them in 16-byte chunks; MOE_ERR_INVALID_ARG otherwise).
 * A layer with MXFP4 or MXFP8 experts needs moe_forward_mx (MOE_ERR_INVALID_ARG
 * here).
 */
int moe_forward(const moe_desc* desc, const void* x, const void* w_router,
                const float* router_bias, const void* w_up, const void* w_gate,
                const void* w_down, const void* ws_up, const void* ws_gate,
                const void* ws_down, void* y, int32_t* topk_idx, float* topk_w,
                int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                moe_stream stream);

/* Scratch held inside the library for moe_forward_noalloc: 64 MiB per GPU. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * moe_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments and results are those of moe_forward without the workspace; the
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine).  Scratch is a device array of MOE_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; the first call on a
 * device looks up that device's copy.  Limit: a layer whose
 * moe_workspace_size exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 * MOE_ERR_TOO_LARGE before any launch.  Decode-sized layers fit, e.g.
 * d=2880, 128 experts, top-4, ffn 2880 at T=512 (40 MiB); d=4096, 8 experts,
 * top-2, ffn 14336 at T=256 (45 MiB); d=7168, 256 experts, top-8, ffn 2048
 * and one shared expert at T=128 (49 MiB).
 * Every call on one GPU uses that GPU's one array and leaves its contents
 * behind (no kernel reads scratch it has not written in the same call):
 * calls that overlap on one GPU (on different streams, or from host threads
 * without ordering) race and give undefined results; order them on one
 * stream.  MOE_ERR_HIP if the device array cannot be looked up.
 */
int moe_forward_noalloc(const moe_desc* desc, const void* x, const void* w_router,
                        const float* router_bias, const void* w_up, const void* w_gate,
                        const void* w_down, const void* ws_up, const void* ws_gate,
                        const void* ws_down, void* y, int32_t* topk_idx, float* topk_w,
                        int32_t* expert_counts, moe_stream stream);

/* Scale arrays of MXFP4 or MXFP8 expert weights (uint8 E8M0, one per 32 elements
 * along K): up, gate [E,ffn,d/32], down [E,d,ffn/32]; shared-expert
 * counterparts [n_shared,...] or NULL when n_shared == 0. */
typedef struct moe_mx_scales {
  const void* up;
  const void* gate;
  const void* down;
  const void* s_up;
  const void* s_gate;
  const void* s_down;
} moe_mx_scales;

/*
 * moe_forward for a layer with expert_format MOE_EXPERTS_MXFP4: w_up, w_gate
 * [E,ffn,d/2], w_down [E,d,ffn/2] (and the shared counterparts) hold the
 * packed E2M1 codes, `scales` their E8M0 scales (16-byte aligned like the
 * codes).  With MOE_EXPERTS_MXFP8 the code arrays hold one E4M3 byte per
 * element: w_up, w_gate [E,ffn,d], w_down [E,d,ffn].  With
 * MOE_FLAG_MX_LINE_ROWS in desc->flags the last dimension of every code
 * array is rounded up to a multiple of 128 bytes (rows on whole lines).  Every other argument
 * is as for moe_forward.  `events` is NULL or points to 6 hipEvents recorded as in
 * moe_forward_timed.  Scale bytes 0 (2^-127) and 255 (NaN) follow the format
 * but results that leave bfloat16's normal range are not defined.
 */
int moe_forward_mx(const moe_desc* desc, const void* x, const void* w_router,
                   const float* router_bias, const void* w_up, const void* w_gate,
                   const void* w_down, const void* ws_up, const void* ws_gate,
                   const void* ws_down, const moe_mx_scales* scales, void* y,
                   int32_t* topk_idx, float* topk_w, int32_t* expert_counts, void* workspace,
                   size_t workspace_bytes, moe_stream stream, void* const* events);

/*
 * moe_forward with timing marks: the same launches on the same stream, with
 * events[i] (a hipEvent_t, or NULL to skip) recorded on `stream` before the
 * router (0), dispatch (1), up/gate GEMM (2), down GEMM (3) and combine (4)
 * kernels, and events[5] after the combine.  `events` points to 6 entries.
 * For measuring each step's duration on the launch stream.
 */
int moe_forward_timed(const moe_desc* desc, const void* x, const void* w_router,
                      const float* router_bias, const void* w_up, const void* w_gate,
                      const void* w_down, const void* ws_up, const void* ws_gate,
                      const void* ws_down, void* y, int32_t* topk_idx, float* topk_w,
                      int32_t* expert_counts, void* workspace, size_t workspace_bytes,
                      moe_stream stream, void* const* events);

/*
 * Step 1-3: router logits, softmax, top-k and renormalisation (page "Mixture
 * of Experts Explained...", steps Score, Normalise, Keep the top k,
 * Renormalise), or the scoring / weighting options of the descriptor.
 * Logits are accumulated in float32; selection compares float32 keys (the
 * logits, or sigmoid scores plus bias), ties to the lower index.
 *   topk_idx [T,k] int32 (required), topk_w [T,k] float32 (required).
 * x and w_router are 16-byte aligned (MOE_ERR_INVALID_ARG otherwise).
 */
int moe_route(const moe_desc* desc, const void* x, const void* w_router,
              const float* router_bias, int32_t* topk_idx, float* topk_w,
              void* workspace, size_t workspace_bytes, moe_stream stream);

/*
 * Step 4: histogram, prefix scan and permutation that group the (token, slot)
 * pairs by expert.  Outputs (all required):
 *   expert_counts [E]        pairs routed to each expert
 *   group_offsets [E+n_shared+1]  first grouped row of each group: routed
 *                 experts 0..E-1 in order, then shared experts; the last entry
 *                 is the row count, T*(k+n_shared) less any dropped pairs
 *   sorted_token  [T*(k+n_shared)] token of each grouped row; within a routed
 *                 group rows follow increasing t*k+j (a stable grouping);
 *                 shared group s holds tokens 0..T-1 in order; entries past
 *                 the row count are not written
 *   slot_row      [T,k]      grouped row of pair (t,j), or -1 when a capacity
 *                 cut dropped the pair
 * With a capacity factor, expert e's group holds min(expert_counts[e], C)
 * rows.
 */
int moe_dispatch(const moe_desc* desc, const int32_t* topk_idx, int32_t* expert_counts,
                 int32_t* group_offsets, int32_t* sorted_token, int32_t* slot_row,
                 void* workspace, size_t workspace_bytes, moe_stream stream);

/*
 * Steps 5-6: grouped expert FFNs over the grouped rows (SwiGLU up/gate, then
 * down).  For grouped row r of group g with token t = sorted_token[r]:
 *   expert_out[r,:] = FFN_g(x[t,:])       float32 [T*(k+n_shared), d]
 * group_offsets / sorted_token as produced by moe_dispatch.  Dense expert
 * weights only (MOE_ERR_INVALID_ARG for MXFP4 or MXFP8).  x and the weight arrays are
 * 16-byte aligned (MOE_ERR_INVALID_ARG otherwise).
 */
int moe_experts(const moe_desc* desc, const void* x, const void* w_up, const void* w_gate,
                const void* w_down, const void* ws_up, const void* ws_gate,
                const void* ws_down, const int32_t* group_offsets,
                const int32_t* sorted_token, float* expert_out, void* workspace,
                size_t workspace_bytes, moe_stream stream);

/*
 * Step 7: weighted combine (page "Mixture of Experts Explained...", step Run
 * and combine; page "Mixture of Experts (MoE)...", "Shared experts"):
 *   y[t,:] = sum_{j<k} topk_w[t,j] * expert_out[slot_row[t,j],:]
 *            + sum_s expert_out[group_offsets[E+s] + t, :]
 * summed in that order, in float32, then stored as y_dtype.  A pair with
 * slot_row -1 (dropped) adds nothing.
 */
int moe_combine(const moe_desc* desc, const float* expert_out, const float* topk_w,
                const int32_t* slot_row, const int32_t* group_offsets, void* y,
                moe_stream stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
