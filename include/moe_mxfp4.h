/*
 * moe_mxfp4.h -- C ABI of libmoe_mxfp4.so: the routed mixture-of-experts layer
 * with MXFP4 expert weights, on one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (sources are web pages on the Deltafin project):
 *  - fp32 router logits l[t][e] = x[t] . Wr[e] (+ b[e]), with fp32 accumulation
 *    ("Tarfa EXACTNESS" page, opening list: fp32 logits, no reduced-precision
 *    accumulate; "Deltafin's custom compiled runtime", section "Complete target
 *    sequence tape": routing yields the top-16 ids in route order with fp32
 *    weights);
 *  - exact top-k: all k selected experts run, none dropped ("Deltafin's custom
 *    compiled runtime", section "Weight fidelity");
 *  - combine weights: softmax over the k selected logits;
 *  - MXFP4 expert weights decoded on the fly: a 4-bit E2M1 code per element
 *    through a 16-entry table, one E8M0 power-of-two scale per 32 elements
 *    along the reduction axis (brain.bigb.es "deltafin", section "The
 *    techniques that bought the 82x": fused MXFP4 dequant + GEMV);
 *  - the SwiGLU expert FFN y = Wd (silu(Wg x) * (Wu x)), activations fp32
 *    ("Deltafin's custom compiled runtime", section "Weight fidelity");
 *  - out[t] = sum_j w[t][j] * y[t][j], summed in rank order j (a fixed
 *    reduction order, after the same page's table of linked sources: batched
 *    expert phases with an ordered reduction).
 *
 * Conventions for every entry point
 *  - All functions are extern "C", never throw, and keep no state between
 *    calls.  They return MOE_OK (0) or a negative moe_status.
 *  - Every argument check runs on the host before anything is enqueued; on an
 *    error nothing is launched and no output is touched.
 *  - Device pointers are plain device addresses; the caller owns every buffer
 *    (the library never allocates, frees or keeps a pointer after returning).
 *    Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    may still run after the call returns: buffers must stay alive until the
 *    stream has passed it.  No entry point synchronises the host, reads device
 *    memory on the host, or allocates, so the forward path can be captured in
 *    a HIP graph.
 *  - Sizes use checked 64-bit arithmetic: an overflow is MOE_ERR_OVERFLOW.
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1u

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = -2,       /* a size is out of range or not a multiple of 32 */
    MOE_ERR_DTYPE = -3,       /* unknown activation dtype */
    MOE_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than moe_workspace_bytes() */
    MOE_ERR_LAYOUT = -6,      /* unknown weight layout id */
    MOE_ERR_UNSUPPORTED = -7, /* valid request outside what the kernels implement */
    MOE_ERR_OVERFLOW = -8,    /* a byte count does not fit in 64 bits / the index types */
    MOE_ERR_DEVICE = -9,      /* a HIP call or kernel launch failed */
    MOE_ERR_ABI = -10,        /* descriptor abi_version / struct_size mismatch */
    MOE_ERR_RANGE = -11       /* an index argument (expert, matrix) is out of range */
} moe_status;

typedef enum moe_dtype {
    MOE_DTYPE_F32 = 0,        /* fp32 activations */
    MOE_DTYPE_BF16 = 1        /* bf16 activations (widened exactly to fp32) */
} moe_dtype;

/* Device weight layout ids. */
#define MOE_LAYOUT_ROWMAJOR_V1 1u
/*
 * MOE_LAYOUT_ROWMAJOR_V1 -- per expert e (experts back to back, e = 0..E-1):
 *   codes  : gate [I][H/2] | up [I][H/2] | down [H][I/2]      (uint8, 3*I*H/2 bytes)
 *   scales : gate [I][H/32] | up [I][H/32] | down [H][I/32]   (uint8 E8M0, 3*I*H/32 bytes)
 * Matrices are [out_features][in_features] row-major.  Element c of a row is
 * the low nibble of byte c/2 when c is even, the high nibble when c is odd.
 * Scale byte [n][c/32] covers elements 32*(c/32) .. 32*(c/32)+31 of row n
 * (blocks run along the reduction axis).  The six tensors of one expert form
 * one contiguous range per buffer.  This is also the logical (interchange)
 * layout, so moe_mxfp4_pack is a validated device copy into it.
 */

typedef struct moe_layer_desc {
    uint32_t abi_version;  /* MOE_ABI_VERSION */
    uint32_t struct_size;  /* sizeof(moe_layer_desc) */
    int32_t hidden;        /* H: 32 <= H, H % 32 == 0 */
    int32_t inter;         /* I: 32 <= I, I % 32 == 0 */
    int32_t n_experts;     /* E >= 1 */
    int32_t top_k_max;     /* largest k used with this layer: 1 <= k <= min(E, 64) */
    uint32_t layout;       /* MOE_LAYOUT_ROWMAJOR_V1 */
    uint32_t reserved;     /* must be 0 */
} moe_layer_desc;

/* ABI version compiled into the library (MOE_ABI_VERSION). */
uint32_t moe_abi_version(void);

/* Static English text for a status code (never NULL). */
const char* moe_status_string(int status);

/* Validate a descriptor: MOE_OK, MOE_ERR_NULL, MOE_ERR_ABI, MOE_ERR_SHAPE,
 * MOE_ERR_LAYOUT or MOE_ERR_UNSUPPORTED (sizes beyond the kernels' limits:
 * H <= 8192, I <= 8192, E <= 4096). */
int moe_layer_check(const moe_layer_desc* desc);

/* Bytes of the device weight buffers of one layer (all E experts). */
int moe_mxfp4_packed_bytes(const moe_layer_desc* desc, size_t* codes_bytes, size_t* scales_bytes);

/* Bytes of device workspace moe_mxfp4_forward / moe_mxfp4_experts need for
 * n_tokens tokens and top-k.  The workspace holds logits, routes, the token ->
 * expert sort, the FFN intermediate and per-(token, rank) expert outputs; its
 * contents on entry do not matter. */
int moe_workspace_bytes(const moe_layer_desc* desc, int32_t n_tokens, int32_t k, size_t* bytes);

/*
 * Pack -- copy `expert_count` experts given back to back in the logical layout
 * (device buffers logical_codes / logical_scales) into the device layout
 * buffers packed_codes / packed_scales at experts expert_begin ..
 * expert_begin + expert_count - 1.  Identity on values.  Lets a caller upload
 * a layer in chunks.  All four pointers are device pointers, 16-byte aligned.
 */
int moe_mxfp4_pack(const moe_layer_desc* desc, const void* logical_codes, const void* logical_scales,
                   int64_t expert_begin, int64_t expert_count, void* packed_codes, void* packed_scales,
                   void* stream);

/*
 * The whole layer (router logits, top-k, softmax, token -> expert sort, expert
 * gate/up + SwiGLU, expert down, rank-ordered combine) for n_tokens tokens.
 *   x            [n_tokens][H], fp32 or bf16 (x_dtype), 16-byte aligned
 *   router_w     [E][H] fp32 row-major
 *   router_bias  [E] fp32 or NULL; added to the logits (moves selection and weights)
 *   packed_codes / packed_scales: the layer's device weights (moe_mxfp4_packed_bytes)
 *   1 <= n_tokens <= 2^20 (MOE_ERR_SHAPE otherwise); 1 <= k <= desc->top_k_max
 *   out          [n_tokens][H] fp32
 *   logits_out   [n_tokens][E] fp32, or NULL
 *   topk_idx_out [n_tokens][k] int32 in rank order (descending logit, ties to the
 *                lower expert id, NaN below every number), or NULL
 *   topk_w_out   [n_tokens][k] fp32 combine weights, or NULL
 *   workspace    device buffer of at least moe_workspace_bytes(desc, n_tokens, k)
 * Deterministic: the same inputs give bit-identical outputs on every call.
 */
int moe_mxfp4_forward(const moe_layer_desc* desc, const void* x, int32_t x_dtype,
                      const float* router_w, const float* router_bias, const void* packed_codes,
                      const void* packed_scales, int32_t n_tokens, int32_t k, float* out,
                      float* logits_out, int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * The expert part of the layer with the routing given: topk_idx [n_tokens][k] int32 (each row k
 * distinct expert ids in [0, E)) and topk_w [n_tokens][k] fp32.  Same output
 * and workspace contract as moe_mxfp4_forward.  Expert ids are not range
 * checked on the device beyond clamping; out-of-range ids give unspecified
 * output (never an out-of-bounds access).
 */
int moe_mxfp4_experts(const moe_layer_desc* desc, const void* x, int32_t x_dtype,
                      const int32_t* topk_idx, const float* topk_w, const void* packed_codes,
                      const void* packed_scales, int32_t n_tokens, int32_t k, float* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-form stages alone (the kernels moe_mxfp4_forward runs for one token),
 * for stage-level checks and timing.  A pair p = t*k + j is token t = p / k of
 * x with expert pair_expert[p] in [0, E).
 * gate/up: h [n_pairs][I] fp32, h[p][i] = silu(g) * u with g = Wg[i] . x[t],
 *     u = Wu[i] . x[t], silu(g) = g / (1 + exp(-g)).
 * down:    y [n_pairs][H] fp32, y[p][n] = Wd[n] . h[p].
 * combine: out[t][n] = (resid[t][n] +) sum_{j<k} w[t][j] * y[t*k+j][n], j ascending;
 *     resid may be NULL or alias out.
 * x has ceil(n_pairs / k) rows.  An expert id outside [0, E) is clamped into
 * it on the device.  Errors, all found before anything is enqueued:
 * MOE_ERR_NULL (a required pointer is NULL), MOE_ERR_DTYPE (x_dtype),
 * MOE_ERR_SHAPE (n_pairs below 1 or above 2^26; n_tokens below 1 or above
 * 2^20; k outside [1, top_k_max] for gate/up or [1, 64] for combine; hidden not
 * a positive multiple of 4), MOE_ERR_ALIGN (x, h, y, out, resid or the packed
 * buffers not 16-byte aligned; combine's w needs none), the descriptor's own
 * errors (moe_layer_check), and MOE_ERR_DEVICE when a launch fails.
 */
int moe_mxfp4_gate_up(const moe_layer_desc* desc, const void* x, int32_t x_dtype,
                      const int32_t* pair_expert, int32_t n_pairs, int32_t k, const void* packed_codes,
                      const void* packed_scales, float* h, void* stream);
int moe_mxfp4_down(const moe_layer_desc* desc, const float* h, const int32_t* pair_expert,
                   int32_t n_pairs, const void* packed_codes, const void* packed_scales, float* y,
                   void* stream);
int moe_combine(const float* y, const float* w, int32_t n_tokens, int32_t k, int32_t hidden,
                const float* resid, float* out, void* stream);

/* Router logits alone: logits [n_tokens][E] = x . router_w^T (+ bias), fp32 accumulation.
 * x [n_tokens][H] (x_dtype), router_w [E][H] fp32 row-major, router_bias [E] or NULL.
 * Errors: MOE_ERR_NULL, MOE_ERR_DTYPE, MOE_ERR_SHAPE (n_tokens outside [1, 2^20]),
 * MOE_ERR_ALIGN (x or router_w not 16-byte aligned), descriptor errors,
 * MOE_ERR_DEVICE. */
int moe_router_logits(const moe_layer_desc* desc, const void* x, int32_t x_dtype,
                      const float* router_w, const float* router_bias, int32_t n_tokens,
                      float* logits, void* stream);

/* Top-k + softmax alone, from given logits [n_tokens][n_experts]: idx [n_tokens][k] in
 * rank order and softmax weights w [n_tokens][k].  1 <= k <= min(E, 64),
 * E <= 4096.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (n_tokens outside [1, 2^20],
 * E below 1, k out of range), MOE_ERR_UNSUPPORTED (E above 4096), MOE_ERR_DEVICE. */
int moe_topk_softmax(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t k,
                     int32_t* idx, float* w, void* stream);

/* Token -> expert sort alone: stable counting sort of the (token, rank) pairs by expert
 * (the grouping the grouped expert GEMMs need; the pages do not describe it).
 *   topk_idx [n_tokens][k] int32: expert ids in [0, E) (an id outside is clamped into it)
 *   expert_offsets [E+1] int32: pairs of expert e are pair_list[offsets[e] .. offsets[e+1])
 *   pair_list [n_tokens*k] int32: pair id t*k + j, ordered by expert, then token, then rank
 *   workspace: device scratch of at least moe_sort_workspace_bytes(E, n_tokens, k)
 *     bytes, 16-byte aligned, owned by the caller and overwritten by the call.  The
 *     size is 0 below 1024 tokens (one workgroup sorts everything; workspace may then
 *     be NULL); from 1024 tokens the pairs are counted in blocks of 256 tokens and the
 *     workspace holds (blocks + 1) * E int32 counts.
 * Errors: MOE_ERR_NULL (idx, offsets or pair list NULL), MOE_ERR_SHAPE (n_tokens,
 * E or k out of range), MOE_ERR_UNSUPPORTED (E above 4096), MOE_ERR_OVERFLOW
 * (n_tokens * k above INT32_MAX), MOE_ERR_WORKSPACE (workspace NULL or too small
 * when the size is not 0), MOE_ERR_ALIGN (workspace not 16-byte aligned),
 * MOE_ERR_DEVICE. */
int moe_sort_workspace_bytes(int32_t n_experts, int32_t n_tokens, int32_t k, size_t* bytes);
int moe_sort_by_expert(const int32_t* topk_idx, int32_t n_tokens, int32_t n_experts, int32_t k,
                       int32_t* expert_offsets, int32_t* pair_list, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Prefill form, stage by stage: the kernels moe_mxfp4_forward runs for more
 * than one bf16 token when H and I are multiples of 256 (the grouped GEMMs on
 * bf16 MFMA), for stage-level checks and timing; the forward runs them over
 * batches of tokens small enough for the limits below.  Other shapes take the
 * decode-form kernels.  After moe_sort_by_expert:
 *  - moe_max_expert_blocks: capacity of the block list for n_pairs pairs,
 *    ceil(n_pairs / 128) + min(n_pairs, n_experts).
 *  - moe_expert_blocks: cut each expert's sorted pairs into blocks of at most
 *    128: blocks [max_blocks][4] int32 {expert, first index into pair_list,
 *    pair count, 0} (16-byte aligned), n_blocks [1] int32 on the device.
 *    max_blocks below the capacity is MOE_ERR_WORKSPACE.
 *  - moe_mxfp4_grouped_gate_up: x bf16 [n_tokens][H]; pair p = t*k + j reads
 *    token t = p / k.  hterm [2][n_tokens*k][I] bf16 receives h = silu(g) * u
 *    as two terms, hterm[0] = bf16(h) and hterm[1] = bf16(h - hterm[0]) (both
 *    round to nearest even), for every pair named by a block.
 *  - moe_mxfp4_grouped_down: y [n_pairs][H] fp32, y[p] = Wd . (hterm[0][p] +
 *    hterm[1][p]), for every pair named by a block.
 * Blocks that do not name a valid expert and pair range, and pair ids outside
 * [0, n_pairs), are skipped on the device.  MOE_ERR_UNSUPPORTED if H or I is
 * not a multiple of 256, x or hterm reaches 1 GiB, or y reaches 2 GiB.
 */
int moe_max_expert_blocks(int32_t n_experts, int32_t n_pairs, int32_t* max_blocks);
int moe_expert_blocks(const int32_t* expert_offsets, int32_t n_experts, int32_t n_pairs, int32_t* blocks,
                      int32_t max_blocks, int32_t* n_blocks, void* stream);
int moe_mxfp4_grouped_gate_up(const moe_layer_desc* desc, const void* x, int32_t n_tokens, int32_t k,
                              const int32_t* pair_list, const int32_t* blocks, const int32_t* n_blocks,
                              int32_t max_blocks, const void* packed_codes, const void* packed_scales, void* hterm,
                              void* stream);
int moe_mxfp4_grouped_down(const moe_layer_desc* desc, const void* hterm, int32_t n_pairs, const int32_t* pair_list,
                           const int32_t* blocks, const int32_t* n_blocks, int32_t max_blocks,
                           const void* packed_codes, const void* packed_scales, float* y, void* stream);

/* Dequantisation alone: dequantise one matrix of one expert from the device layout to
 * fp32, exactly: out = E2M1(code) * 2^(scale - 127), subnormals kept, +-inf on
 * overflow, scale byte 0xFF -> NaN 0x7FC00000.  matrix 0 = gate [I][H],
 * 1 = up [I][H], 2 = down [H][I].  out holds rows x cols fp32.  Errors: MOE_ERR_NULL,
 * MOE_ERR_RANGE (expert outside [0, E) or matrix outside 0..2), MOE_ERR_ALIGN (a buffer
 * not 16-byte aligned), descriptor errors, MOE_ERR_DEVICE. */
int moe_mxfp4_dequant(const moe_layer_desc* desc, const void* packed_codes, const void* packed_scales,
                      int64_t expert, int32_t matrix, float* out, void* stream);

/* RMSNorm with gain, n = r / sqrt(mean(r^2) + eps) * gamma, per token.
 * r, n: [n_tokens][hidden] fp32; gamma [hidden] fp32; hidden % 4 == 0.  Errors:
 * MOE_ERR_NULL, MOE_ERR_SHAPE (n_tokens outside [1, 2^20], hidden not a positive
 * multiple of 4), MOE_ERR_ALIGN (r, gamma or n_out not 16-byte aligned), MOE_ERR_DEVICE. */
int moe_rmsnorm(const float* r, const float* gamma, float eps, int32_t n_tokens, int32_t hidden,
                float* n_out, void* stream);

/* Residual add: r[i] += d[i] for i < n (fp32); n = 0 enqueues nothing.  Errors:
 * MOE_ERR_NULL, MOE_ERR_SHAPE (n negative), MOE_ERR_DEVICE. */
int moe_residual_add(float* r, const float* d, int64_t n, void* stream);

/*
 * Stack -- a stack of n_layers pre-norm MoE layers on one residual stream:
 *   r = upcast(x); for each layer l: r = r + MoE_l(RMSNorm_l(r))
 * Host arrays of n_layers device pointers give each layer's packed codes,
 * packed scales, router weights (and optional biases, NULL array or NULL
 * entries = none) and RMSNorm gains.  residual [n_tokens][H] fp32 receives
 * the result (it may alias nothing else).  Workspace: moe_stack_workspace_bytes.
 * Everything is enqueued on `stream`; the sequence is capture-safe.
 */
int moe_stack_workspace_bytes(const moe_layer_desc* desc, int32_t n_tokens, int32_t k, size_t* bytes);
int moe_mxfp4_stack_forward(const moe_layer_desc* desc, int32_t n_layers,
                            const void* const* packed_codes, const void* const* packed_scales,
                            const float* const* router_w, const float* const* router_bias,
                            const float* const* gamma, float eps, const void* x, int32_t x_dtype,
                            int32_t n_tokens, int32_t k, float* residual, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Stack, graph form: capture moe_mxfp4_stack_forward once into a HIP graph and
 * replay it.  The graph binds the pointers given at creation; a replay
 * recomputes the stack from the current contents of x and the weights.
 * moe_stack_graph_create returns an opaque handle in *graph (free it with
 * moe_stack_graph_destroy); launch enqueues one replay on `stream`.
 */
typedef struct moe_stack_graph moe_stack_graph;
int moe_stack_graph_create(const moe_layer_desc* desc, int32_t n_layers,
                           const void* const* packed_codes, const void* const* packed_scales,
                           const float* const* router_w, const float* const* router_bias,
                           const float* const* gamma, float eps, const void* x, int32_t x_dtype,
                           int32_t n_tokens, int32_t k, float* residual, void* workspace,
                           size_t workspace_bytes, void* stream, moe_stack_graph** graph);
int moe_stack_graph_launch(moe_stack_graph* graph, void* stream);
int moe_stack_graph_destroy(moe_stack_graph* graph);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
