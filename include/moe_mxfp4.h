/*
 * moe_mxfp4.h -- C ABI of libmoe_mxfp4.so: the routed mixture-of-experts layer
 * with MXFP4 expert weights, on one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (sources are web pages on the Deltafin project; each
 * entry point below names the passage that defines it, or says that the pages
 * do not describe it):
 *  - fp32 router logits l[t][e] = x[t] . Wr[e] (+ b[e]), with fp32 accumulation
 *    ("Tarfa EXACTNESS" page, opening list: fp32 logits, no reduced-precision
 *    accumulate; "Deltafin's custom compiled runtime", section "Complete target
 *    sequence tape": routing yields the top-16 ids in route order with fp32
 *    weights);
 *  - exact top-k: all k selected experts run, none dropped ("Deltafin's custom
 *    compiled runtime", section "Weight fidelity");
 *  - combine weights: softmax over the k selected logits (not on the pages;
 *    the tiny one-layer workload this library is measured on states it);
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
 * Conventions for every entry point ("Deltafin's custom compiled runtime": a
 * small versioned C ABI, opening paragraph; descriptor-driven calls, section
 * "Coarse provider binding"; explicit unsupported requests fail early, section
 * "Configuration and device selection"; lengths and offsets in checked
 * arithmetic, section "Model contract and pack authentication")
 *  - All functions are extern "C", never throw, and return MOE_OK (0) or a
 *    negative moe_status.  Apart from the objects they create and destroy
 *    explicitly (the stack graph, the expert residency cache), they keep no
 *    state between calls, and only those object constructors allocate.
 *  - Every argument check runs on the host before anything is enqueued; on an
 *    error nothing is launched and no output is touched.
 *  - Device pointers are plain device addresses; the caller owns every buffer
 *    (the library never allocates, frees or keeps a pointer after returning).
 *    Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *    may still run after the call returns: buffers must stay alive until the
 *    stream has passed it (the borrower's side of the same page's rule that no
 *    pointer is lent to an asynchronous operation that can outlive its
 *    allocation, section "Coarse provider binding").  No entry point
 *    synchronises the host, reads device memory on the host, or allocates, so
 *    the forward path can be captured in a HIP graph.
 *  - Sizes use checked 64-bit arithmetic: an overflow is MOE_ERR_OVERFLOW.
 *  - moe_status and moe_dtype are C enums (the size of an int), so a caller
 *    may also pass and receive them as int.
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
    MOE_ERR_RANGE = -11,      /* an index argument (expert, matrix) is out of range */
    MOE_ERR_SCRATCH_LIMIT = -12, /* moe_mxfp4_forward_noalloc: the call needs more than its static scratch */
    MOE_ERR_POISONED = -13,   /* the residency cache failed terminally earlier and refuses further work */
    MOE_ERR_STATE = -14,      /* a call out of order (a second plan before finish, finish without a plan) */
    MOE_ERR_IO = -15          /* a trace file operation failed, or the trace reached its size limit */
} moe_status;

typedef enum moe_dtype {
    MOE_DTYPE_F32 = 0,        /* fp32 activations */
    MOE_DTYPE_BF16 = 1        /* bf16 activations (widened exactly to fp32) */
} moe_dtype;

/* Device weight layout ids. */
#define MOE_LAYOUT_ROWMAJOR_V1 1u
#define MOE_LAYOUT_SCALE4_V1 2u
/*
 * MOE_LAYOUT_ROWMAJOR_V1 -- per expert e (experts back to back, e = 0..E-1):
 *   codes  : gate [I][H/2] | up [I][H/2] | down [H][I/2]      (uint8, 3*I*H/2 bytes)
 *   scales : gate [I][H/32] | up [I][H/32] | down [H][I/32]   (uint8 E8M0, 3*I*H/32 bytes)
 * Matrices are [out_features][in_features] row-major.  Element c of a row is
 * the low nibble of byte c/2 when c is even, the high nibble when c is odd.
 * Scale byte [n][c/32] covers elements 32*(c/32) .. 32*(c/32)+31 of row n
 * (blocks run along the reduction axis).  The six tensors of one expert form
 * one contiguous range per buffer (brain.bigb.es "deltafin", section "The
 * techniques that bought the 82x": an expert's six tensors are contiguous).
 * This is also the logical (interchange) layout, so moe_mxfp4_pack is a
 * validated device copy into it.
 *
 * MOE_LAYOUT_SCALE4_V1 -- the lossless scale4 side-car ("Deltafin's custom
 * compiled runtime", section "Weight fidelity": scale side-cars coded
 * reversibly, the MXFP4 values and reconstructed scales unchanged; the coding
 * itself is this library's, the pages give none): codes as ROWMAJOR_V1; the
 * scale buffer holds per expert (back to back, 2I + H + 3HI/64 bytes)
 *   bases  : gate [I] | up [I] | down [H]                       (one byte per row)
 *   deltas : gate [I][H/64] | up [I][H/64] | down [H][I/64]     (4 bits per block)
 * Block b of row n has the E8M0 byte base[n] + delta, the even block in the
 * low nibble of byte b/2.  H and I must be multiples of 64.  It is produced
 * by moe_mxfp4_scale4_encode and read by the decode-form kernels and the
 * dequant exports; a forward on it runs the decode form for every token
 * count, and the grouped-GEMM and pack entries refuse it (MOE_ERR_LAYOUT).
 */

/* Layer descriptor: the versioned, size-gated description every layer call
 * takes ("Deltafin's custom compiled runtime", opening paragraph and section
 * "Coarse provider binding"). */
typedef struct moe_layer_desc {
    uint32_t abi_version;  /* MOE_ABI_VERSION */
    uint32_t struct_size;  /* sizeof(moe_layer_desc) */
    int32_t hidden;        /* H: 32 <= H, H % 32 == 0 */
    int32_t inter;         /* I: 32 <= I, I % 32 == 0 */
    int32_t n_experts;     /* E >= 1 */
    int32_t top_k_max;     /* largest k used with this layer: 1 <= k <= min(E, 64) */
    uint32_t layout;       /* MOE_LAYOUT_ROWMAJOR_V1 or MOE_LAYOUT_SCALE4_V1 */
    uint32_t reserved;     /* must be 0 */
} moe_layer_desc;

/* ABI version compiled into the library (MOE_ABI_VERSION), for the caller's
 * version gate ("Deltafin's custom compiled runtime", opening paragraph). */
uint32_t moe_abi_version(void);

/* Static English text for a status code (never NULL; "unknown status" for a
 * value that is not a moe_status).  A convenience, not on the pages. */
const char* moe_status_string(moe_status status);

/* Validate a descriptor ("Deltafin's custom compiled runtime", section
 * "Configuration and device selection": unsupported requests fail early):
 * MOE_OK, MOE_ERR_NULL, MOE_ERR_ABI, MOE_ERR_SHAPE, MOE_ERR_LAYOUT or
 * MOE_ERR_UNSUPPORTED (sizes beyond the kernels' limits: H <= 8192, I <= 8192,
 * E <= 4096). */
moe_status moe_layer_check(const moe_layer_desc* desc);

/* Bytes of the device weight buffers of one layer (all E experts): E times
 * the 3*H*I/2 code bytes and 3*H*I/32 scale bytes of one expert (brain.bigb.es
 * "deltafin", section "The techniques that bought the 82x": one expert is one
 * 17.55 MB range at the K3 shape).  Errors: descriptor errors, MOE_ERR_NULL,
 * MOE_ERR_OVERFLOW. */
moe_status moe_mxfp4_packed_bytes(const moe_layer_desc* desc, size_t* codes_bytes, size_t* scales_bytes);

/* Bytes of device workspace moe_mxfp4_forward / moe_mxfp4_experts need for
 * n_tokens tokens and top-k.  The workspace holds logits, routes, the token ->
 * expert sort, the FFN intermediate and per-(token, rank) expert outputs; its
 * contents on entry do not matter.  Not on the pages (the library's own
 * storage plan; caller-owned so that the library never allocates).  Errors:
 * descriptor errors, MOE_ERR_NULL, MOE_ERR_SHAPE (n_tokens outside [1, 2^20],
 * k outside [1, top_k_max]), MOE_ERR_OVERFLOW. */
moe_status moe_workspace_bytes(const moe_layer_desc* desc, int32_t n_tokens, int32_t k, size_t* bytes);

/*
 * Pack -- copy `expert_count` experts given back to back in the logical layout
 * (device buffers logical_codes / logical_scales) into the device layout
 * buffers packed_codes / packed_scales at experts expert_begin ..
 * expert_begin + expert_count - 1.  Identity on values ("Deltafin's custom
 * compiled runtime", section "Weight fidelity": the released MXFP4 experts stay
 * unchanged; brain.bigb.es "deltafin", section "The techniques that bought the
 * 82x": the six tensors of an expert are one contiguous range).  Lets a caller
 * upload a layer in chunks.  All four pointers are device pointers, 16-byte
 * aligned.  Errors: descriptor errors, MOE_ERR_NULL, MOE_ERR_RANGE (expert
 * range outside [0, E)), MOE_ERR_ALIGN, MOE_ERR_OVERFLOW, MOE_ERR_DEVICE.
 */
moe_status moe_mxfp4_pack(const moe_layer_desc* desc, const void* logical_codes, const void* logical_scales,
                          int64_t expert_begin, int64_t expert_count, void* packed_codes, void* packed_scales,
                          void* stream);

/*
 * The whole layer (router logits, top-k, softmax, token -> expert sort, expert
 * gate/up + SwiGLU, expert down, rank-ordered combine) for n_tokens tokens.
 * Defined by the passages in the file head: "Tarfa EXACTNESS" opening list
 * (fp32 logits, the model's own k); "Deltafin's custom compiled runtime",
 * sections "Complete target sequence tape" (route order, fp32 weights) and
 * "Weight fidelity" (MXFP4 experts unchanged, activations fp32, every selected
 * expert runs); brain.bigb.es "deltafin", section "The techniques that bought
 * the 82x" (fused MXFP4 dequant + GEMV).
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
 * Forms (same results within the output bar): one token, or fp32 x below 9
 * tokens, runs the decode GEMVs; bf16 x from 2 tokens on, and fp32 x from 9
 * on (as three exact bf16 terms), the grouped expert GEMMs, where the shape
 * has them (H and I multiples of 256, 8-bit scales).
 * Deterministic: the same inputs give bit-identical outputs on every call.
 * Errors: descriptor errors, MOE_ERR_NULL, MOE_ERR_DTYPE, MOE_ERR_SHAPE,
 * MOE_ERR_ALIGN (x, router_w, the packed buffers, out or workspace not 16-byte
 * aligned), MOE_ERR_WORKSPACE, MOE_ERR_OVERFLOW, MOE_ERR_DEVICE.
 */
moe_status moe_mxfp4_forward(const moe_layer_desc* desc, const void* x, moe_dtype x_dtype,
                             const float* router_w, const float* router_bias, const void* packed_codes,
                             const void* packed_scales, int32_t n_tokens, int32_t k, float* out,
                             float* logits_out, int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * The whole layer as moe_mxfp4_forward, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): there is no workspace argument.  The workspace
 * lives in a static device array of the library, 64 MiB (67,108,864 bytes),
 * one per GPU, which each GPU the library runs on holds until the process
 * ends; a call uses the array of the current device (stream must belong to
 * it).  A call whose moe_workspace_bytes(desc, n_tokens, k) exceeds 64 MiB
 * returns MOE_ERR_SCRATCH_LIMIT and enqueues nothing (at the K3 shape,
 * H = 7168, I = 1536, E = 896, k = 16, that admits up to 95 tokens).  The
 * array keeps the last call's contents; the forward needs none of it cleared.
 * Calls that overlap on one GPU (on different streams, or from different
 * threads, without ordering between them) race on the array and give
 * undefined output.  The first call on a device looks up the array's device
 * address (hipGetSymbolAddress); no call allocates or frees device memory.
 * Same arguments, outputs and other errors as moe_mxfp4_forward.
 */
moe_status moe_mxfp4_forward_noalloc(const moe_layer_desc* desc, const void* x, moe_dtype x_dtype,
                                     const float* router_w, const float* router_bias, const void* packed_codes,
                                     const void* packed_scales, int32_t n_tokens, int32_t k, float* out,
                                     float* logits_out, int32_t* topk_idx_out, float* topk_w_out, void* stream);

/*
 * The expert part of the layer with the routing given ("Deltafin's custom
 * compiled runtime", section "Complete target sequence tape": the provider
 * receives the authoritative route and its fp32 weights): topk_idx
 * [n_tokens][k] int32 (each row k distinct expert ids in [0, E)) and topk_w
 * [n_tokens][k] fp32.  Same output and workspace contract as
 * moe_mxfp4_forward.  Expert ids outside [0, E) are clamped into it on the
 * device and repeated ids in a row are computed as given; either way every
 * access stays inside the buffers (the output of such a route is the layer
 * evaluated on the clamped ids).
 */
moe_status moe_mxfp4_experts(const moe_layer_desc* desc, const void* x, moe_dtype x_dtype,
                             const int32_t* topk_idx, const float* topk_w, const void* packed_codes,
                             const void* packed_scales, int32_t n_tokens, int32_t k, float* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode-form stages alone (the kernels moe_mxfp4_forward runs for one token),
 * for stage-level checks and timing (brain.bigb.es "deltafin", section "The
 * techniques that bought the 82x": the fused MXFP4 dequant + GEMV; the
 * combine's fixed rank order after "Deltafin's custom compiled runtime", table
 * of linked sources: ordered reduction).  A pair p = t*k + j is token t = p / k
 * of x with expert pair_expert[p] in [0, E).
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
moe_status moe_mxfp4_gate_up(const moe_layer_desc* desc, const void* x, moe_dtype x_dtype,
                             const int32_t* pair_expert, int32_t n_pairs, int32_t k, const void* packed_codes,
                             const void* packed_scales, float* h, void* stream);
moe_status moe_mxfp4_down(const moe_layer_desc* desc, const float* h, const int32_t* pair_expert,
                          int32_t n_pairs, const void* packed_codes, const void* packed_scales, float* y,
                          void* stream);
moe_status moe_combine(const float* y, const float* w, int32_t n_tokens, int32_t k, int32_t hidden,
                       const float* resid, float* out, void* stream);

/* The gate/up stage as the decode-form forward runs it, with the selection
 * fused in: each workgroup takes its pair's expert from the exact top-k of its
 * token's logits [n_tokens][E] (as moe_topk_softmax) and computes h as
 * moe_mxfp4_gate_up does; topk_idx [n_tokens][k] and topk_w [n_tokens][k]
 * receive the selection and its softmax weights ("Tarfa EXACTNESS" page,
 * opening list, and "Deltafin's custom compiled runtime", sections "Weight
 * fidelity" and "Complete target sequence tape", for the selection;
 * brain.bigb.es "deltafin", section "The techniques that bought the 82x",
 * for the fused dequant + GEMV).  Errors: as
 * moe_mxfp4_gate_up, and MOE_ERR_NULL for logits, topk_idx or topk_w. */
moe_status moe_mxfp4_gate_up_select(const moe_layer_desc* desc, const void* x, moe_dtype x_dtype,
                                    const float* logits, int32_t n_tokens, int32_t k, const void* packed_codes,
                                    const void* packed_scales, int32_t* topk_idx, float* topk_w, float* h,
                                    void* stream);

/* Router logits alone: logits [n_tokens][E] = x . router_w^T (+ bias), fp32
 * accumulation ("Tarfa EXACTNESS" page, opening list: fp32 logits with fp32
 * accumulation).  x [n_tokens][H] (x_dtype), router_w [E][H] fp32 row-major,
 * router_bias [E] or NULL.  Errors: MOE_ERR_NULL, MOE_ERR_DTYPE, MOE_ERR_SHAPE
 * (n_tokens outside [1, 2^20]), MOE_ERR_ALIGN (x or router_w not 16-byte
 * aligned), descriptor errors, MOE_ERR_DEVICE. */
moe_status moe_router_logits(const moe_layer_desc* desc, const void* x, moe_dtype x_dtype,
                             const float* router_w, const float* router_bias, int32_t n_tokens,
                             float* logits, void* stream);

/* Top-k + softmax alone, from given logits [n_tokens][n_experts]: idx
 * [n_tokens][k] in rank order and softmax weights w [n_tokens][k].  The
 * selection keeps the model's own k, all of them, in route order ("Tarfa
 * EXACTNESS" page, opening list; "Deltafin's custom compiled runtime",
 * sections "Weight fidelity" and "Complete target sequence tape"); the
 * tie order (lower id first, -0 == +0, NaN last) and the softmax gate are not
 * on the pages.  1 <= k <= min(E, 64), E <= 4096.  Errors: MOE_ERR_NULL,
 * MOE_ERR_SHAPE (n_tokens outside [1, 2^20], E below 1, k out of range),
 * MOE_ERR_UNSUPPORTED (E above 4096), MOE_ERR_DEVICE. */
moe_status moe_topk_softmax(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t k,
                            int32_t* idx, float* w, void* stream);

/* Token -> expert sort alone: stable counting sort of the (token, rank) pairs by expert
 * (the grouping the grouped expert GEMMs need; not on the pages).
 *   topk_idx [n_tokens][k] int32: expert ids in [0, E) (an id outside is clamped into it;
 *     a row that names one expert twice keeps both pairs, in pair order)
 *   expert_offsets [E+1] int32: pairs of expert e are pair_list[offsets[e] .. offsets[e+1])
 *   pair_list [n_tokens*k] int32: pair id t*k + j, ordered by expert, then token, then
 *     rank; always a permutation of 0 .. n_tokens*k - 1, whatever the ids
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
moe_status moe_sort_workspace_bytes(int32_t n_experts, int32_t n_tokens, int32_t k, size_t* bytes);
moe_status moe_sort_by_expert(const int32_t* topk_idx, int32_t n_tokens, int32_t n_experts, int32_t k,
                              int32_t* expert_offsets, int32_t* pair_list, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * Prefill form, stage by stage: the kernels moe_mxfp4_forward runs for more
 * than one bf16 token when H and I are multiples of 256 (the grouped GEMMs on
 * bf16 MFMA), for stage-level checks and timing; the forward runs them over
 * batches of tokens small enough for the limits below.  Other shapes take the
 * decode-form kernels.  The grouping is not on the pages (the pages run one
 * GEMV per expert; brain.bigb.es "deltafin", section "Limitations": prefill
 * touches many experts).  After moe_sort_by_expert:
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
moe_status moe_max_expert_blocks(int32_t n_experts, int32_t n_pairs, int32_t* max_blocks);
moe_status moe_expert_blocks(const int32_t* expert_offsets, int32_t n_experts, int32_t n_pairs, int32_t* blocks,
                             int32_t max_blocks, int32_t* n_blocks, void* stream);
moe_status moe_mxfp4_grouped_gate_up(const moe_layer_desc* desc, const void* x, int32_t n_tokens, int32_t k,
                                     const int32_t* pair_list, const int32_t* blocks, const int32_t* n_blocks,
                                     int32_t max_blocks, const void* packed_codes, const void* packed_scales,
                                     void* hterm, void* stream);
moe_status moe_mxfp4_grouped_down(const moe_layer_desc* desc, const void* hterm, int32_t n_pairs,
                                  const int32_t* pair_list, const int32_t* blocks, const int32_t* n_blocks,
                                  int32_t max_blocks, const void* packed_codes, const void* packed_scales,
                                  float* y, void* stream);

/* Dequantisation alone (brain.bigb.es "deltafin", section "The techniques that
 * bought the 82x": each 4-bit code through a 16-entry table, the E8M0 block
 * scale applied to the fp32 exponent, checked bit for bit against a
 * reference): dequantise one matrix of one expert from the device layout to
 * fp32, exactly: out = E2M1(code) * 2^(scale - 127), subnormals kept, +-inf on
 * overflow, scale byte 0xFF -> NaN 0x7FC00000.  This decodes through the
 * conversion the fp32-operand kernels use (fp32 activations, the decode-form
 * down projection).  matrix 0 = gate [I][H], 1 = up [I][H], 2 = down [H][I].
 * out holds rows x cols fp32.  Errors: MOE_ERR_NULL, MOE_ERR_RANGE (expert
 * outside [0, E) or matrix outside 0..2), MOE_ERR_ALIGN (a buffer not 16-byte
 * aligned), descriptor errors, MOE_ERR_DEVICE. */
moe_status moe_mxfp4_dequant(const moe_layer_desc* desc, const void* packed_codes, const void* packed_scales,
                             int64_t expert, int32_t matrix, float* out, void* stream);

/* Same values (brain.bigb.es "deltafin", section "The techniques that bought
 * the 82x", as above) through the conversion the bf16-activation decode GEMV
 * and both MFMA kernels multiply with: each element decoded to
 * bf16 by the hardware's scaled FP4 -> bf16 conversion, then widened to fp32
 * by placing its 16 bits in the top half.  Every finite E2M1 value times
 * 2^(S-127) fits bf16, so this equals moe_mxfp4_dequant bit for bit where that
 * is finite or infinite; a NaN scale byte gives whatever NaN the conversion
 * produces (not canonicalised).  Same arguments and errors as
 * moe_mxfp4_dequant. */
moe_status moe_mxfp4_dequant_bf16(const moe_layer_desc* desc, const void* packed_codes,
                                  const void* packed_scales, int64_t expert, int32_t matrix, float* out,
                                  void* stream);

/* scale4 encoding ("Deltafin's custom compiled runtime", section "Weight
 * fidelity": lossless scale4 side-cars): desc has layout MOE_LAYOUT_SCALE4_V1;
 * scales8 holds experts expert_begin .. expert_begin + expert_count - 1 back
 * to back in the 8-bit table (3HI/32 bytes each, device memory); their scale4
 * records are written into the layer's scale4 buffer `scale4`.  Each row's
 * base is its smallest scale byte.  A row whose scales span more than 15
 * cannot be coded: the call adds 1 to the device int32 *escapes for each such
 * row (the caller zeroes it first and keeps the 8-bit layout for the layer if
 * it is not 0 after the stream has run).  Errors: descriptor errors,
 * MOE_ERR_LAYOUT (desc not scale4), MOE_ERR_NULL, MOE_ERR_RANGE,
 * MOE_ERR_ALIGN, MOE_ERR_DEVICE. */
moe_status moe_mxfp4_scale4_encode(const moe_layer_desc* desc, const void* scales8, int64_t expert_begin,
                                   int64_t expert_count, void* scale4, int32_t* escapes, void* stream);

/* RMSNorm with gain, n = r / sqrt(mean(r^2) + eps) * gamma, per token (not on
 * the pages; the 12-layer stack workload this library is measured on names
 * it).  r, n: [n_tokens][hidden] fp32; gamma [hidden] fp32; hidden % 4 == 0.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (n_tokens outside [1, 2^20], hidden not
 * a positive multiple of 4), MOE_ERR_ALIGN (r, gamma or n_out not 16-byte
 * aligned), MOE_ERR_DEVICE. */
moe_status moe_rmsnorm(const float* r, const float* gamma, float eps, int32_t n_tokens, int32_t hidden,
                       float* n_out, void* stream);

/* Residual add: r[i] += d[i] for i < n (fp32); n = 0 enqueues nothing (not on
 * the pages; the stack workload's residual stream).  Errors: MOE_ERR_NULL,
 * MOE_ERR_SHAPE (n negative), MOE_ERR_DEVICE. */
moe_status moe_residual_add(float* r, const float* d, int64_t n, void* stream);

/*
 * Stack -- a stack of n_layers pre-norm MoE layers on one residual stream:
 *   r = upcast(x); for each layer l: r = r + MoE_l(RMSNorm_l(r))
 * (the norm and residual are not on the pages; one call advancing every
 * layer of a sequence follows "Deltafin's custom compiled runtime", section
 * "Complete target sequence tape").  Host arrays of n_layers device pointers
 * give each layer's packed codes, packed scales, router weights (and optional
 * biases, NULL array or NULL entries = none) and RMSNorm gains.  residual
 * [n_tokens][H] fp32 receives the result (it may alias nothing else).
 * Workspace: moe_stack_workspace_bytes.  Everything is enqueued on `stream`;
 * the sequence is capture-safe.  Errors: as moe_mxfp4_forward, plus
 * MOE_ERR_SHAPE for n_layers outside [1, 4096].
 */
moe_status moe_stack_workspace_bytes(const moe_layer_desc* desc, int32_t n_tokens, int32_t k, size_t* bytes);
moe_status moe_mxfp4_stack_forward(const moe_layer_desc* desc, int32_t n_layers,
                                   const void* const* packed_codes, const void* const* packed_scales,
                                   const float* const* router_w, const float* const* router_bias,
                                   const float* const* gamma, float eps, const void* x, moe_dtype x_dtype,
                                   int32_t n_tokens, int32_t k, float* residual, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Stack, graph form: capture moe_mxfp4_stack_forward once into a HIP graph and
 * replay it (after "Deltafin's custom compiled runtime", section "Complete
 * target sequence tape": a recorded sequence removes per-operation dispatch).
 * The graph binds the pointers given at creation; a replay recomputes the
 * stack from the current contents of x and the weights.
 * moe_stack_graph_create returns an opaque handle in *graph (free it with
 * moe_stack_graph_destroy, which returns MOE_ERR_DEVICE if HIP fails to free
 * it); launch enqueues one replay on `stream`.  Errors of create: as
 * moe_mxfp4_stack_forward, plus MOE_ERR_DEVICE if capture or instantiation
 * fails.
 */
typedef struct moe_stack_graph moe_stack_graph;
moe_status moe_stack_graph_create(const moe_layer_desc* desc, int32_t n_layers,
                                  const void* const* packed_codes, const void* const* packed_scales,
                                  const float* const* router_w, const float* const* router_bias,
                                  const float* const* gamma, float eps, const void* x, moe_dtype x_dtype,
                                  int32_t n_tokens, int32_t k, float* residual, void* workspace,
                                  size_t workspace_bytes, void* stream, moe_stack_graph** graph);
moe_status moe_stack_graph_launch(moe_stack_graph* graph, void* stream);
moe_status moe_stack_graph_destroy(moe_stack_graph* graph);

#define MOE_CACHE_PREFETCH 1
typedef struct moe_expert_cache moe_expert_cache;
typedef struct moe_cache_stats {
    uint32_t struct_size;     /* set by the caller: sizeof(moe_cache_stats) */
    int32_t capacity;         /* slots in the pool */
    int32_t poisoned;         /* 1 after a terminal failure */
    int32_t alloc_retries;    /* failed pool allocations before the one that succeeded */
    int64_t plans, hits, misses, prefetched, evictions;
    uint64_t bytes_uploaded;  /* host -> device bytes enqueued by finish */
} moe_cache_stats;

/*
 * Host-streamed experts with a device residency cache ("Deltafin's custom
 * compiled runtime", section "CUDA pre-I/O planning and residency"; "How the
 * native runtime works", section "Automatic PILOT prefetch and CUDA expert
 * residency"): the layers' experts live in host memory (logical layout,
 * experts back to back per layer, or any span per expert) and a bounded set
 * of them is resident in a device slot pool.  One layer call is:
 *   1. moe_cache_plan freezes a plan for the call's route ids (host array,
 *      ids in [0, E)): every distinct expert keeps or gets a slot, the hits
 *      first, then the misses in route order, each miss evicting a free slot
 *      or the least recently used one across all layers that the plan does
 *      not use.  slots_out[i] is the slot of ids[i]; miss_ids lists the
 *      misses in order (room for n_ids entries); *n_miss their count.
 *      MOE_ERR_UNSUPPORTED if the union exceeds the capacity, MOE_ERR_RANGE
 *      for a bad layer or id, MOE_ERR_STATE if a plan is already frozen.
 *      flags MOE_CACHE_PREFETCH makes it a prefetch plan (a hint: its
 *      entries become resident like misses, slots_out may be NULL, and it
 *      counts as prefetched, not as hits or misses).
 *   2. moe_cache_finish consumes the plan with one host span per miss (its
 *      codes, 3*H*I/2 bytes, and scales, 3*H*I/32 bytes, in the logical
 *      layout) and enqueues the uploads on `stream`.  With host_pinned the
 *      spans are DMAed directly (they must stay alive until the stream has
 *      passed the copies); otherwise each span is copied on the host into one
 *      of two pinned staging slabs, alternately, and the copy waits for that
 *      slab's previous DMA (an event) before reusing it.  An all-hit plan
 *      uploads nothing.  moe_cache_cancel drops a frozen plan instead.
 *   3. The experts run on the slot pool (moe_cache_slots: codes and scales of
 *      `capacity` experts in the device layout) with every route id replaced
 *      by its slot: moe_mxfp4_experts on a descriptor with n_experts =
 *      capacity.  The output equals the all-resident layer's bit for bit.
 * Uploads, the experts call and any earlier use of an evicted slot must be
 * ordered on one stream (a plan may evict a slot that work already enqueued
 * still reads; stream order keeps the upload after it).
 * moe_cache_create: capacity 0 sizes the pool from free device memory,
 * keeping max(2 GiB, 20%) free, at most 4096 slots; the pool is allocated
 * with up to max_retries further attempts, each a quarter smaller; fails
 * with MOE_ERR_UNSUPPORTED below top_k_max slots.  A failed copy or event
 * poisons the cache: every later call returns MOE_ERR_POISONED.  One caller
 * at a time per cache.  moe_cache_layer_forward runs one whole layer call
 * (router and top-k on the device, the route read back -- this entry
 * synchronises the host with `stream` --, plan, finish from the layer's
 * experts at host_codes / host_scales, experts on the slots) for up to 4096
 * tokens; its workspace is moe_cache_workspace_bytes.
 */
moe_status moe_cache_create(const moe_layer_desc* desc, int32_t n_layers, int32_t capacity, int32_t max_retries,
                            moe_expert_cache** cache);
moe_status moe_cache_destroy(moe_expert_cache* cache);
moe_status moe_cache_slots(moe_expert_cache* cache, void** slot_codes, void** slot_scales, int32_t* capacity);
moe_status moe_cache_get_stats(moe_expert_cache* cache, moe_cache_stats* stats);
moe_status moe_cache_plan(moe_expert_cache* cache, int32_t layer, const int32_t* ids, int32_t n_ids, int32_t flags,
                          int32_t* slots_out, int32_t* miss_ids, int32_t* n_miss);
moe_status moe_cache_finish(moe_expert_cache* cache, const void* const* miss_codes, const void* const* miss_scales,
                            int32_t host_pinned, void* stream);
moe_status moe_cache_cancel(moe_expert_cache* cache);
moe_status moe_cache_workspace_bytes(moe_expert_cache* cache, int32_t n_tokens, int32_t k, size_t* bytes);
moe_status moe_cache_layer_forward(moe_expert_cache* cache, int32_t layer, const void* x, moe_dtype x_dtype,
                                   const float* router_w, const float* router_bias, const void* host_codes,
                                   const void* host_scales, int32_t host_pinned, int32_t n_tokens, int32_t k,
                                   float* out, int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Packed-int8 rows with one fp16 scale per row: the resident-spine matrices
 * of the pages' explicit, non-weight-exact int8 option ("Deltafin's custom
 * compiled runtime", section "Weight fidelity": row rounding and fp16 scales;
 * the 12288 x 7168 packed-int8 shape of section "One native build and test
 * graph").  q [rows][cols] int8 row-major, scales_f16 [rows] IEEE binary16
 * bits; W[n][k] = q[n][k] * s[n], exact in fp32.
 *  - moe_int8_dequant: out [rows][cols] fp32 = W, bit for bit (the fused
 *    int8 -> fp32 + scale copy of brain.bigb.es "deltafin", section "The
 *    techniques that bought the 82x").
 *  - moe_int8_gemv: y [n_tokens][rows] fp32 = x [n_tokens][cols] . W^T, fp32
 *    accumulation, 1 <= n_tokens <= 4, x fp32 or bf16; rows_per_workgroup 0
 *    picks the default split (else a multiple of 8, for tuning).
 * cols a multiple of 16, at most 16384 (MOE_ERR_UNSUPPORTED above); rows at
 * most 2^20.  q, x, y and out 16-byte aligned.  Errors: MOE_ERR_NULL,
 * MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_UNSUPPORTED,
 * MOE_ERR_DEVICE.
 */
moe_status moe_int8_dequant(const int8_t* q, const uint16_t* scales_f16, int32_t rows, int32_t cols, float* out,
                            void* stream);
moe_status moe_int8_gemv(const int8_t* q, const uint16_t* scales_f16, int32_t rows, int32_t cols, const void* x,
                         moe_dtype x_dtype, int32_t n_tokens, float* y, int32_t rows_per_workgroup, void* stream);

/*
 * Matrix-core rate on random operands (a measurement aid, not on the pages):
 * n_workgroups workgroups of 512 threads each run iters rounds of 8
 * independent MFMAs of one kind, with no memory traffic in the loop, and
 * write one float per thread to sink.  kind 0: bf16 16x16x32 (16,384 flops
 * per MFMA); kind 1: fp8 e4m3 x fp4 e2m1, 16x16x128 with unit E8M0 scales
 * (65,536 flops); kind 2: fp4 x fp4, 16x16x128 (65,536 flops).  Timing the
 * call gives the rate the chip sustains under that load, the ceiling of the
 * prefill form's bf16 MFMA and of the MXFP4 alternatives.  operands: 65536
 * random bytes on the device (16-byte aligned; every bit pattern is allowed,
 * NaN operands included); sink: n_workgroups * 512 floats on the device.
 * Errors: MOE_ERR_NULL, MOE_ERR_UNSUPPORTED (kind), MOE_ERR_SHAPE
 * (n_workgroups outside 1 .. 65536, iters outside 1 .. 10^6), MOE_ERR_ALIGN,
 * MOE_ERR_DEVICE.
 */
moe_status moe_mfma_rate(int32_t kind, const void* operands, int32_t n_workgroups, int32_t iters, float* sink,
                         void* stream);

/*
 * Next-layer route hint ("Deltafin's custom compiled runtime", section "Exact
 * next-layer expert prefetch"; "How the native runtime works", section
 * "Automatic PILOT prefetch and CUDA expert residency"): the k experts the
 * next layer's router would select if its input were the current activation
 * r [n_tokens][H] fp32, i.e. the exact top-k of router_w_next .
 * RMSNorm(r; gamma_next, eps) (+ bias), computed with the stack's own norm +
 * router kernel and top-k, so for r equal to the next layer's input the hint
 * is that layer's route.  hint_idx [n_tokens][k] int32 on the device, rank
 * order.  The hint schedules prefetches (moe_cache_plan with
 * MOE_CACHE_PREFETCH) and never enters the computation.  desc is the next
 * layer's descriptor; workspace: moe_route_hint_workspace_bytes.  Errors:
 * descriptor errors, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN,
 * MOE_ERR_WORKSPACE, MOE_ERR_OVERFLOW, MOE_ERR_DEVICE.
 */
moe_status moe_route_hint_workspace_bytes(const moe_layer_desc* desc, int32_t n_tokens, int32_t k, size_t* bytes);
moe_status moe_route_hint(const moe_layer_desc* desc, const float* r, const float* gamma_next, float eps,
                          const float* router_w_next, const float* router_bias_next, int32_t n_tokens, int32_t k,
                          int32_t* hint_idx, void* workspace, size_t workspace_bytes, void* stream);

#define MOE_TRACE_BUFFERED 0
#define MOE_TRACE_SYNC 1
typedef struct moe_trace moe_trace;
/*
 * Router trace ("How the native runtime works", section "Router tracing and
 * offline expert warming"; "Deltafin's custom compiled runtime", section
 * "Router traces and cache warming"): one text line per traced token,
 *   {"layer":L,"pos":P,"ids":[i0,...],"w":["xxxxxxxx",...]}
 * the routed ids in rank order and the 8 hex digits of each combine weight's
 * fp32 bits.  moe_trace_open refuses a path whose last component is a symlink
 * or that is not a regular file (MOE_ERR_IO), truncates it, and caps the
 * trace at max_bytes (0 = 8 GiB): a record that would pass the cap is refused
 * with MOE_ERR_IO and the trace stops.  MOE_TRACE_BUFFERED batches records in
 * a 1 MiB buffer written when full and at close; MOE_TRACE_SYNC writes and
 * syncs each call's records before returning.  moe_trace_record appends
 * n_tokens lines for tokens at positions position .. position + n_tokens - 1
 * from host arrays ids [n_tokens][k] and w [n_tokens][k] (k <= 64).
 * moe_trace_count reads a trace back for offline warming: counts
 * [n_layers][n_experts] receives how often each (layer, expert) was routed and
 * *n_records the line count; a malformed line, an unterminated or over-long
 * line (4096 bytes), an id or layer out of range, a symlink or a file over
 * 8 GiB is MOE_ERR_IO.  Tracing reads routes only and never changes them.
 */
moe_status moe_trace_open(const char* path, int32_t mode, uint64_t max_bytes, moe_trace** trace);
moe_status moe_trace_record(moe_trace* trace, int32_t layer, int64_t position, int32_t n_tokens, int32_t k,
                            const int32_t* ids, const float* w);
moe_status moe_trace_close(moe_trace* trace);
moe_status moe_trace_count(const char* path, int32_t n_layers, int32_t n_experts, int64_t* counts,
                           int64_t* n_records);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
