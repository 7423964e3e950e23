// Host-side launchers of the gfx950 kernels (internal to libmoe_mxfp4).
// Shapes are validated by the C ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

hipError_t launch_router_logits(const void* x, bool x_f32, const float* wr, const float* bias, int T,
                                int H, int E, float* logits, hipStream_t s);
// RMSNorm folded into the fp32 router: logits of n = RMSNorm(r) * gamma, and
// n itself written to nout (bit-identical to k_rmsnorm + k_router_logits).
hipError_t launch_norm_router_logits(const float* r, const float* gamma, float eps, const float* wr,
                                     const float* bias, int T, int H, int E, float* logits, float* nout,
                                     hipStream_t s);
hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                               hipStream_t s);
// Stable sort of the (token, rank) pairs by expert.  ws: sort_workspace_bytes(T, E)
// bytes (may be null when that is 0; with null the one-workgroup sort runs).
size_t sort_workspace_bytes(int T, int E);
// Pairs per expert block of the grouped GEMMs (8 m-tiles of 16).
constexpr int kExpertBlockPairs = 128;
// True when launch_sort_by_expert runs as one workgroup (fewer than 1024
// tokens, or no workspace); it can then also write the expert blocks
// (blocks != nullptr), as launch_expert_blocks would.
bool sort_is_one_workgroup(int T, const void* ws);
hipError_t launch_sort_by_expert(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* pairs,
                                 void* ws, hipStream_t s, int4* blocks = nullptr, int max_blocks = 0,
                                 int32_t* nblocks = nullptr);

// Decode-form GEMVs.  s4: `scales` is the scale4 side-car (per expert: row
// bases gate [I] | up [I] | down [H], then 4-bit deltas gate [I][H/64] |
// up [I][H/64] | down [H][I/64]) instead of the 8-bit table.
hipError_t launch_gateup_gemv(const void* x, bool x_f32, const int32_t* route, int P, int k,
                              const uint8_t* codes, const uint8_t* scales, bool s4, int H, int I, int E,
                              float* hbuf, hipStream_t s);
// Same with the selection fused in: each workgroup takes its pair's expert
// from the exact top-k of its token's logits; route [T][k] and wsel [T][k]
// receive the selection and the softmax weights.
hipError_t launch_gateup_select_gemv(const void* x, bool x_f32, const float* logits, int T, int k,
                                     const uint8_t* codes, const uint8_t* scales, bool s4, int H, int I, int E,
                                     int32_t* route, float* wsel, float* hbuf, hipStream_t s);
hipError_t launch_down_gemv(const float* hbuf, const int32_t* pair_expert, int P, const uint8_t* codes,
                            const uint8_t* scales, bool s4, int H, int I, int E, float* ybuf, hipStream_t s);
hipError_t launch_combine(const float* ybuf, const float* w, int T, int k, int H, const float* resid,
                          float* out, hipStream_t s);

// Prefill form (bf16 activations): expert blocks of at most 128 sorted pairs,
// gate/up + SwiGLU and down grouped GEMMs on MFMA.  hterm holds h as two bf16
// terms, [2][P][I].  grouped_shape_ok: H and I multiples of 256, with the
// gate/up workgroup's scale table fitting LDS beside the activation tiles
// (H <= 11264; layers have H <= 8192).
bool grouped_shape_ok(int64_t H, int64_t I);
int max_expert_blocks(int P, int E);
hipError_t launch_expert_blocks(const int32_t* offsets, int E, int max_blocks, int4* blocks, int32_t* nblocks,
                                hipStream_t s);
// x_terms = 1: x is [T][H] bf16; 3: x is [T][3H], the three exact bf16 terms
// of an fp32 x back to back along K (launch_split3).
hipError_t launch_gateup_mfma(const uint16_t* x, int T, const int32_t* pairs, const int4* blocks,
                              const int32_t* nblocks, int max_blocks, const uint8_t* codes, const uint8_t* scales,
                              int H, int I, int E, int k, int P, uint16_t* hterm, hipStream_t s, int x_terms = 1);
hipError_t launch_down_mfma(const uint16_t* hterm, const int32_t* pairs, const int4* blocks, const int32_t* nblocks,
                            int max_blocks, const uint8_t* codes, const uint8_t* scales, int H, int I, int E, int P,
                            float* ybuf, hipStream_t s);

// Router logits for many bf16 tokens on MFMA (H a multiple of 128).  With
// `part` (router_mfma_splits(T, H) * T * E floats) and few tokens, K slices
// run in workgroups of their own and a second kernel adds their partial sums
// in order; without it one workgroup runs all slices of its tile.  Both give
// the same bits.
int router_mfma_splits(int T, int H);
// reduce = false leaves the partial sums to launch_router_reduce_topk (only
// when the launch splits, router_mfma_splits(T, H) > 1, and T <= 256).
hipError_t launch_router_mfma(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                              float* logits, float* part, hipStream_t s, bool reduce = true);
// The split router's last step and the top-k in one launch: logits[t][e] =
// sum of part[0..nsplit)[t][e] in slice order (+ bias[e]), the bits the
// router's own reduction gives, then the exact top-k + softmax of each token
// as launch_topk_softmax.  One workgroup per token.
hipError_t launch_router_reduce_topk(const float* part, int nsplit, int T, int E, const float* bias, int k,
                                     float* logits, int32_t* idx, float* w, hipStream_t s);

// Packed-int8 rows with fp16 row scales: y [T][N] = x [T][K] . (q * s)^T for
// T <= 4 (rows_per_wg <= 0: the default split), and the fp32 export of q * s.
int int8_rows_per_wg(int N, int K);
hipError_t launch_int8_gemv(const int8_t* q, const uint16_t* s, int N, int K, const void* x, bool x_f32, int T,
                            float* y, int rows_per_wg, hipStream_t st);
hipError_t launch_int8_dequant(const int8_t* q, const uint16_t* s, int N, int K, float* out, hipStream_t st);

// Matrix-core rate on random operands (kind 0 bf16, 1 fp8 x fp4, 2 fp4 x fp4):
// n_workgroups of 512 threads, iters rounds of 8 MFMAs per thread; operands
// 65536 random bytes, sink n_workgroups * 512 floats.
hipError_t launch_mfma_rate(int kind, const void* operands, int n_workgroups, int iters, float* sink,
                            hipStream_t s);

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s);
// via_bf16: decode through the bf16 conversion of the bf16 GEMV and the MFMA
// kernels (widened to fp32), else through the fp32 conversion.  With s4_base
// set, `scales` are the matrix's scale4 deltas [rows][cols/64] and s4_base its
// row bases [rows].
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const uint8_t* s4_base, int rows, int cols,
                          float* out, bool via_bf16, hipStream_t s);
// scale4 encoding of experts [e0, e0 + n) from the 8-bit table (per expert
// 3*H*I/32 bytes, back to back) into the layer's scale4 buffer; every row
// whose block scales span more than 15 adds 1 to *escapes (that row is then
// not representable and the layer must keep the 8-bit table).
hipError_t launch_scale4_encode(const uint8_t* scales8, int64_t e0, int64_t n, int H, int I, uint8_t* scale4,
                                int32_t* escapes, hipStream_t s);
hipError_t launch_rmsnorm(const float* r, const float* gamma, float eps, int T, int H, float* out,
                          hipStream_t s);
hipError_t launch_residual_add(float* r, const float* d, size_t n, hipStream_t s);
hipError_t launch_widen(const void* x, bool x_f32, size_t n, float* out, hipStream_t s);
// fp32 rows x [T][H] as three bf16 terms per element, out [T][3][H] (row t:
// hi of every element, then mid, then lo): hi = bf16(x), mid = bf16(x - hi),
// lo = bf16(x - hi - mid), round to nearest even; hi + mid + lo == x exactly
// for every finite x whose terms stay in bf16's normal range.
hipError_t launch_split3(const float* x, int T, int H, uint16_t* out, hipStream_t s);

}  // namespace moe
