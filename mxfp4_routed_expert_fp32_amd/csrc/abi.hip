// C ABI of libmoe_mxfp4: argument validation, workspace carving and launch
// sequencing.  Every check runs on the host before the first launch, so an
// invalid call enqueues nothing (after "Deltafin's custom compiled runtime",
// section "Configuration and device selection": explicit unsupported requests
// fail early; and section "Model contract and pack authentication": lengths and
// offsets use checked arithmetic).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>

#include "moe_mxfp4.h"
#include <algorithm>

#include "kernels.h"

namespace {

constexpr int kMaxHidden = 8192;
constexpr int kMaxInter = 8192;
constexpr int kMaxExperts = 4096;
constexpr int kMaxTopK = 64;
constexpr int64_t kMaxTokens = 1 << 20;

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool mul_ok(size_t a, size_t b, size_t* r) { return !__builtin_mul_overflow(a, b, r); }
inline bool add_ok(size_t a, size_t b, size_t* r) { return !__builtin_add_overflow(a, b, r); }

moe_status check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->abi_version != MOE_ABI_VERSION || d->struct_size != sizeof(moe_layer_desc)) return MOE_ERR_ABI;
  if (d->reserved != 0) return MOE_ERR_ABI;
  if (d->layout != MOE_LAYOUT_ROWMAJOR_V1 && d->layout != MOE_LAYOUT_SCALE4_V1) return MOE_ERR_LAYOUT;
  if (d->hidden < 32 || d->inter < 32 || d->n_experts < 1 || d->top_k_max < 1) return MOE_ERR_SHAPE;
  if (d->hidden % 32 || d->inter % 32) return MOE_ERR_SHAPE;
  if (d->top_k_max > d->n_experts || d->top_k_max > kMaxTopK) return MOE_ERR_SHAPE;
  if (d->hidden > kMaxHidden || d->inter > kMaxInter || d->n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  // scale4 packs two blocks per delta byte: whole bytes per row need K % 64 == 0
  if (d->layout == MOE_LAYOUT_SCALE4_V1 && (d->hidden % 64 || d->inter % 64)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline bool is_s4(const moe_layer_desc* d) { return d->layout == MOE_LAYOUT_SCALE4_V1; }

// Per-expert byte counts; checked.  scale4: row bases (2I + H bytes) and
// 4-bit deltas (3HI/64 bytes) instead of the 3HI/32-byte table.
moe_status expert_bytes(const moe_layer_desc* d, size_t* cb, size_t* sb) {
  size_t hi;
  if (!mul_ok((size_t)d->hidden, (size_t)d->inter, &hi)) return MOE_ERR_OVERFLOW;
  if (!mul_ok(hi, 3, &hi)) return MOE_ERR_OVERFLOW;
  *cb = hi / 2;
  *sb = is_s4(d) ? hi / 64 + (size_t)2 * d->inter + (size_t)d->hidden : hi / 32;
  return MOE_OK;
}

// Workspace carve: a bump allocator over the caller's buffer, 256-byte aligned.
struct Carve {
  size_t off = 0;
  bool overflow = false;
  size_t take(size_t bytes) {
    size_t a = (off + 255) & ~size_t(255);
    if (a < off) overflow = true;
    size_t end;
    if (!add_ok(a, bytes, &end)) overflow = true;
    off = end;
    return a;
  }
};

struct FwdLayout {
  size_t logits, idx, w, h, y, offsets, pairs, blocks, nblocks, rpart, sortws, xsplit, total;
  int max_blocks;
  bool has_rpart;
};

int64_t grouped_batch(const moe_layer_desc* d, int32_t k, int x_terms);

// fp32 activations take the grouped (prefill) form from this many tokens on,
// as three exact bf16 terms; fewer tokens stream each pair's expert in the
// decode-form GEMVs.
constexpr int32_t kF32GroupedMinTokens = 9;

// The grouped form: bf16 x from two tokens on, fp32 x from
// kF32GroupedMinTokens on (when the shape has one).
bool grouped_form(const moe_layer_desc* d, int32_t T, int32_t k, bool x_f32) {
  if (x_f32) return T >= kF32GroupedMinTokens && grouped_batch(d, k, 3) > 0;
  return T > 1 && grouped_batch(d, k, 1) > 0;
}

moe_status forward_layout(const moe_layer_desc* d, int32_t T, int32_t k, FwdLayout* L) {
  size_t TE, Tk, TkI, TkH;
  if (!mul_ok((size_t)T, (size_t)d->n_experts, &TE) || !mul_ok((size_t)T, (size_t)k, &Tk) ||
      !mul_ok(Tk, (size_t)d->inter, &TkI) || !mul_ok(Tk, (size_t)d->hidden, &TkH))
    return MOE_ERR_OVERFLOW;
  size_t b[7];
  if (!mul_ok(TE, 4, &b[0]) || !mul_ok(Tk, 4, &b[1]) || !mul_ok(Tk, 4, &b[2]) || !mul_ok(TkI, 4, &b[3]) ||
      !mul_ok(TkH, 4, &b[4]) || !mul_ok((size_t)d->n_experts + 1, 4, &b[5]) || !mul_ok(Tk, 4, &b[6]))
    return MOE_ERR_OVERFLOW;
  Carve c;
  L->logits = c.take(b[0]);
  L->idx = c.take(b[1]);
  L->w = c.take(b[2]);
  L->h = c.take(b[3]);
  L->y = c.take(b[4]);
  L->offsets = c.take(b[5]);
  L->pairs = c.take(b[6]);
  L->max_blocks = moe::max_expert_blocks((int)Tk, d->n_experts);
  L->blocks = c.take((size_t)L->max_blocks * 16);
  L->nblocks = c.take(4);
  // partial router sums for few tokens on the MFMA router
  L->has_rpart = d->hidden % 128 == 0 && moe::router_mfma_splits(T, d->hidden) > 1;
  size_t rp = 0;
  if (L->has_rpart && !mul_ok(TE, (size_t)moe::router_mfma_splits(T, d->hidden) * 4, &rp)) return MOE_ERR_OVERFLOW;
  L->rpart = c.take(rp);
  L->sortws = c.take(moe::sort_workspace_bytes(T, d->n_experts));
  // fp32 x in the grouped form: one batch of x as three bf16 terms
  size_t xs = 0;
  if (T >= kF32GroupedMinTokens) {
    const int64_t tb = grouped_batch(d, k, 3);
    if (tb > 0 && !mul_ok((size_t)std::min<int64_t>(T, tb), (size_t)6 * d->hidden, &xs)) return MOE_ERR_OVERFLOW;
  }
  L->xsplit = c.take(xs);
  L->total = c.take(0);
  if (c.overflow) return MOE_ERR_OVERFLOW;
  // pair indices are int32 on the device; MFMA-path byte offsets are 32-bit
  if (Tk > (size_t)INT32_MAX / 8) return MOE_ERR_OVERFLOW;
  return MOE_OK;
}

inline moe_status dev(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

#define MOE_TRY(expr)             \
  do {                            \
    moe_status rc_ = (expr);      \
    if (rc_ != MOE_OK) return rc_; \
  } while (0)

moe_status check_tokens(int32_t T, int32_t k, const moe_layer_desc* d) {
  if (T < 1 || T > kMaxTokens) return MOE_ERR_SHAPE;
  if (k < 1 || k > d->top_k_max) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// The grouped GEMMs tile K by 256 (weights) and 128 (activations), keep the
// gate/up row tile's scales in LDS (which caps H), and address activations
// with 32-bit buffer offsets and an out-of-range sentinel at 1 GiB: x (bf16)
// and the two bf16 terms of h must each stay below that; y (fp32) is stored
// through 32-bit offsets below 2 GiB.

bool grouped_fits(const moe_layer_desc* d, int64_t T, int64_t P) {
  return moe::grouped_shape_ok(d->hidden, d->inter) && T * d->hidden * 2 < (int64_t{1} << 30) &&
         P * d->inter * 4 < (int64_t{1} << 30) && P * d->hidden * 4 < (int64_t{1} << 31);
}

// Tokens per batch of the prefill form (larger T runs in batches of this
// many tokens, which are independent); 0 if the shape has no prefill form.
// x_terms: bf16 terms per activation (1 for bf16 x, 3 for fp32 x).
int64_t grouped_batch(const moe_layer_desc* d, int32_t k, int x_terms) {
  if (is_s4(d) || !moe::grouped_shape_ok(d->hidden, d->inter)) return 0;  // scale4: decode form only
  const int64_t H = d->hidden, I = d->inter;
  int64_t tb = ((int64_t{1} << 30) - 1) / (H * 2 * x_terms);
  tb = std::min(tb, ((int64_t{1} << 30) - 1) / (k * I * 4));
  tb = std::min(tb, ((int64_t{1} << 31) - 1) / (k * H * 4));
  return tb >= 2 ? tb : 0;
}

// Router logits: many bf16 tokens go to the MFMA kernel (fp32 weights split
// into three exact bf16 terms), a few tokens or fp32 tokens to the GEMV.
// `part` (optional) is room for the MFMA router's partial sums.
hipError_t router(const moe_layer_desc* d, const void* x, bool x_f32, const float* wr, const float* bias,
                  int32_t T, float* logits, float* part, hipStream_t s) {
  if (T > 8 && !x_f32 && d->hidden % 128 == 0)
    return moe::launch_router_mfma(static_cast<const uint16_t*>(x), wr, bias, T, d->hidden, d->n_experts, logits,
                                   part, s);
  return moe::launch_router_logits(x, x_f32, wr, bias, T, d->hidden, d->n_experts, logits, s);
}

// Expert part of the layer given the routing (idx, w on the device).  For one token the pairs are
// the k ranks of that token and idx itself is the pair -> expert map.
moe_status run_experts(const moe_layer_desc* d, const void* x, bool x_f32, const int32_t* idx, const float* w,
                const void* codes, const void* scales, int32_t T, int32_t k, float* out,
                const float* resid, char* ws, const FwdLayout& L, hipStream_t s) {
  const int H = d->hidden, I = d->inter, E = d->n_experts;
  const int P = T * k;
  float* h = reinterpret_cast<float*>(ws + L.h);
  float* y = reinterpret_cast<float*>(ws + L.y);
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  const uint8_t* sc = static_cast<const uint8_t*>(scales);
  if (grouped_form(d, T, k, x_f32)) {
    // prefill form, per batch of tokens: sort pairs by expert, grouped GEMMs on
    // MFMA, combine; fp32 x goes to the GEMMs as three exact bf16 terms
    const int xt = x_f32 ? 3 : 1;
    const int64_t tb = grouped_batch(d, k, xt);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* pairs = reinterpret_cast<int32_t*>(ws + L.pairs);
    int4* blocks = reinterpret_cast<int4*>(ws + L.blocks);
    int32_t* nblocks = reinterpret_cast<int32_t*>(ws + L.nblocks);
    uint16_t* hterm = reinterpret_cast<uint16_t*>(h);  // [2][n*k][I] bf16, same bytes as h
    uint16_t* xs = reinterpret_cast<uint16_t*>(ws + L.xsplit);
    for (int64_t t0 = 0; t0 < T; t0 += tb) {
      const int n = (int)std::min<int64_t>(tb, T - t0);
      const int Pn = n * k;
      const uint16_t* xb = static_cast<const uint16_t*>(x) + t0 * H;
      if (x_f32) {
        MOE_TRY(dev(moe::launch_split3(static_cast<const float*>(x) + t0 * H, n, H, xs, s)));
        xb = xs;
      }
      if (moe::sort_is_one_workgroup(n, ws + L.sortws)) {  // the sort also cuts the blocks
        MOE_TRY(dev(moe::launch_sort_by_expert(idx + t0 * k, n, E, k, offsets, pairs, ws + L.sortws, s, blocks,
                                               L.max_blocks, nblocks)));
      } else {
        MOE_TRY(dev(moe::launch_sort_by_expert(idx + t0 * k, n, E, k, offsets, pairs, ws + L.sortws, s)));
        MOE_TRY(dev(moe::launch_expert_blocks(offsets, E, L.max_blocks, blocks, nblocks, s)));
      }
      MOE_TRY(dev(moe::launch_gateup_mfma(xb, n, pairs, blocks, nblocks, L.max_blocks, c, sc, H, I, E, k, Pn, hterm,
                                          s, xt)));
      MOE_TRY(dev(moe::launch_down_mfma(hterm, pairs, blocks, nblocks, L.max_blocks, c, sc, H, I, E, Pn, y, s)));
      MOE_TRY(dev(moe::launch_combine(y, w + t0 * k, n, k, H, resid ? resid + t0 * H : nullptr, out + t0 * H, s)));
    }
    return MOE_OK;
  }
  MOE_TRY(dev(moe::launch_gateup_gemv(x, x_f32, idx, P, k, c, sc, is_s4(d), H, I, E, h, s)));
  MOE_TRY(dev(moe::launch_down_gemv(h, idx, P, c, sc, is_s4(d), H, I, E, y, s)));
  MOE_TRY(dev(moe::launch_combine(y, w, T, k, H, resid, out, s)));
  return MOE_OK;
}

// Checks of a forward / experts call except its workspace; fills the layout.
moe_status check_forward_core(const moe_layer_desc* d, const void* x, moe_dtype x_dtype, const void* codes,
                              const void* scales, int32_t T, int32_t k, const float* out, FwdLayout* L) {
  MOE_TRY(check_desc(d));
  if (!x || !codes || !scales || !out) return MOE_ERR_NULL;
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  MOE_TRY(check_tokens(T, k, d));
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned16(out)) return MOE_ERR_ALIGN;
  return forward_layout(d, T, k, L);
}

moe_status check_forward_args(const moe_layer_desc* d, const void* x, moe_dtype x_dtype, const void* codes,
                       const void* scales, int32_t T, int32_t k, const float* out, const void* ws,
                       size_t ws_bytes, FwdLayout* L) {
  MOE_TRY(check_forward_core(d, x, x_dtype, codes, scales, T, k, out, L));
  if (!ws) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < L->total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// ---------------------------------------------------------------- static scratch (no allocation)
// moe_mxfp4_forward_noalloc keeps the forward's workspace in this file-scope
// device array instead of a caller buffer.  Every GPU the library runs on
// holds its own copy until the process ends.  In host code the array's name
// is only a host-side stand-in: host code uses the device address looked up
// below, never the name.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kScratchDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (hipGetSymbolAddress with that device current) and kept.
moe_status scratch_address(void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return MOE_ERR_DEVICE;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return MOE_ERR_DEVICE;
    g_scratch_addr[dev] = a;
  }
  *p = g_scratch_addr[dev];
  return MOE_OK;
}

moe_status forward_impl(const moe_layer_desc* d, const void* x, moe_dtype x_dtype, const float* router_w,
                 const float* router_bias, const void* codes, const void* scales, int32_t T, int32_t k,
                 float* out, float* logits_out, int32_t* idx_out, float* w_out, void* workspace,
                 const FwdLayout& L, const float* resid, hipStream_t s, const float* norm_gamma = nullptr,
                 float norm_eps = 0.0f, float* norm_out = nullptr) {
  char* ws = static_cast<char*>(workspace);
  float* logits = logits_out ? logits_out : reinterpret_cast<float*>(ws + L.logits);
  int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + L.idx);
  float* w = w_out ? w_out : reinterpret_cast<float*>(ws + L.w);
  const bool xf = x_dtype == MOE_DTYPE_F32;
  if (norm_gamma) {
    // x is an fp32 residual: the router kernel also applies the RMSNorm and
    // writes the normalised rows to norm_out, which the expert kernels read
    MOE_TRY(dev(moe::launch_norm_router_logits(static_cast<const float*>(x), norm_gamma, norm_eps, router_w,
                                               router_bias, T, d->hidden, d->n_experts, logits, norm_out, s)));
    x = norm_out;
  }
  const bool prefill = grouped_form(d, T, k, xf);
  bool selected = false;
  if (!norm_gamma) {
    float* rpart = L.has_rpart ? reinterpret_cast<float*>(ws + L.rpart) : nullptr;
    if (prefill && !xf && rpart && T > 8) {
      // the MFMA router runs its K slices in workgroups of their own; their
      // sum and the top-k run as one launch
      MOE_TRY(dev(moe::launch_router_mfma(static_cast<const uint16_t*>(x), router_w, router_bias, T, d->hidden,
                                          d->n_experts, logits, rpart, s, false)));
      MOE_TRY(dev(moe::launch_router_reduce_topk(rpart, moe::router_mfma_splits(T, d->hidden), T, d->n_experts,
                                                 router_bias, k, logits, idx, w, s)));
      selected = true;
    } else {
      MOE_TRY(dev(router(d, x, xf, router_w, router_bias, T, logits, rpart, s)));
    }
  }
  if (prefill) {
    // prefill form: top-k, then sort + grouped GEMMs
    if (!selected) MOE_TRY(dev(moe::launch_topk_softmax(logits, T, d->n_experts, k, idx, w, s)));
    return run_experts(d, x, xf, idx, w, codes, scales, T, k, out, resid, ws, L, s);
  }
  // decode form: the gate/up kernel selects the experts itself (and writes
  // idx and w for the down and combine kernels)
  const int H = d->hidden, I = d->inter, E = d->n_experts;
  float* h = reinterpret_cast<float*>(ws + L.h);
  float* y = reinterpret_cast<float*>(ws + L.y);
  const uint8_t* c = static_cast<const uint8_t*>(codes);
  const uint8_t* sc = static_cast<const uint8_t*>(scales);
  MOE_TRY(dev(moe::launch_gateup_select_gemv(x, xf, logits, T, k, c, sc, is_s4(d), H, I, E, idx, w, h, s)));
  MOE_TRY(dev(moe::launch_down_gemv(h, idx, T * k, c, sc, is_s4(d), H, I, E, y, s)));
  return dev(moe::launch_combine(y, w, T, k, H, resid, out, s));
}

}  // namespace

extern "C" {

uint32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status status) {
  switch ((int)status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or not a multiple of 32";
    case MOE_ERR_DTYPE: return "unknown activation dtype";
    case MOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_LAYOUT: return "unknown weight layout";
    case MOE_ERR_UNSUPPORTED: return "request outside what the kernels implement";
    case MOE_ERR_OVERFLOW: return "a size computation overflows";
    case MOE_ERR_DEVICE: return "a HIP call or kernel launch failed";
    case MOE_ERR_ABI: return "descriptor ABI version or size mismatch";
    case MOE_ERR_RANGE: return "an index argument is out of range";
    case MOE_ERR_SCRATCH_LIMIT: return "the call needs more than the library's static scratch";
    case MOE_ERR_POISONED: return "the residency cache failed earlier and refuses further work";
    case MOE_ERR_STATE: return "call out of order for the object's state";
    case MOE_ERR_IO: return "a file operation failed, or the trace reached its size limit";
    default: return "unknown status";
  }
}

moe_status moe_layer_check(const moe_layer_desc* desc) { return check_desc(desc); }

moe_status moe_mxfp4_packed_bytes(const moe_layer_desc* d, size_t* codes_bytes, size_t* scales_bytes) {
  MOE_TRY(check_desc(d));
  if (!codes_bytes || !scales_bytes) return MOE_ERR_NULL;
  size_t cb, sb;
  MOE_TRY(expert_bytes(d, &cb, &sb));
  size_t tc, ts;
  if (!mul_ok(cb, (size_t)d->n_experts, &tc) || !mul_ok(sb, (size_t)d->n_experts, &ts)) return MOE_ERR_OVERFLOW;
  *codes_bytes = tc;
  *scales_bytes = ts;
  return MOE_OK;
}

moe_status moe_workspace_bytes(const moe_layer_desc* d, int32_t n_tokens, int32_t k, size_t* bytes) {
  MOE_TRY(check_desc(d));
  if (!bytes) return MOE_ERR_NULL;
  MOE_TRY(check_tokens(n_tokens, k, d));
  FwdLayout L;
  MOE_TRY(forward_layout(d, n_tokens, k, &L));
  *bytes = L.total;
  return MOE_OK;
}

moe_status moe_mxfp4_pack(const moe_layer_desc* d, const void* logical_codes, const void* logical_scales,
                   int64_t expert_begin, int64_t expert_count, void* packed_codes, void* packed_scales,
                   void* stream) {
  MOE_TRY(check_desc(d));
  if (is_s4(d)) return MOE_ERR_LAYOUT;  // scale4 tables come from moe_mxfp4_scale4_encode
  if (!logical_codes || !logical_scales || !packed_codes || !packed_scales) return MOE_ERR_NULL;
  if (expert_begin < 0 || expert_count < 0 || expert_begin > d->n_experts ||
      expert_count > d->n_experts - expert_begin)
    return MOE_ERR_RANGE;
  if (!aligned16(logical_codes) || !aligned16(logical_scales) || !aligned16(packed_codes) ||
      !aligned16(packed_scales))
    return MOE_ERR_ALIGN;
  size_t cb, sb;
  MOE_TRY(expert_bytes(d, &cb, &sb));
  if (sb % 16) return MOE_ERR_UNSUPPORTED;  // 3*H*I/32 is a multiple of 96 for H, I multiples of 32
  size_t c0, s0, cn, sn;
  if (!mul_ok(cb, (size_t)expert_begin, &c0) || !mul_ok(sb, (size_t)expert_begin, &s0) ||
      !mul_ok(cb, (size_t)expert_count, &cn) || !mul_ok(sb, (size_t)expert_count, &sn))
    return MOE_ERR_OVERFLOW;
  hipStream_t s = as_stream(stream);
  MOE_TRY(dev(moe::launch_copy(logical_codes, static_cast<char*>(packed_codes) + c0, cn, s)));
  MOE_TRY(dev(moe::launch_copy(logical_scales, static_cast<char*>(packed_scales) + s0, sn, s)));
  return MOE_OK;
}

moe_status moe_mxfp4_forward(const moe_layer_desc* d, const void* x, moe_dtype x_dtype, const float* router_w,
                      const float* router_bias, const void* packed_codes, const void* packed_scales,
                      int32_t n_tokens, int32_t k, float* out, float* logits_out, int32_t* topk_idx_out,
                      float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream) {
  FwdLayout L;
  MOE_TRY(check_forward_args(d, x, x_dtype, packed_codes, packed_scales, n_tokens, k, out, workspace,
                             workspace_bytes, &L));
  if (!router_w) return MOE_ERR_NULL;
  if (!aligned16(router_w)) return MOE_ERR_ALIGN;
  return forward_impl(d, x, x_dtype, router_w, router_bias, packed_codes, packed_scales, n_tokens, k,
                      out, logits_out, topk_idx_out, topk_w_out, workspace, L, nullptr, as_stream(stream));
}

moe_status moe_mxfp4_forward_noalloc(const moe_layer_desc* d, const void* x, moe_dtype x_dtype,
                                     const float* router_w, const float* router_bias, const void* packed_codes,
                                     const void* packed_scales, int32_t n_tokens, int32_t k, float* out,
                                     float* logits_out, int32_t* topk_idx_out, float* topk_w_out, void* stream) {
  FwdLayout L;
  MOE_TRY(check_forward_core(d, x, x_dtype, packed_codes, packed_scales, n_tokens, k, out, &L));
  if (!router_w) return MOE_ERR_NULL;
  if (!aligned16(router_w)) return MOE_ERR_ALIGN;
  if (L.total > kScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  MOE_TRY(scratch_address(&ws));
  return forward_impl(d, x, x_dtype, router_w, router_bias, packed_codes, packed_scales, n_tokens, k, out,
                      logits_out, topk_idx_out, topk_w_out, ws, L, nullptr, as_stream(stream));
}

moe_status moe_mxfp4_experts(const moe_layer_desc* d, const void* x, moe_dtype x_dtype, const int32_t* topk_idx,
                      const float* topk_w, const void* packed_codes, const void* packed_scales,
                      int32_t n_tokens, int32_t k, float* out, void* workspace, size_t workspace_bytes,
                      void* stream) {
  FwdLayout L;
  MOE_TRY(check_forward_args(d, x, x_dtype, packed_codes, packed_scales, n_tokens, k, out, workspace,
                             workspace_bytes, &L));
  if (!topk_idx || !topk_w) return MOE_ERR_NULL;
  return run_experts(d, x, x_dtype == MOE_DTYPE_F32, topk_idx, topk_w, packed_codes, packed_scales,
                     n_tokens, k, out, nullptr, static_cast<char*>(workspace), L, as_stream(stream));
}

moe_status moe_mxfp4_gate_up(const moe_layer_desc* d, const void* x, moe_dtype x_dtype, const int32_t* pair_expert,
                      int32_t n_pairs, int32_t k, const void* codes, const void* scales, float* h,
                      void* stream) {
  MOE_TRY(check_desc(d));
  if (!x || !pair_expert || !codes || !scales || !h) return MOE_ERR_NULL;
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (n_pairs < 1 || k < 1 || k > d->top_k_max || n_pairs > kMaxTokens * kMaxTopK) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MOE_ERR_ALIGN;
  return dev(moe::launch_gateup_gemv(x, x_dtype == MOE_DTYPE_F32, pair_expert, n_pairs, k,
                                     static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales),
                                     is_s4(d), d->hidden, d->inter, d->n_experts, h, as_stream(stream)));
}

moe_status moe_mxfp4_gate_up_select(const moe_layer_desc* d, const void* x, moe_dtype x_dtype, const float* logits,
                                    int32_t n_tokens, int32_t k, const void* codes, const void* scales,
                                    int32_t* topk_idx, float* topk_w, float* h, void* stream) {
  MOE_TRY(check_desc(d));
  if (!x || !logits || !codes || !scales || !topk_idx || !topk_w || !h) return MOE_ERR_NULL;
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  MOE_TRY(check_tokens(n_tokens, k, d));
  if ((int64_t)n_tokens * k > kMaxTokens * kMaxTopK) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales)) return MOE_ERR_ALIGN;
  return dev(moe::launch_gateup_select_gemv(x, x_dtype == MOE_DTYPE_F32, logits, n_tokens, k,
                                            static_cast<const uint8_t*>(codes), static_cast<const uint8_t*>(scales),
                                            is_s4(d), d->hidden, d->inter, d->n_experts, topk_idx, topk_w, h,
                                            as_stream(stream)));
}

moe_status moe_mxfp4_down(const moe_layer_desc* d, const float* h, const int32_t* pair_expert, int32_t n_pairs,
                   const void* codes, const void* scales, float* y, void* stream) {
  MOE_TRY(check_desc(d));
  if (!h || !pair_expert || !codes || !scales || !y) return MOE_ERR_NULL;
  if (n_pairs < 1 || n_pairs > kMaxTokens * kMaxTopK) return MOE_ERR_SHAPE;
  if (!aligned16(h) || !aligned16(codes) || !aligned16(scales)) return MOE_ERR_ALIGN;
  return dev(moe::launch_down_gemv(h, pair_expert, n_pairs, static_cast<const uint8_t*>(codes),
                                   static_cast<const uint8_t*>(scales), is_s4(d), d->hidden, d->inter, d->n_experts,
                                   y, as_stream(stream)));
}

moe_status moe_combine(const float* y, const float* w, int32_t n_tokens, int32_t k, int32_t hidden, const float* resid,
                float* out, void* stream) {
  if (!y || !w || !out) return MOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kMaxTokens || k < 1 || k > kMaxTopK || hidden < 4 || hidden % 4)
    return MOE_ERR_SHAPE;
  if (!aligned16(y) || !aligned16(out) || (resid && !aligned16(resid))) return MOE_ERR_ALIGN;
  return dev(moe::launch_combine(y, w, n_tokens, k, hidden, resid, out, as_stream(stream)));
}

moe_status moe_router_logits(const moe_layer_desc* d, const void* x, moe_dtype x_dtype, const float* router_w,
                      const float* router_bias, int32_t n_tokens, float* logits, void* stream) {
  MOE_TRY(check_desc(d));
  if (!x || !router_w || !logits) return MOE_ERR_NULL;
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (n_tokens < 1 || n_tokens > kMaxTokens) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(router_w)) return MOE_ERR_ALIGN;
  return dev(router(d, x, x_dtype == MOE_DTYPE_F32, router_w, router_bias, n_tokens, logits, nullptr,
                    as_stream(stream)));
}

moe_status moe_topk_softmax(const float* logits, int32_t n_tokens, int32_t n_experts, int32_t k, int32_t* idx,
                     float* w, void* stream) {
  if (!logits || !idx || !w) return MOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kMaxTokens || n_experts < 1 || k < 1 || k > n_experts || k > kMaxTopK)
    return MOE_ERR_SHAPE;
  if (n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  return dev(moe::launch_topk_softmax(logits, n_tokens, n_experts, k, idx, w, as_stream(stream)));
}

moe_status moe_sort_workspace_bytes(int32_t n_experts, int32_t n_tokens, int32_t k, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kMaxTokens || n_experts < 1 || k < 1 || k > n_experts || k > kMaxTopK)
    return MOE_ERR_SHAPE;
  if (n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  *bytes = moe::sort_workspace_bytes(n_tokens, n_experts);  // per-block counts for many tokens
  return MOE_OK;
}

moe_status moe_sort_by_expert(const int32_t* topk_idx, int32_t n_tokens, int32_t n_experts, int32_t k,
                       int32_t* expert_offsets, int32_t* pair_list, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!topk_idx || !expert_offsets || !pair_list) return MOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kMaxTokens || n_experts < 1 || k < 1 || k > n_experts || k > kMaxTopK)
    return MOE_ERR_SHAPE;
  if (n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)n_tokens * k > INT32_MAX) return MOE_ERR_OVERFLOW;
  const size_t need = moe::sort_workspace_bytes(n_tokens, n_experts);
  if (need > 0 && (!workspace || workspace_bytes < need)) return MOE_ERR_WORKSPACE;
  if (need > 0 && reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return MOE_ERR_ALIGN;
  return dev(moe::launch_sort_by_expert(topk_idx, n_tokens, n_experts, k, expert_offsets, pair_list,
                                        need > 0 ? workspace : nullptr, as_stream(stream)));
}

moe_status moe_max_expert_blocks(int32_t n_experts, int32_t n_pairs, int32_t* max_blocks) {
  if (!max_blocks) return MOE_ERR_NULL;
  if (n_experts < 1 || n_pairs < 1 || (int64_t)n_pairs > (int64_t)kMaxTokens * kMaxTopK) return MOE_ERR_SHAPE;
  if (n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  *max_blocks = moe::max_expert_blocks(n_pairs, n_experts);
  return MOE_OK;
}

moe_status moe_expert_blocks(const int32_t* expert_offsets, int32_t n_experts, int32_t n_pairs, int32_t* blocks,
                      int32_t max_blocks, int32_t* n_blocks, void* stream) {
  if (!expert_offsets || !blocks || !n_blocks) return MOE_ERR_NULL;
  if (n_experts < 1 || n_pairs < 1 || (int64_t)n_pairs > (int64_t)kMaxTokens * kMaxTopK) return MOE_ERR_SHAPE;
  if (n_experts > kMaxExperts) return MOE_ERR_UNSUPPORTED;
  if (max_blocks < moe::max_expert_blocks(n_pairs, n_experts)) return MOE_ERR_WORKSPACE;
  if (!aligned16(blocks)) return MOE_ERR_ALIGN;
  return dev(moe::launch_expert_blocks(expert_offsets, n_experts, max_blocks, reinterpret_cast<int4*>(blocks),
                                       n_blocks, as_stream(stream)));
}

moe_status moe_mxfp4_grouped_gate_up(const moe_layer_desc* d, const void* x, int32_t n_tokens, int32_t k,
                              const int32_t* pair_list, const int32_t* blocks, const int32_t* n_blocks,
                              int32_t max_blocks, const void* packed_codes, const void* packed_scales, void* hterm,
                              void* stream) {
  MOE_TRY(check_desc(d));
  if (is_s4(d)) return MOE_ERR_LAYOUT;  // the grouped GEMMs read the 8-bit table
  if (!x || !pair_list || !blocks || !n_blocks || !packed_codes || !packed_scales || !hterm) return MOE_ERR_NULL;
  MOE_TRY(check_tokens(n_tokens, k, d));
  const int64_t P = (int64_t)n_tokens * k;
  if (!grouped_fits(d, n_tokens, P)) return MOE_ERR_UNSUPPORTED;
  if (max_blocks < 1) return MOE_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(blocks) || !aligned16(packed_codes) || !aligned16(packed_scales) ||
      !aligned16(hterm))
    return MOE_ERR_ALIGN;
  return dev(moe::launch_gateup_mfma(static_cast<const uint16_t*>(x), n_tokens, pair_list,
                                     reinterpret_cast<const int4*>(blocks), n_blocks, max_blocks,
                                     static_cast<const uint8_t*>(packed_codes),
                                     static_cast<const uint8_t*>(packed_scales), d->hidden, d->inter, d->n_experts,
                                     k, (int)P, static_cast<uint16_t*>(hterm), as_stream(stream)));
}

moe_status moe_mxfp4_grouped_down(const moe_layer_desc* d, const void* hterm, int32_t n_pairs, const int32_t* pair_list,
                           const int32_t* blocks, const int32_t* n_blocks, int32_t max_blocks,
                           const void* packed_codes, const void* packed_scales, float* y, void* stream) {
  MOE_TRY(check_desc(d));
  if (is_s4(d)) return MOE_ERR_LAYOUT;  // the grouped GEMMs read the 8-bit table
  if (!hterm || !pair_list || !blocks || !n_blocks || !packed_codes || !packed_scales || !y) return MOE_ERR_NULL;
  if (n_pairs < 1 || (int64_t)n_pairs > (int64_t)kMaxTokens * kMaxTopK) return MOE_ERR_SHAPE;
  if (!grouped_fits(d, 1, n_pairs)) return MOE_ERR_UNSUPPORTED;
  if (max_blocks < 1) return MOE_ERR_SHAPE;
  if (!aligned16(hterm) || !aligned16(blocks) || !aligned16(packed_codes) || !aligned16(packed_scales) ||
      !aligned16(y))
    return MOE_ERR_ALIGN;
  return dev(moe::launch_down_mfma(static_cast<const uint16_t*>(hterm), pair_list,
                                   reinterpret_cast<const int4*>(blocks), n_blocks, max_blocks,
                                   static_cast<const uint8_t*>(packed_codes), static_cast<const uint8_t*>(packed_scales),
                                   d->hidden, d->inter, d->n_experts, n_pairs, y, as_stream(stream)));
}

static moe_status dequant_entry(const moe_layer_desc* d, const void* packed_codes, const void* packed_scales,
                                int64_t expert, int32_t matrix, float* out, bool via_bf16, void* stream) {
  MOE_TRY(check_desc(d));
  if (!packed_codes || !packed_scales || !out) return MOE_ERR_NULL;
  if (expert < 0 || expert >= d->n_experts || matrix < 0 || matrix > 2) return MOE_ERR_RANGE;
  if (!aligned16(packed_codes) || !aligned16(packed_scales) || !aligned16(out)) return MOE_ERR_ALIGN;
  size_t cb, sb;
  MOE_TRY(expert_bytes(d, &cb, &sb));
  const size_t mc = cb / 3;
  const int rows = matrix == 2 ? d->hidden : d->inter;
  const int cols = matrix == 2 ? d->inter : d->hidden;
  const uint8_t* c = static_cast<const uint8_t*>(packed_codes) + (size_t)expert * cb + (size_t)matrix * mc;
  const uint8_t* rec = static_cast<const uint8_t*>(packed_scales) + (size_t)expert * sb;
  if (is_s4(d)) {  // row bases gate [I] | up [I] | down [H], then deltas [rows][cols/64] per matrix
    const size_t I = (size_t)d->inter, H = (size_t)d->hidden, dm = I * H / 64;
    const uint8_t* base = rec + (matrix == 2 ? 2 * I : (size_t)matrix * I);
    const uint8_t* del = rec + 2 * I + H + (size_t)matrix * dm;
    return dev(moe::launch_dequant(c, del, base, rows, cols, out, via_bf16, as_stream(stream)));
  }
  const uint8_t* s = rec + (size_t)matrix * (sb / 3);
  return dev(moe::launch_dequant(c, s, nullptr, rows, cols, out, via_bf16, as_stream(stream)));
}

moe_status moe_mxfp4_dequant(const moe_layer_desc* d, const void* packed_codes, const void* packed_scales,
                             int64_t expert, int32_t matrix, float* out, void* stream) {
  return dequant_entry(d, packed_codes, packed_scales, expert, matrix, out, false, stream);
}

moe_status moe_mxfp4_dequant_bf16(const moe_layer_desc* d, const void* packed_codes, const void* packed_scales,
                                  int64_t expert, int32_t matrix, float* out, void* stream) {
  return dequant_entry(d, packed_codes, packed_scales, expert, matrix, out, true, stream);
}

moe_status moe_mxfp4_scale4_encode(const moe_layer_desc* d, const void* scales8, int64_t expert_begin,
                                   int64_t expert_count, void* scale4, int32_t* escapes, void* stream) {
  MOE_TRY(check_desc(d));
  if (!is_s4(d)) return MOE_ERR_LAYOUT;
  if (!scales8 || !scale4 || !escapes) return MOE_ERR_NULL;
  if (expert_begin < 0 || expert_count < 0 || expert_begin > d->n_experts ||
      expert_count > d->n_experts - expert_begin)
    return MOE_ERR_RANGE;
  if (!aligned16(scale4)) return MOE_ERR_ALIGN;
  return dev(moe::launch_scale4_encode(static_cast<const uint8_t*>(scales8), expert_begin, expert_count, d->hidden,
                                       d->inter, static_cast<uint8_t*>(scale4), escapes, as_stream(stream)));
}

moe_status moe_rmsnorm(const float* r, const float* gamma, float eps, int32_t n_tokens, int32_t hidden, float* n_out,
                void* stream) {
  if (!r || !gamma || !n_out) return MOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kMaxTokens || hidden < 4 || hidden % 4) return MOE_ERR_SHAPE;
  if (!aligned16(r) || !aligned16(gamma) || !aligned16(n_out)) return MOE_ERR_ALIGN;
  return dev(moe::launch_rmsnorm(r, gamma, eps, n_tokens, hidden, n_out, as_stream(stream)));
}

moe_status moe_residual_add(float* r, const float* dlt, int64_t n, void* stream) {
  if (!r || !dlt) return MOE_ERR_NULL;
  if (n < 0) return MOE_ERR_SHAPE;
  return dev(moe::launch_residual_add(r, dlt, (size_t)n, as_stream(stream)));
}

// ---------------------------------------------------------------- packed-int8 rows

static moe_status int8_check(const int8_t* q, const uint16_t* sc, int32_t rows, int32_t cols, const void* out) {
  if (!q || !sc || !out) return MOE_ERR_NULL;
  if (rows < 1 || rows > (1 << 20) || cols < 16 || cols % 16) return MOE_ERR_SHAPE;
  if (cols > 16384) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(out)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

moe_status moe_int8_gemv(const int8_t* q, const uint16_t* scales_f16, int32_t rows, int32_t cols, const void* x,
                         moe_dtype x_dtype, int32_t n_tokens, float* y, int32_t rows_per_workgroup, void* stream) {
  MOE_TRY(int8_check(q, scales_f16, rows, cols, y));
  if (!x) return MOE_ERR_NULL;
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (n_tokens < 1 || n_tokens > 4) return MOE_ERR_SHAPE;
  if (rows_per_workgroup < 0 || rows_per_workgroup % 8 || (int64_t)rows_per_workgroup * cols >= (int64_t{1} << 31))
    return MOE_ERR_SHAPE;
  const int rpw = rows_per_workgroup ? rows_per_workgroup : moe::int8_rows_per_wg(rows, cols);
  if ((size_t)n_tokens * rpw * ((cols + 1023) / 1024) * 4 > 65536) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(x)) return MOE_ERR_ALIGN;
  return dev(moe::launch_int8_gemv(q, scales_f16, rows, cols, x, x_dtype == MOE_DTYPE_F32, n_tokens, y, rpw,
                                   as_stream(stream)));
}

moe_status moe_int8_dequant(const int8_t* q, const uint16_t* scales_f16, int32_t rows, int32_t cols, float* out,
                            void* stream) {
  MOE_TRY(int8_check(q, scales_f16, rows, cols, out));
  return dev(moe::launch_int8_dequant(q, scales_f16, rows, cols, out, as_stream(stream)));
}

// ---------------------------------------------------------------- matrix-core rate

moe_status moe_mfma_rate(int32_t kind, const void* operands, int32_t n_workgroups, int32_t iters, float* sink,
                         void* stream) {
  if (kind < 0 || kind > 2) return MOE_ERR_UNSUPPORTED;
  if (!operands || !sink) return MOE_ERR_NULL;
  if (n_workgroups < 1 || n_workgroups > 65536 || iters < 1 || iters > 1000000) return MOE_ERR_SHAPE;
  if (!aligned16(operands) || !aligned16(sink)) return MOE_ERR_ALIGN;
  return dev(moe::launch_mfma_rate(kind, operands, n_workgroups, iters, sink, as_stream(stream)));
}

// ---------------------------------------------------------------- next-layer route hint

static moe_status hint_layout(const moe_layer_desc* d, int32_t T, int32_t k, size_t* nout_off, size_t* w_off,
                              size_t* total) {
  MOE_TRY(check_desc(d));
  MOE_TRY(check_tokens(T, k, d));
  size_t lg, nb, wb;
  if (!mul_ok((size_t)T * (size_t)d->n_experts, 4, &lg) || !mul_ok((size_t)T * (size_t)d->hidden, 4, &nb) ||
      !mul_ok((size_t)T * (size_t)k, 4, &wb))
    return MOE_ERR_OVERFLOW;
  Carve c;
  c.take(lg);
  *nout_off = c.take(nb);
  *w_off = c.take(wb);
  *total = c.take(0);
  return c.overflow ? MOE_ERR_OVERFLOW : MOE_OK;
}

moe_status moe_route_hint_workspace_bytes(const moe_layer_desc* d, int32_t n_tokens, int32_t k, size_t* bytes) {
  if (!bytes) return MOE_ERR_NULL;
  size_t a, b;
  return hint_layout(d, n_tokens, k, &a, &b, bytes);
}

moe_status moe_route_hint(const moe_layer_desc* d, const float* r, const float* gamma, float eps, const float* router_w,
                          const float* router_bias, int32_t n_tokens, int32_t k, int32_t* hint_idx, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!r || !gamma || !router_w || !hint_idx || !workspace) return MOE_ERR_NULL;
  size_t nout_off, w_off, total;
  MOE_TRY(hint_layout(d, n_tokens, k, &nout_off, &w_off, &total));
  if (d->hidden % 4 || d->hidden > 8192) return MOE_ERR_UNSUPPORTED;
  if (!aligned16(r) || !aligned16(gamma) || !aligned16(router_w) || !aligned16(workspace)) return MOE_ERR_ALIGN;
  if (workspace_bytes < total) return MOE_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* logits = reinterpret_cast<float*>(ws);
  hipStream_t s = as_stream(stream);
  MOE_TRY(dev(moe::launch_norm_router_logits(r, gamma, eps, router_w, router_bias, n_tokens, d->hidden, d->n_experts,
                                             logits, reinterpret_cast<float*>(ws + nout_off), s)));
  return dev(moe::launch_topk_softmax(logits, n_tokens, d->n_experts, k, hint_idx,
                                      reinterpret_cast<float*>(ws + w_off), s));
}

// ---------------------------------------------------------------- layer stack + graph

static moe_status stack_layout(const moe_layer_desc* d, int32_t T, int32_t k, FwdLayout* L, size_t* nbuf_off,
                        size_t* total) {
  MOE_TRY(forward_layout(d, T, k, L));
  size_t nb;
  if (!mul_ok((size_t)T * (size_t)d->hidden, 4, &nb)) return MOE_ERR_OVERFLOW;
  size_t a = (L->total + 255) & ~size_t(255);
  size_t t;
  if (!add_ok(a, nb, &t)) return MOE_ERR_OVERFLOW;
  *nbuf_off = a;
  *total = t;
  return MOE_OK;
}

moe_status moe_stack_workspace_bytes(const moe_layer_desc* d, int32_t n_tokens, int32_t k, size_t* bytes) {
  MOE_TRY(check_desc(d));
  if (!bytes) return MOE_ERR_NULL;
  MOE_TRY(check_tokens(n_tokens, k, d));
  FwdLayout L;
  size_t nb_off, total;
  MOE_TRY(stack_layout(d, n_tokens, k, &L, &nb_off, &total));
  *bytes = total;
  return MOE_OK;
}

static moe_status stack_check(const moe_layer_desc* d, int32_t n_layers, const void* const* codes,
                       const void* const* scales, const float* const* router_w, const float* const* gamma,
                       const void* x, moe_dtype x_dtype, int32_t T, int32_t k, const float* residual,
                       const void* ws, size_t ws_bytes, FwdLayout* L, size_t* nb_off) {
  MOE_TRY(check_desc(d));
  if (n_layers < 1 || n_layers > 4096) return MOE_ERR_SHAPE;
  if (!codes || !scales || !router_w || !gamma || !x || !residual) return MOE_ERR_NULL;
  if (x_dtype != MOE_DTYPE_F32 && x_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  MOE_TRY(check_tokens(T, k, d));
  for (int l = 0; l < n_layers; ++l) {
    if (!codes[l] || !scales[l] || !router_w[l] || !gamma[l]) return MOE_ERR_NULL;
    if (!aligned16(codes[l]) || !aligned16(scales[l]) || !aligned16(router_w[l]) || !aligned16(gamma[l]))
      return MOE_ERR_ALIGN;
  }
  if (!aligned16(x) || !aligned16(residual)) return MOE_ERR_ALIGN;
  size_t total;
  MOE_TRY(stack_layout(d, T, k, L, nb_off, &total));
  if (!ws) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  if (ws_bytes < total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

static moe_status stack_enqueue(const moe_layer_desc* d, int32_t n_layers, const void* const* codes,
                         const void* const* scales, const float* const* router_w,
                         const float* const* router_bias, const float* const* gamma, float eps,
                         const void* x, moe_dtype x_dtype, int32_t T, int32_t k, float* residual, void* ws,
                         const FwdLayout& L, size_t nb_off, hipStream_t s) {
  const size_t n = (size_t)T * d->hidden;
  float* nbuf = reinterpret_cast<float*>(static_cast<char*>(ws) + nb_off);
  MOE_TRY(dev(moe::launch_widen(x, x_dtype == MOE_DTYPE_F32, n, residual, s)));
  for (int l = 0; l < n_layers; ++l) {
    // RMSNorm runs inside the layer's router kernel (same bits as a separate pass), which leaves the
    // normalised rows in nbuf for the expert kernels
    const float* b = router_bias ? router_bias[l] : nullptr;
    MOE_TRY(forward_impl(d, residual, MOE_DTYPE_F32, router_w[l], b, codes[l], scales[l], T, k, residual,
                         nullptr, nullptr, nullptr, ws, L, residual, s, gamma[l], eps, nbuf));
  }
  return MOE_OK;
}

moe_status moe_mxfp4_stack_forward(const moe_layer_desc* d, int32_t n_layers, const void* const* codes,
                            const void* const* scales, const float* const* router_w,
                            const float* const* router_bias, const float* const* gamma, float eps,
                            const void* x, moe_dtype x_dtype, int32_t n_tokens, int32_t k, float* residual,
                            void* workspace, size_t workspace_bytes, void* stream) {
  FwdLayout L;
  size_t nb_off;
  MOE_TRY(stack_check(d, n_layers, codes, scales, router_w, gamma, x, x_dtype, n_tokens, k, residual,
                      workspace, workspace_bytes, &L, &nb_off));
  return stack_enqueue(d, n_layers, codes, scales, router_w, router_bias, gamma, eps, x, x_dtype, n_tokens,
                       k, residual, workspace, L, nb_off, as_stream(stream));
}

struct moe_stack_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

moe_status moe_stack_graph_create(const moe_layer_desc* d, int32_t n_layers, const void* const* codes,
                           const void* const* scales, const float* const* router_w,
                           const float* const* router_bias, const float* const* gamma, float eps,
                           const void* x, moe_dtype x_dtype, int32_t n_tokens, int32_t k, float* residual,
                           void* workspace, size_t workspace_bytes, void* stream, moe_stack_graph** out) {
  if (!out) return MOE_ERR_NULL;
  *out = nullptr;
  FwdLayout L;
  size_t nb_off;
  MOE_TRY(stack_check(d, n_layers, codes, scales, router_w, gamma, x, x_dtype, n_tokens, k, residual,
                      workspace, workspace_bytes, &L, &nb_off));
  // Capture on a private non-blocking stream (default priority) so the
  // caller's stream, which may be the null stream, is never in capture mode.
  hipStream_t cap = nullptr;
  if (hipStreamCreateWithFlags(&cap, hipStreamNonBlocking) != hipSuccess) return MOE_ERR_DEVICE;
  moe_status rc = MOE_OK;
  hipGraph_t g = nullptr;
  if (hipStreamBeginCapture(cap, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(cap);
    return MOE_ERR_DEVICE;
  }
  rc = stack_enqueue(d, n_layers, codes, scales, router_w, router_bias, gamma, eps, x, x_dtype, n_tokens, k,
                     residual, workspace, L, nb_off, cap);
  hipError_t ec = hipStreamEndCapture(cap, &g);
  (void)hipStreamDestroy(cap);
  if (rc != MOE_OK || ec != hipSuccess || !g) {
    if (g) (void)hipGraphDestroy(g);
    return rc != MOE_OK ? rc : MOE_ERR_DEVICE;
  }
  hipGraphExec_t ex = nullptr;
  if (hipGraphInstantiate(&ex, g, nullptr, nullptr, 0) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return MOE_ERR_DEVICE;
  }
  moe_stack_graph* h = new (std::nothrow) moe_stack_graph;
  if (!h) {
    (void)hipGraphExecDestroy(ex);
    (void)hipGraphDestroy(g);
    return MOE_ERR_DEVICE;
  }
  h->graph = g;
  h->exec = ex;
  (void)stream;
  *out = h;
  return MOE_OK;
}

moe_status moe_stack_graph_launch(moe_stack_graph* g, void* stream) {
  if (!g) return MOE_ERR_NULL;
  return dev(hipGraphLaunch(g->exec, as_stream(stream)));
}

moe_status moe_stack_graph_destroy(moe_stack_graph* g) {
  if (!g) return MOE_OK;
  moe_status rc = MOE_OK;
  if (g->exec && hipGraphExecDestroy(g->exec) != hipSuccess) rc = MOE_ERR_DEVICE;
  if (g->graph && hipGraphDestroy(g->graph) != hipSuccess) rc = MOE_ERR_DEVICE;
  delete g;
  return rc;
}

}  // extern "C"
