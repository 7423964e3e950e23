/*
 * CPU oracle for the routed MXFP4 mixture-of-experts layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  It shares no code,
 * header, table or constant generator with the GPU library, and the GPU library
 * never calls it.
 *
 * Plain, slow and written to be checked by eye: every reduction is a single
 * sequential fp32 loop in ascending index order (compiled with
 * -ffp-contract=off, so each step is a separate IEEE multiply and add), and
 * threads only split independent outputs, so results do not depend on the
 * thread count.
 *
 * Sources for what is computed (web pages on the Deltafin project):
 *  - "Deltafin's custom compiled runtime", section "Weight fidelity": expert
 *    weights stay in their released MXFP4 form, target activations stay fp32,
 *    and all selected experts run (no top-k truncation).
 *  - same page, section "Complete target sequence tape": routing hands on the
 *    top-16 expert ids in route order together with their fp32 weights.
 *  - brain.bigb.es "deltafin", section "The techniques that bought the 82x":
 *    the MXFP4 kernel decodes each 4-bit code through a 16-entry table and
 *    applies the E8M0 block scale to the fp32 exponent; all six tensors of an
 *    expert (gate/up/down codes and scales) form one contiguous range.
 *  - "Tarfa EXACTNESS" page, opening list: router top-k is the model's own k,
 *    logits are fp32 with fp32 accumulation.
 * Readings where the pages are silent (table values, nibble order, block axis,
 * gating function, SwiGLU form, matrix orientation, tie order) are stated next
 * to the code that takes them.
 *
 * Parity status of each function is pinned by tests that do not call back
 * into this file's formulas (see the test suite's oracle pin module).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- MXFP4 values */

/* E2M1 value of a 4-bit code, from its bit fields (OCP Microscaling Formats v1.0,
 * FP4 E2M1): bit 3 = sign, bits 2..1 = exponent with bias 1, bit 0 = mantissa.
 * Exponent field 0 is the subnormal case 0.5 * mantissa.  The 16 results form
 * the decode table the pages describe. */
static float e2m1_from_bits(unsigned code) {
    unsigned sign = (code >> 3) & 1u, ex = (code >> 1) & 3u, man = code & 1u;
    double mag = (ex == 0) ? 0.5 * (double)man : ldexp(1.0 + 0.5 * (double)man, (int)ex - 1);
    return (float)(sign ? -mag : mag);
}

void oracle_e2m1_table(float table[16]) {
    for (unsigned c = 0; c < 16; ++c) table[c] = e2m1_from_bits(c);
}

/* E8M0 scale byte -> fp32: 2^(S-127); S = 0xFF is NaN (returned as the
 * canonical quiet NaN 0x7FC00000).  S = 0 gives the subnormal 2^-127. */
float oracle_e8m0_to_f32(uint8_t s) {
    if (s == 0xFF) {
        union { uint32_t u; float f; } c = {0x7FC00000u};
        return c.f;
    }
    return ldexpf(1.0f, (int)s - 127);
}

/* One dequantised element: table value times block scale, as an fp32 product.
 * Every E2M1 value has at most two significant bits, so the product is exact
 * whenever it is representable (subnormal results included) and rounds to
 * +-inf when it is not.  A NaN scale gives the canonical NaN whatever the code. */
static float mx_value(const float table[16], unsigned code, uint8_t s) {
    if (s == 0xFF) return oracle_e8m0_to_f32(s);
    return table[code & 0xFu] * oracle_e8m0_to_f32(s);
}

/* Dequantise a [rows][cols] MXFP4 matrix in the logical layout:
 *   codes [rows][cols/2]: element c of a row is the low nibble of byte c/2 when
 *                         c is even and the high nibble when c is odd;
 *   scales[rows][cols/32]: one E8M0 byte per 32 consecutive elements along the
 *                          row (the reduction axis K).
 * cols must be a multiple of 32. */
void oracle_dequant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                    float* out) {
    float table[16];
    oracle_e2m1_table(table);
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < rows; ++n) {
        for (int64_t c = 0; c < cols; ++c) {
            uint8_t byte = codes[n * (cols / 2) + c / 2];
            unsigned nib = (byte >> (4 * (c & 1))) & 0xFu;
            out[n * cols + c] = mx_value(table, nib, scales[n * (cols / 32) + c / 32]);
        }
    }
}

/* ---------------------------------------------------------------- bf16 input */

/* bf16 -> fp32 by placing the 16 bits in the top half (exact). */
void oracle_bf16_to_f32(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) {
        union { uint32_t u; float f; } c;
        c.u = (uint32_t)in[i] << 16;
        out[i] = c.f;
    }
}

/* ---------------------------------------------------------------- router */

/* logits[t][e] = sum_h x[t][h] * W[e][h]  (+ bias[e]), fp32, ascending h. */
void oracle_router_logits(const float* x, int64_t T, int64_t H, const float* w_router,
                          const float* bias, int64_t E, float* logits) {
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            float acc = 0.0f;
            for (int64_t h = 0; h < H; ++h) acc = acc + x[t * H + h] * w_router[e * H + h];
            if (bias) acc = acc + bias[e];
            logits[t * E + e] = acc;
        }
    }
}

/* Rank order used for selection: a higher logit ranks first; equal logits
 * (IEEE ==, so -0 equals +0) rank by lower expert index; NaN ranks below every
 * number, -inf included, and NaNs among themselves by index. */
static int ranks_before(float a, int64_t ia, float b, int64_t ib) {
    int an = isnan(a), bn = isnan(b);
    if (an || bn) {
        if (an && bn) return ia < ib;
        return bn; /* the non-NaN one ranks first */
    }
    if (a > b) return 1;
    if (a < b) return 0;
    return ia < ib;
}

/* idx[t][0..k) = the k experts first in rank order, listed in rank order.
 * All k selected experts are kept (no capacity limit, no dropping). */
void oracle_topk(const float* logits, int64_t T, int64_t E, int64_t k, int32_t* idx) {
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        unsigned char* taken = (unsigned char*)calloc((size_t)E, 1);
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || ranks_before(l[e], e, l[best], best)) best = e;
            }
            taken[best] = 1;
            idx[t * k + j] = (int32_t)best;
        }
        free(taken);
    }
}

/* Combine weights: softmax over the k selected logits (the plainest gating the
 * workloads name), w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), sum in
 * ascending rank order. */
void oracle_softmax_selected(const float* logits, const int32_t* idx, int64_t T, int64_t E,
                             int64_t k, float* w) {
    float* ex = (float*)malloc(sizeof(float) * (size_t)(k > 0 ? k : 1));
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        float m = l[idx[t * k + 0]];
        float s = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            ex[j] = expf(l[idx[t * k + j]] - m);
            s = s + ex[j];
        }
        for (int64_t j = 0; j < k; ++j) w[t * k + j] = ex[j] / s;
    }
    free(ex);
}

/* ---------------------------------------------------------------- expert FFN */

/* y = Wd (silu(Wg x) * (Wu x)) for one token and one expert, all fp32:
 *   g[i] = sum_h x[h] Wg[i][h], u[i] = sum_h x[h] Wu[i][h]   (ascending h)
 *   a[i] = (g[i] / (1 + exp(-g[i]))) * u[i]                  (silu on the gate)
 *   y[n] = sum_i a[i] Wd[n][i]                                (ascending i)
 * Wg, Wu are [I][H] and Wd is [H][I]: [out_features][in_features]. */
static void expert_ffn(const float* x, int64_t H, int64_t I, const float* wg, const float* wu,
                       const float* wd, float* a, float* y) {
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < I; ++i) {
        float g = 0.0f, u = 0.0f;
        for (int64_t h = 0; h < H; ++h) g = g + x[h] * wg[i * H + h];
        for (int64_t h = 0; h < H; ++h) u = u + x[h] * wu[i * H + h];
        a[i] = (g / (1.0f + expf(-g))) * u;
    }
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < H; ++n) {
        float acc = 0.0f;
        for (int64_t i = 0; i < I; ++i) acc = acc + a[i] * wd[n * I + i];
        y[n] = acc;
    }
}

/* ---------------------------------------------------------------- the layer */

/*
 * out[t] = sum_{j<k} w[t][j] * FFN_{idx[t][j]}(x[t]), summed in ascending rank j.
 *
 *   x           [T][H] fp32 (bf16 inputs widened exactly beforehand)
 *   w_router    [E][H] fp32;  bias [E] or NULL (added to the logits, so it
 *               moves both the selection and the weights)
 *   codes_e[e]  one expert's codes:  gate [I][H/2] | up [I][H/2] | down [H][I/2]
 *   scales_e[e] one expert's scales: gate [I][H/32] | up [I][H/32] | down [H][I/32]
 *               (pointers of experts that are never selected may be NULL)
 *   logits_override [T][E] or NULL: when given, selection and weights use these
 *               logits instead of the ones computed here (comparing two
 *               implementations on identical logits)
 *   out [T][H]; logits_out [T][E], idx_out [T][k], w_out [T][k] may be NULL.
 * Returns 0, -1 on a shape error, -2 when a selected expert has no data, -3 on
 * allocation failure.
 */
int oracle_moe_forward(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, const float* x,
                       const float* w_router, const float* bias, const uint8_t* const* codes_e,
                       const uint8_t* const* scales_e, const float* logits_override, float* out,
                       float* logits_out, int32_t* idx_out, float* w_out, int nthreads) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k < 1 || k > E || H % 32 || I % 32) return -1;
#ifdef _OPENMP
    int saved = omp_get_max_threads();
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int rc = 0;
    float* logits = (float*)malloc(sizeof(float) * (size_t)(T * E + 1));
    int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)(T * k + 1));
    float* w = (float*)malloc(sizeof(float) * (size_t)(T * k + 1));
    float* wg = (float*)malloc(sizeof(float) * (size_t)(I * H));
    float* wu = (float*)malloc(sizeof(float) * (size_t)(I * H));
    float* wd = (float*)malloc(sizeof(float) * (size_t)(H * I));
    float* a = (float*)malloc(sizeof(float) * (size_t)I);
    float* y = (float*)malloc(sizeof(float) * (size_t)(T * k * H + 1));
    if (!logits || !idx || !w || !wg || !wu || !wd || !a || !y) { rc = -3; goto done; }

    if (logits_override)
        memcpy(logits, logits_override, sizeof(float) * (size_t)(T * E));
    else
        oracle_router_logits(x, T, H, w_router, bias, E, logits);
    oracle_topk(logits, T, E, k, idx);
    oracle_softmax_selected(logits, idx, T, E, k, w);

    /* Each distinct selected expert is dequantised once, then applied to every
     * (token, rank) pair that selected it. */
    for (int64_t e = 0; e < E; ++e) {
        int used = 0;
        for (int64_t p = 0; p < T * k; ++p) used |= (idx[p] == e);
        if (!used) continue;
        if (!codes_e[e] || !scales_e[e]) { rc = -2; goto done; }
        const uint8_t* c = codes_e[e];
        const uint8_t* s = scales_e[e];
        oracle_dequant(c, s, I, H, wg);
        oracle_dequant(c + I * H / 2, s + I * H / 32, I, H, wu);
        oracle_dequant(c + 2 * (I * H / 2), s + 2 * (I * H / 32), H, I, wd);
        for (int64_t p = 0; p < T * k; ++p)
            if (idx[p] == e) expert_ffn(x + (p / k) * H, H, I, wg, wu, wd, a, y + p * H);
    }
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < H; ++n) {
            float acc = 0.0f;
            for (int64_t j = 0; j < k; ++j) acc = acc + w[t * k + j] * y[(t * k + j) * H + n];
            out[t * H + n] = acc;
        }
    }
    if (logits_out) memcpy(logits_out, logits, sizeof(float) * (size_t)(T * E));
    if (idx_out) memcpy(idx_out, idx, sizeof(int32_t) * (size_t)(T * k));
    if (w_out) memcpy(w_out, w, sizeof(float) * (size_t)(T * k));
done:
    free(logits); free(idx); free(w); free(wg); free(wu); free(wd); free(a); free(y);
#ifdef _OPENMP
    omp_set_num_threads(saved);
#endif
    return rc;
}

/*
 * The expert part of the layer with the routing given: out[t] = sum_{j<k}
 * w[t][j] * FFN_{idx[t][j]}(x[t]), summed in ascending rank j, with the FFN
 * of expert_ffn.  This is the layer above with its router, top-k and softmax
 * steps replaced by given ids and weights ("Deltafin's custom compiled
 * runtime", section "Complete target sequence tape": the provider receives
 * the route and its fp32 weights).  Ids must lie in [0, E); a row may repeat
 * an id.  Returns 0, -1 on a shape or id error, -2 when a used expert has no
 * data, -3 on allocation failure.
 */
int oracle_moe_experts(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, const float* x,
                       const int32_t* idx, const float* w, const uint8_t* const* codes_e,
                       const uint8_t* const* scales_e, float* out, int nthreads) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k < 1 || H % 32 || I % 32) return -1;
    for (int64_t p = 0; p < T * k; ++p)
        if (idx[p] < 0 || idx[p] >= E) return -1;
#ifdef _OPENMP
    int saved = omp_get_max_threads();
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int rc = 0;
    float* wg = (float*)malloc(sizeof(float) * (size_t)(I * H));
    float* wu = (float*)malloc(sizeof(float) * (size_t)(I * H));
    float* wd = (float*)malloc(sizeof(float) * (size_t)(H * I));
    float* a = (float*)malloc(sizeof(float) * (size_t)I);
    float* y = (float*)malloc(sizeof(float) * (size_t)(T * k * H + 1));
    if (!wg || !wu || !wd || !a || !y) { rc = -3; goto done; }
    for (int64_t e = 0; e < E; ++e) {
        int used = 0;
        for (int64_t p = 0; p < T * k; ++p) used |= (idx[p] == e);
        if (!used) continue;
        if (!codes_e[e] || !scales_e[e]) { rc = -2; goto done; }
        const uint8_t* c = codes_e[e];
        const uint8_t* s = scales_e[e];
        oracle_dequant(c, s, I, H, wg);
        oracle_dequant(c + I * H / 2, s + I * H / 32, I, H, wu);
        oracle_dequant(c + 2 * (I * H / 2), s + 2 * (I * H / 32), H, I, wd);
        for (int64_t p = 0; p < T * k; ++p)
            if (idx[p] == e) expert_ffn(x + (p / k) * H, H, I, wg, wu, wd, a, y + p * H);
    }
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < H; ++n) {
            float acc = 0.0f;
            for (int64_t j = 0; j < k; ++j) acc = acc + w[t * k + j] * y[(t * k + j) * H + n];
            out[t * H + n] = acc;
        }
    }
done:
    free(wg); free(wu); free(wd); free(a); free(y);
#ifdef _OPENMP
    omp_set_num_threads(saved);
#endif
    return rc;
}

/* ---------------------------------------------------------------- error scale */

/*
 * Magnitude scale of each output element, for an elementwise reading of the
 * relative error bar: the layer's last two steps with every input replaced by
 * its absolute value, A[t][n] = sum_j |w[t][j]| sum_i |h_j[i]| |Wd_j[n][i]|,
 * where h_j = silu(Wg_j x[t]) * (Wu_j x[t]) is the intermediate this oracle
 * computes (expert_ffn) and the sums run in double.  A sum evaluated in fp32
 * in any order differs from the exact one by a small multiple of eps times
 * the sum of its terms' magnitudes, so |gpu - oracle| <= tol * A is a
 * per-element bar that stays meaningful where the output itself cancels
 * towards 0.  Not part of the layer's definition: test infrastructure for the
 * comparison.  Same arguments as oracle_moe_experts; A is [T][H] double.
 */
int oracle_moe_abs_scale(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, const float* x,
                         const int32_t* idx, const float* w, const uint8_t* const* codes_e,
                         const uint8_t* const* scales_e, double* A, int nthreads) {
    if (T < 0 || H <= 0 || I <= 0 || E <= 0 || k < 1 || H % 32 || I % 32) return -1;
    for (int64_t p = 0; p < T * k; ++p)
        if (idx[p] < 0 || idx[p] >= E) return -1;
#ifdef _OPENMP
    int saved = omp_get_max_threads();
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int rc = 0;
    float* wg = (float*)malloc(sizeof(float) * (size_t)(I * H));
    float* wu = (float*)malloc(sizeof(float) * (size_t)(I * H));
    float* wd = (float*)malloc(sizeof(float) * (size_t)(H * I));
    float* a = (float*)malloc(sizeof(float) * (size_t)I);
    float* ytmp = (float*)malloc(sizeof(float) * (size_t)H);
    double* y = (double*)malloc(sizeof(double) * (size_t)(T * k * H + 1));
    if (!wg || !wu || !wd || !a || !ytmp || !y) { rc = -3; goto done; }
    for (int64_t e = 0; e < E; ++e) {
        int used = 0;
        for (int64_t p = 0; p < T * k; ++p) used |= (idx[p] == e);
        if (!used) continue;
        if (!codes_e[e] || !scales_e[e]) { rc = -2; goto done; }
        const uint8_t* c = codes_e[e];
        const uint8_t* s = scales_e[e];
        oracle_dequant(c, s, I, H, wg);
        oracle_dequant(c + I * H / 2, s + I * H / 32, I, H, wu);
        oracle_dequant(c + 2 * (I * H / 2), s + 2 * (I * H / 32), H, I, wd);
        for (int64_t p = 0; p < T * k; ++p) {
            if (idx[p] != e) continue;
            expert_ffn(x + (p / k) * H, H, I, wg, wu, wd, a, ytmp);  /* a = h of this pair */
            #pragma omp parallel for schedule(static)
            for (int64_t n = 0; n < H; ++n) {
                double acc = 0.0;
                for (int64_t i = 0; i < I; ++i) acc += fabs((double)a[i]) * fabs((double)wd[n * I + i]);
                y[p * H + n] = acc;
            }
        }
    }
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < H; ++n) {
            double acc = 0.0;
            for (int64_t j = 0; j < k; ++j) acc += fabs((double)w[t * k + j]) * y[(t * k + j) * H + n];
            A[t * H + n] = acc;
        }
    }
done:
    free(wg); free(wu); free(wd); free(a); free(ytmp); free(y);
#ifdef _OPENMP
    omp_set_num_threads(saved);
#endif
    return rc;
}

/* ---------------------------------------------------------------- packed-int8 rows */

/* IEEE binary16 -> fp32, from the bit fields: sign bit 15, exponent bits 14-10
 * (bias 15), mantissa bits 9-0; exponent 0 is subnormal (mantissa * 2^-24),
 * exponent 31 is inf (mantissa 0) or NaN.  Every binary16 value is exact in
 * fp32. */
float oracle_f16_to_f32(uint16_t h) {
    unsigned sign = (h >> 15) & 1u, ex = (h >> 10) & 0x1Fu, man = h & 0x3FFu;
    double mag;
    if (ex == 0x1Fu) {
        if (man) return NAN;
        mag = INFINITY;
    } else if (ex == 0) {
        mag = ldexp((double)man, -24);
    } else {
        mag = ldexp(1.0 + (double)man / 1024.0, (int)ex - 15);
    }
    return (float)(sign ? -mag : mag);
}

/* A resident-spine matrix in packed int8 with one fp16 scale per row (the
 * pages' explicit int8 spine: row rounding and fp16 scales, so not
 * weight-exact with respect to the source weights; "Deltafin's custom
 * compiled runtime", section "Weight fidelity"): W[n][k] = q[n][k] * s[n].
 * The product of an int8 and a binary16 value has at most 7 + 11 significant
 * bits, so it is exact in fp32 (brain.bigb.es "deltafin", section "The
 * techniques that bought the 82x": the fused int8 -> fp32 + scale copy
 * reproduces the weights with max|diff| = 0). */
void oracle_int8_dequant(const int8_t* q, const uint16_t* s, int64_t rows, int64_t cols, float* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < rows; ++n) {
        float sc = oracle_f16_to_f32(s[n]);
        for (int64_t c = 0; c < cols; ++c) out[n * cols + c] = (float)q[n * cols + c] * sc;
    }
}

/* y[t][n] = sum_k W[n][k] * x[t][k], W as oracle_int8_dequant, fp32, ascending k. */
void oracle_int8_gemv(const int8_t* q, const uint16_t* s, int64_t rows, int64_t cols, const float* x,
                      int64_t T, float* y) {
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t n = 0; n < rows; ++n) {
            float sc = oracle_f16_to_f32(s[n]);
            float acc = 0.0f;
            for (int64_t k = 0; k < cols; ++k) acc = acc + ((float)q[n * cols + k] * sc) * x[t * cols + k];
            y[t * rows + n] = acc;
        }
    }
}

/* ---------------------------------------------------------------- stack parts */

/* RMSNorm with gain: n = r * (1 / sqrt(mean(r^2) + eps)) * gamma, per token;
 * the mean is an ascending fp32 sum divided by H. */
void oracle_rmsnorm(const float* r, const float* gamma, float eps, int64_t T, int64_t H, float* n) {
    for (int64_t t = 0; t < T; ++t) {
        float ss = 0.0f;
        for (int64_t h = 0; h < H; ++h) ss = ss + r[t * H + h] * r[t * H + h];
        float inv = 1.0f / sqrtf(ss / (float)H + eps);
        for (int64_t h = 0; h < H; ++h) n[t * H + h] = (r[t * H + h] * inv) * gamma[h];
    }
}

/* Residual update r += d, elementwise fp32. */
void oracle_residual_add(float* r, const float* d, int64_t n) {
    for (int64_t i = 0; i < n; ++i) r[i] = r[i] + d[i];
}
