/*
 * Seeded, counter-based synthetic input generator.
 *
 * Shared by the tests, the benchmark and the CPU reference.  It holds none of
 * the MoE layer's arithmetic: it only produces bytes and floats with the
 * distributions of the workloads (uniform 4-bit codes, E8M0 scale bytes with a
 * uniform exponent, normal activations and router weights, uniform gains).
 *
 * Every value is a pure function of (seed, layer, tensor, item, index), so any
 * expert, token or row can be regenerated alone, on any thread count.
 *
 * Bits come from the SplitMix64 output function (G. Steele, D. Lea, C. Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) applied to a
 * Weyl-sequence counter: draw(key, i) = mix64(key + (i + 1) * golden_gamma).
 * Normals use the Box-Muller transform (cosine branch only), in double.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t draw(uint64_t key, uint64_t i) {
    return mix64(key + (i + 1) * GOLDEN_GAMMA);
}

/* Stream key for one tensor of one item (an expert, a token, a router row). */
uint64_t synth_key(uint64_t seed, uint32_t layer, uint32_t tensor, uint64_t item) {
    uint64_t tag = ((uint64_t)layer << 48) ^ ((uint64_t)tensor << 40) ^ item ^ 0x6A09E667F3BCC909ULL;
    return mix64(seed ^ mix64(tag));
}

uint64_t synth_draw(uint64_t key, uint64_t i) { return draw(key, i); }

/* n uniform random bytes: byte j is byte (j % 8) of draw(key, j / 8).
 * Used for 4-bit code arrays: both nibbles of every byte are uniform over 0..15. */
void synth_bytes(uint64_t key, uint64_t n, uint8_t* out) {
    uint64_t full = n / 8;
    #pragma omp parallel for schedule(static) if (n > (1u << 20))
    for (int64_t w = 0; w < (int64_t)full; ++w) {
        uint64_t v = draw(key, (uint64_t)w);
        for (int b = 0; b < 8; ++b) out[w * 8 + b] = (uint8_t)(v >> (8 * b));
    }
    if (full * 8 < n) {
        uint64_t v = draw(key, full);
        for (uint64_t j = full * 8; j < n; ++j) out[j] = (uint8_t)(v >> (8 * (j % 8)));
    }
}

/* n bytes, each lo + floor(span * u) with u uniform in [0,1): the integer form
 * ((draw >> 32) * span) >> 32 is exact.  Scale bytes with a uniform exponent. */
void synth_uint_range(uint64_t key, uint64_t n, uint32_t lo, uint32_t span, uint8_t* out) {
    #pragma omp parallel for schedule(static) if (n > (1u << 20))
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        uint64_t v = draw(key, (uint64_t)j) >> 32;
        out[j] = (uint8_t)(lo + ((v * span) >> 32));
    }
}

/* n floats ~ N(mean, std^2): Box-Muller in double on draws 2j and 2j+1, then
 * rounded to fp32. */
void synth_normal_f32(uint64_t key, uint64_t n, double mean, double std, float* out) {
    const double two_pi = 6.283185307179586476925286766559;
    #pragma omp parallel for schedule(static) if (n > (1u << 16))
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        double u1 = ((double)((draw(key, 2 * (uint64_t)j) >> 11) + 1)) * 0x1.0p-53; /* (0,1] */
        double u2 = ((double)(draw(key, 2 * (uint64_t)j + 1) >> 11)) * 0x1.0p-53;   /* [0,1) */
        double z = sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
        out[j] = (float)(mean + std * z);
    }
}

/* n floats uniform in [lo, hi), from the top 53 bits of one draw each. */
void synth_uniform_f32(uint64_t key, uint64_t n, double lo, double hi, float* out) {
    #pragma omp parallel for schedule(static) if (n > (1u << 16))
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        double u = (double)(draw(key, (uint64_t)j) >> 11) * 0x1.0p-53;
        out[j] = (float)(lo + (hi - lo) * u);
    }
}

/* fp32 -> bf16 bit pattern, round to nearest even (NaN kept quiet). */
void synth_f32_to_bf16(const float* in, uint64_t n, uint16_t* out) {
    #pragma omp parallel for schedule(static) if (n > (1u << 20))
    for (int64_t j = 0; j < (int64_t)n; ++j) {
        union { float f; uint32_t u; } c;
        c.f = in[j];
        uint32_t u = c.u;
        if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) {
            out[j] = (uint16_t)((u >> 16) | 0x0040u);
        } else {
            uint32_t r = 0x7FFFu + ((u >> 16) & 1u);
            out[j] = (uint16_t)((u + r) >> 16);
        }
    }
}

/* Tensor ids inside the key (kept in step with synth/__init__.py). */
enum { T_X = 1, T_ROUTER_W = 2, T_GATE_CODES = 3, T_UP_CODES = 4, T_DOWN_CODES = 5,
       T_GATE_SCALES = 6, T_UP_SCALES = 7, T_DOWN_SCALES = 8 };

/* One expert in the logical layout.
 * codes_e : gate [inter][hidden/2] | up [inter][hidden/2] | down [hidden][inter/2]
 * scales_e: gate [inter][hidden/32] | up [inter][hidden/32] | down [hidden][inter/32]
 * Scale bytes are 119 + uniform{0..4} (block exponents -8..-4). */
static void expert_one(uint64_t seed, uint32_t layer, int64_t hidden, int64_t inter, uint64_t e,
                       uint8_t* codes_e, uint8_t* scales_e) {
    uint64_t mc = (uint64_t)inter * (uint64_t)hidden / 2, ms = (uint64_t)inter * (uint64_t)hidden / 32;
    synth_bytes(synth_key(seed, layer, T_GATE_CODES, e), mc, codes_e);
    synth_bytes(synth_key(seed, layer, T_UP_CODES, e), mc, codes_e + mc);
    synth_bytes(synth_key(seed, layer, T_DOWN_CODES, e), mc, codes_e + 2 * mc);
    synth_uint_range(synth_key(seed, layer, T_GATE_SCALES, e), ms, 119, 5, scales_e);
    synth_uint_range(synth_key(seed, layer, T_UP_SCALES, e), ms, 119, 5, scales_e + ms);
    synth_uint_range(synth_key(seed, layer, T_DOWN_SCALES, e), ms, 119, 5, scales_e + 2 * ms);
}

void synth_expert(uint64_t seed, uint32_t layer, int64_t hidden, int64_t inter, uint64_t e,
                  uint8_t* codes_e, uint8_t* scales_e) {
    expert_one(seed, layer, hidden, inter, e, codes_e, scales_e);
}

/* Experts [e0, e0 + count) packed back to back into codes / scales. */
void synth_experts(uint64_t seed, uint32_t layer, int64_t hidden, int64_t inter, uint64_t e0,
                   uint64_t count, uint8_t* codes, uint8_t* scales) {
    uint64_t cb = 3ull * (uint64_t)inter * (uint64_t)hidden / 2;
    uint64_t sb = 3ull * (uint64_t)inter * (uint64_t)hidden / 32;
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t j = 0; j < (int64_t)count; ++j)
        expert_one(seed, layer, hidden, inter, e0 + (uint64_t)j, codes + (uint64_t)j * cb,
                   scales + (uint64_t)j * sb);
}
