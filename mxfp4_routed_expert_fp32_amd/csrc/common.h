// Device helpers shared by the gfx950 kernels of libmoe_mxfp4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

namespace moe {

constexpr int kWave = 64;

// E8M0 scale byte as the fp32 scale operand of the gfx950 scaled conversions:
// the byte sits in the fp32 exponent field (the hardware reads it as 2^(S-127),
// S = 0 included, S = 0xFF as NaN).
__device__ __forceinline__ float e8m0_operand(uint32_t s) { return __uint_as_float(s << 23); }

// Two E2M1 codes (byte `SEL` of `codes`: low nibble = even element) times the
// block scale, as exact fp32 values.  The hardware conversion gives exactly
// E2M1(code) * 2^(S-127), rounded to +-inf on overflow and subnormal where
// small; for S = 0xFF it gives a NaN (sign bit set).
template <int SEL>
__device__ __forceinline__ f32x2 fp4x2_to_f32(uint32_t codes, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, scale, SEL);
}

// Same, as bf16 (exact: every finite E2M1 value times 2^(S-127) fits bf16).
template <int SEL>
__device__ __forceinline__ bf16x2 fp4x2_to_bf16(uint32_t codes, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, SEL);
}

// acc + a.x*b.x + a.y*b.y with bf16 products exact in fp32.
__device__ __forceinline__ float dot2_bf16(bf16x2 a, bf16x2 b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) {
  bf16x2 r;
  __builtin_memcpy(&r, &u, 4);
  return r;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// 8 bf16 weights: dword `dw` of a 16-byte code block (8 codes) times the
// block scale, exact.
__device__ __forceinline__ bf16x8 decode8(uint32_t dw, float s) {
  const bf16x2 a = fp4x2_to_bf16<0>(dw, s), b = fp4x2_to_bf16<1>(dw, s);
  const bf16x2 c = fp4x2_to_bf16<2>(dw, s), d = fp4x2_to_bf16<3>(dw, s);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  bf16x8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0x007FFFFFu) ? 0x40u : 0u));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}


// Sum over groups of G consecutive lanes (G a power of two <= 64); every lane
// of a group ends with the group's sum.  The butterfly order is fixed, so the
// result is deterministic.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < G; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ uint4 load_u4(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// Non-temporal 16-byte load for weights that are streamed once.
__device__ __forceinline__ uint4 load_u4_stream(const uint8_t* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  u32x4 v = __builtin_nontemporal_load(q);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

}  // namespace moe

namespace moe {

// DPP lane permutations (GFX9 encodings): quad_perm, row mirrors, row
// broadcasts.  update_dpp with old = 0 leaves lanes of disabled rows at 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Every lane of each 16-lane row receives the row's sum (fixed order).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);  // row_half_mirror
  v += dpp_f<0x140>(v);  // row_mirror
  return v;
}

// Sum over groups of G = 4, 8 or 16 consecutive lanes, every lane of a group
// receiving its group's sum.
template <int G>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(G == 4 || G == 8 || G == 16, "group size");
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  if constexpr (G >= 8) v += dpp_f<0x141>(v);
  if constexpr (G >= 16) v += dpp_f<0x140>(v);
  return v;
}

// Full-wavefront sum, returned in every lane (uniform).
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += dpp_f<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

}  // namespace moe
