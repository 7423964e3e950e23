// Weight pack (device layout copy), dequant export, RMSNorm and residual add.
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------- pack
// The device layout equals the logical row-major layout, so packing a run of
// experts is a 16-byte-vector copy into their place in the layer buffers.
__global__ __launch_bounds__(256) void k_copy16(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                size_t n16) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    dst[i] = src[i];
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  k_copy16<<<dim3((unsigned)blocks), 256, 0, s>>>(static_cast<const uint4*>(src),
                                                  static_cast<uint4*>(dst), n16);
  return hipGetLastError();
}

// ---------------------------------------------------------------- dequant export
// Two exports of E2M1(code) * 2^(S-127), one per gfx950 scaled conversion the
// expert kernels use; each thread decodes 8 elements (one 32-bit word of
// codes).
//  - k_dequant: v_cvt_scalef32_pk_f32_fp4, the conversion of the fp32-operand
//    GEMVs (fp32 activations, and the down projection of the decode form),
//    with the NaN scale byte 0xFF written as the canonical quiet NaN
//    0x7FC00000.
//  - k_dequant_bf16: decode8 (v_cvt_scalef32_pk_bf16_fp4), the conversion of
//    the bf16-activation decode GEMV and of both MFMA kernels, widened to fp32
//    by placing the 16 bits in the top half.  Nothing is canonicalised: the
//    export shows exactly the bits those kernels multiply with.
// The E8M0 byte of block `blk` of row n: the 8-bit table, or (base != null)
// the scale4 row base plus the block's 4-bit delta.
__device__ __forceinline__ uint32_t block_scale(const uint8_t* __restrict__ scales, const uint8_t* __restrict__ base,
                                                size_t n, int cols, int blk) {
  if (!base) return scales[n * (cols / 32) + blk];
  return base[n] + ((scales[n * (cols / 64) + blk / 2] >> ((blk & 1) * 4)) & 15u);
}

__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales,
                                                 const uint8_t* __restrict__ s4_base, int rows, int cols,
                                                 float* __restrict__ out) {
  const size_t words = (size_t)rows * cols / 8;
  const int wpr = cols / 8;
  for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < words; q += (size_t)gridDim.x * 256) {
    const size_t n = q / wpr;
    const int c8 = (int)(q % wpr);
    const uint32_t w = reinterpret_cast<const uint32_t*>(codes)[q];
    const uint32_t sbyte = block_scale(scales, s4_base, n, cols, (c8 * 8) / 32);
    float v[8];
    if (sbyte == 0xFFu) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __uint_as_float(0x7FC00000u);
    } else {
      const float s = e8m0_operand(sbyte);
      f32x2 a = fp4x2_to_f32<0>(w, s), b = fp4x2_to_f32<1>(w, s);
      f32x2 c = fp4x2_to_f32<2>(w, s), d = fp4x2_to_f32<3>(w, s);
      v[0] = a.x; v[1] = a.y; v[2] = b.x; v[3] = b.y; v[4] = c.x; v[5] = c.y; v[6] = d.x; v[7] = d.y;
    }
    float4* o = reinterpret_cast<float4*>(out + n * cols + (size_t)c8 * 8);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

__global__ __launch_bounds__(256) void k_dequant_bf16(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales,
                                                      const uint8_t* __restrict__ s4_base, int rows, int cols,
                                                      float* __restrict__ out) {
  const size_t words = (size_t)rows * cols / 8;
  const int wpr = cols / 8;
  for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < words; q += (size_t)gridDim.x * 256) {
    const size_t n = q / wpr;
    const int c8 = (int)(q % wpr);
    const uint32_t w = reinterpret_cast<const uint32_t*>(codes)[q];
    const uint32_t sbyte = block_scale(scales, s4_base, n, cols, (c8 * 8) / 32);
    const bf16x8 b = decode8(w, e8m0_operand(sbyte));
    uint16_t u[8];
    __builtin_memcpy(u, &b, 16);
    float4* o = reinterpret_cast<float4*>(out + n * cols + (size_t)c8 * 8);
    o[0] = make_float4(bf16_bits_to_f32(u[0]), bf16_bits_to_f32(u[1]), bf16_bits_to_f32(u[2]), bf16_bits_to_f32(u[3]));
    o[1] = make_float4(bf16_bits_to_f32(u[4]), bf16_bits_to_f32(u[5]), bf16_bits_to_f32(u[6]), bf16_bits_to_f32(u[7]));
  }
}

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const uint8_t* s4_base, int rows, int cols,
                          float* out, bool via_bf16, hipStream_t s) {
  const size_t words = (size_t)rows * cols / 8;
  size_t blocks = (words + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (via_bf16)
    k_dequant_bf16<<<dim3((unsigned)blocks), 256, 0, s>>>(codes, scales, s4_base, rows, cols, out);
  else
    k_dequant<<<dim3((unsigned)blocks), 256, 0, s>>>(codes, scales, s4_base, rows, cols, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- scale4 encoding
// One wave per matrix row: the row's smallest scale byte is its base, and
// every block stores scale - base in 4 bits (two blocks per byte, the even
// block in the low nibble).  A row whose scales span more than 15 cannot be
// coded: it adds 1 to *escapes (its deltas are clamped, so the layer must
// keep the 8-bit table).  Rows hold at most 256 blocks (K <= 8192).
__global__ __launch_bounds__(256) void k_scale4_encode(const uint8_t* __restrict__ scales8, int64_t e0, int64_t n,
                                                       int H, int I, uint8_t* __restrict__ scale4,
                                                       int32_t* __restrict__ escapes) {
  const int lane = threadIdx.x % kWave;
  const int64_t rows_per_expert = (int64_t)2 * I + H;
  const int64_t total = n * rows_per_expert;
  const size_t sb = (size_t)3 * I * H / 32, ms = (size_t)I * H / 32, dm = (size_t)I * H / 64;
  const size_t rec = (size_t)2 * I + H + 3 * dm;
  for (int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave; r < total; r += (int64_t)gridDim.x * 4) {
    const int64_t e = e0 + r / rows_per_expert;
    const int64_t rr = r % rows_per_expert;
    const int m = rr < I ? 0 : (rr < 2 * I ? 1 : 2);
    const int64_t row = m == 2 ? rr - 2 * I : rr - (int64_t)m * I;
    const int nb = m == 2 ? I / 32 : H / 32;
    const uint8_t* src = scales8 + (size_t)(e - e0) * sb + (size_t)m * ms + (size_t)row * nb;
    uint32_t lo = 255, hi = 0;
    for (int b = lane; b < nb; b += kWave) {
      const uint32_t v = src[b];
      lo = v < lo ? v : lo;
      hi = v > hi ? v : hi;
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const uint32_t ol = (uint32_t)__shfl_xor((int)lo, off, kWave), oh = (uint32_t)__shfl_xor((int)hi, off, kWave);
      lo = ol < lo ? ol : lo;
      hi = oh > hi ? oh : hi;
    }
    uint8_t* dst = scale4 + (size_t)e * rec;
    if (lane == 0) {
      dst[m == 2 ? (size_t)2 * I + row : (size_t)m * I + row] = (uint8_t)lo;
      if (hi - lo > 15u) atomicAdd(escapes, 1);
    }
    uint8_t* dd = dst + (size_t)2 * I + H + (size_t)m * dm + (size_t)row * (nb / 2);
    for (int i = lane; i < nb / 2; i += kWave) {
      uint32_t d0 = src[2 * i] - lo, d1 = src[2 * i + 1] - lo;
      d0 = d0 > 15u ? 15u : d0;
      d1 = d1 > 15u ? 15u : d1;
      dd[i] = (uint8_t)(d0 | (d1 << 4));
    }
  }
}

hipError_t launch_scale4_encode(const uint8_t* scales8, int64_t e0, int64_t n, int H, int I, uint8_t* scale4,
                                int32_t* escapes, hipStream_t s) {
  const int64_t rows = n * ((int64_t)2 * I + H);
  int64_t blocks = (rows + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  if (blocks == 0) return hipSuccess;
  k_scale4_encode<<<dim3((unsigned)blocks), 256, 0, s>>>(scales8, e0, n, H, I, scale4, escapes);
  return hipGetLastError();
}

// ---------------------------------------------------------------- RMSNorm
// One workgroup per token: ss = sum r^2 (fixed-order block reduction),
// n = (r * (1 / sqrt(ss / H + eps))) * gamma.
__global__ __launch_bounds__(256) void k_rmsnorm(const float* __restrict__ r,
                                                 const float* __restrict__ gamma, float eps, int H,
                                                 float* __restrict__ out) {
  const int t = blockIdx.x;
  const float4* rt = reinterpret_cast<const float4*>(r + (size_t)t * H);
  float ss = 0.0f;
  for (int c = threadIdx.x; c < H / 4; c += 256) {
    float4 v = rt[c];
    ss = fmaf(v.x, v.x, ss);
    ss = fmaf(v.y, v.y, ss);
    ss = fmaf(v.z, v.z, ss);
    ss = fmaf(v.w, v.w, ss);
  }
  __shared__ float red[4];
  ss = group_sum<kWave>(ss);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);
  float4* ot = reinterpret_cast<float4*>(out + (size_t)t * H);
  const float4* g = reinterpret_cast<const float4*>(gamma);
  for (int c = threadIdx.x; c < H / 4; c += 256) {
    float4 v = rt[c], gg = g[c];
    ot[c] = make_float4((v.x * inv) * gg.x, (v.y * inv) * gg.y, (v.z * inv) * gg.z, (v.w * inv) * gg.w);
  }
}

hipError_t launch_rmsnorm(const float* r, const float* gamma, float eps, int T, int H, float* out,
                          hipStream_t s) {
  k_rmsnorm<<<dim3(T), 256, 0, s>>>(r, gamma, eps, H, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- residual / widen
__global__ __launch_bounds__(256) void k_residual_add(float* __restrict__ r, const float* __restrict__ d,
                                                      size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    r[i] = r[i] + d[i];
}

hipError_t launch_residual_add(float* r, const float* d, size_t n, hipStream_t s) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return hipSuccess;
  k_residual_add<<<dim3((unsigned)blocks), 256, 0, s>>>(r, d, n);
  return hipGetLastError();
}

// x (fp32 or bf16) -> fp32 copy.
__global__ __launch_bounds__(256) void k_widen(const void* __restrict__ x, bool x_f32, size_t n,
                                               float* __restrict__ out) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    out[i] = x_f32 ? static_cast<const float*>(x)[i]
                   : bf16_bits_to_f32(static_cast<const uint16_t*>(x)[i]);
}

hipError_t launch_widen(const void* x, bool x_f32, size_t n, float* out, hipStream_t s) {
  size_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks == 0) return hipSuccess;
  k_widen<<<dim3((unsigned)blocks), 256, 0, s>>>(x, x_f32, n, out);
  return hipGetLastError();
}

// Three bf16 terms of fp32 rows (the grouped expert GEMMs' activation operand
// for fp32 x).  x - hi has at most 16 significant bits and x - hi - mid at
// most 8, so both subtractions are exact in fp32 and the three terms add up to
// x (above bf16's largest finite value hi is that value).  A NaN or an
// infinity goes whole into hi (mid and lo are 0).
__global__ __launch_bounds__(256) void k_split3(const float* __restrict__ x, int T, int H,
                                                uint16_t* __restrict__ out) {
  const size_t n = (size_t)T * H;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const float v = x[i];
    uint16_t hi = f32_to_bf16_rne(v);
    uint16_t mid = 0, lo = 0;
    if (isfinite(v)) {
      // above bf16's largest finite value hi would round to infinity: take the
      // largest finite bf16 instead (the rest still fits mid and lo)
      if ((hi & 0x7FFFu) == 0x7F80u) hi = (uint16_t)((hi & 0x8000u) | 0x7F7Fu);
      const float r1 = v - bf16_bits_to_f32(hi);
      mid = f32_to_bf16_rne(r1);
      lo = f32_to_bf16_rne(r1 - bf16_bits_to_f32(mid));
    }
    const size_t t = i / (size_t)H, c = i - t * (size_t)H;
    uint16_t* o = out + t * 3 * (size_t)H + c;
    o[0] = hi;
    o[H] = mid;
    o[2 * (size_t)H] = lo;
  }
}

hipError_t launch_split3(const float* x, int T, int H, uint16_t* out, hipStream_t s) {
  const size_t n = (size_t)T * H;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) return hipSuccess;
  k_split3<<<dim3((unsigned)blocks), 256, 0, s>>>(x, T, H, out);
  return hipGetLastError();
}

}  // namespace moe
