// Packed-int8 rows with one fp16 scale per row: the resident-spine GEMV on the
// decode form's streaming skeleton, and the fused int8 -> fp32 * scale export.
//
// The int8 spine is "Deltafin's custom compiled runtime", section "Weight
// fidelity" (an explicit, non-weight-exact option: row rounding and fp16
// scales), at that page's 12288 x 7168 packed-int8 test shape (section "One
// native build and test graph"); the fused int8 -> fp32 + scale kernel is
// brain.bigb.es "deltafin", section "The techniques that bought the 82x".
// W[n][k] = q[n][k] * s[n] is exact in fp32 (int8 times binary16).
//
// GEMV layout: a workgroup has ceil(K / 1024) waves; wave w covers bytes
// 1024 w .. 1024 w + 1023 of every row, lane l the 16 bytes at 1024 w + 16 l,
// so one load instruction of a wave reads 1 KB of one row and a lane keeps
// its 16 activations per token in registers for every row.  Rows are
// streamed through a ring of loads D - 1 rows ahead; each wave reduces its
// lanes per row (a fixed DPP tree) into LDS, and the workgroup adds the
// waves' partials of a row in wave order and applies the row scale:
// y[t][n] = s[n] * sum_w partial_w (a fixed order, so results are
// deterministic).
#include "common.h"

namespace moe {

namespace {

typedef __amdgpu_buffer_rsrc_t rsrc8_t;
constexpr uint32_t kOOB8 = 0x80000000u;

__device__ __forceinline__ rsrc8_t rsrc8(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float sext_byte(uint32_t w, int b) {
  return (float)(int32_t)((int32_t)(w << (24 - 8 * b)) >> 24);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

constexpr int kInt8Ring = 8;  // rows in flight per wave (7 ahead); 4 measured 20-30% slower

}  // namespace

template <int TT, bool XF32>
__global__ __launch_bounds__(1024) void k_int8_gemv(const int8_t* __restrict__ q, const uint16_t* __restrict__ s,
                                                    int N, int K, const void* __restrict__ x, int rows_per_wg,
                                                    float* __restrict__ y) {
  extern __shared__ float part[];  // [rows_per_wg][nw]
  constexpr int D = kInt8Ring;
  const int nw = blockDim.x / kWave;
  const int lane = threadIdx.x % kWave, wv = threadIdx.x / kWave;
  const int k0 = 1024 * wv + 16 * lane;  // this lane's 16 columns
  const int r0 = blockIdx.x * rows_per_wg;
  const int nrows = min(rows_per_wg, N - r0);
  const rsrc8_t rq = rsrc8(q + (size_t)r0 * K, (uint32_t)((size_t)nrows * K));
  auto load = [&](int r) -> u32x4 {
    const bool ok = r < nrows && k0 < K;
    return __builtin_amdgcn_raw_buffer_load_b128(rq, ok ? (uint32_t)r * (uint32_t)K + (uint32_t)k0 : kOOB8, 0,
                                                 2 /* nt */);
  };
  // the lane's 16 activations per token first, in 16-byte loads (K is a
  // multiple of 16, so a lane's columns are all in range or all past K):
  // loads complete in issue order, so the first row's wait for x then leaves
  // the ring's loads in flight (issued after the ring, that wait would cover
  // them too, in every pass of the loop)
  float xr[TT][16];
  const bool xin = k0 < K;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    if constexpr (XF32) {
      const float4* xp = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)t * K + (xin ? k0 : 0));
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 f = xp[v];
        xr[t][4 * v] = xin ? f.x : 0.0f;
        xr[t][4 * v + 1] = xin ? f.y : 0.0f;
        xr[t][4 * v + 2] = xin ? f.z : 0.0f;
        xr[t][4 * v + 3] = xin ? f.w : 0.0f;
      }
    } else {
      const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + (size_t)t * K + (xin ? k0 : 0));
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const uint4 u = xp[v];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xr[t][8 * v + 2 * j] = xin ? bf16_bits_to_f32(w[j] & 0xFFFFu) : 0.0f;
          xr[t][8 * v + 2 * j + 1] = xin ? bf16_bits_to_f32(w[j] >> 16) : 0.0f;
        }
      }
    }
  }
  // the prologue's loads in ring order (the scheduler may not reorder them:
  // the loop's wait counts assume the oldest load holds the first row)
  u32x4 ring[D];
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    ring[d] = load(d);
    __builtin_amdgcn_sched_barrier(0);
  }
  // every row of the workgroup's range in whole ring passes (rows_per_wg is
  // a multiple of D, so the unrolled ring has no exit inside); rows past N
  // read zeros and their sums are never used
  for (int r = 0; r < rows_per_wg; r += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int row = r + d;
      ring[(d + D - 1) % D] = load(row + D - 1);
      const u32x4 v = ring[d];
      float acc[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t w = v[wd];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float qv = sext_byte(w, b);
#pragma unroll
          for (int t = 0; t < TT; ++t) acc[t] = fmaf(qv, xr[t][4 * wd + b], acc[t]);
        }
      }
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        const float sum = wave_sum(acc[t]);
        if (lane == 0) part[((size_t)t * rows_per_wg + row) * nw + wv] = sum;
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < TT * nrows; i += blockDim.x) {
    const int t = i / nrows, row = i % nrows;
    const float* p = part + ((size_t)t * rows_per_wg + row) * nw;
    float acc = p[0];
    for (int w2 = 1; w2 < nw; ++w2) acc += p[w2];
    y[(size_t)t * N + r0 + row] = acc * f16_bits_to_f32(s[r0 + row]);
  }
}

// out[n][k] = q[n][k] * s[n].  A wave takes 1 KB of q per step: lane l
// loads dwords l, l + 64, l + 128 and l + 192 of it (four independent
// 256-byte loads per wave, in flight together) and writes each as 4 fp32, so
// every store instruction of the wave writes 1 KB of out contiguously.
__global__ __launch_bounds__(256) void k_int8_dequant(const int8_t* __restrict__ q, const uint16_t* __restrict__ s,
                                                      int N, int K, float* __restrict__ out) {
  const size_t ndw = (size_t)N * K / 4;  // dwords of q (K is a multiple of 16)
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const uint32_t* q32 = reinterpret_cast<const uint32_t*>(q);
  f32x4* o4 = reinterpret_cast<f32x4*>(out);
  for (size_t c0 = ((size_t)blockIdx.x * 4 + wave) * 256; c0 < ndw; c0 += (size_t)gridDim.x * 4 * 256) {
    uint32_t w[4];
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t i = c0 + 64 * j + lane;
      const bool ok = i < ndw;
      w[j] = __builtin_nontemporal_load(q32 + (ok ? i : 0));
      sc[j] = f16_bits_to_f32(s[ok ? (i * 4) / K : 0]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t i = c0 + 64 * j + lane;
      if (i < ndw) {
        f32x4 r;
        r.x = sext_byte(w[j], 0) * sc[j];
        r.y = sext_byte(w[j], 1) * sc[j];
        r.z = sext_byte(w[j], 2) * sc[j];
        r.w = sext_byte(w[j], 3) * sc[j];
        o4[i] = r;
      }
    }
  }
}

int int8_rows_per_wg(int N, int K) {
  // about one workgroup per CU of 256 (fewer, longer-streaming workgroups
  // measured faster than four per CU); a multiple of the ring depth
  const int want = 256;
  int r = (N + want - 1) / want;
  r = (r + kInt8Ring - 1) / kInt8Ring * kInt8Ring;
  (void)K;
  return r < kInt8Ring ? kInt8Ring : r;
}

hipError_t launch_int8_gemv(const int8_t* q, const uint16_t* s, int N, int K, const void* x, bool x_f32, int T,
                            float* y, int rows_per_wg, hipStream_t st) {
  const int nw = (K + 1023) / 1024;
  if (rows_per_wg <= 0) rows_per_wg = int8_rows_per_wg(N, K);
  const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg));
  const size_t lds = (size_t)T * rows_per_wg * nw * 4;
  if (lds > 65536) return hipErrorInvalidValue;
#define MOE_I8(TT)                                                                                        \
  if (T == TT) {                                                                                          \
    if (x_f32)                                                                                            \
      k_int8_gemv<TT, true><<<grid, nw * kWave, lds, st>>>(q, s, N, K, x, rows_per_wg, y);                \
    else                                                                                                  \
      k_int8_gemv<TT, false><<<grid, nw * kWave, lds, st>>>(q, s, N, K, x, rows_per_wg, y);               \
    return hipGetLastError();                                                                             \
  }
  MOE_I8(1) MOE_I8(2) MOE_I8(3) MOE_I8(4)
#undef MOE_I8
  return hipErrorInvalidValue;
}

hipError_t launch_int8_dequant(const int8_t* q, const uint16_t* s, int N, int K, float* out, hipStream_t st) {
  const size_t nkb = ((size_t)N * K + 1023) / 1024;  // 1 KB steps of one wave
  size_t blocks = (nkb + 3) / 4;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) return hipSuccess;
  k_int8_dequant<<<dim3((unsigned)blocks), 256, 0, st>>>(q, s, N, K, out);
  return hipGetLastError();
}

}  // namespace moe
