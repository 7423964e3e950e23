// Sustained matrix-core rate on random operands, with no memory traffic in
// the timed loop: the ceiling that bounds the prefill form's grouped GEMMs at
// the clock the chip holds under that load.  It backs the choice of bf16
// MFMA for prefill (bf16 activations are exact only as bf16; an fp8 or fp4
// activation operand would need several terms).  A measurement aid, not on
// the pages.
//
// Each thread takes 32 random bytes as its A and B operands, then runs iters
// rounds of 8 independent accumulator chains of one MFMA kind; the sums go to
// sink so the work cannot be dropped.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {
typedef __attribute__((ext_vector_type(8))) int v8i;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
constexpr int kRateThreads = 512;
constexpr int kRateOperands = 4096;  // 16-byte operand pieces the caller provides
}  // namespace

// KIND 0: bf16 16x16x32; 1: fp8 (e4m3) A x fp4 (e2m1) B, 16x16x128 with
// E8M0 scales 1.0; 2: fp4 x fp4, 16x16x128, scales 1.0.
template <int KIND>
__global__ __launch_bounds__(kRateThreads) void k_mfma_rate(const u32x4* __restrict__ operands, int iters,
                                                            float* __restrict__ sink) {
  const int t = blockIdx.x * kRateThreads + threadIdx.x;
  const u32x4 a0 = operands[(2 * t) % kRateOperands], a1 = operands[(2 * t + 1) % kRateOperands];
  const u32x4 b0 = operands[(2 * t + 777) % kRateOperands], b1 = operands[(2 * t + 778) % kRateOperands];
  const v8i a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
  const v8i b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (KIND == 0) {
        const bf16x8_t x = __builtin_bit_cast(bf16x8_t, u32x4{a0.x, a0.y, a0.z, a0.w});
        const bf16x8_t y = __builtin_bit_cast(bf16x8_t, u32x4{b0.x, b0.y, b0.z, b0.w});
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, acc[j], 0, 0, 0);
      } else if constexpr (KIND == 1) {
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 0, 4, 0, 127, 0, 127);
      } else {
        acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[j], 4, 4, 0, 127, 0, 127);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  sink[t] = s;
}

hipError_t launch_mfma_rate(int kind, const void* operands, int n_workgroups, int iters, float* sink,
                            hipStream_t s) {
  const u32x4* op = static_cast<const u32x4*>(operands);
  const dim3 grid((unsigned)n_workgroups);
  if (kind == 0)
    k_mfma_rate<0><<<grid, kRateThreads, 0, s>>>(op, iters, sink);
  else if (kind == 1)
    k_mfma_rate<1><<<grid, kRateThreads, 0, s>>>(op, iters, sink);
  else if (kind == 2)
    k_mfma_rate<2><<<grid, kRateThreads, 0, s>>>(op, iters, sink);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace moe
