// Decode-form expert kernels (one token): HBM-streaming MXFP4 GEMVs that decode
// the 4-bit codes in registers, plus the rank-ordered combine.
//
// The fused dequant + GEMV follows brain.bigb.es "deltafin", section "The
// techniques that bought the 82x" (table decode of E2M1, E8M0 scale applied to
// the fp32 exponent, one pass over the weights).  Here the decode is the
// gfx950 scaled FP4 conversion, which yields exactly E2M1(code) * 2^(S-127).
//
// Weight layout (row-major, per expert gate | up | down): a row of a
// [rows][K] matrix is K/2 code bytes followed, in the scale buffer, by K/32
// scale bytes.  Lane l of a wave owns the 32-element blocks b = c + LPR*m of
// its row (c = l % LPR), so every load instruction of a wave reads LPR
// consecutive 16-byte blocks of each of 64/LPR rows, and the lane's slice of
// the activation vector stays in registers for all rows the wave streams.
#include "common.h"
#include "kernels.h"

namespace moe {

// 32 products of one block: codes q (16 bytes = 32 nibbles), scale operand s,
// activations as 16 bf16 pairs.  Weights are exact bf16, products exact fp32.
__device__ __forceinline__ float block_dot_bf16(uint4 q, float s, const uint32_t* xp, float acc) {
  acc = dot2_bf16(fp4x2_to_bf16<0>(q.x, s), as_bf16x2(xp[0]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<1>(q.x, s), as_bf16x2(xp[1]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<2>(q.x, s), as_bf16x2(xp[2]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<3>(q.x, s), as_bf16x2(xp[3]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<0>(q.y, s), as_bf16x2(xp[4]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<1>(q.y, s), as_bf16x2(xp[5]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<2>(q.y, s), as_bf16x2(xp[6]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<3>(q.y, s), as_bf16x2(xp[7]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<0>(q.z, s), as_bf16x2(xp[8]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<1>(q.z, s), as_bf16x2(xp[9]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<2>(q.z, s), as_bf16x2(xp[10]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<3>(q.z, s), as_bf16x2(xp[11]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<0>(q.w, s), as_bf16x2(xp[12]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<1>(q.w, s), as_bf16x2(xp[13]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<2>(q.w, s), as_bf16x2(xp[14]), acc);
  acc = dot2_bf16(fp4x2_to_bf16<3>(q.w, s), as_bf16x2(xp[15]), acc);
  return acc;
}

template <int SEL>
__device__ __forceinline__ float quad_fma_f32(uint32_t q, float s, const uint32_t* xf, float acc) {
  f32x2 w = fp4x2_to_f32<SEL>(q, s);
  acc = fmaf(w.x, __uint_as_float(xf[2 * SEL]), acc);
  return fmaf(w.y, __uint_as_float(xf[2 * SEL + 1]), acc);
}

// Same with fp32 activations (32 floats, as bit patterns): exact fp32 weights,
// fp32 FMA.
__device__ __forceinline__ float block_dot_f32(uint4 q, float s, const uint32_t* xf, float acc) {
  acc = quad_fma_f32<0>(q.x, s, xf, acc);
  acc = quad_fma_f32<1>(q.x, s, xf, acc);
  acc = quad_fma_f32<2>(q.x, s, xf, acc);
  acc = quad_fma_f32<3>(q.x, s, xf, acc);
  acc = quad_fma_f32<0>(q.y, s, xf + 8, acc);
  acc = quad_fma_f32<1>(q.y, s, xf + 8, acc);
  acc = quad_fma_f32<2>(q.y, s, xf + 8, acc);
  acc = quad_fma_f32<3>(q.y, s, xf + 8, acc);
  acc = quad_fma_f32<0>(q.z, s, xf + 16, acc);
  acc = quad_fma_f32<1>(q.z, s, xf + 16, acc);
  acc = quad_fma_f32<2>(q.z, s, xf + 16, acc);
  acc = quad_fma_f32<3>(q.z, s, xf + 16, acc);
  acc = quad_fma_f32<0>(q.w, s, xf + 24, acc);
  acc = quad_fma_f32<1>(q.w, s, xf + 24, acc);
  acc = quad_fma_f32<2>(q.w, s, xf + 24, acc);
  acc = quad_fma_f32<3>(q.w, s, xf + 24, acc);
  return acc;
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// Grid: P (token, rank) pairs x `tiles` row tiles; 4 waves per workgroup, RPW
// rows of gate and up per wave.  Lanes: LPR = 64 (one row at a time, 64 blocks
// per load).  Output hbuf[p][i] = silu(g_i) * u_i for pair p = t*k + j.
constexpr int kGU_RPW = 4;
constexpr int kGU_ROWS = 4 * kGU_RPW;

template <bool XF32, int NBL>
__global__ __launch_bounds__(256) void k_gateup_gemv(const void* __restrict__ x,
                                                     const int32_t* __restrict__ route,
                                                     const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int H, int I,
                                                     int E, int k, int tiles, float* __restrict__ hbuf) {
  extern __shared__ uint4 xs_lds[];
  const int j = blockIdx.x / tiles;     // pair (token j / k, rank j % k)
  const int tile = blockIdx.x % tiles;
  int e = route[j];
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  const int nb = H / 32;
  const int xbytes = XF32 ? H * 4 : H * 2;
  const uint4* xg = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) + (size_t)(j / k) * xbytes);
  for (int c = threadIdx.x; c < xbytes / 16; c += 256) xs_lds[c] = xg[c];
  __syncthreads();

  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  constexpr int XW = XF32 ? 32 : 16;  // registers per block of activations
  uint32_t xr[NBL][XW];
#pragma unroll
  for (int m = 0; m < NBL; ++m) {
    const int b = lane + kWave * m;
    if (b < nb) {
      const uint4* src = xs_lds + b * (XW / 4);
#pragma unroll
      for (int v = 0; v < XW / 4; ++v) {
        uint4 u = src[v];
        xr[m][4 * v] = u.x; xr[m][4 * v + 1] = u.y; xr[m][4 * v + 2] = u.z; xr[m][4 * v + 3] = u.w;
      }
    } else {
#pragma unroll
      for (int v = 0; v < XW; ++v) xr[m][v] = 0u;
    }
  }

  const size_t cb = (size_t)3 * I * H / 2, sb = (size_t)3 * I * H / 32;
  const uint8_t* gcod = codes + (size_t)e * cb;
  const uint8_t* ucod = gcod + (size_t)I * H / 2;
  const uint8_t* gsc = scales + (size_t)e * sb;
  const uint8_t* usc = gsc + (size_t)I * H / 32;
  const int rb = H / 2, rs = H / 32;
  const int i0 = tile * kGU_ROWS + wid * kGU_RPW;
#pragma unroll
  for (int r = 0; r < kGU_RPW; ++r) {
    const int i = i0 + r;
    if (i >= I) break;
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int m = 0; m < NBL; ++m) {
      const int b = lane + kWave * m;
      if (b < nb) {
        const uint4 qg = load_u4_stream(gcod + (size_t)i * rb + 16 * b);
        const uint4 qu = load_u4_stream(ucod + (size_t)i * rb + 16 * b);
        const float sg = e8m0_operand(gsc[(size_t)i * rs + b]);
        const float su = e8m0_operand(usc[(size_t)i * rs + b]);
        if constexpr (XF32) {
          ag = block_dot_f32(qg, sg, xr[m], ag);
          au = block_dot_f32(qu, su, xr[m], au);
        } else {
          ag = block_dot_bf16(qg, sg, xr[m], ag);
          au = block_dot_bf16(qu, su, xr[m], au);
        }
      }
    }
    ag = group_sum<kWave>(ag);
    au = group_sum<kWave>(au);
    if (lane == 0) hbuf[(size_t)j * I + i] = silu_mul(ag, au);
  }
}

// ---------------------------------------------------------------- down
// Grid: P pairs x `tiles` row tiles of Wd [H][I]; the pair's h row is staged in
// LDS and each lane keeps its NBL2 blocks of it in registers.  LPR lanes per
// row, 64/LPR rows per load step, kDN_STEPS steps per wave.
constexpr int kDN_STEPS = 4;

template <int LPR, int NBL2>
__global__ __launch_bounds__(256) void k_down_gemv(const float* __restrict__ hbuf,
                                                   const int32_t* __restrict__ pair_expert,
                                                   const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales, int H, int I,
                                                   int E, int tiles, float* __restrict__ ybuf) {
  extern __shared__ float hs_lds[];
  constexpr int RPS = kWave / LPR;
  constexpr int ROWS_W = RPS * kDN_STEPS;
  constexpr int ROWS_G = 4 * ROWS_W;
  const int j = blockIdx.x / tiles;
  const int tile = blockIdx.x % tiles;
  int e = pair_expert[j];
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  const float4* hsrc = reinterpret_cast<const float4*>(hbuf + (size_t)j * I);
  for (int c = threadIdx.x; c < I / 4; c += 256) reinterpret_cast<float4*>(hs_lds)[c] = hsrc[c];
  __syncthreads();

  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int c = lane % LPR, rsub = lane / LPR;
  const int nbk = I / 32;
  uint32_t hr[NBL2][32];
#pragma unroll
  for (int m = 0; m < NBL2; ++m) {
    const int b = c + LPR * m;
#pragma unroll
    for (int v = 0; v < 32; ++v) hr[m][v] = (b < nbk) ? __float_as_uint(hs_lds[32 * b + v]) : 0u;
  }
  const size_t cb = (size_t)3 * I * H / 2, sb = (size_t)3 * I * H / 32;
  const uint8_t* dcod = codes + (size_t)e * cb + (size_t)I * H;
  const uint8_t* dsc = scales + (size_t)e * sb + (size_t)2 * I * H / 32;
  const int rb = I / 2, rs = I / 32;
  const int n0 = tile * ROWS_G + wid * ROWS_W;
#pragma unroll
  for (int s = 0; s < kDN_STEPS; ++s) {
    const int n = n0 + s * RPS + rsub;
    float acc = 0.0f;
    if (n < H) {
#pragma unroll
      for (int m = 0; m < NBL2; ++m) {
        const int b = c + LPR * m;
        if (b < nbk) {
          const uint4 q = load_u4_stream(dcod + (size_t)n * rb + 16 * b);
          const float sc = e8m0_operand(dsc[(size_t)n * rs + b]);
          acc = block_dot_f32(q, sc, hr[m], acc);
        }
      }
    }
    acc = group_sum<LPR>(acc);
    if (c == 0 && n < H) ybuf[(size_t)j * H + n] = acc;
  }
}

// ---------------------------------------------------------------- combine
// out[t][n] = sum_j w[t][j] * y[t*k+j][n], j ascending; optionally added to a
// residual: out = resid + sum (resid may alias out).
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ ybuf,
                                                 const float* __restrict__ w, int T, int k, int H,
                                                 const float* resid, float* out) {
  const size_t n4 = (size_t)T * H / 4;
  for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < n4; q += (size_t)gridDim.x * 256) {
    const size_t flat = 4 * q;
    const int t = (int)(flat / H);
    const int n = (int)(flat % H);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float wj = w[(size_t)t * k + j];
      const float4 y = *reinterpret_cast<const float4*>(ybuf + ((size_t)t * k + j) * H + n);
      acc.x = fmaf(wj, y.x, acc.x);
      acc.y = fmaf(wj, y.y, acc.y);
      acc.z = fmaf(wj, y.z, acc.z);
      acc.w = fmaf(wj, y.w, acc.w);
    }
    if (resid) {
      const float4 r = *reinterpret_cast<const float4*>(resid + flat);
      acc.x = r.x + acc.x; acc.y = r.y + acc.y; acc.z = r.z + acc.z; acc.w = r.w + acc.w;
    }
    *reinterpret_cast<float4*>(out + flat) = acc;
  }
}

// ---------------------------------------------------------------- launchers

template <bool XF32>
static hipError_t gateup_dispatch(int nbl, dim3 grid, size_t lds, hipStream_t s, const void* x,
                                  const int32_t* route, const uint8_t* codes, const uint8_t* scales,
                                  int H, int I, int E, int k, int tiles, float* hbuf) {
  switch (nbl) {
    case 1: k_gateup_gemv<XF32, 1><<<grid, 256, lds, s>>>(x, route, codes, scales, H, I, E, k, tiles, hbuf); break;
    case 2: k_gateup_gemv<XF32, 2><<<grid, 256, lds, s>>>(x, route, codes, scales, H, I, E, k, tiles, hbuf); break;
    case 3: k_gateup_gemv<XF32, 3><<<grid, 256, lds, s>>>(x, route, codes, scales, H, I, E, k, tiles, hbuf); break;
    case 4: k_gateup_gemv<XF32, 4><<<grid, 256, lds, s>>>(x, route, codes, scales, H, I, E, k, tiles, hbuf); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gateup_gemv(const void* x, bool x_f32, const int32_t* route, int P, int k,
                              const uint8_t* codes, const uint8_t* scales, int H, int I, int E,
                              float* hbuf, hipStream_t s) {
  const int nb = H / 32;
  const int nbl = (nb + kWave - 1) / kWave;
  const int tiles = (I + kGU_ROWS - 1) / kGU_ROWS;
  dim3 grid(P * tiles);
  const size_t lds = (size_t)H * (x_f32 ? 4 : 2);
  if (x_f32) return gateup_dispatch<true>(nbl, grid, lds, s, x, route, codes, scales, H, I, E, k, tiles, hbuf);
  return gateup_dispatch<false>(nbl, grid, lds, s, x, route, codes, scales, H, I, E, k, tiles, hbuf);
}

// lanes per row and blocks per lane for a reduction length of nbk blocks:
// the smallest LPR in {4, 8, 16, 32, 64} with nbk <= 4 * LPR and no more idle
// lane slots than a larger LPR would leave.
void down_shape(int nbk, int* lpr, int* nbl2) {
  static const int cand[5] = {4, 8, 16, 32, 64};
  int best = -1, best_idle = 1 << 30;
  for (int i = 0; i < 5; ++i) {
    const int L = cand[i];
    const int nb = (nbk + L - 1) / L;
    if (nb > 4) continue;
    const int idle = nb * L - nbk;
    if (idle < best_idle) { best_idle = idle; best = i; }
  }
  *lpr = cand[best];
  *nbl2 = (nbk + *lpr - 1) / *lpr;
}

#define MOE_DOWN_CASE(L, N)                                                                        \
  if (lpr == L && nbl2 == N) {                                                                   \
    constexpr int ROWS_G = 4 * (kWave / L) * kDN_STEPS;                                           \
    const int tiles = (H + ROWS_G - 1) / ROWS_G;                                                  \
    k_down_gemv<L, N><<<dim3(P * tiles), 256, lds, s>>>(hbuf, pair_expert, codes, scales, H, I, E, \
                                                        tiles, ybuf);                              \
    return hipGetLastError();                                                                      \
  }

hipError_t launch_down_gemv(const float* hbuf, const int32_t* pair_expert, int P, const uint8_t* codes,
                            const uint8_t* scales, int H, int I, int E, float* ybuf, hipStream_t s) {
  int lpr, nbl2;
  down_shape(I / 32, &lpr, &nbl2);
  const size_t lds = (size_t)I * 4;
  MOE_DOWN_CASE(4, 1) MOE_DOWN_CASE(4, 2) MOE_DOWN_CASE(4, 3) MOE_DOWN_CASE(4, 4)
  MOE_DOWN_CASE(8, 1) MOE_DOWN_CASE(8, 2) MOE_DOWN_CASE(8, 3) MOE_DOWN_CASE(8, 4)
  MOE_DOWN_CASE(16, 1) MOE_DOWN_CASE(16, 2) MOE_DOWN_CASE(16, 3) MOE_DOWN_CASE(16, 4)
  MOE_DOWN_CASE(32, 1) MOE_DOWN_CASE(32, 2) MOE_DOWN_CASE(32, 3) MOE_DOWN_CASE(32, 4)
  MOE_DOWN_CASE(64, 1) MOE_DOWN_CASE(64, 2) MOE_DOWN_CASE(64, 3) MOE_DOWN_CASE(64, 4)
  return hipErrorInvalidValue;
}

hipError_t launch_combine(const float* ybuf, const float* w, int T, int k, int H, const float* resid,
                          float* out, hipStream_t s) {
  const size_t n4 = (size_t)T * H / 4;
  size_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_combine<<<dim3((unsigned)blocks), 256, 0, s>>>(ybuf, w, T, k, H, resid, out);
  return hipGetLastError();
}

}  // namespace moe
