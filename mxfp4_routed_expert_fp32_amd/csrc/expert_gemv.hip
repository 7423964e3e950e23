// Decode-form expert kernels: HBM-streaming MXFP4 GEMVs that decode the 4-bit
// codes in registers, plus the rank-ordered combine.
//
// The fused dequant + GEMV follows brain.bigb.es "deltafin", section "The
// techniques that bought the 82x" (E2M1 decode through a 16-entry table, E8M0
// scale applied to the fp32 exponent, one pass over the weights).  Here the
// decode is a gfx950 scaled FP4 conversion: the bf16 form for bf16
// activations, the fp32 form for fp32 activations and for the down
// projection.  The library exports each conversion alone (moe_mxfp4_dequant
// and moe_mxfp4_dequant_bf16), and the tests compare both bit for bit with
// the oracle over every code and scale byte.
//
// Weight layout (row-major, per expert gate | up | down): a row of a
// [rows][K] matrix is K/2 code bytes, plus K/32 scale bytes in the scale
// buffer.
//
// Two forms of each GEMV:
//  - K split across waves (k_gateup_ks for H = 1024 KS, k_down_ks for
//    I = 512 KS, the model's widths): each wave of a workgroup takes a fixed
//    range of 32-element blocks of every row of the workgroup's row range
//    (one block per lane, 32 or 16 lanes per row), so a lane holds one block
//    of activations in registers; the waves' partial sums of a row are added
//    in LDS in wave order, and the workgroup's 8-bit scale rows are copied
//    into LDS once.
//  - Whole rows per wave (k_gateup_gemv, k_down_gemv, other widths): lane l
//    of a wave owns the blocks b = c + LPR*m of its row (c = l % LPR,
//    m < NBL), so each 16-byte load instruction of a wave reads LPR
//    consecutive blocks of each of 64/LPR rows, and the lane's slice of the
//    activation vector stays in registers for every row the wave streams.
// In both, a workgroup owns one (token, rank) pair and a share of its rows;
// the grid is sized to the number of workgroups the GPU holds at once
// (occupancy x CUs), so every workgroup runs once, and weight loads run
// several steps ahead of the compute.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

// Workgroups of `fn` (`threads` threads, `lds` bytes of LDS) the current
// device holds at once.  Queried once per (kernel, LDS size, device) and
// remembered in a fixed table (no heap use on a launch path; when the table
// is full the value is simply queried again).
static int resident_wgs_query(const void* fn, size_t lds, int threads) {
  struct Entry { const void* fn; size_t lds; int dev; int value; };
  constexpr int kSlots = 256;
  static std::mutex mu;
  static Entry table[kSlots];
  static int used = 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  {
    std::lock_guard<std::mutex> g(mu);
    for (int i = 0; i < used; ++i)
      if (table[i].fn == fn && table[i].lds == lds && table[i].dev == dev) return table[i].value;
  }
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, lds) != hipSuccess || per_cu <= 0) per_cu = 1;
  const int v = cus * per_cu;
  std::lock_guard<std::mutex> g(mu);
  if (used < kSlots) table[used++] = Entry{fn, lds, dev, v};
  return v;
}

template <typename F>
static int resident_wgs(F fn, size_t lds, int threads = 256) {
  return resident_wgs_query(reinterpret_cast<const void*>(fn), lds, threads);
}

// Compute units of the current device (remembered per device in a fixed table).
static int cu_count() {
  constexpr int kDevices = 64;
  static std::mutex mu;
  static int table[kDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> g(mu);
  if (dev >= 0 && dev < kDevices && table[dev] > 0) return table[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev >= 0 && dev < kDevices) table[dev] = cus;
  return cus;
}

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
// fp32 FMA.  PIN: a scheduling barrier after each code dword keeps the
// conversions next to their FMAs (hoisted ahead, the 32 converted weights of
// a block are all live at once, which costs the K-split down kernel two
// waves per SIMD).
template <bool PIN = false>
__device__ __forceinline__ float block_dot_f32(uint4 q, float s, const uint32_t* xf, float acc) {
  acc = quad_fma_f32<0>(q.x, s, xf, acc);
  acc = quad_fma_f32<1>(q.x, s, xf, acc);
  acc = quad_fma_f32<2>(q.x, s, xf, acc);
  acc = quad_fma_f32<3>(q.x, s, xf, acc);
  if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
  acc = quad_fma_f32<0>(q.y, s, xf + 8, acc);
  acc = quad_fma_f32<1>(q.y, s, xf + 8, acc);
  acc = quad_fma_f32<2>(q.y, s, xf + 8, acc);
  acc = quad_fma_f32<3>(q.y, s, xf + 8, acc);
  if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
  acc = quad_fma_f32<0>(q.z, s, xf + 16, acc);
  acc = quad_fma_f32<1>(q.z, s, xf + 16, acc);
  acc = quad_fma_f32<2>(q.z, s, xf + 16, acc);
  acc = quad_fma_f32<3>(q.z, s, xf + 16, acc);
  if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
  acc = quad_fma_f32<0>(q.w, s, xf + 24, acc);
  acc = quad_fma_f32<1>(q.w, s, xf + 24, acc);
  acc = quad_fma_f32<2>(q.w, s, xf + 24, acc);
  acc = quad_fma_f32<3>(q.w, s, xf + 24, acc);
  return acc;
}

// Weights are read through raw buffer loads: a resource per matrix (base in
// SGPRs, byte range = the matrix) and a 32-bit offset per lane.  An offset
// past the range returns zeros, which is how blocks past a row's end and rows
// past a matrix's end are read: zero codes with scale byte 0 (a finite
// 2^-127) add exactly 0.  No clamps or branches sit around the loads.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every buffer

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Scales of one matrix: the 8-bit table (one E8M0 byte per 32-element block,
// [rows][nb]), or the scale4 side-car (one base byte per row, [rows], and a
// 4-bit delta per block, two blocks per byte with the even block in the low
// nibble, [rows][nb/2]; the block's E8M0 byte is base + delta).
struct ScaleSrc {
  rsrc_t tab;   // 8-bit table, or scale4 deltas
  rsrc_t base;  // scale4 row bases
  const uint8_t* bptr;  // the same bases, for scalar loads (4-byte aligned)
};

// Scalar (constant address space) view of the row bases: a wave-uniform
// index becomes one s_load_dword, outside the vector memory pipeline.  (Two
// other ways measured slower: a vector load of the base per row, +12% load
// instructions; one vector load of 64 rows' bases read back with readlane,
// which made the compiler wait for all loads every row.)
typedef __attribute__((address_space(4))) const uint32_t scalar_u32;

// The base bytes of rows 4j .. 4j + 3 (j wave-uniform) in one dword.
__device__ __forceinline__ uint32_t bases4(const uint8_t* bptr, int j) {
  return ((scalar_u32*)bptr)[j];  // an address-space cast (C style: reinterpret_cast refuses it)
}

// Scale source of matrix m (0 gate, 1 up, 2 down) of expert e.  scale4
// record of one expert: bases gate [I] | up [I] | down [H], then deltas
// gate [I][H/64] | up [I][H/64] | down [H][I/64].
template <bool S4>
__device__ __forceinline__ ScaleSrc matrix_scales(const uint8_t* scales, int e, int m, int H, int I) {
  if constexpr (S4) {
    const size_t dm = (size_t)I * H / 64;
    const uint8_t* p = scales + (size_t)e * ((size_t)2 * I + H + 3 * dm);
    const size_t boff = m == 2 ? (size_t)2 * I : (size_t)m * I;
    return ScaleSrc{make_rsrc(p + (size_t)2 * I + H + (size_t)m * dm, (uint32_t)dm),
                    make_rsrc(p + boff, (uint32_t)(m == 2 ? H : I)), p + boff};
  } else {
    const uint32_t ms = (uint32_t)((size_t)I * H / 32);
    return ScaleSrc{make_rsrc(scales + (size_t)e * 3 * ms + (size_t)m * ms, ms), make_rsrc(scales, 0u), scales};
  }
}

// One row's worth of a lane's blocks: NBL 16-byte code blocks + scale bytes.
template <int NBL>
struct RowBlocks {
  u32x4 q[NBL];
  uint32_t s[NBL];  // E8M0 byte, or (scale4) the byte holding the block's delta
  uint32_t base;    // scale4: the row's base byte
  uint32_t valid;   // scale4: bit m set when block m exists (a block past the row has scale 0)
};

// Blocks b = c + LPR*m of row `row` (row < 0: none) of a [rows][nb*32] matrix.
template <int LPR, int NBL, bool S4>
__device__ __forceinline__ void load_row(RowBlocks<NBL>& r, rsrc_t codes, const ScaleSrc& sc, int row, int c,
                                         int nb) {
  const uint32_t rc = (uint32_t)row * (uint32_t)(nb * 16);
  const uint32_t rsc = (uint32_t)row * (uint32_t)(S4 ? nb / 2 : nb);
  if constexpr (S4) {
    if constexpr (LPR == kWave) {  // one row per wave: its base by a scalar load
      const int rr = __builtin_amdgcn_readfirstlane(row >= 0 ? row : 0);
      r.base = (bases4(sc.bptr, rr >> 2) >> ((rr & 3) * 8)) & 0xFFu;
    } else {
      r.base = __builtin_amdgcn_raw_buffer_load_b8(sc.base, row >= 0 ? (uint32_t)row : kOOB, 0, 2 /* nt */);
    }
    r.valid = 0u;
  }
#pragma unroll
  for (int m = 0; m < NBL; ++m) {
    const int b = c + LPR * m;
    const bool ok = row >= 0 && b < nb;
    r.q[m] = __builtin_amdgcn_raw_buffer_load_b128(codes, ok ? rc + 16u * b : kOOB, 0, 2 /* nt */);
    if constexpr (S4) {
      r.s[m] = __builtin_amdgcn_raw_buffer_load_b8(sc.tab, ok ? rsc + (uint32_t)(b >> 1) : kOOB, 0, 2 /* nt */);
      r.valid |= ok ? (1u << m) : 0u;
    } else {
      r.s[m] = __builtin_amdgcn_raw_buffer_load_b8(sc.tab, ok ? rsc + b : kOOB, 0, 2 /* nt */);
    }
  }
}

// The E8M0 byte of block m.  scale4: the row base plus the block's nibble
// (sh = 0 for an even block, 4 for an odd one; LPR is even, so all blocks of
// a lane have the parity of its first), read only once the loads have landed;
// a block past the row gets 0, like the 8-bit table's out-of-range read, so
// a NaN or infinite base never meets the zero padding codes.
template <bool S4, int NBL>
__device__ __forceinline__ uint32_t scale_byte(const RowBlocks<NBL>& r, int m, int sh) {
  if constexpr (S4)
    return ((r.valid >> m) & 1u) ? r.base + ((r.s[m] >> sh) & 15u) : 0u;
  else
    return r.s[m];
}

template <bool XF32, int NBL, bool S4, bool PIN = false>
__device__ __forceinline__ float row_dot(const RowBlocks<NBL>& r, const uint32_t (*xr)[XF32 ? 32 : 16], int sh) {
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < NBL; ++m) {
    const float s = e8m0_operand(scale_byte<S4>(r, m, sh));
    const uint4 q = make_uint4(r.q[m].x, r.q[m].y, r.q[m].z, r.q[m].w);
    if constexpr (XF32)
      acc = block_dot_f32<PIN>(q, s, xr[m], acc);
    else
      acc = block_dot_bf16(q, s, xr[m], acc);
  }
  return acc;
}

// Sum over LPR-lane groups; valid at least in the last lane of each group.
template <int LPR>
__device__ __forceinline__ float group_reduce(float v) {
  if constexpr (LPR <= 16) {
    return lane_group_sum<LPR>(v);
  } else if constexpr (LPR == 32) {
    v = row16_sum(v);
    return v + dpp_f<0x142, 0xA>(v);
  } else {
    v = row16_sum(v);
    v += dpp_f<0x142, 0xA>(v);
    return v + dpp_f<0x143, 0xC>(v);
  }
}

// Copies n16 >= 1 16-byte chunks from global memory into LDS with the nthr
// threads me = 0 .. nthr - 1: each thread issues 8 loads before its first LDS
// write, so a batch costs one memory round trip (a load-then-store loop waits
// for every load in turn).  No load or store sits in a branch (the compiler
// would sink a load into its store's branch and wait there): an index past
// the end is clamped to the last chunk, which is then read and written again
// with its own value.
__device__ __forceinline__ void stage_to_lds(uint4* __restrict__ dst, const uint4* __restrict__ src, int n16,
                                             int me, int nthr) {
  constexpr int B = 8;
  for (int c0 = 0; c0 < n16; c0 += B * nthr) {
    uint4 v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int c = c0 + me + u * nthr;
      v[u] = src[c < n16 ? c : n16 - 1];
    }
#pragma unroll
    for (int u = 0; u < B; ++u) {
      const int c = c0 + me + u * nthr;
      dst[c < n16 ? c : n16 - 1] = v[u];
    }
  }
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// Workgroup (pair p, part): wave w takes rows part*4 + w, + 4*parts, ... of
// the gate and up matrices of the pair's expert, LPR = 64 (one row per step),
// the next row loaded while the current one is computed.
// hbuf[p][i] = silu(g_i) * u_i, pair p = t*k + j uses token t = p / k.
// SEL = 0: the pair's expert is route[p].  SEL = MAXV > 0: the workgroup
// selects it itself: wave 0 runs the exact top-k + softmax (topk.h) on the
// token's logits while the token's activations are staged, and the expert of
// rank j = p % k is used; workgroup (p % k == 0, part 0) also writes the
// token's k experts to route[] and their weights to wsel[] for the later
// kernels.  Every workgroup of a token computes the same selection from the
// same logits with the same code, so they agree.
template <bool XF32, int NBL, int SEL, bool S4>
__global__ __launch_bounds__(256) void k_gateup_gemv(const void* __restrict__ x,
                                                     int32_t* __restrict__ route,
                                                     const float* __restrict__ logits,
                                                     float* __restrict__ wsel,
                                                     const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int H, int I,
                                                     int E, int k, int parts, int rpw,
                                                     float* __restrict__ hbuf) {
  extern __shared__ uint4 xs_lds[];
  constexpr int XW = XF32 ? 32 : 16;  // registers per block of activations
  const int p = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int nb = H / 32;
  const int xbytes = XF32 ? H * 4 : H * 2;
  const uint4* xg = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(x) + (size_t)(p / k) * xbytes);
  int e;
  if constexpr (SEL > 0) {
    __shared__ uint64_t cand[2 * kWave];
    __shared__ int32_t chosen;
    // wave 0 selects at once; the other waves stage the activations meanwhile
    if (wid == 0) {
      const int t = p / k;
      int sel;
      float wv;
      const bool writer = part == 0 && p % k == 0;  // the token's workgroup that publishes the selection
      topk_wave<SEL>(logits + (size_t)t * E, E, k, cand, &sel, &wv, writer);
      if (lane == p % k) chosen = sel;
      if (writer && lane < k) {
        route[(size_t)t * k + lane] = sel;
        wsel[(size_t)t * k + lane] = wv;
      }
    } else {
      stage_to_lds(xs_lds, xg, xbytes / 16, threadIdx.x - kWave, 256 - kWave);
    }
    __syncthreads();
    e = __builtin_amdgcn_readfirstlane(chosen);
  } else {
    e = __builtin_amdgcn_readfirstlane(route[p]);
  }
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  const size_t cb = (size_t)3 * I * H / 2;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2);
  const rsrc_t gcod = make_rsrc(codes + (size_t)e * cb, mc);
  const rsrc_t ucod = make_rsrc(codes + (size_t)e * cb + mc, mc);
  const ScaleSrc gsc = matrix_scales<S4>(scales, e, 0, H, I);
  const ScaleSrc usc = matrix_scales<S4>(scales, e, 1, H, I);
  const int sh = (lane & 1) * 4;
  // rows interleaved across the pair's waves
  const int i0 = part * 4 + wid;
  const int istep = parts * 4;
  const int nsteps = i0 < I ? (I - i0 + istep - 1) / istep : 0;

  RowBlocks<NBL> g0, u0, g1, u1;
  load_row<kWave, NBL, S4>(g0, gcod, gsc, nsteps > 0 ? i0 : -1, lane, nb);
  load_row<kWave, NBL, S4>(u0, ucod, usc, nsteps > 0 ? i0 : -1, lane, nb);

  // stage this token's activations (already done when selecting), then keep
  // the lane's blocks in registers
  if constexpr (SEL == 0) {
    stage_to_lds(xs_lds, xg, xbytes / 16, threadIdx.x, 256);
    __syncthreads();
  }
  uint32_t xr[NBL][XW];
#pragma unroll
  for (int m = 0; m < NBL; ++m) {
    const int b = lane + kWave * m;
#pragma unroll
    for (int v = 0; v < XW / 4; ++v) {
      uint4 u = (b < nb) ? xs_lds[b * (XW / 4) + v] : make_uint4(0u, 0u, 0u, 0u);
      xr[m][4 * v] = u.x; xr[m][4 * v + 1] = u.y; xr[m][4 * v + 2] = u.z; xr[m][4 * v + 3] = u.w;
    }
  }

  for (int st = 0; st < nsteps; st += 2) {
    const int i = i0 + st * istep, i1 = i + istep, i2 = i1 + istep;
    const bool has1 = st + 1 < nsteps;
    load_row<kWave, NBL, S4>(g1, gcod, gsc, has1 ? i1 : -1, lane, nb);
    load_row<kWave, NBL, S4>(u1, ucod, usc, has1 ? i1 : -1, lane, nb);
    float ag = wave_sum(row_dot<XF32, NBL, S4>(g0, xr, sh));
    float au = wave_sum(row_dot<XF32, NBL, S4>(u0, xr, sh));
    if (lane == 0) hbuf[(size_t)p * I + i] = silu_mul(ag, au);
    if (!has1) break;
    const bool has2 = st + 2 < nsteps;
    load_row<kWave, NBL, S4>(g0, gcod, gsc, has2 ? i2 : -1, lane, nb);
    load_row<kWave, NBL, S4>(u0, ucod, usc, has2 ? i2 : -1, lane, nb);
    ag = wave_sum(row_dot<XF32, NBL, S4>(g1, xr, sh));
    au = wave_sum(row_dot<XF32, NBL, S4>(u1, xr, sh));
    if (lane == 0) hbuf[(size_t)p * I + i1] = silu_mul(ag, au);
  }
}

// ---------------------------------------------------------------- gate/up + SwiGLU, K split across waves
// For H = 1024*KS (KS in {1, 2, 4, 7, 8}; the model's H = 7168 gives 7): wave
// ks of a 64*KS-thread workgroup takes code blocks 32 ks .. 32 ks + 31 of
// every gate and up row of the workgroup's row range, 32 lanes per row and two
// rows per step (512 contiguous code bytes per row and matrix), so a lane
// keeps one 32-element block of x in registers, loaded straight from memory.
// Low register use lets several waves per SIMD overlap the weight stream with
// the decode and dot-product work.  Each wave reduces its 32 lanes per row and
// leaves the partial sum in LDS; at the end the workgroup adds the KS partials
// of each row in wave order (a fixed order, so results are deterministic) and
// applies SwiGLU.  Weight loads run D - 1 steps ahead; rows_per_wg is a
// multiple of 2 D, so the unrolled ring has no exit inside.
// Scales: the workgroup's rows of both tables (contiguous bytes: 8-bit
// E8M0 bytes, or scale4 deltas and bases) are copied into LDS once before
// the first row, so the only weight loads are the code loads.
// SEL as in k_gateup_gemv; with KS >= 2 waves the selection's per-logit work
// is shared by all of them (topk_wg), and every wave loads x after it.
// Weight steps in flight + 1: 3 with bf16 x, 4 with fp32 x.  Measured on the
// selecting kernel (decode): bf16 31.7-31.9 us at 3 against 32.3 at 4 and
// 32.9 at 5; fp32 (the 12-layer stack) 0.771 ms per token at 4 against 0.788
// at 3 and 0.781 at 5.
template <bool XF32>
constexpr int gu_ks_ring() { return XF32 ? 4 : 3; }
constexpr int kGuKsTabLoads = 2;   // 16-byte scale chunks per thread and matrix
// rows_per_wg * H/32 <= kGuKsTabLoads * 16 * 64 * KS (the table's capacity), in whole ring passes
constexpr int gu_ks_max_rows(int ring) { return 32 * kGuKsTabLoads / (2 * ring) * (2 * ring); }

template <int KS, int D, bool XF32, int SEL, bool S4>
__global__ __launch_bounds__(64 * KS) void k_gateup_ks(const void* __restrict__ x, int32_t* __restrict__ route,
                                                       const float* __restrict__ logits, float* __restrict__ wsel,
                                                       const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales, int H, int I, int E,
                                                       int k, int parts, int rows_per_wg,
                                                       float* __restrict__ hbuf) {
  constexpr int XW = XF32 ? 32 : 16;  // registers per block of x
  // [rows_per_wg][2][KS] partials, then the gate and up scale rows,
  // [rows_per_wg][rb] each (8-bit: rb = H/32 E8M0 bytes; scale4: rb = H/64
  // bytes of deltas, then the rows' bases, [rows_per_wg] each); before them,
  // the selection's scratch
  extern __shared__ __align__(16) float partial[];
  const int p = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const int lane = threadIdx.x % kWave, ks = threadIdx.x / kWave;
  const int c = lane % 32, rsub = lane / 32;
  const int nb = H / 32;
  const int b = ks * 32 + c;  // this lane's block of every row
  const int t = p / k;

  // this lane's 32 activations (with selection, loaded after it: the
  // selection's barriers then wait for nothing in flight, and x arrives
  // alongside the first weights)
  uint32_t xr[1][XW];
  auto load_x = [&]() {
    const u32x4* xp = reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(x) +
                                                     (size_t)t * (XF32 ? H * 4 : H * 2) + (size_t)b * (XW * 4));
#pragma unroll
    for (int v = 0; v < XW / 4; ++v) {
      const u32x4 u = xp[v];
      xr[0][4 * v] = u.x; xr[0][4 * v + 1] = u.y; xr[0][4 * v + 2] = u.z; xr[0][4 * v + 3] = u.w;
    }
  };
  int e;
  if constexpr (SEL > 0) {
    __shared__ int32_t chosen;
    int sel;
    float wv;
    const bool writer = part == 0 && p % k == 0;  // the token's workgroup that publishes the selection
    if constexpr (KS >= 2) {
      // all waves share the per-logit work; wave 0 holds the result.  The
      // scratch is the dynamic LDS, which nothing uses before the selection
      // ends (the launcher makes it at least sizeof(TopkWgLds<KS>)), so the
      // selection adds no LDS to the workgroup.
      TopkWgLds<KS>& tsm = *reinterpret_cast<TopkWgLds<KS>*>(partial);
      topk_wg<KS, (SEL + KS - 1) / KS, SEL>(logits + (size_t)t * E, E, k, tsm, &sel, &wv, writer);
    } else {
      __shared__ uint64_t cand[2 * kWave];
      topk_wave<SEL>(logits + (size_t)t * E, E, k, cand, &sel, &wv, writer);
    }
    if (ks == 0) {
      if (lane == p % k) chosen = sel;
      if (writer && lane < k) {
        route[(size_t)t * k + lane] = sel;
        wsel[(size_t)t * k + lane] = wv;
      }
    }
    __syncthreads();
    e = __builtin_amdgcn_readfirstlane(chosen);
    load_x();
  } else {
    load_x();
    e = __builtin_amdgcn_readfirstlane(route[p]);
  }
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  const size_t cb = (size_t)3 * I * H / 2;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2);
  const rsrc_t gcod = make_rsrc(codes + (size_t)e * cb, mc);
  const rsrc_t ucod = make_rsrc(codes + (size_t)e * cb + mc, mc);
  const ScaleSrc gsc = matrix_scales<S4>(scales, e, 0, H, I);
  const ScaleSrc usc = matrix_scales<S4>(scales, e, 1, H, I);
  const int sh = (c & 1) * 4;
  const int r0 = part * rows_per_wg;
  const int nrows = min(rows_per_wg, I - r0);
  const int steps = rows_per_wg / 2;

  // Both matrices' scale rows r0 .. r0 + nrows - 1, loaded first (the
  // ring's loads behind them need not land before the table is written);
  // rb is a multiple of 16 (H = 1024 KS), so chunks never straddle rows.
  const int rb = S4 ? nb / 2 : nb;
  uint8_t* tab = reinterpret_cast<uint8_t*>(partial + rows_per_wg * 2 * KS);
  uint8_t* tab_base = tab + 2 * rows_per_wg * rb;  // scale4: gate bases, then up bases
  const int tab_n16 = nrows * rb / 16;             // chunks per matrix
  u32x4 tg[kGuKsTabLoads], tu[kGuKsTabLoads];
  uint32_t bg = 0u, bu = 0u;                       // scale4: this thread's row base (one byte a thread)
#pragma unroll
  for (int u = 0; u < kGuKsTabLoads; ++u) {
    const int j = threadIdx.x + u * 64 * KS;
    const uint32_t off = j < tab_n16 ? (uint32_t)r0 * (uint32_t)rb + 16u * j : kOOB;
    tg[u] = __builtin_amdgcn_raw_buffer_load_b128(gsc.tab, off, 0, 2 /* nt */);
    tu[u] = __builtin_amdgcn_raw_buffer_load_b128(usc.tab, off, 0, 2 /* nt */);
  }
  if constexpr (S4) {
    // byte loads: r0 is a multiple of two ring passes, not necessarily of 4
    const uint32_t off = (int)threadIdx.x < nrows ? (uint32_t)r0 + threadIdx.x : kOOB;
    bg = __builtin_amdgcn_raw_buffer_load_b8(gsc.base, off, 0, 2 /* nt */);
    bu = __builtin_amdgcn_raw_buffer_load_b8(usc.base, off, 0, 2 /* nt */);
  }
  auto load = [&](RowBlocks<1>& r, rsrc_t cod, int st) {
    const int n = r0 + 2 * st + rsub;
    const bool ok = st < steps && n < I;
    r.q[0] = __builtin_amdgcn_raw_buffer_load_b128(cod, ok ? (uint32_t)n * (uint32_t)(H / 2) + 16u * b : kOOB, 0,
                                                   2 /* nt */);
    r.s[0] = 0u;  // read from LDS when the step is computed
  };
  RowBlocks<1> gr[D], ur[D];
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    load(gr[d], gcod, d);
    load(ur[d], ucod, d);
  }
#pragma unroll
  for (int u = 0; u < kGuKsTabLoads; ++u) {
    const int j = threadIdx.x + u * 64 * KS;
    if (j < tab_n16) {
      reinterpret_cast<u32x4*>(tab)[j] = tg[u];
      reinterpret_cast<u32x4*>(tab + rows_per_wg * rb)[j] = tu[u];
    }
  }
  if constexpr (S4) {
    if ((int)threadIdx.x < nrows) {
      tab_base[threadIdx.x] = (uint8_t)bg;
      tab_base[rows_per_wg + threadIdx.x] = (uint8_t)bu;
    }
  }
  __syncthreads();

  for (int s0 = 0; s0 < steps; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int st = s0 + d;
      load(gr[(d + D - 1) % D], gcod, st + D - 1);
      load(ur[(d + D - 1) % D], ucod, st + D - 1);
      const int rr = 2 * st + rsub;  // a row past I reads table bytes no result uses
      if constexpr (S4) {
        gr[d].s[0] = tab[rr * rb + (b >> 1)];
        ur[d].s[0] = tab[(rows_per_wg + rr) * rb + (b >> 1)];
        gr[d].base = tab_base[rr];
        ur[d].base = tab_base[rows_per_wg + rr];
        gr[d].valid = ur[d].valid = 1u;  // b < H/32 always
      } else {
        gr[d].s[0] = tab[rr * nb + b];
        ur[d].s[0] = tab[(rows_per_wg + rr) * nb + b];
      }
      const float ag = group_reduce<32>(row_dot<XF32, 1, S4, true>(gr[d], xr, sh));
      const float au = group_reduce<32>(row_dot<XF32, 1, S4, true>(ur[d], xr, sh));
      if (c == 31) {
        partial[(2 * rr) * KS + ks] = ag;
        partial[(2 * rr + 1) * KS + ks] = au;
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nrows; i += 64 * KS) {
    float g = partial[(2 * i) * KS], u = partial[(2 * i + 1) * KS];
#pragma unroll
    for (int k2 = 1; k2 < KS; ++k2) {
      g += partial[(2 * i) * KS + k2];
      u += partial[(2 * i + 1) * KS + k2];
    }
    hbuf[(size_t)p * I + r0 + i] = silu_mul(g, u);
  }
}

// ---------------------------------------------------------------- down
// Workgroup (pair p, part): rows of Wd [H][I] of expert pair_expert[p]; LPR
// lanes per row, RPS = 64/LPR rows per step, `steps` steps per wave, row
// groups interleaved across the pair's waves, weights loaded three steps
// ahead from a ring of four.  The pair's h row is staged in LDS and each lane
// keeps its NBL2 blocks in registers.
template <int LPR, int NBL2, bool S4>
__global__ __launch_bounds__(256) void k_down_gemv(const float* __restrict__ hbuf,
                                                   const int32_t* __restrict__ pair_expert,
                                                   const uint8_t* __restrict__ codes,
                                                   const uint8_t* __restrict__ scales, int H, int I,
                                                   int E, int parts, int steps, float* __restrict__ ybuf) {
  extern __shared__ float hs_lds[];
  constexpr int RPS = kWave / LPR;
  constexpr int D = 4;  // weight loads run D-1 steps ahead
  const int p = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int c = lane % LPR, rsub = lane / LPR;
  int e = __builtin_amdgcn_readfirstlane(pair_expert[p]);
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  const int nbk = I / 32;
  const size_t cb = (size_t)3 * I * H / 2;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2);
  const rsrc_t dcod = make_rsrc(codes + (size_t)e * cb + 2 * (size_t)mc, mc);
  const ScaleSrc dsc = matrix_scales<S4>(scales, e, 2, H, I);
  const int sh = (c & 1) * 4;
  // row groups interleaved across the pair's waves (see k_gateup_gemv)
  const int n_begin = (part * 4 + wid) * RPS + rsub;
  const int n_step = parts * 4 * RPS;

  RowBlocks<NBL2> ring[D];
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    const int n = n_begin + d * n_step;
    load_row<LPR, NBL2, S4>(ring[d], dcod, dsc, (d < steps && n < H) ? n : -1, c, nbk);
  }

  const float4* hsrc = reinterpret_cast<const float4*>(hbuf + (size_t)p * I);
  stage_to_lds(reinterpret_cast<uint4*>(hs_lds), reinterpret_cast<const uint4*>(hsrc), I / 4, threadIdx.x, 256);
  __syncthreads();
  uint32_t hr[NBL2][32];
#pragma unroll
  for (int m = 0; m < NBL2; ++m) {
    const int b = c + LPR * m;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      float4 f = (b < nbk) ? reinterpret_cast<const float4*>(hs_lds)[b * 8 + v] : make_float4(0.f, 0.f, 0.f, 0.f);
      hr[m][4 * v] = __float_as_uint(f.x); hr[m][4 * v + 1] = __float_as_uint(f.y);
      hr[m][4 * v + 2] = __float_as_uint(f.z); hr[m][4 * v + 3] = __float_as_uint(f.w);
    }
  }

  for (int s0 = 0; s0 < steps; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int st = s0 + d;
      if (st >= steps) break;
      const int sn = st + D - 1;
      const int nn = n_begin + sn * n_step;
      load_row<LPR, NBL2, S4>(ring[(d + D - 1) % D], dcod, dsc, (sn < steps && nn < H) ? nn : -1, c, nbk);
      const int n0 = n_begin + st * n_step;
      const float acc = group_reduce<LPR>(row_dot<true, NBL2, S4>(ring[d], hr, sh));
      if (c == LPR - 1 && n0 < H) ybuf[(size_t)p * H + n0] = acc;
    }
  }
}

// ---------------------------------------------------------------- down, K split across waves
constexpr int kDnKsRing = 4;   // weight steps in flight + 1 (measured best of 2..8)
constexpr int kDnKsPerCu = 8;  // workgroups per CU the grid aims at (measured best of 2..12)
// Largest LDS table of row partials per workgroup: with many pairs the grid
// target alone would give one workgroup all H rows (H * KS * 4 bytes, over
// the 160 KiB a workgroup may have at H = 8192, I = 4096); capped, the rows
// are split into more parts instead.
constexpr int kDnKsLdsCap = 16384;
// For I = 512*KS (I/32 = 16*KS blocks per row): wave ks of a workgroup takes
// blocks 16*ks .. 16*ks+15 of every row of the workgroup's row range, 16
// lanes per row and 4 rows per step (256 contiguous code bytes per row), so a
// lane keeps one 32-element block of h in registers (32 fp32) instead of
// three and the kernel runs several waves per SIMD, which lets the weight
// stream and the conversion + FMA work overlap.  Each wave reduces its 16
// lanes per row and leaves the partial sum in LDS; at the end the workgroup
// adds the KS partials of each row in wave order (a fixed order, so results
// are deterministic).  Weight loads run D-1 steps ahead; rows_per_wg is a
// multiple of 4*D, so the unrolled ring has no exit inside.
//
// TAB: the workgroup's scale bytes are copied into LDS once, before the
// first row, by one 16-byte load per thread and chunk; each step then reads
// its scale from LDS instead of issuing a one-byte load per code load.  The
// table holds rows_per_wg rows x rb contiguous bytes of the matrix's scales:
// 8-bit, rb = I/32 E8M0 bytes; scale4, rb = I/64 bytes of deltas, followed
// by the rows' bases (rows_per_wg bytes, loaded a dword per thread).
template <int KS, int D, bool S4, bool TAB>
__global__ __launch_bounds__(64 * KS) void k_down_ks(const float* __restrict__ hbuf,
                                                     const int32_t* __restrict__ pair_expert,
                                                     const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int H, int I, int E,
                                                     int parts, int rows_per_wg, float* __restrict__ ybuf) {
  extern __shared__ float partial[];  // [rows_per_wg][KS], then (TAB) the scale table
  const int p = blockIdx.x / parts;
  const int part = blockIdx.x % parts;
  const int lane = threadIdx.x % kWave, ks = threadIdx.x / kWave;
  const int c = lane % 16, rsub = lane / 16;
  int e = __builtin_amdgcn_readfirstlane(pair_expert[p]);
  e = e < 0 ? 0 : (e >= E ? E - 1 : e);
  const int nbk = I / 32;
  const size_t cb = (size_t)3 * I * H / 2;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2);
  const rsrc_t dcod = make_rsrc(codes + (size_t)e * cb + 2 * (size_t)mc, mc);
  const ScaleSrc dsc = matrix_scales<S4>(scales, e, 2, H, I);
  const int b = ks * 16 + c;  // this lane's block of every row
  const int sh = (c & 1) * 4;
  const int r0 = part * rows_per_wg;
  const int steps = rows_per_wg / 4;

  // TAB: the table's 16-byte chunks (and scale4 bases), loaded first (the
  // ring's loads behind them need not land before the table is written to
  // LDS).  rows_per_wg * rb is a multiple of 16, so the last chunk of a
  // short last part stays inside the delta rows.
  const int rb = S4 ? nbk / 2 : nbk;
  uint8_t* tab = reinterpret_cast<uint8_t*>(partial + rows_per_wg * KS);
  uint8_t* tab_base = tab + rows_per_wg * rb;  // scale4 bases
  const int nrows = min(rows_per_wg, H - r0);
  const int tab_n16 = TAB ? (nrows * rb + 15) / 16 : 0;
  const int tab_nb4 = TAB && S4 ? (nrows + 3) / 4 : 0;
  constexpr int kTabLoads = 2;  // chunks per thread (rows_per_wg * rb <= 2 * 16 * 64 * KS)
  u32x4 tv[kTabLoads];
  uint32_t tbase = 0u;
  if constexpr (TAB) {
#pragma unroll
    for (int u = 0; u < kTabLoads; ++u) {
      const int t = threadIdx.x + u * 64 * KS;
      tv[u] = __builtin_amdgcn_raw_buffer_load_b128(dsc.tab, t < tab_n16 ? (uint32_t)r0 * (uint32_t)rb + 16u * t : kOOB,
                                                    0, 2 /* nt */);
    }
    if constexpr (S4)
      tbase = __builtin_amdgcn_raw_buffer_load_b32(dsc.base, (int)threadIdx.x < tab_nb4 ? (uint32_t)r0 + 4u * threadIdx.x
                                                                                         : kOOB,
                                                   0, 2 /* nt */);
  }
  auto load = [&](RowBlocks<1>& r, int st) {
    const int n = r0 + 4 * st + rsub;
    const bool ok = st < steps && n < H;
    r.q[0] = __builtin_amdgcn_raw_buffer_load_b128(dcod, ok ? (uint32_t)n * (uint32_t)(I / 2) + 16u * b : kOOB, 0, 2);
    if constexpr (TAB) {
      r.s[0] = 0u;  // read from LDS when the step is computed
    } else if constexpr (S4) {
      // rows r0 + 4 st .. + 3 (4-aligned) share one dword of bases: a scalar load
      const int j = (st < steps && r0 + 4 * st < H) ? (r0 + 4 * st) >> 2 : 0;
      r.base = (bases4(dsc.bptr, j) >> (rsub * 8)) & 0xFFu;
      r.s[0] = __builtin_amdgcn_raw_buffer_load_b8(dsc.tab, ok ? (uint32_t)n * (uint32_t)(nbk / 2) + (uint32_t)(b >> 1) : kOOB,
                                                   0, 2 /* nt */);
      r.valid = ok ? 1u : 0u;
    } else {
      r.s[0] = __builtin_amdgcn_raw_buffer_load_b8(dsc.tab, ok ? (uint32_t)n * (uint32_t)nbk + b : kOOB, 0, 2 /* nt */);
    }
  };
  // h before the ring: loads complete in issue order, so the first row's
  // wait for h then leaves the ring's later loads in flight (issued after
  // the ring, that wait would cover them too, and the compiler keeps it in
  // every pass of the loop)
  uint32_t hr[1][32];
  const float4* hp = reinterpret_cast<const float4*>(hbuf + (size_t)p * I + 32 * b);
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const float4 f = hp[v];
    hr[0][4 * v] = __float_as_uint(f.x); hr[0][4 * v + 1] = __float_as_uint(f.y);
    hr[0][4 * v + 2] = __float_as_uint(f.z); hr[0][4 * v + 3] = __float_as_uint(f.w);
  }
  RowBlocks<1> ring[D];
#pragma unroll
  for (int d = 0; d < D - 1; ++d) load(ring[d], d);

  if constexpr (TAB) {
#pragma unroll
    for (int u = 0; u < kTabLoads; ++u) {
      const int t = threadIdx.x + u * 64 * KS;
      if (t < tab_n16) reinterpret_cast<u32x4*>(tab)[t] = tv[u];
    }
    if constexpr (S4)
      if ((int)threadIdx.x < tab_nb4) reinterpret_cast<uint32_t*>(tab_base)[threadIdx.x] = tbase;
    __syncthreads();
  }

  for (int s0 = 0; s0 < steps; s0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int st = s0 + d;
      load(ring[(d + D - 1) % D], st + D - 1);
      if constexpr (TAB) {
        const int rr = 4 * st + rsub;  // a row past H reads bytes no result uses
        if constexpr (S4) {
          ring[d].s[0] = tab[rr * rb + (b >> 1)];
          ring[d].base = tab_base[rr];
          ring[d].valid = 1u;  // b < I/32 always
        } else {
          ring[d].s[0] = tab[rr * nbk + b];
        }
      }
      const float v = lane_group_sum<16>(row_dot<true, 1, S4, true>(ring[d], hr, sh));
      if (c == 15) partial[(4 * st + rsub) * KS + ks] = v;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < rows_per_wg; i += 64 * KS) {
    const int n = r0 + i;
    if (n < H) {
      float acc = partial[i * KS];
#pragma unroll
      for (int k2 = 1; k2 < KS; ++k2) acc += partial[i * KS + k2];
      ybuf[(size_t)p * H + n] = acc;
    }
  }
}

// ---------------------------------------------------------------- combine
// out[t][n] = (resid[t][n] +) sum_j w[t][j] * y[t*k+j][n], j ascending; resid
// may alias out.  Loads are issued in groups of 16 ranks (one group for the
// usual k <= 16), so a thread waits for memory once per group.
__global__ __launch_bounds__(256) void k_combine(const float* __restrict__ ybuf,
                                                const float* __restrict__ w, int T, int k, int H,
                                                const float* resid, float* out) {
  constexpr int G = 16;
  const size_t n4 = (size_t)T * H / 4;
  for (size_t q = (size_t)blockIdx.x * 256 + threadIdx.x; q < n4; q += (size_t)gridDim.x * 256) {
    const size_t flat = 4 * q;
    const int t = (int)(flat / H);
    const int n = (int)(flat % H);
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    if (resid) r = *reinterpret_cast<const float4*>(resid + flat);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j0 = 0; j0 < k; j0 += G) {
      float4 y[G];
      float wj[G];
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int j = j0 + u;
        if (j < k) {
          // read once: a non-temporal load (4096 tokens: 374 -> 330 us)
          const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(ybuf + ((size_t)t * k + j) * H + n));
          y[u] = make_float4(v.x, v.y, v.z, v.w);
          wj[u] = w[(size_t)t * k + j];
        } else {
          y[u] = make_float4(0.f, 0.f, 0.f, 0.f);
          wj[u] = 0.0f;
        }
      }
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (j0 + u < k) {
          acc.x = fmaf(wj[u], y[u].x, acc.x);
          acc.y = fmaf(wj[u], y[u].y, acc.y);
          acc.z = fmaf(wj[u], y[u].z, acc.z);
          acc.w = fmaf(wj[u], y[u].w, acc.w);
        }
      }
    }
    if (resid) {
      acc.x = r.x + acc.x; acc.y = r.y + acc.y; acc.z = r.z + acc.z; acc.w = r.w + acc.w;
    }
    *reinterpret_cast<float4*>(out + flat) = acc;
  }
}

// ---------------------------------------------------------------- launchers

// Rows per wave and workgroups per pair so that about `target` workgroups
// share all pairs equally; `unit` = rows one wave handles per step.
static void split_rows(int rows, int P, int unit, int target, int* parts, int* per_wave) {
  int want = (target + P - 1) / P;
  const int max_parts = (rows + 4 * unit - 1) / (4 * unit);
  if (want > max_parts) want = max_parts;
  if (want < 1) want = 1;
  int pw = (rows + 4 * want - 1) / (4 * want);     // rows per wave
  pw = (pw + unit - 1) / unit * unit;
  *per_wave = pw;
  *parts = (rows + 4 * pw - 1) / (4 * pw);
}

// The K-split gate/up for H = 1024*KS: about as many workgroups as the GPU
// holds at once share all pairs' rows equally (rows per workgroup a multiple
// of two ring passes, at most gu_ks_max_rows so the scale table fits).
template <int KS, bool XF32, int SEL, bool S4>
static hipError_t gateup_ks_launch(int P, hipStream_t s, const void* x, int32_t* route, const float* logits,
                                   float* wsel, const uint8_t* codes, const uint8_t* scales, int H, int I, int E,
                                   int k, float* hbuf) {
  constexpr int D = gu_ks_ring<XF32>();
  constexpr int kMaxRows = gu_ks_max_rows(D);
  static_assert(kMaxRows % (2 * D) == 0, "whole ring passes");
  // the selection (SEL > 0, KS >= 2) keeps its scratch in the same LDS first
  constexpr size_t sel_lds = (SEL > 0 && KS >= 2) ? sizeof(TopkWgLds<KS>) : 0;
  auto lds_for = [&](int rows) {
    return std::max(sel_lds, (size_t)rows * 2 * KS * 4 +
                                 (S4 ? (size_t)2 * rows * (H / 64 + 1) : (size_t)2 * rows * (H / 32)));
  };
  const int target = resident_wgs(k_gateup_ks<KS, D, XF32, SEL, S4>, lds_for(kMaxRows), 64 * KS);
  const int want = (target + P - 1) / P;
  int rows = (I + want - 1) / want;
  rows = (rows + 2 * D - 1) / (2 * D) * (2 * D);
  if (rows > kMaxRows) rows = kMaxRows;
  const int parts = (I + rows - 1) / rows;
  k_gateup_ks<KS, D, XF32, SEL, S4><<<dim3((unsigned)(P * parts)), 64 * KS, lds_for(rows), s>>>(
      x, route, logits, wsel, codes, scales, H, I, E, k, parts, rows, hbuf);
  return hipGetLastError();
}

template <bool XF32, int SEL, bool S4>
static hipError_t gateup_dispatch(int nbl, int P, size_t lds, hipStream_t s, const void* x, int32_t* route,
                                  const float* logits, float* wsel, const uint8_t* codes, const uint8_t* scales,
                                  int H, int I, int E, int k, float* hbuf) {
  if (SEL <= 16 && H % 1024 == 0) {  // K split across H/1024 waves
#define MOE_GUK(KS) \
  return gateup_ks_launch<KS, XF32, (SEL <= 16 ? SEL : 16), S4>(P, s, x, route, logits, wsel, codes, scales, H, I, E, k, hbuf);
    switch (H / 1024) {
      case 1: MOE_GUK(1)
      case 2: MOE_GUK(2)
      case 4: MOE_GUK(4)
      case 7: MOE_GUK(7)
      case 8: MOE_GUK(8)
      default: break;
    }
#undef MOE_GUK
  }
#define MOE_GU(N)                                                                                    \
  {                                                                                                    \
    int parts, rpw;                                                                                    \
    split_rows(I, P, 1, resident_wgs(k_gateup_gemv<XF32, N, SEL, S4>, lds), &parts, &rpw); \
    k_gateup_gemv<XF32, N, SEL, S4><<<dim3((unsigned)(P * parts)), 256, lds, s>>>(                     \
        x, route, logits, wsel, codes, scales, H, I, E, k, parts, rpw, hbuf);                          \
  }
  switch (nbl) {
    case 1: MOE_GU(1); break;
    case 2: MOE_GU(2); break;
    case 3: MOE_GU(3); break;
    case 4: MOE_GU(4); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_GU
  return hipGetLastError();
}

hipError_t launch_gateup_gemv(const void* x, bool x_f32, const int32_t* route, int P, int k,
                              const uint8_t* codes, const uint8_t* scales, bool s4, int H, int I, int E,
                              float* hbuf, hipStream_t s) {
  const int nbl = (H / 32 + kWave - 1) / kWave;
  const size_t lds = (size_t)H * (x_f32 ? 4 : 2);
  int32_t* r = const_cast<int32_t*>(route);  // read only when SEL == 0
#define MOE_GUR(XF, S4_) \
  return gateup_dispatch<XF, 0, S4_>(nbl, P, lds, s, x, r, nullptr, nullptr, codes, scales, H, I, E, k, hbuf);
  if (s4) {
    if (x_f32) MOE_GUR(true, true)
    MOE_GUR(false, true)
  }
  if (x_f32) MOE_GUR(true, false)
  MOE_GUR(false, false)
#undef MOE_GUR
}

template <bool S4>
static hipError_t gateup_select_dispatch(int nbl, int P, size_t lds, hipStream_t s, const void* x, bool x_f32,
                                         const float* logits, int k, const uint8_t* codes, const uint8_t* scales,
                                         int H, int I, int E, int32_t* route, float* wsel, float* hbuf) {
#define MOE_GUS(XF, MV) \
  return gateup_dispatch<XF, MV, S4>(nbl, P, lds, s, x, route, logits, wsel, codes, scales, H, I, E, k, hbuf);
  if (x_f32) {
    if (E <= 256) MOE_GUS(true, 4)
    if (E <= 1024) MOE_GUS(true, 16)
    MOE_GUS(true, 64)
  }
  if (E <= 256) MOE_GUS(false, 4)
  if (E <= 1024) MOE_GUS(false, 16)
  MOE_GUS(false, 64)
#undef MOE_GUS
}

hipError_t launch_gateup_select_gemv(const void* x, bool x_f32, const float* logits, int T, int k,
                                     const uint8_t* codes, const uint8_t* scales, bool s4, int H, int I, int E,
                                     int32_t* route, float* wsel, float* hbuf, hipStream_t s) {
  const int nbl = (H / 32 + kWave - 1) / kWave;
  const size_t lds = (size_t)H * (x_f32 ? 4 : 2);
  const int P = T * k;
  if (s4)
    return gateup_select_dispatch<true>(nbl, P, lds, s, x, x_f32, logits, k, codes, scales, H, I, E, route, wsel,
                                        hbuf);
  return gateup_select_dispatch<false>(nbl, P, lds, s, x, x_f32, logits, k, codes, scales, H, I, E, route, wsel, hbuf);
}

// Lanes per row and blocks per lane for a reduction length of nbk blocks:
// the LPR in {4, 8, 16, 32, 64} with NBL2 = ceil(nbk / LPR) <= 4 that leaves
// the fewest idle lane slots (the smallest such LPR on ties).
void down_shape(int nbk, int* lpr, int* nbl2) {
  static const int cand[5] = {4, 8, 16, 32, 64};
  int best = 4, best_idle = 1 << 30;
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

#define MOE_DOWN_CASE(L, N)                                                                          \
  if (lpr == L && nbl2 == N) {                                                                     \
    int parts, rpw;                                                                                \
    split_rows(H, P, kWave / L, resident_wgs(k_down_gemv<L, N, S4>, lds), &parts, &rpw);          \
    k_down_gemv<L, N, S4><<<dim3((unsigned)(P * parts)), 256, lds, s>>>(hbuf, pair_expert, codes, scales, \
                                                                   H, I, E, parts, rpw / (kWave / L), \
                                                                   ybuf);                            \
    return hipGetLastError();                                                                        \
  }

template <bool S4>
static hipError_t down_dispatch(const float* hbuf, const int32_t* pair_expert, int P, const uint8_t* codes,
                                const uint8_t* scales, int H, int I, int E, float* ybuf, hipStream_t s) {
  const int ks = I % 512 == 0 ? I / 512 : 0;
  if (ks == 2 || ks == 3 || ks == 4 || ks == 6 || ks == 8) {
    // K split across I/512 waves; about kDnKsPerCu workgroups per CU
    constexpr int D = kDnKsRing;
    const int want = (kDnKsPerCu * cu_count() + P - 1) / P;
    int rows = (H + want - 1) / want;
    rows = (rows + 4 * D - 1) / (4 * D) * (4 * D);
    const int max_rows = kDnKsLdsCap / (ks * 4) / (4 * D) * (4 * D);
    if (rows > max_rows) rows = max_rows;
    const int parts = (H + rows - 1) / rows;
    // the LDS scale table when the workgroup's scales fit two 16-byte chunks per thread
    // (scale4: deltas, I/64 bytes a row, then a base byte a row)
    const int rb = S4 ? I / 64 : I / 32;
    const bool tab = rows * rb <= 2 * 16 * 64 * ks && (!S4 || rows <= 4 * 64 * ks);
    const size_t lds = (size_t)rows * ks * 4 + (tab ? (size_t)rows * rb + (S4 ? (size_t)rows : 0) : 0);
    const dim3 grid((unsigned)(P * parts));
#define MOE_DN_KS(KS)                                                                                     \
  if (ks == KS) {                                                                                          \
    if (tab)                                                                                               \
      k_down_ks<KS, D, S4, true><<<grid, 64 * KS, lds, s>>>(hbuf, pair_expert, codes, scales, H, I, E,     \
                                                           parts, rows, ybuf);                             \
    else                                                                                                   \
      k_down_ks<KS, D, S4, false><<<grid, 64 * KS, lds, s>>>(hbuf, pair_expert, codes, scales, H, I, E,    \
                                                            parts, rows, ybuf);                            \
  }
    MOE_DN_KS(2) MOE_DN_KS(3) MOE_DN_KS(4) MOE_DN_KS(6) MOE_DN_KS(8)
#undef MOE_DN_KS
    return hipGetLastError();
  }
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

hipError_t launch_down_gemv(const float* hbuf, const int32_t* pair_expert, int P, const uint8_t* codes,
                            const uint8_t* scales, bool s4, int H, int I, int E, float* ybuf, hipStream_t s) {
  if (s4) return down_dispatch<true>(hbuf, pair_expert, P, codes, scales, H, I, E, ybuf, s);
  return down_dispatch<false>(hbuf, pair_expert, P, codes, scales, H, I, E, ybuf, s);
}

hipError_t launch_combine(const float* ybuf, const float* w, int T, int k, int H, const float* resid,
                          float* out, hipStream_t s) {
  const size_t n4 = (size_t)T * H / 4;
  // one float4 column per thread (measured faster than capping the grid and
  // striding); the cap only bounds the grid for very many tokens
  size_t blocks = (n4 + 255) / 256;
  if (blocks > (1u << 20)) blocks = 1u << 20;
  k_combine<<<dim3((unsigned)blocks), 256, 0, s>>>(ybuf, w, T, k, H, resid, out);
  return hipGetLastError();
}

}  // namespace moe
