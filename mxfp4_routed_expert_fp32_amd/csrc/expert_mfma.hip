// Prefill-form expert kernels: grouped GEMMs over the tokens routed to each
// expert, on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// Exactness: bf16 activations are exact bf16 operands; MXFP4 weights are
// decoded to bf16 exactly (every E2M1 value times a power of two fits bf16);
// products are exact in fp32 and sums are fp32.  The SwiGLU output h (fp32)
// feeds the down projection as two bf16 terms, h = hi + lo with
// hi = bf16(h), lo = bf16(h - hi); the dropped remainder is below 2^-17 |h|.
//
// Work: the token -> expert sort yields, per expert, its (token, rank) pairs
// in token order; those are cut into expert blocks of at most kMB pairs.  A
// workgroup computes one expert block times one tile of output rows.  Block
// index -> (expert block, row tile) is XCD-aware: all row tiles of an expert
// block go to one XCD (hardware hands workgroup b to XCD b % 8), so the
// block's activation rows stay in that XCD's L2 while its row tiles run.
//
// Operand layout of v_mfma_f32_16x16x32_bf16: lane l holds A[m = l%16][k] and
// B[k][n = l%16] for k = 8*(l/16) .. +8; D lane l holds D[4*(l/16) .. +4][l%16].
// Here A = activations (m = token) and B = weights (n = output row).  The K
// axis is permuted the same way on both sides: in MFMA step s of a 128-wide
// K chunk, lane group g = l/16 supplies K = chunk + 32*g + 8*s .. +8, so each
// lane reads one whole 16-byte code block (32 codes) per chunk and uses a
// quarter of it per step.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMB = 128;       // pairs per expert block (8 m-tiles of 16)
constexpr int kKC = 128;       // K per chunk (4 blocks of 32)
constexpr int kLdsRow = kKC + 8;  // bf16 per LDS row (16-byte pad against bank conflicts)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t mk_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------- expert blocks
// blocks[b] = {expert, first index into the sorted pair list, pair count, 0};
// *nblocks = number of blocks.  One workgroup.
__global__ __launch_bounds__(1024) void k_expert_blocks(const int32_t* __restrict__ offsets, int E,
                                                        int4* __restrict__ blocks,
                                                        int32_t* __restrict__ nblocks) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (E + 1023) / 1024;
  const int e0 = tid * per;
  int32_t local = 0;
  for (int e = e0; e < e0 + per && e < E; ++e) local += (offsets[e + 1] - offsets[e] + kMB - 1) / kMB;
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int32_t v = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t b = part[tid] - local;
  for (int e = e0; e < e0 + per && e < E; ++e) {
    const int32_t beg = offsets[e], cnt = offsets[e + 1] - beg;
    for (int32_t m0 = 0; m0 < cnt; m0 += kMB) blocks[b++] = make_int4(e, beg + m0, min(kMB, cnt - m0), 0);
  }
  if (tid == 1023) *nblocks = part[1023];
}

// Workgroup -> (expert block, row tile): row tiles of one block on one XCD.
__device__ __forceinline__ void decode_item(int ntiles, int* eb, int* nt) {
  const int xcd = blockIdx.x % 8, r = blockIdx.x / 8;
  *eb = (r / ntiles) * 8 + xcd;
  *nt = r % ntiles;
}

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

// Stage rows [0, kMB) x K [k0, k0+kKC) of a bf16 source into registers:
// thread t loads 16-byte pieces q = t + 256*v (row q/16, piece q%16).  Rows
// past `cnt` and rows whose source index is negative are zero.
struct AStage {
  uint4 v[8];
};

__device__ __forceinline__ void stage_load(AStage& a, const uint16_t* __restrict__ src, size_t row_stride,
                                           const int32_t* rows_lds, int cnt, int k0) {
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int q = threadIdx.x + 256 * v;
    const int row = q / 16, piece = q % 16;
    const int sr = row < cnt ? rows_lds[row] : -1;
    if (sr >= 0)
      a.v[v] = *reinterpret_cast<const uint4*>(src + (size_t)sr * row_stride + k0 + piece * 8);
    else
      a.v[v] = make_uint4(0u, 0u, 0u, 0u);
  }
}

__device__ __forceinline__ void stage_store(const AStage& a, uint16_t* lds) {
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int q = threadIdx.x + 256 * v;
    const int row = q / 16, piece = q % 16;
    *reinterpret_cast<uint4*>(lds + row * kLdsRow + piece * 8) = a.v[v];
  }
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// Row tile = 128 rows of gate and the same 128 rows of up; wave w owns rows
// 32w .. 32w+31 of the tile (two 16-row n-tiles per matrix).  Output: h as
// two bf16 terms hterm[0][p][i] = hi, hterm[1][p][i] = lo for each pair p.
constexpr int kGU_NT = 128;

__global__ __launch_bounds__(256, 2) void k_gateup_mfma(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pairs, const int4* __restrict__ blocks,
    const int32_t* __restrict__ nblocks, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int H, int I, int k, int P, int ntiles,
    uint16_t* __restrict__ hterm) {
  extern __shared__ uint16_t a_lds[];  // [kMB][kLdsRow]
  __shared__ int32_t tok[kMB], pid[kMB];
  int eb, nt;
  decode_item(ntiles, &eb, &nt);
  if (eb >= *nblocks) return;
  const int4 blk = blocks[eb];
  const int e = blk.x, cnt = blk.z;
  for (int i = threadIdx.x; i < kMB; i += 256) {
    const int p = i < cnt ? pairs[blk.y + i] : -1;
    pid[i] = p;
    tok[i] = p >= 0 ? p / k : -1;
  }
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int nl = lane % 16, g = lane / 16;
  const int mtiles = (cnt + 15) / 16;
  const size_t cb = (size_t)3 * I * H / 2, sb = (size_t)3 * I * H / 32;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2), ms = (uint32_t)((size_t)I * H / 32);
  const rsrc_t rc[2] = {mk_rsrc(codes + (size_t)e * cb, mc), mk_rsrc(codes + (size_t)e * cb + mc, mc)};
  const rsrc_t rs[2] = {mk_rsrc(scales + (size_t)e * sb, ms), mk_rsrc(scales + (size_t)e * sb + ms, ms)};
  const int nb = H / 32;
  const int row0 = nt * kGU_NT + wid * 32;
  // weight fragments: j = matrix*2 + subtile (gate a, gate b, up a, up b)
  uint32_t boff[4], soff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = row0 + 16 * (j % 2) + nl;
    const bool ok = row < I;
    boff[j] = ok ? (uint32_t)row * (uint32_t)(nb * 16) + 16u * g : 0x80000000u;
    soff[j] = ok ? (uint32_t)row * (uint32_t)nb + g : 0x80000000u;
  }
  u32x4 bq[4], bq_n[4];
  uint32_t bs[4], bs_n[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    bq[j] = __builtin_amdgcn_raw_buffer_load_b128(rc[j / 2], boff[j], 0, 2);
    bs[j] = __builtin_amdgcn_raw_buffer_load_b8(rs[j / 2], soff[j], 0, 0);
  }
  __syncthreads();  // tok[] ready
  AStage st;
  stage_load(st, x, (size_t)H, tok, cnt, 0);
  stage_store(st, a_lds);
  __syncthreads();

  f32x4 acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = H / kKC;
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bq_n[j] = __builtin_amdgcn_raw_buffer_load_b128(rc[j / 2], boff[j] + (uint32_t)(c + 1) * 64u, 0, 2);
        bs_n[j] = __builtin_amdgcn_raw_buffer_load_b8(rs[j / 2], soff[j] + (uint32_t)(c + 1) * 4u, 0, 0);
      }
      stage_load(st, x, (size_t)H, tok, cnt, (c + 1) * kKC);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 bf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = decode8(bq[j][s], e8m0_operand(bs[j]));
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mtiles) {
          const bf16x8 af = as_bf16x8(*reinterpret_cast<const uint4*>(a_lds + (m * 16 + nl) * kLdsRow + 32 * g + 8 * s));
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[m][j], 0, 0, 0);
        }
      }
    }
    if (more) {
      __syncthreads();
      stage_store(st, a_lds);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 4; ++j) { bq[j] = bq_n[j]; bs[j] = bs_n[j]; }
    }
  }
  // epilogue: h = silu(g) * u for tokens 4g..4g+3 of each m-tile, row nl of each subtile
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < mtiles) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int i = row0 + 16 * sub + nl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int slot = m * 16 + 4 * g + r;
          const int p = slot < cnt ? pid[slot] : -1;
          if (p >= 0 && i < I) {
            const float h = silu_mul(acc[m][sub][r], acc[m][2 + sub][r]);
            const uint16_t hi = f32_to_bf16_rne(h);
            const uint16_t lo = f32_to_bf16_rne(h - bf16_bits_to_f32(hi));
            hterm[(size_t)p * I + i] = hi;
            hterm[(size_t)P * I + (size_t)p * I + i] = lo;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- down
// Row tile = 128 rows of Wd [H][I]; wave w owns rows 32w .. 32w+31 (two
// n-tiles).  A = the two bf16 terms of h for the block's pairs, both staged
// in LDS; each MFMA step runs once per term into the same accumulator.
// Output y[p][n] (fp32).
constexpr int kDN_NT = 128;

__global__ __launch_bounds__(256, 2) void k_down_mfma(
    const uint16_t* __restrict__ hterm, const int32_t* __restrict__ pairs, const int4* __restrict__ blocks,
    const int32_t* __restrict__ nblocks, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int H, int I, int P, int ntiles, float* __restrict__ ybuf) {
  extern __shared__ uint16_t a_lds[];  // [2 terms][kMB][kLdsRow]
  __shared__ int32_t pid[kMB];
  int eb, nt;
  decode_item(ntiles, &eb, &nt);
  if (eb >= *nblocks) return;
  const int4 blk = blocks[eb];
  const int e = blk.x, cnt = blk.z;
  for (int i = threadIdx.x; i < kMB; i += 256) pid[i] = i < cnt ? pairs[blk.y + i] : -1;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int nl = lane % 16, g = lane / 16;
  const int mtiles = (cnt + 15) / 16;
  const size_t cb = (size_t)3 * I * H / 2, sb = (size_t)3 * I * H / 32;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2), ms = (uint32_t)((size_t)I * H / 32);
  const rsrc_t rc = mk_rsrc(codes + (size_t)e * cb + 2 * (size_t)mc, mc);
  const rsrc_t rs = mk_rsrc(scales + (size_t)e * sb + 2 * (size_t)ms, ms);
  const int nbk = I / 32;
  const int row0 = nt * kDN_NT + wid * 32;
  uint32_t boff[2], soff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = row0 + 16 * j + nl;
    const bool ok = row < H;
    boff[j] = ok ? (uint32_t)row * (uint32_t)(nbk * 16) + 16u * g : 0x80000000u;
    soff[j] = ok ? (uint32_t)row * (uint32_t)nbk + g : 0x80000000u;
  }
  u32x4 bq[2], bq_n[2];
  uint32_t bs[2], bs_n[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    bq[j] = __builtin_amdgcn_raw_buffer_load_b128(rc, boff[j], 0, 2);
    bs[j] = __builtin_amdgcn_raw_buffer_load_b8(rs, soff[j], 0, 0);
  }
  __syncthreads();  // pid[] ready
  uint16_t* lds_hi = a_lds;
  uint16_t* lds_lo = a_lds + kMB * kLdsRow;
  const uint16_t* hsrc_lo = hterm + (size_t)P * I;
  AStage sh, sl;
  stage_load(sh, hterm, (size_t)I, pid, cnt, 0);
  stage_load(sl, hsrc_lo, (size_t)I, pid, cnt, 0);
  stage_store(sh, lds_hi);
  stage_store(sl, lds_lo);
  __syncthreads();

  f32x4 acc[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = I / kKC;
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    if (more) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bq_n[j] = __builtin_amdgcn_raw_buffer_load_b128(rc, boff[j] + (uint32_t)(c + 1) * 64u, 0, 2);
        bs_n[j] = __builtin_amdgcn_raw_buffer_load_b8(rs, soff[j] + (uint32_t)(c + 1) * 4u, 0, 0);
      }
      stage_load(sh, hterm, (size_t)I, pid, cnt, (c + 1) * kKC);
      stage_load(sl, hsrc_lo, (size_t)I, pid, cnt, (c + 1) * kKC);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 bf[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = decode8(bq[j][s], e8m0_operand(bs[j]));
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        if (m < mtiles) {
          const int off = (m * 16 + nl) * kLdsRow + 32 * g + 8 * s;
          const bf16x8 ah = as_bf16x8(*reinterpret_cast<const uint4*>(lds_hi + off));
          const bf16x8 al = as_bf16x8(*reinterpret_cast<const uint4*>(lds_lo + off));
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bf[j], acc[m][j], 0, 0, 0);
            acc[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bf[j], acc[m][j], 0, 0, 0);
          }
        }
      }
    }
    if (more) {
      __syncthreads();
      stage_store(sh, lds_hi);
      stage_store(sl, lds_lo);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 2; ++j) { bq[j] = bq_n[j]; bs[j] = bs_n[j]; }
    }
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < mtiles) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = row0 + 16 * j + nl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int slot = m * 16 + 4 * g + r;
          const int p = slot < cnt ? pid[slot] : -1;
          if (p >= 0 && n < H) ybuf[(size_t)p * H + n] = acc[m][j][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- launchers

int max_expert_blocks(int P, int E) { return (P + kMB - 1) / kMB + (P < E ? P : E); }

hipError_t launch_expert_blocks(const int32_t* offsets, int E, int4* blocks, int32_t* nblocks, hipStream_t s) {
  k_expert_blocks<<<1, 1024, 0, s>>>(offsets, E, blocks, nblocks);
  return hipGetLastError();
}

static unsigned items_grid(int max_blocks, int ntiles) {
  const int rounds = (max_blocks + 7) / 8;
  return (unsigned)rounds * 8u * (unsigned)ntiles;
}

hipError_t launch_gateup_mfma(const uint16_t* x, const int32_t* pairs, const int4* blocks, const int32_t* nblocks,
                              int max_blocks, const uint8_t* codes, const uint8_t* scales, int H, int I, int k,
                              int P, uint16_t* hterm, hipStream_t s) {
  const int ntiles = (I + kGU_NT - 1) / kGU_NT;
  const size_t lds = (size_t)kMB * kLdsRow * 2;
  k_gateup_mfma<<<dim3(items_grid(max_blocks, ntiles)), 256, lds, s>>>(x, pairs, blocks, nblocks, codes, scales,
                                                                        H, I, k, P, ntiles, hterm);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const uint16_t* hterm, const int32_t* pairs, const int4* blocks, const int32_t* nblocks,
                            int max_blocks, const uint8_t* codes, const uint8_t* scales, int H, int I, int P,
                            float* ybuf, hipStream_t s) {
  const int ntiles = (H + kDN_NT - 1) / kDN_NT;
  const size_t lds = (size_t)2 * kMB * kLdsRow * 2;
  k_down_mfma<<<dim3(items_grid(max_blocks, ntiles)), 256, lds, s>>>(hterm, pairs, blocks, nblocks, codes, scales,
                                                                      H, I, P, ntiles, ybuf);
  return hipGetLastError();
}

}  // namespace moe
