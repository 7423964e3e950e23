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

// Stage rows [0, kMB) x K [k0, k0+kKC) of a bf16 source through registers:
// thread t of the 512 moves 16-byte pieces q = t + 512*v (row q/16, piece
// q%16).  Rows past `cnt` (or with a negative source row) are zero.
constexpr int kThreads = 512;
struct AStage {
  uint4 v[4];
};

__device__ __forceinline__ void stage_load(AStage& a, const uint16_t* __restrict__ src, size_t row_stride,
                                           const int32_t* rows_lds, int cnt, int k0) {
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int q = threadIdx.x + kThreads * v;
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
  for (int v = 0; v < 4; ++v) {
    const int q = threadIdx.x + kThreads * v;
    const int row = q / 16, piece = q % 16;
    *reinterpret_cast<uint4*>(lds + row * kLdsRow + piece * 8) = a.v[v];
  }
}

constexpr int kTile = kMB * kLdsRow;  // bf16 elements of one LDS activation tile
constexpr int kDB = 4;                // weight chunks in flight (ring)

// One chunk of one weight row for a lane: 16 code bytes + the block's scale.
struct BChunk {
  u32x4 q;
  uint32_t s;
};

__device__ __forceinline__ BChunk load_bchunk(rsrc_t rc, rsrc_t rs, uint32_t boff, uint32_t soff, int c, bool ok) {
  BChunk b;
  b.q = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? boff + (uint32_t)c * 64u : 0x80000000u, 0, 2);
  b.s = __builtin_amdgcn_raw_buffer_load_b8(rs, ok ? soff + (uint32_t)c * 4u : 0x80000000u, 0, 0);
  return b;
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// Row tile = 128 rows of gate and the same 128 rows of up; wave w (of 8) owns
// rows 16w .. 16w+15 of the tile in both matrices.  Per K chunk: weights of
// chunk c+3 are requested, the activations of chunk c+1 move global -> regs ->
// LDS (double buffer), chunk c is multiplied, one barrier.  Output: h as two
// bf16 terms, hterm[0][p][i] = hi and hterm[1][p][i] = lo, for each pair p.
constexpr int kGU_NT = 128;

__global__ __launch_bounds__(kThreads, 1) void k_gateup_mfma(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pairs, const int4* __restrict__ blocks,
    const int32_t* __restrict__ nblocks, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int H, int I, int k, int P, int ntiles,
    uint16_t* __restrict__ hterm) {
  extern __shared__ uint16_t a_lds[];  // [2][kMB][kLdsRow]
  __shared__ int32_t tok[kMB], pid[kMB];
  int eb, nt;
  decode_item(ntiles, &eb, &nt);
  if (eb >= *nblocks) return;
  const int4 blk = blocks[eb];
  const int e = blk.x, cnt = blk.z;
  for (int i = threadIdx.x; i < kMB; i += kThreads) {
    const int p = i < cnt ? pairs[blk.y + i] : -1;
    pid[i] = p;
    tok[i] = p >= 0 ? p / k : -1;
  }
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int nl = lane % 16, g = lane / 16;
  const int mtiles = (cnt + 15) / 16;
  const size_t cb = (size_t)3 * I * H / 2, sb = (size_t)3 * I * H / 32;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2), ms = (uint32_t)((size_t)I * H / 32);
  const rsrc_t rcg = mk_rsrc(codes + (size_t)e * cb, mc), rcu = mk_rsrc(codes + (size_t)e * cb + mc, mc);
  const rsrc_t rsg = mk_rsrc(scales + (size_t)e * sb, ms), rsu = mk_rsrc(scales + (size_t)e * sb + ms, ms);
  const int nb = H / 32;
  const int row = nt * kGU_NT + wid * 16 + nl;
  const bool rok = row < I;
  const uint32_t boff = (uint32_t)row * (uint32_t)(nb * 16) + 16u * g;
  const uint32_t soff = (uint32_t)row * (uint32_t)nb + g;
  const int nchunks = H / kKC;
  BChunk rg[kDB], ru[kDB];
#pragma unroll
  for (int d = 0; d < kDB - 1; ++d) {
    rg[d] = load_bchunk(rcg, rsg, boff, soff, d, rok && d < nchunks);
    ru[d] = load_bchunk(rcu, rsu, boff, soff, d, rok && d < nchunks);
  }
  __syncthreads();  // tok[] ready
  AStage st;
  stage_load(st, x, (size_t)H, tok, cnt, 0);
  stage_store(st, a_lds);
  __syncthreads();

  f32x4 acc[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < nchunks; c0 += kDB) {
#pragma unroll
    for (int d = 0; d < kDB; ++d) {
      const int c = c0 + d;
      if (c >= nchunks) break;
      const int cn = c + kDB - 1;
      rg[(d + kDB - 1) % kDB] = load_bchunk(rcg, rsg, boff, soff, cn, rok && cn < nchunks);
      ru[(d + kDB - 1) % kDB] = load_bchunk(rcu, rsu, boff, soff, cn, rok && cn < nchunks);
      const bool more = c + 1 < nchunks;
      if (more) stage_load(st, x, (size_t)H, tok, cnt, (c + 1) * kKC);
      const uint16_t* A = a_lds + (d % 2) * kTile;
      const float sg = e8m0_operand(rg[d].s), su = e8m0_operand(ru[d].s);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 bg = decode8(rg[d].q[s], sg), bu = decode8(ru[d].q[s], su);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          if (m < mtiles) {
            const bf16x8 af = as_bf16x8(*reinterpret_cast<const uint4*>(A + (m * 16 + nl) * kLdsRow + 32 * g + 8 * s));
            acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bg, acc[m][0], 0, 0, 0);
            acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bu, acc[m][1], 0, 0, 0);
          }
        }
      }
      if (more) stage_store(st, a_lds + ((d + 1) % 2) * kTile);
      __syncthreads();
    }
  }
  // epilogue: h = silu(g) * u; lane holds row `row` for tokens 4g..4g+3 of each m-tile
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < mtiles) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = m * 16 + 4 * g + r;
        const int p = slot < cnt ? pid[slot] : -1;
        if (p >= 0 && rok) {
          const float h = silu_mul(acc[m][0][r], acc[m][1][r]);
          const uint16_t hi = f32_to_bf16_rne(h);
          const uint16_t lo = f32_to_bf16_rne(h - bf16_bits_to_f32(hi));
          hterm[(size_t)p * I + row] = hi;
          hterm[(size_t)P * I + (size_t)p * I + row] = lo;
        }
      }
    }
  }
}

// ---------------------------------------------------------------- down
// Row tile = 256 rows of Wd [H][I]; wave w (of 8) owns rows 32w .. 32w+31
// (two n-tiles).  A = the two bf16 terms of h for the block's pairs, both
// staged in LDS (double buffered); each MFMA step runs once per term into the
// same accumulator.  Output y[p][n] (fp32).
constexpr int kDN_NT = 256;

__global__ __launch_bounds__(kThreads, 1) void k_down_mfma(
    const uint16_t* __restrict__ hterm, const int32_t* __restrict__ pairs, const int4* __restrict__ blocks,
    const int32_t* __restrict__ nblocks, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int H, int I, int P, int ntiles, float* __restrict__ ybuf) {
  extern __shared__ uint16_t a_lds[];  // [2 buffers][2 terms][kMB][kLdsRow]
  __shared__ int32_t pid[kMB];
  int eb, nt;
  decode_item(ntiles, &eb, &nt);
  if (eb >= *nblocks) return;
  const int4 blk = blocks[eb];
  const int e = blk.x, cnt = blk.z;
  for (int i = threadIdx.x; i < kMB; i += kThreads) pid[i] = i < cnt ? pairs[blk.y + i] : -1;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int nl = lane % 16, g = lane / 16;
  const int mtiles = (cnt + 15) / 16;
  const size_t cb = (size_t)3 * I * H / 2, sb = (size_t)3 * I * H / 32;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2), ms = (uint32_t)((size_t)I * H / 32);
  const rsrc_t rc = mk_rsrc(codes + (size_t)e * cb + 2 * (size_t)mc, mc);
  const rsrc_t rs = mk_rsrc(scales + (size_t)e * sb + 2 * (size_t)ms, ms);
  const int nbk = I / 32;
  int rows[2];
  bool rok[2];
  uint32_t boff[2], soff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    rows[j] = nt * kDN_NT + wid * 32 + 16 * j + nl;
    rok[j] = rows[j] < H;
    boff[j] = (uint32_t)rows[j] * (uint32_t)(nbk * 16) + 16u * g;
    soff[j] = (uint32_t)rows[j] * (uint32_t)nbk + g;
  }
  const int nchunks = I / kKC;
  BChunk rb[kDB][2];
#pragma unroll
  for (int d = 0; d < kDB - 1; ++d)
#pragma unroll
    for (int j = 0; j < 2; ++j) rb[d][j] = load_bchunk(rc, rs, boff[j], soff[j], d, rok[j] && d < nchunks);
  __syncthreads();  // pid[] ready
  const uint16_t* hlo = hterm + (size_t)P * I;
  AStage sh, sl;
  stage_load(sh, hterm, (size_t)I, pid, cnt, 0);
  stage_load(sl, hlo, (size_t)I, pid, cnt, 0);
  stage_store(sh, a_lds);
  stage_store(sl, a_lds + kTile);
  __syncthreads();

  f32x4 acc[8][2];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = 0; c0 < nchunks; c0 += kDB) {
#pragma unroll
    for (int d = 0; d < kDB; ++d) {
      const int c = c0 + d;
      if (c >= nchunks) break;
      const int cn = c + kDB - 1;
#pragma unroll
      for (int j = 0; j < 2; ++j)
        rb[(d + kDB - 1) % kDB][j] = load_bchunk(rc, rs, boff[j], soff[j], cn, rok[j] && cn < nchunks);
      const bool more = c + 1 < nchunks;
      if (more) {
        stage_load(sh, hterm, (size_t)I, pid, cnt, (c + 1) * kKC);
        stage_load(sl, hlo, (size_t)I, pid, cnt, (c + 1) * kKC);
      }
      const uint16_t* Ah = a_lds + (d % 2) * 2 * kTile;
      const uint16_t* Al = Ah + kTile;
      const float s0 = e8m0_operand(rb[d][0].s), s1 = e8m0_operand(rb[d][1].s);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 b0 = decode8(rb[d][0].q[s], s0), b1 = decode8(rb[d][1].q[s], s1);
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          if (m < mtiles) {
            const int off = (m * 16 + nl) * kLdsRow + 32 * g + 8 * s;
            const bf16x8 ah = as_bf16x8(*reinterpret_cast<const uint4*>(Ah + off));
            const bf16x8 al = as_bf16x8(*reinterpret_cast<const uint4*>(Al + off));
            acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b0, acc[m][0], 0, 0, 0);
            acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b1, acc[m][1], 0, 0, 0);
            acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b0, acc[m][0], 0, 0, 0);
            acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b1, acc[m][1], 0, 0, 0);
          }
        }
      }
      if (more) {
        uint16_t* nxt = a_lds + ((d + 1) % 2) * 2 * kTile;
        stage_store(sh, nxt);
        stage_store(sl, nxt + kTile);
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < mtiles) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int slot = m * 16 + 4 * g + r;
          const int p = slot < cnt ? pid[slot] : -1;
          if (p >= 0 && rok[j]) ybuf[(size_t)p * H + rows[j]] = acc[m][j][r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- router logits (many tokens)
// logits[t][e] = x[t] . Wr[e] (+ b[e]) for bf16 activations, on MFMA: each
// fp32 router weight w is split into three bf16 terms w = w0 + w1 + w2
// (w0 = bf16(w), w1 = bf16(w - w0), w2 = w - w0 - w1; exact for every normal
// fp32 whose low terms stay above the bf16 subnormal range), so every
// product is exact and the sum is fp32.  Tile: 128 tokens x 128 experts;
// wave w (of 8) owns experts 16w .. 16w+15, all token m-tiles.
constexpr int kRT_NT = 128;

// Split two fp32 weights into three packed bf16 pairs (term 0, 1, 2).
__device__ __forceinline__ void split3_pair(uint32_t a, uint32_t b, uint32_t& p0, uint32_t& p1, uint32_t& p2) {
  const float wa = __uint_as_float(a), wb = __uint_as_float(b);
  const uint32_t a0 = f32_to_bf16_rne(wa), b0 = f32_to_bf16_rne(wb);
  const float ra = wa - __uint_as_float(a0 << 16), rb = wb - __uint_as_float(b0 << 16);
  const uint32_t a1 = f32_to_bf16_rne(ra), b1 = f32_to_bf16_rne(rb);
  const uint32_t a2 = f32_to_bf16_rne(ra - __uint_as_float(a1 << 16));
  const uint32_t b2 = f32_to_bf16_rne(rb - __uint_as_float(b1 << 16));
  p0 = a0 | (b0 << 16);
  p1 = a1 | (b1 << 16);
  p2 = a2 | (b2 << 16);
}

__device__ __forceinline__ void split3(const u32x4& q0, const u32x4& q1, bf16x8& t0, bf16x8& t1, bf16x8& t2) {
  uint32_t u0[4], u1[4], u2[4];
  split3_pair(q0.x, q0.y, u0[0], u1[0], u2[0]);
  split3_pair(q0.z, q0.w, u0[1], u1[1], u2[1]);
  split3_pair(q1.x, q1.y, u0[2], u1[2], u2[2]);
  split3_pair(q1.z, q1.w, u0[3], u1[3], u2[3]);
  __builtin_memcpy(&t0, &u0, 16);
  __builtin_memcpy(&t1, &u1, 16);
  __builtin_memcpy(&t2, &u2, 16);
}

__global__ __launch_bounds__(kThreads, 1) void k_router_mfma(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ wr,
                                                             const float* __restrict__ bias, int T, int H, int E,
                                                             int ntiles, float* __restrict__ logits) {
  extern __shared__ uint16_t a_lds[];  // [2][kMB][kLdsRow]
  __shared__ int32_t tok[kMB];
  const int mt = blockIdx.x / ntiles, nt = blockIdx.x % ntiles;
  const int t0 = mt * kMB;
  const int cnt = min(kMB, T - t0);
  for (int i = threadIdx.x; i < kMB; i += kThreads) tok[i] = i < cnt ? t0 + i : -1;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int nl = lane % 16, g = lane / 16;
  const int mtiles = (cnt + 15) / 16;
  const int ex = nt * kRT_NT + wid * 16 + nl;
  const bool eok = ex < E;
  const rsrc_t rw = mk_rsrc(wr, (uint32_t)((size_t)E * H * 4));
  const uint32_t woff = (uint32_t)ex * (uint32_t)(H * 4) + 128u * g;  // 32 floats of the lane's K slice
  const int nchunks = H / kKC;
  __syncthreads();
  AStage st;
  stage_load(st, x, (size_t)H, tok, cnt, 0);
  stage_store(st, a_lds);
  u32x4 wq[8];
#pragma unroll
  for (int v = 0; v < 8; ++v)
    wq[v] = __builtin_amdgcn_raw_buffer_load_b128(rw, eok ? woff + 16u * v : 0x80000000u, 0, 0);
  __syncthreads();
  f32x4 acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < nchunks; ++c) {
    const bool more = c + 1 < nchunks;
    bf16x8 bt[4][3];
#pragma unroll
    for (int s = 0; s < 4; ++s) split3(wq[2 * s], wq[2 * s + 1], bt[s][0], bt[s][1], bt[s][2]);
    if (more) {
#pragma unroll
      for (int v = 0; v < 8; ++v)
        wq[v] = __builtin_amdgcn_raw_buffer_load_b128(rw, eok ? woff + (uint32_t)(c + 1) * 512u + 16u * v : 0x80000000u,
                                                       0, 0);
      stage_load(st, x, (size_t)H, tok, cnt, (c + 1) * kKC);
    }
    const uint16_t* A = a_lds + (c % 2) * kTile;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (m < mtiles) {
          const bf16x8 af = as_bf16x8(*reinterpret_cast<const uint4*>(A + (m * 16 + nl) * kLdsRow + 32 * g + 8 * s));
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bt[s][0], acc[m], 0, 0, 0);
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bt[s][1], acc[m], 0, 0, 0);
          acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bt[s][2], acc[m], 0, 0, 0);
        }
      }
    }
    if (more) stage_store(st, a_lds + ((c + 1) % 2) * kTile);
    __syncthreads();
  }
  const float b = (bias && eok) ? bias[ex] : 0.0f;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m < mtiles) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = m * 16 + 4 * g + r;
        if (slot < cnt && eok) logits[(size_t)(t0 + slot) * E + ex] = acc[m][r] + b;
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
  const size_t lds = (size_t)2 * kTile * 2;
  k_gateup_mfma<<<dim3(items_grid(max_blocks, ntiles)), kThreads, lds, s>>>(x, pairs, blocks, nblocks, codes,
                                                                             scales, H, I, k, P, ntiles, hterm);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const uint16_t* hterm, const int32_t* pairs, const int4* blocks, const int32_t* nblocks,
                            int max_blocks, const uint8_t* codes, const uint8_t* scales, int H, int I, int P,
                            float* ybuf, hipStream_t s) {
  const int ntiles = (H + kDN_NT - 1) / kDN_NT;
  const size_t lds = (size_t)4 * kTile * 2;
  k_down_mfma<<<dim3(items_grid(max_blocks, ntiles)), kThreads, lds, s>>>(hterm, pairs, blocks, nblocks, codes,
                                                                           scales, H, I, P, ntiles, ybuf);
  return hipGetLastError();
}

hipError_t launch_router_mfma(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                              float* logits, hipStream_t s) {
  const int ntiles = (E + kRT_NT - 1) / kRT_NT;
  const int mtiles = (T + kMB - 1) / kMB;
  const size_t lds = (size_t)2 * kTile * 2;
  k_router_mfma<<<dim3((unsigned)(mtiles * ntiles)), kThreads, lds, s>>>(x, wr, bias, T, H, E, ntiles, logits);
  return hipGetLastError();
}

}  // namespace moe
