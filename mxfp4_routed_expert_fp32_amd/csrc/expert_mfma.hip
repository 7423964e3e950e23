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
#include <algorithm>
#include <cstdint>

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kMB = kExpertBlockPairs;  // pairs per expert block (8 m-tiles of 16)
constexpr int kKC = 128;       // K per chunk (4 blocks of 32)
constexpr int kLdsRow = kKC + 8;  // bf16 per LDS row (16-byte pad against bank conflicts)

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t mk_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// ---------------------------------------------------------------- expert blocks
// blocks[b] = {expert, first index into the sorted pair list, pair count, 0};
// *nblocks = number of blocks (at most max_blocks are written).  One
// workgroup.
__global__ __launch_bounds__(1024) void k_expert_blocks(const int32_t* __restrict__ offsets, int E, int max_blocks,
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
    for (int32_t m0 = 0; m0 < cnt; m0 += kMB, ++b)
      if (b < max_blocks) blocks[b] = make_int4(e, beg + m0, min(kMB, cnt - m0), 0);
  }
  if (tid == 1023) *nblocks = min(part[1023], max_blocks);
}

// Workgroup -> (expert block, row tile): row tiles of one block on one XCD.
__device__ __forceinline__ void decode_item(int ntiles, int* eb, int* nt) {
  const int xcd = blockIdx.x % 8, r = blockIdx.x / 8;
  *eb = (r / ntiles) * 8 + xcd;
  *nt = r % ntiles;
}

constexpr int kTile = kMB * kLdsRow;  // bf16 elements of one LDS activation tile

// ---------------------------------------------------------------- grouped GEMM pipeline
// Both expert kernels run 8 waves (two per SIMD, so one covers the other's
// waits) over one expert block (<= 128 pairs, MT m-tiles of 16) times one
// tile of output rows; every wave owns two 16-row n-tiles and all MT m-tiles,
// so no weight byte is requested twice.  K runs in 128-wide chunks for the
// activations and in 256-wide superchunks (two chunks) for the weights.
// Per chunk c:
//   1. the activation rows of chunk c+DA are requested into a register ring
//      of DA chunks; at the first chunk of a superchunk the weights of the
//      superchunk DB-1 ahead are requested too (register ring of DB
//      superchunks).  Loads complete for the wait counter in issue order, so
//      a wait for an activation load also waits for every weight load issued
//      before it: the activation ring must reach about as far ahead as the
//      weight ring, or the weight ring's depth is lost;
//   2. chunk c is multiplied: weights decoded to bf16 (exact), activation
//      fragments read from LDS buffer c % 2;
//   3. the activation rows of chunk c+1 are written to LDS buffer (c+1) % 2
//      (last read in chunk c-1, before the previous barrier);
//   4. one barrier.
// Weights: lane group g = l/16 holds code blocks g and g+4 of its row's
// superchunk (16 bytes each, one per chunk), so the 4 groups request both
// halves of a 128-byte line of each of 16 rows back to back; the
// superchunk's 8 scale bytes per row come from the workgroup's LDS scale
// table.  In MFMA step s of chunk c, group g supplies K = 32g + 8s .. +8 of
// the chunk on both operands.
// Every load is an unconditional raw buffer load; rows past the block and
// chunks past K use an out-of-range offset and read 0, so the loop has no
// data-dependent branch and the compiler can count loads in flight exactly.
constexpr int kThr = 512;           // threads per workgroup (8 waves)
constexpr uint32_t kOOB = 0x80000000u;

// Rows of a chunk staged per thread: pieces q = t + 512 v (v < NV), row q/16,
// piece q%16 (16 bytes).  aoff[v] = byte offset of that piece at K origin
// (row base + 16 * piece), or kFar for a row past the block; `kbyte` = byte
// offset of the chunk in the row, or kFar for a chunk past K.  Activation
// buffers are smaller than kFar bytes, so any sum involving kFar is out of
// range (reads 0) and no sum wraps.
constexpr uint32_t kFar = 0x40000000u;

template <int NV>
struct ARegs {
  u32x4 v[NV];
};

template <int NV>
__device__ __forceinline__ void a_offsets(uint32_t* aoff, const uint32_t* row_base) {
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int q = threadIdx.x + kThr * v;
    aoff[v] = row_base[q >> 4] + (uint32_t)(q & 15) * 16u;
  }
}

template <int NV>
__device__ __forceinline__ void a_fetch(ARegs<NV>& a, rsrc_t r, const uint32_t* aoff, uint32_t kbyte) {
#pragma unroll
  for (int v = 0; v < NV; ++v) a.v[v] = __builtin_amdgcn_raw_buffer_load_b128(r, aoff[v] + kbyte, 0, 0);
}

template <int NV>
__device__ __forceinline__ void a_put(const ARegs<NV>& a, uint16_t* buf) {
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int q = threadIdx.x + kThr * v;
    *reinterpret_cast<u32x4*>(buf + (q >> 4) * kLdsRow + (q & 15) * 8) = a.v[v];
  }
}

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* buf, int row, int col) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(buf + row * kLdsRow + col));
}

// Weights of one 16-row n-tile for one superchunk, for this lane.
struct BSuper {
  u32x4 q[2];     // code blocks g (chunk 0) and g+4 (chunk 1)
  uint32_t s[2];  // the superchunk's 8 scale bytes
};

// Codes: boff = row * row_bytes + 16 g (or kOOB for a row past the matrix).
// Half hf of superchunk sc: code block g + 4 hf.
__device__ __forceinline__ void load_bcode_half(BSuper& b, rsrc_t rc, uint32_t boff, int sc, int nsc, int hf) {
  const bool ok = sc < nsc;
  b.q[hf] = __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? boff + (uint32_t)sc * 128u + 64u * (uint32_t)hf : kOOB, 0, 0);
}
__device__ __forceinline__ void load_bcodes(BSuper& b, rsrc_t rc, uint32_t boff, int sc, int nsc) {
  load_bcode_half(b, rc, boff, sc, nsc, 0);
  load_bcode_half(b, rc, boff, sc, nsc, 1);
}

// Scales from this row's line of the LDS scale table; a superchunk past K
// gets scale byte 0 (its codes read 0, and 0 times 2^-127 adds nothing).
__device__ __forceinline__ void load_bscales(BSuper& b, const uint8_t* srow, int sc, int nsc) {
  const bool ok = sc < nsc;
  const u32x2 v = *reinterpret_cast<const u32x2*>(srow + (ok ? sc : 0) * 8);
  b.s[0] = ok ? v[0] : 0u;
  b.s[1] = ok ? v[1] : 0u;
}

// ---------------------------------------------------------------- scale tables
// A workgroup's weight rows are consecutive rows of one matrix, so their E8M0
// scales (nb = K/32 bytes per row) form one contiguous range.  Reading each
// superchunk's 8 scale bytes per row straight from memory touches a new
// 64-byte sector for 8 bytes every time, and those sectors do not survive in
// L2 between touches while the code stream passes through it (measured: HBM
// reads grew by about eight times the scale bytes, and the stream rate fell
// by more than half).  Instead the range is copied once per workgroup into an
// LDS table with whole-line 16-byte loads, rows padded to nb + 8 bytes (an
// 8-byte read per lane over 16 consecutive rows then hits distinct banks for
// the model's nb), and every superchunk reads its 8 bytes from there.
template <int U>
struct SPieces {
  u32x4 v[U];
};

__host__ __device__ constexpr int scale_row_pitch(int nb) { return nb + 8; }

// Requests bytes [first, first + total) of rs as 16-byte pieces q = t + kThr*u.
template <int U>
__device__ __forceinline__ void scales_fetch(SPieces<U>& sp, rsrc_t rs, uint32_t first, uint32_t total) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t flat = (uint32_t)(threadIdx.x + kThr * u) * 16u;
    sp.v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, flat < total ? first + flat : kOOB, 0, 0);
  }
}

// Writes the pieces into rows of nb bytes at pitch scale_row_pitch(nb); a
// piece may straddle two rows (nb % 16 == 8), so each 8-byte half is placed
// on its own.
template <int U>
__device__ __forceinline__ void scales_put(const SPieces<U>& sp, uint8_t* tab, int nb, uint32_t total) {
  const int pitch = scale_row_pitch(nb);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t flat = (uint32_t)(threadIdx.x + kThr * u) * 16u;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t f = flat + 8u * half;
      if (f < total) {
        const uint32_t r = f / (uint32_t)nb, c = f % (uint32_t)nb;
        *reinterpret_cast<u32x2*>(tab + r * pitch + c) =
            half ? u32x2{sp.v[u][2], sp.v[u][3]} : u32x2{sp.v[u][0], sp.v[u][1]};
      }
    }
  }
}

// Per-MT shape: MS m-tiles staged (even; rows past the block read 0), NV
// 16-byte pieces per thread per chunk and activation term.
template <int MT>
struct Shape {
  static constexpr int MS = (MT + 1) / 2 * 2;
  static constexpr int NV = MS * 16 * 16 / kThr;
};

// ---------------------------------------------------------------- activation tiles by DMA
// An activation chunk (rows x 128 bf16, 256 bytes per row) goes from memory
// straight into LDS: buffer_load ... lds writes lane i's 16 bytes at the
// wave's LDS base + 16 i, so no registers or LDS store instructions are
// involved.  LDS rows are 256 bytes with the 16-byte pieces swizzled by row:
// piece p of row r sits in slot p ^ swz_key(r % 16).  A fragment read (16
// rows at one K offset, four such groups) then has no bank conflicts on
// gfx950; measured with the conflict counter, keys p ^ r, rotations and
// padded rows all cost 4 extra cycles per ds_read_b128, this one none.
// Wave w moves blocks b = w + 8 i (i < MS/2) of 4 rows; lane j loads row
// 4b + j/16, the piece that belongs in slot j % 16.  Rows past the block
// read out of range and land as zeros.
typedef __attribute__((address_space(3))) void lds_void_t;
constexpr int kDmaRow = kKC * 2;  // bytes per LDS activation row

__device__ __forceinline__ int swz_key(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

template <int MS>
__device__ __forceinline__ void dma_offsets(uint32_t* doff, const uint32_t* row_base) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < MS / 2; ++i) {
    const int row = 4 * (wid + 8 * i) + lane / 16;
    doff[i] = row_base[row] + (uint32_t)(((lane & 15) ^ swz_key(row & 15)) * 16);
  }
}

// Requests chunk bytes [kbyte, kbyte + 256) of every staged row into `buf`.
template <int MS>
__device__ __forceinline__ void dma_chunk(rsrc_t r, const uint32_t* doff, uint32_t kbyte, uint8_t* buf) {
  const int wid = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < MS / 2; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(buf + (wid + 8 * i) * (4 * kDmaRow)), 16,
                                             doff[i] + kbyte, 0, 0, 0);
}

// Fragment of row m*16 + nl (this lane's), K piece p (0..15) of a swizzled tile.
__device__ __forceinline__ bf16x8 lds_frag_sw(const uint8_t* buf, int m, int nl, int p) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(buf + (m * 16 + nl) * kDmaRow + ((p ^ swz_key(nl)) << 4)));
}

// Waits until at most N vector memory operations of this wave are in flight
// (and, with LDS_DRAIN, for its LDS operations), then joins the workgroup
// barrier.  The barrier carries no memory fence (a fence would wait for every
// load in flight); the empty asm keeps the compiler from moving memory
// accesses across it.  The barriers inside the chunk loops skip the LDS
// drain: the buffer the next DMA overwrites was last read in an earlier
// chunk, and those reads were consumed (hence complete) before this barrier,
// while fragment reads of later chunks may stay in flight across it.  The
// prologue barriers drain, since LDS writes (the scale table) precede them.
template <int N, bool LDS_DRAIN = true>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | ((LDS_DRAIN ? 0x0 : 0xF) << 8));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------- gate/up + SwiGLU
// Row tile = 128 rows of gate and the same 128 rows of up; wave w: n-tile 0
// = gate rows 16w + 0..15, n-tile 1 = the same up rows.  Output: h as two
// bf16 terms, hterm[0][p][i] = hi and hterm[1][p][i] = lo.
constexpr int kGU_NT = 128;
// Weight ring: 4 superchunks (K = 7168 gives 28, whole rounds).
constexpr int kGuDB = 4;
constexpr int kGuPF = 4;  // activation fragments requested ahead of use (2 MFMAs each)
// Scale-table pieces per thread and matrix: 128 rows x nb bytes in 16-byte
// pieces over 512 threads covers nb <= 64 * kGuScaleU, i.e. K <= 12288.
constexpr int kGuScaleU = 6;

// Activation buffers (DMA ring of NB buffers of MS*16 rows, chunks requested
// NB - 1 ahead; a wait for a chunk's DMA also waits for every older weight
// load, so the ring should reach about as far ahead as the weight ring
// allows): 5 up to 2 m-tiles, 4 up to 4; above, 4 (up to 6 m-tiles) or 3
// when they fit LDS beside the scale table (K up to 7424), else 3 or 2.  The
// scale table follows the buffers.
constexpr int gu_nbuf_small(int mt) { return mt <= 2 ? 5 : (mt <= 4 ? 4 : (mt <= 6 ? 3 : 2)); }
constexpr int kGuActSmall = 3 * 96 * kDmaRow;  // holds every small-LDS ring (5x32, 4x64, 3x96, 2x128 rows)
constexpr int kGuActLarge = 3 * 128 * kDmaRow;

// Vector memory operations a wave issues after the DMA of chunk c + 1 (issued
// in chunk c + 1 - da, first thing, da = chunks requested ahead) until its
// wait in chunk c (after the chunk's own loads): the DMAs of the da - 1
// chunks after it (dmaops each) and the weight loads (codeops) of every even
// chunk among the da chunks from c + 1 - da to c.
constexpr int dma_wait_ops(int da, int dmaops, int codeops, int h) {
  const int p0 = ((h + 1 - da) % 2 + 2) % 2;  // parity of chunk c + 1 - da
  const int evens = p0 == 0 ? (da + 1) / 2 : da / 2;
  return (da - 1) * dmaops + codeops * evens;
}

// Replays the issue order of the prologue and the loop (nchunks chunks, weight
// ring db) and checks that every wait count equals the operations issued after
// the DMA it waits for: fewer would wait longer than needed, more would let a
// chunk be read before it is in LDS.  (Stores issued between, at the down
// kernel's tile ends, only lengthen a wait.)
constexpr bool dma_waits_exact(int da, int dmaops, int codeops, int db, int nchunks) {
  int last[256] = {};  // op count when the DMA of a chunk was issued
  int n = 0;
  const int v0 = 2 * (db - 1) > da ? 2 * (db - 1) : da;
  for (int v = -v0; v < 0; ++v) {
    if (v + da >= 0) { n += dmaops; last[v + da] = n; }
    if (v % 2 == 0 && v / 2 + db - 1 >= 0) n += codeops;
  }
  if (n - last[0] != dma_wait_ops(da, dmaops, codeops, 1)) return false;
  for (int sc0 = 0; sc0 < nchunks / 2; sc0 += db)
    for (int d = 0; d < db; ++d)
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * sc0 + 2 * d + h;
        n += dmaops;
        last[c + da] = n;
        if (h == 0) n += codeops;
        if (n - last[c + 1] != dma_wait_ops(da, dmaops, codeops, h)) return false;
      }
  return true;
}
// gate/up: MS/2 DMA instructions and 4 code loads per chunk; (da, MS) as used
static_assert(dma_waits_exact(3, 1, 4, 4, 56) && dma_waits_exact(2, 2, 4, 4, 56) && dma_waits_exact(2, 3, 4, 4, 56) &&
                  dma_waits_exact(1, 3, 4, 4, 56) && dma_waits_exact(1, 4, 4, 4, 56) && dma_waits_exact(3, 1, 4, 4, 2) &&
                  dma_waits_exact(1, 4, 4, 4, 2) && dma_waits_exact(2, 3, 4, 4, 64) && dma_waits_exact(2, 2, 4, 4, 18) &&
                  // three-term activations (fp32 x): K' = 3 H
                  dma_waits_exact(3, 1, 4, 4, 168) && dma_waits_exact(2, 3, 4, 4, 168) &&
                  dma_waits_exact(1, 4, 4, 4, 168) && dma_waits_exact(3, 1, 4, 4, 6),
              "gate/up DMA wait counts");

template <int MT, int DB, int NB, bool MID>
__device__ __forceinline__ void gateup_block(int e, int nt, int H, int I, int P, int xt, rsrc_t rx,
                                             const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                             const int32_t* pid, const uint32_t* row_base, uint8_t* lds,
                                             int act_bytes, uint16_t* __restrict__ hterm) {
  using S = Shape<MT>;
  constexpr int MS = S::MS;
  // chunks requested ahead: NB - 2 when the barrier sits mid-chunk (a buffer
  // is then still read after the barrier that follows its use), else NB - 1
  constexpr int DA = MID ? NB - 2 : NB - 1;
  static_assert(NB >= 2 && NB <= 5 && DA >= 1, "activation buffers");
  constexpr uint32_t kBuf = (uint32_t)MS * 16 * kDmaRow;
  static_assert(NB * MS * 16 * kDmaRow <= kGuActLarge, "ring fits the activation region");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const size_t cb = (size_t)3 * I * H / 2, sb = (size_t)3 * I * H / 32;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2), ms = (uint32_t)((size_t)I * H / 32);
  const rsrc_t rcg = mk_rsrc(codes + (size_t)e * cb, mc), rcu = mk_rsrc(codes + (size_t)e * cb + mc, mc);
  const rsrc_t rsg = mk_rsrc(scales + (size_t)e * sb, ms), rsu = mk_rsrc(scales + (size_t)e * sb + ms, ms);
  const int nb = H / 32;
  const int row = nt * kGU_NT + wid * 16 + nl;
  const bool rok = row < I;
  const uint32_t boff = rok ? (uint32_t)row * (uint32_t)(nb * 16) + 16u * g : kOOB;
  // K' = xt H: the activation row holds xt terms of x back to back (xt = 3:
  // an fp32 x as three bf16 terms), and superchunk sn of K' multiplies weight
  // superchunk sn mod (H / 256); past K' a superchunk reads nothing
  const int nsc_w = H / (2 * kKC);
  const int nchunks = xt * (H / kKC), nsc = nchunks / 2;
  auto wsc = [&](int sn) { return sn < nsc ? sn % nsc_w : nsc_w; };
  // scale table: gate rows, then up rows, of this row tile
  uint8_t* tab = lds + act_bytes;
  const int pitch = scale_row_pitch(nb);
  const uint8_t* tg = tab + (wid * 16 + nl) * pitch;
  const uint8_t* tu = tg + kGU_NT * pitch;
  const uint32_t tfirst = (uint32_t)(nt * kGU_NT) * (uint32_t)nb, ttotal = (uint32_t)kGU_NT * (uint32_t)nb;
  SPieces<kGuScaleU> spg, spu;
  scales_fetch<kGuScaleU>(spg, rsg, tfirst, ttotal);
  scales_fetch<kGuScaleU>(spu, rsu, tfirst, ttotal);

  uint32_t doff[MS / 2];
  dma_offsets<MS>(doff, row_base);
  auto kb_of = [&](int c) -> uint32_t { return c < nchunks ? (uint32_t)c * kDmaRow : kFar; };
  // The prologue issues what the loop would have issued in the chunks before
  // chunk 0, in the loop's order (chunk v: DMA of chunk v + DA, then in even
  // chunks the weight codes of superchunk v/2 + DB - 1), so the loop's wait
  // counts hold from its first chunk on.
  BSuper rg[DB], ru[DB];
  constexpr int V = 2 * (DB - 1) > DA ? 2 * (DB - 1) : DA;
#pragma unroll
  for (int v = -V; v < 0; ++v) {
    if (v + DA >= 0) dma_chunk<MS>(rx, doff, kb_of(v + DA), lds + (v + DA) * kBuf);
    if (v % 2 == 0 && v / 2 + DB - 1 >= 0) {
      const int sn = v / 2 + DB - 1;
      load_bcodes(rg[sn], rcg, boff, wsc(sn), nsc_w);
      load_bcodes(ru[sn], rcu, boff, wsc(sn), nsc_w);
    }
  }
  scales_put<kGuScaleU>(spg, tab, nb, ttotal);
  scales_put<kGuScaleU>(spu, tab + kGU_NT * pitch, nb, ttotal);
  wait_vm_barrier<dma_wait_ops(DA, MS / 2, 4, 1)>();  // chunk 0 (and the scale table) in LDS, as at the end of chunk -1
#pragma unroll
  for (int d = 0; d < DB - 1; ++d) {
    load_bscales(rg[d], tg, wsc(d), nsc_w);
    load_bscales(ru[d], tu, wsc(d), nsc_w);
  }

  f32x4 acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Activation fragments: pair i = s*MT + m (step s, m-tile m) of a chunk;
  // the fragment of pair i + kGuPF is requested before the multiplies of pair
  // i (scheduling barriers keep that order), so LDS latency hides behind
  // 2 kGuPF MFMAs.  With MID the barrier for chunk c + 1 sits kGuPF pairs
  // before the end of chunk c and the requests run on into chunk c + 1, so no
  // chunk starts by waiting for its first fragment.  The ring of RF
  // fragments divides the pairs of one unrolled round.
  constexpr int NQ = 4 * MT, RF = 8;
  static_assert(kGuPF < RF && kGuPF <= NQ && (2 * DB * NQ) % RF == 0, "fragment ring");
  // An even chunk's four weight loads (gate and up halves of one superchunk)
  // go between its multiplies at pairs WP0 + k WS, all before the chunk's
  // wait, so the address unit takes them one at a time instead of in one
  // burst with every other wave's; chunks with few pairs issue them up front.
  // Either way they follow the chunk's DMA, as the wait counts assume.
  constexpr int WLAST = MID ? NQ - kGuPF : NQ;
  constexpr bool kSpread = WLAST >= 5;
  constexpr int WP0 = 1, WS = kSpread ? (WLAST - 2) / 4 : 0;
  static_assert(!kSpread || WP0 + 3 * WS < WLAST, "weight loads before the chunk's wait");
  bf16x8 fa[RF];
  if (MID) {
#pragma unroll
    for (int i = 0; i < kGuPF; ++i) fa[i % RF] = lds_frag_sw(lds, i % MT, nl, 4 * g + i / MT);
  }

  // the ring holds whole superchunks; a phantom superchunk past K reads zeros
  // on both operands and adds nothing
  int slot = 0;  // LDS buffer of the current chunk, c % NB
  for (int sc0 = 0; sc0 < nsc; sc0 += DB) {
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 2 * sc0 + 2 * d + h;  // chunk; c % 2 == h
        {
          // chunk c + DA into the buffer chunk c - 1 used (every wave passed the last barrier after reading it)
          int nslot = slot + DA;
          nslot -= nslot >= NB ? NB : 0;
          dma_chunk<MS>(rx, doff, kb_of(c + DA), lds + nslot * kBuf);
        }
        const int sn = sc0 + d + DB - 1;  // the superchunk an even chunk requests
        const int sw = wsc(sn);           // its weight superchunk
        if (h == 0) {
          if constexpr (!kSpread) {
            load_bcodes(rg[(d + DB - 1) % DB], rcg, boff, sw, nsc_w);
            load_bcodes(ru[(d + DB - 1) % DB], rcu, boff, sw, nsc_w);
          }
          load_bscales(rg[(d + DB - 1) % DB], tg, sw, nsc_w);
          load_bscales(ru[(d + DB - 1) % DB], tu, sw, nsc_w);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the multiply
        const uint8_t* A = lds + slot * kBuf;
        const uint8_t* An = lds + (slot + 1 == NB ? 0 : slot + 1) * kBuf;  // next chunk's buffer
        const float sgv = e8m0_operand((rg[d].s[h] >> (8 * g)) & 0xFFu);
        const float suv = e8m0_operand((ru[d].s[h] >> (8 * g)) & 0xFFu);
        const int q0 = (2 * d + h) * NQ;  // ring position of this chunk's first pair
        if (!MID) {
#pragma unroll
          for (int i = 0; i < kGuPF; ++i) fa[(q0 + i) % RF] = lds_frag_sw(A, i % MT, nl, 4 * g + i / MT);
        }
        bf16x8 bg = decode8(rg[d].q[h][0], sgv), bu = decode8(ru[d].q[h][0], suv);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int st = i / MT, m = i % MT;
          const int j = i + kGuPF;
          if (MID && j == NQ) {
            // chunk c + 1 must be in LDS for every wave before its first read
            if (h == 0) wait_vm_barrier<dma_wait_ops(DA, MS / 2, 4, 0), false>();
            else wait_vm_barrier<dma_wait_ops(DA, MS / 2, 4, 1), false>();
          }
          if (j < NQ) fa[(q0 + j) % RF] = lds_frag_sw(A, j % MT, nl, 4 * g + j / MT);
          else if (MID) fa[(q0 + j) % RF] = lds_frag_sw(An, (j - NQ) % MT, nl, 4 * g + (j - NQ) / MT);
          if (kSpread && h == 0) {
            if (i == WP0) load_bcode_half(rg[(d + DB - 1) % DB], rcg, boff, sw, nsc_w, 0);
            if (i == WP0 + WS) load_bcode_half(rg[(d + DB - 1) % DB], rcg, boff, sw, nsc_w, 1);
            if (i == WP0 + 2 * WS) load_bcode_half(ru[(d + DB - 1) % DB], rcu, boff, sw, nsc_w, 0);
            if (i == WP0 + 3 * WS) load_bcode_half(ru[(d + DB - 1) % DB], rcu, boff, sw, nsc_w, 1);
          }
          if (m == 0 && st > 0) {
            bg = decode8(rg[d].q[h][st], sgv);
            bu = decode8(ru[d].q[h][st], suv);
          }
          __builtin_amdgcn_sched_barrier(0);
          acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[(q0 + i) % RF], bg, acc[m][0], 0, 0, 0);
          acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[(q0 + i) % RF], bu, acc[m][1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (!MID) {
          // chunk c + 1 must be in LDS for every wave before anyone reads it
          if (h == 0) wait_vm_barrier<dma_wait_ops(DA, MS / 2, 4, 0), false>();
          else wait_vm_barrier<dma_wait_ops(DA, MS / 2, 4, 1), false>();
        }
        slot = slot + 1 == NB ? 0 : slot + 1;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no LDS transfer outlives the loop
  // lane holds row `row` for slots m*16 + 4g + r
#pragma unroll
  for (int m = 0; m < MT; ++m) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = pid[m * 16 + 4 * g + r];
      if (p >= 0 && rok) {
        const float hv = silu_mul(acc[m][0][r], acc[m][1][r]);
        const uint16_t hi = f32_to_bf16_rne(hv);
        const uint16_t lo = f32_to_bf16_rne(hv - bf16_bits_to_f32(hi));
        hterm[(size_t)p * I + row] = hi;
        hterm[(size_t)P * I + (size_t)p * I + row] = lo;
      }
    }
  }
}

__global__ __launch_bounds__(kThr, 1) void k_gateup_mfma(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ pairs, const int4* __restrict__ blocks,
    const int32_t* __restrict__ nblocks, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int T, int H, int I, int E, int k, int P, int max_blocks, int ntiles,
    int large, int xt, uint16_t* __restrict__ hterm) {
  extern __shared__ uint4 lds_dyn[];  // activation buffers, then the scale table
  uint8_t* lds8 = reinterpret_cast<uint8_t*>(lds_dyn);
  const int act = large ? kGuActLarge : kGuActSmall;
  __shared__ int32_t pid[kMB];
  __shared__ uint32_t row_base[kMB];
  int eb, nt;
  decode_item(ntiles, &eb, &nt);
  if (eb >= min(*nblocks, max_blocks)) return;
  const int4 blk = blocks[eb];
  const int e = blk.x, cnt = blk.z;
  if (e < 0 || e >= E || cnt < 1 || cnt > kMB || blk.y < 0 || blk.y > P - cnt) return;  // malformed block
  for (int i = threadIdx.x; i < kMB; i += kThr) {
    int p = i < cnt ? pairs[blk.y + i] : -1;
    if (p >= P) p = -1;
    pid[i] = p;
    row_base[i] = p >= 0 ? (uint32_t)(p / k) * (uint32_t)(xt * H * 2) : kFar;
  }
  __syncthreads();
  const rsrc_t rx = mk_rsrc(x, (uint32_t)((size_t)T * xt * H * 2));
  switch ((cnt + 15) / 16) {
    case 1: gateup_block<1, kGuDB, gu_nbuf_small(1), (gu_nbuf_small(1) >= 3)>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm); break;
    case 2: gateup_block<2, kGuDB, gu_nbuf_small(2), (gu_nbuf_small(2) >= 3)>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm); break;
    case 3: gateup_block<3, kGuDB, gu_nbuf_small(3), (gu_nbuf_small(3) >= 3)>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm); break;
    case 4: gateup_block<4, kGuDB, gu_nbuf_small(4), (gu_nbuf_small(4) >= 3)>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm); break;
    case 5: (large ? gateup_block<5, kGuDB, 4, true>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm)
                   : gateup_block<5, kGuDB, 3, true>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm)); break;
    case 6: (large ? gateup_block<6, kGuDB, 4, true>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm)
                   : gateup_block<6, kGuDB, 3, true>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm)); break;
    case 7: (large ? gateup_block<7, kGuDB, 3, true>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm)
                   : gateup_block<7, kGuDB, 2, false>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm)); break;
    default: (large ? gateup_block<8, kGuDB, 3, true>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm)
                   : gateup_block<8, kGuDB, 2, false>(e, nt, H, I, P, xt, rx, codes, scales, pid, row_base, lds8, act, hterm)); break;
  }
}

// ---------------------------------------------------------------- down
// Row tile = 256 rows of Wd [H][I]; wave w: n-tiles = rows 32w + 0..15 and
// 32w + 16..31.  The activations are the two bf16 terms of h for the block's
// pairs, both staged in LDS; each MFMA step runs once per term into the same
// accumulator.  Output y[p][n] (fp32).
// K = I is short (1536: 12 chunks), so a workgroup runs kDnTiles row tiles
// of its expert block back to back: the weight and activation rings run on
// across tile boundaries (the next tile's first weights are in flight while
// this tile finishes), and only the first tile waits for a cold pipeline.
// Scales: for blocks of up to 4 m-tiles, where it fits beside the activation
// ring (I/32 + 8 <= 60 bytes per row, so I <= 1664, which holds the model's
// I = 1536), each tile's 256 rows of scales are staged in an LDS table as in
// gate/up, so a superchunk's 8 bytes per row come from LDS instead of a fresh
// memory sector.  The next tile's scales are requested with the tile's last
// superchunk and written to the table at the tile boundary.  Larger blocks
// and wider I read them from memory per superchunk.
constexpr int kDN_NT = 256;
constexpr int kDnTiles = 4;
// Weight ring: 3 superchunks (K = 1536 gives 6 per tile).
constexpr int dn_db(int mt) { return mt >= 5 ? 2 : 3; }
// fragment pairs (both terms) requested ahead of use (4 MFMAs each); 1 for
// blocks of 7-8 m-tiles, whose accumulators leave no room for more
constexpr int dn_pf(int mt) { return mt >= 7 ? 1 : 2; }

// Codes and scales of one superchunk from memory.  The lane's part of the
// offsets (its row in the first tile, its code block) is a vector offset; the
// workgroup-uniform part (tile and superchunk) is a scalar offset, used only
// when the superchunk is real (ok, uniform): otherwise the vector offset is
// out of range and the scalar offset 0.
// Part 0 and 1: code blocks g and g + 4; part 2: the 8 scale bytes.
__device__ __forceinline__ void load_bsuper_part(BSuper& b, rsrc_t rc, rsrc_t rs, uint32_t vcode, uint32_t vscale,
                                                 uint32_t scode, uint32_t sscale, bool ok, int part) {
  const uint32_t vc = ok ? vcode : kOOB, vs = ok ? vscale : kOOB;
  const uint32_t sc_ = ok ? scode : 0u, ss_ = ok ? sscale : 0u;
  if (part < 2) {
    b.q[part] = __builtin_amdgcn_raw_buffer_load_b128(rc, vc + 64u * (uint32_t)part, sc_, 0);
  } else {
    const u32x2 sv = __builtin_amdgcn_raw_buffer_load_b64(rs, vs, ss_, 0);
    b.s[0] = sv[0];
    b.s[1] = sv[1];
  }
}

// Activation ring (DMA, both terms of a chunk per buffer): 5 buffers up to 2
// m-tiles, 4 up to 4, 3 up to 6, 2 above.
constexpr int dn_nbuf(int mt) { return mt <= 2 ? 5 : (mt <= 4 ? 4 : (mt <= 6 ? 3 : 2)); }
constexpr int kDnActBytes = 3 * 2 * 96 * kDmaRow;  // holds every ring: 5x2x32, 4x2x64, 3x2x96, 2x2x128 rows
// per chunk: MS DMA instructions (two terms), and 6 weight loads (two n-tiles:
// two code blocks and the scales each) in even chunks
static_assert(dma_waits_exact(4, 2, 6, 3, 48) && dma_waits_exact(3, 4, 6, 3, 48) && dma_waits_exact(2, 6, 6, 2, 48) &&
                  dma_waits_exact(1, 8, 6, 2, 48) && dma_waits_exact(4, 2, 6, 3, 24) && dma_waits_exact(1, 8, 6, 2, 8) &&
                  dma_waits_exact(3, 4, 6, 3, 6),
              "down DMA wait counts");
// with the LDS scale table: 4 code loads per even chunk
static_assert(dma_waits_exact(4, 2, 4, 3, 48) && dma_waits_exact(3, 4, 4, 3, 48) && dma_waits_exact(2, 6, 4, 2, 48) &&
                  dma_waits_exact(1, 8, 4, 2, 48) && dma_waits_exact(4, 2, 4, 3, 24) && dma_waits_exact(1, 8, 4, 2, 8) &&
                  dma_waits_exact(3, 4, 4, 3, 6),
              "down DMA wait counts (scale table)");
// 16-byte scale pieces per thread for one tile's table (I/32 <= 52 bytes a row)
constexpr int kDnScaleU = (kDN_NT * 52 + kThr * 16 - 1) / (kThr * 16);
constexpr int kDnTableMaxNb = 52;
static_assert(kDnActBytes + kDN_NT * (kDnTableMaxNb + 8) + 2 * kMB * 4 <= 160 * 1024, "scale table fits");

// Barrier with the LDS drain only (no wait for loads in flight): for LDS
// writes that other waves read after it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Tiles nt0 .. nt0 + kDnTiles - 1 (those below ntiles) of one expert block.
// Superchunk index G runs over the tiles, nscp (the per-tile superchunk
// count rounded up to the ring) per tile; superchunks past K read zeros.
template <int MT, int DB, int NB, bool TAB>
__device__ __forceinline__ void down_block(int e, int nt0, int ntiles, int H, int I, int P, rsrc_t rh,
                                           const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                                           const int32_t* pid, const uint32_t* row_base, uint8_t* lds,
                                           float* __restrict__ ybuf) {
  using S = Shape<MT>;
  constexpr int MS = S::MS;
  constexpr int DA = NB - 1;
  constexpr uint32_t kTerm = (uint32_t)MS * 16 * kDmaRow, kBuf = 2 * kTerm;
  static_assert(NB * kBuf <= kDnActBytes, "ring fits the activation region");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const size_t cb = (size_t)3 * I * H / 2, sb = (size_t)3 * I * H / 32;
  const uint32_t mc = (uint32_t)((size_t)I * H / 2), ms = (uint32_t)((size_t)I * H / 32);
  const rsrc_t rc = mk_rsrc(codes + (size_t)e * cb + 2 * (size_t)mc, mc);
  const rsrc_t rs = mk_rsrc(scales + (size_t)e * sb + 2 * (size_t)ms, ms);
  const rsrc_t ry = mk_rsrc(ybuf, (uint32_t)((size_t)P * H * 4));
  const int nbk = I / 32;
  const int nchunks = I / kKC, nsc = nchunks / 2;
  const int nscp = (nsc + DB - 1) / DB * DB;
  const int ntw = min(kDnTiles, ntiles - nt0);
  const int gend = ntw * nscp;
  const uint32_t lo_off = (uint32_t)((size_t)P * I * 2);  // byte offset of the lo term
  // this lane's two rows of tile t: t * 256 + rbase + 16 j
  const int rbase = nt0 * kDN_NT + wid * 32 + nl;
  // weights of global superchunk G (tile G / nscp, superchunk G % nscp);
  // every row of a real tile is below H (H is a multiple of 256)
  uint32_t vcode[2], vscale[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    vcode[j] = (uint32_t)(rbase + 16 * j) * (uint32_t)(nbk * 16) + 16u * g;
    vscale[j] = (uint32_t)(rbase + 16 * j) * (uint32_t)nbk;
  }
  // scale table (TAB): the current tile's 256 rows, rows of pitch nbk + 8;
  // this lane's rows are wid * 32 + nl (n-tile 0) and 16 further (n-tile 1)
  uint8_t* tab = lds + kDnActBytes;
  const int pitch = scale_row_pitch(nbk);
  const uint8_t* srow = tab + (wid * 32 + nl) * pitch;
  const uint32_t ttotal = (uint32_t)kDN_NT * (uint32_t)nbk;
  SPieces<kDnScaleU> spc;
  if constexpr (TAB) scales_fetch<kDnScaleU>(spc, rs, (uint32_t)(nt0 * kDN_NT) * (uint32_t)nbk, ttotal);
  // NL weight loads per superchunk: per n-tile two code blocks (and, without
  // the table, the 8 scale bytes); load k of superchunk G is n-tile k / PN,
  // part k % PN
  constexpr int PN = TAB ? 2 : 3, NL = 2 * PN;
  auto load_b_part = [&](BSuper (&b)[2], int G, int k) {
    const int t = G / nscp, sc = G - t * nscp;
    const bool ok = G < gend && sc < nsc;
    const uint32_t scode = (uint32_t)t * (uint32_t)(kDN_NT * nbk * 16) + (uint32_t)sc * 128u;
    const uint32_t sscale = (uint32_t)t * (uint32_t)(kDN_NT * nbk) + (uint32_t)sc * 8u;
    load_bsuper_part(b[k / PN], rc, rs, vcode[k / PN], vscale[k / PN], scode, sscale, ok, k % PN);
  };
  auto load_b = [&](BSuper (&b)[2], int G) {
#pragma unroll
    for (int k = 0; k < NL; ++k) load_b_part(b, G, k);
  };
  // As in gate/up, an even chunk's weight loads go one at a time between its
  // multiplies (pairs 1 + k WS, all before the chunk's closing wait) when it
  // has enough pairs, else up front; they always follow the chunk's DMA.
  constexpr int kDnNQ = 4 * MT;
  constexpr bool kDnSpread = kDnNQ >= 8;
  constexpr int kDnWS = kDnSpread ? (kDnNQ - 2) / NL : 0;
  static_assert(!kDnSpread || 1 + (NL - 1) * kDnWS < kDnNQ, "weight loads before the chunk's wait");
  // activations of global chunk q (chunk q % (2 nscp) of its tile; past K or
  // past the last tile: zeros), both terms, into buffer `buf`
  uint32_t doff[MS / 2];
  dma_offsets<MS>(doff, row_base);
  auto dma_q = [&](int q, uint8_t* buf) {
    const int cin = q % (2 * nscp);
    const uint32_t kb = (q < 2 * gend && cin < nchunks) ? (uint32_t)cin * kDmaRow : kFar;
    dma_chunk<MS>(rh, doff, kb, buf);
    dma_chunk<MS>(rh, doff, lo_off + kb, buf + kTerm);
  };

  // prologue: the loop's own issue order for the chunks before chunk 0
  BSuper rb[DB][2];
  constexpr int V = 2 * (DB - 1) > DA ? 2 * (DB - 1) : DA;
#pragma unroll
  for (int v = -V; v < 0; ++v) {
    if (v + DA >= 0) dma_q(v + DA, lds + (v + DA) * kBuf);
    if (v % 2 == 0 && v / 2 + DB - 1 >= 0) load_b(rb[v / 2 + DB - 1], v / 2 + DB - 1);
  }
  if constexpr (TAB) scales_put<kDnScaleU>(spc, tab, nbk, ttotal);
  wait_vm_barrier<dma_wait_ops(NB - 1, MS, NL, 1)>();  // (draining LDS: the table is written)

  f32x4 acc[MT][2];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  int slot = 0;  // LDS buffer of the current chunk
  uint32_t sv[2][2];  // TAB: the current superchunk's scale bytes [n-tile][chunk]
  for (int G0 = 0; G0 < gend; G0 += DB) {
    const bool tile_end = (G0 + DB) % nscp == 0;
    const bool more_tiles = G0 / nscp + 1 < ntw;
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      // the next tile's scales, requested with this tile's last superchunk
      if constexpr (TAB)
        if (d == DB - 1 && tile_end && more_tiles)
          scales_fetch<kDnScaleU>(spc, rs, (uint32_t)((nt0 + G0 / nscp + 1) * kDN_NT) * (uint32_t)nbk, ttotal);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = 2 * G0 + 2 * d + h;  // global chunk
        {
          int nslot = slot + DA;
          nslot -= nslot >= NB ? NB : 0;
          dma_q(q + DA, lds + nslot * kBuf);
        }
        if (!kDnSpread && h == 0) load_b(rb[(d + DB - 1) % DB], G0 + d + DB - 1);
        __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the multiply
        const uint8_t* Ah = lds + slot * kBuf;
        const uint8_t* Al = Ah + kTerm;
        if constexpr (TAB) {
          if (h == 0) {  // the superchunk's 8 bytes of both rows, from the table
            const int sc = (G0 + d) % nscp;
            const bool ok = sc < nsc;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const u32x2 v = *reinterpret_cast<const u32x2*>(srow + j * 16 * pitch + (ok ? sc : 0) * 8);
              sv[j][0] = ok ? v[0] : 0u;
              sv[j][1] = ok ? v[1] : 0u;
            }
          }
        }
        const uint32_t sb0 = TAB ? sv[0][h] : rb[d][0].s[h], sb1 = TAB ? sv[1][h] : rb[d][1].s[h];
        const float s0v = e8m0_operand((sb0 >> (8 * g)) & 0xFFu);
        const float s1v = e8m0_operand((sb1 >> (8 * g)) & 0xFFu);
        // pair i = s*MT + m (step s, m-tile m); both terms' fragments of pair
        // i + kDnPF are requested before the four multiplies of pair i
        constexpr int kDnPF = dn_pf(MT);
        constexpr int NQ = 4 * MT, RF = kDnPF + 1;
        bf16x8 fh[RF], fl[RF];
#pragma unroll
        for (int i = 0; i < kDnPF && i < NQ; ++i) {
          fh[i % RF] = lds_frag_sw(Ah, i % MT, nl, 4 * g + i / MT);
          fl[i % RF] = lds_frag_sw(Al, i % MT, nl, 4 * g + i / MT);
        }
        bf16x8 b0 = decode8(rb[d][0].q[h][0], s0v), b1 = decode8(rb[d][1].q[h][0], s1v);
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
          const int st = i / MT, m = i % MT;
          if (i + kDnPF < NQ) {
            const int j = i + kDnPF;
            fh[j % RF] = lds_frag_sw(Ah, j % MT, nl, 4 * g + j / MT);
            fl[j % RF] = lds_frag_sw(Al, j % MT, nl, 4 * g + j / MT);
          }
          if (kDnSpread && h == 0) {
#pragma unroll
            for (int k = 0; k < NL; ++k)
              if (i == 1 + k * kDnWS) load_b_part(rb[(d + DB - 1) % DB], G0 + d + DB - 1, k);
          }
          if (m == 0 && st > 0) {
            b0 = decode8(rb[d][0].q[h][st], s0v);
            b1 = decode8(rb[d][1].q[h][st], s1v);
          }
          __builtin_amdgcn_sched_barrier(0);
          acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fh[i % RF], b0, acc[m][0], 0, 0, 0);
          acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fh[i % RF], b1, acc[m][1], 0, 0, 0);
          acc[m][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fl[i % RF], b0, acc[m][0], 0, 0, 0);
          acc[m][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fl[i % RF], b1, acc[m][1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (h == 0) wait_vm_barrier<dma_wait_ops(NB - 1, MS, NL, 0), false>();
        else wait_vm_barrier<dma_wait_ops(NB - 1, MS, NL, 1), false>();
        slot = slot + 1 == NB ? 0 : slot + 1;
      }
    }
    if ((G0 + DB) % nscp == 0) {  // a tile ends with this round: store its rows, start the next
      const int t = G0 / nscp;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int p = pid[m * 16 + 4 * g + r];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int row = rbase + t * kDN_NT + 16 * j;
            const uint32_t off = (p >= 0 && row < H) ? ((uint32_t)p * (uint32_t)H + (uint32_t)row) * 4u : kOOB;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[m][j][r]), ry, off, 0, 0);
          }
        }
        acc[m][0] = acc[m][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      if constexpr (TAB) {
        if (more_tiles) {
          // every wave has used this tile's table (its reads fed the
          // multiplies above) before the next tile's rows replace it
          lds_barrier();
          scales_put<kDnScaleU>(spc, tab, nbk, ttotal);
          lds_barrier();
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // no LDS transfer outlives the loop
}

template <bool TAB>
__global__ __launch_bounds__(kThr, 1) void k_down_mfma(
    const uint16_t* __restrict__ hterm, const int32_t* __restrict__ pairs, const int4* __restrict__ blocks,
    const int32_t* __restrict__ nblocks, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, int H, int I, int E, int P, int max_blocks, int ntiles,
    float* __restrict__ ybuf) {
  extern __shared__ uint4 lds_dyn[];  // activation ring
  uint8_t* lds8 = reinterpret_cast<uint8_t*>(lds_dyn);
  __shared__ int32_t pid[kMB];
  __shared__ uint32_t row_base[kMB];
  const int ngroups = (ntiles + kDnTiles - 1) / kDnTiles;
  int eb, ng;
  decode_item(ngroups, &eb, &ng);
  if (eb >= min(*nblocks, max_blocks)) return;
  const int4 blk = blocks[eb];
  const int e = blk.x, cnt = blk.z;
  if (e < 0 || e >= E || cnt < 1 || cnt > kMB || blk.y < 0 || blk.y > P - cnt) return;  // malformed block
  for (int i = threadIdx.x; i < kMB; i += kThr) {
    int p = i < cnt ? pairs[blk.y + i] : -1;
    if (p >= P) p = -1;
    pid[i] = p;
    row_base[i] = p >= 0 ? (uint32_t)p * (uint32_t)(I * 2) : kFar;
  }
  __syncthreads();
  const rsrc_t rh = mk_rsrc(hterm, (uint32_t)((size_t)P * I * 4));
  const int nt0 = ng * kDnTiles;
  // TAB: the launch sized LDS for the scale table (I / 32 <= kDnTableMaxNb).
  // Blocks of up to 4 m-tiles use it; larger ones read their scales per
  // superchunk (measured at 4096 tokens, ~5 m-tiles a block: the table cost
  // 2%; on 1-2 m-tile blocks it saved 5%)
#define DN(M) \
  down_block<M, dn_db(M), dn_nbuf(M), TAB && (M <= 4)>(e, nt0, ntiles, H, I, P, rh, codes, scales, pid, row_base, \
                                                       lds8, ybuf)
  switch ((cnt + 15) / 16) {
    case 1: DN(1); break;
    case 2: DN(2); break;
    case 3: DN(3); break;
    case 4: DN(4); break;
    case 5: DN(5); break;
    case 6: DN(6); break;
    case 7: DN(7); break;
    default: DN(8); break;
  }
}

// ---------------------------------------------------------------- router logits (many tokens)
// logits[t][e] = x[t] . Wr[e] (+ b[e]) for bf16 activations, on MFMA.  Each
// fp32 router weight w is split into three bf16 terms w0 = bf16(w),
// w1 = bf16(w - w0), w2 = bf16(w - w0 - w1), rounding to nearest even; the
// split is exact for every normal fp32 whose low terms stay above the bf16
// subnormal range, so every product is exact and only fp32 sums round.
// Tile: up to 128 tokens (MT m-tiles) x 128 experts; wave w owns experts
// 16w .. 16w+15 and all m-tiles.  K runs in slices of two 128-wide chunks;
// each slice is accumulated from zero and added to the running sum in slice
// order, so the result does not depend on how slices are spread over
// workgroups: a workgroup runs all slices of its tile, or (few tokens, where
// tiles alone cannot fill the chip) each slice runs in a workgroup of its own
// and writes a partial sum that k_router_reduce adds up in the same order.
constexpr int kRT_NT = 128;
constexpr int kRtSlice = 2;          // chunks per slice
constexpr int kRtSplitTokens = 256;  // slices run in workgroups of their own up to this many tokens

// This lane's 32 weights of one chunk: for each 32-wide step st, K = 32 st +
// 8g .. 32 st + 8g + 7 (q[2 st], q[2 st + 1]).  One load instruction then
// takes 16-byte pieces 32 bytes apart from each row, so the four lane groups
// of a row fall in one 128-byte line (and the next instruction fills it)
// instead of four lines; the A fragments are read at the same K.
struct WChunk {
  u32x4 q[8];
};

__device__ __forceinline__ void load_wchunk(WChunk& w, rsrc_t rw, uint32_t woff, int c, int c_end) {
  const bool ok = c < c_end;
#pragma unroll
  for (int v = 0; v < 8; ++v)
    w.q[v] = __builtin_amdgcn_raw_buffer_load_b128(
        rw, ok ? woff + (uint32_t)c * 512u + 128u * (uint32_t)(v >> 1) + 16u * (uint32_t)(v & 1) : kOOB, 0, 0);
}

// Three bf16 terms of 8 fp32 weights (two packed quads), hardware round to
// nearest even.
__device__ __forceinline__ void split3(const u32x4& q0, const u32x4& q1, bf16x8& t0, bf16x8& t1, bf16x8& t2) {
  const uint32_t in[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2 w = {__uint_as_float(in[2 * j]), __uint_as_float(in[2 * j + 1])};
    const bf16x2 a = __builtin_convertvector(w, bf16x2);
    const f32x2 r = w - __builtin_convertvector(a, f32x2);
    const bf16x2 b = __builtin_convertvector(r, bf16x2);
    const bf16x2 c = __builtin_convertvector(r - __builtin_convertvector(b, f32x2), bf16x2);
    t0[2 * j] = a[0]; t0[2 * j + 1] = a[1];
    t1[2 * j] = b[0]; t1[2 * j + 1] = b[1];
    t2[2 * j] = c[0]; t2[2 * j + 1] = c[1];
  }
}

// Chunks [c_begin, c_end) of one tile; c_begin is a slice start.  Writes the
// tile's sums to out[t][e] (row stride E) plus bias when `bias_add`.
template <int MT, int DW>
__device__ __forceinline__ void router_block(rsrc_t rx, rsrc_t rw, const float* __restrict__ bias, bool bias_add,
                                             int H, int E, int nt, int c_begin, int c_end, int t0, int cnt,
                                             const uint32_t* row_base, uint16_t* lds, float* __restrict__ out) {
  using S = Shape<MT>;
  constexpr int NV = S::NV;
  static_assert(DW % kRtSlice == 0, "the weight ring holds whole slices");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int ex = nt * kRT_NT + wid * 16 + nl;
  const uint32_t woff = ex < E ? (uint32_t)ex * (uint32_t)(H * 4) + 32u * g : kOOB;
  const int last_slice = (c_end + kRtSlice - 1) / kRtSlice;  // slices below this index are real
  uint16_t* buf0 = lds;
  uint16_t* buf1 = lds + kTile;

  uint32_t aoff[NV];
  a_offsets<NV>(aoff, row_base);
  ARegs<NV> ar[2];  // chunk c's rows in slot c % 2 (c_begin is even)
  a_fetch<NV>(ar[0], rx, aoff, (uint32_t)c_begin * (kKC * 2));
  WChunk wq[DW];
#pragma unroll
  for (int d = 0; d < DW - 1; ++d) load_wchunk(wq[d], rw, woff, c_begin + d, c_end);
  a_fetch<NV>(ar[1], rx, aoff, c_begin + 1 < c_end ? (uint32_t)(c_begin + 1) * (kKC * 2) : kFar);
  a_put<NV>(ar[0], buf0);
  __syncthreads();

  f32x4 acc[MT], tot[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = tot[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = c_begin; c0 < c_end; c0 += DW) {
#pragma unroll
    for (int d = 0; d < DW; ++d) {
      const int c = c0 + d;  // c % 2 == d % 2
      a_fetch<NV>(ar[d & 1], rx, aoff, c + 2 < c_end ? (uint32_t)(c + 2) * (kKC * 2) : kFar);
      load_wchunk(wq[(d + DW - 1) % DW], rw, woff, c + DW - 1, c_end);
      __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the multiply
      const uint16_t* A = (d & 1) ? buf1 : buf0;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        bf16x8 b0, b1, b2;
        split3(wq[d].q[2 * st], wq[d].q[2 * st + 1], b0, b1, b2);
        // every m-tile's fragment is requested first, then the three terms go
        // term by term over the m-tiles, so consecutive multiplies are
        // independent; each accumulator still takes w0, w1, w2 in that order
        bf16x8 af[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) af[m] = lds_frag(A, m * 16 + nl, 32 * st + 8 * g);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], b0, acc[m], 0, 0, 0);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], b1, acc[m], 0, 0, 0);
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], b2, acc[m], 0, 0, 0);
      }
      if (d % kRtSlice == kRtSlice - 1) {  // end of a slice: fold it into the running sum
        if (c / kRtSlice < last_slice) {
#pragma unroll
          for (int m = 0; m < MT; ++m) tot[m] += acc[m];
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      a_put<NV>(ar[(d + 1) & 1], (d & 1) ? buf0 : buf1);
      __syncthreads();
    }
  }
  if (ex < E) {
    const float b = (bias_add && bias) ? bias[ex] : 0.0f;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = m * 16 + 4 * g + r;
        if (slot < cnt) out[(size_t)(t0 + slot) * E + ex] = bias_add ? tot[m][r] + b : tot[m][r];
      }
    }
  }
}

// Workgroup b: split = b % nsplit, expert tile (b / nsplit) % ntiles, token
// tile b / (nsplit * ntiles).  nsplit == 1: every slice, logits out (with
// bias); otherwise slice `split` only, its partial sums to part[split][t][e].
// xcd_major (nsplit == 1, at most 8 expert tiles): workgroup b runs on XCD
// b % 8 and takes expert tile b % 8 (none past the last) and token tile b / 8,
// so the workgroups of one XCD stream the same router rows through its L2.
__global__ __launch_bounds__(kThr, 1) void k_router_mfma(const uint16_t* __restrict__ x,
                                                        const float* __restrict__ wr,
                                                        const float* __restrict__ bias, int T, int H, int E,
                                                        int ntiles, int nsplit, int xcd_major,
                                                        float* __restrict__ part, float* __restrict__ logits) {
  extern __shared__ uint16_t a_lds[];  // [2][kMB][kLdsRow]
  __shared__ uint32_t row_base[kMB];
  const int split = xcd_major ? 0 : blockIdx.x % nsplit, r = blockIdx.x / nsplit;
  const int nt = xcd_major ? (int)(blockIdx.x % 8) : r % ntiles;
  const int mt = xcd_major ? (int)(blockIdx.x / 8) : r / ntiles;
  if (nt >= ntiles) return;
  const int t0 = mt * kMB;
  const int cnt = min(kMB, T - t0);
  for (int i = threadIdx.x; i < kMB; i += kThr) row_base[i] = i < cnt ? (uint32_t)(t0 + i) * (uint32_t)(H * 2) : kFar;
  __syncthreads();
  const rsrc_t rx = mk_rsrc(x, (uint32_t)((size_t)T * H * 2));
  const rsrc_t rw = mk_rsrc(wr, (uint32_t)((size_t)E * H * 4));
  const int nchunks = H / kKC;
  const bool whole = nsplit == 1;
  const int c_begin = whole ? 0 : split * kRtSlice;
  const int c_end = whole ? nchunks : min(nchunks, c_begin + kRtSlice);
  float* out = whole ? logits : part + (size_t)split * T * E;
  // a workgroup of one slice (two chunks) keeps a two-chunk weight ring, so
  // it runs no chunk past its slice; the bits do not depend on the ring
#define MOE_RB_SMALL(M)                                                                                    \
  if (whole)                                                                                               \
    router_block<M, 4>(rx, rw, bias, whole, H, E, nt, c_begin, c_end, t0, cnt, row_base, a_lds, out);      \
  else                                                                                                     \
    router_block<M, kRtSlice>(rx, rw, bias, whole, H, E, nt, c_begin, c_end, t0, cnt, row_base, a_lds, out);
  switch ((cnt + 15) / 16) {
    case 1: MOE_RB_SMALL(1) break;
    case 2: MOE_RB_SMALL(2) break;
    case 3: MOE_RB_SMALL(3) break;
    case 4: MOE_RB_SMALL(4) break;
    case 5: router_block<5, 2>(rx, rw, bias, whole, H, E, nt, c_begin, c_end, t0, cnt, row_base, a_lds, out); break;
    case 6: router_block<6, 2>(rx, rw, bias, whole, H, E, nt, c_begin, c_end, t0, cnt, row_base, a_lds, out); break;
    case 7: router_block<7, 2>(rx, rw, bias, whole, H, E, nt, c_begin, c_end, t0, cnt, row_base, a_lds, out); break;
    default: router_block<8, 2>(rx, rw, bias, whole, H, E, nt, c_begin, c_end, t0, cnt, row_base, a_lds, out); break;
  }
#undef MOE_RB_SMALL
}

// logits[i] = (sum over splits s in order of part[s][i]) + bias: the same
// additions, in the same order, as a workgroup that runs every slice.
__global__ __launch_bounds__(256) void k_router_reduce(const float* __restrict__ part, int nsplit, int T, int E,
                                                       const float* __restrict__ bias, float* __restrict__ logits) {
  const size_t n = (size_t)T * E;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v = 0.0f;
#pragma unroll 4
  for (int sp = 0; sp < nsplit; ++sp) v += part[(size_t)sp * n + i];
  logits[i] = v + (bias ? bias[i % E] : 0.0f);
}

// ---------------------------------------------------------------- launchers

int max_expert_blocks(int P, int E) { return (P + kMB - 1) / kMB + (P < E ? P : E); }

hipError_t launch_expert_blocks(const int32_t* offsets, int E, int max_blocks, int4* blocks, int32_t* nblocks,
                                hipStream_t s) {
  k_expert_blocks<<<1, 1024, 0, s>>>(offsets, E, max_blocks, blocks, nblocks);
  return hipGetLastError();
}

static unsigned items_grid(int max_blocks, int ntiles) {
  const int rounds = (max_blocks + 7) / 8;
  return (unsigned)rounds * 8u * (unsigned)ntiles;
}

// LDS per workgroup on gfx950, and the kernels' static LDS (pid, row_base).
constexpr size_t kLdsBytes = 160 * 1024;
constexpr size_t kStaticLds = 2 * kMB * 4;
static size_t gu_table_bytes(int H) { return (size_t)2 * kGU_NT * scale_row_pitch(H / 32); }
static bool gu_large(int H) { return kGuActLarge + gu_table_bytes(H) + kStaticLds <= kLdsBytes; }
static size_t gateup_lds(int H) { return (size_t)(gu_large(H) ? kGuActLarge : kGuActSmall) + gu_table_bytes(H); }
static size_t down_lds(int I) {
  const int nb = I / 32;
  return (size_t)kDnActBytes + (nb <= kDnTableMaxNb ? (size_t)kDN_NT * scale_row_pitch(nb) : 0);
}

bool grouped_shape_ok(int64_t H, int64_t I) {
  if (H <= 0 || I <= 0 || H % 256 != 0 || I % 256 != 0) return false;
  if (H / 32 > 64 * kGuScaleU) return false;
  return gateup_lds((int)H) + kStaticLds <= kLdsBytes && down_lds((int)I) + kStaticLds <= kLdsBytes;
}

hipError_t launch_gateup_mfma(const uint16_t* x, int T, const int32_t* pairs, const int4* blocks,
                              const int32_t* nblocks, int max_blocks, const uint8_t* codes, const uint8_t* scales,
                              int H, int I, int E, int k, int P, uint16_t* hterm, hipStream_t s, int x_terms) {
  if (x_terms != 1 && x_terms != 3) return hipErrorInvalidValue;
  const int ntiles = (I + kGU_NT - 1) / kGU_NT;
  const size_t lds = gateup_lds(H);
  k_gateup_mfma<<<dim3(items_grid(max_blocks, ntiles)), kThr, lds, s>>>(
      x, pairs, blocks, nblocks, codes, scales, T, H, I, E, k, P, max_blocks, ntiles, gu_large(H) ? 1 : 0, x_terms,
      hterm);
  return hipGetLastError();
}

hipError_t launch_down_mfma(const uint16_t* hterm, const int32_t* pairs, const int4* blocks, const int32_t* nblocks,
                            int max_blocks, const uint8_t* codes, const uint8_t* scales, int H, int I, int E, int P,
                            float* ybuf, hipStream_t s) {
  const int ntiles = (H + kDN_NT - 1) / kDN_NT;
  const int ngroups = (ntiles + kDnTiles - 1) / kDnTiles;
  const size_t lds = down_lds(I);
  if (I / 32 <= kDnTableMaxNb)
    k_down_mfma<true><<<dim3(items_grid(max_blocks, ngroups)), kThr, lds, s>>>(
        hterm, pairs, blocks, nblocks, codes, scales, H, I, E, P, max_blocks, ntiles, ybuf);
  else
    k_down_mfma<false><<<dim3(items_grid(max_blocks, ngroups)), kThr, lds, s>>>(
        hterm, pairs, blocks, nblocks, codes, scales, H, I, E, P, max_blocks, ntiles, ybuf);
  return hipGetLastError();
}

int router_mfma_splits(int T, int H) {
  return T <= kRtSplitTokens ? (H / kKC + kRtSlice - 1) / kRtSlice : 1;
}

hipError_t launch_router_mfma(const uint16_t* x, const float* wr, const float* bias, int T, int H, int E,
                              float* logits, float* part, hipStream_t s, bool reduce) {
  const int ntiles = (E + kRT_NT - 1) / kRT_NT;
  const size_t lds = (size_t)2 * kTile * 2;
  const int nsplit = part ? router_mfma_splits(T, H) : 1;
  // token batches keep x's 32-bit buffer offsets (and the kFar sentinel) in range
  const int tb = (int)std::min<int64_t>(T, ((int64_t{1} << 29) / ((int64_t)H * 2)) / kMB * kMB);
  for (int t0 = 0; t0 < T; t0 += tb) {
    const int n = std::min(tb, T - t0);
    const int mtiles = (n + kMB - 1) / kMB;
    const int xcd_major = nsplit == 1 && ntiles <= 8 ? 1 : 0;
    const unsigned grid = xcd_major ? (unsigned)(8 * mtiles) : (unsigned)(mtiles * ntiles * nsplit);
    k_router_mfma<<<dim3(grid), kThr, lds, s>>>(x + (size_t)t0 * H, wr, bias, n, H, E, ntiles, nsplit, xcd_major,
                                                part, logits + (size_t)t0 * E);
    if (nsplit > 1 && reduce) {
      const size_t cells = (size_t)n * E;
      k_router_reduce<<<dim3((unsigned)((cells + 255) / 256)), 256, 0, s>>>(part, nsplit, n, E, bias,
                                                                          logits + (size_t)t0 * E);
    }
  }
  return hipGetLastError();
}

}  // namespace moe
