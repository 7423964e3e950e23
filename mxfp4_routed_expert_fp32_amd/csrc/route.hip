// Router logits (fp32), exact top-k with softmax over the selected logits, and
// the stable token -> expert counting sort.
//
// Router: fp32 logits with fp32 accumulation and no reduced-precision products
// ("Tarfa EXACTNESS" page, opening list).  Selection keeps all k experts in
// route order ("Deltafin's custom compiled runtime", sections "Complete target
// sequence tape" and "Weight fidelity").
#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------- router logits
// One workgroup per (expert row, tile of TT tokens).  Thread i owns float4
// columns i + 256*c (c < NW) of the router row; all of the row's loads are
// issued before the FMAs.  The reduction order (DPP within a wave, then the 4
// wave sums in a fixed order) does not depend on timing.
template <bool XF32, int TT, int NW>
__global__ __launch_bounds__(256) void k_router_logits(const void* __restrict__ x,
                                                       const float* __restrict__ wr,
                                                       const float* __restrict__ bias, int T, int H,
                                                       int E, float* __restrict__ logits) {
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * TT;
  const int n4 = H / 4;
  const float4* wrow = reinterpret_cast<const float4*>(wr + (size_t)e * H);
  float4 w[NW];
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    const int q = threadIdx.x + 256 * c;
    if (q < n4) {
      const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(wrow + q));
      w[c] = make_float4(v.x, v.y, v.z, v.w);
    } else {
      w[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  float acc[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    acc[t] = 0.0f;
    if (t0 + t < T) {
      float4 xv[NW];
#pragma unroll
      for (int c = 0; c < NW; ++c) {
        const int q = threadIdx.x + 256 * c;
        if (q < n4) {
          if constexpr (XF32) {
            xv[c] = reinterpret_cast<const float4*>(static_cast<const float*>(x) + (size_t)(t0 + t) * H)[q];
          } else {
            uint2 b = reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(x) + (size_t)(t0 + t) * H)[q];
            xv[c] = make_float4(bf16_bits_to_f32(b.x & 0xFFFFu), bf16_bits_to_f32(b.x >> 16),
                                bf16_bits_to_f32(b.y & 0xFFFFu), bf16_bits_to_f32(b.y >> 16));
          }
        } else {
          xv[c] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int c = 0; c < NW; ++c) {
        acc[t] = fmaf(w[c].x, xv[c].x, acc[t]);
        acc[t] = fmaf(w[c].y, xv[c].y, acc[t]);
        acc[t] = fmaf(w[c].z, xv[c].z, acc[t]);
        acc[t] = fmaf(w[c].w, xv[c].w, acc[t]);
      }
    }
  }
  __shared__ float red[TT][4];
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float v = wave_sum(acc[t]);
    if (lane == 0) red[t][wid] = v;
  }
  __syncthreads();
  if (threadIdx.x < TT && t0 + (int)threadIdx.x < T) {
    const int t = threadIdx.x;
    float v = (red[t][0] + red[t][1]) + (red[t][2] + red[t][3]);
    if (bias) v += bias[e];
    logits[(size_t)(t0 + t) * E + e] = v;
  }
}

// ---------------------------------------------------------------- top-k + softmax
// Rank key of a logit: larger key = earlier in route order.  Higher value
// first; -0 and +0 are equal; NaN is below every number (-inf included); equal
// values go to the lower expert id.  Key 0 is never a valid key.
__device__ __forceinline__ uint64_t rank_key(float v, uint32_t e) {
  uint32_t u = __float_as_uint(v);
  uint32_t ord;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) {
    ord = 0;                                  // NaN
  } else {
    if ((u << 1) == 0) u = 0;                 // -0 -> +0
    ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  return ((uint64_t)ord << 32) | (uint32_t)(~e);
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Largest 64-bit key of the wavefront, returned in every lane.  Lanes of rows
// a broadcast does not reach receive 0, which never wins.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = umax64(v, dpp_u64<0xB1>(v));
  v = umax64(v, dpp_u64<0x4E>(v));
  v = umax64(v, dpp_u64<0x141>(v));
  v = umax64(v, dpp_u64<0x140>(v));
  v = umax64(v, dpp_u64<0x142, 0xA>(v));
  v = umax64(v, dpp_u64<0x143, 0xC>(v));
  const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// Number of lanes whose 64-bit key is larger than this lane's (keys unique),
// through a 64-entry LDS buffer of the wave: every lane writes its key, then
// reads all 64 back two at a time (the same address in every lane, a
// broadcast).  The buffer is free again when the function returns.
__device__ __forceinline__ int rank_in_wave_lds(uint64_t v, uint64_t* buf) {
  const int lane = threadIdx.x % kWave;
  buf[lane] = v;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  int r = 0;
#pragma unroll
  for (int j = 0; j < kWave; j += 2) {
    const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(buf + j);
    r += (kk.x > v ? 1 : 0) + (kk.y > v ? 1 : 0);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  return r;
}


// One wavefront per token; each lane owns experts lane + 64*v, v < MAXV.
// Selection: let L be the k-th largest of the 64 lane maxima.  The k largest
// lane maxima are k keys >= L, so the top k keys are all >= L; these
// candidates (usually a few more than k) are gathered into one key per lane
// and each one's rank among them is its place in the route.  When more than
// 64 keys are >= L (heavy skew inside a few lanes) the wave falls back to k
// rounds of "take the largest remaining key".  Both give the unique order
// defined by rank_key.
template <int MAXV>
__global__ __launch_bounds__(256) void k_topk_softmax(const float* __restrict__ logits, int T, int E,
                                                      int k, int32_t* __restrict__ idx,
                                                      float* __restrict__ wout) {
  __shared__ uint64_t cand[4][kWave];
  __shared__ uint32_t ncand[4];
  __shared__ uint32_t sel_e[4][kWave];
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int t = blockIdx.x * 4 + wid;
  if (t >= T) return;
  const float* l = logits + (size_t)t * E;
  float lv[MAXV];
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int e = lane + kWave * v;
    lv[v] = (e < E) ? l[e] : 0.0f;
  }
  uint64_t key[MAXV];
  uint64_t lmax = 0;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const int e = lane + kWave * v;
    key[v] = (e < E) ? rank_key(lv[v], (uint32_t)e) : 0ull;
    lmax = umax64(lmax, key[v]);
  }
  // L = k-th largest lane maximum (the lane of rank k-1); 0 if fewer lanes hold keys
  const int lrank = rank_in_wave_lds(lmax, cand[wid]);
  const uint64_t sel_lane = __builtin_amdgcn_ballot_w64(lrank == k - 1);
  uint64_t L = 0;
  if (sel_lane) {
    const int src = __builtin_ctzll(sel_lane);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)lmax, src);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(lmax >> 32), src);
    L = ((uint64_t)hi << 32) | lo;
  }
  // candidates: keys >= L
  int mine = 0;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) mine += (key[v] != 0ull && key[v] >= L) ? 1 : 0;
  int total = mine;
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) total += __shfl_xor(total, m, kWave);

  int my_rank = kWave;          // rank of this lane's entry (>= k: not selected)
  uint32_t my_e = 0;
  if (total <= kWave) {
    if (lane == 0) ncand[wid] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      if (key[v] != 0ull && key[v] >= L) {
        const uint32_t pos = atomicAdd(&ncand[wid], 1u);
        cand[wid][pos] = key[v];
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const uint64_t c = (lane < total) ? cand[wid][lane] : 0ull;
    const int r = rank_in_wave_lds(c, cand[wid]);
    if (lane < total) { my_rank = r; my_e = ~(uint32_t)c; }
  } else {
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int v = 0; v < MAXV; ++v) best = umax64(best, key[v]);
      const uint64_t win = wave_max_u64(best);
#pragma unroll
      for (int v = 0; v < MAXV; ++v)
        if (key[v] == win) key[v] = 0;
      if (lane == j) { my_rank = j; my_e = ~(uint32_t)win; }
    }
  }
  // lane r < k receives the entry of rank r
  if (my_rank < k) sel_e[wid][my_rank] = my_e;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int sel = (lane < k) ? (int)sel_e[wid][lane] : 0;
  // softmax over the selected logits, in rank order; each logit is read back
  // from the registers of the lane that holds it (lane sel % 64, slot
  // sel / 64), not from memory
  float lj = 0.0f;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const float x = __shfl(lv[v], sel % kWave, kWave);
    if (sel / kWave == v) lj = x;
  }
  if (lane >= k) lj = 0.0f;
  const float m = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lj)));
  const float ex = (lane < k) ? expf(lj - m) : 0.0f;
  const float s = wave_sum(ex);
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel;
    wout[(size_t)t * k + lane] = ex / s;
  }
}

// ---------------------------------------------------------------- counting sort
// Stable sort of the T*k (token, rank) pairs by expert, in one workgroup:
// histogram -> exclusive scan -> scatter.  Within an expert the pairs are in
// token order: each token selects an expert at most once, so a pair's place
// is the number of earlier tokens that selected the same expert.  Tokens are
// taken 64 at a time; a 64-bit mask per expert records which tokens of the
// chunk selected it, and a popcount below the token's bit gives its place.
constexpr int kSortThreads = 1024;

// running[E] and mask[E] live in LDS (E <= 4096: 48 KB).
__global__ __launch_bounds__(kSortThreads) void k_sort_by_expert(const int32_t* __restrict__ idx,
                                                                 int T, int E, int k,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ pairs) {
  extern __shared__ unsigned long long sort_lds[];
  unsigned long long* mask = sort_lds;                               // [E]
  int32_t* running = reinterpret_cast<int32_t*>(sort_lds + E);       // [E]
  __shared__ int32_t part[kSortThreads];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kSortThreads) { running[e] = 0; mask[e] = 0ull; }
  __syncthreads();
  const int P = T * k;
  for (int p = tid; p < P; p += kSortThreads) {
    int e = idx[p];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    atomicAdd(&running[e], 1);
  }
  __syncthreads();
  // exclusive scan of the counts: each thread owns `per` consecutive experts
  const int per = (E + kSortThreads - 1) / kSortThreads;
  const int e0 = tid * per;
  int32_t local = 0;
  for (int e = e0; e < e0 + per && e < E; ++e) local += running[e];
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kSortThreads; off <<= 1) {
    int32_t v = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t base = part[tid] - local;
  for (int e = e0; e < e0 + per && e < E; ++e) {
    int32_t c = running[e];
    offsets[e] = base;
    running[e] = base;
    base += c;
  }
  if (tid == 0) offsets[E] = P;
  __syncthreads();
  for (int c0 = 0; c0 < T; c0 += 64) {
    const int np = min(64, T - c0) * k;
    const int32_t* ic = idx + (size_t)c0 * k;
    for (int p = tid; p < np; p += kSortThreads) {
      int e = ic[p];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      atomicOr(&mask[e], 1ull << (p / k));
    }
    __syncthreads();
    for (int p = tid; p < np; p += kSortThreads) {
      int e = ic[p];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      const int tl = p / k;
      const unsigned long long m = mask[e];
      const unsigned long long below = m & ((1ull << tl) - 1ull);
      pairs[running[e] + __popcll(below)] = c0 * k + p;
    }
    __syncthreads();
    // the pair of the lowest token of each expert advances that expert's cursor
    for (int p = tid; p < np; p += kSortThreads) {
      int e = ic[p];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      const int tl = p / k;
      const unsigned long long m = mask[e];
      if ((m & ((1ull << tl) - 1ull)) == 0ull) running[e] += __popcll(m);
    }
    __syncthreads();
    for (int p = tid; p < np; p += kSortThreads) {
      int e = ic[p];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);
      mask[e] = 0ull;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------- launchers

template <bool XF32, int TT>
static hipError_t router_dispatch(dim3 grid, hipStream_t s, const void* x, const float* wr, const float* bias,
                                  int T, int H, int E, float* logits) {
  const int nw = (H / 4 + 255) / 256;
#define MOE_RT(N) k_router_logits<XF32, TT, N><<<grid, 256, 0, s>>>(x, wr, bias, T, H, E, logits)
  switch (nw) {
    case 1: MOE_RT(1); break;
    case 2: MOE_RT(2); break;
    case 3: MOE_RT(3); break;
    case 4: MOE_RT(4); break;
    case 5: MOE_RT(5); break;
    case 6: MOE_RT(6); break;
    case 7: MOE_RT(7); break;
    case 8: MOE_RT(8); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_RT
  return hipGetLastError();
}

hipError_t launch_router_logits(const void* x, bool x_f32, const float* wr, const float* bias, int T,
                                int H, int E, float* logits, hipStream_t s) {
  if (T == 1) {
    const dim3 grid(E, 1);
    return x_f32 ? router_dispatch<true, 1>(grid, s, x, wr, bias, T, H, E, logits)
                 : router_dispatch<false, 1>(grid, s, x, wr, bias, T, H, E, logits);
  }
  constexpr int TT = 4;
  const dim3 grid(E, (T + TT - 1) / TT);
  return x_f32 ? router_dispatch<true, TT>(grid, s, x, wr, bias, T, H, E, logits)
               : router_dispatch<false, TT>(grid, s, x, wr, bias, T, H, E, logits);
}

hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                               hipStream_t s) {
  dim3 grid((T + 3) / 4);
  if (E <= 64 * 4)
    k_topk_softmax<4><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  else if (E <= 64 * 16)
    k_topk_softmax<16><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  else
    k_topk_softmax<64><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  return hipGetLastError();
}

hipError_t launch_sort_by_expert(const int32_t* idx, int T, int E, int k, int32_t* offsets,
                                 int32_t* pairs, hipStream_t s) {
  size_t lds = (size_t)E * (sizeof(unsigned long long) + sizeof(int32_t));
  k_sort_by_expert<<<1, kSortThreads, lds, s>>>(idx, T, E, k, offsets, pairs);
  return hipGetLastError();
}

}  // namespace moe
