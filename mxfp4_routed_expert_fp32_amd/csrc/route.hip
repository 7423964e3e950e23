// Router logits (fp32), exact top-k with softmax over the selected logits, and
// the stable token -> expert counting sort.
//
// Router: fp32 logits with fp32 accumulation and no reduced-precision products
// ("Tarfa EXACTNESS" page, opening list).  Selection keeps all k experts in
// route order ("Deltafin's custom compiled runtime", sections "Complete target
// sequence tape" and "Weight fidelity").
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace moe {

// Experts per workgroup of the RMSNorm + router GEMV: the workgroup reads the
// token rows and gamma once for all of them (measured best of 1-4; the plain
// router is best at one).
constexpr int kRouterEpw = 4;

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

// ---------------------------------------------------------------- RMSNorm + router logits
// k_router_logits on n = (r * inv) * gamma, inv = 1 / sqrt(mean(r^2) + eps),
// for fp32 rows r: every workgroup reduces its tokens' r^2 itself, with the
// element order and reduction tree of k_rmsnorm, so n, and the logits, are
// the bits the two separate kernels give.  Workgroup b computes experts
// b EPW .. b EPW + EPW - 1 and also writes their slices of n, float4 columns
// [e S4, e S4 + S4) with S4 = ceil(H/4 / E), for the expert kernels that
// follow; the slices cover every column.
template <int TT, int NW, int EPW>
__global__ __launch_bounds__(256) void k_norm_router_logits(const float* __restrict__ r,
                                                            const float* __restrict__ gamma, float eps,
                                                            const float* __restrict__ wr,
                                                            const float* __restrict__ bias, int T, int H,
                                                            int E, float* __restrict__ logits,
                                                            float* __restrict__ nout) {
  // EPW experts per workgroup share the token rows, gamma and the normalised
  // values; each expert's dot product keeps its own order
  const int e0 = blockIdx.x * EPW;
  const int t0 = blockIdx.y * TT;
  const int n4 = H / 4;
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const float4* g4 = reinterpret_cast<const float4*>(gamma);
  float4 w[EPW][NW], gv[NW], v[TT][NW];
#pragma unroll
  for (int x = 0; x < EPW; ++x) {
    const int e = e0 + x;
    const float4* wrow = reinterpret_cast<const float4*>(wr + (size_t)(e < E ? e : 0) * H);
#pragma unroll
    for (int c = 0; c < NW; ++c) {
      const int q = threadIdx.x + 256 * c;
      if (q < n4 && e < E) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(wrow + q));
        w[x][c] = make_float4(a.x, a.y, a.z, a.w);
      } else {
        w[x][c] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    const int q = threadIdx.x + 256 * c;
    gv[c] = q < n4 ? g4[q] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  __shared__ float red_ss[TT][4], red_dot[TT][EPW][4];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float ss = 0.0f;
    if (t0 + t < T) {
      const float4* rt = reinterpret_cast<const float4*>(r + (size_t)(t0 + t) * H);
#pragma unroll
      for (int c = 0; c < NW; ++c) {
        const int q = threadIdx.x + 256 * c;
        v[t][c] = q < n4 ? rt[q] : make_float4(0.f, 0.f, 0.f, 0.f);
        if (q < n4) {
          ss = fmaf(v[t][c].x, v[t][c].x, ss);
          ss = fmaf(v[t][c].y, v[t][c].y, ss);
          ss = fmaf(v[t][c].z, v[t][c].z, ss);
          ss = fmaf(v[t][c].w, v[t][c].w, ss);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < NW; ++c) v[t][c] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    ss = group_sum<kWave>(ss);
    if (lane == 0) red_ss[t][wid] = ss;
  }
  __syncthreads();
  const int s4 = (n4 + E - 1) / E;
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    float acc[EPW];
#pragma unroll
    for (int x = 0; x < EPW; ++x) acc[x] = 0.0f;
    if (t0 + t < T) {
      const float tot = (red_ss[t][0] + red_ss[t][1]) + (red_ss[t][2] + red_ss[t][3]);
      const float inv = 1.0f / sqrtf(tot / (float)H + eps);
      float4* nt = reinterpret_cast<float4*>(nout + (size_t)(t0 + t) * H);
#pragma unroll
      for (int c = 0; c < NW; ++c) {
        const int q = threadIdx.x + 256 * c;
        const float4 x4 = v[t][c], gg = gv[c];
        const float4 nv = make_float4((x4.x * inv) * gg.x, (x4.y * inv) * gg.y, (x4.z * inv) * gg.z,
                                      (x4.w * inv) * gg.w);
#pragma unroll
        for (int x = 0; x < EPW; ++x) {
          acc[x] = fmaf(w[x][c].x, nv.x, acc[x]);
          acc[x] = fmaf(w[x][c].y, nv.y, acc[x]);
          acc[x] = fmaf(w[x][c].z, nv.z, acc[x]);
          acc[x] = fmaf(w[x][c].w, nv.w, acc[x]);
        }
        // the workgroup writes the slices of n that belong to its experts
        if (q < n4 && q >= e0 * s4 && q < (e0 + EPW) * s4) nt[q] = nv;
      }
    }
#pragma unroll
    for (int x = 0; x < EPW; ++x) {
      const float sv = wave_sum(acc[x]);
      if (lane == 0) red_dot[t][x][wid] = sv;
    }
  }
  __syncthreads();
  if (threadIdx.x < TT * EPW) {
    const int t = threadIdx.x / EPW, x = threadIdx.x % EPW, e = e0 + x;
    if (t0 + t < T && e < E) {
      float o = (red_dot[t][x][0] + red_dot[t][x][1]) + (red_dot[t][x][2] + red_dot[t][x][3]);
      if (bias) o += bias[e];
      logits[(size_t)(t0 + t) * E + e] = o;
    }
  }
}

template <int TT, int EPW>
static hipError_t norm_router_dispatch(dim3 grid, hipStream_t s, const float* r, const float* gamma, float eps,
                                       const float* wr, const float* bias, int T, int H, int E, float* logits,
                                       float* nout) {
  const int nw = (H / 4 + 255) / 256;
#define MOE_NRT(N) \
  k_norm_router_logits<TT, N, EPW><<<grid, 256, 0, s>>>(r, gamma, eps, wr, bias, T, H, E, logits, nout)
  switch (nw) {
    case 1: MOE_NRT(1); break;
    case 2: MOE_NRT(2); break;
    case 3: MOE_NRT(3); break;
    case 4: MOE_NRT(4); break;
    case 5: MOE_NRT(5); break;
    case 6: MOE_NRT(6); break;
    case 7: MOE_NRT(7); break;
    case 8: MOE_NRT(8); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_NRT
  return hipGetLastError();
}

hipError_t launch_norm_router_logits(const float* r, const float* gamma, float eps, const float* wr,
                                     const float* bias, int T, int H, int E, float* logits, float* nout,
                                     hipStream_t s) {
  constexpr int EPW = kRouterEpw;
  const unsigned ge = (unsigned)((E + EPW - 1) / EPW);
  if (T == 1) return norm_router_dispatch<1, EPW>(dim3(ge, 1), s, r, gamma, eps, wr, bias, T, H, E, logits, nout);
  constexpr int TT = 4;
  return norm_router_dispatch<TT, EPW>(dim3(ge, (T + TT - 1) / TT), s, r, gamma, eps, wr, bias, T, H, E, logits,
                                       nout);
}

// ---------------------------------------------------------------- top-k + softmax
// (selection in topk.h)
template <int MAXV>
__global__ __launch_bounds__(256) void k_topk_softmax(const float* __restrict__ logits, int T, int E,
                                                      int k, int32_t* __restrict__ idx,
                                                      float* __restrict__ wout) {
  __shared__ uint64_t cand[4][2 * kWave];
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  const int t = blockIdx.x * 4 + wid;
  if (t >= T) return;
  int sel;
  float wsel;
  topk_wave<MAXV>(logits + (size_t)t * E, E, k, cand[wid], &sel, &wsel);
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel;
    wout[(size_t)t * k + lane] = wsel;
  }
}

// ---------------------------------------------------------------- counting sort
// Stable sort of the T*k (token, rank) pairs by expert: histogram ->
// exclusive scan -> scatter.  Within an expert the pairs are in pair order
// (token, then rank).  Tokens are taken 64 at a time; a 64-bit mask per
// expert records which tokens of the chunk selected it.  When every token of
// the chunk names each expert at most once, a pair's place is the number of
// earlier tokens that selected the same expert (a popcount below the token's
// bit), and the pair of the lowest such token advances the expert's cursor by
// the mask's popcount.  A token that names one expert twice (an invalid
// route, or two out-of-range ids that clamp to the same expert) is seen when
// its second bit is set: atomicOr returns the bit already set.  Such a chunk
// is placed by one thread in pair order instead, so the pair list is still a
// permutation of the pairs and every cursor stays inside its expert's range.
//
// Up to kSortMultiMinTokens tokens one workgroup does everything.  Above, the
// tokens are cut into blocks of kSortBlockTokens: each block's histogram, a
// prefix over blocks per expert, a scan over experts, and a scatter in which
// every block starts from its own cursors -- the same order as one workgroup.
constexpr int kSortThreads = 1024;
constexpr int kSortBlockTokens = 256;
constexpr int kSortMultiMinTokens = 1024;

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// Scatter of tokens [t0, t1) with cursors running[E] (LDS, advanced),
// mask[E] (LDS, zero on entry and exit) and the LDS flag *dup (zero on entry
// and exit); NT threads.
template <int NT>
__device__ void scatter_tokens(const int32_t* __restrict__ idx, int t0, int t1, int E, int k,
                               unsigned long long* mask, int32_t* running, int* dup,
                               int32_t* __restrict__ pairs) {
  const int tid = threadIdx.x;
  for (int c0 = t0; c0 < t1; c0 += 64) {
    const int np = min(64, t1 - c0) * k;
    const int32_t* ic = idx + (size_t)c0 * k;
    for (int p = tid; p < np; p += NT) {
      const unsigned long long bit = 1ull << (p / k);
      if (atomicOr(&mask[clamp_expert(ic[p], E)], bit) & bit) *dup = 1;
    }
    __syncthreads();
    if (*dup) {  // uniform: written before the barrier above, cleared after the one below
      if (tid == 0) {
        for (int p = 0; p < np; ++p) {
          const int e = clamp_expert(ic[p], E);
          pairs[running[e]++] = c0 * k + p;
        }
      }
    } else {
      for (int p = tid; p < np; p += NT) {
        const int e = clamp_expert(ic[p], E);
        const unsigned long long below = mask[e] & ((1ull << (p / k)) - 1ull);
        pairs[running[e] + __popcll(below)] = c0 * k + p;
      }
      __syncthreads();
      // the pair of the lowest token of each expert advances that expert's cursor
      for (int p = tid; p < np; p += NT) {
        const int e = clamp_expert(ic[p], E);
        const unsigned long long m = mask[e];
        if ((m & ((1ull << (p / k)) - 1ull)) == 0ull) running[e] += __popcll(m);
      }
    }
    __syncthreads();
    for (int p = tid; p < np; p += NT) mask[clamp_expert(ic[p], E)] = 0ull;
    if (tid == 0) *dup = 0;
    __syncthreads();
  }
}

// Exclusive scan of counts[E] into offsets[E] (offsets[E] = total) by one
// workgroup of kSortThreads; each thread owns `per` consecutive experts.
// Also writes the scanned values to base_out when it is not null (it may be
// counts itself: a thread reads each of its counts before overwriting it).
__device__ void scan_experts(const int32_t* counts, int E, int32_t* __restrict__ offsets, int32_t* base_out,
                             int32_t* part) {
  const int tid = threadIdx.x;
  const int per = (E + kSortThreads - 1) / kSortThreads;
  const int e0 = tid * per;
  int32_t local = 0;
  for (int e = e0; e < e0 + per && e < E; ++e) local += counts[e];
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < kSortThreads; off <<= 1) {
    const int32_t v = (tid >= off) ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int32_t base = part[tid] - local;
  for (int e = e0; e < e0 + per && e < E; ++e) {
    const int32_t c = counts[e];
    offsets[e] = base;
    if (base_out) base_out[e] = base;
    base += c;
  }
  if (tid == kSortThreads - 1) offsets[E] = part[tid];
}

// One workgroup: running[E] and mask[E] live in LDS (E <= 4096: 48 KB).
// With blocks set it also cuts each expert's pairs into blocks of at most
// kExpertBlockPairs, in expert order: blocks[b] = {expert, first sorted
// index, count, 0} and *nblocks = the count written (at most max_blocks).
__global__ __launch_bounds__(kSortThreads) void k_sort_by_expert(const int32_t* __restrict__ idx,
                                                                 int T, int E, int k,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ pairs,
                                                                 int4* __restrict__ blocks, int max_blocks,
                                                                 int32_t* __restrict__ nblocks) {
  extern __shared__ unsigned long long sort_lds[];
  unsigned long long* mask = sort_lds;                               // [E]
  int32_t* running = reinterpret_cast<int32_t*>(sort_lds + E);       // [E]
  __shared__ int32_t part[kSortThreads];
  __shared__ int dup;
  const int tid = threadIdx.x;
  if (tid == 0) dup = 0;
  for (int e = tid; e < E; e += kSortThreads) { running[e] = 0; mask[e] = 0ull; }
  __syncthreads();
  const int P = T * k;
  for (int p = tid; p < P; p += kSortThreads) atomicAdd(&running[clamp_expert(idx[p], E)], 1);
  __syncthreads();
  scan_experts(running, E, offsets, running, part);  // cursors start at the offsets
  __syncthreads();
  if (blocks) {
    // expert e holds pairs [running[e], running[e + 1]) (the last ends at P)
    const int per = (E + kSortThreads - 1) / kSortThreads;
    const int e0 = tid * per;
    int32_t local = 0;
    for (int e = e0; e < e0 + per && e < E; ++e) {
      const int32_t cnt = (e + 1 < E ? running[e + 1] : P) - running[e];
      local += (cnt + kExpertBlockPairs - 1) / kExpertBlockPairs;
    }
    part[tid] = local;
    __syncthreads();
    for (int off = 1; off < kSortThreads; off <<= 1) {
      const int32_t v = (tid >= off) ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += v;
      __syncthreads();
    }
    int32_t b = part[tid] - local;
    for (int e = e0; e < e0 + per && e < E; ++e) {
      const int32_t beg = running[e], cnt = (e + 1 < E ? running[e + 1] : P) - beg;
      for (int32_t m0 = 0; m0 < cnt; m0 += kExpertBlockPairs, ++b)
        if (b < max_blocks) blocks[b] = make_int4(e, beg + m0, min(kExpertBlockPairs, cnt - m0), 0);
    }
    if (tid == kSortThreads - 1) *nblocks = min(part[kSortThreads - 1], max_blocks);
    __syncthreads();  // the scatter below moves the cursors
  }
  scatter_tokens<kSortThreads>(idx, 0, T, E, k, mask, running, &dup, pairs);
}

// Many tokens, step 1: counts[b][e] = pairs of token block b that chose e.
__global__ __launch_bounds__(256) void k_sort_count(const int32_t* __restrict__ idx, int T, int E, int k,
                                                    int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];  // [E]
  const int b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int p0 = b * kSortBlockTokens * k, p1 = min(T, (b + 1) * kSortBlockTokens) * k;
  for (int p = p0 + threadIdx.x; p < p1; p += 256) atomicAdd(&hist[clamp_expert(idx[p], E)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) counts[(size_t)b * E + e] = hist[e];
}

// Step 2: per expert, counts[b][e] becomes the pairs of blocks before b
// (exclusive prefix over blocks), totals[e] the expert's pair count.
__global__ __launch_bounds__(256) void k_sort_prefix(int32_t* __restrict__ counts, int nblk, int E,
                                                     int32_t* __restrict__ totals) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  int32_t run = 0;
  for (int b = 0; b < nblk; ++b) {
    const int32_t c = counts[(size_t)b * E + e];
    counts[(size_t)b * E + e] = run;
    run += c;
  }
  totals[e] = run;
}

// Step 3: offsets = exclusive scan of totals (one workgroup).
__global__ __launch_bounds__(kSortThreads) void k_sort_offsets(const int32_t* __restrict__ totals, int E,
                                                               int32_t* __restrict__ offsets) {
  __shared__ int32_t part[kSortThreads];
  scan_experts(totals, E, offsets, nullptr, part);
}

// Step 4: block b scatters its tokens from cursors offsets[e] + counts[b][e].
__global__ __launch_bounds__(256) void k_sort_scatter(const int32_t* __restrict__ idx, int T, int E, int k,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ counts,
                                                      int32_t* __restrict__ pairs) {
  extern __shared__ unsigned long long sort_lds[];
  unsigned long long* mask = sort_lds;                          // [E]
  int32_t* running = reinterpret_cast<int32_t*>(sort_lds + E);  // [E]
  __shared__ int dup;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) dup = 0;
  for (int e = threadIdx.x; e < E; e += 256) {
    running[e] = offsets[e] + counts[(size_t)b * E + e];
    mask[e] = 0ull;
  }
  __syncthreads();
  scatter_tokens<256>(idx, b * kSortBlockTokens, min(T, (b + 1) * kSortBlockTokens), E, k, mask, running, &dup,
                      pairs);
}

size_t sort_workspace_bytes(int T, int E) {
  if (T < kSortMultiMinTokens) return 0;
  const size_t nblk = (size_t)(T + kSortBlockTokens - 1) / kSortBlockTokens;
  return (nblk + 1) * (size_t)E * sizeof(int32_t);
}

// ---------------------------------------------------------------- split router's sum + top-k
// One workgroup of 1024 threads per token, one logit per thread (up to 1024
// experts; more loop): its E logits are summed from the router's K-slice
// partials part[sp][t][e] in slice order, from 0, with the bias added last
// (the order of the router's own reduction kernel), kept in LDS and written
// out; wave 0 then selects from LDS.
constexpr int kRedTopkThreads = 1024;
template <int MAXV>
__global__ __launch_bounds__(kRedTopkThreads) void k_router_reduce_topk(const float* __restrict__ part, int nsplit, int T,
                                                            int E, const float* __restrict__ bias, int k,
                                                            float* __restrict__ logits, int32_t* __restrict__ idx,
                                                            float* __restrict__ wout) {
  constexpr int kMaxSplit = 32;  // K slices of 256 for H <= 8192
  __shared__ float lg[kWave * MAXV];
  __shared__ uint64_t cand[2 * kWave];
  const int t = blockIdx.x;
  const size_t n = (size_t)T * E;
  for (int e = threadIdx.x; e < E; e += kRedTopkThreads) {
    const size_t i = (size_t)t * E + e;
    float pv[kMaxSplit];
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp) pv[sp] = sp < nsplit ? part[(size_t)sp * n + i] : 0.0f;
    float v = 0.0f;
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp)
      if (sp < nsplit) v += pv[sp];
    v = v + (bias ? bias[e] : 0.0f);
    lg[e] = v;
    logits[i] = v;
  }
  __syncthreads();
  if (threadIdx.x >= kWave) return;
  int sel;
  float wsel;
  topk_wave<MAXV>(lg, E, k, cand, &sel, &wsel);
  const int lane = threadIdx.x;
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel;
    wout[(size_t)t * k + lane] = wsel;
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

bool sort_is_one_workgroup(int T, const void* ws) { return T < kSortMultiMinTokens || ws == nullptr; }

hipError_t launch_router_reduce_topk(const float* part, int nsplit, int T, int E, const float* bias, int k,
                                     float* logits, int32_t* idx, float* w, hipStream_t s) {
  if (nsplit < 1 || nsplit > 32) return hipErrorInvalidValue;
  const dim3 grid((unsigned)T);
  if (E <= 64 * 4)
    k_router_reduce_topk<4><<<grid, kRedTopkThreads, 0, s>>>(part, nsplit, T, E, bias, k, logits, idx, w);
  else if (E <= 64 * 16)
    k_router_reduce_topk<16><<<grid, kRedTopkThreads, 0, s>>>(part, nsplit, T, E, bias, k, logits, idx, w);
  else
    k_router_reduce_topk<64><<<grid, kRedTopkThreads, 0, s>>>(part, nsplit, T, E, bias, k, logits, idx, w);
  return hipGetLastError();
}

hipError_t launch_sort_by_expert(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* pairs,
                                 void* ws, hipStream_t s, int4* blocks, int max_blocks, int32_t* nblocks) {
  const size_t lds = (size_t)E * (sizeof(unsigned long long) + sizeof(int32_t));
  if (sort_is_one_workgroup(T, ws)) {
    if (blocks && !nblocks) return hipErrorInvalidValue;
    k_sort_by_expert<<<1, kSortThreads, lds, s>>>(idx, T, E, k, offsets, pairs, blocks, max_blocks, nblocks);
    return hipGetLastError();
  }
  if (blocks) return hipErrorInvalidValue;  // the caller runs launch_expert_blocks
  const int nblk = (T + kSortBlockTokens - 1) / kSortBlockTokens;
  int32_t* counts = static_cast<int32_t*>(ws);  // [nblk][E]
  int32_t* totals = counts + (size_t)nblk * E;  // [E]
  k_sort_count<<<nblk, 256, (size_t)E * sizeof(int32_t), s>>>(idx, T, E, k, counts);
  k_sort_prefix<<<(E + 255) / 256, 256, 0, s>>>(counts, nblk, E, totals);
  k_sort_offsets<<<1, kSortThreads, 0, s>>>(totals, E, offsets);
  k_sort_scatter<<<nblk, 256, lds, s>>>(idx, T, E, k, offsets, counts, pairs);
  return hipGetLastError();
}

}  // namespace moe
