// Exact top-k with softmax over the selected logits, one wavefront per
// token; shared by the stand-alone top-k kernel and the decode gate/up
// kernel, which selects its own experts.
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {

// Rank key of expert e's logit v: larger key = earlier in route order.
// Higher value first; -0 and +0 are equal; NaN is below every number (-inf
// included); equal values go to the lower expert id.  The upper word is the
// logit's order as an unsigned integer (rank_ord: x + 0 is x except that -0
// becomes +0, under IEEE round to nearest with denormals kept; then the sign
// bit flips the order of the magnitude bits; NaN gives 0), the lower word is
// ~e.  Key 0 is never a valid key.
__device__ __forceinline__ uint32_t rank_ord(float v) {
  const float y = v + 0.0f;
  const uint32_t u = __float_as_uint(y);
  const uint32_t o = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
  return y == y ? o : 0u;
}

__device__ __forceinline__ uint64_t make_key(uint32_t ord, uint32_t e) { return ((uint64_t)ord << 32) | (uint32_t)(~e); }

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

// The logit a rank key was made from (rank_ord inverted on its upper word):
// exact, except that -0 comes back as +0 and every NaN as one NaN pattern.
__device__ __forceinline__ float key_logit(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// Each candidate's rank among the `total` (<= 64) candidates cand[0, total),
// read in place: entries past `total` must be 0, which never counts.  16
// entries (8 reads) are requested at a time, then compared, so the reads'
// latency is paid once per batch.  Lane i < total gets the rank and key of
// candidate i; other lanes keep theirs (rank kWave: not selected).
__device__ __forceinline__ void rank_candidates(const uint64_t* cand, uint32_t total, int* my_rank,
                                                uint64_t* my_key) {
  const int lane = threadIdx.x % kWave;
  const uint64_t c = ((uint32_t)lane < total) ? cand[lane] : 0ull;
  int r = 0;
  auto batch = [&](int j0) {
    ulonglong2 kk[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) kk[q] = *reinterpret_cast<const ulonglong2*>(cand + j0 + 2 * q);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < 8; ++q) r += (kk[q].x > c ? 1 : 0) + (kk[q].y > c ? 1 : 0);
  };
  batch(0);
  if (total > 16) batch(16);
  if (total > 32) {
    batch(32);
    batch(48);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if ((uint32_t)lane < total) {
    *my_rank = r;
    *my_key = c;
  }
}

// From every lane's (rank, key) (rank >= k: not selected) to lane j < k
// holding the expert of rank j and its softmax weight (lanes >= k: expert 0,
// weight 0); cand (64 keys) is scratch.  weights = false leaves every weight
// 0.
__device__ __forceinline__ void topk_finish(uint64_t* cand, int my_rank, uint64_t my_key, int k, int* sel_out,
                                            float* w_out, bool weights) {
  const int lane = threadIdx.x % kWave;
  // lane r < k receives the key of rank r
  if (my_rank < k) cand[my_rank] = my_key;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const uint64_t kj = (lane < k) ? cand[lane] : 0ull;
  const int sel = (lane < k) ? (int)~(uint32_t)kj : 0;
  *sel_out = sel;
  *w_out = 0.0f;
  if (!weights) return;
  // softmax over the selected logits, in rank order, each logit decoded from
  // its key; lane 0 holds the largest
  const float lj = (lane < k) ? key_logit(kj) : 0.0f;
  const float m = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(lj)));
  const float ex = (lane < k) ? expf(lj - m) : 0.0f;
  const float s = wave_sum(ex);
  *w_out = lane < k ? ex / s : 0.0f;
}

// One wavefront selects for one token; lane l owns experts MAXV*l + v, v <
// MAXV (contiguous, so a row of E % 4 == 0 logits is read with 16-byte
// loads).  Selection: let T be the k-th largest of the 64 lane maxima's top
// 16 key bits (sign, exponent and 7 mantissa bits of the logit; a 16-step
// radix select on ballots), as a 32-bit bound.  At least k keys are >= T, so
// the top k keys all are; these candidates (usually a few more than k) are
// gathered into one key per lane, each lane writing its own at an offset from
// a ballot prefix of the per-lane counts (the others into a dummy half of the
// buffer, so the writes need no branches; the first half is zeroed before,
// so it holds 0 past the candidates), and each one's rank among them, read in
// place, is its place in the route.  When more than 64 keys qualify (heavy
// ties or skew), or fewer than k lanes hold a number (T = 0), the wave falls
// back to k rounds of "take the largest remaining key".
// Both give the unique order of the rank keys.  cand is this wave's LDS
// scratch (2 * 64 keys).
// On return lane j < k holds the expert of rank j in *sel and its softmax
// weight in *wsel (lanes >= k: expert 0, weight 0).  weights = false (a
// wave-uniform flag) skips the softmax and leaves every weight 0, for callers
// that need the experts only.
template <int MAXV>
__device__ __forceinline__ void topk_wave(const float* __restrict__ l, int E, int k, uint64_t* cand,
                                          int* sel_out, float* w_out, bool weights = true) {
  static_assert(MAXV % 4 == 0, "whole 16-byte loads");
  const int lane = threadIdx.x % kWave;
  const int e0 = lane * MAXV;
  float lv[MAXV];
  if ((E & 3) == 0 && (reinterpret_cast<uintptr_t>(l) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < MAXV / 4; ++q) {
      const int e = e0 + 4 * q;  // e < E implies e + 3 < E
      const float4 f = *reinterpret_cast<const float4*>(l + (e < E ? e : 0));
      lv[4 * q] = f.x; lv[4 * q + 1] = f.y; lv[4 * q + 2] = f.z; lv[4 * q + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int v = 0; v < MAXV; ++v) lv[v] = l[e0 + v < E ? e0 + v : 0];
  }
  // upper key words only (the lower word is ~expert, implicit in v); bit v
  // of `alive`: expert e0 + v exists (in the fallback: and is not taken yet)
  using Mask = typename std::conditional<(MAXV > 32), uint64_t, uint32_t>::type;
  constexpr Mask kOne = 1;
  constexpr Mask kAll = MAXV >= 64 ? ~Mask(0) : (kOne << MAXV) - 1;
  const int nh = E - e0;  // experts this lane holds (may be <= 0 or >= MAXV)
  const Mask alive = nh >= MAXV ? kAll : (nh <= 0 ? Mask(0) : (kOne << nh) - 1);
  uint32_t ord[MAXV];
  uint32_t mo = 0;  // upper word of this lane's largest key
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const uint32_t o = v < nh ? rank_ord(lv[v]) : 0u;  // absent experts: 0, like NaN
    ord[v] = o;
    mo = o > mo ? o : mo;
  }
  cand[lane] = 0ull;  // candidates overwrite [0, total); the rest stays 0 for the rank reads
  // T: the largest multiple of 2^16 with at least k lane maxima at or above
  // it, built bit by bit from the top
  uint32_t T = 0;
#pragma unroll
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t c = T | (1u << bit);
    if (__builtin_popcountll(__builtin_amdgcn_ballot_w64(mo >= c)) >= k) T = c;
  }
  // candidates: present keys whose upper word is >= T; lane offsets from a
  // prefix of the per-lane counts, one ballot per count bit
  // (with T > 0, the usual case, absent experts and NaN have key word 0 < T;
  // T = 0, fewer than k lanes hold a number, goes to the fallback below)
  uint32_t cnt = 0;
#pragma unroll
  for (int v = 0; v < MAXV; ++v) cnt += ord[v] >= T ? 1u : 0u;
  uint32_t excl = 0, total = 0;
#pragma unroll
  for (int b = 0; (1 << b) <= MAXV; ++b) {
    const uint64_t m = __builtin_amdgcn_ballot_w64((cnt >> b) & 1u);
    excl += __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
    total += (uint32_t)__builtin_popcountll(m) << b;
  }

  int my_rank = kWave;  // rank of this lane's entry (>= k: not selected)
  uint64_t my_key = 0;
  if (T != 0 && total <= (uint32_t)kWave) {
    uint32_t ptr = excl;
#pragma unroll
    for (int v = 0; v < MAXV; ++v) {
      const bool c = ord[v] >= T;
      cand[c ? ptr : kWave + lane] = make_key(ord[v], (uint32_t)(e0 + v));  // non-candidates: the dummy half
      ptr += c ? 1u : 0u;
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    rank_candidates(cand, total, &my_rank, &my_key);
  } else {
    Mask left = alive;  // present and not taken yet
    for (int j = 0; j < k; ++j) {
      uint64_t best = 0;
#pragma unroll
      for (int v = 0; v < MAXV; ++v)
        best = umax64(best, ((left >> v) & kOne) ? make_key(ord[v], (uint32_t)(e0 + v)) : 0ull);
      const uint64_t win = wave_max_u64(best);
      const uint32_t we = ~(uint32_t)win;  // the winner's expert
      if (we - (uint32_t)e0 < (uint32_t)MAXV) left &= ~(kOne << (we - (uint32_t)e0));
      if (lane == j) { my_rank = j; my_key = win; }
    }
  }
  topk_finish(cand, my_rank, my_key, k, sel_out, w_out, weights);
}

// LDS of topk_wg for a workgroup of KS waves.
template <int KS>
struct TopkWgLds {
  uint32_t gmax[kWave * KS];  // [lane][wave]: each lane's largest key word
  uint64_t cand[2 * kWave];   // candidates; then topk_finish's (and the fallback's) scratch
  uint32_t bound;             // T
  uint32_t count;             // candidate slots claimed
};

// topk_wave's selection with the per-logit work spread over the KS waves of a
// workgroup (all of them call it; wave 0 returns the result, the others
// expert 0 and weight 0).  Lane l of wave w holds experts
// v * 64 KS + 64 w + l, v < MAXW, so each wave's loads are contiguous.
//  1. Every lane makes its keys' upper words and their maximum.
//  2. Wave 0 takes, for each of its lanes g, the largest of lane g's maxima
//     over the waves (64 group maxima, each a distinct key) and finds T as
//     topk_wave does on its lane maxima: at least k keys are >= T, so the top
//     k keys all are.
//  3. Every lane claims slots for its keys >= T with one LDS atomic and
//     writes them there (in no particular order: ranks are counted).
//  4. Wave 0 ranks the candidates and finishes as topk_wave does.
// When more than 64 keys qualify, or T = 0, wave 0 runs topk_wave<MAXV>
// instead.  Both give the unique order of the rank keys, so the result is
// topk_wave's, bit for bit.  E <= 64 KS MAXW and E <= 64 MAXV.  Contains
// workgroup barriers: every wave of the workgroup must call it.
template <int KS, int MAXW, int MAXV>
__device__ __forceinline__ void topk_wg(const float* __restrict__ l, int E, int k, TopkWgLds<KS>& sm, int* sel_out,
                                        float* w_out, bool weights) {
  static_assert(KS >= 2, "one wave: topk_wave");
  const int lane = threadIdx.x % kWave, wid = threadIdx.x / kWave;
  // all loads first (an absent expert's load reads expert 0), then the keys
  float lv[MAXW];
#pragma unroll
  for (int v = 0; v < MAXW; ++v) {
    const int e = v * kWave * KS + wid * kWave + lane;
    lv[v] = l[e < E ? e : 0];
  }
  uint32_t ord[MAXW];
  uint32_t mo = 0;
#pragma unroll
  for (int v = 0; v < MAXW; ++v) {
    const int e = v * kWave * KS + wid * kWave + lane;
    const uint32_t o = e < E ? rank_ord(lv[v]) : 0u;  // absent experts: 0, like NaN
    ord[v] = o;
    mo = o > mo ? o : mo;
  }
  sm.gmax[lane * KS + wid] = mo;
  if (wid == 0) sm.cand[lane] = 0ull;  // rank_candidates reads 0 past the candidates
  if (threadIdx.x == 0) sm.count = 0u;
  __syncthreads();
  if (wid == 0) {
    uint32_t g = 0;
#pragma unroll
    for (int w = 0; w < KS; ++w) {
      const uint32_t m = sm.gmax[lane * KS + w];
      g = m > g ? m : g;
    }
    uint32_t T = 0;
#pragma unroll
    for (int bit = 31; bit >= 16; --bit) {
      const uint32_t c = T | (1u << bit);
      if (__builtin_popcountll(__builtin_amdgcn_ballot_w64(g >= c)) >= k) T = c;
    }
    if (lane == 0) sm.bound = T;
  }
  __syncthreads();
  const uint32_t T = sm.bound;
  if (T != 0) {
    uint32_t n = 0;
#pragma unroll
    for (int v = 0; v < MAXW; ++v) n += ord[v] >= T ? 1u : 0u;
    if (n) {
      uint32_t slot = atomicAdd(&sm.count, n);
#pragma unroll
      for (int v = 0; v < MAXW; ++v) {
        if (ord[v] >= T) {
          if (slot < (uint32_t)kWave) sm.cand[slot] = make_key(ord[v], (uint32_t)(v * kWave * KS + wid * kWave + lane));
          ++slot;
        }
      }
    }
  }
  __syncthreads();
  *sel_out = 0;
  *w_out = 0.0f;
  if (wid != 0) return;
  const uint32_t total = sm.count;
  if (T == 0 || total > (uint32_t)kWave) {
    topk_wave<MAXV>(l, E, k, sm.cand, sel_out, w_out, weights);
    return;
  }
  int my_rank = kWave;
  uint64_t my_key = 0;
  rank_candidates(sm.cand, total, &my_rank, &my_key);
  topk_finish(sm.cand, my_rank, my_key, k, sel_out, w_out, weights);
}

}  // namespace moe
