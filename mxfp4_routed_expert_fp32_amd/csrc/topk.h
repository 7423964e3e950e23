// Exact top-k with softmax over the selected logits, one wavefront per
// token; shared by the stand-alone top-k kernel and the decode gate/up
// kernel, which selects its own experts.
#pragma once

#include "common.h"

namespace moe {

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
// reads the first n back two at a time (the same address in every lane, a
// broadcast).  Keys of lanes n and above must be 0 (they never count).  The
// buffer is free again when the function returns.
__device__ __forceinline__ int rank_in_wave_lds(uint64_t v, uint64_t* buf, int n = kWave) {
  const int lane = threadIdx.x % kWave;
  buf[lane] = v;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  int r = 0;
  for (int j = 0; j < n; j += 2) {
    const ulonglong2 kk = *reinterpret_cast<const ulonglong2*>(buf + j);
    r += (kk.x > v ? 1 : 0) + (kk.y > v ? 1 : 0);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  return r;
}


// One wavefront selects for one token; each lane owns experts lane + 64*v,
// v < MAXV.  Selection: let L be the k-th largest of the 64 lane maxima.  The
// k largest lane maxima are k keys >= L, so the top k keys are all >= L;
// these candidates (usually a few more than k) are gathered into one key per
// lane and each one's rank among them is its place in the route.  When more
// than 64 keys are >= L (heavy skew inside a few lanes) the wave falls back to
// k rounds of "take the largest remaining key".  Both give the unique order
// defined by rank_key.  cand and sel_e are this wave's LDS scratch.
// On return lane j < k holds the expert of rank j in *sel and its softmax
// weight in *wsel (lanes >= k: expert 0, weight 0).
template <int MAXV>
__device__ __forceinline__ void topk_wave(const float* __restrict__ l, int E, int k, uint64_t* cand,
                                          uint32_t* sel_e, int* sel_out, float* w_out) {
  const int lane = threadIdx.x % kWave;
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
  const int lrank = rank_in_wave_lds(lmax, cand);
  const uint64_t sel_lane = __builtin_amdgcn_ballot_w64(lrank == k - 1);
  uint64_t L = 0;
  if (sel_lane) {
    const int src = __builtin_ctzll(sel_lane);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)lmax, src);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(lmax >> 32), src);
    L = ((uint64_t)hi << 32) | lo;
  }
  // candidates: keys >= L, compacted into cand[] in (slot, lane) order: one
  // ballot per slot gives each candidate its position (no atomics)
  uint32_t total = 0;  // the same in every lane
#pragma unroll
  for (int v = 0; v < MAXV; ++v) {
    const bool c = key[v] != 0ull && key[v] >= L;
    const uint64_t b = __builtin_amdgcn_ballot_w64(c);
    const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
    if (c && total + below < (uint32_t)kWave) cand[total + below] = key[v];
    total += (uint32_t)__builtin_popcountll(b);
  }

  int my_rank = kWave;          // rank of this lane's entry (>= k: not selected)
  uint32_t my_e = 0;
  if (total <= (uint32_t)kWave) {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const uint64_t c = ((uint32_t)lane < total) ? cand[lane] : 0ull;
    const int r = rank_in_wave_lds(c, cand, (int)total);  // candidates only (usually about k)
    if ((uint32_t)lane < total) { my_rank = r; my_e = ~(uint32_t)c; }
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
  if (my_rank < k) sel_e[my_rank] = my_e;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const int sel = (lane < k) ? (int)sel_e[lane] : 0;
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
  *sel_out = sel;
  *w_out = lane < k ? ex / s : 0.0f;
}

}  // namespace moe
