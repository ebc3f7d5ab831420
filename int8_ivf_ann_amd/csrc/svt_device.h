// svt_device.h - device helpers shared by the gfx950 kernels of the search library (svt_kernels.hip,
// svt_group.hip): ordering keys, int8 dot products, wave and block primitives, block radix select.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svt {

// ------------------------------------------------------------------------------------------------
// small device helpers

__device__ __forceinline__ uint64_t make_key(int32_t score, uint32_t id) {
  return ((uint64_t)((uint32_t)score ^ 0x80000000u) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ int32_t key_score(uint64_t key) {
  return (int32_t)((uint32_t)(key >> 32) ^ 0x80000000u);
}
__device__ __forceinline__ uint32_t key_id(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }

// 16 int8 products accumulated in int32 with four v_dot4 instructions
__device__ __forceinline__ int32_t dot16(const int4 x, const int4 y, int32_t acc) {
  acc = __builtin_amdgcn_sdot4(x.x, y.x, acc, false);
  acc = __builtin_amdgcn_sdot4(x.y, y.y, acc, false);
  acc = __builtin_amdgcn_sdot4(x.z, y.z, acc, false);
  acc = __builtin_amdgcn_sdot4(x.w, y.w, acc, false);
  return acc;
}

// Sum of v over each group of LPR consecutive lanes (LPR = 1, 2, 4, 8 or 16), valid in the group's first
// lane.  DPP lane moves: quad permutations for lane ^ 1 and lane ^ 2, then row shifts that bring lane
// + 4 and lane + 8 (within a 16-lane row) to the group's first lane.
template <int LPR>
__device__ __forceinline__ int32_t group_sum(int32_t v) {
  if constexpr (LPR >= 2) v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);    // quad_perm 1,0,3,2
  if constexpr (LPR >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);    // quad_perm 2,3,0,1
  if constexpr (LPR >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x104, 0xF, 0xF, true);   // row_shl:4
  if constexpr (LPR >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x108, 0xF, 0xF, true);  // row_shl:8
  return v;
}

// A free slot of an updatable index holds the reserved signature with every bit set, which no live item
// has: the filter rejects it whatever the mask (a mask of zero passes every live item).
__device__ __forceinline__ bool sig_live(uint64_t s0, uint64_t s1, int sig_words) {
  return (s0 & (sig_words == 2 ? s1 : ~0ull)) != ~0ull;
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// number of set bits of `mask` below this lane
__device__ __forceinline__ int mbcnt(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    T u = __shfl_up(v, off);
    if (l >= off) v += u;
  }
  return v;
}

// exclusive block scan of one value per thread; returns the block total in *total.
// wave_tot: LDS scratch of NT/64 + 1 values.
template <int NT, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T *wave_tot, T *total) {
  constexpr int NW = NT / 64;
  const int l = lane_id(), wv = threadIdx.x / 64;
  T inc = wave_incl_scan(v);
  if (l == 63) wave_tot[wv] = inc;
  __syncthreads();
  if (wv == 0) {
    T t = l < NW ? wave_tot[l] : T(0);
    T ti = wave_incl_scan(t);
    if (l < NW) wave_tot[l] = ti - t;           // exclusive wave offsets
    if (l == NW - 1) wave_tot[NW] = ti;         // total
  }
  __syncthreads();
  T r = wave_tot[wv] + inc - v;
  *total = wave_tot[NW];
  __syncthreads();
  return r;
}

// ------------------------------------------------------------------------------------------------
// Block radix select over distinct 64-bit keys.
//
// Returns T such that the keys >= T are exactly the `need` largest keys visited by `for_each`
// (1 <= need <= number of keys).  Passes of 8-bit digits start at the highest bit in which the keys
// differ and stop as soon as the boundary bucket is taken whole.  Every thread of the block calls it.

struct SelScratch {
  uint32_t hist[256];
  unsigned long long kmin, kmax;
  int digit, above;
};

template <int NT, class ForEach>
__device__ uint64_t block_select(ForEach for_each, int need, SelScratch &sh) {
  const int tid = threadIdx.x, l = lane_id();
  if (tid == 0) { sh.kmin = ~0ull; sh.kmax = 0ull; }
  __syncthreads();
  unsigned long long lmin = ~0ull, lmax = 0ull;
  for_each([&](uint64_t key) {
    lmin = key < lmin ? key : lmin;
    lmax = key > lmax ? key : lmax;
  });
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    unsigned long long a = __shfl_xor(lmin, off), b = __shfl_xor(lmax, off);
    lmin = a < lmin ? a : lmin;
    lmax = b > lmax ? b : lmax;
  }
  if (l == 0) { atomicMin(&sh.kmin, lmin); atomicMax(&sh.kmax, lmax); }
  __syncthreads();
  const uint64_t kmin = sh.kmin, kmax = sh.kmax;
  if (kmin == kmax) return kmin;
  const int hb = 63 - __clzll((long long)(kmin ^ kmax));   // highest bit in which keys differ
  int fixed = hb + 1;                                        // bits >= fixed are common to all keys
  int shift = fixed >= 8 ? fixed - 8 : 0;
  uint64_t hi_mask = fixed >= 64 ? 0ull : ~((1ull << fixed) - 1);
  uint64_t prefix = kmin & hi_mask;
  int need_rem = need;
  for (;;) {
    for (int i = tid; i < 256; i += NT) sh.hist[i] = 0u;
    if (tid == 0) { sh.digit = 0; sh.above = 0; }
    __syncthreads();
    const uint64_t m = hi_mask, p = prefix;
    const int s = shift;
    for_each([&](uint64_t key) {
      // Keys cluster in a few buckets (scores are concentrated), and same-address LDS atomics of one
      // wave serialise: the lanes of up to 4 buckets that at least 4 active lanes share add with one
      // atomic per bucket, the rest one each.  Every key is counted once.
      const bool in = (key & m) == p;
      const uint32_t bin = (uint32_t)(key >> s) & 255u;
      bool mine = in;
      uint64_t act = __ballot(mine);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        if (act == 0ull) break;
        const int leader = __ffsll((long long)act) - 1;
        const uint32_t b0 = __shfl(bin, leader);
        const uint64_t same = __ballot(mine && bin == b0);
        if (__popcll(same) < 4) break;
        if (l == leader) atomicAdd(&sh.hist[b0], (uint32_t)__popcll(same));
        if (mine && bin == b0) mine = false;
        act &= ~same;
      }
      if (mine) atomicAdd(&sh.hist[bin], 1u);
    });
    __syncthreads();
    if (tid < 64) {
      uint32_t h0 = sh.hist[4 * l], h1 = sh.hist[4 * l + 1], h2 = sh.hist[4 * l + 2], h3 = sh.hist[4 * l + 3];
      uint32_t sum = h0 + h1 + h2 + h3, suf = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        uint32_t u = __shfl_down(suf, off);
        if (l + off < 64) suf += u;
      }
      uint32_t above = suf - sum;   // keys in buckets above 4l+3
      const uint32_t nr = (uint32_t)need_rem;
      uint32_t hh[4] = {h0, h1, h2, h3};
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < nr && above + hh[j] >= nr) { sh.digit = 4 * l + j; sh.above = (int)above; }
        above += hh[j];
      }
    }
    __syncthreads();
    const int d = sh.digit;
    const int hd = (int)sh.hist[d];
    need_rem -= sh.above;
    prefix |= (uint64_t)d << shift;
    if (hd == need_rem || shift == 0) break;
    fixed = shift;
    hi_mask = ~((1ull << fixed) - 1);
    prefix &= hi_mask;
    shift = fixed >= 8 ? fixed - 8 : 0;
    __syncthreads();
  }
  __syncthreads();
  return prefix;
}

// A bijection of [0, n) that scatters consecutive positions over the whole range: a permutation of
// [0, 2^m) (odd multiplications and an xor-shift, each invertible modulo 2^m), walked until it lands
// below n; the walk ends because every cycle of the permutation holds a position below n (the start).
__device__ __forceinline__ int scatter_index(int pos, int n) {
  const int m = n > 1 ? 32 - __clz(n - 1) : 1;   // 2^m >= n
  const uint32_t mask = m >= 32 ? 0xFFFFFFFFu : ((1u << m) - 1u);
  uint32_t x = (uint32_t)pos;
  do {
    x = (x * 0x9E3779B1u) & mask;
    x ^= x >> ((m >> 1) + 1);
    x = (x * 0x85EBCA77u) & mask;
  } while (x >= (uint32_t)n);
  return (int)x;
}

// Keys held while items are being scanned: (biased score << 32) | position.  They order candidates by
// score like the ordering keys; they are turned into (score, id) keys (make_key) only for the few
// candidates that can still reach a final top k, so the scan never waits on the position -> id table.
__device__ __forceinline__ uint64_t pos_key(int32_t score, int32_t pos) {
  return ((uint64_t)((uint32_t)score ^ 0x80000000u) << 32) | (uint64_t)(uint32_t)pos;
}

// The n best ordering keys of a query, cand[0..n) in LDS (room for 4 NT keys), sorted best first and
// written as row q: ids, int32 scores and scores dequantised as S / (item_scale * query_scale) in double,
// rounded once to float.  Entries nout..k-1 are padding.  All NT threads of the block call it;
// nout <= n <= k <= 2 NT.
// The sort is a bitonic network over 2 NT keys (missing keys are 0, below every real key), two per
// thread (elements 2t and 2t + 1): strides up to 64 pair lanes of one wave and run on shuffles, larger
// strides exchange through LDS, alternating between two halves of cand: a thread reads its partner's
// keys after one barrier, and the next exchange writes the other half, so no second barrier is needed
// (the exchange after that one, which reuses this half, comes after the next exchange's barrier).
template <int NT>
__device__ void emit_sorted(uint64_t *cand, int n, int nout, int q, int k, const float *query_scales,
                            float item_scale, int64_t *out_ids, int32_t *out_scores, float *out_fscores) {
  constexpr int N = 2 * NT;
  const int tid = threadIdx.x;
  uint64_t v[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) v[e] = 2 * tid + e < n ? cand[2 * tid + e] : 0ull;
  __syncthreads();
  int half = 0;   // the half of cand the next exchange writes
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const bool desc = ((2 * tid) & size) == 0;   // the run holding this thread's elements sorts descending
      if (stride == 1) {
        const bool sw = desc ? v[0] < v[1] : v[0] > v[1];
        if (sw) { const uint64_t x = v[0]; v[0] = v[1]; v[1] = x; }
        continue;
      }
      uint64_t p[2];
      const int h = stride >> 1;   // partner thread: tid ^ h
      if (stride <= 64) {
#pragma unroll
        for (int e = 0; e < 2; ++e) p[e] = __shfl_xor(v[e], h);
      } else {
        uint64_t *x = cand + half * N;
#pragma unroll
        for (int e = 0; e < 2; ++e) x[2 * tid + e] = v[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 2; ++e) p[e] = x[2 * (tid ^ h) + e];
        half ^= 1;
      }
      const bool lower = (tid & h) == 0;   // this thread holds the lower index of each pair
      const bool keep_max = lower == desc;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint64_t a = v[e], b = p[e];
        v[e] = keep_max ? (a > b ? a : b) : (a < b ? a : b);
      }
    }
  }
  const float qs = query_scales ? query_scales[q] : item_scale;
  const double denom = (double)item_scale * (double)qs;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = 2 * tid + e;
    if (i < k) {
      const size_t o = (size_t)q * k + i;
      if (i < nout) {
        const int32_t sc = key_score(v[e]);
        out_ids[o] = (int64_t)key_id(v[e]);
        out_scores[o] = sc;
        if (out_fscores) out_fscores[o] = (float)((double)sc / denom);
      } else {
        out_ids[o] = -1;
        out_scores[o] = INT32_MIN;
        if (out_fscores) out_fscores[o] = -__builtin_huge_valf();
      }
    }
  }
}

}  // namespace svt
