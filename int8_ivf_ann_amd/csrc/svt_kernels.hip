// svt_kernels.hip - gfx950 kernels of the fused int8 IVF + Bloom-signature top-k search.
//
// Pipeline per svt_search (all on the caller's stream, no host synchronisation):
//   k_coarse_keys   int8 centroid scores for every (query, cluster), packed as (score, cluster) keys
//   k_coarse_select per query: exact top-nprobe clusters (radix select), probe list in cluster order,
//                   per-query item stream layout; the last workgroup lays out the batch stream
//   k_scan          the fused hot loop: Bloom filter -> int8 dot4 score -> per-workgroup top-k in LDS;
//                   a fixed grid of workgroups splits the concatenated (query, probed item) stream
//                   into equal contiguous chunks; each (workgroup, query) run leaves at most k keys
//   k_merge         per query: exact top-k over its runs' keys (radix select), sorted, written out
//
// Method: "SilverTorch - Index as Model" (Meta engineering post): probe the most promising clusters
// first, filter only inside them with Bloom signatures and bit operations, score only survivors
// with int8 dot products (int32 accumulation, "dp4a"), return a large top-k; "Meta Andromeda"
// summary, System section: per-item intermediates stay in registers and shared memory, only the
// final candidates leave the machine.  The kernel shapes below are designed for CDNA4 (64-wide
// waves, v_dot4 on the VALU, LDS radix selection), not taken from the pages.
//
// Ordering key: ((score ^ 0x80000000) << 32) | (0xFFFFFFFF - id).  Larger key = better: higher score,
// then lower id.  Keys of one query are distinct because item ids are distinct.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svt_internal.h"

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

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// number of set bits of `mask` below this lane
__device__ __forceinline__ int mbcnt(uint64_t mask) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// items per contiguous chunk of the batch stream, shared by k_scan and k_merge
__device__ __forceinline__ int64_t stream_chunk(int64_t L, int32_t P) {
  int64_t c = (L + P - 1) / P;
  return ((c + 63) / 64) * 64;
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
      if ((key & m) == p) atomicAdd(&sh.hist[(key >> s) & 255u], 1u);
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

// ------------------------------------------------------------------------------------------------
// k_coarse_keys: key (s, c) for every query b and cluster c, s = <q_b, centroid_c> (int32).
// One thread per cluster, kCoarseQB queries per workgroup staged in LDS.

template <int LPR>
__global__ __launch_bounds__(256) void k_coarse_keys(const int8_t *__restrict__ centroids, int32_t nlist,
                                                     const int8_t *__restrict__ queries, int32_t B,
                                                     uint64_t *__restrict__ keys, uint32_t *counter) {
  constexpr int D = 16 * LPR;
  __shared__ int4 qs[kCoarseQB][LPR];
  const int tid = threadIdx.x;
  const int b0 = blockIdx.y * kCoarseQB;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) *counter = 0u;
  for (int i = tid; i < kCoarseQB * LPR; i += 256) {
    int qi = i / LPR, ch = i % LPR;
    int b = b0 + qi;
    qs[qi][ch] = b < B ? reinterpret_cast<const int4 *>(queries + (size_t)b * D)[ch] : make_int4(0, 0, 0, 0);
  }
  __syncthreads();
  const int c = blockIdx.x * 256 + tid;
  if (c >= nlist) return;
  int4 row[LPR];
  const int4 *src = reinterpret_cast<const int4 *>(centroids + (size_t)c * D);
#pragma unroll
  for (int ch = 0; ch < LPR; ++ch) row[ch] = src[ch];
#pragma unroll
  for (int qi = 0; qi < kCoarseQB; ++qi) {
    const int b = b0 + qi;
    if (b >= B) break;
    int32_t acc = 0;
#pragma unroll
    for (int ch = 0; ch < LPR; ++ch) acc = dot16(row[ch], qs[qi][ch], acc);
    keys[(size_t)b * nlist + c] = make_key(acc, (uint32_t)c);
  }
}

// ------------------------------------------------------------------------------------------------
// k_coarse_select: one workgroup per query.
//   probes[b][0..nprobe): the nprobe clusters with the largest keys, in ascending cluster id
//   seg[b][j]: offset of probed cluster j in query b's item stream; seg[b][nprobe] = qlen[b]
// The last workgroup to finish turns qlen into the batch stream prefix qstart[0..B].

__global__ __launch_bounds__(kSelThreads) void k_coarse_select(const int32_t *__restrict__ offsets, int32_t nlist,
                                                                int32_t B, int32_t nprobe, Work w) {
  __shared__ SelScratch sel;
  __shared__ int wave_tot[kSelThreads / 64 + 1];
  __shared__ int64_t wave_tot64[kSelThreads / 64 + 1];
  __shared__ int last;
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const uint64_t *row = w.coarse_keys + (size_t)b * nlist;
  uint64_t T = 0;
  if (nprobe < nlist) {
    T = block_select<kSelThreads>(
        [&](auto f) {
          for (int c = tid; c < nlist; c += kSelThreads) f(row[c]);
        },
        nprobe, sel);
  }
  int32_t *probes = w.probes + (size_t)b * nprobe;
  int32_t *seg = w.seg + (size_t)b * (nprobe + 1);
  int base = 0, run = 0;
  for (int c0 = 0; c0 < nlist; c0 += kSelThreads) {
    const int c = c0 + tid;
    const bool take = c < nlist && row[c] >= T;
    const int sz = take ? offsets[c + 1] - offsets[c] : 0;
    int cnt_tot, sz_tot;
    const int idx = block_excl_scan<kSelThreads>(take ? 1 : 0, wave_tot, &cnt_tot);
    const int pre = block_excl_scan<kSelThreads>(sz, wave_tot, &sz_tot);
    if (take && base + idx < nprobe) {
      probes[base + idx] = c;
      seg[base + idx] = run + pre;
    }
    base += cnt_tot;
    run += sz_tot;
  }
  if (tid == 0) {
    seg[nprobe] = run;
    w.qlen[b] = run;
    w.thr[b] = INT32_MIN;
    if (w.stats) { w.stats[2 * (size_t)b] = 0; w.stats[2 * (size_t)b + 1] = 0; }
  }
  // last workgroup: exclusive prefix of qlen over the batch
  __threadfence();
  __syncthreads();
  if (tid == 0) last = (atomicAdd(w.counter, 1u) == (uint32_t)(B - 1)) ? 1 : 0;
  __syncthreads();
  if (!last) return;
  __threadfence();
  int64_t carry = 0;
  for (int i0 = 0; i0 < B; i0 += kSelThreads) {
    const int i = i0 + tid;
    const int64_t v = i < B ? __hip_atomic_load(&w.qlen[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0;
    int64_t tot;
    const int64_t ex = block_excl_scan<kSelThreads>(v, wave_tot64, &tot);
    if (i < B) w.qstart[i] = carry + ex;
    carry += tot;
  }
  if (tid == 0) w.qstart[B] = carry;
}

// ------------------------------------------------------------------------------------------------
// k_scan: the fused filter -> score -> select hot loop.
//
// The batch stream is the concatenation over queries of the items of each query's probed clusters
// (qstart, seg).  Workgroup g owns stream positions [g*chunk, (g+1)*chunk) and walks them in order.
// For each 64-item group a wave loads the 64 signatures with one 128-bit (or 64-bit) load per lane,
// tests (sig & mask) == mask, ballots the result and compacts the survivors into an LDS list; rows of
// survivors only are then fetched, LPR lanes per row with 16-byte loads, and scored with v_dot4.
// A candidate enters the workgroup's LDS list if it beats both the list's own k-th key and the
// query's global bound thr[q]; whenever the list exceeds k keys it is cut back to exactly k by an
// LDS radix select.  When the workgroup leaves a query it writes its <= k keys to slot (g + q).
// Nothing per item is ever written to HBM.

struct ScanArgs {
  DevIndex ix;
  const int8_t *queries;
  const uint64_t *masks;
  Work w;
  int32_t B, nprobe, k, P;
};

struct ScanLds {
  uint64_t list[kListCap];
  uint16_t wl[kScanThreads / 64][64 * kScanGroups];
  SelScratch sel;
  int wave_tot[kScanThreads / 64 + 1];
  unsigned long long kmin;
  int cnt;
};

template <int LPR, int W>
__global__ __launch_bounds__(kScanThreads) void k_scan(ScanArgs a) {
  constexpr int D = 16 * LPR;
  constexpr int RPI = 64 / LPR;                          // rows scored per wave iteration
  constexpr int R = (32 / RPI) > 0 ? (32 / RPI) : 1;     // iterations issued together
  __shared__ ScanLds sm;
  const int tid = threadIdx.x, l = lane_id(), wv = tid / 64, sub = l % LPR;
  const int g = blockIdx.x;
  const int64_t *qstart = a.w.qstart;
  const int64_t L = qstart[a.B];
  const int64_t chunk = stream_chunk(L, a.P);
  const int64_t beg = (int64_t)g * chunk;
  const int64_t end = beg + chunk < L ? beg + chunk : L;
  if (beg >= end) return;
  // first query whose stream range contains beg: largest q with qstart[q] <= beg
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (qstart[mid] <= beg) lo = mid; else hi = mid - 1;
  }
  for (int q = lo; q < a.B && qstart[q] < end; ++q) {
    const int64_t q0 = qstart[q], q1 = qstart[q + 1];
    const int32_t ra = (int32_t)((beg > q0 ? beg : q0) - q0);
    const int32_t rb = (int32_t)((end < q1 ? end : q1) - q0);
    if (ra >= rb) continue;
    // query vector slice held by this lane, request mask
    const int4 qv = reinterpret_cast<const int4 *>(a.queries + (size_t)q * D)[sub];
    uint64_t mk[W];
#pragma unroll
    for (int i = 0; i < W; ++i) mk[i] = a.masks[(size_t)q * W + i];
    if (tid == 0) sm.cnt = 0;
    uint64_t thr_key = 0;            // list's k-th key once the list has been cut (0: none)
    int32_t thr_score = INT32_MIN;
    int64_t n_elig = 0;
    const int32_t *seg = a.w.seg + (size_t)q * (a.nprobe + 1);
    const int32_t *probes = a.w.probes + (size_t)q * a.nprobe;
    // first probed cluster overlapping [ra, rb): largest j with seg[j] <= ra
    int jl = 0, jh = a.nprobe - 1;
    while (jl < jh) {
      int mid = (jl + jh + 1) >> 1;
      if (seg[mid] <= ra) jl = mid; else jh = mid - 1;
    }
    __syncthreads();
    for (int j = jl; j < a.nprobe; ++j) {
      const int32_t s0 = seg[j], s1 = seg[j + 1];
      if (s0 >= rb) break;
      const int32_t t0 = ra > s0 ? ra : s0, t1 = rb < s1 ? rb : s1;
      if (t0 >= t1) continue;
      const int64_t pbase = (int64_t)a.ix.offsets[probes[j]] - s0;   // position = pbase + stream offset
      for (int32_t st = t0; st < t1; st += kScanStep) {
        const int32_t n = (t1 - st) < kScanStep ? (t1 - st) : kScanStep;
        const int64_t p0 = pbase + st;
        const int32_t gthr = __hip_atomic_load(&a.w.thr[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int32_t thr_eff = gthr > thr_score ? gthr : thr_score;
        // --- filter: signatures of kScanGroups x 64 items per wave
        uint64_t sg[kScanGroups][W];
#pragma unroll
        for (int gi = 0; gi < kScanGroups; ++gi) {
          const int i = gi * kScanThreads + wv * 64 + l;
          if (i < n) {
            if constexpr (W == 2) {
              const ulonglong2 v = reinterpret_cast<const ulonglong2 *>(a.ix.sigs)[p0 + i];
              sg[gi][0] = v.x; sg[gi][1] = v.y;
            } else {
              sg[gi][0] = a.ix.sigs[p0 + i];
            }
          } else {
#pragma unroll
            for (int u = 0; u < W; ++u) sg[gi][u] = 0;
          }
        }
        int nw = 0;
#pragma unroll
        for (int gi = 0; gi < kScanGroups; ++gi) {
          const int i = gi * kScanThreads + wv * 64 + l;
          bool pass = i < n;
#pragma unroll
          for (int u = 0; u < W; ++u) pass = pass && ((sg[gi][u] & mk[u]) == mk[u]);
          const uint64_t bal = __ballot(pass);
          if (pass) sm.wl[wv][nw + mbcnt(bal)] = (uint16_t)i;
          nw += __popcll(bal);
        }
        n_elig += nw;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // --- score the survivors: LPR lanes per row, R x RPI rows in flight per wave
        for (int r0 = 0; r0 < nw; r0 += RPI * R) {
          int4 x[R];
          int64_t pos[R];
          bool v[R];
#pragma unroll
          for (int u = 0; u < R; ++u) {
            const int r = r0 + u * RPI + l / LPR;
            v[u] = r < nw;
            const int i = v[u] ? (int)sm.wl[wv][r] : 0;
            pos[u] = p0 + i;
            x[u] = v[u] ? reinterpret_cast<const int4 *>(a.ix.items + (size_t)pos[u] * D)[sub] : make_int4(0, 0, 0, 0);
          }
#pragma unroll
          for (int u = 0; u < R; ++u) {
            int32_t acc = dot16(x[u], qv, 0);
#pragma unroll
            for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
            if (sub == 0 && v[u] && acc >= thr_eff) {
              const uint64_t key = make_key(acc, (uint32_t)a.ix.perm[pos[u]]);
              if (key > thr_key) {
                const int slot = atomicAdd(&sm.cnt, 1);
                sm.list[slot] = key;
              }
            }
          }
        }
        __syncthreads();
        // --- keep the list at most k keys: cut to exactly k, raise the local and global bounds
        if (sm.cnt > a.k) {
          const int cnt = sm.cnt;
          const uint64_t T = block_select<kScanThreads>(
              [&](auto f) {
                for (int i = tid; i < cnt; i += kScanThreads) f(sm.list[i]);
              },
              a.k, sm.sel);
          constexpr int PER = kListCap / kScanThreads;
          uint64_t mine[PER];
          int keep = 0;
#pragma unroll
          for (int u = 0; u < PER; ++u) {
            const int i = tid + u * kScanThreads;
            mine[u] = i < cnt ? sm.list[i] : 0ull;
            keep += (i < cnt && mine[u] >= T) ? 1 : 0;
          }
          if (tid == 0) sm.kmin = ~0ull;
          int tot;
          int off = block_excl_scan<kScanThreads>(keep, sm.wave_tot, &tot);
          unsigned long long mn = ~0ull;
#pragma unroll
          for (int u = 0; u < PER; ++u) {
            const int i = tid + u * kScanThreads;
            if (i < cnt && mine[u] >= T) {
              sm.list[off++] = mine[u];
              mn = mine[u] < mn ? mine[u] : mn;
            }
          }
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) {
            unsigned long long t = __shfl_xor(mn, o);
            mn = t < mn ? t : mn;
          }
          if (l == 0) atomicMin(&sm.kmin, mn);
          __syncthreads();
          thr_key = sm.kmin;
          thr_score = key_score(thr_key);
          if (tid == 0) {
            sm.cnt = tot;
            atomicMax(&a.w.thr[q], thr_score);
          }
          __syncthreads();
        }
      }
    }
    // --- leave the query: publish this run's keys in slot (g + q)
    const int cnt = sm.cnt;
    const size_t slot = (size_t)g + (size_t)q;
    uint64_t *dst = a.w.slot_keys + slot * (size_t)a.k;
    for (int i = tid; i < cnt; i += kScanThreads) dst[i] = sm.list[i];
    if (tid == 0) a.w.slot_cnt[slot] = cnt;
    // per-query counters: items scanned by this run, items that passed the filter
    if (a.w.stats) {
      // n_elig is uniform across the wave: one add per wave
      if (l == 0) atomicAdd((unsigned long long *)&a.w.stats[2 * (size_t)q + 1], (unsigned long long)n_elig);
      if (tid == 0) atomicAdd((unsigned long long *)&a.w.stats[2 * (size_t)q], (unsigned long long)(rb - ra));
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// k_merge: one workgroup per query.  Exact top-k over the keys its (workgroup, query) runs left,
// bitonic sort in LDS, decode, dequantise, write.

struct MergeArgs {
  Work w;
  const float *query_scales;
  float item_scale;
  int32_t B, k, P;
  int64_t *out_ids;
  int32_t *out_scores;
  float *out_fscores;
  int32_t *out_counts;
};

__global__ __launch_bounds__(kSelThreads) void k_merge(MergeArgs a) {
  __shared__ SelScratch sel;
  __shared__ uint64_t buf[kMaxK];
  __shared__ int scnt[kMaxScanWGs + 1];
  __shared__ int wave_tot[kSelThreads / 64 + 1];
  __shared__ int nbuf;
  const int tid = threadIdx.x, l = lane_id(), wv = tid / 64;
  constexpr int NW = kSelThreads / 64;
  const int q = blockIdx.x;
  const int k = a.k;
  const int64_t q0 = a.w.qstart[q], q1 = a.w.qstart[q + 1];
  int total = 0, ns = 0;
  size_t s0 = 0;
  if (q1 > q0) {
    const int64_t chunk = stream_chunk(a.w.qstart[a.B], a.P);
    const int64_t g0 = q0 / chunk, g1 = (q1 - 1) / chunk;
    s0 = (size_t)g0 + (size_t)q;
    ns = (int)(g1 - g0 + 1);
    int part = 0;
    for (int i = tid; i < ns; i += kSelThreads) {
      const int c = a.w.slot_cnt[s0 + i];
      scnt[i] = c;
      part += c;
    }
    block_excl_scan<kSelThreads>(part, wave_tot, &total);
  }
  const uint64_t *keys = a.w.slot_keys;
  auto visit = [&](auto f) {
    for (int s = wv; s < ns; s += NW) {
      const uint64_t *src = keys + (s0 + (size_t)s) * (size_t)k;
      const int c = scnt[s];
      for (int i = l; i < c; i += 64) f(src[i]);
    }
  };
  const int nout = total < k ? total : k;
  uint64_t T = 0;
  if (total > k) T = block_select<kSelThreads>(visit, k, sel);
  if (tid == 0) nbuf = 0;
  __syncthreads();
  if (nout > 0) {
    visit([&](uint64_t key) {
      if (key >= T) {
        const int o = atomicAdd(&nbuf, 1);
        if (o < kMaxK) buf[o] = key;
      }
    });
  }
  __syncthreads();
  // bitonic sort, descending, over the next power of two (padding keys 0 sort last)
  int np2 = 1;
  while (np2 < nout) np2 <<= 1;
  for (int i = nout + tid; i < np2; i += kSelThreads) buf[i] = 0ull;
  __syncthreads();
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < np2; i += kSelThreads) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t x = buf[i], y = buf[j];
          const bool up = (i & size) == 0;   // this run sorts descending
          if (up ? (x < y) : (x > y)) { buf[i] = y; buf[j] = x; }
        }
      }
      __syncthreads();
    }
  }
  const float qs = a.query_scales ? a.query_scales[q] : a.item_scale;
  const double denom = (double)a.item_scale * (double)qs;
  for (int i = tid; i < k; i += kSelThreads) {
    const size_t o = (size_t)q * k + i;
    if (i < nout) {
      const uint64_t key = buf[i];
      const int32_t sc = key_score(key);
      a.out_ids[o] = (int64_t)key_id(key);
      a.out_scores[o] = sc;
      if (a.out_fscores) a.out_fscores[o] = (float)((double)sc / denom);
    } else {
      a.out_ids[o] = -1;
      a.out_scores[o] = INT32_MIN;
      if (a.out_fscores) a.out_fscores[o] = -__builtin_huge_valf();
    }
  }
  if (tid == 0 && a.out_counts) a.out_counts[q] = nout;
}

// ------------------------------------------------------------------------------------------------
// upload: scatter caller rows [i0, i0+n) to their cluster-contiguous positions

__global__ __launch_bounds__(256) void k_scatter_rows(const int8_t *__restrict__ src_rows,
                                                      const uint64_t *__restrict__ src_sigs,
                                                      const int32_t *__restrict__ pos_of, int64_t i0, int64_t n,
                                                      int32_t chunks, int32_t sig_words, int8_t *__restrict__ dst_rows,
                                                      uint64_t *__restrict__ dst_sigs) {
  // one thread per 16-byte chunk of a row
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t r = t / chunks;
  const int c = (int)(t % chunks);
  if (r >= n) return;
  const int64_t p = pos_of[i0 + r];
  reinterpret_cast<int4 *>(dst_rows)[p * chunks + c] = reinterpret_cast<const int4 *>(src_rows)[r * chunks + c];
  for (int u = c; u < sig_words; u += chunks) dst_sigs[p * sig_words + u] = src_sigs[r * sig_words + u];
}

// ------------------------------------------------------------------------------------------------
// launch wrappers

hipError_t launch_coarse_keys(const DevIndex &ix, const int8_t *queries, int32_t B, const Work &w, hipStream_t s) {
  dim3 grid((ix.nlist + 255) / 256, (B + kCoarseQB - 1) / kCoarseQB);
  switch (ix.dim) {
    case 16: k_coarse_keys<1><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_keys, w.counter); break;
    case 32: k_coarse_keys<2><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_keys, w.counter); break;
    case 64: k_coarse_keys<4><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_keys, w.counter); break;
    case 128: k_coarse_keys<8><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_keys, w.counter); break;
    case 256: k_coarse_keys<16><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_keys, w.counter); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_coarse_select(const DevIndex &ix, const SearchShape &sh, const Work &w, hipStream_t s) {
  k_coarse_select<<<sh.B, kSelThreads, 0, s>>>(ix.offsets, ix.nlist, sh.B, sh.nprobe, w);
  return hipGetLastError();
}

template <int LPR>
static void scan_w(const ScanArgs &a, int W, hipStream_t s) {
  if (W == 2)
    k_scan<LPR, 2><<<a.P, kScanThreads, 0, s>>>(a);
  else
    k_scan<LPR, 1><<<a.P, kScanThreads, 0, s>>>(a);
}

hipError_t launch_scan(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const SearchShape &sh,
                       const Work &w, hipStream_t s) {
  ScanArgs a{ix, queries, masks, w, sh.B, sh.nprobe, sh.k, sh.P};
  switch (ix.dim) {
    case 16: scan_w<1>(a, ix.sig_words, s); break;
    case 32: scan_w<2>(a, ix.sig_words, s); break;
    case 64: scan_w<4>(a, ix.sig_words, s); break;
    case 128: scan_w<8>(a, ix.sig_words, s); break;
    case 256: scan_w<16>(a, ix.sig_words, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const DevIndex &ix, const float *query_scales, const SearchShape &sh, const Work &w,
                        int64_t *out_ids, int32_t *out_scores, float *out_fscores, int32_t *out_counts,
                        hipStream_t s) {
  MergeArgs a{w, query_scales, ix.item_scale, sh.B, sh.k, sh.P, out_ids, out_scores, out_fscores, out_counts};
  k_merge<<<sh.B, kSelThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const int8_t *src_rows, const uint64_t *src_sigs, const int32_t *pos_of, int64_t i0,
                               int64_t n, int32_t dim, int32_t sig_words, int8_t *dst_rows, uint64_t *dst_sigs,
                               hipStream_t s) {
  const int chunks = dim / 16;
  const int64_t threads = n * chunks;
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0)
    k_scatter_rows<<<(unsigned)blocks, 256, 0, s>>>(src_rows, src_sigs, pos_of, i0, n, chunks, sig_words, dst_rows,
                                                    dst_sigs);
  return hipGetLastError();
}

}  // namespace svt
