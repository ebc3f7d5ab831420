// svt_largek.hip - searches with k above the fused lists' SVT_MAX_K: an exact top-k by a radix select
// over the eligible items' keys, one digit per pass over the probed clusters, then one pass that keeps
// the k keys at or above the threshold and a sort of those in LDS.
//
// Source: "SilverTorch - Index as Model" (Meta engineering post), the fused Int8 ANN paragraph and the
// compute-cost table: the retrieval kernel supports top-k far beyond the 2048 of GPU FAISS (the
// Spanish page's table row reads "100de miles", taken as hundreds of thousands); the probe, filter and
// score steps are those of the fused search.
//
// Key of an eligible item: (S + 2^23) << 31 | (2^31 - 1 - id), 55 bits.  Its unsigned order is the
// result order, score descending then id ascending, and no key is 0.  The digits are 11 bits wide, from
// bit 44 down: a pass counts, per query, the keys that share the bits fixed so far by their next digit
// (an LDS histogram per workgroup, added to the query's histogram in HBM); k_lk_pick then fixes that
// digit, and a query is done once the digit's bucket is taken whole.  At most 5 passes, usually 2 or 3;
// a pass skips the queries already done.  The collect pass appends every key at or above the
// threshold (exactly min(k, eligible) keys, as keys are distinct) and k_lk_emit sorts them.
//
// Pool mode (when the workspace has room): the coarse stage sets each query's speculative threshold from
// its samples, at the score about 2k eligible items reach, and one scan appends every eligible key at or
// above it to the query's pool (8k keys).  A pool that did not overflow and holds at least k keys (or was
// filled without a threshold) holds the query's top k: k_lk_pool selects them there.  Only the other
// queries run the passes above, each of which reads the query's probed items again.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svt.h"
#include "svt_device.h"
#include "svt_internal.h"

namespace svt {

namespace {

constexpr int kLkThreads = 256;
constexpr int kLkEmitThreads = 1024;

__device__ __forceinline__ uint64_t lk_key(int32_t s, int32_t id) {
  return ((uint64_t)(uint32_t)(s + (1 << 23)) << 31) | (uint64_t)(0x7FFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int32_t lk_score(uint64_t key) { return (int32_t)(key >> 31) - (1 << 23); }
__device__ __forceinline__ int64_t lk_id(uint64_t key) { return (int64_t)(0x7FFFFFFFu - (uint32_t)(key & 0x7FFFFFFFu)); }

__global__ void k_lk_init(int32_t B, int32_t k, Work w) {
  const int64_t n = (int64_t)B * kLkBins;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    w.lk_hist[i] = 0u;
    if (i < B) {
      w.lk_state[i] = LkState{0ull, kLkTopShift, k, 0, 0};
      w.lk_cnt[i] = 0u;
    }
  }
}

struct LkScanArgs {
  DevIndex ix;
  const int8_t *queries;
  const uint64_t *masks;
  Work w;
  int32_t B, nprobe, k, G;
  uint32_t pool_cap;   // pool keys per query (0: no pool mode)
};

enum { kLkCount = 0, kLkCollect = 1, kLkPool = 2 };

// The batch's chunks: query b's stream is cut into ceil(qlen / kLkChunk) chunks, numbered from
// lk_cstart[b]; lk_cstart[B] is their total.  One workgroup.
__global__ __launch_bounds__(1024) void k_lk_chunks(int32_t B, Work w) {
  __shared__ int wave_tot[1024 / 64 + 1];
  int base = 0;
  for (int b0 = 0; b0 < B; b0 += 1024) {
    const int b = b0 + (int)threadIdx.x;
    const int c = b < B ? (int)((w.qlen[b] + kLkChunk - 1) / kLkChunk) : 0;
    int tot;
    const int ex = block_excl_scan<1024>(c, wave_tot, &tot);   // barriers inside
    if (b < B) w.lk_cstart[b] = base + ex;
    base += tot;
  }
  if (threadIdx.x == 0) w.lk_cstart[B] = base;
}

// kLkScanWGs workgroups walk the batch's chunks.  MODE kLkCount: a counting pass (queries still
// selecting); kLkCollect: append the keys at or above the threshold (queries decided by the passes);
// kLkPool: append the keys whose score reaches the speculative threshold to the pool, and count the
// eligible items (every query).  Each thread takes 2 items a step, their signature loads and then their
// row loads issued together; appended keys are staged in LDS and written with one reservation per chunk.
template <int D, int W, int MODE>
__global__ __launch_bounds__(kLkThreads) void k_lk_scan(LkScanArgs a) {
  constexpr bool COLLECT = MODE != kLkCount;
  constexpr int IT = 2;                      // items per thread and step
  constexpr int STEP = IT * kLkThreads;
  __shared__ uint32_t hist[COLLECT ? 1 : kLkBins];   // zero between chunks: each flush clears its bins
  __shared__ uint64_t stage[COLLECT ? kLkChunk : 1];  // a chunk's appended keys
  __shared__ uint32_t stage_n, stage_base;
  const int tid = threadIdx.x, l = lane_id();
  const int32_t n_chunks = a.w.lk_cstart[a.B];
  if (!COLLECT)
    for (int i = tid; i < kLkBins; i += kLkThreads) hist[i] = 0u;
  if (tid == 0) stage_n = 0u;
  __syncthreads();
  for (int t = blockIdx.x; t < n_chunks; t += gridDim.x) {
    // the chunk's query: the largest b with lk_cstart[b] <= t
    int qb = 0, qe = a.B - 1;
    while (qb < qe) {
      const int mid = (qb + qe + 1) >> 1;
      if (a.w.lk_cstart[mid] <= t) qb = mid; else qe = mid - 1;
    }
    const int b = qb;
    const LkState st = a.w.lk_state[b];
    if (MODE == kLkCount && st.done) continue;
    if (MODE == kLkCollect && st.done != kLkDone) continue;
    const int64_t qlen = a.w.qlen[b];
    const int64_t s0 = (int64_t)(t - a.w.lk_cstart[b]) * kLkChunk;
    const int64_t s1 = s0 + kLkChunk < qlen ? s0 + kLkChunk : qlen;
    int my_elig = 0;
    const int32_t sthr = MODE == kLkPool ? a.w.sthr[b] : 0;
    // the query row and masks in registers
    int4 qv[D / 16];
    const int4 *qr = reinterpret_cast<const int4 *>(a.queries + (size_t)b * D);
#pragma unroll
    for (int i = 0; i < D / 16; ++i) qv[i] = qr[i];
    uint64_t mk[kMaxGroups][W];
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g)
#pragma unroll
      for (int x = 0; x < W; ++x) mk[g][x] = g < a.G ? a.masks[((size_t)b * a.G + g) * W + x] : 0ull;
    // keys counted: those whose bits above the digit equal the prefix; kept: those >= the threshold
    const int shift = st.shift;
    const uint64_t hi = ~((1ull << (shift + kLkDigit)) - 1ull);
    const uint64_t prefix = st.prefix;
    const int32_t *seg = a.w.seg + (size_t)b * (a.nprobe + 1);
    const int32_t *pb = a.w.pb + (size_t)b * a.nprobe;
    // the probed cluster holding stream position s0: the largest r with seg[r] <= s0
    int lo = 0, up = a.nprobe - 1;
    while (lo < up) {
      const int mid = (lo + up + 1) >> 1;
      if (seg[mid] <= s0) lo = mid; else up = mid - 1;
    }
    for (int r = lo; r < a.nprobe; ++r) {
      const int64_t r0 = seg[r], r1 = seg[r + 1];
      if (r0 >= s1) break;
      const int64_t e0 = r0 > s0 ? r0 : s0, e1 = r1 < s1 ? r1 : s1;
      const int32_t base = pb[r];
      for (int64_t sb = e0; sb < e1; sb += STEP) {   // uniform trip count: ballots see every lane
        uint64_t sg[IT][2];
        bool ok[IT];
#pragma unroll
        for (int u = 0; u < IT; ++u) {
          const int64_t s = sb + u * kLkThreads + tid;
          sg[u][0] = sg[u][1] = 0ull;
          if (s < e1)
#pragma unroll
            for (int x = 0; x < W; ++x) sg[u][x] = a.ix.sigs[(base + s) * W + x];
        }
#pragma unroll
        for (int u = 0; u < IT; ++u) {
          const int64_t s = sb + u * kLkThreads + tid;
          bool any = false;
#pragma unroll
          for (int g = 0; g < kMaxGroups; ++g) {
            bool pass = g < a.G;
#pragma unroll
            for (int x = 0; x < W; ++x) pass = pass && (sg[u][x] & mk[g][x]) == mk[g][x];
            any = any || pass;
          }
          ok[u] = s < e1 && any && sig_live(sg[u][0], sg[u][1], W);
        }
        int4 xv[IT][D / 16];
#pragma unroll
        for (int u = 0; u < IT; ++u) {
          const int4 *xr = reinterpret_cast<const int4 *>(a.ix.items + (base + sb + u * kLkThreads + tid) * D);
#pragma unroll
          for (int i = 0; i < D / 16; ++i) xv[u][i] = ok[u] ? xr[i] : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < IT; ++u) {
          uint64_t key = 0ull;
          bool keep = ok[u];
          if (ok[u]) {
            int32_t acc = 0;
#pragma unroll
            for (int i = 0; i < D / 16; ++i) {
              acc = __builtin_amdgcn_sdot4(xv[u][i].x, qv[i].x, acc, false);
              acc = __builtin_amdgcn_sdot4(xv[u][i].y, qv[i].y, acc, false);
              acc = __builtin_amdgcn_sdot4(xv[u][i].z, qv[i].z, acc, false);
              acc = __builtin_amdgcn_sdot4(xv[u][i].w, qv[i].w, acc, false);
            }
            if (MODE == kLkPool) {
              ++my_elig;
              keep = acc >= sthr;   // below the speculative threshold: not pooled
            }
            if (keep) key = lk_key(acc, a.ix.perm[base + sb + u * kLkThreads + tid]);
          }
          if constexpr (COLLECT) {
            // kLkCollect: keys at or above the final threshold (0: every eligible key); kLkPool: every
            // key that reached the speculative threshold
            const bool take = keep && (MODE == kLkPool || key >= prefix);
            const uint64_t bal = __ballot(take);
            if (bal) {
              uint32_t at = 0u;
              if (l == 0) at = atomicAdd(&stage_n, (uint32_t)__popcll(bal));
              at = __shfl(at, 0) + (uint32_t)mbcnt(bal);
              if (take) stage[at] = key;   // at most kLkChunk keys a chunk
            }
          } else {
            if (keep && (key & hi) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & (kLkBins - 1)], 1u);
          }
        }
      }
    }
    __syncthreads();
    if (!COLLECT) {   // add the chunk's counts to the query's histogram and clear them
      uint32_t *gh = a.w.lk_hist + (size_t)b * kLkBins;
      for (int i = tid; i < kLkBins; i += kLkThreads)
        if (hist[i]) {
          atomicAdd(&gh[i], hist[i]);
          hist[i] = 0u;
        }
    } else {          // the chunk's keys: one reservation, then the copy
      const uint32_t n = stage_n;
      if (tid == 0) stage_base = n ? atomicAdd(MODE == kLkPool ? a.w.pool_cnt + b : a.w.lk_cnt + b, n) : 0u;
      __syncthreads();
      const uint32_t cap = MODE == kLkPool ? a.pool_cap : (uint32_t)a.k;
      uint64_t *keys = MODE == kLkPool ? a.w.pool + (size_t)b * a.pool_cap : a.w.lk_keys + (size_t)b * a.k;
      for (uint32_t i = tid; i < n; i += kLkThreads)
        if (stage_base + i < cap) keys[stage_base + i] = stage[i];
      if (tid == 0) stage_n = 0u;
    }
    if (MODE == kLkPool) {   // the query's eligible items, for its statistics
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) my_elig += __shfl_xor(my_elig, o);
      if (l == 0 && my_elig && a.w.stats)
        atomicAdd((unsigned long long *)&a.w.stats[2 * (size_t)b + 1], (unsigned long long)my_elig);
    }
    __syncthreads();
  }
}

// Fix the digit counted by the last pass, one workgroup per query.  Thread t holds bins 8 (255 - t) ..
// 8 (255 - t) + 7, so that the block's prefix sums count the keys in higher buckets.  The histogram is
// cleared for the next pass.
__global__ __launch_bounds__(kLkThreads) void k_lk_pick(int32_t B, Work w) {
  static_assert(kLkBins == 8 * kLkThreads, "8 bins per thread");
  __shared__ int wave_tot[kLkThreads / 64 + 1];
  const int b = blockIdx.x, tid = threadIdx.x;
  LkState *sp = w.lk_state + b;
  const LkState st = *sp;
  if (st.done) return;
  uint32_t *gh = w.lk_hist + (size_t)b * kLkBins;
  const int g = kLkThreads - 1 - tid;
  uint32_t h[8];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = gh[8 * g + i];
    sum += (int)h[i];
  }
  int total;
  int above = block_excl_scan<kLkThreads>(sum, wave_tot, &total);   // keys in the buckets above this thread's
#pragma unroll
  for (int i = 0; i < 8; ++i) gh[8 * g + i] = 0u;
  if (st.shift == kLkTopShift && tid == 0 && w.stats) w.stats[2 * (size_t)b + 1] = total;   // every eligible key
  if (total <= st.need) {
    // first pass with at most k eligible keys: every one of them is kept (threshold 0)
    if (tid == 0) *sp = LkState{0ull, st.shift, st.need, kLkDone, 0};
    return;
  }
  if (above < st.need && above + sum >= st.need) {
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (above + (int)h[i] >= st.need) {
        const int d = 8 * g + i;
        const int rem = st.need - above;
        LkState ns = st;
        ns.prefix = st.prefix | ((uint64_t)d << st.shift);
        if ((int)h[i] == rem || st.shift == 0) {
          ns.done = kLkDone;
        } else {
          ns.shift = st.shift - kLkDigit;
          ns.need = rem;
        }
        *sp = ns;
        break;
      }
      above += (int)h[i];
    }
  }
}

// Pool mode: one workgroup per query.  A pool that did not overflow and holds at least k keys, or that
// was filled without a threshold, holds every key at or above the query's k-th best: the k best of it
// (a radix select over the pool, 8 loads in flight per thread) become the collected keys and the query
// is marked kLkFromPool.  Any other query is left to the passes.
// slot_keys: the pool holds the tile scan's (score, slot) keys.  Their k-th best fixes the k-th best score;
// every key at that score or above becomes a (score, id) key in place and every other key 0, and the
// select then runs over those (ties at the k-th score go to the lower ids).
__global__ __launch_bounds__(kLkEmitThreads) void k_lk_pool(int32_t k, uint32_t cap, int32_t slot_keys,
                                                           const int32_t *perm, Work w) {
  __shared__ SelScratch sel;
  __shared__ int wave_tot[kLkEmitThreads / 64 + 1];
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint32_t n = w.pool_cnt[b];
  const int32_t thr = w.sthr[b];
  if (n > cap || (n < (uint32_t)k && thr != INT32_MIN)) return;
  uint64_t *pool = w.pool + (size_t)b * cap;
  const int nn = (int)n;
  auto visit = [&](auto f) {
    for (int i0 = tid; i0 < nn; i0 += 8 * kLkEmitThreads) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kLkEmitThreads;
        v[u] = i < nn ? pool[i] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * kLkEmitThreads < nn) f(v[u]);
    }
  };
  if (slot_keys) {
    // the smallest (score, slot) key with the k-th best score (0: every key), then the conversion
    const uint64_t T1 = nn > k ? block_select<kLkEmitThreads>(visit, k, sel) : 0ull;
    const uint64_t lo = (T1 >> 32) << 32;
    for (int i0 = tid; i0 < nn; i0 += 8 * kLkEmitThreads) {
      uint64_t v[8];
      int32_t id[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kLkEmitThreads;
        v[u] = i < nn ? pool[i] : 0ull;
        id[u] = (i < nn && v[u] >= lo) ? perm[(uint32_t)v[u]] : 0;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kLkEmitThreads;
        if (i < nn) pool[i] = v[u] >= lo ? lk_key(key_score(v[u]), id[u]) : 0ull;
      }
    }
    __syncthreads();   // the converted pool, for every thread of the workgroup
  }
  // the k-th best key (keys are distinct; 0 marks a key below the k-th best score); every key when the
  // pool holds at most k
  const uint64_t T = nn > k ? block_select<kLkEmitThreads>([&](auto f) {
    visit([&](uint64_t v) {
      if (v) f(v);
    });
  }, k, sel) : 1ull;
  uint64_t *keys = w.lk_keys + (size_t)b * k;
  int base = 0;
  for (int i0 = 0; i0 < nn; i0 += 8 * kLkEmitThreads) {   // in the pool's order, 8 keys per thread a round
    uint64_t v[8];
    int take = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kLkEmitThreads + tid;
      v[u] = i < nn ? pool[i] : 0ull;
      take += (i < nn && v[u] >= T && v[u] != 0ull) ? 1 : 0;
    }
    int tot;
    int off = base + block_excl_scan<kLkEmitThreads>(take, wave_tot, &tot);   // barriers inside
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kLkEmitThreads + tid;
      if (i < nn && v[u] >= T && v[u] != 0ull && off < k) keys[off++] = v[u];
    }
    base += tot;
  }
  if (tid == 0) {
    w.lk_cnt[b] = (uint32_t)(base < k ? base : k);
    w.lk_state[b].done = kLkFromPool;
  }
}

// Bitonic sort, descending, of N = E * kLkEmitThreads keys (missing keys are 0, below every real key).
// Thread t holds elements t E .. t E + E - 1 in registers: strides below E are exchanged in registers,
// strides up to 64 E between lanes by shuffles, larger ones through S (N keys of LDS).  The sorted keys
// end in S.
template <int E>
__device__ void lk_sort(uint64_t *S, const uint64_t *keys, int n) {
  constexpr int N = E * kLkEmitThreads;
  const int tid = threadIdx.x;
  for (int i = tid; i < N; i += kLkEmitThreads) S[i] = i < n ? keys[i] : 0ull;
  __syncthreads();
  uint64_t v[E];
#pragma unroll
  for (int e = 0; e < E; ++e) v[e] = S[tid * E + e];
  __syncthreads();
  for (int size = 2; size <= N; size <<= 1) {
    for (int stride = size >> 1; stride >= E; stride >>= 1) {   // partner: thread tid ^ (stride / E)
      const int ts = stride / E;
      uint64_t p[E];
      if (ts < 64) {
#pragma unroll
        for (int e = 0; e < E; ++e) p[e] = __shfl_xor(v[e], ts);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) S[tid * E + e] = v[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) p[e] = S[(tid ^ ts) * E + e];
        __syncthreads();
      }
      const bool lower = (tid & ts) == 0;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const bool desc = ((tid * E + e) & size) == 0;
        const bool keep_max = lower == desc;
        v[e] = keep_max ? (v[e] > p[e] ? v[e] : p[e]) : (v[e] < p[e] ? v[e] : p[e]);
      }
    }
#pragma unroll
    for (int st = E / 2; st >= 1; st >>= 1) {   // within the thread
      if (st < size) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if ((e & st) == 0) {
            const bool desc = ((tid * E + e) & size) == 0;
            const uint64_t x = v[e], y = v[e + st];
            const bool sw = desc ? x < y : x > y;
            v[e] = sw ? y : x;
            v[e + st] = sw ? x : y;
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) S[tid * E + e] = v[e];
  __syncthreads();
}

// Sort each query's collected keys (at most k <= SVT_MAX_K_LARGE) in LDS, best first, and write the row.
__global__ __launch_bounds__(kLkEmitThreads) void k_lk_emit(int32_t k, const float *query_scales, float item_scale,
                                                           Work w, int64_t *out_ids, int32_t *out_scores,
                                                           float *out_fscores, int32_t *out_counts) {
  static_assert(SVT_MAX_K_LARGE == 16 * kLkEmitThreads, "the largest sort holds 16 keys per thread");
  __shared__ uint64_t S[SVT_MAX_K_LARGE];
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint32_t c = w.lk_cnt[b];
  const int n = c < (uint32_t)k ? (int)c : k;
  const uint64_t *keys = w.lk_keys + (size_t)b * k;
  if (n <= 2 * kLkEmitThreads) lk_sort<2>(S, keys, n);
  else if (n <= 4 * kLkEmitThreads) lk_sort<4>(S, keys, n);
  else if (n <= 8 * kLkEmitThreads) lk_sort<8>(S, keys, n);
  else lk_sort<16>(S, keys, n);
  const float qs = query_scales ? query_scales[b] : item_scale;
  const double denom = (double)item_scale * (double)qs;
  for (int i = tid; i < k; i += kLkEmitThreads) {
    const size_t o = (size_t)b * k + i;
    if (i < n) {
      const int32_t sc = lk_score(S[i]);
      out_ids[o] = lk_id(S[i]);
      out_scores[o] = sc;
      if (out_fscores) out_fscores[o] = (float)((double)sc / denom);
    } else {
      out_ids[o] = -1;
      out_scores[o] = INT32_MIN;
      if (out_fscores) out_fscores[o] = -__builtin_huge_valf();
    }
  }
  if (tid == 0 && out_counts) out_counts[b] = n;
}

template <int D, int W>
void lk_scan_launch(const LkScanArgs &a, dim3 grid, int mode, hipStream_t s) {
  if (mode == kLkCollect)
    k_lk_scan<D, W, kLkCollect><<<grid, kLkThreads, 0, s>>>(a);
  else if (mode == kLkPool)
    k_lk_scan<D, W, kLkPool><<<grid, kLkThreads, 0, s>>>(a);
  else
    k_lk_scan<D, W, kLkCount><<<grid, kLkThreads, 0, s>>>(a);
}

template <int D>
void lk_scan_w(const LkScanArgs &a, dim3 grid, int mode, hipStream_t s) {
  if (a.ix.sig_words == 2)
    lk_scan_launch<D, 2>(a, grid, mode, s);
  else
    lk_scan_launch<D, 1>(a, grid, mode, s);
}

}  // namespace

hipError_t launch_large_k(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const float *query_scales,
                          const SearchShape &sh, int64_t max_stream, const Work &w, int64_t *out_ids,
                          int32_t *out_scores, float *out_fscores, int32_t *out_counts, hipStream_t s) {
  const int64_t n_init = (int64_t)sh.B * kLkBins;
  k_lk_init<<<(unsigned)std::min<int64_t>((n_init + 255) / 256, 4096), 256, 0, s>>>(sh.B, sh.k, w);
  const LkScanArgs a{ix, queries, masks, w, sh.B, sh.nprobe, sh.k, sh.G, (uint32_t)sh.pool_cap};
  k_lk_chunks<<<1, 1024, 0, s>>>(sh.B, w);
  // enough workgroups for the batch's chunks (at most kLkScanWGs, which then walk the rest)
  const int64_t most = (int64_t)sh.B * std::max<int64_t>(1, (max_stream + kLkChunk - 1) / kLkChunk);
  const dim3 grid((unsigned)std::min<int64_t>(most, kLkScanWGs));
  auto scan = [&](int mode) -> hipError_t {
    switch (ix.dim) {
      case 16: lk_scan_w<16>(a, grid, mode, s); break;
      case 32: lk_scan_w<32>(a, grid, mode, s); break;
      case 64: lk_scan_w<64>(a, grid, mode, s); break;
      case 128: lk_scan_w<128>(a, grid, mode, s); break;
      case 256: lk_scan_w<256>(a, grid, mode, s); break;
      default: return hipErrorInvalidValue;
    }
    return hipSuccess;
  };
  hipError_t e;
  if (sh.pool_cap > 0) {   // the pools: filled here, or by the tile scan before this call
    if (!sh.lk_tile && (e = scan(kLkPool)) != hipSuccess) return e;
    k_lk_pool<<<sh.B, kLkEmitThreads, 0, s>>>(sh.k, (uint32_t)sh.pool_cap, sh.lk_tile, ix.perm, w);
  }
  for (int pass = 0; pass <= kLkPasses; ++pass) {
    const bool collect = pass == kLkPasses;
    if ((e = scan(collect ? kLkCollect : kLkCount)) != hipSuccess) return e;
    if (!collect) k_lk_pick<<<sh.B, kLkThreads, 0, s>>>(sh.B, w);
  }
  k_lk_emit<<<sh.B, kLkEmitThreads, 0, s>>>(sh.k, query_scales, ix.item_scale, w, out_ids, out_scores, out_fscores,
                                           out_counts);
  return hipGetLastError();
}

}  // namespace svt
