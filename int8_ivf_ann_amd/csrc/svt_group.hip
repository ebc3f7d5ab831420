// svt_group.hip - gfx950 kernels of the grouped search path.  A batch of queries reads each probed
// cluster once for all the queries that probe it, instead of once per query.
//
//   k_gcount, k_gplan, k_gfill, k_gunits
//             work list: the queries of every probed cluster (gq, grouped by cluster), and units of
//             work = tiles of at most kGTile items of one cluster x groups of at most kGMax of the
//             queries probing it
//   k_gscan   persistent workgroups take units from an atomic queue.  A step of 1024 items loads the
//             signatures once and tests them against every request mask of the group; the rows of the
//             items that at least one query accepts are gathered once and scored (v_dot4) for each
//             query that accepted them.  A candidate that reaches the query's proven bound goes to the
//             query's pool in HBM and is counted in the query's score histogram; as soon as k counted
//             candidates lie at or above a bin's lower edge, that edge is the query's new bound.
//   k_pmerge  per query: the exact top k of its pool
// A query whose pool overflows is scanned again query by query (k_scan and k_merge in fallback mode),
// so the result is exact whatever the data.
//
// Method: "SilverTorch - Index as Model" (Meta engineering post): probe the most promising clusters,
// filter inside them with Bloom signatures and bit operations, score the survivors with int8 dot
// products, keep a large top-k on the device and return only the final candidates.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svt_device.h"
#include "svt_internal.h"

namespace svt {

// ------------------------------------------------------------------------------------------------
// work list

// queries probing each cluster (gcnt is zeroed by k_coarse_keys)
__global__ __launch_bounds__(256) void k_gcount(const int32_t *__restrict__ probes, int32_t nprobe,
                                                int32_t *__restrict__ gcnt) {
  const int b = blockIdx.x;
  for (int j = threadIdx.x; j < nprobe; j += 256) atomicAdd(&gcnt[probes[(size_t)b * nprobe + j]], 1);
}

// one workgroup: where each cluster's query list starts in gq, and the first unit of each cluster
__global__ __launch_bounds__(kSelThreads) void k_gplan(DevIndex ix, Work w) {
  __shared__ int wave_tot[kSelThreads / 64 + 1];
  const int tid = threadIdx.x;
  const int nlist = ix.nlist;
  int carry_q = 0, carry_u = 0;
  for (int c0 = 0; c0 < nlist; c0 += kSelThreads) {
    const int c = c0 + tid;
    int nq = 0, nu = 0;
    if (c < nlist) {
      nq = w.gcnt[c];
      const int size = ix.offsets[c + 1] - ix.offsets[c];
      if (nq > 0 && size > 0) nu = ((size + kGTile - 1) / kGTile) * ((nq + kGMax - 1) / kGMax);
    }
    int tq, tu;
    const int eq = block_excl_scan<kSelThreads>(nq, wave_tot, &tq);
    const int eu = block_excl_scan<kSelThreads>(nu, wave_tot, &tu);
    if (c < nlist) {
      w.gstart[c] = carry_q + eq;
      w.ustart[c] = carry_u + eu;
    }
    carry_q += tq;
    carry_u += tu;
  }
  if (tid == 0) {
    w.gstart[nlist] = carry_q;
    w.ustart[nlist] = carry_u;
  }
}

// the queries of each probed cluster (their order inside a cluster is arbitrary)
__global__ __launch_bounds__(256) void k_gfill(const int32_t *__restrict__ probes, int32_t nprobe, Work w) {
  const int b = blockIdx.x;
  for (int j = threadIdx.x; j < nprobe; j += 256) {
    const int c = probes[(size_t)b * nprobe + j];
    const int slot = atomicAdd(&w.gfill[c], 1);
    w.gq[w.gstart[c] + slot] = b;
  }
}

// unit u: the cluster whose units hold u, then its tile and query group
__global__ __launch_bounds__(256) void k_gunits(DevIndex ix, Work w) {
  const int u = blockIdx.x * 256 + threadIdx.x;
  const int nlist = ix.nlist;
  if (u >= w.ustart[nlist]) return;
  int lo = 0, hi = nlist - 1;   // largest c with ustart[c] <= u: a cluster that has units
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (w.ustart[mid] <= u) lo = mid; else hi = mid - 1;
  }
  const int c = lo;
  const int nq = w.gstart[c + 1] - w.gstart[c];
  const int ng = (nq + kGMax - 1) / kGMax;
  const int i = u - w.ustart[c];
  const int t = i / ng, gg = i % ng;
  const int32_t a0 = ix.offsets[c] + t * kGTile, end = ix.offsets[c + 1];
  const int32_t q0 = w.gstart[c] + gg * kGMax, qe = w.gstart[c + 1];
  w.units[u] = GUnit{c, a0, a0 + kGTile < end ? a0 + kGTile : end, q0, q0 + kGMax < qe ? q0 + kGMax : qe, 0, 0, 0};
}

// ------------------------------------------------------------------------------------------------
// k_gscan

struct GScanArgs {
  DevIndex ix;
  const int8_t *queries;
  const uint64_t *masks;
  Work w;
  int32_t B, nprobe, k, P;
  uint32_t pool_cap;
};

constexpr int kStage = 1024;      // candidates staged in LDS before they go to the pools
constexpr int kStageFlush = 512;  // a step that ends with at least this many staged flushes them
constexpr int kGLH = 4;           // queries of a group whose histogram counts are gathered in LDS

struct GScanLds {
  uint16_t wl[kScanThreads * kScanGroups];   // items some query accepts, wave w's at [w * 256, ...)
  uint32_t wq[kScanThreads * kScanGroups];   // for each of them, the group's queries that accept it
  int wcnt[kScanThreads / 64];
  uint64_t gmask[kGMax][2];                  // the group's request masks
  int4 gqv[kGMax][16];                       // the group's query vectors (d <= 256)
  int32_t gq[kGMax], gthr[kGMax], ghlo[kGMax], ghsh[kGMax];
  uint32_t gelig[kGMax];                     // items of the unit each query accepts
  uint32_t gadd[kGMax];                      // candidates the unit gave each query
  uint64_t stage_key[kStage];                // staged candidates: (score, position) key
  uint8_t stage_q[kStage];                   //   and the group index of their query
  uint32_t scnt[kGMax], sbase[kGMax], scur[kGMax];
  int scnt_total;                            // candidates offered to the stage (may exceed kStage)
  uint32_t lh[kGLH][kQHistBins];             // histogram counts of the group's first queries
  int next;                                  // queue position of this workgroup's next unit
};

// Queue position -> unit: a bijection of [0, n) that scatters the units of a cluster (which are numbered
// consecutively) over the whole run.  Otherwise the tiles of a large cluster would all be scanned at
// once, before any of them could raise the bound of the queries probing it.  A permutation of
// [0, 2^m) (odd multiplications and an xor-shift, each invertible modulo 2^m), walked until it lands
// below n; the walk ends because every cycle of the permutation holds a position below n (the start).
__device__ __forceinline__ int scatter_unit(int pos, int n) {
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

template <int LPR, int W>
__global__ __launch_bounds__(kScanThreads, 4) void k_gscan(GScanArgs a) {
  constexpr int D = 16 * LPR;
  constexpr int RPI = 64 / LPR;            // rows covered by one 16-byte load per lane
  constexpr int RB = D <= 128 ? 64 : 32;   // rows a wave requests together
  constexpr int R = RB / RPI;              // row loads per lane in one batch (<= 8)
  constexpr int NWV = kScanThreads / 64;
  __shared__ GScanLds sm;
  const int tid = threadIdx.x, l = lane_id(), wv = tid / 64, sub = l % LPR;
  const uint32_t cap = a.pool_cap;
  const int n_units = a.w.ustart[a.ix.nlist];
  if (tid == 0) sm.next = (int)atomicAdd(&a.w.counter[2], 1u);
  __syncthreads();
  for (;;) {
    const int upos = __builtin_amdgcn_readfirstlane(sm.next);
    if (upos >= n_units) break;
    int next_u = 0;
    if (tid == 0) next_u = (int)atomicAdd(&a.w.counter[2], 1u);
    const GUnit un = a.w.units[scatter_unit(upos, n_units)];
    const int g = un.q1 - un.q0;   // 1 .. kGMax
    for (int j = tid; j < g; j += kScanThreads) {
      const int q = a.w.gq[un.q0 + j];
      sm.gq[j] = q;
#pragma unroll
      for (int t = 0; t < W; ++t) sm.gmask[j][t] = a.masks[(size_t)q * W + t];
      sm.gthr[j] = __hip_atomic_load(&a.w.thr[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      sm.ghlo[j] = a.w.hlo[q];
      sm.ghsh[j] = a.w.hshift[q];
      sm.gelig[j] = 0u;
      sm.gadd[j] = 0u;
      sm.scnt[j] = 0u;
    }
    for (int i = tid; i < kGLH * kQHistBins; i += kScanThreads) sm.lh[i / kQHistBins][i % kQHistBins] = 0u;
    if (tid == 0) sm.scnt_total = 0;
    for (int i = tid; i < g * LPR; i += kScanThreads) {
      const int j = i / LPR, ch = i % LPR;
      sm.gqv[j][ch] = reinterpret_cast<const int4 *>(a.queries + (size_t)a.w.gq[un.q0 + j] * D)[ch];
    }
    __syncthreads();
    // Signatures of a step are requested with the previous step's rows.  Loads are issued
    // unconditionally (lanes past the end read an in-range clamped position and are masked).
    uint64_t sg[kScanGroups][W];
    int32_t sg_n = 0;
    auto load_sigs = [&](int32_t st) {
      const int32_t rem = un.hi - st;
      sg_n = rem <= 0 ? 0 : (rem < kScanStep ? rem : kScanStep);
      const int32_t p0 = rem <= 0 ? un.lo : st;
      const int32_t last = sg_n > 0 ? sg_n - 1 : 0;
#pragma unroll
      for (int gi = 0; gi < kScanGroups; ++gi) {
        const int i = gi * kScanThreads + wv * 64 + l;
        const int32_t p = p0 + (i < last ? i : last);
        if constexpr (W == 2) {
          const ulonglong2 v = reinterpret_cast<const ulonglong2 *>(a.ix.sigs)[p];
          sg[gi][0] = v.x;
          sg[gi][1] = v.y;
        } else {
          sg[gi][0] = a.ix.sigs[p];
        }
      }
    };
    // Move the staged candidates to their pools: one pool reservation per query, then every thread
    // copies entries.  All threads call it, after a barrier that ends the step's appends.
    auto flush_stage = [&]() {
      const int tot = sm.scnt_total < kStage ? sm.scnt_total : kStage;
      if (tid < g) {
        const uint32_t nj = sm.scnt[tid];
        sm.sbase[tid] = nj ? atomicAdd(&a.w.pool_cnt[sm.gq[tid]], nj) : 0u;
        sm.scur[tid] = 0u;
      }
      __syncthreads();
      for (int e = tid; e < tot; e += kScanThreads) {
        const int j = sm.stage_q[e];
        const uint32_t slot = sm.sbase[j] + atomicAdd(&sm.scur[j], 1u);
        if (slot < cap) a.w.pool[(size_t)sm.gq[j] * cap + slot] = sm.stage_key[e];
      }
      __syncthreads();
      if (tid < g) sm.scnt[tid] = 0u;
      if (tid == 0) sm.scnt_total = 0;
    };
    load_sigs(un.lo);
    for (int32_t st = un.lo; st < un.hi; st += kScanStep) {
      const int32_t n = sg_n;
      // --- every request mask of the group against this step's signatures; compact the items at least
      // one query accepts, with the set of queries that accept each
      int nw = 0;
#pragma unroll
      for (int gi = 0; gi < kScanGroups; ++gi) {
        const int i = gi * kScanThreads + wv * 64 + l;
        uint32_t qm = 0u;
        if (i < n) {
          for (int j = 0; j < g; ++j) {
            bool pass = true;
#pragma unroll
            for (int t = 0; t < W; ++t) pass = pass && ((sg[gi][t] & sm.gmask[j][t]) == sm.gmask[j][t]);
            qm |= pass ? (1u << j) : 0u;
          }
        }
        const uint64_t bal = __ballot(qm != 0u);
        if (qm != 0u) {
          const int o = wv * 64 * kScanGroups + nw + mbcnt(bal);
          sm.wl[o] = (uint16_t)i;
          sm.wq[o] = qm;
        }
        nw += __popcll(bal);
        for (int j = 0; j < g; ++j) {
          const uint64_t b = __ballot((qm >> j) & 1u);
          if (l == 0 && b) atomicAdd(&sm.gelig[j], (uint32_t)__popcll(b));
        }
      }
      if (l == 0) sm.wcnt[wv] = nw;
      __syncthreads();
      // --- the step's accepted items are shared out evenly: wave wv takes [rbeg, rend) of the
      // concatenation of the waves' lists
      int pre[NWV + 1];
      pre[0] = 0;
#pragma unroll
      for (int i = 0; i < NWV; ++i) pre[i + 1] = pre[i] + sm.wcnt[i];
      const int total = pre[NWV];
      const int per = (total + NWV - 1) / NWV;
      const int rbeg = wv * per, rend = rbeg + per < total ? rbeg + per : total;
      auto surv_at = [&](int r) -> int {   // LDS index of accepted item r (pre is nondecreasing)
        int adj = 0;
#pragma unroll
        for (int i = 1; i < NWV; ++i) adj = r >= pre[i] ? i * 64 * kScanGroups - pre[i] : adj;
        return r + adj;
      };
      int4 x[R];
      auto load_rows = [&](int r0) {
#pragma unroll
        for (int uu = 0; uu < R; ++uu) {
          const int r = r0 + uu * RPI + l / LPR;
          const int32_t p = st + (r < rend ? (int)sm.wl[surv_at(r)] : 0);
          x[uu] = reinterpret_cast<const int4 *>(a.ix.items + (size_t)p * D)[sub];
        }
      };
      // score each loaded row for every query of the group that accepts it; a candidate reaching the
      // query's bound takes a pool slot (one atomic per wave and query) and is counted in the query's
      // histogram
      auto score_rows = [&](int r0) {
#pragma unroll
        for (int uu = 0; uu < R; ++uu) {
          const int r = r0 + uu * RPI + l / LPR;
          const bool valid = r < rend;
          const int si = valid ? surv_at(r) : 0;
          const uint32_t qm = valid ? sm.wq[si] : 0u;
          for (int j = 0; j < g; ++j) {
            const bool want = (qm >> j) & 1u;
            if (__ballot(want) == 0ull) continue;
            const int32_t acc = group_sum<LPR>(dot16(x[uu], sm.gqv[j][sub], 0));
            const bool ok = sub == 0 && want && acc >= sm.gthr[j];
            const uint64_t b = __ballot(ok);
            if (b == 0ull) continue;
            // the wave's candidates take consecutive stage entries; past the stage's end they go
            // straight to the pool
            int at = 0;
            if (l == 0) at = atomicAdd(&sm.scnt_total, __popcll(b));
            at = __builtin_amdgcn_readfirstlane(at);
            if (ok) {
              const uint64_t key = pos_key(acc, st + (int)sm.wl[si]);
              const int e = at + mbcnt(b);
              const int q = sm.gq[j];
              if (e < kStage) {
                sm.stage_key[e] = key;
                sm.stage_q[e] = (uint8_t)j;
                atomicAdd(&sm.scnt[j], 1u);
              } else {
                const uint32_t slot = atomicAdd(&a.w.pool_cnt[q], 1u);
                if (slot < cap) a.w.pool[(size_t)q * cap + slot] = key;
              }
              const int32_t hlo = sm.ghlo[j];
              int bin = 0;
              if (acc >= hlo) {
                const int32_t bb = (acc - hlo) >> sm.ghsh[j];
                bin = bb < kQHistBins - 1 ? bb : kQHistBins - 1;
              }
              if (j < kGLH) atomicAdd(&sm.lh[j][bin], 1u);
              else atomicAdd(&a.w.ghist[(size_t)q * kQHistBins + bin], 1u);
            }
            if (l == 0) atomicAdd(&sm.gadd[j], (uint32_t)__popcll(b));
          }
        }
      };
      if (rbeg < rend) load_rows(rbeg);
      load_sigs(st + kScanStep);
      // the group's current bounds, requested with the loads and installed after the step
      int32_t thr_pref = INT32_MIN;
      if (wv == 0 && l < g)
        thr_pref = __hip_atomic_load(&a.w.thr[sm.gq[l]], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (rbeg < rend) score_rows(rbeg);
      for (int r0 = rbeg + RB; r0 < rend; r0 += RB) {   // dense filters: further batches
        load_rows(r0);
        score_rows(r0);
      }
      __syncthreads();
      // bounds are read in the scoring phase only, which the next step enters after its barrier
      if (wv == 0 && l < g && thr_pref > sm.gthr[l]) sm.gthr[l] = thr_pref;
      // staged candidates go out when the stage is half full or the unit ends (the decision reads a
      // value no thread changes before the next step's second barrier)
      if (sm.scnt_total >= kStageFlush || st + kScanStep >= un.hi) flush_stage();
    }
    __syncthreads();
    // histogram counts gathered in LDS go to the queries' histograms before the bounds are computed
    for (int i = tid; i < kGLH * kQHistBins; i += kScanThreads) {
      const int j = i / kQHistBins, bin = i % kQHistBins;
      if (j < g) {
        const uint32_t v = sm.lh[j][bin];
        if (v) atomicAdd(&a.w.ghist[(size_t)sm.gq[j] * kQHistBins + bin], v);
      }
    }
    __syncthreads();
    // --- end of the unit: statistics, and new bounds for the queries that received candidates
    for (int j = tid; j < g; j += kScanThreads) {
      const int q = sm.gq[j];
      if (a.w.stats) {
        atomicAdd((unsigned long long *)&a.w.stats[2 * (size_t)q + 1], (unsigned long long)sm.gelig[j]);
        atomicAdd((unsigned long long *)&a.w.stats[2 * (size_t)q], (unsigned long long)(un.hi - un.lo));
      }
    }
    for (int j = wv; j < g; j += NWV) {   // wave-uniform
      if (sm.gadd[j] == 0u) continue;
      const int q = sm.gq[j];
      const uint32_t *gh = a.w.ghist + (size_t)q * kQHistBins;
      constexpr int HPB = kQHistBins / 64;
      uint32_t h[HPB], sum = 0u;
#pragma unroll
      for (int t = 0; t < HPB; ++t) {
        h[t] = __hip_atomic_load(&gh[HPB * l + t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sum += h[t];
      }
      uint32_t suf = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off);
        if (l + off < 64) suf += v;
      }
      uint32_t above = suf - sum;
#pragma unroll
      for (int t = HPB - 1; t >= 0; --t) {
        const int bin = HPB * l + t;
        if (bin >= 1 && above < (uint32_t)a.k && above + h[t] >= (uint32_t)a.k)
          atomicMax(&a.w.thr[q], sm.ghlo[j] + (bin << sm.ghsh[j]));
        above += h[t];
      }
    }
    if (tid == 0) sm.next = next_u;
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// k_pmerge: one workgroup per query whose pool held all its candidates.  The k-th best (score,
// position) key fixes the k-th best score; every key at that score or above becomes a (score, id) key,
// and the exact top k of those is sorted and written.

struct PMergeArgs {
  DevIndex ix;
  Work w;
  const float *query_scales;
  float item_scale;
  int32_t B, k;
  uint32_t pool_cap;
  int64_t *out_ids;
  int32_t *out_scores;
  float *out_fscores;
  int32_t *out_counts;
};

__global__ __launch_bounds__(kSelThreads) void k_pmerge(PMergeArgs a) {
  __shared__ SelScratch sel;
  __shared__ uint64_t cand[kMergeCap];
  __shared__ int wave_tot[kSelThreads / 64 + 1];
  __shared__ int ncand;
  const int q = blockIdx.x, tid = threadIdx.x, k = a.k;
  const uint32_t pc = a.w.pool_cnt[q];
  if (pc > a.pool_cap) return;   // overflowed: merged from the query-by-query scan
  const int n = (int)pc;
  uint64_t *pool = a.w.pool + (size_t)q * a.pool_cap;
  uint64_t lo = 0ull;
  if (n > k) {
    const uint64_t T = block_select<kSelThreads>(
        [&](auto f) {
          for (int i = tid; i < n; i += kSelThreads) f(pool[i]);
        },
        k, sel);
    lo = (T >> 32) << 32;   // the smallest key with the k-th best score
  }
  // keys at or above lo become (score, id) keys in place; their upper half, the score, is unchanged
  for (int i = tid; i < n; i += kSelThreads) {
    const uint64_t v = pool[i];
    if (v >= lo) pool[i] = make_key((int32_t)((uint32_t)(v >> 32) ^ 0x80000000u), (uint32_t)a.ix.perm[(uint32_t)v]);
  }
  if (tid == 0) ncand = 0;
  __syncthreads();
  for (int i = tid; i < n; i += kSelThreads) {
    const uint64_t v = pool[i];
    if (v >= lo) {
      const int o = atomicAdd(&ncand, 1);
      if (o < kMergeCap) cand[o] = v;
    }
  }
  __syncthreads();
  int m = ncand;
  const int nout = n < k ? n : k;
  if (m > kMergeCap) {
    // heavy ties at the k-th score: select among the converted keys in the pool
    const uint64_t Tk = block_select<kSelThreads>(
        [&](auto f) {
          for (int i = tid; i < n; i += kSelThreads) {
            const uint64_t v = pool[i];
            if (v >= lo) f(v);
          }
        },
        k, sel);
    if (tid == 0) ncand = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const uint64_t v = pool[i];
      if (v >= lo && v >= Tk) cand[atomicAdd(&ncand, 1)] = v;   // exactly k distinct keys
    }
    __syncthreads();
    m = k;
  } else if (m > k) {
    const uint64_t Tk = block_select<kSelThreads>(
        [&](auto f) {
          for (int i = tid; i < m; i += kSelThreads) f(cand[i]);
        },
        k, sel);
    constexpr int PER = kMergeCap / kSelThreads;
    uint64_t mine[PER];
    int keep = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSelThreads;
      mine[u] = i < m ? cand[i] : 0ull;
      keep += (i < m && mine[u] >= Tk) ? 1 : 0;
    }
    int tot;
    int off = block_excl_scan<kSelThreads>(keep, wave_tot, &tot);   // barriers inside
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSelThreads;
      if (i < m && mine[u] >= Tk) cand[off++] = mine[u];
    }
    __syncthreads();
    m = k;
  }
  emit_sorted<kSelThreads>(cand, m, nout, q, k, a.query_scales, a.item_scale, a.out_ids, a.out_scores,
                           a.out_fscores);
  if (tid == 0 && a.out_counts) a.out_counts[q] = nout;
}

// ------------------------------------------------------------------------------------------------
// launch wrappers

hipError_t launch_group_plan(const DevIndex &ix, const SearchShape &sh, const Work &w, hipStream_t s) {
  k_gcount<<<sh.B, 256, 0, s>>>(w.probes, sh.nprobe, w.gcnt);
  k_gplan<<<1, kSelThreads, 0, s>>>(ix, w);
  k_gfill<<<sh.B, 256, 0, s>>>(w.probes, sh.nprobe, w);
  k_gunits<<<(sh.max_units + 255) / 256, 256, 0, s>>>(ix, w);
  return hipGetLastError();
}

template <int LPR>
static void gscan_w(const GScanArgs &a, int W, hipStream_t s) {
  if (W == 2)
    k_gscan<LPR, 2><<<a.P, kScanThreads, 0, s>>>(a);
  else
    k_gscan<LPR, 1><<<a.P, kScanThreads, 0, s>>>(a);
}

hipError_t launch_gscan(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const SearchShape &sh,
                        const Work &w, hipStream_t s) {
  GScanArgs a{ix, queries, masks, w, sh.B, sh.nprobe, sh.k, sh.P, (uint32_t)sh.pool_cap};
  switch (ix.dim) {
    case 16: gscan_w<1>(a, ix.sig_words, s); break;
    case 32: gscan_w<2>(a, ix.sig_words, s); break;
    case 64: gscan_w<4>(a, ix.sig_words, s); break;
    case 128: gscan_w<8>(a, ix.sig_words, s); break;
    case 256: gscan_w<16>(a, ix.sig_words, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pool_merge(const DevIndex &ix, const float *query_scales, const SearchShape &sh, const Work &w,
                             int64_t *out_ids, int32_t *out_scores, float *out_fscores, int32_t *out_counts,
                             hipStream_t s) {
  PMergeArgs a{ix, w, query_scales, ix.item_scale, sh.B, sh.k, (uint32_t)sh.pool_cap, out_ids, out_scores,
               out_fscores, out_counts};
  k_pmerge<<<sh.B, kSelThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace svt
