// svt_group.hip - gfx950 kernels of the grouped search path.  A batch of queries reads each probed
// cluster once for all the queries that probe it, instead of once per query.
//
//   k_gcount, k_gplan, k_gfill, k_gunits
//             work list: the queries of every probed cluster (gq, grouped by cluster), and units of
//             work = tiles of at most kGTile items of one cluster x groups of at most kGMax of the
//             queries probing it
//   k_gscan   every wave of the persistent workgroups takes units from an atomic queue on its own.
//             A step of 256 items loads the signatures once and tests them against every request mask
//             of the unit's group; the rows of the items that at least one member accepts are gathered
//             once and scored (v_dot4) for each member that accepted them.  A candidate at or above
//             its query's bound goes to the query's pool in HBM.
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
// k_gscan: every wave of a persistent workgroup works on its own, with no block barrier.  A wave
// takes units from the queue and walks a unit in steps of kGStep items: it loads the step's
// signatures once, tests them against every request mask of the unit's query group, compacts the
// items that at least one member accepts (with the set of members that accept each) into its LDS,
// gathers those rows once and scores each of them (v_dot4) for every member that accepted it.  The
// steps of a unit run as a two-stage pipeline: while the rows of step i are in flight the wave filters
// step i + 1 and requests the signatures of step i + 2.  The next unit is set up (queue position,
// unit, member queries, their masks, bounds and query vectors) one stage per step while the current
// unit runs, and the signatures of its first step are requested with the last step of the current one.
// A candidate at or above its query's bound is staged in LDS; staged candidates go to the queries'
// pools with one pool reservation per member (at the end of a unit, or when the stage is full).

struct GScanArgs {
  DevIndex ix;
  const int8_t *queries;
  const uint64_t *masks;
  Work w;
  int32_t B, nprobe, k, P;
  uint32_t pool_cap;
};

constexpr int kGStep = 256;      // items of one wave step: four 64-item groups
constexpr int kGStage = 256;     // candidates a wave stages in LDS
constexpr int kGRowBatch = 32;   // rows a wave gathers together
constexpr int kGPullMin = 32;    // a flush that gives a member this many candidates pulls its histogram

template <int LPR>
struct GGroup {                  // a unit's query group as the wave uses it
  uint64_t mask[kGMax][2];       // request masks
  int4 qv[kGMax][LPR];           // query vectors
  int32_t q[kGMax];              // query index in the batch
  int32_t thr[kGMax];            // proven bounds (read at set-up, raised by the wave's pulls)
  int32_t hlo[kGMax], hsh[kGMax];  // the queries' histogram bins (lower edge of bin 1, log2 width)
  uint32_t scnt[kGMax];          // staged candidates of each member
  uint32_t sbase[kGMax];         // pool cursor of each member during a flush
};

template <int LPR>
struct GWave {
  uint16_t wl[2][kGStep];        // accepted items of a step (offset in the step); two steps in flight
  uint16_t wq[2][kGStep];        // the members that accept each (bit j: member j)
  uint64_t key[kGStage];         // staged candidates: (score, position) keys
  uint8_t kj[kGStage];           //   and their member
  GGroup<LPR> grp[2];            // the current unit's group and the next unit's
};

// Order of LDS accesses between lanes of one wave (the wave's LDS operations complete in order; this
// keeps the compiler from moving them across each other).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}


template <int LPR, int W>
__global__ __launch_bounds__(kScanThreads, kGScanOcc) void k_gscan(GScanArgs a) {
  constexpr int D = 16 * LPR;
  constexpr int RPI = 64 / LPR;                                  // rows covered by one 16-byte load per lane
  constexpr int RB = RPI > kGRowBatch ? RPI : kGRowBatch;        // rows a wave requests together
  constexpr int R = RB / RPI;                                    // row loads per lane in one batch
  constexpr int QVL = (kGMax * LPR + 63) / 64;                   // query-vector loads per lane in a set-up
  constexpr int NG = kGStep / 64;
  __shared__ GWave<LPR> gws[kScanThreads / 64];
  const int l = lane_id(), sub = l % LPR;
  GWave<LPR> &s = gws[threadIdx.x / 64];
  const uint32_t cap = a.pool_cap;
  const int n_units = a.w.ustart[a.ix.nlist];
  const bool want_stats = a.w.stats != nullptr;

  // --- set-up of the next unit, one stage per call (all values wave-uniform but the per-lane loads)
  int pf = 0;          // 1..4: stage whose loads are in flight; 5: ready in grp[nslot]; 6: queue empty
  int nslot = 0;
  int32_t pf_v = 0, pf_q = 0, pf_thr = INT32_MIN, pf_hlo = 0, pf_hsh = 0;
  uint64_t pf_m[W];
  int4 pf_qa = {}, pf_qb = {}, pf_qc = {}, pf_qd = {};   // query-vector parts in flight (QVL <= 4)
  int32_t n_lo = 0, n_hi = 0, n_g = 0;
  auto pf_start = [&]() {
    pf_v = 0;
    if (l == 0) pf_v = (int)atomicAdd(&a.w.counter[2], 1u);
    pf = 1;
  };
  auto pf_step = [&]() {
    if (pf == 1) {
      const int upos = __builtin_amdgcn_readfirstlane(pf_v);
      if (upos >= n_units) {
        pf = 6;
        return;
      }
      const int u = scatter_index(upos, n_units);
      pf_v = reinterpret_cast<const int32_t *>(a.w.units + u)[l & 7];
      pf = 2;
    } else if (pf == 2) {
      n_lo = __builtin_amdgcn_readlane(pf_v, 1);
      n_hi = __builtin_amdgcn_readlane(pf_v, 2);
      const int q0 = __builtin_amdgcn_readlane(pf_v, 3);
      n_g = __builtin_amdgcn_readlane(pf_v, 4) - q0;
      pf_v = a.w.gq[q0 + (l < n_g ? l : 0)];
      pf = 3;
    } else if (pf == 3) {
      pf_q = pf_v;
#pragma unroll
      for (int t = 0; t < W; ++t) pf_m[t] = a.masks[(size_t)pf_q * W + t];
      pf_thr = __hip_atomic_load(&a.w.thr[pf_q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      pf_hlo = a.w.hlo[pf_q];
      pf_hsh = a.w.hshift[pf_q];
      auto qv_load = [&](int t) -> int4 {
        const int idx = t * 64 + l, j = (idx / LPR) % kGMax;
        const int qj = __shfl(pf_q, j < n_g ? j : 0);
        return reinterpret_cast<const int4 *>(a.queries + (size_t)qj * D)[idx % LPR];
      };
      pf_qa = qv_load(0);
      if constexpr (QVL > 1) pf_qb = qv_load(1);
      if constexpr (QVL > 2) pf_qc = qv_load(2);
      if constexpr (QVL > 3) pf_qd = qv_load(3);
      pf = 4;
    } else if (pf == 4) {
      GGroup<LPR> &G = s.grp[nslot];
      if (l < n_g) {
        G.q[l] = pf_q;
        G.thr[l] = pf_thr;
        G.hlo[l] = pf_hlo;
        G.hsh[l] = pf_hsh;
#pragma unroll
        for (int t = 0; t < W; ++t) G.mask[l][t] = pf_m[t];
        G.scnt[l] = 0u;
      }
      auto qv_store = [&](int t, const int4 v) {
        const int idx = t * 64 + l;
        if (idx < n_g * LPR) G.qv[idx / LPR][idx % LPR] = v;
      };
      qv_store(0, pf_qa);
      if constexpr (QVL > 1) qv_store(1, pf_qb);
      if constexpr (QVL > 2) qv_store(2, pf_qc);
      if constexpr (QVL > 3) qv_store(3, pf_qd);
      pf = 5;
    }
  };

  uint64_t sg[NG][W];
  int32_t sg_n = 0;
  bool sg_pre = false;   // the signatures of the prepared unit's first step are in sg
  // Loads are issued unconditionally (a step that does not exist reads an in-range position and counts
  // no items), so the compiler can count outstanding loads exactly and wait only for the ones it needs.
  auto load_sigs = [&](int32_t st, int32_t end) {   // st: a valid position; no items unless st < end
    const int32_t rem = end - st;
    sg_n = rem <= 0 ? 0 : (rem < kGStep ? rem : kGStep);
    const int32_t last = sg_n > 0 ? sg_n - 1 : 0;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int i = gi * 64 + l;
      const int32_t p = st + (i < last ? i : last);
      if constexpr (W == 2) {
        const ulonglong2 v = reinterpret_cast<const ulonglong2 *>(a.ix.sigs)[p];
        sg[gi][0] = v.x;
        sg[gi][1] = v.y;
      } else {
        sg[gi][0] = a.ix.sigs[p];
      }
    }
  };

  pf_start();
  while (pf < 5) pf_step();
  while (pf == 5) {
    // --- take the prepared unit; the unit after it is set up in the other group slot
    const int slot = nslot;
    nslot ^= 1;
    const int32_t lo = n_lo, hi = n_hi, g = n_g;
    GGroup<LPR> &G = s.grp[slot];
    pf_start();
    uint32_t elig = 0;   // lane j: items of the unit member j accepts
    int stage_n = 0;     // staged candidates (wave-uniform)
    wave_lds_sync();

    // The step in sg into wl/wq[buf]; returns the accepted count.  Member 0 is tested for every group
    // before the loop over the other members, so that the wait for the signatures sits in straight-line
    // code (and leaves the rows requested after them in flight).
    auto filter = [&](int buf) -> int {
      int nw = 0;
      uint32_t qms[NG];
      uint64_t m0[W];
#pragma unroll
      for (int t = 0; t < W; ++t) m0[t] = G.mask[0][t];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        bool pass = gi * 64 + l < sg_n;
#pragma unroll
        for (int t = 0; t < W; ++t) pass = pass && ((sg[gi][t] & m0[t]) == m0[t]);
        qms[gi] = pass ? 1u : 0u;
      }
      for (int j = 1; j < g; ++j) {
        uint64_t mj[W];
#pragma unroll
        for (int t = 0; t < W; ++t) mj[t] = G.mask[j][t];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          bool pass = gi * 64 + l < sg_n;
#pragma unroll
          for (int t = 0; t < W; ++t) pass = pass && ((sg[gi][t] & mj[t]) == mj[t]);
          qms[gi] |= pass ? (1u << j) : 0u;
        }
      }
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const int i = gi * 64 + l;
        const uint32_t qm = qms[gi];
        const uint64_t bal = __ballot(qm != 0u);
        if (qm != 0u) {
          const int o = nw + mbcnt(bal);
          s.wl[buf][o] = (uint16_t)i;
          s.wq[buf][o] = (uint16_t)qm;
        }
        nw += __popcll(bal);
        if (want_stats) {
          for (int j = 0; j < g; ++j) {
            const uint64_t b = __ballot((qm >> j) & 1u);
            elig += l == j ? (uint32_t)__popcll(b) : 0u;
          }
        }
      }
      return nw;
    };
    // Raise member j's bound from its query's histogram: the lower edge of the highest bin at which at
    // least k counted candidates lie at or above (bin 0, everything below the histogram, never
    // counts).  Every candidate is counted once, so a stale read only gives a lower bound.
    auto pull = [&](int j) {
      const int q = G.q[j];
      const int32_t hlo = G.hlo[j], hsh = G.hsh[j];
      constexpr int HPB = kQHistBins / 64;
      uint32_t h[HPB], sum = 0u;
#pragma unroll
      for (int t = 0; t < HPB; ++t) {
        h[t] = __hip_atomic_load(&a.w.ghist[(size_t)q * kQHistBins + HPB * l + t], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        sum += h[t];
      }
      uint32_t suf = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off);
        if (l + off < 64) suf += v;
      }
      uint32_t above = suf - sum;
      int32_t bound = INT32_MIN;
#pragma unroll
      for (int t = HPB - 1; t >= 0; --t) {
        const int bin = HPB * l + t;
        if (bin >= 1 && above < (uint32_t)a.k && above + h[t] >= (uint32_t)a.k) bound = hlo + (bin << hsh);
        above += h[t];
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const int32_t v = __shfl_xor(bound, o);
        bound = v > bound ? v : bound;
      }
      if (l == 0 && bound > G.thr[j]) {
        G.thr[j] = bound;
        atomicMax(&a.w.thr[q], bound);
      }
    };
    // Staged candidates to the pools (one reservation per member, then one slot per candidate) and
    // to their queries' histograms; members that received many pull their bound.
    auto flush = [&]() {
      wave_lds_sync();
      uint32_t c = 0u;
      if (l < g) {
        c = G.scnt[l];
        const uint32_t base = c ? atomicAdd(&a.w.pool_cnt[G.q[l]], c) : 0u;
        G.sbase[l] = base;
        G.scnt[l] = 0u;
      }
      wave_lds_sync();
      for (int e = l; e < stage_n; e += 64) {
        const int j = s.kj[e];
        const uint64_t key = s.key[e];
        const int q = G.q[j];
        const uint32_t at = atomicAdd(&G.sbase[j], 1u);
        if (at < cap) a.w.pool[(size_t)q * cap + at] = key;
        const int32_t sc = (int32_t)((uint32_t)(key >> 32) ^ 0x80000000u), hlo = G.hlo[j];
        int bin = 0;
        if (sc >= hlo) {
          const int32_t bb = (sc - hlo) >> G.hsh[j];
          bin = bb < kQHistBins - 1 ? bb : kQHistBins - 1;
        }
        atomicAdd(&a.w.ghist[(size_t)q * kQHistBins + bin], 1u);
      }
      wave_lds_sync();
      stage_n = 0;
      uint64_t pm = __ballot(c >= (uint32_t)kGPullMin);
      while (pm) {
        const int j = __builtin_ctzll(pm);
        pm &= pm - 1ull;
        pull(j);
      }
      wave_lds_sync();
    };
    int4 x[R];
    auto load_rows = [&](int32_t p0, int buf, int r0, int nrows) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int r = r0 + u * RPI + l / LPR;
        const int32_t p = p0 + (r < nrows ? (int)s.wl[buf][r] : 0);
        x[u] = reinterpret_cast<const int4 *>(a.ix.items + (size_t)p * D)[sub];
      }
    };
    // Score the batch at r0 for every member that accepts each row.  Each row's first member is scored
    // for the whole batch in straight-line code first, so that the wait for the rows sits there (and
    // leaves the signatures requested after them in flight); the loops for further members and the
    // candidate staging follow.
    auto score_rows = [&](int32_t p0, int buf, int r0, int nrows) {
      uint32_t qmv[R];
      int32_t posv[R], acc0[R];
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int r = r0 + u * RPI + l / LPR;
        const bool valid = r < nrows;
        qmv[u] = valid ? (uint32_t)s.wq[buf][r] : 0u;
        posv[u] = p0 + (valid ? (int)s.wl[buf][r] : 0);
        const int j = qmv[u] ? __builtin_ctz(qmv[u]) : 0;
        acc0[u] = group_sum<LPR>(dot16(x[u], G.qv[j][sub], 0));
      }
#pragma unroll
      for (int u = 0; u < R; ++u) {
        uint32_t qm = qmv[u];
        int32_t acc = acc0[u];
        for (;;) {
          if (stage_n > kGStage - RPI) flush();
          const int j = qm ? __builtin_ctz(qm) : 0;
          const bool ok = qm != 0u && sub == 0 && acc >= G.thr[j];
          const uint64_t b = __ballot(ok);
          if (ok) {
            const int e = stage_n + mbcnt(b);
            s.key[e] = pos_key(acc, posv[u]);
            s.kj[e] = (uint8_t)j;
            atomicAdd(&G.scnt[j], 1u);
          }
          stage_n += __popcll(b);
          qm &= qm - 1u;
          if (__ballot(qm != 0u) == 0ull) break;
          const int j2 = qm ? __builtin_ctz(qm) : 0;
          acc = group_sum<LPR>(dot16(x[u], G.qv[j2][sub], 0));
        }
      }
    };

    // After the signatures of the unit's last step: those of the prepared unit's first step when it is
    // ready, else a dummy request.
    int32_t rq_st = lo, rq_end = hi;   // the last request
    auto request_after = [&](int32_t st_next) -> bool {   // returns whether it requested a step of this unit
      const bool own = st_next < hi, pre = !own && pf == 5;
      rq_st = own ? st_next : (pre ? n_lo : lo);
      rq_end = own ? hi : (pre ? n_hi : lo);
      load_sigs(rq_st, rq_end);
      sg_pre = pre;
      return own;
    };
    // --- the unit's steps: iteration i scores step i while step i + 1 is filtered
    if (!sg_pre) load_sigs(lo, hi);
    sg_pre = false;
    int32_t st_sg = lo;   // start of the step whose signatures are in sg
    int n_i = filter(0);
    int32_t p0_i = st_sg;
    bool has_next = request_after(st_sg + kGStep);
    if (has_next) st_sg += kGStep;
    wave_lds_sync();
    load_rows(p0_i, 0, 0, n_i);
    for (int i = 0;; ++i) {
      const int bi = i & 1, bn = bi ^ 1;
      const bool cont = has_next;
      int n_n = 0;
      const int32_t p0_n = st_sg;
      if (cont) {
        n_n = filter(bn);   // waits for step i + 1's signatures; step i's rows keep flying
        has_next = request_after(st_sg + kGStep);
        if (has_next) st_sg += kGStep;
      } else {
        load_sigs(rq_st, rq_end);   // the same request again, so that every iteration issues the same loads
      }
      score_rows(p0_i, bi, 0, n_i);
      for (int r0 = RB; r0 < n_i; r0 += RB) {   // dense filters: further batches
        load_rows(p0_i, bi, r0, n_i);
        score_rows(p0_i, bi, r0, n_i);
      }
      pf_step();
      if (!cont) break;
      wave_lds_sync();
      load_rows(p0_n, bn, 0, n_n);
      n_i = n_n;
      p0_i = p0_n;
    }
    // --- end of the unit
    flush();
    if (want_stats && l < g) {
      const int q = G.q[l];
      atomicAdd((unsigned long long *)&a.w.stats[2 * (size_t)q + 1], (unsigned long long)elig);
      atomicAdd((unsigned long long *)&a.w.stats[2 * (size_t)q], (unsigned long long)(hi - lo));
    }
    while (pf >= 1 && pf <= 4) pf_step();
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

template <int LPR>
static int gscan_occ_w(int W) {
  int n = 0;
  hipError_t e = W == 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gscan<LPR, 2>, kScanThreads, 0)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_gscan<LPR, 1>, kScanThreads, 0);
  return e == hipSuccess ? n : 0;
}

int gscan_blocks_per_cu(int32_t dim, int32_t sig_words) {
  switch (dim) {
    case 16: return gscan_occ_w<1>(sig_words);
    case 32: return gscan_occ_w<2>(sig_words);
    case 64: return gscan_occ_w<4>(sig_words);
    case 128: return gscan_occ_w<8>(sig_words);
    case 256: return gscan_occ_w<16>(sig_words);
    default: return 0;
  }
}

hipError_t launch_gscan(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const SearchShape &sh,
                        const Work &w, hipStream_t s) {
  GScanArgs a{ix, queries, masks, w, sh.B, sh.nprobe, sh.k, sh.GP, (uint32_t)sh.pool_cap};
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
