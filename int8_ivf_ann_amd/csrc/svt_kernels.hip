// svt_kernels.hip - gfx950 kernels of the fused int8 IVF + Bloom-signature top-k search.
//
// Pipeline per svt_search (all on the caller's stream, no host synchronisation):
//   k_coarse_keys   int8 centroid scores for every (query, cluster)
//   k_coarse_select per query: exact top-nprobe clusters (radix select), probe list in cluster order,
//                   per-query item stream layout, filter density and score samples
//   k_plan_*        the work list: every query's stream cut into chunks of about equal estimated cost,
//                   queued by the cluster band they start in
//   k_scan          the fused hot loop: Bloom filter -> int8 dot4 score -> per-workgroup top-k in LDS;
//                   persistent workgroups take chunks from the queue; each chunk leaves at most k keys
//   k_merge         per query: exact top-k over its chunks' keys (radix select), sorted, written out
// The tile path (svt_tile.hip) replaces k_plan_* .. k_merge by a scan that reads each probed cluster once
// per batch; the kernels here then redo the few queries whose candidate pools missed.
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

#include "svt_device.h"
#include "svt_internal.h"

namespace svt {

// ------------------------------------------------------------------------------------------------
// k_coarse_keys: s = <q_b, centroid_c> (int32) for every query b and cluster c; the select forms the
// ordering key (s, c) from it.  One thread per cluster, kCoarseQB queries per workgroup staged in LDS.

template <int LPR>
__global__ __launch_bounds__(256) void k_coarse_keys(const int8_t *__restrict__ centroids, int32_t nlist,
                                                     const int8_t *__restrict__ queries, int32_t B,
                                                     int32_t *__restrict__ scores, uint32_t *counter,
                                                     int32_t *__restrict__ gcnt, int32_t *__restrict__ gfill,
                                                     float *__restrict__ clog) {
  constexpr int D = 16 * LPR;
  __shared__ int4 qs[kCoarseQB][LPR];
  const int tid = threadIdx.x;
  const int b0 = blockIdx.y * kCoarseQB;
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid < 8) counter[tid] = 0u;
  if (gcnt && blockIdx.y == 0 && blockIdx.x * 256 + tid < nlist) {   // tile path: per-cluster counters
    gcnt[blockIdx.x * 256 + tid] = 0;
    gfill[blockIdx.x * 256 + tid] = 0;
    clog[blockIdx.x * 256 + tid] = 0.f;
  }
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
    scores[(size_t)b * nlist + c] = acc;
  }
}

// ------------------------------------------------------------------------------------------------
// k_coarse_select: one workgroup per query.
//   probes[b][0..nprobe): the nprobe clusters with the largest keys, in ascending cluster id
//   seg[b][j]: offset of probed cluster j in query b's item stream; seg[b][nprobe] = qlen[b]
//   qcost[b]: estimated bytes the scan moves for the query: signatures of every probed item plus the
//             rows of the fraction of kCostSamples evenly spaced probed items that pass the filter
// The work list follows in four small kernels (k_plan_*): every query's stream is cut into chunks of
// about equal estimated cost, so that a dense filter does not leave one workgroup with far more bytes.

// <x, q> over NCH 16-byte parts, every part requested before any is used
template <int NCH>
__device__ __forceinline__ int32_t row_dot(const int4 *__restrict__ x, const int4 *__restrict__ q) {
  int4 xv[NCH], qv[NCH];
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    xv[ch] = x[ch];
    qv[ch] = q[ch];
  }
  int32_t s = 0;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) s = dot16(xv[ch], qv[ch], s);
  return s;
}

constexpr int kSelKR = 16;   // coarse keys a select thread keeps in registers (nlist <= kSelThreads * kSelKR)
constexpr int kSelTwoLevel = kSelSegLds / 2 / kSelKR;   // largest nprobe the two-level selection stages

// thr_mode (tile path): 0 no speculative threshold, 1 estimate it from the samples, 2 set it above every
// score (every query with an eligible item is then redone on the query path)
__global__ __launch_bounds__(kSelThreads) void k_coarse_select(DevIndex ix, const int8_t *__restrict__ queries,
                                                                const uint64_t *__restrict__ masks, int32_t G,
                                                                int32_t GT, int32_t B, int32_t nprobe, int32_t k,
                                                                int32_t pool_cap, int32_t thr_mode, Work w) {
  constexpr int NWV = kSelThreads / 64;
  __shared__ SelScratch sel;
  __shared__ int wave_tot[NWV + 1];
  __shared__ int64_t wave_tot64[NWV + 1];
  __shared__ int32_t seg_lds[kSelSegLds + 1];   // the probed clusters, then their stream offsets
  __shared__ union {
    int32_t pb[kSelSegLds];                        // position base of each probed cluster
    uint64_t cand[kSelSegLds / 2];                 // candidates of the two-level selection
  } su;
  __shared__ int ncand_s;
  __shared__ int32_t tcnt[kSelKR * NWV];         // probed clusters per (register slot, wave)
  __shared__ int smax_s;
  __shared__ int32_t tail_s;                     // stream offset of the first probed cluster in the tail bands
  __shared__ unsigned long long live_s;          // live items of the probed clusters
  __shared__ struct {
    int32_t pos[kSelElig];                       // tile path: eligible samples (position, score)
    int32_t sc[kSelElig];
  } se;
  const int tid = threadIdx.x, l = lane_id(), wv = tid / 64;
  const int b = blockIdx.x;
  const int nlist = ix.nlist;
  const int32_t *row = w.coarse_scores + (size_t)b * nlist;
  int32_t *probes = w.probes + (size_t)b * nprobe;
  int32_t *seg = w.seg + (size_t)b * (nprobe + 1);
  int32_t *pb = w.pb + (size_t)b * nprobe;
  const bool in_lds = nprobe <= kSelSegLds;
  const int32_t c_tail = (int32_t)(((int64_t)kTailBand * nlist + kPlanBands - 1) / kPlanBands);
  if (tid == 0) {
    tail_s = INT32_MAX;
    live_s = 0ull;
  }
  int run = 0;   // items of the query's stream
  int64_t my_live = 0;   // live items of the probed clusters this thread visits
  if (nprobe == nlist) {
    // every cluster probed: the probe list is every cluster in order, the stream is the position order
    for (int r = tid; r < nlist; r += kSelThreads) {
      const int32_t o0 = ix.offsets[r];
      my_live += ix.live[r];
      probes[r] = r;
      seg[r] = o0;
      pb[r] = 0;
      if (in_lds) {
        seg_lds[r] = o0;
        su.pb[r] = 0;
      }
    }
    run = ix.offsets[nlist];
    if (tid == 0 && c_tail < nlist) tail_s = ix.offsets[c_tail];
  } else {
  // --- the nprobe largest keys (keys are distinct: the cluster id is part of them)
  uint64_t T = 0;
  if (nlist <= kSelThreads * kSelKR) {
    // keys of clusters tid + i * kSelThreads held in registers; 0 marks a missing cluster (no key is 0)
    uint64_t kr[kSelKR];
#pragma unroll
    for (int i = 0; i < kSelKR; ++i) {
      const int c = i * kSelThreads + tid;
      kr[i] = c < nlist ? make_key(row[c], (uint32_t)c) : 0ull;
    }
    const int nthr = nlist < kSelThreads ? nlist : kSelThreads;   // threads holding at least one key
    if (nprobe < nlist && nprobe <= kSelTwoLevel && nprobe <= nthr) {
      // Two levels.  The nprobe largest of the threads' largest keys are nprobe distinct keys, so the
      // smallest of them, T1, is at or below the nprobe-th largest key: only the nprobe threads whose
      // largest key reaches T1 hold keys >= T1.  Those (at most nprobe * kSelKR) are staged in LDS and
      // the exact selection runs over them.
      uint64_t tmax = 0ull;
#pragma unroll
      for (int i = 0; i < kSelKR; ++i) tmax = kr[i] > tmax ? kr[i] : tmax;
      const uint64_t T1 = block_select<kSelThreads>(
          [&](auto f) {
            if (tmax != 0ull) f(tmax);
          },
          nprobe, sel);
      if (tid == 0) ncand_s = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kSelKR; ++i) {
        const bool take = kr[i] != 0ull && kr[i] >= T1;
        const uint64_t bal = __ballot(take);
        int base = 0;
        if (l == 0 && bal) base = atomicAdd(&ncand_s, __popcll(bal));
        base = __shfl(base, 0);
        if (take) su.cand[base + mbcnt(bal)] = kr[i];
      }
      __syncthreads();
      const int nc = ncand_s;
      T = block_select<kSelThreads>(
          [&](auto f) {
            for (int j = tid; j < nc; j += kSelThreads) f(su.cand[j]);
          },
          nprobe, sel);
      // the threshold separates the candidates only; every other key lies below T1
      T = T > T1 ? T : T1;
      __syncthreads();   // su.cand is reused for the position bases below
    } else if (nprobe < nlist) {
      T = block_select<kSelThreads>(
          [&](auto f) {
#pragma unroll
            for (int i = 0; i < kSelKR; ++i)
              if (i * kSelThreads + tid < nlist) f(kr[i]);
          },
          nprobe, sel);
    }
    // probe list in one pass: a probed cluster's rank is its order by id (register slot, wave, lane)
    uint64_t bal[kSelKR];
#pragma unroll
    for (int i = 0; i < kSelKR; ++i) {
      bal[i] = __ballot(kr[i] != 0ull && kr[i] >= T);
      if (l == 0) tcnt[i * NWV + wv] = __popcll(bal[i]);
    }
    __syncthreads();
    if (wv == 0) {   // exclusive prefix of the kSelKR * NWV counts (in slot-major order)
      constexpr int PL = kSelKR * NWV / 64;
      int v[PL], sum = 0;
#pragma unroll
      for (int u = 0; u < PL; ++u) { v[u] = tcnt[PL * l + u]; sum += v[u]; }
      int run = wave_incl_scan(sum) - sum;
#pragma unroll
      for (int u = 0; u < PL; ++u) { tcnt[PL * l + u] = run; run += v[u]; }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSelKR; ++i) {
      if ((bal[i] >> l) & 1ull) {
        const int r = tcnt[i * NWV + wv] + mbcnt(bal[i]);
        if (r < nprobe) {
          probes[r] = i * kSelThreads + tid;
          if (in_lds) seg_lds[r] = i * kSelThreads + tid;   // the cluster, until its offset replaces it
        }
      }
    }
  } else {
    if (nprobe < nlist) {
      T = block_select<kSelThreads>(
          [&](auto f) {
            for (int c = tid; c < nlist; c += kSelThreads) f(make_key(row[c], (uint32_t)c));
          },
          nprobe, sel);
    }
    int base = 0;
    for (int c0 = 0; c0 < nlist; c0 += kSelThreads) {
      const int c = c0 + tid;
      const bool take = c < nlist && make_key(row[c], (uint32_t)c) >= T;
      int cnt_tot;
      const int idx = block_excl_scan<kSelThreads>(take ? 1 : 0, wave_tot, &cnt_tot);
      if (take && base + idx < nprobe) {
        probes[base + idx] = c;
        if (in_lds) seg_lds[base + idx] = c;
      }
      base += cnt_tot;
    }
  }
  __syncthreads();
  // --- stream offsets: prefix of the probed clusters' sizes in probe order
  for (int r0 = 0; r0 < nprobe; r0 += kSelThreads) {
    const int r = r0 + tid;
    int32_t c = 0, o0 = 0, sz = 0;
    if (r < nprobe) {
      c = in_lds ? seg_lds[r] : probes[r];
      o0 = ix.offsets[c];
      sz = ix.offsets[c + 1] - o0;
      my_live += ix.live[c];
    }
    int tot;
    const int pre = block_excl_scan<kSelThreads>(sz, wave_tot, &tot);
    if (r < nprobe) {
      if (c >= c_tail) atomicMin(&tail_s, run + pre);   // probes ascend, so the first such cluster
      seg[r] = run + pre;
      pb[r] = o0 - (run + pre);
      if (in_lds) {
        seg_lds[r] = run + pre;
        su.pb[r] = o0 - (run + pre);
      }
    }
    run += tot;
  }
  }   // nprobe < nlist
  {
    // the items the search scans for this query: the live items of its probed clusters (the stream also
    // holds the free slots of an updatable index, which no filter passes)
    unsigned long long v = (unsigned long long)my_live;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    __syncthreads();
    if (l == 0 && v) atomicAdd(&live_s, v);
    __syncthreads();
  }
  if (tid == 0) {
    seg[nprobe] = run;
    if (in_lds) seg_lds[nprobe] = run;
    w.qlen[b] = run;
    w.thr[b] = INT32_MIN;
    w.mcnt[b] = 0u;
    if (w.pool_cnt) w.pool_cnt[b] = 0u;
    if (w.stats) { w.stats[2 * (size_t)b] = (int64_t)live_s; w.stats[2 * (size_t)b + 1] = 0; }
  }
  __syncthreads();
  // Evenly spaced samples of the query's probed items: their filter density sizes the query's share of
  // the work list; their scores place the query's score histogram (the bins sit between the mean
  // sample score and twice the largest margin above it).
  //   Query path: one sample per thread, every sample scored.
  //   Tile path: m samples per thread, m growing with the stream (one more per kSampleSpan items, at
  //   most kSampleMax), so that the threshold below rests on enough eligible samples.  The signatures of
  //   a thread's samples are requested together; the eligible samples are compacted in LDS (every
  //   stride-th of them when there are more than kSelElig) and scored by all threads, one row each in
  //   most cases; the histogram sits on their scores.
  const int m = thr_mode == 0 ? 1 : (int)((run + kSampleSpan - 1) / kSampleSpan < kSampleMax
                                              ? ((run + kSampleSpan - 1) / kSampleSpan > 1 ? (run + kSampleSpan - 1) / kSampleSpan : 1)
                                              : kSampleMax);
  const int n_samp = m * kCostSamples;
  const int4 *qr = reinterpret_cast<const int4 *>(queries + (size_t)b * ix.dim);
  auto score_at = [&](int32_t pos) -> int32_t {
    const int4 *xr = reinterpret_cast<const int4 *>(ix.items + (size_t)pos * ix.dim);
    switch (ix.dim) {
      case 16: return row_dot<1>(xr, qr);
      case 32: return row_dot<2>(xr, qr);
      case 64: return row_dot<4>(xr, qr);
      case 128: return row_dot<8>(xr, qr);
      default: return row_dot<16>(xr, qr);
    }
  };
  uint32_t hitm = 0u;        // bit i: sample i of this thread is eligible
  int32_t pos[kSampleMax];
  int have = 0;
  int64_t ssum_t = 0;
  int32_t mx = INT32_MIN;
  if (run > 0) {
    uint64_t mk[kMaxGroups][2];   // the query's G masks (a sample is eligible under any of them)
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g) {
      mk[g][0] = g < G ? masks[((size_t)b * G + g) * ix.sig_words] : 0ull;
      mk[g][1] = (g < G && ix.sig_words == 2) ? masks[((size_t)b * G + g) * ix.sig_words + 1] : 0ull;
    }
    uint64_t sgv[kSampleMax][2];
    int32_t sc0 = 0;
#pragma unroll
    for (int i = 0; i < kSampleMax; ++i) {
      if (i == 0 || i < m) {
        // sample j = i * kSelThreads + tid of n_samp
        const int j = i * kSelThreads + tid;
        const int32_t t = (int32_t)((int64_t)j * run / n_samp);
        if (nprobe == nlist) {
          pos[i] = t;   // every cluster probed, in id order: the stream is the position order
        } else {
          int lo = 0, hi = nprobe - 1;   // largest j with seg[j] <= t
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            const int32_t sv = in_lds ? seg_lds[mid] : seg[mid];
            if (sv <= t) lo = mid; else hi = mid - 1;
          }
          pos[i] = (in_lds ? su.pb[lo] : pb[lo]) + t;
        }
        const uint64_t *sg = ix.sigs + (size_t)pos[i] * ix.sig_words;
        sgv[i][0] = sg[0];
        sgv[i][1] = ix.sig_words == 2 ? sg[1] : 0ull;
        // query path: its one sample is scored whether it passes or not; the row is requested together
        // with the signature
        if (i == 0 && thr_mode == 0) sc0 = score_at(pos[0]);
      } else {   // a thread draws m samples; the rest are never tested
        pos[i] = pos[0];
        sgv[i][0] = sgv[0][0];
        sgv[i][1] = sgv[0][1];
      }
    }
#pragma unroll
    for (int i = 0; i < kSampleMax; ++i) {
      bool any = false;
#pragma unroll
      for (int g = 0; g < kMaxGroups; ++g)
        any = any || (g < G && (sgv[i][0] & mk[g][0]) == mk[g][0] && (sgv[i][1] & mk[g][1]) == mk[g][1]);
      const bool ok = i < m && any && sig_live(sgv[i][0], sgv[i][1], ix.sig_words);
      hitm |= ok ? 1u << i : 0u;
    }
    if (thr_mode == 0) {   // query path: every sample scored
      have = 1;
      ssum_t = sc0;
      mx = sc0;
    }
  }
  const int hit = __popc(hitm);
  int hits;
  const int hoff = block_excl_scan<kSelThreads>(hit, wave_tot, &hits);
  // tile path: the eligible samples compacted in LDS (every stride-th one), then scored
  const int stride = hits > kSelElig ? (hits + kSelElig - 1) / kSelElig : 1;
  const int n_el = (hits + stride - 1) / stride;
  if (thr_mode != 0) {
    int rk = hoff;
#pragma unroll
    for (int i = 0; i < kSampleMax; ++i)
      if ((hitm >> i) & 1u) {
        if (rk % stride == 0) se.pos[rk / stride] = pos[i];
        ++rk;
      }
    __syncthreads();
    for (int e = tid; e < n_el; e += kSelThreads) {
      const int32_t sc = score_at(se.pos[e]);
      se.sc[e] = sc;
      ++have;
      ssum_t += sc;
      mx = sc > mx ? sc : mx;
    }
  }
  if (tid == 0) smax_s = INT32_MIN;
  int haves;
  block_excl_scan<kSelThreads>(have, wave_tot, &haves);
  int64_t ssum;
  block_excl_scan<kSelThreads>(ssum_t, wave_tot64, &ssum);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int32_t t2 = __shfl_xor(mx, o);
    mx = t2 > mx ? t2 : mx;
  }
  if (l == 0) atomicMax(&smax_s, mx);
  for (int i = tid; i < kQHistBins; i += kSelThreads) w.ghist[(size_t)b * kQHistBins + i] = 0u;
  if (thr_mode != 0) {
    // Tile path: the speculative threshold.  The samples are evenly spaced over the query's stream, so
    // r eligible samples at or above a score stand for about r * run / n_samp eligible items (each kept
    // sample stands for stride eligible samples): the r-th best kept score, r for kAlpha * k items (at
    // least kRMin), is the threshold.  A stream the pool can hold whole needs none.  The choice only
    // decides how many candidates the pool receives; a pool that ends below k or above its capacity
    // sends the query to the query path.
    int32_t st = INT32_MIN;
    if (run > pool_cap) {
      const int64_t r0 = ((int64_t)kAlpha * k * n_samp + (int64_t)run * stride - 1) / ((int64_t)run * stride);
      const int r = (int)(r0 > kRMin ? r0 : kRMin);
      if (n_el >= r) {
        __syncthreads();   // se.sc complete
        const uint64_t T = block_select<kSelThreads>(
            [&](auto f) {
              for (int e = tid; e < n_el; e += kSelThreads) f(make_key(se.sc[e], (uint32_t)e));
            },
            r, sel);
        st = key_score(T);
      }
    }
    if (thr_mode == 2) st = INT32_MAX;
    if (tid == 0) w.sthr[b] = st;
  }
  __syncthreads();
  if (tid == 0) {
    const double dens = (double)hits / n_samp;
    if (w.qdens) w.qdens[b] = (float)dens;
    w.qcost[b] = (int64_t)((double)run * (8.0 * ix.sig_words + dens * ix.dim + kItemCost)) + 1;
    w.qtail[2 * (size_t)b] = tail_s < run ? tail_s : run;
    int32_t lo = 0, shift = 0;
    if (haves > 0) {
      lo = (int32_t)(ssum / haves);
      const int64_t hi = (int64_t)smax_s + ((int64_t)smax_s - lo) + 1;
      const uint32_t range = (uint32_t)(hi - lo);
      const int bits = range ? 32 - __clz((int)range) : 0;
      shift = bits > 8 ? bits - 8 : 0;                        // (range >> shift) < kQHistBins
    }
    w.hlo[b] = lo;
    w.hshift[b] = shift;
  }
  // Tile path (w.gcnt set): the query's GT members of each probed cluster are counted, and the log of
  // the fraction of the cluster's items the query does not accept (its sampled density; members taken
  // as independent) is added to the cluster's.  gcnt and clog are zeroed by k_coarse_keys.
  if (w.gcnt) {
    const float dens = (float)((double)hits / n_samp);
    const float lg = log1pf(-(dens < 0.999f ? dens : 0.999f));
    for (int j = tid; j < nprobe; j += kSelThreads) {
      const int c = probes[j];
      atomicAdd(&w.gcnt[c], GT);
      atomicAdd(&w.clog[c], lg);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// The work list.  k_plan_count (one workgroup): the target cost of a chunk from the batch's total
// estimated cost, every query's chunk count and length, and where its chunks start (cstart).
// k_plan_chunks (one workgroup per query, one thread per chunk): each chunk's stream range, the probed
// cluster it starts in and that cluster's band (1/256 of the cluster ids).  k_plan_order (one workgroup): the queue,
// chunks grouped by band, so that chunks of different queries that read the same clusters run at about
// the same time and the second reader finds the data in cache (Infinity Cache: every XCD works through
// the same bands at the same time).  k_plan_small runs the three in one workgroup for batches of a few
// queries, where the launches, not the work, set the stage's time.

// Tile path (redo != 0): a pool proves its query's top k when it holds every candidate it was offered and
// either its threshold admitted every eligible item or at least k candidates reached it (then the k-th
// best score is at or above the threshold, so the top k are all in the pool); every other query is marked
// for redo and only those get chunks.
__device__ __forceinline__ void plan_count(int32_t B, int32_t P, const Work &w, int32_t redo, int32_t k,
                                           uint32_t pool_cap) {
  __shared__ int wave_tot[kSelThreads / 64 + 1];
  __shared__ int64_t wave_tot64[kSelThreads / 64 + 1];
  const int tid = threadIdx.x;
  auto marked = [&](int i) -> bool {   // tile path: query i is redone
    const uint32_t c = w.pool_cnt[i];
    return !(c <= pool_cap && (c >= (uint32_t)k || w.sthr[i] == INT32_MIN));
  };
  int64_t total = 0;
  for (int i0 = 0; i0 < B; i0 += kSelThreads) {
    const int i = i0 + tid;
    int64_t tot;
    bool take = i < B;
    if (take && redo) {
      take = marked(i);
      w.redo[i] = take ? 1 : 0;
    }
    block_excl_scan<kSelThreads>(take ? w.qcost[i] : (int64_t)0, wave_tot64, &tot);
    total += tot;
  }
  // target cost of one chunk: four chunks per workgroup; when that is small, one chunk per workgroup
  // (up to four minimum chunks), since a chunk's set-up and end then outweigh its items; never less than
  // the minimum chunk
  const int64_t tc_four = (total + 4 * (int64_t)P - 1) / (4 * (int64_t)P);
  const int64_t tc_one = (total + P - 1) / P;
  const int64_t tc_small = tc_one < 4 * kMinChunkCost ? tc_one : 4 * kMinChunkCost;
  int64_t Tc = tc_four > tc_small ? tc_four : tc_small;
  Tc = Tc > kMinChunkCost ? Tc : kMinChunkCost;
  int32_t carry = 0;
  for (int i0 = 0; i0 < B; i0 += kSelThreads) {
    const int i = i0 + tid;
    int32_t nch = 0;
    if (i < B) {
      // tile path: only the queries marked for redo get chunks
      const bool skip = redo && !marked(i);
      const int64_t len = skip ? 0 : w.qlen[i], cost = w.qcost[i];
      const int64_t ta = w.qtail[2 * (size_t)i];   // [0, ta): regular chunks; [ta, len): shorter ones
      int32_t na = 0;
      if (len > 0) {
        int64_t cl = (Tc * len + cost - 1) / cost;                          // items of one chunk
        // each region is cut into at most half the chunks a query may have when there are two
        const int64_t per = ta < len ? kMaxChunksPerQuery / 2 : kMaxChunksPerQuery;
        const int64_t cl_min = (len + per - 1) / per;
        cl = cl > cl_min ? cl : cl_min;
        cl = ((cl + 63) / 64) * 64;
        cl = cl < len ? cl : len;
        na = ta > 0 ? (int32_t)((ta + cl - 1) / cl) : 0;
        int32_t nb = 0;
        if (ta < len) {
          int64_t clb = ((cl + kTailDiv - 1) / kTailDiv + 63) / 64 * 64;
          clb = clb > cl_min ? clb : cl_min;
          nb = (int32_t)((len - ta + clb - 1) / clb);
        }
        nch = na + nb;
      }
      w.qtail[2 * (size_t)i + 1] = na;
    }
    int32_t tot;
    const int32_t ex = block_excl_scan<kSelThreads>(nch, wave_tot, &tot);
    if (i < B) w.cstart[i] = carry + ex;
    carry += tot;
  }
  if (tid == 0) w.cstart[B] = carry;
}

__global__ __launch_bounds__(kSelThreads) void k_plan_count(int32_t B, int32_t P, Work w, int32_t redo, int32_t k,
                                                             uint32_t pool_cap) {
  plan_count(B, P, w, redo, k, pool_cap);
}

// The chunks of query q, by NT threads (tid: this thread's index among them).  STAGED: all threads of the
// workgroup call it, and the query's stream offsets are staged in sseg (kSelSegLds + 1 ints of LDS) when
// they fit; otherwise (one wave) they are searched in global memory and no barrier is met.
template <int NT, bool STAGED>
__device__ __forceinline__ void plan_chunks(int q, int tid, int32_t nprobe, int32_t nlist, const Work &w,
                                            int32_t *sseg) {
  const int32_t c0 = w.cstart[q], nch = w.cstart[q + 1] - c0;
  if (nch == 0) return;
  const int64_t len = w.qlen[q], ta = w.qtail[2 * (size_t)q];
  const int32_t na = w.qtail[2 * (size_t)q + 1], nb = nch - na;
  const int32_t *sq = w.seg + (size_t)q * (nprobe + 1);
  const int32_t *pq = w.probes + (size_t)q * nprobe;
  const bool in_lds = STAGED && nprobe <= kSelSegLds;
  if (STAGED) {
    if (in_lds)
      for (int i = tid; i <= nprobe; i += NT) sseg[i] = sq[i];
    __syncthreads();
  }
  // Each region holds its chunks of ceil(region length / chunks) items: none is empty, since that never
  // exceeds the length chosen for the region.
  const int64_t cla = na > 0 ? (ta + na - 1) / na : 0;
  const int64_t clb = nb > 0 ? (len - ta + nb - 1) / nb : 0;
  for (int i = tid; i < nch; i += NT) {
    int64_t l0, l1;
    if (i < na) {
      l0 = (int64_t)i * cla;
      l1 = l0 + cla < ta ? l0 + cla : ta;
    } else {
      l0 = ta + (int64_t)(i - na) * clb;
      l1 = l0 + clb < len ? l0 + clb : len;
    }
    // the probed cluster holding stream offset l0: the largest j with seg[j] <= l0 (empty clusters
    // before it share its offset and are skipped)
    int lo = 0, hi = nprobe - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      const int32_t sv = in_lds ? sseg[mid] : sq[mid];
      if (sv <= l0) lo = mid; else hi = mid - 1;
    }
    w.chunks[c0 + i] = Chunk{q, (int32_t)l0, (int32_t)l1, lo};
    w.cband[c0 + i] = (int)(((int64_t)pq[lo] * kPlanBands) / nlist);
  }
}

__global__ __launch_bounds__(256) void k_plan_chunks(int32_t B, int32_t nprobe, int32_t nlist, Work w) {
  __shared__ int32_t sseg[kSelSegLds + 1];   // the query's stream offsets, when they fit
  plan_chunks<256, true>(blockIdx.x, threadIdx.x, nprobe, nlist, w, sseg);
}

// The queue: a counting sort of the chunks by band.  Inside a band the chunks follow a scattered order
// (scatter_index), which interleaves the queries: consecutive queue entries then belong to different
// queries, so the workgroups running at the same time read the same clusters for different queries
// (measured: both one query's chunks together and chunk order make the scan slower).  The sort is stable
// over that order: wave w of the one workgroup owns scattered positions [w * per, (w + 1) * per); it
// counts their chunks per band, every (wave, band) gets its start from the band totals and the counts of
// the waves before it, and the wave places its chunks, ranking the lanes of a 64-position group that
// share a band with ballots on the band's bits.
__device__ __forceinline__ void plan_order(int32_t B, const Work &w) {
  constexpr int NWV = kSelThreads / 64;
  constexpr int BB = 8;                              // bits of a band
  static_assert(kPlanBands == 1 << BB, "bands are ranked with one ballot per band bit");
  __shared__ uint32_t cnt[NWV][kPlanBands];          // per wave: chunks per band, then next position
  __shared__ uint32_t wave_tot[NWV + 1];
  const int tid = threadIdx.x, l = lane_id(), wv = tid / 64;
  const int n = w.cstart[B];
  const int per = ((n + NWV - 1) / NWV + 63) / 64 * 64;
  const int c_lo = wv * per, c_hi = c_lo + per < n ? c_lo + per : n;
  for (int i = tid; i < NWV * kPlanBands; i += kSelThreads) cnt[i / kPlanBands][i % kPlanBands] = 0u;
  __syncthreads();
  for (int p = c_lo + l; p < c_hi; p += 64) atomicAdd(&cnt[wv][w.cband[scatter_index(p, n)]], 1u);
  __syncthreads();
  // band totals -> band starts (threads of the first kPlanBands), then each wave's start per band
  uint32_t tot = 0u;
  if (tid < kPlanBands)
    for (int v = 0; v < NWV; ++v) tot += cnt[v][tid];
  uint32_t all;
  uint32_t run = block_excl_scan<kSelThreads>(tot, wave_tot, &all);
  if (tid < kPlanBands)
    for (int v = 0; v < NWV; ++v) {
      const uint32_t x = cnt[v][tid];
      cnt[v][tid] = run;
      run += x;
    }
  __syncthreads();
  // each wave places its chunks in order
  for (int c0 = c_lo; c0 < c_hi; c0 += 64) {
    const bool have = c0 + l < c_hi;
    const int c = have ? scatter_index(c0 + l, n) : 0;
    const int b = have ? w.cband[c] : 0;
    uint64_t eq = __ballot(have);
#pragma unroll
    for (int k = 0; k < BB; ++k) {
      const uint64_t m = __ballot((b >> k) & 1);
      eq &= ((b >> k) & 1) ? m : ~m;
    }
    const int rank = mbcnt(eq);
    uint32_t pos = 0u;
    if (have) pos = cnt[wv][b] + (uint32_t)rank;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (have) w.order[pos] = c;
    if (have && rank == 0) cnt[wv][b] += (uint32_t)__popcll(eq);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

__global__ __launch_bounds__(kSelThreads) void k_plan_order(int32_t B, Work w) { plan_order(B, w); }

// The whole work list of a small batch (query path) in one workgroup: counts, each query's chunks in
// turn, the queue.  Each phase reads what the one before wrote to global memory; the workgroup barrier
// between them orders those accesses, since every thread of a workgroup sees global memory through the
// same compute unit.
__global__ __launch_bounds__(kSelThreads) void k_plan_small(int32_t B, int32_t P, int32_t nprobe, int32_t nlist,
                                                             int32_t k, Work w) {
  __shared__ int32_t sseg[kSelSegLds + 1];
  plan_count(B, P, w, 0, k, 0u);
  __syncthreads();
  for (int q = 0; q < B; ++q) {
    plan_chunks<kSelThreads, true>(q, threadIdx.x, nprobe, nlist, w, sseg);
    __syncthreads();   // sseg is reused by the next query
  }
  plan_order(B, w);
}

// The tile path's redo work list in one workgroup: the queries whose pools cannot prove their top k are
// marked and counted (plan_count), each wave cuts the chunks of the marked queries among its share
// (queries wave + 16 j), one at a time, and the queue is built.  Usually no query is marked, and this one
// launch replaces three.
__global__ __launch_bounds__(kSelThreads) void k_plan_redo(int32_t B, int32_t P, int32_t nprobe, int32_t nlist,
                                                            int32_t k, uint32_t pool_cap, Work w) {
  constexpr int NWV = kSelThreads / 64;
  const int l = lane_id(), wv = threadIdx.x / 64;
  plan_count(B, P, w, 1, k, pool_cap);
  __syncthreads();
  for (int base = 0; base < B; base += NWV * 64) {
    const int qi = base + l * NWV + wv;
    uint64_t m = __ballot(qi < B && w.redo[qi] != 0);
    while (m) {
      const int bit = __ffsll((long long)m) - 1;
      m &= m - 1ull;
      plan_chunks<64, false>(base + bit * NWV + wv, l, nprobe, nlist, w, nullptr);
    }
  }
  __syncthreads();
  plan_order(B, w);
}

// ------------------------------------------------------------------------------------------------
// k_scan: the fused filter -> score -> select hot loop.
//
// A query's stream is the concatenation of the items of its probed clusters (seg).  The work list
// cuts every stream into chunks of about equal estimated cost and orders them by the clusters they start
// in; persistent workgroups take chunks in that order with an atomic counter (one chunk ahead) and walk
// each chunk in steps of kScanStep items.
// In a step each wave loads 64 kScanGroups signatures (one 128- or 64-bit load per lane per 64-item group), tests
// (sig & mask) == mask, ballots the result and compacts the survivors' offsets into LDS; it then
// gathers the rows of its survivors (LPR lanes per row, 16-byte loads, about kScanRowBatch rows at once) and
// scores them with v_dot4.  The next step's signatures and the query's current bound are requested
// right after the rows, so a step costs one memory round trip.
// A candidate enters the workgroup's LDS list if it scores at least the best proven bound known to the
// wave; whenever the list could overflow it is cut back towards k by an LDS trim.  Accepted scores are
// also counted in a per-query histogram in HBM shared by all chunks of the query: as soon as k counted
// candidates lie at or above a bin's lower edge, that edge is a proven bound for the whole query.
// At the end of a chunk the workgroup writes the chunk's exact top k keys above the bound to slot c.
// Nothing per item is ever written to HBM.

struct ScanArgs {
  DevIndex ix;
  const int8_t *queries;
  const uint64_t *masks;
  Work w;
  int32_t B, nprobe, k, P;
  // redo of the tile path: only the queries marked for redo have chunks; their statistics were already
  // counted by the tile scan
  int32_t fallback;
  int32_t G;   // masks per query: an item passes when it passes any of them
};

struct ScanLds {
  uint64_t list[kListCap];
  // survivor offsets of three consecutive steps (step i in wl[i % 3], wave w's at [w * 256, ...)); the
  // buffer of step i - 1 is free while step i is scored and serves as scratch of trims and selects
  uint16_t wl[3][kScanThreads * kScanGroups];
  int wave_tot[kScanThreads / 64 + 1];
  unsigned long long kmin;
  uint32_t smin, smax;
  int cnt, cut_bin, cut_above;   // cnt: slot allocation counter of the list
  // keys each wave appended in a step, by step parity: the list length after a step is computed from
  // these by every thread, never read from cnt, which faster waves may already be advancing
  int wadd[2][kScanThreads / 64];
  int wcnt[2][kScanThreads / 64];   // survivors each wave found in a step, by step parity
  // window of the chunk's probed clusters: stream range [t0, t1) and position base (pos = pb + t)
  int32_t seg_t0[kSegWin], seg_t1[kSegWin], seg_pb[kSegWin];
  int seg_n;
  uint32_t qh[kQHistBins];   // scores of candidates accepted since the last push to the query's histogram
  int32_t gbound;            // the query's bound as read once for the whole block
  int next;                  // queue position of this workgroup's next chunk
};

// Keep the keys >= T of list[0..cnt) (T from block_select), in place; returns the count kept and the
// smallest kept key in *kmin_out.  Two rounds over halves of the list keep the register footprint at
// half a list: a round reads its half into registers, then (after a barrier) writes the kept keys at
// or below positions every thread has already read.
__device__ __forceinline__ int keep_at_least(ScanLds &sm, int cnt, uint64_t T, uint64_t *kmin_out) {
  constexpr int HALF = kListCap / 2, PER = HALF / kScanThreads;
  const int tid = threadIdx.x, l = lane_id();
  if (tid == 0) sm.kmin = ~0ull;
  unsigned long long mn = ~0ull;
  int base = 0;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    uint64_t mine[PER];
    int keep = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = r * HALF + tid + u * kScanThreads;
      mine[u] = i < cnt ? sm.list[i] : 0ull;
      keep += (i < cnt && mine[u] >= T) ? 1 : 0;
    }
    int tot;
    int off = base + block_excl_scan<kScanThreads>(keep, sm.wave_tot, &tot);   // barriers inside
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = r * HALF + tid + u * kScanThreads;
      if (i < cnt && mine[u] >= T) {
        sm.list[off++] = mine[u];
        mn = mine[u] < mn ? mine[u] : mn;
      }
    }
    base += tot;
    __syncthreads();
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long t = __shfl_xor(mn, o);
    mn = t < mn ? t : mn;
  }
  if (l == 0) atomicMin(&sm.kmin, mn);
  __syncthreads();
  *kmin_out = sm.kmin;
  __syncthreads();
  return base;
}

// Score-only trim of a list of pos_keys holding more than k keys: histogram the biased scores into
// kTrimBins bins over [min, max], find the bin b* at which the count from the top reaches k and drop
// every key below b*'s lower edge s*.  At least k keys have score >= s*, so no dropped key can be in
// the top k; ties at the edge are all kept.  Returns the count kept; *edge receives s* (biased).
__device__ __forceinline__ int trim_by_score(ScanLds &sm, int cnt, int k, uint32_t *edge, uint32_t *hist) {
  const int tid = threadIdx.x, l = lane_id();
  if (tid == 0) { sm.smin = ~0u; sm.smax = 0u; }
  __syncthreads();
  uint32_t lmin = ~0u, lmax = 0u;
  for (int i = tid; i < cnt; i += kScanThreads) {
    const uint32_t s = (uint32_t)(sm.list[i] >> 32);
    lmin = s < lmin ? s : lmin;
    lmax = s > lmax ? s : lmax;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t a = __shfl_xor(lmin, o), b = __shfl_xor(lmax, o);
    lmin = a < lmin ? a : lmin;
    lmax = b > lmax ? b : lmax;
  }
  if (l == 0) { atomicMin(&sm.smin, lmin); atomicMax(&sm.smax, lmax); }
  for (int i = tid; i < kTrimBins; i += kScanThreads) hist[i] = 0u;
  __syncthreads();
  const uint32_t smin = sm.smin, range = sm.smax - smin;
  const int bits = range ? 32 - __clz(range) : 0;            // range < 2^bits
  const int shift = bits > kTrimBinsLog2 ? bits - kTrimBinsLog2 : 0;   // (range >> shift) < kTrimBins
  for (int i = tid; i < cnt; i += kScanThreads)
    atomicAdd(&hist[((uint32_t)(sm.list[i] >> 32) - smin) >> shift], 1u);
  __syncthreads();
  if (tid < 64) {
    constexpr int PB = kTrimBins / 64;
    uint32_t h[PB], sum = 0;
#pragma unroll
    for (int j = 0; j < PB; ++j) { h[j] = hist[PB * l + j]; sum += h[j]; }
    uint32_t suf = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      uint32_t v = __shfl_down(suf, off);
      if (l + off < 64) suf += v;
    }
    uint32_t above = suf - sum;
#pragma unroll
    for (int j = PB - 1; j >= 0; --j) {
      if (above < (uint32_t)k && above + h[j] >= (uint32_t)k) { sm.cut_bin = PB * l + j; sm.cut_above = (int)above; }
      above += h[j];
    }
  }
  __syncthreads();
  const uint32_t e = smin + ((uint32_t)sm.cut_bin << shift);
  *edge = e;
  uint64_t dummy;
  return keep_at_least(sm, cnt, (uint64_t)e << 32, &dummy);
}

// Replace the pos_keys list[from..cnt) by their (score, id) ordering keys.  The position -> id loads
// of a thread are issued in groups of 8 before any is used.
__device__ __forceinline__ void to_id_keys(ScanLds &sm, int from, int cnt, const int32_t *__restrict__ perm) {
  constexpr int PER = 8;
  const int tid = threadIdx.x;
  for (int i0 = from; i0 < cnt; i0 += PER * kScanThreads) {
    uint32_t id[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = i0 + tid + u * kScanThreads;
      id[u] = i < cnt ? (uint32_t)perm[(uint32_t)sm.list[i]] : 0u;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = i0 + tid + u * kScanThreads;
      if (i < cnt) sm.list[i] = make_key((int32_t)((uint32_t)(sm.list[i] >> 32) ^ 0x80000000u), id[u]);
    }
  }
  __syncthreads();
}

// State of a chunk's candidate list that the cold paths below update.  Normally the list holds
// pos_keys only (id_n == 0).  When score ties at the trim edge keep the list too long, the list is
// switched to exact (score, id) keys and cut to exactly k: from then on list[0..id_n) are id keys and
// the candidates appended after them are pos_keys, converted at the next trim.
struct ListState {
  int32_t thr_s;   // proven bound of the workgroup
  int id_n;        // leading keys of the list that are (score, id) keys
};

// Cut an over-full list back towards k (rare: the bounds reject most candidates).  All threads call
// it; returns the count kept.
__device__ __forceinline__ int trim_list(ScanLds &sm, int cnt, int k, const int32_t *__restrict__ perm,
                                         ListState &st, uint32_t *scratch) {
  const int tid = threadIdx.x;
  int kept = cnt;
  if (st.id_n == 0) {
    uint32_t edge;
    kept = trim_by_score(sm, cnt, k, &edge, scratch);
    const int32_t es = (int32_t)(edge ^ 0x80000000u);
    st.thr_s = es > st.thr_s ? es : st.thr_s;
    if (kept <= kTrimAt) return kept;
  }
  // exact: (score, id) keys throughout, then exactly the k best
  to_id_keys(sm, st.id_n, kept, perm);
  const uint64_t T = block_select<kScanThreads>(
      [&](auto f) {
        for (int i = tid; i < kept; i += kScanThreads) f(sm.list[i]);
      },
      k, *reinterpret_cast<SelScratch *>(scratch));
  uint64_t tk;
  kept = keep_at_least(sm, kept, T, &tk);
  const int32_t ks = key_score(tk);
  st.thr_s = ks > st.thr_s ? ks : st.thr_s;
  st.id_n = kept;
  return kept;
}

// End of a chunk: drop keys below the bound gb, turn the rest into (score, id) keys and cut them to the
// exact top k; *kth receives the smallest kept key when exactly k remain (0 otherwise).  Keys below the
// bound go before the position -> id lookups, so that only survivors pay for them; both key kinds hold
// the biased score in their upper half, so one threshold serves either.  All threads call it; returns
// the count kept.
__device__ __forceinline__ int finish_list(ScanLds &sm, int cnt, int k, int id_n, int32_t gb,
                                           const int32_t *__restrict__ perm, int32_t *thr_q, uint64_t *kth_out,
                                           uint32_t *scratch) {
  const int tid = threadIdx.x, l = lane_id();
  uint64_t kth = 0;
  if (id_n > 0) {   // rare (score ties at a trim): the list already starts with id keys; convert the rest
    to_id_keys(sm, id_n, cnt, perm);
    id_n = cnt;
  }
  if (gb != INT32_MIN) cnt = keep_at_least(sm, cnt, (uint64_t)((uint32_t)gb ^ 0x80000000u) << 32, &kth);
  if (id_n == 0) to_id_keys(sm, 0, cnt, perm);   // ends with a barrier
  if (cnt > k) {
    const uint64_t T = block_select<kScanThreads>(
        [&](auto f) {
          for (int i = tid; i < cnt; i += kScanThreads) f(sm.list[i]);
        },
        k, *reinterpret_cast<SelScratch *>(scratch));
    cnt = keep_at_least(sm, cnt, T, &kth);
    if (tid == 0) atomicMax(thr_q, key_score(kth));
  } else if (cnt == k) {
    if (tid == 0) sm.kmin = ~0ull;
    __syncthreads();
    unsigned long long mn = ~0ull;
    for (int i = tid; i < cnt; i += kScanThreads) mn = sm.list[i] < mn ? sm.list[i] : mn;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      unsigned long long t = __shfl_xor(mn, o);
      mn = t < mn ? t : mn;
    }
    if (l == 0) atomicMin(&sm.kmin, mn);
    __syncthreads();
    kth = sm.kmin;
  }
  *kth_out = cnt == k ? kth : 0ull;
  return cnt;
}

// Three workgroups per CU (168 VGPRs a wave): the pipeline holds a step's rows and the next step's
// signatures in registers across the filter, and spills at four per CU would add waits on every load.
template <int LPR, int W>
__global__ __launch_bounds__(kScanThreads, kScanOcc) void k_scan(ScanArgs a) {
  constexpr int D = 16 * LPR;
  constexpr int RPI = 64 / LPR;                   // rows covered by one 16-byte load per lane
  constexpr int R0 = kScanRowBatch / RPI;
  constexpr int R = R0 < 1 ? 1 : (R0 > 8 ? 8 : R0);   // row loads per lane in one batch (1 to 8)
  constexpr int RB = R * RPI;                     // rows a wave requests together
  __shared__ ScanLds sm;
  const int tid = threadIdx.x, l = lane_id(), wv = tid / 64, sub = l % LPR;
  const int k = a.k;
  const int n_chunks = a.w.cstart[a.B];
  // Persistent workgroups take chunks from the work list until it is empty.  Queue positions: the first
  // two of workgroup i are i and P + i (P workgroups), later ones P * 2 + the counter's next value.  Fixed
  // first claims keep every workgroup from waiting on one counter address at the start, where the
  // atomics of all P workgroups would arrive together and be served one after another.
  const int P = (int)gridDim.x;
  if (tid == 0) sm.next = (int)blockIdx.x;
  __syncthreads();
  int claims = 1;   // positions claimed so far (uniform)
  for (;;) {
    const int qpos = __builtin_amdgcn_readfirstlane(sm.next);
    if (qpos >= n_chunks) break;
    const int c = a.w.order[qpos];
    // the chunk after this one, requested now so the request is answered by the time it is needed
    int next_c = 0;
    if (tid == 0)
      next_c = claims == 1 ? P + (int)blockIdx.x : 2 * P + (int)atomicAdd(&a.w.counter[1], 1u);
    ++claims;
    const Chunk ch = a.w.chunks[c];
    const int q = ch.q;
    const int32_t ra = ch.lo, rb = ch.hi;
    const int32_t hlo = a.w.hlo[q];
    const int hsh = a.w.hshift[q];
    uint32_t *gh = a.w.ghist + (size_t)q * kQHistBins;
    int32_t *thr_q = a.w.thr + q;
    // query vector slice held by this lane, request mask
    const int4 qv = reinterpret_cast<const int4 *>(a.queries + (size_t)q * D)[sub];
    uint64_t mk[kMaxGroups][W];   // the query's masks (groups past G are never tested)
#pragma unroll
    for (int g = 0; g < kMaxGroups; ++g)
#pragma unroll
      for (int i = 0; i < W; ++i) mk[g][i] = g < a.G ? a.masks[((size_t)q * a.G + g) * W + i] : 0ull;
    for (int i = tid; i < kQHistBins; i += kScanThreads) sm.qh[i] = 0u;
    if (tid == 0) sm.cnt = 0;
    // thr_s: proven bound of this workgroup (trims, histogram pulls); gthr: the query's global bound
    // as last read
    int32_t thr_s = INT32_MIN, gthr = __hip_atomic_load(thr_q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int id_n = 0;
    int64_t n_elig = 0;
    const int32_t *seg = a.w.seg + (size_t)q * (a.nprobe + 1);
    const int32_t *pbq = a.w.pb + (size_t)q * a.nprobe;
    // Steps walk the chunk's probed clusters in order.  The clusters are staged in LDS (kSegWin at a
    // time) so that walking them never waits on vector memory.
    struct Cursor {
      int w;            // entry in the LDS window; -1: chunk finished
      int32_t st, t1;   // step start / cluster end, in stream offsets
      int32_t pbase;    // position = pbase + stream offset (positions < 2^31)
    };
    int jwin = ch.j0;   // first probed cluster of the current window
    auto load_window = [&]() {   // all threads; entries jwin .. (first cluster at or past rb)
      __syncthreads();
      if (tid == 0) sm.seg_n = 0;
      __syncthreads();
      for (int i = tid; i < kSegWin && jwin + i < a.nprobe; i += kScanThreads) {
        const int j = jwin + i;
        const int32_t s0 = seg[j], s1 = seg[j + 1];
        if (s0 < rb) {
          sm.seg_t0[i] = ra > s0 ? ra : s0;
          sm.seg_t1[i] = rb < s1 ? rb : s1;
          sm.seg_pb[i] = pbq[j];
          atomicMax(&sm.seg_n, i + 1);
        }
      }
      __syncthreads();
    };
    auto seek = [&](Cursor &cu) {   // from entry cu.w: first entry with items left in [ra, rb)
      for (;;) {
        for (; cu.w < sm.seg_n; ++cu.w) {
          const int32_t t0 = sm.seg_t0[cu.w], t1 = sm.seg_t1[cu.w];
          if (t0 < t1) {
            cu.st = t0; cu.t1 = t1; cu.pbase = sm.seg_pb[cu.w];
            return;
          }
        }
        // window exhausted: another one if the chunk continues past it
        if (sm.seg_n < kSegWin || jwin + kSegWin >= a.nprobe || seg[jwin + kSegWin] >= rb) { cu.w = -1; return; }
        jwin += kSegWin;
        load_window();
        cu.w = 0;
      }
    };
    auto advance = [&](Cursor &cu) {
      cu.st += kScanStep;
      if (cu.st >= cu.t1) { ++cu.w; seek(cu); }
    };
    // bin of a score in the query's histogram: bin 0 holds everything below hlo + 2^hsh, bin b >= 1
    // holds [hlo + b 2^hsh, hlo + (b+1) 2^hsh), the last bin everything above
    auto qbin = [&](int32_t score) -> int {
      if (score < hlo) return 0;
      const int32_t b = (score - hlo) >> hsh;
      return b < kQHistBins - 1 ? b : kQHistBins - 1;
    };
    // Histogram exchange in two halves so that neither waits on memory.  push (all threads, after the
    // step's barrier) adds the counts accepted since the last push to the query's histogram; pull
    // (wave 0) requests the histogram with the next step's loads and, once they have arrived, raises the
    // bound to the lower edge of the highest bin at which at least k counted candidates lie at or above.
    // Every accepted candidate is counted exactly once, so the bound is proven whatever the
    // interleaving; a stale read only yields a lower bound.
    auto hist_push = [&]() {
      for (int i = tid; i < kQHistBins; i += kScanThreads) {
        const uint32_t v = atomicExch(&sm.qh[i], 0u);
        if (v) atomicAdd(&gh[i], v);
      }
    };
    constexpr int HPB = kQHistBins / 64;   // histogram bins per lane of wave 0
    uint32_t hq[HPB];
    auto hist_pull_issue = [&]() {
#pragma unroll
      for (int j = 0; j < HPB; ++j)
        hq[j] = __hip_atomic_load(&gh[HPB * l + j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    auto hist_pull_use = [&]() {   // wave 0 only
      uint32_t sum = 0;
#pragma unroll
      for (int j = 0; j < HPB; ++j) sum += hq[j];
      uint32_t suf = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_down(suf, off);
        if (l + off < 64) suf += v;
      }
      uint32_t above = suf - sum;
      int32_t bound = INT32_MIN;
#pragma unroll
      for (int j = HPB - 1; j >= 0; --j) {
        const int bin = HPB * l + j;
        if (bin >= 1 && above < (uint32_t)k && above + hq[j] >= (uint32_t)k) bound = hlo + (bin << hsh);
        above += hq[j];
      }
      if (bound != INT32_MIN) atomicMax(thr_q, bound);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const int32_t t = __shfl_xor(bound, o);
        bound = t > bound ? t : bound;
      }
      thr_s = bound > thr_s ? bound : thr_s;
    };
    // Loads are issued unconditionally (out-of-range lanes read an in-range clamped address and are
    // masked afterwards), so the compiler can count outstanding loads exactly and wait only for the
    // ones it needs: the rows of this step, not the signatures already requested for the next.
    uint64_t sg[kScanGroups][W];
    int32_t sg_n = 0, sg_p0 = 0;
    auto load_sigs = [&](const Cursor &cu) {
      sg_n = cu.w >= 0 ? ((cu.t1 - cu.st) < kScanStep ? (cu.t1 - cu.st) : kScanStep) : 0;
      const int32_t p0 = cu.w >= 0 ? cu.pbase + cu.st : 0;
      sg_p0 = p0;
      const int32_t last = sg_n > 0 ? sg_n - 1 : 0;
#pragma unroll
      for (int gi = 0; gi < kScanGroups; ++gi) {
        const int i = gi * kScanThreads + wv * 64 + l;
        const int32_t p = p0 + (i < last ? i : last);
        if constexpr (W == 2) {
          const ulonglong2 v = reinterpret_cast<const ulonglong2 *>(a.ix.sigs)[p];
          sg[gi][0] = v.x; sg[gi][1] = v.y;
        } else {
          sg[gi][0] = a.ix.sigs[p];
        }
      }
    };
    // --- The steps of the chunk run as a pipeline.  Iteration i filters step i + 1 (its signatures were
    // requested an iteration earlier), requests the signatures of step i + 2, passes the step barrier,
    // then scores step i, whose rows were requested at the end of iteration i - 1, and requests the rows
    // of step i + 1.  A row gather thus overlaps the next filter and barrier instead of stalling the
    // step.  Survivor lists rotate through three LDS buffers (step i in wl[i % 3]); after the barrier of
    // iteration i every wave has finished scoring step i - 1, so the list length through step i - 1 is
    // known to every thread (per-wave append counts) and the buffer of step i - 1 is free scratch.
    constexpr int NWV = kScanThreads / 64;
    struct Share {           // wave wv scores survivors [rbeg, rend) of a step's concatenated lists
      int pre[NWV + 1];
      int rbeg, rend;
    };
    auto share = [&](int par) -> Share {
      Share s;
      s.pre[0] = 0;
#pragma unroll
      for (int i = 0; i < NWV; ++i) s.pre[i + 1] = s.pre[i] + sm.wcnt[par][i];
      const int total = s.pre[NWV];
      const int per = (total + NWV - 1) / NWV;
      s.rbeg = wv * per;
      s.rend = s.rbeg + per < total ? s.rbeg + per : total;
      return s;
    };
    auto surv_at = [&](const Share &s, int r) -> int {   // index of survivor r in its buffer
      int adj = 0;
#pragma unroll
      for (int i = 1; i < NWV; ++i) adj = r >= s.pre[i] ? i * 64 * kScanGroups - s.pre[i] : adj;
      return r + adj;
    };
    auto filter = [&](int buf) -> int {   // the step in sg into wl[buf]; returns this wave's survivors
      int nw = 0;
#pragma unroll
      for (int gi = 0; gi < kScanGroups; ++gi) {
        const int i = gi * kScanThreads + wv * 64 + l;
        bool any = true;
#pragma unroll
        for (int u = 0; u < W; ++u) any = any && ((sg[gi][u] & mk[0][u]) == mk[0][u]);
#pragma unroll
        for (int g = 1; g < kMaxGroups; ++g) {
          if (g < a.G) {
            bool pg = true;
#pragma unroll
            for (int u = 0; u < W; ++u) pg = pg && ((sg[gi][u] & mk[g][u]) == mk[g][u]);
            any = any || pg;
          }
        }
        const bool pass = i < sg_n && any && sig_live(sg[gi][0], sg[gi][W - 1], W);
        const uint64_t bal = __ballot(pass);
        if (pass) sm.wl[buf][wv * 64 * kScanGroups + nw + mbcnt(bal)] = (uint16_t)i;
        nw += __popcll(bal);
      }
      return nw;
    };
    int4 x[R];
    auto load_rows = [&](int32_t p0, int buf, const Share &s, int r0) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int r = r0 + u * RPI + l / LPR;
        const int32_t p = p0 + (r < s.rend ? (int)sm.wl[buf][surv_at(s, r)] : 0);
        x[u] = reinterpret_cast<const int4 *>(a.ix.items + (size_t)p * D)[sub];
      }
    };
    // score the batch at r0.  The wave's accepted candidates take their list slots with one LDS atomic;
    // a candidate's slot is its rank among them (ballots over the rows of the batch in turn).
    auto score_rows = [&](int32_t p0, int buf, const Share &s, int r0, int32_t thr_eff) -> int {
      uint32_t okm = 0;
      int32_t sc[R];
      int tot = 0;
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int32_t acc = group_sum<LPR>(dot16(x[u], qv, 0));
        const int r = r0 + u * RPI + l / LPR;
        sc[u] = acc;
        const bool ok = sub == 0 && r < s.rend && acc >= thr_eff;
        okm |= ok ? 1u << u : 0u;
        tot += __popcll(__ballot(ok));
      }
      if (tot == 0) return 0;
      int at = 0;
      if (l == 0) at = atomicAdd(&sm.cnt, tot);
      at = __builtin_amdgcn_readfirstlane(at);
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const bool ok = (okm >> u) & 1u;
        const uint64_t b = __ballot(ok);
        if (ok) {
          const int r = r0 + u * RPI + l / LPR;
          sm.list[at + mbcnt(b)] = pos_key(sc[u], p0 + (int)sm.wl[buf][surv_at(s, r)]);
          atomicAdd(&sm.qh[qbin(sc[u])], 1u);
        }
        at += __popcll(b);
      }
      return tot;
    };
    load_window();
    int steps = 0, cnt_base = 0;   // cnt_base: list length through the last step counted
    bool pull = false;
    Cursor cur{0, 0, 0, 0};
    seek(cur);
    // prologue: step 0 filtered, step 1's signatures requested, step 0's first rows requested
    load_sigs(cur);
    Cursor cur_sg = cur;   // the step whose signatures are in sg
    if (cur.w >= 0) advance(cur);
    int32_t p0_i = sg_p0;
    {
      const int nw = filter(0);
      n_elig += nw;
      if (l == 0) sm.wcnt[0][wv] = nw;
    }
    load_sigs(cur);
    cur_sg = cur;
    if (cur.w >= 0) advance(cur);
    __syncthreads();
    Share sh_i = share(0);
    if (sh_i.rbeg < sh_i.rend) load_rows(p0_i, 0, sh_i, sh_i.rbeg);
    int32_t gthr_next = gthr;
    for (int i = 0;; ++i) {
      const bool more = sg_n > 0;   // step i + 1 exists (the same for every thread)
      const int32_t p0_n = sg_p0;
      const int bi = i % 3, bn = (i + 1) % 3, bf = (i + 2) % 3;
      if (more) {
        const int nw = filter(bn);   // waits for step i + 1's signatures; step i's rows keep flying
        n_elig += nw;
        if (l == 0) sm.wcnt[(i + 1) & 1][wv] = nw;
        // the query's global bound and histogram, on exchange steps only
        if (pull) {
          gthr_next = __hip_atomic_load(thr_q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (wv == 0) hist_pull_issue();
        }
        load_sigs(cur);
        cur_sg = cur;
        if (cur.w >= 0) advance(cur);
      }
      __syncthreads();
      // list length through step i - 1; trim when step i's appends could overflow the list
      if (i >= 1) {
#pragma unroll
        for (int w2 = 0; w2 < NWV; ++w2) cnt_base += sm.wadd[(i - 1) & 1][w2];
      }
      if (cnt_base > kTrimAt) {
        ListState st{thr_s, id_n};
        const int kept = trim_list(sm, cnt_base, k, a.ix.perm, st, reinterpret_cast<uint32_t *>(sm.wl[bf]));
        cnt_base = kept;
        thr_s = st.thr_s;
        id_n = st.id_n;
        if (tid == 0) {
          sm.cnt = kept;
          atomicMax(thr_q, thr_s);   // at least k candidates score >= thr_s
        }
        __syncthreads();
        // rows and signatures in flight are requested again rather than held in registers across the trim
        if (sh_i.rbeg < sh_i.rend) load_rows(p0_i, bi, sh_i, sh_i.rbeg);
        load_sigs(cur_sg);
      }
      Share sh_n;
      if (more) sh_n = share((i + 1) & 1);
      // --- score step i
      const int32_t thr_eff = gthr > thr_s ? gthr : thr_s;
      int wtot = sh_i.rbeg < sh_i.rend ? score_rows(p0_i, bi, sh_i, sh_i.rbeg, thr_eff) : 0;
      for (int r0 = sh_i.rbeg + RB; r0 < sh_i.rend; r0 += RB) {   // dense filters: further batches
        load_rows(p0_i, bi, sh_i, r0);
        wtot += score_rows(p0_i, bi, sh_i, r0, thr_eff);
      }
      if (l == 0) sm.wadd[i & 1][wv] = wtot;
      if (pull && more) {
        gthr = gthr_next;
        if (wv == 0) hist_pull_use();
        pull = false;
      }
      // histogram exchange after steps 2, 4, 8, ...: the bound converges within a few exchanges
      ++steps;
      if (steps >= 2 && (steps & (steps - 1)) == 0) {
        hist_push();
        pull = true;
      }
      if (!more) break;
      if (sh_n.rbeg < sh_n.rend) load_rows(p0_n, bn, sh_n, sh_n.rbeg);   // step i + 1's first rows
      sh_i = sh_n;
      p0_i = p0_n;
    }
    __syncthreads();
    {
      // the last step's appends (counted at no later barrier)
      int last = 0;
#pragma unroll
      for (int w2 = 0; w2 < NWV; ++w2) last += sm.wadd[steps & 1 ? 0 : 1][w2];
      cnt_base += last;
    }
    // --- end of the chunk: its exact top k above the query's bound, published in slot c
    hist_push();
    // keys below the query's bound cannot be in its top k.  The branches below contain barriers, so
    // the block uses one value of the bound, read by one thread.
    if (tid == 0) sm.gbound = gthr > thr_s ? gthr : thr_s;
    __syncthreads();
    const int32_t gb = sm.gbound;
    uint64_t kth;
    const int cnt = finish_list(sm, cnt_base, k, id_n, gb, a.ix.perm, thr_q, &kth, reinterpret_cast<uint32_t *>(sm.wl[0]));
    uint64_t *dst = a.w.slot_keys + (size_t)c * (size_t)k;
    for (int i = tid; i < cnt; i += kScanThreads) dst[i] = sm.list[i];
    if (tid == 0) {
      a.w.slot_cnt[c] = cnt;
      // a full slot proves k keys >= its smallest one
      a.w.slot_min[c] = kth;
      sm.next = next_c;
    }
    // per-query counter: items that passed the filter (n_elig is uniform across the wave: one add per
    // wave); the scanned items are counted by k_coarse_select
    if (a.w.stats && !a.fallback) {
      if (l == 0) atomicAdd((unsigned long long *)&a.w.stats[2 * (size_t)q + 1], (unsigned long long)n_elig);
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------------------------------
// Before the merge.  k_merge_gather (persistent workgroups, one slot at a time): the keys of every slot
// at or above its query's final bound, compacted per query with one atomic per slot (the counts start at
// zero from the coarse select).  Every chunk has pushed the candidates it accepted to its query's score
// histogram, so the histogram is final; the lower edge of the highest bin at which at least k counted
// candidates lie at or above is a proven bound on the k-th score (at least k items score that much), as
// is the query's running bound.  A query's top k is among the gathered keys: its true top k all score at
// least the bound.

// The final bound of query q as the smallest key it admits (0: none), by one whole wave; every lane
// returns it.
__device__ __forceinline__ uint64_t merge_bound_key(const Work &w, int q, int32_t k) {
  constexpr int HPB = kQHistBins / 64;
  const int l = lane_id();
  const uint32_t *gh = w.ghist + (size_t)q * kQHistBins;
  uint32_t h[HPB], sum = 0;
#pragma unroll
  for (int j = 0; j < HPB; ++j) { h[j] = gh[HPB * l + j]; sum += h[j]; }
  uint32_t suf = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_down(suf, off);
    if (l + off < 64) suf += v;
  }
  uint32_t above = suf - sum;   // counted candidates in the bins above this lane's
  const int32_t hlo = w.hlo[q];
  const int hsh = w.hshift[q];
  int32_t bound = INT32_MIN;
#pragma unroll
  for (int j = HPB - 1; j >= 0; --j) {
    const int bin = HPB * l + j;
    if (bin >= 1 && above < (uint32_t)k && above + h[j] >= (uint32_t)k) bound = hlo + (bin << hsh);
    above += h[j];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int32_t t = __shfl_xor(bound, o);
    bound = t > bound ? t : bound;
  }
  const int32_t g = w.thr[q];
  bound = g > bound ? g : bound;
  return bound == INT32_MIN ? 0ull : make_key(bound, 0xFFFFFFFFu);   // smallest key of that score
}

__global__ __launch_bounds__(256) void k_merge_gather(Work w, int32_t B, int32_t k, uint32_t cap) {
  constexpr int PER = kMaxK / 256;   // a slot holds at most k <= kMaxK keys: one pass of PER per thread
  __shared__ int wave_tot[256 / 64 + 1];
  __shared__ uint32_t sbase;
  __shared__ unsigned long long sbound;
  const int tid = threadIdx.x;
  const int n = w.cstart[B];
  for (int c = blockIdx.x; c < n; c += gridDim.x) {
    const int q = w.chunks[c].q;
    const int cnt = w.slot_cnt[c];
    const uint64_t *keys = w.slot_keys + (size_t)c * k;
    uint64_t v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = u * 256 + tid;
      v[u] = i < cnt ? keys[i] : 0ull;   // valid keys are never 0
    }
    if (tid < 64) {   // wave 0: the query's bound, while the slot's keys arrive
      const uint64_t b = merge_bound_key(w, q, k);
      if (tid == 0) sbound = b;
    }
    __syncthreads();
    const uint64_t T = sbound;
    int take = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) take += v[u] >= T && v[u] != 0ull ? 1 : 0;
    int tot;
    int off = block_excl_scan<256>(take, wave_tot, &tot);   // barriers inside
    if (tid == 0) sbase = tot > 0 ? atomicAdd(&w.mcnt[q], (uint32_t)tot) : 0u;
    __syncthreads();
    const uint32_t base = sbase;
    uint64_t *dst = w.mkeys + (size_t)q * kGatherCap;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      if (v[u] >= T && v[u] != 0ull) {
        const uint32_t o = base + (uint32_t)off++;
        if (o < cap) dst[o] = v[u];
      }
    }
    __syncthreads();   // sbase and wave_tot are reused for the next slot
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
  int32_t fallback;     // redo of the tile path: only the queries marked for redo are merged here
  uint32_t gather_cap;  // keys gathered per query; a query with more is merged from its slots
  int64_t *out_ids;
  int32_t *out_scores;
  float *out_fscores;
  int32_t *out_counts;
};

__global__ __launch_bounds__(kSelThreads) void k_merge(MergeArgs a) {
  constexpr int kBins = 2048;
  __shared__ SelScratch sel;
  __shared__ union {
    uint64_t cand[kMergeCap];
    uint32_t hist[kBins];
  } mu;
  __shared__ int sprefix[kMaxChunksPerQuery];
  __shared__ int wave_tot[kSelThreads / 64 + 1];
  __shared__ int ncand, cut_bin;
  __shared__ unsigned long long bound;
  __shared__ uint32_t smin, smax;
  uint64_t *cand = mu.cand;
  const int tid = threadIdx.x, l = lane_id();
  const int q = blockIdx.x;
  const int k = a.k;
  if (a.fallback && a.w.redo[q] == 0) return;   // merged from its pool
  // the query's chunks, hence its slots, are cstart[q] .. cstart[q+1]-1 (contiguous in memory)
  const size_t s0 = (size_t)a.w.cstart[q];
  const int ns = a.w.cstart[q + 1] - a.w.cstart[q];
  if (tid == 0) { ncand = 0; bound = 0ull; smin = ~0u; smax = 0u; }
  __syncthreads();
  // The keys gathered above the query's final bound hold its top k.  When all of them were kept
  // (flat), they are the candidates, read as one array; otherwise the slots are read.
  const uint32_t gathered = a.fallback ? ~0u : a.w.mcnt[q];
  const bool flat = gathered <= a.gather_cap;
  const uint64_t *gk = a.w.mkeys + (size_t)q * kGatherCap;
  // 1. counts and a proven lower bound on the k-th key: the largest smallest-key of a full slot
  unsigned long long lb = 0ull;
  int total = flat ? (int)gathered : 0;
  for (int i0 = 0; i0 < (flat ? 0 : ns); i0 += kSelThreads) {
    const int i = i0 + tid;
    const int c = i < ns ? a.w.slot_cnt[s0 + i] : 0;
    if (c == k) {
      const uint64_t m = a.w.slot_min[s0 + i];
      lb = m > lb ? m : lb;
    }
    int tot;
    const int ex = block_excl_scan<kSelThreads>(c, wave_tot, &tot);   // barriers inside
    if (i < ns) sprefix[i] = total + ex;
    total += tot;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    unsigned long long t = __shfl_xor(lb, o);
    lb = t > lb ? t : lb;
  }
  if (l == 0) atomicMax(&bound, lb);
  __syncthreads();
  uint64_t T = total > k ? (uint64_t)bound : 0ull;
  if (!flat && total > k) {
    // every chunk is done: the query's global score bound is final
    const int32_t g = a.w.thr[q];
    if (g != INT32_MIN) {
      const uint64_t gk = make_key(g, 0xFFFFFFFFu);   // smallest key with score g
      T = gk > T ? gk : T;
    }
  }
  // keys >= lo of all slots, visited as one flat range over the valid keys (sprefix[s] = keys before
  // slot s), eight loads in flight per thread
  const uint64_t *keys = a.w.slot_keys + s0 * (size_t)k;
  auto key_at = [&](int f) -> uint64_t {   // f-th valid key, 0 <= f < total
    if (flat) return gk[f];
    int lo = 0, hi = ns - 1;                 // largest slot with sprefix <= f
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sprefix[mid] <= f) lo = mid; else hi = mid - 1;
    }
    return keys[(size_t)lo * k + (f - sprefix[lo])];
  };
  auto visit = [&](uint64_t lo, auto f) {
    for (int i0 = tid; i0 < total; i0 += kSelThreads * 8) {
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * kSelThreads;
        v[u] = i < total ? key_at(i) : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u * kSelThreads < total && v[u] >= lo) f(v[u]);
    }
  };
  // 2. stage the keys >= T in LDS (one LDS atomic per wave); ncand counts them all
  auto stage = [&]() {
    for (int i0 = tid - l; i0 < total; i0 += kSelThreads * 8) {   // wave-uniform trip count
      uint64_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + l + u * kSelThreads;
        v[u] = i < total ? key_at(i) : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool take = i0 + l + u * kSelThreads < total && v[u] >= T;
        const uint64_t bal = __ballot(take);
        int base = 0;
        if (l == 0 && bal) base = atomicAdd(&ncand, __popcll(bal));
        base = __shfl(base, 0);
        const int o = base + mbcnt(bal);
        if (take && o < kMergeCap) cand[o] = v[u];
      }
    }
  };
  stage();
  __syncthreads();
  if (ncand > kMergeCap) {
    // 3. too many for LDS: pin the k-th key's score to one bin of a score histogram over [min, max]
    // and stage again above its lower edge
    uint32_t lmin = ~0u, lmax = 0u;
    visit(T, [&](uint64_t key) {
      const uint32_t sc = (uint32_t)(key >> 32);
      lmin = sc < lmin ? sc : lmin;
      lmax = sc > lmax ? sc : lmax;
    });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      uint32_t x = __shfl_xor(lmin, o), y = __shfl_xor(lmax, o);
      lmin = x < lmin ? x : lmin;
      lmax = y > lmax ? y : lmax;
    }
    if (l == 0) { atomicMin(&smin, lmin); atomicMax(&smax, lmax); }
    for (int i = tid; i < kBins; i += kSelThreads) mu.hist[i] = 0u;
    __syncthreads();
    const uint32_t bmin = smin, range = smax - smin;
    const int bits = range ? 32 - __clz(range) : 0;
    const int shift = bits > 11 ? bits - 11 : 0;          // (range >> shift) < kBins
    visit(T, [&](uint64_t key) { atomicAdd(&mu.hist[((uint32_t)(key >> 32) - bmin) >> shift], 1u); });
    __syncthreads();
    if (tid < 64) {
      constexpr int PB = kBins / 64;
      uint32_t h[PB], sum = 0;
#pragma unroll
      for (int j = 0; j < PB; ++j) { h[j] = mu.hist[PB * l + j]; sum += h[j]; }
      uint32_t suf = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        uint32_t v = __shfl_down(suf, off);
        if (l + off < 64) suf += v;
      }
      uint32_t above = suf - sum;
#pragma unroll
      for (int j = PB - 1; j >= 0; --j) {
        if (above < (uint32_t)k && above + h[j] >= (uint32_t)k) cut_bin = PB * l + j;
        above += h[j];
      }
    }
    __syncthreads();
    // at least k keys have a score >= the edge of the cut bin: smaller keys cannot be in the top k
    const uint32_t edge = bmin + ((uint32_t)cut_bin << shift);
    const uint64_t ek = (uint64_t)edge << 32;
    T = ek > T ? ek : T;
    __syncthreads();   // hist and cand share LDS
    if (tid == 0) ncand = 0;
    __syncthreads();
    stage();
  }
  __syncthreads();
  int n = ncand;
  // gathered keys: the slots' keys at or above the final bound, which include the query's top k (or all of
  // its candidates, when it has fewer than k)
  const int nout = total < k ? total : k;
  if (n > kMergeCap) {
    // the cut bin alone overflows LDS (heavy ties): select over the slots in global memory
    const uint64_t Tk = block_select<kSelThreads>([&](auto f) { visit(T, f); }, k, sel);
    if (tid == 0) ncand = 0;
    __syncthreads();
    visit(Tk, [&](uint64_t key) {
      const int o = atomicAdd(&ncand, 1);
      if (o < kMergeCap) cand[o] = key;
    });
    __syncthreads();
    n = nout;
  } else if (n > k) {
    // exact top k in LDS, compacted in place through registers
    const uint64_t Tk = block_select<kSelThreads>(
        [&](auto f) {
          for (int i = tid; i < n; i += kSelThreads) f(cand[i]);
        },
        k, sel);
    constexpr int PER = kMergeCap / kSelThreads;
    uint64_t mine[PER];
    int keep = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSelThreads;
      mine[u] = i < n ? cand[i] : 0ull;
      keep += (i < n && mine[u] >= Tk) ? 1 : 0;
    }
    int tot;
    int off = block_excl_scan<kSelThreads>(keep, wave_tot, &tot);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * kSelThreads;
      if (i < n && mine[u] >= Tk) cand[off++] = mine[u];
    }
    __syncthreads();
    n = tot;
  }
  // 4. sort the n (= nout) winners and write the query's row
  static_assert(kMergeCap >= 4 * kSelThreads, "emit_sorted needs room for 4 keys per thread");
  emit_sorted<kSelThreads>(cand, n, nout, q, k, a.query_scales, a.item_scale, a.out_ids, a.out_scores, a.out_fscores);
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

// Updates of an updatable index, one thread per 16-byte chunk of a row ("SilverTorch - Index as Model",
// index freshness section: a stream of small in-place updates to the index tensors between snapshots).
// Insert: the row, signature and id go to the free slot the host chose, the cluster's live count grows.
// Delete: the slot's signature becomes the free-slot signature (every bit set) and its id -1.  Re-sign:
// the slot's signature is replaced.  Every update of one batch writes a different slot.
__global__ __launch_bounds__(256) void k_updates(int8_t *__restrict__ items, uint64_t *__restrict__ sigs,
                                                 int32_t *__restrict__ perm, int32_t *__restrict__ live,
                                                 int32_t *__restrict__ slot_of, const UpdOp *__restrict__ ops, int32_t n,
                                                 const int8_t *__restrict__ rows, const uint64_t *__restrict__ new_sigs,
                                                 int32_t chunks, int32_t sig_words) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t i = t / chunks;
  const int c = (int)(t % chunks);
  if (i >= n) return;
  const UpdOp op = ops[i];
  const int64_t p = op.pos;
  if (op.kind == kUpdInsert)   // rows is NULL unless the batch inserts
    reinterpret_cast<int4 *>(items)[p * chunks + c] = reinterpret_cast<const int4 *>(rows)[i * chunks + c];
  if (op.kind == kUpdDelete) {
    for (int u = c; u < sig_words; u += chunks) sigs[p * sig_words + u] = ~0ull;
  } else {   // new_sigs is NULL in a batch of deletes only
    for (int u = c; u < sig_words; u += chunks) sigs[p * sig_words + u] = new_sigs[i * sig_words + u];
  }
  if (c == 0) {
    if (op.kind == kUpdInsert) {
      perm[p] = op.id;
      slot_of[op.id] = (int32_t)p;
      atomicAdd(&live[op.cluster], 1);
    } else if (op.kind == kUpdDelete) {
      perm[p] = -1;
      slot_of[op.id] = -1;
      atomicAdd(&live[op.cluster], -1);
    }
  }
}

// ------------------------------------------------------------------------------------------------
// launch wrappers

hipError_t launch_coarse_keys(const DevIndex &ix, const int8_t *queries, int32_t B, const Work &w, hipStream_t s) {
  dim3 grid((ix.nlist + 255) / 256, (B + kCoarseQB - 1) / kCoarseQB);
  switch (ix.dim) {
    case 16: k_coarse_keys<1><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_scores, w.counter, w.gcnt, w.gfill, w.clog); break;
    case 32: k_coarse_keys<2><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_scores, w.counter, w.gcnt, w.gfill, w.clog); break;
    case 64: k_coarse_keys<4><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_scores, w.counter, w.gcnt, w.gfill, w.clog); break;
    case 128: k_coarse_keys<8><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_scores, w.counter, w.gcnt, w.gfill, w.clog); break;
    case 256: k_coarse_keys<16><<<grid, 256, 0, s>>>(ix.centroids, ix.nlist, queries, B, w.coarse_scores, w.counter, w.gcnt, w.gfill, w.clog); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_coarse_select(const DevIndex &ix, const int8_t *queries, const uint64_t *masks,
                                const SearchShape &sh, const Work &w, hipStream_t s) {
  // speculative thresholds for the tile path's pools and the large-k path's (when it has them)
  const bool pools = sh.path == kPathTile || (sh.path == kPathLargeK && sh.pool_cap > 0);
  const int thr_mode = pools ? (sh.force_redo ? 2 : 1) : 0;
  k_coarse_select<<<sh.B, kSelThreads, 0, s>>>(ix, queries, masks, sh.G, sh.GT, sh.B, sh.nprobe, sh.k,
                                                sh.pool_cap, thr_mode, w);
  return hipGetLastError();
}

hipError_t launch_plan(const DevIndex &ix, const SearchShape &sh, const Work &w, int redo, hipStream_t s) {
  if (redo) {
    k_plan_redo<<<1, kSelThreads, 0, s>>>(sh.B, sh.P, sh.nprobe, ix.nlist, sh.k, (uint32_t)sh.pool_cap, w);
    return hipGetLastError();
  }
  if (sh.B <= kPlanSmallBatch) {
    k_plan_small<<<1, kSelThreads, 0, s>>>(sh.B, sh.P, sh.nprobe, ix.nlist, sh.k, w);
    return hipGetLastError();
  }
  k_plan_count<<<1, kSelThreads, 0, s>>>(sh.B, sh.P, w, redo, sh.k, (uint32_t)sh.pool_cap);
  k_plan_chunks<<<sh.B, 256, 0, s>>>(sh.B, sh.nprobe, ix.nlist, w);
  k_plan_order<<<1, kSelThreads, 0, s>>>(sh.B, w);
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
                       const Work &w, int fallback, hipStream_t s) {
  ScanArgs a{ix, queries, masks, w, sh.B, sh.nprobe, sh.k, sh.P, fallback, sh.G};
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

template <int LPR>
static int scan_occ_w(int W) {
  int n = 0;
  hipError_t e = W == 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_scan<LPR, 2>, kScanThreads, 0)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_scan<LPR, 1>, kScanThreads, 0);
  return e == hipSuccess ? n : 0;
}

int scan_blocks_per_cu(int32_t dim, int32_t sig_words) {
  switch (dim) {
    case 16: return scan_occ_w<1>(sig_words);
    case 32: return scan_occ_w<2>(sig_words);
    case 64: return scan_occ_w<4>(sig_words);
    case 128: return scan_occ_w<8>(sig_words);
    case 256: return scan_occ_w<16>(sig_words);
    default: return 0;
  }
}

hipError_t launch_merge(const DevIndex &ix, const float *query_scales, const SearchShape &sh, const Work &w,
                        int fallback, int64_t *out_ids, int32_t *out_scores, float *out_fscores,
                        int32_t *out_counts, hipStream_t s) {
  MergeArgs a{w, query_scales, ix.item_scale, sh.B, sh.k, sh.P, fallback, (uint32_t)sh.gather_cap, out_ids,
              out_scores, out_fscores, out_counts};
  if (!fallback) {   // the redo of the tile path (rare) merges straight from the chunks' slots
    const int g = sh.max_chunks < kMergeGatherWGs ? sh.max_chunks : kMergeGatherWGs;
    k_merge_gather<<<g, 256, 0, s>>>(w, sh.B, sh.k, (uint32_t)sh.gather_cap);
  }
  k_merge<<<sh.B, kSelThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_updates(int8_t *items, uint64_t *sigs, int32_t *perm, int32_t *live, int32_t *slot_of,
                          const UpdOp *ops, int32_t n, const int8_t *rows, const uint64_t *new_sigs, int32_t dim,
                          int32_t sig_words, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int32_t chunks = dim / 16;
  const int64_t threads = (int64_t)n * chunks;
  k_updates<<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(items, sigs, perm, live, slot_of, ops, n, rows, new_sigs,
                                                                chunks, sig_words);
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
