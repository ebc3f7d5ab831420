// svt_tile.hip - gfx950 kernels of the tile search path: each probed cluster is read once per batch for
// every query that probes it.
//
//   k_tplan1, k_tplan2, k_tfill
//             the union stream: every probed cluster, in cluster order, once per block of at most
//             kTMembers of the queries probing it (an entry); its members (mask, threshold, query); the
//             stream cut into chunks of equal estimated cost (the members per cluster are counted by
//             k_coarse_select)
//   k_tscan   persistent workgroups take chunks from a queue and walk them in steps; each item of an
//             entry is tested against the masks of all the entry's members, the rows any member accepts
//             are gathered once and scored (v_dot4) for each member that accepts them; a score at or
//             above the member's threshold is a candidate for its query's pool
//   k_xscan   nprobe == nlist: the whole catalogue is one stream shared by every query; it is read once
//             per block of kXQ queries and scored with int8 MFMA (16x16x64), the masks applied to the
//             products; a sample pass over every kXStride-th item gives the thresholds (k_xthr)
// A query whose pool cannot prove its top k (fewer than k keys with a threshold above the minimum, or
// more keys than the pool holds) is redone by the query-by-query kernels (marked by k_plan_count).
//   k_pmerge  per query: the exact top k of its pool
//
// Method: "SilverTorch - Index as Model" (Meta engineering post): probe the most promising clusters,
// filter inside them with Bloom signatures and bit operations, score the survivors with int8 dot
// products ("dp4a" in the compute-cost-efficiency section), keep a large top-k on the device;
// "Meta Andromeda" summary, System section: scoring is bound by memory bandwidth, so data are fetched
// once and intermediates stay on chip.  The speculative thresholds, the union stream and the MFMA
// layout are this library's design for CDNA4, not the pages'.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "svt_device.h"
#include "svt_internal.h"

namespace svt {

// ------------------------------------------------------------------------------------------------
// the union stream

// The members of each probed cluster and the log of the fraction of its items no member accepts are
// counted by k_coarse_select (gcnt, clog).

// Each cluster's members in mrec (gstart), its first entry (estart), the union-stream offset of that entry
// (uoff) and the prefix of the clusters' estimated costs (ccost): prefix sums over the clusters in two
// launches.  k_tplan1: one thread per cluster, block prefixes and block totals.  k_tplan2: each
// workgroup adds its block's offset (the sum of the blocks before it); one more writes the totals, the
// stream's length and chunk count in thdr.
__device__ __forceinline__ void tile_cluster(const DevIndex &ix, const Work &w, int c, int64_t v[4]) {
  const int nq = w.gcnt[c];
  const int size = ix.offsets[c + 1] - ix.offsets[c];
  const int ne = (nq > 0 && size > 0) ? (nq + kTMembers - 1) / kTMembers : 0;
  v[0] = nq;
  v[1] = ne;
  v[2] = (int64_t)ne * size;   // the union stream is shorter than 2^31 (checked by the host)
  // estimated bytes and byte equivalents: signatures and per-item work of every entry, per-member
  // tests, the rows of the items some member accepts
  const double acc = ne > 0 ? 1.0 - (double)__expf(w.clog[c]) : 0.0;
  v[3] = ne > 0 ? (int64_t)size * (ne * (8 * ix.sig_words + kTItemCost) + (int64_t)kTMemberCost * nq) +
                      (int64_t)(acc * ix.dim * size) + 1
                : 0;
}

__global__ __launch_bounds__(kSelThreads) void k_tplan1(DevIndex ix, Work w) {
  __shared__ int64_t wave_tot[kSelThreads / 64 + 1];
  const int c = blockIdx.x * kSelThreads + threadIdx.x;
  int64_t v[4] = {0, 0, 0, 0};
  if (c < ix.nlist) tile_cluster(ix, w, c, v);
  int64_t pre[4], tot[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pre[j] = block_excl_scan<kSelThreads>(v[j], wave_tot, &tot[j]);
  if (c < ix.nlist) {
    w.gstart[c] = (int32_t)pre[0];
    w.estart[c] = (int32_t)pre[1];
    w.uoff[c] = (int32_t)pre[2];
    w.ccost[c] = pre[3];
  }
  if (threadIdx.x == 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) w.tblk[4 * blockIdx.x + j] = tot[j];
}

__global__ __launch_bounds__(kSelThreads) void k_tplan2(DevIndex ix, int32_t P, Work w) {
  __shared__ int64_t boff[4];
  const int tid = threadIdx.x, l = lane_id();
  const int nlist = ix.nlist;
  const int nb = (nlist + kSelThreads - 1) / kSelThreads;
  const int blk = blockIdx.x;
  if (tid < 64) {   // this block's offsets (blocks before it), and the totals: one wave over the block sums
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      int64_t before = 0, all = 0;
      for (int b0 = 0; b0 < nb; b0 += 64) {
        const int b = b0 + l;
        const int64_t x = b < nb ? w.tblk[4 * b + v] : 0;
        const int64_t inc = wave_incl_scan(x);
        const int64_t tot = __shfl(inc, 63);
        const int64_t pre = __shfl(inc - x, (blk - b0) & 63);   // offset of block blk within this group
        if (blk >= b0 && blk < b0 + 64) before = all + pre;
        all += tot;
      }
      if (l == 0) boff[v] = blk < nb ? before : all;
    }
  }
  __syncthreads();
  if (blk < nb) {
    const int c = blk * kSelThreads + tid;
    if (blk > 0 && c < nlist) {
      w.gstart[c] += (int32_t)boff[0];
      w.estart[c] += (int32_t)boff[1];
      w.uoff[c] += (int32_t)boff[2];
      w.ccost[c] += boff[3];
    }
  } else if (tid == 0) {   // the last workgroup: totals and the stream's length and chunk count
    w.gstart[nlist] = (int32_t)boff[0];
    w.estart[nlist] = (int32_t)boff[1];
    w.ccost[nlist] = boff[3];
    const int32_t U = (int32_t)boff[2];
    w.thdr[0] = (int32_t)boff[1];
    w.thdr[1] = U;
    w.thdr[2] = U > 0 ? kTChunksPerWave * kTWaves * P : 0;
    w.thdr[3] = 0;
  }
}

// Chunk i of the union stream starts where the estimated cost reaches i / n of the total: inside the
// cluster whose cost range holds that point, at the same fraction of the cluster's union items (rounded
// down to 64).  The starts ascend with i; a chunk may be empty.  ctab[i]: the entry holding the start.
__device__ __forceinline__ void tile_chunk(const DevIndex &ix, int32_t max_tchunks, const Work &w, int i) {
  const int n = w.thdr[2];
  const int32_t U = w.thdr[1];
  if (i > n || i > max_tchunks) return;
  if (i == n) {
    w.cstart_u[n] = U;
    return;
  }
  const int nlist = ix.nlist;
  const int64_t total = w.ccost[nlist];
  const int64_t target = (int64_t)((double)total * i / n);
  int lo = 0, hi = nlist - 1;   // largest c with ccost[c] <= target: its cost range holds target
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (w.ccost[mid] <= target) lo = mid; else hi = mid - 1;
  }
  const int c = lo;
  const int64_t cost = w.ccost[c + 1] - w.ccost[c];
  const int32_t u0 = w.uoff[c];
  const int32_t nu = (c + 1 < nlist ? w.uoff[c + 1] : U) - u0;
  int32_t off = 0;
  if (cost > 0 && nu > 0) {
    off = (int32_t)((double)(target - w.ccost[c]) / (double)cost * (double)nu);
    off = off < nu - 1 ? off : nu - 1;
    off = off / 64 * 64;
  }
  const int size = ix.offsets[c + 1] - ix.offsets[c];
  w.cstart_u[i] = u0 + off;
  w.ctab[i] = w.estart[c] + (size > 0 ? off / size : 0);
}

// the members of each probed cluster: for every query probing it, GT consecutive members, one per request
// mask (masks past the query's G pass nothing: every bit set), with the query's speculative threshold and
// index.  The slots of a query's members start at a multiple of GT, and GT divides kTMembers, so they lie
// in one entry, aligned.  The order of the queries inside a cluster is arbitrary; it changes no result.
__device__ __forceinline__ void tile_members(const int32_t *__restrict__ probes, const uint64_t *__restrict__ masks,
                                             int32_t nprobe, int32_t W, int32_t G, int32_t GT, const Work &w, int b) {
  const int32_t thr = w.sthr[b];
  for (int j = threadIdx.x; j < nprobe; j += 256) {
    const int c = probes[(size_t)b * nprobe + j];
    const int slot = atomicAdd(&w.gfill[c], GT);
    for (int g = 0; g < GT; ++g) {
      const uint64_t *m = masks + ((size_t)b * G + (g < G ? g : 0)) * W;
      const uint64_t m0 = g < G ? m[0] : ~0ull, m1 = g < G ? (W == 2 ? m[1] : 0ull) : ~0ull;
      w.mrec[w.gstart[c] + slot + g] = MRec{m0, m1, thr, b};
    }
  }
}

// entry e: the cluster whose entries hold e and its member block
__device__ __forceinline__ void tile_entry(const DevIndex &ix, int32_t max_entries, const Work &w, int e) {
  const int n_e = w.thdr[0];
  if (e >= n_e || e >= max_entries) return;
  const int nlist = ix.nlist;
  int lo = 0, hi = nlist - 1;   // largest c with estart[c] <= e: the cluster that has entry e
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (w.estart[mid] <= e) lo = mid; else hi = mid - 1;
  }
  const int c = lo;
  const int bi = e - w.estart[c];
  const int32_t pos0 = ix.offsets[c], size = ix.offsets[c + 1] - pos0;
  const int nq = w.gstart[c + 1] - w.gstart[c];
  const int32_t useg = w.uoff[c] + bi * size;
  const int mc = nq - bi * kTMembers < kTMembers ? nq - bi * kTMembers : kTMembers;
  const int ms = w.gstart[c] + bi * kTMembers;
  w.entries[e] = UEntry{useg, size, pos0, ms, mc, 0, 0, 0};
}

// The three independent steps after the prefix sums, in one launch: workgroups [0, B) place the members
// of query blockIdx.x, the next ne_blocks write the entries, the rest cut the chunks.
__global__ __launch_bounds__(256) void k_tfill(DevIndex ix, const int32_t *__restrict__ probes,
                                               const uint64_t *__restrict__ masks, int32_t B, int32_t nprobe,
                                               int32_t G, int32_t GT, int32_t max_entries, int32_t ne_blocks,
                                               int32_t max_tchunks, Work w) {
  const int blk = blockIdx.x;
  if (blk < B)
    tile_members(probes, masks, nprobe, ix.sig_words, G, GT, w, blk);
  else if (blk < B + ne_blocks)
    tile_entry(ix, max_entries, w, (blk - B) * 256 + threadIdx.x);
  else
    tile_chunk(ix, max_tchunks, w, (blk - B - ne_blocks) * 256 + threadIdx.x);
}

// Order of LDS accesses between the lanes of one wave (its LDS operations complete in order; this keeps
// the compiler from moving them across each other).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// raw buffer resource over [base, base + bytes) (gfx9 word 3: 32-bit data format, no swizzle)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes < 0x7FFFFFFF ? (int)bytes : 0x7FFFFFFF);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// ------------------------------------------------------------------------------------------------
// k_tscan: the union stream, chunk by chunk.
//
// Each wave works alone: it takes a chunk from the queue, stages the chunk's entries (a window of them,
// with their members and query vectors) in its part of LDS and walks them in filter steps of 64 kTGroups
// items inside one entry.  A step's signatures are tested against the masks of every member of the entry;
// the items any member accepts go, with their member bits, into the wave's FIFO of survivors.  Every
// iteration then requests the rows of the next batch of FIFO survivors (LPR lanes per row, 16-byte loads)
// and scores the batch requested one iteration earlier against the query vector of each member that
// accepts the row (v_dot4).  The signatures of the next step are requested after each filter, so
// signatures and rows both have one iteration to arrive; every load is issued in every iteration (a
// signature resource clipped to the step, so that items past it read as zero without a memory access;
// lanes without a row re-read the batch's first row), which keeps the compiler's wait counts exact.
// A new step is taken only while the FIFO has room for all of its items besides the batch in flight.
//
// Candidates (score at or above the member's threshold) are staged in LDS with the slot of their (entry
// visit, member) and go to the queries' pools when the stage fills and at the end of the chunk, one pool
// reservation per slot.  Per-slot counters give the accepted items of each query.

struct TScanArgs {
  DevIndex ix;
  const int8_t *queries;
  Work w;
  int32_t B, P;
  uint32_t pool_cap;
  int32_t GT;   // consecutive members per query (one per request mask), aligned in an entry
};

#ifndef SVT_T_WIN_MEMBERS
#define SVT_T_WIN_MEMBERS 16
#endif
#ifndef SVT_T_STAGE
#define SVT_T_STAGE 160
#endif
constexpr int kTF = 512;             // survivors a wave's FIFO holds (a ring)
constexpr int kTWinW = 16;           // entries of a wave's window
constexpr int kTWinMW = SVT_T_WIN_MEMBERS;   // members of those entries
constexpr int kTSlotsW = 64;         // (entry visit, member) slots of a wave's chunk
constexpr int kTStageW = SVT_T_STAGE;        // candidates a wave stages before it writes them to the pools
constexpr uint32_t kNoSlot = 0xFFu;
static_assert(kTWinMW >= kTMembers && kTWinMW <= 256 && kTSlotsW < 255, "survivor metadata fields");

template <int LPR>
struct TWaveLds {
  // the window: stream range of each entry clipped to the chunk, position base (pos = pb + t), first
  // window member, member count, first member in mrec
  int32_t e_t0[kTWinW], e_t1[kTWinW], e_pb[kTWinW], e_m[kTWinW], e_mc[kTWinW], e_ms[kTWinW];
  MRec wm[kTWinMW];                  // members of the window's entries
  int4 wqv[kTWinMW][LPR];            //   and their query vectors
  int32_t fpos[kTF];                 // survivors: position
  uint32_t fmeta[kTF];               //   member bits | first window member << 16 | first slot << 24
  int32_t sq[kTSlotsW];              // query of each slot
  uint32_t scount[kTSlotsW];         // candidates staged for each slot
  uint32_t sbase[kTSlotsW];          // their pool position, reserved at a flush
  uint32_t selig[kTSlotsW];          // items the slot's member accepted
  uint64_t skey[kTStageW];           // staged candidates: (score, position) keys
  uint8_t sslot[kTStageW];           //   their slot
  uint16_t srank[kTStageW];          //   their rank among the slot's staged candidates
};

template <int LPR, int W>
__global__ __launch_bounds__(kScanThreads, kTOcc) void k_tscan(TScanArgs a) {
  constexpr int D = 16 * LPR;
  constexpr int RPI = 64 / LPR;        // rows covered by one 16-byte load per lane
  constexpr int R = kTRowLoads;
  constexpr int RB = R * RPI;          // rows of one batch
  constexpr int G = kTGroups;
  constexpr int GS = 64 * G;           // items of one filter step
  static_assert(RB <= kTF && GS <= kTF, "FIFO");
  __shared__ TWaveLds<LPR> lds[kTWaves];
  const int l = lane_id(), sub = l % LPR;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  TWaveLds<LPR> &S = lds[wv];
  const int n_chunks = a.w.thdr[2];
  const int n_ent = a.w.thdr[0];
  const uint32_t cap = a.pool_cap;
  int64_t *stats = a.w.stats;
  const int GT = a.GT;
  const uint32_t gmask = (1u << GT) - 1u;   // the member bits of one query, at its first member
  for (int i = l; i < kTSlotsW; i += 64) {
    S.scount[i] = 0u;
    S.selig[i] = 0u;
  }
  int stage_n = 0;   // staged candidates (the same value in every lane)
  int nsl = 0;       // slots taken in the chunk
  // staged candidates to their pools: one reservation per slot with staged keys, then the keys
  auto flush = [&]() {
    wave_lds_sync();
    const int ns = nsl < kTSlotsW ? nsl : kTSlotsW;
    for (int s = l; s < ns; s += 64) {
      const uint32_t c = S.scount[s];
      if (c) S.sbase[s] = atomicAdd(&a.w.pool_cnt[S.sq[s]], c);
      S.scount[s] = 0u;
    }
    wave_lds_sync();
    for (int e = l; e < stage_n; e += 64) {
      const int s = S.sslot[e];
      const uint32_t o = S.sbase[s] + S.srank[e];
      if (o < cap) a.w.pool[(size_t)S.sq[s] * cap + o] = S.skey[e];
    }
    wave_lds_sync();
    stage_n = 0;
  };
  // Chunk claims: the first two of wave i (of NW waves) are i and NW + i, later ones NW * 2 + the
  // counter's next value, so that the waves do not all wait on one counter address at the start.
  const int NW = (int)gridDim.x * kTWaves, gw = (int)blockIdx.x * kTWaves + wv;
  int claims = 0;   // chunks claimed so far (uniform across the wave)
  for (;;) {
    int ci = 0;
    if (claims < 2) {
      ci = claims * NW + gw;
    } else {
      if (l == 0) ci = 2 * NW + (int)atomicAdd(&a.w.counter[3], 1u);
      ci = __builtin_amdgcn_readfirstlane(__shfl(ci, 0));
    }
    ++claims;
    if (ci >= n_chunks) break;
    const int32_t ra = a.w.cstart_u[ci], rb = a.w.cstart_u[ci + 1];
    if (ra >= rb) continue;
    int jwin = a.w.ctab[ci];
    int e_n = 0;   // entries in the window
    // the chunk's entries from jwin on, as many as kTWinW entries and kTWinMW members allow
    auto load_window = [&]() {
      UEntry E{0, 0, 0, 0, 0, 0, 0, 0};
      const bool have = jwin + l < n_ent && l < kTWinW;
      if (have) E = a.w.entries[jwin + l];
      const bool valid = have && E.useg < rb;   // entries are in stream order: a prefix of the lanes
      const int mc = valid ? E.mcnt : 0;
      const int inc = wave_incl_scan(mc);
      const bool fit = valid && inc <= kTWinMW;
      const int n = __popcll(__ballot(fit));
      wave_lds_sync();
      if (fit) {
        S.e_t0[l] = ra > E.useg ? ra : E.useg;
        S.e_t1[l] = rb < E.useg + E.len ? rb : E.useg + E.len;
        S.e_pb[l] = E.pos0 - E.useg;
        S.e_m[l] = inc - mc;
        S.e_mc[l] = mc;
        S.e_ms[l] = E.mstart;
      }
      const int nm = n > 0 ? __shfl(inc, n - 1) : 0;
      wave_lds_sync();
      // members and their query vectors: lane t copies part t % LPR of member t / LPR
      for (int mp = l; mp < nm * LPR; mp += 64) {
        const int m = mp / LPR, part = mp % LPR;
        int lo = 0, hi = n - 1;   // the entry of window member m: largest i with e_m[i] <= m
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (S.e_m[mid] <= m) lo = mid; else hi = mid - 1;
        }
        const MRec rec = a.w.mrec[S.e_ms[lo] + (m - S.e_m[lo])];
        if (part == 0) S.wm[m] = rec;
        S.wqv[m][part] = reinterpret_cast<const int4 *>(a.queries + (size_t)rec.q * D)[part];
      }
      wave_lds_sync();
      e_n = n;
    };
    // cursor: entry cw of the window, next step at stream offset cst, entry end ct1, position base cpb;
    // the entry visit's first window member, member count and first slot
    int cw = 0;
    int32_t cst = 0, ct1 = 0, cpb = 0;
    int cmb = 0, cmc = 0;
    uint32_t cslot = kNoSlot;
    // from entry cw on: the first entry of the window with items left (cw == e_n: none); a new entry visit
    // takes a slot per member (a visit without slots counts to HBM)
    auto seek = [&]() {
      for (; cw < e_n; ++cw) {
        const int32_t t0 = __builtin_amdgcn_readfirstlane(S.e_t0[cw]);
        const int32_t t1 = __builtin_amdgcn_readfirstlane(S.e_t1[cw]);
        if (t0 < t1) {
          cst = t0;
          ct1 = t1;
          cpb = __builtin_amdgcn_readfirstlane(S.e_pb[cw]);
          cmb = __builtin_amdgcn_readfirstlane(S.e_m[cw]);
          cmc = __builtin_amdgcn_readfirstlane(S.e_mc[cw]);
          const bool fits = nsl + cmc <= kTSlotsW;
          cslot = fits ? (uint32_t)nsl : kNoSlot;
          if (l < cmc && fits) S.sq[nsl + l] = S.wm[cmb + l].q;
          if (fits) nsl += cmc;
          wave_lds_sync();
          return;
        }
      }
    };
    load_window();
    seek();
    // the step whose signatures are in flight: position of its first item, items, members, slot
    bool sg_live = false;
    int32_t fs_p0 = 0, fs_n = 0;
    int fs_mb = 0, fs_mc = 0;
    uint32_t fs_slot = kNoSlot;
    uint64_t sg[G][W];
    // request the signatures of the step at the cursor (or, with take false, of nothing: the loads read
    // zeros without touching memory)
    auto request_sigs = [&](bool take) {
      const int32_t n = take ? (ct1 - cst < GS ? ct1 - cst : GS) : 0;
      const int32_t p0 = cpb + cst;
      const __amdgpu_buffer_rsrc_t rs = raw_rsrc(a.ix.sigs + (take ? (size_t)p0 * W : 0), (int64_t)n * (8 * W));
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const uint32_t off = (uint32_t)(g * 64 + l) * (8u * W);
        if constexpr (W == 2) {
          typedef int v4i __attribute__((ext_vector_type(4)));
          const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
          sg[g][0] = (uint64_t)(uint32_t)v.x | ((uint64_t)(uint32_t)v.y << 32);
          sg[g][1] = (uint64_t)(uint32_t)v.z | ((uint64_t)(uint32_t)v.w << 32);
        } else {
          typedef int v2i __attribute__((ext_vector_type(2)));
          const v2i v = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
          sg[g][0] = (uint64_t)(uint32_t)v.x | ((uint64_t)(uint32_t)v.y << 32);
        }
      }
      if (take) {
        sg_live = true;
        fs_p0 = p0;
        fs_n = n;
        fs_mb = cmb;
        fs_mc = cmc;
        fs_slot = cslot;
        cst += n;
        if (cst >= ct1) {
          ++cw;
          seek();
        }
      }
    };
    uint32_t head = 0, tail = 0;   // FIFO ring positions (uniform)
    uint32_t bhead = 0;            // first FIFO position of the batch in flight
    // the step in sg against the members of its entry; its survivors to the FIFO
    auto filter = [&]() {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int i = g * 64 + l;
        const bool live = i < fs_n && sig_live(sg[g][0], sg[g][W - 1], W);
        uint32_t qm = 0u;
        for (int j = 0; j < fs_mc; ++j) {
          const uint64_t m0 = S.wm[fs_mb + j].m0;
          bool pass = live && ((sg[g][0] & m0) == m0);
          if constexpr (W == 2) {
            const uint64_t m1 = S.wm[fs_mb + j].m1;
            pass = pass && ((sg[g][1] & m1) == m1);
          }
          qm |= pass ? 1u << j : 0u;
        }
        if (stats) {
          // an item counts once per query: when any of the query's members (its masks) accepts it
          for (int j = 0; j < fs_mc; j += GT) {
            const int cnt = __popcll(__ballot((qm & (gmask << j)) != 0u));
            if (l == 0 && cnt > 0) {
              if (fs_slot != kNoSlot)
                S.selig[fs_slot + j] += (uint32_t)cnt;
              else
                atomicAdd((unsigned long long *)&stats[2 * (size_t)S.wm[fs_mb + j].q + 1], (unsigned long long)cnt);
            }
          }
        }
        const uint64_t bal = __ballot(qm != 0u);
        if (qm != 0u) {
          const uint32_t o = (tail + (uint32_t)mbcnt(bal)) & (kTF - 1);
          S.fpos[o] = fs_p0 + i;
          S.fmeta[o] = qm | ((uint32_t)fs_mb << 16) | (fs_slot << 24);
        }
        tail += (uint32_t)__popcll(bal);
      }
      sg_live = false;
    };
    int4 xa[R], xb[R];
    uint32_t ma[R], mb[R];
    // request the rows of the next batch (n of them) into x / mt
    auto request_rows = [&](int4 (&x)[R], uint32_t (&mt)[R]) -> int {
      const int n = (int)(tail - head) < RB ? (int)(tail - head) : RB;
      wave_lds_sync();
      const int32_t first = n > 0 ? S.fpos[head & (kTF - 1)] : 0;
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const int ri = u * RPI + l / LPR;
        const bool valid = ri < n;
        const uint32_t o = (head + (uint32_t)ri) & (kTF - 1);
        const int32_t pos = valid ? S.fpos[o] : first;
        mt[u] = valid ? S.fmeta[o] : 0u;
        x[u] = reinterpret_cast<const int4 *>(a.ix.items + (size_t)pos * D)[sub];
      }
      bhead = head;
      head += (uint32_t)n;
      return n;
    };
    // a candidate of a member (lanes with ok): staged with its slot; a member without a slot goes to its
    // pool directly
    auto offer = [&](bool ok, int32_t score, uint32_t bpos, uint32_t slot0, int j, int q) {
      if (__ballot(ok) == 0ull) return;
      if (stage_n + 64 > kTStageW) flush();   // rare: an iteration with more candidates than the stage holds
      const uint64_t b = __ballot(ok);
      if (ok) {
        const int32_t pos = S.fpos[bpos & (kTF - 1)];
        const uint64_t key = pos_key(score, pos);
        if (slot0 != kNoSlot) {
          const int e = stage_n + mbcnt(b);
          const uint32_t s = slot0 + (uint32_t)j;
          S.skey[e] = key;
          S.sslot[e] = (uint8_t)s;
          S.srank[e] = (uint16_t)atomicAdd(&S.scount[s], 1u);
        } else {
          const uint32_t o = atomicAdd(&a.w.pool_cnt[q], 1u);
          if (o < cap) a.w.pool[(size_t)q * cap + o] = key;
        }
      }
      stage_n += __popcll(b);   // a lane without a slot leaves an unused stage entry (no harm)
      wave_lds_sync();
    };
    // score the batch in x / mt (rows of FIFO positions bh ..)
    auto score_rows = [&](const int4 (&x)[R], const uint32_t (&mt)[R], uint32_t bh) {
#pragma unroll
      for (int u = 0; u < R; ++u) {
        const uint32_t meta = mt[u];
        uint32_t qm = meta & 0xFFFFu;
        const int mb0 = (int)((meta >> 16) & 0xFFu);
        const uint32_t slot0 = meta >> 24;
        const uint32_t bpos = bh + (uint32_t)(u * RPI + l / LPR);
        int j = qm ? __builtin_ctz(qm) : 0;
        int32_t acc = group_sum<LPR>(dot16(x[u], S.wqv[mb0 + j][sub], 0));
        for (;;) {
          const MRec &m = S.wm[mb0 + j];
          offer(qm != 0u && sub == 0 && acc >= m.thr, acc, bpos, slot0, j, m.q);
          qm &= ~(gmask << (j & ~(GT - 1)));   // the query of member j is done, whichever of its masks passed
          if (__ballot(qm != 0u) == 0ull) break;
          // a further member accepts this row: the same row against its query vector
          j = qm ? __builtin_ctz(qm) : 0;
          acc = group_sum<LPR>(dot16(x[u], S.wqv[mb0 + j][sub], 0));
        }
      }
    };
    // room for a new step: its items at most, besides the survivors not yet scored
    auto room = [&]() { return (int)(tail - bhead) <= kTF - GS; };
    auto more_steps = [&]() { return cw < e_n; };
    // the walk; each iteration: filter the step in flight, request the next step's signatures and the next
    // batch's rows, score the batch requested one iteration earlier
    for (int u = 0; u < R; ++u) mb[u] = 0u;   // the first iteration scores an empty batch
    uint32_t bh_prev = 0;
    auto iteration = [&](int4 (&xr)[R], uint32_t (&mr)[R], const int4 (&xs)[R], const uint32_t (&ms)[R]) -> bool {
      // a stage past half full is written out here, where the loads in flight are the ones this iteration
      // consumes next anyway (the flush waits for every load of the wave)
      if (stage_n > kTStageW / 2) flush();
      if (sg_live) filter();
      request_sigs(more_steps() && room());
      const uint32_t bh_s = bh_prev;
      const int nr = request_rows(xr, mr);
      bh_prev = bhead;
      score_rows(xs, ms, bh_s);   // also an empty batch: every path reads the rows it requested
      return !sg_live && nr == 0 && head == tail && !more_steps();
    };
    for (;;) {
      for (;;) {
        // iterations in pairs, so that the rows requested into xa are always read before the loop ends
        // (an iteration after the one that found nothing left does nothing)
        (void)iteration(xa, ma, xb, mb);
        if (iteration(xb, mb, xa, ma)) break;
      }
      // the window is done (every survivor scored: the FIFO is empty and no batch is in flight); the chunk
      // may continue in the next one
      if (!(e_n > 0 && jwin + e_n < n_ent && a.w.entries[jwin + e_n].useg < rb)) break;
      jwin += e_n;
      load_window();
      cw = 0;
      seek();
    }
    // end of the chunk: staged candidates to the pools, the slots' counts to the statistics
    if (stage_n > 0) flush();
    const int ns = nsl < kTSlotsW ? nsl : kTSlotsW;
    if (stats) {
      for (int s = l; s < ns; s += 64) {
        const int q = S.sq[s];
        if (S.selig[s]) atomicAdd((unsigned long long *)&stats[2 * (size_t)q + 1], (unsigned long long)S.selig[s]);
      }
    }
    wave_lds_sync();
    for (int s = l; s < ns; s += 64) {
      S.scount[s] = 0u;
      S.selig[s] = 0u;
    }
    nsl = 0;
    wave_lds_sync();
  }
}

// ------------------------------------------------------------------------------------------------
// k_xscan: nprobe == nlist.  Every query's stream is the whole catalogue in position order, so one read
// of a 64-item step serves a block of kXQ queries: v_mfma_i32_16x16x64_i8 multiplies 16 queries by 16
// items per K slice of 64 bytes.  Lane layout (gfx950, 16x16x64 int8): lane l supplies row l % 16 of each
// operand with K bytes 16 (l / 16) .. + 15 of the slice, and receives C[4 (l / 16) + r][l % 16], r = 0..3.
// Items are the columns, queries the rows: lane l holds 4 queries x 1 item per (query tile, item tile),
// and tests those items' signatures against those queries' masks after the product.
//
// Each wave works alone, on one query block and a fixed share of the steps: step s of the stream goes to
// the wave with part s mod parts, so the waves of the grid walk the catalogue together and each has the
// same number of steps.  A step's rows and signatures come through buffer loads whose resource starts at
// the step and ends with the catalogue: the per-lane offsets are constants, and items past the end read as
// zero without a memory access.  The loads of the next XNB - 1 steps are in flight while a step is scored
// (XNB register buffers, the loop unrolled XNB times, every load unconditional).  Candidates are staged per
// wave in LDS with their rank among the wave's staged candidates of their query and go to the pools with
// one reservation per query.
// SAMPLE: the stream is every kXStride-th position; each lane keeps its best eligible score per query over
// a step and writes it to the query's sample buffer (one slot per lane and step).

struct XScanArgs {
  DevIndex ix;
  const int8_t *queries;
  const uint64_t *masks;
  Work w;
  int32_t B, n_qb;
  uint32_t cap;       // pool keys (main pass) or sample-buffer entries (sample pass) per query
  int32_t G;          // masks per query (an item is eligible under any of them)
};

struct XWave {
  uint32_t mk[kXQ][4];                     // first request mask of the block's queries (32-bit words)
  uint32_t mkx[kXQ][kMaxGroups - 1][4];    //   and their further masks
  int32_t sc[32][64];        // a step's scores, when it has candidates (entry 8 t + 4 t2 + r, lane)
  uint64_t key[kXStage];     // staged candidates: (score, position) keys
  uint8_t qi[kXStage];       //   their query within the block
  uint16_t rank[kXStage];    //   their rank among the staged candidates of that query
  uint32_t cnt[kXQ];         // staged candidates per query of the block
  uint32_t base[kXQ];        // pool positions reserved at a flush
};

template <int KS, int W, bool SAMPLE, bool MULTI>
__global__ __launch_bounds__(64 * kXWaves, kXOcc) void k_xscan(XScanArgs a) {
  constexpr int XNB = KS >= 4 ? 2 : kXBuffers;   // step buffers in registers
  constexpr int IS = SAMPLE ? kXStride : 1;   // catalogue positions between stream items
  constexpr int MW = 2 * W;                   // 32-bit words of a mask
  __shared__ XWave xw[kXWaves];
  const int l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  XWave &S = xw[wv];
  const int dim = a.ix.dim;
  const int64_t N = a.ix.n_items;
  const int64_t NP = (N + IS - 1) / IS;        // stream length
  const int64_t n_steps = (NP + 63) / 64;
  const int gw = blockIdx.x * kXWaves + wv;
  const int parts = (int)(gridDim.x * kXWaves) / a.n_qb;   // the launch gives every block at least one
  if (gw >= parts * a.n_qb) return;   // waves work alone: no workgroup barrier follows
  const int qb = gw % a.n_qb, part = gw / a.n_qb;
  const int64_t my_steps = part < n_steps ? (n_steps - part + parts - 1) / parts : 0;
  const int lr = l & 15, lg = l >> 4;   // operand row (query or item) and K group of this lane
  const int q0 = qb * kXQ;
  // query operands: rows q0 + 16 t2 + lr, K bytes 64 ks + 16 lg .. + 15 (zero beyond dim or B)
  int4 aop[2][KS];
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2) {
    const int q = q0 + 16 * t2 + lr;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = 64 * ks + 16 * lg;
      const bool ok = q < a.B && off < dim;
      const int4 v = reinterpret_cast<const int4 *>(a.queries + (size_t)(q < a.B ? q : 0) * dim +
                                                    (off < dim ? off : 0))[0];
      aop[t2][ks] = ok ? v : make_int4(0, 0, 0, 0);
    }
  }
  // the block's masks in the wave's LDS (lane j < kXQ writes query q0 + j's); this lane's result rows are
  // queries q0 + 16 t2 + 4 lg + r.  A row past the batch never offers a candidate (threshold above every
  // score) and its count is not written.
  if (l < kXQ) {
    const int qc = q0 + l < a.B ? q0 + l : 0;
    for (int g = 0; g < a.G; ++g)
#pragma unroll
      for (int ww = 0; ww < W; ++ww) {
        const uint64_t m = a.masks[((size_t)qc * a.G + g) * W + ww];
        uint32_t *dst = g == 0 ? S.mk[l] : S.mkx[l][g - 1];
        dst[2 * ww] = (uint32_t)m;
        dst[2 * ww + 1] = (uint32_t)(m >> 32);
      }
    S.cnt[l] = 0u;
  }
  wave_lds_sync();
  int32_t th[2][4];
  uint32_t ec[2][4];   // eligible items per query (sample pass: the lane's best eligible score of the step)
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = q0 + 16 * t2 + 4 * lg + r;
      th[t2][r] = q < a.B ? (SAMPLE ? INT32_MIN : a.w.sthr[q]) : INT32_MAX;
      ec[t2][r] = SAMPLE ? (uint32_t)INT32_MIN : 0u;
    }
  // byte offsets of this lane's parts of a step: rows of items 16 t + lr (K bytes 64 ks + 16 lg) and
  // signature word lg % MW of the same items
  uint32_t roff[4][KS], soff[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint32_t item = (uint32_t)((16 * t + lr) * IS);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int off = 64 * ks + 16 * lg;
      roff[t][ks] = item * (uint32_t)dim + (uint32_t)(off < dim ? off : 0);
    }
    soff[t] = item * (uint32_t)(8 * W) + 4u * (uint32_t)(lg % MW);
  }
  typedef int4 StepRows[4][KS];
  typedef uint32_t StepSigs[4];
  // the j-th step of this wave (j may run past its share: such a step lies past the catalogue and reads
  // zeros without touching memory)
  auto load_step = [&](int64_t j, StepRows &Bo, StepSigs &NS) {
    const int64_t first = (part + j * parts) * 64 * IS;   // catalogue position of the step's item 0
    const int64_t valid = N - first;
    const int64_t at = valid > 0 ? first : 0;
    const __amdgpu_buffer_rsrc_t rr = raw_rsrc(a.ix.items + at * dim, valid * dim);
    const __amdgpu_buffer_rsrc_t rs = raw_rsrc(a.ix.sigs + at * W, valid * (8 * W));
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        typedef int v4i __attribute__((ext_vector_type(4)));
        const v4i v = __builtin_amdgcn_raw_buffer_load_b128(rr, roff[t][ks], 0, 0);
        Bo[t][ks] = make_int4(v.x, v.y, v.z, v.w);
      }
      NS[t] = __builtin_amdgcn_raw_buffer_load_b32(rs, soff[t], 0, 0);
    }
  };
  int stage_n = 0;
  auto flush = [&]() {
    wave_lds_sync();
    if (l < kXQ) {
      const uint32_t c = S.cnt[l];
      uint32_t b = 0u;
      if (c && q0 + l < a.B) b = atomicAdd(&a.w.pool_cnt[q0 + l], c);
      S.base[l] = b;
      S.cnt[l] = 0u;
    }
    wave_lds_sync();
    for (int e = l; e < stage_n; e += 64) {
      const int qi = S.qi[e];
      const uint32_t o = S.base[qi] + S.rank[e];
      const size_t q = (size_t)(q0 + qi);
      if (o < a.cap) a.w.pool[q * a.cap + o] = S.key[e];
    }
    wave_lds_sync();
    stage_n = 0;
  };
  // score the wave's j-th step (rows and signatures in Bo / SG): count the eligible items, offer the
  // candidates (sample pass: keep the best eligible score and write it to the sample buffer)
  auto score_step = [&](int64_t j, const StepRows &Bo, const StepSigs &SG) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    const int64_t s = part + j * parts;
    const int64_t p0 = s * 64;   // stream index of the step's item 0
    uint32_t cbits = 0u;         // bit (8 t + 4 t2 + r): candidate
    v4i acc[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        v4i c = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const v4i av = {aop[t2][ks].x, aop[t2][ks].y, aop[t2][ks].z, aop[t2][ks].w};
          const v4i bv = {Bo[t][ks].x, Bo[t][ks].y, Bo[t][ks].z, Bo[t][ks].w};
          c = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
        }
        acc[t][t2] = c;
      }
    // the complemented signature words of item lr of each tile (an item passes a mask when no mask bit
    // falls on a zero of its signature), gathered from the lanes of the other groups
    uint32_t ns[4][MW];
    bool live[4];   // a free slot (every signature bit set) is eligible for no query
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      uint32_t any = 0u;
#pragma unroll
      for (int ww = 0; ww < MW; ++ww) {
        ns[t][ww] = ~(uint32_t)__shfl((int)SG[t], lr + 16 * ww);
        any |= ns[t][ww];
      }
      live[t] = any != 0u;
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t mq[MW];   // the first mask of this lane's query 16 t2 + 4 lg + r
        const int qi = 16 * t2 + 4 * lg + r;
#pragma unroll
        for (int ww = 0; ww < MW; ++ww) mq[ww] = S.mk[qi][ww];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const bool item_ok = p0 + 16 * t + lr < NP && live[t];
          uint32_t x = 0u;
#pragma unroll
          for (int ww = 0; ww < MW; ++ww) x |= mq[ww] & ns[t][ww];
          bool pass = x == 0u;
          if constexpr (MULTI) {
            for (int g = 1; g < a.G; ++g) {   // further masks of the query: eligible under any of them
              uint32_t xg = 0u;
#pragma unroll
              for (int ww = 0; ww < MW; ++ww) xg |= S.mkx[qi][g - 1][ww] & ns[t][ww];
              pass = pass || xg == 0u;
            }
          }
          const bool el = item_ok && pass;
          if constexpr (SAMPLE) {
            const int32_t cur = (int32_t)ec[t2][r], sc = acc[t][t2][r];
            ec[t2][r] = (uint32_t)(el && sc > cur ? sc : cur);
          } else {
            ec[t2][r] += el ? 1u : 0u;
            const bool cand = el && acc[t][t2][r] >= th[t2][r];
            cbits |= cand ? 1u << (8 * t + 4 * t2 + r) : 0u;
          }
        }
      }
    if constexpr (SAMPLE) {
      // slot 16 s + lr of each of the lane's queries: its best eligible score among the step's items
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = q0 + 16 * t2 + 4 * lg + r;
          if (q < a.B && s < n_steps) a.w.sbuf[(size_t)q * a.cap + 16 * s + lr] = (int32_t)ec[t2][r];
          ec[t2][r] = (uint32_t)INT32_MIN;
        }
      return;
    }
    if (__ballot(cbits != 0u) == 0ull) return;
    // rare: the step's scores go to LDS and its candidates are staged in one loop over the result entries
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 4; ++r) S.sc[8 * t + 4 * t2 + r][l] = acc[t][t2][r];
    wave_lds_sync();
#pragma unroll 1
    for (int c = 0; c < 32; ++c) {
      const bool cand = (cbits >> c) & 1u;
      const uint64_t b = __ballot(cand);
      if (b == 0ull) continue;
      if (stage_n + 64 > kXStage) flush();
      if (cand) {
        const int t = c >> 3, t2 = (c >> 2) & 1, r = c & 3;
        const int e = stage_n + mbcnt(b);
        const int qi = 16 * t2 + 4 * lg + r;
        const int32_t score = S.sc[c][l];
        const int32_t pos = (int32_t)(p0 + 16 * t + lr);
        S.key[e] = pos_key(score, pos);
        S.qi[e] = (uint8_t)qi;
        S.rank[e] = (uint16_t)atomicAdd(&S.cnt[qi], 1u);
      }
      stage_n += __popcll(b);
    }
    wave_lds_sync();
  };
  // the walk: XNB - 1 steps in flight ahead of the one scored
  StepRows rows[XNB];
  StepSigs sigs[XNB];
#pragma unroll
  for (int b = 0; b < XNB - 1; ++b) load_step(b, rows[b], sigs[b]);
  const int64_t n_iter = (my_steps + XNB - 1) / XNB;
  for (int64_t it = 0; it < n_iter; ++it) {
#pragma unroll
    for (int b = 0; b < XNB; ++b) {
      const int64_t j = it * XNB + b;
      load_step(j + XNB - 1, rows[(b + XNB - 1) % XNB], sigs[(b + XNB - 1) % XNB]);
      score_step(j, rows[b], sigs[b]);   // past the share: zero rows, no item in range
    }
  }
  if constexpr (!SAMPLE) {
    if (stage_n > 0) flush();
    // eligible items of each query of the block, summed over the 16 lanes that hold its items
    if (a.w.stats) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint32_t v = ec[t2][r];
          v += __shfl_xor(v, 1);
          v += __shfl_xor(v, 2);
          v += __shfl_xor(v, 4);
          v += __shfl_xor(v, 8);
          const int q = q0 + 16 * t2 + 4 * lg + r;
          if (lr == 0 && q < a.B && v)
            atomicAdd((unsigned long long *)&a.w.stats[2 * (size_t)q + 1], (unsigned long long)v);
        }
    }
  }
}

// Thresholds from the sample pass.  Every slot of a query's sample buffer holds the best eligible score
// among a few sampled items (INT32_MIN when none passed), the slots covering disjoint items.  Each thread
// takes the best of its slots; the r-th best of those per-thread maxima is the threshold, r for kAlpha * k
// items over the whole catalogue (at least kRMin): r distinct sampled items score at or above it.  With
// r far below the thread count it sits close to the r-th best sample.  No threshold when the pool holds
// the whole catalogue or fewer than r threads saw an eligible sample.
__global__ __launch_bounds__(kSelThreads) void k_xthr(Work w, int64_t n_items, int32_t k, int32_t pool_cap,
                                                      int32_t scap, int32_t n_points, int32_t force) {
  __shared__ SelScratch sel;
  __shared__ int wave_tot[kSelThreads / 64 + 1];
  const int q = blockIdx.x, tid = threadIdx.x;
  const int32_t *sb = w.sbuf + (size_t)q * scap;
  int32_t st = INT32_MIN;
  int r = 0;
  if (n_items > pool_cap && n_points > 0) {
    const int64_t r0 = ((int64_t)kAlpha * k * n_points + n_items - 1) / n_items;
    r = (int)(r0 > kRMin ? r0 : kRMin);
  }
  if (r > 0 && r <= kSelThreads) {   // uniform over the block
    int32_t mx = INT32_MIN;
    for (int i0 = tid; i0 < scap; i0 += 8 * kSelThreads) {
      int32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = i0 + u * kSelThreads < scap ? sb[i0 + u * kSelThreads] : INT32_MIN;
#pragma unroll
      for (int u = 0; u < 8; ++u) mx = v[u] > mx ? v[u] : mx;
    }
    int have;
    block_excl_scan<kSelThreads>(mx != INT32_MIN ? 1 : 0, wave_tot, &have);
    if (have >= r) {
      const uint64_t T = block_select<kSelThreads>(
          [&](auto f) {
            if (mx != INT32_MIN) f(make_key(mx, (uint32_t)tid));
          },
          r, sel);
      st = key_score(T);
    }
  }
  if (force) st = INT32_MAX;
  if (tid == 0) w.sthr[q] = st;
}

// ------------------------------------------------------------------------------------------------
// k_pmerge: one workgroup per query whose pool proves its top k.  The k-th best (score, position) key
// fixes the k-th best score; every key at that score or above becomes a (score, id) key, and the exact
// top k of those is sorted and written.  A pool of at most kPoolLds keys is staged in LDS with one
// batch of loads per thread and merged there; a larger one is read from HBM at each step.

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

constexpr int kPoolLds = 19 * kSelThreads;   // pool keys merged in LDS (152 KB of the 160 KB)
static_assert(kPoolLds >= kMergeCap, "the LDS merge holds at least the staging capacity");

// Keep the keys >= lo of cand[0..n) (n <= kPoolLds), in place, as (score, id) keys when to_id; returns
// the count kept.  Each thread reads its keys (and their ids) before the block scan's barriers and
// writes them after.
__device__ __forceinline__ int pool_keep(uint64_t *cand, int n, uint64_t lo, bool to_id, const int32_t *perm,
                                         int *wave_tot) {
  constexpr int PER = kPoolLds / kSelThreads;
  const int tid = threadIdx.x;
  uint64_t kv[PER];
  uint32_t idv[PER];
  int keep = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = u * kSelThreads + tid;
    kv[u] = i < n ? cand[i] : 0ull;
    const bool k_ = i < n && kv[u] >= lo;
    keep += k_ ? 1 : 0;
    idv[u] = (k_ && to_id) ? (uint32_t)perm[(uint32_t)kv[u]] : 0u;
  }
  int tot;
  int off = block_excl_scan<kSelThreads>(keep, wave_tot, &tot);   // barriers inside
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int i = u * kSelThreads + tid;
    if (i < n && kv[u] >= lo)
      cand[off++] = to_id ? make_key((int32_t)((uint32_t)(kv[u] >> 32) ^ 0x80000000u), idv[u]) : kv[u];
  }
  __syncthreads();
  return tot;
}

__global__ __launch_bounds__(kSelThreads) void k_pmerge(PMergeArgs a) {
  __shared__ SelScratch sel;
  __shared__ uint64_t cand[kPoolLds];
  __shared__ int wave_tot[kSelThreads / 64 + 1];
  __shared__ int ncand;
  const int q = blockIdx.x, tid = threadIdx.x, k = a.k;
  if (a.w.redo[q]) return;   // merged by the query path
  const int n = (int)a.w.pool_cnt[q];
  uint64_t *pool = a.w.pool + (size_t)q * a.pool_cap;
  const int nout = n < k ? n : k;
  int m;
  if (n <= kPoolLds) {
    constexpr int PER = kPoolLds / kSelThreads;
    uint64_t v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = u * kSelThreads + tid;
      v[u] = i < n ? pool[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = u * kSelThreads + tid;
      if (i < n) cand[i] = v[u];
    }
    __syncthreads();
    m = n;
    if (n > k) {
      const uint64_t T = block_select<kSelThreads>(
          [&](auto f) {
            for (int i = tid; i < n; i += kSelThreads) f(cand[i]);
          },
          k, sel);
      // every key with the k-th best score or better, as (score, id) keys
      m = pool_keep(cand, n, (T >> 32) << 32, true, a.ix.perm, wave_tot);
      if (m > k) {
        const uint64_t Tk = block_select<kSelThreads>(
            [&](auto f) {
              for (int i = tid; i < m; i += kSelThreads) f(cand[i]);
            },
            k, sel);
        m = pool_keep(cand, m, Tk, false, a.ix.perm, wave_tot);   // exactly k distinct keys
      }
    } else {
      m = pool_keep(cand, n, 0ull, true, a.ix.perm, wave_tot);
    }
  } else {
    // a pool larger than LDS: select in HBM.  Every sweep over the pool loads 8 keys per thread before
    // using any (pool_visit), so a sweep waits for the memory about n / (8 * kSelThreads) times.
    auto pool_visit = [&](auto f) {
      for (int i0 = tid; i0 < n; i0 += 8 * kSelThreads) {
        uint64_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * kSelThreads;
          v[u] = i < n ? pool[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + u * kSelThreads < n) f(i0 + u * kSelThreads, v[u]);
      }
    };
    const uint64_t T = block_select<kSelThreads>([&](auto f) { pool_visit([&](int, uint64_t v) { f(v); }); }, k, sel);
    const uint64_t lo = (T >> 32) << 32;   // the smallest key with the k-th best score
    // keys at or above lo become (score, id) keys in place; their upper half, the score, is unchanged
    pool_visit([&](int i, uint64_t v) {
      if (v >= lo) pool[i] = make_key((int32_t)((uint32_t)(v >> 32) ^ 0x80000000u), (uint32_t)a.ix.perm[(uint32_t)v]);
    });
    if (tid == 0) ncand = 0;
    __syncthreads();
    pool_visit([&](int, uint64_t v) {
      if (v >= lo) {
        const int o = atomicAdd(&ncand, 1);
        if (o < kPoolLds) cand[o] = v;
      }
    });
    __syncthreads();
    m = ncand;
    if (m > kPoolLds) {
      // heavy ties at the k-th score: select among the converted keys in the pool
      const uint64_t Tk = block_select<kSelThreads>(
          [&](auto f) {
            pool_visit([&](int, uint64_t v) {
              if (v >= lo) f(v);
            });
          },
          k, sel);
      if (tid == 0) ncand = 0;
      __syncthreads();
      pool_visit([&](int, uint64_t v) {
        if (v >= lo && v >= Tk) cand[atomicAdd(&ncand, 1)] = v;   // exactly k distinct keys
      });
      __syncthreads();
      m = k;
    } else if (m > k) {
      const uint64_t Tk = block_select<kSelThreads>(
          [&](auto f) {
            for (int i = tid; i < m; i += kSelThreads) f(cand[i]);
          },
          k, sel);
      m = pool_keep(cand, m, Tk, false, a.ix.perm, wave_tot);
    }
  }
  static_assert(kPoolLds >= 4 * kSelThreads, "emit_sorted needs room for 4 keys per thread");
  emit_sorted<kSelThreads>(cand, m, nout, q, k, a.query_scales, a.item_scale, a.out_ids, a.out_scores,
                           a.out_fscores);
  if (tid == 0 && a.out_counts) a.out_counts[q] = nout;
}

// ------------------------------------------------------------------------------------------------
// launch wrappers

hipError_t launch_tile_plan(const DevIndex &ix, const uint64_t *masks, const SearchShape &sh, const Work &w,
                            hipStream_t s) {
  k_tplan1<<<(ix.nlist + kSelThreads - 1) / kSelThreads, kSelThreads, 0, s>>>(ix, w);
  k_tplan2<<<(ix.nlist + kSelThreads - 1) / kSelThreads + 1, kSelThreads, 0, s>>>(ix, sh.TP, w);
  const int ne_blocks = (sh.max_entries + 255) / 256, nc_blocks = (sh.max_tchunks + 256) / 256;
  k_tfill<<<sh.B + ne_blocks + nc_blocks, 256, 0, s>>>(ix, w.probes, masks, sh.B, sh.nprobe, sh.G, sh.GT,
                                                       sh.max_entries, ne_blocks, sh.max_tchunks, w);
  return hipGetLastError();
}

template <int LPR>
static void tscan_w(const TScanArgs &a, int W, hipStream_t s) {
  if (W == 2)
    k_tscan<LPR, 2><<<a.P, kScanThreads, 0, s>>>(a);
  else
    k_tscan<LPR, 1><<<a.P, kScanThreads, 0, s>>>(a);
}

hipError_t launch_tscan(const DevIndex &ix, const int8_t *queries, const SearchShape &sh, const Work &w,
                        hipStream_t s) {
  TScanArgs a{ix, queries, w, sh.B, sh.TP, (uint32_t)sh.pool_cap, sh.GT};
  switch (ix.dim) {
    case 16: tscan_w<1>(a, ix.sig_words, s); break;
    case 32: tscan_w<2>(a, ix.sig_words, s); break;
    case 64: tscan_w<4>(a, ix.sig_words, s); break;
    case 128: tscan_w<8>(a, ix.sig_words, s); break;
    case 256: tscan_w<16>(a, ix.sig_words, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int LPR>
static int tscan_occ_w(int W) {
  int n = 0;
  hipError_t e = W == 2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_tscan<LPR, 2>, kScanThreads, 0)
                        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_tscan<LPR, 1>, kScanThreads, 0);
  return e == hipSuccess ? n : 0;
}

int tscan_blocks_per_cu(int32_t dim, int32_t sig_words) {
  switch (dim) {
    case 16: return tscan_occ_w<1>(sig_words);
    case 32: return tscan_occ_w<2>(sig_words);
    case 64: return tscan_occ_w<4>(sig_words);
    case 128: return tscan_occ_w<8>(sig_words);
    case 256: return tscan_occ_w<16>(sig_words);
    default: return 0;
  }
}

template <int KS, bool SAMPLE>
static void xscan_w(const XScanArgs &a, int W, int grid, hipStream_t s) {
  const bool multi = a.G > 1;   // requests of several masks: a variant, so that one mask costs nothing more
  if (W == 2) {
    if (multi) k_xscan<KS, 2, SAMPLE, true><<<grid, 64 * kXWaves, 0, s>>>(a);
    else k_xscan<KS, 2, SAMPLE, false><<<grid, 64 * kXWaves, 0, s>>>(a);
  } else {
    if (multi) k_xscan<KS, 1, SAMPLE, true><<<grid, 64 * kXWaves, 0, s>>>(a);
    else k_xscan<KS, 1, SAMPLE, false><<<grid, 64 * kXWaves, 0, s>>>(a);
  }
}

template <bool SAMPLE>
static hipError_t xscan_dim(const XScanArgs &a, int dim, int W, int grid, hipStream_t s) {
  switch (dim) {
    case 16:
    case 32:
    case 64: xscan_w<1, SAMPLE>(a, W, grid, s); break;
    case 128: xscan_w<2, SAMPLE>(a, W, grid, s); break;
    case 256: xscan_w<4, SAMPLE>(a, W, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipSuccess;
}

int xscan_blocks_per_cu(int32_t dim, int32_t sig_words) {
  int n = 0;
  hipError_t e = hipSuccess;
  const bool w2 = sig_words == 2;
  switch (dim) {
    case 16:
    case 32:
    case 64:
      e = w2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_xscan<1, 2, false, false>, 64 * kXWaves, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_xscan<1, 1, false, false>, 64 * kXWaves, 0);
      break;
    case 128:
      e = w2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_xscan<2, 2, false, false>, 64 * kXWaves, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_xscan<2, 1, false, false>, 64 * kXWaves, 0);
      break;
    case 256:
      e = w2 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_xscan<4, 2, false, false>, 64 * kXWaves, 0)
             : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_xscan<4, 1, false, false>, 64 * kXWaves, 0);
      break;
    default: return 0;
  }
  return e == hipSuccess ? n : 0;
}

hipError_t launch_exh_scan(const DevIndex &ix, const int8_t *queries, const uint64_t *masks,
                           const SearchShape &sh, const Work &w, hipStream_t s) {
  const int n_qb = (sh.B + kXQ - 1) / kXQ;
  const int64_t N = ix.n_items;
  // every query block needs a wave: at least n_qb waves in the grid
  const int grid = std::max(sh.XP, (n_qb + kXWaves - 1) / kXWaves);
  // sample pass, thresholds, main pass
  XScanArgs as{ix, queries, masks, w, sh.B, n_qb, (uint32_t)sh.scap, sh.G};
  hipError_t e = xscan_dim<true>(as, ix.dim, ix.sig_words, grid, s);
  if (e != hipSuccess) return e;
  k_xthr<<<sh.B, kSelThreads, 0, s>>>(w, N, sh.k, sh.pool_cap, sh.scap, (int32_t)((N + kXStride - 1) / kXStride),
                                      sh.force_redo);
  XScanArgs am{ix, queries, masks, w, sh.B, n_qb, (uint32_t)sh.pool_cap, sh.G};
  e = xscan_dim<false>(am, ix.dim, ix.sig_words, grid, s);
  if (e != hipSuccess) return e;
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
