// svt_internal.h - declarations shared by the host API (svt_api.cpp) and the gfx950 kernels
// (svt_kernels.hip).  Not installed; the public boundary is include/svt.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svt {

constexpr int kMaxK = 2048;          // largest top-k (SVT_MAX_K)
constexpr int kScanThreads = 256;    // fused filter-score-select workgroup: 4 wave64
#ifndef SVT_SCAN_GROUPS
#define SVT_SCAN_GROUPS 5
#endif
constexpr int kScanGroups = SVT_SCAN_GROUPS;   // 64-item groups per wave per step
constexpr int kScanStep = kScanThreads * kScanGroups;   // items per workgroup step (1280)
#ifndef SVT_SCAN_OCC
#define SVT_SCAN_OCC 3
#endif
#ifndef SVT_SCAN_ROW_BATCH
#define SVT_SCAN_ROW_BATCH 40
#endif
constexpr int kScanOcc = SVT_SCAN_OCC;              // query-by-query scan: waves per SIMD (workgroups per CU)
constexpr int kScanRowBatch = SVT_SCAN_ROW_BATCH;   // rows a wave gathers together, rounded down to whole loads
#ifndef SVT_LIST_CAP
#define SVT_LIST_CAP 4096
#endif
constexpr int kListCap = SVT_LIST_CAP;                  // LDS candidate list capacity (keys)
constexpr int kTrimAt = kListCap - kScanStep;           // a list longer than this is trimmed
// a trim cuts the list to at least k keys and must leave room for a step's appends
static_assert(kTrimAt >= kMaxK, "the candidate list must hold k keys plus one step");
constexpr int kTrimBinsLog2 = 9;
constexpr int kTrimBins = 1 << kTrimBinsLog2;           // score histogram bins of a trim
constexpr int kSegWin = 64;                             // probed clusters staged in LDS at a time
constexpr int kQHistBins = 256;                         // bins of a query's global score histogram
constexpr int kSelThreads = 1024;    // coarse-select and merge workgroups
static_assert(2 * kSelThreads >= kMaxK, "the final sort holds two keys per merge thread");
#ifndef SVT_COARSE_QB
#define SVT_COARSE_QB 16
#endif
constexpr int kCoarseQB = SVT_COARSE_QB;   // queries per coarse-score workgroup
constexpr int kMaxScanWGs = 4096;    // upper bound on persistent scan workgroups

// Device-resident index.  Items of cluster c occupy positions [offsets[c], offsets[c+1]); within a
// cluster positions follow item id order.  perm[p] is the caller's id of the item at position p.
struct DevIndex {
  const int8_t *items;      // [n][dim]
  const uint64_t *sigs;     // [n][sig_words]
  const int32_t *perm;      // [n]
  const int32_t *offsets;   // [nlist + 1]
  const int8_t *centroids;  // [nlist][dim]
  int64_t n_items;
  int32_t dim, sig_words, nlist;
  float item_scale;
};

// One unit of scan work: items [lo, hi) of query q's stream (the concatenation, in cluster order, of
// the items of its probed clusters); j0 is the probed cluster that holds stream offset lo.
struct Chunk {
  int32_t q, lo, hi, j0;
};

constexpr int kCostSamples = kSelThreads;   // items sampled per query to estimate its filter density
// Per-item work of the scan besides its bytes (filter, compaction, bookkeeping), in byte equivalents of
// the chunk cost model.  Measured on the 80M-item catalogue at batch 256: 12 to 24 give the shortest
// scan and merge (sparse filters get shorter chunks, dense ones fewer); 0.125 was 2.5 % slower in the
// scan and 40 % slower in the merge.
#ifndef SVT_ITEM_COST
#define SVT_ITEM_COST 16.0
#endif
constexpr double kItemCost = SVT_ITEM_COST;
constexpr int kMaxChunksPerQuery = 2048;    // a query's stream is cut into at most this many chunks
#ifndef SVT_MERGE_CAP
#define SVT_MERGE_CAP 6144
#endif
constexpr int kMergeCap = SVT_MERGE_CAP;      // merge candidates staged in LDS
constexpr int kMergeGatherWGs = 2048;       // persistent workgroups gathering slot keys for the merge
constexpr int kGatherCap = 3 * kMergeCap;   // keys gathered per query above its final bound
static_assert(kMergeCap >= kMaxK && kMergeCap % kSelThreads == 0,
              "the merge stages at least k keys, a whole number per thread");
constexpr int kSelSegLds = 4096;            // probe lists up to this long are searched in LDS
constexpr int64_t kMinChunkCost = 16 << 10; // smallest chunk, in estimated bytes moved
constexpr int kPlanBands = 256;             // cluster-id bands of the scan's queue order
// The queue ends with the chunks of the highest bands.  Items of a query's probed clusters in bands
// kTailBand and above are cut into chunks kTailDiv times shorter, so that the workgroups taking the last
// chunks finish closer together.  kTailBand == kPlanBands: no shorter chunks.
#ifndef SVT_TAIL_BAND
#define SVT_TAIL_BAND 160
#endif
#ifndef SVT_TAIL_DIV
#define SVT_TAIL_DIV 2
#endif
constexpr int kTailBand = SVT_TAIL_BAND;
constexpr int kTailDiv = SVT_TAIL_DIV;
static_assert(kTailBand >= 0 && kTailBand <= kPlanBands && kTailDiv >= 1, "tail region");

// Grouped path: one unit of work is a tile of at most kGTile items of one probed cluster together
// with a group of at most kGMax of the queries that probe that cluster (gq[q0..q1)).
constexpr int kGTile = 4096;
constexpr int kGMax = 16;
constexpr int kGScanOcc = 4;         // grouped scan: workgroups per CU (4 independent waves each)
struct GUnit {
  int32_t c, lo, hi, q0, q1, pad0, pad1, pad2;   // items at positions [lo, hi) of cluster c
};

// Per-search device workspace (carved by the host from the caller's buffer).
struct Work {
  int32_t *coarse_scores;   // [B][nlist]   coarse scores <query, centroid>
  int32_t *probes;          // [B][nprobe]  probed clusters, ascending cluster id
  int32_t *seg;             // [B][nprobe + 1] stream offset of each probed cluster within its query
  int32_t *pb;              // [B][nprobe]  position of stream offset t in probed cluster j: pb[j] + t
  int64_t *qlen;            // [B]          items scanned per query
  int64_t *qcost;           // [B]          estimated bytes the scan moves for the query
  int32_t *qtail;           // [B][2]       stream offset where the query's tail region starts; its first chunk
  int32_t *cstart;          // [B + 1]      first chunk of each query; cstart[B] = number of chunks
  Chunk *chunks;            // [max_chunks] the work list, in query order
  int32_t *order;           // [max_chunks] the order in which the scan takes the chunks
  int32_t *cband;           // [max_chunks] band of the probed cluster each chunk starts in
  int32_t *thr;             // [B]          per-query proven lower bound on the k-th best score
  int32_t *hlo;             // [B]          score at the lower edge of bin 1 of the query's histogram
  int32_t *hshift;          // [B]          bin width of that histogram is 2^hshift
  uint32_t *ghist;          // [B][kQHistBins] scores of every candidate any chunk accepted
  uint32_t *counter;        // [3]          select completion counter, scan and grouped-scan queue heads
  int32_t *slot_cnt;        // [max_chunks] candidates each chunk left
  uint64_t *slot_min;       // [max_chunks] smallest key of a slot holding k keys, else 0
  uint64_t *slot_keys;      // [max_chunks][k] those candidates (score/id keys)
  uint64_t *mbound;         // [B]          the query's final proven bound, as the smallest key it admits
  uint32_t *mcnt;           // [B]          slot keys at or above it (more than kGatherCap: not all kept)
  uint64_t *mkeys;          // [B][kGatherCap] those keys, gathered from the query's slots
  int64_t *stats;           // [B][2] scanned / eligible (caller buffer or workspace)
  // grouped path (null when the search runs query by query)
  int32_t *gcnt;            // [nlist]      queries probing each cluster
  int32_t *gfill;           // [nlist]      fill cursor of each cluster's query list
  int32_t *gstart;          // [nlist + 1]  each cluster's query list in gq
  int32_t *ustart;          // [nlist + 1]  first unit of each cluster; ustart[nlist] = number of units
  int32_t *gq;              // [B * nprobe] queries of every probed cluster, grouped by cluster
  GUnit *units;             // [max_units]
  uint32_t *pool_cnt;       // [B]          candidates offered to each query's pool (> pool_cap: overflow)
  uint64_t *pool;           // [B][pool_cap] (score, position) keys of the candidates
};

struct SearchShape {
  int32_t B, nprobe, k, P, max_chunks;
  int32_t grouped;     // 1: grouped path with the query-by-query scan as fallback for overflowing pools
  int32_t pool_cap;    // keys per query pool
  int32_t max_units;
  int32_t GP;          // persistent workgroups of the grouped scan
  int32_t gather_cap;  // keys the merge gathers per query (at most kGatherCap)
};

// most chunks a search can produce.  The costs of the queries add up to at most 4 P Tc.  Without a tail
// region a query of estimated cost c gets at most c / Tc + 1 chunks; with one, at most kTailDiv c / Tc + 2
// (two regions), or kTailDiv + 1 when it is shorter than one chunk.
inline int32_t max_chunks_for(int32_t B, int32_t P) {
  return kTailBand < kPlanBands ? 4 * kTailDiv * P + (kTailDiv + 1) * B + 1 : 4 * P + B + 1;
}

// launch wrappers (svt_kernels.hip); each returns hipSuccess or the launch error
hipError_t launch_coarse_keys(const DevIndex &ix, const int8_t *queries, int32_t B, const Work &w,
                              hipStream_t s);
hipError_t launch_coarse_select(const DevIndex &ix, const int8_t *queries, const uint64_t *masks,
                                const SearchShape &sh, const Work &w, hipStream_t s);
hipError_t launch_scan(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const SearchShape &sh,
                       const Work &w, hipStream_t s);
// launch_merge: k_merge_bound, k_merge_gather (query-by-query search only), then k_merge
hipError_t launch_merge(const DevIndex &ix, const float *query_scales, const SearchShape &sh, const Work &w,
                        int64_t *out_ids, int32_t *out_scores, float *out_fscores, int32_t *out_counts,
                        hipStream_t s);
// grouped path (svt_group.hip)
hipError_t launch_group_plan(const DevIndex &ix, const SearchShape &sh, const Work &w, hipStream_t s);
hipError_t launch_gscan(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const SearchShape &sh,
                        const Work &w, hipStream_t s);
hipError_t launch_pool_merge(const DevIndex &ix, const float *query_scales, const SearchShape &sh, const Work &w,
                             int64_t *out_ids, int32_t *out_scores, float *out_fscores, int32_t *out_counts,
                             hipStream_t s);
// resident scan workgroups per compute unit for this shape (0 if unknown)
int scan_blocks_per_cu(int32_t dim, int32_t sig_words);
int gscan_blocks_per_cu(int32_t dim, int32_t sig_words);
hipError_t launch_scatter_rows(const int8_t *src_rows, const uint64_t *src_sigs, const int32_t *pos_of,
                               int64_t i0, int64_t n, int32_t dim, int32_t sig_words, int8_t *dst_rows,
                               uint64_t *dst_sigs, hipStream_t s);

}  // namespace svt
