// svt_internal.h - declarations shared by the host API (svt_api.cpp) and the gfx950 kernels
// (svt_kernels.hip).  Not installed; the public boundary is include/svt.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svt.h"

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
// The index in HBM.  Cluster c owns the slots [offsets[c], offsets[c + 1]): its items, in id order at
// upload, then (an updatable index) free slots.  A free slot holds the reserved signature with every bit
// set, which no filter passes, and the id -1; live[c] counts the cluster's items.
struct DevIndex {
  const int8_t *items;      // [n][dim]
  const uint64_t *sigs;     // [n][sig_words]
  const int32_t *perm;      // [n]         id of the item in each slot (-1: free)
  const int32_t *offsets;   // [nlist + 1]
  const int32_t *live;      // [nlist]     items (not free slots) of each cluster
  const int32_t *slot_of;   // [n_ids]     slot of each id (-1: not in the index)
  const int8_t *centroids;  // [nlist][dim]
  int64_t n_items;          // slots
  int64_t n_ids;            // ids: [0, n_ids)
  int32_t dim, sig_words, nlist;
  float item_scale;
};

// One unit of scan work: items [lo, hi) of query q's stream (the concatenation, in cluster order, of
// the items of its probed clusters); j0 is the probed cluster that holds stream offset lo.
struct Chunk {
  int32_t q, lo, hi, j0;
};

constexpr int kCostSamples = kSelThreads;   // items sampled per query to estimate its filter density
constexpr int kSampleMax = 8;               // tile path: samples per select thread, at most
constexpr int64_t kSampleSpan = 256 << 10;  // tile path: one more sample per thread for each this many items
constexpr int kSelElig = 2048;              // tile path: eligible samples the select scores (every stride-th)
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
constexpr int kPlanSmallBatch = 4;          // query path: batches up to this size plan in one workgroup
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

// Tile path.  The batch's probed clusters form one union stream: for every probed cluster, in cluster
// order, one entry per block of at most kTMembers of the queries probing it (a cluster probed by more
// queries appears once per block).  The stream is cut into chunks that the waves of persistent workgroups
// take from a queue; every item of an entry is tested against the masks of the entry's members and the
// rows of the items any member accepts are gathered once and scored for each member that accepts them.
constexpr int kTMembers = 16;        // queries of one union entry (member bits of a survivor: uint16)
constexpr int kTWaves = kScanThreads / 64;   // waves of a tile-scan workgroup (each works alone)
#ifndef SVT_T_CHUNKS
#define SVT_T_CHUNKS 4
#endif
constexpr int kTChunksPerWave = SVT_T_CHUNKS;   // chunks of the union stream per wave of the scan
#ifndef SVT_T_GROUPS
#define SVT_T_GROUPS 4
#endif
constexpr int kTGroups = SVT_T_GROUPS;   // 64-item signature groups of one filter step
#ifndef SVT_T_ROWLOADS
#define SVT_T_ROWLOADS 4
#endif
constexpr int kTRowLoads = SVT_T_ROWLOADS;   // 16-byte row loads per lane of one scored batch
#ifndef SVT_T_OCC
#define SVT_T_OCC 4
#endif
constexpr int kTOcc = SVT_T_OCC;             // tile-scan waves per SIMD the compiler is asked to fit
// Chunks of the union stream are cut at equal estimated cost: per item of an entry, its signature bytes and
// kTItemCost byte equivalents of other work, kTMemberCost per member; the rows of the fraction of items some
// member accepts (from the members' sampled densities).
constexpr int kTItemCost = 16;
constexpr int kTMemberCost = 2;
// Speculative thresholds: a query's threshold is the score that an estimated kAlpha * k of its eligible
// items reach, read off a sample of its items at rank at least kRMin; the pool keeps every candidate at
// or above it.  A pool with fewer than k keys (threshold above the minimum) or more than it holds sends
// its query to the query path.
#ifndef SVT_ALPHA
#define SVT_ALPHA 4
#endif
constexpr int kAlpha = SVT_ALPHA;
constexpr int kRMin = 16;
// Exhaustive batches (nprobe == nlist): the catalogue is streamed once per block of kXQ queries and
// scored with int8 MFMA (16x16x64).  The sample pass scores every kXStride-th item.
constexpr int kXQ = 32;              // queries of one MFMA unit (two 16-row MFMA tiles)
constexpr int kXStride = 256;        // sample pass: every kXStride-th position
constexpr int kXWaves = 4;           // waves of an exhaustive workgroup (each works on its own)
#ifndef SVT_X_BUFFERS
#define SVT_X_BUFFERS 2
#endif
#ifndef SVT_X_OCC
#define SVT_X_OCC 3
#endif
constexpr int kXBuffers = SVT_X_BUFFERS;   // steps of the exhaustive scan in registers (in flight + scored)
constexpr int kXOcc = SVT_X_OCC;           // its waves per SIMD the compiler is asked to fit
constexpr int kXStage = 256;         // candidates a wave of the exhaustive kernel stages in LDS

constexpr int kMaxPlanBlocks = 65536 / kSelThreads;   // blocks of kSelThreads clusters (nlist <= 65536)
struct MRec {                        // one member of a union entry
  uint64_t m0, m1;                   // request mask (m1 = 0 for 64-bit signatures)
  int32_t thr, q;                    // speculative threshold, query index
};
struct UEntry {                      // one entry of the union stream
  int32_t useg, len, pos0, mstart;   // stream offset, items, first position, first member in mrec
  int32_t mcnt, pad0, pad1, pad2;    // members
};

// Per-search device workspace (carved by the host from the caller's buffer).
// Searches with k above SVT_MAX_K (svt_largek.hip): a radix select over 55-bit keys, 11-bit digits from
// bit 44 down, one counting pass over the probed items per digit, then a collect pass
constexpr int kLkDigit = 11, kLkBins = 1 << kLkDigit, kLkTopShift = 44, kLkPasses = 5;
constexpr int kLkChunk = 4096;   // stream positions per chunk of a pass
constexpr int kLkScanWGs = 2048; // workgroups of a pass, walking the batch's chunks
struct LkState {
  uint64_t prefix;   // key bits fixed so far; once done, the threshold (0: every eligible key)
  int32_t shift;     // lowest bit of the digit the next pass counts
  int32_t need;      // keys still to take in the bucket the prefix names
  int32_t done;      // 0: selecting; kLkDone: threshold final; kLkFromPool: the pool gave the k keys
  int32_t pad;
};
constexpr int32_t kLkDone = 1, kLkFromPool = 2;

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
  uint32_t *counter;        // [8]          queue heads (query scan, tile scan, exhaustive sample and scan)
  int32_t *slot_cnt;        // [max_chunks] candidates each chunk left
  uint64_t *slot_min;       // [max_chunks] smallest key of a slot holding k keys, else 0
  uint64_t *slot_keys;      // [max_chunks][k] those candidates (score/id keys)
  uint32_t *mcnt;           // [B]          slot keys at or above the query's final proven bound (more than
                            //              kGatherCap: not all kept)
  uint64_t *mkeys;          // [B][kGatherCap] those keys, gathered from the query's slots
  int64_t *stats;           // [B][2] scanned / eligible (caller buffer or workspace)
  // tile path (null on the query path)
  int32_t *sthr;            // [B]          speculative threshold of each query
  int32_t *redo;            // [B]          1: the query is redone on the query path
  uint32_t *pool_cnt;       // [B]          candidates offered to each query's pool (> pool_cap: overflow)
  uint64_t *pool;           // [B][pool_cap] (score, position) keys at or above the threshold
  int32_t *gcnt;            // [nlist]      queries probing each cluster
  int32_t *gfill;           // [nlist]      fill cursor of each cluster's member list
  int32_t *gstart;          // [nlist + 1]  each cluster's members in mrec
  int32_t *estart;          // [nlist + 1]  each cluster's first union entry
  int32_t *uoff;            // [nlist]      union-stream offset of each cluster's first entry
  MRec *mrec;               // [B * nprobe] members of every probed cluster, grouped by cluster
  UEntry *entries;          // [max_entries]
  int32_t *ctab;            // [max_tchunks] first entry of each chunk
  int32_t *thdr;            // [4]          entries, union-stream length, chunks, 0
  int64_t *tblk;            // [4 * kMaxPlanBlocks] per block of kSelThreads clusters: members, entries, items, cost
  float *qdens;             // [B]          sampled fraction of the query's items that pass its mask
  float *clog;              // [nlist]      sum over the cluster's members of log(1 - density)
  int64_t *ccost;           // [nlist + 1]  prefix of the clusters' estimated costs
  int32_t *cstart_u;        // [max_tchunks + 1] union-stream offset where each chunk starts
  int32_t *sbuf;            // [B][scap]    exhaustive sample pass: per lane and run, the best eligible score
  // searches with k > SVT_MAX_K (null otherwise)
  uint32_t *lk_hist;        // [B][kLkBins] the current pass's digit counts
  LkState *lk_state;        // [B]
  uint32_t *lk_cnt;         // [B]          keys collected
  uint64_t *lk_keys;        // [B][k]       the collected keys, unordered
  int32_t *lk_cstart;       // [B + 1]      first chunk of each query's stream (kLkChunk positions each)
};

enum { kPathQuery = 0, kPathTile = 1, kPathExh = 2, kPathLargeK = 3 };

constexpr int kMaxGroups = 4;   // masks per query (SVT_MAX_MASK_GROUPS)

struct SearchShape {
  int32_t B, nprobe, k, P, max_chunks;
  int32_t path;         // kPath*
  int32_t pool_cap;     // keys per query pool (tile and exhaustive paths)
  int32_t max_entries;  // union entries (tile path)
  int32_t max_tchunks;  // chunks of the union stream
  int32_t TP;           // persistent workgroups of the tile scan
  int32_t XP;           // workgroups of the exhaustive kernel
  int32_t gather_cap;   // keys the merge gathers per query (at most kGatherCap)
  int32_t force_redo;   // every threshold above any score (test of the redo branch)
  int32_t scap;         // exhaustive: slots of a query's sample buffer (16 per run of 64 sampled points)
  int32_t n_sblocks;    // exhaustive: runs of 64 sampled points
  int32_t G;            // request masks per query (masks [B][G][sig_words])
  int32_t GT;           // tile path: members per (query, probed cluster), G rounded up to 1, 2 or 4 (a power of
                        // two dividing kTMembers, so that a query's members never straddle two entries)
  int32_t lk_tile;      // large-k path: the pools are filled by the tile scan ((score, slot) keys)
};

// most chunks a search can produce.  The costs of the queries add up to at most 4 P Tc.  Without a tail
// region a query of estimated cost c gets at most c / Tc + 1 chunks; with one, at most kTailDiv c / Tc + 2
// (two regions), or kTailDiv + 1 when it is shorter than one chunk.
inline int32_t max_chunks_for(int32_t B, int32_t P) {
  return kTailBand < kPlanBands ? 4 * kTailDiv * P + (kTailDiv + 1) * B + 1 : 4 * P + B + 1;
}

// launch wrappers (svt_kernels.hip, svt_tile.hip); each returns hipSuccess or the launch error
hipError_t launch_coarse_keys(const DevIndex &ix, const int8_t *queries, int32_t B, const Work &w, hipStream_t s);
// k_coarse_select: probes, stream layout, samples; tile path: speculative thresholds
hipError_t launch_coarse_select(const DevIndex &ix, const int8_t *queries, const uint64_t *masks,
                                const SearchShape &sh, const Work &w, hipStream_t s);
// the query path's work list (k_plan_count, k_plan_chunks, k_plan_order; k_plan_small for batches of at
// most kPlanSmallBatch queries); redo != 0 (tile path, k_plan_redo): the queries whose pools cannot prove
// their top k are marked in w.redo, and only those get chunks
hipError_t launch_plan(const DevIndex &ix, const SearchShape &sh, const Work &w, int redo, hipStream_t s);
// k_scan; fallback != 0: the redo of the tile path (per-query statistics are not counted again)
hipError_t launch_scan(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const SearchShape &sh,
                       const Work &w, int fallback, hipStream_t s);
// k_merge_gather, k_merge; fallback != 0: only the queries marked for redo, merged from
// their chunks' slots (k_merge alone)
hipError_t launch_merge(const DevIndex &ix, const float *query_scales, const SearchShape &sh, const Work &w,
                        int fallback, int64_t *out_ids, int32_t *out_scores, float *out_fscores,
                        int32_t *out_counts, hipStream_t s);
// tile path (svt_tile.hip)
hipError_t launch_tile_plan(const DevIndex &ix, const uint64_t *masks, const SearchShape &sh, const Work &w,
                            hipStream_t s);
hipError_t launch_tscan(const DevIndex &ix, const int8_t *queries, const SearchShape &sh, const Work &w,
                        hipStream_t s);
hipError_t launch_exh_scan(const DevIndex &ix, const int8_t *queries, const uint64_t *masks,
                           const SearchShape &sh, const Work &w, hipStream_t s);
hipError_t launch_pool_merge(const DevIndex &ix, const float *query_scales, const SearchShape &sh, const Work &w,
                             int64_t *out_ids, int32_t *out_scores, float *out_fscores, int32_t *out_counts,
                             hipStream_t s);
// resident workgroups per compute unit for this shape (0 if unknown)
int scan_blocks_per_cu(int32_t dim, int32_t sig_words);
int tscan_blocks_per_cu(int32_t dim, int32_t sig_words);
int xscan_blocks_per_cu(int32_t dim, int32_t sig_words);
// one update of an updatable index: the slot it writes, the item's id, its cluster, the kind
struct UpdOp {
  int32_t pos, id, cluster, kind;   // kind: kUpdInsert, kUpdDelete, kUpdResign
};
constexpr int32_t kUpdInsert = 0, kUpdDelete = 1, kUpdResign = 2;
// applies n updates (rows[i] / sigs[i]: the payload of update i, where its kind has one)
hipError_t launch_updates(int8_t *items, uint64_t *sigs, int32_t *perm, int32_t *live, int32_t *slot_of,
                          const UpdOp *ops, int32_t n, const int8_t *rows, const uint64_t *new_sigs, int32_t dim,
                          int32_t sig_words, hipStream_t s);
// searches with k > SVT_MAX_K (svt_largek.hip), after the coarse stage; max_stream bounds any query's
// stream (the nprobe largest clusters' slots)
hipError_t launch_large_k(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const float *query_scales,
                          const SearchShape &sh, int64_t max_stream, const Work &w, int64_t *out_ids,
                          int32_t *out_scores, float *out_fscores, int32_t *out_counts, hipStream_t s);
// rerank (svt_rerank.hip): one workgroup per query
hipError_t launch_rerank(const DevIndex &ix, int32_t B, const int8_t *queries, const float *query_scales,
                         int32_t n_cand, const int64_t *cand_ids, const svt_rerank_net &net, int32_t k_out,
                         int64_t *out_ids, float *out_scores, int32_t *out_counts, hipStream_t s);
hipError_t launch_scatter_rows(const int8_t *src_rows, const uint64_t *src_sigs, const int32_t *pos_of,
                               int64_t i0, int64_t n, int32_t dim, int32_t sig_words, int8_t *dst_rows,
                               uint64_t *dst_sigs, hipStream_t s);

// host side of the search entry points (svt_api.cpp)
// sets the thread's last-error message; returns code
int report(int code, const char *fmt, ...);
// validates the arguments of a search; on SVT_OK, its workspace bytes and the device the index lives on
int search_size(const svt_index *ix, int32_t B, int32_t nprobe, int32_t k, const svt_search_options *opts,
                const char *who, size_t *bytes, int *device);
// validates a search and enqueues it on hip_stream with the given workspace; record_events == false: no
// stage-timing events even when timing is on (the event pool would have to grow)
int search_into(const svt_index *ix, int32_t B, const int8_t *queries, const uint64_t *masks,
                const float *query_scales, int32_t nprobe, int32_t k, int64_t *out_ids, int32_t *out_scores,
                float *out_fscores, int32_t *out_counts, int64_t *out_stats, const svt_search_options *opts,
                void *workspace, size_t workspace_bytes, void *hip_stream, bool record_events, const char *who);

}  // namespace svt
