// svt_internal.h - declarations shared by the host API (svt_api.cpp) and the gfx950 kernels
// (svt_kernels.hip).  Not installed; the public boundary is include/svt.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svt {

constexpr int kMaxK = 2048;          // largest top-k (SVT_MAX_K)
constexpr int kScanThreads = 256;    // fused filter-score-select workgroup: 4 wave64
constexpr int kScanGroups = 4;       // 64-item groups per wave per step
constexpr int kScanStep = kScanThreads * kScanGroups;   // items per workgroup step (1024)
constexpr int kListCap = kMaxK + kScanStep;             // LDS candidate list capacity (keys)
constexpr int kSelThreads = 1024;    // coarse-select and merge workgroups
constexpr int kCoarseQB = 8;         // queries per coarse-score workgroup
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

// Per-search device workspace (carved by the host from the caller's buffer).
struct Work {
  uint64_t *coarse_keys;    // [B][nlist]   coarse (score, cluster) keys
  int32_t *probes;          // [B][nprobe]  probed clusters, ascending cluster id
  int32_t *seg;             // [B][nprobe + 1] stream offset of each probed cluster within its query
  int64_t *qlen;            // [B]          items scanned per query
  int64_t *qstart;          // [B + 1]      exclusive prefix of qlen (the batch stream)
  int32_t *thr;             // [B]          per-query proven lower bound on the k-th best score
  uint32_t *counter;        // [1]          completion counter of the select kernel
  int32_t *slot_cnt;        // [P + B]      candidates held by each (workgroup, query) run
  uint64_t *slot_keys;      // [P + B][k]   those candidates (score/id keys)
  int64_t *stats;           // [B][2] scanned / eligible (caller buffer or workspace)
};

struct SearchShape {
  int32_t B, nprobe, k, P;
};

// launch wrappers (svt_kernels.hip); each returns hipSuccess or the launch error
hipError_t launch_coarse_keys(const DevIndex &ix, const int8_t *queries, int32_t B, const Work &w,
                              hipStream_t s);
hipError_t launch_coarse_select(const DevIndex &ix, const SearchShape &sh, const Work &w, hipStream_t s);
hipError_t launch_scan(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const SearchShape &sh,
                       const Work &w, hipStream_t s);
hipError_t launch_merge(const DevIndex &ix, const float *query_scales, const SearchShape &sh, const Work &w,
                        int64_t *out_ids, int32_t *out_scores, float *out_fscores, int32_t *out_counts,
                        hipStream_t s);
hipError_t launch_scatter_rows(const int8_t *src_rows, const uint64_t *src_sigs, const int32_t *pos_of,
                               int64_t i0, int64_t n, int32_t dim, int32_t sig_words, int8_t *dst_rows,
                               uint64_t *dst_sigs, hipStream_t s);

}  // namespace svt
