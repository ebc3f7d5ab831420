// svt_api.cpp - host side of the C ABI declared in include/svt.h: argument validation, the
// cluster-contiguous HBM layout built at upload, per-search workspace carving and kernel launches,
// the Bloom signature helpers and stage timing.  Device work is enqueued on the caller's stream.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <set>
#include <string>
#include <thread>
#include <vector>

#include "svt.h"
#include "svt_internal.h"

using namespace svt;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int fail_hip(hipError_t e, const char *what) {
  return fail(e == hipErrorOutOfMemory ? SVT_ENOMEM : SVT_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr uint32_t kMagic = 0x53565449u;   // "SVTI"

std::mutex g_live_mu;
std::set<const void *> g_live;

bool is_live(const void *p) {
  std::lock_guard<std::mutex> lk(g_live_mu);
  return g_live.count(p) != 0;
}

bool supported_dim(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// stage timing: per-process switch (0 off, 1 every stage, 2 the scan stage only); per-thread record of
// the searches since the last read
std::atomic<int> g_prof_on{0};
constexpr int kStages = 6;
// "plan" and "fallback" are empty when a search runs query by query
const char *const kStageNames[kStages] = {"coarse", "select", "plan", "scan", "fallback", "merge"};
struct ProfState {
  std::vector<hipEvent_t> pool;   // kStages + 1 events per recorded search
  std::vector<int> mode;          // the switch's value when each search was recorded
  int searches = 0;
  ~ProfState() {
    for (auto e : pool) (void)hipEventDestroy(e);
  }
};
thread_local ProfState g_prof;
constexpr int kMaxProfiledSearches = 100000;

}  // namespace

struct svt_index {
  uint32_t magic;
  int device;
  DevIndex dev;
  int8_t *d_items = nullptr;
  uint64_t *d_sigs = nullptr;
  int32_t *d_perm = nullptr;
  int32_t *d_offsets = nullptr;
  int8_t *d_centroids = nullptr;
  int32_t scan_wgs;                 // persistent workgroups of the fused kernel
  int32_t gscan_wgs;                // persistent workgroups of the grouped scan
  int64_t n_tiles;                  // sum over clusters of ceil(size / kGTile)
  int64_t max_cluster_tiles;        // tiles of the largest cluster
};

// ------------------------------------------------------------------------------------------------
extern "C" const char *svt_last_error(void) { return g_err.c_str(); }

static void free_index_memory(svt_index *ix) {
  if (ix->d_items) (void)hipFree(ix->d_items);
  if (ix->d_sigs) (void)hipFree(ix->d_sigs);
  if (ix->d_perm) (void)hipFree(ix->d_perm);
  if (ix->d_offsets) (void)hipFree(ix->d_offsets);
  if (ix->d_centroids) (void)hipFree(ix->d_centroids);
}

extern "C" int svt_index_upload(const svt_index_desc *d, void *hip_stream, svt_index **out) {
  g_err.clear();
  if (!d || !out) return fail(SVT_EINVAL, "svt_index_upload: NULL desc or out");
  *out = nullptr;
  if (d->n_items < 0 || d->n_items >= (int64_t(1) << 31))
    return fail(SVT_EINVAL, "svt_index_upload: n_items %lld out of [0, 2^31)", (long long)d->n_items);
  if (!supported_dim(d->dim)) return fail(SVT_EUNSUPPORTED, "svt_index_upload: dim %d not in {16,32,64,128,256}", d->dim);
  if (d->sig_words != 1 && d->sig_words != 2)
    return fail(SVT_EUNSUPPORTED, "svt_index_upload: sig_words %d not in {1,2}", d->sig_words);
  if (d->nlist < 1 || d->nlist > 65536) return fail(SVT_EINVAL, "svt_index_upload: nlist %d out of [1, 65536]", d->nlist);
  if (!(d->item_scale > 0.f)) return fail(SVT_EINVAL, "svt_index_upload: item_scale must be > 0");
  if (!d->centroids) return fail(SVT_EINVAL, "svt_index_upload: NULL centroids");
  if (d->n_items > 0 && (!d->items || !d->sigs || !d->list_of))
    return fail(SVT_EINVAL, "svt_index_upload: NULL items, sigs or list_of");
  const int64_t n = d->n_items;
  const int32_t dim = d->dim, W = d->sig_words, nlist = d->nlist;
  hipStream_t s = (hipStream_t)hip_stream;

  // host: cluster sizes, offsets, stable cluster-contiguous order
  std::vector<int32_t> offsets(nlist + 1, 0);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t c = d->list_of[i];
    if (c < 0 || c >= nlist) return fail(SVT_EINVAL, "svt_index_upload: list_of[%lld] = %d out of range", (long long)i, c);
    ++offsets[c + 1];
  }
  for (int32_t c = 0; c < nlist; ++c) offsets[c + 1] += offsets[c];
  std::vector<int32_t> perm((size_t)n), pos_of((size_t)n);
  {
    std::vector<int32_t> cur(offsets.begin(), offsets.end() - 1);
    for (int64_t i = 0; i < n; ++i) {
      const int32_t p = cur[d->list_of[i]]++;
      perm[(size_t)p] = (int32_t)i;
      pos_of[(size_t)i] = p;
    }
  }

  svt_index *ix = new (std::nothrow) svt_index();
  if (!ix) return fail(SVT_ENOMEM, "svt_index_upload: host allocation");
  ix->magic = kMagic;
  ix->n_tiles = 0;
  ix->max_cluster_tiles = 0;
  for (int32_t c = 0; c < nlist; ++c) {
    const int64_t t = (offsets[c + 1] - offsets[c] + kGTile - 1) / kGTile;
    ix->n_tiles += t;
    ix->max_cluster_tiles = std::max(ix->max_cluster_tiles, t);
  }
  hipError_t e = hipGetDevice(&ix->device);
  if (e != hipSuccess) { delete ix; return fail_hip(e, "hipGetDevice"); }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, ix->device);
  if (e != hipSuccess) { delete ix; return fail_hip(e, "hipGetDeviceProperties"); }
  {
    // one resident wave of persistent scan workgroups
    const int per_cu = std::max(1, scan_blocks_per_cu(dim, W));
    ix->scan_wgs = std::min(kMaxScanWGs, std::max(64, prop.multiProcessorCount * per_cu));
    const int g_per_cu = std::max(1, gscan_blocks_per_cu(dim, W));
    ix->gscan_wgs = std::min(kMaxScanWGs, std::max(64, prop.multiProcessorCount * g_per_cu));
  }

  int32_t *d_pos_of = nullptr;
  int8_t *stage_rows = nullptr;
  uint64_t *stage_sigs = nullptr;
  auto cleanup_fail = [&](hipError_t err, const char *what) {
    if (d_pos_of) (void)hipFree(d_pos_of);
    if (stage_rows) (void)hipFree(stage_rows);
    if (stage_sigs) (void)hipFree(stage_sigs);
    free_index_memory(ix);
    delete ix;
    return fail_hip(err, what);
  };
  const size_t nb = (size_t)std::max<int64_t>(n, 1);
  if ((e = hipMalloc(&ix->d_items, nb * dim)) != hipSuccess) return cleanup_fail(e, "hipMalloc(items)");
  if ((e = hipMalloc(&ix->d_sigs, nb * W * sizeof(uint64_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(sigs)");
  if ((e = hipMalloc(&ix->d_perm, nb * sizeof(int32_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(perm)");
  if ((e = hipMalloc(&ix->d_offsets, (nlist + 1) * sizeof(int32_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(offsets)");
  if ((e = hipMalloc(&ix->d_centroids, (size_t)nlist * dim)) != hipSuccess) return cleanup_fail(e, "hipMalloc(centroids)");
  if ((e = hipMemcpyAsync(ix->d_offsets, offsets.data(), (nlist + 1) * sizeof(int32_t), hipMemcpyHostToDevice, s)) != hipSuccess)
    return cleanup_fail(e, "copy offsets");
  if ((e = hipMemcpyAsync(ix->d_centroids, d->centroids, (size_t)nlist * dim, hipMemcpyHostToDevice, s)) != hipSuccess)
    return cleanup_fail(e, "copy centroids");
  if (n > 0) {
    if ((e = hipMemcpyAsync(ix->d_perm, perm.data(), (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice, s)) != hipSuccess)
      return cleanup_fail(e, "copy perm");
    // rows and signatures: staged in bounded chunks, scattered on the device to their positions
    if ((e = hipMalloc(&d_pos_of, (size_t)n * sizeof(int32_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(pos_of)");
    if ((e = hipMemcpyAsync(d_pos_of, pos_of.data(), (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice, s)) != hipSuccess)
      return cleanup_fail(e, "copy pos_of");
    const int64_t chunk = std::min<int64_t>(n, std::max<int64_t>(1, (int64_t(256) << 20) / dim));
    if ((e = hipMalloc(&stage_rows, (size_t)chunk * dim)) != hipSuccess) return cleanup_fail(e, "hipMalloc(stage)");
    if ((e = hipMalloc(&stage_sigs, (size_t)chunk * W * sizeof(uint64_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(stage)");
    for (int64_t i0 = 0; i0 < n; i0 += chunk) {
      const int64_t m = std::min(chunk, n - i0);
      if ((e = hipMemcpyAsync(stage_rows, d->items + (size_t)i0 * dim, (size_t)m * dim, hipMemcpyHostToDevice, s)) != hipSuccess)
        return cleanup_fail(e, "copy rows");
      if ((e = hipMemcpyAsync(stage_sigs, d->sigs + (size_t)i0 * W, (size_t)m * W * sizeof(uint64_t), hipMemcpyHostToDevice, s)) != hipSuccess)
        return cleanup_fail(e, "copy sigs");
      if ((e = launch_scatter_rows(stage_rows, stage_sigs, d_pos_of, i0, m, dim, W, ix->d_items, ix->d_sigs, s)) != hipSuccess)
        return cleanup_fail(e, "scatter rows");
      // the staging buffers are reused by the next chunk
      if ((e = hipStreamSynchronize(s)) != hipSuccess) return cleanup_fail(e, "upload sync");
    }
  }
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return cleanup_fail(e, "upload sync");
  if (d_pos_of) (void)hipFree(d_pos_of);
  if (stage_rows) (void)hipFree(stage_rows);
  if (stage_sigs) (void)hipFree(stage_sigs);

  ix->dev.items = ix->d_items;
  ix->dev.sigs = ix->d_sigs;
  ix->dev.perm = ix->d_perm;
  ix->dev.offsets = ix->d_offsets;
  ix->dev.centroids = ix->d_centroids;
  ix->dev.n_items = n;
  ix->dev.dim = dim;
  ix->dev.sig_words = W;
  ix->dev.nlist = nlist;
  ix->dev.item_scale = d->item_scale;
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.insert(ix);
  }
  *out = ix;
  return SVT_OK;
}

extern "C" int svt_index_free(svt_index *ix) {
  g_err.clear();
  if (!ix) return SVT_OK;
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    if (!g_live.count(ix) || ix->magic != kMagic) return fail(SVT_ESTATE, "svt_index_free: not a live index");
    g_live.erase(ix);
  }
  (void)hipDeviceSynchronize();
  free_index_memory(ix);
  ix->magic = 0;
  delete ix;
  return SVT_OK;
}

extern "C" int svt_index_info(const svt_index *ix, int64_t *n_items, int32_t *dim, int32_t *sig_words, int32_t *nlist) {
  g_err.clear();
  if (!ix || !is_live(ix)) return fail(SVT_ESTATE, "svt_index_info: not a live index");
  if (n_items) *n_items = ix->dev.n_items;
  if (dim) *dim = ix->dev.dim;
  if (sig_words) *sig_words = ix->dev.sig_words;
  if (nlist) *nlist = ix->dev.nlist;
  return SVT_OK;
}

// ------------------------------------------------------------------------------------------------
// workspace layout

namespace {

struct Layout {
  size_t coarse_scores, probes, seg, pb, qlen, qcost, qtail, cstart, chunks, order, cband, thr, hlo, hshift, ghist, counter, slot_cnt,
      slot_min, slot_keys, mbound, mcnt, mkeys, stats;
  size_t gcnt, gfill, gstart, ustart, gq, units, pool_cnt, pool;   // grouped path (0 bytes when impossible)
  size_t total;
  int32_t max_chunks;
  int32_t max_units;    // 0: the grouped path does not fit this shape
  int32_t pool_cap;
};

// Grouped searches: candidate pools take at most kPoolBudget bytes in all, at least 16 k and at most
// kPoolMaxKeys keys per query.  Shapes whose work list would not fit an int32 run query by query.
constexpr size_t kPoolBudget = size_t(1) << 30;
constexpr int64_t kPoolMaxKeys = int64_t(1) << 22;
// The grouped path is selected explicitly (SVT_PATH=grouped); by default every batch runs query by
// query, which is faster on every workload measured so far (it keeps an exact top-k per workgroup in LDS,
// the grouped path sends every candidate above the query's bound to HBM).
constexpr int32_t kGroupedMinBatch = 1 << 30;

Layout layout(const svt_index *ix, int32_t B, int32_t nprobe, int32_t k) {
  Layout L{};
  const size_t nlist = (size_t)ix->dev.nlist;
  L.max_chunks = max_chunks_for(B, ix->scan_wgs);
  const size_t C = (size_t)L.max_chunks;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  L.coarse_scores = take((size_t)B * nlist * sizeof(int32_t));
  L.probes = take((size_t)B * nprobe * sizeof(int32_t));
  L.seg = take((size_t)B * (nprobe + 1) * sizeof(int32_t));
  L.pb = take((size_t)B * nprobe * sizeof(int32_t));
  L.qlen = take((size_t)B * sizeof(int64_t));
  L.qcost = take((size_t)B * sizeof(int64_t));
  L.qtail = take((size_t)B * 2 * sizeof(int32_t));
  L.cstart = take((size_t)(B + 1) * sizeof(int32_t));
  L.chunks = take(C * sizeof(Chunk));
  L.order = take(C * sizeof(int32_t));
  L.cband = take(C * sizeof(int32_t));
  L.thr = take((size_t)B * sizeof(int32_t));
  L.hlo = take((size_t)B * sizeof(int32_t));
  L.hshift = take((size_t)B * sizeof(int32_t));
  L.ghist = take((size_t)B * kQHistBins * sizeof(uint32_t));
  L.counter = take(3 * sizeof(uint32_t));
  L.slot_cnt = take(C * sizeof(int32_t));
  L.slot_min = take(C * sizeof(uint64_t));
  L.slot_keys = take(C * (size_t)k * sizeof(uint64_t));
  L.mbound = take((size_t)B * sizeof(uint64_t));
  L.mcnt = take((size_t)B * sizeof(uint32_t));
  L.mkeys = take((size_t)B * kGatherCap * sizeof(uint64_t));
  L.stats = take((size_t)B * 2 * sizeof(int64_t));
  // grouped path: units <= sum_c tiles_c * ceil(queries_c / kGMax), bounded two ways
  const int64_t gpc = ((int64_t)B + kGMax - 1) / kGMax;
  const int64_t u1 = ix->n_tiles * gpc;
  const int64_t u2 = ix->n_tiles + ix->max_cluster_tiles * (((int64_t)B * nprobe + kGMax - 1) / kGMax);
  const int64_t mu = std::max<int64_t>(1, std::min(u1, u2));
  if (mu < (int64_t(1) << 31) - 256) {
    L.max_units = (int32_t)mu;
    const int64_t per_q = (int64_t)(kPoolBudget / 8 / (size_t)std::max(B, 1));
    L.pool_cap = (int32_t)std::min(kPoolMaxKeys, std::max<int64_t>(16 * (int64_t)k, per_q));
    L.gcnt = take(nlist * sizeof(int32_t));
    L.gfill = take(nlist * sizeof(int32_t));
    L.gstart = take((nlist + 1) * sizeof(int32_t));
    L.ustart = take((nlist + 1) * sizeof(int32_t));
    L.gq = take((size_t)B * nprobe * sizeof(int32_t));
    L.units = take((size_t)L.max_units * sizeof(GUnit));
    L.pool_cnt = take((size_t)B * sizeof(uint32_t));
    L.pool = take((size_t)B * (size_t)L.pool_cap * sizeof(uint64_t));
  }
  L.total = o;
  return L;
}

// SVT_OK or the error code (message set)
int check_search_args(const svt_index *ix, int32_t B, int32_t nprobe, int32_t k, const char *who) {
  if (!ix || !is_live(ix) || ix->magic != kMagic) return fail(SVT_ESTATE, "%s: not a live index", who);
  if (B < 0 || B > 65535) return fail(SVT_EINVAL, "%s: n_queries %d out of [0, 65535]", who, B);
  if (nprobe < 1 || nprobe > ix->dev.nlist) return fail(SVT_EINVAL, "%s: nprobe %d out of [1, %d]", who, nprobe, ix->dev.nlist);
  if (k < 1 || k > SVT_MAX_K) return fail(SVT_EINVAL, "%s: k %d out of [1, %d]", who, k, SVT_MAX_K);
  return SVT_OK;
}

}  // namespace

extern "C" size_t svt_search_workspace_size(const svt_index *ix, int32_t n_queries, int32_t nprobe, int32_t k) {
  g_err.clear();
  if (check_search_args(ix, n_queries, nprobe, k, "svt_search_workspace_size") != SVT_OK) return 0;
  return layout(ix, n_queries, nprobe, k).total;
}

extern "C" int svt_search(const svt_index *ix, int32_t B, const int8_t *queries, const uint64_t *masks,
                          const float *query_scales, int32_t nprobe, int32_t k, int64_t *out_ids, int32_t *out_scores,
                          float *out_fscores, int32_t *out_counts, int64_t *out_stats, void *workspace,
                          size_t workspace_bytes, void *hip_stream) {
  g_err.clear();
  const int rc = check_search_args(ix, B, nprobe, k, "svt_search");
  if (rc != SVT_OK) return rc;
  if (B == 0) return SVT_OK;
  if (!queries || !masks || !out_ids || !out_scores || !workspace)
    return fail(SVT_EINVAL, "svt_search: NULL queries, masks, out_ids, out_scores or workspace");
  if (((uintptr_t)workspace & 255) != 0) return fail(SVT_EINVAL, "svt_search: workspace not 256-byte aligned");
  if (((uintptr_t)queries & 15) != 0) return fail(SVT_EINVAL, "svt_search: queries not 16-byte aligned");
  if (((uintptr_t)masks & 7) != 0) return fail(SVT_EINVAL, "svt_search: masks not 8-byte aligned");
  const Layout L = layout(ix, B, nprobe, k);
  if (workspace_bytes < L.total)
    return fail(SVT_EINVAL, "svt_search: workspace %zu bytes < required %zu", workspace_bytes, L.total);
  hipStream_t s = (hipStream_t)hip_stream;
  char *base = (char *)workspace;
  Work w;
  w.coarse_scores = (int32_t *)(base + L.coarse_scores);
  w.probes = (int32_t *)(base + L.probes);
  w.seg = (int32_t *)(base + L.seg);
  w.pb = (int32_t *)(base + L.pb);
  w.qlen = (int64_t *)(base + L.qlen);
  w.qcost = (int64_t *)(base + L.qcost);
  w.qtail = (int32_t *)(base + L.qtail);
  w.cstart = (int32_t *)(base + L.cstart);
  w.chunks = (Chunk *)(base + L.chunks);
  w.order = (int32_t *)(base + L.order);
  w.cband = (int32_t *)(base + L.cband);
  w.thr = (int32_t *)(base + L.thr);
  w.hlo = (int32_t *)(base + L.hlo);
  w.hshift = (int32_t *)(base + L.hshift);
  w.ghist = (uint32_t *)(base + L.ghist);
  w.counter = (uint32_t *)(base + L.counter);
  w.slot_cnt = (int32_t *)(base + L.slot_cnt);
  w.slot_min = (uint64_t *)(base + L.slot_min);
  w.slot_keys = (uint64_t *)(base + L.slot_keys);
  w.mbound = (uint64_t *)(base + L.mbound);
  w.mcnt = (uint32_t *)(base + L.mcnt);
  w.mkeys = (uint64_t *)(base + L.mkeys);
  w.stats = out_stats ? out_stats : (int64_t *)(base + L.stats);
  // path: SVT_PATH=query|grouped forces one; otherwise batches of kGroupedMinBatch or more queries are
  // grouped
  int grouped = B >= kGroupedMinBatch ? 1 : 0;
  if (const char *pe = getenv("SVT_PATH")) {
    if (!strcmp(pe, "query")) grouped = 0;
    else if (!strcmp(pe, "grouped")) grouped = 1;
  }
  if (L.max_units == 0) grouped = 0;
  int32_t pool_cap = L.pool_cap;
  if (const char *pc = getenv("SVT_POOL_CAP")) {   // smaller pools, to exercise the overflow fallback
    const long v = strtol(pc, nullptr, 10);
    if (v >= 1 && v < pool_cap) pool_cap = (int32_t)v;
  }
  w.gcnt = w.gfill = w.gstart = w.ustart = w.gq = nullptr;
  w.units = nullptr;
  w.pool_cnt = nullptr;
  w.pool = nullptr;
  if (grouped) {
    w.gcnt = (int32_t *)(base + L.gcnt);
    w.gfill = (int32_t *)(base + L.gfill);
    w.gstart = (int32_t *)(base + L.gstart);
    w.ustart = (int32_t *)(base + L.ustart);
    w.gq = (int32_t *)(base + L.gq);
    w.units = (GUnit *)(base + L.units);
    w.pool_cnt = (uint32_t *)(base + L.pool_cnt);
    w.pool = (uint64_t *)(base + L.pool);
  }
  int32_t gather_cap = kGatherCap;
  if (const char *gc = getenv("SVT_GATHER_CAP")) {   // fewer gathered keys, to exercise the merge from the slots
    const long v = strtol(gc, nullptr, 10);
    if (v >= 0 && v < gather_cap) gather_cap = (int32_t)v;
  }
  SearchShape sh{B, nprobe, k, ix->scan_wgs, L.max_chunks, grouped, pool_cap, L.max_units, ix->gscan_wgs, gather_cap};

  const int prof_mode = g_prof_on.load(std::memory_order_relaxed);
  const bool prof = prof_mode != 0 && g_prof.searches < kMaxProfiledSearches;
  ProfState &ps = g_prof;
  int ev0 = 0, evn = 0;
  if (prof) {
    if ((int)ps.mode.size() <= ps.searches) ps.mode.resize(ps.searches + 1);
    ps.mode[ps.searches] = prof_mode;
    ev0 = ps.searches * (kStages + 1);
    while ((int)ps.pool.size() < ev0 + kStages + 1) {
      hipEvent_t ev;
      hipError_t er = hipEventCreate(&ev);
      if (er != hipSuccess) return fail_hip(er, "hipEventCreate");
      ps.pool.push_back(ev);
    }
  }
  // mark i ends stage i - 1; the scan stage lies between marks 3 and 4
  auto mark = [&]() -> hipError_t {
    const int i = evn++;
    if (!prof || (prof_mode == 2 && i != 3 && i != 4)) return hipSuccess;
    return hipEventRecord(ps.pool[ev0 + i], s);
  };
  hipError_t e;
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if ((e = launch_coarse_keys(ix->dev, queries, B, w, s)) != hipSuccess) return fail_hip(e, "launch coarse_keys");
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if ((e = launch_coarse_select(ix->dev, queries, masks, sh, w, s)) != hipSuccess)
    return fail_hip(e, "launch coarse_select");
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if (grouped && (e = launch_group_plan(ix->dev, sh, w, s)) != hipSuccess) return fail_hip(e, "launch group plan");
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if (grouped) {
    if ((e = launch_gscan(ix->dev, queries, masks, sh, w, s)) != hipSuccess) return fail_hip(e, "launch gscan");
    if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
    // queries whose pools overflowed, query by query (every other chunk and query returns at once)
    if ((e = launch_scan(ix->dev, queries, masks, sh, w, s)) != hipSuccess) return fail_hip(e, "launch scan");
    if ((e = launch_merge(ix->dev, query_scales, sh, w, out_ids, out_scores, out_fscores, out_counts, s)) !=
        hipSuccess)
      return fail_hip(e, "launch merge");
    if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
    if ((e = launch_pool_merge(ix->dev, query_scales, sh, w, out_ids, out_scores, out_fscores, out_counts, s)) !=
        hipSuccess)
      return fail_hip(e, "launch pool merge");
  } else {
    if ((e = launch_scan(ix->dev, queries, masks, sh, w, s)) != hipSuccess) return fail_hip(e, "launch scan");
    if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
    if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
    if ((e = launch_merge(ix->dev, query_scales, sh, w, out_ids, out_scores, out_fscores, out_counts, s)) !=
        hipSuccess)
      return fail_hip(e, "launch merge");
  }
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if (prof) ++ps.searches;
  return SVT_OK;
}

extern "C" int svt_profile_enable(int on) {
  g_err.clear();
  if (on < 0 || on > 2) return fail(SVT_EINVAL, "svt_profile_enable: mode %d out of [0, 2]", on);
  g_prof_on.store(on);
  return SVT_OK;
}

extern "C" int svt_profile_read(float *stage_ms, const char **stage_names, int32_t max_stages, int32_t *n_stages,
                                int32_t *n_searches) {
  g_err.clear();
  ProfState &ps = g_prof;
  const int ns = ps.searches;
  if (n_stages) *n_stages = kStages;
  if (n_searches) *n_searches = ns;
  double tot[kStages] = {0, 0, 0, 0, 0, 0};
  if (ns > 0) {
    hipError_t e = hipEventSynchronize(ps.pool[ns * (kStages + 1) - 1]);
    if (e != hipSuccess) return fail_hip(e, "hipEventSynchronize");
    for (int r = 0; r < ns; ++r)
      for (int i = 0; i < kStages; ++i) {
        if (ps.mode[r] == 2 && i != 3) continue;   // scan-only record
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, ps.pool[r * (kStages + 1) + i], ps.pool[r * (kStages + 1) + i + 1]);
        if (e != hipSuccess) return fail_hip(e, "hipEventElapsedTime");
        tot[i] += ms;
      }
  }
  for (int i = 0; i < kStages && i < max_stages; ++i) {
    if (stage_ms) stage_ms[i] = (float)tot[i];
    if (stage_names) stage_names[i] = kStageNames[i];
  }
  ps.searches = 0;
  return SVT_OK;
}

// ------------------------------------------------------------------------------------------------
// Bloom signature helpers (host).  splitmix64 (Steele, Lea, Flood, OOPSLA 2014) seeded with the token
// key; output j selects bit out_j >> (64 - log2(64 * sig_words)).

namespace {

inline uint64_t sm64_next(uint64_t &st) {
  uint64_t z = (st += 0x9E3779B97F4A7C15ULL);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

inline void token_bits(uint64_t key, int h, int W, uint64_t *sig) {
  const int shift = 64 - (W == 1 ? 6 : 7);
  uint64_t st = key;
  for (int j = 0; j < h; ++j) {
    const uint64_t b = sm64_next(st) >> shift;
    sig[b >> 6] |= 1ULL << (b & 63);
  }
}

}  // namespace

extern "C" int svt_bloom_mask(const uint64_t *token_keys, int32_t n_tokens, int32_t n_hashes, int32_t sig_words,
                              uint64_t *out) {
  g_err.clear();
  if (!out || n_tokens < 0 || (n_tokens > 0 && !token_keys) || n_hashes < 1 || n_hashes > 16)
    return fail(SVT_EINVAL, "svt_bloom_mask: invalid arguments");
  if (sig_words != 1 && sig_words != 2) return fail(SVT_EUNSUPPORTED, "svt_bloom_mask: sig_words %d", sig_words);
  uint64_t m[2] = {0, 0};
  for (int32_t t = 0; t < n_tokens; ++t) token_bits(token_keys[t], n_hashes, sig_words, m);
  for (int32_t w = 0; w < sig_words; ++w) out[w] = m[w];
  return SVT_OK;
}

extern "C" int svt_bloom_sign(const uint64_t *token_keys, int64_t n_items, int32_t tokens_per_item, int32_t n_hashes,
                              int32_t sig_words, uint64_t *out, int32_t n_threads) {
  g_err.clear();
  if (n_items < 0 || tokens_per_item < 0 || (n_items > 0 && (!out || (tokens_per_item > 0 && !token_keys))) ||
      n_hashes < 1 || n_hashes > 16)
    return fail(SVT_EINVAL, "svt_bloom_sign: invalid arguments");
  if (sig_words != 1 && sig_words != 2) return fail(SVT_EUNSUPPORTED, "svt_bloom_sign: sig_words %d", sig_words);
  int nt = n_threads > 0 ? n_threads : (int)std::max(1u, std::thread::hardware_concurrency());
  nt = (int)std::min<int64_t>(nt, std::max<int64_t>(1, n_items / 4096));
  auto work = [&](int64_t i0, int64_t i1) {
    for (int64_t i = i0; i < i1; ++i) {
      uint64_t m[2] = {0, 0};
      for (int32_t t = 0; t < tokens_per_item; ++t)
        token_bits(token_keys[i * tokens_per_item + t], n_hashes, sig_words, m);
      for (int32_t w = 0; w < sig_words; ++w) out[i * sig_words + w] = m[w];
    }
  };
  if (nt <= 1) {
    work(0, n_items);
    return SVT_OK;
  }
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t) th.emplace_back(work, n_items * t / nt, n_items * (t + 1) / nt);
  for (auto &x : th) x.join();
  return SVT_OK;
}
