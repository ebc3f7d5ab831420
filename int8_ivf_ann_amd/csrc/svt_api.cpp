// svt_api.cpp - host side of the C ABI declared in include/svt.h: argument validation, the
// cluster-contiguous HBM layout built at upload, per-search workspace carving and kernel launches,
// the Bloom signature helpers and stage timing.  Device work is enqueued on the caller's stream.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
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

int vfail(int code, const char *fmt, va_list ap) {
  char buf[512];
  vsnprintf(buf, sizeof buf, fmt, ap);
  g_err = buf;
  return code;
}

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int r = vfail(code, fmt, ap);
  va_end(ap);
  return r;
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
  int32_t *d_live = nullptr;
  int32_t *d_slot_of = nullptr;                // [max(n_items, id_capacity)] slot of each id (-1: absent)
  int8_t *d_centroids = nullptr;
  int64_t n_live = 0;                          // items (not free slots)
  // updatable index: the host's record of the layout, which chooses every update's slot
  bool updatable = false;
  int64_t id_capacity = 0;
  std::vector<int32_t> slot_of;                // [id_capacity] slot of each id (-1: not in the index)
  std::vector<int32_t> offsets_h;              // [nlist + 1] cluster slot ranges
  std::vector<std::vector<int32_t>> free_h;    // free slots of each cluster (a stack, lowest slot on top)
  void *d_stage = nullptr;                     // device staging of an update batch
  size_t stage_bytes = 0;
  std::vector<int64_t> top_slots;               // [nlist + 1] slots of the j largest clusters (a query's stream bound)
  int32_t scan_wgs;                 // persistent workgroups of the query-by-query scan
  int32_t tscan_wgs;                // persistent workgroups of the tile scan
  int32_t xscan_wgs;                // workgroups of the exhaustive MFMA scan
};

// ------------------------------------------------------------------------------------------------
extern "C" const char *svt_last_error(void) { return g_err.c_str(); }

static void free_index_memory(svt_index *ix) {
  if (ix->d_items) (void)hipFree(ix->d_items);
  if (ix->d_sigs) (void)hipFree(ix->d_sigs);
  if (ix->d_perm) (void)hipFree(ix->d_perm);
  if (ix->d_offsets) (void)hipFree(ix->d_offsets);
  if (ix->d_live) (void)hipFree(ix->d_live);
  if (ix->d_slot_of) (void)hipFree(ix->d_slot_of);
  if (ix->d_centroids) (void)hipFree(ix->d_centroids);
  if (ix->d_stage) (void)hipFree(ix->d_stage);
}

namespace {

bool sig_reserved(const uint64_t *sig, int32_t W) {
  uint64_t a = ~0ull;
  for (int32_t u = 0; u < W; ++u) a &= sig[u];
  return a == ~0ull;
}

// Upload; with updatable, each cluster gets max(slack_min, ceil(slack_frac * size)) free slots after its
// items and the host keeps the layout record that places later updates.
int upload(const svt_index_desc *d, bool updatable, int64_t id_capacity, int32_t slack_min, float slack_frac,
           void *hip_stream, svt_index **out, const char *who) {
  if (!d || !out) return fail(SVT_EINVAL, "%s: NULL desc or out", who);
  *out = nullptr;
  if (d->n_items < 0 || d->n_items >= (int64_t(1) << 31))
    return fail(SVT_EINVAL, "%s: n_items %lld out of [0, 2^31)", who, (long long)d->n_items);
  if (!supported_dim(d->dim)) return fail(SVT_EUNSUPPORTED, "%s: dim %d not in {16,32,64,128,256}", who, d->dim);
  if (d->sig_words != 1 && d->sig_words != 2)
    return fail(SVT_EUNSUPPORTED, "%s: sig_words %d not in {1,2}", who, d->sig_words);
  if (d->nlist < 1 || d->nlist > 65536) return fail(SVT_EINVAL, "%s: nlist %d out of [1, 65536]", who, d->nlist);
  if (!(d->item_scale > 0.f)) return fail(SVT_EINVAL, "%s: item_scale must be > 0", who);
  if (!d->centroids) return fail(SVT_EINVAL, "%s: NULL centroids", who);
  if (d->n_items > 0 && (!d->items || !d->sigs || !d->list_of))
    return fail(SVT_EINVAL, "%s: NULL items, sigs or list_of", who);
  const int64_t n = d->n_items;
  const int32_t dim = d->dim, W = d->sig_words, nlist = d->nlist;
  hipStream_t s = (hipStream_t)hip_stream;

  if (updatable) {
    if (id_capacity < n || id_capacity > INT32_MAX)
      return fail(SVT_EINVAL, "%s: id_capacity %lld out of [n_items, 2^31)", who, (long long)id_capacity);
    if (slack_min < 0 || !(slack_frac >= 0.f) || slack_frac > 64.f)
      return fail(SVT_EINVAL, "%s: slack_min %d < 0 or slack_frac %g out of [0, 64]", who, slack_min, (double)slack_frac);
  }

  // host: cluster sizes, slot ranges (items, then free slots), stable cluster-contiguous order
  std::vector<int64_t> size(nlist, 0);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t c = d->list_of[i];
    if (c < 0 || c >= nlist) return fail(SVT_EINVAL, "%s: list_of[%lld] = %d out of range", who, (long long)i, c);
    ++size[c];
    if (sig_reserved(d->sigs + (size_t)i * W, W))
      return fail(SVT_EINVAL, "%s: item %lld has every signature bit set (reserved for free slots)", who, (long long)i);
  }
  std::vector<int32_t> offsets(nlist + 1, 0);
  {
    int64_t at = 0;
    for (int32_t c = 0; c < nlist; ++c) {
      offsets[c] = (int32_t)at;
      const int64_t slack = updatable ? std::max<int64_t>(slack_min, (int64_t)std::ceil((double)slack_frac * size[c])) : 0;
      at += size[c] + slack;
      if (at >= (int64_t(1) << 31)) return fail(SVT_EINVAL, "%s: more than 2^31 slots", who);
    }
    offsets[nlist] = (int32_t)at;
  }
  const int64_t n_slots = offsets[nlist];
  std::vector<int32_t> perm((size_t)n_slots, -1), pos_of((size_t)n), live((size_t)nlist);
  {
    std::vector<int32_t> cur(offsets.begin(), offsets.end() - 1);
    for (int64_t i = 0; i < n; ++i) {
      const int32_t p = cur[d->list_of[i]]++;
      perm[(size_t)p] = (int32_t)i;
      pos_of[(size_t)i] = p;
    }
    for (int32_t c = 0; c < nlist; ++c) live[(size_t)c] = (int32_t)size[c];
  }

  svt_index *ix = new (std::nothrow) svt_index();
  if (!ix) return fail(SVT_ENOMEM, "%s: host allocation", who);
  ix->magic = kMagic;
  hipError_t e = hipGetDevice(&ix->device);
  if (e != hipSuccess) { delete ix; return fail_hip(e, "hipGetDevice"); }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, ix->device);
  if (e != hipSuccess) { delete ix; return fail_hip(e, "hipGetDeviceProperties"); }
  {
    // one resident wave of persistent scan workgroups
    const int per_cu = std::max(1, scan_blocks_per_cu(dim, W));
    ix->scan_wgs = std::min(kMaxScanWGs, std::max(64, prop.multiProcessorCount * per_cu));
    const int t_per_cu = std::max(1, tscan_blocks_per_cu(dim, W));
    ix->tscan_wgs = std::min(kMaxScanWGs, std::max(64, prop.multiProcessorCount * t_per_cu));
    const int x_per_cu = std::max(1, xscan_blocks_per_cu(dim, W));
    ix->xscan_wgs = std::min(kMaxScanWGs, std::max(64, prop.multiProcessorCount * x_per_cu));
  }

  int8_t *stage_rows = nullptr;
  uint64_t *stage_sigs = nullptr;
  auto cleanup_fail = [&](hipError_t err, const char *what) {
    if (stage_rows) (void)hipFree(stage_rows);
    if (stage_sigs) (void)hipFree(stage_sigs);
    free_index_memory(ix);
    delete ix;
    return fail_hip(err, what);
  };
  const size_t nb = (size_t)std::max<int64_t>(n_slots, 1);
  if ((e = hipMalloc(&ix->d_items, nb * dim)) != hipSuccess) return cleanup_fail(e, "hipMalloc(items)");
  if ((e = hipMalloc(&ix->d_sigs, nb * W * sizeof(uint64_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(sigs)");
  if ((e = hipMalloc(&ix->d_perm, nb * sizeof(int32_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(perm)");
  if ((e = hipMalloc(&ix->d_offsets, (nlist + 1) * sizeof(int32_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(offsets)");
  if ((e = hipMalloc(&ix->d_live, (size_t)nlist * sizeof(int32_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(live)");
  if ((e = hipMalloc(&ix->d_centroids, (size_t)nlist * dim)) != hipSuccess) return cleanup_fail(e, "hipMalloc(centroids)");
  if ((e = hipMemcpyAsync(ix->d_offsets, offsets.data(), (nlist + 1) * sizeof(int32_t), hipMemcpyHostToDevice, s)) != hipSuccess)
    return cleanup_fail(e, "copy offsets");
  if ((e = hipMemcpyAsync(ix->d_live, live.data(), (size_t)nlist * sizeof(int32_t), hipMemcpyHostToDevice, s)) != hipSuccess)
    return cleanup_fail(e, "copy live counts");
  if ((e = hipMemcpyAsync(ix->d_centroids, d->centroids, (size_t)nlist * dim, hipMemcpyHostToDevice, s)) != hipSuccess)
    return cleanup_fail(e, "copy centroids");
  if (n_slots > n) {
    // free slots: the reserved signature, zero rows (the items' slots are overwritten below)
    if ((e = hipMemsetAsync(ix->d_sigs, 0xFF, (size_t)n_slots * W * sizeof(uint64_t), s)) != hipSuccess)
      return cleanup_fail(e, "fill free slots");
    if ((e = hipMemsetAsync(ix->d_items, 0, (size_t)n_slots * dim, s)) != hipSuccess) return cleanup_fail(e, "fill free slots");
  }
  if (n_slots > 0 &&
      (e = hipMemcpyAsync(ix->d_perm, perm.data(), (size_t)n_slots * sizeof(int32_t), hipMemcpyHostToDevice, s)) != hipSuccess)
    return cleanup_fail(e, "copy perm");
  // id -> slot: the uploaded ids, then (updatable) the ids not yet used
  const int64_t n_ids = std::max<int64_t>(n, updatable ? id_capacity : 0);
  if ((e = hipMalloc(&ix->d_slot_of, (size_t)std::max<int64_t>(n_ids, 1) * sizeof(int32_t))) != hipSuccess)
    return cleanup_fail(e, "hipMalloc(slot_of)");
  if (n_ids > n &&
      (e = hipMemsetAsync(ix->d_slot_of + n, 0xFF, (size_t)(n_ids - n) * sizeof(int32_t), s)) != hipSuccess)
    return cleanup_fail(e, "fill slot_of");
  if (n > 0 &&
      (e = hipMemcpyAsync(ix->d_slot_of, pos_of.data(), (size_t)n * sizeof(int32_t), hipMemcpyHostToDevice, s)) != hipSuccess)
    return cleanup_fail(e, "copy slot_of");
  if (n > 0) {
    // rows and signatures: staged in bounded chunks, scattered on the device to their slots
    const int64_t chunk = std::min<int64_t>(n, std::max<int64_t>(1, (int64_t(256) << 20) / dim));
    if ((e = hipMalloc(&stage_rows, (size_t)chunk * dim)) != hipSuccess) return cleanup_fail(e, "hipMalloc(stage)");
    if ((e = hipMalloc(&stage_sigs, (size_t)chunk * W * sizeof(uint64_t))) != hipSuccess) return cleanup_fail(e, "hipMalloc(stage)");
    for (int64_t i0 = 0; i0 < n; i0 += chunk) {
      const int64_t m = std::min(chunk, n - i0);
      if ((e = hipMemcpyAsync(stage_rows, d->items + (size_t)i0 * dim, (size_t)m * dim, hipMemcpyHostToDevice, s)) != hipSuccess)
        return cleanup_fail(e, "copy rows");
      if ((e = hipMemcpyAsync(stage_sigs, d->sigs + (size_t)i0 * W, (size_t)m * W * sizeof(uint64_t), hipMemcpyHostToDevice, s)) != hipSuccess)
        return cleanup_fail(e, "copy sigs");
      if ((e = launch_scatter_rows(stage_rows, stage_sigs, ix->d_slot_of, i0, m, dim, W, ix->d_items, ix->d_sigs, s)) != hipSuccess)
        return cleanup_fail(e, "scatter rows");
      // the staging buffers are reused by the next chunk
      if ((e = hipStreamSynchronize(s)) != hipSuccess) return cleanup_fail(e, "upload sync");
    }
  }
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return cleanup_fail(e, "upload sync");
  if (stage_rows) (void)hipFree(stage_rows);
  if (stage_sigs) (void)hipFree(stage_sigs);

  ix->dev.items = ix->d_items;
  ix->dev.sigs = ix->d_sigs;
  ix->dev.perm = ix->d_perm;
  ix->dev.offsets = ix->d_offsets;
  ix->dev.live = ix->d_live;
  ix->dev.slot_of = ix->d_slot_of;
  ix->dev.n_ids = n_ids;
  ix->dev.centroids = ix->d_centroids;
  ix->dev.n_items = n_slots;
  ix->dev.dim = dim;
  ix->dev.sig_words = W;
  ix->dev.nlist = nlist;
  ix->dev.item_scale = d->item_scale;
  ix->n_live = n;
  {
    std::vector<int64_t> sz((size_t)nlist);
    for (int32_t c = 0; c < nlist; ++c) sz[(size_t)c] = (int64_t)offsets[c + 1] - offsets[c];
    std::sort(sz.begin(), sz.end(), std::greater<int64_t>());
    ix->top_slots.assign((size_t)nlist + 1, 0);
    for (int32_t c = 0; c < nlist; ++c) ix->top_slots[(size_t)c + 1] = ix->top_slots[(size_t)c] + sz[(size_t)c];
  }
  if (updatable) {
    ix->updatable = true;
    ix->id_capacity = id_capacity;
    ix->slot_of.assign((size_t)id_capacity, -1);
    for (int64_t i = 0; i < n; ++i) ix->slot_of[(size_t)i] = pos_of[(size_t)i];
    ix->offsets_h = offsets;
    ix->free_h.resize((size_t)nlist);
    for (int32_t c = 0; c < nlist; ++c)
      for (int32_t p = offsets[c + 1] - 1; p >= offsets[c] + (int32_t)size[c]; --p) ix->free_h[(size_t)c].push_back(p);
  }
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    g_live.insert(ix);
  }
  *out = ix;
  return SVT_OK;
}

}  // namespace

extern "C" int svt_index_upload(const svt_index_desc *d, void *hip_stream, svt_index **out) {
  g_err.clear();
  return upload(d, false, 0, 0, 0.f, hip_stream, out, "svt_index_upload");
}

extern "C" int svt_index_upload_updatable(const svt_index_desc *d, int64_t id_capacity, int32_t slack_min,
                                          float slack_frac, void *hip_stream, svt_index **out) {
  g_err.clear();
  return upload(d, true, id_capacity, slack_min, slack_frac, hip_stream, out, "svt_index_upload_updatable");
}

extern "C" int svt_index_free(svt_index *ix, void *hip_stream) {
  g_err.clear();
  if (!ix) return SVT_OK;
  {
    std::lock_guard<std::mutex> lk(g_live_mu);
    if (!g_live.count(ix) || ix->magic != kMagic) return fail(SVT_ESTATE, "svt_index_free: not a live index");
    g_live.erase(ix);
  }
  // the caller's searches on this index ran on hip_stream: they end before the memory is released
  const hipError_t e = hipStreamSynchronize((hipStream_t)hip_stream);
  free_index_memory(ix);
  ix->magic = 0;
  delete ix;
  if (e != hipSuccess) return fail_hip(e, "svt_index_free: hipStreamSynchronize");
  return SVT_OK;
}

extern "C" int svt_index_info(const svt_index *ix, int64_t *n_items, int32_t *dim, int32_t *sig_words, int32_t *nlist) {
  g_err.clear();
  if (!ix || !is_live(ix)) return fail(SVT_ESTATE, "svt_index_info: not a live index");
  if (n_items) *n_items = ix->n_live;
  if (dim) *dim = ix->dev.dim;
  if (sig_words) *sig_words = ix->dev.sig_words;
  if (nlist) *nlist = ix->dev.nlist;
  return SVT_OK;
}

namespace {

// The checks every update batch shares; SVT_OK or the error (message set)
int check_update(svt_index *ix, int32_t n, const int64_t *ids, const char *who) {
  if (!ix || !is_live(ix) || ix->magic != kMagic) return fail(SVT_ESTATE, "%s: not a live index", who);
  if (!ix->updatable) return fail(SVT_ESTATE, "%s: the index was not uploaded as updatable", who);
  if (n < 0) return fail(SVT_EINVAL, "%s: n %d < 0", who, n);
  if (n > 0 && !ids) return fail(SVT_EINVAL, "%s: NULL ids", who);
  return SVT_OK;
}

// ids of one batch: each in [0, id_capacity), no id twice, each present (present) or absent (!present)
int check_ids(svt_index *ix, int32_t n, const int64_t *ids, bool present, const char *who) {
  std::vector<int64_t> sorted(ids, ids + n);
  std::sort(sorted.begin(), sorted.end());
  for (int32_t i = 0; i < n; ++i) {
    const int64_t id = sorted[(size_t)i];
    if (id < 0 || id >= ix->id_capacity)
      return fail(SVT_EINVAL, "%s: id %lld out of [0, %lld)", who, (long long)id, (long long)ix->id_capacity);
    if (i > 0 && sorted[(size_t)i - 1] == id) return fail(SVT_EINVAL, "%s: id %lld twice in one batch", who, (long long)id);
    const bool in = ix->slot_of[(size_t)id] >= 0;
    if (in != present)
      return fail(SVT_EINVAL, "%s: id %lld is %s the index", who, (long long)id, in ? "already in" : "not in");
  }
  return SVT_OK;
}

int32_t cluster_of_slot(const svt_index *ix, int32_t p) {
  return (int32_t)(std::upper_bound(ix->offsets_h.begin(), ix->offsets_h.end(), p) - ix->offsets_h.begin()) - 1;
}

// Stage a batch (ops, then rows, then signatures) on the device, apply it on s and wait for it.
int apply_updates(svt_index *ix, const std::vector<UpdOp> &ops, const int8_t *rows, const uint64_t *sigs,
                  hipStream_t s, const char *who) {
  const int32_t n = (int32_t)ops.size(), dim = ix->dev.dim, W = ix->dev.sig_words;
  const size_t ob = align256((size_t)n * sizeof(UpdOp));
  const size_t rb = rows ? align256((size_t)n * dim) : 0;
  const size_t sb = sigs ? (size_t)n * W * sizeof(uint64_t) : 0;
  const size_t need = ob + rb + sb;
  hipError_t e;
  if (need > ix->stage_bytes) {
    // the previous batch finished before its call returned: the old staging is idle
    if (ix->d_stage) (void)hipFree(ix->d_stage);
    ix->d_stage = nullptr;
    ix->stage_bytes = 0;
    if ((e = hipMalloc(&ix->d_stage, need)) != hipSuccess) return fail_hip(e, who);
    ix->stage_bytes = need;
  }
  char *base = (char *)ix->d_stage;
  if ((e = hipMemcpyAsync(base, ops.data(), (size_t)n * sizeof(UpdOp), hipMemcpyHostToDevice, s)) != hipSuccess)
    return fail_hip(e, who);
  if (rows && (e = hipMemcpyAsync(base + ob, rows, (size_t)n * dim, hipMemcpyHostToDevice, s)) != hipSuccess)
    return fail_hip(e, who);
  if (sigs && (e = hipMemcpyAsync(base + ob + rb, sigs, sb, hipMemcpyHostToDevice, s)) != hipSuccess)
    return fail_hip(e, who);
  if ((e = launch_updates(ix->d_items, ix->d_sigs, ix->d_perm, ix->d_live, ix->d_slot_of, (const UpdOp *)base, n,
                          rows ? (const int8_t *)(base + ob) : nullptr,
                          sigs ? (const uint64_t *)(base + ob + rb) : nullptr, dim, W, s)) != hipSuccess)
    return fail_hip(e, who);
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return fail_hip(e, who);
  return SVT_OK;
}

}  // namespace

extern "C" int svt_index_insert(svt_index *ix, int32_t n, const int64_t *ids, const int8_t *rows, const uint64_t *sigs,
                                const int32_t *list_of, void *hip_stream) {
  g_err.clear();
  const char *who = "svt_index_insert";
  int rc = check_update(ix, n, ids, who);
  if (rc != SVT_OK || n == 0) return rc;
  if (!rows || !sigs || !list_of) return fail(SVT_EINVAL, "%s: NULL rows, sigs or list_of", who);
  if ((rc = check_ids(ix, n, ids, false, who)) != SVT_OK) return rc;
  const int32_t nlist = ix->dev.nlist, W = ix->dev.sig_words;
  std::vector<int32_t> want((size_t)nlist, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t c = list_of[i];
    if (c < 0 || c >= nlist) return fail(SVT_EINVAL, "%s: list_of[%d] = %d out of range", who, i, c);
    if (sig_reserved(sigs + (size_t)i * W, W))
      return fail(SVT_EINVAL, "%s: item %d has every signature bit set (reserved for free slots)", who, i);
    if (++want[(size_t)c] > (int32_t)ix->free_h[(size_t)c].size())
      return fail(SVT_ENOSPACE, "%s: cluster %d has %zu free slots, the batch needs more (upload with more slack)", who,
                  c, ix->free_h[(size_t)c].size());
  }
  std::vector<UpdOp> ops((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t c = list_of[i];
    const int32_t p = ix->free_h[(size_t)c].back();
    ix->free_h[(size_t)c].pop_back();
    ix->slot_of[(size_t)ids[i]] = p;
    ops[(size_t)i] = UpdOp{p, (int32_t)ids[i], c, kUpdInsert};
  }
  ix->n_live += n;
  return apply_updates(ix, ops, rows, sigs, (hipStream_t)hip_stream, who);
}

extern "C" int svt_index_delete(svt_index *ix, int32_t n, const int64_t *ids, void *hip_stream) {
  g_err.clear();
  const char *who = "svt_index_delete";
  int rc = check_update(ix, n, ids, who);
  if (rc != SVT_OK || n == 0) return rc;
  if ((rc = check_ids(ix, n, ids, true, who)) != SVT_OK) return rc;
  std::vector<UpdOp> ops((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = ix->slot_of[(size_t)ids[i]];
    const int32_t c = cluster_of_slot(ix, p);
    ops[(size_t)i] = UpdOp{p, (int32_t)ids[i], c, kUpdDelete};
    ix->slot_of[(size_t)ids[i]] = -1;
  }
  // freed slots go back on top of their clusters' stacks, lowest slot last pushed
  std::vector<UpdOp> by_slot(ops);
  std::sort(by_slot.begin(), by_slot.end(), [](const UpdOp &a, const UpdOp &b) { return a.pos > b.pos; });
  for (const UpdOp &op : by_slot) ix->free_h[(size_t)op.cluster].push_back(op.pos);
  ix->n_live -= n;
  return apply_updates(ix, ops, nullptr, nullptr, (hipStream_t)hip_stream, who);
}

extern "C" int svt_index_resign(svt_index *ix, int32_t n, const int64_t *ids, const uint64_t *sigs, void *hip_stream) {
  g_err.clear();
  const char *who = "svt_index_resign";
  int rc = check_update(ix, n, ids, who);
  if (rc != SVT_OK || n == 0) return rc;
  if (!sigs) return fail(SVT_EINVAL, "%s: NULL sigs", who);
  if ((rc = check_ids(ix, n, ids, true, who)) != SVT_OK) return rc;
  const int32_t W = ix->dev.sig_words;
  for (int32_t i = 0; i < n; ++i)
    if (sig_reserved(sigs + (size_t)i * W, W))
      return fail(SVT_EINVAL, "%s: signature %d has every bit set (reserved for free slots)", who, i);
  std::vector<UpdOp> ops((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = ix->slot_of[(size_t)ids[i]];
    ops[(size_t)i] = UpdOp{p, (int32_t)ids[i], cluster_of_slot(ix, p), kUpdResign};
  }
  return apply_updates(ix, ops, nullptr, sigs, (hipStream_t)hip_stream, who);
}

// ------------------------------------------------------------------------------------------------
// workspace layout

namespace {

struct Layout {
  size_t coarse_scores, probes, seg, pb, qlen, qcost, qtail, cstart, chunks, order, cband, thr, hlo, hshift, ghist, counter,
      slot_cnt, slot_min, slot_keys, mcnt, mkeys, stats;
  // tile and exhaustive paths (absent on the query path)
  size_t sthr, redo, pool_cnt, pool, gcnt, gfill, gstart, estart, uoff, mrec, entries, ctab, thdr, tblk, sbuf;
  size_t qdens, clog, ccost, cstart_u;
  size_t lk_hist, lk_state, lk_cnt, lk_keys, lk_cstart;   // large-k path
  size_t total;
  SearchShape sh;
};

// Batches of at least this many queries take the tile path by default: their queries share enough
// probed clusters for one read per batch to pay for the union work list and the pools (at 80M items,
// nprobe 64, the query path is faster at 32 queries and the tile path at 256).
constexpr int32_t kTileMinBatch = 128;
// The union stream is indexed with 32-bit offsets.
constexpr int64_t kMaxUnion = (int64_t(1) << 31) - (int64_t(1) << 20);

int32_t mask_groups(const svt_search_options *o) { return (o && o->mask_groups > 1) ? o->mask_groups : 1; }
// members per (query, probed cluster) on the tile path
int32_t tile_groups(int32_t G) { return G <= 1 ? 1 : (G <= 2 ? 2 : 4); }

bool tile_fits(const svt_index *ix, int32_t B, int32_t nprobe, int32_t GT) {
  const int64_t blocks = ((int64_t)B * GT + kTMembers - 1) / kTMembers;
  return ix->dev.n_items * blocks < kMaxUnion && (int64_t)B * nprobe * GT < kMaxUnion;
}

int resolve_path(const svt_index *ix, int32_t B, int32_t nprobe, int32_t k, const svt_search_options *o) {
  const int want = o ? o->path : SVT_PATH_AUTO;
  if (want == SVT_PATH_LARGE_K || k > SVT_MAX_K) return kPathLargeK;
  if (want == SVT_PATH_QUERY || ix->dev.n_items == 0) return kPathQuery;
  const bool exh = nprobe == ix->dev.nlist;
  const int32_t GT = tile_groups(mask_groups(o));
  if (want == SVT_PATH_TILE) {
    if (exh) return kPathExh;
    return tile_fits(ix, B, nprobe, GT) ? kPathTile : kPathQuery;
  }
  if (exh && B >= 2) return kPathExh;
  if (B >= kTileMinBatch && tile_fits(ix, B, nprobe, GT)) return kPathTile;
  return kPathQuery;
}

// SVT_OK or SVT_EINVAL (message set)
int check_options(const svt_search_options *o, const char *who) {
  if (!o) return SVT_OK;
  if (o->path != SVT_PATH_AUTO && o->path != SVT_PATH_QUERY && o->path != SVT_PATH_TILE && o->path != SVT_PATH_LARGE_K)
    return fail(SVT_EINVAL, "%s: unknown path %d", who, o->path);
  if (o->pool_keys < 0) return fail(SVT_EINVAL, "%s: pool_keys %d < 0", who, o->pool_keys);
  if (o->flags & ~(SVT_OPT_MERGE_FROM_SLOTS | SVT_OPT_FORCE_REDO))
    return fail(SVT_EINVAL, "%s: unknown flag bits 0x%x", who, o->flags);
  if (o->mask_groups < 0 || o->mask_groups > SVT_MAX_MASK_GROUPS)
    return fail(SVT_EINVAL, "%s: mask_groups %d out of [0, %d]", who, o->mask_groups, SVT_MAX_MASK_GROUPS);
  for (int i = 0; i < 4; ++i)
    if (o->reserved[i] != 0) return fail(SVT_EINVAL, "%s: reserved word %d is not 0", who, i);
  return SVT_OK;
}

Layout layout(const svt_index *ix, int32_t B, int32_t nprobe, int32_t k, const svt_search_options *o) {
  Layout L{};
  const size_t nlist = (size_t)ix->dev.nlist;
  SearchShape &sh = L.sh;
  sh.B = B;
  sh.nprobe = nprobe;
  sh.k = k;
  sh.P = ix->scan_wgs;
  sh.max_chunks = max_chunks_for(B, ix->scan_wgs);
  sh.path = resolve_path(ix, B, nprobe, k, o);
  sh.gather_cap = (o && (o->flags & SVT_OPT_MERGE_FROM_SLOTS)) ? 0 : kGatherCap;
  sh.force_redo = (o && (o->flags & SVT_OPT_FORCE_REDO)) ? 1 : 0;
  sh.TP = ix->tscan_wgs;
  sh.XP = ix->xscan_wgs;
  sh.G = mask_groups(o);
  sh.GT = tile_groups(sh.G);
  const size_t C = (size_t)sh.max_chunks;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align256(bytes);
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
  L.counter = take(8 * sizeof(uint32_t));
  L.slot_cnt = take(C * sizeof(int32_t));
  L.slot_min = take(C * sizeof(uint64_t));
  const bool lk = sh.path == kPathLargeK;
  L.slot_keys = take(C * (size_t)(lk ? 1 : k) * sizeof(uint64_t));   // the large-k path keeps no slots
  L.mcnt = take((size_t)B * sizeof(uint32_t));
  L.mkeys = take((size_t)B * kGatherCap * sizeof(uint64_t));
  L.stats = take((size_t)B * 2 * sizeof(int64_t));
  if (lk) {
    // pool mode: 8k keys per query (or the options' pool_keys), while the pools take at most 1 GiB
    const int64_t def = ((int64_t)8 * k + 4095) / 4096 * 4096;
    const int64_t cap = (o && o->pool_keys > 0) ? o->pool_keys : def;
    sh.pool_cap = (int64_t)B * cap * 8 <= ((int64_t)1 << 30) ? (int32_t)cap : 0;
    // the tile scan fills the pools for batches the tile path would take (at least kTileMinBatch queries,
    // a union plan that fits, not every cluster probed); otherwise the large-k path's own pooled scan
    sh.lk_tile = sh.pool_cap > 0 && B >= kTileMinBatch && nprobe < (int32_t)nlist && ix->dev.n_items > 0 &&
                         tile_fits(ix, B, nprobe, sh.GT) ? 1 : 0;
    if (sh.pool_cap > 0) {
      L.sthr = take((size_t)B * sizeof(int32_t));
      L.pool_cnt = take((size_t)B * sizeof(uint32_t));
      L.pool = take((size_t)B * (size_t)sh.pool_cap * sizeof(uint64_t));
    }
    L.lk_hist = take((size_t)B * kLkBins * sizeof(uint32_t));
    L.lk_state = take((size_t)B * sizeof(LkState));
    L.lk_cnt = take((size_t)B * sizeof(uint32_t));
    L.lk_keys = take((size_t)B * (size_t)k * sizeof(uint64_t));
    L.lk_cstart = take((size_t)(B + 1) * sizeof(int32_t));
  }
  if (sh.path == kPathTile || sh.path == kPathExh) {
    const int64_t def = std::max<int64_t>(4096, ((int64_t)16 * k + 4095) / 4096 * 4096);
    sh.pool_cap = (int32_t)((o && o->pool_keys > 0) ? o->pool_keys : def);
    L.sthr = take((size_t)B * sizeof(int32_t));
    L.redo = take((size_t)B * sizeof(int32_t));
    L.pool_cnt = take((size_t)B * sizeof(uint32_t));
    L.pool = take((size_t)B * (size_t)sh.pool_cap * sizeof(uint64_t));
  }
  if (sh.path == kPathTile || sh.lk_tile) {
    const int64_t blocks = ((int64_t)B * sh.GT + kTMembers - 1) / kTMembers;
    sh.max_entries =
        (int32_t)std::max<int64_t>(1, std::min<int64_t>((int64_t)nlist * blocks, (int64_t)B * nprobe * sh.GT));
    sh.max_tchunks = kTChunksPerWave * kTWaves * sh.TP + 2;
    L.gcnt = take(nlist * sizeof(int32_t));
    L.gfill = take(nlist * sizeof(int32_t));
    L.gstart = take((nlist + 1) * sizeof(int32_t));
    L.estart = take((nlist + 1) * sizeof(int32_t));
    L.uoff = take(nlist * sizeof(int32_t));
    L.mrec = take((size_t)B * nprobe * sh.GT * sizeof(MRec));
    L.entries = take((size_t)sh.max_entries * sizeof(UEntry));
    L.ctab = take((size_t)sh.max_tchunks * sizeof(int32_t));
    L.thdr = take(4 * sizeof(int32_t));
    L.tblk = take(4 * kMaxPlanBlocks * sizeof(int64_t));
    L.qdens = take((size_t)B * sizeof(float));
    L.clog = take(nlist * sizeof(float));
    L.ccost = take((nlist + 1) * sizeof(int64_t));
    L.cstart_u = take((size_t)(sh.max_tchunks + 1) * sizeof(int32_t));
  }
  if (sh.path == kPathExh) {
    const int64_t N = ix->dev.n_items;
    const int64_t points = (N + kXStride - 1) / kXStride;   // sample pass: every kXStride-th position
    sh.n_sblocks = (int32_t)((points + 63) / 64);            // runs of 64 points
    sh.scap = 16 * sh.n_sblocks;                             // slots per query: one per lane and run
    L.sbuf = take((size_t)B * (size_t)sh.scap * sizeof(int32_t));
  }
  L.total = off;
  return L;
}

// SVT_OK or the error code (message set)
int check_search_args(const svt_index *ix, int32_t B, int32_t nprobe, int32_t k, const svt_search_options *o,
                      const char *who) {
  if (!ix || !is_live(ix) || ix->magic != kMagic) return fail(SVT_ESTATE, "%s: not a live index", who);
  if (B < 0 || B > 65535) return fail(SVT_EINVAL, "%s: n_queries %d out of [0, 65535]", who, B);
  if (nprobe < 1 || nprobe > ix->dev.nlist) return fail(SVT_EINVAL, "%s: nprobe %d out of [1, %d]", who, nprobe, ix->dev.nlist);
  if (k < 1 || k > SVT_MAX_K_LARGE) return fail(SVT_EINVAL, "%s: k %d out of [1, %d]", who, k, SVT_MAX_K_LARGE);
  const int rc = check_options(o, who);
  if (rc != SVT_OK) return rc;
  if (k > SVT_MAX_K && o && o->path != SVT_PATH_AUTO && o->path != SVT_PATH_LARGE_K)
    return fail(SVT_EINVAL, "%s: k %d above %d needs the large-k path (path %d requested)", who, k, SVT_MAX_K, o->path);
  return SVT_OK;
}

Work carve(const Layout &L, void *workspace, int64_t *out_stats) {
  char *base = (char *)workspace;
  const SearchShape &sh = L.sh;
  Work w{};
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
  w.mcnt = (uint32_t *)(base + L.mcnt);
  w.mkeys = (uint64_t *)(base + L.mkeys);
  w.stats = out_stats ? out_stats : (int64_t *)(base + L.stats);
  if (sh.path == kPathLargeK) {
    if (sh.pool_cap > 0) {
      w.sthr = (int32_t *)(base + L.sthr);
      w.pool_cnt = (uint32_t *)(base + L.pool_cnt);
      w.pool = (uint64_t *)(base + L.pool);
    }
    w.lk_hist = (uint32_t *)(base + L.lk_hist);
    w.lk_state = (LkState *)(base + L.lk_state);
    w.lk_cnt = (uint32_t *)(base + L.lk_cnt);
    w.lk_keys = (uint64_t *)(base + L.lk_keys);
    w.lk_cstart = (int32_t *)(base + L.lk_cstart);
  }
  if (sh.path == kPathTile || sh.path == kPathExh) {
    w.sthr = (int32_t *)(base + L.sthr);
    w.redo = (int32_t *)(base + L.redo);
    w.pool_cnt = (uint32_t *)(base + L.pool_cnt);
    w.pool = (uint64_t *)(base + L.pool);
  }
  if (sh.path == kPathTile || sh.lk_tile) {
    w.gcnt = (int32_t *)(base + L.gcnt);
    w.gfill = (int32_t *)(base + L.gfill);
    w.gstart = (int32_t *)(base + L.gstart);
    w.estart = (int32_t *)(base + L.estart);
    w.uoff = (int32_t *)(base + L.uoff);
    w.mrec = (MRec *)(base + L.mrec);
    w.entries = (UEntry *)(base + L.entries);
    w.ctab = (int32_t *)(base + L.ctab);
    w.thdr = (int32_t *)(base + L.thdr);
    w.tblk = (int64_t *)(base + L.tblk);
    w.qdens = (float *)(base + L.qdens);
    w.clog = (float *)(base + L.clog);
    w.ccost = (int64_t *)(base + L.ccost);
    w.cstart_u = (int32_t *)(base + L.cstart_u);
  }
  if (sh.path == kPathExh) w.sbuf = (int32_t *)(base + L.sbuf);
  return w;
}

// Enqueue the search of a validated call on stream s.
int enqueue_search(const svt_index *ix, const SearchShape &sh, const Work &w, const int8_t *queries,
                   const uint64_t *masks, const float *query_scales, int64_t *out_ids, int32_t *out_scores,
                   float *out_fscores, int32_t *out_counts, bool record_events, hipStream_t s) {
  const int prof_mode = record_events ? g_prof_on.load(std::memory_order_relaxed) : 0;
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
  const DevIndex &dx = ix->dev;
  hipError_t e;
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if ((e = launch_coarse_keys(dx, queries, sh.B, w, s)) != hipSuccess) return fail_hip(e, "launch coarse_keys");
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  {
    SearchShape cs = sh;
    // large-k path: the threshold rank (for kAlpha * k candidates) is set for k / 2, so that a pool of 8k
    // keys expects about 2k candidates
    if (sh.path == kPathLargeK) cs.k = std::max(1, (sh.k + 1) / 2);
    if ((e = launch_coarse_select(dx, queries, masks, cs, w, s)) != hipSuccess) return fail_hip(e, "launch coarse_select");
  }
  if (sh.path == kPathLargeK) {
    if ((e = mark()) != hipSuccess) return fail_hip(e, "event");   // end of the select stage
    if (sh.lk_tile && (e = launch_tile_plan(dx, masks, sh, w, s)) != hipSuccess) return fail_hip(e, "launch tile plan");
    if ((e = mark()) != hipSuccess) return fail_hip(e, "event");   // end of the plan stage
    if (sh.lk_tile && (e = launch_tscan(dx, queries, sh, w, s)) != hipSuccess) return fail_hip(e, "launch tile scan");
    if ((e = launch_large_k(dx, queries, masks, query_scales, sh, ix->top_slots[(size_t)sh.nprobe], w, out_ids,
                            out_scores, out_fscores, out_counts, s)) != hipSuccess)
      return fail_hip(e, "launch large-k passes");
    for (int i = 0; i < 3; ++i)   // the passes are the scan stage; no fallback, no merge
      if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
    if (prof) ++ps.searches;
    return SVT_OK;
  }
  if (sh.path == kPathQuery && (e = launch_plan(dx, sh, w, 0, s)) != hipSuccess) return fail_hip(e, "launch plan");
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if (sh.path == kPathTile && (e = launch_tile_plan(dx, masks, sh, w, s)) != hipSuccess)
    return fail_hip(e, "launch tile plan");
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if (sh.path == kPathQuery) e = launch_scan(dx, queries, masks, sh, w, 0, s);
  else if (sh.path == kPathTile) e = launch_tscan(dx, queries, sh, w, s);
  else e = launch_exh_scan(dx, queries, masks, sh, w, s);
  if (e != hipSuccess) return fail_hip(e, "launch scan");
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if (sh.path != kPathQuery) {
    // the queries whose pools cannot prove their top k, query by query (rare: a quarter of the scan's
    // workgroups; the work list and chunk sizes follow that count)
    SearchShape rs = sh;
    rs.P = std::max(1, sh.P / 4);
    if ((e = launch_plan(dx, rs, w, 1, s)) != hipSuccess) return fail_hip(e, "launch plan");
    if ((e = launch_scan(dx, queries, masks, rs, w, 1, s)) != hipSuccess) return fail_hip(e, "launch scan");
    if ((e = launch_merge(dx, query_scales, rs, w, 1, out_ids, out_scores, out_fscores, out_counts, s)) != hipSuccess)
      return fail_hip(e, "launch merge");
  }
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if (sh.path == kPathQuery)
    e = launch_merge(dx, query_scales, sh, w, 0, out_ids, out_scores, out_fscores, out_counts, s);
  else
    e = launch_pool_merge(dx, query_scales, sh, w, out_ids, out_scores, out_fscores, out_counts, s);
  if (e != hipSuccess) return fail_hip(e, "launch merge");
  if ((e = mark()) != hipSuccess) return fail_hip(e, "event");
  if (prof) ++ps.searches;
  return SVT_OK;
}

// pointer checks shared by the search entry points; SVT_OK or SVT_EINVAL (message set)
int check_search_ptrs(const int8_t *queries, const uint64_t *masks, const int64_t *out_ids, const int32_t *out_scores,
                      const char *who) {
  if (!queries || !masks || !out_ids || !out_scores)
    return fail(SVT_EINVAL, "%s: NULL queries, masks, out_ids or out_scores", who);
  if (((uintptr_t)queries & 15) != 0) return fail(SVT_EINVAL, "%s: queries not 16-byte aligned", who);
  if (((uintptr_t)masks & 7) != 0) return fail(SVT_EINVAL, "%s: masks not 8-byte aligned", who);
  if (((uintptr_t)out_ids & 7) != 0 || ((uintptr_t)out_scores & 3) != 0)
    return fail(SVT_EINVAL, "%s: out_ids not 8-byte or out_scores not 4-byte aligned", who);
  return SVT_OK;
}

}  // namespace

namespace svt {

int report(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  const int r = vfail(code, fmt, ap);
  va_end(ap);
  return r;
}

int search_size(const svt_index *ix, int32_t B, int32_t nprobe, int32_t k, const svt_search_options *opts,
                const char *who, size_t *bytes, int *device) {
  const int rc = check_search_args(ix, B, nprobe, k, opts, who);
  if (rc != SVT_OK) return rc;
  *bytes = layout(ix, B, nprobe, k, opts).total;
  *device = ix->device;
  return SVT_OK;
}

int search_into(const svt_index *ix, int32_t B, const int8_t *queries, const uint64_t *masks,
                const float *query_scales, int32_t nprobe, int32_t k, int64_t *out_ids, int32_t *out_scores,
                float *out_fscores, int32_t *out_counts, int64_t *out_stats, const svt_search_options *opts,
                void *workspace, size_t workspace_bytes, void *hip_stream, bool record_events, const char *who) {
  int rc = check_search_args(ix, B, nprobe, k, opts, who);
  if (rc != SVT_OK) return rc;
  if (B == 0) return SVT_OK;
  if ((rc = check_search_ptrs(queries, masks, out_ids, out_scores, who)) != SVT_OK) return rc;
  if (((uintptr_t)out_fscores & 3) || ((uintptr_t)out_counts & 3) || ((uintptr_t)out_stats & 7) ||
      ((uintptr_t)query_scales & 3))
    return fail(SVT_EINVAL, "%s: misaligned out_fscores, out_counts, out_stats or query_scales", who);
  if (!workspace) return fail(SVT_EINVAL, "%s: NULL workspace", who);
  if (((uintptr_t)workspace & 255) != 0) return fail(SVT_EINVAL, "%s: workspace not 256-byte aligned", who);
  const Layout L = layout(ix, B, nprobe, k, opts);
  if (workspace_bytes < L.total)
    return fail(SVT_EINVAL, "%s: workspace %zu bytes < required %zu", who, workspace_bytes, L.total);
  const Work w = carve(L, workspace, out_stats);
  return enqueue_search(ix, L.sh, w, queries, masks, query_scales, out_ids, out_scores, out_fscores, out_counts,
                        record_events, (hipStream_t)hip_stream);
}

}  // namespace svt

extern "C" size_t svt_search_workspace_size(const svt_index *ix, int32_t n_queries, int32_t nprobe, int32_t k,
                                            const svt_search_options *opts) {
  g_err.clear();
  if (check_search_args(ix, n_queries, nprobe, k, opts, "svt_search_workspace_size") != SVT_OK) return 0;
  return layout(ix, n_queries, nprobe, k, opts).total;
}

extern "C" int svt_rerank(const svt_index *ix, int32_t B, const int8_t *queries, const float *query_scales,
                          int32_t n_cand, const int64_t *cand_ids, const svt_rerank_net *net, int32_t k_out,
                          int64_t *out_ids, float *out_scores, int32_t *out_counts, void *hip_stream) {
  g_err.clear();
  const char *who = "svt_rerank";
  if (!ix || !is_live(ix) || ix->magic != kMagic) return fail(SVT_ESTATE, "%s: not a live index", who);
  if (B < 0 || B > 65535) return fail(SVT_EINVAL, "%s: n_queries %d out of [0, 65535]", who, B);
  if (n_cand < 0 || n_cand > SVT_RERANK_MAX_CAND)
    return fail(SVT_EINVAL, "%s: n_cand %d out of [0, %d]", who, n_cand, SVT_RERANK_MAX_CAND);
  if (k_out < 1 || k_out > SVT_RERANK_MAX_OUT)
    return fail(SVT_EINVAL, "%s: k_out %d out of [1, %d]", who, k_out, SVT_RERANK_MAX_OUT);
  if (!net) return fail(SVT_EINVAL, "%s: NULL net", who);
  if (net->n_experts < 1 || net->n_experts > SVT_RERANK_MAX_EXPERTS)
    return fail(SVT_EINVAL, "%s: n_experts %d out of [1, %d]", who, net->n_experts, SVT_RERANK_MAX_EXPERTS);
  if (net->hidden < 1 || net->n_experts * net->hidden > SVT_RERANK_MAX_UNITS)
    return fail(SVT_EINVAL, "%s: hidden %d: need 1 <= hidden and n_experts * hidden <= %d", who, net->hidden,
                SVT_RERANK_MAX_UNITS);
  if (B == 0) return SVT_OK;
  if (!net->gate_w || !net->gate_b || !net->w1 || !net->b1 || !net->w2 || !net->b2)
    return fail(SVT_EINVAL, "%s: NULL net weight", who);
  if (!queries || !out_ids || !out_scores || (n_cand > 0 && !cand_ids))
    return fail(SVT_EINVAL, "%s: NULL queries, cand_ids or outputs", who);
  if (((uintptr_t)cand_ids & 7) || ((uintptr_t)out_ids & 7) || ((uintptr_t)out_scores & 3) ||
      ((uintptr_t)out_counts & 3) || ((uintptr_t)query_scales & 3))
    return fail(SVT_EINVAL, "%s: misaligned cand_ids, outputs or query_scales", who);
  for (const float *wp : {net->gate_w, net->gate_b, net->w1, net->b1, net->w2, net->b2})
    if ((uintptr_t)wp & 3) return fail(SVT_EINVAL, "%s: misaligned net weight", who);
  const hipError_t e = launch_rerank(ix->dev, B, queries, query_scales, n_cand, cand_ids, *net, k_out, out_ids,
                                     out_scores, out_counts, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail_hip(e, "launch_rerank");
  return SVT_OK;
}

extern "C" int svt_search_path(const svt_index *ix, int32_t n_queries, int32_t nprobe, int32_t k,
                               const svt_search_options *opts) {
  g_err.clear();
  const int rc = check_search_args(ix, n_queries, nprobe, k, opts, "svt_search_path");
  if (rc != SVT_OK) return rc;
  switch (resolve_path(ix, n_queries, nprobe, k, opts)) {
    case kPathLargeK: return SVT_PATH_LARGE_K;
    case kPathTile: return SVT_PATH_TILE;
    case kPathExh: return SVT_PATH_EXHAUSTIVE;
    default: return SVT_PATH_QUERY;
  }
}

extern "C" int svt_search(const svt_index *ix, int32_t B, const int8_t *queries, const uint64_t *masks,
                          const float *query_scales, int32_t nprobe, int32_t k, int64_t *out_ids, int32_t *out_scores,
                          float *out_fscores, int32_t *out_counts, int64_t *out_stats, const svt_search_options *opts,
                          void *workspace, size_t workspace_bytes, void *hip_stream) {
  g_err.clear();
  return search_into(ix, B, queries, masks, query_scales, nprobe, k, out_ids, out_scores, out_fscores, out_counts,
                     out_stats, opts, workspace, workspace_bytes, hip_stream, true, "svt_search");
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
