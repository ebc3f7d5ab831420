/*
 * svt.h - C ABI of the fused int8 IVF + Bloom-signature top-k search library for AMD MI355X (gfx950).
 *
 * What the library computes (the "index as model" retrieval path):
 *   for each query b
 *     1. coarse probe: score all int8 centroids with int8 dot products (int32 accumulation) and keep
 *        the nprobe best clusters, ties to the lower cluster id
 *        ["SilverTorch - Index as Model", "How each component worked before": probe the most
 *         promising clusters first; "The pure-PyTorch decision": large probe counts, 64 probes];
 *     2. filter: inside those clusters only, an item is eligible iff every bit of the request mask is
 *        set in its Bloom signature, (sig & mask) == mask over every signature word
 *        [same post, Bloom index filter paragraph: compact per-item signature checked against the
 *         request with simple bit operations];
 *     3. score: int8 . int8 with int32 accumulation for eligible items only
 *        [same post, fused Int8 ANN paragraph and compute-cost-efficiency section ("dp4a")];
 *     4. select: the k best eligible items by (score desc, item id asc), kept on chip and merged for
 *        k <= 2048 (larger k, up to SVT_MAX_K_LARGE: a radix select over repeated passes, see
 *        SVT_PATH_LARGE_K); only the final candidates are written out
 *        [same post: no recall loss observed at 64 probes, top-2048; "Meta Andromeda" summary, System
 *         section: intermediates stay in registers and shared memory, targeting + scoring + top-K
 *         on one machine, only the final candidates return].
 *   Scores are also returned dequantised: f = S / (item_scale * query_scale) computed in double and
 *   rounded once to float (a reading: the pages do not state the float mapping).
 *
 * Conventions for every entry point
 *   - Return value: SVT_OK (0) or a negative SVT_E* code; svt_last_error() then holds a message
 *     (thread-local, valid until the next call on the same thread).
 *   - Arguments are validated on the host before anything is enqueued; on error no output is written.
 *   - "device" pointers are HIP device memory of the device the index lives on; "host" pointers are
 *     ordinary host memory.  hip_stream is a hipStream_t (NULL = the default stream).
 *   - The library never takes ownership of caller memory.
 */
#ifndef SVT_H
#define SVT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SVT_OK = 0,
  SVT_EINVAL = -1,       /* invalid argument (NULL pointer, out-of-range size, bad layout)         */
  SVT_ENOMEM = -2,       /* device or host allocation failed                                        */
  SVT_EDEVICE = -3,      /* a HIP runtime call or kernel launch failed                              */
  SVT_EUNSUPPORTED = -4, /* valid but unsupported shape (dimension, signature width)                 */
  SVT_ESTATE = -5,       /* object in the wrong state (freed or foreign index, not updatable)        */
  SVT_ENOSPACE = -6      /* an insert finds no free slot in its cluster                              */
};

#define SVT_MAX_K 2048        /* largest top-k of the fused paths (per-workgroup lists in LDS)        */
#define SVT_MAX_K_LARGE 16384 /* largest top-k per query: k > SVT_MAX_K takes the large-k path        */
#define SVT_MAX_SIG_WORDS 2   /* signatures of 64 or 128 bits                                       */

/* Opaque, library-owned index resident in HBM. */
typedef struct svt_index svt_index;

/* Host description of a catalogue to upload.  Item i (0 <= i < n_items) is row i of every array;
 * its id in search results is i. */
typedef struct {
  int64_t n_items;            /* 0 <= n_items < 2^31                                                */
  int32_t dim;                /* 16, 32, 64, 128 or 256 (int8 components per vector)                */
  int32_t sig_words;          /* 1 (64-bit) or 2 (128-bit) Bloom signatures                         */
  int32_t nlist;              /* number of IVF clusters, 1 <= nlist <= 65536                        */
  const int8_t *items;        /* host, [n_items][dim] row-major int8 item embeddings                */
  const uint64_t *sigs;       /* host, [n_items][sig_words] Bloom signatures                        */
  const int32_t *list_of;     /* host, [n_items] cluster of each item, each in [0, nlist)           */
  const int8_t *centroids;    /* host, [nlist][dim] int8 coarse centroids                           */
  float item_scale;           /* > 0; float value of an int8 component is x / item_scale            */
} svt_index_desc;

/*
 * svt_index_upload - copy a catalogue into device memory in the search layout.
 * The items of each cluster become contiguous (clusters in id order, items within a cluster in id
 * order); rows, signatures and ids are stored structure-of-arrays in HBM ("index as model": the item
 * index is a tensor inside the model, "SilverTorch - Index as Model", opening section).
 * The device is the current HIP device.  The call enqueues its copies on hip_stream and synchronises
 * that stream before returning; the caller may free its host arrays afterwards.
 * Errors: SVT_EINVAL (NULL desc/out, NULL array with n_items > 0, sizes out of range, list_of entry out
 * of range), SVT_EUNSUPPORTED (dim or sig_words not listed above), SVT_ENOMEM, SVT_EDEVICE.
 * On success *out owns the device memory until svt_index_free.
 */
int svt_index_upload(const svt_index_desc *desc, void *hip_stream, svt_index **out);

/*
 * svt_index_upload_updatable - svt_index_upload for an index that takes in-place updates afterwards
 * (svt_index_insert, svt_index_delete, svt_index_resign): the freshness of "SilverTorch - Index as
 * Model" (index freshness section), where the index tensors receive a continuous stream of small,
 * targeted in-place updates between full snapshots.
 * Each cluster gets max(slack_min, ceil(slack_frac * its item count)) free slots after its items; a free
 * slot holds the reserved signature with every bit set (which no filter passes, whatever the mask) and
 * the id -1, so searches scan it at the cost of its signature and never return it.  Ids of later
 * inserts are any unused ids in [0, id_capacity).  The host keeps a record of the layout (an int32 per
 * id and per free slot) that places each update.
 *   id_capacity  n_items <= id_capacity < 2^31
 *   slack_min    >= 0;  slack_frac  in [0, 64]
 * Other arguments, errors and ownership as svt_index_upload; also SVT_EINVAL for a bad id_capacity or
 * slack, or more than 2^31 slots.  Items whose signature has every bit set are rejected (SVT_EINVAL) by
 * both uploads: that signature marks free slots.
 */
int svt_index_upload_updatable(const svt_index_desc *d, int64_t id_capacity, int32_t slack_min, float slack_frac,
                               void *hip_stream, svt_index **out);

/*
 * In-place updates of an updatable index (same section of the same page).  Each call takes a batch from
 * host memory, checks all of it (on any error nothing changes), chooses the slots on the host, copies
 * the batch to the device, applies it with one kernel on hip_stream and synchronises that stream before
 * returning.  Searches see the index as of the updates enqueued before them on their stream: searches
 * in flight on other streams must not overlap an update.  A search after the updates returns exactly
 * what a search of the updated catalogue (the items present, with their current signatures) returns.
 *   svt_index_insert  n items: ids (unused, distinct), rows [n][dim] int8, sigs [n][sig_words], list_of
 *                     [n] cluster of each; each goes to a free slot of its cluster (lowest slot first)
 *   svt_index_delete  n present, distinct ids: their slots become free
 *   svt_index_resign  n present, distinct ids: their signatures become sigs [n][sig_words]
 * All pointers are host pointers.  Errors: SVT_ESTATE (freed index, or one not uploaded as updatable),
 * SVT_EINVAL (n < 0, NULL pointer with n > 0, an id out of range, repeated, already present (insert) or
 * absent (delete, resign), a cluster out of range, a reserved signature), SVT_ENOSPACE (a cluster without
 * enough free slots for the batch), SVT_ENOMEM / SVT_EDEVICE (device staging or kernel; the index is then
 * undefined).  n == 0 is a no-op.
 */
int svt_index_insert(svt_index *ix, int32_t n, const int64_t *ids, const int8_t *rows, const uint64_t *sigs,
                     const int32_t *list_of, void *hip_stream);
int svt_index_delete(svt_index *ix, int32_t n, const int64_t *ids, void *hip_stream);
int svt_index_resign(svt_index *ix, int32_t n, const int64_t *ids, const uint64_t *sigs, void *hip_stream);

/* svt_index_free - release an index and its device memory.
 * hip_stream: the stream the caller's searches on this index ran on (NULL = the default stream); the
 * call synchronises that stream before freeing.  Searches enqueued on other streams must have
 * completed (the caller synchronises them); the device as a whole is not synchronised.
 * NULL ix is accepted (no-op).  SVT_ESTATE if ix is not a live index from svt_index_upload;
 * SVT_EDEVICE if the stream synchronisation fails (the index is then still freed). */
int svt_index_free(svt_index *ix, void *hip_stream);

/* svt_index_info - shape of an uploaded index (n_items: the items present, not free slots); any output
 * pointer may be NULL. */
int svt_index_info(const svt_index *ix, int64_t *n_items, int32_t *dim, int32_t *sig_words, int32_t *nlist);

/*
 * Search paths.  Every path returns the same, exact result (tested element by element); they differ in
 * how the probed clusters are read.
 *   SVT_PATH_AUTO   chosen from the batch shape alone (never from query values): the tile path for
 *                   batches whose queries share probed clusters, the query path otherwise
 *   SVT_PATH_QUERY  query by query: each query's probed clusters are read for that query, an exact
 *                   top-k is kept per workgroup in LDS and merged ("SilverTorch - Index as Model":
 *                   probe the most promising clusters first, filter only inside them, score only the
 *                   survivors)
 *   SVT_PATH_TILE   each probed cluster is read once per batch for every query that probes it
 *                   (the union of the batch's probed clusters is streamed once); with nprobe == nlist
 *                   the catalogue is streamed once and scored for the whole batch with int8 MFMA.
 *                   Candidates at or above a per-query threshold estimated from a sample of the
 *                   query's items are kept in per-query pools; a query whose pool holds fewer than k
 *                   candidates (with a threshold above the minimum) or overflows is redone on the query
 *                   path, so the result stays exact whatever the data.
 *   SVT_PATH_LARGE_K  any k up to SVT_MAX_K_LARGE (the path every search with k > SVT_MAX_K takes;
 *                   also selectable for smaller k).  One scan keeps every eligible item whose score
 *                   reaches a threshold estimated from the query's samples (about 2k of them) in a
 *                   per-query pool; a pool that proves the top k is selected and sorted.  Any other
 *                   query runs an exact radix select over its eligible items' (score, id) keys, one
 *                   11-bit digit per pass over its probed items (at most 5 passes), then one pass that
 *                   keeps the keys at or above its threshold and an LDS sort of those
 *                   ["SilverTorch - Index as Model", fused Int8 ANN paragraph and compute-cost table:
 *                    top-k well beyond GPU FAISS's 2048].  Each pass reads the probed items again.
 */
enum { SVT_PATH_AUTO = 0, SVT_PATH_QUERY = 1, SVT_PATH_TILE = 2, SVT_PATH_EXHAUSTIVE = 3, SVT_PATH_LARGE_K = 4 };

/* svt_search_options.flags */
#define SVT_OPT_MERGE_FROM_SLOTS 1u  /* query path: the merge reads every chunk's slot instead of the keys
                                        gathered above each query's final bound (a test of that branch)  */
#define SVT_OPT_FORCE_REDO 2u        /* tile and large-k paths: every query's threshold is set above any
                                        score, so every query with an eligible item is redone on the
                                        query path (tile) or goes through the digit passes (large k)
                                        (a test of those branches)                                      */

/*
 * Options of one search.  A NULL pointer, or a zero-initialised struct, selects the defaults.  The
 * workspace size depends on the options: pass the same options to svt_search_workspace_size and
 * svt_search.
 *   path       SVT_PATH_AUTO (default), SVT_PATH_QUERY, SVT_PATH_TILE or SVT_PATH_LARGE_K; with
 *              k > SVT_MAX_K only SVT_PATH_AUTO and SVT_PATH_LARGE_K are accepted
 *   pool_keys  tile path: candidate keys kept per query (0 = default, 16 k rounded up to 4096); large-k
 *              path: the same, default 8 k rounded up to 4096 (no pools when the batch's pools would
 *              exceed 1 GiB); a smaller value makes more pools overflow (their queries are redone, or go
 *              through the digit passes)
 *   flags      OR of SVT_OPT_* above
 *   mask_groups  G in [0, SVT_MAX_MASK_GROUPS]: each query brings G request masks ([B][G][sig_words]) and an
 *              item is eligible when its signature passes at least one of them (a targeting rule set as a
 *              disjunction of conjunctive masks, "Meta Andromeda" summary, System section: the targeting
 *              matcher).  A mask with every bit set passes no item: it pads a query with fewer masks.
 *              0 is the same as 1.
 * Errors (returned by the calls that take the options): SVT_EINVAL for an unknown path, a negative
 * pool_keys, unknown flag bits, mask_groups out of range or non-zero reserved words.
 */
#define SVT_MAX_MASK_GROUPS 4  /* masks per request at most                                            */

typedef struct {
  int32_t path;
  int32_t pool_keys;
  uint32_t flags;
  int32_t mask_groups;   /* masks per query (0 or 1: one); an item is eligible when it passes any of them */
  int32_t reserved[4];   /* must be 0 */
} svt_search_options;

/*
 * svt_search_workspace_size - bytes of device workspace svt_search needs for these sizes and options.
 * Returns 0 if the arguments are invalid (see svt_search; svt_last_error() then says why).  The size
 * never depends on query values.
 */
size_t svt_search_workspace_size(const svt_index *ix, int32_t n_queries, int32_t nprobe, int32_t k,
                                 const svt_search_options *opts);

/*
 * svt_search_path - the path a search with these sizes and options takes: SVT_PATH_QUERY, SVT_PATH_TILE,
 * SVT_PATH_EXHAUSTIVE (the tile path's MFMA scan of the whole catalogue, nprobe == nlist) or
 * SVT_PATH_LARGE_K.  It depends
 * on the index, n_queries, nprobe and the options only, never on query values.  No device work.
 * Errors (negative return): those of svt_search_workspace_size's arguments (SVT_EINVAL, SVT_ESTATE).
 */
int svt_search_path(const svt_index *ix, int32_t n_queries, int32_t nprobe, int32_t k, const svt_search_options *opts);

/*
 * svt_search - batched fused search (steps 1-4 above), asynchronous on hip_stream.
 *   queries       device, [n_queries][dim] int8, row-major, 16-byte aligned
 *   masks         device, [n_queries][G][sig_words] uint64 request masks (see svt_bloom_mask; G = the options'
 *                 mask_groups, 1 by default), 8-byte aligned
 *   query_scales  device, [n_queries] float > 0, or NULL to use the index's item_scale
 *   nprobe        1 <= nprobe <= nlist
 *   k             1 <= k <= SVT_MAX_K_LARGE (above SVT_MAX_K: the large-k path)
 *   out_ids       device, [n_queries][k] int64: item ids, best first; -1 past out_counts[b]
 *   out_scores    device, [n_queries][k] int32: exact int8 dot products; INT32_MIN past the count
 *   out_fscores   device, [n_queries][k] float or NULL: S / (item_scale * query_scale); -inf padding
 *   out_counts    device, [n_queries] int32 or NULL: min(k, number of eligible items in the probed
 *                 clusters)
 *   out_stats     device, [n_queries][2] int64 or NULL: items scanned in the probed clusters, items
 *                 that passed the filter and were scored
 *   opts          search options or NULL (defaults)
 *   workspace     device, at least svt_search_workspace_size(ix, n_queries, nprobe, k, opts) bytes,
 *                 256-byte aligned; contents on entry are ignored, contents on exit are unspecified
 * Result rows are sorted by (score desc, id asc) and identical for any batch composition and path.
 * n_queries == 0 returns SVT_OK without enqueuing anything.
 * Errors: SVT_EINVAL (NULL required pointer, n_queries < 0 or > 65535, nprobe or k out of range,
 * misaligned queries, masks, workspace, outputs or query_scales (each aligned to its element size),
 * workspace too small, invalid options), SVT_ESTATE (freed
 * index), SVT_EDEVICE (launch failure).  On any error nothing is enqueued and no output is written.
 * Concurrency: the index is read-only; concurrent calls are safe if each uses its own workspace and
 * outputs.  Outputs are valid once hip_stream has been synchronised.
 */
int svt_search(const svt_index *ix, int32_t n_queries, const int8_t *queries, const uint64_t *masks,
               const float *query_scales, int32_t nprobe, int32_t k, int64_t *out_ids, int32_t *out_scores,
               float *out_fscores, int32_t *out_counts, int64_t *out_stats, const svt_search_options *opts,
               void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * svt_search_noalloc - svt_search without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, results and errors are those of svt_search; the workspace is a static device array of
 * SVT_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, held until the process ends.
 * The call allocates no device memory: on its first call on a GPU it looks up that GPU's copy of the
 * array (hipGetSymbolAddress), and it records no stage-timing events.
 *   Errors, besides those of svt_search: SVT_EINVAL when this call's svt_search_workspace_size exceeds
 *   SVT_NOALLOC_SCRATCH_BYTES, or when the current device is not the one the index was uploaded on;
 *   SVT_EDEVICE when the array's address cannot be obtained.
 * Concurrency: every call on one GPU uses the same array, which keeps the previous call's contents (the
 * search clears what it needs).  Calls whose executions overlap on one GPU (two streams, two threads
 * or two processes' work in flight at once) race on it and may return wrong results: serialise them,
 * e.g. issue them all on one stream.
 */
#define SVT_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
int svt_search_noalloc(const svt_index *ix, int32_t n_queries, const int8_t *queries, const uint64_t *masks,
                       const float *query_scales, int32_t nprobe, int32_t k, int64_t *out_ids, int32_t *out_scores,
                       float *out_fscores, int32_t *out_counts, int64_t *out_stats, const svt_search_options *opts,
                       void *hip_stream);

/*
 * svt_rerank - re-score each query's retrieved candidates with a small gated mixture of experts over
 * the query-candidate interaction, fused with the fetch of the candidates' rows and the final top-k
 * ["SilverTorch - Index as Model", recommendation-quality section: retrieved candidates re-scored by
 *  neural modules (MLP, mixture of logits, multi-task heads); "Meta Andromeda" summary, System section:
 *  embedding fetch, interaction and scoring in one kernel with intermediates on chip].  The pages give no
 * formula; this library computes, in float32, for query q and candidate row x:
 *   q^ = q / query_scale, x^ = x / item_scale, z = q^ * x^ (elementwise)
 *   g  = softmax(gate_w q^ + gate_b)                      (E experts)
 *   r  = sum_e g_e (w2_e . relu(w1_e z + b1_e) + b2_e)    (hidden width H per expert)
 * and returns the k_out best candidates by (r desc, id asc).
 *   net           host struct of device pointers (float32, row-major): gate_w [E][dim], gate_b [E],
 *                 w1 [E][H][dim], b1 [E][H], w2 [E][H], b2 [E]; 1 <= E <= SVT_RERANK_MAX_EXPERTS,
 *                 H >= 1, E * H <= SVT_RERANK_MAX_UNITS
 *   queries       device, [n_queries][dim] int8 (the search's queries)
 *   query_scales  device, [n_queries] float > 0, or NULL to use the index's item_scale
 *   cand_ids      device, [n_queries][n_cand] int64: the candidates of each query, e.g. svt_search's
 *                 out_ids.  Entries that are negative or not an id present in the index are skipped; a
 *                 repeated id is scored, and may be returned, once per occurrence.
 *   n_cand        0 <= n_cand <= SVT_RERANK_MAX_CAND
 *   k_out         1 <= k_out <= SVT_RERANK_MAX_OUT
 *   out_ids       device, [n_queries][k_out] int64, best first; -1 past out_counts[b]
 *   out_scores    device, [n_queries][k_out] float: r; -inf padding
 *   out_counts    device, [n_queries] int32 or NULL: min(k_out, candidates scored)
 * The index must not be updated while the call runs.  n_queries == 0 returns SVT_OK without enqueuing.
 * Errors: SVT_EINVAL (NULL required pointer, n_queries < 0 or > 65535, n_cand, k_out, E or H out of
 * range, a pointer not aligned to its element size), SVT_ESTATE (freed index), SVT_EDEVICE (launch
 * failure); on error nothing is enqueued.
 * The call allocates no device memory; concurrent calls with their own outputs are safe.
 */
#define SVT_RERANK_MAX_EXPERTS 8
#define SVT_RERANK_MAX_UNITS 64
#define SVT_RERANK_MAX_CAND 4096
#define SVT_RERANK_MAX_OUT 2048
typedef struct {
  int32_t n_experts;   /* E */
  int32_t hidden;      /* H */
  const float *gate_w, *gate_b, *w1, *b1, *w2, *b2;
} svt_rerank_net;
int svt_rerank(const svt_index *ix, int32_t n_queries, const int8_t *queries, const float *query_scales,
               int32_t n_cand, const int64_t *cand_ids, const svt_rerank_net *net, int32_t k_out,
               int64_t *out_ids, float *out_scores, int32_t *out_counts, void *hip_stream);

/* svt_last_error - message of the last failed call on this thread ("" if none). */
const char *svt_last_error(void);

/*
 * svt_bloom_mask - host helper: request mask = OR of the Bloom bits of each required token
 * (Bloom index filter paragraph of "SilverTorch - Index as Model").  Bits of one token: a splitmix64
 * stream (Steele, Lea, Flood, OOPSLA 2014) seeded with the token key; output j < n_hashes selects bit
 * out_j >> (64 - log2(64 * sig_words)); bit b is bit (b & 63) of word (b >> 6).
 *   token_keys host [n_tokens] (n_tokens may be 0: all-zero mask, every item eligible)
 *   out        host [sig_words]
 * Errors: SVT_EINVAL (NULL pointers, n_tokens < 0, n_hashes < 1 or > 16), SVT_EUNSUPPORTED (sig_words).
 */
int svt_bloom_mask(const uint64_t *token_keys, int32_t n_tokens, int32_t n_hashes, int32_t sig_words,
                   uint64_t *out);

/*
 * svt_bloom_sign - host helper: item signatures, each the svt_bloom_mask of the item's tokens
 * (an item receives its compact signature when it is published, same paragraph).
 *   token_keys host [n_items][tokens_per_item]; out host [n_items][sig_words]
 *   n_threads  host threads to use (<= 0: hardware concurrency)
 */
int svt_bloom_sign(const uint64_t *token_keys, int64_t n_items, int32_t tokens_per_item, int32_t n_hashes,
                   int32_t sig_words, uint64_t *out, int32_t n_threads);

/*
 * Stage timing.  While enabled (per process), svt_search records HIP events on hip_stream around its
 * stages (the calling thread keeps up to 100000 searches).  svt_profile_read synchronises on the last
 * recorded event and returns, for each stage in launch order, the elapsed milliseconds summed over every
 * search this thread recorded since the previous read, then forgets them.  Stages:
 *   "coarse"   centroid scores
 *   "select"   top-nprobe per query, stream layout, samples and thresholds, query-path work list
 *   "plan"     tile path: the batch's probed clusters and the queries of each
 *   "scan"     the fused filter -> score -> select kernel of the path taken (k_scan, k_tscan or k_xscan
 *              with its sample pass)
 *   "fallback" tile path: redo of the queries whose pools missed (work list, k_scan, merge)
 *   "merge"    the final top-k per query
 * Stages a path does not run measure only the gap between two event records.
 *   on      0 off (default), 1 every stage (seven event records per search), 2 the scan stage only
 *           (two event records per search; the other stages read 0); any other value: SVT_EINVAL
 *   stage_ms, stage_names  host arrays of max_stages entries (either may be NULL)
 *   n_stages               receives the number of stages (6); n_searches the number of searches summed
 */
int svt_profile_enable(int on);
int svt_profile_read(float *stage_ms, const char **stage_names, int32_t max_stages, int32_t *n_stages,
                     int32_t *n_searches);

#ifdef __cplusplus
}
#endif

#endif /* SVT_H */
