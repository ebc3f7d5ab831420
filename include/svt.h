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
 *     4. select: the k best eligible items by (score desc, item id asc), k <= 2048, kept on chip and
 *        merged; only the final candidates are written out
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
  SVT_ESTATE = -5        /* object in the wrong state (freed or foreign index)                       */
};

#define SVT_MAX_K 2048        /* largest top-k per query                                            */
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

/* svt_index_free - release an index and its device memory (synchronises the device first).
 * NULL is accepted (no-op).  SVT_ESTATE if ix is not a live index from svt_index_upload. */
int svt_index_free(svt_index *ix);

/* svt_index_info - shape of an uploaded index; any output pointer may be NULL. */
int svt_index_info(const svt_index *ix, int64_t *n_items, int32_t *dim, int32_t *sig_words, int32_t *nlist);

/*
 * svt_search_workspace_size - bytes of device workspace svt_search needs for these sizes.
 * Returns 0 if the arguments are invalid (see svt_search).  The size never depends on query values.
 */
size_t svt_search_workspace_size(const svt_index *ix, int32_t n_queries, int32_t nprobe, int32_t k);

/*
 * svt_search - batched fused search (steps 1-4 above), asynchronous on hip_stream.
 *   queries       device, [n_queries][dim] int8, row-major
 *   masks         device, [n_queries][sig_words] uint64 request masks (see svt_bloom_mask)
 *   query_scales  device, [n_queries] float > 0, or NULL to use the index's item_scale
 *   nprobe        1 <= nprobe <= nlist
 *   k             1 <= k <= SVT_MAX_K
 *   out_ids       device, [n_queries][k] int64: item ids, best first; -1 past out_counts[b]
 *   out_scores    device, [n_queries][k] int32: exact int8 dot products; INT32_MIN past the count
 *   out_fscores   device, [n_queries][k] float or NULL: S / (item_scale * query_scale); -inf padding
 *   out_counts    device, [n_queries] int32 or NULL: min(k, number of eligible items in the probed
 *                 clusters)
 *   out_stats     device, [n_queries][2] int64 or NULL: items scanned in the probed clusters, items
 *                 that passed the filter and were scored
 *   workspace     device, at least svt_search_workspace_size(ix, n_queries, nprobe, k) bytes, 256-byte
 *                 aligned; contents on entry are ignored, contents on exit are unspecified
 * Result rows are sorted by (score desc, id asc) and identical for any batch composition.
 * n_queries == 0 returns SVT_OK without enqueuing anything.
 * Errors: SVT_EINVAL (NULL required pointer, n_queries < 0 or > 65535, nprobe or k out of range,
 * workspace too small or misaligned), SVT_ESTATE (freed index), SVT_EDEVICE (launch failure).
 * Concurrency: the index is read-only; concurrent calls are safe if each uses its own workspace and
 * outputs.  Outputs are valid once hip_stream has been synchronised.
 */
int svt_search(const svt_index *ix, int32_t n_queries, const int8_t *queries, const uint64_t *masks,
               const float *query_scales, int32_t nprobe, int32_t k, int64_t *out_ids, int32_t *out_scores,
               float *out_fscores, int32_t *out_counts, int64_t *out_stats, void *workspace,
               size_t workspace_bytes, void *hip_stream);

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
 * recorded event and returns, for each stage in launch order ("coarse", "select", "plan", "scan",
 * "fallback", "merge"), the elapsed milliseconds summed over every search this thread recorded since
 * the previous read, then forgets them.  "plan" and "fallback" hold work only on the grouped path (set
 * by the environment variable SVT_PATH=grouped; SVT_PATH=query forces the query-by-query path); on the
 * query-by-query path they measure only the gap between two event records.
 *   on      0 off (default), 1 every stage (seven event records per search), 2 the scan stage only
 *           (two event records per search; the other stages read 0); any other value: SVT_EINVAL
 *   stage_ms, stage_names  host arrays of max_stages entries (either may be NULL)
 *   n_stages               receives the number of stages (6); n_searches the number of searches summed
 */
int svt_profile_enable(int on);
/*
 * Environment variables read by svt_search on every call (tests use them to force rare paths):
 *   SVT_PATH=query|grouped   the search path (default query)
 *   SVT_POOL_CAP=n           grouped path: at most n candidate keys per query pool (overflow -> rescan)
 *   SVT_GATHER_CAP=n         query path: at most n keys gathered per query for the merge (more -> the
 *                            merge reads the chunks' slots)
 */
int svt_profile_read(float *stage_ms, const char **stage_names, int32_t max_stages, int32_t *n_stages,
                     int32_t *n_searches);

#ifdef __cplusplus
}
#endif

#endif /* SVT_H */
