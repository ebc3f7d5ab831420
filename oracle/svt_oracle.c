/*
 * svt_oracle.c - CPU oracle for the fused int8 IVF + Bloom-signature top-k search.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  The GPU library never links, includes or calls it, and it shares no
 * code with the GPU library (each side has its own splitmix64, its own Bloom bit mapping, its own
 * scoring and selection).
 *
 * Plain, slow, obviously correct: scalar loops, qsort, no SIMD, no blocking, no fusion.  Each step
 * follows the method as the pages state it; where they are silent the reading is named in the
 * comment and listed with the other readings in the design notes.
 *
 * Method, as stated in "SilverTorch - Index as Model" (Meta engineering post; Chinese translation
 * and Spanish machine translation), "How each component worked before" and "The pure-PyTorch
 * decision" sections:
 *   1. coarse: pick the most promising clusters first (IVF probes; the number of probes is a
 *      parameter, e.g. 64);
 *   2. filter only inside those clusters, with a compact per-item Bloom signature checked against
 *      the request by simple bit operations;
 *   3. score only the survivors, int8 item embeddings, int8 dot products with int32 accumulation
 *      ("dp4a", compute-cost-efficiency section);
 *   4. return a large top-k (e.g. top-2048).
 *
 * Parity pins (tests): splitmix64 published outputs; Bloom no-false-negative invariant and the exact
 * false-positive closed form; nprobe = nlist reduces to exhaustive filtered int8 MIPS top-k computed
 * with numpy's library routines; the probe set satisfies the top-nprobe order invariant; tie-heavy
 * inputs pin the id tie-break; dequantisation is checked against exact rational arithmetic.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ORACLE_MUTANT (default 0) plants one deliberate mistake per value; the test suite builds each
 * mutant separately and checks that the pins reject it.  Never set in a normal build.              */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* ---------------------------------------------------------------------------------------------- */
/* splitmix64 (Steele, Lea, Flood, OOPSLA 2014; Vigna's public-domain reference): advance the state
 * by the golden gamma, then apply the variant-13 finaliser.                                         */
uint64_t oracle_splitmix64_next(uint64_t *state) {
  uint64_t z = (*state += 0x9E3779B97F4A7C15ULL);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* ---------------------------------------------------------------------------------------------- */
/* Bloom bits of one token (Bloom index filter paragraph: each item receives a compact signature
 * when it is published).  Reading: a splitmix64 stream seeded with the token key; the j-th output
 * (j < n_hashes) selects bit  out_j >> (64 - log2(64 * sig_words))  of the signature.              */
void oracle_token_bits(uint64_t key, int32_t n_hashes, int32_t sig_words, uint64_t *sig) {
  int32_t m_log2 = (sig_words == 1) ? 6 : (sig_words == 2) ? 7 : (sig_words == 4) ? 8 : 9;
  uint64_t state = key;
  for (int32_t j = 0; j < n_hashes; ++j) {
    uint64_t h = oracle_splitmix64_next(&state);
#if ORACLE_MUTANT == 6
    uint64_t bit = (h >> (64 - m_log2 - 1)) & ((1u << m_log2) - 1);
#else
    uint64_t bit = h >> (64 - m_log2);
#endif
    sig[bit >> 6] |= (uint64_t)1 << (bit & 63);
  }
}

/* item signatures: OR of the bits of each item's tokens                                           */
void oracle_signatures(const uint64_t *tokens, int64_t n_items, int32_t tokens_per_item,
                       int32_t n_hashes, int32_t sig_words, uint64_t *out) {
  for (int64_t i = 0; i < n_items; ++i) {
    uint64_t *s = out + i * sig_words;
    for (int32_t w = 0; w < sig_words; ++w) s[w] = 0;
    for (int32_t t = 0; t < tokens_per_item; ++t)
      oracle_token_bits(tokens[i * tokens_per_item + t], n_hashes, sig_words, s);
  }
}

/* request mask: OR of the bits of the tokens the request requires                                 */
void oracle_mask(const uint64_t *req_tokens, int32_t n_req, int32_t n_hashes, int32_t sig_words,
                 uint64_t *out) {
  for (int32_t w = 0; w < sig_words; ++w) out[w] = 0;
  for (int32_t t = 0; t < n_req; ++t) oracle_token_bits(req_tokens[t], n_hashes, sig_words, out);
}

/* eligibility (Bloom index filter: "simple bit operations"): reading = conjunctive test, every bit
 * of the mask must be set in the signature, over all words                                         */
static int eligible(const uint64_t *sig, const uint64_t *mask, int32_t sig_words) {
#if ORACLE_MUTANT == 2
  for (int32_t w = 0; w < sig_words; ++w)
    if (mask[w] && !(sig[w] & mask[w])) return 0;
  return 1;
#else
  for (int32_t w = 0; w < sig_words; ++w)
    if ((sig[w] & mask[w]) != mask[w]) return 0;
  return 1;
#endif
}

/* int8 . int8 with int32 accumulation ("dp4a" in the compute-cost-efficiency section)              */
static int32_t dot_i8(const int8_t *a, const int8_t *b, int32_t d) {
  int32_t s = 0;
#if ORACLE_MUTANT == 5
  for (int32_t j = 0; j + 1 < d; ++j) s += (int32_t)a[j] * (int32_t)b[j];
#else
  for (int32_t j = 0; j < d; ++j) s += (int32_t)a[j] * (int32_t)b[j];
#endif
  return s;
}

/* ---------------------------------------------------------------------------------------------- */
typedef struct { int32_t score; int64_t id; } cand;

/* order: score descending, then id ascending (reading: the pages give no tie rule; ties go to the
 * lower id, which makes the answer unique)                                                         */
static int cand_cmp(const void *pa, const void *pb) {
  const cand *a = (const cand *)pa, *b = (const cand *)pb;
  if (a->score != b->score) return a->score > b->score ? -1 : 1;
#if ORACLE_MUTANT == 1
  return (a->id > b->id) ? -1 : (a->id < b->id) ? 1 : 0;
#else
  return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;
#endif
}

/* coarse probe (pick the most promising clusters first): all nlist int32 centroid scores, sorted by
 * (score desc, cluster id asc), first nprobe taken.  probes_out receives them in rank order.       */
void oracle_coarse(const int8_t *centroids, int32_t nlist, int32_t dim, const int8_t *q, int32_t nprobe,
                   int32_t *probes_out, int32_t *scores_out) {
  cand *cs = (cand *)malloc(sizeof(cand) * (size_t)nlist);
  for (int32_t c = 0; c < nlist; ++c) {
#if ORACLE_MUTANT == 4
    cs[c].score = -dot_i8(q, centroids + (size_t)c * dim, dim);
#else
    cs[c].score = dot_i8(q, centroids + (size_t)c * dim, dim);
#endif
    cs[c].id = c;
    if (scores_out) scores_out[c] = cs[c].score;
  }
  qsort(cs, (size_t)nlist, sizeof(cand), cand_cmp);
  for (int32_t r = 0; r < nprobe; ++r) probes_out[r] = (int32_t)cs[r].id;
  free(cs);
}

/* dequantisation (reading: the pages are silent; scores map back to float as
 * S / (item_scale * query_scale), computed in double and rounded once to float)                    */
float oracle_dequant(int32_t score, float item_scale, float query_scale) {
#if ORACLE_MUTANT == 7
  return (float)((double)score / (double)item_scale);
#else
  return (float)((double)score / ((double)item_scale * (double)query_scale));
#endif
}

/* ---------------------------------------------------------------------------------------------- */
typedef struct {
  const int8_t *items; const uint64_t *sigs; const int32_t *list_of; int64_t n_items;
  int32_t dim, sig_words;
  const int8_t *centroids; int32_t nlist; float item_scale;
  const int8_t *queries; const uint64_t *masks; const float *query_scales;
  int32_t mask_groups;
  int32_t nprobe, k;
  int64_t *out_ids; int32_t *out_scores; float *out_fscores; int32_t *out_counts; int64_t *out_stats;
  int32_t q0, q1;
} job;

static void search_one(const job *J, int32_t b, char *probed, int32_t *probes, cand **buf, int64_t *cap) {
  const int32_t d = J->dim, W = J->sig_words;
  const int8_t *q = J->queries + (size_t)b * d;
  const int32_t G = J->mask_groups;
  const uint64_t *mask = J->masks + (size_t)b * G * W;   /* G masks of W words */
  /* 1. coarse */
  oracle_coarse(J->centroids, J->nlist, d, q, J->nprobe, probes, NULL);
  memset(probed, 0, (size_t)J->nlist);
#if ORACLE_MUTANT == 3
  for (int32_t r = 0; r + 1 < J->nprobe; ++r) probed[probes[r]] = 1;
#else
  for (int32_t r = 0; r < J->nprobe; ++r) probed[probes[r]] = 1;
#endif
  /* 2 + 3. filter inside the probed clusters, score the survivors */
  int64_t n = 0, scanned = 0;
  for (int64_t i = 0; i < J->n_items; ++i) {
    if (!probed[J->list_of[i]]) continue;
    ++scanned;
    /* a request of several masks (targeting rules, "Meta Andromeda" summary, System section: the
     * targeting matcher): reading = an item is eligible when it passes at least one of them */
    int ok = 0;
#if ORACLE_MUTANT == 8
    for (int32_t g = 0; g < 1 && !ok; ++g) ok = eligible(J->sigs + (size_t)i * W, mask + (size_t)g * W, W);
#else
    for (int32_t g = 0; g < G && !ok; ++g) ok = eligible(J->sigs + (size_t)i * W, mask + (size_t)g * W, W);
#endif
    if (!ok) continue;
    if (n == *cap) {
      *cap = *cap ? *cap * 2 : 4096;
      *buf = (cand *)realloc(*buf, sizeof(cand) * (size_t)*cap);
    }
    (*buf)[n].score = dot_i8(q, J->items + (size_t)i * d, d);
    (*buf)[n].id = i;
    ++n;
  }
  /* 4. top-k by (score desc, id asc) */
  qsort(*buf, (size_t)n, sizeof(cand), cand_cmp);
  int64_t cnt = n < J->k ? n : J->k;
  float qs = J->query_scales ? J->query_scales[b] : J->item_scale;
  for (int32_t r = 0; r < J->k; ++r) {
    size_t o = (size_t)b * J->k + r;
    if (r < cnt) {
      J->out_ids[o] = (*buf)[r].id;
      J->out_scores[o] = (*buf)[r].score;
      if (J->out_fscores) J->out_fscores[o] = oracle_dequant((*buf)[r].score, J->item_scale, qs);
    } else {
      J->out_ids[o] = -1;
      J->out_scores[o] = INT32_MIN;
      if (J->out_fscores) J->out_fscores[o] = -INFINITY;
    }
  }
  if (J->out_counts) J->out_counts[b] = (int32_t)cnt;
  if (J->out_stats) { J->out_stats[2 * (size_t)b] = scanned; J->out_stats[2 * (size_t)b + 1] = n; }
}

static void *search_worker(void *arg) {
  const job *J = (const job *)arg;
  char *probed = (char *)malloc((size_t)J->nlist);
  int32_t *probes = (int32_t *)malloc(sizeof(int32_t) * (size_t)J->nlist);
  cand *buf = NULL;
  int64_t cap = 0;
  for (int32_t b = J->q0; b < J->q1; ++b) search_one(J, b, probed, probes, &buf, &cap);
  free(probed); free(probes); free(buf);
  return NULL;
}

/* Full search for n_queries queries, each with mask_groups masks of sig_words words ([n_queries]
 * [mask_groups][sig_words]); an item is eligible when it passes any of its query's masks.  Outputs
 * [n_queries][k] with padding id -1, score INT32_MIN, fscore -inf past count.  out_stats (nullable)
 * receives per query: items scanned in the probed clusters, eligible items scored.  Queries are split
 * over n_threads threads (no other change).  Returns 0, or -1 on invalid arguments.               */
int oracle_search_groups(const int8_t *items, const uint64_t *sigs, const int32_t *list_of, int64_t n_items,
                         int32_t dim, int32_t sig_words, const int8_t *centroids, int32_t nlist, float item_scale,
                         int32_t n_queries, const int8_t *queries, const uint64_t *masks, int32_t mask_groups,
                         const float *query_scales, int32_t nprobe, int32_t k, int64_t *out_ids,
                         int32_t *out_scores, float *out_fscores, int32_t *out_counts, int64_t *out_stats,
                         int32_t n_threads) {
  if (n_queries < 0 || nprobe < 1 || nprobe > nlist || k < 1 || dim < 1 || sig_words < 1 || mask_groups < 1)
    return -1;
  if (n_queries == 0) return 0;
  int32_t nt = n_threads < 1 ? 1 : n_threads;
  if (nt > n_queries) nt = n_queries;
  job *jobs = (job *)calloc((size_t)nt, sizeof(job));
  pthread_t *th = (pthread_t *)calloc((size_t)nt, sizeof(pthread_t));
  for (int32_t t = 0; t < nt; ++t) {
    job *J = &jobs[t];
    J->items = items; J->sigs = sigs; J->list_of = list_of; J->n_items = n_items;
    J->dim = dim; J->sig_words = sig_words; J->centroids = centroids; J->nlist = nlist;
    J->item_scale = item_scale; J->queries = queries; J->masks = masks; J->query_scales = query_scales;
    J->mask_groups = mask_groups;
    J->nprobe = nprobe; J->k = k; J->out_ids = out_ids; J->out_scores = out_scores;
    J->out_fscores = out_fscores; J->out_counts = out_counts; J->out_stats = out_stats;
    J->q0 = (int32_t)((int64_t)n_queries * t / nt);
    J->q1 = (int32_t)((int64_t)n_queries * (t + 1) / nt);
    pthread_create(&th[t], NULL, search_worker, J);
  }
  for (int32_t t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  free(jobs); free(th);
  return 0;
}

/* The same with one mask per query ([n_queries][sig_words]).                                     */
int oracle_search(const int8_t *items, const uint64_t *sigs, const int32_t *list_of, int64_t n_items,
                  int32_t dim, int32_t sig_words, const int8_t *centroids, int32_t nlist, float item_scale,
                  int32_t n_queries, const int8_t *queries, const uint64_t *masks, const float *query_scales,
                  int32_t nprobe, int32_t k, int64_t *out_ids, int32_t *out_scores, float *out_fscores,
                  int32_t *out_counts, int64_t *out_stats, int32_t n_threads) {
  return oracle_search_groups(items, sigs, list_of, n_items, dim, sig_words, centroids, nlist, item_scale, n_queries,
                              queries, masks, 1, query_scales, nprobe, k, out_ids, out_scores, out_fscores,
                              out_counts, out_stats, n_threads);
}
