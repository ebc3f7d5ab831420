// svt_largek.hip - searches with k above the fused lists' SVT_MAX_K: an exact top-k by a radix select
// over the eligible items' keys, one digit per pass over the probed clusters, then one pass that keeps
// the k keys at or above the threshold and a sort of those in LDS.
//
// Source: "SilverTorch - Index as Model" (Meta engineering post), the fused Int8 ANN paragraph and the
// compute-cost table: the retrieval kernel supports top-k far beyond the 2048 of GPU FAISS (the
// Spanish page's table row reads "100de miles", taken as hundreds of thousands); the probe, filter and
// score steps are those of the fused search.
//
// Key of an eligible item: (S + 2^23) << 31 | (2^31 - 1 - id), 55 bits.  Its unsigned order is the
// result order, score descending then id ascending, and no key is 0.  The digits are 11 bits wide, from
// bit 44 down: a pass counts, per query, the keys that share the bits fixed so far by their next digit
// (an LDS histogram per workgroup, added to the query's histogram in HBM); k_lk_pick then fixes that
// digit, and a query is done once the digit's bucket is taken whole.  At most 5 passes, usually 2 or 3;
// a pass skips the queries already done.  The collect pass appends every key at or above the
// threshold (exactly min(k, eligible) keys, as keys are distinct) and k_lk_emit sorts them.
//
// Each pass reads the query's probed items again, so the cost is (passes + 1) query-path scans: the
// price of an exact result without per-query storage for all the candidates.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svt.h"
#include "svt_device.h"
#include "svt_internal.h"

namespace svt {

namespace {

constexpr int kLkThreads = 256;
constexpr int kLkEmitThreads = 1024;

__device__ __forceinline__ uint64_t lk_key(int32_t s, int32_t id) {
  return ((uint64_t)(uint32_t)(s + (1 << 23)) << 31) | (uint64_t)(0x7FFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ int32_t lk_score(uint64_t key) { return (int32_t)(key >> 31) - (1 << 23); }
__device__ __forceinline__ int64_t lk_id(uint64_t key) { return (int64_t)(0x7FFFFFFFu - (uint32_t)(key & 0x7FFFFFFFu)); }

__global__ void k_lk_init(int32_t B, int32_t k, Work w) {
  const int64_t n = (int64_t)B * kLkBins;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    w.lk_hist[i] = 0u;
    if (i < B) {
      w.lk_state[i] = LkState{0ull, kLkTopShift, k, 0, 0};
      w.lk_cnt[i] = 0u;
    }
  }
}

struct LkScanArgs {
  DevIndex ix;
  const int8_t *queries;
  const uint64_t *masks;
  Work w;
  int32_t nprobe, k, G;
};

// One workgroup per (chunk of kLkChunk stream positions, query).  COLLECT = false: a counting pass;
// COLLECT = true: append the keys at or above each query's threshold.
template <int D, int W, bool COLLECT>
__global__ __launch_bounds__(kLkThreads) void k_lk_scan(LkScanArgs a) {
  __shared__ uint32_t hist[COLLECT ? 1 : kLkBins];
  const int b = blockIdx.y, tid = threadIdx.x, l = lane_id();
  const LkState st = a.w.lk_state[b];
  if (!COLLECT && st.done) return;
  const int64_t qlen = a.w.qlen[b];
  const int64_t s0 = (int64_t)blockIdx.x * kLkChunk;
  if (s0 >= qlen) return;
  const int64_t s1 = s0 + kLkChunk < qlen ? s0 + kLkChunk : qlen;
  if (!COLLECT) {
    for (int i = tid; i < kLkBins; i += kLkThreads) hist[i] = 0u;
    __syncthreads();
  }
  // the query row and masks in registers
  int4 qv[D / 16];
  const int4 *qr = reinterpret_cast<const int4 *>(a.queries + (size_t)b * D);
#pragma unroll
  for (int i = 0; i < D / 16; ++i) qv[i] = qr[i];
  uint64_t mk[kMaxGroups][W];
#pragma unroll
  for (int g = 0; g < kMaxGroups; ++g)
#pragma unroll
    for (int x = 0; x < W; ++x) mk[g][x] = g < a.G ? a.masks[((size_t)b * a.G + g) * W + x] : 0ull;
  // keys counted: those whose bits above the digit equal the prefix; kept: those >= the threshold
  const int shift = st.shift;
  const uint64_t hi = ~((1ull << (shift + kLkDigit)) - 1ull);
  const uint64_t prefix = st.prefix;
  const int32_t *seg = a.w.seg + (size_t)b * (a.nprobe + 1);
  const int32_t *pb = a.w.pb + (size_t)b * a.nprobe;
  // the probed cluster holding stream position s0: the largest r with seg[r] <= s0
  int lo = 0, up = a.nprobe - 1;
  while (lo < up) {
    const int mid = (lo + up + 1) >> 1;
    if (seg[mid] <= s0) lo = mid; else up = mid - 1;
  }
  uint32_t *cnt = a.w.lk_cnt + b;
  uint64_t *keys = a.w.lk_keys + (size_t)b * a.k;
  for (int r = lo; r < a.nprobe; ++r) {
    const int64_t r0 = seg[r], r1 = seg[r + 1];
    if (r0 >= s1) break;
    const int64_t e0 = r0 > s0 ? r0 : s0, e1 = r1 < s1 ? r1 : s1;
    const int32_t base = pb[r];
    for (int64_t sb = e0; sb < e1; sb += kLkThreads) {   // uniform trip count: ballots see every lane
      const int64_t s = sb + tid;
      bool ok = false;
      uint64_t key = 0ull;
      if (s < e1) {
        const int64_t pos = base + s;
        uint64_t sg[2] = {0ull, 0ull};
#pragma unroll
        for (int x = 0; x < W; ++x) sg[x] = a.ix.sigs[pos * W + x];
        bool any = false;
#pragma unroll
        for (int g = 0; g < kMaxGroups; ++g) {
          bool pass = g < a.G;
#pragma unroll
          for (int x = 0; x < W; ++x) pass = pass && (sg[x] & mk[g][x]) == mk[g][x];
          any = any || pass;
        }
        ok = any && sig_live(sg[0], sg[1], W);
        if (ok) {
          const int4 *xr = reinterpret_cast<const int4 *>(a.ix.items + pos * D);
          int32_t acc = 0;
#pragma unroll
          for (int i = 0; i < D / 16; ++i) {
            const int4 xv = xr[i];
            acc = __builtin_amdgcn_sdot4(xv.x, qv[i].x, acc, false);
            acc = __builtin_amdgcn_sdot4(xv.y, qv[i].y, acc, false);
            acc = __builtin_amdgcn_sdot4(xv.z, qv[i].z, acc, false);
            acc = __builtin_amdgcn_sdot4(xv.w, qv[i].w, acc, false);
          }
          key = lk_key(acc, a.ix.perm[pos]);
        }
      }
      if constexpr (COLLECT) {
        const bool take = ok && key >= prefix;   // prefix: the final threshold (0: every eligible key)
        const uint64_t bal = __ballot(take);
        if (bal) {
          uint32_t at = 0u;
          if (l == 0) at = atomicAdd(cnt, (uint32_t)__popcll(bal));
          at = __shfl(at, 0) + (uint32_t)mbcnt(bal);
          if (take && at < (uint32_t)a.k) keys[at] = key;
        }
      } else {
        if (ok && (key & hi) == prefix) atomicAdd(&hist[(uint32_t)(key >> shift) & (kLkBins - 1)], 1u);
      }
    }
  }
  if (!COLLECT) {
    __syncthreads();
    uint32_t *gh = a.w.lk_hist + (size_t)b * kLkBins;
    for (int i = tid; i < kLkBins; i += kLkThreads)
      if (hist[i]) atomicAdd(&gh[i], hist[i]);
  }
}

// Fix the digit counted by the last pass, one workgroup per query.  Thread t holds bins 8 (255 - t) ..
// 8 (255 - t) + 7, so that the block's prefix sums count the keys in higher buckets.  The histogram is
// cleared for the next pass.
__global__ __launch_bounds__(kLkThreads) void k_lk_pick(int32_t B, Work w) {
  static_assert(kLkBins == 8 * kLkThreads, "8 bins per thread");
  __shared__ int wave_tot[kLkThreads / 64 + 1];
  const int b = blockIdx.x, tid = threadIdx.x;
  LkState *sp = w.lk_state + b;
  const LkState st = *sp;
  if (st.done) return;
  uint32_t *gh = w.lk_hist + (size_t)b * kLkBins;
  const int g = kLkThreads - 1 - tid;
  uint32_t h[8];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = gh[8 * g + i];
    sum += (int)h[i];
  }
  int total;
  int above = block_excl_scan<kLkThreads>(sum, wave_tot, &total);   // keys in the buckets above this thread's
#pragma unroll
  for (int i = 0; i < 8; ++i) gh[8 * g + i] = 0u;
  if (st.shift == kLkTopShift && tid == 0 && w.stats) w.stats[2 * (size_t)b + 1] = total;   // every eligible key
  if (total <= st.need) {
    // first pass with at most k eligible keys: every one of them is kept (threshold 0)
    if (tid == 0) *sp = LkState{0ull, st.shift, st.need, 1, 0};
    return;
  }
  if (above < st.need && above + sum >= st.need) {
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (above + (int)h[i] >= st.need) {
        const int d = 8 * g + i;
        const int rem = st.need - above;
        LkState ns = st;
        ns.prefix = st.prefix | ((uint64_t)d << st.shift);
        if ((int)h[i] == rem || st.shift == 0) {
          ns.done = 1;
        } else {
          ns.shift = st.shift - kLkDigit;
          ns.need = rem;
        }
        *sp = ns;
        break;
      }
      above += (int)h[i];
    }
  }
}

// Sort each query's collected keys (at most k <= SVT_MAX_K_LARGE) in LDS, best first, and write the row.
__global__ __launch_bounds__(kLkEmitThreads) void k_lk_emit(int32_t k, const float *query_scales, float item_scale,
                                                           Work w, int64_t *out_ids, int32_t *out_scores,
                                                           float *out_fscores, int32_t *out_counts) {
  __shared__ uint64_t S[SVT_MAX_K_LARGE];
  const int b = blockIdx.x, tid = threadIdx.x;
  const uint32_t c = w.lk_cnt[b];
  const int n = c < (uint32_t)k ? (int)c : k;
  int P = 1;
  while (P < n) P <<= 1;
  const uint64_t *keys = w.lk_keys + (size_t)b * k;
  for (int i = tid; i < P; i += kLkEmitThreads) S[i] = i < n ? keys[i] : 0ull;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = tid; p < P / 2; p += kLkEmitThreads) {
        const int i = 2 * stride * (p / stride) + p % stride;
        const bool desc = (i & size) == 0;
        const uint64_t x = S[i], y = S[i + stride];
        if (desc ? x < y : x > y) {
          S[i] = y;
          S[i + stride] = x;
        }
      }
      __syncthreads();
    }
  }
  const float qs = query_scales ? query_scales[b] : item_scale;
  const double denom = (double)item_scale * (double)qs;
  for (int i = tid; i < k; i += kLkEmitThreads) {
    const size_t o = (size_t)b * k + i;
    if (i < n) {
      const int32_t sc = lk_score(S[i]);
      out_ids[o] = lk_id(S[i]);
      out_scores[o] = sc;
      if (out_fscores) out_fscores[o] = (float)((double)sc / denom);
    } else {
      out_ids[o] = -1;
      out_scores[o] = INT32_MIN;
      if (out_fscores) out_fscores[o] = -__builtin_huge_valf();
    }
  }
  if (tid == 0 && out_counts) out_counts[b] = n;
}

template <int D, int W>
void lk_scan_launch(const LkScanArgs &a, dim3 grid, bool collect, hipStream_t s) {
  if (collect)
    k_lk_scan<D, W, true><<<grid, kLkThreads, 0, s>>>(a);
  else
    k_lk_scan<D, W, false><<<grid, kLkThreads, 0, s>>>(a);
}

template <int D>
void lk_scan_w(const LkScanArgs &a, dim3 grid, bool collect, hipStream_t s) {
  if (a.ix.sig_words == 2)
    lk_scan_launch<D, 2>(a, grid, collect, s);
  else
    lk_scan_launch<D, 1>(a, grid, collect, s);
}

}  // namespace

hipError_t launch_large_k(const DevIndex &ix, const int8_t *queries, const uint64_t *masks, const float *query_scales,
                          const SearchShape &sh, int64_t max_stream, const Work &w, int64_t *out_ids,
                          int32_t *out_scores, float *out_fscores, int32_t *out_counts, hipStream_t s) {
  const int64_t n_init = (int64_t)sh.B * kLkBins;
  k_lk_init<<<(unsigned)std::min<int64_t>((n_init + 255) / 256, 4096), 256, 0, s>>>(sh.B, sh.k, w);
  const LkScanArgs a{ix, queries, masks, w, sh.nprobe, sh.k, sh.G};
  const int64_t chunks = std::max<int64_t>(1, (max_stream + kLkChunk - 1) / kLkChunk);
  const dim3 grid((unsigned)chunks, (unsigned)sh.B);
  for (int pass = 0; pass <= kLkPasses; ++pass) {
    const bool collect = pass == kLkPasses;
    switch (ix.dim) {
      case 16: lk_scan_w<16>(a, grid, collect, s); break;
      case 32: lk_scan_w<32>(a, grid, collect, s); break;
      case 64: lk_scan_w<64>(a, grid, collect, s); break;
      case 128: lk_scan_w<128>(a, grid, collect, s); break;
      case 256: lk_scan_w<256>(a, grid, collect, s); break;
      default: return hipErrorInvalidValue;
    }
    if (!collect) k_lk_pick<<<sh.B, kLkThreads, 0, s>>>(sh.B, w);
  }
  k_lk_emit<<<sh.B, kLkEmitThreads, 0, s>>>(sh.k, query_scales, ix.item_scale, w, out_ids, out_scores, out_fscores,
                                           out_counts);
  return hipGetLastError();
}

}  // namespace svt
