// svt_rerank.hip - fused rerank of retrieved candidates on gfx950: fetch each candidate's int8 row, form
// its interaction with the query, score it with a small gated mixture of experts, keep the best.
//
// Score of candidate x for query q (float32 arithmetic):
//   q^ = q / query_scale, x^ = x / item_scale, z = q^ * x^ (elementwise)
//   g = softmax(gate_w q^ + gate_b)                       over the E experts
//   r = sum_e g_e (w2_e . relu(w1_e z + b1_e) + b2_e)     hidden width H per expert
// and the result is the k_out best candidates by (r desc, id asc).
//
// Sources: "SilverTorch - Index as Model" (Meta engineering post), recommendation-quality section: the
// retrieved candidates are re-scored by neural modules (MLP, mixture of logits, multi-task heads);
// "Meta Andromeda" summary, System section: fetching the candidates' embeddings, their interaction with
// the request and the scoring run fused in one kernel, intermediates on chip.  The formula is this
// library's reading; the pages give none.
//
// The first layer is a dense contraction per query: P[c][u] = sum_f x_c[f] * V[u][f] with
// V[u][f] = w1[u][f] * q^[f] / item_scale, over the candidates' raw int8 rows (exact in float32), so it
// runs on the float32 matrix cores (v_mfma_f32_16x16x4_f32, one 16-candidate x 16-unit tile per
// instruction and 4 features).  One workgroup of 1024 threads per query:
//   1. every global read of the set-up is issued before any is waited on: the candidates' ids, then
//      their slots (id -> slot map), w1 and the other weights;
//   2. the candidates present in the index are compacted to the front of an LDS array; V is built in LDS
//      as the B operand of every step (a float4 per lane and step: the 4 unit tiles of the padded 64
//      units); the gate, g_e w2 and sum_e g_e b2 are set once;
//   3. each wave takes 16-candidate tiles: lane (i, k) loads bytes [k d/4, (k + 1) d/4) of candidate i's
//      row (the K order of A and B follows that split) and issues the next tile's loads before the
//      current tile's d/4 x 4 instructions; the epilogue applies b1, relu and g w2 per unit and sums the
//      64 units across lanes;
//   4. the scores become (score, id) keys; a radix select finds the k_out-th largest and the keys above
//      it (and enough equal to it) are compacted;
//   5. they are ordered by rank counting (1 to 4 threads count the keys above each one, no barrier) when
//      at most 1024 remain, else by a bitonic sort in LDS.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "svt.h"
#include "svt_device.h"
#include "svt_internal.h"

namespace svt {

namespace {

#ifndef SVT_RR_THREADS
#define SVT_RR_THREADS 1024
#endif
constexpr int kRThreads = SVT_RR_THREADS;
constexpr int kRWaves = kRThreads / 64;
constexpr int kRUnits = 64;                      // E * H, padded with zero units
constexpr int kRMaxCand = SVT_RERANK_MAX_CAND;
constexpr int kRMaxOut = SVT_RERANK_MAX_OUT;
constexpr int kRMaxExperts = SVT_RERANK_MAX_EXPERTS;
static_assert(SVT_RERANK_MAX_UNITS == kRUnits, "4 unit tiles of 16");
static_assert(kRMaxCand % 16 == 0 && kRMaxCand % kRThreads == 0, "whole tiles, whole thread rows");
constexpr int kRPer = kRMaxCand / kRThreads;      // candidates per thread at most
static_assert(kRMaxOut <= kRMaxCand, "the sort runs in the key array");

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kVbRow = 4 * 64 + 4;

struct RerankArgs {
  DevIndex ix;
  const int8_t *queries;
  const float *query_scales;
  int32_t n_cand;
  const int64_t *cand_ids;
  svt_rerank_net net;
  int32_t k_out;
  int64_t *out_ids;
  float *out_scores;
  int32_t *out_counts;
};

template <int D>
struct RerankLds {
  // step s, lane (j, k): V[16 t + j][k d/4 + s] at vb[s][4 (16 k + j) + t] for the unit tiles t = 0..3,
  // read as one float4.  Plain floats: each is written by its own thread (a store into a vector element
  // would rewrite all four).  Rows padded by 4 floats so that consecutive steps start 4 banks apart.
  alignas(16) float vb[D / 4][kVbRow];
  float v_row[D];               // q^ / item_scale
  float b1[kRUnits], gw2[kRUnits];
  float logit[kRMaxExperts], b2[kRMaxExperts];
  float bg;                     // sum_e g_e b2_e
  union alignas(16) {
    int2 cand[kRMaxCand];       // (slot, id) of each candidate; slot -1: none (also past n_cand)
    uint64_t keys[kRMaxCand];   // (score, id) key of each candidate once scored; 0: none
  };
  SelScratch sel;
  int wave_tot[kRWaves + 1];
};

// float -> uint32 whose unsigned order is the float order (the scores are finite)
__device__ __forceinline__ uint32_t float_order(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_float(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// lane's d/4 bytes of a row: D/16 dwords (zeros for no candidate)
template <int D>
struct RowPart {
  int32_t w[D / 16];
};

template <int D>
__device__ __forceinline__ RowPart<D> load_part(const int8_t *items, int32_t slot, int k) {
  RowPart<D> p;
  if (slot < 0) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) p.w[i] = 0;
    return p;
  }
  const int8_t *src = items + (size_t)slot * D + k * (D / 4);
  if constexpr (D >= 64) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const int4 v = reinterpret_cast<const int4 *>(src)[i];
      p.w[4 * i] = v.x;
      p.w[4 * i + 1] = v.y;
      p.w[4 * i + 2] = v.z;
      p.w[4 * i + 3] = v.w;
    }
  } else if constexpr (D == 32) {
    const int2 v = *reinterpret_cast<const int2 *>(src);
    p.w[0] = v.x;
    p.w[1] = v.y;
  } else {
    p.w[0] = *reinterpret_cast<const int32_t *>(src);
  }
  return p;
}

template <int D>
__global__ __launch_bounds__(kRThreads) void k_rerank(RerankArgs a) {
  __shared__ RerankLds<D> S;
  constexpr int kVPer = kRUnits * D / kRThreads;   // entries of w1 (padded to 64 units) per thread
  static_assert((kRUnits * D) % kRThreads == 0, "whole rows of w1 per pass");
  const int b = blockIdx.x, tid = threadIdx.x, l = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
  const int E = a.net.n_experts, H = a.net.hidden, U = E * H;
  const int n_cand = a.n_cand;
  const float iscale = a.ix.item_scale;
  const float qscale = a.query_scales ? a.query_scales[b] : iscale;
  // 1. every global read of the set-up in flight together: the candidates' ids, then their slots;
  //    the weights; q^ / item_scale and the gate logits
  const int64_t *cids = a.cand_ids + (size_t)b * n_cand;
  int64_t id[kRPer];
#pragma unroll
  for (int u = 0; u < kRPer; ++u) {
    const int c = u * kRThreads + tid;
    id[u] = c < n_cand ? cids[c] : -1;
  }
  float w[kVPer];   // w1 entry i (unit i / d, feature i % d; coalesced)
#pragma unroll
  for (int j = 0; j < kVPer; ++j) {
    const int i = j * kRThreads + tid;
    w[j] = i / D < U ? a.net.w1[i] : 0.f;
  }
  int32_t slot[kRPer];
  int n_mine = 0;
#pragma unroll
  for (int u = 0; u < kRPer; ++u) {
    slot[u] = (id[u] >= 0 && id[u] < a.ix.n_ids) ? a.ix.slot_of[id[u]] : -1;
    n_mine += slot[u] >= 0 ? 1 : 0;
  }
  const int8_t *q = a.queries + (size_t)b * D;
  for (int f = tid; f < D; f += kRThreads) S.v_row[f] = ((float)q[f] / qscale) / iscale;
  if (tid < kRUnits) {
    S.b1[tid] = tid < U ? a.net.b1[tid] : 0.f;
    S.gw2[tid] = tid < U ? a.net.w2[tid] : 0.f;   // times g of the unit's expert below
  }
  if (wv < E) {   // wave e: logit e = gate_w[e] . q^ + gate_b[e]
    float s = 0.f;
    for (int f = l; f < D; f += 64) s = fmaf(a.net.gate_w[(size_t)wv * D + f], (float)q[f] / qscale, s);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (l == 0) {
      S.logit[wv] = s + a.net.gate_b[wv];
      S.b2[wv] = a.net.b2[wv];
    }
  }
  // 2. the candidates present in the index, compacted to the front (any order: keys carry the ids)
  int n_valid;
  int pos = block_excl_scan<kRThreads>(n_mine, S.wave_tot, &n_valid);   // barriers inside
#pragma unroll
  for (int u = 0; u < kRPer; ++u)
    if (slot[u] >= 0) S.cand[pos++] = make_int2(slot[u], (int32_t)id[u]);
  const int n_tiles = (n_valid + 15) / 16;
  if (tid < 16 * n_tiles - n_valid) S.cand[n_valid + tid] = make_int2(-1, -1);
  // V in the B-operand layout; units past U are zero
#pragma unroll
  for (int j = 0; j < kVPer; ++j) {
    const int i = j * kRThreads + tid;
    const int u = i / D, f = i % D;
    const int k = f / (D / 4), s = f % (D / 4), t = u / 16, jj = u % 16;
    S.vb[s][4 * (16 * k + jj) + t] = w[j] * S.v_row[f];
  }
  // the gate: softmax of the logits (each of the first 64 threads, for its unit)
  if (tid < kRUnits) {
    float mx = S.logit[0];
    for (int e = 1; e < E; ++e) mx = fmaxf(mx, S.logit[e]);
    float sum = 0.f, bg = 0.f;
    for (int e = 0; e < E; ++e) {
      const float ge = expf(S.logit[e] - mx);
      sum += ge;
      bg = fmaf(ge, S.b2[e], bg);
    }
    const float inv = 1.f / sum;
    if (tid < U) S.gw2[tid] = (expf(S.logit[tid / H] - mx) * inv) * S.gw2[tid];
    if (tid == 0) S.bg = bg * inv;
  }
  __syncthreads();
  // 3. the tiles of this wave
  const int i_row = l % 16, k_part = l / 16;
  const float bg = S.bg;
  float b1v[4], gw2v[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    b1v[t] = S.b1[16 * t + i_row];
    gw2v[t] = S.gw2[16 * t + i_row];
  }
  int tile = wv;
  RowPart<D> next{};
  if (tile < n_tiles) next = load_part<D>(a.ix.items, S.cand[16 * tile + i_row].x, k_part);
  for (; tile < n_tiles; tile += kRWaves) {
    const RowPart<D> cur = next;
    const int tn = tile + kRWaves;
    if (tn < n_tiles) next = load_part<D>(a.ix.items, S.cand[16 * tn + i_row].x, k_part);
    f32x4 acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 4; ++s) {
      const float x = (float)(int8_t)(cur.w[s / 4] >> (8 * (s % 4)));
      const f32x4 v = *reinterpret_cast<const f32x4 *>(&S.vb[s][4 * l]);
#pragma unroll
      for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, v[t], acc[t], 0, 0, 0);
    }
    // lane (j, k) holds P[candidate 4 k + r][unit 16 t + j]
    float part[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sacc = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) sacc = fmaf(gw2v[t], fmaxf(acc[t][r] + b1v[t], 0.f), sacc);
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) sacc += __shfl_xor(sacc, off);
      part[r] = sacc;
    }
    if (i_row == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int c = 16 * tile + 4 * k_part + r;
        const int2 e = S.cand[c];
        S.keys[c] = e.x >= 0
                        ? ((uint64_t)float_order(part[r] + bg) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e.y)
                        : 0ull;
      }
    }
  }
  __syncthreads();
  // 4. the k_out best keys of keys[0 .. n_valid)
  const int k_out = a.k_out;
  const int nout = n_valid < k_out ? n_valid : k_out;
  uint64_t T = 0ull;   // keep keys > T, then keys == T up to k_out (T = 0: every key)
  if (n_valid > k_out)
    T = block_select<kRThreads>(
        [&](auto f) {
          for (int i = tid; i < n_valid; i += kRThreads) f(S.keys[i]);
        },
        k_out, S.sel);
  uint64_t mine[kRPer];
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int u = 0; u < kRPer; ++u) {
    const int i = u * kRThreads + tid;
    mine[u] = i < n_valid ? S.keys[i] : 0ull;
    n_gt += mine[u] > T ? 1 : 0;
    n_eq += (T != 0ull && mine[u] == T) ? 1 : 0;
  }
  int tot;
  const int off = block_excl_scan<kRThreads>(n_gt | (n_eq << 16), S.wave_tot, &tot);   // barriers inside
  int o_gt = off & 0xFFFF, o_eq = off >> 16;
  const int tot_gt = tot & 0xFFFF;
#pragma unroll
  for (int u = 0; u < kRPer; ++u) {
    if (mine[u] > T) {
      S.keys[o_gt++] = mine[u];
    } else if (T != 0ull && mine[u] == T) {
      if (tot_gt + o_eq < nout) S.keys[tot_gt + o_eq] = mine[u];
      ++o_eq;
    }
  }
  __syncthreads();
  // 5. order the nout kept keys (descending) and write them
  const size_t ob = (size_t)b * k_out;
  if (nout <= kRThreads) {
    // rank of each key: the keys above it, and the equal ones stored before it (repeated ids); tpk
    // adjacent lanes share a key, each counting over its own slice of the keys
    const int tpk = nout <= kRThreads / 4 ? 4 : nout <= kRThreads / 2 ? 2 : 1;
    if (wv * 64 < nout * tpk) {
      const int i = tid / tpk, part = tid % tpk;
      const uint64_t my = i < nout ? S.keys[i] : 0ull;
      auto above = [&](uint64_t kj, int j) { return (kj > my || (kj == my && j < i)) ? 1 : 0; };
      const int len = (((nout + tpk - 1) / tpk) + 7) & ~7;   // slice length, a multiple of 8
      const int j0 = part * len, j1 = min(nout, j0 + len);
      int rank = 0, j = j0;
      for (; j + 8 <= j1; j += 8) {   // 8 keys per round, their reads in flight together
        const ulonglong2 *k2 = reinterpret_cast<const ulonglong2 *>(&S.keys[j]);
        const ulonglong2 x0 = k2[0], x1 = k2[1], x2 = k2[2], x3 = k2[3];
        rank += above(x0.x, j) + above(x0.y, j + 1) + above(x1.x, j + 2) + above(x1.y, j + 3) +
                above(x2.x, j + 4) + above(x2.y, j + 5) + above(x3.x, j + 6) + above(x3.y, j + 7);
      }
      for (; j < j1; ++j) rank += above(S.keys[j], j);
      for (int o = 1; o < tpk; o <<= 1) rank += __shfl_xor(rank, o);
      if (i < nout && part == 0) {
        a.out_ids[ob + rank] = (int64_t)(0xFFFFFFFFu - (uint32_t)my);
        a.out_scores[ob + rank] = order_float((uint32_t)(my >> 32));
      }
    }
  } else {
    // bitonic sort, padded with zero keys to a power of two
    int P = 1;
    while (P < nout) P <<= 1;
    for (int i = nout + tid; i < P; i += kRThreads) S.keys[i] = 0ull;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int p = tid; p < P / 2; p += kRThreads) {
          const int i = 2 * stride * (p / stride) + p % stride;
          const bool desc = (i & size) == 0;
          const uint64_t x = S.keys[i], y = S.keys[i + stride];
          if (desc ? x < y : x > y) {
            S.keys[i] = y;
            S.keys[i + stride] = x;
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < nout; i += kRThreads) {
      const uint64_t key = S.keys[i];
      a.out_ids[ob + i] = (int64_t)(0xFFFFFFFFu - (uint32_t)key);
      a.out_scores[ob + i] = order_float((uint32_t)(key >> 32));
    }
  }
  for (int i = nout + tid; i < k_out; i += kRThreads) {
    a.out_ids[ob + i] = -1;
    a.out_scores[ob + i] = -INFINITY;
  }
  if (tid == 0 && a.out_counts) a.out_counts[b] = nout;
}

}  // namespace

hipError_t launch_rerank(const DevIndex &ix, int32_t B, const int8_t *queries, const float *query_scales,
                         int32_t n_cand, const int64_t *cand_ids, const svt_rerank_net &net, int32_t k_out,
                         int64_t *out_ids, float *out_scores, int32_t *out_counts, hipStream_t s) {
  const RerankArgs a{ix, queries, query_scales, n_cand, cand_ids, net, k_out, out_ids, out_scores, out_counts};
  switch (ix.dim) {
    case 16: k_rerank<16><<<B, kRThreads, 0, s>>>(a); break;
    case 32: k_rerank<32><<<B, kRThreads, 0, s>>>(a); break;
    case 64: k_rerank<64><<<B, kRThreads, 0, s>>>(a); break;
    case 128: k_rerank<128><<<B, kRThreads, 0, s>>>(a); break;
    case 256: k_rerank<256><<<B, kRThreads, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svt
