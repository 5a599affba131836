// Verification of D drafts against D+1 target rows: greedy prefix match and speculative
// sampling after temperature, top-k and top-p.
//
// Sources: [HB14] "14. MTP: speculative decoding with the built-in draft head", the speculative
// loop of section "The draft head" (verify two positions, accept the guess and the next token on
// a hit); [DLM] "The decoding loop and MTP", items 2-3 (7 distributions checked in order, the
// first refused guess replaced by the model's pick, one more token when all hold, a guess kept
// with its post-warp probability, otherwise a draw from the other candidates; temperature, top-k
// and top-p applied in turn); [YL] "MTP 原理详解" 三 stages 3-4 (accept when P/Q >= U, resample
// on rejection, 1..D+1 tokens per round).
//
// Each verifier is a short chain of kernels: workgroups scan chunks of every row, then rows are
// merged, then one workgroup per sequence takes the sequence's decisions.
#include <float.h>

#include "common.h"
#include "verify.h"

namespace mtp {

// workgroup argmax (value desc, index asc) of one value per thread
__device__ __forceinline__ void wg_argmax(float& v, int& i, float* sv, int* si) {
  wave_argmax(v, i);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wid] = v;
    si[wid] = i;
  }
  __syncthreads();
  v = sv[0];
  i = si[0];
#pragma unroll
  for (int w = 1; w < 4; ++w)
    if (better(sv[w], si[w], v, i)) {
      v = sv[w];
      i = si[w];
    }
  __syncthreads();
}

// ---------------------------------------------------------------------------------------------
// greedy
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(kWG) void k_verify_greedy(VerifyArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int c = blockIdx.x, row = blockIdx.y;
  const float* x = a.tl + (long)row * a.V;
  const int beg = c * a.chunk, end = min(a.V, beg + a.chunk);
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  if ((a.V & 3) == 0) {
    for (int k = beg + 4 * threadIdx.x; k < end; k += 4 * kWG) {
      const uint4 u = ld_stream(x + k);
      const float f[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (better(f[e], k + e, bv, bi)) {
          bv = f[e];
          bi = k + e;
        }
    }
  } else {
    for (int k = beg + threadIdx.x; k < end; k += kWG)
      if (better(x[k], k, bv, bi)) {
        bv = x[k];
        bi = k;
      }
  }
  wg_argmax(bv, bi, sv, si);
  if (threadIdx.x == 0) {
    a.part_v[(long)row * a.nchunk + c] = bv;
    a.part_i[(long)row * a.nchunk + c] = bi;
  }
}

// one workgroup per sequence: argmax of each of its D+1 rows, then the prefix match
__global__ __launch_bounds__(kWG) void k_verify_greedy_final(VerifyArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ int st[kMaxDraft + 1];
  const int b = blockIdx.x, rows_per_seq = a.D + 1;
  for (int j = 0; j < rows_per_seq; ++j) {
    const long row = (long)b * rows_per_seq + j;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int k = threadIdx.x; k < a.nchunk; k += kWG) {
      const float v = a.part_v[row * a.nchunk + k];
      const int i = a.part_i[row * a.nchunk + k];
      if (better(v, i, bv, bi)) {
        bv = v;
        bi = i;
      }
    }
    wg_argmax(bv, bi, sv, si);
    if (threadIdx.x == 0) st[j] = bi;
  }
  if (threadIdx.x == 0) {
    const int* d = a.drafts + (long)b * a.D;
    int n = 0;
    while (n < a.D && st[n] == d[n]) ++n;
    int32_t* out = a.out + (long)b * rows_per_seq;
    for (int j = 0; j < n; ++j) out[j] = d[j];
    out[n] = st[n];
    for (int j = n + 1; j < rows_per_seq; ++j) out[j] = -1;
    a.n_accept[b] = n;
    a.crop[b] = a.ctx_len[b] + 1 + n;
  }
}

// ---------------------------------------------------------------------------------------------
// sampling: top-k selection
// ---------------------------------------------------------------------------------------------
// LDS of the top-k pass: the candidate buffer and the per-thread maxima.
struct TopkSmem {
  float v[kTopCap];
  int i[kTopCap];
  float tm[kWG];
  float v2[kTopSmall];  // second-level candidates of the final selection
  int i2[kTopSmall];
  int cnt, cnt2;
};

// bitonic sort of n (power of two <= kTopCap) (v, i) pairs in LDS, best first
__device__ void bitonic_sort_pairs(float* v, int* id, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = threadIdx.x; t < n; t += kWG) {
        const int p = t ^ j;
        if (p > t) {
          const bool first_best = (t & k) == 0;  // this half ends best-first
          const bool p_better = better(v[p], id[p], v[t], id[t]);
          if (p_better == first_best) {
            const float tv = v[t];
            v[t] = v[p];
            v[p] = tv;
            const int ti = id[t];
            id[t] = id[p];
            id[p] = ti;
          }
        }
      }
      __syncthreads();
    }
  }
}

// bitonic sort of kWG floats (one per thread), descending
__device__ void bitonic_sort_desc(float* v) {
  const int t = threadIdx.x;
  for (int k = 2; k <= kWG; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int p = t ^ j;
      if (p > t) {
        const bool desc = (t & k) == 0;
        if ((v[p] > v[t]) == desc) {
          const float tv = v[t];
          v[t] = v[p];
          v[p] = tv;
        }
      }
      __syncthreads();
    }
  }
}

// Warped distribution of one row from its sorted top-k candidates: probabilities of the kept
// prefix (temperature softmax over the k candidates, then top-p: a candidate stays while the
// mass ranked before it is below p; the first always stays), renormalised.  Runs on one thread.
__device__ int warp_row(const float* tv, int n, float T, float top_p, float* prob) {
  float S = 0.f;
  for (int k = 0; k < n; ++k) {
    prob[k] = expf((tv[k] - tv[0]) / T);
    S += prob[k];
  }
  int m = n;
  if (top_p < 1.f) {
    float before = 0.f;
    m = 0;
    for (int k = 0; k < n; ++k) {
      const float pk = prob[k] / S;
      if (k > 0 && !(before < top_p)) break;
      before += pk;
      ++m;
    }
  }
  float Z = 0.f;
  for (int k = 0; k < m; ++k) Z += prob[k];
  for (int k = 0; k < m; ++k) prob[k] = prob[k] / Z;
  return m;
}

__device__ float lookup(const int* ids, const float* prob, int m, int tok) {
  for (int k = 0; k < m; ++k)
    if (ids[k] == tok) return prob[k];
  return 0.f;
}

// Inverse-CDF draw over (id, weight) pairs in ascending id order: the smallest id whose
// cumulative weight exceeds u * total.  Sorts the pairs by id in place.
__device__ int draw_ascending(int* ids, float* w, int m, float u) {
  for (int a = 1; a < m; ++a) {  // insertion sort by id (m <= 128)
    const int ki = ids[a];
    const float kw = w[a];
    int b = a - 1;
    while (b >= 0 && ids[b] > ki) {
      ids[b + 1] = ids[b];
      w[b + 1] = w[b];
      --b;
    }
    ids[b + 1] = ki;
    w[b + 1] = kw;
  }
  float S = 0.f;
  for (int k = 0; k < m; ++k) S += w[k];
  const float t = u * S;
  float c = 0.f;
  int last = -1;
  for (int k = 0; k < m; ++k) {
    if (w[k] <= 0.f) continue;
    c += w[k];
    last = ids[k];
    if (c > t) return ids[k];
  }
  return last;  // u * S rounded onto S
}

// One workgroup per row streams the row once.  Items at or above a threshold are appended to an
// LDS candidate buffer; the threshold starts as the K-th largest of the per-thread maxima of the
// first tile (K threads hold an item at least that large, so it never exceeds the row's K-th
// best) and rises to the K-th best candidate whenever the buffer has to be compacted.  At the
// end the candidates are sorted (value desc, id asc) and the first K written.
constexpr int kTile = kWG * 16;  // items per tile: four float4 per thread

// Item e of tile `base` for thread t: ids base + 4 (t + kWG q) + r, e = 4 q + r.
__device__ __forceinline__ void load_tile(const float* x, int V, int base, bool vec, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k0 = base + 4 * (threadIdx.x + kWG * q);
    if (vec && k0 + 3 < V) {
      const float4 f = *reinterpret_cast<const float4*>(x + k0);
      v[4 * q] = f.x;
      v[4 * q + 1] = f.y;
      v[4 * q + 2] = f.z;
      v[4 * q + 3] = f.w;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * q + r] = k0 + r < V ? x[k0 + r] : -INFINITY;
    }
  }
}

// Sort the S buffered candidates (padded to a power of two) best first; keeps the first `keep`.
__device__ int sort_candidates(TopkSmem& sm, int S, int keep) {
  int n2 = 1;
  while (n2 < S) n2 <<= 1;
  for (int t = S + threadIdx.x; t < n2; t += kWG) {
    sm.v[t] = -INFINITY;
    sm.i[t] = 0x7fffffff;
  }
  __syncthreads();
  bitonic_sort_pairs(sm.v, sm.i, n2);
  return min(keep, S);
}

__global__ __launch_bounds__(kWG) void k_topk_stream(VerifyArgs a) {
  __shared__ TopkSmem sm;
  const int row = blockIdx.x, K = a.top_k, V = a.V;
  const int tgt_rows = a.B * (a.D + 1);
  const float* x = row < tgt_rows ? a.tl + (long)row * V : a.dl + (long)(row - tgt_rows) * V;
  const bool vec = (reinterpret_cast<uintptr_t>(x) & 15) == 0;
  float cur[16], nxt[16];
  load_tile(x, V, 0, vec, cur);
  {  // threshold from the first tile
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, cur[e]);
    sm.tm[threadIdx.x] = tmax;
    if (threadIdx.x == 0) sm.cnt = 0;
    __syncthreads();
    bitonic_sort_desc(sm.tm);
  }
  float theta = sm.tm[K - 1];
  // Append the tile's items at or above the threshold, then compact if the next tile might not
  // fit in the buffer.  Tiles alternate between two register buffers, so the next tile's loads
  // stay in flight while this one is filtered.
  auto filter = [&](const float (&v)[16], int base) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int k = base + 4 * (threadIdx.x + kWG * (e >> 2)) + (e & 3);
      if (k < V && v[e] >= theta) {
        const int pos = atomicAdd(&sm.cnt, 1);
        sm.v[pos] = v[e];
        sm.i[pos] = k;
      }
    }
    __syncthreads();
    const int S = sm.cnt;
    __syncthreads();  // every thread has read the count before the next tile appends
    if (S > kTopCap - kTile && base + kTile < V) {
      const int n = sort_candidates(sm, S, K);
      if (n == K) theta = sm.v[K - 1];
      __syncthreads();
      if (threadIdx.x == 0) sm.cnt = n;
      __syncthreads();
    }
  };
  for (int base = 0; base < V; base += 2 * kTile) {
    if (base + kTile < V) load_tile(x, V, base + kTile, vec, nxt);
    filter(cur, base);
    if (base + kTile >= V) break;
    if (base + 2 * kTile < V) load_tile(x, V, base + 2 * kTile, vec, cur);
    filter(nxt, base + kTile);
  }
  // Final selection.  The K-th largest of the per-thread maxima over the S candidates bounds
  // the K-th best from below again; the few candidates at or above it are ranked by counting
  // (rank = candidates ranked before it, value desc, id asc) straight into their output slots.
  // If too many remain (ties), the whole buffer is sorted instead.
  const int S = sm.cnt;
  float* ov = a.top_v + (long)row * K;
  int* oi = a.top_i + (long)row * K;
  float tmax = -INFINITY;
  for (int c = threadIdx.x; c < S; c += kWG) tmax = fmaxf(tmax, sm.v[c]);
  sm.tm[threadIdx.x] = tmax;
  if (threadIdx.x == 0) sm.cnt2 = 0;
  __syncthreads();
  bitonic_sort_desc(sm.tm);
  const float theta2 = sm.tm[K - 1];
  for (int c = threadIdx.x; c < S; c += kWG)
    if (sm.v[c] >= theta2) {
      const int pos = atomicAdd(&sm.cnt2, 1);
      if (pos < kTopSmall) {
        sm.v2[pos] = sm.v[c];
        sm.i2[pos] = sm.i[c];
      }
    }
  __syncthreads();
  const int S2 = sm.cnt2;
  int n;
  if (S2 <= kTopSmall) {
    n = min(K, S2);
    for (int c = threadIdx.x; c < S2; c += kWG) {
      const float cv = sm.v2[c];
      const int ci = sm.i2[c];
      int r = 0;
      for (int d = 0; d < S2; ++d) r += better(sm.v2[d], sm.i2[d], cv, ci) ? 1 : 0;
      if (r < K) {
        ov[r] = cv;
        oi[r] = ci;
      }
    }
  } else {
    n = sort_candidates(sm, S, K);
    for (int t = threadIdx.x; t < n; t += kWG) {
      ov[t] = sm.v[t];
      oi[t] = sm.i[t];
    }
  }
  for (int t = n + threadIdx.x; t < K; t += kWG) {
    ov[t] = -INFINITY;
    oi[t] = -1;
  }
  if (threadIdx.x == 0) a.top_n[row] = n;
}

// one workgroup per sequence (one thread does the work): accept / reject / draw
__global__ __launch_bounds__(64) void k_sample_decide(VerifyArgs a) {
  const int b = blockIdx.x;
  const int K = a.top_k;
  const int tgt_rows = a.B * (a.D + 1);
  __shared__ float P[kMaxTopK], Q[kMaxTopK], w[kMaxTopK];  // probabilities, draft probs, residual
  __shared__ int ids[kMaxTopK];
  if (threadIdx.x != 0) return;
  // ---- the sequence's decision, one thread, working in LDS ----
  const float T = a.temperature;
  int32_t* out = a.out + (long)b * (a.D + 1);
  int n_acc = 0;
  int tok = -1;
  for (int j = 0; j < a.D; ++j) {
    const int tr = b * (a.D + 1) + j;
    const float* tv = a.top_v + (long)tr * K;
    const int* ti = a.top_i + (long)tr * K;
    const int mP = warp_row(tv, a.top_n[tr], T, a.top_p, P);
    const int d = a.drafts[(long)b * a.D + j];
    const float Pd = lookup(ti, P, mP, d);
    float Qd = 1.f;
    int mQ = 0;
    const int* qi = nullptr;
    if (a.q_mode == 1) {
      const int dr = tgt_rows + b * a.D + j;
      qi = a.top_i + (long)dr * K;
      mQ = warp_row(a.top_v + (long)dr * K, a.top_n[dr], T, a.top_p, Q);
      Qd = lookup(qi, Q, mQ, d);
    }
    const float u = a.u_accept[(long)b * a.D + j];
    const bool accept = Pd > 0.f && (Qd == 0.f || u <= Pd / Qd);
    if (accept) {
      out[j] = d;
      ++n_acc;
      continue;
    }
    // residual max(0, P - Q); its support lies inside P's kept set
    float rs = 0.f;
    for (int k = 0; k < mP; ++k) {
      ids[k] = ti[k];
      const float q = a.q_mode == 1 ? lookup(qi, Q, mQ, ti[k]) : (ti[k] == d ? 1.f : 0.f);
      w[k] = fmaxf(P[k] - q, 0.f);
      rs += w[k];
    }
    if (!(rs > 0.f))
      for (int k = 0; k < mP; ++k) w[k] = P[k];
    tok = draw_ascending(ids, w, mP, a.u_sample[b]);
    break;
  }
  if (tok < 0) {  // every draft held: one more token from row D
    const int tr = b * (a.D + 1) + a.D;
    const int mP = warp_row(a.top_v + (long)tr * K, a.top_n[tr], T, a.top_p, P);
    for (int k = 0; k < mP; ++k) {
      ids[k] = a.top_i[(long)tr * K + k];
      w[k] = P[k];
    }
    tok = draw_ascending(ids, w, mP, a.u_sample[b]);
  }
  out[n_acc] = tok;
  for (int j = n_acc + 1; j <= a.D; ++j) out[j] = -1;
  a.n_accept[b] = n_acc;
  a.crop[b] = a.ctx_len[b] + 1 + n_acc;
}

hipError_t run_verify(const VerifyArgs& a, hipStream_t st) {
  if (a.greedy) {
    hipLaunchKernelGGL(k_verify_greedy, dim3(a.nchunk, a.B * (a.D + 1)), dim3(kWG), 0, st, a);
    hipLaunchKernelGGL(k_verify_greedy_final, dim3(a.B), dim3(kWG), 0, st, a);
  } else {
    const int rows = a.B * (a.D + 1) + (a.q_mode == 1 ? a.B * a.D : 0);
    hipLaunchKernelGGL(k_topk_stream, dim3(rows), dim3(kWG), 0, st, a);
    hipLaunchKernelGGL(k_sample_decide, dim3(a.B), dim3(64), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace mtp
