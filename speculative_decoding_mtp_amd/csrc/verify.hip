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
// One workgroup per (chunk, sequence) takes the chunk's argmax of the sequence's rows 0, 1, ... in
// order.  Greedy verification stops at the first row whose argmax is not the draft it judges
// ([YL 三 stage 3]), so no row after that one is needed: once this chunk holds an element ranked
// above row j's draft (value desc, id asc), the draft cannot be row j's argmax, the sequence stops
// at row j or before, and the workgroup skips the later rows.  Every row the decision needs (each
// row up to the first mismatch) is therefore scanned by every chunk.
// Each draft's own target logit is loaded up front, and while row j is reduced the next row's
// slice is already in flight (slices of at most 4096 logits, up to four float4 per thread), so a
// row costs one memory latency only when its predecessor was needed.
__device__ __forceinline__ void chunk_best4(const uint4 u, int k, int end, float& bv, int& bi) {
  const float f[4] = {__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w)};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (k + e < end && better(f[e], k + e, bv, bi)) {
      bv = f[e];
      bi = k + e;
    }
}

__global__ __launch_bounds__(kWG) void k_verify_greedy(VerifyArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  __shared__ float s_vd[kMaxDraft];
  __shared__ int s_d[kMaxDraft];
  const int c = blockIdx.x, R = a.D + 1;
  const int beg = c * a.chunk, end = min(a.V, beg + a.chunk);
  // without the walk (small calls, where latency rather than bytes decides) every workgroup
  // takes one row, blockIdx.y = b * (D + 1) + j, and no row is skipped
  const int b = a.walk ? blockIdx.y : blockIdx.y / R;
  const int j0 = a.walk ? 0 : blockIdx.y - b * R, j1 = a.walk ? R : j0 + 1;
  for (int t = threadIdx.x; t < a.D && a.walk; t += kWG) {
    const int d = a.drafts[(long)b * a.D + t];
    const bool ok = d >= 0 && d < a.V;
    s_d[t] = ok ? d : -1;
    s_vd[t] = ok ? a.tl[((long)b * R + t) * a.V + d] : 0.f;
  }
  // slices of up to 4096 logits: up to four float4 per thread, the next row's held in registers
  const bool pipelined = (a.V & 3) == 0 && end - beg <= 16 * kWG;
  const int nsw = (end - beg + 4 * kWG - 1) / (4 * kWG);
  const int k4 = beg + 4 * threadIdx.x;
  uint4 cur[4], nxt[4];
  auto load_row = [&](long row, uint4 (&r)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (s < nsw) r[s] = ld_stream(a.tl + row * a.V + min(k4 + 4 * kWG * s, (end - 1) & ~3));
  };
  if (pipelined) load_row((long)b * R + j0, cur);
  __syncthreads();
  for (int j = j0; j < j1; ++j) {
    const long row = (long)b * R + j;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    if (pipelined) {
      if (j + 1 < j1) load_row(row + 1, nxt);  // the next row in flight
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (s < nsw) chunk_best4(cur[s], k4 + 4 * kWG * s, end, bv, bi);
#pragma unroll
      for (int s = 0; s < 4; ++s) cur[s] = nxt[s];
    } else {
      const float* x = a.tl + row * a.V;
      if ((a.V & 3) == 0) {
        for (int k = k4; k < end; k += 4 * kWG) chunk_best4(ld_stream(x + k), k, end, bv, bi);
      } else {
        for (int k = beg + threadIdx.x; k < end; k += kWG)
          if (better(x[k], k, bv, bi)) {
            bv = x[k];
            bi = k;
          }
      }
    }
    wg_argmax(bv, bi, sv, si);  // every thread holds the chunk's argmax
    if (threadIdx.x == 0) {
      a.part_v[row * a.nchunk + c] = bv;
      a.part_i[row * a.nchunk + c] = bi;
    }
    if (!a.walk || j == a.D) break;
    const int d = s_d[j];
    if (d < 0) break;                           // no valid draft: the sequence stops here
    if (better(bv, bi, s_vd[j], d)) break;      // ranked above the draft: row j rejects it
  }
}

// one workgroup per sequence: the argmax of rows 0, 1, ... from the chunk partials, up to the
// first row whose argmax differs from its draft; then the emitted tokens and lengths
__global__ __launch_bounds__(kWG) void k_verify_greedy_final(VerifyArgs a) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int b = blockIdx.x, rows_per_seq = a.D + 1;
  const int* d = a.drafts + (long)b * a.D;
  int n = 0, last = 0;
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
    wg_argmax(bv, bi, sv, si);  // uniform
    last = bi;
    if (j == a.D || bi != d[j]) break;
    n = j + 1;
  }
  if (threadIdx.x == 0) {
    int32_t* out = a.out + (long)b * rows_per_seq;
    for (int j = 0; j < n; ++j) out[j] = d[j];
    out[n] = last;
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

// ---- wave-parallel pieces of the decision (one wave per sequence; candidate k of a row sits in
// lane k % 64, slot k / 64, so K <= 128 takes two slots per lane)

__device__ __forceinline__ float wave_incl_scan(float v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

// A row's warped distribution from its sorted top-k candidates (value desc): temperature
// softmax over the n candidates, then top-p (a candidate stays while the mass ranked before it
// is below p; the first always stays), renormalised.  p[s] is candidate 64 s + lane's
// probability (0 outside the kept prefix); returns the kept count m.
__device__ int warp_row_wave(const float* tv, const int n, float T, float top_p, float (&p)[2]) {
  const int lane = threadIdx.x & 63;
  const float t0 = tv[0];
  float e[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int k = 64 * s + lane;
    e[s] = k < n ? expf((tv[k] - t0) / T) : 0.f;
  }
  const float c0 = wave_incl_scan(e[0]);
  const float tot0 = __shfl(c0, 63, 64);
  const float c1 = wave_incl_scan(e[1]) + tot0;
  const float S = __shfl(c1, 63, 64);
  int m = n;
  if (top_p < 1.f) {
    const float before[2] = {c0 - e[0], c1 - e[1]};
    int kept = 0;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k = 64 * s + lane;
      kept += (k < n && (k == 0 || before[s] / S < top_p)) ? 1 : 0;
    }
    m = (int)wave_sum((float)kept);
  }
  float z = 0.f;
#pragma unroll
  for (int s = 0; s < 2; ++s) z += (64 * s + lane < m) ? e[s] : 0.f;
  const float Z = wave_sum(z);
#pragma unroll
  for (int s = 0; s < 2; ++s) p[s] = (64 * s + lane < m) ? e[s] / Z : 0.f;
  return m;
}

// Inverse-CDF draw over the weights w of ids (candidate slots as above, m of them) in ascending
// id order: the smallest id whose cumulative weight exceeds u * total; weights <= 0 are never
// drawn (if u * total rounds onto the total, the last positive one is).  sw/si: LDS, 128 each.
__device__ int draw_ascending_wave(const int (&id)[2], const float (&w)[2], int m, float u, float* sw, int* si) {
  const int lane = threadIdx.x & 63;
  // rank of each candidate by id among the m (ids are distinct)
  int r[2] = {0, 0};
#pragma unroll
  for (int s = 0; s < 2; ++s) si[64 * s + lane] = id[s];
  __syncthreads();
  for (int j = 0; j < m; ++j) {
    const int o = si[j];
#pragma unroll
    for (int s = 0; s < 2; ++s) r[s] += o < id[s] ? 1 : 0;
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < 2; ++s)
    if (64 * s + lane < m) {
      sw[r[s]] = w[s] > 0.f ? w[s] : 0.f;
      si[r[s]] = id[s];
    }
  __syncthreads();
  float x[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) x[s] = 64 * s + lane < m ? sw[64 * s + lane] : 0.f;
  const float c0 = wave_incl_scan(x[0]);
  const float tot0 = __shfl(c0, 63, 64);
  const float c1 = wave_incl_scan(x[1]) + tot0;
  const float S = __shfl(c1, 63, 64);
  const float t = u * S;
  const unsigned long long hit0 = __ballot(x[0] > 0.f && c0 > t);
  const unsigned long long hit1 = __ballot(x[1] > 0.f && c1 > t);
  int pos = -1;
  if (hit0)
    pos = __ffsll((long long)hit0) - 1;
  else if (hit1)
    pos = 64 + __ffsll((long long)hit1) - 1;
  else {  // the last positive weight
    const unsigned long long pz0 = __ballot(x[0] > 0.f), pz1 = __ballot(x[1] > 0.f);
    if (pz1)
      pos = 64 + 63 - __clzll((long long)pz1);
    else if (pz0)
      pos = 63 - __clzll((long long)pz0);
  }
  const int tok = pos >= 0 ? si[pos] : -1;
  __syncthreads();
  return tok;
}

// One workgroup per row streams the row once.  Items at or above a threshold are appended to an
// LDS candidate buffer; the threshold starts as the K-th largest of the per-thread maxima of the
// first tile (K threads hold an item at least that large, so it never exceeds the row's K-th
// best) and rises to the K-th best candidate whenever the buffer has to be compacted.  At the
// end the candidates are sorted (value desc, id asc) and the first K written.
constexpr int kTile = kWG * 16;  // items per tile: four float4 per thread
static_assert(kTopCap >= kMaxTopK + kTile / 4, "the slow pass appends a quarter tile after a compaction");
static_assert((kTopCap & (kTopCap - 1)) == 0, "the candidate sort pads to a power of two");
static_assert(kMaxTopK <= 128, "the decision keeps two candidates per lane");

// Item e of tile `base` for thread t: ids base + 4 (t + kWG q) + r, e = 4 q + r.
// One tile: items base + 4 (tid + kWG q) + r, q, r < 4.  Every load is issued unconditionally (a
// clamped in-bounds address, items past V masked to -inf), so the loads of one tile can be in
// flight together with the next tile's.  VEC: float4 loads (the row is 16-byte aligned and V a
// multiple of 4, so a group of four is either wholly inside the row or wholly past it).
template <bool VEC>
__device__ __forceinline__ void load_tile(const float* x, int V, int base, float (&v)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k0 = base + 4 * (threadIdx.x + kWG * q);
    if constexpr (VEC) {  // each logit is read once: streamed past L2
      const float4 f = ld_stream_f4(x + min(k0, V - 4));
      const bool in = k0 < V;
      v[4 * q] = in ? f.x : -INFINITY;
      v[4 * q + 1] = in ? f.y : -INFINITY;
      v[4 * q + 2] = in ? f.z : -INFINITY;
      v[4 * q + 3] = in ? f.w : -INFINITY;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = x[min(k0 + r, V - 1)];
        v[4 * q + r] = k0 + r < V ? f : -INFINITY;
      }
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

// The top K of the V items at x (value desc, position asc) into ov / oi, the count into *on (when
// not NULL).  An output id is the item's position plus id_base, or id_map[position].
template <bool VEC>
__device__ __forceinline__ void topk_row(const VerifyArgs& a, TopkSmem& sm, const float* x, int V, float* ov,
                                         int* oi, int* on, int id_base, const int* id_map) {
  const int K = a.top_k;
  auto out_id = [&](int pos) { return id_map ? id_map[pos] : pos + id_base; };
  float cur[16], nxt[16];
  load_tile<VEC>(x, V, 0, cur);
  float rmax = -INFINITY;  // this thread's running maximum
#pragma unroll
  for (int e = 0; e < 16; ++e) rmax = fmaxf(rmax, cur[e]);
  // K-th largest of the per-thread maxima: K distinct items are at least this large
  auto bound = [&]() {
    sm.tm[threadIdx.x] = rmax;
    __syncthreads();
    bitonic_sort_desc(sm.tm);
    const float b = sm.tm[K - 1];
    __syncthreads();
    return b;
  };
  if (threadIdx.x == 0) sm.cnt = 0;
  float theta = bound();
  // Fast pass: no barriers while streaming (the threshold is raised once, after four tiles);
  // appends past the buffer are counted, not stored, and send the row to the slow pass.
  auto append = [&](const float (&v)[16], int base) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int k = base + 4 * (threadIdx.x + kWG * (e >> 2)) + (e & 3);
      if (k < V) {
        rmax = fmaxf(rmax, v[e]);
        if (v[e] >= theta) {
          const int pos = atomicAdd(&sm.cnt, 1);
          if (pos < kTopCap) {
            sm.v[pos] = v[e];
            sm.i[pos] = k;
          }
        }
      }
    }
  };
  for (int base = 0; base < V; base += 2 * kTile) {
    // loads are unconditional (past the row they are clamped and masked): the compiler can then
    // count them and keep the next tile in flight while this one is scanned
    load_tile<VEC>(x, V, base + kTile, nxt);
    append(cur, base);
    if (base + kTile >= V) break;
    load_tile<VEC>(x, V, base + 2 * kTile, cur);
    append(nxt, base + kTile);
    if (base == 2 * kTile && base + 2 * kTile < V) theta = fmaxf(theta, bound());
  }
  __syncthreads();
  if (sm.cnt > kTopCap) {
    // Slow pass (the threshold let too many items through, e.g. heavy ties): stream the row
    // again, compacting the buffer to its top K whenever the next tile might not fit.
    __syncthreads();
    if (threadIdx.x == 0) sm.cnt = 0;
    __syncthreads();
    for (int base = 0; base < V; base += kTile) {
      load_tile<VEC>(x, V, base, cur);
#pragma unroll
      for (int h = 0; h < 4; ++h) {  // a quarter tile (at most kTile / 4 appends) at a time
#pragma unroll
        for (int e = 4 * h; e < 4 * h + 4; ++e) {
          const int k = base + 4 * (threadIdx.x + kWG * (e >> 2)) + (e & 3);
          if (k < V && cur[e] >= theta) {
            const int pos = atomicAdd(&sm.cnt, 1);
            sm.v[pos] = cur[e];
            sm.i[pos] = k;
          }
        }
        __syncthreads();
        const int S = sm.cnt;
        __syncthreads();
        if (S > kTopCap - kTile / 4) {
          const int n = sort_candidates(sm, S, K);
          if (n == K) theta = sm.v[K - 1];
          __syncthreads();
          if (threadIdx.x == 0) sm.cnt = n;
          __syncthreads();
        }
      }
    }
  }
  // Final selection.  The K-th largest of the per-thread maxima over the S candidates bounds
  // the K-th best from below again; the few candidates at or above it are ranked by counting
  // (rank = candidates ranked before it, value desc, id asc) straight into their output slots.
  // If too many remain (ties), the whole buffer is sorted instead.
  const int S = sm.cnt;
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
        oi[r] = out_id(ci);
      }
    }
  } else {
    n = sort_candidates(sm, S, K);
    for (int t = threadIdx.x; t < n; t += kWG) {
      ov[t] = sm.v[t];
      oi[t] = out_id(sm.i[t]);
    }
  }
  for (int t = n + threadIdx.x; t < K; t += kWG) {
    ov[t] = -INFINITY;
    oi[t] = -1;
  }
  if (on && threadIdx.x == 0) *on = n;
}

__device__ __forceinline__ const float* topk_src(const VerifyArgs& a, int row) {
  const int tgt_rows = a.B * (a.D + 1);
  return row < tgt_rows ? a.tl + (long)row * a.V : a.dl + (long)(row - tgt_rows) * a.V;
}

__device__ __forceinline__ bool vec_ok(const float* x, int n) {
  return (reinterpret_cast<uintptr_t>(x) & 15) == 0 && (n & 3) == 0;
}

// One workgroup per row.
__global__ __launch_bounds__(kWG) void k_topk_stream(VerifyArgs a) {
  __shared__ TopkSmem sm;
  const int row = blockIdx.x, K = a.top_k;
  const float* x = topk_src(a, row);
  float* ov = a.top_v + (long)row * K;
  int* oi = a.top_i + (long)row * K;
  if (vec_ok(x, a.V))
    topk_row<true>(a, sm, x, a.V, ov, oi, a.top_n + row, 0, nullptr);
  else
    topk_row<false>(a, sm, x, a.V, ov, oi, a.top_n + row, 0, nullptr);
}

// Few rows: workgroup (c, row) takes the top K of items [c chunk, (c + 1) chunk) of the row ...
__global__ __launch_bounds__(kWG) void k_topk_chunks(VerifyArgs a) {
  __shared__ TopkSmem sm;
  const int c = blockIdx.x, row = blockIdx.y, K = a.top_k;
  const int c0 = c * a.tk_chunk, n = min(a.tk_chunk, a.V - c0);
  const float* x = topk_src(a, row) + c0;
  const long slot = ((long)row * a.tk_nchunk + c) * K;
  if (vec_ok(x, n))
    topk_row<true>(a, sm, x, n, a.cand_v + slot, a.cand_i + slot, nullptr, c0, nullptr);
  else
    topk_row<false>(a, sm, x, n, a.cand_v + slot, a.cand_i + slot, nullptr, c0, nullptr);
}

// ... and one workgroup per row then takes the top K of the row's chunk candidates.  Candidates
// sit in chunk order (ascending ids) and, inside a chunk, best first with ascending ids among
// equal values, so ordering them by (value desc, position asc) is ordering them by (value desc,
// id asc): the result equals the one-pass selection over the whole row.
__global__ __launch_bounds__(kWG) void k_topk_merge(VerifyArgs a) {
  __shared__ TopkSmem sm;
  const int row = blockIdx.x, K = a.top_k, n = a.tk_nchunk * K;
  const float* x = a.cand_v + (long)row * n;
  const int* ids = a.cand_i + (long)row * n;
  float* ov = a.top_v + (long)row * K;
  int* oi = a.top_i + (long)row * K;
  if (vec_ok(x, n))
    topk_row<true>(a, sm, x, n, ov, oi, a.top_n + row, 0, ids);
  else
    topk_row<false>(a, sm, x, n, ov, oi, a.top_n + row, 0, ids);
}

// One wave per sequence: accept / reject / draw ([DLM "MTP speculative decoding"] item 3, [YL 三
// stage 3]).  P_j = warp(target row j); Q_j = one-hot at the draft (q_mode 0) or warp(draft row
// j) (q_mode 1).  Draft j is accepted iff P_j(d) > 0 and U_j <= P_j(d) / Q_j(d); at the first
// rejection a token is drawn from normalize(max(0, P_j - Q_j)) (P_j if that is all zero), and
// if every draft holds, from P_D.
__global__ __launch_bounds__(64) void k_sample_decide(VerifyArgs a) {
  __shared__ float sw[kMaxTopK], sq[kMaxTopK];
  __shared__ int si[kMaxTopK], sqi[kMaxTopK];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int K = a.top_k;
  const int tgt_rows = a.B * (a.D + 1);
  const float T = a.temperature;
  int n_acc = 0, tok = -1;
  float P[2];
  int id[2];
  auto load_row = [&](int r, float (&p)[2], int (&ids)[2]) {
    const int m = warp_row_wave(a.top_v + (long)r * K, a.top_n[r], T, a.top_p, p);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int k = 64 * s + lane;
      ids[s] = k < m ? a.top_i[(long)r * K + k] : -1;
    }
    return m;
  };
  for (int j = 0; j < a.D && tok < 0; ++j) {
    const int mP = load_row(b * (a.D + 1) + j, P, id);
    const int d = a.drafts[(long)b * a.D + j];
    const float Pd = wave_sum((id[0] == d ? P[0] : 0.f) + (id[1] == d ? P[1] : 0.f));
    float Qd = 1.f;
    int mQ = 0;
    if (a.q_mode == 1) {
      float Qp[2];
      int qid[2];
      mQ = load_row(tgt_rows + b * a.D + j, Qp, qid);
      Qd = wave_sum((qid[0] == d ? Qp[0] : 0.f) + (qid[1] == d ? Qp[1] : 0.f));
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        sq[64 * s + lane] = Qp[s];
        sqi[64 * s + lane] = qid[s];
      }
      __syncthreads();
    }
    const float u = a.u_accept[(long)b * a.D + j];
    if (Pd > 0.f && (Qd == 0.f || u <= Pd / Qd)) {
      if (lane == 0) a.out[(long)b * (a.D + 1) + j] = d;
      ++n_acc;
      continue;
    }
    // residual max(0, P - Q); its support lies inside P's kept set
    float w[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float q = 0.f;
      if (a.q_mode == 1) {
        for (int k = 0; k < mQ; ++k) q = sqi[k] == id[s] ? sq[k] : q;
      } else {
        q = id[s] == d ? 1.f : 0.f;
      }
      w[s] = 64 * s + lane < mP ? fmaxf(P[s] - q, 0.f) : 0.f;
    }
    if (!(wave_sum(w[0] + w[1]) > 0.f)) {
      w[0] = P[0];
      w[1] = P[1];
    }
    tok = draw_ascending_wave(id, w, mP, a.u_sample[b], sw, si);
    if (tok < 0) tok = -2;  // nothing drawable: keep the row's outcome as a rejection
  }
  if (tok == -1) {  // every draft held: one more token from row D
    const int mP = load_row(b * (a.D + 1) + a.D, P, id);
    tok = draw_ascending_wave(id, P, mP, a.u_sample[b], sw, si);
  }
  if (lane == 0) {
    int32_t* out = a.out + (long)b * (a.D + 1);
    out[n_acc] = tok < 0 ? -1 : tok;
    for (int j = n_acc + 1; j <= a.D; ++j) out[j] = -1;
    a.n_accept[b] = n_acc;
    a.crop[b] = a.ctx_len[b] + 1 + n_acc;
  }
}

// ---------------------------------------------------------------------------------------------
// sampling over the whole vocabulary: top-k off (or above the candidate buffer), top-p on the rest
// ---------------------------------------------------------------------------------------------
// [DLM "Why a hand-written decoding loop"]: temperature, then top-k, then top-p, in that order.
// The kept set of a row is a prefix of the tokens ranked by (logit desc, id asc) -- the same
// ranking as scaled logits, since T > 0 -- so it is described by its last member.  One workgroup
// per row finds it by radix selection over order-preserving 32-bit keys of the logits, 8 bits per
// pass: by count for the k-th token, by weight for the token whose inclusive mass first reaches
// p times the mass of the top-k set (the token that crosses p is kept).  Equal keys are taken in
// ascending id order with a scan over the row.  Weights exp((l - lmax) / T) are summed as 2^-40
// fixed-point integers, so every sum (and every decision) is the same from run to run.
constexpr double kFix = 1099511627776.0;  // 2^40

__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);  // -0 ranks with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ unsigned long long fix_weight(float l, float lmax, float T) {
  return (unsigned long long)((double)expf((l - lmax) / T) * kFix + 0.5);
}
// rank order: token i is ranked at or before the boundary (key, id)
__device__ __forceinline__ bool kept_by(uint32_t k, int i, uint32_t bk, int bi) {
  return k > bk || (k == bk && i <= bi);
}

// Block-wide exclusive scan of one 64-bit value per thread (256 threads); returns the thread's
// exclusive prefix, *total the sum.  s64: __shared__ unsigned long long[kWG].
__device__ unsigned long long scan_u64(unsigned long long v, unsigned long long* s64, unsigned long long* total) {
  const int tid = threadIdx.x;
  s64[tid] = v;
  __syncthreads();
  for (int off = 1; off < kWG; off <<= 1) {
    const unsigned long long add = tid >= off ? s64[tid - off] : 0ull;
    __syncthreads();
    s64[tid] += add;
    __syncthreads();
  }
  const unsigned long long incl = s64[tid];
  *total = s64[kWG - 1];
  __syncthreads();
  return incl - v;
}

struct FullSmem {
  unsigned long long hist[256];
  unsigned long long s64[kWG];
  float red[4];
  int pick, pick_id;
  unsigned long long pick_above;
};

// The row's search.  Each thread walks a contiguous id segment [seg0, seg1) wherever the order of
// ids matters (the tie scans), and strided elements elsewhere.
__global__ __launch_bounds__(kWG) void k_full_select(VerifyArgs a) {
  __shared__ FullSmem sm;
  const int row = blockIdx.x, tid = threadIdx.x, V = a.V;
  const float T = a.temperature;
  const int tgt_rows = a.B * (a.D + 1);
  const float* x = row < tgt_rows ? a.tl + (long)row * V : a.dl + (long)(row - tgt_rows) * V;
  const int seg = (V + kWG - 1) / kWG, seg0 = min(V, tid * seg), seg1 = min(V, seg0 + seg);
  // the row maximum
  float mx = -INFINITY;
  for (int i = tid; i < V; i += kWG) mx = fmaxf(mx, x[i]);
  mx = wave_max(mx);
  if ((tid & 63) == 0) sm.red[tid >> 6] = mx;
  __syncthreads();
  const float lmax = fmaxf(fmaxf(sm.red[0], sm.red[1]), fmaxf(sm.red[2], sm.red[3]));
  __syncthreads();
  // top-k boundary: the k-th token in rank order (none when top-k is off)
  uint32_t tk = 0;
  int ik = 0x7fffffff;
  const bool use_k = a.top_k > 0 && a.top_k < V;
  if (use_k) {
    uint32_t prefix = 0, mask = 0;
    unsigned long long need = (unsigned long long)a.top_k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      sm.hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < V; i += kWG) {
        const uint32_t k = order_key(x[i]);
        if ((k & mask) == prefix) atomicAdd(&sm.hist[(k >> shift) & 255], 1ull);
      }
      __syncthreads();
      if (tid == 0) {
        unsigned long long cum = 0;
        int d = 255;
        for (; d > 0; --d) {
          if (cum + sm.hist[d] >= need) break;
          cum += sm.hist[d];
        }
        sm.pick = d;
        sm.pick_above = cum;
      }
      __syncthreads();
      need -= sm.pick_above;
      prefix |= (uint32_t)sm.pick << shift;
      mask |= 255u << shift;
      __syncthreads();
    }
    tk = prefix;
    // the need-th lowest id among the tokens whose key is tk
    unsigned long long c = 0;
    for (int i = seg0; i < seg1; ++i) c += order_key(x[i]) == tk ? 1ull : 0ull;
    unsigned long long tot;
    const unsigned long long before = scan_u64(c, sm.s64, &tot);
    if (before < need && need <= before + c) {
      unsigned long long cnt = before;
      for (int i = seg0; i < seg1; ++i)
        if (order_key(x[i]) == tk && ++cnt == need) {
          sm.pick_id = i;
          break;
        }
    }
    __syncthreads();
    ik = sm.pick_id;
    __syncthreads();
  }
  // the top-k set's weight
  unsigned long long z = 0;
  for (int i = tid; i < V; i += kWG)
    if (!use_k || kept_by(order_key(x[i]), i, tk, ik)) z += fix_weight(x[i], lmax, T);
  unsigned long long zk;
  (void)scan_u64(z, sm.s64, &zk);
  uint32_t bk = tk;
  int bi = ik;
  unsigned long long zkept = zk;
  if (a.top_p < 1.f) {
    // top-p boundary inside the top-k set: the token whose inclusive mass first reaches p * zk
    const double target = (double)a.top_p * (double)zk;
    uint32_t prefix = 0, mask = 0;
    unsigned long long above = 0;
    bool crossed = true;
    for (int shift = 24; shift >= 0 && crossed; shift -= 8) {
      sm.hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < V; i += kWG) {
        const uint32_t k = order_key(x[i]);
        if ((k & mask) == prefix && (!use_k || kept_by(k, i, tk, ik)))
          atomicAdd(&sm.hist[(k >> shift) & 255], fix_weight(x[i], lmax, T));
      }
      __syncthreads();
      if (tid == 0) {
        unsigned long long cum = above;
        int d = 255;
        for (; d >= 0; --d) {
          if ((double)(cum + sm.hist[d]) >= target) break;
          cum += sm.hist[d];
        }
        sm.pick = d;
        sm.pick_above = cum;
      }
      __syncthreads();
      if (sm.pick < 0) {
        crossed = false;  // rounding left the whole set below p: keep all of it
      } else {
        above = sm.pick_above;
        prefix |= (uint32_t)sm.pick << shift;
        mask |= 255u << shift;
      }
      __syncthreads();
    }
    if (crossed) {
      // among the tokens with key == prefix (inside the top-k set), ascending ids until the
      // inclusive mass reaches the target
      unsigned long long c = 0;
      for (int i = seg0; i < seg1; ++i) {
        const uint32_t k = order_key(x[i]);
        if (k == prefix && (!use_k || kept_by(k, i, tk, ik))) c += fix_weight(x[i], lmax, T);
      }
      unsigned long long tot;
      const unsigned long long before = scan_u64(c, sm.s64, &tot);
      if ((double)(above + before) < target && (double)(above + before + c) >= target) {
        unsigned long long cum = above + before;
        for (int i = seg0; i < seg1; ++i) {
          const uint32_t k = order_key(x[i]);
          if (k == prefix && (!use_k || kept_by(k, i, tk, ik))) {
            cum += fix_weight(x[i], lmax, T);
            if ((double)cum >= target) {
              sm.pick_id = i;
              sm.pick_above = cum;
              break;
            }
          }
        }
      }
      __syncthreads();
      bk = prefix;
      bi = sm.pick_id;
      zkept = sm.pick_above;
    }
  }
  if (tid == 0) {
    FullRow f;
    f.lmax = lmax;
    f.key = bk;
    f.id = bi;
    f.pad = 0;
    f.zk = zkept;
    f.pad2 = 0;
    a.rowinfo[row] = f;
  }
}

// One workgroup per sequence: the decisions of k_sample_decide with the whole-vocabulary kept
// sets.  P_j(i) = w_i / zk for kept i; the draw takes the smallest id whose inclusive cumulative
// fixed-point weight exceeds u times the total, over the row in ascending id order.
__global__ __launch_bounds__(kWG) void k_full_decide(VerifyArgs a) {
  __shared__ unsigned long long s64[kWG];
  __shared__ int s_tok;
  const int b = blockIdx.x, tid = threadIdx.x, V = a.V;
  const float T = a.temperature;
  const int tgt_rows = a.B * (a.D + 1);
  const int seg = (V + kWG - 1) / kWG, seg0 = min(V, tid * seg), seg1 = min(V, seg0 + seg);
  auto prob = [&](int row, int i) -> double {  // P of token i under row's warp
    const FullRow f = a.rowinfo[row];
    const float* x = row < tgt_rows ? a.tl + (long)row * V : a.dl + (long)(row - tgt_rows) * V;
    const float l = x[i];
    if (!kept_by(order_key(l), i, f.key, f.id)) return 0.0;
    return (double)fix_weight(l, f.lmax, T) / (double)f.zk;
  };
  // inverse-CDF draw over the row's residual (qrow >= 0: max(0, P - Q) against that row; qrow ==
  // -1: P without the one-hot draft d; qrow == -2: P itself); falls back to P when all zero
  auto draw = [&](int prow, int qrow, int d, float u) -> int {
    const FullRow fp = a.rowinfo[prow];
    const float* xp = a.tl + (long)prow * V;
    FullRow fq = fp;
    const float* xq = xp;
    if (qrow >= 0) {
      fq = a.rowinfo[qrow];
      xq = a.dl + (long)(qrow - tgt_rows) * V;
    }
    auto weight = [&](int i, bool resid) -> unsigned long long {
      const float l = xp[i];
      if (!kept_by(order_key(l), i, fp.key, fp.id)) return 0ull;
      const unsigned long long wp = fix_weight(l, fp.lmax, T);
      if (!resid || qrow == -2) return wp;
      if (qrow == -1) return i == d ? 0ull : wp;
      const double P = (double)wp / (double)fp.zk;
      const float lq = xq[i];
      const double Q = kept_by(order_key(lq), i, fq.key, fq.id) ? (double)fix_weight(lq, fq.lmax, T) / (double)fq.zk : 0.0;
      return P > Q ? (unsigned long long)((P - Q) * kFix + 0.5) : 0ull;
    };
    bool resid = qrow != -2;
    for (int attempt = 0; attempt < 2; ++attempt) {
      unsigned long long c = 0;
      for (int i = seg0; i < seg1; ++i) c += weight(i, resid);
      unsigned long long S;
      const unsigned long long before = scan_u64(c, s64, &S);
      if (S == 0ull) {
        resid = false;  // max(0, P - Q) is all zero: draw from P
        continue;
      }
      const double t = (double)u * (double)S;
      if (tid == 0) s_tok = -1;
      __syncthreads();
      if ((double)before <= t && (double)(before + c) > t) {
        unsigned long long cum = before;
        for (int i = seg0; i < seg1; ++i) {
          cum += weight(i, resid);
          if ((double)cum > t) {
            s_tok = i;
            break;
          }
        }
      }
      __syncthreads();
      int tok = s_tok;
      if (tok < 0) {  // u * S rounded onto S: the last id with weight
        for (int i = V - 1 - tid; i >= 0 && tok < 0; i -= kWG)
          if (weight(i, resid) > 0ull) tok = i;
        s64[tid] = (unsigned long long)(tok < 0 ? -1 : tok);
        __syncthreads();
        if (tid == 0) {
          long long best = -1;
          for (int k = 0; k < kWG; ++k) best = max(best, (long long)s64[k]);
          s_tok = (int)best;
        }
        __syncthreads();
        tok = s_tok;
      }
      __syncthreads();
      return tok;
    }
    return -1;
  };
  int n_acc = 0, tok = -1;
  for (int j = 0; j < a.D && tok < 0; ++j) {
    const int prow = b * (a.D + 1) + j, d = a.drafts[(long)b * a.D + j];
    const int qrow = a.q_mode == 1 ? tgt_rows + b * a.D + j : -1;
    double Pd = 0.0, Qd = 1.0;
    if (d >= 0 && d < V) {
      Pd = prob(prow, d);
      if (qrow >= 0) Qd = prob(qrow, d);
    }
    const float u = a.u_accept[(long)b * a.D + j];
    if (Pd > 0.0 && (Qd == 0.0 || (double)u <= Pd / Qd)) {
      if (tid == 0) a.out[(long)b * (a.D + 1) + j] = d;
      ++n_acc;
      continue;
    }
    tok = draw(prow, qrow, d, a.u_sample[b]);
    if (tok < 0) tok = -2;
  }
  if (tok == -1) tok = draw(b * (a.D + 1) + a.D, -2, -1, a.u_sample[b]);
  if (tid == 0) {
    int32_t* out = a.out + (long)b * (a.D + 1);
    out[n_acc] = tok < 0 ? -1 : tok;
    for (int j = n_acc + 1; j <= a.D; ++j) out[j] = -1;
    a.n_accept[b] = n_acc;
    a.crop[b] = a.ctx_len[b] + 1 + n_acc;
  }
}

hipError_t run_verify(const VerifyArgs& a, hipStream_t st) {
  if (a.greedy) {
    hipLaunchKernelGGL(k_verify_greedy, dim3(a.nchunk, a.walk ? a.B : a.B * (a.D + 1)), dim3(kWG), 0, st, a);
    hipLaunchKernelGGL(k_verify_greedy_final, dim3(a.B), dim3(kWG), 0, st, a);
  } else if (a.full) {
    const int rows = a.B * (a.D + 1) + (a.q_mode == 1 ? a.B * a.D : 0);
    hipLaunchKernelGGL(k_full_select, dim3(rows), dim3(kWG), 0, st, a);
    hipLaunchKernelGGL(k_full_decide, dim3(a.B), dim3(kWG), 0, st, a);
  } else {
    const int rows = a.B * (a.D + 1) + (a.q_mode == 1 ? a.B * a.D : 0);
    if (a.tk_nchunk > 1) {
      hipLaunchKernelGGL(k_topk_chunks, dim3(a.tk_nchunk, rows), dim3(kWG), 0, st, a);
      hipLaunchKernelGGL(k_topk_merge, dim3(rows), dim3(kWG), 0, st, a);
    } else {
      hipLaunchKernelGGL(k_topk_stream, dim3(rows), dim3(kWG), 0, st, a);
    }
    hipLaunchKernelGGL(k_sample_decide, dim3(a.B), dim3(64), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace mtp
