// Decode attention of the draft head: grouped-query causal softmax attention of each row over
// the head's own KV cache, split over the cached positions and merged in a second pass.
//
// [HB14] "14. MTP: speculative decoding with the built-in draft head", section "The draft head":
// the head's decoder layer is full attention with RoPE over its own KV cache; rows attend to
// every cached position up to their own.  Scores q.k / sqrt(hd), softmax, weighted sum of V.
#include "common.h"
#include "draft.h"
#include "gemv.h"

namespace mtp {

// The compact row of row 0 of sequence b: the valid rows of the sequences before it (the row
// order of the MFMA GEMMs' split activations).  Thread t < B counts sequence t into s_cnt; call
// with the whole workgroup (it contains a barrier).
__device__ int attn_compact_base(const AttnArgs& a, int b, int* s_cnt) {
  for (int t = threadIdx.x; t < a.B; t += blockDim.x)
    s_cnt[t] = a.rows ? a.rows[t] : count_rows(a.tok + (long)t * a.tok_sb, a.rps, a.V, a.len[t], a.max_len, nullptr);
  __syncthreads();
  int c = 0;
  for (int t = 0; t < b; ++t) c += s_cnt[t];
  return c;
}

// One output value: at `o` of out, and split into bf16 hi + lo at `c` of a.shi / a.slo (when set).
__device__ __forceinline__ void attn_store(const AttnArgs& a, float* out, long o, long c, float v) {
  out[o] = v;
  if (a.shi) {
    const uint32_t h = bf16_rne(v);
    a.shi[c] = (uint16_t)h;
    a.slo[c] = (uint16_t)bf16_rne(v - __uint_as_float(h << 16));
  }
}

// Max and sum over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes of a query column), by the
// in-register half swaps: with both operands x, a swap returns x[l] and its partner in the two
// results of every lane, so one max (or add, commutative) per swap leaves every lane with the
// same value.
__device__ __forceinline__ float col_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float col_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// ---------------------------------------------------------------------------------------------
// decode attention, split over the cached positions (fp32 caches: VALU kernel)
// ---------------------------------------------------------------------------------------------
constexpr int kTile = 64;  // cached positions per LDS tile
constexpr int kQB = 32;    // queries per pass

// Workgroup (s, kvh, b) handles positions [s*chunk, min(T, (s+1)*chunk)) of sequence b, where
// T = len[b] + rows, for every query (row i, query head kvh*G + g) of the sequence.  K/V tiles
// of 64 positions go through registers (the next tile is fetched while the current one is
// used) into LDS, values transposed back to [position][channel]; an online softmax keeps
// (m, l, o) per query.  Output per query: the unnormalised o, the running max m and the sum l.
template <class W, int HD>
__global__ __launch_bounds__(kWG) void k_attn(AttnArgs a) {
  using T = typename W::T;
  constexpr int VE = W::VE;               // elements per 16-byte vector
  constexpr int VPR = HD / VE;            // vectors per cached row
  constexpr int NV = kTile * VPR / kWG;   // vectors per thread per tile and matrix
  constexpr int LDR = HD + VE;            // padded LDS row (elements)
  constexpr int SPT = kQB / 4;            // score accumulators per thread
  constexpr int QG = kWG / HD;            // query groups in the PV phase
  constexpr int QPT = kQB / QG;           // PV accumulators per thread
  constexpr int QW = kQB / 4;             // softmax queries per wave
  __shared__ __align__(16) T sK[kTile * LDR];
  __shared__ __align__(16) T sV[kTile * LDR];
  __shared__ __align__(16) float sQ[kQB * HD];
  __shared__ float sS[kQB * (kTile + 1)];           // scores [q][p], padded rows
  __shared__ __align__(16) float sP[kTile * kQB];   // probabilities [p][q]
  __shared__ float sAlpha[kQB];
  __shared__ int s_n;

  const int tid = threadIdx.x;
  // blockIdx.y = kv head + nkv * (query-block group): many queries (a prefill) also spread over
  // the grid: this workgroup takes query blocks qgrp, qgrp + nqgrp, ... of the sequence
  const int s = blockIdx.x, kvh = blockIdx.y % a.nkv, b = blockIdx.z;
  const int qgrp = blockIdx.y / a.nkv, nqgrp = gridDim.y / a.nkv;
  const int G = a.nq / a.nkv;
  const int L0 = a.len[b];
  if (tid == 0) s_n = a.rows ? a.rows[b] : count_rows(a.tok + (long)b * a.tok_sb, a.rps, a.V, L0, a.max_len, nullptr);
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;
  const int Tn = L0 + (a.shared ? 0 : n);
  const int chunk = attn_chunk(Tn, a.nsplit);
  const int p_beg = s * chunk;
  if (p_beg >= Tn) return;
  const int p_end = min(Tn, p_beg + chunk);
  const int NQ = n * G;
  const T* Kb = reinterpret_cast<const T*>(a.kc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  const T* Vt = reinterpret_cast<const T*>(a.vc) + ((long)b * a.nkv + kvh) * a.max_len * HD;  // [HD][max_len]
  const float scale = 1.0f / sqrtf(float(HD));
  const int dpv = tid % HD, qg = tid / HD;

  for (int q0 = qgrp * kQB; q0 < NQ; q0 += kQB * nqgrp) {
    const int nqb = min(kQB, NQ - q0);
    // positions past the last row of this pass are masked for every query: not visited
    const int p_stop = min(p_end, L0 + (q0 + nqb - 1) / G + 1);
    uint4 kr[NV], vr[NV];
    auto fetch = [&](int t0) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int idx = tid + v * kWG, pr = idx / VPR, c = idx - pr * VPR;
        const int p = t0 + pr;
        kr[v] = p < p_end ? ld16(Kb + (long)p * HD + c * VE) : make_uint4(0, 0, 0, 0);
        // values: VE positions of one channel; positions past the range are zero
        const int d = idx / (kTile / VE), pv = t0 + (idx - d * (kTile / VE)) * VE;
        vr[v] = pv < p_end ? ld16(Vt + (long)d * a.max_len + pv) : make_uint4(0, 0, 0, 0);
        if (pv < p_end && pv + VE > p_end) vr[v] = W::keep_first(vr[v], p_end - pv);
      }
    };
    fetch(p_beg);
    for (int idx = tid; idx < kQB * HD; idx += kWG) {
      const int ql = idx / HD, d = idx - ql * HD;
      float v = 0.f;
      if (ql < nqb) {
        const int qi = q0 + ql, i = qi / G, gg = qi - i * G;
        const long row = (long)b * a.rps + i;
        v = a.q[(row * a.nq + (kvh * G + gg)) * HD + d];
      }
      sQ[idx] = v;
    }
    float m_run[QW], l_run[QW];  // wave-uniform running max and sum of the wave's queries
#pragma unroll
    for (int k = 0; k < QW; ++k) {
      m_run[k] = -INFINITY;
      l_run[k] = 0.f;
    }
    float o[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) o[k] = 0.f;

    for (int t0 = p_beg; t0 < p_stop; t0 += kTile) {
      __syncthreads();  // the previous tile is no longer read
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int idx = tid + v * kWG, pr = idx / VPR, c = idx - pr * VPR;
        *reinterpret_cast<uint4*>(sK + pr * LDR + c * VE) = kr[v];
        const int d = idx / (kTile / VE), pl = (idx - d * (kTile / VE)) * VE;
        T ve[VE];
        __builtin_memcpy(ve, &vr[v], 16);
#pragma unroll
        for (int e = 0; e < VE; ++e) sV[(pl + e) * LDR + d] = ve[e];  // transposed into [p][d]
      }
      __syncthreads();
      if (t0 + kTile < p_stop) fetch(t0 + kTile);  // in flight while this tile is used
      {  // scores: thread -> position pl, queries qs + 4k
        const int pl = tid & (kTile - 1), qs = tid >> 6;
        float acc[SPT];
#pragma unroll
        for (int k = 0; k < SPT; ++k) acc[k] = 0.f;
#pragma unroll 4
        for (int d0 = 0; d0 < HD; d0 += VE) {
          float kf[VE];
          W::cvt(*reinterpret_cast<const uint4*>(sK + pl * LDR + d0), kf);
#pragma unroll
          for (int k = 0; k < SPT; ++k) {
            if (qs + 4 * k < nqb) {  // wave-uniform: only the live queries read Q from LDS
              const float* qp = sQ + (qs + 4 * k) * HD + d0;
#pragma unroll
              for (int e = 0; e < VE; ++e) acc[k] = fmaf(qp[e], kf[e], acc[k]);
            }
          }
        }
        const int p = t0 + pl;
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
          const int ql = qs + 4 * k;
          const int i = (q0 + ql) / G;
          const bool ok = ql < nqb && p < p_end && p <= L0 + i;
          sS[ql * (kTile + 1) + pl] = ok ? acc[k] * scale : -INFINITY;
        }
      }
      __syncthreads();
      {  // online softmax: wave w owns queries w, w+4, ...; lane = position in the tile
        const int lane = tid & 63, wid = tid >> 6;
#pragma unroll
        for (int k = 0; k < QW; ++k) {
          const int ql = wid + 4 * k;
          if (ql >= nqb) continue;  // wave-uniform
          const float sc = sS[ql * (kTile + 1) + lane];
          const float m_new = fmaxf(m_run[k], wave_max_dpp(sc));
          float alpha = 1.f, e = 0.f;
          if (m_new != -INFINITY) {
            alpha = (m_run[k] == -INFINITY) ? 0.f : expf(m_run[k] - m_new);
            e = (sc == -INFINITY) ? 0.f : expf(sc - m_new);
          }
          sP[lane * kQB + ql] = e;
          l_run[k] = l_run[k] * alpha + wave_sum_dpp(e);
          m_run[k] = m_new;
          if (lane == 0) sAlpha[ql] = alpha;
        }
      }
      __syncthreads();
      {  // o = o * alpha + P V: thread -> dim dpv, queries qg*QPT .. qg*QPT+QPT-1
#pragma unroll
        for (int k = 0; k < QPT; ++k) o[k] *= sAlpha[qg * QPT + k];
        const int live4 = (min(QPT, max(0, nqb - qg * QPT)) + 3) / 4;  // float4 groups with live queries
#pragma unroll 4
        for (int pl = 0; pl < kTile; ++pl) {
          const float v = W::get(sV, pl * LDR + dpv);
          const float4* pp = reinterpret_cast<const float4*>(sP + pl * kQB + qg * QPT);
#pragma unroll
          for (int k4 = 0; k4 < QPT / 4; ++k4) {
            if (k4 >= live4) continue;  // wave-uniform
            const float4 pv = pp[k4];
            o[4 * k4 + 0] = fmaf(pv.x, v, o[4 * k4 + 0]);
            o[4 * k4 + 1] = fmaf(pv.y, v, o[4 * k4 + 1]);
            o[4 * k4 + 2] = fmaf(pv.z, v, o[4 * k4 + 2]);
            o[4 * k4 + 3] = fmaf(pv.w, v, o[4 * k4 + 3]);
          }
        }
      }
    }
    float* P = a.part + (((long)b * a.nkv + kvh) * a.nsplit + s) * (long)a.qstride * (HD + 2);
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int ql = qg * QPT + k;
      if (ql < nqb) P[(long)(q0 + ql) * (HD + 2) + dpv] = o[k];
    }
    if ((tid & 63) == 0) {
#pragma unroll
      for (int k = 0; k < QW; ++k) {
        const int ql = (tid >> 6) + 4 * k;
        if (ql < nqb) {
          P[(long)(q0 + ql) * (HD + 2) + HD] = m_run[k];
          P[(long)(q0 + ql) * (HD + 2) + HD + 1] = l_run[k];
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 heads: decode attention on MFMA (v_mfma_f32_16x16x32_bf16), same split and partials
// ---------------------------------------------------------------------------------------------
// Workgroup (s, kvh, b) as above.  Each wave walks its own 32-position slices of the range
// (wave w takes slices w, w + 4, ...) with its own online softmax, and the four waves are merged
// in LDS at the end.  Per slice, with queries in tiles of 16 (NQT tiles per pass):
// * scores, transposed: S^T[p][q] = sum_d K[p][d] Q[q][d] with K as the A operand straight from
//   the cache and Q (fp32, split into bf16 hi + lo) as B.  The A row m of sub-tile t is position
//   8 (m / 4) + 4 t + m % 4 of the slice, so that result element r of lane (h = l / 16, j = l % 16)
//   in sub-tile t is position 8 h + 4 t + r: each lane ends up with 8 consecutive positions of
//   query column j;
// * softmax over those 8 scores, reduced over the four lanes of the column (in base 2: one
//   v_exp_f32 per probability; the maxima handed to the combine in natural units);
// * O^T[d][q] += sum_p V^T[d][p] P[q][p] with V^T (the cache holds values transposed) as A and
//   the lane's 8 probabilities (split hi + lo) as B: the K index 8 h + e of a lane is exactly its
//   position 8 h + e.
// Masked positions get probability 0; values past the range are zeroed before the product.
template <int HD, int NQT>
__global__ __launch_bounds__(kWG) void k_attn_mfma(AttnArgs a) {
  constexpr int NS = HD / 32;   // q.k steps
  constexpr int ND = HD / 16;   // 16-channel tiles of the output
  constexpr int QB = 16 * NQT;  // queries per pass
  constexpr int OP = HD + 4;    // padded LDS row of the merged output
  constexpr int QP = HD + 8;    // padded LDS row of the split queries (bf16)
  __shared__ float sm[4][QB], sl[4][QB];
  __shared__ __align__(16) float sO[QB * OP];
  __shared__ __align__(16) __bf16 sQ[2 * QB * QP];  // [hi/lo][query][channel]
  __shared__ int s_n;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, j = lane & 15, hq = lane >> 4;
  // blockIdx.y = kv head + nkv * (query-block group): many queries (a prefill) also spread over
  // the grid: this workgroup takes query blocks qgrp, qgrp + nqgrp, ... of the sequence
  const int s = blockIdx.x, kvh = blockIdx.y % a.nkv, b = blockIdx.z;
  const int qgrp = blockIdx.y / a.nkv, nqgrp = gridDim.y / a.nkv;
  const int G = a.nq / a.nkv;
  const int L0 = a.len[b];
  if (tid == 0) s_n = a.rows ? a.rows[b] : count_rows(a.tok + (long)b * a.tok_sb, a.rps, a.V, L0, a.max_len, nullptr);
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;
  const int Tn = L0 + (a.shared ? 0 : n);
  const int chunk = attn_chunk(Tn, a.nsplit);
  const int p_beg = s * chunk;
  if (p_beg >= Tn) return;
  const int p_end = min(Tn, p_beg + chunk);
  const int NQ = n * G;
  __shared__ int s_cnt[kMaxBatch];
  const int cbase = a.shi ? attn_compact_base(a, b, s_cnt) : 0;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.kc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  const uint16_t* Vt = reinterpret_cast<const uint16_t*>(a.vc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  // scores and running maxima in base 2 (times log2(e) / sqrt(hd)): one v_exp_f32 per probability
  const float c2 = 1.4426950408889634f / sqrtf(float(HD));
  const int krow = 8 * (j >> 2) + (j & 3);  // this lane's K row in sub-tile 0 (+4 in sub-tile 1)

  for (int q0 = qgrp * QB; q0 < NQ; q0 += QB * nqgrp) {
    // positions past the last row of this pass are masked for every query: not visited
    const int p_stop = min(p_end, L0 + (min(NQ, q0 + QB) - 1) / G + 1);
    // queries of this pass as bf16 hi + lo in LDS (B operand of the scores); absent ones zero
    for (int idx = tid; idx < QB * (HD / 8); idx += kWG) {
      const int q = idx / (HD / 8), c = idx - q * (HD / 8), qi = q0 + q;
      float f[8];
      if (qi < NQ) {
        const int i = qi / G, g = qi - i * G;
        const float* qp = a.q + (((long)b * a.rps + i) * a.nq + kvh * G + g) * HD + 8 * c;
        const float4 x0 = *reinterpret_cast<const float4*>(qp);
        const float4 x1 = *reinterpret_cast<const float4*>(qp + 4);
        f[0] = x0.x; f[1] = x0.y; f[2] = x0.z; f[3] = x0.w;
        f[4] = x1.x; f[5] = x1.y; f[6] = x1.z; f[7] = x1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.f;
      }
      bf16x8_t h, l;
      split_bf16x8(f, h, l);
      *reinterpret_cast<bf16x8_t*>(sQ + q * QP + 8 * c) = h;
      *reinterpret_cast<bf16x8_t*>(sQ + (QB + q) * QP + 8 * c) = l;
    }
    int lim[NQT];  // last position query column j may attend (-1: no query)
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int qi = q0 + 16 * qt + j;
      lim[qt] = qi < NQ ? L0 + qi / G : -1;
    }
    __syncthreads();
    float m_run[NQT], l_run[NQT];
    f32x4_t acc[ND][NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      m_run[qt] = -INFINITY;
      l_run[qt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt][qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // operands of one slice: K rows (A of the scores) and V^T rows (A of the output)
    uint4 ck[2][NS], cv[ND];
    // Loads are unconditional from clamped, in-range addresses (rows past the range are
    // masked as scores; value positions past the range are zeroed).
    auto load = [&](int pw, uint4 (&kk)[2][NS], uint4 (&vv)[ND]) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int p = min(pw + krow + 4 * t, p_end - 1);
        const uint16_t* kp = Kb + (long)p * HD + 8 * hq;
#pragma unroll
        for (int st = 0; st < NS; ++st) kk[t][st] = ld16(kp + 32 * st);
      }
      const int pv = pw + 8 * hq;
      const uint16_t* vp = Vt + min(pv, (p_end - 1) & ~7) + (long)j * a.max_len;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) vv[dt] = ld16(vp + (long)(16 * dt) * a.max_len);
    };
    // Two waves per SIMD hide the load latency of each other's slices (a register prefetch of
    // the next slice would cost that occupancy).
    for (int pw = p_beg + 32 * wid; pw < p_stop; pw += 128) {
      load(pw, ck, cv);
      __builtin_amdgcn_sched_barrier(0);  // all of the slice's loads are issued before any use
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        f32x4_t sc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const bf16x8_t kop = __builtin_bit_cast(bf16x8_t, ck[t][st]);
            const bf16x8_t qh = *reinterpret_cast<const bf16x8_t*>(sQ + (16 * qt + j) * QP + 32 * st + 8 * hq);
            const bf16x8_t ql = *reinterpret_cast<const bf16x8_t*>(sQ + (QB + 16 * qt + j) * QP + 32 * st + 8 * hq);
            sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qh, sc[t], 0, 0, 0);
            sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, ql, sc[t], 0, 0, 0);
          }
        }
        float pe[8];
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = pw + 8 * hq + e;
          const float v = (p < p_end && p <= lim[qt]) ? sc[e >> 2][e & 3] * c2 : -INFINITY;
          pe[e] = v;
          mx = fmaxf(mx, v);
        }
        mx = col_max(mx);
        const float m_new = fmaxf(m_run[qt], mx);
        float alpha = 1.f, rs = 0.f;
        if (m_new != -INFINITY) {
          alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);  // 0 while m_run is -inf
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pe[e] = __builtin_amdgcn_exp2f(pe[e] - m_new);  // masked: exp2(-inf) = 0
            rs += pe[e];
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) pe[e] = 0.f;
        }
        rs = col_sum(rs);
        l_run[qt] = l_run[qt] * alpha + rs;
        m_run[qt] = m_new;
        bf16x8_t ph, pl;  // probabilities as bf16 hi + lo (hardware round to nearest even)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ph[e] = (__bf16)pe[e];
          pl[e] = (__bf16)(pe[e] - (float)ph[e]);
        }
        // value positions of this lane past the range are zeroed (they may hold anything)
        const int keep = p_end - (pw + 8 * hq);
        uint32_t vm[4];
#pragma unroll
        for (int w = 0; w < 4; ++w)
          vm[w] = (2 * w < keep ? 0x0000ffffu : 0u) | (2 * w + 1 < keep ? 0xffff0000u : 0u);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
          acc[dt][qt] *= alpha;
          const uint4 vr = cv[dt];
          const bf16x8_t vop =
              __builtin_bit_cast(bf16x8_t, make_uint4(vr.x & vm[0], vr.y & vm[1], vr.z & vm[2], vr.w & vm[3]));
          acc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, ph, acc[dt][qt], 0, 0, 0);
          acc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pl, acc[dt][qt], 0, 0, 0);
        }
      }
    }
    // merge the four waves: o = sum_w o_w 2^{m_w - M}, l = sum_w l_w 2^{m_w - M} (base-2 maxima)
    if (hq == 0) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        sm[wid][16 * qt + j] = m_run[qt];
        sl[wid][16 * qt + j] = l_run[qt];
      }
    }
    __syncthreads();
    float cw[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int q = 16 * qt + j;
      const float M = fmaxf(fmaxf(sm[0][q], sm[1][q]), fmaxf(sm[2][q], sm[3][q]));
      cw[qt] = m_run[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qt] - M);
    }
    for (int w = 0; w < 4; ++w) {
      if (wid == w) {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            float4* op = reinterpret_cast<float4*>(sO + (16 * qt + j) * OP + 16 * dt + 4 * hq);
            const f32x4_t v = acc[dt][qt] * cw[qt];
            if (w == 0) {
              *op = make_float4(v[0], v[1], v[2], v[3]);
            } else {
              const float4 o = *op;
              *op = make_float4(o.x + v[0], o.y + v[1], o.z + v[2], o.w + v[3]);
            }
          }
      }
      __syncthreads();
    }
    if (a.out) {  // the only split: normalise here and write the output rows (no combine pass)
      for (int q = tid; q < QB; q += kWG) {  // thread q alone reads and writes column q
        const float M = fmaxf(fmaxf(sm[0][q], sm[1][q]), fmaxf(sm[2][q], sm[3][q]));
        float L = 0.f;
        for (int w = 0; w < 4; ++w)
          if (sm[w][q] != -INFINITY) L += sl[w][q] * __builtin_amdgcn_exp2f(sm[w][q] - M);
        sl[0][q] = L;
      }
      __syncthreads();
      for (int idx = tid; idx < QB * HD; idx += kWG) {
        const int q = idx / HD, d = idx - q * HD, qi = q0 + q;
        if (qi < NQ) {
          const int i = qi / G, g = qi - i * G;
          attn_store(a, a.out, (((long)b * a.rps + i) * a.nq + kvh * G + g) * HD + d,
                     (long)(cbase + i) * a.nq * HD + (kvh * G + g) * HD + d, sO[q * OP + d] / sl[0][q]);
        }
      }
    } else {
      float* P = a.part + (((long)b * a.nkv + kvh) * a.nsplit + s) * (long)a.qstride * (HD + 2);
      for (int idx = tid; idx < QB * HD; idx += kWG) {
        const int q = idx / HD, d = idx - q * HD;
        if (q0 + q < NQ) P[(long)(q0 + q) * (HD + 2) + d] = sO[q * OP + d];
      }
      for (int q = tid; q < QB; q += kWG) {
        if (q0 + q < NQ) {
          const float M = fmaxf(fmaxf(sm[0][q], sm[1][q]), fmaxf(sm[2][q], sm[3][q]));
          float L = 0.f;
          for (int w = 0; w < 4; ++w)
            if (sm[w][q] != -INFINITY) L += sl[w][q] * __builtin_amdgcn_exp2f(sm[w][q] - M);
          P[(long)(q0 + q) * (HD + 2) + HD] = M * 0.6931471805599453f;  // the combine's natural units
          P[(long)(q0 + q) * (HD + 2) + HD + 1] = L;
        }
      }
    }
    __syncthreads();  // sm, sl, sO are reused by the next pass
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 heads, many queries per kv head (a prefill; one split): the MFMA attention above with the
// queries spread over the waves instead of the positions.  Workgroup (query block, kv head,
// sequence) takes 64 queries -- 16 per wave, each wave with its own online softmax over every
// position its queries may attend, so no merge across waves -- and walks the positions in
// 64-position tiles staged once in LDS for all four waves: keys [position][channel] and values
// transposed [channel][position] (as the cache holds them), each thread moving 16-byte pieces
// of whole rows; the next tile's loads are in flight while the current one is multiplied (one
// barrier per tile).  Per 32-position slice of a tile the products are those of k_attn_mfma:
// S^T = K Q^T with Q (split bf16 hi + lo) held in registers for the whole walk and O^T += V^T P^T.
// The softmax runs once per tile over the lane's sixteen positions (one max, sum and rescale of
// the output per 64 positions), in base 2: scores times log2(e) / sqrt(hd), probabilities by
// v_exp_f32, split into bf16 hi + lo by the hardware conversion (round to nearest even); tiles
// inside every query's causal reach skip the masks.  The softmax is VALU work, not MFMA: per
// slice it had cost 13 VALU instructions per MFMA.  LDS rows are XOR-swizzled in 16-byte slots so that
// the sixteen rows a quarter-wave reads fall on distinct banks: key row r slot s at
// s ^ ((r & 3) | (r >> 3 & 3) << 2), value row d slot s at s ^ ((d ^ d >> 3) & 7).  Value
// positions past the range are stored as zeros (the cache may hold anything there); key rows
// past it re-read the last one and their scores are masked.
constexpr int kPfQ = 64;   // queries per workgroup
constexpr int kPfT = 64;   // positions per LDS tile

__device__ __forceinline__ int pf_kswz(int r) { return (r & 3) | ((r >> 3) & 3) << 2; }

__device__ __forceinline__ int pf_vswz(int d) { return (d ^ (d >> 3)) & 7; }

__global__ __launch_bounds__(kWG, 2) void k_attn_prefill(AttnArgs a) {
  constexpr int HD = 128, NS = HD / 32, ND = HD / 16;
  __shared__ __align__(16) uint16_t sK[2][kPfT * HD];
  __shared__ __align__(16) uint16_t sV[2][HD * kPfT];
  __shared__ int s_n;
  __shared__ int s_cnt[kMaxBatch];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, j = lane & 15, hq = lane >> 4;
  // the first half of the grid takes the query blocks longest first, the second half shortest
  // first: workgroups i and i + half, which tend to share a compute unit, get complementary walks
  const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int half = gridDim.x * gridDim.y * gridDim.z / 2;
  const int qblk = lin < half ? gridDim.x - 1 - blockIdx.x : blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.nq / a.nkv;
  const int L0 = a.len[b];
  if (tid == 0) s_n = a.rows ? a.rows[b] : count_rows(a.tok + (long)b * a.tok_sb, a.rps, a.V, L0, a.max_len, nullptr);
  const int cbase = a.shi ? attn_compact_base(a, b, s_cnt) : 0;  // contains a barrier
  __syncthreads();
  const int n = s_n;
  const int NQ = n * G, q0 = qblk * kPfQ;
  if (n == 0 || q0 >= NQ) return;
  const int Tn = L0 + (a.shared ? 0 : n);
  // positions past the last query row of the block are masked for every query: not visited
  const int p_end = min(Tn, L0 + (min(NQ, q0 + kPfQ) - 1) / G + 1);
  const int ntile = (p_end + kPfT - 1) / kPfT;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.kc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  const uint16_t* Vt = reinterpret_cast<const uint16_t*>(a.vc) + ((long)b * a.nkv + kvh) * a.max_len * HD;

  // this wave's 16 queries as the B operand of the scores, split bf16 hi + lo (zero if absent)
  const int qi = q0 + 16 * wid + j;
  const int qrow = qi / G, qg = qi - qrow * G;
  bf16x8_t qh[NS], ql[NS];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    float f[8];
    if (qi < NQ) {
      const float* qp = a.q + (((long)b * a.rps + qrow) * a.nq + kvh * G + qg) * HD + 32 * st + 8 * hq;
      const float4 x0 = *reinterpret_cast<const float4*>(qp);
      const float4 x1 = *reinterpret_cast<const float4*>(qp + 4);
      f[0] = x0.x; f[1] = x0.y; f[2] = x0.z; f[3] = x0.w;
      f[4] = x1.x; f[5] = x1.y; f[6] = x1.z; f[7] = x1.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = 0.f;
    }
    split_bf16x8(f, qh[st], ql[st]);
  }
  const int lim = qi < NQ ? L0 + qrow : -1;  // last position query column j may attend

  // staging: thread t moves key slots z = t + 256 k (row z / 16, slot z % 16) and value slots
  // (channel z / 8, slot z % 8) of a tile
  uint4 gk[4], gv[4];
  auto gload = [&](int p0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int z = tid + kWG * k;
      const int pr = min(p0 + (z >> 4), p_end - 1);
      gk[k] = ld16(Kb + (long)pr * HD + 8 * (z & 15));
      const int pv = min(p0 + 8 * (z & 7), (p_end - 1) & ~7);
      gv[k] = ld16(Vt + (long)(z >> 3) * a.max_len + pv);
    }
  };
  auto sstore = [&](int buf, int p0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int z = tid + kWG * k;
      const int r = z >> 4, d = z >> 3, sv = z & 7;
      *reinterpret_cast<uint4*>(&sK[buf][r * HD + 8 * ((z & 15) ^ pf_kswz(r))]) = gk[k];
      // value positions p0 + 8 sv + e past the range are zeroed
      const int keep = p_end - (p0 + 8 * sv);
      uint4 v = gv[k];
      if (keep < 8) {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = (2 * q < keep ? w[q] & 0x0000ffffu : 0u) | (2 * q + 1 < keep ? w[q] & 0xffff0000u : 0u);
        v = make_uint4(w[0], w[1], w[2], w[3]);
      }
      *reinterpret_cast<uint4*>(&sV[buf][d * kPfT + 8 * (sv ^ pf_vswz(d))]) = v;
    }
  };

  // running max and sum in base-2 units: scores are taken times log2(e) / sqrt(hd), so that one
  // v_exp_f32 gives each probability
  float m_run = -INFINITY, l_run = 0.f;
  f32x4_t acc[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int krow = 8 * (j >> 2) + (j & 3);  // this lane's key row in sub-tile 0 of a slice (+4 in 1)
  const float c2 = 1.4426950408889634f / sqrtf(float(HD));
  // the first query of the wave attends the fewest positions; a tile that ends within its reach
  // (and within the range) needs no mask when all sixteen queries are present
  const int q_first = q0 + 16 * wid;
  const int lim_all = q_first + 15 < NQ ? L0 + q_first / G : -1;

  gload(0);
  sstore(0, 0);
  __syncthreads();
  for (int t = 0; t < ntile; ++t) {
    const int p0 = t * kPfT, buf = t & 1;
    if (t + 1 < ntile) gload(p0 + kPfT);
    __builtin_amdgcn_sched_barrier(0);  // the next tile's loads are issued before this one's use
    // scores of the tile: lane (j, hq) holds positions p0 + 32 sl + 8 hq + e of query column j
    float pe[2][8];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      f32x4_t sc[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        sc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        const int r = 32 * sl + krow + 4 * tt;
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          const bf16x8_t kop =
              *reinterpret_cast<const bf16x8_t*>(&sK[buf][r * HD + 8 * ((4 * st + hq) ^ pf_kswz(r))]);
          sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qh[st], sc[tt], 0, 0, 0);
          sc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, ql[st], sc[tt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[sl][e] = sc[e >> 2][e & 3] * c2;
    }
    if (!(p0 + kPfT - 1 <= lim_all && p0 + kPfT <= p_end)) {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = p0 + 32 * sl + 8 * hq + e;
          if (!(p < p_end && p <= lim)) pe[sl][e] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
      for (int e = 0; e < 8; ++e) mx = fmaxf(mx, pe[sl][e]);
    mx = col_max(mx);
    const float m_new = fmaxf(m_run, mx);
    float alpha = 1.f, rs = 0.f;
    if (m_new != -INFINITY) {
      alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while m_run is -inf
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pe[sl][e] = __builtin_amdgcn_exp2f(pe[sl][e] - m_new);  // masked: exp2(-inf) = 0
          rs += pe[sl][e];
        }
    } else {
#pragma unroll
      for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int e = 0; e < 8; ++e) pe[sl][e] = 0.f;
    }
    rs = col_sum(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) acc[dt] *= alpha;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      // probabilities as bf16 hi + lo (hardware round to nearest even)
      bf16x8_t ph, pl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ph[e] = (__bf16)pe[sl][e];
        pl[e] = (__bf16)(pe[sl][e] - (float)ph[e]);
      }
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        const int d = 16 * dt + j;
        const bf16x8_t vop =
            *reinterpret_cast<const bf16x8_t*>(&sV[buf][d * kPfT + 8 * ((4 * sl + hq) ^ pf_vswz(d))]);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, ph, acc[dt], 0, 0, 0);
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pl, acc[dt], 0, 0, 0);
      }
    }
    if (t + 1 < ntile) sstore(buf ^ 1, p0 + kPfT);  // that buffer's readers passed the last barrier
    __syncthreads();
  }
  // lane (j, hq) holds channels 16 dt + 4 hq + r of query column j
  if (qi < NQ && l_run > 0.f) {
    const float inv = 1.0f / l_run;
    const long o = (((long)b * a.rps + qrow) * a.nq + kvh * G + qg) * HD;
    const long c = (long)(cbase + qrow) * a.nq * HD + (kvh * G + qg) * HD;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = 16 * dt + 4 * hq + r;
        attn_store(a, a.out, o + d, c + d, acc[dt][r] * inv);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 heads with a batch of sequences (B x kv heads fill the GPU): the same MFMA attention with
// the keys and values staged through LDS.  Reading K and V^T straight in the operand layout
// fetches 64 bytes of each of 16 rows per load instruction, a pattern that streams well below
// the read ceiling; here each wave fetches SP-position superslices row-contiguously -- keys as
// four 256-byte rows per load, values as 64 / (SP / 8) channel rows of 2 SP bytes -- into a
// private LDS tile (XOR-swizzled in 16-byte units) and reads the operands from there.  NB
// superslices per wave are in flight in registers while one is used; the tile is the wave's own,
// so the streaming loop has no barrier.  Per 32-position half the products are those of
// k_attn_mfma.  NWV waves per workgroup (NWV x tile bytes of LDS) share the position range
// round-robin and merge at the end.
// The cache is read once per step and is larger than the caches, so keys are loaded
// nontemporally; values too when every 2 SP-byte segment of a value row is a whole 128-byte line
// (max_len a multiple of 64).  Otherwise each segment straddles two lines and cached loads let
// L2 serve the shared line once.  Measured at 32 sequences x 8 kv heads x 8192 positions:
// 187 -> 167 us (0.67 -> 0.75 of the HBM peak) with line-aligned rows.
template <int NQT, int NWV, int SP, int NB, bool VNT>
__global__ __launch_bounds__(64 * NWV) void k_attn_lds(AttnArgs a) {
  constexpr int HD = 128;
  constexpr int NT = 64 * NWV;  // threads
  constexpr int NS = HD / 32;   // q.k steps
  constexpr int ND = HD / 16;   // 16-channel tiles of the output
  constexpr int QB = 16 * NQT;  // queries per pass
  constexpr int OP = HD + 4;    // padded LDS row of the merged output
  constexpr int QP = HD + 8;    // padded LDS row of the split queries (bf16)
  constexpr int KT = SP * HD * 2;   // bytes of a key tile: SP rows x 256 B (16 units)
  constexpr int VU = SP / 8;        // 16-byte units of a value channel row
  constexpr int VT = HD * SP * 2;   // bytes of a value tile: 128 channel rows x 2 SP bytes
  constexpr int LK = SP / 4;        // key loads per lane and superslice (4 rows each)
  constexpr int VR = 64 / VU;       // value channel rows per load
  constexpr int LV = HD / VR;       // value loads per lane and superslice
  static_assert(SP == 32 || SP == 64, "superslices of one or two 32-position halves");
  __shared__ float sm[NWV][QB], sl[NWV][QB];
  __shared__ __align__(16) __bf16 sQ[2 * QB * QP];  // [hi/lo][query][channel]
  __shared__ __align__(16) char sKV[NWV][KT + VT];   // each wave's tiles
  __shared__ int s_n;
  // the merged output reuses the tiles: it is written after every wave has left the streaming
  // loop (behind a barrier) and read before the next pass stores tiles again (another barrier)
  float* sO = reinterpret_cast<float*>(&sKV[0][0]);
  static_assert(QB * OP * 4 <= NWV * (KT + VT), "merged output fits in the tiles");
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, j = lane & 15, hq = lane >> 4;
  const int s = blockIdx.x, kvh = blockIdx.y % a.nkv, b = blockIdx.z;
  const int qgrp = blockIdx.y / a.nkv, nqgrp = gridDim.y / a.nkv;
  const int G = a.nq / a.nkv;
  const int L0 = a.len[b];
  if (tid == 0) s_n = a.rows ? a.rows[b] : count_rows(a.tok + (long)b * a.tok_sb, a.rps, a.V, L0, a.max_len, nullptr);
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;
  const int Tn = L0 + (a.shared ? 0 : n);
  const int chunk = attn_chunk(Tn, a.nsplit);
  const int p_beg = s * chunk;
  if (p_beg >= Tn) return;
  const int p_end = min(Tn, p_beg + chunk);
  const int NQ = n * G;
  __shared__ int s_cnt[kMaxBatch];
  const int cbase = a.shi ? attn_compact_base(a, b, s_cnt) : 0;
  const uint16_t* Kb = reinterpret_cast<const uint16_t*>(a.kc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  const uint16_t* Vt = reinterpret_cast<const uint16_t*>(a.vc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  // scores and running maxima in base 2 (times log2(e) / sqrt(hd)): one v_exp_f32 per probability
  const float c2 = 1.4426950408889634f / sqrtf(float(HD));
  const int krow = 8 * (j >> 2) + (j & 3);  // this lane's K row in sub-tile 0 (+4 in sub-tile 1)
  char* tK = sKV[wid];
  char* tV = sKV[wid] + KT;
  // value rows: 16 distinct banks for the 16 rows a quarter wave reads at one unit
  auto vswz = [](int r) { return SP == 64 ? (r & 7) ^ ((r >> 3) & 1) : (r >> 2) & 3; };

  for (int q0 = qgrp * QB; q0 < NQ; q0 += QB * nqgrp) {
    const int p_stop = min(p_end, L0 + (min(NQ, q0 + QB) - 1) / G + 1);
    for (int idx = tid; idx < QB * (HD / 8); idx += NT) {
      const int q = idx / (HD / 8), c = idx - q * (HD / 8), qi = q0 + q;
      float f[8];
      if (qi < NQ) {
        const int i = qi / G, g = qi - i * G;
        const float* qp = a.q + (((long)b * a.rps + i) * a.nq + kvh * G + g) * HD + 8 * c;
        const float4 x0 = *reinterpret_cast<const float4*>(qp);
        const float4 x1 = *reinterpret_cast<const float4*>(qp + 4);
        f[0] = x0.x; f[1] = x0.y; f[2] = x0.z; f[3] = x0.w;
        f[4] = x1.x; f[5] = x1.y; f[6] = x1.z; f[7] = x1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.f;
      }
      bf16x8_t h, l;
      split_bf16x8(f, h, l);
      *reinterpret_cast<bf16x8_t*>(sQ + q * QP + 8 * c) = h;
      *reinterpret_cast<bf16x8_t*>(sQ + (QB + q) * QP + 8 * c) = l;
    }
    int lim[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const int qi = q0 + 16 * qt + j;
      lim[qt] = qi < NQ ? L0 + qi / G : -1;
    }
    __syncthreads();
    float m_run[NQT], l_run[NQT];
    f32x4_t acc[ND][NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      m_run[qt] = -INFINITY;
      l_run[qt] = 0.f;
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) acc[dt][qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    // this pass's queries as B operands: one 16-query tile is held in registers for the whole
    // pass, two are read from LDS at each use (registers for the second tile's accumulators)
    constexpr bool QREG = NQT == 1;
    bf16x8_t qH[QREG ? NQT : 1][NS], qL[QREG ? NQT : 1][NS];
    if constexpr (QREG) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          qH[qt][st] = *reinterpret_cast<const bf16x8_t*>(sQ + (16 * qt + j) * QP + 32 * st + 8 * hq);
          qL[qt][st] = *reinterpret_cast<const bf16x8_t*>(sQ + (QB + 16 * qt + j) * QP + 32 * st + 8 * hq);
        }
    }
    auto qop = [&](int qt, int st, int lo) {
      if constexpr (QREG) return lo ? qL[qt][st] : qH[qt][st];
      return *reinterpret_cast<const bf16x8_t*>(sQ + (lo * QB + 16 * qt + j) * QP + 32 * st + 8 * hq);
    };
    // superslice loads, unconditional from clamped in-range addresses: key row 4 i + lane / 16
    // (unit lane % 16); value channel row VR i + lane / VU (unit lane % VU = 8 positions)
    uint4 rk[NB][LK], rv[NB][LV];
    auto load = [&](uint4 (&k)[LK], uint4 (&v)[LV], int pw) {
#pragma unroll
      for (int i = 0; i < LK; ++i) {
        const int p = min(pw + 4 * i + (lane >> 4), p_end - 1);
        k[i] = ld_stream(Kb + (long)p * HD + 8 * (lane & 15));
      }
#pragma unroll
      for (int i = 0; i < LV; ++i) {
        const int d = VR * i + lane / VU;
        const int pv = min(pw + 8 * (lane % VU), (p_end - 1) & ~7);
        v[i] = VNT ? ld_stream(Vt + (long)d * a.max_len + pv) : ld16(Vt + (long)d * a.max_len + pv);
      }
    };
    // a buffer into the wave's tiles; value positions past the range become zero
    auto store = [&](const uint4 (&k)[LK], const uint4 (&v)[LV], int pw) {
#pragma unroll
      for (int i = 0; i < LK; ++i) {
        const int r = 4 * i + (lane >> 4), u = lane & 15;
        *reinterpret_cast<uint4*>(tK + r * 256 + ((u ^ (r & 15)) << 4)) = k[i];
      }
#pragma unroll
      for (int i = 0; i < LV; ++i) {
        const int d = VR * i + lane / VU, uv = lane % VU;
        const int keep = p_end - (pw + 8 * uv);
        uint4 x = v[i];
        if (keep < 8) {
          uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= keep) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
          x = make_uint4(w[0], w[1], w[2], w[3]);
        }
        *reinterpret_cast<uint4*>(tV + d * (2 * SP) + ((uv ^ vswz(d)) << 4)) = x;
      }
    };
    auto compute = [&](int pw) {
#pragma unroll
      for (int hh = 0; hh < SP / 32; ++hh) {  // 32-position halves
        const int ph = pw + 32 * hh;
        if (ph >= p_stop) break;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
          f32x4_t sc[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            sc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            const int r = 32 * hh + krow + 4 * t;
#pragma unroll
            for (int st = 0; st < NS; ++st) {
              const int u = 4 * st + hq;
              const bf16x8_t kop = *reinterpret_cast<const bf16x8_t*>(tK + r * 256 + ((u ^ (r & 15)) << 4));
              sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop(qt, st, 0), sc[t], 0, 0, 0);
              sc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop(qt, st, 1), sc[t], 0, 0, 0);
            }
          }
          float pe[8];
          float mx = -INFINITY;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int p = ph + 8 * hq + e;
            const float v = (p < p_end && p <= lim[qt]) ? sc[e >> 2][e & 3] * c2 : -INFINITY;
            pe[e] = v;
            mx = fmaxf(mx, v);
          }
          mx = col_max(mx);
          const float m_new = fmaxf(m_run[qt], mx);
          float alpha = 1.f, rs = 0.f;
          if (m_new != -INFINITY) {
            alpha = __builtin_amdgcn_exp2f(m_run[qt] - m_new);  // 0 while m_run is -inf
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              pe[e] = __builtin_amdgcn_exp2f(pe[e] - m_new);  // masked: exp2(-inf) = 0
              rs += pe[e];
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) pe[e] = 0.f;
          }
          rs = col_sum(rs);
          l_run[qt] = l_run[qt] * alpha + rs;
          m_run[qt] = m_new;
          bf16x8_t pH, pL;  // probabilities as bf16 hi + lo (hardware round to nearest even)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pH[e] = (__bf16)pe[e];
            pL[e] = (__bf16)(pe[e] - (float)pH[e]);
          }
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            acc[dt][qt] *= alpha;
            const int d = 16 * dt + j, u = 4 * hh + hq;
            const bf16x8_t vop = *reinterpret_cast<const bf16x8_t*>(tV + d * (2 * SP) + ((u ^ vswz(d)) << 4));
            acc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pH, acc[dt][qt], 0, 0, 0);
            acc[dt][qt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pL, acc[dt][qt], 0, 0, 0);
          }
        }
      }
    };
    // wave w takes superslices w, w + NWV, ... ; loads past the end re-read the clamped last
    // position (cached) and are not used, so every iteration issues the same loads
    constexpr int STEP = NWV * SP;
    const int pw0 = p_beg + SP * wid;
#pragma unroll
    for (int c = 0; c < NB; ++c) load(rk[c], rv[c], pw0 + c * STEP);
    for (int pw = pw0; pw < p_stop; pw += NB * STEP) {
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        const int pc = pw + c * STEP;
        if (c == 0 || pc < p_stop) store(rk[c], rv[c], pc);
        load(rk[c], rv[c], pc + NB * STEP);
        if (c == 0 || pc < p_stop) compute(pc);
      }
    }
    // merge the waves: o = sum_w o_w 2^{m_w - M}, l = sum_w l_w 2^{m_w - M} (base-2 maxima)
    if (hq == 0) {
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        sm[wid][16 * qt + j] = m_run[qt];
        sl[wid][16 * qt + j] = l_run[qt];
      }
    }
    __syncthreads();
    auto row_max = [&](int q) {
      float M = sm[0][q];
#pragma unroll
      for (int w = 1; w < NWV; ++w) M = fmaxf(M, sm[w][q]);
      return M;
    };
    float cw[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      const float M = row_max(16 * qt + j);
      cw[qt] = m_run[qt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[qt] - M);
    }
    for (int w = 0; w < NWV; ++w) {
      if (wid == w) {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
          for (int dt = 0; dt < ND; ++dt) {
            float4* op = reinterpret_cast<float4*>(sO + (16 * qt + j) * OP + 16 * dt + 4 * hq);
            const f32x4_t v = acc[dt][qt] * cw[qt];
            if (w == 0) {
              *op = make_float4(v[0], v[1], v[2], v[3]);
            } else {
              const float4 o = *op;
              *op = make_float4(o.x + v[0], o.y + v[1], o.z + v[2], o.w + v[3]);
            }
          }
      }
      __syncthreads();
    }
    auto row_sum = [&](int q, float M) {
      float L = 0.f;
      for (int w = 0; w < NWV; ++w)
        if (sm[w][q] != -INFINITY) L += sl[w][q] * __builtin_amdgcn_exp2f(sm[w][q] - M);
      return L;
    };
    if (a.out) {  // the only split: normalise here and write the output rows (no combine pass)
      for (int q = tid; q < QB; q += NT) sl[0][q] = row_sum(q, row_max(q));
      __syncthreads();
      for (int idx = tid; idx < QB * HD; idx += NT) {
        const int q = idx / HD, d = idx - q * HD, qi = q0 + q;
        if (qi < NQ) {
          const int i = qi / G, g = qi - i * G;
          attn_store(a, a.out, (((long)b * a.rps + i) * a.nq + kvh * G + g) * HD + d,
                     (long)(cbase + i) * a.nq * HD + (kvh * G + g) * HD + d, sO[q * OP + d] / sl[0][q]);
        }
      }
    } else {
      float* P = a.part + (((long)b * a.nkv + kvh) * a.nsplit + s) * (long)a.qstride * (HD + 2);
      for (int idx = tid; idx < QB * HD; idx += NT) {
        const int q = idx / HD, d = idx - q * HD;
        if (q0 + q < NQ) P[(long)(q0 + q) * (HD + 2) + d] = sO[q * OP + d];
      }
      for (int q = tid; q < QB; q += NT) {
        if (q0 + q < NQ) {
          const float M = row_max(q);
          P[(long)(q0 + q) * (HD + 2) + HD] = M * 0.6931471805599453f;  // the combine's natural units
          P[(long)(q0 + q) * (HD + 2) + HD + 1] = row_sum(q, M);
        }
      }
    }
    __syncthreads();  // sm, sl, sO are reused by the next pass
  }
}

// Merge the split partials of one (row, query head): o = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}.
// kWG / HD thread groups take every (kWG / HD)-th split, summed in LDS at the end.
template <int HD>
__global__ __launch_bounds__(kWG) void k_attn_combine(AttnArgs a, float* out) {
  constexpr int NG = kWG / HD;
  __shared__ float sw[kMaxSplit];
  __shared__ float sl[kMaxSplit];
  __shared__ float so[NG][HD];
  __shared__ float sL[NG];
  const int item = blockIdx.x, tid = threadIdx.x, d = tid % HD, grp = tid / HD;
  const int row = item / a.nq, h = item - row * a.nq;
  const int b = row / a.rps, i = row - b * a.rps;
  const int n = a.rows ? a.rows[b] : count_rows(a.tok + (long)b * a.tok_sb, a.rps, a.V, a.len[b], a.max_len, nullptr);
  if (i >= n) return;
  __shared__ int s_cnt[kMaxBatch];
  const int cbase = a.shi ? attn_compact_base(a, b, s_cnt) : 0;
  const int G = a.nq / a.nkv, kvh = h / G, qi = i * G + (h - kvh * G);
  const int Tn = a.len[b] + (a.shared ? 0 : n);
  const int chunk = attn_chunk(Tn, a.nsplit);
  const int ns = min(a.nsplit, (Tn + chunk - 1) / chunk);
  const long sstride = (long)a.qstride * (HD + 2);
  const float* P = a.part + ((long)b * a.nkv + kvh) * a.nsplit * sstride + (long)qi * (HD + 2);
  for (int s = tid; s < ns; s += kWG) {
    const float l = P[s * sstride + HD + 1];
    sw[s] = l > 0.f ? P[s * sstride + HD] : -INFINITY;
    sl[s] = l;
  }
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, sw[s]);
  __syncthreads();
  for (int s = tid; s < ns; s += kWG) sw[s] = sl[s] > 0.f ? expf(sw[s] - M) : 0.f;
  __syncthreads();
  float L = 0.f, O = 0.f;
#pragma unroll 8
  for (int s = grp; s < ns; s += NG) {
    L = fmaf(sl[s], sw[s], L);
    O = fmaf(P[s * sstride + d], sw[s], O);
  }
  so[grp][d] = O;
  if (d == 0) sL[grp] = L;
  __syncthreads();
  if (grp == 0) {
    float Ot = so[0][d], Lt = sL[0];
#pragma unroll
    for (int q = 1; q < NG; ++q) {
      Ot += so[q][d];
      Lt += sL[q];
    }
    attn_store(a, out, ((long)row * a.nq + h) * HD + d, (long)(cbase + i) * a.nq * HD + h * HD + d, Ot / Lt);
  }
}

// bf16 caches take the MFMA kernel: one query tile per pass, or two when a sequence has more
// than 16 queries and the cache is large enough that a second pass over it would cost more than
// the two-tile kernel's lower occupancy (64 MB of keys and values); fp32 caches the VALU kernel.
// Query-block groups per (split, kv head, sequence): enough to give the launch ~2048 workgroups
// when a sequence has many query blocks.
inline int attn_qgroups(const AttnArgs& a, int qb) {
  const int blocks = (a.qstride + qb - 1) / qb;
  const int want = 2048 / (a.nsplit * a.nkv * a.B);
  const int g = blocks < want ? blocks : want;
  return g < 1 ? 1 : g;
}

template <int HD>
void launch_attention(AttnArgs a, int wdtype, float* out, hipStream_t st) {
  a.out = nullptr;
  if (wdtype == MTP_BF16) {
    if (a.nsplit == 1) a.out = out;
    const double kv_bytes = 4.0 * a.B * a.nkv * (double)a.max_len * HD;
    if constexpr (HD == 128) {
      // a batch whose (sequence, kv head) pairs fill the GPU on their own, over a long cache:
      // the LDS-staged kernel (one wave per SIMD, registers free for the prefetch), for up to
      // two query tiles per kv head
      if (a.B * a.nkv >= 128 && a.max_len >= 1024 && a.qstride <= 32) {
        if (a.qstride <= 16) {
          dim3 grid(a.nsplit, a.nkv * attn_qgroups(a, 16), a.B);
          if (a.max_len % 64 == 0)
            hipLaunchKernelGGL((k_attn_lds<1, 4, 64, 1, true>), grid, dim3(kWG), 0, st, a);
          else
            hipLaunchKernelGGL((k_attn_lds<1, 4, 64, 1, false>), grid, dim3(kWG), 0, st, a);
        } else {
          // two query tiles (a catch-up of a few rows per sequence): 32-position superslices keep
          // the operands and the prefetch in registers (64 spill); their value rows are 64-byte
          // half lines, so the loads stay cached
          dim3 grid(a.nsplit, a.nkv * attn_qgroups(a, 32), a.B);
          hipLaunchKernelGGL((k_attn_lds<2, 4, 32, 1, false>), grid, dim3(kWG), 0, st, a);
        }
        if (!a.out) hipLaunchKernelGGL((k_attn_combine<HD>), dim3(a.B * a.rps * a.nq), dim3(kWG), 0, st, a, out);
        return;
      }
    }
    if constexpr (HD == 128) {
      // many queries per kv head in one split (a prefill): query blocks over the grid, K/V tiles
      // through LDS once per 64 queries
      if (a.nsplit == 1 && a.qstride >= 256) {
        dim3 grid((a.qstride + kPfQ - 1) / kPfQ, a.nkv, a.B);
        hipLaunchKernelGGL(k_attn_prefill, grid, dim3(kWG), 0, st, a);
        return;
      }
    }
    if (a.qstride <= 16 || kv_bytes < 64.0 * 1024 * 1024) {
      dim3 grid(a.nsplit, a.nkv * attn_qgroups(a, 16), a.B);
      hipLaunchKernelGGL((k_attn_mfma<HD, 1>), grid, dim3(kWG), 0, st, a);
    } else {
      dim3 grid(a.nsplit, a.nkv * attn_qgroups(a, 32), a.B);
      hipLaunchKernelGGL((k_attn_mfma<HD, 2>), grid, dim3(kWG), 0, st, a);
    }
  } else {
    dim3 grid(a.nsplit, a.nkv * attn_qgroups(a, kQB), a.B);
    hipLaunchKernelGGL((k_attn<F32, HD>), grid, dim3(kWG), 0, st, a);
  }
  if (!a.out) hipLaunchKernelGGL((k_attn_combine<HD>), dim3(a.B * a.rps * a.nq), dim3(kWG), 0, st, a, out);
}

hipError_t run_attention(const AttnArgs& a, int hd, int wdtype, float* out, hipStream_t st) {
  if (hd == 128)
    launch_attention<128>(a, wdtype, out, st);
  else
    launch_attention<64>(a, wdtype, out, st);
  return hipGetLastError();
}

}  // namespace mtp
