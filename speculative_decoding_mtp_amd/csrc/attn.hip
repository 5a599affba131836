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

// ---------------------------------------------------------------------------------------------
// decode attention, split over the cached positions
// ---------------------------------------------------------------------------------------------
// Workgroup (s, kvh, b) handles positions [s*chunk, min(T, (s+1)*chunk)) of sequence b, where
// T = len[b] + rows, for all queries (row i, query head kvh*G + g) of the sequence.  K/V tiles of
// 64 positions are staged through LDS; an online softmax keeps (m, l, o) per query.  Output per
// query: the unnormalised o, the running max m and the sum l.
constexpr int kTile = 64;  // cached positions per LDS tile
constexpr int kQB = 32;    // queries per pass

// Workgroup (s, kvh, b) handles positions [s*chunk, min(T, (s+1)*chunk)) of sequence b, where
// T = len[b] + rows, for every query (row i, query head kvh*G + g) of the sequence.  K/V tiles
// of 64 positions go through registers (the next tile is fetched while the current one is
// used) into LDS; an online softmax keeps (m, l, o) per query.  Output per query: the
// unnormalised o, the running max m and the sum l.
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
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.nq / a.nkv;
  const int L0 = a.len[b];
  if (tid == 0) s_n = count_rows(a.tok + (long)b * a.tok_sb, a.rps, a.V, L0, a.max_len, nullptr);
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;
  const int Tn = L0 + n;
  const int chunk = attn_chunk(Tn, a.nsplit);
  const int p_beg = s * chunk;
  if (p_beg >= Tn) return;
  const int p_end = min(Tn, p_beg + chunk);
  const int NQ = n * G;
  const T* Kb = reinterpret_cast<const T*>(a.kc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  const T* Vb = reinterpret_cast<const T*>(a.vc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  const float scale = 1.0f / sqrtf(float(HD));
  const int dpv = tid % HD, qg = tid / HD;

  for (int q0 = 0; q0 < NQ; q0 += kQB) {
    const int nqb = min(kQB, NQ - q0);
    uint4 kr[NV], vr[NV];
    auto fetch = [&](int t0) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int idx = tid + v * kWG, pr = idx / VPR, c = idx - pr * VPR;
        const int p = t0 + pr;
        kr[v] = p < p_end ? ld16(Kb + (long)p * HD + c * VE) : make_uint4(0, 0, 0, 0);
        vr[v] = p < p_end ? ld16(Vb + (long)p * HD + c * VE) : make_uint4(0, 0, 0, 0);
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

    for (int t0 = p_beg; t0 < p_end; t0 += kTile) {
      __syncthreads();  // the previous tile is no longer read
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int idx = tid + v * kWG, pr = idx / VPR, c = idx - pr * VPR;
        *reinterpret_cast<uint4*>(sK + pr * LDR + c * VE) = kr[v];
        *reinterpret_cast<uint4*>(sV + pr * LDR + c * VE) = vr[v];
      }
      __syncthreads();
      if (t0 + kTile < p_end) fetch(t0 + kTile);  // in flight while this tile is used
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

// Merge the split partials of one (row, query head): o = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}.
template <int HD>
__global__ __launch_bounds__(HD) void k_attn_combine(AttnArgs a, float* out) {
  __shared__ float sw[kMaxSplit];
  __shared__ float sl[kMaxSplit];
  const int item = blockIdx.x, d = threadIdx.x;
  const int row = item / a.nq, h = item - row * a.nq;
  const int b = row / a.rps, i = row - b * a.rps;
  const int n = count_rows(a.tok + (long)b * a.tok_sb, a.rps, a.V, a.len[b], a.max_len, nullptr);
  if (i >= n) return;
  const int G = a.nq / a.nkv, kvh = h / G, qi = i * G + (h - kvh * G);
  const int Tn = a.len[b] + n;
  const int chunk = attn_chunk(Tn, a.nsplit);
  const int ns = min(a.nsplit, (Tn + chunk - 1) / chunk);
  const long sstride = (long)a.qstride * (HD + 2);
  const float* P = a.part + ((long)b * a.nkv + kvh) * a.nsplit * sstride + (long)qi * (HD + 2);
  for (int s = d; s < ns; s += HD) {
    const float l = P[s * sstride + HD + 1];
    sw[s] = l > 0.f ? P[s * sstride + HD] : -INFINITY;
    sl[s] = l;
  }
  __syncthreads();
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, sw[s]);
  __syncthreads();
  for (int s = d; s < ns; s += HD) sw[s] = sl[s] > 0.f ? expf(sw[s] - M) : 0.f;
  __syncthreads();
  float L = 0.f, O = 0.f;
#pragma unroll 8
  for (int s = 0; s < ns; ++s) {
    L = fmaf(sl[s], sw[s], L);
    O = fmaf(P[s * sstride + d], sw[s], O);
  }
  out[((long)row * a.nq + h) * HD + d] = O / L;
}

hipError_t run_attention(const AttnArgs& a, int hd, int wdtype, float* out, hipStream_t st) {
  dim3 grid(a.nsplit, a.nkv, a.B);
  const int items = a.B * a.rps * a.nq;
  if (hd == 128) {
    if (wdtype == MTP_BF16)
      hipLaunchKernelGGL((k_attn<BF16, 128>), grid, dim3(kWG), 0, st, a);
    else
      hipLaunchKernelGGL((k_attn<F32, 128>), grid, dim3(kWG), 0, st, a);
    hipLaunchKernelGGL((k_attn_combine<128>), dim3(items), dim3(128), 0, st, a, out);
  } else {
    if (wdtype == MTP_BF16)
      hipLaunchKernelGGL((k_attn<BF16, 64>), grid, dim3(kWG), 0, st, a);
    else
      hipLaunchKernelGGL((k_attn<F32, 64>), grid, dim3(kWG), 0, st, a);
    hipLaunchKernelGGL((k_attn_combine<64>), dim3(items), dim3(64), 0, st, a, out);
  }
  return hipGetLastError();
}

}  // namespace mtp
