// Decode attention of the draft head: grouped-query causal softmax attention of each row over
// the head's own KV cache, split over the cached positions and merged in a second pass.
//
// [HB14] "14. MTP: speculative decoding with the built-in draft head", section "The draft head":
// the head's decoder layer is full attention with RoPE over its own KV cache; rows attend to
// every cached position up to their own.  Scores q.k / sqrt(hd), softmax, weighted sum of V.
#include "common.h"
#include "draft.h"

namespace mtp {

// ---------------------------------------------------------------------------------------------
// decode attention, split over the cached positions
// ---------------------------------------------------------------------------------------------
// Workgroup (s, kvh, b) handles positions [s*chunk, min(T, (s+1)*chunk)) of sequence b, where
// T = len[b] + rows, for all queries (row i, query head kvh*G + g) of the sequence.  K/V tiles of
// 64 positions are staged through LDS; an online softmax keeps (m, l, o) per query.  Output per
// query: the unnormalised o, the running max m and the sum l.
constexpr int kTile = 64;
constexpr int kQB = 32;

template <class W, int HD>
__global__ __launch_bounds__(kWG) void k_attn(AttnArgs a) {
  using T = typename W::T;
  constexpr int VE = W::VE;
  constexpr int LDR = HD + VE;  // padded tile row (elements)
  __shared__ __align__(16) T sK[kTile * LDR];
  __shared__ __align__(16) T sV[kTile * LDR];
  __shared__ __align__(16) float sQ[kQB * HD];
  __shared__ float sS[kQB * kTile];
  __shared__ float sAlpha[kQB];
  __shared__ int s_n;

  const int tid = threadIdx.x;
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.nq / a.nkv;
  if (tid == 0) s_n = count_rows(a.tok + (long)b * a.tok_sb, a.rps, a.V, a.len[b], a.max_len, nullptr);
  __syncthreads();
  const int n = s_n;
  if (n == 0) return;
  const int L0 = a.len[b];
  const int Tn = L0 + n;
  const int chunk = attn_chunk(Tn, a.nsplit);
  const int p_beg = s * chunk;
  if (p_beg >= Tn) return;
  const int p_end = min(Tn, p_beg + chunk);
  const int NQ = n * G;
  const T* Kb = reinterpret_cast<const T*>(a.kc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  const T* Vb = reinterpret_cast<const T*>(a.vc) + ((long)b * a.nkv + kvh) * a.max_len * HD;
  const float scale = 1.0f / sqrtf(float(HD));

  for (int q0 = 0; q0 < NQ; q0 += kQB) {
    const int nqb = min(kQB, NQ - q0);
    // queries of this block -> LDS
    for (int idx = tid; idx < nqb * HD; idx += kWG) {
      const int ql = idx / HD, d = idx - ql * HD;
      const int qi = q0 + ql, i = qi / G, gg = qi - i * G;
      const long row = (long)b * a.rps + i;
      sQ[idx] = a.q[(row * a.nq + (kvh * G + gg)) * HD + d];
    }
    float m_run = -INFINITY, l_run = 0.f;  // owned by thread tid < nqb
    constexpr int QPT = kQB / (kWG / HD);  // PV accumulators per thread
    float o[QPT];
#pragma unroll
    for (int k = 0; k < QPT; ++k) o[k] = 0.f;
    const int dpv = tid % HD, qsub = tid / HD;

    for (int t0 = p_beg; t0 < p_end; t0 += kTile) {
      __syncthreads();
      // stage K and V tiles (16-byte vectors)
      constexpr int VPR = HD / VE;  // vectors per row
      for (int idx = tid; idx < kTile * VPR; idx += kWG) {
        const int pr = idx / VPR, c = idx - pr * VPR;
        const int p = t0 + pr;
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (p < p_end) {
          kv = ld16(Kb + (long)p * HD + c * VE);
          vv = ld16(Vb + (long)p * HD + c * VE);
        }
        *reinterpret_cast<uint4*>(sK + pr * LDR + c * VE) = kv;
        *reinterpret_cast<uint4*>(sV + pr * LDR + c * VE) = vv;
      }
      __syncthreads();
      // scores: thread -> position pl, queries qs, qs+4, ...
      {
        const int pl = tid & (kTile - 1), qs = tid >> 6;
        constexpr int SPT = kQB / 4;
        float acc[SPT];
#pragma unroll
        for (int k = 0; k < SPT; ++k) acc[k] = 0.f;
#pragma unroll 4
        for (int d0 = 0; d0 < HD; d0 += VE) {
          float kf[VE];
          W::cvt(*reinterpret_cast<const uint4*>(sK + pl * LDR + d0), kf);
#pragma unroll
          for (int k = 0; k < SPT; ++k) {
            const float* qp = sQ + (qs + 4 * k) * HD + d0;
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[k] = fmaf(qp[e], kf[e], acc[k]);
          }
        }
        const int p = t0 + pl;
#pragma unroll
        for (int k = 0; k < SPT; ++k) {
          const int ql = qs + 4 * k;
          if (ql < nqb) {
            const int qi = q0 + ql, i = qi / G;
            const bool ok = p < p_end && p <= L0 + i;
            sS[ql * kTile + pl] = ok ? acc[k] * scale : -INFINITY;
          }
        }
      }
      __syncthreads();
      // online softmax update, one thread per query
      if (tid < nqb) {
        float* srow = sS + tid * kTile;
        float tmax = -INFINITY;
        for (int k = 0; k < kTile; ++k) tmax = fmaxf(tmax, srow[k]);
        const float m_new = fmaxf(m_run, tmax);
        float alpha, lsum = 0.f;
        if (m_new == -INFINITY) {
          alpha = 1.f;
          for (int k = 0; k < kTile; ++k) srow[k] = 0.f;
        } else {
          alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
          for (int k = 0; k < kTile; ++k) {
            const float e = (srow[k] == -INFINITY) ? 0.f : expf(srow[k] - m_new);
            srow[k] = e;
            lsum += e;
          }
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        sAlpha[tid] = alpha;
      }
      __syncthreads();
      // o = o * alpha + P V
#pragma unroll
      for (int k = 0; k < QPT; ++k) {
        const int ql = qsub + (kWG / HD) * k;
        if (ql < nqb) {
          float acc = o[k] * sAlpha[ql];
          const float* prow = sS + ql * kTile;
          for (int pl = 0; pl < kTile; ++pl) acc = fmaf(prow[pl], W::get(sV, pl * LDR + dpv), acc);
          o[k] = acc;
        }
      }
    }
    // write partials
    float* P = a.part + (((long)b * a.nkv + kvh) * a.nsplit + s) * (long)a.qstride * (HD + 2);
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int ql = qsub + (kWG / HD) * k;
      if (ql < nqb) P[(long)(q0 + ql) * (HD + 2) + dpv] = o[k];
    }
    if (tid < nqb) {
      P[(long)(q0 + tid) * (HD + 2) + HD] = m_run;
      P[(long)(q0 + tid) * (HD + 2) + HD + 1] = l_run;
    }
    __syncthreads();
  }
}

// Merge the split partials: o = sum_s o_s e^{m_s - M} / sum_s l_s e^{m_s - M}.
template <int HD>
__global__ __launch_bounds__(kWG) void k_attn_combine(AttnArgs a, float* out) {
  const int per = kWG / HD;
  const int item = blockIdx.x * per + threadIdx.x / HD;  // (row, head)
  const int d = threadIdx.x % HD;
  const int R = a.B * a.rps;
  if (item >= R * a.nq) return;
  const int row = item / a.nq, h = item - row * a.nq;
  const int b = row / a.rps, i = row - b * a.rps;
  const int n = count_rows(a.tok + (long)b * a.tok_sb, a.rps, a.V, a.len[b], a.max_len, nullptr);
  if (i >= n) return;
  const int G = a.nq / a.nkv, kvh = h / G, qi = i * G + (h - kvh * G);
  const int T = a.len[b] + n;
  const int chunk = attn_chunk(T, a.nsplit);
  const float* P = a.part + ((long)b * a.nkv + kvh) * a.nsplit * (long)a.qstride * (HD + 2) + (long)qi * (HD + 2);
  const long sstride = (long)a.qstride * (HD + 2);
  float M = -INFINITY;
  for (int s = 0; s < a.nsplit && s * chunk < T; ++s) {
    const float l = P[s * sstride + HD + 1];
    if (l > 0.f) M = fmaxf(M, P[s * sstride + HD]);
  }
  float L = 0.f, O = 0.f;
  for (int s = 0; s < a.nsplit && s * chunk < T; ++s) {
    const float l = P[s * sstride + HD + 1];
    if (l > 0.f) {
      const float e = expf(P[s * sstride + HD] - M);
      L = fmaf(l, e, L);
      O = fmaf(P[s * sstride + d], e, O);
    }
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
    hipLaunchKernelGGL((k_attn_combine<128>), dim3((items + 1) / 2), dim3(kWG), 0, st, a, out);
  } else {
    if (wdtype == MTP_BF16)
      hipLaunchKernelGGL((k_attn<BF16, 64>), grid, dim3(kWG), 0, st, a);
    else
      hipLaunchKernelGGL((k_attn<F32, 64>), grid, dim3(kWG), 0, st, a);
    hipLaunchKernelGGL((k_attn_combine<64>), dim3((items + 3) / 4), dim3(kWG), 0, st, a, out);
  }
  return hipGetLastError();
}

}  // namespace mtp
