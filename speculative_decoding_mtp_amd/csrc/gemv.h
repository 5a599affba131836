// Weight-streaming GEMV for the draft head (few activation rows, bf16 or fp32 weights,
// fp32 activations and accumulation).
//
// y[a][m] = sum_k W[row(m)][k] * x[a][k] for every logical output row m and activation row a.
//
// Layout of the work: the 256 threads of a workgroup split K into 16-byte weight chunks
// (chunk c = tid + 256*j, j < nx), so one wave-wide load reads 1 KB of a weight row and the
// whole workgroup reads 4 KB contiguous.  Each thread keeps its slice of RB activation rows in
// registers for the whole kernel and streams ROWS weight rows at a time through it; the ROWS*RB
// partial dot products are reduced across the workgroup once per ROWS rows.  Workgroups take
// row groups in a grid-stride loop.  Activation rows beyond RB are handled in further passes
// over the weights.  A policy class supplies the activation prologue (raw loads, RMSNorm), the
// logical-row -> weight-row map and the epilogue.
#pragma once

#include "common.h"

namespace mtp {

constexpr int kMaxBatch = 256;  // sequences per drafter call (per-sequence row counts live in LDS)

template <int VE>
__device__ __forceinline__ void load_f32_vec(const float* p, float (&f)[VE]) {
  if constexpr (VE == 8) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
  }
}

template <class W>
__device__ __forceinline__ void load_w_vec(const typename W::T* p, float (&f)[W::VE]) {
  W::cvt(ld16(p), f);
}

// Policy hooks (all __device__):
//   static constexpr int kNorm;             0: none, 1: RMSNorm of the whole row, 2: separate
//                                           RMSNorms of [0, split) and [split, K)
//   void setup(int* s_n)                    fill per-sequence row counts (then the kernel syncs)
//   void act(int a, const int* s_n, int& row, bool& valid)
//   void load_x(int row, int k, float (&f)[VE])   raw activations k..k+VE-1 of a row
//   void gain_vec(int k, float (&g)[VE])    norm gains k..k+VE-1 (kNorm > 0)
//   const T* wrow(int m)                    weight row of logical row m (m < N)
//   void epilogue(int m0, const float* tile, const int* rows, const bool* valid, int nval)
//                                           tile[q*RB + r] = y[a0+r][m0+q]; called by all threads
//   void act_block_done(int a0, ...)        after the last row group of an activation block
//   void finish()                           once per workgroup at the end
template <class W, int RB, int NXM, int ROWS, class P>
__global__ __launch_bounds__(kWG, 2) void k_gemv(P p) {
  using T = typename W::T;
  constexpr int VE = W::VE;
  __shared__ float s_red[4 * ROWS * RB];
  __shared__ float s_tile[ROWS * RB];
  __shared__ float s_norm[8 * RB];
  __shared__ int s_n[kMaxBatch];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;

  p.setup(s_n);
  __syncthreads();

  const int Kc = p.K / VE;
  const int nx = (Kc + kWG - 1) / kWG;
  const int ngroups = (p.N + ROWS - 1) / ROWS;

  for (int a0 = 0; a0 < p.nact; a0 += RB) {
    int rows[RB];
    bool valid[RB];
    bool any = false;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      p.act(a0 + r, s_n, rows[r], valid[r]);
      any |= valid[r];
    }
    if (!any) continue;  // uniform across the workgroup

    float x[RB][NXM][VE];
    float ss[2 * RB];
#pragma unroll
    for (int r = 0; r < 2 * RB; ++r) ss[r] = 0.f;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
#pragma unroll
      for (int j = 0; j < NXM; ++j) {
        const int c = tid + j * kWG;
        if (valid[r] && j < nx && c < Kc) {
          p.load_x(rows[r], c * VE, x[r][j]);
          if constexpr (P::kNorm > 0) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < VE; ++e) s += x[r][j][e] * x[r][j][e];
            const int half = (P::kNorm == 2 && c * VE >= p.split) ? 1 : 0;
            ss[2 * r + half] += s;
          }
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) x[r][j][e] = 0.f;
        }
      }
    }
    if constexpr (P::kNorm > 0) {
      wg_sum<2 * RB>(ss, s_norm);
#pragma unroll
      for (int r = 0; r < RB; ++r) {
        float sc0, sc1;
        if constexpr (P::kNorm == 2) {
          sc0 = 1.0f / sqrtf(ss[2 * r] / float(p.split) + p.eps);
          sc1 = 1.0f / sqrtf(ss[2 * r + 1] / float(p.K - p.split) + p.eps);
        } else {
          sc0 = sc1 = 1.0f / sqrtf((ss[2 * r] + ss[2 * r + 1]) / float(p.K) + p.eps);
        }
#pragma unroll
        for (int j = 0; j < NXM; ++j) {
          const int c = tid + j * kWG;
          if (j < nx && c < Kc) {
            const int k0 = c * VE;
            const float sc = (P::kNorm == 2 && k0 >= p.split) ? sc1 : sc0;
            float gv[VE];
            p.gain_vec(k0, gv);
#pragma unroll
            for (int e = 0; e < VE; ++e) x[r][j][e] = x[r][j][e] * sc * gv[e];
          }
        }
      }
    }

    for (int g = blockIdx.x; g < ngroups; g += gridDim.x) {
      const int m0 = g * ROWS;
      const T* wp[ROWS];
#pragma unroll
      for (int q = 0; q < ROWS; ++q) wp[q] = (m0 + q < p.N) ? p.wrow(m0 + q) : nullptr;
      float acc[ROWS][RB];
#pragma unroll
      for (int q = 0; q < ROWS; ++q)
#pragma unroll
        for (int r = 0; r < RB; ++r) acc[q][r] = 0.f;

#pragma unroll
      for (int j = 0; j < NXM; ++j) {
        const int c = tid + j * kWG;
        if (j < nx && c < Kc) {
          uint4 wv[ROWS];
#pragma unroll
          for (int q = 0; q < ROWS; ++q)
            wv[q] = wp[q] ? ld_stream(wp[q] + (long)c * VE) : make_uint4(0, 0, 0, 0);
#pragma unroll
          for (int q = 0; q < ROWS; ++q) {
            float wf[VE];
            W::cvt(wv[q], wf);
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
              for (int e = 0; e < VE; ++e) acc[q][r] = fmaf(wf[e], x[r][j][e], acc[q][r]);
          }
        }
      }
      // reduce ROWS*RB partial sums over the workgroup
#pragma unroll
      for (int q = 0; q < ROWS; ++q)
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const float s = wave_sum(acc[q][r]);
          if (lane == 0) s_red[wid * ROWS * RB + q * RB + r] = s;
        }
      __syncthreads();
      if (tid < ROWS * RB)
        s_tile[tid] = s_red[tid] + s_red[ROWS * RB + tid] + s_red[2 * ROWS * RB + tid] + s_red[3 * ROWS * RB + tid];
      __syncthreads();
      p.template epilogue<ROWS, RB>(m0, s_tile, rows, valid, a0);
    }
    p.template act_block_done<RB>(a0, rows, valid);
  }
  p.finish(s_n);
}

}  // namespace mtp
