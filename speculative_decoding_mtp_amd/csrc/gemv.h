// Weight-streaming GEMV for the draft head (few activation rows, bf16 or fp32 weights,
// fp32 activations and fp32 accumulation).
//
//   y[a][m] = sum_k W[row(m)][k] * x[a][k]   for every logical output row m, activation row a.
//
// Two layouts of the same computation:
//
// * k_gemv_w ("wave rows", rows of up to 64*4 16-byte chunks): every wave owns whole weight
//   rows.  Lane l reads chunks c = l + 64 j of a row, so one load instruction covers 1 KB of a
//   row and a wave keeps RW*NJ loads (about 16) in flight.  The lane's slice of RB activation
//   rows stays in registers for the whole kernel.  Row sums are wave reductions through DPP
//   moves and lane reads: no LDS traffic and no barrier in the streaming loop; the waves of a
//   workgroup are independent.
// * k_gemv_s ("split K", wider rows): the 256 threads of a workgroup share each row (chunk
//   c = tid + 256 j); partial sums meet in LDS once per ROWS rows, the next rows' weights in
//   flight meanwhile.
//
// Activation rows beyond RB are handled in further passes over the weights.  A policy class
// supplies the activation prologue (raw loads, RMSNorm), the logical-row -> weight-row map and
// the stores; the argmax over logical rows (the lm_head) is tracked by the kernel.
#pragma once

#include "common.h"

namespace mtp {

constexpr int kMaxBatch = 256;  // sequences per drafter call (per-sequence row counts live in LDS)
static_assert(kMaxBatch == kWG, "one sequence per thread in the policies' setup");

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

// DPP lane move (gfx9 encodings: quad_perm 0x00-0xff, row_mirror 0x140, row_half_mirror 0x141)
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over the 64 lanes of a wave; the result is wave-uniform.  Pairs lanes i^1 and i^2 inside
// each quad, then mirrors inside each 8-lane half row and each 16-lane row (every lane of a row
// then holds the row sum), and adds the four row sums read from lanes 0, 16, 32, 48.  Must be
// called with all lanes active.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_mov<0xb1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4e>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Maximum over the 64 lanes of a wave, wave-uniform (same lane pattern as wave_sum_dpp).
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_mov<0xb1>(v));
  v = fmaxf(v, dpp_mov<0x4e>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Policy hooks (all __device__):
//   static constexpr int kNorm;     0: none, 1: RMSNorm of the row, 2: RMSNorms of [0, split) and
//                                   [split, K) separately
//   static constexpr bool kPair;    outputs come as logical-row pairs (m even, m + 1)
//   static constexpr bool kArgmax;  track the argmax over logical rows of every activation row
//   static constexpr bool kVocab;   output rows are a vocabulary (wider MFMA row groups)
//   void setup(int* s_n, int* s_len) per-sequence row counts and cache lengths into LDS (the
//                                   kernel then syncs); also in halves: SeqPre setup_load() issues
//                                   the loads, setup_store(pre, s_n, s_len) counts and writes
//   static constexpr bool kEarlyRows; row_of(a) gives activation a's row before the counts exist
//   void act(int a, const int* s_n, int& row, bool& valid)
//   void load_x(int row, int k, float (&f)[VE])     raw activations k..k+VE-1 of a row
//   uint4 gain_raw(int k)                            16 bytes of norm gains from column k (kNorm > 0)
//   const T* wrow(int m)                            weight row of logical row m < N
//   void store(int m, int a, int row, float v)      (!kPair)
//   void store_pair(int m, int a, int row, float v0, float v1)   (kPair)
//   void partial(int a, float v, int i)             (kArgmax) this workgroup's best of row a
//   void finish(const int* s_n)                     once per workgroup at the end

// Register slice of RB activation rows: x[r][j] holds the VE activations of chunk
// c = cbase + j * cstride (zero outside the row and for invalid rows), RMS-normalised when the
// policy asks.  issue_slice starts the loads -- every one at an in-bounds address (the row from
// row_of()/act() and the column clamped), none behind a branch, the norm gains of the thread's
// columns with them -- and norm_slice masks and normalises once the rows' validity is known;
// `reduce(s0, s1)` turns per-thread sums of squares into row totals.
template <class W, int RB, int NJ, class P>
__device__ __forceinline__ void issue_slice(const P& p, const int (&rows)[RB], int cbase, int cstride, int Kc,
                                            float (&x)[RB][NJ][W::VE], uint4 (&graw)[NJ]) {
  constexpr int VE = W::VE;
  if constexpr (P::kNorm > 0) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) graw[j] = p.gain_raw(min(cbase + j * cstride, Kc - 1) * VE);
  }
#pragma unroll
  for (int r = 0; r < RB; ++r)
#pragma unroll
    for (int j = 0; j < NJ; ++j) p.load_x(rows[r], min(cbase + j * cstride, Kc - 1) * VE, x[r][j]);
}

template <class W, int RB, int NJ, class P, class Reduce>
__device__ __forceinline__ void norm_slice(const P& p, const bool (&valid)[RB], int cbase, int cstride, int Kc,
                                           float (&x)[RB][NJ][W::VE], const uint4 (&graw)[NJ], Reduce reduce) {
  constexpr int VE = W::VE;
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int c = cbase + j * cstride;
      const bool live = valid[r] && c < Kc;
#pragma unroll
      for (int e = 0; e < VE; ++e) x[r][j][e] = live ? x[r][j][e] : 0.f;
      if constexpr (P::kNorm > 0) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) s = fmaf(x[r][j][e], x[r][j][e], s);
        if (P::kNorm == 2 && c * VE >= p.split)
          s1 += s;
        else
          s0 += s;
      }
    }
    if constexpr (P::kNorm > 0) {
      reduce(s0, s1);
      float sc0, sc1;
      if constexpr (P::kNorm == 2) {
        sc0 = 1.0f / sqrtf(s0 / float(p.split) + p.eps);
        sc1 = 1.0f / sqrtf(s1 / float(p.K - p.split) + p.eps);
      } else {
        sc0 = sc1 = 1.0f / sqrtf(s0 / float(p.K) + p.eps);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = cbase + j * cstride;
        if (c < Kc) {
          const int k0 = c * VE;
          const float sc = (P::kNorm == 2 && k0 >= p.split) ? sc1 : sc0;
          float gv[VE];
          W::cvt(graw[j], gv);
#pragma unroll
          for (int e = 0; e < VE; ++e) x[r][j][e] = x[r][j][e] * sc * gv[e];
        }
      }
    }
  }
}

// Hand the reduced, wave-uniform tile v[q][r] to the policy: item (q, r) -- or pair (q, q+1) --
// is stored by one lane.
template <int RW, int RB, class P>
__device__ __forceinline__ void store_tile(P& p, int m0, int a0, const int (&rows)[RB], const bool (&valid)[RB],
                                           const float (&v)[RW][RB], int lane) {
  if constexpr (P::kPair) {
#pragma unroll
    for (int q = 0; q < RW; q += 2)
#pragma unroll
      for (int r = 0; r < RB; ++r)
        if (lane == ((q / 2) * RB + r) % kWave && valid[r] && m0 + q < p.N)
          p.store_pair(m0 + q, a0 + r, rows[r], v[q][r], v[q + 1][r]);
  } else {
#pragma unroll
    for (int q = 0; q < RW; ++q)
#pragma unroll
      for (int r = 0; r < RB; ++r)
        if (lane == (q * RB + r) % kWave && valid[r] && m0 + q < p.N) p.store(m0 + q, a0 + r, rows[r], v[q][r]);
  }
}

// Combine the per-wave argmax of RB activation rows across the workgroup and hand it to the
// policy (thread r).  Contains barriers: call with the whole workgroup.
template <int RB, class P>
__device__ __forceinline__ void argmax_partials(P& p, int a0, const float (&bv)[RB], const int (&bi)[RB], float* sv,
                                                int* si) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0)
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      sv[wid * RB + r] = bv[r];
      si[wid * RB + r] = bi[r];
    }
  __syncthreads();
  if (threadIdx.x < RB) {
    const int r = threadIdx.x;
    float v = sv[r];
    int i = si[r];
    for (int w = 1; w < 4; ++w)
      if (better(sv[w * RB + r], si[w * RB + r], v, i)) {
        v = sv[w * RB + r];
        i = si[w * RB + r];
      }
    p.partial(a0 + r, v, i);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------------------
template <class W, int RB, int NJ, int RW, class P>
__global__ __launch_bounds__(kWG) void k_gemv_w(P p) {
  using T = typename W::T;
  constexpr int VE = W::VE;
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  __shared__ float s_bv[4 * RB];
  __shared__ int s_bi[4 * RB];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int Kc = p.K / VE;
  const int ngroups = (p.N + RW - 1) / RW;
  const int wave = blockIdx.x * 4 + wid, nwaves = gridDim.x * 4;
  uint4 wv[RW][NJ];
  auto load_group = [&](int g) {
    const int m0 = g * RW;
#pragma unroll
    for (int q = 0; q < RW; ++q) {
      const T* wp = p.wrow(min(m0 + q, p.N - 1));
#pragma unroll
      for (int j = 0; j < NJ; ++j) wv[q][j] = ld_stream(wp + (long)min(lane + j * kWave, Kc - 1) * VE);
    }
  };
  // Issue order: the per-sequence count inputs, the first activation block (when its rows are
  // known without the counts), then this wave's first weights; the counts are written to LDS
  // once their own loads are back, with the later loads still in flight.
  const auto pre = p.setup_load();
  int rows[RB];
  bool valid[RB];
  float x[RB][NJ][VE];
  uint4 graw[NJ];
  if constexpr (P::kEarlyRows) {
#pragma unroll
    for (int r = 0; r < RB; ++r) rows[r] = p.row_of(r);
    issue_slice<W, RB, NJ>(p, rows, lane, kWave, Kc, x, graw);
  }
  if (wave < ngroups) load_group(wave);
  p.setup_store(pre, s_n, s_len);
  __syncthreads();

  for (int a0 = 0; a0 < p.nact; a0 += RB) {
    bool any = false;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      p.act(a0 + r, s_n, rows[r], valid[r]);
      any |= valid[r];
    }
    if (!any) continue;  // uniform across the workgroup; the prefetched group is the next block's first
    if (!P::kEarlyRows || a0 > 0) issue_slice<W, RB, NJ>(p, rows, lane, kWave, Kc, x, graw);
    norm_slice<W, RB, NJ>(p, valid, lane, kWave, Kc, x, graw, [](float& s0, float& s1) {
      s0 = wave_sum_dpp(s0);
      s1 = wave_sum_dpp(s1);
    });
    float bv[RB];
    int bi[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      bv[r] = -INFINITY;
      bi[r] = 0x7fffffff;
    }
    for (int g = wave; g < ngroups; g += nwaves) {
      const int m0 = g * RW;
      float acc[RW][RB];
#pragma unroll
      for (int q = 0; q < RW; ++q) {
#pragma unroll
        for (int r = 0; r < RB; ++r) acc[q][r] = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          float wf[VE];
          W::cvt(wv[q][j], wf);
#pragma unroll
          for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[q][r] = fmaf(wf[e], x[r][j][e], acc[q][r]);
        }
      }
      // next group's weights (this block's next group, or the next block's first) are loaded
      // while this group is reduced and stored
      const int gn = g + nwaves < ngroups ? g + nwaves : (a0 + RB < p.nact ? wave : -1);
      if (gn >= 0) load_group(gn);
#pragma unroll
      for (int q = 0; q < RW; ++q)
#pragma unroll
        for (int r = 0; r < RB; ++r) acc[q][r] = wave_sum_dpp(acc[q][r]);
      store_tile<RW, RB>(p, m0, a0, rows, valid, acc, lane);
      if constexpr (P::kArgmax) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int q = 0; q < RW; ++q)
            if (m0 + q < p.N && better(acc[q][r], m0 + q, bv[r], bi[r])) {
              bv[r] = acc[q][r];
              bi[r] = m0 + q;
            }
      }
    }
    if constexpr (P::kArgmax) argmax_partials<RB>(p, a0, bv, bi, s_bv, s_bi);
  }
  p.finish(s_n);
}

// ---------------------------------------------------------------------------------------------
template <class W, int RB, int NXM, int ROWS, class P>
__global__ __launch_bounds__(kWG) void k_gemv_s(P p) {
  constexpr int VE = W::VE;
  __shared__ float s_red[4 * ROWS * RB];
  __shared__ float s_norm[8];
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  __shared__ float s_bv[4 * RB];
  __shared__ int s_bi[4 * RB];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int Kc = p.K / VE;
  const int ngroups = (p.N + ROWS - 1) / ROWS;
  uint4 wv[NXM][ROWS];
  // chunk c = tid + j * kWG of rows m0 .. m0 + ROWS - 1; lanes past the row end read a clamped
  // chunk (multiplied by x = 0)
  auto load_group = [&](int g) {
    const int m0 = g * ROWS;
#pragma unroll
    for (int j = 0; j < NXM; ++j)
      if (j * kWG < Kc)  // uniform
#pragma unroll
        for (int q = 0; q < ROWS; ++q)
          wv[j][q] = ld_stream(p.wrow(min(m0 + q, p.N - 1)) + (long)min(tid + j * kWG, Kc - 1) * VE);
  };
  // issue order as in k_gemv_w: count inputs, first activation block, first weights
  const auto pre = p.setup_load();
  int rows[RB];
  bool valid[RB];
  float x[RB][NXM][VE];
  uint4 graw[NXM];
  if constexpr (P::kEarlyRows) {
#pragma unroll
    for (int r = 0; r < RB; ++r) rows[r] = p.row_of(r);
    issue_slice<W, RB, NXM>(p, rows, tid, kWG, Kc, x, graw);
  }
  if ((int)blockIdx.x < ngroups) load_group(blockIdx.x);
  p.setup_store(pre, s_n, s_len);
  __syncthreads();

  for (int a0 = 0; a0 < p.nact; a0 += RB) {
    bool any = false;
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      p.act(a0 + r, s_n, rows[r], valid[r]);
      any |= valid[r];
    }
    if (!any) continue;  // uniform; the prefetched group is the next block's first
    if (!P::kEarlyRows || a0 > 0) issue_slice<W, RB, NXM>(p, rows, tid, kWG, Kc, x, graw);
    norm_slice<W, RB, NXM>(p, valid, tid, kWG, Kc, x, graw, [&](float& s0, float& s1) {
      s0 = wave_sum_dpp(s0);
      s1 = wave_sum_dpp(s1);
      if (lane == 0) {
        s_norm[wid] = s0;
        s_norm[4 + wid] = s1;
      }
      __syncthreads();
      s0 = (s_norm[0] + s_norm[1]) + (s_norm[2] + s_norm[3]);
      s1 = (s_norm[4] + s_norm[5]) + (s_norm[6] + s_norm[7]);
      __syncthreads();
    });
    float bv[RB];
    int bi[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      bv[r] = -INFINITY;
      bi[r] = 0x7fffffff;
    }
    for (int g = blockIdx.x; g < ngroups; g += gridDim.x) {
      const int m0 = g * ROWS;
      float acc[ROWS][RB];
#pragma unroll
      for (int q = 0; q < ROWS; ++q)
#pragma unroll
        for (int r = 0; r < RB; ++r) acc[q][r] = 0.f;
#pragma unroll
      for (int j = 0; j < NXM; ++j) {
        if (j * kWG < Kc) {  // uniform
#pragma unroll
          for (int q = 0; q < ROWS; ++q) {
            float wf[VE];
            W::cvt(wv[j][q], wf);
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
              for (int e = 0; e < VE; ++e) acc[q][r] = fmaf(wf[e], x[r][j][e], acc[q][r]);
          }
        }
      }
      // the next group's weights (this block's next, or the next block's first) in flight
      // while this group is reduced and stored
      const int gn = g + (int)gridDim.x < ngroups ? g + (int)gridDim.x : (a0 + RB < p.nact ? (int)blockIdx.x : -1);
      if (gn >= 0) load_group(gn);
#pragma unroll
      for (int q = 0; q < ROWS; ++q)
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const float s = wave_sum_dpp(acc[q][r]);
          if (lane == 0) s_red[wid * ROWS * RB + q * RB + r] = s;
        }
      __syncthreads();
#pragma unroll
      for (int q = 0; q < ROWS; ++q)
#pragma unroll
        for (int r = 0; r < RB; ++r) {
          const int k = q * RB + r;
          acc[q][r] = (s_red[k] + s_red[ROWS * RB + k]) + (s_red[2 * ROWS * RB + k] + s_red[3 * ROWS * RB + k]);
        }
      __syncthreads();
      if (wid == 0) store_tile<ROWS, RB>(p, m0, a0, rows, valid, acc, lane);
      if constexpr (P::kArgmax) {
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
          for (int q = 0; q < ROWS; ++q)
            if (m0 + q < p.N && better(acc[q][r], m0 + q, bv[r], bi[r])) {
              bv[r] = acc[q][r];
              bi[r] = m0 + q;
            }
      }
    }
    if constexpr (P::kArgmax) argmax_partials<RB>(p, a0, bv, bi, s_bv, s_bi);
  }
  p.finish(s_n);
}

}  // namespace mtp
