// GEMMs on bf16 MFMA for draft steps with many activation rows (a batch of sequences, a
// prefill).
//
//   y[row][m] = sum_k W[m][k] * x[row][k],   W bf16 [N][K], x fp32 (after the policy's norm)
//
// k_prep and the skinny k_gemm_mfma below (k_gemm_tile, further down, takes calls with hundreds
// of rows):
// * k_prep: one workgroup per activation row; the policy's prologue (raw loads, RMSNorm, gains)
//   gives the fp32 row, which is written as two bf16 rows hi = bf16(x), lo = bf16(x - hi)
//   (x = hi + lo to about 2^-17 relative), compacted over the valid rows.  rowmap / amap record
//   each compact row's padded row and activation index; `count` the number of compact rows.
// * k_gemm_mfma: each workgroup owns 4 waves x NT tiles of 16 weight rows and a range of K
//   (the whole of K, or one of `ksplit` ranges when there are few row groups), walked in
//   chunks of 128.  Per chunk the workgroup stages the compact activations (hi and lo, up to MG
//   tiles of 16 rows) in LDS, and every wave streams its weight rows once from HBM, the next
//   chunk's weights in flight while this one is multiplied.  In step s of a chunk, lane l holds
//   columns 32 s + 8 (l / 16) .. +7 of row l % 16, so the four lanes of a row read 64
//   contiguous bytes per load.  v_mfma_f32_16x16x32_bf16 consumes the chunk in four steps; the
//   activations are read with the same column order, so the dot products are unchanged.  Two
//   MFMAs (hi, lo) per step keep fp32-like accuracy.  Rows beyond MG tiles are handled in
//   further passes.  With K split, raw partial sums go to a buffer and k_splitk_reduce adds
//   them in range order and applies the policy's store.
// Operand layout of v_mfma_f32_16x16x32_bf16 (checked on the device): lane l supplies
// A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16], e < 8; result r of lane l is
// D[4 (l / 16) + r][l % 16].
#pragma once

#include <type_traits>

#include "gemv.h"

namespace mtp {

constexpr int kMfmaKC = 128;          // K per LDS chunk
constexpr int kMfmaLdr = kMfmaKC + 8; // padded LDS row (bf16 elements)

struct MfmaBufs {
  uint16_t *xhi, *xlo;  // [cap][K] compact split activations
  int* rowmap;          // [cap] padded row of a compact row
  int* amap;            // [cap] activation index of a compact row
  int* count;           // number of compact rows
  float* part;          // split-K partial sums [ksplit][cap][N] (NULL: no split)
  int ksplit, cap;      // K ranges; activation rows the partial buffer is laid out for
  long part_cap;        // floats available at part
};

// One workgroup per activation index a (grid = nact).  The first KEEP chunks of each thread
// stay in registers, with their gains, across the norm reduction (KEEP = 12 holds rows of up to
// 24576 columns, chosen for rows wider than 8192; 4 otherwise); their loads are issued
// unconditionally from clamped columns -- before the row counts are in LDS when the row is
// known without them -- so the row arrives in one memory round trip.  The hi / lo rows are
// written 16 bytes at a time.
template <class W, class P, int KEEP>
__global__ __launch_bounds__(kWG) void k_prep(P p, MfmaBufs mb) {
  constexpr int VE = W::VE;
  static_assert(VE == 8, "bf16 weights");
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  __shared__ float red[8];
  const int a = blockIdx.x, tid = threadIdx.x;
  const int Kc = p.K / VE;
  float keep[KEEP][VE];
  uint4 gk[KEEP];
  auto issue = [&](int row) {
#pragma unroll
    for (int i = 0; i < KEEP; ++i) {
      const int ch = min(tid + i * kWG, Kc - 1);
      p.load_x(row, ch * VE, keep[i]);
      if constexpr (P::kNorm > 0) gk[i] = p.gain_raw(ch * VE);
    }
  };
  const auto pre = p.setup_load();
  if constexpr (P::kEarlyRows) issue(p.row_of(a));
  p.setup_store(pre, s_n, s_len);
  __syncthreads();
  int row;
  bool valid;
  p.act(a, s_n, row, valid);
  // compact index: activations before this one that are valid
  int c = 0, total = 0;
  if (P::kArgmax) {  // one activation per sequence with rows
    for (int b = 0; b < p.B; ++b) {
      const int v = s_n[b] > 0 ? 1 : 0;
      if (b < a) c += v;
      total += v;
    }
  } else {
    const int b = a / p.rps, i = a - b * p.rps;
    for (int bb = 0; bb < p.B; ++bb) {
      if (bb < b) c += s_n[bb];
      total += s_n[bb];
    }
    c += i;
  }
  if (a == 0 && tid == 0) *mb.count = total;
  if (!valid) return;
  if constexpr (!P::kEarlyRows) issue(row);
  float ss[2] = {0.f, 0.f};
  auto sumsq = [&](const float (&f)[VE], int ch) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) s = fmaf(f[e], f[e], s);
    if (P::kNorm == 2 && ch * VE >= p.split)
      ss[1] += s;
    else
      ss[0] += s;
  };
  if constexpr (P::kNorm > 0) {
#pragma unroll
    for (int i = 0; i < KEEP; ++i)
      if (tid + i * kWG < Kc) sumsq(keep[i], tid + i * kWG);
    for (int ch = tid + KEEP * kWG; ch < Kc; ch += kWG) {
      float f[VE];
      p.load_x(row, ch * VE, f);
      sumsq(f, ch);
    }
    wg_sum<2>(ss, red);
  }
  float sc0 = 1.f, sc1 = 1.f;
  if constexpr (P::kNorm == 2) {
    sc0 = 1.0f / sqrtf(ss[0] / float(p.split) + p.eps);
    sc1 = 1.0f / sqrtf(ss[1] / float(p.K - p.split) + p.eps);
  } else if constexpr (P::kNorm == 1) {
    sc0 = sc1 = 1.0f / sqrtf(ss[0] / float(p.K) + p.eps);
  }
  uint16_t* hi = mb.xhi + (long)c * p.K;
  uint16_t* lo = mb.xlo + (long)c * p.K;
  auto emit = [&](const float (&f)[VE], const uint4& graw, int ch) {
    float g[VE];
    if constexpr (P::kNorm > 0) {
      W::cvt(graw, g);
    } else {
#pragma unroll
      for (int e = 0; e < VE; ++e) g[e] = 1.f;
    }
    const float sc = (P::kNorm == 2 && ch * VE >= p.split) ? sc1 : sc0;
    uint32_t h2[VE / 2], l2[VE / 2];
#pragma unroll
    for (int e = 0; e < VE; e += 2) {
      const float x0 = P::kNorm > 0 ? f[e] * sc * g[e] : f[e];
      const float x1 = P::kNorm > 0 ? f[e + 1] * sc * g[e + 1] : f[e + 1];
      const uint32_t a0 = bf16_rne(x0), a1 = bf16_rne(x1);
      const uint32_t b0 = bf16_rne(x0 - __uint_as_float(a0 << 16)), b1 = bf16_rne(x1 - __uint_as_float(a1 << 16));
      h2[e / 2] = a0 | (a1 << 16);
      l2[e / 2] = b0 | (b1 << 16);
    }
    *reinterpret_cast<uint4*>(hi + ch * VE) = make_uint4(h2[0], h2[1], h2[2], h2[3]);
    *reinterpret_cast<uint4*>(lo + ch * VE) = make_uint4(l2[0], l2[1], l2[2], l2[3]);
  };
#pragma unroll
  for (int i = 0; i < KEEP; ++i)
    if (tid + i * kWG < Kc) emit(keep[i], gk[i], tid + i * kWG);
  for (int ch = tid + KEEP * kWG; ch < Kc; ch += kWG) {
    float f[VE];
    p.load_x(row, ch * VE, f);
    uint4 graw = make_uint4(0, 0, 0, 0);
    if constexpr (P::kNorm > 0) graw = p.gain_raw(ch * VE);
    emit(f, graw, ch);
  }
  if (tid == 0) {
    mb.rowmap[c] = row;
    mb.amap[c] = a;
  }
}

// NT weight-row tiles (16 rows each) per wave, MG activation tiles (16 compact rows) per pass.
template <class P, int NT, int MG>
__global__ __launch_bounds__(kWG, MG <= 4 ? 2 : 1) void k_gemm_mfma(P p, MfmaBufs mb) {
  using T = uint16_t;
  constexpr int WR = NT * 16;          // weight rows per wave
  constexpr int WL = WR / 4;           // weight loads per lane and chunk (four rows per load)
  constexpr bool DB = MG <= 2;         // double-buffered activation staging
  constexpr bool RP = MG >= 4;         // single buffer, next chunk's activations held in registers
  constexpr int NB = DB ? 2 : 1;
  constexpr int AV = 2 * MG * 16 * (kMfmaKC / 8);  // 16-byte activation vectors per chunk (hi + lo)
  constexpr int PER = (AV + kWG - 1) / kWG;
  __shared__ __align__(16) uint16_t sA[NB][2][MG * 16 * kMfmaLdr];  // [buffer][hi/lo][row][k]
  __shared__ __align__(16) uint16_t sW[4][WR * kMfmaLdr];            // each wave's weight tile
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  __shared__ float s_bv[4 * MG * 16];
  __shared__ int s_bi[4 * MG * 16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int jl = lane & 15, hq = lane >> 4;  // column of the tile, quarter of the wave
  uint16_t* myW = sW[wid];
  p.setup(s_n, s_len);
  const int count = *mb.count;
  __syncthreads();
  const int Kc = p.K / kMfmaKC;  // K is a multiple of 128 on this path
  const int rows_per_wg = 4 * WR;
  const int ngroups = (p.N + rows_per_wg - 1) / rows_per_wg;
  const int ks = mb.part ? mb.ksplit : 1;           // K ranges per row group
  const int kper = (Kc + ks - 1) / ks;

  const int npass = (count + MG * 16 - 1) / (MG * 16);  // passes of MG activation tiles
  const int per_pass = ngroups * ks;
  // lm_head (argmax) walks the passes in order (each workgroup's running bests are flushed per
  // pass); the other policies spread their (pass, row group, K range) items over the grid
  const int outer = P::kArgmax ? npass : (npass > 0 ? 1 : 0);
  for (int op = 0; op < outer; ++op) {
   const int n_items = P::kArgmax ? per_pass : npass * per_pass;
   for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
    const int pass = P::kArgmax ? op : it / per_pass;
    const int gk = P::kArgmax ? it : it - pass * per_pass;
    const int mg0 = pass * MG * 16;
    const int mrows = min(MG * 16, count - mg0);
    const int mt = (mrows + 15) / 16;
    const int srows = mt * 16;                        // staged rows (zero past mrows)
    const int nav = 2 * srows * (kMfmaKC / 8);        // staged vectors per chunk
    uint4 st[PER];
    // the pass's activations of chunk kc: vector idx -> (hi/lo, row, 8-column group)
    auto aload = [&](int kc) {
#pragma unroll
      for (int v = 0; v < PER; ++v) {
        const int idx = tid + kWG * v;
        const int half = idx / (srows * (kMfmaKC / 8)), rem = idx - half * (srows * (kMfmaKC / 8));
        const int r = rem / (kMfmaKC / 8), cv = rem - r * (kMfmaKC / 8);
        st[v] = (idx < nav && r < mrows)
                    ? ld16((half ? mb.xlo : mb.xhi) + (long)(mg0 + r) * p.K + kc * kMfmaKC + cv * 8)
                    : make_uint4(0, 0, 0, 0);
      }
    };
    auto astore = [&](int buf) {
#pragma unroll
      for (int v = 0; v < PER; ++v) {
        const int idx = tid + kWG * v;
        const int half = idx / (srows * (kMfmaKC / 8)), rem = idx - half * (srows * (kMfmaKC / 8));
        const int r = rem / (kMfmaKC / 8), cv = rem - r * (kMfmaKC / 8);
        if (idx < nav) *reinterpret_cast<uint4*>(&sA[buf][half][r * kMfmaLdr + cv * 8]) = st[v];
      }
    };
    {
      const int g = gk / ks, kpart = gk - g * ks;
      const int kc_beg = kpart * kper, kc_end = min(Kc, kc_beg + kper);
      const int n0 = g * rows_per_wg + wid * WR;
      f32x4_t acc[MG][NT];
#pragma unroll
      for (int m = 0; m < MG; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      // Weights are read row-contiguous: load i of a lane takes 16 bytes at column 8 (l % 16) of
      // the wave's row 4 i + l / 16, so sixteen lanes read 256 contiguous bytes of one row.  The
      // wave moves them through its own LDS tile into the MFMA operand layout.
      const T* wrow[WL];
#pragma unroll
      for (int i = 0; i < WL; ++i) wrow[i] = p.wrow(min(n0 + 4 * i + hq, p.N - 1)) + 8 * jl;
      uint4 wn[WL];
      auto wload = [&](int kc) {
#pragma unroll
        for (int i = 0; i < WL; ++i) wn[i] = ld_stream(wrow[i] + kc * kMfmaKC);
      };
      if (kc_beg < kc_end) {
        __syncthreads();  // the previous item's readers are done with the staging buffers
        wload(kc_beg);
        aload(kc_beg);
        astore(0);
        __syncthreads();
      }
      for (int kc = kc_beg; kc < kc_end; ++kc) {
        const int buf = DB ? ((kc - kc_beg) & 1) : 0;
#pragma unroll
        for (int i = 0; i < WL; ++i)  // this chunk's weights into the wave's tile
          *reinterpret_cast<uint4*>(&myW[(4 * i + hq) * kMfmaLdr + 8 * jl]) = wn[i];
        if (!DB && !RP && kc > kc_beg) {  // single buffer: stage this chunk now
          __syncthreads();
          aload(kc);
          astore(0);
          __syncthreads();
        }
        if (kc + 1 < kc_end) {  // the next chunk in flight while this one is multiplied
          wload(kc + 1);
          if (DB || RP) aload(kc + 1);
        }
#pragma unroll
        for (int m = 0; m < MG; ++m) {
          if (m < mt) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const int kk = 32 * s + 8 * hq;
              const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&sA[buf][0][(m * 16 + jl) * kMfmaLdr + kk]);
              const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&sA[buf][1][(m * 16 + jl) * kMfmaLdr + kk]);
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                const bf16x8_t bw = *reinterpret_cast<const bf16x8_t*>(&myW[(t * 16 + jl) * kMfmaLdr + kk]);
                acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw, acc[m][t], 0, 0, 0);
                acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw, acc[m][t], 0, 0, 0);
              }
            }
          }
        }
        if (DB) {
          if (kc + 1 < kc_end) astore(buf ^ 1);
          __syncthreads();
        } else if (RP && kc + 1 < kc_end) {
          __syncthreads();  // every wave is done with this chunk's activations
          astore(0);
          __syncthreads();
        }
      }
      if (mb.part) {  // split-K: raw partial sums, reduced and stored by k_splitk_reduce
#pragma unroll
        for (int m = 0; m < MG; ++m) {
          if (m >= mt) continue;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int col = n0 + t * 16 + jl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int cr = mg0 + m * 16 + 4 * hq + r;
              if (cr < count && col < p.N) mb.part[((long)kpart * mb.cap + cr) * p.N + col] = acc[m][t][r];
            }
          }
        }
        continue;
      }
      // epilogue: lane holds rows 4 hq + r of each activation tile, column jl of each weight tile
#pragma unroll
      for (int m = 0; m < MG; ++m) {
        if (m >= mt) continue;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int col = n0 + t * 16 + jl;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int cr = mg0 + m * 16 + 4 * hq + r;
            const float v = acc[m][t][r];
            const float partner = __shfl_xor(v, 1, kWave);
            if (cr < count && col < p.N) {
              const int row = mb.rowmap[cr], a = mb.amap[cr];
              if constexpr (P::kPair) {
                if ((jl & 1) == 0) p.store_pair(col, a, row, v, partner);
              } else {
                p.store(col, a, row, v);
              }
            }
          }
        }
      }
      if constexpr (P::kArgmax) {
        // running best per compact row over this group's columns, lowest id on ties
#pragma unroll
        for (int m = 0; m < MG; ++m) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const int col = n0 + t * 16 + jl;
              if (m < mt && col < p.N && better(acc[m][t][r], col, bv, bi)) {
                bv = acc[m][t][r];
                bi = col;
              }
            }
#pragma unroll
            for (int o = 8; o > 0; o >>= 1) {  // over the 16 lanes of this quarter
              const float ov = __shfl_xor(bv, o, kWave);
              const int oi = __shfl_xor(bi, o, kWave);
              if (better(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
              }
            }
            const int k = m * 16 + 4 * hq + r;
            if (jl == 0) {
              if (gk == (int)blockIdx.x) {
                s_bv[wid * MG * 16 + k] = bv;
                s_bi[wid * MG * 16 + k] = bi;
              } else if (better(bv, bi, s_bv[wid * MG * 16 + k], s_bi[wid * MG * 16 + k])) {
                s_bv[wid * MG * 16 + k] = bv;
                s_bi[wid * MG * 16 + k] = bi;
              }
            }
          }
        }
      }
    }
   }
    if constexpr (P::kArgmax) {
      const int mg0 = op * MG * 16, mrows = min(MG * 16, count - mg0);
      __syncthreads();
      for (int k = tid; k < mrows; k += kWG) {
        float v = -INFINITY;
        int i = 0x7fffffff;
        if ((int)blockIdx.x < ngroups * ks)
          for (int w = 0; w < 4; ++w)
            if (better(s_bv[w * MG * 16 + k], s_bi[w * MG * 16 + k], v, i)) {
              v = s_bv[w * MG * 16 + k];
              i = s_bi[w * MG * 16 + k];
            }
        p.partial(mb.amap[mg0 + k], v, i);
      }
      __syncthreads();
    }
  }
  p.finish(s_n);
}

// ---------------------------------------------------------------------------------------------
// Large tiles for calls with hundreds of activation rows (a prefill).  The skinny kernel above
// streams the whole weight matrix once per 64-row pass; here each workgroup owns a 128
// (compact activation rows) x 128 (weight rows) output tile and walks K in 32-column chunks
// with both operands staged in LDS (double-buffered, one barrier per chunk, two chunks in
// flight from memory), so the weights of
// a column group are read once per 128 rows and every staged element feeds four MFMA tiles.
// The four waves split the tile 2 x 2 (64 x 64 each: 4 x 4 MFMA tiles, hi and lo activation
// products into the same accumulators).  Global loads are row-contiguous (four threads x 16 B
// = one row's 64-byte chunk slice), issued two chunks ahead of the one multiplied, every
// one unconditional: rows past the count or the matrix re-read the last valid row, and their
// outputs are never stored.  LDS rows are padded to 40 bf16 (20 dwords): the sixteen rows a
// quarter-wave reads for one operand fall on distinct banks.  K must be a multiple of 64.
constexpr int kTileM = 128, kTileN = 128, kTileK = 32, kTileLd = kTileK + 8;
constexpr int kTileRows = 256;  // activation rows from which the large tiles are used

template <class P>
__global__ __launch_bounds__(kWG, 2) void k_gemm_tile(P p, MfmaBufs mb) {
  __shared__ __align__(16) uint16_t sA[2][2][kTileM * kTileLd];  // [buffer][hi/lo][row][k]
  __shared__ __align__(16) uint16_t sB[2][kTileN * kTileLd];     // [buffer][weight row][k]
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int jl = lane & 15, hq = lane >> 4;
  const int wm = wid & 1, wn = wid >> 1;  // this wave's 64 x 64 quarter of the tile
  p.setup(s_n, s_len);
  const int count = *mb.count;
  __syncthreads();
  const int nrt = (count + kTileM - 1) / kTileM;
  const int nct = (p.N + kTileN - 1) / kTileN;
  const int nk = p.K / kTileK;
  // staging map: thread t moves 16 bytes of row (t / 4) + 64 h at column 8 (t % 4) of a chunk
  const int lr = tid >> 2, lc = 8 * (tid & 3);
  for (int it = blockIdx.x; it < nrt * nct; it += gridDim.x) {
    const int i = it % nrt, j = it / nrt;  // consecutive items share the weight column group
    const uint16_t* arow_hi[2];
    const uint16_t* arow_lo[2];
    const uint16_t* brow[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cr = min(i * kTileM + lr + 64 * h, count - 1);
      arow_hi[h] = mb.xhi + (long)cr * p.K + lc;
      arow_lo[h] = mb.xlo + (long)cr * p.K + lc;
      brow[h] = reinterpret_cast<const uint16_t*>(p.wrow(min(j * kTileN + lr + 64 * h, p.N - 1))) + lc;
    }
    // two chunks in flight: register slot S holds chunk kc while kc is staged, then receives
    // kc + 2 (the K loop is unrolled by two so that slots are compile-time; K / 32 is even)
    uint4 ga[2][2][2], gb[2][2];  // [slot][hi/lo][half], [slot][half]
    auto gload = [&](int kc, uint4 (&a)[2][2], uint4 (&b)[2]) {
      const int k0 = kc * kTileK;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        b[h] = ld_stream(brow[h] + k0);
        a[0][h] = ld16(arow_hi[h] + k0);
        a[1][h] = ld16(arow_lo[h] + k0);
      }
    };
    auto sstore = [&](int buf, const uint4 (&a)[2][2], const uint4 (&b)[2]) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = lr + 64 * h;
        *reinterpret_cast<uint4*>(&sB[buf][r * kTileLd + lc]) = b[h];
        *reinterpret_cast<uint4*>(&sA[buf][0][r * kTileLd + lc]) = a[0][h];
        *reinterpret_cast<uint4*>(&sA[buf][1][r * kTileLd + lc]) = a[1][h];
      }
    };
    f32x4_t acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the padded row and activation index of this lane's 16 output rows, fetched up front (the
    // epilogue would otherwise wait for each pair of loads in turn)
    int orow[4][4], oact[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int cr = min(i * kTileM + wm * 64 + m * 16 + 4 * hq + r, count - 1);
        orow[m][r] = mb.rowmap[cr];
        oact[m][r] = mb.amap[cr];
      }
    __syncthreads();  // the previous item's readers are done with both buffers
    gload(0, ga[0], gb[0]);
    gload(1, ga[1], gb[1]);
    sstore(0, ga[0], gb[0]);
    __syncthreads();
    auto chunk = [&](auto slot, int kc) {
      constexpr int S = decltype(slot)::value;  // == kc & 1, also the LDS buffer of chunk kc
      // chunk kc + 2 into the slot chunk kc came in (the last chunk again near the end: every
      // load unconditional, so the compiler waits for one chunk's loads, not all)
      gload(min(kc + 2, nk - 1), ga[S], gb[S]);
#pragma unroll
      for (int s = 0; s < kTileK / 32; ++s) {
        const int kk = 32 * s + 8 * hq;
        bf16x8_t bw[4];
#pragma unroll
        for (int n = 0; n < 4; ++n)
          bw[n] = *reinterpret_cast<const bf16x8_t*>(&sB[S][(wn * 64 + n * 16 + jl) * kTileLd + kk]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int ra = (wm * 64 + m * 16 + jl) * kTileLd + kk;
          const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&sA[S][0][ra]);
          const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&sA[S][1][ra]);
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw[n], acc[m][n], 0, 0, 0);
            acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw[n], acc[m][n], 0, 0, 0);
          }
        }
      }
      // chunk kc + 1 (requested an iteration ago) into the other buffer, last read before the
      // previous barrier
      if (kc + 1 < nk) sstore(S ^ 1, ga[S ^ 1], gb[S ^ 1]);
      __syncthreads();
    };
    for (int kc = 0; kc < nk; kc += 2) {
      chunk(std::integral_constant<int, 0>{}, kc);
      chunk(std::integral_constant<int, 1>{}, kc + 1);
    }
    // epilogue: lane holds compact rows 4 hq + r of each 16-row tile, column jl of each weight tile
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int col = j * kTileN + wn * 64 + n * 16 + jl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int cr = i * kTileM + wm * 64 + m * 16 + 4 * hq + r;
          const float v = acc[m][n][r];
          const float partner = __shfl_xor(v, 1, kWave);
          if (cr < count && col < p.N) {
            if constexpr (P::kPair) {
              if ((jl & 1) == 0) p.store_pair(col, oact[m][r], orow[m][r], v, partner);
            } else {
              p.store(col, oact[m][r], orow[m][r], v);
            }
          }
        }
      }
  }
  p.finish(s_n);
}

// Sum the split-K partials of each (compact row, column) in split order and store them through
// the policy (pairs for pair policies).  One thread per output (or output pair).
template <class P>
__global__ __launch_bounds__(kWG) void k_splitk_reduce(P p, MfmaBufs mb) {
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  p.setup(s_n, s_len);
  __syncthreads();
  const int count = *mb.count;
  const int step = P::kPair ? 2 : 1;
  const long items = (long)count * (p.N / step);
  for (long it = (long)blockIdx.x * kWG + threadIdx.x; it < items; it += (long)gridDim.x * kWG) {
    const int cr = (int)(it / (p.N / step));
    const int col = (int)(it - (long)cr * (p.N / step)) * step;
    float v0 = 0.f, v1 = 0.f;
    for (int k = 0; k < mb.ksplit; ++k) {
      const float* pp = mb.part + ((long)k * mb.cap + cr) * p.N + col;
      v0 += pp[0];
      if (P::kPair) v1 += pp[1];
    }
    const int row = mb.rowmap[cr], a = mb.amap[cr];
    if constexpr (P::kPair)
      p.store_pair(col, a, row, v0, v1);
    else
      p.store(col, a, row, v0);
  }
}

}  // namespace mtp
