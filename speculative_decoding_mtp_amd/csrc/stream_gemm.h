// Weight-streaming GEMM on bf16 MFMA for draft steps with a batch of activation rows (a batch of
// sequences, a catch-up call, a target pass, a short prefill):
//
//   y[row][m] = sum_k W[m][k] * x[row][k],   W bf16 [N][K], x fp32 carried as bf16 hi + lo
//
// The activations have been normalised and split by k_prep (mfma_gemm.h) into compact bf16 rows
// hi = bf16(x), lo = bf16(x - hi).  The weights are read once per pass of up to 16*MT activation
// rows; everything here is arranged so that the weight stream never waits on anything else.
//
// * Work: a workgroup of NW waves owns a set of NW*NT 16-row weight tiles and one range of K (the
//   whole of K, or one of ks parts whose raw sums k_splitk_reduce adds up in order).  The host
//   picks NW (7..9), NT and ks per matrix so that sets x parts cover the compute units evenly.
// * Weights: each wave streams its own NT tiles in 64-column chunks (128 bytes of a row): load i
//   of a lane takes 16 bytes of row 8 i + lane / 8, so one instruction reads eight rows x 128
//   contiguous bytes.  D chunks are in flight in registers; each chunk goes through the wave's
//   own LDS tile (written and read by that wave only, no barrier) into the MFMA operand layout.
// * Activations: staged in LDS in ranges of RC chunks, three range buffers.  While range r is
//   multiplied, every iteration loads one slice of range r + 2 (a fixed number of 16-byte loads
//   per thread) and writes the slice it loaded D iterations earlier; a range is therefore in LDS
//   before the barrier at its start, which only has to wait for LDS writes.  Every iteration of
//   the K loop issues the same number of vector-memory loads (the loop runs a whole number of
//   D-chunk groups; loads past the end re-read cached addresses and only the multiplications are
//   skipped), so the compiler's waits are exact and nothing drains the weight loads in flight.
// * MFMA: v_mfma_f32_16x16x32_bf16 with the activations as the A operand (16 rows x 32 k) and the
//   weights as the B operand (32 k x 16 weight rows), two products per step (hi and lo).
//   Operand layout (gfx950): lane l supplies A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16],
//   e < 8; result r of lane l is D[4 (l / 16) + r][l % 16].
// * LDS layouts are XOR-swizzled in 16-byte units so that the 16 lanes of a quarter wave, which
//   read one unit of 16 different rows, hit distinct banks: weight tile rows are 8 units long,
//   unit u of row r stored at u ^ ((r & 7) ^ ((r >> 3) & 1)); activation rows hold 16k units,
//   unit u of row r at u ^ (r & 15).
#pragma once

#include "mfma_gemm.h"

namespace mtp {

constexpr int kSgKC = 64;        // K per chunk (128 bytes of a weight row)
constexpr int kSgMaxWaves = 9;   // waves per workgroup at most

// Waves a workgroup may have with NT tiles per wave and 16 MT-row passes: bounded by the LDS of
// the weight tiles next to the activation ranges (and, through the launch bound, the registers).
constexpr int sg_max_waves(int NT, int MT) { return NT * MT >= 16 ? 6 : NT >= 3 ? 8 : kSgMaxWaves; }

template <int MT, int AC = (MT <= 2 ? 256 : 128)>
struct SgShape {
  static constexpr int ROWS = 16 * MT;                 // activation rows per pass
  static constexpr int ACOLS = AC;                     // activation columns per staged range
  static constexpr int RC = ACOLS / kSgKC;             // chunks per range
  static constexpr int D = RC < 3 ? RC : 3;            // weight chunks in flight per wave
  static constexpr int UNITS = ACOLS / 8;              // 16-byte units per staged activation row
  static constexpr int HALF = ROWS * ACOLS * 2;        // bytes of the hi (or lo) rows of a range
  static constexpr int BUF = 2 * HALF;                 // bytes of one range buffer
  static constexpr int SLICE = 2 * ROWS * 8;           // 16-byte pieces of one chunk of a range
  static_assert(UNITS % 16 == 0, "activation rows of whole 16-unit swizzle groups");
  static_assert(RC >= D, "a range must cover the chunks in flight");
};

// The work decomposition chosen on the host.
struct SgPlan {
  int nw;     // waves per workgroup
  int sets;   // sets of nw * NT weight tiles
  int ks;     // K parts
  int kper;   // chunks per K part
};

__device__ __forceinline__ int sg_wswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// KPT: activation pieces each thread loads per chunk (ceil(SLICE / threads)); the same count in
// every thread keeps the loads per iteration fixed.
template <class P, int NT, int MT, int KPT, int AC = (MT <= 2 ? 256 : 128)>
__global__ __launch_bounds__(64 * sg_max_waves(NT, MT)) void k_gemm_stream(P p, MfmaBufs mb, SgPlan pl) {
  using S = SgShape<MT, AC>;
  constexpr int D = S::D, RC = S::RC;
  constexpr int WMAX = sg_max_waves(NT, MT);
  constexpr int WL = 2 * NT;              // weight loads per lane and chunk
  constexpr int WT = NT * 16 * 128;       // bytes of a wave's weight tile
  __shared__ __align__(16) char s_act[3][S::BUF];
  __shared__ __align__(16) char s_w[WMAX][WT];
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  __shared__ float s_bv[(P::kArgmax ? WMAX * S::ROWS : 1)];
  __shared__ int s_bi[(P::kArgmax ? WMAX * S::ROWS : 1)];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int jl = lane & 15, hq = lane >> 4;
  const int nw = pl.nw, nthreads = 64 * nw;
  char* myW = s_w[wid];
  p.setup(s_n, s_len);
  const int count = *mb.count;
  __syncthreads();
  const int K = p.K;
  const int nk = K / kSgKC;
  const int set_rows = nw * NT * 16;
  const int npass = (count + S::ROWS - 1) / S::ROWS;
  const int per_pass = pl.sets * pl.ks;
  // lm_head (argmax) walks the passes in order, flushing each workgroup's running bests per pass;
  // the other policies spread (pass, set, K part) items over the grid
  const int outer = P::kArgmax ? npass : (npass > 0 ? 1 : 0);
  for (int op = 0; op < outer; ++op) {
    const int n_items = P::kArgmax ? per_pass : npass * per_pass;
    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
      const int pass = P::kArgmax ? op : it / per_pass;
      const int rest = P::kArgmax ? it : it - pass * per_pass;
      const int set = rest / pl.ks, kpart = rest - set * pl.ks;
      const int mg0 = pass * S::ROWS;
      const int mrows = min(S::ROWS, count - mg0);
      const int mt = (mrows + 15) / 16;
      const int kc0 = kpart * pl.kper;
      const int nkc = min(nk, kc0 + pl.kper) - kc0;
      const int n0 = set * set_rows + wid * NT * 16;
      const int nranges = (nkc + RC - 1) / RC;

      // weight rows of this lane's loads; chunk c adds c * 64 elements
      const uint16_t* wsrc[WL];
#pragma unroll
      for (int i = 0; i < WL; ++i)
        wsrc[i] = reinterpret_cast<const uint16_t*>(p.wrow(min(n0 + 8 * i + (lane >> 3), p.N - 1))) +
                  (long)kc0 * kSgKC + 8 * (lane & 7);
      // piece q (< SLICE) of chunk slice s of range r: (half, row, unit v of the chunk); pieces past
      // SLICE (spare threads) repeat the last one, an address another lane already reads
      auto act_src = [&](int r, int s, int q) {
        q = min(q, S::SLICE - 1);
        const int half = q / (S::ROWS * 8), row = (q >> 3) % S::ROWS, v = q & 7;
        const int col = min((kc0 + r * RC + s) * kSgKC + 8 * v, K - 8);
        return (half ? mb.xlo : mb.xhi) + (long)(mg0 + min(row, mrows - 1)) * K + col;
      };
      auto act_put = [&](int r, int s, int q, uint4 v16) {
        if (q < S::SLICE) {
          const int half = q / (S::ROWS * 8), row = (q >> 3) % S::ROWS, v = q & 7;
          *reinterpret_cast<uint4*>(s_act[r % 3] + half * S::HALF + row * (S::UNITS * 16) +
                                    (((8 * s + v) ^ (row & 15)) << 4)) = v16;
        }
      };
      f32x4_t acc[MT][NT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[m][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      uint4 wr[D][WL];
      uint4 ar[D][KPT];
      __syncthreads();  // the previous item's readers are done with the range buffers
      // ranges 0 and 1 (their loads first, then the first weight chunks, then the LDS writes)
      {
        uint4 pre[2][RC][KPT];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int s = 0; s < RC; ++s)
#pragma unroll
            for (int k = 0; k < KPT; ++k) pre[r][s][k] = ld16(act_src(min(r, nranges - 1), s, tid + k * nthreads));
#pragma unroll
        for (int d = 0; d < D; ++d)
#pragma unroll
          for (int i = 0; i < WL; ++i) wr[d][i] = ld_stream(wsrc[i] + min(d, nkc - 1) * kSgKC);
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int s = 0; s < RC; ++s)
#pragma unroll
            for (int k = 0; k < KPT; ++k) act_put(r, s, tid + k * nthreads, pre[r][s][k]);
      }
      const int nkc_pad = (nkc + D - 1) / D * D;
      for (int c0 = 0; c0 < nkc_pad; c0 += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          const int c = c0 + d;
          const int r = c / RC, cr = c - r * RC;
          if (cr == 0) {  // range r is complete in LDS once every wave's writes of it are done
            __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));  // lgkmcnt(0); vmcnt, expcnt untouched
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
          }
          // this chunk's weights into the wave's tile (swizzled), the next load into the slot
#pragma unroll
          for (int i = 0; i < WL; ++i) {
            const int row = 8 * i + (lane >> 3), u = lane & 7;
            *reinterpret_cast<uint4*>(myW + row * 128 + ((u ^ sg_wswz(row)) << 4)) = wr[d][i];
          }
#pragma unroll
          for (int i = 0; i < WL; ++i) wr[d][i] = ld_stream(wsrc[i] + min(c + D, nkc - 1) * kSgKC);
          // the activation slice loaded D iterations ago (range r' + 2 for its chunk c - D in range
          // r'), then this iteration's slice of range r + 2
          if (c >= D) {
            const int cp = c - D, rp = cp / RC;
            if (rp + 2 < nranges) {
#pragma unroll
              for (int k = 0; k < KPT; ++k) act_put(rp + 2, cp - rp * RC, tid + k * nthreads, ar[d][k]);
            }
          }
#pragma unroll
          for (int k = 0; k < KPT; ++k) ar[d][k] = ld16(act_src(min(r + 2, nranges - 1), cr, tid + k * nthreads));
          if (c < nkc) {
            const char* ab = s_act[r % 3];
#pragma unroll
            for (int s = 0; s < kSgKC / 32; ++s) {
              const int uw = 4 * s + hq;       // unit of the chunk in a weight-tile row
              const int ua = cr * 8 + uw;      // unit in an activation row of the range
              bf16x8_t bw[NT];
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                const int row = 16 * t + jl;
                bw[t] = *reinterpret_cast<const bf16x8_t*>(myW + row * 128 + ((uw ^ sg_wswz(row)) << 4));
              }
#pragma unroll
              for (int m = 0; m < MT; ++m) {
                if (m < mt) {
                  const int row = 16 * m + jl;
                  const int off = row * (S::UNITS * 16) + ((ua ^ (row & 15)) << 4);
                  const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(ab + off);
                  const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(ab + S::HALF + off);
#pragma unroll
                  for (int t = 0; t < NT; ++t) {
                    acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw[t], acc[m][t], 0, 0, 0);
                    acc[m][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw[t], acc[m][t], 0, 0, 0);
                  }
                }
              }
            }
          }
        }
      }
      if (mb.part) {  // split K: raw partial sums, reduced and stored by k_splitk_reduce
#pragma unroll
        for (int m = 0; m < MT; ++m) {
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
      for (int m = 0; m < MT; ++m) {
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
                if ((jl & 1) == 0) {
                  if constexpr (P::kSplitOut) {
                    if (mb.shi)
                      p.store_pair_split(col, a, row, cr, v, partner, mb.shi, mb.slo);
                    else
                      p.store_pair(col, a, row, v, partner);
                  } else {
                    p.store_pair(col, a, row, v, partner);
                  }
                }
              } else {
                p.store(col, a, row, v);
              }
            }
          }
        }
      }
      if constexpr (P::kArgmax) {
        // running best per compact row over this workgroup's columns, lowest id on ties
#pragma unroll
        for (int m = 0; m < MT; ++m) {
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
              if (it == (int)blockIdx.x) {
                s_bv[wid * S::ROWS + k] = bv;
                s_bi[wid * S::ROWS + k] = bi;
              } else if (better(bv, bi, s_bv[wid * S::ROWS + k], s_bi[wid * S::ROWS + k])) {
                s_bv[wid * S::ROWS + k] = bv;
                s_bi[wid * S::ROWS + k] = bi;
              }
            }
          }
        }
      }
    }
    if constexpr (P::kArgmax) {
      const int mg0 = op * S::ROWS, mrows = min(S::ROWS, count - mg0);
      __syncthreads();
      for (int k = tid; k < mrows; k += blockDim.x) {
        float v = -INFINITY;
        int i = 0x7fffffff;
        if ((int)blockIdx.x < per_pass)
          for (int w = 0; w < nw; ++w)
            if (better(s_bv[w * S::ROWS + k], s_bi[w * S::ROWS + k], v, i)) {
              v = s_bv[w * S::ROWS + k];
              i = s_bi[w * S::ROWS + k];
            }
        p.partial(mb.amap[mg0 + k], v, i);
      }
      __syncthreads();
    }
  }
  p.finish(s_n);
}

}  // namespace mtp
