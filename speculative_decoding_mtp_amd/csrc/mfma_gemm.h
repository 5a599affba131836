// MFMA GEMMs for draft steps with many activation rows (a batch of sequences, a prefill):
//
//   y[row][m] = sum_k W[m][k] * x[row][k],   W bf16 [N][K], x fp32 (after the policy's norm)
//
// * k_prep: one workgroup per activation row; the policy's prologue (raw loads, RMSNorm, gains)
//   gives the fp32 row, which is written as two bf16 rows hi = bf16(x), lo = bf16(x - hi)
//   (x = hi + lo to about 2^-17 relative), compacted over the valid rows.  rowmap / amap record
//   each compact row's padded row and activation index; `count` the number of compact rows.
//   Those compact rows feed the weight-streaming GEMM (stream_gemm.h) and, for calls with
//   hundreds of rows, k_gemm_tile below.
// * k_gemm_tile: 128 x 256 output tiles with both operands staged in LDS (a prefill).
// * k_splitk_reduce: sums split-K partials in range order and applies the policy's store.
// Operand layout of v_mfma_f32_16x16x32_bf16 (checked on the device): lane l supplies
// A[l % 16][8 (l / 16) + e] and B[8 (l / 16) + e][l % 16], e < 8; result r of lane l is
// D[4 (l / 16) + r][l % 16].
#pragma once

#include <type_traits>

#include "gemv.h"

namespace mtp {

constexpr int kMfmaKC = 128;  // MFMA paths take K in whole 128-column chunks

struct MfmaBufs {
  uint16_t *xhi, *xlo;  // [cap][K] compact split activations
  int* rowmap;          // [cap] padded row of a compact row
  int* amap;            // [cap] activation index of a compact row
  int* count;           // number of compact rows
  float* part;          // split-K partial sums [ksplit][cap][N] (NULL: no split)
  int ksplit, cap;      // K ranges; activation rows the partial buffer is laid out for
  long part_cap;        // floats available at part
  uint16_t *shi, *slo;  // NULL, or where a policy with kSplitOut also writes its outputs split
                        // hi / lo (compact rows of width N / 2) for the next GEMM
};

// One workgroup per activation index a (grid = nact).  The first KEEP chunks of each thread
// stay in registers, with their gains, across the norm reduction (KEEP = 12 holds rows of up to
// 24576 columns, chosen for rows wider than 8192; otherwise 4, 2 or 1, no more than the row
// needs, so that fewer registers let more rows run at once); their loads are issued
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

// A split-K GEMM whose outputs are the residual stream (eh_proj, o_proj, down_proj) followed by a
// GEMM that normalises that stream (QKV, gate/up, lm_head): one workgroup per row sums the
// row's partials in split order and stores it through P (as k_splitk_reduce does), keeps it in
// registers and prepares Pn's split activations from it (as k_prep does: the same chunks per
// thread, the same sums, so the activations are bit-identical) -- one launch instead of two.
// Rows are P's activation rows; with an argmax Pn (one row per sequence) only each sequence's
// last valid row is prepared, at the sequence's compact index.  Requires P::N == Pn::K and
// N <= KEEP * kWG * 8.  The compact maps and count written are Pn's.
template <class W, class P, class Pn, int KEEP>
__global__ __launch_bounds__(kWG) void k_reduce_prep(P p, Pn pn, MfmaBufs mb) {
  constexpr int VE = 8;
  static_assert(!P::kPair && Pn::kNorm == 1, "a residual-stream reduction feeding one RMSNorm");
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  __shared__ float red[8];
  const int a = blockIdx.x, tid = threadIdx.x;
  const int N = p.N, Kc = N / VE;
  p.setup(s_n, s_len);
  __syncthreads();
  int row;
  bool valid;
  p.act(a, s_n, row, valid);
  const int b = a / p.rps, i = a - b * p.rps;
  int c = 0, total = 0, cs = 0, nseq = 0;  // compact index (P's rows, and Pn's for argmax)
  for (int bb = 0; bb < p.B; ++bb) {
    const int nb = s_n[bb];
    if (bb < b) {
      c += nb;
      cs += nb > 0 ? 1 : 0;
    }
    total += nb;
    nseq += nb > 0 ? 1 : 0;
  }
  c += i;
  if (a == 0 && tid == 0) *mb.count = Pn::kArgmax ? nseq : total;
  if (!valid) return;
  // partial sums in split order; the loads of QS splits of every chunk are issued together
  // (chunk columns clamped, so every load is in bounds and unconditional)
  constexpr int QS = KEEP <= 4 ? 4 : 1;
  float v[KEEP][VE];
#pragma unroll
  for (int k = 0; k < KEEP; ++k)
#pragma unroll
    for (int e = 0; e < VE; ++e) v[k][e] = 0.f;
  const float* pc = mb.part + (long)c * N;
  const long sstride = (long)mb.cap * N;
  for (int sp = 0; sp < mb.ksplit; sp += QS) {
    float4 u[QS][KEEP][2];
#pragma unroll
    for (int q = 0; q < QS; ++q)
#pragma unroll
      for (int k = 0; k < KEEP; ++k) {
        const float* pp = pc + (long)min(sp + q, mb.ksplit - 1) * sstride + min(tid + k * kWG, Kc - 1) * VE;
        u[q][k][0] = *reinterpret_cast<const float4*>(pp);
        u[q][k][1] = *reinterpret_cast<const float4*>(pp + 4);
      }
#pragma unroll
    for (int q = 0; q < QS; ++q)
      if (sp + q < mb.ksplit) {
#pragma unroll
        for (int k = 0; k < KEEP; ++k) {
          v[k][0] += u[q][k][0].x; v[k][1] += u[q][k][0].y; v[k][2] += u[q][k][0].z; v[k][3] += u[q][k][0].w;
          v[k][4] += u[q][k][1].x; v[k][5] += u[q][k][1].y; v[k][6] += u[q][k][1].z; v[k][7] += u[q][k][1].w;
        }
      }
  }
  float x[KEEP][VE];
#pragma unroll
  for (int k = 0; k < KEEP; ++k) {
    const int ch = tid + k * kWG;
    if (ch < Kc) {
#pragma unroll
      for (int e = 0; e < VE; ++e) x[k][e] = p.reduce_store(ch * VE + e, a, row, v[k][e]);
    }
  }
  int cn = c;
  if constexpr (Pn::kArgmax) {  // the sequence's last valid row only (uniform per workgroup)
    if (i != s_n[b] - 1) return;
    cn = cs;
  }
  float ss[2] = {0.f, 0.f};
#pragma unroll
  for (int k = 0; k < KEEP; ++k)
    if (tid + k * kWG < Kc) {
      float sq = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) sq = fmaf(x[k][e], x[k][e], sq);
      ss[0] += sq;
    }
  wg_sum<2>(ss, red);
  const float sc = 1.0f / sqrtf(ss[0] / float(pn.K) + pn.eps);
  uint16_t* hi = mb.xhi + (long)cn * pn.K;
  uint16_t* lo = mb.xlo + (long)cn * pn.K;
#pragma unroll
  for (int k = 0; k < KEEP; ++k) {
    const int ch = tid + k * kWG;
    if (ch < Kc) {
      float g[VE];
      W::cvt(pn.gain_raw(ch * VE), g);
      uint32_t h2[VE / 2], l2[VE / 2];
#pragma unroll
      for (int e = 0; e < VE; e += 2) {
        const float x0 = x[k][e] * sc * g[e], x1 = x[k][e + 1] * sc * g[e + 1];
        const uint32_t a0 = bf16_rne(x0), a1 = bf16_rne(x1);
        const uint32_t b0 = bf16_rne(x0 - __uint_as_float(a0 << 16)), b1 = bf16_rne(x1 - __uint_as_float(a1 << 16));
        h2[e / 2] = a0 | (a1 << 16);
        l2[e / 2] = b0 | (b1 << 16);
      }
      *reinterpret_cast<uint4*>(hi + ch * VE) = make_uint4(h2[0], h2[1], h2[2], h2[3]);
      *reinterpret_cast<uint4*>(lo + ch * VE) = make_uint4(l2[0], l2[1], l2[2], l2[3]);
    }
  }
  if (tid == 0) {
    mb.rowmap[cn] = row;
    mb.amap[cn] = Pn::kArgmax ? b : a;
  }
}

// ---------------------------------------------------------------------------------------------
// Large tiles for calls with hundreds of activation rows (a prefill).  The streaming kernel
// (stream_gemm.h) reads the whole weight matrix once per 64-row pass; here each workgroup of
// eight waves owns a 128 (compact activation rows) x 256 (weight rows) output tile -- or one of
// `ksplit` K ranges of it, when the tiles alone would leave compute units idle -- and walks K in
// 32-column chunks with both operands staged in LDS.  The waves split the tile 2 x 4 (64 x 64
// each: 4 x 4 MFMA tiles, hi and lo activation products into the same accumulators).  What
// limits this GEMM is the operand traffic from L2 (hi + lo activations at 4 bytes per element,
// weights at 2): per output it falls as 4 / 256 + 2 / 128 bytes per K column here, against
// 4 / 128 + 2 / 128 for a 128 x 128 tile (2048 x 12288 x 2048: 328 -> 259 us).
// Global loads take whole 128-byte lines: a line of a row holds two consecutive chunks, and a
// load of its 64-byte halves one chunk apart fetched most lines twice.  So each thread loads 16
// bytes of rows of each operand per pair of chunks; the pair is stored at the start of every odd
// chunk into the two of three LDS buffers not being read (32 KB each: hi, lo and weights; one
// workgroup per compute unit) and the next pair's loads are issued right after, two chunks ahead
// of their use.  Rows are unpadded, the four 16-byte slots of row r XOR-swizzled by
// ((r >> 1) ^ (r >> 3)) & 3 so that the sixteen rows a quarter-wave reads for one operand fall on
// distinct banks.  Work items are taken in contiguous ranges per XCD (workgroup b runs on XCD
// b % 8), so the tiles sharing a column group, or a row group, share that XCD's L2.  Every load
// is unconditional: rows past the count or the matrix re-read the last valid row (their outputs
// are never stored) and pairs past the range re-read its last pair.  The chunks are multiplied in
// the same order as in one pass over K, so a single range gives the same sums whatever the
// staging.  K must be a multiple of 64; the host keeps every K range non-empty.
constexpr int kTileM = 128, kTileN = 256, kTileK = 32, kTileThreads = 512;
constexpr int kTileOpA = kTileM * kTileK, kTileOpB = kTileN * kTileK;  // bf16 per operand and buffer
constexpr int kTileBuf = 2 * kTileOpA + kTileOpB;                       // hi, lo, weights
constexpr int kTileRows = 256;     // activation rows from which the large tiles are used
constexpr int kTileMinPairs = 16;  // K pairs (64 columns) per range at least when split

__device__ __forceinline__ int tile_swz(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }

template <class P>
__global__ __launch_bounds__(kTileThreads, 1) void k_gemm_tile(P p, MfmaBufs mb) {
  static_assert(kTileM == 128 && kTileN == 256 && kTileK == 32 && kTileThreads == 512, "the staging map below");
  __shared__ __align__(16) uint16_t sm[3 * kTileBuf];  // [buffer][hi, lo, weights][row][32]
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int jl = lane & 15, hq = lane >> 4;
  const int wm = wid & 1, wn = wid >> 1;  // this wave's 64 x 64 part of the tile
  p.setup(s_n, s_len);                    // threads past the batch (kMaxBatch) take no sequence
  const int count = *mb.count;
  __syncthreads();
  const int ks = mb.part ? mb.ksplit : 1;
  const int nrt = (count + kTileM - 1) / kTileM;
  const int nct = (p.N + kTileN - 1) / kTileN;
  const int npall = p.K / (2 * kTileK), pp = (npall + ks - 1) / ks;
  const int total = nrt * nct * ks, per = (total + 7) / 8;
  // staging map: thread t moves 16 bytes (slot t % 8 of the 128-byte line) of rows t / 8 + 64 h
  const int pr = tid >> 3, pc = tid & 7;
  const int fj = tile_swz(jl);  // the swizzle of rows 16 k + jl is fj ^ (2 k & 3)
  for (int u = blockIdx.x; u < 8 * per; u += gridDim.x) {
    const int it = (u & 7) * per + (u >> 3);  // XCD u % 8 takes items [x per, (x + 1) per)
    if (it >= total) continue;
    const int s = it % ks, t = it / ks;   // the K ranges of a tile run side by side
    const int i = t % nrt, j = t / nrt;   // consecutive tiles share the weight column group
    const int p0 = s * pp, np = min(npall, p0 + pp) - p0, nk = 2 * np;
    long ao[2];
    const uint16_t* brow[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) ao[h] = (long)min(i * kTileM + pr + 64 * h, count - 1) * p.K + 64 * p0 + 8 * pc;
#pragma unroll
    for (int h = 0; h < 4; ++h)
      brow[h] = reinterpret_cast<const uint16_t*>(p.wrow(min(j * kTileN + pr + 64 * h, p.N - 1))) + 64 * p0 + 8 * pc;
    uint4 ga[2][2], gb[4];  // one pair of chunks: [hi, lo][row group], [row group]
    auto gload = [&](int pair) {
      const int k0 = 64 * pair;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ga[0][h] = ld16(mb.xhi + ao[h] + k0);
        ga[1][h] = ld16(mb.xlo + ao[h] + k0);
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) gb[h] = ld_stream(brow[h] + k0);
    };
    // chunks c (held by the lanes with pc < 4) and c + 1 (pc >= 4) into their buffers
    auto sstore = [&](int c) {
      const int b0 = c % 3, b1 = b0 == 2 ? 0 : b0 + 1;
      const int base = ((pc >> 2) ? b1 : b0) * kTileBuf;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = pr + 64 * h;
        const int off = base + r * kTileK + 8 * ((pc & 3) ^ tile_swz(r));
        *reinterpret_cast<uint4*>(&sm[off]) = ga[0][h];
        *reinterpret_cast<uint4*>(&sm[off + kTileOpA]) = ga[1][h];
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int r = pr + 64 * h;
        *reinterpret_cast<uint4*>(&sm[base + 2 * kTileOpA + r * kTileK + 8 * ((pc & 3) ^ tile_swz(r))]) = gb[h];
      }
    };
    f32x4_t acc[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) acc[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int c) {
      const uint16_t* sb = sm + (c % 3) * kTileBuf;
      bf16x8_t bw[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int R = wn * 64 + n * 16 + jl;
        bw[n] = *reinterpret_cast<const bf16x8_t*>(sb + 2 * kTileOpA + R * kTileK + 8 * (hq ^ fj ^ ((2 * n) & 3)));
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int o = (wm * 64 + m * 16 + jl) * kTileK + 8 * (hq ^ fj ^ ((2 * m) & 3));
        const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(sb + o);
        const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(sb + kTileOpA + o);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bw[n], acc[m][n], 0, 0, 0);
          acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bw[n], acc[m][n], 0, 0, 0);
        }
      }
    };
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
    __syncthreads();  // the previous item's readers are done with every buffer
    gload(0);
    sstore(0);
    gload(min(1, np - 1));
    __syncthreads();
    for (int c = 0; c < nk; c += 2) {
      compute(c);
      __syncthreads();  // chunk c - 1's buffer and chunk c's are free
      if (c + 2 < nk) {
        sstore(c + 2);
        gload(min(c / 2 + 2, np - 1));
      }
      // the loads stay ahead of the chunk's MFMAs (the compiler would sink them to its end)
      __builtin_amdgcn_sched_barrier(0);
      compute(c + 1);
      __syncthreads();
    }
    if constexpr (P::kPair && P::kRolledStore) {
      if (ks == 1) {
        // a long pair store (RoPE and the cache append): unrolled over the lane's 64 outputs it
        // made the kernel ten times larger than the others (and slower, on instruction fetch).
        // Each half of this wave's 64 x 64 outputs goes through its own 8 KB of the free LDS as
        // fp32 [row][column]; lane l then stores column pair l % 32 of rows l / 32, + 2, ...
        float* sE = reinterpret_cast<float*>(sm) + wid * 32 * 64;
        const int c0 = j * kTileN + wn * 64;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
          for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
              for (int r = 0; r < 4; ++r) sE[(m * 16 + 4 * hq + r) * 64 + n * 16 + jl] = acc[2 * hf + m][n][r];
          __builtin_amdgcn_wave_barrier();
#pragma unroll 1
          for (int e = lane; e < 32 * 32; e += 64) {
            const int rr = e >> 5, cp = 2 * (e & 31);
            const int cr = i * kTileM + wm * 64 + 32 * hf + rr;
            if (cr < count && c0 + cp < p.N) {
              const float2 v = *reinterpret_cast<const float2*>(&sE[rr * 64 + cp]);
              p.store_pair(c0 + cp, mb.amap[cr], mb.rowmap[cr], v.x, v.y);
            }
          }
          __builtin_amdgcn_wave_barrier();  // the second half reuses the region
        }
        continue;  // the next item's first barrier waits for these reads
      }
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
            if (ks > 1) {
              mb.part[((long)s * mb.cap + cr) * p.N + col] = v;
            } else if constexpr (P::kPair && P::kRolledStore) {
              // stored by the rolled epilogue above
            } else if constexpr (P::kPair) {
              if ((jl & 1) == 0) {
                if constexpr (P::kSplitOut) {
                  if (mb.shi)
                    p.store_pair_split(col, oact[m][r], orow[m][r], cr, v, partner, mb.shi, mb.slo);
                  else
                    p.store_pair(col, oact[m][r], orow[m][r], v, partner);
                } else {
                  p.store_pair(col, oact[m][r], orow[m][r], v, partner);
                }
              }
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
// the policy (pairs for pair policies).  One thread per four consecutive outputs (16-byte partial
// loads; N % 4 == 0, as every matrix of the MFMA path has), each summed in split order as before.
template <class P>
__global__ __launch_bounds__(kWG) void k_splitk_reduce(P p, MfmaBufs mb) {
  __shared__ int s_n[kMaxBatch];
  __shared__ int s_len[kMaxBatch];
  p.setup(s_n, s_len);
  __syncthreads();
  const int count = *mb.count;
  const int nq = p.N / 4;
  const long items = (long)count * nq;
  for (long it = (long)blockIdx.x * kWG + threadIdx.x; it < items; it += (long)gridDim.x * kWG) {
    const int cr = (int)(it / nq);
    const int col = (int)(it - (long)cr * nq) * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < mb.ksplit; ++k) {
      const float4 q = *reinterpret_cast<const float4*>(mb.part + ((long)k * mb.cap + cr) * p.N + col);
      v[0] += q.x;
      v[1] += q.y;
      v[2] += q.z;
      v[3] += q.w;
    }
    const int row = mb.rowmap[cr], a = mb.amap[cr];
    if constexpr (P::kPair) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (P::kSplitOut) {
          if (mb.shi)
            p.store_pair_split(col + 2 * h, a, row, cr, v[2 * h], v[2 * h + 1], mb.shi, mb.slo);
          else
            p.store_pair(col + 2 * h, a, row, v[2 * h], v[2 * h + 1]);
        } else {
          p.store_pair(col + 2 * h, a, row, v[2 * h], v[2 * h + 1]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) p.store(col + e, a, row, v[e]);
    }
  }
}

}  // namespace mtp
