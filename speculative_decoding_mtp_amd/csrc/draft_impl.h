// Draft-head step: GEMV policies and the kernel sequence, templated on the weight type.
// Instantiated once per weight type in draft_bf16.hip and draft_f32.hip.
//
// One draft step over R = B * rows_per_seq padded rows (a row is valid when its token is
// non-negative, inside the vocabulary and its position fits the cache):
//   eh_proj   : x = W_eh [rms(E[tok]) * g_e ; rms(h) * g_h]           (embedding half first)
//   per layer : q,k,v = W_qkv rms(x) * g_in, RoPE(q,k) at pos, k,v -> cache[pos]
//               o = softmax(q K^T / sqrt(hd)) V over positions 0..pos   (split over T, combined)
//               x += W_o o
//               x += W_d (silu(W_g m) * W_u m),  m = rms(x) * g_post
//   lm_head   : g = rms(x) * g_f; logits = W_lm g for each sequence's last row; argmax with the
//               lowest id on ties; the last workgroup writes the draft and grows len[b].
// Sources: [HB14] "14. MTP: speculative decoding with the built-in draft head", section "The
// draft head"; [YL] "MTP 原理详解" sections 二.1-二.3 and 三 stages 1-2.
#pragma once

#include <functional>
#include <type_traits>

#include "draft.h"
#include "gemv.h"
#include "mfma_gemm.h"
#include "stream_gemm.h"

namespace mtp {

// ---------------------------------------------------------------------------------------------
// common part of every drafter GEMV policy: row addressing and validity
// ---------------------------------------------------------------------------------------------
template <class W>
struct PBase {
  using T = typename W::T;
  static constexpr bool kPair = false;
  static constexpr bool kArgmax = false;
  static constexpr bool kVocab = false;  // output rows are a vocabulary (MFMA: 128 rows per workgroup)
  static constexpr bool kSplitOut = false;  // can also write its outputs split for the next GEMM
  // the pair store is long (RoPE): a tile epilogue calls it from a loop, not unrolled per output
  static constexpr bool kRolledStore = false;
  const int32_t* tok;
  int tok_sb;
  int B, rps;
  const int32_t* len;
  int max_len, V;
  int K, N, nact, split;
  float eps;
  const int* rows;      // NULL, or valid rows counted once for the step
  const int* lds_len;  // cache lengths in LDS, set by setup()
  int dense = 0;        // host hint: every row of the call is valid (the target's verify pass)

  // Per-sequence row counts and cache lengths into LDS, in two halves so that a kernel can put
  // its weight loads between them: setup_load issues thread b's loads (sequence b = thread;
  // B <= kMaxBatch == kWG; clamped, so every lane loads in bounds), setup_store counts and
  // writes.  setup() does both.
  struct SeqPre {
    int len, r;
    int t[8];
  };
  __device__ SeqPre setup_load() const {
    SeqPre q;
    const int b = min((int)threadIdx.x, B - 1);
    q.len = len[b];
    q.r = (rows ? rows : len)[b];
    const int32_t* tb = tok + (long)b * tok_sb;
#pragma unroll
    for (int e = 0; e < 8; ++e) q.t[e] = tb[min(e, rps - 1)];
    return q;
  }
  __device__ void setup_store(const SeqPre& q, int* s_n, int* s_len) {
    const int b = threadIdx.x;
    if (b < B) {
      s_len[b] = q.len;
      s_n[b] = rows ? q.r
                    : (rps <= 8 ? count_tokens8(q.t, rps, V, q.len, max_len, nullptr)
                                : count_rows(tok + (long)b * tok_sb, rps, V, q.len, max_len, nullptr));
    }
    lds_len = s_len;
  }
  __device__ void setup(int* s_n, int* s_len) { setup_store(setup_load(), s_n, s_len); }
  // activation rows are known before the counts (row = activation index): a kernel may issue
  // the first block's activation loads before setup
  static constexpr bool kEarlyRows = true;
  __device__ int row_of(int a) const { return a < B * rps ? a : 0; }
  // row is always a row of the call (0 for an index past the end): activation loads are issued
  // for every row before validity masks them
  __device__ void act(int a, const int* s_n, int& row, bool& valid) const {
    row = 0;
    valid = false;
    if (a < B * rps) {
      const int b = a / rps, i = a - b * rps;
      row = a;
      valid = i < s_n[b];
    }
  }
  __device__ void store(int, int, int, float) {}
  __device__ void store_pair(int, int, int, float, float) {}
  __device__ void partial(int, float, int) {}
  __device__ void finish(const int*) {}
};

// eh_proj over [embedding ; hidden], each half RMS-normalised with its own gain
template <class W>
struct PEhProj : PBase<W> {
  using T = typename W::T;
  static constexpr int kNorm = 2;
  const T *embed, *enorm, *hnorm, *w;
  const float* hin;
  int hin_sb, H;
  float* xout;

  // Branch-free: both halves are read at in-bounds addresses (a padding row's token is clamped
  // into the vocabulary; its values are masked by the caller) and the right one is kept.
  __device__ void load_x(int row, int k, float (&f)[W::VE]) const {
    const int b = row / this->rps, i = row - b * this->rps;
    const int t = min(max(this->tok[(long)b * this->tok_sb + i], 0), this->V - 1);
    const bool emb = k < H;
    float e[W::VE], h[W::VE];
    W::cvt(ld16(embed + (long)t * H + (emb ? k : 0)), e);
    load_f32_vec<W::VE>(hin + ((long)b * hin_sb + i) * H + (emb ? 0 : k - H), h);
#pragma unroll
    for (int j = 0; j < W::VE; ++j) f[j] = emb ? e[j] : h[j];
  }
  __device__ uint4 gain_raw(int k) const { return ld16(k < H ? enorm + k : hnorm + (k - H)); }
  __device__ const T* wrow(int m) const { return w + (long)m * (2 * H); }
  __device__ void store(int m, int, int row, float v) { xout[(long)row * H + m] = v; }
  // store, returning the residual-stream value written
  __device__ float reduce_store(int m, int, int row, float v) {
    xout[(long)row * H + m] = v;
    return v;
  }
};

// sin r and cos r for |r| <= pi/4 by their Taylor series through r^11 / 11! and r^12 / 12!: the
// first omitted terms are below 1e-11 there, far under float rounding.  Horner in float.
__device__ __forceinline__ void sincos_quarter(float r, float& s, float& c) {
  const float r2 = r * r;
  s = fmaf(r * r2,
           fmaf(r2, fmaf(r2, fmaf(r2, fmaf(r2, -2.5052108385441720e-8f, 2.7557319223985893e-6f),
                                 -1.9841269841269841e-4f),
                       8.3333333333333333e-3f),
                -1.6666666666666667e-1f),
           r);
  c = fmaf(r2,
           fmaf(r2, fmaf(r2, fmaf(r2, fmaf(r2, fmaf(r2, 2.0876756987868099e-9f, -2.7557319223985891e-7f),
                                         2.4801587301587302e-5f),
                                 -1.3888888888888889e-3f),
                       4.1666666666666667e-2f),
                -0.5f),
           1.0f);
}

// Q/K/V projection of rms(x) with RoPE on q and k and the K/V append.  Logical rows are
// ordered per head as (0, hd/2, 1, hd/2+1, ...) so a rotation pair is one (even, odd) pair.
template <class W>
struct PQKV : PBase<W> {
  using T = typename W::T;
  static constexpr int kNorm = 1;
  static constexpr bool kPair = true;
  const T *g, *wq, *wk, *wv;
  const float* xin;
  int H, nq, nkv, hd;
  double log_theta;
  float* qout;
  T *kc, *vc;  // this layer's cache: keys [B][nkv][max_len][hd], values [B][nkv][hd][max_len]
  int pos_off;  // row i of sequence b sits at position len[b] + i + pos_off
  const double* inv_freq;  // theta^(-2u/hd), u < hd/2, in LDS (set by setup)

  // Per-sequence rows and cache lengths, and the rotation frequencies (exp in double once per
  // workgroup instead of once per output pair).
  __device__ void setup_store(const typename PBase<W>::SeqPre& q, int* s_n, int* s_len) {
    PBase<W>::setup_store(q, s_n, s_len);
    __shared__ double s_inv_freq[64];  // head_dim <= 128
    for (int u = threadIdx.x; u < (hd >> 1); u += kWG)
      s_inv_freq[u] = exp(-2.0 * double(u) / double(hd) * log_theta);
    inv_freq = s_inv_freq;
  }
  __device__ void setup(int* s_n, int* s_len) { setup_store(this->setup_load(), s_n, s_len); }

  __device__ void load_x(int row, int k, float (&f)[W::VE]) const { load_f32_vec<W::VE>(xin + (long)row * H + k, f); }
  __device__ uint4 gain_raw(int k) const { return ld16(g + k); }
  static constexpr bool kRolledStore = true;
  __device__ const T* wrow(int m) const {
    const int head = m / hd, mm = m - head * hd;
    const int dim = (mm >> 1) + (mm & 1) * (hd >> 1);
    if (head < nq) return wq + ((long)head * hd + dim) * H;
    if (head < nq + nkv) return wk + ((long)(head - nq) * hd + dim) * H;
    return wv + ((long)(head - nq - nkv) * hd + dim) * H;
  }
  __device__ void store_pair(int m, int, int row, float v0, float v1) {
    const int head = m / hd, u = (m - head * hd) >> 1, half = hd >> 1;
    const int b = row / this->rps, i = row - b * this->rps;
    const int pos = this->lds_len[b] + i + pos_off;
    if (head < nq + nkv) {
      // rotate q and k by pos * theta^(-2u/hd): the angle in double, reduced to [-pi/4, pi/4]
      // in double (quadrant k, two-part pi/2), sine and cosine of the remainder in float by their
      // Taylor series (a library sincosf, inlined at every store, made these kernels up to ten
      // times larger), then placed by the quadrant: sin(r + k pi/2), cos(r + k pi/2)
      const double ang = double(pos) * inv_freq[u];
      const double kq = rint(ang * 0.6366197723675814);  // 2 / pi
      const double red = fma(-kq, 6.123233995736766e-17, fma(-kq, 1.5707963267948966, ang));
      float sq, cq;
      sincos_quarter(float(red), sq, cq);
      const int q = int(kq) & 3;  // ang >= 0
      const float sf = q == 0 ? sq : q == 1 ? cq : q == 2 ? -sq : -cq;
      const float cf = q == 0 ? cq : q == 1 ? -sq : q == 2 ? -cq : sq;
      const float a0 = v0 * cf - v1 * sf, a1 = v1 * cf + v0 * sf;
      v0 = a0;
      v1 = a1;
    }
    if (head < nq) {
      float* qp = qout + (long)row * nq * hd + (long)head * hd;
      qp[u] = v0;
      qp[u + half] = v1;
    } else if (head < nq + nkv) {  // key row at position pos
      T* dst = kc + (((long)b * nkv + head - nq) * this->max_len + pos) * hd;
      dst[u] = W::put(v0);
      dst[u + half] = W::put(v1);
    } else {  // value channels u and u + hd/2 at position pos (values are stored transposed)
      T* dst = vc + ((long)b * nkv + head - nq - nkv) * this->max_len * hd + pos;
      dst[(long)u * this->max_len] = W::put(v0);
      dst[(long)(u + half) * this->max_len] = W::put(v1);
    }
  }
};

// y = W a added into the residual stream (o_proj and down_proj)
template <class W>
struct PResidual : PBase<W> {
  using T = typename W::T;
  static constexpr int kNorm = 0;
  const T* w;
  const float* ain;  // [R][K]
  float* xres;       // [R][N]

  __device__ void load_x(int row, int k, float (&f)[W::VE]) const {
    load_f32_vec<W::VE>(ain + (long)row * this->K + k, f);
  }
  __device__ const T* wrow(int m) const { return w + (long)m * this->K; }
  __device__ void store(int m, int, int row, float v) { xres[(long)row * this->N + m] += v; }
  // store, returning the residual-stream value written
  __device__ float reduce_store(int m, int, int row, float v) {
    const float x = xres[(long)row * this->N + m] + v;
    xres[(long)row * this->N + m] = x;
    return x;
  }
};

// gate/up of rms(x), interleaved as (gate f, up f); stores silu(gate) * up
template <class W>
struct PGateUp : PBase<W> {
  using T = typename W::T;
  static constexpr int kNorm = 1;
  static constexpr bool kPair = true;
  const T *g, *wg, *wu;
  const float* xin;
  int H, F;
  float* aout;  // [R][F]

  __device__ void load_x(int row, int k, float (&f)[W::VE]) const { load_f32_vec<W::VE>(xin + (long)row * H + k, f); }
  __device__ uint4 gain_raw(int k) const { return ld16(g + k); }
  __device__ const T* wrow(int m) const { return ((m & 1) ? wu : wg) + (long)(m >> 1) * H; }
  __device__ void store_pair(int m, int, int row, float gt, float up) {
    aout[(long)row * F + (m >> 1)] = gt / (1.0f + expf(-gt)) * up;
  }
  // the same value, split into bf16 hi + lo at compact row cr of down_proj's activations instead
  // (the split k_prep would make of it): the down projection then takes it without a
  // preparation, so the fp32 row (read only by that preparation) is not written
  static constexpr bool kSplitOut = true;
  __device__ void store_pair_split(int m, int, int, int cr, float gt, float up, uint16_t* shi, uint16_t* slo) {
    const float y = gt / (1.0f + expf(-gt)) * up;
    const uint32_t h = bf16_rne(y);
    shi[(long)cr * F + (m >> 1)] = (uint16_t)h;
    slo[(long)cr * F + (m >> 1)] = (uint16_t)bf16_rne(y - __uint_as_float(h << 16));
  }
};

// final RMSNorm + lm_head + argmax for each sequence's last row; output hiddens; finalisation
template <class W>
struct PLmHead : PBase<W> {
  using T = typename W::T;
  static constexpr int kNorm = 1;
  static constexpr bool kArgmax = true;
  static constexpr bool kEarlyRows = false;  // the row of sequence b is its last valid one
  const T *g, *w;
  const float* xin;
  int H;
  float* logits;  // NULL or row b at logits + b * lg_sb
  long lg_sb;
  float* part_v;  // [B][gridDim]
  int* part_i;

  __device__ void act(int a, const int* s_n, int& row, bool& valid) const {
    valid = a < this->B && s_n[a] > 0;
    row = valid ? a * this->rps + s_n[a] - 1 : 0;
  }
  __device__ void load_x(int row, int k, float (&f)[W::VE]) const { load_f32_vec<W::VE>(xin + (long)row * H + k, f); }
  __device__ uint4 gain_raw(int k) const { return ld16(g + k); }
  __device__ const T* wrow(int m) const { return w + (long)m * H; }
  __device__ void store(int m, int a, int, float v) {
    if (logits) logits[(long)a * lg_sb + m] = v;
  }
  __device__ void partial(int a, float v, int i) {
    if (a < this->B) {
      part_v[(long)a * gridDim.x + blockIdx.x] = v;
      part_i[(long)a * gridDim.x + blockIdx.x] = i;
    }
  }
  __device__ void finish(const int* s_n) {
    // activation blocks with no valid row were skipped: their partials must still be written
    for (int a = threadIdx.x; a < this->B; a += kWG)
      if (s_n[a] == 0) {
        part_v[(long)a * gridDim.x + blockIdx.x] = -INFINITY;
        part_i[(long)a * gridDim.x + blockIdx.x] = 0x7fffffff;
      }
  }
};

// The target's output layer: final RMSNorm + lm_head for every valid row, logits stored
// [row][V] (row = b * rps + i).
template <class W>
struct PLogits : PBase<W> {
  using T = typename W::T;
  static constexpr int kNorm = 1;
  static constexpr bool kVocab = true;
  const T *g, *w;
  const float* xin;
  int H;
  float* logits;

  __device__ void load_x(int row, int k, float (&f)[W::VE]) const { load_f32_vec<W::VE>(xin + (long)row * H + k, f); }
  __device__ uint4 gain_raw(int k) const { return ld16(g + k); }
  __device__ const T* wrow(int m) const { return w + (long)m * H; }
  __device__ void store(int m, int, int row, float v) { logits[(long)row * this->N + m] = v; }
};

// The target's input: x[row] = E[tok] (fp32) for the valid rows; one workgroup per row.
template <class W>
__global__ __launch_bounds__(kWG) void k_embed_rows(const void* embed, const int32_t* tok, int tok_sb, int rps,
                                                    int V, const int32_t* len, int max_len, int H, float* x,
                                                    const int* rows) {
  using T = typename W::T;
  constexpr int VE = W::VE;
  __shared__ int s_n;
  const int row = blockIdx.x, b = row / rps, i = row - b * rps;
  if (threadIdx.x == 0)
    s_n = rows ? rows[b] : count_rows(tok + (long)b * tok_sb, rps, V, len[b], max_len, nullptr);
  __syncthreads();
  if (i >= s_n) return;
  const T* e = reinterpret_cast<const T*>(embed) + (long)tok[(long)b * tok_sb + i] * H;
  for (int k = threadIdx.x * VE; k < H; k += kWG * VE) {
    float f[VE];
    W::cvt(ld16(e + k), f);
#pragma unroll
    for (int j = 0; j < VE; ++j) x[(long)row * H + k + j] = f[j];
  }
}

// dst = rms(x) * g over one row of H floats (H a multiple of 8) by one wave: float4 loads, four
// in flight per lane, the row read twice (the second time from cache).
template <class W>
__device__ __forceinline__ void wave_rms_row(const float* x, float* dst, const typename W::T* g, int H, float eps,
                                             int lane) {
  const float4* xr = reinterpret_cast<const float4*>(x);
  float4* d4 = reinterpret_cast<float4*>(dst);
  const int H4 = H >> 2;
  float ss = 0.f;
#pragma unroll 4
  for (int c = lane; c < H4; c += 64) {
    const float4 v = xr[c];
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float sc = 1.0f / sqrtf(ss / float(H) + eps);
#pragma unroll 4
  for (int c = lane; c < H4; c += 64) {
    const float4 v = xr[c];
    const int k = 4 * c;
    d4[c] = make_float4(v.x * sc * W::get(g, k), v.y * sc * W::get(g, k + 1), v.z * sc * W::get(g, k + 2),
                        v.w * sc * W::get(g, k + 3));
  }
}

// After the lm_head: one workgroup per sequence reduces the per-workgroup argmax partials
// (the lowest id among equal maxima), writes the draft, grows len[b], records device errors,
// and writes the post-norm hidden of the rows the caller wants.
template <class W>
__global__ __launch_bounds__(kWG) void k_lm_finalize(LmFinal f) {
  using T = typename W::T;
  __shared__ float sv[4];
  __shared__ int si[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  int flags = 0;
  const int n = f.rows ? f.rows[b] : count_rows(f.tok + (long)b * f.tok_sb, f.rps, f.V, f.len[b], f.max_len, &flags);
  if (f.rows) flags = f.rows[f.B + b];
  float v = -INFINITY;
  int id = 0x7fffffff;
  for (int k = tid; k < f.nparts; k += kWG) {
    const float pv = f.part_v[(long)b * f.nparts + k];
    const int pi = f.part_i[(long)b * f.nparts + k];
    if (better(pv, pi, v, id)) {
      v = pv;
      id = pi;
    }
  }
  wave_argmax(v, id);
  if ((tid & 63) == 0) {
    sv[tid >> 6] = v;
    si[tid >> 6] = id;
  }
  __syncthreads();
  if (tid == 0) {  // the argmax of the workgroup, before sv is reused for the norm
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], sv[0], si[0])) {
        sv[0] = sv[w];
        si[0] = si[w];
      }
    v = sv[0];
    id = si[0];
  }
  __syncthreads();
  const T* g = reinterpret_cast<const T*>(f.gain);
  const int lane = tid & 63, wid = tid >> 6;
  if (f.hout && f.hout_last && n > 0 && f.H <= 8 * 4 * kWG) {
    // the last row only (a draft step's fed-back hidden): the whole workgroup, float4 loads held
    // in registers across the norm reduction
    const float4* xr = reinterpret_cast<const float4*>(f.x + ((long)b * f.rps + n - 1) * f.H);
    float4* dst = reinterpret_cast<float4*>(f.hout + (long)b * f.hout_sb * f.H);
    const int H4 = f.H >> 2;
    float4 xv[8];
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = tid + j * kWG;
      xv[j] = c < H4 ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) ss += xv[j].x * xv[j].x + xv[j].y * xv[j].y + xv[j].z * xv[j].z + xv[j].w * xv[j].w;
    ss = wave_sum(ss);
    if (lane == 0) sv[wid] = ss;
    __syncthreads();
    const float sc = 1.0f / sqrtf((sv[0] + sv[1] + sv[2] + sv[3]) / float(f.H) + f.eps);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = tid + j * kWG;
      if (c < H4) {
        const int k = 4 * c;
        dst[c] = make_float4(xv[j].x * sc * W::get(g, k), xv[j].y * sc * W::get(g, k + 1),
                             xv[j].z * sc * W::get(g, k + 2), xv[j].w * sc * W::get(g, k + 3));
      }
    }
  } else if (f.hout) {
    // every valid row (or the last of a wider one): wave w normalises rows first + w, first + w + 4, ...
    for (int i = (f.hout_last ? n - 1 : 0) + wid; i < n; i += kWG / 64)
      wave_rms_row<W>(f.x + ((long)b * f.rps + i) * f.H, f.hout + ((long)b * f.hout_sb + (f.hout_last ? 0 : i)) * f.H,
                      g, f.H, f.eps, lane);
  }
  if (tid == 0) {
    if (f.draft) f.draft[(long)b * f.dr_sb] = n > 0 ? id : -1;
    if (f.grow) f.len[b] = f.len[b] + n;
    if (flags) atomicOr(f.status, flags);
  }
}

// The post-norm hiddens of many rows (a prefill): one wave per row of the flattened [B][rps]
// rows, launched before k_lm_finalize grows the cache lengths.
template <class W>
__global__ __launch_bounds__(kWG) void k_hidden_out(LmFinal f) {
  using T = typename W::T;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kWG / 64) + (threadIdx.x >> 6);
  if (row >= f.B * f.rps) return;
  const int b = row / f.rps, i = row - b * f.rps;
  const int n = f.rows ? f.rows[b] : count_rows(f.tok + (long)b * f.tok_sb, f.rps, f.V, f.len[b], f.max_len, nullptr);
  if (i >= n || (f.hout_last && i != n - 1)) return;
  wave_rms_row<W>(f.x + (long)row * f.H, f.hout + ((long)b * f.hout_sb + (f.hout_last ? 0 : i)) * f.H,
                  reinterpret_cast<const T*>(f.gain), f.H, f.eps, lane);
}

// k_lm_finalize, with the hiddens of many-row calls written by k_hidden_out first.
template <class W>
hipError_t launch_finalize(LmFinal f, hipStream_t st) {
  if (f.hout && f.rps >= 8) {
    hipLaunchKernelGGL((k_hidden_out<W>), dim3((f.B * f.rps + kWG / 64 - 1) / (kWG / 64)), dim3(kWG), 0, st, f);
    f.hout = nullptr;
  }
  hipLaunchKernelGGL((k_lm_finalize<W>), dim3(f.B), dim3(kWG), 0, st, f);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// launch selection
// ---------------------------------------------------------------------------------------------
// Workgroups that can be resident at once for a kernel (occupancy x compute units), cached.
template <class K>
int resident_cap(K kernel, int* cache, int threads = kWG) {
  if (*cache == 0) {
    int dev = 0, cus = 0, nb = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    (void)hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(kernel), threads, 0);
    *cache = (nb < 1 ? 1 : nb) * (cus < 1 ? 1 : cus);
  }
  return *cache;
}

// Launch the planned variant with a grid of at most one resident wave of workgroups (the
// kernels loop over row groups), so no partial second wave of workgroups trails the first.
// The bf16 MFMA path (K a multiple of the 128-wide chunk) takes 16 or more activation rows, and
// fewer when the VALU GEMV would stream a large matrix more than once (more rows than it holds
// per pass).  A matrix of at most 32 MB stays on the GEMV for up to four passes: the passes after
// the first re-read it from the last-level cache, blocks of rows with no valid row are skipped
// (a catch-up call usually has one or two of its rows valid), and the MFMA path's preparation,
// split-K reduction and few workgroups (a small matrix has few weight tiles) cost more.  A call
// whose rows are all valid (the target's verify pass over D + 1 positions) has no blocks to skip:
// more rows than one GEMV pass holds take the MFMA path, whose fused preparations and reductions
// then chain through the layer (4-layer 2048-hidden stand-in at 7 rows: 0.540 -> 0.500 ms).
template <class W, class P>
bool use_mfma(const P& p, const MfmaBufs* mb) {
  if (!mb || !std::is_same<W, BF16>::value || p.K % kMfmaKC != 0) return false;  // K: whole 128-wide chunks
  if (p.nact >= 16) return true;
  const int rb = plan_gemv(p.nact, p.K, W::VE, p.N).rb;
  if (p.nact <= rb) return false;
  if (p.dense) return true;
  const long bytes = (long)p.N * p.K * (long)sizeof(typename W::T);
  return bytes > (32l << 20) || (p.nact + rb - 1) / rb > 4;
}

// Optional HIP events recorded around a GEMV/GEMM's main kernel (not its preparation or
// reduction launches), with that kernel's name.
struct KTimer {
  hipEvent_t b = nullptr, e = nullptr;
  const char** name = nullptr;
  void begin(hipStream_t st, const char* n) const {
    if (b) (void)hipEventRecord(b, st);
    if (b && name) *name = n;
  }
  void end(hipStream_t st) const {
    if (e) (void)hipEventRecord(e, st);
  }
};

// Compute units of the current device, cached.
inline int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (cus < 1) cus = 1;
  }
  return cus;
}

// Work decomposition of k_gemm_stream for an N x K matrix and up to nact activation rows: waves
// per workgroup, tiles per wave and K parts chosen to minimise the estimated time of the weight
// stream -- (rounds of workgroups over the compute units) x (bytes one workgroup streams) -- plus
// the split-K partial sums written and read back.  One workgroup runs per compute unit (LDS).
// How many rows are valid is known only on the device, so the plan fills the GPU with the items
// of one pass of 16 MT rows; a call with more valid rows takes one more round per extra pass.
struct SgChoice {
  SgPlan pl;
  int nt, mt, items;
};
inline SgChoice plan_stream(int N, int K, int nact, bool whole_rows, long part_room, int cap) {
  const int cus = device_cus();
  SgChoice best{};
  best.mt = nact <= 32 ? 2 : 4;
  const int nk = K / kSgKC, tiles = (N + 15) / 16;
  const int rc = best.mt <= 2 ? SgShape<2>::RC : SgShape<4>::RC;
  double best_t = 1e300;
  const int ks_opts[7] = {1, 2, 3, 4, 6, 8, 12};
  for (int nw = 7; nw <= kSgMaxWaves; ++nw)
    for (int nt = 1; nt <= 2; ++nt)
      for (int ks : ks_opts) {
        if (whole_rows && ks > 1) continue;
        // every K part holds at least two ranges (and so is never empty)
        if (ks > 1 && (nk / ks < 2 * rc || (long)(ks - 1) * ((nk + ks - 1) / ks) >= nk ||
                       (long)ks * cap * N > part_room))
          continue;
        const int sets = (tiles + nw * nt - 1) / (nw * nt);
        const long items = (long)sets * ks;
        const long rounds = (items + cus - 1) / cus;
        const double per_item = (double)nw * nt * 16 * ((double)K / ks) * 2;
        double t = rounds * per_item * cus;                           // bytes-equivalent of the stream
        if (ks > 1) t += 2.0 * ks * nact * (double)N * 4 + 4.0e7;     // partials + the reduce launch
        if (nt == 1 && best.mt == 4) t *= 1.5;                        // 64-row passes: operand reads
        if (t < best_t * 0.999) {
          best_t = t;
          best.pl.nw = nw;
          best.nt = nt;
          best.pl.ks = ks;
          best.pl.sets = sets;
          best.pl.kper = (nk + ks - 1) / ks;
          best.items = (int)items;
        }
      }
  return best;
}

// Replaces the split-K reduction after a stream GEMM (k_reduce_prep: the reduction fused with the
// next GEMM's activation split); `used` is set when it ran, so the next GEMM skips its own split.
using ReduceHook = std::function<hipError_t(const MfmaBufs&)>;
// split: a kSplitOut GEMM also writes its outputs split for the next GEMM (into mb.shi / slo).
struct ReduceCtx {
  const ReduceHook* hook = nullptr;
  bool split = false;
  bool* used = nullptr;
};

template <class P, int NT, int MT, int KPT, int AC = (MT <= 2 ? 256 : 128)>
hipError_t launch_stream_t(P& p, hipStream_t st, int* grid_used, const MfmaBufs& mb, const KTimer& tm,
                           const SgChoice& ch, const ReduceCtx& rc) {
  if (KPT * 64 * ch.pl.nw < SgShape<MT, AC>::SLICE || ch.pl.nw > sg_max_waves(NT, MT))
    return hipErrorInvalidConfiguration;
  MfmaBufs m = mb;
  if (ch.pl.ks <= 1) m.part = nullptr;
  m.ksplit = ch.pl.ks;
  if (!rc.split) m.shi = m.slo = nullptr;
  if (rc.split && rc.used) *rc.used = true;  // the epilogue or the reduction below writes them
  int grid = min(ch.items, device_cus());
  grid = max(1, min(grid, kMaxGemvGrid));
  if (grid_used) *grid_used = grid;
  static const char* const names[2][7] = {
      {"", "k_gemm_stream<NT=1,MT=2>", "k_gemm_stream<NT=2,MT=2>", "k_gemm_stream<NT=3,MT=2>",
       "k_gemm_stream<NT=4,MT=2>", "k_gemm_stream<NT=5,MT=2>", "k_gemm_stream<NT=6,MT=2>"},
      {"", "k_gemm_stream<NT=1,MT=4>", "k_gemm_stream<NT=2,MT=4>", "k_gemm_stream<NT=3,MT=4>",
       "k_gemm_stream<NT=4,MT=4>", "k_gemm_stream<NT=5,MT=4>", "k_gemm_stream<NT=6,MT=4>"}};
  static_assert(NT >= 1 && NT <= 6 && (MT == 2 || MT == 4), "kernel name table");
  const char* name = names[MT == 4][NT];
  tm.begin(st, name);
  hipLaunchKernelGGL((k_gemm_stream<P, NT, MT, KPT, AC>), dim3(grid), dim3(64 * ch.pl.nw), 0, st, p, m, ch.pl);
  tm.end(st);
  if (m.part && rc.hook) {
    const hipError_t e = (*rc.hook)(m);
    if (rc.used) *rc.used = e == hipSuccess;
    return e;
  }
  if (m.part) {
    const long items = (long)m.cap * (p.N / 4);
    const int rgrid = (int)std::min<long>((items + kWG - 1) / kWG, 4096);
    hipLaunchKernelGGL((k_splitk_reduce<P>), dim3(rgrid), dim3(kWG), 0, st, p, m);
  }
  return hipGetLastError();
}

// The skinny MFMA GEMM: lm_head (argmax) and the target's lm_head keep whole rows (no split K)
// with two tiles per wave; the other matrices take the planned decomposition.
template <class P>
hipError_t launch_stream(P& p, hipStream_t st, int* grid_used, const MfmaBufs& mb, const KTimer& tm,
                         const ReduceCtx& rc) {
  const bool whole = P::kArgmax || P::kVocab;
  SgChoice ch;
  if (whole) {
    ch.mt = p.nact <= 32 ? 2 : 4;
    ch.nt = 2;
    if (ch.mt == 2) {
      // tiles per wave (8 waves): the fewest rounds of workgroups over the compute units, each
      // round weighted by the tiles one workgroup streams over its measured share of the HBM
      // peak (two tiles 0.76, three 0.80, four or five 0.82); 151936 rows take five tiles (238
      // sets in one round) where four would need 297 sets, two rounds
      const int tiles = (p.N + 15) / 16, cus = device_cus();
      double best = 1e300;
      for (int nt = 2; nt <= 5; ++nt) {
        const int sets = (tiles + 8 * nt - 1) / (8 * nt);
        const double t = (double)((sets + cus - 1) / cus) * nt / (nt == 2 ? 0.76 : nt == 3 ? 0.80 : 0.82);
        if (t < best * 0.999) {
          best = t;
          ch.nt = nt;
        }
      }
    }
    ch.pl.nw = 8;
    ch.pl.ks = 1;
    ch.pl.kper = p.K / kSgKC;
    ch.pl.sets = (p.N + 8 * ch.nt * 16 - 1) / (8 * ch.nt * 16);
    const int npass = P::kArgmax ? 1 : (p.nact + 16 * ch.mt - 1) / (16 * ch.mt);
    ch.items = npass * ch.pl.sets;
  } else {
    ch = plan_stream(p.N, p.K, p.nact, false, mb.part ? mb.part_cap : 0, mb.cap);
  }
  // activation pieces per thread and chunk: ceil(SLICE / threads); 512 pieces (32-row passes):
  // 2 with 7 waves, 1 with 8 or 9; 1024 pieces (64-row passes): 3 with 7 waves, 2 with 8 or 9
  const bool seven = ch.pl.nw == 7;
  if constexpr (P::kArgmax || P::kVocab) {  // 8 waves; 32-row passes with three or more tiles
    // take 128-column activation ranges (fewer activation operand reads per weight byte)
    if (ch.mt == 2) {
      switch (ch.nt) {
        case 3: return launch_stream_t<P, 3, 2, 1, 128>(p, st, grid_used, mb, tm, ch, rc);
        case 4: return launch_stream_t<P, 4, 2, 1, 128>(p, st, grid_used, mb, tm, ch, rc);
        case 5: return launch_stream_t<P, 5, 2, 1, 128>(p, st, grid_used, mb, tm, ch, rc);
        default: return launch_stream_t<P, 2, 2, 1>(p, st, grid_used, mb, tm, ch, rc);
      }
    }
    return launch_stream_t<P, 2, 4, 2>(p, st, grid_used, mb, tm, ch, rc);
  } else {
    if (ch.mt == 2) {
      if (ch.nt == 2)
        return seven ? launch_stream_t<P, 2, 2, 2>(p, st, grid_used, mb, tm, ch, rc)
                     : launch_stream_t<P, 2, 2, 1>(p, st, grid_used, mb, tm, ch, rc);
      return seven ? launch_stream_t<P, 1, 2, 2>(p, st, grid_used, mb, tm, ch, rc)
                   : launch_stream_t<P, 1, 2, 1>(p, st, grid_used, mb, tm, ch, rc);
    }
    if (ch.nt == 2)
      return seven ? launch_stream_t<P, 2, 4, 3>(p, st, grid_used, mb, tm, ch, rc)
                   : launch_stream_t<P, 2, 4, 2>(p, st, grid_used, mb, tm, ch, rc);
    return seven ? launch_stream_t<P, 1, 4, 3>(p, st, grid_used, mb, tm, ch, rc)
                 : launch_stream_t<P, 1, 4, 2>(p, st, grid_used, mb, tm, ch, rc);
  }
}

// rc: a split-K stream GEMM's reduction may be replaced (the fused reduction + next split);
// prepped: the split activations were already written by the previous GEMM's fused reduction.
template <class W, class P>
hipError_t launch_gemv(P& p, hipStream_t st, int* grid_used = nullptr, const MfmaBufs* mb = nullptr,
                       const KTimer& tm = KTimer(), const ReduceCtx& rc = ReduceCtx(), bool prepped = false) {
  if constexpr (std::is_same<W, BF16>::value) {
    if (use_mfma<W>(p, mb)) {
      // the whole row in registers, with no more chunks per thread than the row has (fewer
      // registers: more rows resident; the chunks and sums are the same for every choice)
      if (prepped) {
      } else if (p.K > 4 * kWG * W::VE) {  // rows wider than 8192
        hipLaunchKernelGGL((k_prep<W, P, 12>), dim3(p.nact), dim3(kWG), 0, st, p, *mb);
      } else if (p.K > 2 * kWG * W::VE) {
        hipLaunchKernelGGL((k_prep<W, P, 4>), dim3(p.nact), dim3(kWG), 0, st, p, *mb);
      } else if (p.K > kWG * W::VE) {
        hipLaunchKernelGGL((k_prep<W, P, 2>), dim3(p.nact), dim3(kWG), 0, st, p, *mb);
      } else {
        hipLaunchKernelGGL((k_prep<W, P, 1>), dim3(p.nact), dim3(kWG), 0, st, p, *mb);
      }
      if constexpr (!P::kArgmax) {
        // hundreds of rows (a prefill, by the activation count, an upper bound of the valid
        // rows): 128 x 256 output tiles, even when they do not fill the GPU -- the streaming
        // kernel would read the weights once per 64 rows (2048 rows of a 3072 x 2048 QKV: 1.2 ms
        // against ~0.1 ms)
        static int cap = 0;
        const long tiles = (long)((p.nact + kTileM - 1) / kTileM) * ((p.N + kTileN - 1) / kTileN);
        if (p.nact >= kTileRows) {
          const int slots = resident_cap(k_gemm_tile<P>, &cap, kTileThreads);
          // K ranges side by side while they all fit the resident slots (one workgroup per
          // compute unit; 2048 rows of down_proj, 2048 x 6144: 211 -> 125 us at two ranges; QKV's
          // 192 tiles stay whole: two ranges would take 1.5 rounds), each range at least
          // kTileMinPairs pairs of chunks, the partials within the buffer
          const int npairs = p.K / (2 * kTileK);
          int ks = 1;
          while (mb->part && tiles * (ks + 1) <= slots && npairs >= kTileMinPairs * (ks + 1) &&
                 (long)(ks + 1) * mb->cap * p.N <= mb->part_cap)
            ++ks;
          MfmaBufs m = *mb;
          m.ksplit = ks;
          if (ks <= 1) m.part = nullptr;
          if (!rc.split) m.shi = m.slo = nullptr;
          const int grid = (int)std::min<long>(tiles * ks, slots);
          if (grid_used) *grid_used = grid;
          tm.begin(st, "k_gemm_tile");
          hipLaunchKernelGGL((k_gemm_tile<P>), dim3(grid), dim3(kTileThreads), 0, st, p, m);
          tm.end(st);
          if (m.part && rc.hook) {
            const hipError_t e = (*rc.hook)(m);
            if (rc.used) *rc.used = e == hipSuccess;
            return e;
          }
          if (m.part) {
            const long items = (long)m.cap * (p.N / 4);
            const int rgrid = (int)std::min<long>((items + kWG - 1) / kWG, 4096);
            hipLaunchKernelGGL((k_splitk_reduce<P>), dim3(rgrid), dim3(kWG), 0, st, p, m);
          }
          // the split activations of a kSplitOut policy: by the tile epilogue or the reduction
          if (rc.split && rc.used) *rc.used = true;
          return hipGetLastError();
        }
      }
      // 32-row passes for a batch of serial steps, 64-row passes above (by the activation count,
      // an upper bound of the valid rows)
      return launch_stream(p, st, grid_used, *mb, tm, rc);
    }
  }
  const GemvPlan pl = plan_gemv(p.nact, p.K, W::VE, p.N);
  if (pl.kind == 0) {
#define MTP_W(NJ_, RB_, RW_)                                                                 \
  if (pl.nj == NJ_ && pl.rb == RB_ && pl.rw == RW_) {                                         \
    static int cap = 0;                                                                      \
    const int grid = min(pl.grid, resident_cap(k_gemv_w<W, RB_, NJ_, RW_, P>, &cap));       \
    if (grid_used) *grid_used = grid;                                                        \
    tm.begin(st, "k_gemv_w (VALU GEMV, whole rows per wave)");                                \
    hipLaunchKernelGGL((k_gemv_w<W, RB_, NJ_, RW_, P>), dim3(grid), dim3(kWG), 0, st, p);    \
    tm.end(st);                                                                              \
    return hipGetLastError();                                                                \
  }
    MTP_W(1, 1, 16) MTP_W(1, 2, 16) MTP_W(1, 4, 16) MTP_W(2, 1, 8) MTP_W(2, 2, 8) MTP_W(2, 4, 8)
    MTP_W(1, 1, 8) MTP_W(1, 2, 8) MTP_W(1, 4, 8) MTP_W(1, 1, 4) MTP_W(1, 2, 4) MTP_W(1, 4, 4)
    MTP_W(1, 1, 2) MTP_W(1, 2, 2) MTP_W(1, 4, 2) MTP_W(2, 1, 4) MTP_W(2, 2, 4) MTP_W(2, 4, 4)
    MTP_W(2, 1, 2) MTP_W(2, 2, 2) MTP_W(2, 4, 2)
    MTP_W(4, 1, 2) MTP_W(4, 2, 2)
#undef MTP_W
  } else {
#define MTP_S(NX_, RB_, RW_)                                                                 \
  if (pl.nj == NX_ && pl.rb == RB_ && pl.rw == RW_) {                                          \
    static int cap = 0;                                                                      \
    const int grid = min(pl.grid, resident_cap(k_gemv_s<W, RB_, NX_, RW_, P>, &cap));        \
    if (grid_used) *grid_used = grid;                                                        \
    tm.begin(st, "k_gemv_s (VALU GEMV, rows split over the workgroup)");                      \
    hipLaunchKernelGGL((k_gemv_s<W, RB_, NX_, RW_, P>), dim3(grid), dim3(kWG), 0, st, p);    \
    tm.end(st);                                                                              \
    return hipGetLastError();                                                                \
  }
    MTP_S(2, 1, 8) MTP_S(2, 2, 8) MTP_S(2, 4, 8) MTP_S(2, 1, 4) MTP_S(2, 2, 4) MTP_S(2, 4, 4)
    MTP_S(2, 1, 2) MTP_S(2, 2, 2) MTP_S(2, 4, 2) MTP_S(4, 1, 2) MTP_S(4, 2, 2) MTP_S(4, 4, 2)
    MTP_S(8, 1, 2) MTP_S(8, 2, 2) MTP_S(16, 1, 2)
    MTP_S(4, 1, 8) MTP_S(4, 2, 8) MTP_S(4, 4, 8) MTP_S(8, 1, 8) MTP_S(8, 2, 8) MTP_S(16, 1, 8)
    MTP_S(4, 1, 4) MTP_S(4, 2, 4) MTP_S(4, 4, 4) MTP_S(8, 1, 4) MTP_S(8, 2, 4) MTP_S(16, 1, 4)
#undef MTP_S
  }
  return hipErrorInvalidValue;
}

// The per-step row counts when the call has many rows per sequence, else NULL.
inline const int* step_rows(const StepArgs& s) { return s.shared || s.rps > kInlineRows ? s.ws.rows : nullptr; }

template <class W, class P>
void fill_base(P& p, const StepArgs& s) {
  p.tok = s.tok;
  p.tok_sb = s.tok_sb;
  p.B = s.B;
  p.rps = s.rps;
  p.len = s.kv_len;
  p.max_len = s.max_len;
  p.V = s.cfg.vocab;
  p.eps = s.cfg.rms_eps;
  p.split = 0;
  p.rows = step_rows(s);
  p.dense = s.target;
}

// Policy pairs whose split-K reduction and next activation split run as one k_reduce_prep: a
// GEMM writing the residual stream followed by one that normalises it.
template <class P, class Pn>
struct CanFuse : std::false_type {};
template <class W>
struct CanFuse<PEhProj<W>, PQKV<W>> : std::true_type {};
template <class W>
struct CanFuse<PResidual<W>, PGateUp<W>> : std::true_type {};
template <class W>
struct CanFuse<PResidual<W>, PQKV<W>> : std::true_type {};
template <class W>
struct CanFuse<PResidual<W>, PLmHead<W>> : std::true_type {};

template <class W, class P, class Pn>
hipError_t launch_reduce_prep(const P& p, const Pn& pn, const MfmaBufs& m, hipStream_t st) {
  // as many chunks per thread as the row needs (the 2048-wide rows of a prefill: one chunk, 38
  // registers instead of 146, so more rows resident at once)
  if (p.N <= kWG * 8)
    hipLaunchKernelGGL((k_reduce_prep<W, P, Pn, 1>), dim3(p.nact), dim3(kWG), 0, st, p, pn, m);
  else if (p.N <= 2 * kWG * 8)
    hipLaunchKernelGGL((k_reduce_prep<W, P, Pn, 2>), dim3(p.nact), dim3(kWG), 0, st, p, pn, m);
  else if (p.N <= 4 * kWG * 8)
    hipLaunchKernelGGL((k_reduce_prep<W, P, Pn, 4>), dim3(p.nact), dim3(kWG), 0, st, p, pn, m);
  else
    hipLaunchKernelGGL((k_reduce_prep<W, P, Pn, 12>), dim3(p.nact), dim3(kWG), 0, st, p, pn, m);
  return hipGetLastError();
}

// Where the next GEMM of a step finds its split activations already written: nowhere (it runs
// its own k_prep), in the primary buffers (a fused reduction), or in the SwiGLU split buffers
// (written by the gate/up GEMM for down_proj).
enum class Prepped { kNo, kPrimary, kSwiglu };

template <class P, class Pn>
struct SplitsFor : std::false_type {};
template <class W>
struct SplitsFor<PGateUp<W>, PResidual<W>> : std::true_type {};

// Launch one GEMM of the step.  With a following GEMM `next` that can take its outputs already
// prepared (both on the MFMA path, the row width within the fused kernel's registers), either
// the split-K reduction is replaced by k_reduce_prep or the GEMM writes the split itself;
// `prepped` carries what ran into the next launch.
template <class W, class P, class Pn>
hipError_t step_gemm(P& p, const Pn* next, const MfmaBufs* mb, hipStream_t st, Prepped& prepped,
                     int* grid_used = nullptr, const KTimer& tm = KTimer()) {
  const Prepped have = prepped;
  prepped = Prepped::kNo;
  MfmaBufs alt;
  const MfmaBufs* use = mb;
  if (mb && have == Prepped::kSwiglu) {
    alt = *mb;
    alt.xhi = mb->shi;
    alt.xlo = mb->slo;
    use = &alt;
  }
  ReduceHook hook;
  ReduceCtx rc;
  bool used = false, split = false;
  if constexpr (std::is_same<W, BF16>::value && CanFuse<P, Pn>::value) {
    if (next && mb && p.N == next->K && p.N % 8 == 0 && p.N <= 12 * kWG * 8 && use_mfma<W>(p, mb) &&
        use_mfma<W>(*next, mb)) {
      // the next GEMM's activations go to the primary buffers (this GEMM has finished with them)
      hook = [&p, next, st, mb](const MfmaBufs& m) {
        MfmaBufs m2 = m;
        m2.xhi = mb->xhi;
        m2.xlo = mb->xlo;
        return launch_reduce_prep<W>(p, *next, m2, st);
      };
      rc.hook = &hook;
      rc.used = &used;
    }
  }
  if constexpr (std::is_same<W, BF16>::value && SplitsFor<P, Pn>::value) {
    if (next && mb && mb->shi && 2 * next->K == p.N && use_mfma<W>(p, mb) && use_mfma<W>(*next, mb)) {
      rc.split = split = true;
      rc.used = &used;
    }
  }
  const hipError_t e = launch_gemv<W>(p, st, grid_used, use, tm, rc, have != Prepped::kNo);
  if (used) prepped = split ? Prepped::kSwiglu : Prepped::kPrimary;
  return e;
}

template <class W>
hipError_t run_step_t(const StepArgs& s) {
  using T = typename W::T;
  const mtp_config& c = s.cfg;
  const int H = c.hidden, F = c.ffn, nq = c.n_heads, nkv = c.n_kv_heads, hd = c.head_dim;
  const int R = s.B * s.rps;
  hipError_t e;
  const MfmaBufs mbuf = {s.ws.xhi, s.ws.xlo, s.ws.rowmap, s.ws.amap, s.ws.mcount, s.ws.kpart, 1, s.B * s.rps,
                         s.ws.kpart_cap, s.ws.shi, s.ws.slo};
  const MfmaBufs* mb = s.ws.xhi ? &mbuf : nullptr;

  if (step_rows(s) && (e = count_step_rows(s)) != hipSuccess) return e;
  const mtp_layer_weights* layers = s.target ? s.tw->layers : s.w->layers;
  // the step's GEMM policies, built ahead so that each launch knows the GEMM after it
  auto layer_off = [&](int l) { return (long)(s.kv_layer ? s.kv_layer[l] : l) * s.B * nkv * s.max_len * hd; };
  auto make_qkv = [&](int l) {  // q/k/v + RoPE + append
    const mtp_layer_weights& lw = layers[l];
    PQKV<W> p;
    fill_base<W>(p, s);
    p.K = H;
    p.N = (nq + (s.shared ? 0 : 2 * nkv)) * hd;  // a head reading another cache projects q only
    p.nact = R;
    p.g = (const T*)lw.in_norm;
    p.wq = (const T*)lw.wq;
    p.wk = (const T*)lw.wk;
    p.wv = (const T*)lw.wv;
    p.xin = s.ws.x;
    p.H = H;
    p.nq = nq;
    p.nkv = nkv;
    p.hd = hd;
    p.log_theta = log((double)c.rope_theta);
    p.qout = s.ws.q;
    p.kc = (T*)s.kc + layer_off(l);
    p.vc = (T*)s.vc + layer_off(l);
    p.pos_off = s.pos_off;
    return p;
  };
  auto make_lm = [&]() {  // final norm + lm_head + argmax
    PLmHead<W> p;
    fill_base<W>(p, s);
    p.K = H;
    p.N = c.vocab;
    p.nact = s.B;
    p.g = (const T*)s.w->final_norm;
    p.w = (const T*)s.w->lm_head;
    p.xin = s.ws.x;
    p.H = H;
    p.logits = s.logits;
    p.lg_sb = s.lg_sb;
    p.part_v = s.ws.lm_part_v;
    p.part_i = s.ws.lm_part_i;
    return p;
  };
  const bool head = !s.target && !s.no_head;
  PLmHead<W> plm;
  if (head) plm = make_lm();
  Prepped prepped = Prepped::kNo;  // where the next GEMM's split activations already are
  PQKV<W> pqkv = make_qkv(0);
  if (s.target) {  // the target's input: token embeddings
    hipLaunchKernelGGL((k_embed_rows<W>), dim3(R), dim3(kWG), 0, s.stream, s.tw->embed, s.tok, s.tok_sb, s.rps,
                       c.vocab, s.kv_len, s.max_len, H, s.ws.x, step_rows(s));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {  // eh_proj
    PEhProj<W> p;
    fill_base<W>(p, s);
    p.K = 2 * H;
    p.N = H;
    p.nact = R;
    p.split = H;
    p.embed = (const T*)s.w->embed;
    p.enorm = (const T*)s.w->enorm;
    p.hnorm = (const T*)s.w->hnorm;
    p.w = (const T*)s.w->eh_proj;
    p.hin = s.hin;
    p.hin_sb = s.hin_sb;
    p.H = H;
    p.xout = s.ws.x;
    if ((e = step_gemm<W>(p, &pqkv, mb, s.stream, prepped)) != hipSuccess) return e;
  }
  for (int l = 0; l < c.n_layers; ++l) {
    const mtp_layer_weights& lw = layers[l];
    if ((e = step_gemm<W>(pqkv, (const PQKV<W>*)nullptr, mb, s.stream, prepped)) != hipSuccess) return e;
    PResidual<W> po;  // o_proj + residual
    fill_base<W>(po, s);
    po.K = nq * hd;
    po.N = H;
    po.nact = R;
    po.w = (const T*)lw.wo;
    po.ain = s.ws.attn_out;
    po.xres = s.ws.x;
    {  // attention
      AttnArgs a;
      a.q = s.ws.q;
      a.kc = (const T*)s.kc + layer_off(l);
      a.vc = (const T*)s.vc + layer_off(l);
      a.tok = s.tok;
      a.tok_sb = s.tok_sb;
      a.len = s.kv_len;
      a.B = s.B;
      a.rps = s.rps;
      a.nq = nq;
      a.nkv = nkv;
      a.max_len = s.max_len;
      a.V = c.vocab;
      a.nsplit = s.nsplit;
      a.qstride = s.rps * (nq / nkv);
      a.part = s.ws.attn_part;
      a.rows = step_rows(s);
      a.shared = s.shared;
      a.shi = a.slo = nullptr;
      if (mb && use_mfma<W>(po, mb)) {  // o_proj's split activations straight from the attention
        a.shi = mb->xhi;
        a.slo = mb->xlo;
      }
      if ((e = run_attention(a, hd, c.wdtype, s.ws.attn_out, s.stream)) != hipSuccess) return e;
      if (a.shi) prepped = Prepped::kPrimary;
    }
    PGateUp<W> pgu;  // gate/up + SwiGLU
    fill_base<W>(pgu, s);
    pgu.K = H;
    pgu.N = 2 * F;
    pgu.nact = R;
    pgu.g = (const T*)lw.post_norm;
    pgu.wg = (const T*)lw.wgate;
    pgu.wu = (const T*)lw.wup;
    pgu.xin = s.ws.x;
    pgu.H = H;
    pgu.F = F;
    pgu.aout = s.ws.act;
    if ((e = step_gemm<W>(po, &pgu, mb, s.stream, prepped)) != hipSuccess) return e;
    PResidual<W> pdn;  // down + residual
    fill_base<W>(pdn, s);
    pdn.K = F;
    pdn.N = H;
    pdn.nact = R;
    pdn.w = (const T*)lw.wdown;
    pdn.ain = s.ws.act;
    pdn.xres = s.ws.x;
    if ((e = step_gemm<W>(pgu, &pdn, mb, s.stream, prepped)) != hipSuccess) return e;
    {  // then the next layer's q/k/v or the lm_head
      PResidual<W>& p = pdn;
      if (l + 1 < c.n_layers) {
        pqkv = make_qkv(l + 1);
        e = step_gemm<W>(p, &pqkv, mb, s.stream, prepped);
      } else {
        e = step_gemm<W>(p, head ? &plm : nullptr, mb, s.stream, prepped);
      }
      if (e != hipSuccess) return e;
    }
  }
  if (s.target) {  // final norm + lm_head over every valid row, hiddens, len
    PLogits<W> p;
    fill_base<W>(p, s);
    p.K = H;
    p.N = c.vocab;
    p.nact = R;
    p.g = (const T*)s.tw->final_norm;
    p.w = (const T*)s.tw->lm_head;
    p.xin = s.ws.x;
    p.H = H;
    p.logits = s.logits;
    if ((e = launch_gemv<W>(p, s.stream, nullptr, mb)) != hipSuccess) return e;
    LmFinal f;
    f.B = s.B;
    f.tok = s.tok;
    f.tok_sb = s.tok_sb;
    f.rps = s.rps;
    f.V = c.vocab;
    f.len = s.kv_len;
    f.max_len = s.max_len;
    f.part_v = nullptr;
    f.part_i = nullptr;
    f.nparts = 0;
    f.x = s.ws.x;
    f.gain = s.tw->final_norm;
    f.H = H;
    f.eps = c.rms_eps;
    f.hout = s.hout;
    f.hout_sb = s.hout_sb;
    f.hout_last = 0;
    f.draft = nullptr;
    f.dr_sb = 0;
    f.status = s.ws.status;
    f.rows = step_rows(s);
    f.grow = !s.shared;
    return launch_finalize<W>(f, s.stream);
  }
  if (s.no_head) {  // K/V appended: only the lengths (and device errors) remain
    LmFinal f = {};
    f.B = s.B;
    f.tok = s.tok;
    f.tok_sb = s.tok_sb;
    f.rps = s.rps;
    f.V = c.vocab;
    f.len = s.kv_len;
    f.max_len = s.max_len;
    f.x = s.ws.x;
    f.H = H;
    f.status = s.ws.status;
    f.rows = step_rows(s);
    f.grow = 1;
    return launch_finalize<W>(f, s.stream);
  }
  {  // final norm + lm_head + argmax + finalisation
    int grid = 0;
    KTimer tm;
    tm.b = s.ev_begin;
    tm.e = s.ev_end;
    tm.name = s.ev_name;
    e = step_gemm<W>(plm, (const PQKV<W>*)nullptr, mb, s.stream, prepped, &grid, tm);
    if (e != hipSuccess) return e;
    LmFinal f;
    f.B = s.B;
    f.tok = s.tok;
    f.tok_sb = s.tok_sb;
    f.rps = s.rps;
    f.V = c.vocab;
    f.len = s.kv_len;
    f.max_len = s.max_len;
    f.part_v = s.ws.lm_part_v;
    f.part_i = s.ws.lm_part_i;
    f.nparts = grid;
    f.x = s.ws.x;
    f.gain = s.w->final_norm;
    f.H = H;
    f.eps = c.rms_eps;
    f.hout = s.hout;
    f.hout_sb = s.hout_sb;
    f.hout_last = s.hout_last;
    f.draft = s.draft;
    f.dr_sb = s.dr_sb;
    f.status = s.ws.status;
    f.rows = step_rows(s);
    f.grow = !s.shared;
    e = launch_finalize<W>(f, s.stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace mtp
