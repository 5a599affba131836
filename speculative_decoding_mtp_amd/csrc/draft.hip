// Draft-head kernels: the GEMV policies of one MTP step and the decode attention.
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
#include "draft.h"
#include "gemv.h"

namespace mtp {

// ---------------------------------------------------------------------------------------------
// common part of every drafter GEMV policy: row addressing and validity
// ---------------------------------------------------------------------------------------------
template <class W>
struct PBase {
  using T = typename W::T;
  const int32_t* tok;
  int tok_sb;
  int B, rps;
  const int32_t* len;
  int max_len, V;
  int K, N, nact, split;
  float eps;

  __device__ void setup(int* s_n) const {
    for (int b = threadIdx.x; b < B; b += kWG)
      s_n[b] = count_rows(tok + (long)b * tok_sb, rps, V, len[b], max_len, nullptr);
  }
  __device__ void act(int a, const int* s_n, int& row, bool& valid) const {
    row = a;
    valid = false;
    if (a < B * rps) {
      const int b = a / rps, i = a - b * rps;
      valid = i < s_n[b];
    }
  }
  template <int RB>
  __device__ void act_block_done(int, const int (&)[RB], const bool (&)[RB]) {}
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

  __device__ void load_x(int row, int k, float (&f)[W::VE]) const {
    const int b = row / this->rps, i = row - b * this->rps;
    if (k < H) {
      const int t = this->tok[(long)b * this->tok_sb + i];
      W::cvt(ld16(embed + (long)t * H + k), f);
    } else {
      load_f32_vec<W::VE>(hin + ((long)b * hin_sb + i) * H + (k - H), f);
    }
  }
  __device__ void gain_vec(int k, float (&f)[W::VE]) const { W::cvt(ld16(k < H ? enorm + k : hnorm + (k - H)), f); }
  __device__ const T* wrow(int m) const { return w + (long)m * (2 * H); }
  template <int ROWS, int RB>
  __device__ void epilogue(int m0, const float* tile, const int (&rows)[RB], const bool (&valid)[RB], int) {
    for (int idx = threadIdx.x; idx < ROWS * RB; idx += kWG) {
      const int q = idx / RB, r = idx % RB;
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
        if (rr == r && valid[rr] && m0 + q < this->N) xout[(long)rows[rr] * H + m0 + q] = tile[idx];
    }
  }
};

// Q/K/V projection of rms(x) with RoPE on q and k and the K/V append.  Logical rows are
// ordered per head as (0, hd/2, 1, hd/2+1, ...) so a rotation pair lands in one tile.
template <class W>
struct PQKV : PBase<W> {
  using T = typename W::T;
  static constexpr int kNorm = 1;
  const T *g, *wq, *wk, *wv;
  const float* xin;
  int H, nq, nkv, hd;
  double log_theta;
  float* qout;
  T *kc, *vc;  // this layer's cache [B][nkv][max_len][hd]

  __device__ void load_x(int row, int k, float (&f)[W::VE]) const { load_f32_vec<W::VE>(xin + (long)row * H + k, f); }
  __device__ void gain_vec(int k, float (&f)[W::VE]) const { W::cvt(ld16(g + k), f); }
  __device__ const T* wrow(int m) const {
    const int head = m / hd, mm = m - head * hd;
    const int dim = (mm >> 1) + (mm & 1) * (hd >> 1);
    if (head < nq) return wq + ((long)head * hd + dim) * H;
    if (head < nq + nkv) return wk + ((long)(head - nq) * hd + dim) * H;
    return wv + ((long)(head - nq - nkv) * hd + dim) * H;
  }
  template <int ROWS, int RB>
  __device__ void epilogue(int m0, const float* tile, const int (&rows)[RB], const bool (&valid)[RB], int) {
    for (int idx = threadIdx.x; idx < (ROWS / 2) * RB; idx += kWG) {
      const int qq = idx / RB, r = idx % RB;
      int row = -1;
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
        if (rr == r && valid[rr]) row = rows[rr];
      const int m = m0 + 2 * qq;
      if (row < 0 || m >= this->N) continue;
      const int head = m / hd, u = (m - head * hd) >> 1, half = hd >> 1;
      float v0 = tile[(2 * qq) * RB + r], v1 = tile[(2 * qq + 1) * RB + r];
      const int b = row / this->rps, i = row - b * this->rps;
      const int pos = this->len[b] + i;
      if (head < nq + nkv) {
        const double ang = double(pos) * exp(-2.0 * double(u) / double(hd) * log_theta);
        double s, c;
        sincos(ang, &s, &c);
        const float cf = float(c), sf = float(s);
        const float a0 = v0 * cf - v1 * sf, a1 = v1 * cf + v0 * sf;
        v0 = a0;
        v1 = a1;
      }
      if (head < nq) {
        float* qp = qout + (long)row * nq * hd + (long)head * hd;
        qp[u] = v0;
        qp[u + half] = v1;
      } else {
        const int kvh = head < nq + nkv ? head - nq : head - nq - nkv;
        T* dst = (head < nq + nkv ? kc : vc) + (((long)b * nkv + kvh) * this->max_len + pos) * hd;
        dst[u] = W::put(v0);
        dst[u + half] = W::put(v1);
      }
    }
  }
};

// y = W a with the result added into the residual stream (o_proj and down_proj)
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
  __device__ void gain_vec(int, float (&f)[W::VE]) const {
#pragma unroll
    for (int e = 0; e < W::VE; ++e) f[e] = 1.f;
  }
  __device__ const T* wrow(int m) const { return w + (long)m * this->K; }
  template <int ROWS, int RB>
  __device__ void epilogue(int m0, const float* tile, const int (&rows)[RB], const bool (&valid)[RB], int) {
    for (int idx = threadIdx.x; idx < ROWS * RB; idx += kWG) {
      const int q = idx / RB, r = idx % RB;
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
        if (rr == r && valid[rr] && m0 + q < this->N) xres[(long)rows[rr] * this->N + m0 + q] += tile[idx];
    }
  }
};

// gate/up of rms(x) interleaved as (gate f, up f); writes silu(gate) * up
template <class W>
struct PGateUp : PBase<W> {
  using T = typename W::T;
  static constexpr int kNorm = 1;
  const T *g, *wg, *wu;
  const float* xin;
  int H, F;
  float* aout;  // [R][F]

  __device__ void load_x(int row, int k, float (&f)[W::VE]) const { load_f32_vec<W::VE>(xin + (long)row * H + k, f); }
  __device__ void gain_vec(int k, float (&f)[W::VE]) const { W::cvt(ld16(g + k), f); }
  __device__ const T* wrow(int m) const { return ((m & 1) ? wu : wg) + (long)(m >> 1) * H; }
  template <int ROWS, int RB>
  __device__ void epilogue(int m0, const float* tile, const int (&rows)[RB], const bool (&valid)[RB], int) {
    for (int idx = threadIdx.x; idx < (ROWS / 2) * RB; idx += kWG) {
      const int qq = idx / RB, r = idx % RB;
      const int m = m0 + 2 * qq;
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
        if (rr == r && valid[rr] && m < this->N) {
          const float gt = tile[(2 * qq) * RB + r], up = tile[(2 * qq + 1) * RB + r];
          aout[(long)rows[rr] * F + (m >> 1)] = gt / (1.0f + expf(-gt)) * up;
        }
    }
  }
};

// final RMSNorm + lm_head + argmax for each sequence's last row; output hiddens; finalisation
template <class W>
struct PLmHead : PBase<W> {
  using T = typename W::T;
  static constexpr int kNorm = 1;
  const T *g, *w;
  const float* xin;
  int H;
  float* logits;  // NULL or row b at logits + b * lg_sb
  long lg_sb;
  float* part_v;  // [B][gridDim]
  int* part_i;
  float* hout;  // row (b,i) at hout + (b*hout_sb + (last ? 0 : i)) * H
  int hout_sb, hout_last;
  int32_t* draft;  // draft of b at draft[b * dr_sb]
  int dr_sb;
  int32_t* len_w;
  int* status;
  unsigned* ticket;
  float bv[8];
  int bi[8];

  __device__ void setup(int* s_n) {
    PBase<W>::setup(s_n);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      bv[r] = -INFINITY;
      bi[r] = 0x7fffffff;
    }
  }
  __device__ void act(int a, const int* s_n, int& row, bool& valid) const {
    valid = a < this->B && s_n[a] > 0;
    row = valid ? a * this->rps + s_n[a] - 1 : 0;
  }
  __device__ void load_x(int row, int k, float (&f)[W::VE]) const { load_f32_vec<W::VE>(xin + (long)row * H + k, f); }
  __device__ void gain_vec(int k, float (&f)[W::VE]) const { W::cvt(ld16(g + k), f); }
  __device__ const T* wrow(int m) const { return w + (long)m * H; }
  template <int ROWS, int RB>
  __device__ void epilogue(int m0, const float* tile, const int (&rows)[RB], const bool (&valid)[RB], int a0) {
    if (logits) {
      for (int idx = threadIdx.x; idx < ROWS * RB; idx += kWG) {
        const int q = idx / RB, r = idx % RB;
        if (a0 + r < this->B && m0 + q < this->N) logits[(long)(a0 + r) * lg_sb + m0 + q] = tile[idx];
      }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (threadIdx.x == r && valid[r]) {
        for (int q = 0; q < ROWS; ++q) {
          const int m = m0 + q;
          if (m < this->N && better(tile[q * RB + r], m, bv[r], bi[r])) {
            bv[r] = tile[q * RB + r];
            bi[r] = m;
          }
        }
      }
  }
  template <int RB>
  __device__ void act_block_done(int a0, const int (&)[RB], const bool (&)[RB]) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
      if (threadIdx.x == r) {
        if (a0 + r < this->B) {
          part_v[(long)(a0 + r) * gridDim.x + blockIdx.x] = bv[r];
          part_i[(long)(a0 + r) * gridDim.x + blockIdx.x] = bi[r];
        }
        bv[r] = -INFINITY;
        bi[r] = 0x7fffffff;
      }
  }
  __device__ void finish(const int* s_n) {
    __shared__ float red[8];
    __shared__ int s_last;
    const int tid = threadIdx.x;
    // activation blocks with no valid row were skipped: their partials must still be written
    for (int a = tid; a < this->B; a += kWG)
      if (s_n[a] == 0) {
        part_v[(long)a * gridDim.x + blockIdx.x] = -INFINITY;
        part_i[(long)a * gridDim.x + blockIdx.x] = 0x7fffffff;
      }
    // post-norm hidden of every row the caller wants, rows spread over the workgroups
    const int R = this->B * this->rps;
    for (int row = blockIdx.x; row < R; row += gridDim.x) {
      const int b = row / this->rps, i = row - b * this->rps;
      const int n = s_n[b];
      if (i >= n || (hout_last && i != n - 1)) continue;  // uniform over the workgroup
      const float* xr = xin + (long)row * H;
      float ss[1] = {0.f};
      for (int k = tid; k < H; k += kWG) ss[0] += xr[k] * xr[k];
      wg_sum<1>(ss, red);
      const float sc = 1.0f / sqrtf(ss[0] / float(H) + this->eps);
      float* dst = hout + ((long)b * hout_sb + (hout_last ? 0 : i)) * H;
      for (int k = tid; k < H; k += kWG) dst[k] = xr[k] * sc * W::get(g, k);
    }
    // last workgroup: argmax over the per-workgroup partials, drafts, lengths, status
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(ticket, 1u) == gridDim.x - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int b = tid; b < this->B; b += kWG) {
      int flags = 0;
      const int n = count_rows(this->tok + (long)b * this->tok_sb, this->rps, this->V, this->len[b], this->max_len, &flags);
      int d = -1;
      if (n > 0) {
        float v = -INFINITY;
        int id = 0x7fffffff;
        for (unsigned wg = 0; wg < gridDim.x; ++wg) {
          const float pv = part_v[(long)b * gridDim.x + wg];
          const int pi = part_i[(long)b * gridDim.x + wg];
          if (better(pv, pi, v, id)) {
            v = pv;
            id = pi;
          }
        }
        d = id;
      }
      draft[(long)b * dr_sb] = d;
      len_w[b] = this->len[b] + n;
      if (flags) atomicOr(status, flags);
    }
    if (tid == 0) *ticket = 0u;
  }
};

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

// ---------------------------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------------------------
namespace {

struct Variant {
  int rb, nxm;
};

// Register slice per thread: nxm chunks (the next power of two >= K / VE / 256) of rb activation
// rows, rb * nxm <= 16 and rb <= 8.
Variant pick_variant(int nact, int K, int VE) {
  const int Kc = K / VE;
  const int nx = (Kc + kWG - 1) / kWG;
  int nxm = 1;
  while (nxm < nx) nxm *= 2;
  int rb = 1;
  while (rb < 8 && rb * 2 <= nact && rb * 2 * nxm <= 16) rb *= 2;
  return Variant{rb, nxm};
}

int gemv_grid(int N, int rows) {
  const int groups = (N + rows - 1) / rows;
  return groups < 1024 ? groups : 1024;
}

template <class W, int ROWS, class P>
hipError_t launch_gemv(P& p, hipStream_t st) {
  const Variant v = pick_variant(p.nact, p.K, W::VE);
  if (v.nxm > 16) return hipErrorInvalidValue;
  const int grid = gemv_grid(p.N, ROWS);
#define MTP_GEMV_CASE(RB_, NX_) \
  if (v.rb == RB_ && v.nxm == NX_) { hipLaunchKernelGGL((k_gemv<W, RB_, NX_, ROWS, P>), dim3(grid), dim3(kWG), 0, st, p); return hipGetLastError(); }
  MTP_GEMV_CASE(1, 1) MTP_GEMV_CASE(2, 1) MTP_GEMV_CASE(4, 1) MTP_GEMV_CASE(8, 1)
  MTP_GEMV_CASE(1, 2) MTP_GEMV_CASE(2, 2) MTP_GEMV_CASE(4, 2) MTP_GEMV_CASE(8, 2)
  MTP_GEMV_CASE(1, 4) MTP_GEMV_CASE(2, 4) MTP_GEMV_CASE(4, 4)
  MTP_GEMV_CASE(1, 8) MTP_GEMV_CASE(2, 8)
  MTP_GEMV_CASE(1, 16)
#undef MTP_GEMV_CASE
  return hipErrorInvalidValue;
}

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
}

}  // namespace

int lm_head_grid(const mtp_config& cfg) { return gemv_grid(cfg.vocab, kLmRows); }

template <class W>
hipError_t run_step_t(const StepArgs& s) {
  using T = typename W::T;
  const mtp_config& c = s.cfg;
  const int H = c.hidden, F = c.ffn, nq = c.n_heads, nkv = c.n_kv_heads, hd = c.head_dim;
  const int R = s.B * s.rps;
  hipError_t e;

  {  // eh_proj
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
    if ((e = launch_gemv<W, 8>(p, s.stream)) != hipSuccess) return e;
  }
  for (int l = 0; l < c.n_layers; ++l) {
    const mtp_layer_weights& lw = s.w->layers[l];
    const long layer_off = (long)l * s.B * nkv * s.max_len * hd;
    {  // q/k/v + RoPE + append
      PQKV<W> p;
      fill_base<W>(p, s);
      p.K = H;
      p.N = (nq + 2 * nkv) * hd;
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
      p.kc = (T*)s.kc + layer_off;
      p.vc = (T*)s.vc + layer_off;
      if ((e = launch_gemv<W, 8>(p, s.stream)) != hipSuccess) return e;
    }
    {  // attention
      AttnArgs a;
      a.q = s.ws.q;
      a.kc = (const T*)s.kc + layer_off;
      a.vc = (const T*)s.vc + layer_off;
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
      dim3 grid(s.nsplit, nkv, s.B);
      if (hd == 128) {
        hipLaunchKernelGGL((k_attn<W, 128>), grid, dim3(kWG), 0, s.stream, a);
        const int per = kWG / 128;
        hipLaunchKernelGGL((k_attn_combine<128>), dim3((R * nq + per - 1) / per), dim3(kWG), 0, s.stream, a,
                           s.ws.attn_out);
      } else {
        hipLaunchKernelGGL((k_attn<W, 64>), grid, dim3(kWG), 0, s.stream, a);
        const int per = kWG / 64;
        hipLaunchKernelGGL((k_attn_combine<64>), dim3((R * nq + per - 1) / per), dim3(kWG), 0, s.stream, a,
                           s.ws.attn_out);
      }
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {  // o_proj + residual
      PResidual<W> p;
      fill_base<W>(p, s);
      p.K = nq * hd;
      p.N = H;
      p.nact = R;
      p.w = (const T*)lw.wo;
      p.ain = s.ws.attn_out;
      p.xres = s.ws.x;
      if ((e = launch_gemv<W, 8>(p, s.stream)) != hipSuccess) return e;
    }
    {  // gate/up + SwiGLU
      PGateUp<W> p;
      fill_base<W>(p, s);
      p.K = H;
      p.N = 2 * F;
      p.nact = R;
      p.g = (const T*)lw.post_norm;
      p.wg = (const T*)lw.wgate;
      p.wu = (const T*)lw.wup;
      p.xin = s.ws.x;
      p.H = H;
      p.F = F;
      p.aout = s.ws.act;
      if ((e = launch_gemv<W, 8>(p, s.stream)) != hipSuccess) return e;
    }
    {  // down + residual
      PResidual<W> p;
      fill_base<W>(p, s);
      p.K = F;
      p.N = H;
      p.nact = R;
      p.w = (const T*)lw.wdown;
      p.ain = s.ws.act;
      p.xres = s.ws.x;
      if ((e = launch_gemv<W, 8>(p, s.stream)) != hipSuccess) return e;
    }
  }
  {  // final norm + lm_head + argmax + finalisation
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
    p.hout = s.hout;
    p.hout_sb = s.hout_sb;
    p.hout_last = s.hout_last;
    p.draft = s.draft;
    p.dr_sb = s.dr_sb;
    p.len_w = s.kv_len;
    p.status = s.ws.status;
    p.ticket = s.ws.ticket_lm;
    if (s.ev_begin) (void)hipEventRecord(s.ev_begin, s.stream);
    e = launch_gemv<W, kLmRows>(p, s.stream);
    if (s.ev_end) (void)hipEventRecord(s.ev_end, s.stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t run_step(const StepArgs& s) {
  return s.cfg.wdtype == MTP_BF16 ? run_step_t<BF16>(s) : run_step_t<F32>(s);
}

}  // namespace mtp
