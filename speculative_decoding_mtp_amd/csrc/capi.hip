// C ABI of the MTP step: argument checks, workspace carving, kernel sequencing, timers.
// The declarations and their contracts are in include/mtp.h.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "draft.h"
#include "gemv.h"
#include "state.h"
#include "verify.h"

using namespace mtp;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MTP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

// ------------------------------------------------------------------ timers
struct Timer {
  std::vector<hipEvent_t> begin, end;
  int max = 0, count = 0;
  bool armed = false;
};
Timer g_timers[3];
const char* g_timer_name[3] = {"", "", ""};

void timer_events(int kernel, hipEvent_t* b, hipEvent_t* e) {
  *b = nullptr;
  *e = nullptr;
  Timer& t = g_timers[kernel];
  if (t.armed && t.count < t.max) {
    *b = t.begin[t.count];
    *e = t.end[t.count];
    ++t.count;
  }
}

// ------------------------------------------------------------------ config checks
int check_cfg(const mtp_config* c) {
  if (!c) return fail(MTP_ERR_ARG, "cfg is NULL");
  if (c->wdtype != MTP_F32 && c->wdtype != MTP_BF16) return fail(MTP_ERR_DTYPE, "unknown wdtype %d", c->wdtype);
  if (c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->ffn <= 0 || c->vocab <= 0 || c->n_layers <= 0)
    return fail(MTP_ERR_ARG, "config sizes must be positive");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(MTP_ERR_SHAPE, "head_dim must be 64 or 128");
  if (c->n_heads % c->n_kv_heads) return fail(MTP_ERR_SHAPE, "n_heads must be a multiple of n_kv_heads");
  if (c->hidden % 8 || c->ffn % 8) return fail(MTP_ERR_SHAPE, "hidden and ffn must be multiples of 8");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return fail(MTP_ERR_ARG, "rope_theta > 0 and rms_eps >= 0");
  const int ve = c->wdtype == MTP_BF16 ? 8 : 4;
  const int kmax = 16 * kWG * ve;
  const int ks[4] = {2 * c->hidden, c->hidden, c->n_heads * c->head_dim, c->ffn};
  for (int k : ks)
    if (k > kmax) return fail(MTP_ERR_SHAPE, "an input width of %d exceeds %d", k, kmax);
  return MTP_OK;
}

// need_kv = 0: a head reading another model's cache never reads wk / wv.
int check_layers(const mtp_config* c, const mtp_layer_weights* layers, bool need_kv = true) {
  if (!layers) return fail(MTP_ERR_ARG, "weights.layers is NULL");
  for (int l = 0; l < c->n_layers; ++l) {
    const mtp_layer_weights& L = layers[l];
    const void* lp[9] = {L.in_norm, L.wq, L.wo, L.post_norm, L.wgate, L.wup, L.wdown, L.wk, L.wv};
    for (int i = 0; i < (need_kv ? 9 : 7); ++i)
      if (!lp[i] || !aligned16(lp[i])) return fail(MTP_ERR_ARG, "layer %d: a weight pointer is NULL or misaligned", l);
  }
  return MTP_OK;
}

int check_weights(const mtp_config* c, const mtp_weights* w, bool need_kv = true) {
  if (!w) return fail(MTP_ERR_ARG, "weights is NULL");
  const void* top[6] = {w->embed, w->enorm, w->hnorm, w->eh_proj, w->final_norm, w->lm_head};
  for (const void* p : top)
    if (!p || !aligned16(p)) return fail(MTP_ERR_ARG, "a weight pointer is NULL or not 16-byte aligned");
  return check_layers(c, w->layers, need_kv);
}

int check_target_weights(const mtp_config* c, const mtp_target_weights* w) {
  if (!w) return fail(MTP_ERR_ARG, "target weights is NULL");
  const void* top[3] = {w->embed, w->final_norm, w->lm_head};
  for (const void* p : top)
    if (!p || !aligned16(p)) return fail(MTP_ERR_ARG, "a target weight pointer is NULL or not 16-byte aligned");
  return check_layers(c, w->layers);
}

int check_kv(const mtp_kv* kv) {
  if (!kv) return fail(MTP_ERR_ARG, "kv is NULL");
  if (!kv->k || !kv->v || !kv->len || !aligned16(kv->k) || !aligned16(kv->v))
    return fail(MTP_ERR_ARG, "kv pointers must be non-NULL and 16-byte aligned");
  if (kv->batch < 1 || kv->batch > kMaxBatch) return fail(MTP_ERR_ARG, "kv.batch must be in [1, %d]", kMaxBatch);
  if (kv->max_len < 8 || kv->max_len % 8) return fail(MTP_ERR_ARG, "kv.max_len must be a positive multiple of 8");
  return MTP_OK;
}

// ------------------------------------------------------------------ drafter workspace
struct DraftLayout {
  size_t off[17];
  size_t total;
  int nsplit;  // attention splits the partial buffer is laid out for
};

DraftLayout draft_layout(const mtp_config& c, int B, int rps, int D, int max_len) {
  const size_t R = (size_t)B * (rps < 1 ? 1 : rps);
  const int nsplit = attn_nsplit(B, c.n_kv_heads, max_len, (rps < 1 ? 1 : rps) * (c.n_heads / c.n_kv_heads));
  const size_t G = c.n_heads / c.n_kv_heads;
  size_t kmax = 2 * (size_t)c.hidden;
  if ((size_t)c.ffn > kmax) kmax = c.ffn;
  if ((size_t)c.n_heads * c.head_dim > kmax) kmax = (size_t)c.n_heads * c.head_dim;
  const bool mfma = c.wdtype == MTP_BF16 && R >= 3;  // more rows than one VALU GEMV pass may hold
  const size_t sizes[17] = {
      256 + (size_t)B * 8,                                                   // status word, row counts
      R * c.hidden * 4,                                                      // x
      R * c.n_heads * c.head_dim * 4,                                        // q
      (size_t)B * c.n_kv_heads * nsplit * (rps * G) * (c.head_dim + 2) * 4, // attention partials
      R * c.n_heads * c.head_dim * 4,                                        // attention output
      R * c.ffn * 4,                                                         // act
      (size_t)B * kMaxGemvGrid * 4,                                          // lm partial values
      (size_t)B * kMaxGemvGrid * 4,                                          // lm partial ids
      (size_t)B * (D < 1 ? 1 : D) * c.hidden * 4,                            // step hiddens
      mfma ? R * kmax * 2 : 0,                                               // split activations, hi
      mfma ? R * kmax * 2 : 0,                                               // split activations, lo
      mfma ? R * 4 : 0,                                                      // compact row map
      mfma ? R * 4 : 0,                                                      // compact activation map
      mfma ? (size_t)4 : (size_t)0,                                          // compact count
      mfma ? R * c.ffn * 2 : 0,                                              // SwiGLU output split, hi
      mfma ? R * c.ffn * 2 : 0,                                              // SwiGLU output split, lo
      mfma ? R * kPartCols * 4 : 0};                                         // split-K partials (last)
  DraftLayout L;
  size_t o = 0;
  for (int i = 0; i < 17; ++i) {
    L.off[i] = o;
    o += up256(sizes[i]);
  }
  L.total = o;
  L.nsplit = nsplit;
  return L;
}

DraftWs carve(void* ws, const DraftLayout& L) {
  char* base = static_cast<char*>(ws);
  DraftWs w;
  w.status = reinterpret_cast<int*>(base);
  w.rows = reinterpret_cast<int*>(base + 256);
  w.x = reinterpret_cast<float*>(base + L.off[1]);
  w.q = reinterpret_cast<float*>(base + L.off[2]);
  w.attn_part = reinterpret_cast<float*>(base + L.off[3]);
  w.attn_out = reinterpret_cast<float*>(base + L.off[4]);
  w.act = reinterpret_cast<float*>(base + L.off[5]);
  w.lm_part_v = reinterpret_cast<float*>(base + L.off[6]);
  w.lm_part_i = reinterpret_cast<int*>(base + L.off[7]);
  w.hid_fb = reinterpret_cast<float*>(base + L.off[8]);
  const bool mfma = L.off[10] > L.off[9];
  w.xhi = mfma ? reinterpret_cast<uint16_t*>(base + L.off[9]) : nullptr;
  w.xlo = mfma ? reinterpret_cast<uint16_t*>(base + L.off[10]) : nullptr;
  w.rowmap = mfma ? reinterpret_cast<int*>(base + L.off[11]) : nullptr;
  w.amap = mfma ? reinterpret_cast<int*>(base + L.off[12]) : nullptr;
  w.mcount = mfma ? reinterpret_cast<int*>(base + L.off[13]) : nullptr;
  w.shi = mfma ? reinterpret_cast<uint16_t*>(base + L.off[14]) : nullptr;
  w.slo = mfma ? reinterpret_cast<uint16_t*>(base + L.off[15]) : nullptr;
  w.kpart = mfma ? reinterpret_cast<float*>(base + L.off[16]) : nullptr;
  w.kpart_cap = mfma ? (long)((L.total - L.off[16]) / 4) : 0;
  return w;
}

int draft_common(const mtp_config* cfg, const mtp_weights* w, const mtp_kv* kv, int rps, int D, const int32_t* tokens,
                 const float* hidden_in, void* ws, size_t ws_bytes, DraftLayout* L) {
  int rc;
  if ((rc = check_cfg(cfg)) || (rc = check_weights(cfg, w)) || (rc = check_kv(kv))) return rc;
  if (rps < 1) return fail(MTP_ERR_ARG, "rows_per_seq must be >= 1");
  if (!tokens || !hidden_in || !aligned16(hidden_in)) return fail(MTP_ERR_ARG, "tokens / hidden_in NULL or misaligned");
  if (!ws || !aligned16(ws)) return fail(MTP_ERR_ARG, "workspace NULL or misaligned");
  *L = draft_layout(*cfg, kv->batch, rps, D, kv->max_len);
  if (ws_bytes < L->total)
    return fail(MTP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, L->total);
  return MTP_OK;
}

StepArgs base_step(const mtp_config* cfg, const mtp_weights* w, const mtp_kv* kv, void* ws, const DraftLayout& L,
                   hipStream_t st) {
  StepArgs s;
  s.cfg = *cfg;
  s.w = w;
  s.tw = nullptr;
  s.target = 0;
  s.kc = kv->k;
  s.vc = kv->v;
  s.kv_len = kv->len;
  s.B = kv->batch;
  s.max_len = kv->max_len;
  s.nsplit = L.nsplit;
  s.ws = carve(ws, L);
  s.stream = st;
  s.logits = nullptr;
  s.lg_sb = 0;
  s.ev_begin = s.ev_end = nullptr;
  s.ev_name = &g_timer_name[MTP_KERNEL_LM_HEAD];
  s.shared = 0;
  s.pos_off = 0;
  s.kv_layer = nullptr;
  s.no_head = 0;
  return s;
}

// Checks spec_verify's arguments and lays its scratch out from `base` (a workspace, or the
// library's own array): the greedy chunk argmax partials, or the sampling top-k buffers.  *used
// is the number of bytes this call needs from base (exact, unlike the workspace-size bound).
int verify_setup(int32_t B, int32_t D, int32_t V, const float* target_logits, const int32_t* drafts,
                 const float* draft_logits, const mtp_sampling* sp, const float* u_accept, const float* u_sample,
                 const int32_t* ctx_len, int32_t* n_accept, int32_t* out_tokens, int32_t* crop_len, char* base,
                 VerifyArgs* out, size_t* used) {
  if (B < 1 || D < 1 || V < 1) return fail(MTP_ERR_ARG, "B, D, V must be positive");
  if (D > kMaxDraft) return fail(MTP_ERR_ARG, "D must be <= %d", kMaxDraft);
  if (!target_logits || !drafts || !ctx_len || !n_accept || !out_tokens || !crop_len)
    return fail(MTP_ERR_ARG, "a required pointer is NULL");
  if (!aligned16(target_logits)) return fail(MTP_ERR_ARG, "target_logits misaligned");
  VerifyArgs a = {};
  a.B = B;
  a.D = D;
  a.V = V;
  a.greedy = !sp || !(sp->temperature > 0.f);
  a.tl = target_logits;
  a.drafts = drafts;
  a.ctx_len = ctx_len;
  a.n_accept = n_accept;
  a.out = out_tokens;
  a.crop = crop_len;
  size_t o = 256;
  const int rows = B * (D + 1) + (!a.greedy && sp->q_mode == 1 ? B * D : 0);
  if (a.greedy) {
    // Early exit: when the logits run to hundreds of MB the scan is bound by bytes, and each
    // workgroup walks its chunk of a sequence's rows in order, stopping where the sequence must
    // (about 1024 workgroups over the sequences); below that, latency decides, and every row is
    // scanned at once (about 1024 workgroups over the rows).  Chunks of at least 1024 logits, at
    // most 1024 chunks.
    a.walk = (double)rows * V * 4.0 >= 256.0 * 1024 * 1024;
    const int over = a.walk ? B : rows;
    int target = (1024 + over - 1) / over;
    if (target > 1024) target = 1024;
    int chunk = (V + target - 1) / target;
    chunk = (chunk + 1023) & ~1023;
    a.chunk = chunk;
    a.nchunk = (V + chunk - 1) / chunk;
    a.part_v = reinterpret_cast<float*>(base + o);
    o += up256((size_t)rows * a.nchunk * 4);
    a.part_i = reinterpret_cast<int*>(base + o);
    o += up256((size_t)rows * a.nchunk * 4);
  } else {
    if (sp->q_mode != 0 && sp->q_mode != 1) return fail(MTP_ERR_ARG, "q_mode must be 0 or 1");
    if (sp->q_mode == 1 && (!draft_logits || !aligned16(draft_logits)))
      return fail(MTP_ERR_ARG, "q_mode 1 needs draft_logits");
    if (!u_accept || !u_sample) return fail(MTP_ERR_ARG, "sampling needs u_accept and u_sample");
    const int K = sp->top_k;
    a.q_mode = sp->q_mode;
    a.top_k = K;
    a.temperature = sp->temperature;
    a.top_p = sp->top_p;
    a.dl = draft_logits;
    a.u_accept = u_accept;
    a.u_sample = u_sample;
    a.full = K < 1 || K > kMaxTopK;
    if (a.full) {  // top-k off, or more than the candidate buffer holds: the whole vocabulary
      a.rowinfo = reinterpret_cast<FullRow*>(base + o);
      o += up256((size_t)rows * sizeof(FullRow));
      *out = a;
      *used = o;
      return MTP_OK;
    }
    a.top_v = reinterpret_cast<float*>(base + o);
    o += up256((size_t)rows * K * 4);
    a.top_i = reinterpret_cast<int*>(base + o);
    o += up256((size_t)rows * K * 4);
    a.top_n = reinterpret_cast<int*>(base + o);
    o += up256((size_t)rows * 4);
    topk_split(rows, V, &a.tk_nchunk, &a.tk_chunk);
    a.cand_v = nullptr;
    a.cand_i = nullptr;
    if (a.tk_nchunk > 1) {
      a.cand_v = reinterpret_cast<float*>(base + o);
      o += up256((size_t)rows * a.tk_nchunk * K * 4);
      a.cand_i = reinterpret_cast<int*>(base + o);
      o += up256((size_t)rows * a.tk_nchunk * K * 4);
    }
  }
  *out = a;
  *used = o;
  return MTP_OK;
}

int verify_launch(const VerifyArgs& a, hipStream_t stream) {
  hipEvent_t eb, ee;
  timer_events(MTP_KERNEL_VERIFY, &eb, &ee);
  if (eb) {
    (void)hipEventRecord(eb, stream);
    g_timer_name[MTP_KERNEL_VERIFY] = a.greedy ? "spec_verify (greedy: chunk argmax + prefix match)"
                                               : "spec_verify (top-k scan, merge, decide)";
  }
  const hipError_t e = run_verify(a, stream);
  if (ee) (void)hipEventRecord(ee, stream);
  return e == hipSuccess ? MTP_OK : hip_fail(e, "spec_verify launch");
}

// ------------------------------------------------------------------ scratch of spec_verify_noalloc
// A file-scope device array, one copy per GPU for the life of the process.  Host code must not use
// the symbol's name as a device address: its address on each device comes from
// hipGetSymbolAddress, taken once per device (with that device current) and kept here.
__device__ __align__(256) char scratch[MTP_VERIFY_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(char** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MTP_ERR_ARG, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e == hipSuccess ? hipErrorInvalidSymbol : e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *ptr = static_cast<char*>(g_scratch_ptr[dev]);
  return MTP_OK;
}

}  // namespace

namespace mtp {
int attn_nsplit(int B, int nkv, int max_len, int qrows) {
  // about one workgroup per compute unit: a single decode row per sequence then gets chunks of
  // 128+ positions (every wave of a workgroup has a 32-position slice; two splits per unit left
  // half the waves idle), and a batch of 32 sequences x 8 kv heads runs unsplit, with no
  // combine launch
  int n = (256 + B * nkv - 1) / (B * nkv);
  if (n > kMaxSplit) n = kMaxSplit;
  // many queries per kv head (a long prefill): bound the partials to 8192 query rows per head
  const int qcap = 8192 / (qrows < 1 ? 1 : qrows);
  if (n > qcap) n = qcap;
  const int cap = (max_len + 63) / 64;
  if (n > cap) n = cap;
  return n < 1 ? 1 : n;
}
}  // namespace mtp

extern "C" {

const char* mtp_last_error(void) { return g_err.c_str(); }

int mtp_draft_workspace_size(const mtp_config* cfg, int32_t batch, int32_t rows_per_seq, int32_t D, int32_t max_len,
                             size_t* bytes) {
  int rc;
  if ((rc = check_cfg(cfg))) return rc;
  if (!bytes) return fail(MTP_ERR_ARG, "bytes is NULL");
  if (batch < 1 || batch > kMaxBatch || rows_per_seq < 1 || max_len < 1 || D < 0)
    return fail(MTP_ERR_ARG, "batch in [1, %d], rows_per_seq >= 1, max_len >= 1, D >= 0", kMaxBatch);
  *bytes = draft_layout(*cfg, batch, rows_per_seq, D, max_len).total;
  return MTP_OK;
}

int mtp_target_workspace_size(const mtp_config* cfg, int32_t batch, int32_t rows_per_seq, int32_t max_len,
                              size_t* bytes) {
  return mtp_draft_workspace_size(cfg, batch, rows_per_seq, 1, max_len, bytes);
}

int mtp_target_forward(const mtp_config* cfg, const mtp_target_weights* w, const mtp_kv* kv, int32_t rows_per_seq,
                       const int32_t* tokens, float* hidden_out, float* logits_out, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  int rc;
  if ((rc = check_cfg(cfg)) || (rc = check_target_weights(cfg, w)) || (rc = check_kv(kv))) return rc;
  if (rows_per_seq < 1) return fail(MTP_ERR_ARG, "rows_per_seq must be >= 1");
  if (!tokens) return fail(MTP_ERR_ARG, "tokens is NULL");
  if (!logits_out || !aligned16(logits_out)) return fail(MTP_ERR_ARG, "logits_out NULL or misaligned");
  if (hidden_out && !aligned16(hidden_out)) return fail(MTP_ERR_ARG, "hidden_out misaligned");
  if (!ws || !aligned16(ws)) return fail(MTP_ERR_ARG, "workspace NULL or misaligned");
  const DraftLayout L = draft_layout(*cfg, kv->batch, rows_per_seq, 1, kv->max_len);
  if (ws_bytes < L.total) return fail(MTP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, L.total);
  StepArgs s = base_step(cfg, nullptr, kv, ws, L, stream);
  s.tw = w;
  s.target = 1;
  s.rps = rows_per_seq;
  s.tok = tokens;
  s.tok_sb = rows_per_seq;
  s.hin = nullptr;
  s.hin_sb = 0;
  s.hout = hidden_out;
  s.hout_sb = rows_per_seq;
  s.hout_last = 0;
  s.draft = nullptr;
  s.dr_sb = 0;
  s.logits = logits_out;
  s.lg_sb = cfg->vocab;
  const hipError_t e = run_step(s);
  return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_target_forward launch");
}

int mtp_draft_step(const mtp_config* cfg, const mtp_weights* w, const mtp_kv* kv, int32_t rows_per_seq,
                   const int32_t* tokens, const float* hidden_in, float* hidden_out, int32_t* draft_out,
                   float* logits_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  DraftLayout L;
  int rc = draft_common(cfg, w, kv, rows_per_seq, 0, tokens, hidden_in, ws, ws_bytes, &L);
  if (rc) return rc;
  if (!hidden_out || !draft_out || !aligned16(hidden_out)) return fail(MTP_ERR_ARG, "hidden_out / draft_out");
  if (hidden_out == hidden_in) return fail(MTP_ERR_ARG, "hidden_out may not alias hidden_in");
  if (logits_out && !aligned16(logits_out)) return fail(MTP_ERR_ARG, "logits_out misaligned");
  StepArgs s = base_step(cfg, w, kv, ws, L, stream);
  s.rps = rows_per_seq;
  s.tok = tokens;
  s.tok_sb = rows_per_seq;
  s.hin = hidden_in;
  s.hin_sb = rows_per_seq;
  s.hout = hidden_out;
  s.hout_sb = rows_per_seq;
  s.hout_last = 0;
  s.draft = draft_out;
  s.dr_sb = 1;
  s.logits = logits_out;
  s.lg_sb = cfg->vocab;
  timer_events(MTP_KERNEL_LM_HEAD, &s.ev_begin, &s.ev_end);
  const hipError_t e = run_step(s);
  return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_draft_step launch");
}

int mtp_draft_loop(const mtp_config* cfg, const mtp_weights* w, const mtp_kv* kv, int32_t D, int32_t rows_per_seq,
                   const int32_t* tokens, const float* hidden_in, int32_t* drafts, float* hiddens,
                   float* draft_logits, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (D < 1) return fail(MTP_ERR_ARG, "D must be >= 1");
  DraftLayout L;
  int rc = draft_common(cfg, w, kv, rows_per_seq, D, tokens, hidden_in, ws, ws_bytes, &L);
  if (rc) return rc;
  if (!drafts) return fail(MTP_ERR_ARG, "drafts is NULL");
  if ((hiddens && !aligned16(hiddens)) || (draft_logits && !aligned16(draft_logits)))
    return fail(MTP_ERR_ARG, "hiddens / draft_logits misaligned");
  StepArgs s = base_step(cfg, w, kv, ws, L, stream);
  const int H = cfg->hidden;
  float* hbuf = hiddens ? hiddens : s.ws.hid_fb;
  for (int k = 0; k < D; ++k) {
    if (k == 0) {
      s.rps = rows_per_seq;
      s.tok = tokens;
      s.tok_sb = rows_per_seq;
      s.hin = hidden_in;
      s.hin_sb = rows_per_seq;
    } else {
      s.rps = 1;
      s.tok = drafts + (k - 1);
      s.tok_sb = D;
      s.hin = hbuf + (long)(k - 1) * H;
      s.hin_sb = D;
    }
    s.hout = hbuf + (long)k * H;
    s.hout_sb = D;
    s.hout_last = 1;
    s.draft = drafts + k;
    s.dr_sb = D;
    s.logits = draft_logits ? draft_logits + (long)k * cfg->vocab : nullptr;
    s.lg_sb = (long)D * cfg->vocab;
    timer_events(MTP_KERNEL_LM_HEAD, &s.ev_begin, &s.ev_end);
    const hipError_t e = run_step(s);
    if (e != hipSuccess) return hip_fail(e, "mtp_draft_loop launch");
  }
  return MTP_OK;
}

int mtp_draft_loop_shared_kv(const mtp_config* cfg, const mtp_weights* w, const mtp_kv* target_kv,
                             int32_t target_layers, const int32_t* kv_layer, int32_t D, const int32_t* tokens,
                             const float* hidden_in, int32_t* drafts, float* hiddens, float* draft_logits, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  int rc;
  if ((rc = check_cfg(cfg)) || (rc = check_weights(cfg, w, false)) || (rc = check_kv(target_kv))) return rc;
  if (D < 1) return fail(MTP_ERR_ARG, "D must be >= 1");
  if (target_layers < 1) return fail(MTP_ERR_ARG, "target_layers must be >= 1");
  if (!kv_layer) return fail(MTP_ERR_ARG, "kv_layer is NULL");
  for (int l = 0; l < cfg->n_layers; ++l)
    if (kv_layer[l] < 0 || kv_layer[l] >= target_layers)
      return fail(MTP_ERR_ARG, "kv_layer[%d] = %d outside [0, %d)", l, kv_layer[l], target_layers);
  if (!tokens || !hidden_in || !aligned16(hidden_in)) return fail(MTP_ERR_ARG, "tokens / hidden_in NULL or misaligned");
  if (!drafts) return fail(MTP_ERR_ARG, "drafts is NULL");
  if ((hiddens && !aligned16(hiddens)) || (draft_logits && !aligned16(draft_logits)))
    return fail(MTP_ERR_ARG, "hiddens / draft_logits misaligned");
  if (!ws || !aligned16(ws)) return fail(MTP_ERR_ARG, "workspace NULL or misaligned");
  const DraftLayout L = draft_layout(*cfg, target_kv->batch, 1, D, target_kv->max_len);
  if (ws_bytes < L.total) return fail(MTP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, L.total);
  StepArgs s = base_step(cfg, w, target_kv, ws, L, stream);
  s.shared = 1;
  s.kv_layer = kv_layer;
  s.rps = 1;
  const int H = cfg->hidden;
  float* hbuf = hiddens ? hiddens : s.ws.hid_fb;
  for (int k = 0; k < D; ++k) {
    s.pos_off = k - 1;  // step k + 1 sits at len[b] - 1 + k
    s.tok = k == 0 ? tokens : drafts + (k - 1);
    s.tok_sb = k == 0 ? 1 : D;
    s.hin = k == 0 ? hidden_in : hbuf + (long)(k - 1) * H;
    s.hin_sb = k == 0 ? 1 : D;
    s.hout = hbuf + (long)k * H;
    s.hout_sb = D;
    s.hout_last = 1;
    s.draft = drafts + k;
    s.dr_sb = D;
    s.logits = draft_logits ? draft_logits + (long)k * cfg->vocab : nullptr;
    s.lg_sb = (long)D * cfg->vocab;
    timer_events(MTP_KERNEL_LM_HEAD, &s.ev_begin, &s.ev_end);
    const hipError_t e = run_step(s);
    if (e != hipSuccess) return hip_fail(e, "mtp_draft_loop_shared_kv launch");
  }
  return MTP_OK;
}

int mtp_draft_loop_multi(const mtp_config* cfg, const mtp_weights* modules, int32_t M, const mtp_kv* kvs, int32_t D,
                         int32_t rows_per_seq, const int32_t* tokens, const float* hidden_in, int32_t* drafts,
                         float* hiddens, float* draft_logits, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M < 1 || !modules || !kvs) return fail(MTP_ERR_ARG, "M >= 1 modules and caches needed");
  if (D < 1) return fail(MTP_ERR_ARG, "D must be >= 1");
  int rc;
  if ((rc = check_cfg(cfg))) return rc;
  for (int m = 0; m < M; ++m) {
    if ((rc = check_weights(cfg, &modules[m])) || (rc = check_kv(&kvs[m]))) return rc;
    if (kvs[m].batch != kvs[0].batch || kvs[m].max_len != kvs[0].max_len)
      return fail(MTP_ERR_ARG, "every module's cache needs the same batch and max_len");
  }
  if (rows_per_seq < 1) return fail(MTP_ERR_ARG, "rows_per_seq must be >= 1");
  if (!tokens || !hidden_in || !aligned16(hidden_in)) return fail(MTP_ERR_ARG, "tokens / hidden_in NULL or misaligned");
  if (!drafts) return fail(MTP_ERR_ARG, "drafts is NULL");
  if ((hiddens && !aligned16(hiddens)) || (draft_logits && !aligned16(draft_logits)))
    return fail(MTP_ERR_ARG, "hiddens / draft_logits misaligned");
  if (!ws || !aligned16(ws)) return fail(MTP_ERR_ARG, "workspace NULL or misaligned");
  const int rmax = M > 1 && D - 1 > rows_per_seq ? D - 1 : rows_per_seq;
  const DraftLayout L = draft_layout(*cfg, kvs[0].batch, rmax, D, kvs[0].max_len);
  if (ws_bytes < L.total) return fail(MTP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, L.total);
  const int H = cfg->hidden;
  float* hbuf = hiddens ? hiddens : carve(ws, L).hid_fb;
  std::vector<int> seen(M, 1);  // chain steps whose rows each module's cache holds
  for (int m = 0; m < M; ++m) {  // catch-up: every module appends the settled rows
    StepArgs s = base_step(cfg, &modules[m], &kvs[m], ws, L, stream);
    s.rps = rows_per_seq;
    s.tok = tokens;
    s.tok_sb = rows_per_seq;
    s.hin = hidden_in;
    s.hin_sb = rows_per_seq;
    s.no_head = m > 0;
    s.hout = hbuf;
    s.hout_sb = D;
    s.hout_last = 1;
    s.draft = drafts;
    s.dr_sb = D;
    s.logits = draft_logits;
    s.lg_sb = (long)D * cfg->vocab;
    if (m == 0) timer_events(MTP_KERNEL_LM_HEAD, &s.ev_begin, &s.ev_end);
    const hipError_t e = run_step(s);
    if (e != hipSuccess) return hip_fail(e, "mtp_draft_loop_multi launch");
  }
  for (int k = 2; k <= D; ++k) {  // step k: module (k-1) mod M over the chain rows it has not seen
    const int m = (k - 1) % M, lo = seen[m];
    StepArgs s = base_step(cfg, &modules[m], &kvs[m], ws, L, stream);
    s.rps = k - lo;
    s.tok = drafts + (lo - 1);
    s.tok_sb = D;
    s.hin = hbuf + (long)(lo - 1) * H;
    s.hin_sb = D;
    s.hout = hbuf + (long)(k - 1) * H;
    s.hout_sb = D;
    s.hout_last = 1;
    s.draft = drafts + (k - 1);
    s.dr_sb = D;
    s.logits = draft_logits ? draft_logits + (long)(k - 1) * cfg->vocab : nullptr;
    s.lg_sb = (long)D * cfg->vocab;
    timer_events(MTP_KERNEL_LM_HEAD, &s.ev_begin, &s.ev_end);
    const hipError_t e = run_step(s);
    if (e != hipSuccess) return hip_fail(e, "mtp_draft_loop_multi launch");
    seen[m] = k;
  }
  return MTP_OK;
}

int spec_verify_workspace_size(int32_t B, int32_t D, int32_t V, const mtp_sampling* sp, size_t* bytes) {
  if (!bytes) return fail(MTP_ERR_ARG, "bytes is NULL");
  if (B < 1 || D < 1 || V < 1) return fail(MTP_ERR_ARG, "B, D, V must be positive");
  const bool greedy = !sp || !(sp->temperature > 0.f);
  const size_t rows = (size_t)B * (D + 1) + (size_t)(!greedy && sp->q_mode == 1 ? B * D : 0);
  if (D > kMaxDraft) return fail(MTP_ERR_ARG, "D must be <= %d", kMaxDraft);
  size_t t = 256;
  if (greedy) {
    const size_t nchunk = 1024;  // upper bound of the chunk count chosen at launch
    t += 2 * up256(rows * nchunk * 4);
  } else if (sp->top_k < 1 || sp->top_k > kMaxTopK) {  // the whole vocabulary
    t += up256(rows * sizeof(FullRow));
  } else {
    const int K = sp->top_k;
    t += 2 * up256(rows * K * 4) + up256(rows * 4);
    int nch = 1, chunk = V;
    topk_split((int)rows, V, &nch, &chunk);
    if (nch > 1) t += 2 * up256(rows * nch * K * 4);  // per-chunk candidates
  }
  *bytes = t;
  return MTP_OK;
}

int spec_verify(int32_t B, int32_t D, int32_t V, const float* target_logits, const int32_t* drafts,
                const float* draft_logits, const mtp_sampling* sp, const float* u_accept, const float* u_sample,
                const int32_t* ctx_len, int32_t* n_accept, int32_t* out_tokens, int32_t* crop_len, void* ws,
                size_t ws_bytes, hipStream_t stream) {
  size_t need;
  int rc = spec_verify_workspace_size(B, D, V, sp, &need);
  if (rc) return rc;
  if (!ws || !aligned16(ws)) return fail(MTP_ERR_ARG, "workspace NULL or misaligned");
  if (ws_bytes < need) return fail(MTP_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, need);
  VerifyArgs a;
  size_t used;
  if ((rc = verify_setup(B, D, V, target_logits, drafts, draft_logits, sp, u_accept, u_sample, ctx_len, n_accept,
                         out_tokens, crop_len, static_cast<char*>(ws), &a, &used)))
    return rc;
  return verify_launch(a, stream);
}

int spec_verify_noalloc(int32_t B, int32_t D, int32_t V, const float* target_logits, const int32_t* drafts,
                        const float* draft_logits, const mtp_sampling* sp, const float* u_accept,
                        const float* u_sample, const int32_t* ctx_len, int32_t* n_accept, int32_t* out_tokens,
                        int32_t* crop_len, hipStream_t stream) {
  char* base = nullptr;
  int rc = scratch_for_current_device(&base);
  if (rc) return rc;
  VerifyArgs a;
  size_t used;
  if ((rc = verify_setup(B, D, V, target_logits, drafts, draft_logits, sp, u_accept, u_sample, ctx_len, n_accept,
                         out_tokens, crop_len, base, &a, &used)))
    return rc;
  if (used > MTP_VERIFY_SCRATCH_BYTES)
    return fail(MTP_ERR_WORKSPACE, "this call needs %zu bytes of scratch; the library's array holds %u", used,
                (unsigned)MTP_VERIFY_SCRATCH_BYTES);
  return verify_launch(a, stream);
}

int kv_crop(const mtp_kv* kv, const int32_t* new_len, hipStream_t stream) {
  if (!kv || !kv->len || !new_len) return fail(MTP_ERR_ARG, "kv / kv.len / new_len is NULL");
  if (kv->batch < 1) return fail(MTP_ERR_ARG, "kv.batch must be positive");
  const hipError_t e = run_kv_crop(kv->len, new_len, kv->batch, stream);
  return e == hipSuccess ? MTP_OK : hip_fail(e, "kv_crop launch");
}

int mtp_state_snapshot(const void* state, void* snap, size_t bytes_per_seq, int32_t B, hipStream_t stream) {
  if (!state || !snap || !aligned16(state) || !aligned16(snap)) return fail(MTP_ERR_ARG, "state / snap");
  if (B < 1 || bytes_per_seq == 0 || bytes_per_seq % 16) return fail(MTP_ERR_ARG, "B >= 1, bytes_per_seq % 16 == 0");
  const hipError_t e = run_copy_states(snap, state, bytes_per_seq, B, nullptr, 0, stream);
  return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_state_snapshot launch");
}

int mtp_state_restore(void* state, const void* snap, size_t bytes_per_seq, int32_t B, const int32_t* n_accept,
                      int32_t D, hipStream_t stream) {
  if (!state || !snap || !n_accept || !aligned16(state) || !aligned16(snap))
    return fail(MTP_ERR_ARG, "state / snap / n_accept");
  if (B < 1 || bytes_per_seq == 0 || bytes_per_seq % 16) return fail(MTP_ERR_ARG, "B >= 1, bytes_per_seq % 16 == 0");
  const hipError_t e = run_copy_states(state, snap, bytes_per_seq, B, n_accept, D, stream);
  return e == hipSuccess ? MTP_OK : hip_fail(e, "mtp_state_restore launch");
}

int mtp_check(void* ws, hipStream_t stream) {
  if (!ws) return fail(MTP_ERR_ARG, "ws is NULL");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  int flags = 0;
  e = hipMemcpy(&flags, ws, sizeof(int), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  if (!flags) return MTP_OK;
  const int zero = 0;
  e = hipMemcpy(ws, &zero, sizeof(int), hipMemcpyHostToDevice);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
  if (flags & kFlagCapacity) return fail(MTP_ERR_CAPACITY, "KV cache capacity exceeded; rows were skipped");
  return fail(MTP_ERR_TOKEN, "token id outside the vocabulary; rows were skipped");
}

int mtp_timer_start(int32_t kernel, int32_t max_launches) {
  if (kernel != MTP_KERNEL_LM_HEAD && kernel != MTP_KERNEL_VERIFY) return fail(MTP_ERR_ARG, "unknown kernel id");
  if (max_launches < 1) return fail(MTP_ERR_ARG, "max_launches must be positive");
  Timer& t = g_timers[kernel];
  while ((int)t.begin.size() < max_launches) {
    hipEvent_t a, b;
    hipError_t e = hipEventCreate(&a);
    if (e == hipSuccess) e = hipEventCreate(&b);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreate");
    t.begin.push_back(a);
    t.end.push_back(b);
  }
  t.max = max_launches;
  t.count = 0;
  t.armed = true;
  return MTP_OK;
}

const char* mtp_timer_kernel_name(int32_t kernel) {
  if (kernel != MTP_KERNEL_LM_HEAD && kernel != MTP_KERNEL_VERIFY) return "";
  return g_timer_name[kernel];
}

int mtp_timer_read(int32_t kernel, float* total_ms, int32_t* launches) {
  if (kernel != MTP_KERNEL_LM_HEAD && kernel != MTP_KERNEL_VERIFY) return fail(MTP_ERR_ARG, "unknown kernel id");
  if (!total_ms || !launches) return fail(MTP_ERR_ARG, "NULL output");
  Timer& t = g_timers[kernel];
  t.armed = false;
  float sum = 0.f;
  for (int i = 0; i < t.count; ++i) {
    hipError_t e = hipEventSynchronize(t.end[i]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, t.begin[i], t.end[i]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    sum += ms;
  }
  *total_ms = sum;
  *launches = t.count;
  return MTP_OK;
}

}  // extern "C"
