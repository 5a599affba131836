"""Plain float64 CPU oracle of the MTP draft head, the verifier and crop/rollback.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.  Everything runs one row of one sequence at a time, in
float64, in the order the pages give; matrix-vector products use NumPy.

Citation keys: [HB14] handbook chapter 14 "MTP: speculative decoding with the
built-in draft head"; [DLM] "The decoding loop and MTP"; [YL] "MTP
(Multi-Token Prediction) 原理详解".  Where the pages leave a step open the
reading taken is stated in the function's docstring.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

F64 = np.float64

__all__ = [
    "rms_norm", "rope", "round_kv", "silu", "attend", "argmax_lowest",
    "OracleModel", "KVCache", "decoder_block", "mtp_row", "draft_step", "draft_loop",
    "greedy_verify", "warp", "sample", "residual", "sampling_verify", "spec_verify",
    "kv_crop", "state_snapshot", "state_restore", "spec_decode", "VerifyResult",
    "TargetModel", "target_row", "target_forward", "DenseTarget",
    "shared_block", "mtp_row_shared", "draft_loop_shared", "draft_loop_multi",
]


# --------------------------------------------------------------------------------------------
# O1  RMSNorm
# --------------------------------------------------------------------------------------------
def rms_norm(x, gain, eps: float) -> np.ndarray:
    """RMSNorm of one vector: x / sqrt(mean(x^2) + eps), times the gain.

    [HB14 "The draft head"]: the head normalises the next-token embedding and
    the main model's hidden with one RMSNorm each before the projection, and
    normalises its output with a third one; the main model's hidden is itself
    taken after the main model's final RMSNorm."""
    x = np.asarray(x, dtype=F64)
    return x / np.sqrt(np.mean(x * x) + eps) * np.asarray(gain, dtype=F64)


# --------------------------------------------------------------------------------------------
# O2  rotary position embedding
# --------------------------------------------------------------------------------------------
def rope(x, pos: int, theta: float) -> np.ndarray:
    """Rotate one head vector (last axis = head_dim) to position ``pos``.

    [HB14 "The draft head"] builds cos/sin tables for the positions of the rows
    and hands them to the decoder layer; the layer's internals are not listed.
    Reading: the rotate-half form over the whole head dim, frequency of pair i
    equal to theta^(-2i/hd); pair i couples element i with element i + hd/2."""
    x = np.asarray(x, dtype=F64)
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=F64)
    ang = float(pos) * np.power(float(theta), -2.0 * i / hd)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def round_kv(x, kvdtype: str) -> np.ndarray:
    """Round values to the KV-cache storage type, round to nearest, ties to even.

    The pages keep K and V in the model's dtype; reading: the cache stores the
    weight dtype, so fp32 for fp32 heads and bf16 (8 significant bits) for bf16
    heads."""
    x = np.asarray(x, dtype=F64)
    if kvdtype == "f32":
        return x.astype(np.float32).astype(F64)
    m, e = np.frexp(x)                      # x = m * 2^e with 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)   # rint: half to even


def silu(z) -> np.ndarray:
    """SiLU(z) = z / (1 + exp(-z)), the gate of the SwiGLU feed-forward."""
    z = np.asarray(z, dtype=F64)
    return z / (1.0 + np.exp(-z))


def attend(q, K, V) -> np.ndarray:
    """Softmax attention of one query over the cached keys and values.

    q: [hd]; K, V: [T][hd] (every cached position the query may see).  Scores
    are q.k / sqrt(hd); the result is the softmax-weighted sum of V rows."""
    q = np.asarray(q, dtype=F64)
    K = np.asarray(K, dtype=F64)
    V = np.asarray(V, dtype=F64)
    s = (K @ q) / np.sqrt(q.shape[-1])
    p = np.exp(s - s.max())
    p = p / p.sum()
    return p @ V


def argmax_lowest(logits):
    """Greedy choice: the largest logit, the lowest id among equal values.

    [DLM "Why a hand-written decoding loop"]: of two equally likely tokens the
    greedy pick is the lower id.  Also returns the decision margin: the gap
    between the chosen value and the best of the others (0 on a tie)."""
    l = np.asarray(logits)
    i = int(np.argmax(l))                   # first occurrence of the maximum = lowest id
    if l.shape[-1] == 1:
        return i, float("inf")
    best = l[i]
    other = np.max(np.concatenate([l[:i], l[i + 1:]]))
    return i, float(F64(best) - F64(other))


# --------------------------------------------------------------------------------------------
# model and cache containers
# --------------------------------------------------------------------------------------------
class OracleModel:
    """The MTP head's configuration and its weights, held as float64.

    [HB14 "The draft head"]: a 2H->H projection without bias, two input
    RMSNorms, one full-attention decoder layer, a final RMSNorm; the token
    embedding and lm_head are the main model's.  [YL 二.1] names the same parts
    enorm, hnorm, eh_proj, mtp_block and the shared head."""

    def __init__(self, cfg, weights):
        self.cfg = cfg
        f = lambda a: np.asarray(a, dtype=F64)
        self.embed = weights.embed            # gathered one row at a time
        self.enorm, self.hnorm = f(weights.enorm), f(weights.hnorm)
        self.eh_proj = f(weights.eh_proj)
        self.layers = []
        for lw in weights.layers:
            self.layers.append(dict(in_norm=f(lw.in_norm), wq=f(lw.wq), wk=f(lw.wk), wv=f(lw.wv),
                                    wo=f(lw.wo), post_norm=f(lw.post_norm), wgate=f(lw.wgate),
                                    wup=f(lw.wup), wdown=f(lw.wdown)))
        self.final_norm = f(weights.final_norm)
        self.lm_head = f(weights.lm_head)


class KVCache:
    """The head's own K/V cache: per layer and sequence, [n_kv][T_max][hd].

    Values are stored already rounded to the KV dtype (both fit in float32).
    ``len[b]`` is the number of valid positions; position p lives in slot p.
    [HB14 "The draft head"]: the draft state is an attention cache of shape
    [batch, heads, T, d] that a rollback truncates along T."""

    def __init__(self, cfg, batch: int, max_len: int):
        self.cfg = cfg
        self.max_len = max_len
        shape = (cfg.n_layers, batch, cfg.n_kv_heads, max_len, cfg.head_dim)
        self.K = np.zeros(shape, dtype=np.float32)
        self.V = np.zeros(shape, dtype=np.float32)
        self.len = np.zeros(batch, dtype=np.int64)

    def load_prefix(self, K, V, length: int) -> None:
        """Place given (already rounded) K/V for positions [0, length) and set len."""
        self.K[:, :, :, :length] = K[:, :, :, :length]
        self.V[:, :, :, :length] = V[:, :, :, :length]
        self.len[:] = length


# --------------------------------------------------------------------------------------------
# O3  the decoder block
# --------------------------------------------------------------------------------------------
def decoder_block(model: OracleModel, layer: int, cache: KVCache, b: int, x, pos: int) -> np.ndarray:
    """One pre-norm decoder block for one row of sequence ``b`` at position ``pos``.

    The pages only import the full-attention decoder layer [HB14 "The draft
    head"]; the SwiGLU feed-forward is named by the workload.  Reading (stated
    because the pages leave it open): RMSNorm, Q/K/V projections without bias,
    RoPE on q and k, append k and v to the cache at ``pos`` in the cache dtype,
    grouped-query causal attention over positions 0..pos (query head h reads kv
    head h // (nq/nkv)), output projection and residual; then RMSNorm,
    down(silu(gate m) * up m) and residual."""
    cfg = model.cfg
    w = model.layers[layer]
    nq, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    x = np.asarray(x, dtype=F64)
    a = rms_norm(x, w["in_norm"], cfg.rms_eps)
    q = (w["wq"] @ a).reshape(nq, hd)
    k = (w["wk"] @ a).reshape(nkv, hd)
    v = (w["wv"] @ a).reshape(nkv, hd)
    q = rope(q, pos, cfg.rope_theta)
    k = rope(k, pos, cfg.rope_theta)
    if pos >= cache.max_len:
        raise IndexError(f"position {pos} beyond the cache capacity {cache.max_len}")
    cache.K[layer, b, :, pos] = round_kv(k, cfg.wdtype)
    cache.V[layer, b, :, pos] = round_kv(v, cfg.wdtype)
    group = nq // nkv
    o = np.empty((nq, hd), dtype=F64)
    for h in range(nq):
        g = h // group
        o[h] = attend(q[h], cache.K[layer, b, g, :pos + 1], cache.V[layer, b, g, :pos + 1])
    x = x + w["wo"] @ o.reshape(-1)
    m = rms_norm(x, w["post_norm"], cfg.rms_eps)
    x = x + w["wdown"] @ (silu(w["wgate"] @ m) * (w["wup"] @ m))
    return x


# --------------------------------------------------------------------------------------------
# O4  one MTP row
# --------------------------------------------------------------------------------------------
def mtp_row(model: OracleModel, cache: KVCache, b: int, tok: int, hidden, pos: int):
    """The draft head on one row: (token, hidden, position) -> (g, draft, logits, margin).

    [HB14 "The draft head"]: project cat(norm(e_{t+1}), norm(h_t)) from 2H to H,
    embedding half first, run the decoder layer with its own KV cache at the
    row's position, normalise; the shared output layer gives the prediction for
    position t+2.  [YL 二.2] has the same order ([embedding, previous hidden]).
    Every layer of the stack runs on every step (one module reused for all D
    steps, [YL 二.3] single-module).  Reading: the returned hidden g is the
    post-final-norm vector, the one lm_head reads, and the one fed back to the
    next step.  The position-0 embedding mask of [YL 二.2] is not applied: the
    rows here never sit at position 0 of a sequence with a real prompt."""
    cfg = model.cfg
    if not (0 <= tok < cfg.vocab):
        raise IndexError(f"token {tok} outside the vocabulary")
    e = np.asarray(model.embed[tok], dtype=F64)
    cat = np.concatenate([rms_norm(e, model.enorm, cfg.rms_eps),
                          rms_norm(hidden, model.hnorm, cfg.rms_eps)])
    x = model.eh_proj @ cat
    for layer in range(cfg.n_layers):
        x = decoder_block(model, layer, cache, b, x, pos)
    g = rms_norm(x, model.final_norm, cfg.rms_eps)
    logits = model.lm_head @ g
    draft, margin = argmax_lowest(logits)
    return g, draft, logits, margin


# --------------------------------------------------------------------------------------------
# the target's verify forward (a dense stand-in main model)
# --------------------------------------------------------------------------------------------
class TargetModel:
    """A dense main model sharing the MTP head's token embedding and output layer.

    [HB14 "The draft head"]: the head takes the main model's embedding table and
    lm_head, and the main model hands it its last hidden state; the main model
    returns logits for every position it is given (the verify pass over the
    current token and the D drafts).  The pages do not describe the main model's
    layers.  Reading: a stack of the same pre-norm decoder blocks as the head's
    (O3), a final RMSNorm, and the shared lm_head; its hidden is the post-norm
    vector (the one its lm_head reads), as in the head."""

    def __init__(self, cfg, target_weights):
        self.cfg = cfg
        f = lambda a: np.asarray(a, dtype=F64)
        self.embed = target_weights.embed
        self.layers = []
        for lw in target_weights.layers:
            self.layers.append(dict(in_norm=f(lw.in_norm), wq=f(lw.wq), wk=f(lw.wk), wv=f(lw.wv),
                                    wo=f(lw.wo), post_norm=f(lw.post_norm), wgate=f(lw.wgate),
                                    wup=f(lw.wup), wdown=f(lw.wdown)))
        self.final_norm = f(target_weights.final_norm)
        self.lm_head = f(target_weights.lm_head)


def target_row(model: TargetModel, cache: KVCache, b: int, tok: int, pos: int):
    """The target on one row: x = E[tok], every block at ``pos`` (appending its
    K/V), g = rms(x; g_final), logits = W_lm g.  Returns (g, logits)."""
    cfg = model.cfg
    if not (0 <= tok < cfg.vocab):
        raise IndexError(f"token {tok} outside the vocabulary")
    x = np.asarray(model.embed[tok], dtype=F64)
    for layer in range(cfg.n_layers):
        x = decoder_block(model, layer, cache, b, x, pos)
    g = rms_norm(x, model.final_norm, cfg.rms_eps)
    return g, model.lm_head @ g


def target_forward(model: TargetModel, cache: KVCache, tokens):
    """The target over ``tokens[B][rows]`` (valid prefix of each row = the
    non-negative tokens), row i of sequence b at position len[b] + i; len grows
    by the valid rows.  Returns hiddens [B][rows][H] and logits [B][rows][V]
    (zeros for invalid rows)."""
    tokens = np.asarray(tokens)
    B, R = tokens.shape
    cfg = model.cfg
    hid = np.zeros((B, R, cfg.hidden))
    logits = np.zeros((B, R, cfg.vocab))
    for b in range(B):
        n = _valid_rows(tokens[b])
        p0 = int(cache.len[b])
        for i in range(n):
            hid[b, i], logits[b, i] = target_row(model, cache, b, int(tokens[b, i]), p0 + i)
        cache.len[b] = p0 + n
    return hid, logits


class DenseTarget:
    """``spec_decode``'s target interface over a TargetModel (batch 1): the
    state is its KV cache; there is no recurrent state (an empty table)."""

    def __init__(self, model: TargetModel, max_len: int):
        self.model, self.max_len = model, max_len

    def new_state(self):
        return KVCache(self.model.cfg, 1, self.max_len)

    def forward(self, st, tokens):
        h, lg = target_forward(self.model, st, np.asarray([list(tokens)]))
        return lg[0], h[0]

    def length(self, st):
        return int(st.len[0])

    def crop(self, st, n):
        kv_crop(st, [n])

    def recurrent(self, st):
        return np.zeros((1, 0), np.uint8)

    def set_recurrent(self, st, b):
        pass


# --------------------------------------------------------------------------------------------
# O5  one draft call and the serial D-loop
# --------------------------------------------------------------------------------------------
def _valid_rows(tok_row) -> int:
    n = 0
    for t in tok_row:
        if t < 0:
            break
        n += 1
    return n


def draft_step(model: OracleModel, cache: KVCache, tokens, hiddens, want_logits: bool = True):
    """One head call over a padded batch of rows.

    tokens [B][R] int (a negative token marks padding; the valid rows of a
    sequence are a prefix), hiddens [B][R][H].  Row i of sequence b sits at
    position len[b] + i and appends its K/V there; the call then sets
    len[b] += valid rows.  Returns (hidden_out [B][R][H] (zeros on padding),
    draft [B] (-1 for a sequence with no rows), logits [B][V] of each
    sequence's last row, margin [B]).

    This is both the prompt-length prefill of [HB14 "The draft head"] (every
    prompt position paired with its next token, start 0) and the catch-up after
    a verification (two rows at pos-2 on a hit, one row at pos-1 on a miss)."""
    tokens = np.asarray(tokens)
    B, R = tokens.shape
    H, V = model.cfg.hidden, model.cfg.vocab
    hid_out = np.zeros((B, R, H), dtype=F64)
    drafts = np.full(B, -1, dtype=np.int64)
    logits = np.zeros((B, V), dtype=F64) if want_logits else None
    margins = np.full(B, np.inf)
    for b in range(B):
        n = _valid_rows(tokens[b])
        if cache.len[b] + n > cache.max_len:
            raise IndexError("KV cache capacity exceeded")
        for i in range(n):
            g, d, lg, mg = mtp_row(model, cache, b, int(tokens[b, i]), hiddens[b][i], int(cache.len[b]) + i)
            hid_out[b, i] = g
        cache.len[b] += n
        if n:
            drafts[b], margins[b] = d, mg
            if want_logits:
                logits[b] = lg
    return hid_out, drafts, logits, margins


def draft_loop(model: OracleModel, cache: KVCache, tokens, hiddens, D: int, want_logits: bool = True):
    """Catch-up call, then D-1 serial steps each fed its own hidden and draft.

    [YL 三 stage 1]: the first draft comes from (settled token, target hidden);
    [YL 三 stage 2]: each further step takes the previous draft token and the
    head's previous output hidden.  The serial step k (k >= 2) sits one
    position after step k-1.  Returns drafts [B][D], hiddens [B][D][H] (the g
    of each step's last row), logits [B][D][V], margins [B][D]."""
    tokens = np.asarray(tokens)
    B = tokens.shape[0]
    H, V = model.cfg.hidden, model.cfg.vocab
    drafts = np.full((B, D), -1, dtype=np.int64)
    hid = np.zeros((B, D, H), dtype=F64)
    logits = np.zeros((B, D, V), dtype=F64) if want_logits else None
    margins = np.full((B, D), np.inf)
    hout, d, lg, mg = draft_step(model, cache, tokens, hiddens, want_logits)
    for b in range(B):
        n = _valid_rows(tokens[b])
        if n:
            hid[b, 0] = hout[b, n - 1]
    drafts[:, 0], margins[:, 0] = d, mg
    if want_logits:
        logits[:, 0] = lg
    for k in range(1, D):
        tk = np.where(drafts[:, k - 1:k] >= 0, drafts[:, k - 1:k], -1)
        hout, d, lg, mg = draft_step(model, cache, tk, hid[:, k - 1:k], want_logits)
        drafts[:, k], margins[:, k] = d, mg
        hid[:, k] = hout[:, 0]
        if want_logits:
            logits[:, k] = lg
    return drafts, hid, logits, margins


# --------------------------------------------------------------------------------------------
# several MTP modules: one per draft position
# --------------------------------------------------------------------------------------------
def draft_loop_multi(models: Sequence[OracleModel], caches: Sequence[KVCache], tokens, hiddens, D: int,
                     want_logits: bool = True):
    """The D-step draft loop over M modules, each with its own cache.

    [YL 二.3]: the predictor holds several MTP layers; a single module is
    reused for every step, the layer chosen by the step index modulo the
    number of layers, and multi-module MTP gives each draft position its own
    layer.  [YL 五]: the multi-module form needs a re-prefill to repair the
    stale KV that rejected tokens leave.  Readings: step k (1-based) uses
    module (k-1) mod M at the position the single-module loop gives it (one
    past step k-1); every module keeps, like the single module's cache, the
    K/V of every row of the sequence it is asked about:
      * catch-up (re-prefill after a verification): every module appends the
        catch-up rows (the settled positions, with the main model's hiddens);
        module 0's last row gives draft 1;
      * step k >= 2: module m = (k-1) mod M first appends the rows of this
        round's chain it has not seen yet (positions of steps s_m+1 .. k-1,
        fed (d_j, g_j) as the single module is), then its own row; the last
        row gives draft k.
    A stale row (a rejected draft's) is removed by the caller's crop of every
    module's cache and recomputed by the next catch-up.  With M = 1 this is
    ``draft_loop``; with M identical modules it equals ``draft_loop`` exactly.
    tokens/hiddens: the catch-up rows as in ``draft_step``.  Returns drafts
    [B][D], hiddens [B][D][H], logits [B][D][V], margins [B][D]."""
    M = len(models)
    assert M >= 1 and len(caches) == M
    tokens = np.asarray(tokens)
    B = tokens.shape[0]
    H, V = models[0].cfg.hidden, models[0].cfg.vocab
    drafts = np.full((B, D), -1, dtype=np.int64)
    hid = np.zeros((B, D, H), dtype=F64)
    logits = np.zeros((B, D, V), dtype=F64) if want_logits else None
    margins = np.full((B, D), np.inf)
    for m in range(M):
        hout, d, lg, mg = draft_step(models[m], caches[m], tokens, hiddens, want_logits)
        if m == 0:
            for b in range(B):
                n = _valid_rows(tokens[b])
                if n:
                    hid[b, 0] = hout[b, n - 1]
            drafts[:, 0], margins[:, 0] = d, mg
            if want_logits:
                logits[:, 0] = lg
    seen = [1] * M  # chain steps whose rows each module holds (the catch-up's last row is step 1's)
    for k in range(2, D + 1):
        m = (k - 1) % M
        lo = seen[m]
        # rows of steps lo+1 .. k: step j's row is fed (d_{j-1}, g_{j-1})
        tk = np.where(drafts[:, lo - 1:k - 1] >= 0, drafts[:, lo - 1:k - 1], -1)
        hout, d, lg, mg = draft_step(models[m], caches[m], tk, hid[:, lo - 1:k - 1], want_logits)
        for b in range(B):
            n = _valid_rows(tk[b])
            if n:
                hid[b, k - 1] = hout[b, n - 1]
        drafts[:, k - 1], margins[:, k - 1] = d, mg
        if want_logits:
            logits[:, k - 1] = lg
        seen[m] = k
    return drafts, hid, logits, margins


# --------------------------------------------------------------------------------------------
# a head with no cache of its own: it reads the main model's keys and values
# --------------------------------------------------------------------------------------------
def shared_block(model: OracleModel, layer: int, tcache: KVCache, tlayer: int, b: int, x, pos: int) -> np.ndarray:
    """The head's decoder block when it keeps no K/V ([DLM "MTP speculative
    decoding"] item 1: the drafter has no KV cache and reads the main model's
    keys and values).  q = W_q rms(x), rotated at ``pos``; the keys and values
    are the main model's cache of layer ``tlayer`` for sequence ``b``, positions
    [0, len_b); nothing is appended.  Readings: every cached position is visible
    (the main model has only cached positions before the row's); the head's own
    q/kv head grouping is used over the main model's kv heads (same count and
    head size); an empty cache contributes a zero attention output.  The output
    projection and the SwiGLU part are those of the ordinary block."""
    cfg = model.cfg
    w = model.layers[layer]
    nq, nkv, hd = cfg.n_heads, cfg.n_kv_heads, cfg.head_dim
    x = np.asarray(x, dtype=F64)
    a = rms_norm(x, w["in_norm"], cfg.rms_eps)
    q = rope((w["wq"] @ a).reshape(nq, hd), pos, cfg.rope_theta)
    L = int(tcache.len[b])
    group = nq // nkv
    o = np.zeros((nq, hd), dtype=F64)
    if L > 0:
        for h in range(nq):
            g = h // group
            o[h] = attend(q[h], tcache.K[tlayer, b, g, :L], tcache.V[tlayer, b, g, :L])
    x = x + w["wo"] @ o.reshape(-1)
    m = rms_norm(x, w["post_norm"], cfg.rms_eps)
    x = x + w["wdown"] @ (silu(w["wgate"] @ m) * (w["wup"] @ m))
    return x


def mtp_row_shared(model: OracleModel, tcache: KVCache, kv_layers, b: int, tok: int, hidden, pos: int):
    """``mtp_row`` for a head that reads the main model's cache: head layer l
    attends over the main model's layer ``kv_layers[l]``.  Returns (g, draft,
    logits, margin)."""
    cfg = model.cfg
    if not (0 <= tok < cfg.vocab):
        raise IndexError(f"token {tok} outside the vocabulary")
    e = np.asarray(model.embed[tok], dtype=F64)
    cat = np.concatenate([rms_norm(e, model.enorm, cfg.rms_eps),
                          rms_norm(hidden, model.hnorm, cfg.rms_eps)])
    x = model.eh_proj @ cat
    for layer in range(cfg.n_layers):
        x = shared_block(model, layer, tcache, int(kv_layers[layer]), b, x, pos)
    g = rms_norm(x, model.final_norm, cfg.rms_eps)
    logits = model.lm_head @ g
    draft, margin = argmax_lowest(logits)
    return g, draft, logits, margin


def draft_loop_shared(model: OracleModel, tcache: KVCache, kv_layers, tokens, hiddens, D: int,
                      want_logits: bool = True):
    """D serial draft steps of a head that reads the main model's cache.

    tokens [B]: the settled next token x_n (negative: no drafts for the
    sequence); hiddens [B][H]: the main model's hidden at its last cached
    position.  With no cache of its own the head needs no catch-up rows: step 1
    is the row (x_n, h) at the main model's last cached position len_b - 1,
    step k (k >= 2) the row (d_{k-1}, g_{k-1}) one position later each time
    ([YL 三 stage 2] feeding, as in ``draft_loop``).  The main model's cache
    and its length are read only.  A sequence whose main-model cache is empty
    has no hidden to start from and gets no drafts.  Returns drafts [B][D],
    hiddens [B][D][H], logits [B][D][V], margins [B][D]."""
    tokens = np.asarray(tokens).reshape(-1)
    B = tokens.shape[0]
    H, V = model.cfg.hidden, model.cfg.vocab
    drafts = np.full((B, D), -1, dtype=np.int64)
    hid = np.zeros((B, D, H), dtype=F64)
    logits = np.zeros((B, D, V), dtype=F64) if want_logits else None
    margins = np.full((B, D), np.inf)
    for b in range(B):
        L = int(tcache.len[b])
        if tokens[b] < 0 or L == 0:
            continue
        tok, h = int(tokens[b]), hiddens[b]
        for k in range(D):
            g, d, lg, mg = mtp_row_shared(model, tcache, kv_layers, b, tok, h, L - 1 + k)
            drafts[b, k], hid[b, k], margins[b, k] = d, g, mg
            if want_logits:
                logits[b, k] = lg
            tok, h = d, g
    return drafts, hid, logits, margins


# --------------------------------------------------------------------------------------------
# O6  greedy verification
# --------------------------------------------------------------------------------------------
@dataclass
class VerifyResult:
    n_accept: np.ndarray        # [B]
    out_tokens: np.ndarray      # [B][D+1], -1 after the emitted tokens
    crop_len: np.ndarray        # [B] = ctx_len + 1 + n_accept
    margins: List[List[float]]  # per sequence, the margins of every decision taken, in order
    margin_pos: List[List[int]] = None  # per sequence, the output position j each margin decides

    def trusted_prefix(self, b: int, margin: float) -> int:
        """How many of sequence b's emitted tokens follow only from decisions whose margin is at
        least ``margin`` (all a+1 of them when every margin is): the tokens before the first
        position holding a closer decision."""
        for m, j in zip(self.margins[b], self.margin_pos[b]):
            if m < margin:
                return j
        return int(self.n_accept[b]) + 1


def greedy_verify(target_logits, drafts, ctx_len) -> VerifyResult:
    """Greedy prefix match of D drafts against D+1 target rows.

    Target row j (the target's output at the position holding the settled
    token for j = 0, draft j otherwise) judges draft j+1 [HB14 "The draft head"
    loop steps 2-3; DLM item 2; YL 三 stage 3].  a = length of the prefix with
    argmax(target[j]) == d_{j+1}; emitted: d_1..d_a then argmax(target[a]),
    which is the correction when a < D and the extra token when all drafts
    hold [DLM item 2; YL 三 stage 4].  The target keeps ctx_len + 1 + a
    positions: the settled token plus the accepted drafts."""
    target_logits = np.asarray(target_logits)
    drafts = np.asarray(drafts)
    B, D = drafts.shape
    n_acc = np.zeros(B, dtype=np.int64)
    out = np.full((B, D + 1), -1, dtype=np.int64)
    crop = np.zeros(B, dtype=np.int64)
    margins, mpos = [], []
    for b in range(B):
        ms, mp = [], []
        a = 0
        while True:
            t, m = argmax_lowest(target_logits[b, a])
            ms.append(m)
            mp.append(a)
            if a < D and t == drafts[b, a]:
                out[b, a] = t
                a += 1
                continue
            out[b, a] = t
            break
        n_acc[b] = a
        crop[b] = int(ctx_len[b]) + 1 + a
        margins.append(ms)
        mpos.append(mp)
    return VerifyResult(n_acc, out, crop, margins, mpos)


# --------------------------------------------------------------------------------------------
# O7  temperature, top-k, top-p
# --------------------------------------------------------------------------------------------
def warp(logits, temperature: float, top_k: int, top_p: float):
    """The sampling distribution after temperature, then top-k, then top-p.

    [DLM "Why a hand-written decoding loop"]: temperature, top-k and top-p are
    applied in turn, then a token is drawn.  Readings: tokens are ranked by
    scaled logit descending, id ascending on ties; top-k keeps exactly the
    first k (k <= 0 or k >= V keeps all); the softmax is taken over the kept
    set; top-p walks the kept set in the same order and keeps a token when the
    probability mass before it is below p (so the token that crosses p stays and
    at least one token is kept; p >= 1 keeps all); the result is renormalised.
    Temperature 0 is greedy (one-hot at the lowest-id maximum).

    Returns (w [V] float64 summing to 1, margins list)."""
    l = np.asarray(logits, dtype=F64)
    V = l.shape[-1]
    if temperature <= 0.0:
        i, m = argmax_lowest(l)
        w = np.zeros(V)
        w[i] = 1.0
        return w, [m]
    z = l / temperature
    order = np.lexsort((np.arange(V), -z))          # primary: z descending; ties: id ascending
    margins = []
    if 0 < top_k < V:
        kept = order[:top_k]
        margins.append(float(z[order[top_k - 1]] - z[order[top_k]]))
    else:
        kept = order
    zk = z[kept]
    pi = np.exp(zk - zk[0])
    pi = pi / pi.sum()
    if top_p < 1.0:
        before = np.concatenate([[0.0], np.cumsum(pi)[:-1]])   # mass ranked strictly ahead
        keep = before < top_p
        keep[0] = True                                          # the top token always stays
        margins.append(float(np.min(np.abs(before - top_p))))
        kept, pi = kept[keep], pi[keep]
    w = np.zeros(V)
    w[kept] = pi / pi.sum()
    return w, margins


# --------------------------------------------------------------------------------------------
# O9  inverse-CDF sampling
# --------------------------------------------------------------------------------------------
def sample(weights, u: float):
    """Draw one id from non-negative weights with the uniform ``u`` in [0, 1).

    Reading (the pages only say "sample"): the smallest id i whose cumulative
    weight, summed in ascending id order, exceeds u * total.  Returns (id,
    margin) where margin = the distance of u * total to the nearest cumulative
    boundary around the chosen id, divided by the total."""
    w = np.asarray(weights, dtype=F64)
    c = np.cumsum(w)
    S = c[-1]
    t = float(u) * S
    i = int(np.searchsorted(c, t, side="right"))
    if i >= w.shape[-1]:                     # u * S rounded onto S: take the last id with weight
        i = int(np.nonzero(w > 0)[0][-1])
    lo = c[i - 1] if i > 0 else 0.0
    margin = min(abs(c[i] - t), abs(t - lo)) / S
    return i, float(margin)


# --------------------------------------------------------------------------------------------
# O8  speculative-sampling verification
# --------------------------------------------------------------------------------------------
def residual(P, Q) -> np.ndarray:
    """The distribution a rejected draft is replaced from: max(0, P - Q), or P when that is all zero.

    [YL 三 stage 3] (garbled; read as the positive part of P - Q), [DLM item 3]
    ("drawn from the other candidates" when Q is one-hot).  Left unnormalised:
    ``sample`` scales by the total."""
    r = np.maximum(np.asarray(P, dtype=F64) - np.asarray(Q, dtype=F64), 0.0)
    return r if r.sum() > 0.0 else np.asarray(P, dtype=F64)


def sampling_verify(target_logits, drafts, draft_logits, temperature: float, top_k: int, top_p: float,
                    q_mode: int, u_accept, u_sample, ctx_len) -> VerifyResult:
    """Speculative sampling over D drafts and D+1 target rows.

    For j = 0..D-1, with P_j = warp(target[j]) and Q_j the draft distribution:
    draft d_{j+1} is kept when P_j(d) > 0 and U_j <= P_j(d) / Q_j(d)
    [YL 三 stage 3 rejection rule; DLM item 3 "kept with its probability"].  At
    the first rejection one token is drawn from normalize(max(0, P_j - Q_j))
    (if that is all zero, from P_j) and the round ends; if all D drafts hold,
    one more token is drawn from P_D [DLM item 2].  The draw is ``sample`` with
    u_sample.  q_mode 0: Q_j is one-hot at d_{j+1} (a greedy drafter), so the
    residual is P_j without d_{j+1}, the "other candidates" of [DLM item 3].
    q_mode 1: Q_j = warp(draft_logits[j]) with the same settings.  Readings:
    the garbled residual formula of [YL 三 stage 3] is read as
    normalize(max(0, P - Q)); when Q_j(d) = 0 and P_j(d) > 0 the ratio is taken
    as infinite (accept).
    """
    target_logits = np.asarray(target_logits)
    drafts = np.asarray(drafts)
    B, D = drafts.shape
    n_acc = np.zeros(B, dtype=np.int64)
    out = np.full((B, D + 1), -1, dtype=np.int64)
    crop = np.zeros(B, dtype=np.int64)
    margins, mpos = [], []
    for b in range(B):
        ms = []
        pos = []                             # the output position each margin belongs to
        a = 0
        tok = None
        while a < D:
            P, mp = warp(target_logits[b, a], temperature, top_k, top_p)
            ms += mp
            d = int(drafts[b, a])
            if q_mode == 0:
                Q = np.zeros_like(P)
                Q[d] = 1.0
            else:
                Q, mq = warp(draft_logits[b, a], temperature, top_k, top_p)
                ms += mq
            ratio = np.inf if Q[d] == 0.0 else P[d] / Q[d]
            u = float(u_accept[b, a])
            if np.isfinite(ratio):
                ms.append(abs(ratio - u))
            pos += [a] * (len(ms) - len(pos))
            if P[d] > 0.0 and u <= ratio:
                out[b, a] = d
                a += 1
                continue
            tok, m = sample(residual(P, Q), float(u_sample[b]))
            ms.append(m)
            break
        if tok is None:                      # every draft held: one more token from row D
            P, mp = warp(target_logits[b, D], temperature, top_k, top_p)
            ms += mp
            tok, m = sample(P, float(u_sample[b]))
            ms.append(m)
        pos += [a] * (len(ms) - len(pos))
        out[b, a] = tok
        n_acc[b] = a
        crop[b] = int(ctx_len[b]) + 1 + a
        margins.append(ms)
        mpos.append(pos)
    return VerifyResult(n_acc, out, crop, margins, mpos)


def spec_verify(target_logits, drafts, ctx_len, sampling=None, draft_logits=None,
                u_accept=None, u_sample=None) -> VerifyResult:
    """Greedy verify when ``sampling`` is None or its temperature is 0, else speculative sampling."""
    if sampling is None or sampling.temperature <= 0.0:
        return greedy_verify(target_logits, drafts, ctx_len)
    return sampling_verify(target_logits, drafts, draft_logits, sampling.temperature, sampling.top_k,
                           sampling.top_p, sampling.q_mode, u_accept, u_sample, ctx_len)


# --------------------------------------------------------------------------------------------
# O10  crop, snapshot, restore
# --------------------------------------------------------------------------------------------
def kv_crop(cache: KVCache, new_len) -> None:
    """Truncate each sequence's cache to new_len[b] positions.

    [HB14 "The draft head"]: rolling back an attention cache keeps its first n
    positions; after a miss the head's own cache is cut to the main model's
    position.  [DLM item 2]: the cache is cut back after the first rejected
    guess."""
    for b, n in enumerate(np.asarray(new_len)):
        if n < 0 or n > cache.max_len:
            raise ValueError("crop length out of range")
        cache.len[b] = int(n)


def state_snapshot(state) -> np.ndarray:
    """A byte-for-byte copy of a recurrent state [B][bytes] taken before verification.

    [HB14, paragraph after the loop]: a recurrent memory table cannot be
    truncated, so the tables and convolution windows are copied before the
    verification pass."""
    return np.array(state, dtype=np.uint8, copy=True)


def state_restore(state, snap, n_accept, D: int) -> None:
    """Copy the snapshot back, in place, for every sequence that rejected a draft (n_accept < D)."""
    for b, a in enumerate(np.asarray(n_accept)):
        if a < D:
            state[b, :] = snap[b, :]


# --------------------------------------------------------------------------------------------
# the generalised decode loop (greedy), used to check that the output equals plain greedy
# --------------------------------------------------------------------------------------------
def spec_decode(target, model: OracleModel, prompt: Sequence[int], max_new: int, D: int,
                draft_override=None):
    """Greedy speculative decoding with the MTP head, D drafts per round.

    ``target`` provides: new_state(), forward(state, tokens) -> (logits
    [T][V], hiddens [T][H]) appending T positions, length(state), crop(state,
    n), recurrent(state) -> uint8 [1][bytes] view of its recurrent tables and
    set_recurrent(state, bytes).  Follows the loop of [HB14 "The draft head"]
    (prefill, draft, snapshot, verify, accept or roll back and re-run, head
    catch-up) with the D-draft verification of [YL 三] and [DLM item 2]:

    * main prefill; the settled token x is its last argmax;
    * head prefill: rows (h_i, x_{i+1}) for every prompt position;
    * each round: D drafts; snapshot; target over [x, d_1..d_D]; greedy verify;
      if some draft failed, restore the recurrent state, crop the target's
      cache to its pre-round length and re-run [x, d_1..d_a]; crop the head's
      cache to the pre-round length; catch-up rows (h_{n+i}, x_{n+i+1}).

    ``draft_override(out, drafts) -> drafts`` lets a test replace the head's
    guesses (the output must not depend on them).  Returns (tokens, rounds,
    accepted drafts)."""
    ts = target.new_state()
    logits, hid = target.forward(ts, list(prompt))
    x, _ = argmax_lowest(logits[-1])
    out = [x]
    n = len(prompt)
    cache = KVCache(model.cfg, 1, n + max_new + D + 2)
    tokens = np.array([list(prompt[1:]) + [x]])
    hiddens = np.asarray(hid)[None]
    rounds = hits = 0
    while len(out) < max_new:
        drafts, _, _, _ = draft_loop(model, cache, tokens, hiddens, D, want_logits=False)
        if draft_override is not None:
            drafts = np.asarray(draft_override(list(out), drafts))
        snap = state_snapshot(target.recurrent(ts))
        tl, th = target.forward(ts, [x] + [int(t) for t in drafts[0]])
        res = greedy_verify(np.asarray(tl)[None], drafts, [n])
        a = int(res.n_accept[0])
        emitted = [int(t) for t in res.out_tokens[0, :a + 1]]
        rounds += 1
        hits += a
        if a < D:
            rec = target.recurrent(ts)
            state_restore(rec, snap, res.n_accept, D)
            target.set_recurrent(ts, rec)
            target.crop(ts, n)
            _, th = target.forward(ts, [x] + [int(t) for t in drafts[0, :a]])
        assert target.length(ts) == res.crop_len[0]
        kv_crop(cache, [n])
        tokens = np.array([emitted])
        hiddens = np.asarray(th)[None, :a + 1]
        out += emitted
        x = emitted[-1]
        n += a + 1
    return out, rounds, hits
