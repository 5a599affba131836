"""Seeded synthetic inputs for the MTP speculative-decoding step.

This module is shared by the CPU oracle, the tests and the benchmark.  It only
draws random numbers and lays them out; it holds none of the method's
arithmetic (no normalisation, projection, attention, sampling or verification).

Every tensor is drawn from its own numpy ``Generator(PCG64)`` stream, keyed by
``(config index, stream id[, round])`` so that any part can be regenerated on
its own.  Streams: 0 weights, 1 embedding, 2 hiddens, 3 KV prefix, 4 tokens,
5 target-logit noise, 6 uniforms, 7 verifier logits, 8 recurrent state.

Weights are drawn as float32 N(0, 0.02) and, for bf16 configurations, rounded
to the nearest bf16 value (ties to even) here, once.  Those rounded values are
the weights: the oracle reads them as float64, the device path reads the bf16
bit patterns.  RMSNorm gains are 1.
"""
from __future__ import annotations

import dataclasses
import os
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np

# stream ids
S_WEIGHTS, S_EMBED, S_HIDDEN, S_KV, S_TOKENS, S_NOISE, S_UNIF, S_VLOGITS, S_STATE, S_TARGET = range(10)


@dataclass(frozen=True)
class Sampling:
    temperature: float
    top_k: int
    top_p: float
    q_mode: int = 0  # 0: draft distribution is one-hot at the greedy draft; 1: warped draft logits


@dataclass(frozen=True)
class MTPConfig:
    """A drafter workload: the MTP head's shape plus the round schedule."""
    index: int
    name: str
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_layers: int
    rope_theta: float
    rms_eps: float
    wdtype: str            # "f32" or "bf16"; the KV cache uses the same type
    embed_std: float
    batch: int
    D: int
    ctx: int               # positions already in the MTP cache before round 0
    prefill_rows: int      # >0: those positions are produced by an MTP prefill call
    rounds: int
    noise_std: float       # target logits = draft logits + N(0, noise_std)
    sampling: Optional[Sampling] = None
    state_bytes_per_seq: int = 0   # recurrent-state bytes snapshotted per round

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def wbytes(self) -> int:
        return 4 if self.wdtype == "f32" else 2

    def replace(self, **kw) -> "MTPConfig":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class VerifyConfig:
    """A verifier-only workload."""
    index: int
    name: str
    batch: int
    D: int
    vocab: int
    draft_std: float
    sigmas: Tuple[float, ...]
    sampling: Sampling
    max_ctx: int


# p1's recurrent snapshot: 18 memory tables plus conv windows, about 19 MB per
# sequence (handbook ch.14, the paragraph after the speculative loop).
P1_STATE_BYTES = 19 * 1024 * 1024

CONFIGS: Dict[str, MTPConfig] = {
    "tiny": MTPConfig(1, "mtp-tiny-h256-v4096-f32-b1-d1-prefill128", 256, 4, 4, 64, 688, 4096, 1,
                      1e4, 1e-6, "f32", 1.0, 1, 1, 128, 128, 64, 1.0),
    "qwen": MTPConfig(2, "mtp-h2048-q16kv4-f6144-v151936-bf16-b1-d1-ctx4096", 2048, 16, 4, 128, 6144,
                      151936, 1, 1e4, 1e-6, "bf16", 0.02, 1, 1, 4096, 0, 64, 0.5,
                      state_bytes_per_seq=P1_STATE_BYTES),
    "drafter4": MTPConfig(3, "mtp-4layer-h1024-q8kv2-f4096-v262144-bf16-b1-d6-ctx2048", 1024, 8, 2, 128,
                          4096, 262144, 4, 1e4, 1e-6, "bf16", 1.0, 1, 6, 2048, 0, 64, 1.0,
                          Sampling(1.0, 64, 0.95, 0)),
    "dsv3": MTPConfig(4, "mtp-h7168-q56kv8-f18432-v129280-bf16-b32-d3-ctx8192", 7168, 56, 8, 128, 18432,
                      129280, 1, 1e4, 1e-6, "bf16", 0.02, 32, 3, 8192, 0, 16, 0.7),
}

VERIFY_CONFIGS: Dict[str, VerifyConfig] = {
    "stress": VerifyConfig(5, "verify-b256-d4-v151936-f32", 256, 4, 151936, 3.0, (0.3, 1.0, 3.0),
                           Sampling(0.7, 50, 0.9, 0), 8192),
}


def gen(cfg_index: int, stream: int, sub: int = 0, block: Optional[int] = None) -> np.random.Generator:
    """The PCG64 stream for (config, stream, sub-key[, block])."""
    key = [1000 * cfg_index + stream, sub] if block is None else [1000 * cfg_index + stream, sub, block]
    return np.random.Generator(np.random.PCG64(key))


_BLOCK = 1 << 22          # elements per independently seeded block of a large tensor
_WORKERS = min(16, os.cpu_count() or 1)


def _normal_blocks(cfg_index: int, stream: int, sub: int, shape, std: float, wdtype: str) -> np.ndarray:
    """N(0, std) float32 of ``shape`` in the config's dtype, drawn in blocks of whole leading-axis
    rows (about 2^22 elements each), block i from its own stream (config, stream, sub, i), the
    blocks filled in parallel threads (NumPy's generators release the GIL while filling)."""
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(shape[0], -1)
    row = flat.shape[1]
    rows_per = max(1, _BLOCK // max(row, 1))
    starts = list(range(0, shape[0], rows_per))

    def fill(i):
        lo, hi = starts[i], min(starts[i] + rows_per, shape[0])
        gen(cfg_index, stream, sub, i).standard_normal((hi - lo, row), dtype=np.float32, out=flat[lo:hi])
        if std != 1.0:
            flat[lo:hi] *= np.float32(std)
        if wdtype != "f32":
            flat[lo:hi] = bf16_bits_to_f32(to_bf16_bits(flat[lo:hi]))

    if len(starts) == 1:
        fill(0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(_WORKERS) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(g: np.random.Generator, shape, std: float) -> np.ndarray:
    a = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


@dataclass
class LayerWeights:
    in_norm: np.ndarray    # [H]
    wq: np.ndarray         # [nq*hd][H]
    wk: np.ndarray         # [nkv*hd][H]
    wv: np.ndarray         # [nkv*hd][H]
    wo: np.ndarray         # [H][nq*hd]
    post_norm: np.ndarray  # [H]
    wgate: np.ndarray      # [F][H]
    wup: np.ndarray        # [F][H]
    wdown: np.ndarray      # [H][F]


@dataclass
class Weights:
    """All tensors float32 holding values exactly representable in the config's wdtype."""
    embed: np.ndarray       # [V][H]
    enorm: np.ndarray       # [H]
    hnorm: np.ndarray       # [H]
    eh_proj: np.ndarray     # [H][2H]   (input = [embedding half ; hidden half])
    layers: list
    final_norm: np.ndarray  # [H]
    lm_head: np.ndarray     # [V][H]


def make_weights(cfg: MTPConfig, std: float = 0.02) -> Weights:
    """The head's matrices N(0, std) in the config's dtype, each tensor from its own sub-key of the
    weights stream (in the order eh_proj, then per layer q, k, v, o, gate, up, down, then lm_head);
    the embedding N(0, embed_std) from the embedding stream; gains 1."""
    H, F = cfg.hidden, cfg.ffn
    key = iter(range(1 << 20))
    w = lambda *shape: _normal_blocks(cfg.index, S_WEIGHTS, next(key), shape, std, cfg.wdtype)
    ones = lambda n: np.ones(n, dtype=np.float32)
    eh = w(H, 2 * H)
    layers = []
    for _ in range(cfg.n_layers):
        layers.append(LayerWeights(ones(H), w(cfg.q_dim, H), w(cfg.kv_dim, H), w(cfg.kv_dim, H),
                                   w(H, cfg.q_dim), ones(H), w(F, H), w(F, H), w(H, F)))
    lm = w(cfg.vocab, H)
    embed = _normal_blocks(cfg.index, S_EMBED, 0, (cfg.vocab, H), cfg.embed_std, cfg.wdtype)
    return Weights(embed, ones(H), ones(H), eh, layers, ones(H), lm)


@dataclass
class TargetWeights:
    """A dense stand-in main model: its own decoder layers and final norm; the token embedding
    and the output layer are the head's (shared, as the MTP head shares the main model's)."""
    embed: np.ndarray       # [V][H]
    layers: list
    final_norm: np.ndarray  # [H]
    lm_head: np.ndarray     # [V][H]


def make_target_weights(cfg: MTPConfig, n_layers: int, head: Weights, std: float = 0.02) -> TargetWeights:
    """n_layers target blocks with the head's dimensions, matrices N(0, std) in the config's
    dtype, gains 1; embedding and lm_head taken from ``head``."""
    H, F = cfg.hidden, cfg.ffn
    key = iter(range(1 << 20))
    w = lambda *shape: _normal_blocks(cfg.index, S_TARGET, next(key), shape, std, cfg.wdtype)
    ones = lambda n: np.ones(n, dtype=np.float32)
    layers = [LayerWeights(ones(H), w(cfg.q_dim, H), w(cfg.kv_dim, H), w(cfg.kv_dim, H), w(H, cfg.q_dim), ones(H),
                           w(F, H), w(F, H), w(H, F)) for _ in range(n_layers)]
    return TargetWeights(head.embed, layers, ones(H), head.lm_head)


def make_kv_prefix(cfg: MTPConfig, length: Optional[int] = None):
    """Random post-RoPE K and V for positions [0, length): N(0,1) in the KV dtype.

    Returns float32 arrays K, V of shape [L][B][nkv][length][hd]."""
    T = cfg.ctx if length is None else length
    shape = (cfg.n_layers * cfg.batch * cfg.n_kv_heads, T, cfg.head_dim)
    full = (cfg.n_layers, cfg.batch, cfg.n_kv_heads, T, cfg.head_dim)
    K = _normal_blocks(cfg.index, S_KV, 0, shape, 1.0, cfg.wdtype).reshape(full)
    V = _normal_blocks(cfg.index, S_KV, 1, shape, 1.0, cfg.wdtype).reshape(full)
    return K, V


def make_prefill(cfg: MTPConfig, rows: Optional[int] = None):
    """Prompt rows for an MTP prefill: tokens uniform over V, hiddens N(0,1).

    Returns tokens int32 [B][R], hiddens float32 [B][R][H]."""
    R = cfg.prefill_rows if rows is None else rows
    g = gen(cfg.index, S_TOKENS, 0)
    toks = g.integers(0, cfg.vocab, size=(cfg.batch, R), dtype=np.int32)
    gh = gen(cfg.index, S_HIDDEN, 0)
    hid = _normal(gh, (cfg.batch, R, cfg.hidden), 1.0)
    return toks, hid


def make_first_round(cfg: MTPConfig):
    """The first catch-up: one row per sequence (settled token, last target hidden)."""
    g = gen(cfg.index, S_TOKENS, 1)
    toks = g.integers(0, cfg.vocab, size=(cfg.batch, 1), dtype=np.int32)
    gh = gen(cfg.index, S_HIDDEN, 1)
    hid = _normal(gh, (cfg.batch, 1, cfg.hidden), 1.0)
    return toks, hid


def make_round_hiddens(cfg: MTPConfig, rnd: int) -> np.ndarray:
    """Target hiddens at the D+1 verified positions of round ``rnd``: N(0,1), [B][D+1][H]."""
    g = gen(cfg.index, S_HIDDEN, 100 + rnd)
    return _normal(g, (cfg.batch, cfg.D + 1, cfg.hidden), 1.0)


def make_round_noise(cfg: MTPConfig, rnd: int, std: Optional[float] = None) -> np.ndarray:
    """Target-logit noise of round ``rnd``: N(0, noise_std), [B][D+1][V] float32."""
    return _normal_blocks(cfg.index, S_NOISE, rnd, (cfg.batch * (cfg.D + 1), cfg.vocab),
                          cfg.noise_std if std is None else std, "f32").reshape(cfg.batch, cfg.D + 1, cfg.vocab)


def make_round_uniforms(cfg_index: int, B: int, D: int, rnd: int):
    """u_accept [B][D] and u_sample [B], float32 in [0, 1)."""
    g = gen(cfg_index, S_UNIF, rnd)
    return g.random((B, D), dtype=np.float32), g.random(B, dtype=np.float32)


def make_state(B: int, nbytes: int, cfg_index: int = 0) -> np.ndarray:
    """An opaque recurrent state: uint8 [B][nbytes]."""
    g = gen(cfg_index, S_STATE)
    return g.integers(0, 256, size=(B, nbytes), dtype=np.uint8)


def make_verify_inputs(vc: VerifyConfig, sigma: float, batch: Optional[int] = None):
    """Verifier-only inputs: draft logits N(0, draft_std), target = draft + N(0, sigma).

    Drafts are left to the caller (greedy drafts are the argmax of the draft
    logits, which is method arithmetic).  Returns draft_logits [B][D][V],
    target_logits [B][D+1][V] (position D gets its own draw), ctx_len [B]."""
    B = vc.batch if batch is None else batch
    si = {s: i for i, s in enumerate(vc.sigmas)}.get(sigma, 99)
    g = gen(vc.index, S_VLOGITS, si)
    dl = _normal(g, (B, vc.D, vc.vocab), vc.draft_std)
    tgt = np.empty((B, vc.D + 1, vc.vocab), dtype=np.float32)
    tgt[:, :vc.D] = dl + _normal(g, (B, vc.D, vc.vocab), sigma)
    tgt[:, vc.D] = _normal(g, (B, vc.vocab), vc.draft_std) + _normal(g, (B, vc.vocab), sigma)
    gc = gen(vc.index, S_TOKENS, si)
    ctx = gc.integers(1, vc.max_ctx + 1, size=B, dtype=np.int32)
    return dl, tgt, ctx
