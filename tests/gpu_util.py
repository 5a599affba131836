"""Helpers shared by the GPU parity tests: upload synthetic inputs, compare with the oracle."""
import numpy as np
import torch

import speculative_decoding_mtp_amd as M
from synth import MTPConfig, to_bf16_bits


def config(cfg: MTPConfig) -> M.Config:
    return M.Config(cfg.hidden, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim, cfg.ffn, cfg.vocab, cfg.n_layers,
                    cfg.rope_theta, cfg.rms_eps, M.MTP_BF16 if cfg.wdtype == "bf16" else M.MTP_F32)


def to_dev(a: np.ndarray, wdtype: str) -> torch.Tensor:
    """float32 values (exact in the weight dtype) -> device tensor of that dtype."""
    if wdtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    bits = to_bf16_bits(a).view(np.int16)
    return torch.from_numpy(bits).cuda().view(torch.bfloat16)


def upload_weights(cfg: MTPConfig, w) -> M.Weights:
    d = lambda a: to_dev(a, cfg.wdtype)
    t = dict(embed=d(w.embed), enorm=d(w.enorm), hnorm=d(w.hnorm), eh_proj=d(w.eh_proj),
             final_norm=d(w.final_norm), lm_head=d(w.lm_head), layers=[])
    for lw in w.layers:
        t["layers"].append(dict(in_norm=d(lw.in_norm), wq=d(lw.wq), wk=d(lw.wk), wv=d(lw.wv), wo=d(lw.wo),
                                post_norm=d(lw.post_norm), wgate=d(lw.wgate), wup=d(lw.wup), wdown=d(lw.wdown)))
    return M.Weights(config(cfg), t)


def upload_target_weights(cfg: MTPConfig, tw) -> M.TargetWeights:
    """``cfg`` describes the target (its n_layers)."""
    d = lambda a: to_dev(a, cfg.wdtype)
    t = dict(embed=d(tw.embed), final_norm=d(tw.final_norm), lm_head=d(tw.lm_head), layers=[])
    for lw in tw.layers:
        t["layers"].append(dict(in_norm=d(lw.in_norm), wq=d(lw.wq), wk=d(lw.wk), wv=d(lw.wv), wo=d(lw.wo),
                                post_norm=d(lw.post_norm), wgate=d(lw.wgate), wup=d(lw.wup), wdown=d(lw.wdown)))
    return M.TargetWeights(config(cfg), t)


def kv_from_numpy(cfg: MTPConfig, K: np.ndarray, V: np.ndarray, length: int, max_len: int) -> M.KVCache:
    kv = M.KVCache(config(cfg), K.shape[1], max_len)
    kv.k[:, :, :, :length] = to_dev(K[:, :, :, :length], cfg.wdtype)
    kv.v[:, :, :, :, :length] = to_dev(np.swapaxes(V[:, :, :, :length], -1, -2), cfg.wdtype)
    kv.len.fill_(length)
    return kv


def i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def f32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def max_rel(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max_i |gpu - ref| / max_i |ref| over a tensor."""
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(gpu, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


MARGIN = 1e-4   # decisions whose oracle margin is below this are not required to match
