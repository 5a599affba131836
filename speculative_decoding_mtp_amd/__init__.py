"""Python binding of libmtp_hip.so, the MI355X (gfx950) MTP speculative-decoding step.

Argument marshalling only: every function here checks tensor devices, dtypes and shapes,
passes raw device pointers and the current HIP stream to the C ABI declared in
include/mtp.h, and raises ``MTPError`` on a non-zero status.  All compute runs in the HIP
kernels of the library.  PyTorch provides device memory and streams.

The library must have been built (``python -m speculative_decoding_mtp_amd.build``); importing
this package without it raises ImportError.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmtp_hip.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m speculative_decoding_mtp_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

MTP_F32, MTP_BF16 = 0, 1
MTP_KERNEL_LM_HEAD, MTP_KERNEL_VERIFY = 1, 2
STATUS = {0: "MTP_OK", -1: "MTP_ERR_ARG", -2: "MTP_ERR_SHAPE", -3: "MTP_ERR_DTYPE", -4: "MTP_ERR_CAPACITY",
          -5: "MTP_ERR_WORKSPACE", -6: "MTP_ERR_HIP", -7: "MTP_ERR_TOKEN"}


class MTPError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


# ---------------------------------------------------------------- C structs
class MtpConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("wdtype", ctypes.c_int32)]


class MtpLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("in_norm", "wq", "wk", "wv", "wo", "post_norm", "wgate", "wup", "wdown")]


class MtpWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("enorm", ctypes.c_void_p), ("hnorm", ctypes.c_void_p),
                ("eh_proj", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(MtpLayerWeights))]


class MtpTargetWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(MtpLayerWeights))]


class MtpKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("len", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_len", ctypes.c_int32)]


class MtpSampling(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("top_k", ctypes.c_int32), ("top_p", ctypes.c_float),
                ("q_mode", ctypes.c_int32)]


_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_sigs = {
    "mtp_last_error": ([], ctypes.c_char_p),
    "mtp_draft_workspace_size": ([ctypes.POINTER(MtpConfig), _I, _I, _I, _I, ctypes.POINTER(_SZ)], _I),
    "mtp_draft_step": ([ctypes.POINTER(MtpConfig), ctypes.POINTER(MtpWeights), ctypes.POINTER(MtpKV), _I, _P, _P, _P,
                        _P, _P, _P, _SZ, _P], _I),
    "mtp_draft_loop": ([ctypes.POINTER(MtpConfig), ctypes.POINTER(MtpWeights), ctypes.POINTER(MtpKV), _I, _I, _P, _P,
                        _P, _P, _P, _P, _SZ, _P], _I),
    "mtp_draft_loop_multi": ([ctypes.POINTER(MtpConfig), ctypes.POINTER(MtpWeights), _I, ctypes.POINTER(MtpKV), _I, _I,
                              _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "mtp_draft_loop_shared_kv": ([ctypes.POINTER(MtpConfig), ctypes.POINTER(MtpWeights), ctypes.POINTER(MtpKV), _I,
                                  ctypes.POINTER(_I), _I, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "spec_verify_workspace_size": ([_I, _I, _I, ctypes.POINTER(MtpSampling), ctypes.POINTER(_SZ)], _I),
    "spec_verify": ([_I, _I, _I, _P, _P, _P, ctypes.POINTER(MtpSampling), _P, _P, _P, _P, _P, _P, _P, _SZ, _P], _I),
    "spec_verify_noalloc": ([_I, _I, _I, _P, _P, _P, ctypes.POINTER(MtpSampling), _P, _P, _P, _P, _P, _P, _P], _I),
    "kv_crop": ([ctypes.POINTER(MtpKV), _P, _P], _I),
    "mtp_state_snapshot": ([_P, _P, _SZ, _I, _P], _I),
    "mtp_state_restore": ([_P, _P, _SZ, _I, _P, _I, _P], _I),
    "mtp_check": ([_P, _P], _I),
    "mtp_target_workspace_size": ([ctypes.POINTER(MtpConfig), _I, _I, _I, ctypes.POINTER(_SZ)], _I),
    "mtp_target_forward": ([ctypes.POINTER(MtpConfig), ctypes.POINTER(MtpTargetWeights), ctypes.POINTER(MtpKV), _I,
                            _P, _P, _P, _P, _SZ, _P], _I),
    "mtp_timer_start": ([_I, _I], _I),
    "mtp_timer_read": ([_I, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(_I)], _I),
    "mtp_timer_kernel_name": ([_I], ctypes.c_char_p),
}
for _name, (_args, _res) in _sigs.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_sigs)


def _check(rc: int) -> None:
    if rc != 0:
        raise MTPError(rc, _lib.mtp_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor", numel: Optional[int] = None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")
    return t.data_ptr()


# ---------------------------------------------------------------- model / cache holders
@dataclass
class Config:
    hidden: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    n_layers: int
    rope_theta: float
    rms_eps: float
    wdtype: int

    def c(self) -> MtpConfig:
        return MtpConfig(self.hidden, self.n_heads, self.n_kv_heads, self.head_dim, self.ffn, self.vocab,
                         self.n_layers, self.rope_theta, self.rms_eps, self.wdtype)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.wdtype == MTP_BF16 else torch.float32


class Weights:
    """Device weight tensors of the head, kept alive with the C struct that points at them.

    ``tensors``: dict with embed, enorm, hnorm, eh_proj, final_norm, lm_head and ``layers`` (a
    list of dicts with in_norm, wq, wk, wv, wo, post_norm, wgate, wup, wdown), all contiguous
    device tensors of the config's dtype."""

    def __init__(self, cfg: Config, tensors: dict):
        self.cfg = cfg
        self.t = tensors
        dt = cfg.torch_dtype
        for k in ("embed", "enorm", "hnorm", "eh_proj", "final_norm", "lm_head"):
            _ptr(tensors[k], dt, k)
        self._layers = (MtpLayerWeights * cfg.n_layers)()
        for i, lw in enumerate(tensors["layers"]):
            for k in ("in_norm", "wq", "wk", "wv", "wo", "post_norm", "wgate", "wup", "wdown"):
                setattr(self._layers[i], k, _ptr(lw[k], dt, f"layers[{i}].{k}"))
        self.c = MtpWeights(tensors["embed"].data_ptr(), tensors["enorm"].data_ptr(), tensors["hnorm"].data_ptr(),
                            tensors["eh_proj"].data_ptr(), tensors["final_norm"].data_ptr(),
                            tensors["lm_head"].data_ptr(), self._layers)


class TargetWeights:
    """Device weight tensors of the dense stand-in target: ``tensors`` holds embed, final_norm,
    lm_head and ``layers`` (as in Weights), kept alive with the C struct."""

    def __init__(self, cfg: Config, tensors: dict):
        self.cfg = cfg
        self.t = tensors
        dt = cfg.torch_dtype
        for k in ("embed", "final_norm", "lm_head"):
            _ptr(tensors[k], dt, k)
        self._layers = (MtpLayerWeights * cfg.n_layers)()
        for i, lw in enumerate(tensors["layers"]):
            for k in ("in_norm", "wq", "wk", "wv", "wo", "post_norm", "wgate", "wup", "wdown"):
                setattr(self._layers[i], k, _ptr(lw[k], dt, f"layers[{i}].{k}"))
        self.c = MtpTargetWeights(tensors["embed"].data_ptr(), tensors["final_norm"].data_ptr(),
                                  tensors["lm_head"].data_ptr(), self._layers)


def round_max_len(n: int) -> int:
    """The smallest cache capacity >= n that is a multiple of 64 (the library accepts multiples
    of 8; with 64 every 64-position segment of a bf16 value row sits on one 128-byte line)."""
    return -(-int(n) // 64) * 64


class KVCache:
    """The head's cache: keys [n_layers][batch][n_kv_heads][max_len][head_dim], values transposed
    [n_layers][batch][n_kv_heads][head_dim][max_len], lengths [batch].  max_len: multiple of 8."""

    def __init__(self, cfg: Config, batch: int, max_len: int, device="cuda", n_layers: Optional[int] = None):
        if max_len < 8 or max_len % 8:
            raise MTPError(-1, f"max_len must be a positive multiple of 8, got {max_len}")
        L = cfg.n_layers if n_layers is None else n_layers
        self.k = torch.zeros((L, batch, cfg.n_kv_heads, max_len, cfg.head_dim), dtype=cfg.torch_dtype, device=device)
        self.v = torch.zeros((L, batch, cfg.n_kv_heads, cfg.head_dim, max_len), dtype=cfg.torch_dtype, device=device)
        self.n_layers = L
        self.len = torch.zeros(batch, dtype=torch.int32, device=device)
        self.batch, self.max_len = batch, max_len

    def c(self) -> MtpKV:
        return MtpKV(self.k.data_ptr(), self.v.data_ptr(), self.len.data_ptr(), self.batch, self.max_len)


def sampling(temperature: float, top_k: int, top_p: float, q_mode: int = 0) -> MtpSampling:
    return MtpSampling(temperature, top_k, top_p, q_mode)


# ---------------------------------------------------------------- entry points (same names as the C ABI)
def mtp_draft_workspace_size(cfg: Config, batch: int, rows_per_seq: int, D: int, max_len: int) -> int:
    n = _SZ()
    _check(_lib.mtp_draft_workspace_size(ctypes.byref(cfg.c()), batch, rows_per_seq, D, max_len, ctypes.byref(n)))
    return n.value


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (16-byte aligned: torch allocations are 256-byte aligned)."""
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def mtp_target_workspace_size(cfg: Config, batch: int, rows_per_seq: int, max_len: int) -> int:
    n = _SZ()
    _check(_lib.mtp_target_workspace_size(ctypes.byref(cfg.c()), batch, rows_per_seq, max_len, ctypes.byref(n)))
    return n.value


def mtp_target_forward(cfg: Config, w: TargetWeights, kv: KVCache, rows_per_seq: int, tokens, hidden_out,
                       logits_out, ws: torch.Tensor, stream=None) -> None:
    B, H = kv.batch, cfg.hidden
    R = B * rows_per_seq
    _check(_lib.mtp_target_forward(
        ctypes.byref(cfg.c()), ctypes.byref(w.c), ctypes.byref(kv.c()), rows_per_seq,
        _ptr(tokens, torch.int32, "tokens", R), _ptr(hidden_out, torch.float32, "hidden_out", R * H),
        _ptr(logits_out, torch.float32, "logits_out", R * cfg.vocab), _ptr(ws, None, "ws"), ws.numel(),
        _stream(stream)))


def mtp_draft_step(cfg: Config, w: Weights, kv: KVCache, rows_per_seq: int, tokens, hidden_in, hidden_out,
                   draft_out, logits_out, ws: torch.Tensor, stream=None) -> None:
    B, H = kv.batch, cfg.hidden
    R = B * rows_per_seq
    _check(_lib.mtp_draft_step(
        ctypes.byref(cfg.c()), ctypes.byref(w.c), ctypes.byref(kv.c()), rows_per_seq,
        _ptr(tokens, torch.int32, "tokens", R), _ptr(hidden_in, torch.float32, "hidden_in", R * H),
        _ptr(hidden_out, torch.float32, "hidden_out", R * H), _ptr(draft_out, torch.int32, "draft_out", B),
        _ptr(logits_out, torch.float32, "logits_out", B * cfg.vocab), _ptr(ws, None, "ws"), ws.numel(),
        _stream(stream)))


def mtp_draft_loop(cfg: Config, w: Weights, kv: KVCache, D: int, rows_per_seq: int, tokens, hidden_in, drafts,
                   hiddens, draft_logits, ws: torch.Tensor, stream=None) -> None:
    B, H = kv.batch, cfg.hidden
    R = B * rows_per_seq
    _check(_lib.mtp_draft_loop(
        ctypes.byref(cfg.c()), ctypes.byref(w.c), ctypes.byref(kv.c()), D, rows_per_seq,
        _ptr(tokens, torch.int32, "tokens", R), _ptr(hidden_in, torch.float32, "hidden_in", R * H),
        _ptr(drafts, torch.int32, "drafts", B * D), _ptr(hiddens, torch.float32, "hiddens", B * D * H),
        _ptr(draft_logits, torch.float32, "draft_logits", B * D * cfg.vocab), _ptr(ws, None, "ws"), ws.numel(),
        _stream(stream)))


def mtp_draft_loop_multi(cfg: Config, modules: Sequence[Weights], kvs: Sequence[KVCache], D: int, rows_per_seq: int,
                         tokens, hidden_in, drafts, hiddens, draft_logits, ws: torch.Tensor, stream=None) -> None:
    M = len(modules)
    if M < 1 or len(kvs) != M:
        raise MTPError(-1, "one cache per module needed")
    B, H = kvs[0].batch, cfg.hidden
    R = B * rows_per_seq
    ws_arr = (MtpWeights * M)(*[w.c for w in modules])
    kv_arr = (MtpKV * M)(*[kv.c() for kv in kvs])
    _check(_lib.mtp_draft_loop_multi(
        ctypes.byref(cfg.c()), ws_arr, M, kv_arr, D, rows_per_seq,
        _ptr(tokens, torch.int32, "tokens", R), _ptr(hidden_in, torch.float32, "hidden_in", R * H),
        _ptr(drafts, torch.int32, "drafts", B * D), _ptr(hiddens, torch.float32, "hiddens", B * D * H),
        _ptr(draft_logits, torch.float32, "draft_logits", B * D * cfg.vocab), _ptr(ws, None, "ws"), ws.numel(),
        _stream(stream)))


def mtp_draft_loop_shared_kv(cfg: Config, w: Weights, target_kv: KVCache, kv_layer, D: int, tokens, hidden_in,
                             drafts, hiddens, draft_logits, ws: torch.Tensor, stream=None) -> None:
    B, H = target_kv.batch, cfg.hidden
    if len(kv_layer) != cfg.n_layers:
        raise MTPError(-1, f"kv_layer needs {cfg.n_layers} entries")
    layers = (_I * cfg.n_layers)(*[int(x) for x in kv_layer])
    _check(_lib.mtp_draft_loop_shared_kv(
        ctypes.byref(cfg.c()), ctypes.byref(w.c), ctypes.byref(target_kv.c()), target_kv.n_layers, layers, D,
        _ptr(tokens, torch.int32, "tokens", B), _ptr(hidden_in, torch.float32, "hidden_in", B * H),
        _ptr(drafts, torch.int32, "drafts", B * D), _ptr(hiddens, torch.float32, "hiddens", B * D * H),
        _ptr(draft_logits, torch.float32, "draft_logits", B * D * cfg.vocab), _ptr(ws, None, "ws"), ws.numel(),
        _stream(stream)))


def spec_verify_workspace_size(B: int, D: int, V: int, sp: Optional[MtpSampling]) -> int:
    n = _SZ()
    _check(_lib.spec_verify_workspace_size(B, D, V, ctypes.byref(sp) if sp is not None else None, ctypes.byref(n)))
    return n.value


def spec_verify(B: int, D: int, V: int, target_logits, drafts, draft_logits, sp: Optional[MtpSampling], u_accept,
                u_sample, ctx_len, n_accept, out_tokens, crop_len, ws: torch.Tensor, stream=None) -> None:
    _check(_lib.spec_verify(
        B, D, V, _ptr(target_logits, torch.float32, "target_logits", B * (D + 1) * V),
        _ptr(drafts, torch.int32, "drafts", B * D), _ptr(draft_logits, torch.float32, "draft_logits", B * D * V),
        ctypes.byref(sp) if sp is not None else None, _ptr(u_accept, torch.float32, "u_accept", B * D),
        _ptr(u_sample, torch.float32, "u_sample", B), _ptr(ctx_len, torch.int32, "ctx_len", B),
        _ptr(n_accept, torch.int32, "n_accept", B), _ptr(out_tokens, torch.int32, "out_tokens", B * (D + 1)),
        _ptr(crop_len, torch.int32, "crop_len", B), _ptr(ws, None, "ws"), ws.numel(), _stream(stream)))


def spec_verify_noalloc(B: int, D: int, V: int, target_logits, drafts, draft_logits, sp: Optional[MtpSampling],
                        u_accept, u_sample, ctx_len, n_accept, out_tokens, crop_len, stream=None) -> None:
    """spec_verify with the library's own per-GPU scratch array instead of a workspace."""
    _check(_lib.spec_verify_noalloc(
        B, D, V, _ptr(target_logits, torch.float32, "target_logits", B * (D + 1) * V),
        _ptr(drafts, torch.int32, "drafts", B * D), _ptr(draft_logits, torch.float32, "draft_logits", B * D * V),
        ctypes.byref(sp) if sp is not None else None, _ptr(u_accept, torch.float32, "u_accept", B * D),
        _ptr(u_sample, torch.float32, "u_sample", B), _ptr(ctx_len, torch.int32, "ctx_len", B),
        _ptr(n_accept, torch.int32, "n_accept", B), _ptr(out_tokens, torch.int32, "out_tokens", B * (D + 1)),
        _ptr(crop_len, torch.int32, "crop_len", B), _stream(stream)))


def kv_crop(kv: KVCache, new_len, stream=None) -> None:
    _check(_lib.kv_crop(ctypes.byref(kv.c()), _ptr(new_len, torch.int32, "new_len", kv.batch), _stream(stream)))


def mtp_state_snapshot(state: torch.Tensor, snap: torch.Tensor, bytes_per_seq: int, B: int, stream=None) -> None:
    _check(_lib.mtp_state_snapshot(_ptr(state, None, "state"), _ptr(snap, None, "snap"), bytes_per_seq, B,
                                   _stream(stream)))


def mtp_state_restore(state: torch.Tensor, snap: torch.Tensor, bytes_per_seq: int, B: int, n_accept, D: int,
                      stream=None) -> None:
    _check(_lib.mtp_state_restore(_ptr(state, None, "state"), _ptr(snap, None, "snap"), bytes_per_seq, B,
                                  _ptr(n_accept, torch.int32, "n_accept", B), D, _stream(stream)))


def mtp_check(ws: torch.Tensor, stream=None) -> None:
    _check(_lib.mtp_check(_ptr(ws, None, "ws"), _stream(stream)))


def mtp_timer_start(kernel: int, max_launches: int) -> None:
    _check(_lib.mtp_timer_start(kernel, max_launches))


def mtp_timer_read(kernel: int):
    ms = ctypes.c_float()
    n = _I()
    _check(_lib.mtp_timer_read(kernel, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def mtp_timer_kernel_name(kernel: int) -> str:
    return _lib.mtp_timer_kernel_name(kernel).decode()
