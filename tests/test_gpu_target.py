"""The target's verify forward on the GPU (a dense stand-in main model that shares the head's
embedding and lm_head, [HB14 "The draft head"]) against the oracle, and the whole loop on the
GPU -- target prefill, head prefill, draft loop, target verify pass, greedy verify, crops --
giving exactly the target's plain greedy output (the greedy identity of [HB14 "Acceptance rate
and speed-up"], [DLM] item 3).

Bar: logits and hiddens within max relative error 1e-4 (fp32) / 2e-3 (bf16); K/V within 1e-5
(fp32) or one bf16 ulp (rare rounding flips of values computed in fp32 vs float64);
emitted tokens identical up to the first plain-greedy decision whose top-2 logit gap is below
1e-4 (none occur for these seeds)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, make_target_weights, make_weights

pytestmark = pytest.mark.gpu

M = pytest.importorskip("speculative_decoding_mtp_amd")
from tests.gpu_util import MARGIN, config, i32, max_rel, upload_target_weights, upload_weights  # noqa: E402


def _target(cfg, layers, std=0.02):
    w = make_weights(cfg)
    tcfg = dataclasses.replace(cfg, n_layers=layers)
    tw = make_target_weights(cfg, layers, w, std)
    return w, tcfg, tw


@pytest.mark.parametrize("kind", ["tiny", "bf16", "bf16_mfma"])
def test_target_forward_matches_oracle(kind):
    if kind == "tiny":
        cfg, B, rows, tol = CONFIGS["tiny"].replace(index=31, embed_std=1.0), 2, 4, 1e-4
    else:
        cfg = CONFIGS["tiny"].replace(index=32, wdtype="bf16", n_heads=4, n_kv_heads=2, head_dim=128, hidden=512,
                                      ffn=1024, vocab=5000, embed_std=1.0)
        B, rows, tol = (2, 4, 2e-3) if kind == "bf16" else (5, 4, 2e-3)   # 20 rows: the MFMA path
    _, tcfg, tw = _target(cfg, 2, std=0.05)
    tm = O.TargetModel(tcfg, tw)
    c, gw = config(tcfg), upload_target_weights(tcfg, tw)
    max_len = 64
    kv = M.KVCache(c, B, max_len)
    cache = O.KVCache(tcfg, B, max_len)
    g = np.random.default_rng(5)
    ws = M.new_workspace(M.mtp_target_workspace_size(c, B, 16, max_len))
    # a 16-row prefill, then a verify-shaped call whose second sequence has a short valid prefix
    for r, toks in enumerate([g.integers(0, cfg.vocab, (B, 16)), g.integers(0, cfg.vocab, (B, rows))]):
        toks = toks.astype(np.int32)
        if r == 1:
            toks[1, 2:] = -1
        R = toks.shape[1]
        hid = torch.zeros(B, R, cfg.hidden, device="cuda")
        lg = torch.full((B, R, cfg.vocab), 7.0, device="cuda")
        M.mtp_target_forward(c, gw, kv, R, i32(toks), hid, lg, ws)
        M.mtp_check(ws)
        h_o, l_o = O.target_forward(tm, cache, toks)
        assert np.array_equal(kv.len.cpu().numpy(), cache.len)
        hg, lgn = hid.cpu().numpy(), lg.cpu().numpy()
        for b in range(B):
            n = int((toks[b] >= 0).cumprod().sum())
            assert max_rel(hg[b, :n], h_o[b, :n]) < tol, (kind, r, b)
            assert max_rel(lgn[b, :n], l_o[b, :n]) < tol, (kind, r, b)
            assert (lgn[b, n:] == 7.0).all()                     # rows past the valid prefix untouched
    # K/V: equal up to rare one-ulp rounding flips of the cache dtype (fp32 vs float64 inputs)
    L = int(cache.len.max())
    kv_tol = 1e-5 if cfg.wdtype == "f32" else 2.0 ** -7
    assert max_rel(kv.k[..., :L, :].float().cpu().numpy(), cache.K[..., :L, :]) < kv_tol
    assert max_rel(kv.v[..., :L].transpose(-1, -2).float().cpu().numpy(), cache.V[..., :L, :]) < kv_tol


class _GpuLoop:
    """The decode loop with every step on the GPU (batch 1)."""

    def __init__(self, cfg, w, tcfg, tw, max_len):
        self.cfg, self.tcfg = cfg, tcfg
        self.c, self.tc = config(cfg), config(tcfg)
        self.gw, self.tgw = upload_weights(cfg, w), upload_target_weights(tcfg, tw)
        self.max_len = max_len
        self.tws = M.new_workspace(M.mtp_target_workspace_size(self.tc, 1, 64, max_len))

    def target(self, kv, toks):
        R = len(toks)
        hid = torch.zeros(1, R, self.cfg.hidden, device="cuda")
        lg = torch.zeros(1, R, self.cfg.vocab, device="cuda")
        M.mtp_target_forward(self.tc, self.tgw, kv, R, i32([toks]), hid, lg, self.tws)
        return hid, lg

    def plain_greedy(self, prompt, n_new):
        kv = M.KVCache(self.tc, 1, self.max_len)
        _, lg = self.target(kv, prompt)
        out, margins = [], []
        row = lg[0, -1]
        while len(out) < n_new:
            top = torch.topk(row, 2).values.cpu().numpy()
            x = int(torch.argmax(row))
            out.append(x)
            margins.append(float(top[0] - top[1]))
            _, lg = self.target(kv, [x])
            row = lg[0, -1]
        return out, margins

    def spec(self, prompt, n_new, D, override=None):
        tkv, hkv = M.KVCache(self.tc, 1, self.max_len), M.KVCache(self.c, 1, self.max_len)
        hid, lg = self.target(tkv, prompt)
        x = int(torch.argmax(lg[0, -1]))
        out, n = [x], len(prompt)
        rps = max(len(prompt), D + 1)
        ws = M.new_workspace(M.mtp_draft_workspace_size(self.c, 1, rps, D, self.max_len))
        vws = M.new_workspace(M.spec_verify_workspace_size(1, D, self.cfg.vocab, None))
        toks = np.full((1, rps), -1, np.int32)
        toks[0, :len(prompt)] = list(prompt[1:]) + [x]
        hin = torch.zeros(1, rps, self.cfg.hidden, device="cuda")
        hin[0, :len(prompt)] = hid[0]
        drafts = torch.zeros(1, D, dtype=torch.int32, device="cuda")
        n_acc = torch.zeros(1, dtype=torch.int32, device="cuda")
        out_t = torch.zeros(1, D + 1, dtype=torch.int32, device="cuda")
        crop = torch.zeros(1, dtype=torch.int32, device="cuda")
        rounds = hits = 0
        while len(out) < n_new:
            M.mtp_draft_loop(self.c, self.gw, hkv, D, rps, i32(toks), hin, drafts, None, None, ws)
            if override is not None:
                drafts = i32(override(list(out), drafts.cpu().numpy()))
            vt = [x] + [int(t) for t in drafts[0].cpu().numpy()]
            th, tl = self.target(tkv, vt)
            M.spec_verify(1, D, self.cfg.vocab, tl, drafts, None, None, None, None, i32([n]), n_acc, out_t, crop, vws)
            a = int(n_acc[0])
            emitted = [int(t) for t in out_t[0, :a + 1].cpu().numpy()]
            M.kv_crop(tkv, crop)
            M.kv_crop(hkv, i32([n]))
            M.mtp_check(ws)
            assert int(tkv.len[0]) == n + 1 + a and int(hkv.len[0]) == n
            toks = np.full((1, rps), -1, np.int32)
            toks[0, :a + 1] = emitted
            hin = torch.zeros(1, rps, self.cfg.hidden, device="cuda")
            hin[0, :a + 1] = th[0, :a + 1]
            out += emitted
            x, n = emitted[-1], n + a + 1
            rounds, hits = rounds + 1, hits + a
        return out, rounds, hits


@pytest.mark.parametrize("D", [1, 3])
def test_gpu_loop_is_plain_greedy(D):
    cfg = CONFIGS["tiny"].replace(index=33 + D, embed_std=1.0)
    w, tcfg, tw = _target(cfg, 2, std=0.05)
    loop = _GpuLoop(cfg, w, tcfg, tw, 256)
    prompt = [int(t) for t in np.random.default_rng(D).integers(0, cfg.vocab, 9)]
    n_new = 48
    plain, margins = loop.plain_greedy(prompt, n_new + D + 2)
    cut = next((i for i, m in enumerate(margins) if m < MARGIN), len(plain))
    assert cut > n_new // 2
    rng = np.random.default_rng(7 + D)

    def mix(out, drafts):
        d = np.array(drafts)
        for j in range(D):
            if len(out) + j < len(plain) and rng.random() < 0.7:
                d[0, j] = plain[len(out) + j]
        return d
    for over in (None, mix):
        out, rounds, hits = loop.spec(prompt, n_new, D, over)
        k = min(len(out), cut)
        assert out[:k] == plain[:k]
        assert len(out) == 1 + rounds + hits
        if over is mix:
            assert hits > 0
