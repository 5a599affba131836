"""GPU parity of the draft head against the oracle, through the C ABI.

Bar: draft tokens and verify outputs bit-exact except where the oracle's top-2 logit gap is
below 1e-4 (then the oracle's token is fed to both sides); hiddens and logits within max
relative error 1e-4 for fp32 weights and 2e-3 for bf16 weights (fp32 against float64 arithmetic on
identical bf16 operands)."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, make_first_round, make_kv_prefix, make_prefill, make_round_hiddens, make_round_noise, \
    make_weights

pytestmark = pytest.mark.gpu

M = pytest.importorskip("speculative_decoding_mtp_amd")
from tests.gpu_util import MARGIN, config, f32, i32, kv_from_numpy, max_rel, upload_weights  # noqa: E402


def _tol(cfg):
    return 1e-4 if cfg.wdtype == "f32" else 2e-3


def _setup(cfg, max_extra=64):
    w = make_weights(cfg)
    model = O.OracleModel(cfg, w)
    c = config(cfg)
    gw = upload_weights(cfg, w)
    max_len = M.round_max_len(cfg.ctx + cfg.rounds * (cfg.D + 1) + max_extra)
    return w, model, c, gw, max_len


def test_prefill_rows_match_oracle():
    """The 128-row head prefill of the tiny fp32 head: every row's hidden, the last row's
    logits and draft, and the appended K/V."""
    cfg = CONFIGS["tiny"]
    _, model, c, gw, max_len = _setup(cfg)
    toks, hid = make_prefill(cfg)
    R = toks.shape[1]
    kv = M.KVCache(c, 1, max_len)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, 1, R, 1, max_len))
    hout = torch.zeros(1, R, cfg.hidden, device="cuda")
    draft = torch.zeros(1, dtype=torch.int32, device="cuda")
    logits = torch.zeros(1, cfg.vocab, device="cuda")
    M.mtp_draft_step(c, gw, kv, R, i32(toks), f32(hid), hout, draft, logits, ws)
    M.mtp_check(ws)
    cache = O.KVCache(cfg, 1, max_len)
    h_o, d_o, l_o, m_o = O.draft_step(model, cache, toks, hid)
    assert int(kv.len[0]) == R == cache.len[0]
    assert max_rel(hout.cpu().numpy(), h_o) < 1e-4
    assert max_rel(logits.cpu().numpy(), l_o) < 1e-4
    if m_o[0] >= MARGIN:
        assert int(draft[0]) == d_o[0]
    assert max_rel(kv.k[:, :, :, :R].float().cpu().numpy(), cache.K[:, :, :, :R]) < 1e-5
    assert max_rel(kv.v[..., :R].transpose(-1, -2).float().cpu().numpy(), cache.V[:, :, :, :R]) < 1e-5


def _run_rounds(cfg, rounds, seq_check=None):
    """Chained rounds: catch-up + serial drafts (compared with the oracle), target logits from
    the oracle's logits plus seeded noise, greedy verify (compared), crop, next catch-up."""
    w, model, c, gw, max_len = _setup(cfg)
    B, D, H, V = cfg.batch, cfg.D, cfg.hidden, cfg.vocab
    kv = M.KVCache(c, B, max_len)
    cache = O.KVCache(cfg, B, max_len)
    if cfg.prefill_rows:
        toks, hid = make_prefill(cfg)
    else:
        K, Vv = make_kv_prefix(cfg)
        kv = kv_from_numpy(cfg, K, Vv, cfg.ctx, max_len)
        cache.load_prefix(K, Vv, cfg.ctx)
        toks, hid = make_first_round(cfg)
    rps_max = max(toks.shape[1], D + 1)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, B, rps_max, D, max_len))
    vws = M.new_workspace(M.spec_verify_workspace_size(B, D, V, None))
    drafts = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    hids = torch.zeros(B, D, H, device="cuda")
    dlog = torch.zeros(B, D, V, device="cuda")
    n_acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.zeros(B, D + 1, dtype=torch.int32, device="cuda")
    crop = torch.zeros(B, dtype=torch.int32, device="cuda")
    stats = dict(accepted=0, rounds=0, excluded=0)
    tol = _tol(cfg)
    for r in range(rounds):
        rps = toks.shape[1]
        M.mtp_draft_loop(c, gw, kv, D, rps, i32(toks), f32(hid), drafts, hids, dlog, ws)
        M.mtp_check(ws)
        d_o, h_o, l_o, m_o = O.draft_loop(model, cache, toks, hid, D)
        ctx = cache.len.copy() - (D - 1)                  # positions after the catch-up
        assert np.array_equal(kv.len.cpu().numpy(), cache.len)
        dg, hg, lg = drafts.cpu().numpy(), hids.cpu().numpy(), dlog.cpu().numpy()
        for b in range(B):
            for k in range(D):
                assert max_rel(hg[b, k], h_o[b, k]) < tol, (r, b, k)
                assert max_rel(lg[b, k], l_o[b, k]) < tol, (r, b, k)
                if m_o[b, k] < MARGIN:
                    stats["excluded"] += 1
                    break                                   # later steps may follow another draft
                assert dg[b, k] == d_o[b, k], (r, b, k)
        noise = make_round_noise(cfg, r)
        tl = np.empty((B, D + 1, V), np.float32)
        tl[:, :D] = l_o.astype(np.float32)
        tl[:, D] = l_o[:, D - 1].astype(np.float32)
        tl += noise
        # teacher forcing: both verifiers judge the oracle's drafts
        M.spec_verify(B, D, V, f32(tl), i32(d_o), None, None, None, None, i32(ctx), n_acc, out, crop, vws)
        res = O.greedy_verify(tl, d_o, ctx)
        assert np.array_equal(n_acc.cpu().numpy(), res.n_accept), r
        assert np.array_equal(out.cpu().numpy(), res.out_tokens), r
        assert np.array_equal(crop.cpu().numpy(), res.crop_len), r
        M.kv_crop(kv, i32(ctx))
        O.kv_crop(cache, ctx)
        stats["accepted"] += int(res.n_accept.sum())
        stats["rounds"] += 1
        toks = res.out_tokens.astype(np.int32)
        hid = make_round_hiddens(cfg, r)
    return stats


def test_tiny_fp32_64_rounds():
    cfg = CONFIGS["tiny"]
    s = _run_rounds(cfg, cfg.rounds)
    assert s["rounds"] == 64


def test_tiny_batched_d3_with_acceptance():
    # three sequences, three drafts, little noise: the accept and bonus paths are exercised
    cfg = CONFIGS["tiny"].replace(index=11, batch=3, D=3, noise_std=0.002, rounds=12)
    s = _run_rounds(cfg, cfg.rounds)
    assert s["accepted"] > 0


def test_two_layer_bf16_small_head():
    cfg = CONFIGS["tiny"].replace(index=12, wdtype="bf16", n_layers=2, n_heads=4, n_kv_heads=2, head_dim=128,
                                  hidden=512, ffn=1024, vocab=5000, batch=2, D=2, prefill_rows=0, ctx=300,
                                  noise_std=0.01, rounds=6, embed_std=1.0)
    _run_rounds(cfg, cfg.rounds)


def test_batched_bf16_head_mfma_path():
    # 20 sequences and two drafts: 60 padded catch-up rows and 20 rows per serial step take the
    # bf16 MFMA path (split-bf16 activations); the oracle stays the plain float64 definition
    cfg = CONFIGS["tiny"].replace(index=13, wdtype="bf16", n_heads=2, n_kv_heads=1, head_dim=128, hidden=256,
                                  ffn=512, vocab=3000, batch=20, D=2, prefill_rows=0, ctx=200, noise_std=0.01,
                                  rounds=5, embed_std=1.0)
    s = _run_rounds(cfg, cfg.rounds)
    assert s["accepted"] > 0
