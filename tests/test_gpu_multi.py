"""GPU parity of the multi-module draft loop ([YL 二.3, 五]) through mtp_draft_loop_multi: chained
rounds of catch-up (re-prefill of every module) + D draft steps over M modules, greedy
verification and a crop of every module's cache, compared with the oracle round by round.

Bar as for the single-module loop: drafts bit-exact while the oracle's top-2 gap is at least
1e-4 (later steps of that round are then not compared); hiddens and logits within 1e-4 (fp32) or
2e-3 (bf16) max relative error; cache lengths exact.  Both verifiers judge the oracle's drafts."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, make_first_round, make_kv_prefix, make_round_hiddens, make_round_noise, make_weights

pytestmark = pytest.mark.gpu

M_ = pytest.importorskip("speculative_decoding_mtp_amd")
from tests.gpu_util import MARGIN, config, f32, i32, kv_from_numpy, max_rel, upload_weights  # noqa: E402


def _modules(cfg, M):
    """M modules sharing module 0's embedding and lm_head (the shared head of [YL 二.1])."""
    ws = [make_weights(cfg.replace(index=cfg.index + 100 * m)) for m in range(M)]
    for w in ws[1:]:
        w.embed, w.lm_head = ws[0].embed, ws[0].lm_head
    return ws


def _rounds(cfg, M, rounds):
    B, D, H, V = cfg.batch, cfg.D, cfg.hidden, cfg.vocab
    c = config(cfg)
    ws = _modules(cfg, M)
    models = [O.OracleModel(cfg, w) for w in ws]
    gws = [upload_weights(cfg, w) for w in ws]
    max_len = M_.round_max_len(cfg.ctx + rounds * (D + 1) + 2 * D + 8)
    kvs, caches = [], []
    for m in range(M):
        K, Vv = make_kv_prefix(cfg.replace(index=cfg.index + 100 * m))
        kvs.append(kv_from_numpy(cfg, K, Vv, cfg.ctx, max_len))
        oc = O.KVCache(cfg, B, max_len)
        oc.load_prefix(K, Vv, cfg.ctx)
        caches.append(oc)
    toks, hid = make_first_round(cfg)
    ws_dev = M_.new_workspace(M_.mtp_draft_workspace_size(c, B, max(D + 1, D - 1), D, max_len))
    vws = M_.new_workspace(M_.spec_verify_workspace_size(B, D, V, None))
    drafts = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    hids = torch.zeros(B, D, H, device="cuda")
    dlog = torch.zeros(B, D, V, device="cuda")
    n_acc = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.zeros(B, D + 1, dtype=torch.int32, device="cuda")
    crop = torch.zeros(B, dtype=torch.int32, device="cuda")
    tol = 1e-4 if cfg.wdtype == "f32" else 2e-3
    compared = 0
    for r in range(rounds):
        rps = toks.shape[1]
        n_rows = np.array([int(np.argmax(np.append(t < 0, True))) for t in toks])
        ctx = caches[0].len.copy() + n_rows                     # positions after the catch-up
        M_.mtp_draft_loop_multi(c, gws, kvs, D, rps, i32(toks), f32(hid), drafts, hids, dlog, ws_dev)
        M_.mtp_check(ws_dev)
        d_o, h_o, l_o, m_o = O.draft_loop_multi(models, caches, toks, hid, D)
        for m in range(M):
            assert np.array_equal(kvs[m].len.cpu().numpy(), caches[m].len), (r, m)
        dg, hg, lg = drafts.cpu().numpy(), hids.cpu().numpy(), dlog.cpu().numpy()
        for b in range(B):
            for k in range(D):
                assert max_rel(hg[b, k], h_o[b, k]) < tol, (r, b, k)
                assert max_rel(lg[b, k], l_o[b, k]) < tol, (r, b, k)
                if m_o[b, k] < MARGIN:
                    break
                assert dg[b, k] == d_o[b, k], (r, b, k)
                compared += 1
        tl = np.empty((B, D + 1, V), np.float32)
        tl[:, :D] = l_o
        tl[:, D] = l_o[:, D - 1]
        tl += make_round_noise(cfg, r)
        M_.spec_verify(B, D, V, f32(tl), i32(d_o), None, None, None, None, i32(ctx), n_acc, out, crop, vws)
        res = O.greedy_verify(tl, d_o, ctx)
        assert np.array_equal(out.cpu().numpy(), res.out_tokens), r
        for m in range(M):
            M_.kv_crop(kvs[m], i32(ctx))
            O.kv_crop(caches[m], ctx)
        toks = res.out_tokens.astype(np.int32)
        hid = make_round_hiddens(cfg, r)
    return compared


def test_tiny_fp32_three_modules():
    cfg = CONFIGS["tiny"].replace(index=71, batch=2, D=3, ctx=40, prefill_rows=0, noise_std=0.05)
    assert _rounds(cfg, 3, 6) >= 18


def test_bf16_two_modules_five_drafts_mfma_rows():
    # steps of module 1 carry up to 3 chain rows at batch 3: the MFMA GEMM path
    cfg = CONFIGS["tiny"].replace(index=72, wdtype="bf16", n_layers=2, n_heads=8, n_kv_heads=2, head_dim=128,
                                  hidden=512, ffn=1024, vocab=5000, batch=3, D=5, ctx=70, prefill_rows=0,
                                  noise_std=0.05)
    assert _rounds(cfg, 2, 3) >= 15


def test_one_module_equals_the_single_module_loop():
    cfg = CONFIGS["tiny"].replace(index=73, batch=2, D=3, ctx=24, prefill_rows=0)
    c = config(cfg)
    w = make_weights(cfg)
    gw = upload_weights(cfg, w)
    K, Vv = make_kv_prefix(cfg)
    a, b = kv_from_numpy(cfg, K, Vv, cfg.ctx, 64), kv_from_numpy(cfg, K, Vv, cfg.ctx, 64)
    toks, hid = make_first_round(cfg)
    ws = M_.new_workspace(M_.mtp_draft_workspace_size(c, 2, 1, 3, 64))
    out = [(torch.zeros(2, 3, dtype=torch.int32, device="cuda"), torch.zeros(2, 3, cfg.hidden, device="cuda"))
           for _ in range(2)]
    M_.mtp_draft_loop(c, gw, a, 3, 1, i32(toks), f32(hid), out[0][0], out[0][1], None, ws)
    M_.mtp_draft_loop_multi(c, [gw], [b], 3, 1, i32(toks), f32(hid), out[1][0], out[1][1], None, ws)
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v) and torch.equal(a.len, b.len)
