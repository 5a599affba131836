"""Full-size parity of the draft head and verifier, in the launch configuration bench.py uses
(the same entry points, workspace sizing and kernels), on sampled outputs the oracle can
compute one by one.

Workloads: the single-layer bf16 head (H 2048, 16/4 heads, FFN 6144, vocab 151936, 4096-position
context), the 4-layer bf16 drafter (H 1024, 8/2 heads, FFN 4096, vocab 262144, D 6, sampling
verify), and the large single-module head (H 7168, 56/8 heads, FFN 18432, vocab 129280, B 32,
D 3, 8192-position context) on three sampled sequences.  Bar: drafts exact except where the
oracle's top-2 gap is below 1e-4, hiddens and logits within max relative error 2e-2."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, gen, make_first_round, make_kv_prefix, make_round_noise, make_weights

pytestmark = [pytest.mark.gpu]

M = pytest.importorskip("speculative_decoding_mtp_amd")
from tests.gpu_util import MARGIN, config, f32, i32, kv_from_numpy, max_rel, upload_weights  # noqa: E402

TOL = 2e-2


def _round(cfg, seqs, rounds=1):
    """Run `rounds` rounds on the GPU for the whole batch; check sequences `seqs` with the oracle."""
    w = make_weights(cfg)
    c, gw = config(cfg), upload_weights(cfg, w)
    B, D, H, V = cfg.batch, cfg.D, cfg.hidden, cfg.vocab
    max_len = M.round_max_len(cfg.ctx + rounds * (D + 1) + 8)
    K, Vv = make_kv_prefix(cfg)
    kv = kv_from_numpy(cfg, K, Vv, cfg.ctx, max_len)
    model = O.OracleModel(cfg, w)
    cache = O.KVCache(cfg, len(seqs), max_len)
    cache.load_prefix(K[:, seqs], Vv[:, seqs], cfg.ctx)
    del K, Vv
    toks, hid = make_first_round(cfg)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, B, D + 1, D, max_len))
    drafts = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    hids = torch.zeros(B, D, H, device="cuda")
    dlog = torch.zeros(B, D, V, device="cuda")
    excluded = 0
    for r in range(rounds):
        M.mtp_draft_loop(c, gw, kv, D, toks.shape[1], i32(toks), f32(hid), drafts, hids, dlog, ws)
        M.mtp_check(ws)
        d_o, h_o, l_o, m_o = O.draft_loop(model, cache, toks[seqs], hid[seqs], D)
        dg, hg, lg = drafts.cpu().numpy()[seqs], hids.cpu().numpy()[seqs], dlog.cpu().numpy()[seqs]
        assert np.array_equal(kv.len.cpu().numpy()[seqs], cache.len)
        for j in range(len(seqs)):
            for k in range(D):
                assert max_rel(hg[j, k], h_o[j, k]) < TOL, (r, j, k)
                assert max_rel(lg[j, k], l_o[j, k]) < TOL, (r, j, k)
                if m_o[j, k] < MARGIN:
                    excluded += 1
                    break
                assert dg[j, k] == d_o[j, k], (r, j, k)
        yield dict(d_o=d_o, l_o=l_o, kv=kv, cache=cache, drafts=drafts, dlog=dlog, c=c, r=r)
        # next round: a forced two-row catch-up (one accepted draft) on every sequence
        ctx = cache.len - (D - 1)
        O.kv_crop(cache, ctx)
        full_ctx = kv.len.cpu().numpy() - (D - 1)
        M.kv_crop(kv, i32(full_ctx))
        toks = np.full((B, D + 1), -1, np.int32)
        toks[:, 0] = dg[0, 0] if len(dg) else 0
        toks[:, 1] = np.arange(B) % V
        g = gen(cfg.index, 2, 500 + r)
        hid = g.standard_normal((B, D + 1, H), dtype=np.float32)
    assert excluded <= len(seqs) * rounds


def test_qwen_head_full_size():
    cfg = CONFIGS["qwen"]
    for st in _round(cfg, [0], rounds=2):
        # greedy verify of the round against target logits = oracle logits + noise
        D, V = cfg.D, cfg.vocab
        l_o = st["l_o"]
        tl = np.concatenate([l_o, l_o[:, D - 1:D]], axis=1).astype(np.float32) + make_round_noise(cfg, st["r"])
        ctx = (st["cache"].len - (D - 1)).astype(np.int32)
        vws = M.new_workspace(M.spec_verify_workspace_size(1, D, V, None))
        n = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = torch.zeros(1, D + 1, dtype=torch.int32, device="cuda")
        crop = torch.zeros(1, dtype=torch.int32, device="cuda")
        M.spec_verify(1, D, V, f32(tl), i32(st["d_o"]), None, None, None, None, i32(ctx), n, out, crop, vws)
        r = O.greedy_verify(tl, st["d_o"], ctx)
        assert np.array_equal(out.cpu().numpy(), r.out_tokens)
        assert np.array_equal(crop.cpu().numpy(), r.crop_len)


def test_four_layer_drafter_full_size_with_sampling_verify():
    cfg = CONFIGS["drafter4"]
    sp = cfg.sampling
    for st in _round(cfg, [0], rounds=1):
        D, V = cfg.D, cfg.vocab
        l_o = st["l_o"]
        tl = np.concatenate([l_o, l_o[:, D - 1:D]], axis=1).astype(np.float32) + make_round_noise(cfg, 0)
        ctx = (st["cache"].len - (D - 1)).astype(np.int32)
        g = gen(cfg.index, 6, 0)
        ua, us = g.random((1, D), dtype=np.float32), g.random(1, dtype=np.float32)
        csp = M.sampling(sp.temperature, sp.top_k, sp.top_p, sp.q_mode)
        vws = M.new_workspace(M.spec_verify_workspace_size(1, D, V, csp))
        n = torch.zeros(1, dtype=torch.int32, device="cuda")
        out = torch.zeros(1, D + 1, dtype=torch.int32, device="cuda")
        crop = torch.zeros(1, dtype=torch.int32, device="cuda")
        M.spec_verify(1, D, V, f32(tl), i32(st["d_o"]), None, csp, f32(ua), f32(us), i32(ctx), n, out, crop, vws)
        r = O.sampling_verify(tl, st["d_o"], None, sp.temperature, sp.top_k, sp.top_p, sp.q_mode, ua, us, ctx)
        if min(r.margins[0]) >= MARGIN:
            assert np.array_equal(out.cpu().numpy(), r.out_tokens)
            assert np.array_equal(crop.cpu().numpy(), r.crop_len)


@pytest.mark.timeout(600)
def test_large_single_module_head_batch32_sampled():
    cfg = CONFIGS["dsv3"]
    for st in _round(cfg, [0, 17, 31], rounds=1):
        pass
