"""Full-size parity of the two widened draft loops, in the launch configuration bench.py uses, on
sampled outputs the oracle computes one by one:

* mtp_draft_loop_shared_kv at the 4-layer drafter's size (H 1024, 8/2 heads, FFN 4096, vocab
  262144, D 6) reading a 2-layer main-model cache of 2048 positions, head layer l -> layer l mod 2;
* mtp_draft_loop_multi with three modules at the large head's size (H 7168, 56/8 heads, FFN 18432,
  vocab 129280, B 32, D 3, 8192-position caches), three sampled sequences.

Bar: drafts exact except where the oracle's top-2 gap is below 1e-4 (later steps of that sequence
are then not compared), hiddens and logits within max relative error 2e-3, lengths exact."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, make_first_round, make_kv_prefix, make_weights

pytestmark = [pytest.mark.gpu]

M = pytest.importorskip("speculative_decoding_mtp_amd")
from tests.gpu_util import MARGIN, config, f32, i32, kv_from_numpy, max_rel, to_dev, upload_weights  # noqa: E402

TOL = 2e-3


def _compare(dg, hg, lg, d_o, h_o, l_o, m_o):
    compared = 0
    for j in range(d_o.shape[0]):
        for k in range(d_o.shape[1]):
            assert max_rel(hg[j, k], h_o[j, k]) < TOL, (j, k)
            assert max_rel(lg[j, k], l_o[j, k]) < TOL, (j, k)
            if m_o[j, k] < MARGIN:
                break
            assert dg[j, k] == d_o[j, k], (j, k)
            compared += 1
    return compared


@pytest.mark.timeout(600)
def test_shared_kv_drafter_full_size():
    cfg = CONFIGS["drafter4"]
    B, D, H, V, T = cfg.batch, cfg.D, cfg.hidden, cfg.vocab, 2
    w = make_weights(cfg)
    c, gw = config(cfg), upload_weights(cfg, w)
    model = O.OracleModel(cfg, w)
    max_len = M.round_max_len(cfg.ctx + 1 + 64)
    tcfg = cfg.replace(n_layers=T, index=cfg.index + 50)
    K, Vv = make_kv_prefix(tcfg, cfg.ctx + 1)
    kv = M.KVCache(c, B, max_len, n_layers=T)
    kv.k[:, :, :, :cfg.ctx + 1] = to_dev(K, cfg.wdtype)
    kv.v[:, :, :, :, :cfg.ctx + 1] = to_dev(np.ascontiguousarray(np.swapaxes(Vv, -1, -2)), cfg.wdtype)
    kv.len.fill_(cfg.ctx + 1)
    ref = O.KVCache(tcfg, B, max_len)
    ref.load_prefix(K, Vv, cfg.ctx + 1)
    del K, Vv
    kv_layer = [l % T for l in range(cfg.n_layers)]
    toks, hid = make_first_round(cfg)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, B, 1, D, max_len))
    drafts = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    hids = torch.zeros(B, D, H, device="cuda")
    dlog = torch.zeros(B, D, V, device="cuda")
    M.mtp_draft_loop_shared_kv(c, gw, kv, kv_layer, D, i32(toks[:, 0]), f32(hid[:, 0]), drafts, hids, dlog, ws)
    M.mtp_check(ws)
    d_o, h_o, l_o, m_o = O.draft_loop_shared(model, ref, kv_layer, toks[:, 0], hid[:, 0], D)
    assert kv.len.cpu().tolist() == [cfg.ctx + 1] * B
    assert _compare(drafts.cpu().numpy(), hids.cpu().numpy(), dlog.cpu().numpy(), d_o, h_o, l_o, m_o) >= 1


def _rotated(w, m):
    """Module m: module 0's matrices with their rows rotated by m (distinct weights, no new draws);
    gains, embedding and lm_head shared."""
    import copy
    r = copy.copy(w)
    r.eh_proj = np.roll(w.eh_proj, m, axis=0)
    r.layers = []
    for lw in w.layers:
        nl = copy.copy(lw)
        for name in ("wq", "wk", "wv", "wo", "wgate", "wup", "wdown"):
            setattr(nl, name, np.roll(getattr(lw, name), m, axis=0))
        r.layers.append(nl)
    return r


@pytest.mark.timeout(900)
def test_three_modules_large_head_batch32_sampled():
    cfg = CONFIGS["dsv3"]
    Mm, seqs = 3, [0, 17, 31]
    B, D, H, V = cfg.batch, cfg.D, cfg.hidden, cfg.vocab
    c = config(cfg)
    w0 = make_weights(cfg)
    # the oracle converts weights to float64: convert the shared tables once
    w0.embed, w0.lm_head = w0.embed.astype(np.float64), w0.lm_head.astype(np.float64)
    ws_ = [w0] + [_rotated(w0, m) for m in range(1, Mm)]
    gws = [upload_weights(cfg, w) for w in ws_]
    max_len = M.round_max_len(cfg.ctx + 1 + 2 * (D + 1) + 64)
    kvs, caches = [], []
    for m in range(Mm):
        K, Vv = make_kv_prefix(cfg.replace(index=cfg.index + 100 * m))
        kvs.append(kv_from_numpy(cfg, K, Vv, cfg.ctx, max_len))
        oc = O.KVCache(cfg, len(seqs), max_len)
        oc.load_prefix(K[:, seqs], Vv[:, seqs], cfg.ctx)
        caches.append(oc)
        del K, Vv
    models = [O.OracleModel(cfg, w) for w in ws_]
    toks, hid = make_first_round(cfg)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, B, max(D + 1, D - 1), D, max_len))
    drafts = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    hids = torch.zeros(B, D, H, device="cuda")
    dlog = torch.zeros(B, D, V, device="cuda")
    M.mtp_draft_loop_multi(c, gws, kvs, D, toks.shape[1], i32(toks), f32(hid), drafts, hids, dlog, ws)
    M.mtp_check(ws)
    d_o, h_o, l_o, m_o = O.draft_loop_multi(models, caches, toks[seqs], hid[seqs], D)
    for m in range(Mm):
        assert np.array_equal(kvs[m].len.cpu().numpy()[seqs], caches[m].len), m
    got = _compare(drafts.cpu().numpy()[seqs], hids.cpu().numpy()[seqs], dlog.cpu().numpy()[seqs], d_o, h_o, l_o, m_o)
    assert got >= len(seqs)
