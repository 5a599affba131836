"""Parity of the batched bf16 head -- a batch whose (sequence, kv head) pairs fill the GPU, over
caches of 1000+ positions, which takes the LDS-staged decode attention -- against the oracle.

Ragged per-sequence cache lengths (not multiples of the 64-position superslice), catch-up calls
of one to four rows per sequence (some sequences without rows), query groups of 2 and 8 per kv
head (the LDS-staged kernel with one query tile up to 16 queries per kv head, with two tiles the
catch-up of 4 rows x 8; 32 sequences x 4 kv heads take two splits and the combine), and capacities
of 1280 and 1288 positions (value rows on whole 128-byte
lines, read nontemporally, or straddling lines, read through the cache).  Every sequence's hiddens, logits and draft of
each step and the appended K/V are compared.  Bar: 2e-3 max relative error on hiddens and logits
(bf16 weights and K/V on both sides, fp32 against float64 arithmetic), K/V within one bf16 ulp,
drafts exact unless the oracle's top-2 gap is below 1e-4."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, gen, make_weights

pytestmark = pytest.mark.gpu

M = pytest.importorskip("speculative_decoding_mtp_amd")
from tests.gpu_util import MARGIN, config, f32, i32, max_rel, to_dev, upload_weights  # noqa: E402

TOL = 2e-3
KV_ULP = 2.0 ** -7


@pytest.mark.parametrize("max_len", [1280, 1288])
@pytest.mark.parametrize("nq", [8, 32])
def test_batched_head_with_ragged_caches_matches_oracle(nq, max_len):
    nkv, B, D = 4, 32, 2
    cfg = CONFIGS["tiny"].replace(index=61, wdtype="bf16", hidden=256, n_heads=nq, n_kv_heads=nkv, head_dim=128,
                                  ffn=512, vocab=2000, embed_std=1.0, batch=B, D=D)
    w = make_weights(cfg)
    model = O.OracleModel(cfg, w)
    c, gw = config(cfg), upload_weights(cfg, w)
    g = gen(61, 3, nq)
    lens = g.integers(1, 1200, size=B)
    lens[:3] = [1, 63, 1151]
    K = (g.standard_normal((1, B, nkv, max_len, 128), dtype=np.float32))
    Vv = (g.standard_normal((1, B, nkv, max_len, 128), dtype=np.float32))
    from synth import bf16_bits_to_f32, to_bf16_bits
    K = bf16_bits_to_f32(to_bf16_bits(K))
    Vv = bf16_bits_to_f32(to_bf16_bits(Vv))
    kv = M.KVCache(c, B, max_len)
    kv.k.copy_(to_dev(K, "bf16"))
    kv.v.copy_(to_dev(np.ascontiguousarray(np.swapaxes(Vv, -1, -2)), "bf16"))
    kv.len.copy_(i32(lens))
    cache = O.KVCache(cfg, B, max_len)
    cache.K[:] = K
    cache.V[:] = Vv
    cache.len[:] = lens
    rps = 4
    nrows = g.integers(0, rps + 1, size=B)
    nrows[:4] = [4, 1, 0, 3]
    toks = np.full((B, rps), -1, np.int32)
    for b in range(B):
        toks[b, :nrows[b]] = g.integers(0, cfg.vocab, size=nrows[b])
    hid = g.standard_normal((B, rps, cfg.hidden), dtype=np.float32)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, B, rps, D, max_len))
    drafts = torch.zeros(B, D, dtype=torch.int32, device="cuda")
    hids = torch.zeros(B, D, cfg.hidden, device="cuda")
    dlog = torch.zeros(B, D, cfg.vocab, device="cuda")
    M.mtp_draft_loop(c, gw, kv, D, rps, i32(toks), f32(hid), drafts, hids, dlog, ws)
    M.mtp_check(ws)
    d_o, h_o, l_o, m_o = O.draft_loop(model, cache, toks, hid, D)
    assert np.array_equal(kv.len.cpu().numpy(), cache.len)
    dg, hg, lg = drafts.cpu().numpy(), hids.cpu().numpy(), dlog.cpu().numpy()
    compared = 0
    for b in range(B):
        if nrows[b] == 0:
            assert np.all(dg[b] == -1)
            continue
        for k in range(D):
            assert max_rel(hg[b, k], h_o[b, k]) < TOL, (b, k)
            assert max_rel(lg[b, k], l_o[b, k]) < TOL, (b, k)
            if m_o[b, k] < MARGIN:
                break
            assert dg[b, k] == d_o[b, k], (b, k)
            compared += 1
        p0, p1 = int(lens[b]), int(lens[b]) + int(nrows[b])   # the catch-up rows' K/V
        kg = kv.k[0, b, :, p0:p1].float().cpu().numpy()
        vg = kv.v[0, b, :, :, p0:p1].transpose(-1, -2).float().cpu().numpy()
        for p in range(p1 - p0):
            assert max_rel(kg[:, p], cache.K[0, b, :, p0 + p]) < KV_ULP, (b, p)
            assert max_rel(vg[:, p], cache.V[0, b, :, p0 + p]) < KV_ULP, (b, p)
    assert compared >= B
