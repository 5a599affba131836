"""MTP prefill at prompt length ([HB14 "The draft head"]: after the main model's prefill the head
runs over the whole prompt, each position paired with its next token): thousands of rows in one
mtp_draft_step call, through the MFMA GEMM path in 128-row passes and causal multi-query
attention.

* parity with the oracle on a small bf16 head at 2048 rows: every row's K/V (up to rare one-ulp
  flips of bf16 rounding), the hiddens of sampled rows and the last row's logits and draft;
* at the 2048-hidden head's full size: one 2048-row call equals two 1024-row calls (the same
  cache, hiddens and draft), a property that holds at any size.

bf16 bar: max relative error 1e-3 on hiddens and logits (bf16 weights on both sides, fp32 against
float64 arithmetic; measured at most 9e-6, printed by each case)."""
import numpy as np
import pytest
import torch

import oracle as O
from synth import CONFIGS, make_prefill, make_weights

pytestmark = pytest.mark.gpu

M = pytest.importorskip("speculative_decoding_mtp_amd")
from tests.gpu_util import MARGIN, config, f32, i32, max_rel, upload_weights  # noqa: E402

TOL = 1e-3  # bf16 weights on both sides, fp32 against float64 arithmetic (measured <= 9e-6)


def _prefill(c, gw, kv, toks, hid, ws):
    B, R = toks.shape
    H = hid.shape[-1]
    hout = torch.zeros(B, R, H, device="cuda")
    draft = torch.zeros(B, dtype=torch.int32, device="cuda")
    logits = torch.zeros(B, c.vocab, device="cuda")
    M.mtp_draft_step(c, gw, kv, R, i32(toks), f32(hid), hout, draft, logits, ws)
    M.mtp_check(ws)
    return hout, draft, logits


def test_prefill_2048_rows_matches_oracle():
    cfg = CONFIGS["tiny"].replace(index=41, wdtype="bf16", n_heads=4, n_kv_heads=2, head_dim=128, hidden=256,
                                  ffn=512, vocab=3000, embed_std=1.0, prefill_rows=2048)
    w = make_weights(cfg)
    model = O.OracleModel(cfg, w)
    c, gw = config(cfg), upload_weights(cfg, w)
    toks, hid = make_prefill(cfg)
    R = toks.shape[1]
    max_len = M.round_max_len(R + 8)
    kv = M.KVCache(c, 1, max_len)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, 1, R, 1, max_len))
    hout, draft, logits = _prefill(c, gw, kv, toks, hid, ws)
    cache = O.KVCache(cfg, 1, max_len)
    h_o, d_o, l_o, m_o = O.draft_step(model, cache, toks, hid)
    assert int(kv.len[0]) == R == cache.len[0]
    ulp = 2.0 ** -7
    assert max_rel(kv.k[..., :R, :].float().cpu().numpy(), cache.K[..., :R, :]) < ulp
    assert max_rel(kv.v[..., :R].transpose(-1, -2).float().cpu().numpy(), cache.V[..., :R, :]) < ulp
    rows = list(range(0, R, 61)) + list(range(R - 8, R))
    hg = hout.cpu().numpy()
    eh = max(max_rel(hg[0, i], h_o[0, i]) for i in rows)
    el = max_rel(logits.cpu().numpy(), l_o)
    print("prefill 2048 rows: hidden", eh, "logits", el, flush=True)
    assert eh < TOL and el < TOL, (eh, el)
    if m_o[0] >= MARGIN:
        assert int(draft[0]) == d_o[0]


def test_prefill_in_one_call_equals_two_calls_at_full_size():
    cfg = CONFIGS["qwen"]
    w = make_weights(cfg)
    c, gw = config(cfg), upload_weights(cfg, w)
    R = 2048
    toks, hid = make_prefill(cfg, R)
    max_len = M.round_max_len(R + 8)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, 1, R, 1, max_len))
    kv1 = M.KVCache(c, 1, max_len)
    h1, d1, l1 = _prefill(c, gw, kv1, toks, hid, ws)
    kv2 = M.KVCache(c, 1, max_len)
    half = R // 2
    ha, _, _ = _prefill(c, gw, kv2, toks[:, :half], hid[:, :half], ws)
    hb, d2, l2 = _prefill(c, gw, kv2, toks[:, half:], hid[:, half:], ws)
    assert int(kv1.len[0]) == int(kv2.len[0]) == R
    # the same arithmetic per row except the attention split and pass boundaries: fp32 rounding
    ulp = 2.0 ** -7
    assert max_rel(kv1.k[..., :R, :].float().cpu().numpy(), kv2.k[..., :R, :].float().cpu().numpy()) < ulp
    assert max_rel(kv1.v[..., :R].float().cpu().numpy(), kv2.v[..., :R].float().cpu().numpy()) < ulp
    h2 = torch.cat([ha, hb], dim=1)
    assert max_rel(h1.cpu().numpy(), h2.cpu().numpy()) < 1e-3
    assert max_rel(l1.cpu().numpy(), l2.cpu().numpy()) < 1e-3
    top = torch.topk(l1[0], 2).values
    if float(top[0] - top[1]) >= MARGIN:
        assert int(d1[0]) == int(d2[0])


@pytest.mark.parametrize("wdtype", ["f32", "bf16"])
def test_ragged_batched_prefill_matches_oracle(wdtype):
    """Three sequences in one 40-row call, more rows per sequence than the kernels count inline
    (the per-call row-count pass): 40, 23 and 1 valid rows, the rest padded with -1, over caches
    that already hold 0, 5 and 17 positions."""
    cfg = CONFIGS["tiny"].replace(index=43, wdtype=wdtype, batch=3, prefill_rows=40)
    w = make_weights(cfg)
    model = O.OracleModel(cfg, w)
    c, gw = config(cfg), upload_weights(cfg, w)
    toks, hid = make_prefill(cfg)
    n = [40, 23, 1]
    for b in range(3):
        toks[b, n[b]:] = -1
    start = [0, 5, 17]
    max_len = M.round_max_len(64)
    kv = M.KVCache(c, 3, max_len)
    cache = O.KVCache(cfg, 3, max_len)
    pre_t, pre_h = make_prefill(cfg.replace(index=44), 17)
    for b in range(3):  # the cache prefixes: earlier one-sequence prefills
        pt = np.full((3, 17), -1, np.int32)
        pt[b, :start[b]] = pre_t[b, :start[b]]
        if start[b]:
            _prefill(c, gw, kv, pt, pre_h, M.new_workspace(M.mtp_draft_workspace_size(c, 3, 17, 1, max_len)))
            O.draft_step(model, cache, pt, pre_h)
    assert kv.len.cpu().tolist() == start
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, 3, 40, 1, max_len))
    hout, draft, logits = _prefill(c, gw, kv, toks, hid, ws)
    h_o, d_o, l_o, m_o = O.draft_step(model, cache, toks, hid)
    assert kv.len.cpu().tolist() == list(cache.len) == [s + k for s, k in zip(start, n)]
    tol, ktol = (1e-4, 1e-5) if wdtype == "f32" else (TOL, 2.0 ** -7)
    hg, lg, dg = hout.cpu().numpy(), logits.cpu().numpy(), draft.cpu().numpy()
    for b in range(3):
        T = start[b] + n[b]
        assert max_rel(kv.k[:, b, :, :T].float().cpu().numpy(), cache.K[:, b, :, :T]) < ktol, b
        assert max_rel(kv.v[:, b, ..., :T].transpose(-1, -2).float().cpu().numpy(), cache.V[:, b, :, :T]) < ktol, b
        eh, el = max_rel(hg[b, :n[b]], h_o[b, :n[b]]), max_rel(lg[b], l_o[b])
        print("ragged prefill", wdtype, b, "hidden", eh, "logits", el, flush=True)
        assert eh < tol and el < tol, (b, eh, el)
        if m_o[b] >= MARGIN:
            assert dg[b] == d_o[b], b


@pytest.mark.parametrize("case", ["capacity", "token"])
def test_many_row_call_reports_errors(case):
    """The device error flags of a 24-row call come from the per-call row count: a sequence that
    outgrows its cache keeps the rows that fit, a token outside the vocabulary ends its rows."""
    cfg = CONFIGS["tiny"].replace(batch=2)
    c, gw = config(cfg), upload_weights(cfg, make_weights(cfg))
    kv = M.KVCache(c, 2, 32)
    toks = np.arange(48, dtype=np.int32).reshape(2, 24)
    toks[1, 10:] = -1
    if case == "capacity":
        kv.len.copy_(i32([16, 0]))
        want, code = [32, 10], -4
    else:
        toks[0, 20] = cfg.vocab
        want, code = [20, 10], -7
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, 2, 24, 1, 32))
    hid = torch.randn(2, 24, cfg.hidden, device="cuda")
    d = torch.zeros(2, dtype=torch.int32, device="cuda")
    M.mtp_draft_step(c, gw, kv, 24, i32(toks), hid, torch.zeros_like(hid), d, None, ws)
    with pytest.raises(M.MTPError) as e:
        M.mtp_check(ws)
    assert e.value.code == code
    assert kv.len.cpu().tolist() == want


def test_prefill_one_split_attention_ragged_with_prefix():
    """Calls with more than 4096 query rows per kv head take one split and the prefill attention
    (query blocks over the waves, K/V tiles in LDS): 8 query heads on one kv head at 640 rows per
    sequence, two sequences with 640 and 517 valid rows, after a 40-row call that left 37 and 20
    positions in the caches (so the causal windows start past position 0 and differ per
    sequence, and the last tiles are partial).  Every valid row's hidden and K/V, the logits and
    the drafts against the oracle's two draft_step calls."""
    cfg = CONFIGS["tiny"].replace(index=43, wdtype="bf16", n_heads=8, n_kv_heads=1, head_dim=128, hidden=256,
                                  ffn=512, vocab=3000, embed_std=1.0, batch=2, prefill_rows=0)
    w = make_weights(cfg)
    model = O.OracleModel(cfg, w)
    c, gw = config(cfg), upload_weights(cfg, w)
    rng = np.random.default_rng(cfg.index)
    B, H = 2, cfg.hidden
    max_len = M.round_max_len(640 + 40 + 8)
    kv = M.KVCache(c, B, max_len)
    cache = O.KVCache(cfg, B, max_len)
    ws = M.new_workspace(M.mtp_draft_workspace_size(c, B, 640, 1, max_len))
    ulp = 2.0 ** -7
    for rows, valid in ((40, [37, 20]), (640, [640, 517])):
        toks = rng.integers(0, cfg.vocab, size=(B, rows)).astype(np.int32)
        for b, n in enumerate(valid):
            toks[b, n:] = -1
        hid = rng.standard_normal((B, rows, H)).astype(np.float32)
        hout, draft, logits = _prefill(c, gw, kv, toks, hid, ws)
        h_o, d_o, l_o, m_o = O.draft_step(model, cache, toks, hid)
        assert kv.len.cpu().tolist() == cache.len.tolist()
        hg, lg = hout.cpu().numpy(), logits.cpu().numpy()
        for b, n in enumerate(valid):
            eh = max(max_rel(hg[b, i], h_o[b, i]) for i in range(n))
            el = max_rel(lg[b], l_o[b])
            print("one-split prefill", rows, b, "hidden", eh, "logits", el, flush=True)
            assert eh < TOL and el < TOL, (rows, b, eh, el)
            if m_o[b] >= MARGIN:
                assert int(draft[b]) == d_o[b], (rows, b)
    L = cache.len.tolist()
    kg = kv.k.float().cpu().numpy()
    vg = kv.v.transpose(-1, -2).float().cpu().numpy()
    for b in range(B):
        assert max_rel(kg[:, b, :, :L[b]], cache.K[:, b, :, :L[b]]) < ulp, b
        assert max_rel(vg[:, b, :, :L[b]], cache.V[:, b, :, :L[b]]) < ulp, b
