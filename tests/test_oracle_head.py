"""Pins of the oracle's MTP head and its draft calls: concat order, the shared
embedding / lm_head, row positions, catch-up bookkeeping, crop, the serial loop."""
import numpy as np
import pytest

import oracle as O
from synth import MTPConfig


def _cfg(**kw):
    base = dict(index=91, name="t", hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, ffn=40, vocab=512,
                n_layers=1, rope_theta=1e4, rms_eps=1e-6, wdtype="f32", embed_std=1.0, batch=2, D=3, ctx=0,
                prefill_rows=0, rounds=1, noise_std=1.0)
    base.update(kw)
    return MTPConfig(**base)


class _W:
    pass


def _weights(cfg, rng, identity_block=False):
    H, F = cfg.hidden, cfg.ffn
    w = _W()
    w.embed = rng.standard_normal((cfg.vocab, H))
    w.enorm = w.hnorm = w.final_norm = np.ones(H)
    w.eh_proj = rng.standard_normal((H, 2 * H)) * 0.1
    w.layers = []
    for _ in range(cfg.n_layers):
        lw = _W()
        lw.in_norm = lw.post_norm = np.ones(H)
        lw.wq = rng.standard_normal((cfg.q_dim, H)) * 0.2
        lw.wk = rng.standard_normal((cfg.kv_dim, H)) * 0.2
        lw.wv = rng.standard_normal((cfg.kv_dim, H)) * 0.2
        lw.wo = np.zeros((H, cfg.q_dim)) if identity_block else rng.standard_normal((H, cfg.q_dim)) * 0.1
        lw.wgate = rng.standard_normal((F, H)) * 0.2
        lw.wup = rng.standard_normal((F, H)) * 0.2
        lw.wdown = np.zeros((H, F)) if identity_block else rng.standard_normal((H, F)) * 0.1
        w.layers.append(lw)
    w.lm_head = rng.standard_normal((cfg.vocab, H))
    return w


def test_copy_head_reads_the_embedding_half_first():
    # eh_proj = [I 0], an identity block and lm_head = the embedding table: the head
    # must return the token it was given.  With [0 I] and the hidden set to E[j] it
    # must return j.  A swapped concat order fails both.
    cfg = _cfg()
    rng = np.random.default_rng(11)
    w = _weights(cfg, rng, identity_block=True)
    H = cfg.hidden
    w.lm_head = w.embed
    w.eh_proj = np.concatenate([np.eye(H), np.zeros((H, H))], axis=1)
    m = O.OracleModel(cfg, w)
    for tok in [0, 7, 300, 511]:
        _, d, _, _ = O.mtp_row(m, O.KVCache(cfg, 1, 4), 0, tok, rng.standard_normal(H), 2)
        assert d == tok
    w.eh_proj = np.concatenate([np.zeros((H, H)), np.eye(H)], axis=1)
    m = O.OracleModel(cfg, w)
    for j in [3, 100, 499]:
        _, d, _, _ = O.mtp_row(m, O.KVCache(cfg, 1, 4), 0, 5, w.embed[j] * 3.0, 2)
        assert d == j


def test_head_output_is_the_final_norm_and_feeds_lm_head():
    cfg = _cfg()
    rng = np.random.default_rng(12)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    g, d, logits, margin = O.mtp_row(m, O.KVCache(cfg, 1, 4), 0, 9, rng.standard_normal(cfg.hidden), 1)
    assert abs(np.mean(g * g) - 1.0) < 1e-5                # unit RMS after the final norm (gain 1)
    np.testing.assert_allclose(logits, m.lm_head @ g, atol=1e-12)
    assert d == int(np.argmax(logits)) and margin > 0


def test_catch_up_rows_equal_single_row_calls_and_set_lengths():
    cfg = _cfg(n_layers=2)
    rng = np.random.default_rng(13)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    H = cfg.hidden
    toks = np.array([[5, 6, 7], [8, 9, -1]])               # sequence 1 has a padded third row
    hid = rng.standard_normal((2, 3, H))
    c1 = O.KVCache(cfg, 2, 16)
    c1.len[:] = [4, 2]
    pre = rng.standard_normal(c1.K.shape).astype(np.float32)
    c1.K[:], c1.V[:] = pre, pre * 0.5
    c2 = O.KVCache(cfg, 2, 16)
    c2.K[:], c2.V[:], c2.len[:] = c1.K, c1.V, c1.len
    h1, d1, l1, _ = O.draft_step(m, c1, toks, hid)
    assert list(c1.len) == [7, 4]
    assert not np.any(h1[1, 2])
    for i in range(3):
        t = toks[:, i:i + 1]                                # [[7], [-1]] on the last call
        h2, d2, l2, _ = O.draft_step(m, c2, t, hid[:, i:i + 1])
        for b in range(2):
            if toks[b, i] >= 0:
                np.testing.assert_array_equal(h1[b, i], h2[b, 0])
    assert list(c2.len) == [7, 4]
    np.testing.assert_array_equal(c1.K, c2.K)
    np.testing.assert_array_equal(d1, [O.argmax_lowest(l1[0])[0], O.argmax_lowest(l1[1])[0]])


def test_crop_makes_later_rows_ignore_stale_entries():
    cfg = _cfg(batch=1)
    rng = np.random.default_rng(14)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    H = cfg.hidden
    hid = rng.standard_normal((1, 6, H))
    fresh = O.KVCache(cfg, 1, 16)
    O.draft_step(m, fresh, np.array([[1, 2, 3]]), hid[:, :3])
    g_ref, d_ref, _, _ = O.draft_step(m, fresh, np.array([[4]]), hid[:, 5:6])
    dirty = O.KVCache(cfg, 1, 16)
    O.draft_step(m, dirty, np.array([[1, 2, 3, 10, 11]]), hid[:, :5])   # two rows later rolled back
    O.kv_crop(dirty, [3])
    g, d, _, _ = O.draft_step(m, dirty, np.array([[4]]), hid[:, 5:6])
    np.testing.assert_array_equal(g, g_ref)
    assert d[0] == d_ref[0]


def test_draft_loop_feeds_back_its_own_draft_and_hidden_one_position_later():
    cfg = _cfg(batch=1, n_layers=2)
    rng = np.random.default_rng(15)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    H = cfg.hidden
    toks, hid = np.array([[3, 4]]), rng.standard_normal((1, 2, H))
    ca = O.KVCache(cfg, 1, 32)
    ca.len[:] = 5
    drafts, hs, logits, _ = O.draft_loop(m, ca, toks, hid, 4)
    assert ca.len[0] == 5 + 2 + 3
    cb = O.KVCache(cfg, 1, 32)
    cb.len[:] = 5
    hout, d, _, _ = O.draft_step(m, cb, toks, hid)
    assert d[0] == drafts[0, 0]
    np.testing.assert_array_equal(hout[0, 1], hs[0, 0])
    g = hout[0, 1]
    for k in range(1, 4):
        g2, dk, lk, _ = O.mtp_row(m, cb, 0, int(drafts[0, k - 1]), g, 5 + 2 + k - 1)
        assert dk == drafts[0, k]
        np.testing.assert_array_equal(g2, hs[0, k])
        np.testing.assert_array_equal(lk, logits[0, k])
        g = g2


def test_capacity_and_token_range_errors():
    cfg = _cfg(batch=1)
    m = O.OracleModel(cfg, _weights(cfg, np.random.default_rng(16)))
    c = O.KVCache(cfg, 1, 3)
    with pytest.raises(IndexError):
        O.draft_step(m, c, np.array([[1, 2, 3, 4]]), np.zeros((1, 4, cfg.hidden)))
    with pytest.raises(IndexError):
        O.draft_step(m, O.KVCache(cfg, 1, 3), np.array([[cfg.vocab]]), np.zeros((1, 1, cfg.hidden)))
