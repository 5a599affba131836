"""Pins of the oracle's head that keeps no cache of its own and reads the main model's keys and
values ([DLM "MTP speculative decoding"] item 1): equality with the own-cache head where the two
must agree, the layer map, read-only use of the main model's cache, the row positions and the
feeding of the serial steps, and a closed form of the attention over the main model's keys."""
import math

import numpy as np
import pytest

import oracle as O
from synth import MTPConfig


def _cfg(**kw):
    base = dict(index=92, name="t", hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, ffn=40, vocab=512,
                n_layers=2, rope_theta=1e4, rms_eps=1e-6, wdtype="f32", embed_std=1.0, batch=2, D=3, ctx=0,
                prefill_rows=0, rounds=1, noise_std=1.0)
    base.update(kw)
    return MTPConfig(**base)


class _W:
    pass


def _weights(cfg, rng):
    H, F = cfg.hidden, cfg.ffn
    w = _W()
    w.embed = rng.standard_normal((cfg.vocab, H))
    w.enorm = w.hnorm = w.final_norm = np.ones(H)
    w.eh_proj = rng.standard_normal((H, 2 * H)) * 0.1
    w.layers = []
    for _ in range(cfg.n_layers):
        lw = _W()
        lw.in_norm = lw.post_norm = np.ones(H)
        lw.wq = rng.standard_normal((cfg.q_dim, H)) * 0.3
        lw.wk = rng.standard_normal((cfg.kv_dim, H)) * 0.3
        lw.wv = rng.standard_normal((cfg.kv_dim, H)) * 0.3
        lw.wo = rng.standard_normal((H, cfg.q_dim)) * 0.1
        lw.wgate = rng.standard_normal((F, H)) * 0.2
        lw.wup = rng.standard_normal((F, H)) * 0.2
        lw.wdown = rng.standard_normal((H, F)) * 0.1
        w.layers.append(lw)
    w.lm_head = rng.standard_normal((cfg.vocab, H))
    return w


def _filled_cache(cfg, model, rng, n, B=1, max_len=32):
    """An own-cache head's cache after a prefill of n rows per sequence, and that call's outputs."""
    cache = O.KVCache(cfg, B, max_len)
    toks = rng.integers(0, cfg.vocab, size=(B, n))
    hid = rng.standard_normal((B, n, cfg.hidden))
    hout, d, lg, _ = O.draft_step(model, cache, toks, hid)
    return cache, toks, hid, hout, d, lg


def test_first_step_equals_the_own_cache_heads_last_row():
    # The own-cache head's last prefill row at position n-1 attends over positions 0..n-1 of its
    # cache, its own K/V included.  A head that reads that same cache (identity layer map) at
    # position n-1 sees exactly those keys and values: the first step must agree bit for bit.
    cfg = _cfg()
    rng = np.random.default_rng(21)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    n = 9
    cache, toks, hid, hout, d, lg = _filled_cache(cfg, m, rng, n)
    drafts, hs, logits, _ = O.draft_loop_shared(m, cache, [0, 1], toks[:, -1], hid[:, -1], 1)
    assert drafts[0, 0] == d[0]
    np.testing.assert_array_equal(hs[0, 0], hout[0, n - 1])
    np.testing.assert_array_equal(logits[0, 0], lg[0])


def test_head_layer_l_reads_main_model_layer_map_l():
    # Swapping the two layers of the main model's cache and the map together changes nothing;
    # swapping only the cache changes the result.
    cfg = _cfg(batch=1)
    rng = np.random.default_rng(22)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    cache, toks, hid, *_ = _filled_cache(cfg, m, rng, 7)
    swapped = O.KVCache(cfg, 1, cache.max_len)
    swapped.K[:], swapped.V[:] = cache.K[::-1], cache.V[::-1]
    swapped.len[:] = cache.len
    a = O.draft_loop_shared(m, cache, [0, 1], toks[:, -1], hid[:, -1], 2)
    b = O.draft_loop_shared(m, swapped, [1, 0], toks[:, -1], hid[:, -1], 2)
    c = O.draft_loop_shared(m, swapped, [0, 1], toks[:, -1], hid[:, -1], 2)
    np.testing.assert_array_equal(a[1], b[1])
    assert not np.allclose(a[1], c[1])
    # both head layers may read one main-model layer
    d = O.draft_loop_shared(m, cache, [1, 1], toks[:, -1], hid[:, -1], 1)
    e = O.draft_loop_shared(m, swapped, [0, 0], toks[:, -1], hid[:, -1], 1)
    np.testing.assert_array_equal(d[1], e[1])


def test_main_model_cache_is_read_only_and_only_its_valid_prefix_is_seen():
    cfg = _cfg(batch=1)
    rng = np.random.default_rng(23)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    cache, toks, hid, *_ = _filled_cache(cfg, m, rng, 6)
    K0, V0, len0 = cache.K.copy(), cache.V.copy(), cache.len.copy()
    a = O.draft_loop_shared(m, cache, [0, 1], toks[:, -1], hid[:, -1], 3)
    np.testing.assert_array_equal(cache.K, K0)
    np.testing.assert_array_equal(cache.V, V0)
    np.testing.assert_array_equal(cache.len, len0)
    cache.K[:, :, :, 6:] = 50.0       # slots at and past len: stale, never read
    cache.V[:, :, :, 6:] = -50.0
    b = O.draft_loop_shared(m, cache, [0, 1], toks[:, -1], hid[:, -1], 3)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_rows_sit_at_len_minus_one_plus_k_and_feed_back_draft_and_hidden(monkeypatch):
    cfg = _cfg()
    rng = np.random.default_rng(24)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    cache = O.KVCache(cfg, 2, 32)
    cache.K[:] = rng.standard_normal(cache.K.shape).astype(np.float32)
    cache.V[:] = rng.standard_normal(cache.V.shape).astype(np.float32)
    cache.len[:] = [5, 11]
    toks = np.array([3, 400])
    hid = rng.standard_normal((2, cfg.hidden))
    calls = []
    orig = O.mtp_row_shared

    def spy(model, tc, kvl, b, tok, hidden, pos):
        out = orig(model, tc, kvl, b, tok, hidden, pos)
        calls.append((b, tok, np.array(hidden), pos, out))
        return out

    monkeypatch.setattr(O, "mtp_row_shared", spy)
    import oracle.mtp as OM
    monkeypatch.setattr(OM, "mtp_row_shared", spy)
    drafts, hs, _, _ = O.draft_loop_shared(m, cache, [0, 1], toks, hid, 4)
    assert [(c[0], c[3]) for c in calls] == [(0, 4), (0, 5), (0, 6), (0, 7), (1, 10), (1, 11), (1, 12), (1, 13)]
    for b in range(2):
        mine = [c for c in calls if c[0] == b]
        assert mine[0][1] == toks[b]
        np.testing.assert_array_equal(mine[0][2], hid[b])
        for k in range(1, 4):
            assert mine[k][1] == drafts[b, k - 1]
            np.testing.assert_array_equal(mine[k][2], hs[b, k - 1])
    np.testing.assert_array_equal(cache.len, [5, 11])


def test_sequences_without_a_token_or_a_cache_get_no_drafts():
    cfg = _cfg(batch=3)
    rng = np.random.default_rng(25)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    cache = O.KVCache(cfg, 3, 16)
    cache.K[:] = rng.standard_normal(cache.K.shape).astype(np.float32)
    cache.V[:] = rng.standard_normal(cache.V.shape).astype(np.float32)
    cache.len[:] = [4, 0, 4]
    drafts, hs, logits, _ = O.draft_loop_shared(m, cache, [0, 1], np.array([7, 7, -1]),
                                                rng.standard_normal((3, cfg.hidden)), 2)
    assert (drafts[0] >= 0).all()
    assert (drafts[1:] == -1).all()
    assert not hs[1:].any() and not logits[1:].any()
    with pytest.raises(IndexError):
        O.draft_loop_shared(m, cache, [0, 1], np.array([cfg.vocab, -1, -1]),
                            rng.standard_normal((3, cfg.hidden)), 1)


def test_block_attention_over_two_main_model_keys_closed_form():
    # One query head of size 2, W_q = I, no MLP: q is the rotated unit-RMS input.  Key 0 is zero
    # (score 0), key 1 is c; the output mixes the two values by sigmoid(s1), s1 = (R_pos q).c / sqrt 2.
    cfg = _cfg(hidden=2, n_heads=1, n_kv_heads=1, head_dim=2, ffn=1, n_layers=1, batch=1)
    lw = _W()
    lw.in_norm = lw.post_norm = np.ones(2)
    lw.wq = np.eye(2)
    lw.wk = lw.wv = np.zeros((2, 2))
    lw.wo = np.eye(2)
    lw.wgate, lw.wup, lw.wdown = np.zeros((1, 2)), np.zeros((1, 2)), np.zeros((2, 1))
    w = _W()
    w.embed = np.zeros((cfg.vocab, 2))
    w.enorm = w.hnorm = w.final_norm = np.ones(2)
    w.eh_proj = np.zeros((2, 4))
    w.layers = [lw]
    w.lm_head = np.zeros((cfg.vocab, 2))
    m = O.OracleModel(cfg, w)
    cache = O.KVCache(cfg, 1, 8)
    c = np.array([1.5, -0.5])
    v0, v1 = np.array([2.0, 0.0]), np.array([0.0, -4.0])
    cache.K[0, 0, 0, 1], cache.V[0, 0, 0, 0], cache.V[0, 0, 0, 1] = c, v0, v1
    cache.len[:] = 2
    x = np.array([0.3, 1.1])
    for pos in [1, 2, 5]:
        y = O.shared_block(m, 0, cache, 0, 0, x, pos)
        a = x / math.sqrt(np.mean(x * x) + cfg.rms_eps)
        th = float(pos)                                      # head_dim 2: one pair, frequency 1
        q = np.array([a[0] * math.cos(th) - a[1] * math.sin(th), a[1] * math.cos(th) + a[0] * math.sin(th)])
        s1 = q @ c / math.sqrt(2.0)
        p1 = 1.0 / (1.0 + math.exp(-s1))
        np.testing.assert_allclose(y, x + (1 - p1) * v0 + p1 * v1, rtol=0, atol=1e-12)
    cache.len[:] = 0                                          # empty: zero attention output
    np.testing.assert_allclose(O.shared_block(m, 0, cache, 0, 0, x, 3), x, atol=0)
