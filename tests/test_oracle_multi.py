"""Pins of the oracle's multi-module draft loop ([YL 二.3, 五]): one module reproduces the
single-module loop, identical modules reproduce it too (every module's cache included), step k is
drafted by module (k-1) mod M, each module holds every row of the chain it is asked about, and a
crop plus the next catch-up removes the rows of rejected drafts."""
import numpy as np
import pytest

import oracle as O
from synth import MTPConfig


def _cfg(**kw):
    base = dict(index=93, name="t", hidden=64, n_heads=4, n_kv_heads=2, head_dim=16, ffn=40, vocab=512,
                n_layers=1, rope_theta=1e4, rms_eps=1e-6, wdtype="f32", embed_std=1.0, batch=3, D=5, ctx=0,
                prefill_rows=0, rounds=1, noise_std=1.0)
    base.update(kw)
    return MTPConfig(**base)


class _W:
    pass


def _weights(cfg, rng, embed=None, lm_head=None):
    H, F = cfg.hidden, cfg.ffn
    w = _W()
    w.embed = rng.standard_normal((cfg.vocab, H)) if embed is None else embed
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
    w.lm_head = rng.standard_normal((cfg.vocab, H)) if lm_head is None else lm_head
    return w


def _prefilled(cfg, model, rng, T=6):
    cache = O.KVCache(cfg, cfg.batch, 64)
    O.draft_step(model, cache, rng.integers(0, cfg.vocab, size=(cfg.batch, T)),
                 rng.standard_normal((cfg.batch, T, cfg.hidden)))
    return cache


def _copy(cache):
    c = O.KVCache(cache.cfg, cache.len.shape[0], cache.max_len)
    c.K[:], c.V[:], c.len[:] = cache.K, cache.V, cache.len
    return c


def _catch_up(cfg, rng):
    toks = rng.integers(0, cfg.vocab, size=(cfg.batch, 3))
    toks[1, 1:] = -1                     # one sequence with a single catch-up row
    return toks, rng.standard_normal((cfg.batch, 3, cfg.hidden))


@pytest.mark.parametrize("M", [1, 2, 3, 5])
def test_identical_modules_reproduce_the_single_module_loop(M):
    cfg = _cfg()
    rng = np.random.default_rng(31)
    m = O.OracleModel(cfg, _weights(cfg, rng))
    base = _prefilled(cfg, m, rng)
    toks, hid = _catch_up(cfg, rng)
    single = _copy(base)
    ref = O.draft_loop(m, single, toks, hid, cfg.D)
    caches = [_copy(base) for _ in range(M)]
    got = O.draft_loop_multi([m] * M, caches, toks, hid, cfg.D)
    for a, b in zip(ref, got):
        np.testing.assert_array_equal(a, b)
    # module (k-1) mod M last drafted step k; its cache holds every row up to that step's
    last = [max(k for k in range(1, cfg.D + 1) if (k - 1) % M == j) if j < min(M, cfg.D) else 1 for j in range(M)]
    for j, c in enumerate(caches):
        L = c.len - (cfg.D - last[j])
        assert (c.len == single.len - (cfg.D - last[j])).all()
        for b in range(cfg.batch):
            np.testing.assert_array_equal(c.K[:, b, :, :L[b]], single.K[:, b, :, :L[b]])
            np.testing.assert_array_equal(c.V[:, b, :, :L[b]], single.V[:, b, :, :L[b]])


def test_step_k_is_drafted_by_module_k_minus_1_mod_M():
    # Module j maps token t to perm_j(t): one-hot embeddings (V <= H) shared by all modules,
    # eh_proj = [P_j 0], blocks that add nothing, lm_head = the embedding table.
    cfg = _cfg(vocab=48, batch=1, D=5)
    H, V = cfg.hidden, cfg.vocab
    rng = np.random.default_rng(32)
    E = np.zeros((V, H))
    E[np.arange(V), np.arange(V)] = 1.0
    perms, models = [], []
    for j in range(3):
        p = rng.permutation(V)
        P = np.eye(H)
        P[:V, :V] = 0.0
        P[p, np.arange(V)] = 1.0          # e_t -> e_{p[t]}
        w = _weights(cfg, rng, embed=E, lm_head=E)
        w.eh_proj = np.concatenate([P, np.zeros((H, H))], axis=1)
        for lw in w.layers:
            lw.wo = np.zeros_like(lw.wo)
            lw.wdown = np.zeros_like(lw.wdown)
        perms.append(p)
        models.append(O.OracleModel(cfg, w))
    caches = [O.KVCache(cfg, 1, 32) for _ in range(3)]
    x = 7
    d, *_ = O.draft_loop_multi(models, caches, np.array([[x]]), rng.standard_normal((1, 1, H)), 5)
    t, want = x, []
    for k in range(5):
        t = perms[k % 3][t]
        want.append(t)
    assert d[0].tolist() == want


def test_each_module_holds_the_rows_of_the_chain_it_was_asked_about():
    # M = D = 3: after the catch-up every module holds the catch-up rows; module 1 then appends
    # step 2's row, module 2 the rows of steps 2 and 3 (step 2's is re-computed with its own
    # weights), so the module lengths end at catch-up + 0, + 1 and + 2.
    cfg = _cfg(D=3)
    rng = np.random.default_rng(33)
    models = [O.OracleModel(cfg, _weights(cfg, rng)) for _ in range(3)]
    base = [_prefilled(cfg, mm, rng) for mm in models]
    toks, hid = _catch_up(cfg, rng)
    n_rows = np.array([(t >= 0).sum() for t in toks])
    caches = [_copy(c) for c in base]
    d, h, _, _ = O.draft_loop_multi(models, caches, toks, hid, 3)
    for j, extra in enumerate([0, 1, 2]):
        assert (caches[j].len == base[j].len + n_rows + extra).all()
    # module 2 by hand: catch-up, then one call over the rows of steps 2 and 3
    c2 = _copy(base[2])
    O.draft_step(models[2], c2, toks, hid)
    hout, d3, _, _ = O.draft_step(models[2], c2, d[:, :2], h[:, :2])
    np.testing.assert_array_equal(d3, d[:, 2])
    np.testing.assert_array_equal(hout[:, 1], h[:, 2])
    np.testing.assert_array_equal(c2.K, caches[2].K)


def test_crop_and_catch_up_remove_the_rows_of_rejected_drafts():
    # A first speculative round drafts, the caches are cropped back to the settled length, the
    # next round's catch-up appends the settled rows: every module then equals a module that only
    # ever saw the settled rows, and the next round drafts the same.
    cfg = _cfg(D=3, batch=2)
    rng = np.random.default_rng(34)
    models = [O.OracleModel(cfg, _weights(cfg, rng)) for _ in range(3)]
    base = [_prefilled(cfg, mm, rng) for mm in models]
    toks1, hid1 = _catch_up(cfg, rng)
    toks1[1, 1:] = rng.integers(0, cfg.vocab, size=2)
    run = [_copy(c) for c in base]
    O.draft_loop_multi(models, run, toks1, hid1, 3)
    n0 = base[0].len.copy()
    for c in run:
        O.kv_crop(c, n0)
    toks2 = rng.integers(0, cfg.vocab, size=(2, 4))
    hid2 = rng.standard_normal((2, 4, cfg.hidden))
    a = O.draft_loop_multi(models, run, toks2, hid2, 3)
    clean = [_copy(c) for c in base]
    b = O.draft_loop_multi(models, clean, toks2, hid2, 3)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
    for c1, c2 in zip(run, clean):
        np.testing.assert_array_equal(c1.len, c2.len)
        for bb in range(2):
            L = c1.len[bb]
            np.testing.assert_array_equal(c1.K[:, bb, :, :L], c2.K[:, bb, :, :L])
