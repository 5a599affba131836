"""Pins of the oracle's target verify forward (a dense stand-in main model sharing the head's
embedding and output layer, [HB14 "The draft head"]): the output norm, agreement with the
head's own row path when the head's projection passes the embedding through, causality of a
multi-row call, and the greedy identity of speculative decoding against it."""
import dataclasses

import numpy as np
import pytest

import oracle as O
from synth import MTPConfig, make_target_weights, make_weights
from tests.toy_target import plain_greedy


def _cfg(layers=1, eps=1e-6, index=95):
    return MTPConfig(index, "target", 32, 4, 2, 8, 48, 64, layers, 1e4, eps, "f32", 1.0, 1, 1, 0, 0, 1, 1.0)


def test_zero_layers_gives_a_unit_rms_hidden_and_its_projection():
    cfg = _cfg(layers=0)
    w = make_weights(cfg, std=0.3)
    tm = O.TargetModel(cfg, make_target_weights(cfg, 0, w))
    cache = O.KVCache(cfg, 1, 8)
    g, logits = O.target_row(tm, cache, 0, 5, 3)
    assert abs(np.mean(g * g) - 1.0) < 1e-4           # RMSNorm with unit gains
    assert np.allclose(logits, np.asarray(w.lm_head, np.float64) @ g, rtol=0, atol=1e-12)
    g2, _ = O.target_row(tm, cache, 0, 5, 0)           # no attention: the position does not matter
    assert np.array_equal(g, g2)


def test_target_row_equals_the_head_row_when_eh_proj_passes_the_embedding():
    # eps = 0 and embedding rows of exact unit RMS make rms(e) = e; with eh_proj = [I, 0] the
    # head's input is the embedding itself, so both row paths see the same x.
    cfg = _cfg(layers=2, eps=0.0)
    w = make_weights(cfg, std=0.3)
    e = np.asarray(w.embed, np.float64)
    w.embed = (e / np.sqrt(np.mean(e * e, axis=1, keepdims=True))).astype(np.float64)
    w.eh_proj = np.concatenate([np.eye(cfg.hidden), np.zeros((cfg.hidden, cfg.hidden))], axis=1)
    head = O.OracleModel(cfg, w)
    tw = make_target_weights(cfg, 2, w)
    tw.layers = w.layers                               # the head's own blocks
    tm = O.TargetModel(cfg, tw)
    ch, ct = O.KVCache(cfg, 1, 16), O.KVCache(cfg, 1, 16)
    rng = np.random.default_rng(3)
    for pos, tok in enumerate(rng.integers(0, cfg.vocab, 6)):
        gh, _, lh, _ = O.mtp_row(head, ch, 0, int(tok), rng.standard_normal(cfg.hidden), pos)
        gt, lt = O.target_row(tm, ct, 0, int(tok), pos)
        assert np.allclose(gh, gt, rtol=0, atol=1e-12) and np.allclose(lh, lt, rtol=0, atol=1e-12)
    assert np.array_equal(ch.K, ct.K) and np.array_equal(ch.V, ct.V)


def test_multi_row_call_equals_rows_one_by_one():
    cfg = _cfg(layers=2)
    w = make_weights(cfg, std=0.3)
    tm = O.TargetModel(cfg, make_target_weights(cfg, 2, w, std=0.3))
    toks = np.array([[7, 3, 9, 1, -1], [2, 2, -1, -1, -1]])
    c1, c2 = O.KVCache(cfg, 2, 16), O.KVCache(cfg, 2, 16)
    c1.len[:] = c2.len[:] = 0
    h1, l1 = O.target_forward(tm, c1, toks)
    for i in range(toks.shape[1]):
        col = np.where(np.arange(toks.shape[1])[None, :] == i, toks, -1)[:, i:i + 1]
        col = np.where((toks[:, :i + 1] >= 0).all(axis=1, keepdims=True), col, -1)
        h, lg = O.target_forward(tm, c2, col)
        for b in range(2):
            if col[b, 0] >= 0:
                assert np.allclose(h[b, 0], h1[b, i], rtol=0, atol=1e-12)
                assert np.allclose(lg[b, 0], l1[b, i], rtol=0, atol=1e-12)
    assert list(c1.len) == [4, 2] and list(c2.len) == [4, 2]
    assert not l1[1, 2:].any()                         # rows past the valid prefix stay zero


@pytest.mark.parametrize("D", [1, 3])
def test_spec_decoding_against_the_dense_target_is_plain_greedy(D):
    cfg = _cfg(layers=1, index=96 + D)
    w = make_weights(cfg, std=0.3)
    tw = make_target_weights(cfg, 2, w, std=0.3)
    target = O.DenseTarget(O.TargetModel(dataclasses.replace(cfg, n_layers=2), tw), 256)
    head = O.OracleModel(cfg, w)
    prompt = [3, 14, 15, 9, 2]
    plain = plain_greedy(target, prompt, 40 + D + 2)
    rng = np.random.default_rng(D)

    def mix(out, drafts):
        d = np.array(drafts)
        for j in range(d.shape[1]):
            if len(out) + j < len(plain) and rng.random() < 0.7:
                d[0, j] = plain[len(out) + j]
        return d
    for over in (None, mix):
        out, rounds, hits = O.spec_decode(target, head, prompt, 40, D, draft_override=over)
        assert out[:len(plain)] == plain[:len(out)] and len(out) >= 40
        assert len(out) == 1 + rounds + hits
