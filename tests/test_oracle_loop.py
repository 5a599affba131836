"""Greedy identity of the oracle's decode loop: speculative decoding with the MTP
head gives exactly the plain greedy output of the target, whatever the head
guesses ([HB14] "Acceptance rate and speed-up": identical token by token;
[DLM] item 3).  Also the token count 1 + rounds + accepted drafts."""
import numpy as np
import pytest

import oracle as O
from synth import MTPConfig, make_weights
from tests.toy_target import HashTarget, TinyHybridTarget, plain_greedy


def _head(seed=0, V=64, H=32, layers=1):
    cfg = MTPConfig(92 + seed, "loop", H, 2, 1, 16, 48, V, layers, 1e4, 1e-6, "f32", 1.0, 1, 1, 0, 0, 1, 1.0)
    w = make_weights(cfg, std=0.3)
    return cfg, w, O.OracleModel(cfg, w)


def _mixing_override(plain, p, seed):
    rng = np.random.default_rng(seed)

    def f(out, drafts):
        d = np.array(drafts)
        for j in range(d.shape[1]):
            idx = len(out) + j
            if idx < len(plain) and rng.random() < p:
                d[0, j] = plain[idx]
        return d
    return f


@pytest.mark.slow
@pytest.mark.parametrize("D", [1, 3, 6])
@pytest.mark.parametrize("kind", ["hash", "hybrid"])
def test_spec_greedy_equals_plain_greedy(D, kind):
    cfg, w, model = _head(seed=D)
    target = HashTarget(cfg.vocab, cfg.hidden) if kind == "hash" else TinyHybridTarget(w.embed, seed=D)
    prompt = list(np.random.default_rng(D).integers(0, cfg.vocab, 7))
    max_new = 220
    plain = plain_greedy(target, prompt, max_new + D + 2)
    for p in (0.0, 0.6, 1.0):
        over = None if p == 0.0 else _mixing_override(plain, p, seed=D)
        out, rounds, hits = O.spec_decode(target, model, prompt, max_new, D, draft_override=over)
        assert out[:len(plain)] == plain[:len(out)] and len(out) >= max_new
        assert len(out) == 1 + rounds + hits
        if p == 0.6:
            assert rounds >= 64 and 0 < hits < rounds * D
        if p == 1.0:
            assert hits == rounds * D


@pytest.mark.slow
def test_spec_greedy_with_a_four_layer_head():
    cfg, w, model = _head(seed=9, layers=4)
    target = TinyHybridTarget(w.embed, seed=9)
    prompt = [3, 1, 4, 1, 5]
    plain = plain_greedy(target, prompt, 80)
    out, rounds, hits = O.spec_decode(target, model, prompt, 60, 6,
                                      draft_override=_mixing_override(plain, 0.7, 9))
    assert out[:len(plain)] == plain[:len(out)]
    assert len(out) == 1 + rounds + hits


def test_identity_check_detects_a_planted_loop_mistake(monkeypatch):
    # Planted mistake in the oracle: keep one draft more than the prefix match allows.
    cfg, w, model = _head(seed=1)
    target = TinyHybridTarget(w.embed, seed=1)
    prompt = [5, 6, 7]
    plain = plain_greedy(target, prompt, 40)
    real = O.greedy_verify

    def bad(tl, dr, ctx):
        r = real(tl, dr, ctx)
        a = int(r.n_accept[0])
        if a < dr.shape[1]:
            r.out_tokens[0, a] = dr[0, a]
            r.out_tokens[0, a + 1] = int(np.argmax(tl[0, a + 1]))
            r.n_accept[0] = a + 1
            r.crop_len[0] += 1
        return r
    import oracle.mtp as OM
    monkeypatch.setattr(OM, "greedy_verify", bad)
    out, _, _ = O.spec_decode(target, model, prompt, 30, 1)
    assert out[:len(plain)] != plain[:len(out)]
