"""Pins of the oracle's building blocks (RMSNorm, RoPE, KV rounding, attention,
the decoder block) against closed forms, invariants and library routines."""
import math

import numpy as np
import pytest
import torch

import oracle as O
from synth import MTPConfig, to_bf16_bits, bf16_bits_to_f32


# ---------------------------------------------------------------- RMSNorm
def test_rms_norm_closed_form():
    # [3, 4]: mean of squares 12.5, so the result is [3, 4] / sqrt(12.5)
    y = O.rms_norm([3.0, 4.0], [1.0, 1.0], 0.0)
    np.testing.assert_allclose(y, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=0, atol=1e-15)
    # eps enters under the square root
    y = O.rms_norm([1.0, 1.0], [1.0, 1.0], 3.0)
    np.testing.assert_allclose(y, [0.5, 0.5], atol=1e-15)
    # the gain multiplies each output element
    y = O.rms_norm([2.0, 0.0], [3.0, 7.0], 0.0)
    np.testing.assert_allclose(y, [3 * math.sqrt(2.0), 0.0], atol=1e-14)


def test_rms_norm_invariants():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(257)
    y = O.rms_norm(x, np.ones(257), 0.0)
    assert abs(np.sqrt(np.mean(y * y)) - 1.0) < 1e-14
    np.testing.assert_allclose(O.rms_norm(5.5 * x, np.ones(257), 0.0), y, atol=1e-14)


# ---------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).standard_normal((3, 64))
    np.testing.assert_array_equal(O.rope(x, 0, 1e4), x)


def test_rope_two_dims_is_a_plane_rotation_by_pos_radians():
    # head_dim 2: one pair with frequency theta^0 = 1, so position p rotates by p radians
    np.testing.assert_allclose(O.rope([1.0, 0.0], 1, 1e4), [math.cos(1), math.sin(1)], atol=1e-15)
    np.testing.assert_allclose(O.rope([0.0, 1.0], 2, 1e4), [-math.sin(2), math.cos(2)], atol=1e-15)


def test_rope_pairing_and_frequencies():
    # head_dim 4, theta 100: pair (0,2) turns at 1 rad/position, pair (1,3) at 100^(-1/2) = 0.1
    y = O.rope([0.0, 1.0, 0.0, 0.0], 5, 100.0)
    np.testing.assert_allclose(y, [0.0, math.cos(0.5), 0.0, math.sin(0.5)], atol=1e-15)
    y = O.rope([1.0, 0.0, 0.0, 0.0], 5, 100.0)
    np.testing.assert_allclose(y, [math.cos(5), 0.0, math.sin(5), 0.0], atol=1e-15)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for m, n in [(7, 3), (4000, 17), (129, 129)]:
        assert abs(np.linalg.norm(O.rope(q, m, 1e4)) - np.linalg.norm(q)) < 1e-12
        d0 = O.rope(q, m, 1e4) @ O.rope(k, n, 1e4)
        d1 = O.rope(q, m + 250, 1e4) @ O.rope(k, n + 250, 1e4)
        assert abs(d0 - d1) < 1e-10


# ---------------------------------------------------------------- KV rounding
def test_bf16_rounding_ties_to_even():
    one = 1.0
    assert O.round_kv([one], "bf16")[0] == 1.0
    assert O.round_kv([1 + 2.0 ** -8], "bf16")[0] == 1.0                  # halfway, down to even
    assert O.round_kv([1 + 3 * 2.0 ** -8], "bf16")[0] == 1 + 2.0 ** -6    # halfway, up to even
    assert O.round_kv([1 + 2.0 ** -8 + 2.0 ** -20], "bf16")[0] == 1 + 2.0 ** -7
    assert O.round_kv([-(2 - 2.0 ** -9)], "bf16")[0] == -2.0               # carry into the exponent


def test_bf16_rounding_matches_torch_on_float32_values():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 3
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(O.round_kv(x.astype(np.float64), "bf16"), ref.astype(np.float64))
    # the input generator's own bf16 rounding agrees as well
    np.testing.assert_array_equal(bf16_bits_to_f32(to_bf16_bits(x)), ref)


def test_f32_rounding_is_float32_cast():
    x = np.random.default_rng(4).standard_normal(1000)
    np.testing.assert_array_equal(O.round_kv(x, "f32"), x.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- SiLU and attention
def test_silu_values():
    assert O.silu(0.0) == 0.0
    assert abs(O.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(O.silu(40.0) - 40.0) < 1e-12
    assert abs(O.silu(-40.0)) < 1e-15


def test_attention_single_position_returns_its_value():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((1, 16))
    np.testing.assert_allclose(O.attend(rng.standard_normal(16), rng.standard_normal((1, 16)), v), v[0],
                               atol=1e-15)


def test_attention_zero_query_is_the_mean():
    rng = np.random.default_rng(6)
    V = rng.standard_normal((9, 16))
    np.testing.assert_allclose(O.attend(np.zeros(16), rng.standard_normal((9, 16)), V), V.mean(0), atol=1e-14)


def test_attention_scale_is_one_over_sqrt_head_dim():
    # head_dim 4 -> scale 1/2.  Key 0 scores 0, key 1 scores (2 ln 3)/2 = ln 3: weights 1/4 and 3/4.
    q = np.array([2 * math.log(3), 0, 0, 0])
    K = np.array([[0.0, 0, 0, 0], [1.0, 0, 0, 0]])
    V = np.array([[4.0, 0, 0, 0], [0.0, 8, 0, 0]])
    np.testing.assert_allclose(O.attend(q, K, V), [1.0, 6.0, 0, 0], atol=1e-14)


# ---------------------------------------------------------------- decoder block
def _tiny_cfg(**kw):
    base = dict(index=90, name="t", hidden=16, n_heads=4, n_kv_heads=2, head_dim=4, ffn=12, vocab=32,
                n_layers=1, rope_theta=1e4, rms_eps=1e-6, wdtype="f32", embed_std=1.0, batch=1, D=1, ctx=0,
                prefill_rows=0, rounds=1, noise_std=1.0)
    base.update(kw)
    return MTPConfig(**base)


class _W:
    pass


def _model(cfg, rng, **over):
    H, F = cfg.hidden, cfg.ffn
    lw = _W()
    lw.in_norm, lw.post_norm = np.ones(H), np.ones(H)
    lw.wq = rng.standard_normal((cfg.q_dim, H))
    lw.wk = rng.standard_normal((cfg.kv_dim, H))
    lw.wv = rng.standard_normal((cfg.kv_dim, H))
    lw.wo = rng.standard_normal((H, cfg.q_dim))
    lw.wgate, lw.wup = rng.standard_normal((F, H)), rng.standard_normal((F, H))
    lw.wdown = rng.standard_normal((H, F))
    for k, v in over.items():
        setattr(lw, k, v)
    w = _W()
    w.embed = rng.standard_normal((cfg.vocab, H))
    w.enorm = w.hnorm = w.final_norm = np.ones(H)
    w.eh_proj = rng.standard_normal((H, 2 * H))
    w.layers = [lw]
    w.lm_head = rng.standard_normal((cfg.vocab, H))
    return O.OracleModel(cfg, w)


def test_block_with_zero_output_projections_is_identity():
    cfg = _tiny_cfg()
    rng = np.random.default_rng(7)
    m = _model(cfg, rng, wo=np.zeros((16, 16)), wdown=np.zeros((16, 12)))
    cache = O.KVCache(cfg, 1, 8)
    x = rng.standard_normal(16)
    np.testing.assert_array_equal(O.decoder_block(m, 0, cache, 0, x, 3), x)
    assert np.any(cache.K[0, 0, :, 3] != 0) and not np.any(cache.K[0, 0, :, 4:])


def test_block_at_position_zero_attends_to_its_own_value_with_grouped_heads():
    # At position 0 the only visible key is the row's own: each query head h gets
    # v of kv head h // (nq/nkv).  With the MLP switched off the block adds Wo @ o.
    cfg = _tiny_cfg()
    rng = np.random.default_rng(8)
    m = _model(cfg, rng, wdown=np.zeros((16, 12)))
    cache = O.KVCache(cfg, 1, 8)
    x = rng.standard_normal(16)
    y = O.decoder_block(m, 0, cache, 0, x, 0)
    a = x / np.sqrt(np.mean(x * x) + cfg.rms_eps)
    v = (m.layers[0]["wv"] @ a).reshape(2, 4)
    o = np.concatenate([v[0], v[0], v[1], v[1]])           # heads 0,1 -> kv 0; heads 2,3 -> kv 1
    np.testing.assert_allclose(y, x + m.layers[0]["wo"] @ o, atol=1e-5)  # v is stored as float32


def test_block_swiglu_gate_and_up_roles():
    # ffn 1: gate = alpha, up = beta exactly; down writes element 0.  The block adds silu(alpha)*beta.
    cfg = _tiny_cfg(ffn=1)
    rng = np.random.default_rng(9)
    x = np.ones(16)
    mvec = x / np.sqrt(1.0 + cfg.rms_eps)
    alpha, beta = 1.0, 3.0
    wd = np.zeros((16, 1))
    wd[0, 0] = 1.0
    m = _model(cfg, rng, wo=np.zeros((16, 16)), wgate=(alpha * mvec / (mvec @ mvec))[None],
               wup=(beta * mvec / (mvec @ mvec))[None], wdown=wd)
    y = O.decoder_block(m, 0, O.KVCache(cfg, 1, 4), 0, x, 1)
    expect = x.copy()
    expect[0] += beta / (1.0 + math.exp(-alpha))
    np.testing.assert_allclose(y, expect, atol=1e-12)


def test_block_is_causal_over_the_cache():
    cfg = _tiny_cfg()
    rng = np.random.default_rng(10)
    m = _model(cfg, rng)
    c1, c2 = O.KVCache(cfg, 1, 16), O.KVCache(cfg, 1, 16)
    pre = rng.standard_normal((1, 1, 2, 16, 4)).astype(np.float32)
    c1.K[:], c1.V[:] = pre, pre
    c2.K[:], c2.V[:] = pre, pre
    c2.K[0, 0, :, 6:] = 99.0                                 # slots after the row's position
    c2.V[0, 0, :, 6:] = -99.0
    x = rng.standard_normal(16)
    np.testing.assert_array_equal(O.decoder_block(m, 0, c1, 0, x, 5), O.decoder_block(m, 0, c2, 0, x, 5))


def test_argmax_lowest_id_on_ties_and_margin():
    assert O.argmax_lowest([0.0, 3.0, 1.0, 3.0]) == (1, 0.0)
    i, m = O.argmax_lowest([0.0, 3.0, 1.0, 2.5])
    assert i == 1 and abs(m - 0.5) < 1e-15
