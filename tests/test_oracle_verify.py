"""Pins of the oracle's verifier: the pages' worked examples, the warp order
rules against counting definitions, the sampler, the special cases that reduce
to greedy, a chi-square test of exactness over 20,000 rounds, an exact
enumeration on tiny vocabularies, and a planted-mistake negative control."""
import itertools
import json
import os

import numpy as np
import pytest
from scipy import stats

import oracle as O
import oracle.mtp as OM


# ---------------------------------------------------------------- worked examples
def test_greedy_worked_examples(golden_dir):
    doc = json.load(open(os.path.join(golden_dir, "greedy_worked_examples.json")))
    for case in doc["cases"]:
        tl = np.array([case["target_logits"]])
        r = O.greedy_verify(tl, np.array([case["drafts"]]), [case["ctx_len"]])
        e = case["expect"]
        assert r.n_accept[0] == e["n_accept"], case["name"]
        assert list(r.out_tokens[0]) == e["out_tokens"], case["name"]
        assert r.crop_len[0] == e["crop_len"], case["name"]
        assert 1 + r.n_accept[0] + 1 == e["tokens_with_settled"], case["name"]
        # the same cases through the sampling verifier with top-k 1 (greedy for any uniforms)
        for u in [0.0, 0.37, 1 - 2.0 ** -24]:
            D = case["D"]
            rs = O.sampling_verify(tl, np.array([case["drafts"]]), None, 1.0, 1, 1.0, 0,
                                   np.full((1, D), u), np.array([u]), [case["ctx_len"]])
            assert list(rs.out_tokens[0]) == e["out_tokens"], case["name"]


def test_emitted_count_is_one_to_d_plus_one():
    # [YL] stage 4: one forward gives between 1 and D+1 tokens
    rng = np.random.default_rng(20)
    for _ in range(200):
        D = int(rng.integers(1, 7))
        tl = rng.integers(0, 3, size=(1, D + 1, 4)).astype(float)
        dr = rng.integers(0, 4, size=(1, D))
        r = O.greedy_verify(tl, dr, [0])
        k = int(np.sum(r.out_tokens[0] >= 0))
        assert 1 <= k <= D + 1 and k == r.n_accept[0] + 1
        assert np.all(r.out_tokens[0, k:] == -1)


def test_trusted_prefix_stops_at_the_first_close_decision():
    # greedy, D = 3: target rows 0 and 1 agree with the drafts by clear gaps, row 2 has a tie
    # (margin 0) between the draft and a lower id, so only the first two tokens are trusted
    tl = np.array([[[0.0, 5.0, 0.0, 0.0], [0.0, 0.0, 5.0, 0.0], [0.0, 4.0, 0.0, 4.0], [9.0, 0.0, 0.0, 0.0]]])
    r = O.greedy_verify(tl, np.array([[1, 2, 3]]), [10])
    assert r.n_accept[0] == 2 and list(r.out_tokens[0]) == [1, 2, 1, -1]
    assert r.margin_pos[0] == [0, 1, 2]
    assert r.trusted_prefix(0, 1e-4) == 2
    assert r.trusted_prefix(0, 0.0) == 3            # every margin >= 0: all a + 1 tokens
    # sampling: every margin is tagged with the output position it decides, in order
    rng = np.random.default_rng(3)
    for _ in range(50):
        D = int(rng.integers(1, 5))
        tl = rng.normal(size=(1, D + 1, 7))
        dr = rng.integers(0, 7, size=(1, D))
        rs = O.sampling_verify(tl, dr, None, 0.9, 4, 0.8, 0, rng.random((1, D)), rng.random(1), [0])
        pos = rs.margin_pos[0]
        assert len(pos) == len(rs.margins[0]) and pos == sorted(pos)
        assert pos[-1] == rs.n_accept[0] and pos[0] == 0
        j = rs.trusted_prefix(0, 1e-4)
        assert 0 <= j <= rs.n_accept[0] + 1
        assert all(m >= 1e-4 for m, p in zip(rs.margins[0], pos) if p < j)


# ---------------------------------------------------------------- warp
def _warp_by_counting(l, T, k, p):
    """Independent definitions: a token survives top-k when fewer than k tokens rank
    strictly ahead of it (higher scaled logit, or equal with a lower id); it survives
    top-p when the kept mass ranked strictly ahead of it is below p, or when it is the top token."""
    z = np.asarray(l, float) / T
    V = len(z)
    ahead = lambda i, j: z[j] > z[i] or (z[j] == z[i] and j < i)
    keep_k = [i for i in range(V) if (k <= 0 or k >= V) or sum(ahead(i, j) for j in range(V)) < k]
    e = {i: np.exp(z[i] - z.max()) for i in keep_k}
    s = sum(e.values())
    pi = {i: e[i] / s for i in keep_k}
    keep_p = [i for i in keep_k if p >= 1.0 or sum(pi[j] for j in keep_k if ahead(i, j)) < p
              or not any(ahead(i, j) for j in keep_k)]
    w = np.zeros(V)
    for i in keep_p:
        w[i] = pi[i]
    return w / w.sum()


@pytest.mark.parametrize("T,k,p", [(1.0, 0, 1.0), (0.7, 5, 1.0), (1.0, 0, 0.6), (0.7, 4, 0.9), (2.0, 9, 0.3),
                                   (1.0, 1, 0.95), (0.5, 30, 0.999)])
def test_warp_matches_counting_definition(T, k, p):
    rng = np.random.default_rng(21)
    for _ in range(30):
        l = np.round(rng.standard_normal(24) * 2, 1)         # rounding plants ties
        w, _ = O.warp(l, T, k, p)
        np.testing.assert_allclose(w, _warp_by_counting(l, T, k, p), atol=1e-13)


def test_warp_top_p_keeps_the_crossing_token():
    l = np.log(np.array([0.5, 0.3, 0.2]))
    np.testing.assert_allclose(O.warp(l, 1.0, 0, 0.5)[0], [1, 0, 0], atol=1e-15)   # mass before id 1 is 0.5
    np.testing.assert_allclose(O.warp(l, 1.0, 0, 0.51)[0], [0.625, 0.375, 0], atol=1e-14)
    np.testing.assert_allclose(O.warp(l, 1.0, 0, 0.0)[0], [1, 0, 0], atol=1e-15)


def test_warp_temperature_zero_is_greedy():
    w, _ = O.warp([1.0, 5.0, 5.0, 2.0], 0.0, 0, 1.0)
    np.testing.assert_array_equal(w, [0, 1, 0, 0])


# ---------------------------------------------------------------- sampler
def test_sample_inverse_cdf_in_ascending_id_order():
    w = [0.2, 0.3, 0.5]
    assert O.sample(w, 0.0)[0] == 0
    assert O.sample(w, 0.19)[0] == 0
    assert O.sample(w, 0.2)[0] == 1          # boundary belongs to the next id
    assert O.sample(w, 0.49)[0] == 1
    assert O.sample(w, 0.5)[0] == 2
    assert O.sample(w, 1 - 2.0 ** -24)[0] == 2
    assert O.sample([0, 0, 2.0, 0, 2.0], 0.0)[0] == 2   # zero-weight ids are never drawn
    assert O.sample([0, 0, 2.0, 0, 2.0], 0.75)[0] == 4
    assert O.sample([0.0, 3.0, 0.0], 0.999999)[0] == 1


# ---------------------------------------------------------------- special cases
def test_top_k_one_is_greedy_for_any_uniforms():
    rng = np.random.default_rng(22)
    B, D, V = 64, 4, 50
    tl = np.round(rng.standard_normal((B, D + 1, V)), 1)
    dr = np.argmax(tl[:, :D] + rng.standard_normal((B, D, V)) * 0.3, axis=-1)
    g = O.greedy_verify(tl, dr, np.zeros(B, int))
    for qm in (0, 1):
        s = O.sampling_verify(tl, dr, tl[:, :D], 0.8, 1, 0.9, qm, rng.random((B, D)), rng.random(B),
                              np.zeros(B, int))
        np.testing.assert_array_equal(s.out_tokens, g.out_tokens)
        np.testing.assert_array_equal(s.n_accept, g.n_accept)


def test_tiny_temperature_is_greedy():
    rng = np.random.default_rng(23)
    B, D, V = 64, 3, 40
    tl = rng.standard_normal((B, D + 1, V))
    dr = np.argmax(tl[:, :D] + rng.standard_normal((B, D, V)) * 0.5, axis=-1)
    g = O.greedy_verify(tl, dr, np.zeros(B, int))
    s = O.sampling_verify(tl, dr, None, 1e-9, 0, 1.0, 0, rng.random((B, D)), rng.random(B), np.zeros(B, int))
    np.testing.assert_array_equal(s.out_tokens, g.out_tokens)


def test_draft_distribution_equal_to_target_always_accepts():
    rng = np.random.default_rng(24)
    B, D, V = 32, 4, 30
    tl = rng.standard_normal((B, D + 1, V))
    dr = np.array([[O.sample(O.warp(tl[b, j], 0.9, 10, 0.9)[0], rng.random())[0] for j in range(D)]
                   for b in range(B)])
    s = O.sampling_verify(tl, dr, tl[:, :D], 0.9, 10, 0.9, 1, rng.random((B, D)) * (1 - 1e-7), rng.random(B),
                          np.zeros(B, int))
    assert np.all(s.n_accept == D)


def test_uniform_zero_accepts_exactly_the_drafts_with_mass():
    # P = [0.5, 0.5, 0, 0, 0, 0]: draft 0 has mass and U = 0 keeps it; draft 4 has none
    row = np.array([0.0, 0.0] + [-np.inf] * 4)
    tl = np.array([[row, np.zeros(6)]])
    s = O.sampling_verify(tl, np.array([[0]]), None, 1.0, 0, 1.0, 0, np.zeros((1, 1)), np.zeros(1), [0])
    assert s.n_accept[0] == 1
    s = O.sampling_verify(tl, np.array([[4]]), None, 1.0, 0, 1.0, 0, np.zeros((1, 1)), np.zeros(1), [0])
    assert s.n_accept[0] == 0 and s.out_tokens[0, 0] == 0


def test_uniform_near_one_rejects_unless_ratio_reaches_it():
    l = np.log(np.array([0.6, 0.4]))
    tl = np.array([[l, l]])
    u = np.array([[1 - 2.0 ** -24]])
    s = O.sampling_verify(tl, np.array([[0]]), None, 1.0, 0, 1.0, 0, u, np.array([0.0]), [0])
    assert s.n_accept[0] == 0 and s.out_tokens[0, 0] == 1   # residual = P without the draft
    tl1 = np.array([[[0.0, -np.inf], l]])
    s = O.sampling_verify(tl1, np.array([[0]]), None, 1.0, 0, 1.0, 0, u, np.array([0.0]), [0])
    assert s.n_accept[0] == 1                                # P(d) = 1 >= U


# ---------------------------------------------------------------- exactness by chi-square
def _tables(seed, V=8, D=2):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((D + 1, V)) * 1.2, rng.standard_normal((D, V)) * 1.2


def _chi2_round_outputs(T, k, p, q_mode, n=20000, seed=25):
    tl, dl = _tables(seed)
    D, V = dl.shape
    rng = np.random.default_rng(seed + 1)
    P = [O.warp(tl[j], T, k, p)[0] for j in range(D + 1)]
    Q = [O.warp(dl[j], T, k, p)[0] for j in range(D)]
    if q_mode == 0:
        drafts = np.tile(np.argmax(dl, axis=-1), (n, 1))
    else:
        ud = rng.random((n, D))
        drafts = np.array([[O.sample(Q[j], ud[i, j])[0] for j in range(D)] for i in range(n)])
    r = O.sampling_verify(np.broadcast_to(tl, (n, D + 1, V)), drafts, np.broadcast_to(dl, (n, D, V)), T, k, p,
                          q_mode, rng.random((n, D)), rng.random(n), np.zeros(n, int))
    # categories: (first token, second token or STOP)
    obs = {}
    for i in range(n):
        key = (int(r.out_tokens[i, 0]), int(r.out_tokens[i, 1]) if r.n_accept[i] >= 1 else -1)
        obs[key] = obs.get(key, 0) + 1
    # exact probabilities: the first token follows P0; it continues only by accepting
    # its draft, which happens with probability min(Q0(y), P0(y)) (one-hot Q0 in q_mode 0),
    # and then the second token follows P1.
    Q0 = np.eye(V)[int(np.argmax(dl[0]))] if q_mode == 0 else Q[0]
    exp = {}
    for y in range(V):
        cont = min(Q0[y], P[0][y])
        if P[0][y] - cont > 0:
            exp[(y, -1)] = P[0][y] - cont
        for z in range(V):
            if cont * P[1][z] > 0:
                exp[(y, z)] = cont * P[1][z]
    if not set(obs) <= set(exp):                 # an output the target can never give
        return 0.0
    keys = sorted(exp)
    f_obs = np.array([obs.get(kk, 0) for kk in keys], float)
    f_exp = np.array([exp[kk] for kk in keys]) * n
    # pool tiny cells so the chi-square approximation holds
    small = f_exp < 5
    if small.any():
        f_obs = np.append(f_obs[~small], f_obs[small].sum())
        f_exp = np.append(f_exp[~small], f_exp[small].sum())
    return stats.chisquare(f_obs, f_exp).pvalue


@pytest.mark.slow
@pytest.mark.parametrize("T,k,p", [(1.0, 0, 1.0), (0.8, 5, 0.85)])
@pytest.mark.parametrize("q_mode", [0, 1])
def test_sampling_verify_output_follows_the_target_distribution(T, k, p, q_mode):
    assert _chi2_round_outputs(T, k, p, q_mode) > 1e-3


@pytest.mark.slow
def test_negative_control_resampling_from_p_is_detected(monkeypatch):
    # Planted mistake in the oracle: replace a rejected draft from P instead of max(0, P - Q).
    monkeypatch.setattr(OM, "residual", lambda P, Q: np.asarray(P, float))
    assert _chi2_round_outputs(1.0, 0, 1.0, 1) < 1e-6


# ---------------------------------------------------------------- exact enumeration
def _exact_round_distribution(tl, dl, T, k, p, q_mode):
    """Probability of every complete round output, integrating the uniforms exactly.

    The oracle is evaluated at one point inside every cell of a partition of
    [0,1)^(D+1) on which its decisions cannot change: the accept thresholds
    min(1, P/Q) split each u_accept axis, and the cumulative boundaries of every
    distribution a round can draw from split the u_sample axis."""
    D, V = dl.shape
    P = [O.warp(tl[j], T, k, p)[0] for j in range(D + 1)]
    Q = [O.warp(dl[j], T, k, p)[0] for j in range(D)]
    dists = [O.residual(P[j], Q[j]) for j in range(D)] + [P[D]]
    if q_mode == 0:
        dists += [O.residual(P[j], np.eye(V)[d]) for j in range(D) for d in range(V)]
    cuts = {0.0, 1.0}
    for w in dists:
        c = np.cumsum(w) / np.sum(w)
        cuts |= set(np.clip(c, 0, 1).tolist())
    cuts = sorted(cuts)
    us_pts = [((a + b) / 2, b - a) for a, b in zip(cuts[:-1], cuts[1:]) if b - a > 1e-15]
    out = {}
    tuples = itertools.product(range(V), repeat=D)
    for dr in tuples:
        if q_mode == 0:
            pd = 1.0 if list(dr) == [int(np.argmax(dl[j])) for j in range(D)] else 0.0
        else:
            pd = float(np.prod([Q[j][dr[j]] for j in range(D)]))
        if pd == 0.0:
            continue
        axes = []
        for j in range(D):
            q = 1.0 if q_mode == 0 else Q[j][dr[j]]
            thr = min(1.0, P[j][dr[j]] / q) if P[j][dr[j]] > 0 else 0.0
            pts = []
            if thr > 0:
                pts.append((thr / 2, thr))
            if thr < 1:
                pts.append(((thr + 1) / 2, 1 - thr))
            axes.append(pts)
        for combo in itertools.product(*axes):
            ua = np.array([[c[0] for c in combo]])
            wa = float(np.prod([c[1] for c in combo]))
            for us, ws in us_pts:
                r = O.sampling_verify(tl[None], np.array([dr]), dl[None], T, k, p, q_mode, ua, np.array([us]), [0])
                key = tuple(int(t) for t in r.out_tokens[0] if t >= 0)
                out[key] = out.get(key, 0.0) + pd * wa * ws
    return out


@pytest.mark.slow
@pytest.mark.parametrize("V,D,T,k,p,q_mode", [(5, 2, 1.0, 0, 1.0, 1), (4, 3, 0.9, 3, 0.9, 1),
                                              (5, 2, 1.2, 4, 0.8, 0), (4, 3, 1.0, 0, 1.0, 0)])
def test_exact_enumeration_matches_autoregressive_target(V, D, T, k, p, q_mode):
    rng = np.random.default_rng(100 + V * 10 + D)
    tl, dl = rng.standard_normal((D + 1, V)), rng.standard_normal((D, V))
    dist = _exact_round_distribution(tl, dl, T, k, p, q_mode)
    P = [O.warp(tl[j], T, k, p)[0] for j in range(D + 1)]
    assert abs(sum(dist.values()) - 1.0) < 1e-12
    # each emitted token, given the tokens before it and that the round went on, follows P_i
    for i in range(D + 1):
        prefixes = {s[:i] for s in dist if len(s) > i}
        for pre in prefixes:
            tot = sum(v for s, v in dist.items() if len(s) > i and s[:i] == pre)
            for y in range(V):
                m = sum(v for s, v in dist.items() if len(s) > i and s[:i] == pre and s[i] == y)
                assert abs(m / tot - P[i][y]) < 1e-12, (i, pre, y)


@pytest.mark.slow
def test_exact_enumeration_detects_a_planted_residual_mistake(monkeypatch):
    monkeypatch.setattr(OM, "residual", lambda P, Q: np.asarray(P, float))
    with pytest.raises(AssertionError):
        test_exact_enumeration_matches_autoregressive_target(5, 2, 1.0, 0, 1.0, 1)
