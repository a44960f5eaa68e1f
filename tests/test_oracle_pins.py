"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, never against a retyped copy of the oracle's own formulas.

* hand-worked fixtures (tests/golden/*.json, each with its citation);
* exact rational arithmetic for the fp32 survival product;
* brute-force optimality of the budgeted schedule on tiny batches;
* losslessness: the emitted token's distribution equals the target softmax
  (stratified uniform grids for one position, Monte Carlo chi-square for three),
  with the softmax taken from scipy;
* the closed form P(accepted length >= L) = prod_{k<=L} alpha_k (DSpark Guide,
  "1. The Mathematics of Suffix Decay"), and its beta_k form for redrawn drafts;
* q == p accepts everything; greedy equals planted argmaxes; inverse CDF equals
  numpy.searchsorted.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _arr(x, dtype=np.float32):
    return np.array([[float(v) if not isinstance(v, str) else float(v) for v in row] for row in x],
                    dtype=dtype)


# ------------------------------------------------------------------ schedule

@pytest.mark.parametrize("case", _load("schedule_cases.json")["cases"], ids=lambda c: c["name"])
def test_schedule_golden(case):
    conf = np.array(case["conf"], dtype=np.float32)
    L, mask, C = oracle.schedule(conf, case["threshold"], case["budget"], case["min_len"])
    assert C.tolist() == case["survival"]
    assert L.tolist() == case["lengths"]
    K = conf.shape[1]
    for b, l in enumerate(case["lengths"]):
        assert mask[b].tolist() == [1] * l + [0] * (K - l)


def test_survival_exact_rational_bound():
    """Each fp32 multiply is correctly rounded, so after k-1 multiplies the
    product is within (1 + 2^-24)^(k-1) - 1 of the exact rational product
    (plus 2^-150 once values fall into the subnormal range)."""
    rng = np.random.default_rng(7)
    conf = rng.uniform(0.0, 1.0, size=(64, 16)).astype(np.float32)
    conf[0] = np.float32(1e-20)          # underflows through the subnormals
    conf[1, 3] = 0.0
    C = oracle.survival(conf)
    for b in range(conf.shape[0]):
        exact = Fraction(1)
        for k in range(conf.shape[1]):
            exact *= Fraction(float(conf[b, k]))
            rel = (1 + Fraction(1, 2 ** 24)) ** k - 1
            err = abs(Fraction(float(C[b, k])) - exact)
            assert err <= rel * exact + Fraction(1, 2 ** 149) * k, (b, k)
    assert C[0, 1] > 0 and C[0, 1] < np.finfo(np.float32).tiny   # subnormal kept, not flushed
    assert (C[1, 3:] == 0).all()


def _random_conf(rng, B, K):
    c = rng.uniform(0.0, 1.0, size=(B, K)) ** rng.uniform(0.05, 1.0, size=(B, 1))
    return c.astype(np.float32)


def test_schedule_invariants():
    rng = np.random.default_rng(11)
    for trial in range(300):
        B = int(rng.integers(1, 12))
        K = int(rng.integers(1, 10))
        min_len = int(rng.integers(0, 2))
        conf = _random_conf(rng, B, K)
        tau = float(rng.uniform(0, 0.9))
        budget = int(rng.integers(B * min_len, B * K + 3)) if rng.random() < 0.8 else -1
        L, mask, C = oracle.schedule(conf, tau, budget, min_len)
        Lthr = oracle.threshold_lengths(C, tau, min_len)
        assert (L >= min_len).all() and (L <= Lthr).all() and (L <= K).all()
        for b in range(B):
            assert mask[b].tolist() == [1] * int(L[b]) + [0] * (K - int(L[b]))
            # threshold rule: every verified position survives unless it is a floor slot
            for k in range(1, int(Lthr[b]) + 1):
                assert C[b, k - 1] >= np.float32(tau) or k <= min_len
        if budget < 0 or Lthr.sum() <= budget:
            assert (L == Lthr).all()
        else:
            assert L.sum() == budget


def test_schedule_bruteforce_optimal():
    """For monotone survival the greedy fill is optimal: among all admissible
    length vectors with sum <= budget it maximises the total survival of the
    verified positions (exchange argument), and it is the unique optimum when
    all C are distinct."""
    rng = np.random.default_rng(5)
    for trial in range(150):
        B = int(rng.integers(1, 4))
        K = int(rng.integers(1, 5))
        min_len = int(rng.integers(0, 2))
        conf = _random_conf(rng, B, K)
        tau = float(rng.uniform(0, 0.5))
        C = oracle.survival(conf)
        Lthr = oracle.threshold_lengths(C, tau, min_len)
        budget = int(rng.integers(B * min_len, int(Lthr.sum()) + 1))
        L, _, _ = oracle.schedule(conf, tau, budget, min_len)
        Cd = C.astype(np.float64)

        def score(Lv):
            return sum(float(Cd[b, :Lv[b]].sum()) for b in range(B))

        best, best_vecs = -1.0, []
        for Lv in itertools.product(*[range(min_len, int(Lthr[b]) + 1) for b in range(B)]):
            if sum(Lv) > budget:
                continue
            s = score(Lv)
            if s > best + 1e-12:
                best, best_vecs = s, [Lv]
            elif abs(s - best) <= 1e-12:
                best_vecs.append(Lv)
        assert abs(score(L) - best) <= 1e-12
        if len(set(C.ravel().tolist())) == C.size and all(Cd[b, k] > 0 for b in range(B) for k in range(K)):
            assert tuple(L.tolist()) in best_vecs and len(best_vecs) == 1


def test_schedule_monotone_in_threshold_and_budget():
    rng = np.random.default_rng(3)
    for trial in range(100):
        B, K = 6, 8
        conf = _random_conf(rng, B, K)
        taus = sorted(rng.uniform(0, 0.8, size=4))
        prev = None
        for t in taus:
            L, _, _ = oracle.schedule(conf, float(t), -1, 1)
            if prev is not None:
                assert (L <= prev).all()
            prev = L
        prev = None
        for bud in range(B, B * K + 1, 5):
            L, _, _ = oracle.schedule(conf, 0.05, bud, 1)
            if prev is not None:
                assert (L >= prev).all()
            prev = L


# ------------------------------------------------------------------ verify

@pytest.mark.parametrize("case", _load("verify_cases.json")["cases"], ids=lambda c: c["name"])
def test_verify_golden(case):
    V, K = case["V"], case["K"]
    target = _arr(case["target"]).reshape(1, K + 1, V)
    draft = _arr(case["draft"]).reshape(1, K, V)
    drafted = np.array([case["drafted"]], dtype=np.int32)
    lengths = np.array([case["length"]], dtype=np.int32)
    temp = np.array([case["T"]], dtype=np.float32)
    u = np.array([case["uniforms"]], dtype=np.float32)
    r = oracle.verify(target, draft, drafted, lengths, temp, u)
    assert int(r["accepted"][0]) == case["accepted"]
    assert r["tokens"][0].tolist() == case["tokens"]
    assert r["flags"] == 0


def test_greedy_planted_argmax():
    rng = np.random.default_rng(17)
    for trial in range(60):
        K = int(rng.integers(1, 9))
        V = int(rng.integers(2, 300))
        target = rng.normal(0, 1, size=(1, K + 1, V)).astype(np.float32)
        amax = rng.integers(0, V, size=K + 1)
        for j in range(K + 1):
            target[0, j, amax[j]] = 10.0
            if V > 2 and rng.random() < 0.5:        # a planted tie above the argmax
                hi = int(rng.integers(amax[j], V))
                if hi != amax[j]:
                    target[0, j, hi] = 10.0
        m = int(rng.integers(0, K + 1))
        drafted = amax[:K].copy()
        if m < K:
            drafted[m] = (amax[m] + 1 + int(rng.integers(0, V - 1))) % V
        L = int(rng.integers(0, K + 1))
        r = oracle.verify_greedy(target, drafted[None].astype(np.int32), np.array([L], np.int32))
        a = min(m, L)
        assert int(r["accepted"][0]) == a
        assert r["tokens"][0, :a].tolist() == amax[:a].tolist()
        assert int(r["tokens"][0, a]) == int(amax[a])
        assert (r["tokens"][0, a + 1:] == -1).all()


def test_q_equals_p_accepts_everything():
    rng = np.random.default_rng(19)
    B, K, V = 40, 6, 97
    target = (3 * rng.normal(size=(B, K + 1, V))).astype(np.float32)
    draft = target[:, :K].copy()
    drafted = rng.integers(0, V, size=(B, K)).astype(np.int32)
    lengths = rng.integers(0, K + 1, size=B).astype(np.int32)
    temp = rng.choice([0.5, 1.0, 1.7], size=B).astype(np.float32)
    u = rng.random(size=(B, K + 1)).astype(np.float32)
    r = oracle.verify(target, draft, drafted, lengths, temp, u)
    assert (r["accepted"] == lengths).all()
    assert (r["p_tok"] == r["q_tok"]).all()


def test_probabilities_match_scipy_softmax():
    rng = np.random.default_rng(23)
    B, K, V = 12, 4, 513
    target = (4 * rng.normal(size=(B, K + 1, V))).astype(np.float32)
    draft = (4 * rng.normal(size=(B, K, V))).astype(np.float32)
    drafted = rng.integers(0, V, size=(B, K)).astype(np.int32)
    temp = rng.uniform(0.3, 2.0, size=B).astype(np.float32)
    u = rng.random(size=(B, K + 1)).astype(np.float32)
    r = oracle.verify(target, draft, drafted, None, temp, u)
    for b in range(B):
        T = float(temp[b])
        for k in range(K):
            p = scipy.special.softmax(target[b, k].astype(np.float64) / T)[drafted[b, k]]
            q = scipy.special.softmax(draft[b, k].astype(np.float64) / T)[drafted[b, k]]
            assert r["p_tok"][b, k] == pytest.approx(p, rel=1e-12)
            assert r["q_tok"][b, k] == pytest.approx(q, rel=1e-12)


def test_softmax_special_cases():
    V = 1000
    const = np.full(V, 3.25)
    assert np.allclose(oracle.softmax_T(const, 1.0), 1.0 / V, rtol=1e-14, atol=0)
    assert np.allclose(oracle.softmax_T(const, 0.37), 1.0 / V, rtol=1e-14, atol=0)
    spike = np.zeros(V)
    spike[123] = 100.0
    p = oracle.softmax_T(spike, 1.0)
    assert p[123] == pytest.approx(1.0 - (V - 1) * math.exp(-100.0), rel=1e-14)
    x = np.random.default_rng(2).normal(size=V) * 5
    assert np.allclose(oracle.softmax_T(x, 2.5), oracle.softmax_T(x / 2.5, 1.0), rtol=1e-12)
    x[7] = -np.inf
    assert oracle.softmax_T(x, 1.0)[7] == 0.0


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(29)
    for trial in range(300):
        V = int(rng.integers(1, 60))
        mass = rng.random(V) * (rng.random(V) < 0.7)
        if mass.sum() == 0:
            mass[int(rng.integers(0, V))] = 1.0
        u = float(np.float32(rng.random()))
        t, d = oracle.inverse_cdf(mass, u)
        cdf = np.cumsum(mass)
        expect = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
        if expect >= V:
            expect = int(np.nonzero(mass > 0)[0][-1])
        assert t == expect
        assert mass[t] > 0


def _lossless_setup(rng, V, K, spread=2.0):
    target = (spread * rng.normal(size=(K + 1, V))).astype(np.float32)
    draft = (target[:K] + 1.3 * rng.normal(size=(K, V))).astype(np.float32)
    return target, draft


def test_lossless_stratified_single_position():
    """One drafted position: the emitted token must be distributed as the
    target softmax p_1, and the bonus as p_2, up to the grid resolution.
    Weights q(y) and the reference p come from scipy's softmax."""
    rng = np.random.default_rng(31)
    V, N = 5, 2048
    for T in (1.0, 0.6):
        target, draft = _lossless_setup(rng, V, 1)
        p1 = scipy.special.softmax(target[0].astype(np.float64) / T)
        p2 = scipy.special.softmax(target[1].astype(np.float64) / T)
        q1 = scipy.special.softmax(draft[0].astype(np.float64) / T)
        grid = ((np.arange(N) + 0.5) / N).astype(np.float32)
        out = np.zeros(V)
        bonus = np.zeros(V)
        for y in range(V):
            n = N
            tg = np.broadcast_to(target, (n, 2, V))
            dr = np.broadcast_to(draft, (n, 1, V))
            dy = np.full((n, 1), y, np.int32)
            tt = np.full(n, T, np.float32)
            # accept fraction over a u0 grid
            u = np.stack([grid, np.full(n, 0.5, np.float32)], axis=1)
            r = oracle.verify(tg, dr, dy, None, tt, u)
            acc = r["accepted"].mean()
            # draw distribution with the accept test forced to fail
            u = np.stack([np.full(n, np.float32(1 - 2 ** -24)), grid], axis=1)
            r2 = oracle.verify(tg, dr, dy, None, tt, u)
            if acc < 1.0:
                assert (r2["accepted"] == 0).all()
                draw = np.bincount(r2["tokens"][:, 0], minlength=V) / n
                out += q1[y] * (1 - acc) * draw
            out[y] += q1[y] * acc
            # bonus on full acceptance, u1 grid
            u = np.stack([np.zeros(n, np.float32), grid], axis=1)
            r3 = oracle.verify(tg, dr, dy, None, tt, u)
            if (r3["accepted"] == 1).all():
                bonus = np.bincount(r3["tokens"][:, 1], minlength=V) / n
        assert np.abs(out - p1).max() <= 3.0 / N, (out, p1)
        assert np.abs(bonus - p2).max() <= 1.0 / N + 1e-12


def test_lossless_monte_carlo_three_positions():
    """K = 3 with drafts y_k ~ q_k: for each position k, the token emitted
    there (draft kept, or the correction) among requests that reached k is
    distributed as p_k; the bonus (all three accepted) as p_4."""
    rng = np.random.default_rng(37)
    V, K, n = 5, 3, 30000
    T = 1.0
    target, draft = _lossless_setup(rng, V, K, spread=1.5)
    P = [scipy.special.softmax(target[j].astype(np.float64) / T) for j in range(K + 1)]
    Q = [scipy.special.softmax(draft[j].astype(np.float64) / T) for j in range(K)]
    drafted = np.stack([rng.choice(V, size=n, p=Q[k]) for k in range(K)], axis=1).astype(np.int32)
    u = rng.random(size=(n, K + 1)).astype(np.float32)
    r = oracle.verify(np.broadcast_to(target, (n, K + 1, V)), np.broadcast_to(draft, (n, K, V)),
                      drafted, None, np.full(n, T, np.float32), u)
    a = r["accepted"]
    for k in range(K + 1):
        reached = a >= k
        emitted = r["tokens"][reached, k]
        counts = np.bincount(emitted, minlength=V)
        expect = P[k] * reached.sum()
        stat, pval = scipy.stats.chisquare(counts, expect)
        assert pval > 1e-4, (k, counts, expect)


def test_expected_accepted_length_closed_form():
    """Guide, "1. The Mathematics of Suffix Decay": with fixed drafts and
    independent uniforms P(a >= L) = prod_{k<=L} alpha_k, so
    E[a] = sum_L prod_{k<=L} alpha_k.  With drafts redrawn from q each time,
    alpha_k is replaced by beta_k = sum_v min(p_k, q_k)(v)."""
    rng = np.random.default_rng(41)
    V, K, n = 7, 4, 20000
    T = 0.8
    target, draft = _lossless_setup(rng, V, K, spread=1.2)
    P = [scipy.special.softmax(target[j].astype(np.float64) / T) for j in range(K + 1)]
    Q = [scipy.special.softmax(draft[j].astype(np.float64) / T) for j in range(K)]
    y = np.array([int(np.argmax(Q[k])) for k in range(K)], np.int32)
    alpha = [min(1.0, P[k][y[k]] / Q[k][y[k]]) for k in range(K)]
    expect = sum(np.prod(alpha[:L]) for L in range(1, K + 1))
    u = rng.random(size=(n, K + 1)).astype(np.float32)
    r = oracle.verify(np.broadcast_to(target, (n, K + 1, V)), np.broadcast_to(draft, (n, K, V)),
                      np.broadcast_to(y, (n, K)), None, np.full(n, T, np.float32), u)
    a = r["accepted"].astype(np.float64)
    assert abs(a.mean() - expect) <= 5 * a.std() / math.sqrt(n) + 1e-9
    for L in range(1, K + 1):
        frac = (a >= L).mean()
        pL = float(np.prod(alpha[:L]))
        assert abs(frac - pL) <= 5 * math.sqrt(pL * (1 - pL) / n) + 1e-9

    beta = [float(np.minimum(P[k], Q[k]).sum()) for k in range(K)]
    expect_b = sum(np.prod(beta[:L]) for L in range(1, K + 1))
    ys = np.stack([rng.choice(V, size=n, p=Q[k]) for k in range(K)], axis=1).astype(np.int32)
    u = rng.random(size=(n, K + 1)).astype(np.float32)
    r = oracle.verify(np.broadcast_to(target, (n, K + 1, V)), np.broadcast_to(draft, (n, K, V)),
                      ys, None, np.full(n, T, np.float32), u)
    a = r["accepted"].astype(np.float64)
    assert abs(a.mean() - expect_b) <= 5 * a.std() / math.sqrt(n) + 1e-9


def test_boundary_distance_reported():
    V = 3
    target = np.array([[[math.log(2), 0, 0], [0, 0, 0]]], np.float32)
    draft = np.array([[[0, math.log(2), 0]]], np.float32)
    p = scipy.special.softmax(target[0, 0].astype(np.float64))
    q = scipy.special.softmax(draft[0, 0].astype(np.float64))
    alpha = p[1] / q[1]
    u0 = np.float32(alpha)            # the fp32 uniform nearest alpha
    r = oracle.verify(target, draft, np.array([[1]], np.int32), None, np.ones(1, np.float32),
                      np.array([[u0, 0.5]], np.float32))
    assert r["dist"][0] <= 1e-7
    r = oracle.verify(target, draft, np.array([[1]], np.int32), None, np.ones(1, np.float32),
                      np.array([[0.9, 0.5]], np.float32))
    assert r["dist"][0] > 0.3


def test_device_status_flags():
    rng = np.random.default_rng(43)
    B, K, V = 1, 3, 16
    target = rng.normal(size=(B, K + 1, V)).astype(np.float32)
    draft = rng.normal(size=(B, K, V)).astype(np.float32)
    y = np.array([[1, 2, 3]], np.int32)
    T = np.ones(B, np.float32)
    u = np.full((B, K + 1), 0.5, np.float32)
    assert oracle.verify(target, draft, y, None, T, u)["flags"] == 0
    assert oracle.verify(target, draft, np.array([[1, V, 3]], np.int32), None, T, u)["flags"] & oracle.DEV_BAD_TOKEN
    assert oracle.verify(target, draft, y, None, -T, u)["flags"] & oracle.DEV_BAD_TEMP
    bad_u = u.copy()
    bad_u[0, K] = 1.0
    assert oracle.verify(target, draft, y, None, T, bad_u)["flags"] & oracle.DEV_BAD_UNIFORM
    nan_t = target.copy()
    nan_t[0, 1, 5] = np.nan
    assert oracle.verify(nan_t, draft, y, None, T, u)["flags"] & oracle.DEV_NONFINITE
    # a row past the scheduled length is never read
    assert oracle.verify(nan_t, draft, y, np.array([0], np.int32), T, u)["flags"] == 0
    # -inf is a legal logit (masked token)
    ninf = target.copy()
    ninf[0, 0, 0] = -np.inf
    assert oracle.verify(ninf, draft, y, None, T, u)["flags"] == 0


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049], np.uint16)
    w = oracle.widen(bits)
    assert w.tolist()[:6] == [1.0, -2.0, math.inf, -math.inf, 2.0 ** -133, -0.0]
    assert w[6] == 3.140625


def test_inverse_cdf_edges():
    """Token order is ascending id; the first id whose cumulative mass
    strictly exceeds u*Z is drawn, so a zero-mass id is never drawn and a
    uniform landing exactly on a CDF step goes to the next id."""
    assert oracle.inverse_cdf(np.array([0.0, 0.0, 0.5, 0.5]), 0.0)[0] == 2
    assert oracle.inverse_cdf(np.array([0.25, 0.25, 0.5]), 0.5)[0] == 2
    assert oracle.inverse_cdf(np.array([0.25, 0.0, 0.75]), 0.25)[0] == 2
    assert oracle.inverse_cdf(np.array([0.5, 0.5, 0.0]), np.nextafter(1.0, 0.0))[0] == 1


def test_nonfinite_row_rules():
    """A read row with NaN or +Inf, or without any finite logit, is flagged;
    rows are checked whatever the drafted ids are."""
    B, K, V = 1, 2, 8
    t = np.zeros((B, K + 1, V), np.float32)
    d = np.zeros((B, K, V), np.float32)
    y = np.array([[1, 2]], np.int32)
    T = np.ones(B, np.float32)
    u = np.full((B, K + 1), 0.5, np.float32)
    allinf = t.copy()
    allinf[0, 2] = -np.inf
    assert oracle.verify(allinf, d, y, None, T, u)["flags"] == oracle.DEV_NONFINITE
    pinf = t.copy()
    pinf[0, 0, 3] = np.inf
    f = oracle.verify(pinf, d, np.array([[1, V]], np.int32), None, T, u)["flags"]
    assert f == oracle.DEV_NONFINITE | oracle.DEV_BAD_TOKEN
    # greedy reads no draft row
    dn = d.copy()
    dn[0, 0, 0] = np.nan
    assert oracle.verify(t, dn, y, None, np.zeros(B, np.float32), u)["flags"] == 0
    assert oracle.verify(t, dn, y, None, T, u)["flags"] == oracle.DEV_NONFINITE
