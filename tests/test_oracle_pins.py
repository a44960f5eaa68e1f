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


# ------------------------------------------------- load-aware threshold, budget

CURVE = _load("throughput_curve.json")


def test_curve_slopes_reproduce_the_printed_gains():
    # the page's marginal-gain column for batch sizes 2..32 is the segment
    # slope rounded to a whole number; 64 and 128 are documented misprints
    c = np.array(CURVE["curve"], dtype=np.float64)
    slopes = np.diff(c[:, 1]) / np.diff(c[:, 0])
    printed = CURVE["printed_marginal_gain"][1:]
    for i in range(5):
        assert round(slopes[i] + 1e-9) == printed[i], (i, slopes[i], printed[i])
    assert slopes[5] == 4.0625 and slopes[6] == 1.09375


@pytest.mark.parametrize("case", CURVE["budget_cases"], ids=lambda c: f"cost{c['slot_cost']}")
def test_curve_budget_page_table(case):
    budget, flags = oracle.curve_budget(CURVE["curve"], case["slot_cost"], case["B"], case["min_len"])
    assert flags == 0
    assert budget == case["budget"]
    assert budget == max(case["B"] * case["min_len"], case["xstar"] - case["B"])


def _token_scan_budget(curve, cost, B, min_len):
    # one token at a time along the piecewise-linear curve (exact fractions):
    # the pass grows while the next token's gain covers the cost
    xs = [Fraction(int(x)) for x, _ in curve]
    ts = [Fraction(float(t)) for _, t in curve]

    def T(x):
        for i in range(1, len(xs)):
            if x <= xs[i]:
                return ts[i - 1] + (ts[i] - ts[i - 1]) * (x - xs[i - 1]) / (xs[i] - xs[i - 1])
        return ts[-1]
    x = xs[0]
    cost = Fraction(float(np.float32(cost)))
    while x < xs[-1] and T(x + 1) - T(x) >= cost:
        x += 1
    return max(B * min_len, int(x) - B)


def test_curve_budget_equals_token_by_token_scan():
    rng = np.random.default_rng(5)
    for _ in range(300):
        n = int(rng.integers(1, 9))
        xs = np.cumsum(rng.integers(1, 9, size=n)).astype(np.float32)
        ts = np.cumsum(rng.uniform(-20, 80, size=n)).astype(np.float32)
        curve = np.stack([xs, ts], axis=1)
        cost = float(rng.uniform(-10, 60))
        B, ml = int(rng.integers(1, 6)), int(rng.integers(0, 3))
        slopes = np.diff(ts.astype(np.float64)) / np.diff(xs.astype(np.float64))
        if np.any(np.abs(slopes - np.float32(cost)) < 1e-6):
            continue  # a slope equal to the cost up to rounding: both readings hold
        got, flags = oracle.curve_budget(curve, cost, B, ml)
        assert flags == 0
        assert got == _token_scan_budget(curve, cost, B, ml)


def test_curve_budget_monotone_in_cost_and_edge_cases():
    c = CURVE["curve"]
    costs = np.linspace(-5, 50, 111)
    budgets = [oracle.curve_budget(c, k, 4, 1)[0] for k in costs]
    assert all(a >= b for a, b in zip(budgets, budgets[1:]))
    assert oracle.curve_budget(np.zeros((0, 2)), 1.0, 4, 1) == (-1, 0)
    assert oracle.curve_budget([[3, 10]], 1.0, 2, 1) == (2, 0)          # one point: x* = 3, 3 - 2 = 1 < floor 2
    for bad in ([[2, 10], [2, 20]], [[0, 10]], [[1.5, 10]], [[1, float("nan")]], [[4, 1], [3, 2]]):
        assert oracle.curve_budget(bad, 1.0, 2, 1) == (-1, oracle.DEV_BAD_CURVE)


def test_load_factor_closed_forms():
    f32 = np.float32
    assert oracle.load_factor(10, 10, 0, 4) == (f32(0.6), 0)
    assert oracle.load_factor(0, 10, 4, 4) == (f32(0.4), 0)
    assert oracle.load_factor(10, 10, 4, 4) == (f32(1.0), 0)
    assert oracle.load_factor(0, 10, 0, 4) == (f32(0.0), 0)
    assert oracle.load_factor(25, 10, 4, 4) == (f32(1.0), 0)             # past Q_max: clamped
    lf, fl = oracle.load_factor(5, 10, 2, 4)
    assert fl == 0 and abs(float(lf) - 0.5) < 1e-7                        # 0.6 * 0.5 + 0.4 * 0.5
    for q, m in ((float("nan"), 1.0), (1.0, float("inf")), (-1.0, 0.0)):
        assert oracle.load_factor(q, 10, m, 4) == (f32(1.0), oracle.DEV_BAD_LOAD)


@pytest.mark.parametrize("case", CURVE["threshold_cases"], ids=lambda c: f"lf{c['lf']}-{c['tau_min']}")
def test_load_threshold_page_values(case):
    tau = oracle.load_threshold(case["lf"], case["tau_min"], case["tau_max"])
    assert abs(float(tau) - case["tau"]) <= 1e-7


def test_load_threshold_endpoints_and_monotone():
    f32 = np.float32
    for lo, hi in ((0.20, 0.75), (0.25, 0.75), (0.0, 1.0), (0.3, 0.3)):
        assert oracle.load_threshold(0.0, lo, hi) == f32(lo)
        assert abs(float(oracle.load_threshold(1.0, lo, hi)) - float(f32(hi))) <= float(np.spacing(f32(hi)))
        taus = [float(oracle.load_threshold(x, lo, hi)) for x in np.linspace(0, 1, 101, dtype=np.float32)]
        assert all(a <= b for a, b in zip(taus, taus[1:]))
    # the code listing's 0.25 + 0.50 * LF^2, in exact arithmetic
    for x in np.linspace(0, 1, 37, dtype=np.float32):
        exact = 0.25 + 0.5 * float(x) ** 2
        assert abs(float(oracle.load_threshold(x, 0.25, 0.75)) - exact) <= 2e-7


def test_load_aware_schedule_shortens_under_load():
    # more load -> a higher threshold -> no request verifies more positions
    rng = np.random.default_rng(9)
    conf = rng.uniform(0.6, 1.0, size=(12, 8)).astype(np.float32)
    curve = CURVE["curve"]
    prev = None
    for q in np.linspace(0, 10, 11):
        L, mask, C, tau, budget, flags = oracle.schedule_load_aware(
            conf, (q, 2.0), 10.0, 8.0, 0.2, 0.75, curve, 0.0, 1)
        assert flags == 0 and budget == 128 - 12
        assert np.array_equal(L, oracle.threshold_lengths(C, tau, 1))  # budget 116 never binds here
        if prev is not None:
            assert np.all(L <= prev)
        prev = L
    # an idle engine (LF = 0) verifies with tau_min, a saturated one with tau_max
    L0 = oracle.schedule_load_aware(conf, (0, 0), 10, 8, 0.2, 0.75, [], 0.0, 1)
    L1 = oracle.schedule_load_aware(conf, (10, 8), 10, 8, 0.2, 0.75, [], 0.0, 1)
    assert float(L0[3]) == np.float32(0.2) and L0[4] == -1
    assert abs(float(L1[3]) - 0.75) < 1e-7


# ------------------------------------------------------------ online calibration

def test_calibrate_closed_forms():
    # dyadic scores, exact in fp32: logit(x) = ln r with r = x / (1 - x)
    x = np.array([[0.75, 0.875, 0.5, 0.2, 0.0, 1.0, 0.37]], dtype=np.float32)
    c, flags = oracle.calibrate(x, [2.0, 0.5, 7.0, 1.0, 3.0, 3.0, 1.0])
    assert flags == 0
    assert abs(c[0, 0] - math.sqrt(3.0) / (1.0 + math.sqrt(3.0))) < 1e-15  # r = 3, temperature 2
    assert abs(c[0, 1] - 49.0 / 50.0) < 1e-15      # r = 7, temperature 1/2: r^2 / (1 + r^2)
    assert c[0, 2] == 0.5                            # the midpoint is fixed by every temperature
    assert abs(c[0, 3] - float(np.float32(0.2))) < 1e-15   # temperature 1: the identity
    assert c[0, 4] == 0.0 and c[0, 5] == 1.0
    assert abs(c[0, 6] - float(np.float32(0.37))) < 1e-15
    # symmetry about 1/2, and a higher temperature pulls scores toward 1/2
    r = np.random.default_rng(1).uniform(0.01, 0.99, size=(50, 1)).astype(np.float32)
    lo, _ = oracle.calibrate(r, [1.7])
    hi, _ = oracle.calibrate((1 - r.astype(np.float64)).astype(np.float32), [1.7])
    assert np.all(np.abs(lo + hi - 1.0) < 1e-7)
    t2, _ = oracle.calibrate(r, [2.5])
    assert np.all(np.abs(t2 - 0.5) <= np.abs(lo - 0.5) + 1e-15)
    _, f = oracle.calibrate(np.array([[0.5, 1.5]], np.float32), [1.0, 1.0])
    assert f == oracle.DEV_BAD_CONF
    _, f = oracle.calibrate(np.array([[0.5]], np.float32), [0.0])
    assert f == oracle.DEV_BAD_CONF


def test_evaluated_positions_by_hand():
    ran, ok = oracle.evaluated_positions([3, 3, 0, 4], [1, 3, 0, 0], 4)
    assert ran.astype(int).tolist() == [[1, 1, 0, 0], [1, 1, 1, 0], [0, 0, 0, 0], [1, 0, 0, 0]]
    assert ok.astype(int).tolist() == [[1, 0, 0, 0], [1, 1, 1, 0], [0, 0, 0, 0], [0, 0, 0, 0]]


def test_temperature_step_page_example():
    # Deep Dive, "Online Adaptation": position 5 predicted 0.70 but accepted
    # 0.55 -> its temperature goes up (by learning rate * 0.15)
    K = 5
    win = oracle.CalibrationWindow(K)
    cal = np.full((20, K), 0.7, dtype=np.float32)
    lengths = np.full(20, K, dtype=np.int32)
    # position 5 runs in every request; 11 of 20 accept it
    accepted = np.array([5] * 11 + [4] * 9, dtype=np.int32)
    win.observe(cal, lengths, accepted)
    th = win.update(np.ones(K, np.float32), 0.015625, 0.05)
    assert abs(th[4] - (1.0 + 0.015625 * (float(np.float32(0.7)) - 0.55))) < 1e-12
    assert th[4] > 1.0
    # positions 1-4 ran and were accepted everywhere: underconfident, so down
    assert np.all(th[:4] < 1.0)


def test_ece_by_hand():
    win = oracle.CalibrationWindow(1, n_bins=10)
    win.observe(np.full((10, 1), 0.9, np.float32), np.ones(10, np.int32), np.array([1] * 9 + [0]))
    assert abs(win.ece() - abs(9 - 10 * float(np.float32(0.9))) / 10) < 1e-12   # ~0
    win.reset()
    win.observe(np.full((10, 1), 0.9, np.float32), np.ones(10, np.int32), np.array([1] * 7 + [0] * 3))
    assert abs(win.ece() - 0.2) < 1e-7
    # two bins: 4 tokens at 0.25 (1 accepted) and 4 at 0.85 (4 accepted)
    win = oracle.CalibrationWindow(1, n_bins=10)
    c = np.array([[0.25]] * 4 + [[0.85]] * 4, np.float32)
    win.observe(c, np.ones(8, np.int32), np.array([1, 0, 0, 0, 1, 1, 1, 1]))
    exact = (abs(1 - 4 * float(np.float32(0.25))) + abs(4 - 4 * float(np.float32(0.85)))) / 8
    assert abs(win.ece() - exact) < 1e-12 and abs(exact - 0.075) < 1e-7
    assert win.bn.tolist() == [0, 0, 4, 0, 0, 0, 0, 0, 4, 0]
    # the top edge falls in the last bin
    win = oracle.CalibrationWindow(1, n_bins=4)
    win.observe(np.array([[1.0]], np.float32), np.ones(1, np.int32), np.ones(1, np.int32))
    assert win.bn.tolist() == [0, 0, 0, 1] and win.ece() == 0.0


def test_online_loop_converges_to_the_true_temperature():
    # raw scores are overconfident: a token with raw score s is accepted with
    # probability sigmoid(logit(s) / 1.6); the loop should find ~1.6 and
    # bring the ECE down (Deep Dive, "Online Adaptation")
    rng = np.random.default_rng(7)
    K, B, true_t = 1, 512, 1.6
    theta = np.ones(K)
    win = oracle.CalibrationWindow(K)
    eces = []
    for w in range(120):
        for _ in range(8):
            raw = rng.uniform(0.55, 0.99, size=(B, K)).astype(np.float32)
            cal, _ = oracle.calibrate(raw, theta.astype(np.float32))
            p_true, _ = oracle.calibrate(raw, [true_t])
            acc = (rng.random((B, K)) < p_true).astype(np.int32)[:, 0]
            theta, ece = oracle.calib_observe(win, theta, cal, np.ones(B, np.int32), acc, 1.0, 0.05, 8)
        eces.append(ece)
    assert abs(theta[0] - true_t) < 0.1, theta
    assert np.mean(eces[:3]) > 0.05 and np.mean(eces[-40:]) < 0.02, (np.mean(eces[:3]), np.mean(eces[-40:]))


# ------------------------------------------------------ Markov logit-bias draft

def _fixed_point(rng, shape):
    # multiples of 2^-8 in [-1, 1]: bf16-exact, and every sum of up to 256
    # products is exact in fp32
    return oracle.bf16_round((rng.integers(-256, 257, size=shape) / 256.0).astype(np.float32))


def test_bf16_round_against_exact_rounding():
    rng = np.random.default_rng(2)
    x = (rng.normal(size=4000) * 10.0 ** rng.integers(-3, 4, size=4000)).astype(np.float32)
    x[:4] = [1.00390625, 1.005859375, 1.01171875, -1.00390625]    # ties go to even
    got = oracle.widen(oracle.bf16_round(x))
    for v, g in zip(x.astype(np.float64), got):
        # the two bf16 neighbours of v, and the nearest (even on a tie)
        m, e = math.frexp(v)
        step = 2.0 ** (e - 8)
        lo = math.floor(v / step) * step
        hi = lo + step
        want = lo if (v - lo < hi - v or (v - lo == hi - v and int(round(lo / step)) % 2 == 0)) else hi
        assert g == want, (v, g, want)


def test_markov_bias_is_the_exact_sum():
    rng = np.random.default_rng(3)
    for fixed in (True, False):
        U = _fixed_point(rng, (40, 32)) if fixed else oracle.bf16_round(rng.normal(size=(40, 32)).astype(np.float32))
        Vm = _fixed_point(rng, (40, 32)) if fixed else oracle.bf16_round(rng.normal(size=(40, 32)).astype(np.float32))
        U64, V64 = oracle.widen(U), oracle.widen(Vm)
        for prev in (0, 7, 39):
            got = oracle.markov_bias(U64, V64, prev)
            exact = np.array([math.fsum(U64[v] * V64[prev]) for v in range(40)])
            if fixed:
                assert np.array_equal(got, exact)
            else:
                assert np.allclose(got, exact, rtol=1e-12, atol=1e-12)


def test_markov_zero_scale_is_plain_sampling():
    rng = np.random.default_rng(4)
    B, K, V, r = 3, 4, 60, 16
    base = oracle.bf16_round(rng.normal(size=(B, K, V)).astype(np.float32) * 3)
    U, Vm = _fixed_point(rng, (V, r)), _fixed_point(rng, (V, r))
    u = rng.random((B, K)).astype(np.float32)
    T = np.array([1.0, 0.7, 1.3], np.float32)
    c, y, q, _ = oracle.markov_draft(base, U, Vm, 0.0, [1, 2, 3], T, u)
    assert np.array_equal(c, base)
    for b in range(B):
        for k in range(K):
            p = scipy.special.softmax(oracle.widen(base[b, k]) / float(T[b]))
            want = int(np.searchsorted(np.cumsum(p), float(u[b, k]) * np.sum(p), side="right"))
            assert y[b, k] == want and abs(q[b, k] - p[want]) < 1e-12


def test_markov_one_hot_rows_give_a_column_bias():
    # Vm rows one-hot: the bias of the previous token t is the column U[:, j(t)]
    rng = np.random.default_rng(5)
    V, r, K = 48, 16, 6
    j_of = rng.integers(0, r, size=V)
    Vm = np.zeros((V, r), np.float32)
    Vm[np.arange(V), j_of] = 1.0
    Vm = oracle.bf16_round(Vm)
    U = _fixed_point(rng, (V, r))
    base = oracle.bf16_round(rng.normal(size=(1, K, V)).astype(np.float32))
    s = 0.75
    c, y, q, _ = oracle.markov_draft(base, U, Vm, s, [5], np.zeros(1, np.float32), np.zeros((1, K), np.float32))
    prev = 5
    Uw = oracle.widen(U)
    for k in range(K):
        row = oracle.widen(base[0, k]).astype(np.float32) + np.float32(s) * Uw[:, j_of[prev]].astype(np.float32)
        want = oracle.bf16_round(row.astype(np.float32))
        assert np.array_equal(c[0, k], want)
        assert y[0, k] == int(np.argmax(oracle.widen(want)))      # greedy: first maximum
        prev = y[0, k]


def test_markov_bias_depends_on_the_previous_token_only():
    rng = np.random.default_rng(6)
    V, r, K = 40, 16, 3
    U, Vm = _fixed_point(rng, (V, r)), _fixed_point(rng, (V, r))
    base = np.repeat(oracle.bf16_round(rng.normal(size=(1, K, V)).astype(np.float32)), 2, axis=0)
    c, y, _, _ = oracle.markov_draft(base, U, Vm, 1.0, [9, 9], np.zeros(2, np.float32), np.zeros((2, K), np.float32))
    assert np.array_equal(c[0], c[1]) and np.array_equal(y[0], y[1])
    c2, y2, _, _ = oracle.markov_draft(base[:1, 1:], U, Vm, 1.0, [int(y[0, 0])], np.zeros(1, np.float32),
                                       np.zeros((1, K - 1), np.float32))
    # the block restarted after its first token reproduces the rest of the block
    assert np.array_equal(c2[0], c[0, 1:]) and np.array_equal(y2[0], y[0, 1:])


def test_markov_draws_follow_the_corrected_softmax():
    # stratified uniforms: the draw frequencies equal softmax(corrected) to 1/N
    rng = np.random.default_rng(8)
    V, r, N = 12, 16, 2048
    U, Vm = _fixed_point(rng, (V, r)), _fixed_point(rng, (V, r))
    base = oracle.bf16_round(rng.normal(size=(1, 1, V)).astype(np.float32))
    counts = np.zeros(V)
    for i in range(N):
        _, y, _, _ = oracle.markov_draft(base, U, Vm, 2.0, [3], np.ones(1, np.float32),
                                         np.array([[(i + 0.5) / N]], np.float32))
        counts[y[0, 0]] += 1
    c, _, _, _ = oracle.markov_draft(base, U, Vm, 2.0, [3], np.ones(1, np.float32), np.zeros((1, 1), np.float32))
    p = scipy.special.softmax(oracle.widen(c[0, 0]))
    assert np.all(np.abs(counts / N - p) <= 1.0 / N + 1e-9)
