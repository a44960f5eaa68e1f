"""Precision of the draw and accept decisions where it is hardest: drafts
close to the target, whose residual max(0, p - q) has little mass.

The parity rule lets the HIP path differ from the oracle only where the
oracle's uniform lies within 1e-6 of a decision edge.  These tests hold the
library to a third of that: uniforms placed 3e-7 from exact edges (computed by
the oracle in fp64) must give exactly the oracle's decision.  The drafts are
the target plus N(0, sigma^2) logit noise with sigma 0.01-0.05, so that the
residual mass Z at a rejection ranges down to 1e-6 (Deep Dive, "Speculative
Decoding From First Principles": the correction is drawn from the normalised
positive part of p - q)."""
import math

import numpy as np
import pytest
import torch

import draft_verification_dspark_amd as ds
import oracle
from parity import compare_verify, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
MARGIN = 3e-7


def _rows(B, K, V, dtype, sigma, T, seed, heads=True):
    """LM-shaped target rows (N(0, 9) plus 20 Zipf-boosted heads), drafts =
    target + sigma * N(0, 1), drafted tokens from the draft softmax."""
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    x = 3.0 * torch.randn((B, K + 1, V), generator=g, device=DEV)
    if heads:
        beta = math.log(V) + 4.5 + 2.0
        boost = beta - 1.1 * torch.log(torch.arange(1, 21, device=DEV, dtype=torch.float32))
        ids = torch.rand((B * (K + 1), V), generator=g, device=DEV).topk(20, dim=1).indices
        x.view(B * (K + 1), V).scatter_add_(1, ids, boost.expand(B * (K + 1), 20).contiguous())
    d = x[:, :K] + sigma * torch.randn((B, K, V), generator=g, device=DEV)
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    tgt, dft = x.to(st).contiguous(), d.to(st).contiguous()
    temp = torch.full((B,), float(T), device=DEV)
    probs = torch.softmax(dft.float() / float(T), -1)
    y = torch.multinomial(probs.view(B * K, V), 1, generator=g).view(B, K).int().contiguous()
    u = torch.rand((B, K + 1), generator=g, device=DEV).contiguous()
    return tgt, dft, y, temp, u


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("sigma", [0.01, 0.02, 0.05])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_residual_parity(dtype, sigma, T):
    # accept uniforms just below 1 reject wherever alpha < 1 - 2^-20, so that
    # almost every request draws a correction from a small residual
    B, K, V = 48, 8, 151936
    tgt, dft, y, temp, u = _rows(B, K, V, dtype, sigma, T, seed=int(sigma * 1e4) + int(T * 10))
    u[:, :K] = 1.0 - 2.0 ** -20
    print(f"small residual {dtype} sigma={sigma} T={T}", flush=True)
    out = ds.verify(tgt, dft, y, None, temp, u)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in out.items()}
    L = np.full(B, K, np.int32)
    th, dh, yh, Th, uh = host(tgt), host(dft), host(y), host(temp), host(u)
    ref = oracle.verify(th, dh, yh, L, Th, uh)
    rep = compare_verify(g, ref, L, Th)
    zs = []
    for b in range(B):
        a = int(ref["accepted"][b])
        if a < L[b]:
            p = oracle.softmax_T(oracle.widen(th[b, a]), float(Th[b]))
            q = oracle.softmax_T(oracle.widen(dh[b, a]), float(Th[b]))
            zs.append(float(np.maximum(p - q, 0.0).sum()))
    print(f"  residual draws {len(zs)}, Z min {min(zs):.2e} median {np.median(zs):.2e}; "
          f"mismatches {rep.n_mismatch} (boundary {rep.n_boundary}); smallest distance of a "
          f"uniform to its edge {np.min(ref['dist']):.2e}", flush=True)
    assert len(zs) >= B // 2
    rep.assert_ok()
    assert int(g["dev_status"][0]) == 0


def _replicate(row_t, row_d, n):
    """n requests with K = 1 sharing one (target, draft) row pair: target rows
    [n, 2, V] (row 1, the bonus row, is the target row again), draft [n, 1, V]."""
    t = torch.stack([row_t, row_t]).unsqueeze(0).expand(n, 2, -1).contiguous()
    d = row_d.view(1, 1, -1).expand(n, 1, -1).contiguous()
    return t, d


def _edge_uniforms(F, mass, rng, n_edges):
    """Uniforms (fp32) near the CDF edges of the n_edges tokens with the most
    mass and of a few random ones with mass: starting 3e-7 inside and outside
    each edge, stepping outwards by 3e-7 until the oracle's draw at that
    uniform is between 0.9 and 3 margins from the nearest edge of the token it
    selects (tiny-mass tokens put edges almost everywhere)."""
    order = np.argsort(-mass)
    picks = list(order[:n_edges]) + list(rng.choice(np.nonzero(mass > 0)[0], 8))
    Fprev = np.concatenate([[0.0], F[:-1]])
    us = []
    for t in picks:
        for edge, side in ((Fprev[t], 1.0), (F[t], -1.0), (F[t], 1.0), (Fprev[t], -1.0)):
            for k in range(1, 6):
                x = edge + side * k * MARGIN
                if not (0.0 <= x < 1.0):
                    break
                u32 = np.float32(x)
                dist = oracle.inverse_cdf(mass, float(u32))[1]
                if 0.9 * MARGIN <= dist <= 3 * MARGIN:
                    us.append(u32)
                    break
    return np.array(us, np.float32)


@pytest.mark.parametrize("T", [1.0, 0.7])
@pytest.mark.parametrize("sigma", [0.01, 0.05])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_residual_draw_at_cdf_edges(dtype, sigma, T):
    # one row pair, many requests: each rejects at position 1 and draws its
    # correction with a uniform 3e-7 from an edge of the exact residual CDF
    V = 151936
    tgt, dft, _, _, _ = _rows(1, 1, V, dtype, sigma, T, seed=7 + int(sigma * 1e3) + int(T * 10))
    th, dh = host(tgt), host(dft)
    p = oracle.softmax_T(oracle.widen(th[0, 0]), T)
    q = oracle.softmax_T(oracle.widen(dh[0, 0]), T)
    r = np.maximum(p - q, 0.0)
    Z = r.sum()
    F = np.cumsum(r) / Z
    rng = np.random.default_rng(1)
    us = _edge_uniforms(F, r, rng, 48)
    n = len(us)
    # the drafted token with the smallest p/q; an accept uniform halfway
    # between its alpha and 1 rejects it far from the accept edge
    ratio = np.where(q > 0, p / np.maximum(q, 1e-300), np.inf)
    y0 = int(np.argmin(ratio))
    alpha0 = float(ratio[y0])
    assert alpha0 < 1.0 - 1e-4
    u_acc = np.float32(alpha0 + (1.0 - alpha0) / 2)
    t, d = _replicate(tgt[0, 0], dft[0, 0], n)
    y = torch.full((n, 1), y0, dtype=torch.int32, device=DEV)
    temp = torch.full((n,), float(T), device=DEV)
    u = torch.empty((n, 2), dtype=torch.float32, device=DEV)
    u[:, 0] = float(u_acc)
    u[:, 1] = torch.from_numpy(us).to(DEV)
    print(f"residual edges {dtype} sigma={sigma} T={T}: Z {Z:.2e}, alpha {alpha0:.6f}, "
          f"{n} uniforms", flush=True)
    out = ds.verify(t, d, y, None, temp, u)
    torch.cuda.synchronize()
    assert np.all(host(out["accepted"]) == 0)
    got = host(out["tokens"])[:, 0]
    want = np.array([oracle.inverse_cdf(r, float(v))[0] for v in us])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(us[i]), int(got[i]), int(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_bonus_draw_at_cdf_edges(dtype):
    # full acceptance (accept uniform 0), the bonus token drawn with a uniform
    # 3e-7 from an edge of the target row's CDF
    V, T = 151936, 0.7
    tgt, dft, _, _, _ = _rows(1, 1, V, dtype, 0.5, T, seed=29)
    th = host(tgt)
    p = oracle.softmax_T(oracle.widen(th[0, 0]), T)
    F = np.cumsum(p) / p.sum()
    us = _edge_uniforms(F, p, np.random.default_rng(2), 48)
    n = len(us)
    t, d = _replicate(tgt[0, 0], dft[0, 0], n)
    y0 = int(np.argmax(p))                   # p(y) > 0: u = 0 < alpha accepts it
    y = torch.full((n, 1), y0, dtype=torch.int32, device=DEV)
    temp = torch.full((n,), T, device=DEV)
    u = torch.zeros((n, 2), dtype=torch.float32, device=DEV)
    u[:, 1] = torch.from_numpy(us).to(DEV)
    out = ds.verify(t, d, y, None, temp, u)
    torch.cuda.synchronize()
    assert np.all(host(out["accepted"]) == 1)
    got = host(out["tokens"])[:, 1]
    want = np.array([oracle.inverse_cdf(p, float(v))[0] for v in us])
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(us[i]), int(got[i]), int(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_accept_test_at_alpha_edges(dtype):
    # every position's accept uniform 3e-7 below or above its alpha (fp64,
    # oracle): the accepted counts follow exactly
    B, K, V, T = 64, 8, 151936, 1.0
    tgt, dft, y, temp, _ = _rows(B, K, V, dtype, 0.3, T, seed=41)
    th, dh, yh = host(tgt), host(dft), host(y)
    alpha = np.zeros((B, K))
    for b in range(B):
        for k in range(K):
            pk = oracle.softmax_T(oracle.widen(th[b, k]), T)[yh[b, k]]
            qk = oracle.softmax_T(oracle.widen(dh[b, k]), T)[yh[b, k]]
            alpha[b, k] = 0.0 if pk == 0 else (1.0 if qk == 0 else min(1.0, pk / qk))
    rng = np.random.default_rng(3)
    side = rng.choice([-1.0, 1.0], size=(B, K))
    side[:, :2] = -1.0                       # the first positions accept, so later ones are tested
    uu = np.float32(alpha + side * MARGIN)
    # alpha within the margin of 0 or 1 has no edge to straddle: a uniform of
    # 0.5 decides those far from the edge
    near_end = (alpha < 2 * MARGIN) | (alpha > 1.0 - 2 * MARGIN)
    uu[near_end] = np.float32(0.5)
    dist = np.abs(uu.astype(np.float64) - alpha)
    assert (dist >= 0.9 * MARGIN).all()
    print(f"accept edges {dtype}: {int((~near_end).sum())} of {B * K} uniforms {MARGIN:.0e} "
          f"from alpha", flush=True)
    u = torch.zeros((B, K + 1), dtype=torch.float32, device=DEV)
    u[:, :K] = torch.from_numpy(uu).to(DEV)
    u[:, K] = 0.5
    out = ds.verify(tgt, dft, y, None, temp, u)
    torch.cuda.synchronize()
    acc = host(out["accepted"])
    want = np.zeros(B, np.int64)
    for b in range(B):
        k = 0
        while k < K and uu[b, k] < alpha[b, k]:
            k += 1
        want[b] = k
    assert np.array_equal(acc, want), (acc, want)
