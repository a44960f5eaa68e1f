"""Seeded synthetic inputs for block verification and scheduling.

This module only *makes inputs*.  It holds no step of the verified path: no
survival product, no truncation, no budget, no accept test, no residual and no
inverse-CDF draw.  It imitates the upstream drafter (which samples the drafted
tokens from its own softmax and reports a per-position confidence) with plain
torch calls, and hands every value — logits, drafted ids, confidences,
temperatures and the pre-drawn uniforms — to both the HIP library and the CPU
oracle.  Both sides then compute from these stored values only.

The recipe follows the five benchmark workloads used by the build (vocabulary
sizes of Qwen3-8B, 151 936, and DeepSeek-V4, 129 280; K = 8 or 16 drafted
positions; temperatures 0 / 0.6 / 0.7 / 1.0).  The pages measure on GSM8K,
HumanEval, MT-Bench, Alpaca and MATH with trained drafters; those are not
available here, so these seeded, LM-shaped synthetic rows stand in for them:

* target row (b, j):  x = sigma_t * N(0, 1) per vocabulary entry; in every
  workload but the tiny one, 20 distinct ids per row get a Zipf-ranked boost
  ``beta_V - 1.1 * ln(rank)``, ``beta_V = ln V + sigma_t^2 / 2 + 2`` (a peaked,
  LM-like head holding most of the mass);
* draft row (b, j), j < K: ``x_j + eps`` with a per-workload noise law
  (plain Gaussian, per-request sigma, AR(1) across positions, or a two-class
  mixture);
* storage: generated in fp32, rounded to bf16 (round-to-nearest-even) except
  for the tiny fp32 workload;
* drafted y_{b,k} ~ softmax(draft_{b,k-1} / T_b) (lowest-index argmax at T=0);
* confidence c_{b,k}: q(y) (at T = 1 for T = 0 requests), optionally times a
  position decay or passed through a per-position sigmoid-temperature map;
* uniforms: U[0, 1) fp32, ``[B, K + 1]``.

Seeds: stream ``s`` of workload ``n`` with offset ``o`` uses
``torch.Generator(device).manual_seed(1000 * n + s + o)``.  Streams:
1 target noise, 2 head ids, 3 draft noise, 4 noise classes / per-request sigma,
5 temperatures, 6 drafted tokens, 7 uniforms.  The same seed gives different
numbers on the CPU and on the GPU generator; every consumer takes the tensors
this module returns, never regenerates them.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import torch

# name, B, K, V, dtype, threshold, budget (-1 = none), sigma_t, zipf heads
WORKLOADS = {
    1: dict(name="tiny", B=1, K=4, V=1024, dtype="f32", threshold=0.0, budget=-1,
            sigma_t=2.0, heads=False),
    2: dict(name="b16-k8-v32000", B=16, K=8, V=32000, dtype="bf16", threshold=0.1,
            budget=128, sigma_t=3.0, heads=True),
    3: dict(name="b64-k16-v151936", B=64, K=16, V=151936, dtype="bf16", threshold=0.2,
            budget=512, sigma_t=3.0, heads=True),
    4: dict(name="b256-k16-v129280", B=256, K=16, V=129280, dtype="bf16", threshold=0.15,
            budget=2048, sigma_t=3.0, heads=True),
    5: dict(name="b1024-k8-v151936", B=1024, K=8, V=151936, dtype="bf16", threshold=0.3,
            budget=3072, sigma_t=3.0, heads=True),
}

N_HEADS = 20
ZIPF_S = 1.1


@dataclasses.dataclass
class Workload:
    """One batch of inputs.  Tensor shapes: target [B,K+1,V], draft [B,K,V]
    (bf16 or fp32), drafted int32 [B,K], conf fp32 [B,K], temperature fp32 [B],
    uniforms fp32 [B,K+1].  ``greedy_drafted`` holds the draft argmax ids used
    for the greedy (T = 0) run of workload 2."""
    wid: int
    name: str
    B: int
    K: int
    V: int
    dtype: str
    target: torch.Tensor
    draft: torch.Tensor
    drafted: torch.Tensor
    conf: torch.Tensor
    temperature: torch.Tensor
    uniforms: torch.Tensor
    threshold: float
    budget: int
    min_len: int
    greedy_drafted: Optional[torch.Tensor] = None
    seed_offset: int = 0

    def hashes(self) -> dict:
        out = {}
        for k in ("target", "draft", "drafted", "conf", "temperature", "uniforms"):
            t = getattr(self, k).detach().contiguous().cpu()
            out[k] = hashlib.sha256(t.view(torch.uint8).numpy().tobytes()
                                    if t.dtype != torch.bfloat16 else
                                    t.view(torch.int16).numpy().tobytes()).hexdigest()[:16]
        return out


def _gen(device, wid, stream, offset):
    g = torch.Generator(device=device)
    g.manual_seed(1000 * wid + stream + offset)
    return g


def _draft_noise(wid, B, K, V, device, offset, n_rows_shape):
    """eps [B, K, V] fp32 for workload ``wid``."""
    g3 = _gen(device, wid, 3, offset)
    g4 = _gen(device, wid, 4, offset)
    if wid == 1:
        return 0.5 * torch.randn(n_rows_shape, generator=g3, device=device)
    if wid == 2:
        return torch.randn(n_rows_shape, generator=g3, device=device)
    if wid == 3:
        sig = 0.3 + 1.7 * torch.rand((B, 1, 1), generator=g4, device=device)
        return sig * torch.randn(n_rows_shape, generator=g3, device=device)
    if wid == 4:
        rho, sig = 0.7, 1.0
        xi = torch.randn(n_rows_shape, generator=g3, device=device)
        eps = torch.empty_like(xi)
        eps[:, 0] = sig * xi[:, 0]
        for j in range(1, K):
            eps[:, j] = rho * eps[:, j - 1] + sig * math.sqrt(1.0 - rho * rho) * xi[:, j]
        return eps
    if wid == 5:
        n_hi = int(round(0.3 * B))
        perm = torch.randperm(B, generator=g4, device=device)
        sig = torch.full((B,), 0.3, device=device)
        sig[perm[:n_hi]] = 2.5
        return sig.view(B, 1, 1) * torch.randn(n_rows_shape, generator=g3, device=device)
    raise ValueError(wid)


def make(wid: int, seed_offset: int = 0, device="cpu", B: Optional[int] = None,
         K: Optional[int] = None, V: Optional[int] = None) -> Workload:
    """Build workload ``wid`` (1..5) with optional size overrides (same recipe)."""
    spec = dict(WORKLOADS[wid])
    B = spec["B"] if B is None else int(B)
    K = spec["K"] if K is None else int(K)
    V = spec["V"] if V is None else int(V)
    dev = torch.device(device)
    sigma_t = spec["sigma_t"]

    g1 = _gen(dev, wid, 1, seed_offset)
    x = sigma_t * torch.randn((B, K + 1, V), generator=g1, device=dev)
    if spec["heads"] and V >= N_HEADS:
        g2 = _gen(dev, wid, 2, seed_offset)
        beta = math.log(V) + sigma_t * sigma_t / 2.0 + 2.0
        boost = beta - ZIPF_S * torch.log(torch.arange(1, N_HEADS + 1, device=dev,
                                                       dtype=torch.float32))
        ids = torch.rand((B * (K + 1), V), generator=g2, device=dev).topk(N_HEADS, dim=1).indices
        x.view(B * (K + 1), V).scatter_add_(1, ids, boost.expand(B * (K + 1), N_HEADS).contiguous())
    d = x[:, :K] + _draft_noise(wid, B, K, V, dev, seed_offset, (B, K, V))

    store = torch.bfloat16 if spec["dtype"] == "bf16" else torch.float32
    target = x.to(store).contiguous()
    draft = d.to(store).contiguous()
    del x, d

    # temperatures
    if wid in (1, 2, 3):
        temp = torch.ones(B, device=dev)
    elif wid == 4:
        temp = torch.full((B,), 0.7, device=dev)
    else:
        g5 = _gen(dev, wid, 5, seed_offset)
        choice = torch.tensor([0.0, 0.6, 1.0], device=dev)
        temp = choice[torch.randint(0, 3, (B,), generator=g5, device=dev)]
    temp = temp.float().contiguous()

    # the drafter: y ~ softmax(d / T) from the stored draft values
    g6 = _gen(dev, wid, 6, seed_offset)
    dv = draft.float()
    t_eff = torch.where(temp > 0, temp, torch.ones_like(temp)).view(B, 1, 1)
    logp = torch.log_softmax(dv / t_eff, dim=-1)
    probs = logp.exp().view(B * K, V)
    y_s = torch.multinomial(probs, 1, generator=g6).view(B, K)
    y_g = dv.argmax(dim=-1)
    greedy_req = (temp == 0).view(B, 1)
    drafted = torch.where(greedy_req, y_g, y_s).to(torch.int32).contiguous()
    # confidence = q(y) at T (T = 1 for greedy requests)
    logp1 = torch.log_softmax(dv, dim=-1)
    q_at_T = logp.gather(-1, drafted.long().unsqueeze(-1)).squeeze(-1).exp()
    q_at_1 = logp1.gather(-1, drafted.long().unsqueeze(-1)).squeeze(-1).exp()
    q = torch.where(greedy_req, q_at_1, q_at_T)
    del dv, logp, logp1, probs
    kk = torch.arange(1, K + 1, device=dev, dtype=torch.float32)
    if wid == 3:
        conf = q * (0.95 ** kk)
    elif wid == 4:
        qt = q.clamp(1e-6, 1 - 1e-6)
        theta = 1.0 + 0.05 * (kk - 1.0)
        conf = torch.sigmoid(torch.log(qt / (1 - qt)) / theta)
    else:
        conf = q
    conf = conf.float().contiguous()

    g7 = _gen(dev, wid, 7, seed_offset)
    uniforms = torch.rand((B, K + 1), generator=g7, device=dev).float().contiguous()

    greedy_drafted = None
    if wid == 2:
        greedy_drafted = y_g.to(torch.int32).contiguous()

    return Workload(wid=wid, name=spec["name"], B=B, K=K, V=V, dtype=spec["dtype"],
                    target=target, draft=draft, drafted=drafted, conf=conf,
                    temperature=temp, uniforms=uniforms, threshold=float(spec["threshold"]),
                    budget=int(spec["budget"]), min_len=1, greedy_drafted=greedy_drafted,
                    seed_offset=seed_offset)


def to_numpy(t: torch.Tensor):
    """Host copy for the oracle: bf16 tensors become uint16 bit patterns."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()
