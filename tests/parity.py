"""Comparison of the HIP library's outputs with the CPU oracle.

The rules: schedule outputs (lengths, mask, survival) must match bit for bit;
accepted counts and emitted tokens must match exactly except for requests
where the oracle reports a uniform within 1e-6 of a decision edge (counted as
boundary exceptions); p(y) and q(y) must agree to 1e-5 relative, or both be
below 1e-30.  Greedy outputs must match exactly."""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
import workloads

REL_TOL = 1e-5
TINY = 1e-30


@dataclasses.dataclass
class VerifyReport:
    n_requests: int
    n_mismatch: int
    n_boundary: int
    failures: list
    worst_prob_rel: float

    def assert_ok(self):
        assert not self.failures, f"{len(self.failures)} unexplained mismatches, first: {self.failures[:3]}"


def compare_schedule(gpu, ref):
    lengths, mask, surv = [np.asarray(x) for x in gpu]
    rl, rm, rs = ref
    assert np.array_equal(lengths, rl), (np.nonzero(lengths != rl), lengths[:8], rl[:8])
    assert np.array_equal(mask, rm)
    # bitwise equality of the fp32 survival (NaN-free inputs)
    assert np.array_equal(surv.view(np.uint32), rs.view(np.uint32))


def compare_verify(gpu: dict, ref: dict, lengths, temperature, requests=None) -> VerifyReport:
    acc = gpu["accepted"]
    tok = gpu["tokens"]
    B = acc.shape[0]
    idx = range(B) if requests is None else requests
    failures = []
    n_mis = n_bnd = 0
    worst = 0.0
    for b in idx:
        if ref.get("req_flags") is not None and ref["req_flags"][b]:
            continue                       # outputs unspecified for flagged requests
        same = acc[b] == ref["accepted"][b] and np.array_equal(tok[b], ref["tokens"][b])
        if not same:
            n_mis += 1
            if ref["dist"][b] <= oracle.BOUNDARY:
                n_bnd += 1
            else:
                failures.append((int(b), int(acc[b]), int(ref["accepted"][b]), tok[b].tolist(),
                                 ref["tokens"][b].tolist(), float(ref["dist"][b])))
        if gpu.get("p_tok") is not None and temperature[b] > 0:
            L = int(lengths[b])
            for name in ("p_tok", "q_tok"):
                g = gpu[name][b, :L].astype(np.float64)
                o = ref[name][b, :L]
                both_tiny = (np.abs(g) < TINY) & (o < TINY)
                rel = np.where(both_tiny, 0.0, np.abs(g - o) / np.maximum(o, 1e-300))
                if rel.size:
                    worst = max(worst, float(rel.max()))
                bad = rel > REL_TOL
                if bad.any():
                    failures.append((int(b), name, g[bad].tolist(), o[bad].tolist()))
    return VerifyReport(len(list(idx)), n_mis, n_bnd, failures, worst)


def host(t):
    return workloads.to_numpy(t)
