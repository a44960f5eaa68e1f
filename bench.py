"""Benchmark: verified draft positions per second and achieved HBM bandwidth of
confidence-scheduled block verification on one MI355X.

One step = the schedule and the verification of one batch of the
V=151936, B=64, K=16 workload (bf16 logits, T=1, threshold 0.2, budget 512;
seeded synthetic inputs resident in HBM), as one dspark_schedule_verify call,
which works the schedule out inside the streaming launch.  Six input sets
(seed offsets 0, 100, ..., 500; 641 MB each) rotate so that no step reads
logits left in the 256 MB last-level cache by the step before.

Order of the run:
1. warm-up steps;
2. one step per input set, then the accounting: per set the verified
   positions (sum_b L_b) and the algorithmic bytes, from outputs that a step
   has written; every length, accepted count and byte count is checked
   against its bounds before use;
3. the timed region: the K steps launched back to back on one stream,
   behind a spin kernel that lets the host queue them all first;
4. kernel timing: the streaming launches of the same steps alone
   (dspark_schedule_verify_phase, STREAM half), back to back between one
   event pair; the same steps again, each as its two halves with events
   around the streaming launch (the spread, dispatch included); and whole
   calls with events around the call;
5. context: the same steps as two calls (dspark_schedule, dspark_verify), the
   plain read of the same bytes (libdspark_bench.so), the other hot-path
   rows (``--no-rows`` skips them; their streaming launches are timed back
   to back as above, their whole calls between events);
6. the CPU baseline: the oracle on the host's cores (one worker process per
   core, at most 16, requests split statically), which also checks the GPU's
   outputs of input set 0 request by request (``parity``).

Prints ONE JSON line on stdout.  ``value`` = verified positions per second of
schedule + verify.  ``roofline`` reports the dominant kernel, the streaming
launch (k_stream_rows), against the 8 TB/s HBM peak: its algorithmic bytes
per launch, s*V*sum_b rows_b with rows_b = 2 L_b + 1 (T > 0) or L_b + 1
(T = 0), over its mean duration launched back to back; ``call_*`` the same
for the whole call (streaming bytes plus the rejected row pairs it re-reads).
``traffic`` is the HBM bytes per launch that rocprofv3 counters measured for
the same kernel (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel of known
size), used only while the kernel sources hash to the recorded value.

--calibrate-copy N runs, after the timed steps, a plain elementwise copy of
N MiB (read N MiB, write N MiB) five times: the reference kernel of known size
for the FETCH_SIZE / WRITE_SIZE counter runs.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SPIN_CYCLES = 20_000_000  # GPU clock cycles the pre-queued spin kernel runs for
MAX_CPU_WORKERS = 16
PMC_SUMMARY = os.path.join(ROOT, "profiles", "k_stream_rows_b64_k16_v151936_pmc.md")
KERNEL_SOURCES = [os.path.join(ROOT, "draft_verification_dspark_amd", "csrc", f)
                  for f in ("verify.hip", "device.hpp", "args.hpp", "schedule_core.hpp",
                            "schedule_args.hpp")]
BENCH_LIB = os.path.join(ROOT, "draft_verification_dspark_amd", "libdspark_bench.so")
METRIC = "verified draft positions/sec and achieved HBM GB/s vs peak (V=151936, B=64, K=16)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- accounting

class AccountingError(ValueError):
    pass


def account_set(lengths, accepted, temperature, K: int, V: int, s: int) -> dict:
    """Positions and algorithmic bytes of one verified batch, from the outputs
    a step wrote.  Raises AccountingError when a length or accepted count is
    out of its bounds (0 <= L <= K, 0 <= a <= L), which is what outputs that
    no step has written look like.

    rows of the streaming pass: 2 L + 1 for T > 0 (target rows 0..L, draft
    rows 0..L-1), L + 1 for T = 0; the call adds the rejected row pair
    (2 rows) of every sampled request with a < L; the early-exit bound is what
    a verifier stopping at the first rejection would read."""
    import numpy as np
    L = np.asarray(lengths).astype(np.int64)
    a = np.asarray(accepted).astype(np.int64)
    T = np.asarray(temperature, dtype=np.float32)
    if L.shape != a.shape or L.shape != T.shape or L.ndim != 1:
        raise AccountingError(f"shapes {L.shape} {a.shape} {T.shape}")
    if (L < 0).any() or (L > K).any():
        raise AccountingError(f"lengths outside [0, {K}]: {L[(L < 0) | (L > K)][:8]}")
    if (a < 0).any() or (a > L).any():
        raise AccountingError(f"accepted outside [0, L]: {a[(a < 0) | (a > L)][:8]}")
    soft = T > 0
    stream_rows = np.where(soft, 2 * L + 1, L + 1)
    call_rows = stream_rows + np.where(soft & (a < L), 2, 0)
    early_rows = np.where(soft, 2 * (a + 1) + 2 * (a < L), a + 1)
    out = dict(positions=int(L.sum()), stream_bytes=int(s * V * stream_rows.sum()),
               call_bytes=int(s * V * call_rows.sum()),
               early_exit_bytes=int(s * V * early_rows.sum()),
               accepted_sum=int(a.sum()))
    full = s * V * len(L) * (2 * K + 1 + 2)
    if not (0 <= out["stream_bytes"] <= out["call_bytes"] <= full):
        raise AccountingError(f"bytes {out} above the full-length bound {full}")
    return out


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per streaming launch from the committed counter summary, if
    it was taken on the current kernel sources (else None)."""
    try:
        with open(PMC_SUMMARY) as f:
            txt = f.read()
    except OSError:
        return None, "no counter summary"
    m_h = re.search(r"source_sha256:\s*([0-9a-f]{64})", txt)
    m_t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not (m_h and m_t):
        return None, "counter summary unreadable"
    if m_h.group(1) != kernel_source_hash():
        return None, "kernel changed since the counters were taken"
    return float(m_t.group(1)), "rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-kernel scaled"


def tensor_sha256(t) -> str:
    """SHA-256 of a tensor's bytes (bf16 as its 16-bit patterns)."""
    import torch
    h = t.detach().contiguous().cpu()
    if h.dtype == torch.bfloat16:
        h = h.view(torch.int16)
    return hashlib.sha256(h.numpy().tobytes()).hexdigest()


# ---------------------------------------------------------------- timing helpers

def time_calls(fn, reps, stream, torch):
    """Median and mean (ms) of `reps` calls of fn(), each between two events.
    A spin kernel queued first keeps the GPU busy while the host queues the
    calls, so that the events time the GPU work, not the host's launch
    overhead."""
    ts = []
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        ts.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ts)
    return ms[len(ms) // 2], sum(ms) / len(ms)


def time_phases(call, reps, stream, torch, np):
    """Mean streaming-launch time and median whole-call time (ms) over `reps`
    calls: call(i, phases) enqueues the STREAM half, then the FINISH half,
    with events around the first half and around both."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in evs:
        for x in e:
            x.record(stream)  # creates the HIP events
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
    for i, (e0, e1, e2) in enumerate(evs):
        e0.record(stream)
        call(i, 1)
        e1.record(stream)
        call(i, 2)
        e2.record(stream)
    torch.cuda.synchronize()
    st = [a.elapsed_time(b) for a, b, _ in evs]
    ca = sorted(a.elapsed_time(c) for a, _, c in evs)
    return float(np.mean(st)), ca[len(ca) // 2], st


def time_stream_back_to_back(call, reps, stream, torch):
    """Mean streaming-launch time (ms): `reps` STREAM halves call(i, 1)
    launched back to back, one event pair around them all, so that no launch
    waits on an event (each pair of events around a single launch also spans
    its dispatch).  Rotating over the input sets keeps the reads from the
    last-level cache as in the timed steps."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
    e0.record(stream)
    for i in range(reps):
        call(i, 1)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def probe_offset(k: int, nbytes: int, span: int, stride: int) -> int:
    """Offset of the k-th plain read of `nbytes` (a multiple of 16) in a buffer
    of `span` bytes: at least `stride` past the previous read, 256-aligned,
    and the read ends inside the buffer."""
    if not (16 <= nbytes <= span - 256) or nbytes % 16:
        raise ValueError(f"read probe of {nbytes} bytes: outside [16, {span - 256}] or not a "
                         f"multiple of 16")
    step = max(stride, nbytes) // 256 * 256 + 256
    room = span - nbytes
    off = (k * step) % room // 256 * 256
    assert 0 <= off and off + nbytes <= span
    return off


class ReadProbe:
    """Plain contiguous reads (dspark_bench_read_probe) of a given byte count,
    each call at an offset at least 300 MB past the previous one in a 2.2 GB
    buffer, so that, like the rotating input sets, no call reads bytes left
    in the 256 MB last-level cache by the calls before it."""

    SPAN = 2_200_000_000
    STRIDE = 300_000_000

    def __init__(self, torch, dev):
        if not os.path.exists(BENCH_LIB):
            raise RuntimeError(f"{BENCH_LIB} is not built; run python -m "
                               "draft_verification_dspark_amd.build")
        self.lib = ctypes.CDLL(BENCH_LIB)
        self.lib.dspark_bench_read_probe.argtypes = [ctypes.c_void_p, ctypes.c_size_t,
                                                     ctypes.c_void_p, ctypes.c_void_p]
        self.lib.dspark_bench_read_probe.restype = ctypes.c_int
        self.torch = torch
        self.buf = torch.empty(self.SPAN, dtype=torch.uint8, device=dev)  # contents irrelevant
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)
        self.k = 0

    def call(self, nbytes, stream):
        nbytes = nbytes // 16 * 16
        off = probe_offset(self.k, nbytes, self.SPAN, self.STRIDE)
        self.k += 1
        st = self.lib.dspark_bench_read_probe(self.buf.data_ptr() + off, nbytes,
                                              self.sink.data_ptr(), stream.cuda_stream)
        if st != 0:
            raise RuntimeError(f"dspark_bench_read_probe returned {st}")

    def timed(self, nbytes, reps, stream, np):
        """Mean duration (ms) of `reps` calls launched back to back, one event
        pair around them all (as the streaming launches are timed), the host
        queued ahead."""
        torch = self.torch
        for _ in range(4):
            self.call(nbytes, stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(SPIN_CYCLES)
        e0.record(stream)
        for _ in range(reps):
            self.call(nbytes, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps


# ---------------------------------------------------------------- CPU baseline

_W = {}


def _cpu_worker_init(specs, root):
    """Attach the shared input arrays (a worker process of the CPU baseline)."""
    from multiprocessing import shared_memory

    import numpy as np
    if root not in sys.path:
        sys.path.insert(0, root)
    for name, (shm_name, shape, dtype) in specs.items():
        shm = shared_memory.SharedMemory(name=shm_name)
        _W[name + "_shm"] = shm
        _W[name] = np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf)


def _cpu_worker_verify(job):
    """The oracle's verification of this worker's requests."""
    import oracle
    lengths, part = job
    r = oracle.verify(_W["target"], _W["draft"], _W["drafted"], lengths, _W["temperature"],
                      _W["uniforms"], requests=part)
    keep = ("accepted", "tokens", "p_tok", "q_tok", "dist", "req_flags")
    return part, {k: r[k][part] for k in keep}


def _cpu_worker_ping(_):
    import oracle  # noqa: F401  (imported before the timing starts)
    return os.getpid()


def cpu_baseline(host: dict, threshold, budget, min_len, seconds: float, log):
    """The oracle (schedule, then verify) on full steps of one input set,
    requests split statically over one worker process per core (at most 16);
    returns the rate and the oracle's outputs of the first step."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    import numpy as np

    import oracle
    n = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
    B = host["drafted"].shape[0]
    parts = [list(range(i, B, n)) for i in range(n) if i < B]
    shms, specs = [], {}
    try:
        for k in ("target", "draft", "drafted", "temperature", "uniforms"):
            a = np.ascontiguousarray(host[k])
            shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            shms.append(shm)
            np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
            specs[k] = (shm.name, a.shape, a.dtype.str)
        ctx = mp.get_context("spawn")  # fresh interpreters: the workers never touch the GPU
        with ctx.Pool(len(parts), initializer=_cpu_worker_init, initargs=(specs, ROOT)) as pool:
            pool.map(_cpu_worker_ping, range(len(parts)))
            runs, pos, first = 0, 0, None
            t0 = time.perf_counter()
            while True:
                L, mask, surv = oracle.schedule(host["conf"], threshold, budget, min_len)
                res = pool.map(_cpu_worker_verify, [(L, p) for p in parts])
                if first is None:
                    first = dict(lengths=L, mask=mask, survival=surv, res=res)
                runs += 1
                pos += int(L.sum())
                el = time.perf_counter() - t0
                if el >= seconds or runs >= 200:
                    break
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    log(f"cpu oracle: {runs} steps in {el:.1f} s on {len(parts)} worker processes")
    return dict(rate=pos / el, runs=runs, seconds=el, cores=len(parts), model=model,
                first=first)


def parity_of_sample(first, gpu: dict, temperature, K):
    """The GPU's outputs of one input set against the oracle's, request by
    request: schedule bit for bit; accepted and tokens exact except where the
    oracle's uniform lies within 1e-6 of a decision edge (a boundary
    exception); p(y) and q(y) within 1e-5 relative."""
    import numpy as np

    import oracle
    out = dict(requests=0, schedule_exact=True, mismatches=0, boundary_exceptions=0,
               failures=0, worst_prob_rel=0.0, min_boundary_distance=None)
    if not (np.array_equal(first["lengths"], gpu["lengths"])
            and np.array_equal(first["mask"], gpu["mask"])
            and np.array_equal(first["survival"].view(np.uint32),
                               gpu["survival"].view(np.uint32))):
        out["schedule_exact"] = False
    dmin = np.inf
    for part, r in first["res"]:
        for i, b in enumerate(part):
            out["requests"] += 1
            if r["req_flags"][i]:
                out["failures"] += 1
                continue
            dmin = min(dmin, float(r["dist"][i]))
            same = (gpu["accepted"][b] == r["accepted"][i]
                    and np.array_equal(gpu["tokens"][b], r["tokens"][i]))
            if not same:
                out["mismatches"] += 1
                if r["dist"][i] <= oracle.BOUNDARY:
                    out["boundary_exceptions"] += 1
                else:
                    out["failures"] += 1
            if temperature[b] > 0:
                L = int(first["lengths"][b])
                for name in ("p_tok", "q_tok"):
                    g = gpu[name][b, :L].astype(np.float64)
                    o = r[name][i][:L]
                    tiny = (np.abs(g) < 1e-30) & (o < 1e-30)
                    rel = np.where(tiny, 0.0, np.abs(g - o) / np.maximum(o, 1e-300))
                    if rel.size:
                        out["worst_prob_rel"] = max(out["worst_prob_rel"], float(rel.max()))
                    if (rel > 1e-5).any():
                        out["failures"] += 1
    out["min_boundary_distance"] = None if dmin == np.inf else dmin
    return out


# ---------------------------------------------------------------- other rows

def row_measurements(ds, workloads, sets, outs, ws_v, dev, stream, torch, np, log, probe,
                     until=None):
    """The hot-path rows the headline step does not exercise, each timed
    apart (not part of `value`): the greedy rule, full-length blocks, a length
    sweep against the plain read, the schedule with a binding budget, the
    load-aware schedule, online calibration, Markov drafting and a
    mixed-temperature batch of 1024 requests.  With `until`, the rows run in
    that order and stop after the one of that name (for profiling a row)."""
    rows = {}

    def stop():
        return until is not None and until in rows
    n = len(sets)
    B, K, V = sets[0].B, sets[0].K, sets[0].V
    s = 2

    # G1: greedy rule on the same logits and scheduled lengths
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    st_ = torch.zeros(1, dtype=torch.int32, device=dev)

    def greedy(i, ph=3):
        ds.verify_greedy(sets[i % n].target, sets[i % n].drafted, outs[i % n]["lengths"],
                         accepted=acc, tokens=tok, dev_status=st_, ws=ws_v, stream=stream, phases=ph)
    for i in range(n):
        greedy(i)
    gb = [s * V * int((outs[i]["lengths"].cpu().numpy().astype(np.int64) + 1).sum()) for i in range(n)]
    _, t_c, _ = time_phases(greedy, 24, stream, torch, np)
    t_s = time_stream_back_to_back(greedy, 24, stream, torch)
    gbs = float(np.mean(gb)) / (t_s / 1e3) / 1e9
    rows["G1_verify_greedy"] = {"workload": "b64-k16-v151936 logits, scheduled lengths",
                                "stream_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                                "stream_us_mean": round(t_s * 1e3, 2), "call_us_median": round(t_c * 1e3, 2)}
    if stop():
        return rows

    # V1-V5 at full length: every block verified to K
    full = torch.full((B,), K, dtype=torch.int32, device=dev)
    accf = torch.empty(B, dtype=torch.int32, device=dev)
    tokf = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    ptf = torch.empty((B, K), dtype=torch.float32, device=dev)
    qtf = torch.empty((B, K), dtype=torch.float32, device=dev)

    def vlen(lx):
        def call(i, ph=3):
            w = sets[i % n]
            ds.verify(w.target, w.draft, w.drafted, lx, w.temperature, w.uniforms, accepted=accf,
                      tokens=tokf, p_tok=ptf, q_tok=qtf, dev_status=st_, ws=ws_v, stream=stream,
                      phases=ph)
        return call
    vfull = vlen(full)
    for i in range(n):
        vfull(i)
    fb = s * V * B * (2 * K + 1)
    _, t_c, _ = time_phases(vfull, 18, stream, torch, np)
    t_s = time_stream_back_to_back(vfull, 18, stream, torch)
    gbs = fb / (t_s / 1e3) / 1e9
    rows["V_full_length"] = {"workload": "b64-k16-v151936, every length = K (641.8 MB per pass)",
                             "stream_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                             "stream_us_mean": round(t_s * 1e3, 2), "call_us_median": round(t_c * 1e3, 2),
                             "positions_per_s": round(B * K / (t_c / 1e3), 1)}
    if stop():
        return rows

    # The streaming pass against its byte count: every length = L for several
    # L, a least-squares line through (bytes, time), and the plain contiguous
    # read of the same byte counts beside it.
    sweep = []
    for Lx in (0, 2, 4, 8, 16):
        vl = vlen(torch.full((B,), Lx, dtype=torch.int32, device=dev))
        for i in range(n):
            vl(i)
        by = s * V * B * (2 * Lx + 1)
        t_s = time_stream_back_to_back(vl, 18, stream, torch)
        t_p = probe.timed(by, 18, stream, np)
        sweep.append((by, t_s * 1e3, t_p * 1e3))
    xb = np.array([x[0] for x in sweep], dtype=np.float64)
    fit_s = np.polyfit(xb, [x[1] for x in sweep], 1)
    fit_p = np.polyfit(xb, [x[2] for x in sweep], 1)
    rows["V_length_sweep"] = {
        "workload": "b64-k16-v151936 logits, every length = L for L in 0, 2, 4, 8, 16",
        "points": [{"L": Lx, "bytes": int(by), "stream_us": round(ts, 2), "read_us": round(tp, 2)}
                   for Lx, (by, ts, tp) in zip((0, 2, 4, 8, 16), sweep)],
        "stream_slope_gbs": round(1e-3 / fit_s[0], 1), "stream_intercept_us": round(fit_s[1], 2),
        "read_slope_gbs": round(1e-3 / fit_p[0], 1), "read_intercept_us": round(fit_p[1], 2),
        "note": "read = dspark_bench_read_probe, a plain contiguous read of the same bytes in the "
                "same launch shape"}
    if stop():
        return rows

    # S3 and the mixed batch: workload b1024-k8-v151936 (temperatures 0 / 0.6 / 1)
    w5 = workloads.make(5, device=dev)
    B5, K5, V5 = w5.B, w5.K, w5.V
    ws_s5 = ds.workspace(ds.OP_SCHEDULE, B5, K5, 1, dev)
    ws_v5 = ds.workspace(ds.OP_VERIFY, B5, K5, V5, dev)
    L5 = torch.empty(B5, dtype=torch.int32, device=dev)
    m5 = torch.empty((B5, K5), dtype=torch.uint8, device=dev)
    c5 = torch.empty((B5, K5), dtype=torch.float32, device=dev)
    st5 = torch.zeros(1, dtype=torch.int32, device=dev)
    ds.schedule(w5.conf, w5.threshold, -1, w5.min_len, lengths=L5, mask=m5, survival=c5,
                dev_status=st5, ws=ws_s5, stream=stream)
    l_thr = int(L5.sum().item())

    def sched5():
        ds.schedule(w5.conf, w5.threshold, w5.budget, w5.min_len, lengths=L5, mask=m5,
                    survival=c5, dev_status=st5, ws=ws_s5, stream=stream)
    sched5()
    t_med, _ = time_calls(sched5, 30, stream, torch)
    rows["S1_S3_schedule_b1024"] = {"workload": "b1024-k8, threshold 0.3, budget 3072",
                                    "threshold_lengths_sum": l_thr, "budget": w5.budget,
                                    "budget_binds": l_thr > w5.budget,
                                    "call_us_median": round(t_med * 1e3, 2)}
    half = max(B5 * w5.min_len, l_thr // 2)

    def sched5b():
        ds.schedule(w5.conf, w5.threshold, half, w5.min_len, lengths=L5, mask=m5,
                    survival=c5, dev_status=st5, ws=ws_s5, stream=stream)
    sched5b()
    t_med, _ = time_calls(sched5b, 30, stream, torch)
    rows["S3_schedule_binding_b1024"] = {"workload": "b1024-k8, threshold 0.3, budget = half the "
                                                     "threshold lengths",
                                         "budget": half, "call_us_median": round(t_med * 1e3, 2)}
    # the load-aware schedule: threshold and budget derived on the device from
    # an engine load and the Deep Dive's throughput-curve table, its batch
    # sizes scaled 8x to tokens per forward pass
    curve = torch.tensor([[1, 35], [2, 67], [4, 125], [8, 220], [16, 360], [32, 520], [64, 650],
                          [128, 720]], dtype=torch.float32, device=dev)
    curve[:, 0] *= 8
    curve[:, 1] *= 8
    load = torch.tensor([48.0, 0.7], dtype=torch.float32, device=dev)  # queue 48 of 128, 70 % memory
    for name, conf_t, Bx, Kx in (("NEXT1_schedule_load_aware_b64", sets[0].conf, B, K),
                                 ("NEXT1_schedule_load_aware_b1024", w5.conf, B5, K5)):
        Lx = torch.empty(Bx, dtype=torch.int32, device=dev)
        mx = torch.empty((Bx, Kx), dtype=torch.uint8, device=dev)
        cx = torch.empty((Bx, Kx), dtype=torch.float32, device=dev)
        tx = torch.empty(1, dtype=torch.float32, device=dev)
        bx = torch.empty(1, dtype=torch.int32, device=dev)
        sx = torch.zeros(1, dtype=torch.int32, device=dev)
        wsx = ds.workspace(ds.OP_SCHEDULE, Bx, Kx, 1, dev)

        def sched_la():
            ds.schedule_load_aware(conf_t, load, 128.0, 1.0, 0.20, 0.75, curve, 2.0, 1,
                                   lengths=Lx, mask=mx, survival=cx, tau_out=tx, budget_out=bx,
                                   dev_status=sx, ws=wsx, stream=stream)
        sched_la()
        t_med, _ = time_calls(sched_la, 30, stream, torch)
        rows[name] = {"workload": f"b{Bx}-k{Kx} confidences, load 48/128 queue and 0.7 memory, "
                                  "tau 0.20..0.75, throughput curve of the Deep Dive x8, slot cost 2",
                      "tau": round(float(tx.item()), 6), "budget": int(bx.item()),
                      "lengths_sum": int(Lx.sum().item()), "call_us_median": round(t_med * 1e3, 2)}
    # online calibration: temperature scaling of the raw scores, and one
    # round into the calibration window (every 4th call ends a window)
    for name, conf_t, Bx, Kx, acc_t in (("NEXT2_calibration_b64", sets[0].conf, B, K, outs[0]["acc"]),
                                       ("NEXT2_calibration_b1024", w5.conf, B5, K5, None)):
        th = torch.linspace(1.0, 1.5, Kx, dtype=torch.float32, device=dev)
        calx = torch.empty((Bx, Kx), dtype=torch.float32, device=dev)
        sx = torch.zeros(1, dtype=torch.int32, device=dev)
        state = ds.calib_state(Kx, 10, dev)
        ece = torch.zeros(1, dtype=torch.float32, device=dev)
        accx = acc_t if acc_t is not None else torch.zeros(Bx, dtype=torch.int32, device=dev)
        Lx = outs[0]["lengths"] if acc_t is not None else torch.full((Bx,), Kx, dtype=torch.int32,
                                                                      device=dev)

        def cal_call():
            ds.calibrate(conf_t, th, out=calx, dev_status=sx, stream=stream)

        def obs_call():
            ds.calib_observe(calx, Lx, accx, th, 0.01, 0.05, 4, 10, state, ece_out=ece,
                             dev_status=sx, stream=stream)
        cal_call()
        obs_call()
        t_cal, _ = time_calls(cal_call, 30, stream, torch)
        t_obs, _ = time_calls(obs_call, 32, stream, torch)
        rows[name] = {"workload": f"b{Bx}-k{Kx} scores, 10 ECE bins, window 4 rounds",
                      "calibrate_us_median": round(t_cal * 1e3, 2),
                      "observe_us_median": round(t_obs * 1e3, 2),
                      "call_us_median": round((t_cal + t_obs) * 1e3, 2)}
    # Markov logit-bias drafting of the workload's block (rank 256): per
    # position an MFMA contraction over U (V x r) and a draw per request
    r_m = 256
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    Um = (0.05 * torch.randn((V, r_m), generator=g, device=dev)).to(torch.bfloat16)
    Vmm = (0.05 * torch.randn((V, r_m), generator=g, device=dev)).to(torch.bfloat16)
    y0m = torch.randint(0, V, (B,), generator=g, device=dev, dtype=torch.int32)
    um = torch.rand((B, K), generator=g, device=dev)
    cm = torch.empty_like(sets[0].draft)
    ym = torch.empty((B, K), dtype=torch.int32, device=dev)
    qm = torch.empty((B, K), dtype=torch.float32, device=dev)
    stm = torch.zeros(1, dtype=torch.int32, device=dev)
    wsm = ds.workspace(ds.OP_MARKOV_DRAFT, B, K, V, dev)

    def draft_call():
        ds.markov_draft(sets[0].draft, Um, Vmm, 0.1, y0m, sets[0].temperature, um, corrected=cm,
                        drafted=ym, q_tok=qm, dev_status=stm, ws=wsm, stream=stream)
    draft_call()
    t_med, _ = time_calls(draft_call, 10, stream, torch)
    step_bytes = V * r_m * 2 + 2 * B * V * s       # U once, base rows read, corrected rows written
    step_flops = 2.0 * V * r_m * B
    rows["NEXT3_markov_draft_b64"] = {
        "workload": f"b{B}-k{K}-v{V}, rank {r_m}, bf16 (U, V ~ N(0, 0.05^2)), T = 1",
        "call_us_median": round(t_med * 1e3, 2), "us_per_position": round(t_med * 1e3 / K, 2),
        "bytes_per_position": step_bytes, "hbm_gbs": round(step_bytes * K / (t_med / 1e3) / 1e9, 1),
        "mfma_tflops": round(step_flops * K / (t_med / 1e3) / 1e12, 2)}
    sched5()  # back to the configured lengths for the verify row
    a5 = torch.empty(B5, dtype=torch.int32, device=dev)
    t5 = torch.empty((B5, K5 + 1), dtype=torch.int32, device=dev)
    p5 = torch.empty((B5, K5), dtype=torch.float32, device=dev)
    q5 = torch.empty((B5, K5), dtype=torch.float32, device=dev)

    def v5(i, ph=3):
        ds.verify(w5.target, w5.draft, w5.drafted, L5, w5.temperature, w5.uniforms, accepted=a5,
                  tokens=t5, p_tok=p5, q_tok=q5, dev_status=st5, ws=ws_v5, stream=stream, phases=ph)
    v5(0)
    torch.cuda.synchronize()
    L = L5.cpu().numpy().astype(np.int64)
    T = w5.temperature.cpu().numpy()
    b5 = s * V5 * int((((2 * L + 1) * (T > 0)) + ((L + 1) * (T == 0))).sum())
    _, t_c, _ = time_phases(v5, 12, stream, torch, np)
    t_s = time_stream_back_to_back(v5, 12, stream, torch)
    gbs = b5 / (t_s / 1e3) / 1e9
    rows["V_G1_mixed_b1024"] = {"workload": "b1024-k8-v151936, temperatures 0 / 0.6 / 1, scheduled",
                                "positions": int(L.sum()), "stream_bytes": b5,
                                "stream_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                                "stream_us_mean": round(t_s * 1e3, 2),
                                "call_us_median": round(t_c * 1e3, 2),
                                "positions_per_s": round(int(L.sum()) / (t_c / 1e3), 1)}
    flags = {"G1/full": int(st_.item()), "b1024": int(st5.item()), "markov": int(stm.item())}
    assert not any(flags.values()), f"device status flags set: {flags}"
    log("rows: " + "; ".join(
        f"{k} {v.get('stream_gbs', v.get('call_us_median', v.get('stream_slope_gbs')))}"
        for k, v in rows.items()))
    return rows


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--sets", type=int, default=6)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the separate timings of the other hot-path rows")
    ap.add_argument("--rows-until", default=None, metavar="ROW",
                    help="run the rows in order and stop after this one (G1_verify_greedy, "
                         "V_full_length or V_length_sweep; for profiling a row)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this path runs on a "
              f"single device and has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.sets < 1:
        print("--steps >= 1, --warmup >= 0 and --sets >= 1 are required", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import draft_verification_dspark_amd as ds
    import workloads

    ds.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"device: {torch.cuda.get_device_name(dev)}")

    sets = [workloads.make(args.workload, seed_offset=100 * i, device=dev) for i in range(args.sets)]
    w0 = sets[0]
    B, K, V = w0.B, w0.K, w0.V
    s = 2 if w0.dtype == "bf16" else 4
    log(f"workload {w0.name}: B={B} K={K} V={V} {w0.dtype}; {args.sets} input sets")

    # preallocated outputs and workspace (the library never allocates)
    outs = []
    for w in sets:
        outs.append(dict(
            lengths=torch.empty(B, dtype=torch.int32, device=dev),
            mask=torch.empty((B, K), dtype=torch.uint8, device=dev),
            surv=torch.empty((B, K), dtype=torch.float32, device=dev),
            acc=torch.empty(B, dtype=torch.int32, device=dev),
            tok=torch.empty((B, K + 1), dtype=torch.int32, device=dev),
            pt=torch.empty((B, K), dtype=torch.float32, device=dev),
            qt=torch.empty((B, K), dtype=torch.float32, device=dev),
            st=torch.zeros(1, dtype=torch.int32, device=dev)))
    stream = torch.cuda.current_stream(dev)
    ws_s = ds.workspace(ds.OP_SCHEDULE, B, K, 1, dev)
    ws_v = ds.workspace(ds.OP_VERIFY, B, K, V, dev)
    ws_sv = ds.workspace(ds.OP_SCHEDULE_VERIFY, B, K, V, dev)

    def step(i, phases=ds.PHASE_ALL):
        """One step (or one half of it): dspark_schedule_verify of input set i."""
        w, o = sets[i % len(sets)], outs[i % len(sets)]
        ds.schedule_verify(w.conf, w.threshold, w.budget, w.min_len, w.target, w.draft, w.drafted,
                           w.temperature, w.uniforms, lengths=o["lengths"], mask=o["mask"],
                           survival=o["surv"], accepted=o["acc"], tokens=o["tok"], p_tok=o["pt"],
                           q_tok=o["qt"], dev_status=o["st"], ws=ws_sv, stream=stream,
                           phases=phases)

    def step_two_calls(i):
        """The same step as two calls: dspark_schedule, then dspark_verify."""
        w, o = sets[i % len(sets)], outs[i % len(sets)]
        ds.schedule(w.conf, w.threshold, w.budget, w.min_len, lengths=o["lengths"], mask=o["mask"],
                    survival=o["surv"], dev_status=o["st"], ws=ws_s, stream=stream)
        ds.verify(w.target, w.draft, w.drafted, o["lengths"], w.temperature, w.uniforms,
                  accepted=o["acc"], tokens=o["tok"], p_tok=o["pt"], q_tok=o["qt"],
                  dev_status=o["st"], ws=ws_v, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # every input set verified once, so that the accounting reads outputs a
    # step has written (whatever --warmup is)
    for i in range(len(sets)):
        step(i)
    torch.cuda.synchronize()
    acct, gpu_out = [], []
    for i in range(len(sets)):
        o, w = outs[i], sets[i]
        if int(o["st"].item()) != 0:
            raise RuntimeError(f"device status {int(o['st'].item())} on input set {i}")
        hostd = {k: workloads.to_numpy(o[k]) for k in ("lengths", "mask", "surv", "acc", "tok",
                                                        "pt", "qt")}
        acct.append(account_set(hostd["lengths"], hostd["acc"], workloads.to_numpy(w.temperature),
                                K, V, s))
        gpu_out.append(hostd)
    log("accounting: positions per set " + str([a["positions"] for a in acct]))

    # Timed region: K steps launched directly on one stream with nothing
    # between the calls.
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)  # the host queues all K steps while it runs
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per = [acct[i % len(sets)] for i in range(args.steps)]
    n_pos = sum(a["positions"] for a in per)
    s_bytes = sum(a["stream_bytes"] for a in per)
    c_bytes = sum(a["call_bytes"] for a in per)
    e_bytes = sum(a["early_exit_bytes"] for a in per)
    value = n_pos / (total_ms / 1e3)
    log(f"timed {args.steps} steps: {total_ms:.3f} ms, {total_ms / args.steps * 1e3:.1f} us/step, "
        f"{value:.0f} positions/s")

    # Kernel timing: the streaming launches of the same steps back to back
    # (the launch time the roofline uses); the same steps as their two halves,
    # events around the streaming launch (its spread, and the time with the
    # dispatch); then whole calls, events around the call.
    b2b_ms = time_stream_back_to_back(lambda i, ph: step(i, ph), args.steps, stream, torch)
    str_mean, _, str_ms = time_phases(lambda i, ph: step(i, ph), args.steps, stream, torch, np)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for e in ev:
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in ev]
    stream_gbs = s_bytes / (b2b_ms * args.steps / 1e3) / 1e9
    stream_ev_gbs = s_bytes / (sum(str_ms) / 1e3) / 1e9
    call_gbs = c_bytes / (sum(call_ms) / 1e3) / 1e9
    log(f"streaming launch mean {b2b_ms * 1e3:.2f} us back to back ({stream_gbs:.0f} GB/s), "
        f"{np.mean(str_ms) * 1e3:.2f} us between events ({stream_ev_gbs:.0f} GB/s); call "
        f"median {np.median(call_ms) * 1e3:.2f} us ({call_gbs:.0f} GB/s)")

    # the same steps as two calls (schedule, then verify), timed the same way
    for i in range(len(sets)):
        step_two_calls(i)
    torch.cuda.synchronize()
    t2a = torch.cuda.Event(enable_timing=True)
    t2b = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
    t2a.record(stream)
    for i in range(args.steps):
        step_two_calls(i)
    t2b.record(stream)
    torch.cuda.synchronize()
    two_ms = t2a.elapsed_time(t2b)
    log(f"the same {args.steps} steps as two calls: {two_ms / args.steps * 1e3:.1f} us/step")
    traffic, traffic_note = measured_traffic()

    # the plain contiguous read of the same byte count in the same launch
    # shape, and of 2 GB: what a kernel that only reads achieves
    probe = ReadProbe(torch, dev)
    ref_bytes = round(s_bytes / args.steps) // 16 * 16
    ref_ms = probe.timed(ref_bytes, 30, stream, np)
    ref_gbs = ref_bytes / (ref_ms / 1e3) / 1e9
    big_bytes = 2_000_000_000
    big_ms = probe.timed(big_bytes, 8, stream, np)
    big_gbs = big_bytes / (big_ms / 1e3) / 1e9

    def pct(x, q):
        return round(float(np.percentile(np.asarray(x) * 1e3, q)), 2)

    hashes = {f"set{i}": {k: tensor_sha256(getattr(w, k))
                          for k in ("target", "draft", "drafted", "conf", "temperature", "uniforms")}
              for i, w in enumerate(sets)}
    mean_acc = float(np.mean([a["accepted_sum"] / B for a in acct]))
    waste = float(np.mean([1 - a["accepted_sum"] / max(1, a["positions"]) for a in acct]))

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w0.name}: V={V}, B={B}, K={K}, bf16 logits, T=1, threshold 0.2, budget 512",
            "logits": w0.dtype,
            "arithmetic": "bf16 logits widened exactly to fp32; fp32 exponentials, fp64 sums and "
                          "probabilities",
            "input_sets": len(sets),
            "step": "dspark_schedule_verify (schedule inside the streaming launch)",
            "two_call_us_per_step": round(two_ms / args.steps * 1e3, 2),
            "positions_per_set": [a["positions"] for a in acct],
            "stream_bytes_per_set": [a["stream_bytes"] for a in acct],
            "call_bytes_per_set": [a["call_bytes"] for a in acct],
            "input_sha256": hashes,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_stream_rows (streaming launch of dspark_schedule_verify, schedule worked "
                      "out inside)",
            "achieved": round(stream_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(stream_gbs / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "traffic_note": traffic_note,
            "algorithmic_bytes_per_launch": round(s_bytes / args.steps),
            "launch_us_mean": round(b2b_ms * 1e3, 2),
            "kernel_timing": "the STREAM halves of dspark_schedule_verify_phase (the streaming "
                             "launch alone) of the timed steps launched back to back on the "
                             "call's stream, one event pair around them all, mean per launch",
            "launch_us_between_events": {
                "mean": round(float(np.mean(str_ms)) * 1e3, 2),
                "p10_p50_p90": [pct(str_ms, 10), pct(str_ms, 50), pct(str_ms, 90)],
                "gbs": round(stream_ev_gbs, 1),
                "note": "an event pair around each STREAM half, the FINISH half after it: "
                        "each interval also spans the launch's dispatch"},
            "call_bytes_per_call": round(c_bytes / args.steps),
            "call_achieved": round(call_gbs, 1),
            "call_frac": round(call_gbs / HBM_PEAK_GBS, 4),
            "call_us_median": round(float(np.median(call_ms)) * 1e3, 2),
            "call_us_p10_p90": [pct(call_ms, 10), pct(call_ms, 90)],
            "call_note": "the whole dspark_schedule_verify call: streaming bytes plus the rejected "
                         "row pairs re-read, over the call's event-timed duration",
            "early_exit_bytes_per_call": round(e_bytes / args.steps),
            "read_ceiling_2gb": {"gbs": round(big_gbs, 1), "frac": round(big_gbs / HBM_PEAK_GBS, 4),
                                 "note": "dspark_bench_read_probe over 2 GB, 8 calls back to back"},
            "contiguous_read_reference": {
                "bytes": ref_bytes, "us_mean": round(ref_ms * 1e3, 2), "gbs": round(ref_gbs, 1),
                "frac": round(ref_gbs / HBM_PEAK_GBS, 4),
                "note": "dspark_bench_read_probe: the same bytes read contiguously, same launch "
                        "shape, 30 calls back to back at rotating offsets, mean per call"},
        },
        "accepted_mean": round(mean_acc, 3),
        "waste_ratio": round(waste, 4),
    }
    result["rows"] = None if args.no_rows else row_measurements(
        ds, workloads, sets, outs, ws_v, dev, stream, torch, np, log, probe, until=args.rows_until)

    if args.calibrate_copy > 0:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.rand(n, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            torch.add(src, 0.0, out=dst)   # reads and writes n*4 bytes
        torch.cuda.synchronize()
        log(f"calibration copy: 5 x {args.calibrate_copy} MiB read + written")
        del src, dst

    if not args.no_cpu_baseline:
        cw = sets[0]
        host = {k: workloads.to_numpy(getattr(cw, k))
                for k in ("conf", "target", "draft", "drafted", "temperature", "uniforms")}
        cb = cpu_baseline(host, cw.threshold, cw.budget, cw.min_len, args.cpu_seconds, log)
        g0 = gpu_out[0]
        par = parity_of_sample(cb["first"], dict(lengths=g0["lengths"], mask=g0["mask"],
                                                 survival=g0["surv"], accepted=g0["acc"],
                                                 tokens=g0["tok"], p_tok=g0["pt"], q_tok=g0["qt"]),
                               host["temperature"], K)
        result["cpu_baseline"] = {
            "value": round(cb["rate"], 2),
            "unit": "positions/s",
            "cores": cb["cores"],
            "kind": "oracle",
            "model": cb["model"],
            "sample": f"{cb['runs']} full step(s) (oracle schedule, then oracle verify of all {B} "
                      f"requests) of {cw.name} seed+0 in {cb['seconds']:.1f} s wall; numpy fp64, "
                      f"{cb['cores']} worker processes, requests split statically",
        }
        result["parity"] = dict(par, input_set="set0 (seed+0)",
                                note="GPU outputs of the accounting pass against the CPU oracle's "
                                     "first step; boundary exceptions are mismatches where the "
                                     "oracle's uniform lies within 1e-6 of a decision edge")
        log(f"parity set0: {par}")
        if par["failures"] or not par["schedule_exact"]:
            print(json.dumps(result), flush=True)
            raise SystemExit("GPU outputs disagree with the oracle")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
