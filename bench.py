"""Benchmark: verified draft positions per second and achieved HBM bandwidth of
confidence-scheduled block verification on one MI355X.

One step = the schedule and the verification of one batch of the
V=151936, B=64, K=16 workload (bf16 logits, T=1, threshold 0.2, budget 512;
seeded synthetic inputs resident in HBM), as one dspark_schedule_verify call,
which works the schedule out inside the streaming launch; the same steps as
two calls (dspark_schedule, then dspark_verify) are timed beside it
(``config.two_call_us_per_step``).  Six input sets (seed offsets
0, 100, ..., 500; 641 MB each) rotate so that no step reads logits left in the
256 MB last-level cache by the step before.

The timed region launches the K steps directly on one stream with nothing
in between, behind a spin kernel that lets the host queue them all first
(``--graphs`` replays each step from its own HIP graph instead, which is
slower on this stack).  Kernel times (the call, the streaming
pass) come from a separate pass over the same steps with events around each
call and, recorded by the library on the same stream, around each streaming
launch.

Prints ONE JSON line on stdout.  ``value`` = sum of verified positions
(sum_b L_b) per second of schedule + verify.  ``roofline`` reports the
dominant kernel, the streaming pass (k_stream_rows), against the 8 TB/s HBM
peak: its algorithmic bytes per launch, s*V*sum_b rows_b with rows_b = 2 L_b + 1
(T > 0) or L_b + 1 (T = 0), over its average duration, timed with HIP events
that the library records on its own stream around that launch.  ``traffic`` is
the HBM bytes per launch that rocprofv3 counters measured for the same kernel
(profiles/k_stream_rows_b64_k16_v151936_pmc.md), used only while the kernel
sources still hash to the recorded value.  ``contiguous_read_reference`` times
dspark_read_probe, a plain read of the same byte count in the same launch
shape, as the yardstick of what a read-only kernel reaches at this size.  ``cpu_baseline`` times the CPU
oracle on a bounded sample of the same workload.

``rows`` times, apart from the step, the hot-path rows the step does not
exercise: the greedy rule on the same logits, full-length blocks, the
schedule with a binding budget, the load-aware schedule (threshold and budget
from an engine load and a throughput curve), online calibration (temperature
scaling and one round into the calibration window), Markov logit-bias drafting
of the workload's block and a mixed-temperature batch of 1024 requests
(``--no-rows`` skips them).  ``V_length_sweep`` times the streaming pass at
uniform lengths 0..16 beside the plain read of the same bytes and fits each
with a line: bandwidth (slope) and fixed cost per launch (intercept).

--calibrate-copy N runs, after the timed steps, a plain elementwise copy of
N MiB (read N MiB, write N MiB) five times: the reference kernel of known size
for the FETCH_SIZE / WRITE_SIZE counter runs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SPIN_CYCLES = 20_000_000  # GPU clock cycles the pre-queued spin kernel runs for
PMC_SUMMARY = os.path.join(ROOT, "profiles", "k_stream_rows_b64_k16_v151936_pmc.md")
KERNEL_SOURCES = [os.path.join(ROOT, "draft_verification_dspark_amd", "csrc", f)
                  for f in ("verify.hip", "device.hpp", "args.hpp", "schedule_core.hpp",
                            "schedule_args.hpp")]
METRIC = "verified draft positions/sec and achieved HBM GB/s vs peak (V=151936, B=64, K=16)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(w, lengths, accepted, temperature) -> int:
    """Bytes the whole verify call must read (streaming pass + residual rows)."""
    s = 2 if w.dtype == "bf16" else 4
    L = lengths.astype("int64")
    a = accepted.astype("int64")
    T = temperature
    soft = T > 0
    rows = ((2 * L + 1) + 2 * (a < L)) * soft + (L + 1) * (~soft)
    return int(s * w.V * rows.sum())


def early_exit_bytes(w, lengths, accepted, temperature) -> int:
    """The early-exit lower bound: the rows a verifier that could stop at the
    first rejection would still read, s*V*sum[2(a+1) + 2*rejected] for T > 0
    and s*V*sum(a+1) for T = 0; beside the streaming pass's bytes it shows
    the over-read of rows past the first rejection."""
    s = 2 if w.dtype == "bf16" else 4
    L = lengths.astype("int64")
    a = accepted.astype("int64")
    soft = temperature > 0
    rows = (2 * (a + 1) + 2 * (a < L)) * soft + (a + 1) * (~soft)
    return int(s * w.V * rows.sum())


def stream_bytes(w, lengths, temperature) -> int:
    """Bytes the streaming pass must read: every scheduled row once."""
    s = 2 if w.dtype == "bf16" else 4
    L = lengths.astype("int64")
    soft = temperature > 0
    rows = (2 * L + 1) * soft + (L + 1) * (~soft)
    return int(s * w.V * rows.sum())


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


def time_calls(fn, reps, stream, torch):
    """Median and mean of `reps` calls of fn(), each between two events.  A
    spin kernel queued first keeps the GPU busy while the host queues the
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


class ReadProbe:
    """Plain contiguous reads (dspark_read_probe) of a given byte count, each
    call at an offset at least 300 MB past the previous one in a 2.2 GB
    buffer, so that, like the rotating input sets, no call reads bytes left
    in the 256 MB last-level cache by the calls before it."""

    SPAN = 2_200_000_000
    STRIDE = 300_000_000

    def __init__(self, ds, torch, dev):
        self.ds, self.torch = ds, torch
        self.buf = torch.empty(self.SPAN, dtype=torch.uint8, device=dev)  # contents irrelevant
        self.sink = torch.zeros(4, dtype=torch.int32, device=dev)
        self.k = 0

    def call(self, nbytes, stream):
        nbytes = nbytes // 16 * 16
        step = max(self.STRIDE, nbytes) // 256 * 256 + 256
        room = self.SPAN - nbytes
        off = (self.k * step) % room // 256 * 256
        self.k += 1
        self.ds.read_probe(self.buf[off:], nbytes, self.sink, stream)

    def timed(self, nbytes, reps, stream, np):
        """Mean event-timed duration (ms) of `reps` calls, the host queued ahead."""
        torch = self.torch
        for _ in range(4):
            self.call(nbytes, stream)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for e in evs:
            for x in e:
                x.record(stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(SPIN_CYCLES)
        for e0, e1 in evs:
            e0.record(stream)
            self.call(nbytes, stream)
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.mean([a.elapsed_time(b) for a, b in evs]))


def row_measurements(ds, workloads, sets, outs, ws_v, dev, stream, torch, np, log, probe):
    """The hot-path rows the headline step does not exercise, each timed
    apart (not part of `value`): the greedy rule, full-length blocks, a
    binding budget, the load-aware schedule, online calibration, Markov
    drafting and a mixed-temperature batch of 1024 requests."""
    rows = {}
    n = len(sets)
    B, K, V = sets[0].B, sets[0].K, sets[0].V
    s = 2

    def stream_timed(call, reps):
        """Mean streaming-pass time (events recorded by the library) and
        median whole-call time over `reps` calls; call(i, before, after)."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
                torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for e in evs:
            for x in e:
                x.record(stream)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            torch.cuda._sleep(SPIN_CYCLES)  # the host queues ahead of the GPU
        for i, (c0, s0, s1, c1) in enumerate(evs):
            c0.record(stream)
            ds.dspark_set_stream_events(s0, s1)
            call(i)
            ds.dspark_set_stream_events(None, None)
            c1.record(stream)
        torch.cuda.synchronize()
        st = [s0.elapsed_time(s1) for _, s0, s1, _ in evs]
        ca = sorted(c0.elapsed_time(c1) for c0, _, _, c1 in evs)
        return float(np.mean(st)), ca[len(ca) // 2]

    # G1: greedy rule on the same logits and scheduled lengths
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    st_ = torch.zeros(1, dtype=torch.int32, device=dev)
    for i in range(n):
        ds.verify_greedy(sets[i].target, sets[i].drafted, outs[i]["lengths"], accepted=acc,
                         tokens=tok, dev_status=st_, ws=ws_v, stream=stream)
    gb = [s * V * int((outs[i]["lengths"].cpu().numpy().astype(np.int64) + 1).sum()) for i in range(n)]
    t_s, t_c = stream_timed(lambda i: ds.verify_greedy(
        sets[i % n].target, sets[i % n].drafted, outs[i % n]["lengths"], accepted=acc, tokens=tok,
        dev_status=st_, ws=ws_v, stream=stream), 24)
    gbs = float(np.mean(gb)) / (t_s / 1e3) / 1e9
    rows["G1_verify_greedy"] = {"workload": "b64-k16-v151936 logits, scheduled lengths",
                                "stream_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                                "stream_us_mean": round(t_s * 1e3, 2), "call_us_median": round(t_c * 1e3, 2)}

    # V1-V5 at full length: every block verified to K
    full = torch.full((B,), K, dtype=torch.int32, device=dev)
    accf = torch.empty(B, dtype=torch.int32, device=dev)
    tokf = torch.empty((B, K + 1), dtype=torch.int32, device=dev)
    ptf = torch.empty((B, K), dtype=torch.float32, device=dev)
    qtf = torch.empty((B, K), dtype=torch.float32, device=dev)

    def vfull(i):
        w = sets[i % n]
        ds.verify(w.target, w.draft, w.drafted, full, w.temperature, w.uniforms, accepted=accf,
                  tokens=tokf, p_tok=ptf, q_tok=qtf, dev_status=st_, ws=ws_v, stream=stream)
    for i in range(n):
        vfull(i)
    fb = s * V * B * (2 * K + 1)
    t_s, t_c = stream_timed(vfull, 18)
    gbs = fb / (t_s / 1e3) / 1e9
    rows["V_full_length"] = {"workload": "b64-k16-v151936, every length = K (641.8 MB per pass)",
                             "stream_gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                             "stream_us_mean": round(t_s * 1e3, 2), "call_us_median": round(t_c * 1e3, 2),
                             "positions_per_s": round(B * K / (t_c / 1e3), 1)}

    # The streaming pass against its byte count: every length = L for several
    # L, a least-squares line through (bytes, time), and the plain contiguous
    # read of the same byte counts beside it.  The slope is the pass's
    # bandwidth once it runs; the intercept its fixed cost per launch.
    sweep = []
    for Lx in (0, 2, 4, 8, 16):
        lx = torch.full((B,), Lx, dtype=torch.int32, device=dev)

        def vl(i, lx=lx):
            w = sets[i % n]
            ds.verify(w.target, w.draft, w.drafted, lx, w.temperature, w.uniforms, accepted=accf,
                      tokens=tokf, p_tok=ptf, q_tok=qtf, dev_status=st_, ws=ws_v, stream=stream)
        for i in range(n):
            vl(i)
        by = s * V * B * (2 * Lx + 1)
        t_s, _ = stream_timed(vl, 18)
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
        "note": "read = dspark_read_probe, a plain contiguous read of the same bytes in the same "
                "launch shape"}

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
    # the same confidences under a budget that binds (half the threshold
    # lengths): the radix select of the budget cut runs
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
    Um = ((torch.randint(-256, 257, (V, r_m), generator=g, device=dev).float() / 256.0)
          .to(torch.bfloat16))
    Vmm = ((torch.randint(-256, 257, (V, r_m), generator=g, device=dev).float() / 256.0)
           .to(torch.bfloat16))
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
        "workload": f"b{B}-k{K}-v{V}, rank {r_m}, bf16 (U, V fixed-point synthetic), T = 1",
        "call_us_median": round(t_med * 1e3, 2), "us_per_position": round(t_med * 1e3 / K, 2),
        "bytes_per_position": step_bytes, "hbm_gbs": round(step_bytes * K / (t_med / 1e3) / 1e9, 1),
        "mfma_tflops": round(step_flops * K / (t_med / 1e3) / 1e12, 2)}
    sched5()  # back to the configured lengths for the verify row
    a5 = torch.empty(B5, dtype=torch.int32, device=dev)
    t5 = torch.empty((B5, K5 + 1), dtype=torch.int32, device=dev)
    p5 = torch.empty((B5, K5), dtype=torch.float32, device=dev)
    q5 = torch.empty((B5, K5), dtype=torch.float32, device=dev)

    def v5(i):
        ds.verify(w5.target, w5.draft, w5.drafted, L5, w5.temperature, w5.uniforms, accepted=a5,
                  tokens=t5, p_tok=p5, q_tok=q5, dev_status=st5, ws=ws_v5, stream=stream)
    v5(0)
    torch.cuda.synchronize()
    L = L5.cpu().numpy().astype(np.int64)
    T = w5.temperature.cpu().numpy()
    b5 = s * V5 * int((((2 * L + 1) * (T > 0)) + ((L + 1) * (T == 0))).sum())
    t_s, t_c = stream_timed(v5, 12)
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
    ap.add_argument("--graphs", action="store_true",
                    help="replay each timed step from its own HIP graph (slower on this stack)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this path runs on a "
              f"single device and has no multi-GPU mode", file=sys.stderr)
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
    log(f"workload {w0.name}: B={B} K={K} V={V} {w0.dtype}; {args.sets} input sets")

    # preallocated outputs and workspaces (the library never allocates)
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
    ws_s = ds.workspace(ds.OP_SCHEDULE, B, K, 1, dev)
    ws_v = ds.workspace(ds.OP_VERIFY, B, K, V, dev)
    ws_sv = ds.workspace(ds.OP_SCHEDULE_VERIFY, B, K, V, dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, cur, ev=None):
        """One step on stream `cur`: dspark_schedule_verify (the schedule
        worked out inside the streaming pass); with `ev` = three events:
        around the call, and (recorded by the library) around the streaming
        launch."""
        w, o = sets[i % len(sets)], outs[i % len(sets)]
        if ev is not None:
            ev[0].record(cur)
            ds.dspark_set_stream_events(ev[1], ev[2])
        ds.schedule_verify(w.conf, w.threshold, w.budget, w.min_len, w.target, w.draft, w.drafted,
                           w.temperature, w.uniforms, lengths=o["lengths"], mask=o["mask"],
                           survival=o["surv"], accepted=o["acc"], tokens=o["tok"], p_tok=o["pt"],
                           q_tok=o["qt"], dev_status=o["st"], ws=ws_sv, stream=cur)
        if ev is not None:
            ds.dspark_set_stream_events(None, None)
            ev[3].record(cur)

    def step_two_calls(i, cur):
        """The same step as two calls: dspark_schedule, then dspark_verify."""
        w, o = sets[i % len(sets)], outs[i % len(sets)]
        ds.schedule(w.conf, w.threshold, w.budget, w.min_len, lengths=o["lengths"], mask=o["mask"],
                    survival=o["surv"], dev_status=o["st"], ws=ws_s, stream=cur)
        ds.verify(w.target, w.draft, w.drafted, o["lengths"], w.temperature, w.uniforms,
                  accepted=o["acc"], tokens=o["tok"], p_tok=o["pt"], q_tok=o["qt"],
                  dev_status=o["st"], ws=ws_v, stream=cur)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # per-set positions and algorithmic bytes (outputs are deterministic per set)
    pos, nbytes, sbytes, mbytes, accs = [], [], [], [], []
    for i in range(len(sets)):
        o, w = outs[i], sets[i]
        L = o["lengths"].cpu().numpy()
        a = o["acc"].cpu().numpy()
        T = w.temperature.cpu().numpy()
        assert int(o["st"].item()) == 0, "device status flags set on synthetic inputs"
        pos.append(int(L.sum()))
        nbytes.append(algorithmic_bytes(w, L, a, T))
        sbytes.append(stream_bytes(w, L, T))
        mbytes.append(early_exit_bytes(w, L, a, T))
        accs.append((a, L))

    # Kernel timing pass: direct launches with events around the call and,
    # recorded by the library on the same stream, around the streaming
    # launch.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in ev:
        for x in e:
            x.record(stream)           # creates the HIP events
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)  # the host queues ahead: events time GPU work only
    for i in range(args.steps):
        step(i, stream, ev[i])
    torch.cuda.synchronize()
    ver_ms = [e[0].elapsed_time(e[3]) for e in ev]
    str_ms = [e[1].elapsed_time(e[2]) for e in ev]
    assert all(0 < t <= v for t, v in zip(str_ms, ver_ms)), "stream events outside the call"

    # Timed region: K steps launched directly on one stream with nothing
    # between the calls (an event between kernels delays the next one); with
    # --graphs each step is replayed from its own HIP graph instead.
    graphs = None
    if args.graphs:
        try:
            graphs = []
            for i in range(args.steps):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(i, torch.cuda.current_stream(dev))
                graphs.append(g)
            for g in graphs[: len(sets)]:
                g.replay()             # first replays are warm-up
            torch.cuda.synchronize()
        except Exception as ex:        # no graph support: launch directly
            log(f"graph capture unavailable ({ex}); timing direct launches")
            graphs = None
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # a spin kernel queued first: the host queues all K steps while it runs,
    # so the region times the GPU's work, not the host's launch rate
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
    t_start.record(stream)
    for i in range(args.steps):
        if graphs is not None:
            graphs[i].replay()
        else:
            step(i, stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    n_pos = sum(pos[i % len(sets)] for i in range(args.steps))
    n_bytes = sum(nbytes[i % len(sets)] for i in range(args.steps))
    s_bytes = sum(sbytes[i % len(sets)] for i in range(args.steps))
    value = n_pos / (total_ms / 1e3)
    verify_gbs = n_bytes / (sum(ver_ms) / 1e3) / 1e9
    stream_gbs = s_bytes / (sum(str_ms) / 1e3) / 1e9
    log(f"timed {args.steps} steps ({'graphs' if graphs is not None else 'direct'}): {total_ms:.3f} ms, "
        f"{total_ms / args.steps * 1e3:.1f} us/step; kernel pass: schedule + verify call median "
        f"{np.median(ver_ms)*1e3:.1f} us ({verify_gbs:.0f} GB/s); streaming pass median "
        f"{np.median(str_ms)*1e3:.1f} us ({stream_gbs:.0f} GB/s)")
    # the same steps as two calls (schedule, then verify), timed the same way
    for i in range(args.warmup):
        step_two_calls(i, stream)
    torch.cuda.synchronize()
    t2a = torch.cuda.Event(enable_timing=True)
    t2b = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
    t2a.record(stream)
    for i in range(args.steps):
        step_two_calls(i, stream)
    t2b.record(stream)
    torch.cuda.synchronize()
    two_ms = t2a.elapsed_time(t2b)
    log(f"the same {args.steps} steps as two calls: {two_ms / args.steps * 1e3:.1f} us/step")
    # the streaming pass alone (dspark_verify after dspark_schedule), its
    # launch timed by library-recorded events as above
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in ev2:
        for x in e:
            x.record(stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        torch.cuda._sleep(SPIN_CYCLES)
    for i in range(args.steps):
        w, o = sets[i % len(sets)], outs[i % len(sets)]
        ds.schedule(w.conf, w.threshold, w.budget, w.min_len, lengths=o["lengths"], mask=o["mask"],
                    survival=o["surv"], dev_status=o["st"], ws=ws_s, stream=stream)
        ev2[i][2].record(stream)
        ds.dspark_set_stream_events(ev2[i][0], ev2[i][1])
        ds.verify(w.target, w.draft, w.drafted, o["lengths"], w.temperature, w.uniforms,
                  accepted=o["acc"], tokens=o["tok"], p_tok=o["pt"], q_tok=o["qt"],
                  dev_status=o["st"], ws=ws_v, stream=stream)
        ds.dspark_set_stream_events(None, None)
        ev2[i][3].record(stream)
    torch.cuda.synchronize()
    alone_ms = [e[0].elapsed_time(e[1]) for e in ev2]
    vonly_ms = [e[2].elapsed_time(e[3]) for e in ev2]
    alone_gbs = s_bytes / (sum(alone_ms) / 1e3) / 1e9
    mean_acc = float(np.mean([a.mean() for a, _ in accs]))
    waste = float(np.mean([1 - a.sum() / max(1, L.sum()) for a, L in accs]))
    traffic, traffic_note = measured_traffic()
    # the plain contiguous read of the same byte count in the same launch
    # shape: what a kernel that only reads achieves at this size
    probe = ReadProbe(ds, torch, dev)
    ref_bytes = round(s_bytes / args.steps) // 16 * 16
    ref_ms = probe.timed(ref_bytes, 30, stream, np)
    ref_gbs = ref_bytes / (ref_ms / 1e3) / 1e9
    # and of 2 GB: the read bandwidth this GPU reaches at all
    big_bytes = 2_000_000_000
    big_ms = probe.timed(big_bytes, 8, stream, np)
    big_gbs = big_bytes / (big_ms / 1e3) / 1e9

    def pct(x, q):
        return round(float(np.percentile(np.asarray(x) * 1e3, q)), 2)
    # every input set scheduled once (short runs leave some unscheduled), so
    # that the rows read valid lengths
    for i in range(len(sets)):
        w, o = sets[i], outs[i]
        ds.schedule(w.conf, w.threshold, w.budget, w.min_len, lengths=o["lengths"], mask=o["mask"],
                    survival=o["surv"], dev_status=o["st"], ws=ws_s, stream=stream)
    torch.cuda.synchronize()

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
            "input_sets": len(sets),
            "launch": "hip graph per step" if graphs is not None else "direct",
            "step": "dspark_schedule_verify (schedule inside the streaming launch)",
            "two_call_us_per_step": round(two_ms / args.steps * 1e3, 2),
            "positions_per_step": pos,
            "verify_bytes_per_call": nbytes,
            "stream_bytes_per_call": sbytes,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "k_stream_rows<FUSED> (streaming pass of dspark_schedule_verify, schedule "
                      "worked out inside)",
            "achieved": round(stream_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(stream_gbs / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else round(traffic),
            "traffic_note": traffic_note,
            "algorithmic_bytes_per_launch": round(s_bytes / args.steps),
            "launch_us_mean": round(float(np.mean(str_ms)) * 1e3, 2),
            "call_gbs": round(verify_gbs, 1),
            "call_us_median": round(float(np.median(ver_ms)) * 1e3, 2),
            "kernel_timing": "separate pass over the same steps, events around each call and "
                             "(library-recorded, same stream) around each streaming launch; the "
                             "streaming launch works out the schedule as well",
            "launch_us_p10_p50_p90": [pct(str_ms, 10), pct(str_ms, 50), pct(str_ms, 90)],
            "call_us_p10_p90": [pct(ver_ms, 10), pct(ver_ms, 90)],
            "early_exit": {
                "bytes_per_call": round(sum(mbytes[i % len(sets)] for i in range(args.steps))
                                        / args.steps),
                "verify_bytes_per_call": round(n_bytes / args.steps),
                "note": "the rows a verifier stopping at the first rejection would read, beside "
                        "the whole call's algorithmic bytes (streaming pass + residual rows)"},
            "streaming_pass_alone": {
                "us_mean": round(float(np.mean(alone_ms)) * 1e3, 2), "gbs": round(alone_gbs, 1),
                "frac": round(alone_gbs / HBM_PEAK_GBS, 4),
                "verify_call_us_p10_p50_p90": [pct(vonly_ms, 10), pct(vonly_ms, 50),
                                               pct(vonly_ms, 90)],
                "note": "the streaming launch of dspark_verify after a separate dspark_schedule "
                        "(no schedule inside), same steps, same event timing"},
            "read_ceiling_2gb": {"gbs": round(big_gbs, 1), "frac": round(big_gbs / HBM_PEAK_GBS, 4),
                                 "note": "dspark_read_probe over 2 GB, events around the call"},
            "contiguous_read_reference": {
                "bytes": ref_bytes, "us_mean": round(ref_ms * 1e3, 2), "gbs": round(ref_gbs, 1),
                "frac": round(ref_gbs / HBM_PEAK_GBS, 4),
                "note": "dspark_read_probe: the same bytes read contiguously, same launch shape, "
                        "events around the call"},
        },
        "accepted_mean": round(mean_acc, 3),
        "waste_ratio": round(waste, 4),
        "rows": None if args.no_rows else row_measurements(ds, workloads, sets, outs, ws_v, dev,
                                                             stream, torch, np, log, probe),
    }

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
        import oracle
        cw = sets[0]
        conf = workloads.to_numpy(cw.conf)
        tgt = workloads.to_numpy(cw.target)
        dft = workloads.to_numpy(cw.draft)
        y = workloads.to_numpy(cw.drafted)
        T = workloads.to_numpy(cw.temperature)
        u = workloads.to_numpy(cw.uniforms)
        runs, cpu_pos, t0 = 0, 0, time.perf_counter()
        while True:
            L, _, _ = oracle.schedule(conf, cw.threshold, cw.budget, cw.min_len)
            oracle.verify(tgt, dft, y, L, T, u)
            runs += 1
            cpu_pos += int(L.sum())
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or runs >= 400:
                break
        result["cpu_baseline"] = {
            "value": round(cpu_pos / el, 2),
            "unit": "positions/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"{runs} full step(s) (schedule + verify, all {B} requests) of {cw.name} "
                      f"seed+0, {el:.1f} s wall, numpy fp64, single thread",
        }
        log(f"cpu oracle: {runs} runs in {el:.1f} s")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
