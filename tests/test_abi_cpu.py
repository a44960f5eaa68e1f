"""The C ABI library on the CPU: it loads, exports every function the header
declares, and its synchronous argument checks return before any GPU call."""
import ctypes
import os
import re

import pytest

import draft_verification_dspark_amd as ds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header="dspark.h", prefix="DSPARK_API"):
    with open(os.path.join(ROOT, "include", header)) as f:
        src = f.read()
    return re.findall(prefix + r"\s+[\w\s\*]+?\b(dspark_\w+)\s*\(", src)


def test_exports_every_declared_symbol():
    lib = ds.load_library()
    names = _declared()
    assert set(names) == set(ds.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    # the measurement aids live in the benchmark's library only
    for n in ("dspark_read_probe", "dspark_set_stream_events", "dspark_bench_read_probe"):
        assert not hasattr(lib, n), n


BENCH_LIB = os.path.join(ROOT, "draft_verification_dspark_amd", "libdspark_bench.so")


def test_bench_library_exports_its_header():
    lib = ctypes.CDLL(BENCH_LIB)
    names = _declared("dspark_bench.h", r'__attribute__\(\(visibility\("default"\)\)\)')
    assert names == ["dspark_bench_read_probe"]
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(8):
        assert ds.dspark_status_string(s)
    assert ds.dspark_status_string(99) == "unknown status"


def test_workspace_sizes():
    w = ds.dspark_workspace_bytes
    assert w(ds.OP_VERIFY, 0, 4, 10) == 0
    assert w(ds.OP_VERIFY, 1, 65, 10) == 0
    assert w(7, 1, 1, 1) == 0
    a = w(ds.OP_VERIFY, 64, 16, 151936)
    assert a > 0 and a % 256 == 0
    assert w(ds.OP_VERIFY, 128, 16, 151936) > a
    assert w(ds.OP_VERIFY_GREEDY, 64, 16, 151936) == a
    assert w(ds.OP_SCHEDULE, 64, 16, 1) >= 64 * 16 * 4 + 64 * 4
    assert w(ds.OP_MARKOV_DRAFT, 64, 16, 151936) >= 64 * (151936 // 64) * 16


P = 4096  # any 256-aligned non-null "pointer": the checks never dereference it


@pytest.mark.parametrize("args,code", [
    ((None, 4, 4, 0.1, -1, 1, P, None, None, P, P, 10 ** 6, None), 1),
    ((P, 0, 4, 0.1, -1, 1, P, None, None, P, P, 10 ** 6, None), 2),
    ((P, 4, 0, 0.1, -1, 1, P, None, None, P, P, 10 ** 6, None), 2),
    ((P, 4, 4, 0.1, 3, 1, P, None, None, P, P, 10 ** 6, None), 4),
    ((P, 4, 4, 0.1, -1, 5, P, None, None, P, P, 10 ** 6, None), 4),
    ((P, 4, 4, 0.1, -1, -1, P, None, None, P, P, 10 ** 6, None), 4),
    ((P, 4, 4, 0.1, -1, 1, P, None, None, P, P, 8, None), 5),
    ((P, 4, 4, 0.1, -1, 1, P, None, None, P, P + 8, 10 ** 6, None), 5),
])
def test_schedule_argument_errors(args, code):
    assert ds.load_library().dspark_schedule(*args) == code


def _la(**kw):
    a = dict(conf=P, B=4, K=4, load=P, qmax=10.0, mmax=8.0, tmin=0.2, tmax=0.75, curve=P, n=8,
             cost=1.0, ml=1, L=P, mask=None, surv=None, tout=None, bout=None, st=P, ws=P,
             nb=10 ** 6, stream=None)
    a.update(kw)
    return ds.load_library().dspark_schedule_load_aware(
        a["conf"], a["B"], a["K"], a["load"], a["qmax"], a["mmax"], a["tmin"], a["tmax"], a["curve"],
        a["n"], a["cost"], a["ml"], a["L"], a["mask"], a["surv"], a["tout"], a["bout"], a["st"],
        a["ws"], a["nb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(load=None), 1), (dict(conf=None), 1), (dict(B=0), 2), (dict(ml=5), 4), (dict(nb=8), 5),
    (dict(qmax=0.0), 7), (dict(mmax=-1.0), 7), (dict(qmax=float("inf")), 7),
    (dict(tmin=0.8), 7), (dict(tmin=-0.1), 7), (dict(tmax=float("nan")), 7),
    (dict(n=65), 7), (dict(n=-1), 7), (dict(curve=None), 7), (dict(cost=float("nan")), 7),
])
def test_schedule_load_aware_argument_errors(kw, code):
    assert _la(**kw) == code


@pytest.mark.parametrize("args,code", [
    ((None, P, 4, 4, P, P, None), 1), ((P, None, 4, 4, P, P, None), 1), ((P, P, 4, 4, None, P, None), 1),
    ((P, P, 0, 4, P, P, None), 2), ((P, P, 4, 0, P, P, None), 2), ((P, P, 4, 65, P, P, None), 2),
])
def test_calibrate_argument_errors(args, code):
    assert ds.load_library().dspark_calibrate(*args) == code


def test_calib_state_bytes():
    f = ds.load_library().dspark_calib_state_bytes
    assert f(16, 10) == 8 * (1 + 3 * 16 + 3 * 10)
    assert f(0, 10) == 0 and f(65, 10) == 0 and f(4, 0) == 0 and f(4, 65) == 0


def _obs(**kw):
    a = dict(c=P, L=None, acc=P, B=4, K=4, th=P, lr=0.01, tmin=0.05, win=10, nb=10, st=P,
             sb=10 ** 4, ece=None, ds_=P, stream=None)
    a.update(kw)
    return ds.load_library().dspark_calib_observe(a["c"], a["L"], a["acc"], a["B"], a["K"], a["th"],
                                                  a["lr"], a["tmin"], a["win"], a["nb"], a["st"],
                                                  a["sb"], a["ece"], a["ds_"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(c=None), 1), (dict(acc=None), 1), (dict(th=None), 1), (dict(st=None), 1), (dict(ds_=None), 1),
    (dict(B=0), 2), (dict(K=65), 2), (dict(lr=float("nan")), 7), (dict(tmin=0.0), 7),
    (dict(win=0), 7), (dict(nb=0), 7), (dict(nb=65), 7), (dict(sb=8), 5), (dict(st=P + 4), 5),
])
def test_calib_observe_argument_errors(kw, code):
    assert _obs(**kw) == code


def _md(**kw):
    a = dict(base=P, dtype=1, B=2, K=3, V=100, U=P, Vm=P, r=64, scale=1.0, y0=P, T=P, u=P, c=P,
             y=P, q=None, st=P, ws=P, nb=10 ** 9, stream=None)
    a.update(kw)
    return ds.load_library().dspark_markov_draft(
        a["base"], a["dtype"], a["B"], a["K"], a["V"], a["U"], a["Vm"], a["r"], a["scale"], a["y0"],
        a["T"], a["u"], a["c"], a["y"], a["q"], a["st"], a["ws"], a["nb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(base=None), 1), (dict(U=None), 1), (dict(Vm=None), 1), (dict(y0=None), 1), (dict(c=None), 1),
    (dict(B=0), 2), (dict(K=0), 2), (dict(V=0), 2), (dict(r=8), 2), (dict(r=24), 2), (dict(r=272), 2),
    (dict(dtype=5), 3), (dict(U=P + 8), 7), (dict(nb=16), 5),
])
def test_markov_draft_argument_errors(kw, code):
    assert _md(**kw) == code


def _v(**kw):
    a = dict(t=P, d=P, dtype=1, B=2, K=4, V=100, y=P, L=None, T=P, u=P, acc=P, tok=P, pt=None,
             qt=None, st=P, ws=P, nb=10 ** 9, stream=None)
    a.update(kw)
    return ds.load_library().dspark_verify(a["t"], a["d"], a["dtype"], a["B"], a["K"], a["V"],
                                           a["y"], a["L"], a["T"], a["u"], a["acc"], a["tok"],
                                           a["pt"], a["qt"], a["st"], a["ws"], a["nb"], a["stream"])


def test_verify_argument_errors():
    assert _v(t=None) == 1
    assert _v(d=None) == 1
    assert _v(u=None) == 1
    assert _v(st=None) == 1
    assert _v(B=0) == 2
    assert _v(K=65) == 2
    assert _v(V=0) == 2
    assert _v(dtype=2) == 3
    assert _v(nb=16) == 5
    assert _v(ws=P + 64) == 5
    lib = ds.load_library()
    # greedy needs no draft, temperature or uniforms
    assert lib.dspark_verify_greedy(P, 1, 2, 4, 100, P, None, P, P, P, P, 16, None) == 5
    assert lib.dspark_verify_greedy(P, 1, 2, 4, 100, None, None, P, P, P, P, 10 ** 9, None) == 1


def test_binding_refuses_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("draft_verification_dspark_amd")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(RuntimeError):
            mod.load_library(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


def test_read_probe_argument_errors():
    # checks come before any launch: NULL pointers, sizes, alignment
    lib = ctypes.CDLL(BENCH_LIB)
    f = lib.dspark_bench_read_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert f(None, 16, P, None) == 1
    assert f(P, 16, None, None) == 1
    assert f(P, 0, P, None) == ds.ERR_PARAM
    assert f(P, 24, P, None) == ds.ERR_PARAM
    assert f(P + 8, 32, P, None) == ds.ERR_PARAM


def test_phase_argument_errors():
    lib = ds.load_library()
    args = (P, P, 1, 2, 4, 100, P, None, P, P, P, P, None, None, P, P, 10 ** 9, None)
    assert lib.dspark_verify_phase(0, *args) == ds.ERR_PARAM
    assert lib.dspark_verify_phase(4, *args) == ds.ERR_PARAM
    assert lib.dspark_verify_phase(-1, *args) == ds.ERR_PARAM
    # a split call keeps one launch batch (2048 requests) in the workspace
    big = (P, P, 1, 2049, 4, 100, P, None, P, P, P, P, None, None, P, P, 10 ** 12, None)
    assert lib.dspark_verify_phase(1, *big) == 2
    assert lib.dspark_verify_phase(2, *big) == 2
    g = (P, 1, 2, 4, 100, P, None, P, P, P, P, 16, None)
    assert lib.dspark_verify_greedy_phase(1, *g) == 5
    assert lib.dspark_verify_greedy_phase(5, *g[:-2], 10 ** 9, None) == ds.ERR_PARAM
    sv = (P, 0.1, -1, 1, P, None, None, P, P, 1, 2, 4, 100, P, P, P, P, P, None, None, P, P,
          10 ** 9, None)
    assert lib.dspark_schedule_verify_phase(3, *sv[:-2], 8, None) == 5
    assert lib.dspark_schedule_verify_phase(7, *sv) == ds.ERR_PARAM


# ---------------------------------------------------------------- binding checks

def _cpu_case(B=2, K=4, V=64):
    import torch
    t = torch.zeros((B, K + 1, V), dtype=torch.bfloat16)
    d = torch.zeros((B, K, V), dtype=torch.bfloat16)
    y = torch.zeros((B, K), dtype=torch.int32)
    T = torch.ones(B, dtype=torch.float32)
    u = torch.zeros((B, K + 1), dtype=torch.float32)
    c = torch.ones((B, K), dtype=torch.float32)
    return t, d, y, T, u, c


def _bad_outputs(B=2, K=4):
    import torch
    return [
        ("accepted", torch.zeros(B + 1, dtype=torch.int32)),
        ("accepted", torch.zeros(B, dtype=torch.int64)),
        ("tokens", torch.zeros((B, K), dtype=torch.int32)),
        ("tokens", torch.zeros((K + 1, B), dtype=torch.int32).t()),   # not contiguous
        ("p_tok", torch.zeros((B, K), dtype=torch.float64)),
        ("q_tok", torch.zeros((B, K + 1), dtype=torch.float32)),
        ("dev_status", torch.zeros(2, dtype=torch.int32)),
        ("dev_status", torch.zeros(1, dtype=torch.float32)),
    ]


@pytest.mark.parametrize("i", range(8))
def test_verify_binding_refuses_bad_outputs(i):
    t, d, y, T, u, _ = _cpu_case()
    name, bad = _bad_outputs()[i]
    with pytest.raises(ValueError, match=name):
        ds.verify(t, d, y, None, T, u, **{name: bad})


@pytest.mark.parametrize("i", range(8))
def test_schedule_verify_binding_refuses_bad_outputs(i):
    t, d, y, T, u, c = _cpu_case()
    name, bad = _bad_outputs()[i]
    with pytest.raises(ValueError, match=name):
        ds.schedule_verify(c, 0.1, -1, 1, t, d, y, T, u, **{name: bad})


@pytest.mark.parametrize("i", [0, 1, 2, 3, 6, 7])
def test_verify_greedy_binding_refuses_bad_outputs(i):
    t, _, y, _, _, _ = _cpu_case()
    name, bad = _bad_outputs()[i]
    with pytest.raises(ValueError, match=name):
        ds.verify_greedy(t, y, None, **{name: bad})


def test_schedule_binding_refuses_bad_outputs():
    import torch
    c = torch.ones((3, 4), dtype=torch.float32)
    for kw in (dict(lengths=torch.zeros(4, dtype=torch.int32)),
               dict(mask=torch.zeros((3, 4), dtype=torch.bool)),
               dict(survival=torch.zeros((4, 3), dtype=torch.float32)),
               dict(dev_status=torch.zeros(1, dtype=torch.int64))):
        with pytest.raises(ValueError, match=next(iter(kw))):
            ds.schedule(c, 0.1, -1, 1, **kw)


def test_binding_refuses_a_small_workspace():
    t, d, y, T, u, _ = _cpu_case()

    class Small:
        nbytes, ptr = 16, P
    with pytest.raises(ValueError, match="workspace"):
        ds.verify(t, d, y, None, T, u, ws=Small())


def _sv(conf=P, thr=0.1, budget=-1, ml=1, L=P, t=P, d=P, dtype=1, B=2, K=4, V=100, y=P, T=P,
        u=P, acc=P, tok=P, st=P, ws=P, nb=10 ** 9):
    lib = ds.load_library()
    return lib.dspark_schedule_verify(conf, thr, budget, ml, L, None, None, t, d, dtype, B, K, V,
                                      y, T, u, acc, tok, None, None, st, ws, nb, None)


def test_schedule_verify_argument_errors():
    # the checks of both halves come before any launch
    assert _sv(ws=None) == 1
    assert _sv(conf=None) == 1
    assert _sv(L=None) == 1
    assert _sv(t=None) == 1
    assert _sv(d=None) == 1
    assert _sv(u=None) == 1
    assert _sv(B=0) == 2
    assert _sv(K=65) == 2
    assert _sv(V=0) == 2
    assert _sv(dtype=2) == 3
    assert _sv(budget=1, ml=1) == 4          # budget below B * min_len
    assert _sv(ml=5) == 4
    need = ds.dspark_workspace_bytes(ds.OP_SCHEDULE_VERIFY, 2, 4, 100)
    assert _sv(nb=need - 1) == 5
    assert _sv(ws=P + 64) == 5


def test_schedule_verify_workspace_is_both_layouts():
    w = ds.dspark_workspace_bytes
    for B, K, V in ((64, 16, 151936), (1, 4, 1024), (1024, 8, 151936)):
        v = w(ds.OP_VERIFY, B, K, V)
        s = w(ds.OP_SCHEDULE, B, K, 1)
        assert w(ds.OP_SCHEDULE_VERIFY, B, K, V) == (v + 255) // 256 * 256 + s
    assert w(ds.OP_SCHEDULE_VERIFY, 1, 65, 10) == 0


def test_noalloc_size_checks_come_first():
    # no-alloc call: sizes are checked before the scratch's address is
    # looked up (no GPU call), and sizes past the 16 MiB scratch are refused
    lib = ds.load_library()
    args = lambda B, K, V: (P, 0.3, -1, 1, P, None, None, P, P, 1, B, K, V, P, P, P, P, P, None,
                            None, P, None)
    assert lib.dspark_schedule_verify_noalloc(*args(1024, 8, 151936)) == 8
    assert lib.dspark_schedule_verify_noalloc(*args(0, 8, 151936)) == 2
    assert lib.dspark_schedule_verify_noalloc(*args(4, 65, 100)) == 2
    assert ds.dspark_workspace_bytes(ds.OP_SCHEDULE_VERIFY, 330, 16, 151936) <= ds.SCRATCH_BYTES
    assert ds.dspark_workspace_bytes(ds.OP_SCHEDULE_VERIFY, 331, 16, 151936) > ds.SCRATCH_BYTES
    assert "scratch" in ds.dspark_status_string(8)
