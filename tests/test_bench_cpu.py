"""The benchmark's host-side accounting on the CPU: positions and bytes come
only from outputs within their bounds, and the plain-read yardstick never
reads past its buffer."""
import numpy as np
import pytest

import bench

K, V, S = 16, 151936, 2


def test_accounting_of_a_known_batch():
    L = np.array([3, 0, 16, 5], np.int32)
    a = np.array([1, 0, 16, 5], np.int32)
    T = np.array([1.0, 1.0, 0.7, 0.0], np.float32)
    r = bench.account_set(L, a, T, K, V, S)
    # rows: 2L+1 for T > 0, L+1 for T = 0; +2 for a sampled request with a < L
    stream_rows = 7 + 1 + 33 + 6
    assert r["positions"] == 24
    assert r["stream_bytes"] == S * V * stream_rows
    assert r["call_bytes"] == S * V * (stream_rows + 2)
    assert r["early_exit_bytes"] == S * V * ((2 * 2 + 2) + 2 + 2 * 17 + 6)
    assert r["accepted_sum"] == 22


def test_accounting_refuses_unwritten_outputs():
    # what torch.empty buffers that no step wrote can hold: arbitrary int32s
    rng = np.random.default_rng(0)
    garbage = rng.integers(-2 ** 31, 2 ** 31 - 1, size=64, dtype=np.int64).astype(np.int32)
    ok = np.full(64, 4, np.int32)
    T = np.ones(64, np.float32)
    with pytest.raises(bench.AccountingError):
        bench.account_set(garbage, ok, T, K, V, S)
    with pytest.raises(bench.AccountingError):
        bench.account_set(ok, garbage, T, K, V, S)


@pytest.mark.parametrize("L,a", [([17], [0]), ([-1], [0]), ([4], [5]), ([4], [-1])])
def test_accounting_bounds(L, a):
    with pytest.raises(bench.AccountingError):
        bench.account_set(np.array(L, np.int32), np.array(a, np.int32), np.ones(1, np.float32),
                          K, V, S)


def test_accounting_stays_below_the_full_length_bound():
    L = np.full(64, K, np.int32)
    a = np.zeros(64, np.int32)
    r = bench.account_set(L, a, np.ones(64, np.float32), K, V, S)
    assert r["call_bytes"] == S * V * 64 * (2 * K + 1 + 2)


def test_read_probe_offsets_stay_inside_the_buffer():
    span, stride = bench.ReadProbe.SPAN, bench.ReadProbe.STRIDE
    for nbytes in (16, 82_450_608, 641_785_856, 2_000_000_000, span - 256):
        for k in range(40):
            off = bench.probe_offset(k, nbytes, span, stride)
            assert off % 256 == 0 and off + nbytes <= span
    for bad in (0, 8, 24, span, span - 16, 124190097207 * 80):
        with pytest.raises(ValueError):
            bench.probe_offset(0, bad, span, stride)


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
