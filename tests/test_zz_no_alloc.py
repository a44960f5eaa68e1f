"""dspark_schedule_verify_noalloc (the built-in device scratch in place of a
caller workspace) against dspark_schedule_verify with a workspace: the same
outputs, bit for bit, on two calls in a row, the second with a smaller
input; sizes past the scratch are refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import draft_verification_dspark_amd as ds
import oracle
import workloads
from parity import compare_schedule, compare_verify, host

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
KEYS = ("lengths", "mask", "survival", "accepted", "tokens", "p_tok", "q_tok", "dev_status")


def _noalloc_through_abi(w):
    """The C ABI called directly, every output preallocated."""
    B, K = w.B, w.K
    out = dict(lengths=torch.empty(B, dtype=torch.int32, device=DEV),
               mask=torch.empty((B, K), dtype=torch.uint8, device=DEV),
               survival=torch.empty((B, K), dtype=torch.float32, device=DEV),
               accepted=torch.empty(B, dtype=torch.int32, device=DEV),
               tokens=torch.empty((B, K + 1), dtype=torch.int32, device=DEV),
               p_tok=torch.empty((B, K), dtype=torch.float32, device=DEV),
               q_tok=torch.empty((B, K), dtype=torch.float32, device=DEV),
               dev_status=torch.zeros(1, dtype=torch.int32, device=DEV))
    lib = ds.load_library()
    st = lib.dspark_schedule_verify_noalloc(
        w.conf.data_ptr(), float(w.threshold), int(w.budget), int(w.min_len),
        out["lengths"].data_ptr(), out["mask"].data_ptr(), out["survival"].data_ptr(),
        w.target.data_ptr(), w.draft.data_ptr(), ds.DSPARK_BF16, B, K, w.V,
        w.drafted.data_ptr(), w.temperature.data_ptr(), w.uniforms.data_ptr(),
        out["accepted"].data_ptr(), out["tokens"].data_ptr(), out["p_tok"].data_ptr(),
        out["q_tok"].data_ptr(), out["dev_status"].data_ptr(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, ds.dspark_status_string(st)
    return out


def test_noalloc_matches_the_workspace_call_twice_second_smaller():
    cases = [workloads.make(3, device=DEV),                               # b64-k16-v151936
             workloads.make(3, device=DEV, B=24, V=70001, seed_offset=100)]
    for i, w in enumerate(cases):
        print(f"no-alloc call {i}: {w.name} B={w.B} K={w.K} V={w.V}", flush=True)
        got = _noalloc_through_abi(w)
        ref = ds.schedule_verify(w.conf, w.threshold, w.budget, w.min_len, w.target, w.draft,
                                 w.drafted, w.temperature, w.uniforms)
        torch.cuda.synchronize()
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), k
        # and the oracle's bar, on the same inputs
        ref_s = oracle.schedule(host(w.conf), w.threshold, w.budget, w.min_len)
        compare_schedule((host(got["lengths"]), host(got["mask"]), host(got["survival"])), ref_s)
        g = {k: host(got[k]) for k in ("accepted", "tokens", "p_tok", "q_tok", "dev_status")}
        ro = oracle.verify(host(w.target), host(w.draft), host(w.drafted), ref_s[0],
                           host(w.temperature), host(w.uniforms))
        compare_verify(g, ro, ref_s[0], host(w.temperature)).assert_ok()
        assert int(g["dev_status"][0]) == 0


def test_noalloc_refuses_sizes_past_the_scratch():
    lib = ds.load_library()
    P = 4096
    B, K, V = 1024, 8, 151936            # 24 MB of workspace: more than the 16 MiB scratch
    assert ds.dspark_workspace_bytes(ds.OP_SCHEDULE_VERIFY, B, K, V) > ds.SCRATCH_BYTES
    st = lib.dspark_schedule_verify_noalloc(P, 0.3, 3072, 1, P, None, None, P, P, 1, B, K, V, P,
                                            P, P, P, P, None, None, P, None)
    assert st == ds.ERR_SCRATCH
    assert "scratch" in ds.dspark_status_string(st)
