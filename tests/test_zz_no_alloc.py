"""The decode step without a workspace (adamas_decode_step_noalloc, for callers
that cannot allocate): through the C ABI, two calls in a row -- the 32K
Llama-3.1-8B-shaped layer, then a smaller ragged batch -- each equal to
adamas_decode_step on the same inputs (selections, distances and query codes
bit for bit, the output within the 2e-3 bar and, since the kernels are the
same, bit for bit too)."""
import numpy as np
import pytest

import workloads as W
from helpers import DeviceCase, assert_out_close, from_dev

pytestmark = pytest.mark.gpu


def run_both(A, torch, wl, budget):
    case = DeviceCase(wl, A, torch)
    ref = case.decode(budget, want_debug=True)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
    sel = torch.full((wl.B, wl.Hq, budget), -7, dtype=torch.int32, device="cuda")
    dist = torch.zeros((wl.B, wl.Hq, wl.cap), dtype=torch.int16, device="cuda")
    qc = torch.zeros((wl.B, wl.Hq, 32), dtype=torch.uint8, device="cuda")
    A.decode_step_noalloc(case.q, case.k, case.v, case.codes, case.kv_len, budget, wl.scale, out, sel_idx=sel,
                          dist=dist, q_codes=qc)
    torch.cuda.synchronize()
    got = (from_dev(out), from_dev(sel), from_dev(dist, np.uint16), from_dev(qc))
    return ref, got


def test_noalloc_matches_workspace_entry_point_twice():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import sparse_attention_long_fwht_amd as A
    cases = [(W.llama(0, cap=32768, budget=128), 128),
             (W.llama(81, cap=3000, budget=300, B=2, Hq=8, Hkv=2, kv_len=np.array([3000, 1537], np.int32)), 300)]
    for wl, budget in cases:  # the second call is the smaller input
        ref, got = run_both(A, torch, wl, budget)
        o_r, s_r, d_r, q_r = ref
        o, s, d, q = got
        assert np.array_equal(q, q_r)
        for b in range(wl.B):
            L = int(wl.kv_len[b])
            assert np.array_equal(d[b, :, :L], d_r[b, :, :L])
        assert np.array_equal(s, s_r)
        assert_out_close(o, o_r)
        assert np.array_equal(o, o_r)
