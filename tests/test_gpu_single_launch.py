"""The single-launch decode step (scan, in-kernel hand-off, select + attend in
one kernel) against the two-kernel step and the oracle: bit-identical
selections and outputs, on the shapes that take it (and a check that they do),
through HIP graph replays (every replay is a new generation of the hand-off
flags), with a workspace shared with two-kernel calls in between."""
import numpy as np
import pytest

import workloads as W
from helpers import DeviceCase, from_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import sparse_attention_long_fwht_amd as A
    import oracle
    yield A, torch, oracle
    A.decode_launch_mode(0)


def both_modes(case, budget, **kw):
    """decode() in launch mode 1 and 0; returns both results and launch counts."""
    A = case.A
    res, counts = [], []
    for mode in (1, 0):
        A.decode_launch_mode(mode)
        res.append(case.decode(budget, want_debug=True, **kw))
        counts.append(A.last_launch_count())
    A.decode_launch_mode(0)
    return res, counts


def assert_same(r1, r0):
    for a, b in zip(r1, r0):
        assert np.array_equal(a, b)


CASES = {
    "tiny": (lambda: W.tiny(), None, {}),
    "ragged_b2": (lambda: W.llama(90, cap=5000, budget=128, B=2, Hq=8, Hkv=2,
                                  kv_len=np.array([5000, 1777], np.int32)), 128, {}),
    "group8": (lambda: W.llama(91, cap=8192, budget=64, B=1, Hq=8, Hkv=1), 64, {}),
    "llama32k_b128": (lambda: W.llama(0, cap=32768, budget=128), 128, {}),
    "llama32k_b1024": (lambda: W.llama(0, cap=32768, budget=1024), 1024, {}),
    "forced": (lambda: W.llama(92, cap=6000, budget=200, B=2, Hq=8, Hkv=2), 200, dict(sink=4, recent=32)),
    "append": (lambda: W.llama(93, cap=4000, budget=100, B=2, Hq=8, Hkv=2,
                               kv_len=np.array([4000, 2500], np.int32)), 100, dict(append=True)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_single_launch_equals_two_kernels_and_oracle(env, name):
    A, torch, oracle = env
    make, budget, kw = CASES[name]
    wl = make()
    budget = budget or wl.budget
    case = DeviceCase(wl, A, torch)
    if kw.get("append"):
        # the appended key: encode everything but position len-1, let the step add it
        codes = oracle.encode_keys(wl.k, wl.kv_len - 1)
        case.codes.copy_(to_dev(codes, torch))
    (r1, r0), (n1, n0) = both_modes(case, budget, **kw)
    assert n1 == 1 and n0 == 2, (n1, n0)
    assert_same(r1, r0)
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
    fk = {k: v for k, v in kw.items() if k in ("sink", "recent")}
    out_r, sel_r, dist_r, qc_r = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, budget, wl.scale,
                                                    threads=8, **fk)
    out, sel, dist, qc = r1
    assert np.array_equal(sel, sel_r)
    assert np.array_equal(qc, qc_r)
    from helpers import assert_out_close
    assert_out_close(out, out_r)
    if kw.get("append"):
        assert np.array_equal(from_dev(case.codes), codes_ref)


def test_larger_shapes_take_two_kernels(env):
    """Past 64 (batch, kv head) groups or 32 chunks per group the step runs as
    two kernels, in either mode."""
    A, torch, oracle = env
    wl = W.llama(94, cap=2048, budget=16, B=9, Hq=64, Hkv=8)  # 72 groups
    case = DeviceCase(wl, A, torch)
    A.decode_launch_mode(1)
    case.decode(16, want_debug=False)
    A.decode_launch_mode(0)
    assert A.last_launch_count() == 2


def test_single_launch_graph_replays_and_shared_workspace(env):
    """A graph of single-launch steps replayed again and again, with two-kernel
    calls on the same workspace in between: every replay equals the eager step
    bit for bit (each call expects new flag values)."""
    A, torch, oracle = env
    wl = W.llama(95, cap=16384, budget=128, B=1, Hq=32, Hkv=8)
    case = DeviceCase(wl, A, torch)
    ws = A.alloc_workspace(A.decode_workspace_size(1, 32, 8, 16384, 128))
    ws.fill_(0)
    out = torch.empty((1, 32, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((1, 32, 128), dtype=torch.int32, device="cuda")

    def step():
        A.decode_step(case.q, case.k, case.v, case.codes, case.kv_len, 128, wl.scale, out, ws, sel_idx=sel)

    A.decode_launch_mode(1)
    step()
    torch.cuda.synchronize()
    assert A.last_launch_count() == 1
    ref = (out.clone(), sel.clone())
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(3):
            step()
    torch.cuda.synchronize()
    for i in range(6):
        out.zero_()
        sel.fill_(-5)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(sel, ref[1]), "replay %d" % i
        if i % 2 == 1:  # two-kernel calls on the same workspace, then eager single-launch ones
            A.decode_launch_mode(0)
            step()
            A.decode_launch_mode(1)
            step()
            torch.cuda.synchronize()
            assert torch.equal(out, ref[0]) and torch.equal(sel, ref[1])
    A.decode_launch_mode(0)
