"""HIP-graph replay of the decode step (the benchmark times graph replays).

The step's launches are captured once and replayed several times, with eager
work and synchronisations between replays; every replay must reproduce the
eager result bit for bit (same kernels, same inputs, deterministic).
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from helpers import DeviceCase, assert_out_close, from_dev

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    import torch
    import sparse_attention_long_fwht_amd as A

    wl = W.llama(40, cap=20000, budget=200, B=2, kv_len=np.array([20000, 11111], np.int32))
    case = DeviceCase(wl, A, torch)
    start = case.kv_len - 1
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((wl.B, wl.Hq, wl.budget), dtype=torch.int32, device="cuda")
    ws = A.alloc_workspace(A.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap, wl.budget))

    def step():
        A.encode_keys(case.k, case.kv_len, case.codes, start=start)
        A.decode_step(case.q, case.k, case.v, case.codes, case.kv_len, wl.budget, wl.scale, out, ws, sel_idx=sel)

    step()
    torch.cuda.synchronize()
    ref_out, ref_sel = from_dev(out).copy(), from_dev(sel).copy()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        sel.fill_(-5)
        # eager work between replays (a dense call on the same stream)
        dout = torch.empty_like(out)
        A.dense_decode_attention(case.q, case.k, case.v, case.kv_len, wl.scale, dout,
                                 A.alloc_workspace(A.dense_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(out), ref_out), "replay %d: out differs" % i
        got_sel = from_dev(sel)
        bad = np.argwhere(got_sel != ref_sel)
        assert len(bad) == 0, "replay %d: sel_idx differs at %d entries, first %s: got %s want %s" % (
            i, len(bad), bad[:6].tolist(), [int(got_sel[tuple(x)]) for x in bad[:6]],
            [int(ref_sel[tuple(x)]) for x in bad[:6]])


def test_profile_events_time_each_kernel_and_change_nothing():
    """adamas_profile_events: each launch is bracketed by its event pair; the
    results equal those of an untimed call."""
    import ctypes
    import torch
    import sparse_attention_long_fwht_amd as A

    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    evs = []
    for _ in range(4):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    wl = W.llama(43, cap=9000, budget=300, B=1)
    case = DeviceCase(wl, A, torch)
    ref = case.decode(want_debug=False)
    for mode, launches in ((0, 2), (1, 1)):  # two kernels; the single-launch step
        A.decode_launch_mode(mode)
        A.profile_events(evs)
        try:
            got = case.decode(want_debug=False)
        finally:
            A.profile_events(None)
            A.decode_launch_mode(0)
        assert A.last_launch_count() == launches
        for x, y in zip(ref[:2], got[:2]):
            assert np.array_equal(x, y)
        for i in range(launches):
            ms = ctypes.c_float()
            assert hip.hipEventElapsedTime(ctypes.byref(ms), evs[2 * i], evs[2 * i + 1]) == 0
            assert 0.0 < ms.value < 100.0


def test_graph_replay_forced_and_paged():
    """The paged step with forced positions and the fused append, captured once
    and replayed with eager work in between: every replay equals the eager call."""
    import torch
    import sparse_attention_long_fwht_amd as A
    from helpers import paginate, to_dev

    wl = W.llama(44, cap=6000, budget=256, B=2, kv_len=np.array([6000, 3333], np.int32))
    page = 64
    kp, table = paginate(wl.k, page, np.random.default_rng(1))
    vp, _ = paginate(wl.v, page, np.random.default_rng(1))
    k, v, tab = to_dev(kp, torch), to_dev(vp, torch), to_dev(table, torch)
    q, kv_len = to_dev(wl.q, torch), to_dev(wl.kv_len, torch)
    pages = A.Pages(tab, page, capacity=wl.cap)
    codes = torch.zeros((kp.shape[0], wl.Hkv, page, 32), dtype=torch.uint8, device="cuda")
    A.encode_keys(k, kv_len, codes, pages=pages, num_q_heads=wl.Hq)
    mask = torch.zeros((wl.B, (wl.cap + 31) // 32), dtype=torch.int32, device="cuda")
    mask[:, 3] = 0x1010  # positions 100 and 108 of each sequence
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((wl.B, wl.Hq, wl.budget), dtype=torch.int32, device="cuda")
    ws = A.alloc_workspace(A.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap, wl.budget))

    def step():
        A.decode_step(q, k, v, codes, kv_len, wl.budget, wl.scale, out, ws, sel_idx=sel, append=True, sink=4,
                      recent=32, mask=mask, pages=pages)

    step()
    torch.cuda.synchronize()
    ref_out, ref_sel = from_dev(out).copy(), from_dev(sel).copy()
    assert np.all(np.isin([100, 108], ref_sel[0, 0])) and np.all(np.isin(np.arange(4), ref_sel[1, 3]))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        sel.fill_(-5)
        torch.zeros(1 << 20, device="cuda").add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(out), ref_out), "replay %d: out differs" % i
        assert np.array_equal(from_dev(sel), ref_sel), "replay %d: sel_idx differs" % i



def test_dense_graph_replays_and_stale_workspace():
    """The dense baseline merges a group's chunk partials in the block that finds
    all of them tagged with the group's current generation (a word in the
    workspace, advanced by every call).  Replays of a captured graph, eager calls
    on the same workspace between them, and workspaces holding arbitrary bytes
    all give the eager result bit for bit, and that result is the oracle's dense
    attention."""
    import torch
    import sparse_attention_long_fwht_amd as A
    import oracle

    # (an idle slot: drawn with length 1, then emptied)
    wl = W.llama(23, cap=6000, budget=8, B=3, Hq=8, Hkv=2, kv_len=np.array([6000, 3111, 1], np.int32))
    wl = dataclasses.replace(wl, kv_len=np.array([6000, 3111, 0], np.int32))
    case = DeviceCase(wl, A, torch, encode=False)
    ref = case.dense()  # (poisoned workspace)
    assert_out_close(ref, oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale, threads=16))
    ws = A.alloc_workspace(A.dense_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap))
    gen = torch.Generator(device="cuda")
    for seed in range(3):  # arbitrary workspace contents, then the same workspace reused
        gen.manual_seed(seed)
        ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=gen))
        for _ in range(2):
            out = torch.full((wl.B, wl.Hq, 128), float("nan"), dtype=torch.float32, device="cuda")
            A.dense_decode_attention(case.q, case.k, case.v, case.kv_len, wl.scale, out, ws)
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(out), ref)
    # a captured call replayed, eager calls on the same workspace in between
    gout = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
    call = lambda: A.dense_decode_attention(case.q, case.k, case.v, case.kv_len, wl.scale, gout, ws)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for i in range(5):
        gout.fill_(float("nan"))
        if i % 2:
            eout = torch.empty_like(gout)
            A.dense_decode_attention(case.q, case.k, case.v, case.kv_len, wl.scale, eout, ws)
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(eout), ref), "eager call between replays %d" % i
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(gout), ref), "replay %d" % i
