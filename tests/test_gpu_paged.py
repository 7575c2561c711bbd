"""GPU parity of the paged entry points (adamas_paged_encode_keys,
adamas_paged_decode_step, dense_paged_decode_attention) against the CPU oracle.

The oracle defines the step on the logical (contiguous) cache; the tests
scatter the same seeded workload into shuffled page pools (tests/helpers.py
paginate) and compare codes, distances, selections and outputs with the oracle
on the contiguous arrays -- and, bit for bit, with the library's own contiguous
path.  Page sizes from 1 to 512, ragged lengths with partial last pages,
shared prefix pages, append, forced positions, and the 32K and batched
configurations.
"""
import numpy as np
import pytest

import workloads as W
from helpers import assert_out_close, from_dev, paginate, to_dev, unpaginate, DeviceCase

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import sparse_attention_long_fwht_amd as A
    import oracle
    return A, torch, oracle


class PagedCase:
    """A workload in shuffled page pools, its codes encoded by the paged entry point."""

    def __init__(self, wl, A, torch, page, seed=0, table=None, pools=None):
        rng = np.random.default_rng(seed)
        self.wl, self.A, self.torch, self.page = wl, A, torch, page
        if pools is None:
            kp, table = paginate(wl.k, page, rng)
            vp, _ = paginate(wl.v, page, np.random.default_rng(seed))  # (same permutation: same seed)
        else:
            kp, vp = pools
        self.table_np = table
        self.k = to_dev(kp, torch)
        self.v = to_dev(vp, torch)
        self.table = to_dev(table, torch)
        self.kv_len = to_dev(wl.kv_len.astype(np.int32), torch)
        self.q = to_dev(wl.q, torch)
        self.pages = A.Pages(self.table, page, capacity=wl.cap)
        self.codes = torch.zeros((kp.shape[0], wl.Hkv, page, 32), dtype=torch.uint8, device="cuda")
        A.encode_keys(self.k, self.kv_len, self.codes, pages=self.pages)

    def logical_codes(self):
        return unpaginate(from_dev(self.codes), self.table_np, self.wl.cap)

    def decode(self, budget, append=False, **forced):
        A, torch, wl = self.A, self.torch, self.wl
        out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
        sel = torch.full((wl.B, wl.Hq, budget), -7, dtype=torch.int32, device="cuda")
        dist = torch.zeros((wl.B, wl.Hq, wl.cap), dtype=torch.int16, device="cuda")
        qc = torch.zeros((wl.B, wl.Hq, 32), dtype=torch.uint8, device="cuda")
        ws = A.alloc_workspace(A.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap, budget))
        ws.fill_(0xFF)
        A.decode_step(self.q, self.k, self.v, self.codes, self.kv_len, budget, wl.scale, out, ws, sel_idx=sel,
                      dist=dist, q_codes=qc, append=append, pages=self.pages, **forced)
        torch.cuda.synchronize()
        return from_dev(out), from_dev(sel), from_dev(dist, np.uint16), from_dev(qc)

    def dense(self):
        A, torch, wl = self.A, self.torch, self.wl
        out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
        ws = A.alloc_workspace(A.dense_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap))
        A.dense_decode_attention(self.q, self.k, self.v, self.kv_len, wl.scale, out, ws, pages=self.pages)
        torch.cuda.synchronize()
        return from_dev(out)


def check_paged(case, oracle, budget, check_dist=True, **forced):
    wl = case.wl
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
    codes = case.logical_codes()
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(codes[b, :, :L], codes_ref[b, :, :L]), "key codes differ (b=%d)" % b
    out_r, sel_r, dist_r, qc_r = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, budget, wl.scale,
                                                    threads=8, want_dist=check_dist, **forced)
    out, sel, dist, qc = case.decode(budget, **forced)
    assert np.array_equal(qc, qc_r)
    if check_dist:
        for b in range(wl.B):
            L = int(wl.kv_len[b])
            assert np.array_equal(dist[b, :, :L], dist_r[b, :, :L]), "distances differ (b=%d)" % b
    assert np.array_equal(sel, sel_r), "selected indices differ"
    assert_out_close(out, out_r)
    return out, sel


def ragged(seed, budget):
    return W.llama(seed, cap=3000, budget=budget, B=3, Hq=8, Hkv=2, kv_len=np.array([3000, 1537, 1], np.int32))


@pytest.mark.parametrize("page", [1, 16, 64, 512])
def test_paged_encode_matches_oracle(env, page):
    A, torch, oracle = env
    wl = ragged(50, 64)
    case = PagedCase(wl, A, torch, page, seed=page)
    ref = oracle.encode_keys(wl.k, wl.kv_len)
    got = case.logical_codes()
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(got[b, :, :L], ref[b, :, :L])


@pytest.mark.parametrize("page,budget", [(16, 64), (64, 700), (256, 7), (1, 64)])
def test_paged_decode_ragged(env, page, budget):
    """Against the oracle, and bit for bit against the contiguous path."""
    A, torch, oracle = env
    wl = ragged(51, budget)
    out, sel = check_paged(PagedCase(wl, A, torch, page, seed=7), oracle, budget)
    out_c, sel_c, _, _ = DeviceCase(wl, A, torch).decode(budget)
    assert np.array_equal(sel, sel_c) and np.array_equal(out, out_c)


def test_paged_empty_sequences(env):
    """Idle slots (kv_len 0) in a paged batch: nothing selected, out 0, dense too."""
    import dataclasses
    A, torch, oracle = env
    wl = W.llama(53, cap=3000, budget=64, B=4, Hq=8, Hkv=2, kv_len=np.array([3000, 1, 1537, 1], np.int32))
    wl = dataclasses.replace(wl, kv_len=np.array([3000, 0, 1537, 0], np.int32))
    case = PagedCase(wl, A, torch, 16, seed=9)
    out, sel = check_paged(case, oracle, 64)
    assert np.all(out[[1, 3]] == 0.0) and np.all(sel[[1, 3]] == -1)
    dense = case.dense()
    assert np.all(dense[[1, 3]] == 0.0)
    assert_out_close(dense, oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale, threads=8))


@pytest.mark.parametrize("page", [1, 8, 16, 64, 1024])
def test_paged_dense(env, page):
    """Pages under 16 positions (a tile's rows on several pages: one table entry
    per row) and of 16 or more (one entry per tile): the same output as the
    contiguous cache, bit for bit."""
    A, torch, oracle = env
    wl = ragged(52, 64)
    case = PagedCase(wl, A, torch, page, seed=3)
    assert_out_close(case.dense(), oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale, threads=8))
    assert np.array_equal(case.dense(), DeviceCase(wl, A, torch).dense())


def test_paged_shared_prefix(env):
    """Sequences 0 and 1 share their first 1024 positions (equal K/V, one set of
    physical pages in the table of both)."""
    A, torch, oracle = env
    wl = ragged(53, 128)
    P = 64
    wl.k[1, :, :1024] = wl.k[0, :, :1024]
    wl.v[1, :, :1024] = wl.v[0, :, :1024]
    rng = np.random.default_rng(11)
    kp, table = paginate(wl.k, P, rng)
    vp, _ = paginate(wl.v, P, np.random.default_rng(11))
    table[1, :1024 // P] = table[0, :1024 // P]  # the shared pages
    check_paged(PagedCase(wl, A, torch, P, table=table, pools=(kp, vp)), oracle, 128)


def test_paged_append_forced(env):
    """append = 1 with sinks and a window: the new key's code lands in its page."""
    A, torch, oracle = env
    wl = ragged(54, 64)
    case = PagedCase(wl, A, torch, 32, seed=5)
    # wipe the last position's code in its page: the step must write it
    for b in range(wl.B):
        p = int(wl.kv_len[b]) - 1
        case.codes[int(case.table_np[b, p // 32]), :, p % 32] = 0
    out, sel, _, _ = case.decode(64, append=True, sink=2, recent=8)
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
    got = case.logical_codes()
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(got[b, :, :L], codes_ref[b, :, :L])
    out_r, sel_r, _, _ = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, 64, wl.scale, threads=8,
                                            sink=2, recent=8)
    assert np.array_equal(sel, sel_r)
    assert_out_close(out, out_r)


def test_paged_llama32k(env):
    A, torch, oracle = env
    wl = W.llama(0, cap=32768, budget=128)
    check_paged(PagedCase(wl, A, torch, 64, seed=1), oracle, 128)


def test_paged_batched16(env):
    A, torch, oracle = env
    wl = W.batched(0)
    check_paged(PagedCase(wl, A, torch, 128, seed=2), oracle, 256, check_dist=False)
