"""GPU parity of the decode step with forced positions (sinks, a recent window,
a bitmap of special tokens) against the CPU oracle.

Blog sections 3.2 and 6 keep special tokens at full attention; the paper builds
on the attention-sink work (citation map).  Reading (shared with the oracle):
sinks and the recent window are always selected; the mask's special tokens take
the rest of the budget first, lower positions first; what remains goes to the
other positions by (distance, position).  Bars as everywhere: indices,
codes and distances exact, out within 2e-3 of the row norm.
"""
import numpy as np
import pytest

import workloads as W
from helpers import DeviceCase, assert_out_close, from_dev
from test_gpu_parity import check_decode

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import sparse_attention_long_fwht_amd as A
    import oracle
    return A, torch, oracle


def special_mask(B, cap, per_b, seed, beyond=0):
    """uint32 [B][ceil(cap/32)] bitmap with `per_b` random positions per entry
    (plus `beyond` bits set past every length, which must be ignored)."""
    rng = np.random.default_rng(seed)
    words = (cap + 31) // 32
    m = np.zeros((B, words), np.uint32)
    for b in range(B):
        for p in rng.choice(cap, per_b, replace=False):
            m[b, p // 32] |= np.uint32(1 << (int(p) % 32))
    return m


def ragged(seed, budget, cap=3000, lens=(3000, 1537, 1)):
    return W.llama(seed, cap=cap, budget=budget, B=len(lens), Hq=8, Hkv=2, kv_len=np.array(lens, np.int32))


@pytest.mark.parametrize("sink,recent", [(4, 16), (1, 0), (0, 33), (32, 32)])
def test_forced_sink_recent_ragged(env, sink, recent):
    A, torch, oracle = env
    check_decode(DeviceCase(ragged(40, 64), A, torch), oracle, sink=sink, recent=recent)


def test_forced_mask_special_tokens(env):
    """A bitmap of special tokens plus one sink; bits past kv_len are ignored."""
    A, torch, oracle = env
    wl = ragged(41, 128)
    mask = special_mask(wl.B, wl.cap, 40, seed=1)
    check_decode(DeviceCase(wl, A, torch), oracle, sink=1, recent=0, mask=mask)


def test_forced_mask_more_than_budget(env):
    """Every third position forced, budget 64: the 64 lowest forced positions."""
    A, torch, oracle = env
    wl = ragged(42, 64)
    words = (wl.cap + 31) // 32
    bits = np.zeros(words * 32, np.uint8)
    bits[::3] = 1
    mask = np.packbits(bits.reshape(-1, 32)[:, ::-1], axis=1).view(">u4").astype(np.uint32).reshape(1, words)
    mask = np.repeat(mask, wl.B, axis=0)
    check_decode(DeviceCase(wl, A, torch), oracle, mask=mask)
    _, sel, _, _ = DeviceCase(wl, A, torch).decode(64, mask=mask)
    assert np.array_equal(sel[0, 0], np.arange(0, 192, 3))


def test_forced_window_kept_when_mask_overflows(env):
    """Every even position is a special token, more than the budget: sinks and
    window are still all kept, the lowest special tokens fill the rest."""
    A, torch, oracle = env
    wl = ragged(47, 30)
    mask = np.full((wl.B, (wl.cap + 31) // 32), 0x55555555, np.uint32)
    check_decode(DeviceCase(wl, A, torch), oracle, sink=3, recent=8, mask=mask)


def test_forced_large_splits(env):
    """Budget 8192 at 32K: splits of 1024 rows, forced ranks past the first 512
    rows of a split."""
    A, torch, oracle = env
    wl = W.llama(3, cap=32768, budget=8192)
    check_decode(DeviceCase(wl, A, torch), oracle, sink=600, recent=1000, check_dist=False)


def test_forced_exactly_the_budget(env):
    """sink + recent == budget: the selection is the forced set itself."""
    A, torch, oracle = env
    wl = ragged(43, 48)
    check_decode(DeviceCase(wl, A, torch), oracle, sink=16, recent=32)
    _, sel, _, _ = DeviceCase(wl, A, torch).decode(48, sink=16, recent=32)
    assert np.array_equal(sel[0, 0], np.concatenate([np.arange(16), np.arange(3000 - 32, 3000)]))


def test_forced_wide_window(env):
    """A 700-position recent window at budget 1024: chunks hold hundreds of
    forced entries at key 0 (the select kernel's bitmap emission)."""
    A, torch, oracle = env
    check_decode(DeviceCase(ragged(44, 1024), A, torch), oracle, sink=4, recent=700)


def test_forced_empty_equals_plain(env):
    """No forced position through the forced entry point: sink = recent = 0
    (plain keys) and an all-zero mask (keys shifted by one) both reproduce the
    plain step exactly, out bit for bit."""
    A, torch, oracle = env
    case = DeviceCase(ragged(45, 96), A, torch)
    out0, sel0, dist0, qc0 = case.decode(96)
    for kw in (dict(sink=0, recent=0), dict(mask=np.zeros((3, 94), np.uint32))):
        out, sel, dist, qc = case.decode(96, **kw)
        assert np.array_equal(sel, sel0) and np.array_equal(out, out0)
        assert np.array_equal(dist, dist0) and np.array_equal(qc, qc0)


def test_forced_append(env):
    """append = 1 with a recent window: the new key's code is written and the
    key is selected."""
    A, torch, oracle = env
    wl = ragged(46, 64)
    case = DeviceCase(wl, A, torch)
    for b in range(wl.B):  # wipe the last codes: the step must write them
        case.codes[b, :, int(wl.kv_len[b]) - 1] = 0
    out, sel, _, _ = case.decode(64, sink=2, recent=8, append=True)
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
    assert np.array_equal(from_dev(case.codes), codes_ref)
    out_r, sel_r, _, _ = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, 64, wl.scale, threads=8,
                                            sink=2, recent=8)
    assert np.array_equal(sel, sel_r)
    assert_out_close(out, out_r)


def test_forced_llama32k(env):
    """The Llama-shaped 32K configuration, budget 128, with 4 sinks, a 64-token
    window and 32 special tokens."""
    A, torch, oracle = env
    wl = W.llama(0, cap=32768, budget=128)
    mask = special_mask(1, 32768, 32, seed=2)
    check_decode(DeviceCase(wl, A, torch), oracle, sink=4, recent=64, mask=mask)


def test_forced_batched16(env):
    """16 ragged sequences of 16K-32K, budget 256, per-sequence windows."""
    A, torch, oracle = env
    wl = W.batched(0)
    check_decode(DeviceCase(wl, A, torch), oracle, sink=8, recent=128, check_dist=False)
