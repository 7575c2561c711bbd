"""GPU parity: the HIP library against the CPU oracle on the same seeded inputs.

Every call goes through the C ABI (ctypes binding).  Integer results (key codes,
query codes, distances, selected indices) must match the oracle exactly; the
attention output must be within 2e-3 of the oracle relative to the row norm.
Cases span several chunks and a ragged tail, the GQA group sizes 1/2/4/8, the
edge cases (kv_len 1, budget 1, budget >= kv_len, heavy ties, boundary values of
the bucketing), and the full configurations: tiny (1K), Llama-shaped 32K with
budgets 128 and 1024, the batched ragged 16 x [16K, 32K] case and 512K.
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from helpers import DeviceCase, assert_out_close, from_dev, paginate, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import sparse_attention_long_fwht_amd as A
    import oracle
    return A, torch, oracle


def check_decode(case, oracle, budget=None, threads=8, check_dist=True, **forced):
    """forced: sink / recent / mask (host uint32 [B][words]) for both sides."""
    wl = case.wl
    budget = wl.budget if budget is None else budget
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
    codes_gpu = from_dev(case.codes)
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(codes_gpu[b, :, :L], codes_ref[b, :, :L]), "key codes differ (b=%d)" % b
    out_r, sel_r, dist_r, qc_r = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, budget, wl.scale,
                                                    threads=threads, want_dist=check_dist, **forced)
    out, sel, dist, qc = case.decode(budget, want_debug=True, **forced)
    assert np.array_equal(qc, qc_r), "query codes differ"
    if check_dist:
        for b in range(wl.B):
            L = int(wl.kv_len[b])
            assert np.array_equal(dist[b, :, :L], dist_r[b, :, :L]), "distances differ (b=%d)" % b
    assert np.array_equal(sel, sel_r), "selected indices differ"
    return assert_out_close(out, out_r)


# ---------------------------------------------------------------- key encode


def test_encode_keys_tiny(env):
    A, torch, oracle = env
    wl = W.tiny()
    case = DeviceCase(wl, A, torch)
    assert np.array_equal(from_dev(case.codes), oracle.encode_keys(wl.k, wl.kv_len))


def test_encode_keys_boundary_values(env):
    """Keys whose transform lands exactly on -t, 0 and +t, all-zero and -0 keys,
    subnormal keys: codes must match bit for bit."""
    A, torch, oracle = env
    rng = np.random.default_rng(30)
    H = np.array([[(-1) ** bin(i & j).count("1") for j in range(128)] for i in range(128)], np.int64)
    rows = []
    for _ in range(200):
        z = np.zeros(128, np.int64)
        idx = rng.choice(128, 6, replace=False)
        z[idx] = rng.choice([-2, -1, 1, 2], 6)
        rows.append((H @ z).astype(np.float32))      # transform = 128 z exactly: values 0, +-t, +-2t
    rows.append(np.zeros(128, np.float32))
    rows.append(np.full(128, -0.0, np.float32))
    sub = np.zeros(128, np.float32)
    sub[:5] = np.array([1e-39, -2e-39, 3e-40, 0.0, -1e-38], np.float32)
    rows.append(sub)
    for _ in range(20):
        rows.append((rng.standard_normal(128) * 1e-38).astype(np.float32))
    kb = W.f32_to_bf16(np.stack(rows)).reshape(1, 1, -1, 128)
    n = kb.shape[2]
    kv_len = np.array([n], np.int32)
    k = to_dev(kb, torch)
    codes = torch.zeros((1, 1, n, 32), dtype=torch.uint8, device="cuda")
    A.encode_keys(k, to_dev(kv_len, torch), codes)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(codes), oracle.encode_keys(kb, kv_len))


def test_encode_keys_llama32k(env):
    A, torch, oracle = env
    wl = W.llama(0, cap=32768, budget=128)
    case = DeviceCase(wl, A, torch)
    assert np.array_equal(from_dev(case.codes), oracle.encode_keys(wl.k, wl.kv_len))


def test_encode_append_matches_prefill(env):
    A, torch, oracle = env
    wl = W.llama(31, cap=3000, budget=64, B=3, Hq=8, Hkv=2, kv_len=np.array([3000, 1537, 1], np.int32))
    case = DeviceCase(wl, A, torch)
    start = to_dev(wl.kv_len - 1, torch)
    appended = torch.zeros_like(case.codes)
    A.encode_keys(case.k, case.kv_len, appended, start=start)
    torch.cuda.synchronize()
    full, app = from_dev(case.codes), from_dev(appended)
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(app[b, :, L - 1], full[b, :, L - 1])
        assert not app[b, :, : L - 1].any() and not app[b, :, L:].any()


# ---------------------------------------------------------------- decode step


def test_decode_tiny(env):
    A, torch, oracle = env
    case = DeviceCase(W.tiny(), A, torch)
    check_decode(case, oracle)


@pytest.mark.parametrize("budget", [1, 7, 64, 700, 5000])
def test_decode_ragged_multi_chunk(env, budget):
    """3000-slot cache (several chunks + ragged tail), lengths 3000 / 1537 / 1."""
    A, torch, oracle = env
    wl = W.llama(32, cap=3000, budget=budget, B=3, Hq=8, Hkv=2, kv_len=np.array([3000, 1537, 1], np.int32))
    check_decode(DeviceCase(wl, A, torch), oracle)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 1), (16, 2)])
def test_decode_group_sizes(env, Hq, Hkv):
    A, torch, oracle = env
    wl = W.llama(33, cap=2100, budget=96, B=2, Hq=Hq, Hkv=Hkv, kv_len=np.array([2100, 999], np.int32))
    check_decode(DeviceCase(wl, A, torch), oracle)


@pytest.mark.parametrize("distinct", [8, 4])
def test_decode_heavy_ties(env, distinct):
    """Many keys share one code (`distinct` codes tiled over the cache), so the
    threshold bin holds hundreds of ties: the lower positions must win.  With 4
    codes a chunk holds more than 64 entries at or below the threshold, which
    takes the select kernel's bitmap emission; with 8, exactly 64 (the widest
    in-register sort)."""
    A, torch, oracle = env
    wl = W.llama(34, cap=4096, budget=300, B=1, Hq=4, Hkv=1)
    rep = wl.k[0, 0, :distinct].copy()
    wl.k[0, 0] = np.tile(rep, (4096 // distinct, 1))
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
    _, _, dist_r, _ = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, wl.budget, wl.scale, threads=8)
    widest = max_chunk_entries(wl, dist_r, wl.budget)
    assert (widest > 64) if distinct == 4 else (widest == 64), widest
    check_decode(DeviceCase(wl, A, torch), oracle)


def max_chunk_entries(wl, dist, budget):
    """Largest number of positions at or below the threshold distance T in one
    chunk, over all heads (the select kernel sorts up to 64 of them in
    registers, more through a bitmap)."""
    chunk, _ = chunking(wl.cap, wl.B * wl.Hkv, wl.Hq // wl.Hkv)
    worst = 0
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        k_eff = min(budget, L)
        for h in range(wl.Hq):
            d = dist[b, h, :L].astype(np.int64)
            T = int(np.sort(d)[k_eff - 1])
            for c0 in range(0, L, chunk):
                worst = max(worst, int((d[c0:c0 + chunk] <= T).sum()))
    return worst


def chunking(cap, groups=1, R=4):
    """The library's chunk size: 512 positions, doubled up to 4096 until a head
    has at most 64 chunks and the scan has at most 256 blocks, one per (b, kv
    head, chunk); then 8192 if that takes fewer rounds of resident scan blocks
    (blocks per compute unit by LDS, at most 4)."""
    chunk = 512
    blocks = lambda ch: groups * -(-cap // ch)
    while chunk < 4096 and (chunk * 64 < cap or blocks(chunk) > 256):
        chunk *= 2
    if chunk == 4096:
        def rounds(ch):
            lds = R * (448 * 4 + 392 * 2 + 36) + 32 + R * ch * 2
            slots = 256 * max(1, min(4, 163840 // lds))
            return -(-blocks(ch) // slots)
        if rounds(8192) < rounds(4096):
            chunk = 8192
    return chunk, None


def thresholds(wl, dist, budget):
    """The threshold distance T (the k-th smallest) of every (b, q head)."""
    out = []
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        for h in range(wl.Hq):
            out.append(int(np.sort(dist[b, h, :L])[min(budget, L) - 1]))
    return out


def pm1_query(seed):
    """A bf16 query whose transform is exactly a +-1 vector (codes 0 and 3 only):
    its negation is at distance 384, itself at distance 0."""
    H = np.array([[1.0]], np.float32)
    while H.shape[0] < 128:
        H = np.block([[H, H], [H, -H]])
    s = np.where(np.random.default_rng(seed).random(128) < 0.5, -1.0, 1.0).astype(np.float32)
    qv = (H @ s) / 128.0  # multiples of 1/64 in [-1, 1]: exact in bf16, and H @ qv == s exactly
    return W.f32_to_bf16(qv.astype(np.float32)), W.f32_to_bf16(-qv.astype(np.float32))


def test_decode_threshold_extremes(env):
    """Thresholds at the ends of the distance range and far from the smallest
    distance: (a) 40 chunks of 1024, budget 38000, one key equal to query head
    0 (its least distance is 0, its threshold far above); (b) one chunk holding
    keys at distance 0 and 384 beside random keys; (c) T = 384, the last
    distance: 10 keys at distance 0, 590 at 384, budget 100 (90 ties at 384,
    the lowest positions win); (d) T = 0 with more keys at distance 0 than the
    budget (the lowest 64 of 200 win)."""
    A, torch, oracle = env
    wa = W.llama(50, cap=40000, budget=38000, B=1, Hq=8, Hkv=2)
    wa.k[0, 0, 2600] = wa.q[0, 0]
    wb = W.llama(51, cap=2048, budget=520, B=1, Hq=2, Hkv=1)
    q, nq = pm1_query(7)
    wb.q[0, 0] = q
    wb.k[0, 0, 0:100] = nq
    wb.k[0, 0, 100:110] = q
    wc = W.llama(52, cap=600, budget=100, B=1, Hq=1, Hkv=1)
    q, nq = pm1_query(8)
    wc.q[0, 0] = q
    wc.k[0, 0, :590] = nq
    wc.k[0, 0, 590:] = q
    wd = W.llama(53, cap=3000, budget=64, B=1, Hq=1, Hkv=1)
    rng = np.random.default_rng(9)
    wd.k[0, 0, np.sort(rng.choice(3000, 200, replace=False))] = wd.q[0, 0]
    for wl, want in ((wa, None), (wb, None), (wc, 384), (wd, 0)):
        codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
        _, _, dist_r, _ = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, wl.budget, wl.scale, threads=8)
        T = thresholds(wl, dist_r, wl.budget)
        if want is not None:
            assert T[0] == want, T
        if wl is wa:
            assert int(dist_r[0, 0].min()) == 0 and T[0] > 128, T
        check_decode(DeviceCase(wl, A, torch), oracle)


def test_decode_budget_twice_capacity(env):
    """A budget twice the capacity with sel_idx: every position is kept, in
    ascending order, and the -1 tail (written by all of a head's blocks) runs
    to the end of the row."""
    A, torch, oracle = env
    wl = W.llama(71, cap=3000, budget=6000, B=2, Hq=8, Hkv=2, kv_len=np.array([3000, 1537], np.int32))
    case = DeviceCase(wl, A, torch)
    check_decode(case, oracle)
    _, sel, _, _ = case.decode(want_debug=False)
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(sel[b, :, :L], np.broadcast_to(np.arange(L, dtype=np.int32), (wl.Hq, L)))
        assert np.all(sel[b, :, L:] == -1)


def test_decode_sixteen_pass_chunks(env):
    """Chunks of 8192 positions (the sixteen-pass scan: three sequences of one
    kv head with eight query heads need two rounds of resident scan blocks at
    4096 and one at 8192), ragged lengths, one ending inside a pass."""
    A, torch, oracle = env
    wl = W.llama(54, cap=524288, budget=512, B=3, Hq=8, Hkv=1,
                 kv_len=np.array([524288, 300001, 9000], np.int32))
    assert chunking(wl.cap, wl.B * wl.Hkv, 8)[0] == 8192
    check_decode(DeviceCase(wl, A, torch), oracle, threads=16)


@pytest.mark.parametrize("budget", [300, 2500])
def test_decode_multipass_chunks_ragged(env, budget):
    """Chunks of 2048 positions (four passes of the scan block, each loading the
    next pass's codes while it computes), kv_len ending inside a pass."""
    A, torch, oracle = env
    wl = W.llama(52, cap=100000, budget=budget, B=2, Hq=8, Hkv=2, kv_len=np.array([99999, 61234], np.int32))
    assert chunking(wl.cap, wl.B * wl.Hkv)[0] == 2048
    check_decode(DeviceCase(wl, A, torch), oracle)


def test_decode_full_budget_equals_dense(env):
    A, torch, oracle = env
    wl = W.llama(35, cap=1500, budget=2000, B=2, Hq=8, Hkv=2, kv_len=np.array([1500, 733], np.int32))
    case = DeviceCase(wl, A, torch)
    out, sel, _, _ = case.decode(2000)
    dense = case.dense()
    ref = oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale)
    assert_out_close(out, ref)
    assert_out_close(dense, ref)
    assert np.array_equal(sel[0, :, :1500], np.broadcast_to(np.arange(1500), (8, 1500)))
    assert np.all(sel[1, :, 733:] == -1)


def test_decode_is_deterministic(env):
    A, torch, oracle = env
    wl = W.llama(36, cap=8192, budget=256, B=1)
    case = DeviceCase(wl, A, torch)
    a = case.decode()
    b = case.decode()
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_decode_reused_workspace_new_inputs(env):
    """One workspace, three calls with different inputs (A, B, A): each result
    must match the oracle for its own inputs, so nothing is carried over."""
    A, torch, oracle = env
    wa = W.llama(38, cap=6000, budget=150, B=2, Hq=8, Hkv=2, kv_len=np.array([6000, 3001], np.int32))
    wb = W.llama(39, cap=6000, budget=150, B=2, Hq=8, Hkv=2, kv_len=np.array([4500, 6000], np.int32))
    ca, cb = DeviceCase(wa, A, torch), DeviceCase(wb, A, torch)
    ws = A.alloc_workspace(A.decode_workspace_size(2, 8, 2, 6000, 150))
    ws.fill_(0xFF)
    refs = {}
    for name, wl in (("a", wa), ("b", wb)):
        codes = oracle.encode_keys(wl.k, wl.kv_len)
        refs[name] = oracle.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, 150, wl.scale)
    for name, case in (("a", ca), ("b", cb), ("a", ca)):
        out = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
        sel = torch.empty((2, 8, 150), dtype=torch.int32, device="cuda")
        A.decode_step(case.q, case.k, case.v, case.codes, case.kv_len, 150, case.wl.scale, out, ws, sel_idx=sel)
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(sel), refs[name][1]), name
        assert_out_close(from_dev(out), refs[name][0], what="out(%s)" % name)


def check_append_decode(A, torch, oracle, wl, budget=None):
    """Codes hold every key but the last; adamas_append_decode_step must encode
    key kv_len-1 and then match the oracle step on the complete codes."""
    budget = wl.budget if budget is None else budget
    case = DeviceCase(wl, A, torch, encode=False)
    end_prev = to_dev(np.maximum(wl.kv_len - 1, 0), torch)  # (an empty sequence has nothing to append)
    A.encode_keys(case.k, end_prev, case.codes)  # positions [0, len-1)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
    sel = torch.empty((wl.B, wl.Hq, budget), dtype=torch.int32, device="cuda")
    qc = torch.empty((wl.B, wl.Hq, 32), dtype=torch.uint8, device="cuda")
    ws = A.alloc_workspace(A.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap, budget))
    ws.fill_(0xFF)
    A.decode_step(case.q, case.k, case.v, case.codes, case.kv_len, budget, wl.scale, out, ws, sel_idx=sel,
                  q_codes=qc, append=True)
    torch.cuda.synchronize()
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
    codes = from_dev(case.codes)
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(codes[b, :, :L], codes_ref[b, :, :L]), "codes after append (b=%d)" % b
        assert not codes[b, :, L:].any(), "append wrote past kv_len (b=%d)" % b
    out_r, sel_r, _, qc_r = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, budget, wl.scale, threads=16,
                                               want_dist=False)
    assert np.array_equal(from_dev(qc), qc_r)
    assert np.array_equal(from_dev(sel), sel_r)
    return assert_out_close(from_dev(out), out_r)


def test_append_decode_ragged(env):
    A, torch, oracle = env
    wl = W.llama(41, cap=3000, budget=100, B=3, Hq=8, Hkv=2, kv_len=np.array([3000, 1537, 1], np.int32))
    check_append_decode(A, torch, oracle, wl)
    wl = W.llama(42, cap=5000, budget=64, B=2, Hq=8, Hkv=1, kv_len=np.array([4097, 512], np.int32))
    check_append_decode(A, torch, oracle, wl)


@pytest.mark.parametrize("cap", [1, 5, 63, 64, 65, 511, 513])
def test_decode_capacities_below_a_chunk(env, cap):
    """Caches smaller than (or just past) one scan chunk and one encode pass,
    full and partly filled, with budgets below, at and above the length."""
    A, torch, oracle = env
    lens = np.array([cap, max(1, cap // 2), 1], np.int32)
    for budget in sorted({1, max(1, cap // 3), cap, cap + 7}):
        wl = W.llama(60 + cap, cap=cap, budget=budget, B=3, Hq=8, Hkv=2, kv_len=lens)
        check_decode(DeviceCase(wl, A, torch), oracle)
        out = DeviceCase(wl, A, torch, encode=False).dense()
        assert_out_close(out, oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale))


def test_decode_largest_int32_budget(env):
    """Any positive int32 budget: past the capacity the step plans and selects
    exactly as at budget = capacity (every position kept), bit for bit."""
    A, torch, oracle = env
    wl = W.llama(70, cap=3000, budget=3000, B=2, Hq=8, Hkv=2, kv_len=np.array([3000, 1537], np.int32))
    case = DeviceCase(wl, A, torch)
    outs = []
    for budget in (3000, 2 ** 31 - 1):
        out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
        ws = A.alloc_workspace(A.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap, budget))
        A.decode_step(case.q, case.k, case.v, case.codes, case.kv_len, budget, wl.scale, out, ws)
        torch.cuda.synchronize()
        outs.append(from_dev(out))
    assert np.array_equal(outs[0], outs[1])
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
    out_r, _, _, _ = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, 3000, wl.scale, threads=8,
                                        want_dist=False)
    assert_out_close(outs[1], out_r)


def with_empty_slots(seed, budget):
    """Idle batch slots (kv_len 0) between a full, a ragged and a length-1
    sequence (the workload is drawn with length 1 there, then emptied)."""
    wl = W.llama(seed, cap=3000, budget=budget, B=5, Hq=8, Hkv=2, kv_len=np.array([3000, 1, 1537, 1, 1], np.int32))
    return dataclasses.replace(wl, kv_len=np.array([3000, 0, 1537, 0, 1], np.int32))


@pytest.mark.parametrize("variant", ["plain", "forced", "append", "dense"])
def test_empty_sequences(env, variant):
    """An empty sequence selects nothing (sel_idx all -1) and gets out exactly 0;
    the other entries match the oracle as usual."""
    A, torch, oracle = env
    wl = with_empty_slots(43, 96)
    if variant == "dense":
        out = DeviceCase(wl, A, torch, encode=False).dense()
        assert np.all(out[[1, 3]] == 0.0)
        assert_out_close(out, oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale))
    elif variant == "append":
        check_append_decode(A, torch, oracle, wl)
    else:
        case = DeviceCase(wl, A, torch)
        kw = dict(sink=4, recent=16) if variant == "forced" else {}
        check_decode(case, oracle, **kw)
        out, sel, _, _ = case.decode(wl.budget, want_debug=False, **kw)
        assert np.all(out[[1, 3]] == 0.0) and np.all(sel[[1, 3]] == -1)


def test_empty_sequences_several_splits(env):
    """The same with a budget that spreads a head over several blocks."""
    A, torch, oracle = env
    wl = with_empty_slots(44, 1024)
    check_decode(DeviceCase(wl, A, torch), oracle, budget=1024)


def test_append_decode_llama32k(env):
    A, torch, oracle = env
    check_append_decode(A, torch, oracle, W.llama(0, cap=32768, budget=128))


@pytest.mark.parametrize("budget", [128, 1024])
def test_decode_llama32k(env, budget):
    """Llama-3.1-8B-shaped layer: 32 q heads / 8 kv heads, 32K context."""
    A, torch, oracle = env
    wl = W.llama(0, cap=32768, budget=budget)
    err = check_decode(DeviceCase(wl, A, torch), oracle, threads=16)
    print("llama32k budget %d: worst relative error %.2e" % (budget, err))


def test_decode_batched16(env):
    """16 sequences with ragged lengths in [16K, 32K], budget 256 (chunks of
    4096 positions: eight passes per scan block; one 256-row block per head)."""
    A, torch, oracle = env
    wl = W.batched(0)
    err = check_decode(DeviceCase(wl, A, torch), oracle, threads=16)
    print("batched16: worst relative error %.2e" % err)


def test_decode_long512k(env):
    """512K context, budget 1024: the whole step runs on the GPU at full size and
    every KV group and query head is compared with the oracle (key codes, query
    codes, distances, selections, outputs)."""
    A, torch, oracle = env
    wl = W.llama(0, cap=524288, budget=1024, name="long512k")
    case = DeviceCase(wl, A, torch)
    out, sel, dist, qc = case.decode(want_debug=True)
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len, threads=16)
    assert np.array_equal(from_dev(case.codes), codes_ref)
    o_r, s_r, d_r, q_r = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, wl.budget, wl.scale,
                                            threads=16)
    assert np.array_equal(qc, q_r)
    assert np.array_equal(dist, d_r)
    assert np.array_equal(sel, s_r)
    err = assert_out_close(out, o_r)
    print("long512k: all 32 heads, worst relative error %.2e" % err)


def test_decode_long512k_largest_budget(env):
    """The largest supported budget at the largest capacity (245760 of 524288
    positions: 64 splits of 3840 rows per head, chunks of 8192); every head
    checked."""
    A, torch, oracle = env
    assert A.decode_workspace_size(1, 32, 8, 524288, 245760) > 0
    assert A.decode_workspace_size(1, 32, 8, 524288, 245761) == 0
    wl = W.llama(4, cap=524288, budget=245760, name="long512k_k240k")
    case = DeviceCase(wl, A, torch)
    out, sel, _, _ = case.decode(want_debug=False)
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len, threads=16)
    assert np.array_equal(from_dev(case.codes), codes_ref)
    o_r, s_r, _, _ = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, wl.budget, wl.scale, threads=16,
                                        want_dist=False)
    assert np.array_equal(sel, s_r)
    assert_out_close(out, o_r)


def test_decode_many_heads(env):
    """32768 query heads (batch 1024 x 32 / 8 heads, 96 positions each, ragged):
    grids of 8192 scan and 32768 select blocks."""
    A, torch, oracle = env
    rng = np.random.default_rng(60)
    lens = rng.integers(1, 97, 1024).astype(np.int32)
    wl = W.llama(60, cap=96, budget=16, B=1024, kv_len=lens, n_planted=1)
    check_decode(DeviceCase(wl, A, torch), oracle, budget=16, threads=16)


# ---------------------------------------------------------------- dense baseline


def test_dense_tiny_and_ragged(env):
    A, torch, oracle = env
    for wl in (W.tiny(), W.llama(37, cap=5000, budget=1, B=2, Hq=8, Hkv=2, kv_len=np.array([5000, 2049], np.int32))):
        case = DeviceCase(wl, A, torch, encode=False)
        assert_out_close(case.dense(), oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale))


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (8, 1), (16, 2)])
def test_dense_group_sizes(env, Hq, Hkv):
    A, torch, oracle = env
    wl = W.llama(38, cap=3100, budget=1, B=2, Hq=Hq, Hkv=Hkv, kv_len=np.array([3100, 1], np.int32))
    case = DeviceCase(wl, A, torch, encode=False)
    assert_out_close(case.dense(), oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale))


@pytest.mark.parametrize("Hq", [8, 4])
def test_dense_many_chunks(env, Hq):
    """One kv head at 128K positions: 128 chunks per group (the most a group
    has), so the merge runs several batches of chunks and its second half of
    lanes; the second sequence's 69 chunks end mid-chunk."""
    A, torch, oracle = env
    wl = W.llama(42, cap=131072, budget=1, B=2, Hq=Hq, Hkv=1, kv_len=np.array([131072, 70001], np.int32))
    case = DeviceCase(wl, A, torch, encode=False)
    assert_out_close(case.dense(), oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale, threads=16))


def test_encode_keys_arbitrary_ranges(env):
    """Ranges [start[b], end[b]) anywhere in the cache (empty ones included):
    exactly those rows are written, equal to the oracle's codes; the rest of
    the poisoned code buffer is left as it was."""
    A, torch, oracle = env
    wl = W.llama(39, cap=4000, budget=8, B=4, Hq=8, Hkv=2)
    start = np.array([0, 1234, 3999, 2000], np.int32)
    end = np.array([4000, 1300, 3999, 3001], np.int32)
    case = DeviceCase(wl, A, torch, encode=False)
    case.codes.fill_(0xA5)
    A.encode_keys(case.k, to_dev(end, torch), case.codes, start=to_dev(start, torch))
    torch.cuda.synchronize()
    got = from_dev(case.codes)
    ref = oracle.encode_keys(wl.k, end, start=start)
    for b in range(wl.B):
        s, e = int(start[b]), int(end[b])
        assert np.array_equal(got[b, :, s:e], ref[b, :, s:e])
        assert np.all(got[b, :, :s] == 0xA5) and np.all(got[b, :, e:] == 0xA5)


def test_encode_keys_bounded(env):
    """adamas_encode_keys_bounded writes exactly what adamas_encode_keys writes,
    whatever the bound: one key per sequence with max_rows = 1, whole ragged
    ranges with a bound far below their lengths (every block then walks many
    passes) and one above the capacity; and the paged form into shuffled pages."""
    A, torch, oracle = env
    wl = W.llama(41, cap=3000, budget=8, B=3, Hq=8, Hkv=2, kv_len=np.array([3000, 1537, 1], np.int32))
    case = DeviceCase(wl, A, torch, encode=False)
    end = to_dev(wl.kv_len, torch)
    ref = oracle.encode_keys(wl.k, wl.kv_len)
    # appended keys
    start = to_dev(wl.kv_len - 1, torch)
    case.codes.fill_(0x5A)
    A.encode_keys(case.k, end, case.codes, start=start, max_rows=1)
    torch.cuda.synchronize()
    got = from_dev(case.codes)
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(got[b, :, L - 1], ref[b, :, L - 1])
        assert np.all(got[b, :, : L - 1] == 0x5A) and np.all(got[b, :, L:] == 0x5A)
    # whole ranges, bounds too small and too large
    for bound in (5, 64, 65, 1 << 30):
        case.codes.fill_(0x5A)
        A.encode_keys(case.k, end, case.codes, max_rows=bound)
        torch.cuda.synchronize()
        got = from_dev(case.codes)
        for b in range(wl.B):
            L = int(wl.kv_len[b])
            assert np.array_equal(got[b, :, :L], ref[b, :, :L]), bound
            assert np.all(got[b, :, L:] == 0x5A), bound
    # paged pools (pages of 64, shuffled), bound 1 for the appended keys
    page = 64
    pool_k, table = paginate(wl.k, page, np.random.default_rng(5))
    num_pages = pool_k.shape[0]
    pk = to_dev(pool_k, torch)
    pcodes = torch.full((num_pages, wl.Hkv, page, 32), 0x5A, dtype=torch.uint8, device="cuda")
    pages = A.Pages(to_dev(table, torch), page, capacity=wl.cap)
    A.encode_keys(pk, end, pcodes, start=start, pages=pages, max_rows=1)
    torch.cuda.synchronize()
    pc = from_dev(pcodes)
    for b in range(wl.B):
        p = int(wl.kv_len[b]) - 1
        row = table[b, p // page]
        assert np.array_equal(pc[row, :, p % page], ref[b, :, p])


def test_dense_llama32k(env):
    A, torch, oracle = env
    wl = W.llama(0, cap=32768, budget=128)
    case = DeviceCase(wl, A, torch, encode=False)
    assert_out_close(case.dense(), oracle.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale, threads=16))
