"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test states what pins it: a closed form of the Sylvester-Hadamard matrix,
hand-derived fixtures under tests/golden/, exact integer arithmetic, invariants
of the distance and of top-k, or closed forms of softmax attention.  A numpy
re-derivation of the encode is used only on inputs where fp32 is exact, so it
checks the oracle from a different direction (matrix product, searchsorted,
packbits) rather than retyping its loops.

Sources: Adamas paper abstracts (v1 and v2): Hadamard transform, bucketing,
2-bit compression, Manhattan / distance-based top-k, gather of the original KV
for sparse attention.  ADAMAS blog (jsqmd.com) sections 2.1 (transform),
2.2 (dynamic thresholds), 2.3 (Manhattan distance), 3.1 (compressed cache).
"""
import os

import numpy as np
import pytest

import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def sylvester(n=128):
    """Closed form of the natural-order Sylvester-Hadamard matrix: (-1)^popcount(i&j)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    x = i & j
    pc = np.zeros_like(x)
    while np.any(x):
        pc += x & 1
        x >>= 1
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- transform


def test_fwht_columns_are_sylvester_hadamard(oracle_mod):
    """Applying the transform to unit vectors yields H; H is the Sylvester matrix and H H^T = 128 I."""
    H = np.stack([oracle_mod.fwht128(np.eye(128, dtype=np.float32)[i]) for i in range(128)], axis=1)
    Hi = H.astype(np.int64)
    assert np.array_equal(H, Hi.astype(np.float32))
    assert np.array_equal(Hi, sylvester())
    assert np.array_equal(Hi @ Hi.T, 128 * np.eye(128, dtype=np.int64))
    assert np.array_equal(Hi, Hi.T)


def test_fwht_exact_on_integers(oracle_mod):
    """For integer inputs |x| < 2^16 every partial sum is exact in fp32: y == H x in int64."""
    rng = np.random.default_rng(1)
    H = sylvester()
    for _ in range(20):
        x = rng.integers(-(2 ** 16) + 1, 2 ** 16, 128)
        y = oracle_mod.fwht128(x.astype(np.float32))
        assert np.array_equal(y.astype(np.int64), H @ x)


def test_fwht_involution_on_integers(oracle_mod):
    """H H = 128 I: transforming twice multiplies by 128 (exact for small integers)."""
    rng = np.random.default_rng(2)
    x = rng.integers(-1000, 1000, 128).astype(np.float32)
    y = oracle_mod.fwht128(oracle_mod.fwht128(x))
    assert np.array_equal(y, 128 * x)


def test_fwht_preserves_dot_products_up_to_d(oracle_mod):
    """(Hq).(Hk) = 128 q.k, the invariant behind transforming both q and k."""
    rng = np.random.default_rng(3)
    for _ in range(10):
        q = rng.integers(-200, 200, 128)
        k = rng.integers(-200, 200, 128)
        hq = oracle_mod.fwht128(q.astype(np.float32)).astype(np.int64)
        hk = oracle_mod.fwht128(k.astype(np.float32)).astype(np.int64)
        assert int(hq @ hk) == 128 * int(q @ k)


def test_fwht_error_bound_on_bf16(oracle_mod):
    """Seven rounded stages: |y - Hx| <= ((1+u)^7 - 1) * sum|x| per coordinate, u = 2^-24."""
    rng = np.random.default_rng(4)
    H = sylvester().astype(np.float64)
    bound_factor = (1 + 2.0 ** -24) ** 7 - 1
    for _ in range(50):
        xb = W.f32_to_bf16(rng.standard_normal(128).astype(np.float32) * rng.lognormal(0, 2, 128).astype(np.float32))
        x = W.bf16_to_f32(xb).astype(np.float64)
        y = oracle_mod.fwht128(x.astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(y - H @ x) <= bound_factor * np.abs(x).sum() * (1 + 1e-12))


def test_fwht_stage_order_golden(oracle_mod):
    """Hand-derived rounding case (tests/golden/fwht_stage_order.txt) fixes the stage order."""
    x = np.zeros(128, np.float32)
    want = {}
    for tag, idx, val in read_golden("fwht_stage_order.txt"):
        if tag == "x":
            x[int(idx)] = np.float32(float.fromhex(val))
        else:
            want[int(idx)] = np.float32(float.fromhex(val))
    y = oracle_mod.fwht128(x)
    for i, v in want.items():
        assert y[i] == v, (i, y[i].hex() if hasattr(y[i], "hex") else y[i], v)


# ---------------------------------------------------------------- bucketing


def test_bucketize_boundary_golden(oracle_mod):
    rows = read_golden("bucketize_boundaries.txt")
    y = np.zeros(128, np.float32)
    want = np.full(128, 2, np.uint8)  # zeros elsewhere: 0 is not below 0, is below t=4
    for i, r in enumerate(rows):
        y[i] = np.float32(float.fromhex(r[0]))
        want[i] = int(r[1])
    got = oracle_mod.bucketize128(y)
    assert np.array_equal(got, want), np.nonzero(got != want)


def test_bucketize_all_zero_vector(oracle_mod):
    """t = 0 and no value is below 0 or t: every code is 3 (literal strict tests)."""
    assert np.all(oracle_mod.bucketize128(np.zeros(128, np.float32)) == 3)
    z = np.zeros(128, np.float32)
    z[::2] = -0.0
    assert np.all(oracle_mod.bucketize128(z) == 3)


def test_bucketize_max_taken_over_every_coordinate(oracle_mod):
    """A lone +-10 at coordinate i sets t = 5; values +-1, +-3 then code 1/1/2/2.
    If the maximum skipped coordinate i, t would be 1.5 and +-3 would code 0/3."""
    base = np.tile(np.array([-3.0, -1.0, 1.0, 3.0], np.float32), 32)
    for i in range(128):
        for big in (10.0, -10.0):
            y = base.copy()
            y[i] = big
            want = np.where(base < 0, 1, 2).astype(np.uint8)
            want[i] = 3 if big > 0 else 0
            assert np.array_equal(oracle_mod.bucketize128(y), want), (i, big)


def test_bucketize_scale_invariance(oracle_mod):
    """Thresholds scale with max|y|, so codes(2^j y) == codes(y) exactly."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        y = (rng.standard_normal(128) * 10).astype(np.float32)
        c = oracle_mod.bucketize128(y)
        for j in (-20, -3, -1, 1, 5, 30):
            assert np.array_equal(oracle_mod.bucketize128(np.ldexp(y, j).astype(np.float32)), c)


def test_bucketize_monotone_and_symmetric(oracle_mod):
    """Codes never decrease with the value; negating a vector maps code c to 3-c (no ties, no zeros)."""
    rng = np.random.default_rng(6)
    for _ in range(20):
        y = rng.standard_normal(128).astype(np.float32)
        c = oracle_mod.bucketize128(y)
        order = np.argsort(y, kind="stable")
        assert np.all(np.diff(c[order].astype(int)) >= 0)
        t = 0.5 * np.abs(y).max()
        if np.all(y != 0) and np.all(np.abs(y) != t):
            assert np.array_equal(oracle_mod.bucketize128(-y), 3 - c)


def test_bucketize_matches_searchsorted(oracle_mod):
    """Code = number of thresholds (-t, 0, t) that the value is not below."""
    rng = np.random.default_rng(7)
    for _ in range(50):
        y = (rng.standard_normal(128) * rng.lognormal(0, 1)).astype(np.float32)
        t = np.float32(0.5) * np.abs(y).max()
        thr = np.array([-t, 0.0, t], np.float32)
        want = np.searchsorted(thr, y, side="right").astype(np.uint8)
        assert np.array_equal(oracle_mod.bucketize128(y), want)


# ---------------------------------------------------------------- packing


def test_pack_pattern_golden(oracle_mod):
    rows = read_golden("pack_pattern.txt")
    want = np.array([int(b, 16) for b in rows[0]], np.uint8)
    got = oracle_mod.pack128((np.arange(128) % 4).astype(np.uint8))
    assert np.array_equal(got, want)


def test_pack_single_coordinate(oracle_mod):
    """A lone code at coordinate i lands at bit i%8 of byte i/8 of its plane(s)."""
    for i in (0, 1, 7, 8, 63, 64, 100, 127):
        for code in (1, 2, 3):
            c = np.zeros(128, np.uint8)
            c[i] = code
            p = oracle_mod.pack128(c)
            want = np.zeros(32, np.uint8)
            if code & 1:
                want[i // 8] = 1 << (i % 8)
            if code & 2:
                want[16 + i // 8] = 1 << (i % 8)
            assert np.array_equal(p, want), (i, code)


def test_pack_roundtrip_and_packbits(oracle_mod):
    rng = np.random.default_rng(8)
    for _ in range(50):
        c = rng.integers(0, 4, 128).astype(np.uint8)
        p = oracle_mod.pack128(c)
        assert np.array_equal(oracle_mod.unpack128(p), c)
        lo = np.packbits(c & 1, bitorder="little")
        hi = np.packbits(c >> 1, bitorder="little")
        assert np.array_equal(p, np.concatenate([lo, hi]))


def test_encode_vector_exact_rederivation(oracle_mod):
    """On small-integer bf16 inputs the fp32 transform is exact, so a numpy path
    (H matrix product, searchsorted thresholds, packbits) must give the same bytes."""
    rng = np.random.default_rng(9)
    H = sylvester()
    for _ in range(100):
        xi = rng.integers(-100, 101, 128)
        xb = W.f32_to_bf16(xi.astype(np.float32))
        assert np.array_equal(W.bf16_to_f32(xb), xi.astype(np.float32))
        y = (H @ xi).astype(np.float32)
        t = np.float32(0.5) * np.abs(y).max()
        c = np.searchsorted(np.array([-t, 0.0, t], np.float32), y, side="right").astype(np.uint8)
        want = np.concatenate([np.packbits(c & 1, bitorder="little"), np.packbits(c >> 1, bitorder="little")])
        assert np.array_equal(oracle_mod.encode_vector(xb), want)


def test_encode_vector_is_composition(oracle_mod):
    rng = np.random.default_rng(10)
    for _ in range(20):
        xb = W.f32_to_bf16(rng.standard_normal(128).astype(np.float32) * 3)
        y = oracle_mod.fwht128(W.bf16_to_f32(xb))
        assert np.array_equal(oracle_mod.encode_vector(xb), oracle_mod.pack128(oracle_mod.bucketize128(y)))


# ---------------------------------------------------------------- distance


def test_distance_closed_forms(oracle_mod):
    pk = oracle_mod.pack128
    zeros = pk(np.zeros(128, np.uint8))
    threes = pk(np.full(128, 3, np.uint8))
    ones = pk(np.ones(128, np.uint8))
    pattern = pk((np.arange(128) % 4).astype(np.uint8))
    assert oracle_mod.distance(zeros, threes) == 384
    assert oracle_mod.distance(threes, zeros) == 384
    # |1 - (i mod 4)| = 1, 0, 1, 2 per group of four -> 32 * 4 = 128
    assert oracle_mod.distance(ones, pattern) == 128
    # |0 - (i mod 4)| sums to 32 * 6 = 192
    assert oracle_mod.distance(zeros, pattern) == 192
    for i in (0, 9, 64, 127):
        for a in range(4):
            for b in range(4):
                ca = np.full(128, 1, np.uint8)
                cb = ca.copy()
                ca[i] = a
                cb[i] = b
                assert oracle_mod.distance(pk(ca), pk(cb)) == abs(a - b)


def test_distance_metric_axioms(oracle_mod):
    rng = np.random.default_rng(11)
    pk = oracle_mod.pack128
    for _ in range(100):
        a, b, c = (pk(rng.integers(0, 4, 128).astype(np.uint8)) for _ in range(3))
        dab, dba = oracle_mod.distance(a, b), oracle_mod.distance(b, a)
        assert oracle_mod.distance(a, a) == 0
        assert dab == dba
        assert 0 <= dab <= 384
        assert oracle_mod.distance(a, c) <= dab + oracle_mod.distance(b, c)


# ---------------------------------------------------------------- top-k


def check_topk_definition(d, budget, sel, k_eff):
    """Selected set = the k_eff smallest (distance, position) pairs, ascending, -1 padded."""
    n = d.shape[0]
    assert k_eff == min(budget, n)
    S = sel[:k_eff]
    assert np.all(sel[k_eff:] == -1)
    assert np.all(np.diff(S) > 0)
    assert S.min(initial=0) >= 0 and (k_eff == 0 or S.max() < n)
    chosen = np.zeros(n, bool)
    chosen[S] = True
    if k_eff and (~chosen).any():
        worst_in = max((int(d[p]), int(p)) for p in S)
        best_out = min((int(d[p]), int(p)) for p in np.nonzero(~chosen)[0])
        assert worst_in < best_out


def test_topk_definition_with_ties(oracle_mod):
    rng = np.random.default_rng(12)
    for _ in range(300):
        n = int(rng.integers(1, 40))
        d = rng.integers(0, 4, n).astype(np.uint16)  # heavy ties
        for budget in (1, 2, n // 2 + 1, n, n + 3):
            sel, k_eff = oracle_mod.topk(d, budget)
            check_topk_definition(d, budget, sel, k_eff)


def test_topk_brute_force_tiny(oracle_mod):
    """Exhaustive: among all k-subsets, the chosen one minimises the sorted (d, p) key list."""
    from itertools import combinations
    rng = np.random.default_rng(13)
    for _ in range(60):
        n = int(rng.integers(1, 8))
        d = rng.integers(0, 3, n).astype(np.uint16)
        k = int(rng.integers(1, n + 1))
        best = min(combinations(range(n), k), key=lambda s: sorted((int(d[p]), p) for p in s))
        sel, k_eff = oracle_mod.topk(d, k)
        assert list(sel[:k_eff]) == sorted(best)


def test_topk_all_equal_and_budget_over_len(oracle_mod):
    d = np.full(50, 7, np.uint16)
    sel, k_eff = oracle_mod.topk(d, 10)
    assert k_eff == 10 and list(sel) == list(range(10))
    sel, k_eff = oracle_mod.topk(d, 64)
    assert k_eff == 50 and list(sel[:50]) == list(range(50)) and np.all(sel[50:] == -1)


# ---------------------------------------------------------------- forced positions
# Blog sections 3.2 and 6 (special tokens keep full attention); the paper builds
# on attention-sink work (citation map).  Reading: sinks and the recent window
# (force 2) are always kept; special tokens of the caller's mask (force 1) take
# the rest of the budget first, lower positions first; then the other positions
# by (distance, position).


def test_topk_forced_brute_force_tiny(oracle_mod):
    """Exhaustive: the chosen k-subset holds every force-2 position, then the
    lowest force-1 positions that fit, and, among subsets that hold those,
    minimises the sorted (d, p) list of its other members."""
    from itertools import combinations
    rng = np.random.default_rng(31)
    for _ in range(300):
        n = int(rng.integers(1, 9))
        d = rng.integers(0, 3, n).astype(np.uint16)
        k = int(rng.integers(1, n + 1))
        f = np.where(rng.random(n) < 0.3, 1, 0).astype(np.uint8)
        always = rng.choice(n, int(rng.integers(0, k + 1)), replace=False)
        f[always] = 2
        A = set(always.tolist())
        P = [p for p in range(n) if f[p] == 1]
        want = A | set(P[:k - len(A)])
        subsets = [s for s in combinations(range(n), k) if want <= set(s)]
        best = min(subsets, key=lambda s: sorted((int(d[p]), p) for p in s if p not in want))
        sel, k_eff = oracle_mod.topk_forced(d, f, k)
        assert k_eff == k and list(sel[:k_eff]) == sorted(best)


def test_topk_forced_reductions(oracle_mod):
    rng = np.random.default_rng(32)
    for _ in range(100):
        n = int(rng.integers(1, 60))
        d = rng.integers(0, 6, n).astype(np.uint16)
        budget = int(rng.integers(1, n + 4))
        plain = oracle_mod.topk(d, budget)
        # no forced position (and a NULL mask): the plain top-k
        none = oracle_mod.topk_forced(d, np.zeros(n, np.uint8), budget)
        assert np.array_equal(none[0], plain[0]) and none[1] == plain[1]
        nul = oracle_mod.topk_forced(d, None, budget)
        assert np.array_equal(nul[0], plain[0])
        # forcing positions the plain top-k keeps anyway changes nothing
        f = np.zeros(n, np.uint8)
        kept = plain[0][:plain[1]]
        f[kept[rng.random(kept.size) < 0.5]] = 1
        assert np.array_equal(oracle_mod.topk_forced(d, f, budget)[0], plain[0])
        # forced (either kind) = exactly k positions: the selection is that set
        k = min(budget, n)
        F = np.sort(rng.choice(n, k, replace=False))
        for kind in (1, 2):
            f = np.zeros(n, np.uint8)
            f[F] = kind
            sel, k_eff = oracle_mod.topk_forced(d, f, budget)
            assert k_eff == k and np.array_equal(sel[:k], F)
        # more preferred positions than the budget: the lowest ones
        f = np.ones(n, np.uint8)
        sel, k_eff = oracle_mod.topk_forced(d, f, budget)
        assert np.array_equal(sel[:k], np.arange(k))


def test_topk_forced_distances_shifted_equivalence(oracle_mod):
    """Giving every forced position a distance below all others (a transform
    done here in numpy on the inputs) makes the plain top-k agree, as long as
    at most k_eff positions are forced."""
    rng = np.random.default_rng(33)
    for _ in range(100):
        n = int(rng.integers(1, 80))
        d = rng.integers(0, 385, n).astype(np.uint16)
        budget = int(rng.integers(1, n + 4))
        k_eff = min(budget, n)
        nf = int(rng.integers(0, k_eff + 1))
        f = np.zeros(n, np.uint8)
        f[rng.choice(n, nf, replace=False)] = 1
        shifted = np.where(f == 1, 0, d.astype(np.int64) + 1).astype(np.uint16)
        assert np.array_equal(oracle_mod.topk_forced(d, f, budget)[0], oracle_mod.topk(shifted, budget)[0])


def test_decode_forced_sink_recent_mask(oracle_mod):
    """The whole step with sinks, a recent window and a mask: every forced
    position is selected, the rest is the plain top-k of the others (numpy
    lexsort over the oracle's own distances), and out is attention over it."""
    wl = small_case(seed=24)
    codes = oracle_mod.encode_keys(wl.k, wl.kv_len)
    sink, recent, budget = 4, 6, 40
    words = (wl.cap + 31) // 32
    mask = np.zeros((wl.B, words), np.uint32)
    special = [(0, 77), (0, 250), (1, 3), (1, 120), (1, 200)]  # (b, position); 200 >= len of b = 1
    for b, p in special:
        mask[b, p // 32] |= np.uint32(1 << (p % 32))
    out, sel, dist, _ = oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, budget, wl.scale,
                                               sink=sink, recent=recent, mask=mask)
    group = wl.Hq // wl.Hkv
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        F = set(range(sink)) | set(range(L - recent, L)) | {p for bb, p in special if bb == b and p < L}
        for h in range(wl.Hq):
            k_eff = min(budget, L)
            S = sel[b, h, :k_eff]
            assert F <= set(S.tolist()) and np.all(sel[b, h, k_eff:] == -1)
            rest = np.array(sorted(set(range(L)) - F))
            d = dist[b, h, rest].astype(np.int64)
            others = np.sort(rest[np.lexsort((rest, d))[:k_eff - len(F)]])
            assert np.array_equal(np.sort(np.concatenate([np.array(sorted(F)), others])), S)
            g = h // group
            # (the step takes the scale as fp32)
            o = oracle_mod.attention_rows(wl.q[b, h], wl.k[b, g], wl.v[b, g], S, float(np.float32(wl.scale)))
            assert np.array_equal(out[b, h], o)


def test_decode_forced_window_kept_when_mask_overflows(oracle_mod):
    """A mask with more special tokens than the budget: the sinks and the
    window are still all kept, and the lowest special tokens outside them fill
    the rest."""
    wl = small_case(seed=26)
    codes = oracle_mod.encode_keys(wl.k, wl.kv_len)
    words = (wl.cap + 31) // 32
    mask = np.full((wl.B, words), 0x55555555, np.uint32)  # every even position
    sink, recent, budget = 3, 8, 30
    _, sel, _, _ = oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, budget, wl.scale, sink=sink,
                                          recent=recent, mask=mask)
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        always = list(range(sink)) + list(range(L - recent, L))
        evens = [p for p in range(sink, L - recent) if p % 2 == 0][:budget - len(always)]
        for h in range(wl.Hq):
            assert np.array_equal(sel[b, h], np.array(sorted(always + evens)))


def test_decode_forced_full_window_is_dense(oracle_mod):
    """recent = budget >= kv_len: every position is forced, so the step is dense attention."""
    wl = small_case(seed=25)
    codes = oracle_mod.encode_keys(wl.k, wl.kv_len)
    out, _, _, _ = oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, 300, wl.scale, recent=300)
    dense = oracle_mod.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale)
    assert np.array_equal(out, dense)


def test_decode_forced_invalid_arguments(oracle_mod):
    wl = small_case()
    codes = oracle_mod.encode_keys(wl.k, wl.kv_len)
    for kw in (dict(sink=-1), dict(recent=-2), dict(sink=20, recent=13)):
        with pytest.raises(ValueError):
            oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, 32, 0.1, **kw)
    with pytest.raises(ValueError):  # mask narrower than ceil(cap / 32) words
        oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, 32, 0.1, mask=np.zeros((2, 9), np.uint32))


# ---------------------------------------------------------------- attention


def bf(x):
    return W.f32_to_bf16(np.asarray(x, np.float32))


def test_attention_single_row_is_that_v_row(oracle_mod):
    rng = np.random.default_rng(14)
    K = bf(rng.standard_normal((10, 128)))
    V = bf(rng.standard_normal((10, 128)) * 5)
    q = bf(rng.standard_normal(128))
    out = oracle_mod.attention_rows(q, K, V, np.array([6], np.int32), 0.1)
    assert np.array_equal(out, W.bf16_to_f32(V[6]))


def test_attention_zero_query_is_mean(oracle_mod):
    rng = np.random.default_rng(15)
    K = bf(rng.standard_normal((20, 128)))
    V = bf(rng.standard_normal((20, 128)))
    pos = np.array([1, 4, 5, 19], np.int32)
    out = oracle_mod.attention_rows(bf(np.zeros(128)), K, V, pos, 1.0)
    want = W.bf16_to_f32(V[pos]).astype(np.float64).mean(axis=0)
    assert np.allclose(out, want, rtol=1e-6, atol=1e-7)


def test_attention_two_rows_closed_form(oracle_mod):
    """Scores 0 and ln 3 give weights 1/4 and 3/4."""
    K = np.zeros((2, 128), np.float32)
    K[1, 0] = 1.0
    V = np.zeros((2, 128), np.float32)
    V[0, :] = 4.0
    V[1, :] = -8.0
    q = np.zeros(128, np.float32)
    q[0] = 1.0
    out = oracle_mod.attention_rows(bf(q), bf(K), bf(V), np.array([0, 1], np.int32), float(np.log(3.0)))
    assert np.allclose(out, 0.25 * 4.0 + 0.75 * -8.0, rtol=1e-6)


def test_attention_large_scores_do_not_overflow(oracle_mod):
    K = np.zeros((3, 128), np.float32)
    K[:, 0] = [100.0, 200.0, 300.0]
    V = np.eye(3, 128, dtype=np.float32)
    q = np.zeros(128, np.float32)
    q[0] = 100.0
    out = oracle_mod.attention_rows(bf(q), bf(K), bf(V), np.array([0, 1, 2], np.int32), 1.0)
    assert np.all(np.isfinite(out)) and out[2] == 1.0 and out[0] == 0.0


# ---------------------------------------------------------------- whole step


def small_case(seed=20, B=2, Hq=4, Hkv=2, cap=300, lens=(300, 157), budget=32):
    wl = W.llama(seed, cap=cap, budget=budget, B=B, Hq=Hq, Hkv=Hkv, kv_len=np.array(lens, np.int32))
    return wl


def test_decode_full_budget_equals_dense(oracle_mod):
    wl = small_case(budget=400)
    codes = oracle_mod.encode_keys(wl.k, wl.kv_len)
    out, sel, _, _ = oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, 400, wl.scale)
    dense = oracle_mod.dense_attention(wl.q, wl.k, wl.v, wl.kv_len, wl.scale)
    assert np.array_equal(out, dense)
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(sel[b, :, :L], np.broadcast_to(np.arange(L), (wl.Hq, L)))


def test_decode_gqa_head_mapping(oracle_mod):
    """Query head h reads KV head h // (Hq/Hkv): V = +1 in KV head 0 and -1 in KV head 1."""
    B, Hq, Hkv, cap = 1, 4, 2, 64
    rng = np.random.default_rng(21)
    k = bf(rng.standard_normal((B, Hkv, cap, 128)))
    v = np.empty((B, Hkv, cap, 128), np.uint16)
    v[:, 0] = bf(np.ones((cap, 128)))
    v[:, 1] = bf(-np.ones((cap, 128)))
    q = bf(rng.standard_normal((B, Hq, 128)))
    kv_len = np.array([cap], np.int32)
    codes = oracle_mod.encode_keys(k, kv_len)
    out, _, _, _ = oracle_mod.decode_step(q, k, v, codes, kv_len, 8, 0.1)
    assert np.all(out[0, 0:2] == 1.0) and np.all(out[0, 2:4] == -1.0)


def test_decode_batch_is_independent(oracle_mod):
    wl = small_case()
    codes = oracle_mod.encode_keys(wl.k, wl.kv_len)
    out, sel, dist, qc = oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, wl.budget, wl.scale)
    for b in range(wl.B):
        o1, s1, d1, q1 = oracle_mod.decode_step(wl.q[b:b + 1], wl.k[b:b + 1], wl.v[b:b + 1], codes[b:b + 1],
                                                wl.kv_len[b:b + 1], wl.budget, wl.scale)
        assert np.array_equal(o1[0], out[b]) and np.array_equal(s1[0], sel[b])
        assert np.array_equal(d1[0], dist[b]) and np.array_equal(q1[0], qc[b])


def test_decode_empty_sequence(oracle_mod):
    """A sequence with no cached position (an idle batch slot) selects nothing
    and gets the zero vector, by the empty-sum reading; the other entries are
    what they are alone, with and without forced positions, and dense attention
    agrees."""
    wl = small_case()
    codes = oracle_mod.encode_keys(wl.k, wl.kv_len)
    lens = wl.kv_len.copy()
    lens[0] = 0
    for kw in ({}, dict(sink=2, recent=3)):
        out, sel, dist, _ = oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, lens, wl.budget, wl.scale, **kw)
        assert np.all(out[0] == 0.0) and np.all(sel[0] == -1) and np.all(dist[0] == 0)
        o1, s1, d1, _ = oracle_mod.decode_step(wl.q[1:], wl.k[1:], wl.v[1:], codes[1:], lens[1:], wl.budget,
                                               wl.scale, **kw)
        assert np.array_equal(o1, out[1:]) and np.array_equal(s1, sel[1:]) and np.array_equal(d1, dist[1:])
    dense = oracle_mod.dense_attention(wl.q, wl.k, wl.v, lens, wl.scale)
    assert np.all(dense[0] == 0.0)
    assert np.array_equal(dense[1:], oracle_mod.dense_attention(wl.q[1:], wl.k[1:], wl.v[1:], lens[1:], wl.scale))
    assert np.all(oracle_mod.attention_rows(wl.q[0, 0], wl.k[0, 0], wl.v[0, 0], np.zeros(0, np.int32), 0.1) == 0.0)


def test_decode_rederived_in_numpy(oracle_mod):
    """Independent numpy path for the step after encoding: unpackbits distances,
    lexsort top-k, fp64 softmax attention."""
    wl = small_case(seed=22)
    codes = oracle_mod.encode_keys(wl.k, wl.kv_len)
    out, sel, dist, qc = oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, wl.budget, wl.scale)
    group = wl.Hq // wl.Hkv

    def unpack(c):
        bits = np.unpackbits(c.reshape(-1, 2, 16), axis=-1, bitorder="little").astype(np.int64)
        return bits[:, 0, :] + 2 * bits[:, 1, :]

    for b in range(wl.B):
        L = int(wl.kv_len[b])
        for h in range(wl.Hq):
            g = h // group
            assert np.array_equal(qc[b, h], oracle_mod.encode_vector(wl.q[b, h]))
            d = np.abs(unpack(codes[b, g, :L]) - unpack(qc[b, h][None])).sum(axis=1)
            assert np.array_equal(dist[b, h, :L], d)
            k_eff = min(wl.budget, L)
            order = np.lexsort((np.arange(L), d))[:k_eff]
            S = np.sort(order)
            assert np.array_equal(sel[b, h, :k_eff], S) and np.all(sel[b, h, k_eff:] == -1)
            qf = W.bf16_to_f32(wl.q[b, h]).astype(np.float64)
            Kf = W.bf16_to_f32(wl.k[b, g, S]).astype(np.float64)
            Vf = W.bf16_to_f32(wl.v[b, g, S]).astype(np.float64)
            s = wl.scale * (Kf @ qf)
            w = np.exp(s - s.max())
            o = (w[:, None] * Vf).sum(0) / w.sum()
            assert np.allclose(out[b, h], o, rtol=1e-6, atol=1e-6 * np.abs(o).max())


def test_append_equals_prefill_row(oracle_mod):
    wl = small_case(seed=23)
    full = oracle_mod.encode_keys(wl.k, wl.kv_len)
    start = wl.kv_len - 1
    app = oracle_mod.encode_keys(wl.k, wl.kv_len, start=start)
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(app[b, :, L - 1], full[b, :, L - 1])
        assert not app[b, :, : L - 1].any() and not app[b, :, L:].any()


def test_invalid_arguments_rejected(oracle_mod):
    wl = small_case()
    codes = oracle_mod.encode_keys(wl.k, wl.kv_len)
    with pytest.raises(ValueError):
        oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, np.array([-1, 5], np.int32), 8, 0.1)
    with pytest.raises(ValueError):
        oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, np.array([wl.cap + 1, 5], np.int32), 8, 0.1)
    with pytest.raises(ValueError):
        oracle_mod.decode_step(wl.q, wl.k, wl.v, codes, wl.kv_len, 0, 0.1)
    with pytest.raises(ValueError):
        oracle_mod.encode_keys(wl.k, np.array([301, 5], np.int32))
