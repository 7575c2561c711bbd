"""Seeded random configurations against the CPU oracle: batch 1-4, group sizes
1/2/4/8, 1-3 KV heads, capacities 1-6000, ragged lengths (1 .. capacity),
budgets from 1 to twice the capacity, with or without forced positions
(sinks / window / special tokens), contiguous or paged (page sizes 1-256),
with or without the fused key append.  Every case checks key codes, query
codes, distances and selections exactly and the output within 2e-3 of the row
norm, as the hand-picked cases do."""
import numpy as np
import pytest

import workloads as W
from helpers import DeviceCase, assert_out_close, from_dev, paginate, to_dev, unpaginate

pytestmark = pytest.mark.gpu

N_CASES = 64


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import sparse_attention_long_fwht_amd as A
    import oracle
    return A, torch, oracle


def draw(seed):
    rng = np.random.default_rng(1000 + seed)
    R = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.integers(1, 4))
    B = int(rng.integers(1, 5))
    cap = int(rng.choice([1, 7, 64, 513, 1024, 2500, 6000]))
    lens = rng.integers(1, cap + 1, B).astype(np.int32)
    budget = int(rng.integers(1, 2 * cap + 2))
    cfg = dict(R=R, Hkv=Hkv, B=B, cap=cap, lens=lens, budget=budget, append=bool(rng.random() < 0.5))
    if rng.random() < 0.4:
        sink = int(rng.integers(0, budget + 1))
        recent = int(rng.integers(0, budget - sink + 1))
        cfg["forced"] = dict(sink=sink, recent=recent)
        if rng.random() < 0.5:
            words = (cap + 31) // 32
            mask = np.zeros((B, words), np.uint32)
            for b in range(B):
                for p in rng.choice(cap, min(cap, int(rng.integers(1, 20))), replace=False):
                    mask[b, p // 32] |= np.uint32(1 << (int(p) % 32))
            cfg["forced"]["mask"] = mask
    if rng.random() < 0.4:
        cfg["page"] = int(rng.choice([1, 4, 16, 64, 256]))
    return cfg


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(env, seed):
    A, torch, oracle = env
    cfg = draw(seed)
    print("case", seed, {k: v for k, v in cfg.items() if k not in ("lens",)}, "lens", cfg["lens"].tolist()[:4],
          flush=True)
    wl = W.llama(2000 + seed, cap=cfg["cap"], budget=cfg["budget"], B=cfg["B"], Hq=cfg["R"] * cfg["Hkv"],
                 Hkv=cfg["Hkv"], kv_len=cfg["lens"], n_planted=4)
    forced = cfg.get("forced", {})
    budget = cfg["budget"]
    codes_ref = oracle.encode_keys(wl.k, wl.kv_len)
    out_r, sel_r, dist_r, qc_r = oracle.decode_step(wl.q, wl.k, wl.v, codes_ref, wl.kv_len, budget, wl.scale,
                                                    threads=8, **forced)
    page = cfg.get("page")
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
    sel = torch.full((wl.B, wl.Hq, budget), -7, dtype=torch.int32, device="cuda")
    dist = torch.zeros((wl.B, wl.Hq, wl.cap), dtype=torch.int16, device="cuda")
    qc = torch.zeros((wl.B, wl.Hq, 32), dtype=torch.uint8, device="cuda")
    ws = A.alloc_workspace(A.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap, budget))
    ws.fill_(0xFF)
    kw = dict(forced)
    if "mask" in kw:
        kw["mask"] = to_dev(kw["mask"].view(np.int32), torch)
    if page is None:
        case = DeviceCase(wl, A, torch)
        if cfg["append"]:  # the step must write the last code itself
            for b in range(wl.B):
                case.codes[b, :, int(wl.kv_len[b]) - 1] = 0
        A.decode_step(case.q, case.k, case.v, case.codes, case.kv_len, budget, wl.scale, out, ws, sel_idx=sel,
                      dist=dist, q_codes=qc, append=cfg["append"], **kw)
        torch.cuda.synchronize()
        codes = from_dev(case.codes)
    else:
        kp, table = paginate(wl.k, page, np.random.default_rng(seed))
        vp, _ = paginate(wl.v, page, np.random.default_rng(seed))
        kd, vd, td = to_dev(kp, torch), to_dev(vp, torch), to_dev(table, torch)
        kv_len = to_dev(wl.kv_len, torch)
        pages = A.Pages(td, page, capacity=wl.cap)
        cp = torch.zeros((kp.shape[0], wl.Hkv, page, 32), dtype=torch.uint8, device="cuda")
        A.encode_keys(kd, kv_len, cp, pages=pages, num_q_heads=wl.Hq)
        if cfg["append"]:
            for b in range(wl.B):
                p = int(wl.kv_len[b]) - 1
                cp[int(table[b, p // page]), :, p % page] = 0
        A.decode_step(to_dev(wl.q, torch), kd, vd, cp, kv_len, budget, wl.scale, out, ws, sel_idx=sel, dist=dist,
                      q_codes=qc, append=cfg["append"], pages=pages, **kw)
        torch.cuda.synchronize()
        codes = unpaginate(from_dev(cp), table, wl.cap)
    for b in range(wl.B):
        L = int(wl.kv_len[b])
        assert np.array_equal(codes[b, :, :L], codes_ref[b, :, :L]), "codes differ (b=%d)" % b
        assert np.array_equal(from_dev(dist, np.uint16)[b, :, :L], dist_r[b, :, :L]), "distances differ (b=%d)" % b
    assert np.array_equal(from_dev(qc), qc_r)
    assert np.array_equal(from_dev(sel), sel_r), "selected indices differ"
    assert_out_close(from_dev(out), out_r)
