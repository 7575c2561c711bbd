"""Seeded synthetic decode-step inputs shaped like the pages' workloads.

This module holds no step of the method: it only draws numbers and stores them as
bf16 bit patterns.  Both the oracle and the GPU library are fed from it.

The pages evaluate on Llama-3.1-8B-Instruct at 32K context (paper abstracts) with
real data; no weights or datasets are used here.  These generators stand in for
that with its attention shape (32 query heads, 8 KV heads, head_dim 128) and with
value distributions chosen to exercise the method: heavy per-channel scales
(outlier channels, which the Hadamard transform is meant to spread) and queries
built from a few planted keys, so that a good selection exists.

Recipes (numpy.random.default_rng(seed); draws happen in the order listed;
values are drawn in fp32 and rounded to bf16 with round-to-nearest-even):

* tiny       B=1, Hq=Hkv=1, N=1024, budget 64.
             K, V ~ N(0,1) [1,1,N,128]; ch = choice(128, 4, no replace);
             K[...,ch] *= 20, V[...,ch] *= 20; P = choice(N, 8, no replace);
             q = sum_{p in P} K_bf16[p] + N(0, 0.5^2) noise.
* llama      B, Hq=32, Hkv=8, cap, kv_len (default: all = cap).
             Per (b, kv head): s_K, s_V ~ LogNormal(0, 1) per channel [128];
             K = N(0,1) * s_K, V = N(0,1) * s_V, each (tensor, b, kv head) slice
             from its own stream default_rng([seed, 1 for K / 2 for V, b, g]);
             per (b, q head h): P_h = choice(kv_len[b], 16, no replace),
             q_h = sum_{p in P_h} K_bf16[b, g(h), p] + N(0, 0.5^2) noise.
             Positions >= kv_len[b] hold a bf16 NaN so that any read past the
             valid length poisons the result.
* batched    B=16, cap=32768: kv_len[b] = integers(16384, 32768, endpoint=True)
             drawn first for all b, then the llama recipe.  Budget 256.
"""
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

HEAD_DIM = 128
BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16(x: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = (u >> np.uint32(16)) & np.uint32(1)
    t += np.uint32(0x7FFF)
    t += u
    t >>= np.uint32(16)
    if out is None:
        return t.astype(np.uint16)
    out[...] = t
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    q: np.ndarray          # uint16 [B][Hq][128]
    k: np.ndarray          # uint16 [B][Hkv][cap][128]
    v: np.ndarray          # uint16 [B][Hkv][cap][128]
    kv_len: np.ndarray     # int32 [B]
    budget: int
    planted: List[np.ndarray] = field(default_factory=list)  # per (b*Hq + h): planted positions
    seed: int = 0

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def Hq(self) -> int:
        return self.q.shape[1]

    @property
    def Hkv(self) -> int:
        return self.k.shape[1]

    @property
    def cap(self) -> int:
        return self.k.shape[2]

    @property
    def scale(self) -> float:
        return float(1.0 / np.sqrt(HEAD_DIM))


def tiny(seed: int = 0, n: int = 1024, budget: int = 64) -> Workload:
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((1, 1, n, HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((1, 1, n, HEAD_DIM), dtype=np.float32)
    ch = rng.choice(HEAD_DIM, 4, replace=False)
    k[..., ch] *= 20.0
    v[..., ch] *= 20.0
    kb = f32_to_bf16(k)
    vb = f32_to_bf16(v)
    P = rng.choice(n, 8, replace=False)
    q = bf16_to_f32(kb[0, 0, P]).sum(axis=0) + rng.normal(0.0, 0.5, HEAD_DIM).astype(np.float32)
    qb = f32_to_bf16(q.astype(np.float32)).reshape(1, 1, HEAD_DIM)
    return Workload("tiny", qb, kb, vb, np.array([n], np.int32), budget, [np.sort(P)], seed)


def llama(seed: int = 0, cap: int = 32768, budget: int = 128, B: int = 1, Hq: int = 32, Hkv: int = 8,
          kv_len: Optional[np.ndarray] = None, rng: Optional[np.random.Generator] = None,
          name: Optional[str] = None, n_planted: int = 16) -> Workload:
    rng = np.random.default_rng(seed) if rng is None else rng
    if kv_len is None:
        kv_len = np.full(B, cap, np.int32)
    kv_len = np.asarray(kv_len, np.int32)
    assert kv_len.shape == (B,) and kv_len.min() >= 1 and kv_len.max() <= cap and Hq % Hkv == 0
    group = Hq // Hkv
    sK = rng.lognormal(0.0, 1.0, (B, Hkv, HEAD_DIM)).astype(np.float32)
    sV = rng.lognormal(0.0, 1.0, (B, Hkv, HEAD_DIM)).astype(np.float32)
    k = np.empty((B, Hkv, cap, HEAD_DIM), np.uint16)
    v = np.empty((B, Hkv, cap, HEAD_DIM), np.uint16)

    def fill(job):
        # each (tensor, b, kv head) slice has its own stream, so slices fill in parallel
        tag, b, g = job
        dst, scl = (k, sK) if tag == 0 else (v, sV)
        buf = np.random.default_rng([seed, 1 + tag, b, g]).standard_normal((cap, HEAD_DIM), dtype=np.float32)
        buf *= scl[b, g]
        f32_to_bf16(buf, out=dst[b, g])

    jobs = [(t, b, g) for t in (0, 1) for b in range(B) for g in range(Hkv)]
    with ThreadPoolExecutor(max_workers=min(16, len(jobs))) as ex:
        list(ex.map(fill, jobs))
    q = np.empty((B, Hq, HEAD_DIM), np.uint16)
    planted = []
    for b in range(B):
        L = int(kv_len[b])
        for h in range(Hq):
            g = h // group
            P = rng.choice(L, min(n_planted, L), replace=False)
            qf = bf16_to_f32(k[b, g, P]).sum(axis=0) + rng.normal(0.0, 0.5, HEAD_DIM).astype(np.float32)
            q[b, h] = f32_to_bf16(qf.astype(np.float32))
            planted.append(np.sort(P))
    for b in range(B):
        L = int(kv_len[b])
        if L < cap:
            k[b, :, L:] = BF16_NAN
            v[b, :, L:] = BF16_NAN
    nm = name or ("llama_b%d_n%d_k%d" % (B, cap, budget))
    return Workload(nm, q, k, v, kv_len, budget, planted, seed)


def batched_lengths(rng: np.random.Generator, B: int = 16, cap: int = 32768, lo: int = 16384) -> np.ndarray:
    """The batched recipe's lengths: uniform integers in [lo, cap], drawn first."""
    return rng.integers(lo, cap, size=B, endpoint=True).astype(np.int32)


def batched(seed: int = 0, B: int = 16, cap: int = 32768, budget: int = 256, lo: int = 16384) -> Workload:
    rng = np.random.default_rng(seed)
    kv_len = batched_lengths(rng, B, cap, lo)
    return llama(seed, cap=cap, budget=budget, B=B, kv_len=kv_len, rng=rng,
                 name="batched_b%d_n%d_k%d" % (B, cap, budget))


def by_name(name: str, seed: int = 0) -> Workload:
    """Named configurations used by the tests and the benchmark."""
    if name == "tiny":
        return tiny(seed)
    if name == "llama32k_k128":
        return llama(seed, cap=32768, budget=128)
    if name == "llama32k_k1024":
        return llama(seed, cap=32768, budget=1024)
    if name == "batched16":
        return batched(seed)
    if name == "long512k":
        return llama(seed, cap=524288, budget=1024, name="long512k")
    if name.startswith("sweep_"):
        # sweep_<N>_<budget>, e.g. sweep_4096_64
        _, n, kb = name.split("_")
        return llama(seed, cap=int(n), budget=int(kb), name=name)
    raise KeyError(name)
