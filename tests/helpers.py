"""Shared helpers for the GPU parity tests: host<->device marshalling of the
seeded workloads and the parity bars.

Bars (from the method's integer/float split): codes, distances, query codes and
selected indices are integers and must match the oracle exactly; the attention
output must satisfy max_j |o_gpu - o_ref| <= 2e-3 * ||o_ref||_2 per (b, h) row
(bf16 inputs, fp32 accumulation on the GPU vs fp64 in the oracle).
"""
import numpy as np

OUT_RTOL = 2e-3


def to_dev(a, torch):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def from_dev(t, dtype=None):
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def assert_out_close(got, ref, rtol=OUT_RTOL, what="out"):
    got = np.asarray(got, np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    assert np.all(np.isfinite(got)), "%s has non-finite values" % what
    err = np.abs(got - ref).max(axis=1)
    bound = rtol * np.linalg.norm(ref, axis=1)
    worst = int(np.argmax(err / np.maximum(bound, 1e-30)))
    assert np.all(err <= bound), "%s row %d: max|err| %.3e > %.3e" % (what, worst, err[worst], bound[worst])
    return float((err / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)).max())


class DeviceCase:
    """A workload uploaded to the GPU with its codes encoded by the library."""

    def __init__(self, wl, A, torch, encode=True):
        self.wl = wl
        self.A = A
        self.torch = torch
        self.q = to_dev(wl.q, torch)
        self.k = to_dev(wl.k, torch)
        self.v = to_dev(wl.v, torch)
        self.kv_len = to_dev(wl.kv_len.astype(np.int32), torch)
        self.codes = torch.zeros((wl.B, wl.Hkv, wl.cap, 32), dtype=torch.uint8, device="cuda")
        if encode:
            A.encode_keys(self.k, self.kv_len, self.codes)

    def decode(self, budget=None, want_debug=True, sink=None, recent=None, mask=None, append=False):
        """One decode step through the C ABI; sink / recent / mask (a host uint32
        [B][words] bitmap) select the forced-position entry point."""
        A, torch, wl = self.A, self.torch, self.wl
        mask_dev = None if mask is None else to_dev(np.ascontiguousarray(mask, np.uint32).view(np.int32), torch)
        budget = wl.budget if budget is None else budget
        out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
        sel = torch.full((wl.B, wl.Hq, budget), -7, dtype=torch.int32, device="cuda")
        dist = torch.zeros((wl.B, wl.Hq, wl.cap), dtype=torch.int16, device="cuda") if want_debug else None
        qc = torch.zeros((wl.B, wl.Hq, 32), dtype=torch.uint8, device="cuda") if want_debug else None
        ws = A.alloc_workspace(A.decode_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap, budget))
        ws.fill_(0xFF)  # poison: any read of scratch not written by this call shows up
        A.decode_step(self.q, self.k, self.v, self.codes, self.kv_len, budget, wl.scale, out, ws, sel_idx=sel,
                      dist=dist, q_codes=qc, sink=sink, recent=recent, mask=mask_dev, append=append)
        torch.cuda.synchronize()
        return (from_dev(out), from_dev(sel), None if dist is None else from_dev(dist, np.uint16),
                None if qc is None else from_dev(qc))

    def dense(self):
        A, torch, wl = self.A, self.torch, self.wl
        out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device="cuda")
        ws = A.alloc_workspace(A.dense_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.cap))
        ws.fill_(0xFF)
        A.dense_decode_attention(self.q, self.k, self.v, self.kv_len, wl.scale, out, ws)
        torch.cuda.synchronize()
        return from_dev(out)


def paginate(a, page, rng, spare=3, fill=0):
    """Scatter a contiguous cache [B][H][cap][D] into a page pool [N][H][page][D]:
    sequence b's logical page j goes to physical page table[b][j], a random
    permutation over N = B * ceil(cap / page) + spare pages (the spare pages and
    the tail of a last partial page hold `fill`).  Returns (pool, table)."""
    B, H, cap, D = a.shape
    mp = -(-cap // page)
    n = B * mp + spare
    table = rng.permutation(n)[:B * mp].reshape(B, mp).astype(np.int32)
    padded = np.full((B, H, mp * page, D), fill, a.dtype)
    padded[:, :, :cap] = a
    pool = np.full((n, H, page, D), fill, a.dtype)
    pool[table.reshape(-1)] = padded.reshape(B, H, mp, page, D).transpose(0, 2, 1, 3, 4).reshape(B * mp, H, page, D)
    return pool, table


def unpaginate(pool, table, cap):
    """The contiguous view [B][H][cap][D] of a page pool through its table."""
    B, mp = table.shape
    n, H, page, D = pool.shape
    out = pool[table.reshape(-1)].reshape(B, mp, H, page, D).transpose(0, 2, 1, 3, 4).reshape(B, H, mp * page, D)
    return out[:, :, :cap]
