"""Python binding of libadamas.so (the Adamas decode step on gfx950).

Argument marshalling only: every step of the path runs in the HIP kernels behind
the C ABI declared in include/adamas.h.  Tensors are torch tensors on the current
HIP device; bf16 tensors may be torch.bfloat16 or any 2-byte dtype holding the
bf16 bit patterns.  Calls enqueue on the current torch stream unless `stream` is
given.  There is no CPU fallback: importing this package fails if the library has
not been built (python -c "import __graft_entry__ as g; g.build()").
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libadamas.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libadamas.so is not built at %s; build it with sparse_attention_long_fwht_amd/build.py"
                      % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

HEAD_DIM = 128
CODE_BYTES = 32

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_WORKSPACE = 3
ERR_HIP = 4


class Dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32)]


class Forced(ctypes.Structure):
    _fields_ = [("sink", ctypes.c_int32), ("recent", ctypes.c_int32), ("mask", ctypes.c_void_p),
                ("mask_words", ctypes.c_int32)]


class _PagesC(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


class Pages:
    """A paged cache description: block_table int32 [B][max_pages] (device),
    positions per page (a power of two), and the longest a sequence may grow
    (default max_pages * page_size).  The K/V pools passed with it are
    [num_pages][Hkv][page_size][128], the codes pool [num_pages][Hkv][page_size][32]."""

    def __init__(self, block_table, page_size, capacity=None):
        if block_table.dim() != 2 or block_table.element_size() != 4:
            raise ValueError("block_table must be int32 [batch][max_pages]")
        self.table = block_table
        self.page_size = int(page_size)
        self.capacity = int(capacity) if capacity is not None else block_table.shape[1] * self.page_size

    def c(self, num_pages):
        return _PagesC(_ptr(self.table, "block_table", 4), self.table.shape[1], self.page_size, int(num_pages))


_vp = ctypes.c_void_p
_dims_p = ctypes.POINTER(Dims)
_pages_p = ctypes.POINTER(_PagesC)
_lib.adamas_encode_keys.argtypes = [_dims_p, _vp, _vp, _vp, _vp, _vp]
_lib.adamas_encode_keys.restype = ctypes.c_int
_lib.adamas_decode_workspace_size.argtypes = [_dims_p, ctypes.c_int32]
_lib.adamas_decode_workspace_size.restype = ctypes.c_size_t
_lib.adamas_decode_step.argtypes = [_dims_p, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_float, _vp, _vp,
                                    _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.adamas_decode_step.restype = ctypes.c_int
_lib.adamas_decode_step_noalloc.argtypes = [_dims_p, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, ctypes.c_float, _vp,
                                            _vp, _vp, _vp, _vp]
_lib.adamas_decode_step_noalloc.restype = ctypes.c_int
_lib.adamas_append_decode_step.argtypes = _lib.adamas_decode_step.argtypes
_lib.adamas_append_decode_step.restype = ctypes.c_int
_lib.adamas_forced_decode_step.argtypes = [_dims_p, ctypes.POINTER(Forced), ctypes.c_int32, _vp, _vp, _vp, _vp, _vp,
                                           ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                           _vp]
_lib.adamas_forced_decode_step.restype = ctypes.c_int
_lib.adamas_paged_encode_keys.argtypes = [_dims_p, _pages_p, _vp, _vp, _vp, _vp, _vp]
_lib.adamas_paged_encode_keys.restype = ctypes.c_int
_lib.adamas_encode_keys_bounded.argtypes = [_dims_p, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp]
_lib.adamas_encode_keys_bounded.restype = ctypes.c_int
_lib.adamas_paged_encode_keys_bounded.argtypes = [_dims_p, _pages_p, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp]
_lib.adamas_paged_encode_keys_bounded.restype = ctypes.c_int
_lib.adamas_paged_decode_step.argtypes = [_dims_p, _pages_p, ctypes.POINTER(Forced), ctypes.c_int32, _vp, _vp, _vp,
                                          _vp, _vp, ctypes.c_int32, ctypes.c_float, _vp, _vp, _vp, _vp, _vp,
                                          ctypes.c_size_t, _vp]
_lib.adamas_paged_decode_step.restype = ctypes.c_int
_lib.dense_paged_decode_attention.argtypes = [_dims_p, _pages_p, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp,
                                              ctypes.c_size_t, _vp]
_lib.dense_paged_decode_attention.restype = ctypes.c_int
_lib.dense_decode_workspace_size.argtypes = [_dims_p]
_lib.dense_decode_workspace_size.restype = ctypes.c_size_t
_lib.dense_decode_attention.argtypes = [_dims_p, _vp, _vp, _vp, _vp, ctypes.c_float, _vp, _vp, ctypes.c_size_t,
                                        _vp]
_lib.dense_decode_attention.restype = ctypes.c_int
_lib.adamas_status_string.argtypes = [ctypes.c_int]
_lib.adamas_status_string.restype = ctypes.c_char_p
_lib.adamas_profile_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32]
_lib.adamas_profile_events.restype = ctypes.c_int
_lib.adamas_decode_launch_mode.argtypes = [ctypes.c_int32]
_lib.adamas_decode_launch_mode.restype = ctypes.c_int
_lib.adamas_last_launch_count.argtypes = []
_lib.adamas_last_launch_count.restype = ctypes.c_int32
_lib.adamas_abi_version.argtypes = []
_lib.adamas_abi_version.restype = ctypes.c_int32

EXPORTED_SYMBOLS = ("adamas_encode_keys", "adamas_decode_workspace_size", "adamas_decode_step",
                    "adamas_decode_step_noalloc",
                    "adamas_append_decode_step", "adamas_forced_decode_step", "adamas_paged_encode_keys",
                    "adamas_encode_keys_bounded", "adamas_paged_encode_keys_bounded",
                    "adamas_paged_decode_step", "dense_decode_workspace_size", "dense_decode_attention",
                    "dense_paged_decode_attention", "adamas_profile_events", "adamas_status_string",
                    "adamas_abi_version", "adamas_decode_launch_mode", "adamas_last_launch_count")


class AdamasError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


def status_string(status: int) -> str:
    return _lib.adamas_status_string(int(status)).decode()


def abi_version() -> int:
    return int(_lib.adamas_abi_version())


def dims(batch: int, num_q_heads: int, num_kv_heads: int, capacity: int, head_dim: int = HEAD_DIM) -> Dims:
    return Dims(int(batch), int(num_q_heads), int(num_kv_heads), int(head_dim), int(capacity))


def _ptr(t, name, itemsize=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if itemsize is not None and t.element_size() != itemsize:
        raise ValueError("%s must have %d-byte elements" % (name, itemsize))
    return t.data_ptr()


def _shape(t, name, shape, device=None):
    """Raise unless t (if given) has exactly `shape` and lives on `device`: the
    kernels index every buffer by the dims, so a short buffer would be written
    past its end rather than rejected."""
    if t is None:
        return
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, [int(x) for x in shape], list(t.shape)))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, the other tensors on %s" % (name, t.device, device))


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(status, where):
    if status != OK:
        raise AdamasError(status, where)


def encode_keys(k, end, codes, start=None, stream=None, num_q_heads=None, pages=None, max_rows=None):
    """Encode keys at positions [start[b], end[b]) of k [B][Hkv][cap][128] into codes [B][Hkv][cap][32]
    (with `pages`: of the pools k [num_pages][Hkv][page][128] into codes [num_pages][Hkv][page][32]).
    max_rows: the caller's bound on end[b] - start[b] (adamas_encode_keys_bounded: it sizes the launch)."""
    if k.dim() != 4:
        raise ValueError("k must be 4-D")
    dev = k.device
    if pages is None:
        B, Hkv, cap, hd = k.shape
        _shape(codes, "codes", (B, Hkv, cap, CODE_BYTES), dev)
        _shape(end, "end", (B,), dev)
        _shape(start, "start", (B,), dev)
        d = dims(B, num_q_heads or Hkv, Hkv, cap, hd)
        if max_rows is not None:
            st = _lib.adamas_encode_keys_bounded(ctypes.byref(d), _ptr(k, "k", 2),
                                                 _ptr(start, "start", 4, optional=True), _ptr(end, "end", 4),
                                                 int(max_rows), _ptr(codes, "codes", 1), _stream(stream))
            _check(st, "adamas_encode_keys_bounded")
            return
        st = _lib.adamas_encode_keys(ctypes.byref(d), _ptr(k, "k", 2), _ptr(start, "start", 4, optional=True),
                                     _ptr(end, "end", 4), _ptr(codes, "codes", 1), _stream(stream))
        _check(st, "adamas_encode_keys")
        return
    num_pages, Hkv, page, hd = k.shape
    B = pages.table.shape[0]
    if page != pages.page_size:
        raise ValueError("the k pool holds pages of %d positions, the page table %d" % (page, pages.page_size))
    _shape(codes, "codes", (num_pages, Hkv, page, CODE_BYTES), dev)
    _shape(end, "end", (B,), dev)
    _shape(start, "start", (B,), dev)
    _shape(pages.table, "block_table", pages.table.shape, dev)
    d = dims(B, num_q_heads or Hkv, Hkv, pages.capacity, hd)
    pc = pages.c(num_pages)
    if max_rows is not None:
        st = _lib.adamas_paged_encode_keys_bounded(ctypes.byref(d), ctypes.byref(pc), _ptr(k, "k", 2),
                                                   _ptr(start, "start", 4, optional=True), _ptr(end, "end", 4),
                                                   int(max_rows), _ptr(codes, "codes", 1), _stream(stream))
        _check(st, "adamas_paged_encode_keys_bounded")
        return
    st = _lib.adamas_paged_encode_keys(ctypes.byref(d), ctypes.byref(pc), _ptr(k, "k", 2),
                                       _ptr(start, "start", 4, optional=True), _ptr(end, "end", 4),
                                       _ptr(codes, "codes", 1), _stream(stream))
    _check(st, "adamas_paged_encode_keys")


def decode_workspace_size(B, Hq, Hkv, cap, budget, head_dim=HEAD_DIM) -> int:
    return int(_lib.adamas_decode_workspace_size(ctypes.byref(dims(B, Hq, Hkv, cap, head_dim)), int(budget)))


def dense_workspace_size(B, Hq, Hkv, cap, head_dim=HEAD_DIM) -> int:
    return int(_lib.dense_decode_workspace_size(ctypes.byref(dims(B, Hq, Hkv, cap, head_dim))))


def alloc_workspace(nbytes, device=None):
    """A device byte tensor usable as workspace (torch allocations are 256-byte aligned)."""
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device or "cuda")


def _check_shapes(q, k, v, codes, kv_len, out, pages):
    """The shapes shared by the decode step and dense attention: q [B][Hq][hd],
    k and v [B][Hkv][cap][hd] (with pages: pools [num_pages][Hkv][page][hd]),
    codes k's leading dims by 32, kv_len [B], out [B][Hq][128].  Returns B, Hq,
    Hkv and the capacity."""
    if q.dim() != 3 or k.dim() != 4:
        raise ValueError("q must be [batch][q heads][head_dim] and k 4-D")
    B, Hq, hd = q.shape
    n0, Hkv, rows, _ = k.shape
    dev = q.device
    _shape(k, "k", (n0, Hkv, rows, hd), dev)
    _shape(v, "v", k.shape, dev)
    _shape(codes, "codes", (n0, Hkv, rows, CODE_BYTES), dev)
    _shape(kv_len, "kv_len", (B,), dev)
    _shape(out, "out", (B, Hq, HEAD_DIM), dev)
    if pages is None:
        if n0 != B:
            raise ValueError("k has %d sequences, q %d" % (n0, B))
        return B, Hq, Hkv, rows
    if rows != pages.page_size:
        raise ValueError("the k pool holds pages of %d positions, the page table %d" % (rows, pages.page_size))
    if pages.table.shape[0] != B:
        raise ValueError("the page table has %d rows, q %d sequences" % (pages.table.shape[0], B))
    _shape(pages.table, "block_table", pages.table.shape, dev)
    return B, Hq, Hkv, pages.capacity


def decode_step(q, k, v, codes, kv_len, budget, scale, out, workspace, sel_idx=None, dist=None, q_codes=None,
                stream=None, append=False, sink=None, recent=None, mask=None, pages=None):
    """One Adamas decode step; writes out [B][Hq][128] fp32 (and the optional outputs).

    append=True calls adamas_append_decode_step: the key at kv_len[b]-1 is
    encoded into `codes` first (no separate encode launch).  Any of sink /
    recent / mask (int32 [B][words] device bitmap, bit p % 32 of word p / 32)
    calls adamas_forced_decode_step with those forced positions.  `pages`
    (a Pages) calls adamas_paged_decode_step: k, v and codes are then pools."""
    B, Hq, Hkv, cap = _check_shapes(q, k, v, codes, kv_len, out, pages)
    hd = q.shape[2]
    _shape(sel_idx, "sel_idx", (B, Hq, int(budget)), q.device)
    _shape(dist, "dist", (B, Hq, cap), q.device)
    _shape(q_codes, "q_codes", (B, Hq, CODE_BYTES), q.device)
    if mask is not None:
        if mask.dim() != 2:
            raise ValueError("mask must be [batch][words]")
        _shape(mask, "mask", (B, mask.shape[1]), q.device)
    d = dims(B, Hq, Hkv, cap, hd)
    tail = (_ptr(q, "q", 2), _ptr(k, "k", 2), _ptr(v, "v", 2), _ptr(codes, "codes", 1), _ptr(kv_len, "kv_len", 4),
            int(budget), float(scale), _ptr(out, "out", 4), _ptr(sel_idx, "sel_idx", 4, optional=True),
            _ptr(dist, "dist", 2, optional=True), _ptr(q_codes, "q_codes", 1, optional=True),
            _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream(stream))
    forced = not (sink is None and recent is None and mask is None)
    if not forced and pages is None:
        fn = _lib.adamas_append_decode_step if append else _lib.adamas_decode_step
        _check(fn(ctypes.byref(d), *tail), "adamas_append_decode_step" if append else "adamas_decode_step")
        return
    f = None
    if forced:
        f = Forced(int(sink or 0), int(recent or 0), _ptr(mask, "mask", 4, optional=True),
                   0 if mask is None else int(mask.shape[1]))
    if pages is None:
        st = _lib.adamas_forced_decode_step(ctypes.byref(d), ctypes.byref(f), 1 if append else 0, *tail)
        _check(st, "adamas_forced_decode_step")
        return
    pc = pages.c(k.shape[0])
    st = _lib.adamas_paged_decode_step(ctypes.byref(d), ctypes.byref(pc), ctypes.byref(f) if f is not None else None,
                                       1 if append else 0, *tail)
    _check(st, "adamas_paged_decode_step")


NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_step_noalloc(q, k, v, codes, kv_len, budget, scale, out, sel_idx=None, dist=None, q_codes=None,
                        stream=None):
    """adamas_decode_step with the library's static scratch instead of a
    workspace (no device allocation by the call); concurrent calls on one GPU
    race.  Same arguments and results as decode_step without append/forced/pages."""
    B, Hq, Hkv, cap = _check_shapes(q, k, v, codes, kv_len, out, None)
    _shape(sel_idx, "sel_idx", (B, Hq, int(budget)), q.device)
    _shape(dist, "dist", (B, Hq, cap), q.device)
    _shape(q_codes, "q_codes", (B, Hq, CODE_BYTES), q.device)
    d = dims(B, Hq, Hkv, cap, q.shape[2])
    st = _lib.adamas_decode_step_noalloc(ctypes.byref(d), _ptr(q, "q", 2), _ptr(k, "k", 2), _ptr(v, "v", 2),
                                         _ptr(codes, "codes", 1), _ptr(kv_len, "kv_len", 4), int(budget),
                                         float(scale), _ptr(out, "out", 4),
                                         _ptr(sel_idx, "sel_idx", 4, optional=True),
                                         _ptr(dist, "dist", 2, optional=True),
                                         _ptr(q_codes, "q_codes", 1, optional=True), _stream(stream))
    _check(st, "adamas_decode_step_noalloc")


def dense_decode_attention(q, k, v, kv_len, scale, out, workspace, stream=None, pages=None):
    """Dense decode attention over every position < kv_len[b]; writes out [B][Hq][128] fp32
    (with `pages`: k and v are pools, see Pages)."""
    B, Hq, Hkv, cap = _check_shapes(q, k, v, None, kv_len, out, pages)
    d = dims(B, Hq, Hkv, cap, q.shape[2])
    tail = (_ptr(q, "q", 2), _ptr(k, "k", 2), _ptr(v, "v", 2), _ptr(kv_len, "kv_len", 4), float(scale),
            _ptr(out, "out", 4), _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream))
    if pages is None:
        _check(_lib.dense_decode_attention(ctypes.byref(d), *tail), "dense_decode_attention")
        return
    pc = pages.c(k.shape[0])
    _check(_lib.dense_paged_decode_attention(ctypes.byref(d), ctypes.byref(pc), *tail),
           "dense_paged_decode_attention")


def decode_launch_mode(mode):
    """Later decode steps on this thread: 0 = two kernels (default), 1 = one
    kernel where the shape allows it.  Results are the same either way."""
    _check(_lib.adamas_decode_launch_mode(int(mode)), "adamas_decode_launch_mode")


def last_launch_count():
    """Kernels launched by this thread's last decode step (1 or 2)."""
    return int(_lib.adamas_last_launch_count())


def profile_events(events):
    """Time later calls on this thread kernel by kernel: `events` is a list of raw
    hipEvent_t handles (ints); launch i is bracketed by events[2i], events[2i+1].
    Pass None or [] to switch timing off."""
    n = len(events) if events else 0
    arr = (ctypes.c_void_p * max(n, 1))(*(events or [None]))
    _check(_lib.adamas_profile_events(arr if n else None, n), "adamas_profile_events")


def raw_library():
    """The ctypes handle of libadamas.so (for callers that pass raw pointers)."""
    return _lib
