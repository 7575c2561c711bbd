"""ctypes front end of the C oracle (adamas_oracle.c).

TEST INFRASTRUCTURE: only tests/, the smoke check and the benchmark's CPU
baseline may import this package.  It takes and returns numpy arrays on the
host; bf16 tensors travel as their uint16 bit patterns.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_f32p = ctypes.POINTER(ctypes.c_float)


def lib():
    """Load liboracle.so, compiling it first if it is absent (or the library
    that ADAMAS_ORACLE_LIB names, e.g. the sanitizer build)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ADAMAS_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        i32 = ctypes.c_int32
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_fwht128.argtypes = [_f32p, _f32p]
        L.oracle_fwht128.restype = None
        L.oracle_bucketize128.argtypes = [_f32p, _u8p]
        L.oracle_bucketize128.restype = None
        L.oracle_pack128.argtypes = [_u8p, _u8p]
        L.oracle_pack128.restype = None
        L.oracle_unpack128.argtypes = [_u8p, _u8p]
        L.oracle_unpack128.restype = None
        L.oracle_encode_vector.argtypes = [_u16p, _u8p]
        L.oracle_encode_vector.restype = None
        L.oracle_distance.argtypes = [_u8p, _u8p]
        L.oracle_distance.restype = ctypes.c_int
        L.oracle_topk.argtypes = [_u16p, i32, i32, _i32p]
        L.oracle_topk.restype = i32
        L.oracle_attention_rows.argtypes = [_u16p, _u16p, _u16p, _i32p, i32, ctypes.c_double, _f32p]
        L.oracle_attention_rows.restype = None
        L.oracle_encode_keys.argtypes = [i32, i32, i32, _u16p, _i32p, _i32p, _u8p, i32]
        L.oracle_encode_keys.restype = ctypes.c_int
        L.oracle_decode_step.argtypes = [i32, i32, i32, i32, _u16p, _u16p, _u16p, _u8p, _i32p, i32,
                                         ctypes.c_float, _f32p, _i32p, _u16p, _u8p, i32]
        L.oracle_decode_step.restype = ctypes.c_int
        L.oracle_topk_forced.argtypes = [_u16p, _u8p, i32, i32, _i32p]
        L.oracle_topk_forced.restype = i32
        L.oracle_decode_step_forced.argtypes = [i32, i32, i32, i32, _u16p, _u16p, _u16p, _u8p, _i32p, i32,
                                                ctypes.c_float, i32, i32, _u32p, i32, _f32p, _i32p, _u16p,
                                                _u8p, i32]
        L.oracle_decode_step_forced.restype = ctypes.c_int
        L.oracle_dense_attention.argtypes = [i32, i32, i32, i32, _u16p, _u16p, _u16p, _i32p,
                                             ctypes.c_float, _f32p, i32]
        L.oracle_dense_attention.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a, ptype):
    if a is None:
        return ctypes.cast(None, ptype)
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ptype)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def bf16_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16 array) to float32."""
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def fwht128(x):
    x = _c(x, np.float32)
    assert x.shape == (128,)
    y = np.empty(128, np.float32)
    lib().oracle_fwht128(_ptr(x, _f32p), _ptr(y, _f32p))
    return y


def bucketize128(y):
    y = _c(y, np.float32)
    assert y.shape == (128,)
    c = np.empty(128, np.uint8)
    lib().oracle_bucketize128(_ptr(y, _f32p), _ptr(c, _u8p))
    return c


def pack128(codes):
    c = _c(codes, np.uint8)
    assert c.shape == (128,)
    out = np.empty(32, np.uint8)
    lib().oracle_pack128(_ptr(c, _u8p), _ptr(out, _u8p))
    return out


def unpack128(packed):
    p = _c(packed, np.uint8)
    assert p.shape == (32,)
    out = np.empty(128, np.uint8)
    lib().oracle_unpack128(_ptr(p, _u8p), _ptr(out, _u8p))
    return out


def encode_vector(x_bf16):
    x = _c(x_bf16, np.uint16)
    assert x.shape == (128,)
    out = np.empty(32, np.uint8)
    lib().oracle_encode_vector(_ptr(x, _u16p), _ptr(out, _u8p))
    return out


def distance(a32, b32):
    a = _c(a32, np.uint8)
    b = _c(b32, np.uint8)
    assert a.shape == (32,) and b.shape == (32,)
    return int(lib().oracle_distance(_ptr(a, _u8p), _ptr(b, _u8p)))


def topk(dist, budget):
    d = _c(dist, np.uint16)
    sel = np.empty(budget, np.int32)
    k_eff = lib().oracle_topk(_ptr(d, _u16p), int(d.shape[0]), int(budget), _ptr(sel, _i32p))
    return sel, int(k_eff)


def topk_forced(dist, forced, budget):
    """Top-k with forced positions.  forced: uint8 array like dist (2 = always
    kept, 1 = preferred, 0 = ordinary), or None."""
    d = _c(dist, np.uint16)
    f = None if forced is None else _c(forced, np.uint8)
    assert f is None or f.shape == d.shape
    sel = np.empty(budget, np.int32)
    k_eff = lib().oracle_topk_forced(_ptr(d, _u16p), _ptr(f, _u8p), int(d.shape[0]), int(budget),
                                     _ptr(sel, _i32p))
    return sel, int(k_eff)


def attention_rows(q, k_head, v_head, pos, scale):
    q = _c(q, np.uint16)
    kh = _c(k_head, np.uint16)
    vh = _c(v_head, np.uint16)
    p = _c(pos, np.int32)
    assert q.shape == (128,) and kh.shape[-1] == 128 and vh.shape == kh.shape
    assert p.size == 0 or (p.min() >= 0 and p.max() < kh.shape[0])  # (no rows: the zero vector)
    out = np.empty(128, np.float32)
    lib().oracle_attention_rows(_ptr(q, _u16p), _ptr(kh, _u16p), _ptr(vh, _u16p), _ptr(p, _i32p),
                                int(p.size), float(scale), _ptr(out, _f32p))
    return out


def encode_keys(k, end, start=None, codes=None, threads=1):
    """Encode positions [start[b], end[b]) of k (uint16 [B][Hkv][cap][128]).

    Returns the codes array (uint8 [B][Hkv][cap][32]); rows outside the ranges
    keep their previous contents (zeros for a fresh array).  threads > 1 encodes
    independent rows in parallel (same arithmetic per row).
    """
    k = _c(k, np.uint16)
    B, Hkv, cap, d = k.shape
    assert d == 128
    end = _c(end, np.int32)
    start = None if start is None else _c(start, np.int32)
    if codes is None:
        codes = np.zeros((B, Hkv, cap, 32), np.uint8)
    assert codes.shape == (B, Hkv, cap, 32) and codes.dtype == np.uint8 and codes.flags["C_CONTIGUOUS"]
    rc = lib().oracle_encode_keys(B, Hkv, cap, _ptr(k, _u16p), _ptr(start, _i32p), _ptr(end, _i32p),
                                  _ptr(codes, _u8p), int(threads))
    if rc != 0:
        raise ValueError("oracle_encode_keys: invalid arguments")
    return codes


def decode_step(q, k, v, codes, kv_len, budget, scale, threads=1, want_dist=True, sink=0, recent=0,
                mask=None):
    """Full decode step on the host.  Returns (out, sel_idx, dist, q_codes).

    dist rows are zero at positions >= kv_len[b] (never written by the oracle).
    sink / recent / mask (uint32 [B][words], bit p % 32 of word p / 32) name
    the forced positions; all three absent gives the plain top-k.
    """
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    codes = _c(codes, np.uint8)
    kv_len = _c(kv_len, np.int32)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    assert d == 128 and v.shape == k.shape and codes.shape == (B, Hkv, cap, 32)
    out = np.empty((B, Hq, 128), np.float32)
    sel = np.empty((B, Hq, budget), np.int32)
    dist = np.zeros((B, Hq, cap), np.uint16) if want_dist else None
    qc = np.empty((B, Hq, 32), np.uint8)
    if sink == 0 and recent == 0 and mask is None:
        rc = lib().oracle_decode_step(B, Hq, Hkv, cap, _ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p),
                                      _ptr(codes, _u8p), _ptr(kv_len, _i32p), int(budget), float(scale),
                                      _ptr(out, _f32p), _ptr(sel, _i32p), _ptr(dist, _u16p), _ptr(qc, _u8p),
                                      int(threads))
    else:
        m = None if mask is None else _c(mask, np.uint32)
        assert m is None or (m.ndim == 2 and m.shape[0] == B)
        rc = lib().oracle_decode_step_forced(B, Hq, Hkv, cap, _ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p),
                                             _ptr(codes, _u8p), _ptr(kv_len, _i32p), int(budget), float(scale),
                                             int(sink), int(recent), _ptr(m, _u32p),
                                             0 if m is None else int(m.shape[1]), _ptr(out, _f32p),
                                             _ptr(sel, _i32p), _ptr(dist, _u16p), _ptr(qc, _u8p), int(threads))
    if rc != 0:
        raise ValueError("oracle_decode_step: invalid arguments")
    return out, sel, dist, qc


def dense_attention(q, k, v, kv_len, scale, threads=1):
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    kv_len = _c(kv_len, np.int32)
    B, Hq, d = q.shape
    _, Hkv, cap, _ = k.shape
    out = np.empty((B, Hq, 128), np.float32)
    rc = lib().oracle_dense_attention(B, Hq, Hkv, cap, _ptr(q, _u16p), _ptr(k, _u16p), _ptr(v, _u16p),
                                      _ptr(kv_len, _i32p), float(scale), _ptr(out, _f32p), int(threads))
    if rc != 0:
        raise ValueError("oracle_dense_attention: invalid arguments")
    return out
