"""Binding of libllama_glue.so (include/llama_glue.h): the fused elementwise
kernels of the Llama-shaped decoder stack.  Argument marshalling only; the
library must be built (sparse_attention_long_fwht_amd/build.py)."""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libllama_glue.so")
if not os.path.exists(LIB_PATH):
    raise ImportError("libllama_glue.so is not built at %s; build it with sparse_attention_long_fwht_amd/build.py"
                      % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
_lib.llama_add_rmsnorm.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _f32, _vp]
_lib.llama_add_rmsnorm.restype = _i32
_lib.llama_rope_append.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]
_lib.llama_rope_append.restype = _i32
_lib.llama_silu_mul.argtypes = [_vp, _vp, _i32, _i32, _vp]
_lib.llama_silu_mul.restype = _i32

EXPORTED_SYMBOLS = ("llama_add_rmsnorm", "llama_rope_append", "llama_silu_mul")


def _p(t):
    if t is None:
        return None
    if not (t.is_cuda and t.is_contiguous()):
        raise ValueError("device tensors, contiguous")
    return t.data_ptr()


def _shape(t, name, shape):
    """The kernels index by the dims they are given: a buffer of another shape
    is rejected rather than read or written past its end."""
    if t is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError("%s must have shape %s, got %s" % (name, [int(x) for x in shape], list(t.shape)))


def _s():
    return torch.cuda.current_stream().cuda_stream


def _check(rc, name):
    if rc != 0:
        raise RuntimeError("%s failed (status %d)" % (name, rc))


def add_rmsnorm(x, delta, x_out, w, h, eps):
    """x_out = x + delta (delta may be None; x_out may be x or None); h = rmsnorm(x_out) * w."""
    rows, hidden = x.shape
    _shape(delta, "delta", x.shape)
    _shape(x_out, "x_out", x.shape)
    _shape(w, "w", (hidden,))
    _shape(h, "h", x.shape)
    _check(_lib.llama_add_rmsnorm(_p(x), _p(delta), _p(x_out), _p(w), _p(h), rows, hidden, float(eps), _s()),
           "llama_add_rmsnorm")


def rope_append(qkv, pos, inv_freq, q_out, k_cache, v_cache):
    """Rotary q/k of the new token at pos[b], q to q_out, k/v rows into the caches."""
    B, Hkv, cap, hd = k_cache.shape
    Hq = q_out.shape[1]
    _shape(k_cache, "k_cache", (B, Hkv, cap, 128))
    _shape(v_cache, "v_cache", k_cache.shape)
    _shape(q_out, "q_out", (B, Hq, 128))
    _shape(qkv, "qkv", (B, (Hq + 2 * Hkv) * 128))
    _shape(pos, "pos", (B,))
    _shape(inv_freq, "inv_freq", (64,))
    _check(_lib.llama_rope_append(_p(qkv), _p(pos), _p(inv_freq), _p(q_out), _p(k_cache), _p(v_cache), B,
                                  Hq, Hkv, cap, _s()), "llama_rope_append")


def silu_mul(gu, out):
    rows, ffn = out.shape
    _shape(gu, "gu", (rows, 2 * ffn))
    _check(_lib.llama_silu_mul(_p(gu), _p(out), rows, ffn, _s()), "llama_silu_mul")


def raw_library():
    return _lib
