"""CPU oracle for the A16W4 MoE layer -- TEST INFRASTRUCTURE ONLY.

A ctypes front end over libmoe_oracle.so (plain C, float64 arithmetic except
the float32 integer decisions of the requantization). Only the tests, the
package smoke check and the benchmark's CPU-baseline leg may import this
package; the product path never does. It shares no code with the GPU path.

Functions that have no independent pin say "parity unpinned" here and in the
C source; at present every exported function is pinned by a test in
tests/test_oracle_*.py.
"""
import ctypes
import os

import numpy as np

from . import build as _build

FMT_MXFP4 = 0
FMT_INT4G32 = 1

_lib = None


def lib():
    """The oracle library: oracle/libmoe_oracle.so (built on first use), or
    the file MOE_ORACLE_LIB names (the sanitizer build of the same source)."""
    global _lib
    if _lib is None:
        path = os.environ.get("MOE_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i = ctypes.c_int
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [i]
        L.oracle_e8m0_value.restype = ctypes.c_double
        L.oracle_e8m0_value.argtypes = [i]
        L.oracle_nibble.restype = i
        L.oracle_nibble.argtypes = [p, i]
        L.oracle_bf16_value.restype = ctypes.c_double
        L.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_bf16_rne.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16_rne.argtypes = [ctypes.c_float]
        L.oracle_dequant.restype = None
        L.oracle_dequant.argtypes = [p, p, i, i, i, p]
        L.oracle_route_topk.restype = None
        L.oracle_route_topk.argtypes = [p, i, i, i, i, p, p]
        L.oracle_align_capacity.restype = ctypes.c_int64
        L.oracle_align_capacity.argtypes = [i, i, i, i]
        L.oracle_align_sort.restype = None
        L.oracle_align_sort.argtypes = [p, i, i, i, i, p, p, p, p]
        L.oracle_moe_forward.restype = None
        L.oracle_moe_forward.argtypes = [p, p, p, p, p, i, p, p, i, i, i, i, i, p, i, p]
        L.oracle_moe_forward_ex.restype = None
        L.oracle_moe_forward_ex.argtypes = [p, p, p, p, p, p, p, ctypes.c_double, i, p, p, i, i, i, i, i,
                                            p, i, p]
        L.oracle_requant_int4g32.restype = None
        L.oracle_requant_int4g32.argtypes = [p, p, i, i, i, i, i, p, p]
        L.oracle_num_threads.restype = i
        L.oracle_set_num_threads.argtypes = [i]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def e8m0_value(byte: int) -> float:
    return lib().oracle_e8m0_value(int(byte))


def nibble(row_bytes, k: int) -> int:
    row = _c(row_bytes, np.uint8)
    return lib().oracle_nibble(_ptr(row), int(k))


def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_value(int(bits))


def f32_to_bf16(v: float) -> int:
    return lib().oracle_f32_to_bf16_rne(float(v))


def dequant(w, scale, fmt: int, K: int):
    """Dequantize a packed [rows, K/2] weight with its [rows, K/32] scales."""
    w = _c(w, np.uint8)
    rows = w.size // (K // 2)
    scale = _c(scale, np.uint8 if fmt == FMT_MXFP4 else np.uint16)
    out = np.empty((rows, K), dtype=np.float64)
    lib().oracle_dequant(_ptr(w), _ptr(scale), int(fmt), rows, int(K), _ptr(out))
    return out


def route_topk(logits, topk: int, renormalize: bool = True):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, topk), dtype=np.int32)
    w = np.empty((T, topk), dtype=np.float32)
    lib().oracle_route_topk(_ptr(logits), T, E, int(topk), int(bool(renormalize)),
                            _ptr(ids), _ptr(w))
    return ids, w


def align_capacity(T: int, topk: int, E: int, bm: int) -> int:
    return int(lib().oracle_align_capacity(T, topk, E, bm))


def align_sort(ids, E: int, bm: int):
    ids = _c(ids, np.int32)
    T, topk = ids.shape
    cap = align_capacity(T, topk, E, bm)
    sorted_ids = np.empty(cap, dtype=np.int32)
    block_expert = np.empty(cap // bm, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    npp = np.empty(1, dtype=np.int32)
    lib().oracle_align_sort(_ptr(ids), T, topk, int(E), int(bm), _ptr(sorted_ids),
                            _ptr(block_expert), _ptr(offsets), _ptr(npp))
    return sorted_ids, block_expert, offsets, int(npp[0])


def moe_forward(x_bf16, w13, w13_scale, w2, w2_scale, fmt, ids, weights,
                I: int, tokens=None, w13_bias=None, w2_bias=None, swiglu_limit=0.0):
    """out[len(tokens) or T, H] float64. x_bf16 holds bf16 bit patterns.
    w13_bias [E, 2I] / w2_bias [E, H]: optional bf16 bit patterns;
    swiglu_limit > 0 clamps gate and up to [-limit, limit] before SwiGLU."""
    x = _c(x_bf16, np.uint16)
    T, H = x.shape
    w13 = _c(w13, np.uint8)
    w2 = _c(w2, np.uint8)
    sdt = np.uint8 if fmt == FMT_MXFP4 else np.uint16
    w13s = _c(w13_scale, sdt)
    w2s = _c(w2_scale, sdt)
    E = w13.shape[0]
    assert w13.shape == (E, 2 * I, H // 2) and w2.shape == (E, H, I // 2)
    assert w13s.shape == (E, 2 * I, H // 32) and w2s.shape == (E, H, I // 32)
    ids = _c(ids, np.int32)
    weights = _c(weights, np.float32)
    topk = ids.shape[1]
    if tokens is None:
        tok = None
        n = T
    else:
        tok = _c(tokens, np.int32)
        n = tok.size
        assert np.all((tok >= 0) & (tok < T))
    b13 = None if w13_bias is None else _c(w13_bias, np.uint16)
    b2 = None if w2_bias is None else _c(w2_bias, np.uint16)
    assert b13 is None or b13.shape == (E, 2 * I)
    assert b2 is None or b2.shape == (E, H)
    out = np.empty((n, H), dtype=np.float64)
    lib().oracle_moe_forward_ex(_ptr(x), _ptr(w13), _ptr(w13s), _ptr(b13), _ptr(w2), _ptr(w2s),
                                _ptr(b2), float(swiglu_limit), int(fmt), _ptr(ids), _ptr(weights),
                                T, H, int(I), E, topk, _ptr(tok), n, _ptr(out))
    return out


def requant_int4g32(w, scale_e8m0, lo: int = 0, hi: int = None, out=None):
    """Requantize experts [lo, hi) of w [E, N, K/2] (+ e8m0 [E, N, K/32]).

    Returns (codes uint8 [E, N, K/2], scales uint16 bf16 bits [E, N, K/32]);
    pass out=(codes, scales) to fill preallocated arrays chunk by chunk."""
    w = _c(w, np.uint8)
    s = _c(scale_e8m0, np.uint8)
    E, N, Kh = w.shape
    K = Kh * 2
    hi = E if hi is None else hi
    if out is None:
        codes = np.zeros((E, N, K // 2), dtype=np.uint8)
        scales = np.zeros((E, N, K // 32), dtype=np.uint16)
    else:
        codes, scales = out
    lib().oracle_requant_int4g32(_ptr(w), _ptr(s), E, N, K, int(lo), int(hi),
                                 _ptr(codes), _ptr(scales))
    return codes, scales


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(int(n))
