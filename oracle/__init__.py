"""fp64 CPU oracle for decode attention: test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library
(``decode_attention_fdec_amd``) and imports nothing from it; the two meet only
through the seeded input generators in ``synth``.

The arithmetic lives in ``oracle.c`` (plain C, double precision, one loop per
definition); this module only marshals numpy arrays into it. What each
function follows on the pages is stated in the header of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at another build of oracle.c (a planted-mistake
# copy, built on the CPU) to check that the pins catch it.
_LIB_OVERRIDE = os.environ.get("ORACLE_LIB_OVERRIDE")

F16, BF16, FP8 = 0, 1, 2  # FP8: float8 e4m3fn caches (queries stay 16-bit)


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


class _KV(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("Hq", ctypes.c_int), ("Hkv", ctypes.c_int), ("D", ctypes.c_int),
        ("dtype", ctypes.c_int),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("page_size", ctypes.c_int), ("capacity", ctypes.c_int),
        ("s_outer", ctypes.c_int64), ("s_token", ctypes.c_int64), ("s_head", ctypes.c_int64),
        ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int),
        ("prefix_pages", ctypes.c_void_p), ("prefix_len", ctypes.c_int),
        ("k_descale", ctypes.c_void_p), ("v_descale", ctypes.c_void_p),
        ("batch_idx", ctypes.c_void_p), ("leftpad", ctypes.c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=True)
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.oracle_decode.argtypes = [ctypes.POINTER(_KV), P, P, ctypes.c_double, P, P, ctypes.c_int]
        lib.oracle_decode_multi.argtypes = [ctypes.POINTER(_KV), P, P, ctypes.c_int, ctypes.c_double, P, P,
                                            ctypes.c_int]
        lib.oracle_partials.argtypes = [ctypes.POINTER(_KV), P, P, ctypes.c_double, ctypes.c_int,
                                        P, P, P, P, ctypes.c_int]
        lib.oracle_merge.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_int, P, P]
        lib.oracle_rope_neox.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_double]
        lib.oracle_append.argtypes = [ctypes.POINTER(_KV), P, P, P, P, P, P, ctypes.c_int,
                                      ctypes.c_double, P]
        lib.oracle_decode_elems.argtypes = [P, ctypes.c_int, ctypes.c_int64, P]
        lib.oracle_decode_f8.argtypes = [P, ctypes.c_int64, P]
        lib.oracle_encode_elems.argtypes = [P, ctypes.c_int, ctypes.c_int64, P]
        lib.oracle_encode_f8.argtypes = [P, ctypes.c_int64, P]
        lib.oracle_now.restype = ctypes.c_double
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _bits(a) -> np.ndarray:
    """Raw bit patterns (C order): uint16 for fp16/bf16, uint8 for float8 e4m3fn."""
    if isinstance(a, np.ndarray):
        assert a.dtype in (np.uint16, np.uint8)
        return np.ascontiguousarray(a)
    import torch  # only for unpacking torch tensors handed in by tests

    a = a.detach().cpu().contiguous()
    if a.dtype == torch.float8_e4m3fn:
        return np.ascontiguousarray(a.view(torch.uint8).numpy())
    assert a.dtype in (torch.float16, torch.bfloat16)
    return np.ascontiguousarray(a.view(torch.int16).numpy().view(np.uint16))


def dtype_code(a) -> int:
    import torch

    if a.dtype == torch.float8_e4m3fn:
        return FP8
    return F16 if a.dtype == torch.float16 else BF16


def _i32(a) -> np.ndarray:
    if a is None:
        return None
    if not isinstance(a, np.ndarray):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data


def to_f64(bits, dtype: int) -> np.ndarray:
    """Exact fp16/bf16/float8 -> double conversion by the oracle's own field decoders."""
    b = _bits(bits)
    out = np.empty(b.shape, dtype=np.float64)
    if dtype == FP8:
        assert b.dtype == np.uint8
        _load().oracle_decode_f8(_ptr(b), b.size, _ptr(out))
    else:
        assert b.dtype == np.uint16
        _load().oracle_decode_elems(_ptr(b), dtype, b.size, _ptr(out))
    return out


def from_f64(x: np.ndarray, dtype: int) -> np.ndarray:
    """Round doubles once (nearest, ties to even) onto fp16/bf16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_encode_elems(_ptr(x), dtype, x.size, _ptr(out))
    return out


def f32_to_f8(x) -> np.ndarray:
    """Nearest float8 e4m3fn codes (ties to even, saturating at +-448) of binary32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().oracle_encode_f8(_ptr(x), x.size, _ptr(out))
    return out


class KV:
    """One KV cache as the oracle reads it (raw bits + geometry)."""

    def __init__(self, k, v, dtype: int, Hq: int, B: int, page_size: int = 0,
                 page_table=None, prefix_pages=None, prefix_len: int = 0, k_descale=None, v_descale=None,
                 batch_idx=None, leftpad=None):
        self.k = _bits(k)
        self.v = _bits(v)
        assert self.k.shape == self.v.shape and self.k.ndim == 4
        self.dtype = dtype
        self.B, self.Hq = B, Hq
        self.page_size = page_size
        _, n1, self.Hkv, self.D = self.k.shape
        self.capacity = n1 if page_size == 0 else 0
        # plain C-order strides of [outer, token, head, D]
        self.strides = (n1 * self.Hkv * self.D, self.Hkv * self.D, self.D)
        self.page_table = _i32(page_table)
        self.prefix_pages = _i32(prefix_pages)
        self.prefix_len = prefix_len
        self.k_descale = _f64(k_descale, (B, self.Hkv))
        self.v_descale = _f64(v_descale, (B, self.Hkv))
        self.batch_idx = _i32(batch_idx)  # contiguous caches: cache row of request b
        self.leftpad = _i32(leftpad)      # first valid row of request b
        for a in (self.batch_idx, self.leftpad):
            assert a is None or a.shape == (B,)

    def _struct(self) -> _KV:
        s = _KV()
        s.B, s.Hq, s.Hkv, s.D = self.B, self.Hq, self.Hkv, self.D
        s.dtype = self.dtype
        s.k, s.v = _ptr(self.k), _ptr(self.v)
        s.page_size, s.capacity = self.page_size, self.capacity
        s.s_outer, s.s_token, s.s_head = self.strides
        s.page_table = _ptr(self.page_table)
        s.max_pages = 0 if self.page_table is None else self.page_table.shape[1]
        s.prefix_pages = _ptr(self.prefix_pages)
        s.prefix_len = self.prefix_len
        s.k_descale = _ptr(self.k_descale)
        s.v_descale = _ptr(self.v_descale)
        s.batch_idx = _ptr(self.batch_idx)
        s.leftpad = _ptr(self.leftpad)
        return s


def _f64(a, shape):
    if a is None:
        return None
    if not isinstance(a, np.ndarray):
        a = a.detach().cpu().double().numpy()
    a = np.ascontiguousarray(a, dtype=np.float64)
    assert a.shape == shape
    return a


def _q64(q, dtype):
    """Queries in double: a float64 array as is, a tensor by its own dtype, bits by `dtype`."""
    if isinstance(q, np.ndarray):
        if q.dtype == np.float64:
            return np.ascontiguousarray(q)
        return to_f64(q, dtype)
    return to_f64(q, dtype_code(q))


def decode(kv: KV, q, lens, scale: float, nthreads: int = 0):
    """Plain attention for every (b, h): returns out [B,Hq,D] and lse [B,Hq] in float64."""
    q64 = _q64(q, kv.dtype)
    lens = _i32(lens)
    assert q64.shape == (kv.B, kv.Hq, kv.D) and lens.shape == (kv.B,)
    out = np.empty((kv.B, kv.Hq, kv.D), dtype=np.float64)
    lse = np.empty((kv.B, kv.Hq), dtype=np.float64)
    s = kv._struct()
    _load().oracle_decode(ctypes.byref(s), _ptr(q64), _ptr(lens), float(scale), _ptr(out),
                          _ptr(lse), int(nthreads))
    return out, lse


def decode_multi(kv: KV, q, lens, scale: float, nthreads: int = 0):
    """q_len query tokens per request, causal: q [B, q_len, Hq, D] -> out [B, q_len, Hq, D], lse [B, Hq, q_len]."""
    if isinstance(q, np.ndarray) and q.dtype == np.float64:
        q64 = np.ascontiguousarray(q)
    else:
        q64 = to_f64(q, dtype_code(q) if not isinstance(q, np.ndarray) else kv.dtype)
    lens = _i32(lens)
    B, q_len, Hq, D = q64.shape
    assert (B, Hq, D) == (kv.B, kv.Hq, kv.D) and lens.shape == (kv.B,)
    out = np.empty((B, q_len, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq, q_len), dtype=np.float64)
    s = kv._struct()
    _load().oracle_decode_multi(ctypes.byref(s), _ptr(q64), _ptr(lens), int(q_len), float(scale), _ptr(out),
                                _ptr(lse), int(nthreads))
    return out, lse


def partials(kv: KV, q, lens, scale: float, bounds, nthreads: int = 0):
    """Map-stage states for explicit boundaries bounds [B, S+1]: (po, pm, pd) in float64."""
    q64 = _q64(q, kv.dtype)
    lens = _i32(lens)
    bounds = _i32(bounds)
    S = bounds.shape[1] - 1
    po = np.empty((kv.B, kv.Hq, S, kv.D), dtype=np.float64)
    pm = np.empty((kv.B, kv.Hq, S), dtype=np.float64)
    pd = np.empty((kv.B, kv.Hq, S), dtype=np.float64)
    s = kv._struct()
    _load().oracle_partials(ctypes.byref(s), _ptr(q64), _ptr(lens), float(scale), S,
                            _ptr(bounds), _ptr(po), _ptr(pm), _ptr(pd), int(nthreads))
    return po, pm, pd


def merge(po, pm, pd):
    """Reduce-stage merge of states [B,Hq,S,D] / [B,Hq,S] into (out, lse) float64."""
    po = np.ascontiguousarray(po, dtype=np.float64)
    pm = np.ascontiguousarray(pm, dtype=np.float64)
    pd = np.ascontiguousarray(pd, dtype=np.float64)
    B, Hq, S, D = po.shape
    out = np.empty((B, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    _load().oracle_merge(_ptr(po), _ptr(pm), _ptr(pd), B, Hq, S, D, _ptr(out), _ptr(lse))
    return out, lse


def rope_neox(x, pos: int, rotary_dim: int, base: float = 10000.0) -> np.ndarray:
    """NeoX rotary of the last axis of x (any leading shape), in double."""
    x = np.array(x, dtype=np.float64, copy=True, order="C")
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        _load().oracle_rope_neox(_ptr(row), D, rotary_dim, int(pos), float(base))
        flat[r] = row
    return flat.reshape(x.shape)


def append(kv: KV, k_new, v_new, q, cache_seqlens, rotary_dim: int, base: float = 10000.0):
    """KV append (+ NeoX rotary when rotary_dim > 0) on copies of kv's caches.

    Returns (k_cache_bits, v_cache_bits, q_rotated_f64, kv_after) where kv_after
    reads the updated caches.
    """
    kc = kv.k.copy()
    vc = kv.v.copy()
    kn, vn = _bits(k_new), _bits(v_new)
    q64 = _q64(q, kv.dtype)
    cs = _i32(cache_seqlens)
    q_out = np.empty_like(q64)
    after = KV.__new__(KV)
    after.__dict__.update(kv.__dict__)
    after.k, after.v = kc, vc
    s = after._struct()
    _load().oracle_append(ctypes.byref(s), _ptr(kc), _ptr(vc), _ptr(kn), _ptr(vn), _ptr(q64),
                          _ptr(cs), int(rotary_dim), float(base), _ptr(q_out))
    return kc, vc, q_out, after


def now() -> float:
    return _load().oracle_now()


def max_threads() -> int:
    return _load().oracle_max_threads()
