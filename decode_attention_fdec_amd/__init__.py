"""Python binding for libfdec (split-KV decode attention on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libfdec.so``. torch supplies device memory and the current
stream. The names follow the C ABI in ``include/fdec.h``:

    plan, plan_rules, split_chunk, workspace_size, Workspace,
    decode, decode_partials, merge_states, cascade_decode, cascade_workspace_size

If ``libfdec.so`` has not been built, importing works but every call raises
``FdecError``; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfdec.so")

FDEC_OK, FDEC_ERR_INVALID_ARG, FDEC_ERR_UNSUPPORTED, FDEC_ERR_WORKSPACE, FDEC_ERR_HIP = range(5)
FDEC_F16, FDEC_BF16, FDEC_FP8_E4M3 = 0, 1, 2
MAX_SPLITS = 256


class FdecError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[{status}] {msg}")
        self.status = status


class FdecKV(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("dtype", ctypes.c_int), ("num_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int),
        ("page_size", ctypes.c_int), ("capacity", ctypes.c_int),
        ("s_outer", ctypes.c_int64), ("s_token", ctypes.c_int64), ("s_head", ctypes.c_int64),
        ("page_table", ctypes.c_void_p), ("max_pages_per_seq", ctypes.c_int),
        ("k_descale", ctypes.c_void_p), ("v_descale", ctypes.c_void_p),
        ("cache_batch_idx", ctypes.c_void_p), ("cache_leftpad", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int),
    ]


class FdecAppend(ctypes.Structure):
    _fields_ = [
        ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
        ("rope_cos", ctypes.c_void_p), ("rope_sin", ctypes.c_void_p),
        ("rotary_dim", ctypes.c_int), ("rope_max_pos", ctypes.c_int),
    ]


_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libfdec.so (after torch, so it binds to torch's HIP runtime)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise FdecError(FDEC_ERR_HIP, f"{p} is not built; run __graft_entry__.build() "
                        "or python -m decode_attention_fdec_amd.build")
    lib = ctypes.CDLL(p)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fdec_status_string.restype = ctypes.c_char_p
    lib.fdec_status_string.argtypes = [I]
    lib.fdec_last_error.restype = ctypes.c_char_p
    lib.fdec_last_error.argtypes = []
    lib.fdec_plan.argtypes = [I, I, I, P, I, I, I, ctypes.POINTER(I)]
    lib.fdec_plan_kv.argtypes = [I, I, I, P, I, I, I, I, ctypes.POINTER(I)]
    lib.fdec_plan_rules.argtypes = [I, I, I, I, ctypes.POINTER(I)]
    lib.fdec_split_chunk.restype = ctypes.c_int64
    lib.fdec_split_chunk.argtypes = [I, I]
    lib.fdec_workspace_size.restype = Z
    lib.fdec_workspace_size.argtypes = [I, I, I, I, I]
    lib.fdec_workspace_init.argtypes = [P, Z, P]
    lib.fdec_decode.argtypes = [P, I, I, ctypes.POINTER(FdecKV), P, I, F, ctypes.POINTER(FdecAppend), I,
                                P, P, P, Z, P]
    lib.fdec_decode_noalloc.argtypes = [P, I, I, ctypes.POINTER(FdecKV), P, I, F, ctypes.POINTER(FdecAppend), I,
                                        P, P, P]
    lib.fdec_decode_partials.argtypes = [P, I, I, ctypes.POINTER(FdecKV), P, I, F,
                                         ctypes.POINTER(FdecAppend), P, P, P, P]
    lib.fdec_merge_states.argtypes = [P, P, P, I, I, I, I, P, P, P]
    lib.fdec_cascade_decode.argtypes = [P, I, I, ctypes.POINTER(FdecKV), P, I, P, I, I, F, P, P, P, Z, P]
    lib.fdec_probe_read.argtypes = [P, Z, P, P]
    lib.fdec_probe_copy.argtypes = [P, P, Z, P]
    lib.fdec_trace_start.argtypes = [I]
    lib.fdec_trace_stop.argtypes = [P, P, I, ctypes.POINTER(I)]
    lib.fdec_probe_stream.argtypes = [P, Z, P, I, I, P]
    lib.fdec_cascade_plan.argtypes = [I, I, I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.fdec_cascade_plan_kv.argtypes = [I, I, I, I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.fdec_cascade_workspace_size.restype = Z
    lib.fdec_cascade_workspace_size.argtypes = [I, I, I, I, I, I]
    lib.fdec_decode_balanced.argtypes = [P, I, I, ctypes.POINTER(FdecKV), P, I, F, P, P, P, Z, P]
    lib.fdec_decode_multi.argtypes = [P, I, I, I, ctypes.POINTER(FdecKV), P, I, F, P, P, P, Z, P]
    lib.fdec_decode_multi_balanced.argtypes = [P, I, I, I, ctypes.POINTER(FdecKV), P, I, F, P, P, P, Z, P]
    lib.fdec_balanced_workspace_size.restype = Z
    lib.fdec_balanced_workspace_size.argtypes = [I, I, I, I, I]
    lib.fdec_check_inputs.argtypes = [I, ctypes.POINTER(FdecKV), P, ctypes.POINTER(FdecAppend), P, I,
                                      ctypes.POINTER(I), ctypes.POINTER(I), P]
    lib.fdec_set_debug.restype = None
    lib.fdec_set_debug.argtypes = [I]
    lib.fdec_debug_enabled.argtypes = []
    if path is None:
        _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != FDEC_OK:
        lib = load_library()
        raise FdecError(rc, f"{lib.fdec_status_string(rc).decode()}: {lib.fdec_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float16:
        return FDEC_F16
    if dt == torch.bfloat16:
        return FDEC_BF16
    if dt == torch.float8_e4m3fn:
        return FDEC_FP8_E4M3
    raise FdecError(FDEC_ERR_UNSUPPORTED, f"dtype {dt} not built (float16, bfloat16, float8_e4m3fn)")


def _check_q(q: torch.Tensor, k: torch.Tensor) -> None:
    """q has the cache's dtype (bf16 for a float8 cache) and is contiguous."""
    want = torch.bfloat16 if k.dtype == torch.float8_e4m3fn else k.dtype
    if q.dtype != want or not q.is_contiguous():
        raise FdecError(FDEC_ERR_INVALID_ARG, f"q must be contiguous {want} for a {k.dtype} cache")


def make_kv(k: torch.Tensor, v: torch.Tensor, page_table: Optional[torch.Tensor] = None,
            k_descale: Optional[torch.Tensor] = None, v_descale: Optional[torch.Tensor] = None,
            cache_batch_idx: Optional[torch.Tensor] = None,
            cache_leftpad: Optional[torch.Tensor] = None) -> FdecKV:
    """Describe a cache: contiguous [rows, cap, Hkv, D] or paged [P, page_size, Hkv, D] (+ page_table).

    Float8 caches take k_descale / v_descale: contiguous [B, Hkv] float32 device tensors (or None = 1).
    cache_batch_idx (contiguous caches) / cache_leftpad: contiguous [B] int32 device tensors or None.
    """
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype or k.dim() != 4:
        raise FdecError(FDEC_ERR_INVALID_ARG, "k and v must be 4-D with equal shapes, strides and dtypes")
    if k.stride(3) != 1:
        raise FdecError(FDEC_ERR_INVALID_ARG, "the head_dim axis of k/v must be contiguous")
    kv = FdecKV()
    kv.k, kv.v = k.data_ptr(), v.data_ptr()
    kv.dtype = _dtype_code(k.dtype)
    kv.num_kv_heads, kv.head_dim = k.shape[2], k.shape[3]
    kv.s_outer, kv.s_token, kv.s_head = k.stride(0), k.stride(1), k.stride(2)
    kv.num_blocks = k.shape[0]  # pages of a pool / rows of a contiguous cache
    if page_table is None:
        kv.page_size, kv.capacity = 0, k.shape[1]
        kv.page_table, kv.max_pages_per_seq = None, 0
    else:
        if page_table.dtype != torch.int32 or not page_table.is_contiguous() or page_table.dim() != 2:
            raise FdecError(FDEC_ERR_INVALID_ARG, "page_table must be a contiguous 2-D int32 tensor")
        kv.page_size = k.shape[1]
        kv.max_pages_per_seq = page_table.shape[1]
        kv.capacity = kv.page_size * kv.max_pages_per_seq
        kv.page_table = page_table.data_ptr()
    for name, d in (("k_descale", k_descale), ("v_descale", v_descale)):
        if d is not None:
            if d.dtype != torch.float32 or not d.is_contiguous():
                raise FdecError(FDEC_ERR_INVALID_ARG, f"{name} must be a contiguous float32 tensor")
            setattr(kv, name, d.data_ptr())
    for name, d in (("cache_batch_idx", cache_batch_idx), ("cache_leftpad", cache_leftpad)):
        if d is not None:
            if d.dtype != torch.int32 or not d.is_contiguous() or d.dim() != 1:
                raise FdecError(FDEC_ERR_INVALID_ARG, f"{name} must be a contiguous 1-D int32 tensor")
            setattr(kv, name, d.data_ptr())
    return kv


def make_append(k_new: torch.Tensor, v_new: torch.Tensor, rope_cos: Optional[torch.Tensor] = None,
                rope_sin: Optional[torch.Tensor] = None, rotary_dim: int = 0) -> FdecAppend:
    a = FdecAppend()
    a.k_new, a.v_new = k_new.data_ptr(), v_new.data_ptr()
    a.rotary_dim = rotary_dim
    if rotary_dim > 0:
        a.rope_cos, a.rope_sin = rope_cos.data_ptr(), rope_sin.data_ptr()
        a.rope_max_pos = rope_cos.shape[0]
    return a


def plan(B: int, Hq: int, Hkv: int, seq_lens_host: Optional[Sequence[int]], capacity: int,
         page_size: int = 0, cu_count: int = 256, kv_dtype=None) -> int:
    """fdec_plan, or fdec_plan_kv when kv_dtype (a torch dtype or an fdec_dtype code) is given."""
    lib = load_library()
    out = ctypes.c_int(0)
    arr = None
    if seq_lens_host is not None:
        vals = [int(x) for x in seq_lens_host]
        arr = (ctypes.c_int32 * len(vals))(*vals)
    lens = ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None
    if kv_dtype is None:
        _check(lib.fdec_plan(B, Hq, Hkv, lens, capacity, page_size, cu_count, ctypes.byref(out)))
    else:
        code = kv_dtype if isinstance(kv_dtype, int) else _dtype_code(kv_dtype)
        _check(lib.fdec_plan_kv(B, Hq, Hkv, lens, capacity, page_size, code, cu_count, ctypes.byref(out)))
    return out.value


def plan_rules(B: int, Hkv: int, sm_count: int, max_splits: int = 128) -> int:
    out = ctypes.c_int(0)
    _check(load_library().fdec_plan_rules(B, Hkv, sm_count, max_splits, ctypes.byref(out)))
    return out.value


def split_chunk(capacity: int, num_splits: int) -> int:
    return int(load_library().fdec_split_chunk(capacity, num_splits))


def workspace_size(B: int, Hq: int, Hkv: int, head_dim: int, num_splits: int) -> int:
    return int(load_library().fdec_workspace_size(B, Hq, Hkv, head_dim, num_splits))


def cascade_workspace_size(B: int, Hq: int, Hkv: int, head_dim: int, splits_prefix: int,
                           splits_suffix: int) -> int:
    return int(load_library().fdec_cascade_workspace_size(B, Hq, Hkv, head_dim, splits_prefix, splits_suffix))


class Workspace:
    """A device workspace (uint8 tensor) prepared with fdec_workspace_init."""

    def __init__(self, nbytes: int, device="cuda"):
        self.buf = torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _check(load_library().fdec_workspace_init(self.buf.data_ptr(), self.buf.numel(),
                                                  _stream(self.buf.device)))

    @property
    def nbytes(self) -> int:
        return self.buf.numel()


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
           page_table: Optional[torch.Tensor] = None, num_splits: int = 0, softmax_scale: float = 0.0,
           append: Optional[FdecAppend] = None, fused: bool = False, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, workspace: Optional[Workspace] = None,
           return_lse: bool = True, k_descale: Optional[torch.Tensor] = None,
           v_descale: Optional[torch.Tensor] = None, cache_batch_idx: Optional[torch.Tensor] = None,
           cache_leftpad: Optional[torch.Tensor] = None):
    """fdec_decode: returns (out [B, Hq, D] fp32, lse [B, Hq] fp32 or None)."""
    lib = load_library()
    B, Hq, D = q.shape
    kv = make_kv(k, v, page_table, k_descale, v_descale, cache_batch_idx, cache_leftpad)
    _check_q(q, k)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    S = num_splits if num_splits > 0 else plan(B, Hq, kv.num_kv_heads, None, kv.capacity, kv.page_size,
                                               kv_dtype=kv.dtype)
    if workspace is None:
        workspace = Workspace(workspace_size(B, Hq, kv.num_kv_heads, D, S), q.device)
    _check(lib.fdec_decode(q.data_ptr(), B, Hq, ctypes.byref(kv), seq_lens.data_ptr(), S,
                           float(softmax_scale), ctypes.byref(append) if append is not None else None,
                           int(bool(fused)), out.data_ptr(), _ptr(lse), workspace.buf.data_ptr(),
                           workspace.nbytes, _stream(q.device)))
    return out, lse


def decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                   page_table: Optional[torch.Tensor] = None, num_splits: int = 0, softmax_scale: float = 0.0,
                   append: Optional[FdecAppend] = None, fused: bool = False, out: Optional[torch.Tensor] = None,
                   lse: Optional[torch.Tensor] = None, return_lse: bool = True,
                   k_descale: Optional[torch.Tensor] = None, v_descale: Optional[torch.Tensor] = None,
                   cache_batch_idx: Optional[torch.Tensor] = None, cache_leftpad: Optional[torch.Tensor] = None):
    """fdec_decode_noalloc: fdec_decode on the library's own device scratch (no workspace).

    Allocates nothing when out (and lse, or return_lse=False) are passed in."""
    lib = load_library()
    B, Hq, D = q.shape
    kv = make_kv(k, v, page_table, k_descale, v_descale, cache_batch_idx, cache_leftpad)
    _check_q(q, k)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    _check(lib.fdec_decode_noalloc(q.data_ptr(), B, Hq, ctypes.byref(kv), seq_lens.data_ptr(), int(num_splits),
                                   float(softmax_scale), ctypes.byref(append) if append is not None else None,
                                   int(bool(fused)), out.data_ptr(), _ptr(lse), _stream(q.device)))
    return out, lse


def decode_multi(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                 page_table: Optional[torch.Tensor] = None, num_splits: int = 0, softmax_scale: float = 0.0,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[Workspace] = None, return_lse: bool = True,
                 k_descale: Optional[torch.Tensor] = None, v_descale: Optional[torch.Tensor] = None,
                 cache_batch_idx: Optional[torch.Tensor] = None, cache_leftpad: Optional[torch.Tensor] = None):
    """fdec_decode_multi: q [B, q_len, Hq, D] -> (out [B, q_len, Hq, D] fp32, lse [B, Hq, q_len] fp32 or None)."""
    lib = load_library()
    if q.dim() != 4 or not q.is_contiguous():
        raise FdecError(FDEC_ERR_INVALID_ARG, "q must be a contiguous [B, q_len, Hq, D] tensor")
    B, q_len, Hq, D = q.shape
    kv = make_kv(k, v, page_table, k_descale, v_descale, cache_batch_idx, cache_leftpad)
    _check_q(q, k)
    if out is None:
        out = torch.empty(B, q_len, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, q_len, dtype=torch.float32, device=q.device)
    S = num_splits if num_splits > 0 else plan(B, Hq, kv.num_kv_heads, None, kv.capacity, kv.page_size,
                                               kv_dtype=kv.dtype)
    if workspace is None:
        workspace = Workspace(workspace_size(B * q_len, Hq, kv.num_kv_heads, D, S), q.device)
    _check(lib.fdec_decode_multi(q.data_ptr(), B, q_len, Hq, ctypes.byref(kv), seq_lens.data_ptr(), S,
                                 float(softmax_scale), out.data_ptr(), _ptr(lse), workspace.buf.data_ptr(),
                                 workspace.nbytes, _stream(q.device)))
    return out, lse


def decode_multi_balanced(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                          page_table: Optional[torch.Tensor] = None, num_blocks: int = 0, softmax_scale: float = 0.0,
                          out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[Workspace] = None, return_lse: bool = True,
                          k_descale: Optional[torch.Tensor] = None, v_descale: Optional[torch.Tensor] = None,
                          cache_batch_idx: Optional[torch.Tensor] = None,
                          cache_leftpad: Optional[torch.Tensor] = None):
    """fdec_decode_multi_balanced: q [B, q_len, Hq, D] -> (out [B, q_len, Hq, D], lse [B, Hq, q_len] or None)."""
    lib = load_library()
    if q.dim() != 4 or not q.is_contiguous():
        raise FdecError(FDEC_ERR_INVALID_ARG, "q must be a contiguous [B, q_len, Hq, D] tensor")
    B, q_len, Hq, D = q.shape
    kv = make_kv(k, v, page_table, k_descale, v_descale, cache_batch_idx, cache_leftpad)
    _check_q(q, k)
    if out is None:
        out = torch.empty(B, q_len, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, q_len, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = Workspace(balanced_workspace_size(B, q_len * Hq, kv.num_kv_heads, D, num_blocks), q.device)
    _check(lib.fdec_decode_multi_balanced(q.data_ptr(), B, q_len, Hq, ctypes.byref(kv), seq_lens.data_ptr(),
                                          int(num_blocks), float(softmax_scale), out.data_ptr(), _ptr(lse),
                                          workspace.buf.data_ptr(), workspace.nbytes, _stream(q.device)))
    return out, lse


def balanced_workspace_size(B: int, Hq: int, Hkv: int, D: int, num_blocks: int = 0) -> int:
    n = load_library().fdec_balanced_workspace_size(B, Hq, Hkv, D, num_blocks)
    if n == 0:
        raise FdecError(FDEC_ERR_INVALID_ARG, "fdec_balanced_workspace_size: bad arguments")
    return n


def decode_balanced(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                    page_table: Optional[torch.Tensor] = None, num_blocks: int = 0, softmax_scale: float = 0.0,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[Workspace] = None, return_lse: bool = True,
                    k_descale: Optional[torch.Tensor] = None, v_descale: Optional[torch.Tensor] = None,
                    cache_batch_idx: Optional[torch.Tensor] = None, cache_leftpad: Optional[torch.Tensor] = None):
    """fdec_decode_balanced: returns (out [B, Hq, D] fp32, lse [B, Hq] fp32 or None)."""
    lib = load_library()
    B, Hq, D = q.shape
    kv = make_kv(k, v, page_table, k_descale, v_descale, cache_batch_idx, cache_leftpad)
    _check_q(q, k)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = Workspace(balanced_workspace_size(B, Hq, kv.num_kv_heads, D, num_blocks), q.device)
    _check(lib.fdec_decode_balanced(q.data_ptr(), B, Hq, ctypes.byref(kv), seq_lens.data_ptr(), int(num_blocks),
                                    float(softmax_scale), out.data_ptr(), _ptr(lse), workspace.buf.data_ptr(),
                                    workspace.nbytes, _stream(q.device)))
    return out, lse


def decode_partials(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor,
                    num_splits: int, page_table: Optional[torch.Tensor] = None, softmax_scale: float = 0.0,
                    append: Optional[FdecAppend] = None, part_o: Optional[torch.Tensor] = None,
                    part_m: Optional[torch.Tensor] = None, part_d: Optional[torch.Tensor] = None,
                    k_descale: Optional[torch.Tensor] = None, v_descale: Optional[torch.Tensor] = None,
                    cache_batch_idx: Optional[torch.Tensor] = None, cache_leftpad: Optional[torch.Tensor] = None):
    """fdec_decode_partials: returns (part_o [B,Hq,S,D], part_m [B,Hq,S], part_d [B,Hq,S]) fp32."""
    lib = load_library()
    B, Hq, D = q.shape
    kv = make_kv(k, v, page_table, k_descale, v_descale, cache_batch_idx, cache_leftpad)
    _check_q(q, k)
    S = num_splits
    if part_o is None:
        part_o = torch.empty(B, Hq, S, D, dtype=torch.float32, device=q.device)
        part_m = torch.empty(B, Hq, S, dtype=torch.float32, device=q.device)
        part_d = torch.empty(B, Hq, S, dtype=torch.float32, device=q.device)
    _check(lib.fdec_decode_partials(q.data_ptr(), B, Hq, ctypes.byref(kv), seq_lens.data_ptr(), S,
                                    float(softmax_scale),
                                    ctypes.byref(append) if append is not None else None,
                                    part_o.data_ptr(), part_m.data_ptr(), part_d.data_ptr(),
                                    _stream(q.device)))
    return part_o, part_m, part_d


def merge_states(part_o: torch.Tensor, part_m: torch.Tensor, part_d: torch.Tensor,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """fdec_merge_states: (out [B,Hq,D], lse [B,Hq]) from states [B,Hq,S,D] / [B,Hq,S]."""
    lib = load_library()
    B, Hq, S, D = part_o.shape
    for t in (part_o, part_m, part_d):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise FdecError(FDEC_ERR_INVALID_ARG, "states must be contiguous float32")
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=part_o.device)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=part_o.device)
    _check(lib.fdec_merge_states(part_o.data_ptr(), part_m.data_ptr(), part_d.data_ptr(), B, Hq, S, D,
                                 out.data_ptr(), _ptr(lse), _stream(part_o.device)))
    return out, lse


PROBE_BLOCKS = 2048


def probe_read(src: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fdec_probe_read: stream every byte of `src` (a calibration probe)."""
    if sink is None:
        sink = torch.empty(PROBE_BLOCKS, dtype=torch.int32, device=src.device)
    _check(load_library().fdec_probe_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(),
                                          _stream(src.device)))
    return sink


def trace_start(max_events: int = 4096) -> None:
    """fdec_trace_start: record stage-timing events for this thread's next calls."""
    _check(load_library().fdec_trace_start(int(max_events)))


def trace_stop():
    """fdec_trace_stop: (intervals_ms, kinds) of the trace; kind k >= 1 marks the end of a call's
    k-th kernel (the interval is that kernel's time), 0 the start of a call."""
    lib = load_library()
    cap = 1 << 20
    n = ctypes.c_int(0)
    ms = (ctypes.c_float * 8192)()
    kinds = (ctypes.c_int * 8192)()
    _check(lib.fdec_trace_stop(ctypes.cast(ms, ctypes.c_void_p), ctypes.cast(kinds, ctypes.c_void_p), 8192,
                               ctypes.byref(n)))
    m = max(0, min(n.value - 1, 8192, cap))
    return [float(ms[i]) for i in range(m)], [int(kinds[i]) for i in range(m)]


CHECK_LENGTH, CHECK_PAGE, CHECK_LEFTPAD, CHECK_BATCH_IDX, CHECK_ROPE_POS, CHECK_PREFIX_PAGE = 1, 2, 4, 8, 16, 32


def check_inputs(k: torch.Tensor, v: torch.Tensor, seq_lens: torch.Tensor, page_table: Optional[torch.Tensor] = None,
                 append: Optional[FdecAppend] = None, prefix_pages: Optional[torch.Tensor] = None,
                 prefix_len: int = 0, cache_batch_idx: Optional[torch.Tensor] = None,
                 cache_leftpad: Optional[torch.Tensor] = None):
    """fdec_check_inputs: (flags, first flagged request) of the device data a call would trust."""
    kv = make_kv(k, v, page_table, cache_batch_idx=cache_batch_idx, cache_leftpad=cache_leftpad)
    flags, first = ctypes.c_int(0), ctypes.c_int(0)
    _check(load_library().fdec_check_inputs(seq_lens.shape[0], ctypes.byref(kv), seq_lens.data_ptr(),
                                            ctypes.byref(append) if append is not None else None,
                                            _ptr(prefix_pages), prefix_len, ctypes.byref(flags),
                                            ctypes.byref(first), _stream(k.device)))
    return flags.value, first.value


def set_debug(on: bool) -> None:
    """fdec_set_debug: every decode call checks its device data first (and refuses bad data)."""
    load_library().fdec_set_debug(int(bool(on)))


def debug_enabled() -> bool:
    return bool(load_library().fdec_debug_enabled())


PROBE_STATIC, PROBE_TICKETS = 0, 1


def probe_stream(src: torch.Tensor, mode: int = PROBE_STATIC, per_cu: int = 1,
                 sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fdec_probe_stream over the bytes of src (LDS-DMA streaming read); returns the sink.

    The sink's last word is the ticket counter: a new sink is zeroed, and each call leaves it zero."""
    lib = load_library()
    if sink is None:
        sink = torch.zeros(PROBE_BLOCKS + 1, dtype=torch.int32, device=src.device)
    _check(lib.fdec_probe_stream(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), int(mode),
                                 int(per_cu), _stream(src.device)))
    return sink


def probe_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """fdec_probe_copy: plain copy of src's bytes into dst (a calibration probe)."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise FdecError(FDEC_ERR_INVALID_ARG, "dst smaller than src")
    _check(load_library().fdec_probe_copy(dst.data_ptr(), src.data_ptr(), n, _stream(src.device)))


def cascade_plan(B: int, Hq: int, Hkv: int, prefix_len: int, capacity: int, page_size: int,
                 cu_count: int = 256, kv_dtype=None):
    """fdec_cascade_plan, or fdec_cascade_plan_kv when kv_dtype (a torch dtype or an fdec_dtype
    code) is given: (splits_prefix, splits_suffix)."""
    sp, ss = ctypes.c_int(0), ctypes.c_int(0)
    lib = load_library()
    if kv_dtype is None:
        _check(lib.fdec_cascade_plan(B, Hq, Hkv, prefix_len, capacity, page_size, cu_count, ctypes.byref(sp),
                                     ctypes.byref(ss)))
    else:
        code = kv_dtype if isinstance(kv_dtype, int) else _dtype_code(kv_dtype)
        _check(lib.fdec_cascade_plan_kv(B, Hq, Hkv, prefix_len, capacity, page_size, code, cu_count,
                                        ctypes.byref(sp), ctypes.byref(ss)))
    return sp.value, ss.value


def cascade_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, page_table: torch.Tensor,
                   prefix_pages: torch.Tensor, prefix_len: int, suffix_lens: torch.Tensor,
                   splits_prefix: int = 0, splits_suffix: int = 0, softmax_scale: float = 0.0,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   workspace: Optional[Workspace] = None, cache_leftpad: Optional[torch.Tensor] = None,
                   k_descale: Optional[torch.Tensor] = None, v_descale: Optional[torch.Tensor] = None):
    """fdec_cascade_decode: shared prefix + per-request suffix, merged exactly (no left padding)."""
    lib = load_library()
    B, Hq, D = q.shape
    kv = make_kv(k, v, page_table, k_descale, v_descale, cache_leftpad=cache_leftpad)
    _check_q(q, k)
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=q.device)
    if splits_prefix <= 0 or splits_suffix <= 0:
        # as fdec_cascade_decode plans: a planned count fits beside a count the caller gave
        sp, ss = cascade_plan(B, Hq, kv.num_kv_heads, prefix_len, kv.capacity, kv.page_size, kv_dtype=k.dtype)
        if splits_prefix <= 0:
            splits_prefix = max(1, min(sp, MAX_SPLITS - splits_suffix)) if splits_suffix > 0 else sp
        if splits_suffix <= 0:
            splits_suffix = max(1, min(ss, MAX_SPLITS - splits_prefix))
    if workspace is None:
        workspace = Workspace(cascade_workspace_size(B, Hq, kv.num_kv_heads, D, splits_prefix, splits_suffix),
                              q.device)
    _check(lib.fdec_cascade_decode(q.data_ptr(), B, Hq, ctypes.byref(kv), _ptr(prefix_pages), prefix_len,
                                   suffix_lens.data_ptr(), splits_prefix, splits_suffix, float(softmax_scale),
                                   out.data_ptr(), _ptr(lse), workspace.buf.data_ptr(), workspace.nbytes,
                                   _stream(q.device)))
    return out, lse
