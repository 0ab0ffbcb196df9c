"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host before any launch (no GPU needed: every call here fails
validation, so nothing reaches the HIP runtime)."""
import ctypes
import os
import re

import pytest
import torch

import decode_attention_fdec_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            src = open(os.path.join(ROOT, "include", fn)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(fdec_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["fdec_plan", "fdec_decode", "fdec_merge_states", "fdec_decode_partials",
                     "fdec_cascade_decode", "fdec_workspace_size", "fdec_workspace_init",
                     "fdec_status_string", "fdec_last_error", "fdec_plan_rules", "fdec_split_chunk"]:
        assert required in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_declared_symbol(fdec, name):
    lib = ctypes.CDLL(F.LIB_PATH)
    assert hasattr(lib, name), f"{name} declared in include/ but not exported"


def test_status_strings(fdec):
    lib = F.load_library()
    for s in range(5):
        assert lib.fdec_status_string(s)
    assert lib.fdec_status_string(99) == b"unknown status"


# Fake, 256-byte aligned "device" addresses: validation must reject the call
# before anything dereferences them.
FAKE = 0x10000


def kv_struct(**over):
    kv = F.FdecKV()
    kv.k, kv.v = FAKE, FAKE + 0x1000
    kv.dtype, kv.num_kv_heads, kv.head_dim = F.FDEC_BF16, 8, 128
    kv.page_size, kv.capacity = 0, 4096
    kv.s_outer, kv.s_token, kv.s_head = 4096 * 8 * 128, 8 * 128, 128
    kv.page_table, kv.max_pages_per_seq = None, 0
    for k, v in over.items():
        setattr(kv, k, v)
    return kv


def call_decode(kv, B=1, Hq=32, num_splits=4, ws_bytes=1 << 30, append=None, fused=0, q=FAKE,
                seq=FAKE, out=FAKE, scale=0.0, ws=FAKE):
    lib = F.load_library()
    return lib.fdec_decode(q, B, Hq, ctypes.byref(kv), seq, num_splits, scale,
                           ctypes.byref(append) if append else None, fused, out, None, ws, ws_bytes,
                           None)


def last_error():
    return F.load_library().fdec_last_error().decode()


@pytest.mark.parametrize("ps", [8, 24, 1, -16])
def test_page_size_must_be_multiple_of_16(fdec, ps):
    kv = kv_struct(page_size=ps, page_table=FAKE, max_pages_per_seq=64, capacity=0)
    assert call_decode(kv) == F.FDEC_ERR_INVALID_ARG
    assert "page_size" in last_error()


def test_head_ratio_must_divide(fdec):
    assert call_decode(kv_struct(num_kv_heads=5), Hq=32) == F.FDEC_ERR_INVALID_ARG


def test_unsupported_shapes_are_reported_as_unsupported(fdec):
    assert call_decode(kv_struct(head_dim=96)) == F.FDEC_ERR_UNSUPPORTED
    assert call_decode(kv_struct(head_dim=256)) == F.FDEC_ERR_UNSUPPORTED
    assert call_decode(kv_struct(dtype=7)) == F.FDEC_ERR_UNSUPPORTED  # not an fdec_dtype
    assert call_decode(kv_struct(num_kv_heads=2), Hq=32) == F.FDEC_ERR_UNSUPPORTED  # G = 16


def test_null_and_misaligned_pointers(fdec):
    assert call_decode(kv_struct(), q=None) == F.FDEC_ERR_INVALID_ARG
    assert call_decode(kv_struct(), seq=None) == F.FDEC_ERR_INVALID_ARG
    assert call_decode(kv_struct(), out=None) == F.FDEC_ERR_INVALID_ARG
    assert call_decode(kv_struct(k=FAKE + 2)) == F.FDEC_ERR_INVALID_ARG
    assert call_decode(kv_struct(s_token=8 * 128 + 4)) == F.FDEC_ERR_INVALID_ARG
    assert call_decode(kv_struct(), q=FAKE + 8) == F.FDEC_ERR_INVALID_ARG


def test_bad_split_counts(fdec):
    assert call_decode(kv_struct(), num_splits=-1) == F.FDEC_ERR_INVALID_ARG
    assert call_decode(kv_struct(), num_splits=F.MAX_SPLITS + 1) == F.FDEC_ERR_INVALID_ARG


def test_workspace_too_small_is_reported_not_allocated(fdec):
    need = F.workspace_size(1, 32, 8, 128, 4)
    assert need > 0
    assert call_decode(kv_struct(), ws_bytes=need - 1) == F.FDEC_ERR_WORKSPACE
    assert str(need) in last_error()
    assert call_decode(kv_struct(), ws=None) == F.FDEC_ERR_WORKSPACE


def test_paged_cache_checks(fdec):
    kv = kv_struct(page_size=16, page_table=None, max_pages_per_seq=64, capacity=0)
    assert call_decode(kv) == F.FDEC_ERR_INVALID_ARG
    kv = kv_struct(page_size=16, page_table=FAKE, max_pages_per_seq=64, capacity=1000)
    assert call_decode(kv) == F.FDEC_ERR_INVALID_ARG  # capacity != pages * page_size


def test_append_checks(fdec):
    a = F.FdecAppend()
    a.k_new, a.v_new, a.rotary_dim = FAKE, FAKE, 3
    assert call_decode(kv_struct(), append=a) == F.FDEC_ERR_INVALID_ARG
    a.rotary_dim = 64  # rotary without tables
    assert call_decode(kv_struct(), append=a) == F.FDEC_ERR_INVALID_ARG
    a.rotary_dim, a.k_new = 0, None
    assert call_decode(kv_struct(), append=a) == F.FDEC_ERR_INVALID_ARG


def test_bad_fused_flag_and_scale(fdec):
    assert call_decode(kv_struct(), fused=2) == F.FDEC_ERR_INVALID_ARG
    assert call_decode(kv_struct(), scale=float("nan")) == F.FDEC_ERR_INVALID_ARG


def test_merge_states_validation(fdec):
    lib = F.load_library()
    assert lib.fdec_merge_states(FAKE, FAKE, FAKE, 1, 32, 0, 128, FAKE, None, None) == F.FDEC_ERR_INVALID_ARG
    assert lib.fdec_merge_states(FAKE, FAKE, FAKE, 1, 32, 300, 128, FAKE, None, None) == F.FDEC_ERR_INVALID_ARG
    assert lib.fdec_merge_states(FAKE, FAKE, FAKE, 1, 32, 4, 80, FAKE, None, None) == F.FDEC_ERR_UNSUPPORTED
    assert lib.fdec_merge_states(None, FAKE, FAKE, 1, 32, 4, 128, FAKE, None, None) == F.FDEC_ERR_INVALID_ARG


def test_partials_validation(fdec):
    lib = F.load_library()
    kv = kv_struct()
    assert lib.fdec_decode_partials(FAKE, 1, 32, ctypes.byref(kv), FAKE, 0, 0.0, None, FAKE, FAKE, FAKE,
                                    None) == F.FDEC_ERR_INVALID_ARG
    assert lib.fdec_decode_partials(FAKE, 1, 32, ctypes.byref(kv), FAKE, 4, 0.0, None, None, FAKE, FAKE,
                                    None) == F.FDEC_ERR_INVALID_ARG


def test_empty_batch_is_a_no_op(fdec):
    # B = 0 returns OK without touching any pointer
    assert call_decode(kv_struct(), B=0, q=None, seq=None, out=None, ws=None) == F.FDEC_OK


def test_workspace_size_grows_with_splits(fdec):
    a = F.workspace_size(32, 32, 8, 128, 8)
    b = F.workspace_size(32, 32, 8, 128, 16)
    assert b > a >= 32 * 32 * 8 * (128 + 2) * 4
    assert F.workspace_size(1, 32, 8, 128, 0) == 0


def test_split_chunk_rule(fdec):
    assert F.split_chunk(1024, 4) == 256
    assert F.split_chunk(131072, 16) == 8192
    assert F.split_chunk(100, 3) == 48  # ceil(100/3) = 34 -> 48
    assert F.split_chunk(5, 1) == 16
    assert F.split_chunk(0, 4) == 0


def test_cascade_validation(fdec):
    lib = F.load_library()
    kv = kv_struct()  # contiguous: the cascade needs pages
    args = lambda kv, plen, pages: (FAKE, 2, 32, ctypes.byref(kv), pages, plen, FAKE, 2, 2, 0.0, FAKE, None,
                                    FAKE, 1 << 30, None)
    assert lib.fdec_cascade_decode(*args(kv, 64, FAKE)) == F.FDEC_ERR_INVALID_ARG
    kvp = kv_struct(page_size=64, page_table=FAKE, max_pages_per_seq=32, capacity=0)
    assert lib.fdec_cascade_decode(*args(kvp, 64, None)) == F.FDEC_ERR_INVALID_ARG  # no prefix pages
    assert lib.fdec_cascade_decode(*args(kvp, -1, FAKE)) == F.FDEC_ERR_INVALID_ARG
    kv64 = kv_struct(page_size=64, page_table=FAKE, max_pages_per_seq=32, capacity=0, head_dim=64)
    assert lib.fdec_cascade_decode(*args(kv64, 64, FAKE)) == F.FDEC_ERR_UNSUPPORTED
    small = F.cascade_workspace_size(2, 32, 8, 128, 2, 2) - 1
    assert lib.fdec_cascade_decode(FAKE, 2, 32, ctypes.byref(kvp), FAKE, 64, FAKE, 2, 2, 0.0, FAKE, None, FAKE,
                                   small, None) == F.FDEC_ERR_WORKSPACE


def test_cascade_plan_for_float8_pools(fdec, monkeypatch):
    import torch

    # G = 4 with Hkv a multiple of 4: prefix and suffix share one launch, with at
    # most one block of each per compute unit: 128-row prefix chunks on three
    # quarters of the 256 units for 16-bit pools (12 splits x 8 KV heads x 2
    # chunks), on all of them for float8 pools (16 splits), and one suffix block
    # per unit
    monkeypatch.delenv("FDEC_CASCADE_PATH", raising=False)
    assert F.cascade_plan(64, 32, 8, 16384, 2048, 64, kv_dtype=torch.bfloat16) == F.cascade_plan(64, 32, 8, 16384,
                                                                                                  2048, 64)
    assert F.cascade_plan(64, 32, 8, 16384, 2048, 64) == (12, 128)
    assert F.cascade_plan(64, 32, 8, 16384, 2048, 64, kv_dtype=torch.float8_e4m3fn) == (16, 128)
    # separate prefix and suffix kernels (forced, or two KV heads per suffix block):
    # 256-row prefix chunks, and float8 pools take two suffix blocks per compute
    # unit within the 256 states a merge holds
    for Hq, Hkv, env in ((32, 8, "two"), (8, 2, None)):
        if env:
            monkeypatch.setenv("FDEC_CASCADE_PATH", env)
        sp, ss = F.cascade_plan(64, Hq, Hkv, 16384, 2048, 64, kv_dtype=torch.float8_e4m3fn)
        sp16, ss16 = F.cascade_plan(64, Hq, Hkv, 16384, 2048, 64)
        assert sp == sp16 and ss == min(2 * ss16, F.MAX_SPLITS - sp)
        monkeypatch.delenv("FDEC_CASCADE_PATH", raising=False)
    assert F.cascade_plan(4, 8, 4, 500, 512, 16, kv_dtype=torch.float8_e4m3fn)[1] == \
        F.plan(4, 8, 4, None, 512, 16, kv_dtype=torch.float8_e4m3fn)
    lib = F.load_library()
    a, b = ctypes.c_int(0), ctypes.c_int(0)
    assert lib.fdec_cascade_plan_kv(4, 8, 4, 500, 512, 16, 9, 256, ctypes.byref(a), ctypes.byref(b)) == \
        F.FDEC_ERR_INVALID_ARG


def test_cascade_plan(fdec):
    sp, ss = F.cascade_plan(64, 32, 8, 16384, 2048, 64)
    assert 8 * sp * 2 <= 256 and 1 <= ss and sp + ss <= F.MAX_SPLITS  # at most one prefix block per unit
    sp, ss = F.cascade_plan(2, 8, 2, 100, 256, 16)
    assert sp == 1  # fewer than 256 prefix tokens: one split
    sp, ss = F.cascade_plan(1, 8, 8, 0, 64, 16)
    assert sp >= 1 and ss >= 1


def call_balanced(kv, B=2, Hq=32, num_blocks=16, ws_bytes=1 << 30, out=FAKE, ws=FAKE):
    lib = F.load_library()
    return lib.fdec_decode_balanced(FAKE, B, Hq, ctypes.byref(kv), FAKE, num_blocks, 0.0, out, None, ws,
                                    ws_bytes, None)


def test_balanced_validation(fdec):
    # only the matrix-core kernels' head_dim 128
    assert call_balanced(kv_struct(head_dim=64, s_outer=4096 * 8 * 64, s_token=8 * 64, s_head=64)) == \
        F.FDEC_ERR_UNSUPPORTED
    assert call_balanced(kv_struct(), num_blocks=-1) == F.FDEC_ERR_INVALID_ARG
    assert call_balanced(kv_struct(), num_blocks=F.MAX_SPLITS + 1) == F.FDEC_ERR_INVALID_ARG
    assert call_balanced(kv_struct(), out=None) == F.FDEC_ERR_INVALID_ARG
    need = F.balanced_workspace_size(2, 32, 8, 128, 16)
    assert call_balanced(kv_struct(), ws_bytes=need - 1) == F.FDEC_ERR_WORKSPACE
    assert str(need) in last_error()
    # tiles of all requests must be countable in 31 bits
    assert call_balanced(kv_struct(capacity=1 << 30, s_outer=(1 << 30) * 1024), B=64) == F.FDEC_ERR_INVALID_ARG


def test_balanced_workspace_size(fdec):
    # the fused path's counters [B, Hkv] int32 (kept clear for it), meta [B, 2] int32, then m, d and O~
    # for Hq x (num_blocks + B) slots, each array 256-byte aligned
    def up(n):
        return (n + 255) // 256 * 256
    B, Hq, D, nb = 3, 32, 128, 10
    slots = Hq * (nb + B)
    want = up(up(up(up(B * 8 * 4) + B * 8) + slots * 4) + slots * 4) + up(slots * D * 4)
    assert F.balanced_workspace_size(B, Hq, 8, D, nb) == want
    with pytest.raises(F.FdecError):
        F.balanced_workspace_size(B, Hq, 8, D, 257)


def test_fp8_validation(fdec):
    lib = F.load_library()
    fp8 = dict(dtype=F.FDEC_FP8_E4M3)
    # strides must be multiples of 16 bytes: 16 float8 elements
    assert call_decode(kv_struct(s_head=8, **fp8)) == F.FDEC_ERR_INVALID_ARG
    # the balanced split takes float8 at head_dim 128 only
    assert call_balanced(kv_struct(head_dim=64, s_outer=4096 * 8 * 64, s_token=8 * 64, s_head=64, **fp8)) == \
        F.FDEC_ERR_UNSUPPORTED
    # an append into a float8 cache is checked like any other
    a = F.FdecAppend()
    a.k_new, a.v_new = FAKE, FAKE
    a.rotary_dim = 3
    assert call_decode(kv_struct(**fp8), append=a) == F.FDEC_ERR_INVALID_ARG
    assert "rotary_dim" in last_error()
    # the cascade takes float8 pools under the same checks as 16-bit ones
    kvp = kv_struct(page_size=64, page_table=FAKE, max_pages_per_seq=32, capacity=0, head_dim=64, s_outer=64 * 8 * 64,
                    s_token=8 * 64, s_head=64, **fp8)
    assert lib.fdec_cascade_decode(FAKE, 2, 32, ctypes.byref(kvp), FAKE, 64, FAKE, 2, 2, 0.0, FAKE, None,
                                   FAKE, 1 << 30, None) == F.FDEC_ERR_UNSUPPORTED
    assert "head_dim" in last_error()
    # an unknown element type
    assert call_decode(kv_struct(dtype=3)) == F.FDEC_ERR_UNSUPPORTED


def test_batch_idx_and_leftpad_validation(fdec):
    lib = F.load_library()
    # cache_batch_idx is for contiguous caches only
    kvp = kv_struct(page_size=16, page_table=FAKE, max_pages_per_seq=64, capacity=0, cache_batch_idx=FAKE)
    assert call_decode(kvp) == F.FDEC_ERR_INVALID_ARG
    assert "cache_batch_idx" in last_error()
    # no left padding with a shared prefix
    kvc = kv_struct(page_size=64, page_table=FAKE, max_pages_per_seq=32, capacity=0, cache_leftpad=FAKE)
    assert lib.fdec_cascade_decode(FAKE, 2, 32, ctypes.byref(kvc), FAKE, 64, FAKE, 2, 2, 0.0, FAKE, None,
                                   FAKE, 1 << 30, None) == F.FDEC_ERR_UNSUPPORTED
    assert "leftpad" in last_error()


def test_binding_checks_index_tensors(fdec):
    k = torch.zeros(2, 32, 2, 128, dtype=torch.float16)
    for bad in (torch.zeros(2, dtype=torch.int64), torch.zeros(2, 2, dtype=torch.int32),
                torch.zeros(4, dtype=torch.int32)[::2]):
        with pytest.raises(F.FdecError):
            F.make_kv(k, k, cache_batch_idx=bad)
        with pytest.raises(F.FdecError):
            F.make_kv(k, k, cache_leftpad=bad)
    kv = F.make_kv(k, k, cache_batch_idx=torch.zeros(2, dtype=torch.int32),
                   cache_leftpad=torch.zeros(2, dtype=torch.int32))
    assert kv.cache_batch_idx and kv.cache_leftpad


def call_noalloc(kv, B=1, Hq=32, num_splits=4, fused=0, q=FAKE, seq=FAKE, out=FAKE):
    lib = F.load_library()
    return lib.fdec_decode_noalloc(q, B, Hq, ctypes.byref(kv), seq, num_splits, 0.0, None, fused, out, None, None)


def test_noalloc_validates_like_decode_and_bounds_its_scratch(fdec):
    # the argument checks of fdec_decode, then the scratch bound, all before any HIP call
    assert call_noalloc(kv_struct(num_kv_heads=5)) == F.FDEC_ERR_INVALID_ARG
    assert call_noalloc(kv_struct(head_dim=96)) == F.FDEC_ERR_UNSUPPORTED
    assert call_noalloc(kv_struct(), q=None) == F.FDEC_ERR_INVALID_ARG
    assert call_noalloc(kv_struct(), num_splits=-1) == F.FDEC_ERR_INVALID_ARG
    assert call_noalloc(kv_struct(), fused=2) == F.FDEC_ERR_INVALID_ARG
    # states of B * Hq * S splits beyond FDEC_NOALLOC_SCRATCH_BYTES - 64 KiB
    assert call_noalloc(kv_struct(), B=64, Hq=64, num_splits=256) == F.FDEC_ERR_WORKSPACE
    assert "scratch" in last_error()
    # more than 16384 (request, KV head) counters
    assert call_noalloc(kv_struct(num_kv_heads=8, capacity=16), B=4096, Hq=8, num_splits=1) == F.FDEC_ERR_WORKSPACE
    # B = 0 is a valid empty call
    assert call_noalloc(kv_struct(), B=0) == F.FDEC_OK


def test_trace_arguments_and_an_empty_trace(fdec):
    lib = F.load_library()
    assert lib.fdec_trace_start(1) == F.FDEC_ERR_INVALID_ARG
    assert lib.fdec_trace_start(16) == F.FDEC_OK
    n = ctypes.c_int(-1)
    assert lib.fdec_trace_stop(None, None, 0, ctypes.byref(n)) == F.FDEC_OK
    assert n.value == 0
    # failing calls launch nothing and record nothing
    assert lib.fdec_trace_start(16) == F.FDEC_OK
    assert call_decode(kv_struct(num_kv_heads=5)) == F.FDEC_ERR_INVALID_ARG
    assert lib.fdec_trace_stop(None, None, 0, ctypes.byref(n)) == F.FDEC_OK
    assert n.value == 0


def test_check_inputs_validation_and_debug_switch(fdec):
    lib = F.load_library()
    flags, first = ctypes.c_int(0), ctypes.c_int(0)
    kv = kv_struct()
    # malformed arguments are refused before any HIP call
    assert lib.fdec_check_inputs(1, ctypes.byref(kv), FAKE, None, None, 0, None, None, None) == F.FDEC_ERR_INVALID_ARG
    assert lib.fdec_check_inputs(-1, ctypes.byref(kv), FAKE, None, None, 0, ctypes.byref(flags), None,
                                 None) == F.FDEC_ERR_INVALID_ARG
    assert lib.fdec_check_inputs(1, ctypes.byref(kv), None, None, None, 0, ctypes.byref(flags), None,
                                 None) == F.FDEC_ERR_INVALID_ARG
    # a prefix needs a paged pool
    assert lib.fdec_check_inputs(1, ctypes.byref(kv), FAKE, None, FAKE, 16, ctypes.byref(flags), ctypes.byref(first),
                                 None) == F.FDEC_ERR_INVALID_ARG
    assert "prefix" in last_error()
    assert lib.fdec_check_inputs(1, ctypes.byref(kv_struct(num_blocks=-2)), FAKE, None, None, 0,
                                 ctypes.byref(flags), None, None) == F.FDEC_ERR_INVALID_ARG
    # the debug switch is process-wide and needs no GPU
    was = lib.fdec_debug_enabled()
    lib.fdec_set_debug(1)
    assert lib.fdec_debug_enabled() == 1
    lib.fdec_set_debug(0)
    assert lib.fdec_debug_enabled() == 0
    lib.fdec_set_debug(was)


def test_cascade_plans_one_count_beside_the_other(fdec):
    # a planned suffix count fits beside an explicit prefix count (and the other
    # way round): the planner alone would give 1 + 255 here
    lib = F.load_library()
    kvp = kv_struct(page_size=16, page_table=FAKE, max_pages_per_seq=4, capacity=0, num_kv_heads=4)
    sp, ss = F.cascade_plan(40, 16, 4, 15, 64, 16)
    assert sp + ss == F.MAX_SPLITS
    n = lib.fdec_cascade_workspace_size(40, 16, 4, 128, 3, ss)
    # explicit 3 + planned: accepted up to the workspace check (too small on purpose)
    assert lib.fdec_cascade_decode(FAKE, 40, 16, ctypes.byref(kvp), FAKE, 15, FAKE, 3, 0, 0.0, FAKE, None, FAKE, 16,
                                   None) == F.FDEC_ERR_WORKSPACE
    assert "splits" in last_error() and str(F.MAX_SPLITS - 3) in last_error()
    assert n > 0
