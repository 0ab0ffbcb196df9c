"""fdec_decode_noalloc (the entry point for callers that cannot allocate) against
fdec_decode, through the C ABI.

The no-allocation call runs fdec_decode's kernels on the library's own device
scratch, so its output must equal fdec_decode's bitwise (and so meet the
oracle's bar). Two calls in a row share that scratch, the second with a smaller
input; fused and two-kernel calls both start from whatever the previous call
left there. A call whose states do not fit is rejected before any launch.
"""
import ctypes
import math

import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import assert_parity, check_append_k, okv, oracle_decode, to_dev
from synth import BF16, F16, append_case, contiguous_case, paged_case, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


def _noalloc(lib, d, case, S, fused, append=None):
    kv = F.make_kv(d["k"], d["v"], d["page_table"], d["k_descale"], d["v_descale"], d["cache_batch_idx"],
                   d["cache_leftpad"])
    out = torch.full((case.B, case.Hq, case.D), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((case.B, case.Hq), float("nan"), dtype=torch.float32, device="cuda")
    rc = lib.fdec_decode_noalloc(d["q"].data_ptr(), case.B, case.Hq, ctypes.byref(kv), d["seq_lens"].data_ptr(), S,
                                 0.0, ctypes.byref(append) if append is not None else None, int(fused),
                                 out.data_ptr(), lse.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, lib.fdec_last_error()
    return out, lse


def _workspace_call(d, case, S, fused, append=None):
    return F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=S, fused=fused,
                    append=append, k_descale=d["k_descale"], v_descale=d["v_descale"],
                    cache_batch_idx=d["cache_batch_idx"], cache_leftpad=d["cache_leftpad"])


@pytest.mark.parametrize("fused", [False, True])
def test_two_calls_in_a_row_match_fdec_decode(fused):
    lib = F.load_library()
    # a large call first (the 128k-token GQA request, 128 splits: 2 MB of states),
    # then a smaller paged batch, then a smaller still contiguous MHA call
    calls = [
        (workload("c2"), 128),
        (paged_case(401, 5, 32, 8, 128, [3000, 17, 0, 900, 2048], 16, BF16, extra_pages=3, pad="nan"), 7),
        (contiguous_case(402, 2, 8, 8, 64, [300, 41], 512, F16, pad="nan"), 3),
    ]
    for i, (case, S) in enumerate(calls):
        d = to_dev(case)
        o_n, l_n = _noalloc(lib, d, case, S, fused)
        o_w, l_w = _workspace_call(d, case, S, fused)
        torch.cuda.synchronize()
        assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w), f"call {i} ({case.name}) fused={fused}"
        if i > 0:  # the small calls against the oracle too
            ref_out, ref_lse = oracle_decode(case)
            assert_parity(o_n, l_n, ref_out, ref_lse, case.dtype, f"no-alloc call {i}")


def test_fused_after_two_kernel_calls_and_back():
    """The counters start at zero for a fused call whatever the previous calls left
    in the scratch (here: two-kernel states of a larger call over the same bytes)."""
    lib = F.load_library()
    big = paged_case(403, 8, 32, 8, 128, [4000] * 8, 16, BF16, extra_pages=2, pad="nan")
    small = paged_case(404, 3, 32, 8, 128, [1000, 5, 2500], 16, BF16, extra_pages=2, pad="nan")
    db, ds = to_dev(big), to_dev(small)
    for fused_big, fused_small in ((False, True), (True, False), (True, True)):
        _noalloc(lib, db, big, 40, fused_big)
        o_n, l_n = _noalloc(lib, ds, small, 9, fused_small)
        o_w, l_w = _workspace_call(ds, small, 9, False)
        torch.cuda.synchronize()
        assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w), (fused_big, fused_small)


def test_append_through_no_alloc_matches_fdec_decode():
    lib = F.load_library()
    case = append_case(405, 3, 32, 8, 128, 600, F16, rotary_dim=128, pad="nan", cache_seqlens=[0, 301, 599])
    d1, d2 = to_dev(case), to_dev(case)
    a1 = F.make_append(d1["k_new"], d1["v_new"], d1["rope_cos"], d1["rope_sin"], case.rotary_dim)
    a2 = F.make_append(d2["k_new"], d2["v_new"], d2["rope_cos"], d2["rope_sin"], case.rotary_dim)
    o_n, l_n = _noalloc(lib, d1, case, 5, False, a1)
    o_w, l_w = _workspace_call(d2, case, 5, False, a2)
    torch.cuda.synchronize()
    assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w)
    # the caches (NaN padding included) bitwise: both calls wrote the same rows
    assert torch.equal(d1["k"].view(torch.int16), d2["k"].view(torch.int16))
    assert torch.equal(d1["v"].view(torch.int16), d2["v"].view(torch.int16))
    kc, vc, q_rot, after = oracle.append(okv(case), case.k_new, case.v_new, case.q, case.seq_lens, case.rotary_dim,
                                         case.rope_base)
    ref_out, ref_lse = oracle.decode(after, q_rot, case.seq_lens + 1, 1 / math.sqrt(case.D))
    check_append_k(d1["k"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16), kc, case, "no-alloc")
    assert_parity(o_n, l_n, ref_out, ref_lse, case.dtype, "no-alloc append")


def test_too_large_for_the_scratch_is_rejected():
    lib = F.load_library()
    case = contiguous_case(406, 64, 64, 8, 128, [16] * 64, 16, BF16)
    d = to_dev(case)
    kv = F.make_kv(d["k"], d["v"])
    out = torch.zeros(case.B, case.Hq, case.D, dtype=torch.float32, device="cuda")
    rc = lib.fdec_decode_noalloc(d["q"].data_ptr(), case.B, case.Hq, ctypes.byref(kv), d["seq_lens"].data_ptr(), 256,
                                 0.0, None, 0, out.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert rc == F.FDEC_ERR_WORKSPACE
    assert b"scratch" in lib.fdec_last_error()
    torch.cuda.synchronize()
    assert int(out.abs().sum()) == 0  # nothing launched
