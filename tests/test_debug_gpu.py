"""The device-data check (fdec_check_inputs) and the debug mode, through the C ABI.

Out-of-range device data (page ids past the pool, lengths past the capacity,
left padding past the length, cache rows past the cache, rotary positions past
the tables, prefix pages past the pool) only ever reaches the check kernel,
whose reads stay within the shapes the call declares, or a decode call in the
debug mode, which checks first and launches nothing; every valid case also
runs the decode itself, which must give the same bits with the mode on and off.
"""
import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import to_dev
from synth import BF16, F16, append_case, cascade_case, contiguous_case, paged_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    F.set_debug(False)


def _paged():
    return paged_case(201, 4, 16, 4, 128, [16, 31, 500, 2], 16, BF16, extra_pages=4, pad="nan")


def _check(case, d, **kw):
    return F.check_inputs(d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], **kw)


def test_valid_inputs_pass_the_check():
    for case in (_paged(), contiguous_case(202, 3, 8, 2, 128, [0, 7, 300], 300, F16, pad="nan")):
        d = to_dev(case)
        assert _check(case, d) == (0, -1)


def test_page_ids_out_of_the_pool_are_flagged():
    case = _paged()
    d = to_dev(case)
    pool = case.k.shape[0]
    for b, j, bad in ((2, 5, pool), (1, 1, -1), (3, 0, pool + 1000)):
        table = d["page_table"].clone()
        table[b, j] = bad
        flags, first = F.check_inputs(d["k"], d["v"], d["seq_lens"], page_table=table)
        assert flags == F.CHECK_PAGE and first == b, (b, j, bad)
    # an entry past the request's pages is never read: -1 (or anything) there is fine
    table = d["page_table"].clone()
    table[0, 5] = pool + 7
    assert F.check_inputs(d["k"], d["v"], d["seq_lens"], page_table=table) == (0, -1)


def test_lengths_leftpad_rows_and_positions_are_flagged():
    case = contiguous_case(203, 3, 8, 2, 128, [10, 20, 30], 64, BF16, pad="zero")
    d = to_dev(case)
    lens = torch.tensor([10, 65, 30], dtype=torch.int32, device="cuda")  # 65 > capacity 64
    assert F.check_inputs(d["k"], d["v"], lens) == (F.CHECK_LENGTH, 1)
    lens = torch.tensor([10, -1, 30], dtype=torch.int32, device="cuda")
    assert F.check_inputs(d["k"], d["v"], lens)[0] == F.CHECK_LENGTH
    lp = torch.tensor([0, 21, 0], dtype=torch.int32, device="cuda")  # past seq_lens[1] = 20
    assert F.check_inputs(d["k"], d["v"], d["seq_lens"], cache_leftpad=lp) == (F.CHECK_LEFTPAD, 1)
    idx = torch.tensor([0, 2, 3], dtype=torch.int32, device="cuda")  # the cache has rows 0..2
    assert F.check_inputs(d["k"], d["v"], d["seq_lens"], cache_batch_idx=idx) == (F.CHECK_BATCH_IDX, 2)
    # an append writes row seq_lens[b]: a full request has no room
    ap = append_case(204, 2, 8, 2, 128, 64, F16, rotary_dim=128, cache_seqlens=[63, 5])
    da = to_dev(ap)
    a = F.make_append(da["k_new"], da["v_new"], da["rope_cos"], da["rope_sin"], 128)
    assert F.check_inputs(da["k"], da["v"], da["seq_lens"], append=a) == (0, -1)
    full = torch.tensor([64, 5], dtype=torch.int32, device="cuda")  # (its position 64 is past the tables too)
    assert F.check_inputs(da["k"], da["v"], full, append=a) == (F.CHECK_LENGTH | F.CHECK_ROPE_POS, 0)
    # rotary tables shorter than the position
    short = F.make_append(da["k_new"], da["v_new"], da["rope_cos"][:10].contiguous(),
                          da["rope_sin"][:10].contiguous(), 128)
    assert F.check_inputs(da["k"], da["v"], da["seq_lens"], append=short) == (F.CHECK_ROPE_POS, 0)


def test_pages_below_the_left_padding_are_not_read():
    # request 2 (length 500, 32 pages) with 100 rows of left padding: its first tile
    # starts at row 96, on page 6; pages 0..5 are never read and may hold -1
    case = _paged()
    d = to_dev(case)
    table = d["page_table"].clone()
    table[2, :6] = -1
    lp = torch.tensor([0, 0, 100, 0], dtype=torch.int32, device="cuda")
    assert F.check_inputs(d["k"], d["v"], d["seq_lens"], page_table=table, cache_leftpad=lp) == (0, -1)
    table[2, 6] = -1  # the page holding row 96 is read
    assert F.check_inputs(d["k"], d["v"], d["seq_lens"], page_table=table, cache_leftpad=lp) == (F.CHECK_PAGE, 2)


def test_prefix_pages_are_flagged():
    case = cascade_case(205, 3, 16, 4, 128, prefix_len=100, ps=16, suffix_lens=[0, 5, 40], dtype=BF16,
                        pad="nan")
    d = to_dev(case)
    ok = F.check_inputs(d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], prefix_pages=d["prefix_pages"],
                        prefix_len=100)
    assert ok == (0, -1)
    bad = d["prefix_pages"].clone()
    bad[6] = case.k.shape[0]
    assert F.check_inputs(d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], prefix_pages=bad,
                          prefix_len=100) == (F.CHECK_PREFIX_PAGE, 3)


def test_debug_mode_refuses_bad_data_and_keeps_the_bits():
    case = _paged()
    d = to_dev(case)
    ref_out, ref_lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=5)
    torch.cuda.synchronize()
    F.set_debug(True)
    try:
        assert F.debug_enabled()
        out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=5)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        table = d["page_table"].clone()
        table[2, 7] = case.k.shape[0] + 3
        sentinel = torch.full_like(ref_out, 7.0)
        for fused in (False, True):
            with pytest.raises(F.FdecError) as e:
                F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=table, num_splits=5, fused=fused,
                         out=sentinel)
            assert e.value.status == F.FDEC_ERR_INVALID_ARG and "out of range" in str(e.value)
        with pytest.raises(F.FdecError):
            F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=table)
        torch.cuda.synchronize()
        assert torch.all(sentinel == 7.0)  # nothing ran
        # the cascade checks its shared prefix too
        cc = cascade_case(206, 3, 16, 4, 128, prefix_len=100, ps=16, suffix_lens=[0, 5, 40], dtype=BF16,
                          pad="nan")
        dc = to_dev(cc)
        bad = dc["prefix_pages"].clone()
        bad[0] = -5
        with pytest.raises(F.FdecError):
            F.cascade_decode(dc["q"], dc["k"], dc["v"], dc["page_table"], bad, 100, dc["seq_lens"])
    finally:
        F.set_debug(False)
    assert not F.debug_enabled()


def test_debug_mode_under_graph_capture():
    """The check waits for its result on the host, so a call made while its stream
    is capturing launches unchecked: the captured graph replays the eager result
    bit for bit, and the same call made eagerly is still checked."""
    case = _paged()
    d = to_dev(case)
    ws = F.Workspace(F.workspace_size(case.B, case.Hq, case.Hkv, case.D, 5), torch.device("cuda"))
    out = torch.empty(case.B, case.Hq, case.D, dtype=torch.float32, device="cuda")
    lse = torch.empty(case.B, case.Hq, dtype=torch.float32, device="cuda")

    def step(table):
        F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=table, num_splits=5, out=out, lse=lse,
                 workspace=ws)

    step(d["page_table"])
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    F.set_debug(True)
    try:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                step(d["page_table"])
        torch.cuda.synchronize()
        for _ in range(3):
            out.zero_()
            lse.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        table = d["page_table"].clone()
        table[2, 7] = case.k.shape[0] + 3
        with pytest.raises(F.FdecError):
            step(table)
    finally:
        F.set_debug(False)
