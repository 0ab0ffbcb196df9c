"""Balanced split (fdec_decode_balanced) against the fp64 oracle, through the C ABI.

The tiles of all requests are cut into equal ranges whatever the length mix,
so the cases mix very long and very short requests, empty requests, more
blocks than tiles, one block for everything, and both cache layouts.
"""
import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import assert_parity, oracle_decode, to_dev
from synth import BF16, F16, FP8, contiguous_case, paged_case, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


def run(case, num_blocks):
    d = to_dev(case)
    out, lse = F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                                 num_blocks=num_blocks, k_descale=d["k_descale"], v_descale=d["v_descale"])
    torch.cuda.synchronize()
    return out, lse


CASES = [
    ("contig_mixed_bf16", lambda: contiguous_case(81, 5, 16, 4, 128, [3000, 1, 0, 17, 700], 3072, BF16, pad="nan")),
    ("paged16_mixed_f16", lambda: paged_case(82, 6, 32, 8, 128, [2500, 0, 33, 16, 1, 900], 16, F16, extra_pages=5,
                                             pad="nan")),
    ("paged48_bf16", lambda: paged_case(83, 3, 8, 2, 128, [481, 48, 1000], 48, BF16, extra_pages=2, pad="nan")),
    ("many_short_f16", lambda: contiguous_case(84, 70, 4, 1, 128, [(7 * i) % 53 for i in range(70)], 64, F16,
                                               pad="nan")),
    ("all_empty_bf16", lambda: contiguous_case(85, 3, 8, 2, 128, [0, 0, 0], 32, BF16, pad="nan")),
    # groups of eight query heads per KV head
    ("g8_paged16_bf16", lambda: paged_case(87, 5, 64, 8, 128, [2500, 0, 33, 1, 900], 16, BF16, extra_pages=3,
                                           pad="nan")),
    ("g8_contig_f16", lambda: contiguous_case(88, 3, 16, 2, 128, [1000, 17, 2000], 2048, F16, pad="nan")),
    ("g8_paged32_fp8", lambda: paged_case(89, 4, 32, 4, 128, [700, 64, 0, 1500], 32, FP8, extra_pages=2,
                                          pad="nan")),
]


@pytest.mark.parametrize("name,builder", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("num_blocks", [1, 3, 64, 256, 0])
def test_balanced_matches_oracle(name, builder, num_blocks):
    case = builder()
    ref_out, ref_lse = oracle_decode(case)
    out, lse = run(case, num_blocks)
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{name} blocks={num_blocks}")


def test_balanced_repeats_bitwise_and_agrees_with_uniform_splits():
    case = paged_case(86, 8, 32, 8, 128, None, 16, BF16, max_pages=128, pad="nan", lens_range=(1, 2048))
    o1, l1 = run(case, 0)
    o2, l2 = run(case, 0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    d = to_dev(case)
    ou, lu = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=8)
    torch.cuda.synchronize()
    assert (o1 - ou).abs().max().item() < 1e-5
    assert ((l1 - lu).abs() / lu.abs().clamp(min=1)).max().item() < 1e-6


@pytest.mark.parametrize("name", ["c2", "c3", "c2g8"])
def test_balanced_full_size_workloads(name):
    case = workload(name, pad="nan")
    ref_out, ref_lse = oracle_decode(case)
    out, lse = run(case, 0)
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{name} balanced")


def test_balanced_graph_replay_follows_new_lengths():
    # the ranges come from seq_lens on the device, so one captured graph serves
    # every length mix; each replay is checked against the oracle
    # every request owns pages for 1279 tokens, so any length up to that is in bounds
    case = paged_case(87, 4, 16, 4, 128, [1279] * 4, 16, BF16, max_pages=80, extra_pages=2, pad="nan")
    assert int((case.page_table >= 0).sum(dim=1).min()) * 16 >= 1279
    d = to_dev(case)
    out = torch.empty(4, 16, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(4, 16, dtype=torch.float32, device="cuda")
    ws = F.Workspace(F.balanced_workspace_size(4, 16, 4, 128, 32), torch.device("cuda"))
    lens_dev = d["seq_lens"].clone()
    F.decode_balanced(d["q"], d["k"], d["v"], lens_dev, page_table=d["page_table"], num_blocks=32, out=out,
                      lse=lse, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            F.decode_balanced(d["q"], d["k"], d["v"], lens_dev, page_table=d["page_table"], num_blocks=32,
                              out=out, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    for lens in ([1000, 10, 400, 777], [5, 1270, 0, 64], [1279, 1, 1, 1], [1000, 10, 400, 777]):
        lens_dev.copy_(torch.tensor(lens, dtype=torch.int32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        case.seq_lens = torch.tensor(lens, dtype=torch.int32)
        ref_out, ref_lse = oracle_decode(case)
        assert_parity(out.clone(), lse.clone(), ref_out, ref_lse, case.dtype, f"graph replay lens={lens}")


@pytest.mark.parametrize("first", ["balanced", "multi_balanced", "cascade"])
def test_shared_workspace_keeps_fused_counters(first):
    """A workspace used by a balanced-split call (whose per-request records are
    device metadata) then serves a fused fdec_decode unchanged: the fused
    output equals the two-kernel output bitwise, and the arrival counters are
    back at zero afterwards."""
    case = paged_case(91, 4, 32, 8, 128, [1500, 3, 700, 64], 16, BF16, extra_pages=2, pad="nan")
    d = to_dev(case)
    S = 6
    size = max(F.workspace_size(case.B, case.Hq, case.Hkv, 128, S),
               F.balanced_workspace_size(case.B, case.Hq, case.Hkv, 128, 0),
               F.balanced_workspace_size(case.B, 2 * case.Hq, case.Hkv, 128, 0),
               F.cascade_workspace_size(case.B, case.Hq, case.Hkv, 128, 4, 4))
    ws = F.Workspace(size)
    if first == "balanced":
        F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], workspace=ws)
    elif first == "multi_balanced":
        q2 = torch.cat([d["q"][:, None], d["q"][:, None]], 1).contiguous()
        F.decode_multi_balanced(q2, d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], workspace=ws)
    else:
        F.cascade_decode(d["q"], d["k"], d["v"], d["page_table"], d["page_table"][0], 32, d["seq_lens"],
                         splits_prefix=4, splits_suffix=4, workspace=ws)
    o_f, l_f = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=S,
                        fused=True, workspace=ws)
    o_2, l_2 = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=S)
    torch.cuda.synchronize()
    assert torch.equal(o_f, o_2) and torch.equal(l_f, l_2)
    counters = ws.buf[: case.B * case.Hkv * 4].view(torch.int32)
    assert int(counters.abs().sum()) == 0
    ref_out, ref_lse = oracle_decode(case)
    assert_parity(o_f, l_f, ref_out, ref_lse, case.dtype, f"fused after {first}")


@pytest.mark.parametrize("lens,nb", [([3000, 1, 0, 17, 700], 64), ([0] * 3 + [5000], 7),
                                     ([(13 * i) % 400 for i in range(70)], 256), ([1600], 1),
                                     ([100] * 9, 3)])
def test_device_records_follow_the_partition_rule(lens, nb):
    """The (first slot, piece count) records the kernel writes per request equal the
    partition rule that tests/test_balanced_partition.py checks on the CPU, so that
    check pins the device code."""
    from test_balanced_partition import partition

    B = len(lens)
    case = contiguous_case(93, B, 16, 4, 128, lens, max(max(lens), 1), BF16, pad="nan")
    d = to_dev(case)
    ws = F.Workspace(F.balanced_workspace_size(B, case.Hq, case.Hkv, 128, nb))
    ws.buf.fill_(0x7f)  # records the kernel does not write would show up
    F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], num_blocks=nb, workspace=ws)
    torch.cuda.synchronize()
    off = (B * case.Hkv * 4 + 255) // 256 * 256  # after the fused path's counters
    got = ws.buf[off: off + 8 * B].view(torch.int32).cpu().view(B, 2).tolist()
    meta, _ = partition(lens, nb)
    assert [tuple(x) for x in got] == [meta[j] for j in range(B)]
