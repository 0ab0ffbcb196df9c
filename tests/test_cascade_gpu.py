"""GPU parity of the cascade path (shared prefix on matrix cores + suffix
split-KV + merge) against the fp64 oracle over [prefix; suffix]."""
import math

import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import assert_cascade_parity, assert_parity, oracle_decode, to_dev
from synth import BF16, F16, FP8, cascade_case, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)


def run_cascade(case, sp=0, ss=0, scale=0.0):
    d = to_dev(case)
    out, lse = F.cascade_decode(d["q"], d["k"], d["v"], d["page_table"], d["prefix_pages"], case.prefix_len,
                                d["seq_lens"], sp, ss, softmax_scale=scale, k_descale=d["k_descale"],
                                v_descale=d["v_descale"])
    torch.cuda.synchronize()
    return out, lse


CASES = [
    ("ragged_bf16_g4", lambda: cascade_case(71, 3, 16, 4, 128, prefix_len=100, ps=16, suffix_lens=[0, 5, 40],
                                            dtype=BF16, pad="nan", extra_pages=2)),
    ("ragged_f16_g4", lambda: cascade_case(72, 3, 16, 4, 128, prefix_len=333, ps=16, suffix_lens=[17, 1, 64],
                                           dtype=F16, pad="nan", extra_pages=2)),
    ("g1_ps64", lambda: cascade_case(73, 2, 8, 8, 128, prefix_len=700, ps=64, suffix_lens=[100, 300],
                                     dtype=BF16, pad="nan")),
    ("g8_ps32", lambda: cascade_case(74, 5, 16, 2, 128, prefix_len=512, ps=32, suffix_lens=[31, 32, 33, 0, 5],
                                     dtype=F16, pad="nan")),
    ("rows_over_256", lambda: cascade_case(75, 70, 8, 2, 128, prefix_len=200, ps=16, suffix_range=(0, 40),
                                           dtype=BF16, pad="nan")),
    ("empty_prefix", lambda: cascade_case(76, 3, 8, 2, 128, prefix_len=0, ps=16, suffix_lens=[10, 0, 70],
                                          dtype=BF16, pad="nan")),
    # float8 pools (the pages' FP8 KV cache): the prefix kernel's float8 tiles,
    # the suffix on the balanced split (G = 4) or the uniform map kernels
    ("fp8_ragged_g4", lambda: cascade_case(78, 3, 16, 4, 128, prefix_len=100, ps=16, suffix_lens=[0, 5, 40],
                                           dtype=FP8, pad="nan", extra_pages=2)),
    ("fp8_g1_ps64", lambda: cascade_case(79, 2, 8, 8, 128, prefix_len=700, ps=64, suffix_lens=[100, 300],
                                         dtype=FP8, pad="nan")),
    ("fp8_g8_ps32", lambda: cascade_case(80, 5, 16, 2, 128, prefix_len=512, ps=32, suffix_lens=[31, 32, 33, 0, 5],
                                         dtype=FP8, pad="nan")),
    ("fp8_rows_over_256", lambda: cascade_case(81, 70, 8, 2, 128, prefix_len=333, ps=16, suffix_range=(0, 40),
                                               dtype=FP8, pad="nan")),
    ("fp8_g2", lambda: cascade_case(82, 4, 8, 4, 128, prefix_len=129, ps=48, suffix_lens=[1, 2, 100, 47],
                                    dtype=FP8, pad="nan")),
]


@pytest.mark.parametrize("name,builder", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("sp,ss", [(1, 1), (3, 2), (0, 0)])
def test_cascade_matches_oracle(name, builder, sp, ss):
    case = builder()
    ref_out, ref_lse = oracle_decode(case)
    out, lse = run_cascade(case, sp, ss)
    assert_cascade_parity(case, out, lse, ref_out, ref_lse, f"{name} sp={sp} ss={ss}")


def test_cascade_equals_plain_decode_over_concatenated_pages():
    case = cascade_case(77, 4, 32, 8, 128, prefix_len=256, ps=16, suffix_lens=[5, 100, 16, 0], dtype=BF16,
                        pad="nan")
    out_c, lse_c = run_cascade(case, 2, 2)
    n_pre = case.prefix_pages.numel()
    table = torch.full((4, n_pre + case.page_table.shape[1]), -1, dtype=torch.int32)
    for b in range(4):
        table[b, :n_pre] = case.prefix_pages
        table[b, n_pre:] = case.page_table[b]
    d = to_dev(case)
    out_p, lse_p = F.decode(d["q"], d["k"], d["v"], (case.seq_lens + 256).to("cuda"), page_table=table.cuda(),
                            num_splits=4)
    torch.cuda.synchronize()
    assert (out_c - out_p).abs().max().item() < 3e-3
    assert ((lse_c - lse_p).abs() / lse_p.abs().clamp(min=1)).max().item() < 1e-4


def test_cascade_full_workload():
    case = workload("c5", pad="nan")
    ref_out, ref_lse = oracle_decode(case)
    out, lse = run_cascade(case)
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, "c5")


def test_fp8_cascade_full_workload():
    case = workload("c5f8", pad="nan")
    ref_out, ref_lse = oracle_decode(case)
    out, lse = run_cascade(case)
    assert_cascade_parity(case, out, lse, ref_out, ref_lse, "c5f8")


@pytest.mark.parametrize("sp,ss", [(1, 1), (3, 2)])
@pytest.mark.parametrize("suffix", [True, False])
def test_fp8_cascade_is_bitwise_the_bf16_cascade_on_the_same_values(sp, ss, suffix):
    # descales 1/32 (a power of two): code / 32 is exact in bf16, the score scale and
    # the state scale change by a power of two only, so the matrix cores see the same
    # operands and the float8 pool gives the bf16 pool's bits
    case = cascade_case(81, 70, 8, 2, 128, prefix_len=333, ps=16, suffix_range=(0, 40),
                        suffix_lens=None if suffix else [0] * 70, dtype=FP8, pad="zero")
    case.k_descale = torch.full((70, 2), 1.0 / 32)
    case.v_descale = case.k_descale.clone()
    o8, l8 = run_cascade(case, sp, ss)
    bf = cascade_case(81, 70, 8, 2, 128, prefix_len=333, ps=16, suffix_range=(0, 40),
                      suffix_lens=None if suffix else [0] * 70, dtype=FP8, pad="zero")
    bf.k = (case.k.to(torch.float32) / 32).to(BF16)
    bf.v = (case.v.to(torch.float32) / 32).to(BF16)
    assert torch.equal(bf.k.to(torch.float32) * 32, case.k.to(torch.float32))
    bf.k_descale = bf.v_descale = None
    bf.dtype = BF16
    ob, lb = run_cascade(bf, sp, ss)
    assert torch.equal(o8, ob) and torch.equal(l8, lb)


def test_fp8_cascade_equals_fp8_decode_over_concatenated_pages():
    case = cascade_case(83, 4, 32, 8, 128, prefix_len=256, ps=16, suffix_lens=[5, 100, 16, 0], dtype=FP8,
                        pad="nan")
    out_c, lse_c = run_cascade(case, 2, 2)
    n_pre = case.prefix_pages.numel()
    table = torch.full((4, n_pre + case.page_table.shape[1]), -1, dtype=torch.int32)
    for b in range(4):
        table[b, :n_pre] = case.prefix_pages
        table[b, n_pre:] = case.page_table[b]
    d = to_dev(case)
    out_p, lse_p = F.decode(d["q"], d["k"], d["v"], (case.seq_lens + 256).to("cuda"), page_table=table.cuda(),
                            num_splits=4, k_descale=d["k_descale"], v_descale=d["v_descale"])
    torch.cuda.synchronize()
    assert (out_c - out_p).abs().max().item() < 3e-3
    assert ((lse_c - lse_p).abs() / lse_p.abs().clamp(min=1)).max().item() < 1e-4


@pytest.mark.parametrize("dtype", [BF16, F16, FP8])
@pytest.mark.parametrize("B,Hkv,sp,ss", [(5, 4, 3, 7), (70, 8, 0, 0), (33, 8, 2, 130)])
def test_single_launch_is_bitwise_the_two_launches(monkeypatch, dtype, B, Hkv, sp, ss):
    """With G = 4 and Hkv a multiple of 4 the prefix and suffix blocks share one
    launch; each query row's prefix state is computed the same way in a 4-wave
    block as in the 8-wave prefix kernel, and the suffix blocks are the balanced
    kernel's, so at the same split counts the outputs are bit for bit those of
    the two launches (FDEC_CASCADE_PATH=two). Row counts that are not multiples
    of 128 (20, 132) leave partly empty prefix blocks; 130 suffix blocks per
    group of KV heads exceed one per compute unit."""
    case = cascade_case(400 + B, B, 4 * Hkv, Hkv, 128, 900, 64, suffix_range=(0, 300), dtype=dtype, pad="nan",
                        extra_pages=2)
    d = to_dev(case)
    if sp == 0:
        sp, ss = F.cascade_plan(B, 4 * Hkv, Hkv, case.prefix_len, case.capacity, 64, kv_dtype=dtype)

    def run():
        out, lse = F.cascade_decode(d["q"], d["k"], d["v"], d["page_table"], d["prefix_pages"], case.prefix_len,
                                    d["seq_lens"], sp, ss, k_descale=d["k_descale"], v_descale=d["v_descale"])
        torch.cuda.synchronize()
        return out, lse

    monkeypatch.delenv("FDEC_CASCADE_PATH", raising=False)
    o1, l1 = run()
    monkeypatch.setenv("FDEC_CASCADE_PATH", "two")
    o2, l2 = run()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"B={B} Hkv={Hkv} sp={sp} ss={ss}"
    ref_out, ref_lse = oracle_decode(case)
    assert_cascade_parity(case, o1, l1, ref_out, ref_lse, f"single launch B={B} Hkv={Hkv}")


@pytest.mark.parametrize("dtype", [BF16, FP8])
def test_cascade_many_requests(dtype):
    """300 requests of G = 4 (1200 query rows per KV head, ten 128-row prefix
    chunks): the planned single launch then has fewer prefix splits than row
    chunks need for one block per compute unit, and more blocks of one role than
    the other."""
    case = cascade_case(431, 300, 32, 8, 128, 2048, 64, suffix_range=(0, 64), dtype=dtype, pad="nan",
                        extra_pages=2)
    # 192 (16-bit) or 256 (float8) prefix blocks at most, over 8 KV heads x 10 chunks
    sp, ss = F.cascade_plan(300, 32, 8, case.prefix_len, case.capacity, 64, kv_dtype=dtype)
    assert (sp, ss) == ((2 if dtype == BF16 else 3), 128)
    ref_out, ref_lse = oracle_decode(case)
    out, lse = run_cascade(case)
    assert_cascade_parity(case, out, lse, ref_out, ref_lse, f"300 requests {dtype}")


@pytest.mark.parametrize("name", ["c5", "c5f8"])
@pytest.mark.parametrize("sp,ss", [(32, 64), (24, 200), (1, 1)])
def test_single_launch_role_counts_bitwise(monkeypatch, name, sp, ss):
    """The full shared-prefix workloads with prefix and suffix block counts far
    apart (512 prefix blocks against 128 suffix blocks: whole runs of paired
    roles, then prefix blocks alone; 384 against 400; 16 against 2): the single
    launch equals the two launches bit for bit."""
    case = workload(name, pad="nan")
    monkeypatch.delenv("FDEC_CASCADE_PATH", raising=False)
    o1, l1 = run_cascade(case, sp, ss)
    monkeypatch.setenv("FDEC_CASCADE_PATH", "two")
    o2, l2 = run_cascade(case, sp, ss)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{name} sp={sp} ss={ss}"
    assert torch.isfinite(o1).all()
