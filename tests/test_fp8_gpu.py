"""Float8 (e4m3fn) KV caches against the fp64 oracle, through the C ABI.

The pages' FP8 KV cache: K and V stored as float8 e4m3fn with one fp32 descale
per (request, KV head) each, queries in bf16. Each case runs the uniform splits
(two kernels and the single-kernel merge), the map stage alone and the balanced
split, on the matrix-core map kernel (G = 4, 8 at head_dim 128) and on the
vector one (every other shape); padding rows and unused pages hold NaN.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import assert_parity, check_fp8_append, okv, oracle_decode, to_dev
from synth import FP8, append_case, contiguous_case, paged_case, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


CASES = [
    ("contig_tail", lambda: contiguous_case(91, 4, 16, 4, 128, [1, 15, 17, 1000], 1024, FP8, pad="nan")),
    ("contig_empty", lambda: contiguous_case(92, 3, 32, 8, 128, [0, 33, 0], 64, FP8, pad="nan")),
    ("paged16", lambda: paged_case(93, 4, 16, 4, 128, [16, 31, 500, 2], 16, FP8, extra_pages=4, pad="nan")),
    ("paged32", lambda: paged_case(94, 3, 32, 8, 128, [64, 95, 1500], 32, FP8, extra_pages=3, pad="nan")),
    ("paged48", lambda: paged_case(95, 3, 8, 2, 128, [48, 49, 480], 48, FP8, extra_pages=2, pad="nan")),
]


def run(case, num_splits=0, fused=False, descales=True):
    d = to_dev(case)
    kd, vd = (d["k_descale"], d["v_descale"]) if descales else (None, None)
    out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                        num_splits=num_splits, fused=fused, k_descale=kd, v_descale=vd)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("name,builder", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("num_splits", [1, 5, 32, 0])
def test_fp8_decode_matches_oracle(name, builder, num_splits):
    case = builder()
    ref_out, ref_lse = oracle_decode(case)
    for fused in (False, True):
        out, lse = run(case, num_splits, fused)
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{name} S={num_splits} fused={fused}")


@pytest.mark.parametrize("name,builder", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("num_blocks", [1, 3, 64, 0])
def test_fp8_balanced_matches_oracle(name, builder, num_blocks):
    case = builder()
    ref_out, ref_lse = oracle_decode(case)
    d = to_dev(case)
    out, lse = F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                                 num_blocks=num_blocks, k_descale=d["k_descale"], v_descale=d["v_descale"])
    torch.cuda.synchronize()
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{name} blocks={num_blocks}")


def test_fp8_without_descales_means_unit_descales():
    case = paged_case(96, 2, 8, 2, 128, [300, 77], 16, FP8, extra_pages=1, pad="nan")
    out, lse = run(case, 4, descales=False)
    case.k_descale = torch.ones_like(case.k_descale)
    case.v_descale = torch.ones_like(case.v_descale)
    ref_out, ref_lse = oracle_decode(case)
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, "unit descales")


def test_fp8_map_stage_states_match_oracle_states():
    lens = [1, 33, 300, 1000]
    case = contiguous_case(97, 4, 16, 4, 128, lens, 1024, FP8, pad="nan")
    S = 7
    d = to_dev(case)
    po, pm, pd = F.decode_partials(d["q"], d["k"], d["v"], d["seq_lens"], S, k_descale=d["k_descale"],
                                   v_descale=d["v_descale"])
    torch.cuda.synchronize()
    chunk = F.split_chunk(case.capacity, S)
    bounds = np.array([[min(i * chunk, case.capacity) for i in range(S + 1)]] * 4, dtype=np.int32)
    rpo, rpm, rpd = oracle.partials(okv(case), case.q, case.seq_lens, 1 / math.sqrt(128), bounds)
    gpo, gpm, gpd = (t.cpu().double().numpy() for t in (po, pm, pd))
    fin = np.isfinite(rpm)
    assert np.array_equal(np.isfinite(gpm), fin)
    assert np.all(gpd[~fin] == 0) and np.all(gpo[~fin] == 0)
    np.testing.assert_allclose(gpm[fin], rpm[fin], rtol=0, atol=1e-5 * np.abs(rpm[fin]).max() + 1e-5)
    np.testing.assert_allclose(gpd[fin], rpd[fin], rtol=1e-4)
    err = np.abs(gpo - rpo)[fin] / rpd[fin][:, None]
    assert err.max() < 1e-3


@pytest.mark.parametrize("name,mode", [("c2f8", "two"), ("c3f8", "bal"), ("c3f8", "two"), ("c1f8", "two"),
                                       ("c2g2f8", "two")])
def test_fp8_full_size_workloads(name, mode):
    case = workload(name, pad="nan")
    ref_out, ref_lse = oracle_decode(case)
    d = to_dev(case)
    if mode == "bal":
        out, lse = F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                                     k_descale=d["k_descale"], v_descale=d["v_descale"])
    else:
        B, Hq, _ = case.q.shape
        S = F.plan(B, Hq, case.Hkv, case.seq_lens.tolist(), case.capacity, case.page_size, kv_dtype=case.dtype)
        out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=S,
                            k_descale=d["k_descale"], v_descale=d["v_descale"])
    torch.cuda.synchronize()
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{name} {mode}")


# the vector map kernel: group sizes and head dims the matrix-core kernel does
# not take, and G = 4 / 8 forced onto it
VECTOR_CASES = [
    ("g1_contig_d128", lambda: contiguous_case(110, 3, 8, 8, 128, [1, 300, 1000], 1024, FP8, pad="nan")),
    ("g2_paged16_d128", lambda: paged_case(111, 4, 16, 8, 128, [16, 31, 500, 0], 16, FP8, extra_pages=4,
                                           pad="nan")),
    ("g2_paged32_d64", lambda: paged_case(112, 3, 8, 4, 64, [64, 95, 777], 32, FP8, extra_pages=3, pad="nan")),
    ("g8_contig_d64", lambda: contiguous_case(113, 2, 16, 2, 64, [17, 600], 640, FP8, pad="nan")),
    ("g1_paged48_d64", lambda: paged_case(114, 2, 4, 4, 64, [48, 481], 48, FP8, extra_pages=2, pad="nan")),
]


@pytest.mark.parametrize("name,builder", VECTOR_CASES, ids=[c[0] for c in VECTOR_CASES])
@pytest.mark.parametrize("num_splits", [1, 5, 0])
def test_fp8_vector_kernel_matches_oracle(name, builder, num_splits):
    case = builder()
    ref_out, ref_lse = oracle_decode(case)
    for fused in (False, True):
        out, lse = run(case, num_splits, fused)
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{name} S={num_splits} fused={fused}")


@pytest.mark.parametrize("G", [4, 8])
def test_fp8_matrix_core_shapes_on_the_vector_kernel(G, monkeypatch):
    case = paged_case(115 + G, 3, 2 * G, 2, 128, [33, 400, 1000], 16, FP8, extra_pages=2, pad="nan")
    ref_out, ref_lse = oracle_decode(case)
    mo, ml = run(case, 6)
    monkeypatch.setenv("FDEC_MAP_PATH", "vector")
    vo, vl = run(case, 6)
    assert_parity(vo, vl, ref_out, ref_lse, case.dtype, f"G={G} vector kernel")
    assert (vo - mo).abs().max().item() < 1e-4


def test_fp8_vector_kernel_states_match_oracle_states():
    lens = [1, 33, 300, 1000]
    case = contiguous_case(119, 4, 8, 4, 128, lens, 1024, FP8, pad="nan")  # G = 2
    S = 7
    d = to_dev(case)
    po, pm, pd = F.decode_partials(d["q"], d["k"], d["v"], d["seq_lens"], S, k_descale=d["k_descale"],
                                   v_descale=d["v_descale"])
    torch.cuda.synchronize()
    chunk = F.split_chunk(case.capacity, S)
    bounds = np.array([[min(i * chunk, case.capacity) for i in range(S + 1)]] * 4, dtype=np.int32)
    rpo, rpm, rpd = oracle.partials(okv(case), case.q, case.seq_lens, 1 / math.sqrt(128), bounds)
    gpo, gpm, gpd = (t.cpu().double().numpy() for t in (po, pm, pd))
    fin = np.isfinite(rpm)
    assert np.array_equal(np.isfinite(gpm), fin)
    assert np.all(gpd[~fin] == 0) and np.all(gpo[~fin] == 0)
    np.testing.assert_allclose(gpm[fin], rpm[fin], rtol=0, atol=1e-5 * np.abs(rpm[fin]).max() + 1e-5)
    np.testing.assert_allclose(gpd[fin], rpd[fin], rtol=1e-4)
    err = np.abs(gpo - rpo)[fin] / rpd[fin][:, None]
    assert err.max() < 1e-3


def test_fp8_balanced_split_at_g1_g2():
    """One query token at G = 1 and 2 on the balanced split: the 16x16x32 kernel
    (float8 tiles), its 16-row block padded, against the oracle."""
    for G in (1, 2):
        case = paged_case(98 + G, 7, 8 * G, 8, 128, [40, 0, 3000, 1, 777, 64, 65], 16, FP8, extra_pages=2,
                          pad="nan")
        d = to_dev(case)
        ref_out, ref_lse = oracle_decode(case)
        for nb in (1, 5, 0):
            out, lse = F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                                         num_blocks=nb, k_descale=d["k_descale"], v_descale=d["v_descale"])
            torch.cuda.synchronize()
            assert_parity(out, lse, ref_out, ref_lse, FP8, f"float8 balanced G={G} nb={nb}")


# ---------------------------------------------------------------- append into a float8 cache
# ("Inference Cookbook / 推理优化" §3.3-3.4 append and rotary, §7.2 FP8 KV cache:
# the new row is stored as codes of value / descale, then attended to)

@pytest.mark.parametrize("G,rd,paged,S,fused", [
    (1, 128, False, 4, False), (2, 0, True, 3, True), (4, 128, True, 7, False), (4, 64, False, 1, True),
    (8, 128, False, 5, False), (8, 0, True, 2, True), (2, 128, False, 32, False)])
def test_fp8_append_matches_oracle(G, rd, paged, S, fused):
    case = append_case(181 + G + rd, 3, 2 * G, 2, 128, 300, FP8, rotary_dim=rd, pad="nan",
                       page_size=16 if paged else 0, cache_seqlens=[0, 150, 299])
    check_fp8_append(case, S, fused, f"fp8 append G={G} rd={rd} paged={paged} S={S}")


def test_fp8_append_head_dim_64():
    case = append_case(188, 3, 8, 2, 64, 300, FP8, rotary_dim=64, pad="nan", cache_seqlens=[5, 150, 298])
    check_fp8_append(case, 3, False, "fp8 append D=64")


def test_fp8_append_with_batch_idx_and_leftpad():
    case = append_case(189, 3, 8, 2, 128, 256, FP8, rotary_dim=128, pad="zero", cache_seqlens=[40, 0, 255])
    case.cache_batch_idx = torch.tensor([2, 0, 1], dtype=torch.int32)
    case.cache_leftpad = torch.tensor([7, 0, 100], dtype=torch.int32)
    check_fp8_append(case, 4, False, "fp8 append batch_idx + leftpad")


def test_fp8_append_at_the_append_workload_size():
    # the append + rotary workload's shapes (4 requests, 32 query heads, 8 KV
    # heads, 2048 rows, rotary 128) with a float8 cache
    case = append_case(4, 4, 32, 8, 128, 2048, FP8, rotary_dim=128, pad="nan")
    n_off = check_fp8_append(case, 0, False, "fp8 append workload")
    assert n_off <= 2
