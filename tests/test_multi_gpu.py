"""Multi-token (speculative) decode on the GPU against the fp64 oracle, through the C ABI.

q_len query tokens per request share each KV tile; token i is the request's
row L - q_len + i and sees rows [leftpad, L - q_len + i]. Covered: q_len from
1 to 16 (one wave holds up to 4 tokens, more run as groups of 4), contiguous
and paged caches, every cache dtype, left padding and a cache row index,
requests shorter than q_len, the lse layout [B, Hq, q_len], q_len = 1 against
the single-query decode bitwise, and a full 128k-token request.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import OUT_TOL, LSE_RTOL, okv, to_dev
from synth import BF16, F16, FP8, contiguous_case, indexed_case, multi_query, pad_left, paged_case, workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


def check(out, lse, ref_out, ref_lse, dtype, what):
    o = out.cpu().double().numpy()
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ref_out).max()
    assert err <= OUT_TOL[dtype], f"{what}: max-abs out error {err:.3g}"
    l = lse.cpu().double().numpy()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: lse finiteness differs"
    assert np.all(l[~fin] == ref_lse[~fin])
    if fin.any():
        rel = (np.abs(l[fin] - ref_lse[fin]) / np.maximum(np.abs(ref_lse[fin]), 1.0)).max()
        assert rel <= LSE_RTOL, f"{what}: lse relative error {rel:.3g}"


def run(case, q, S, **extra):
    d = to_dev(case)
    out, lse = F.decode_multi(q.to("cuda"), d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                              num_splits=S, k_descale=d["k_descale"], v_descale=d["v_descale"],
                              cache_batch_idx=d["cache_batch_idx"], cache_leftpad=d["cache_leftpad"], **extra)
    torch.cuda.synchronize()
    return out, lse


LENS = [700, 3, 1, 64, 65, 2000]  # requests shorter than q_len, tile-edge lengths


@pytest.mark.parametrize("q_len", [1, 2, 3, 4, 5, 8, 16])
@pytest.mark.parametrize("kind", ["contig_bf16", "paged_f16", "paged_fp8"])
@pytest.mark.parametrize("S", [1, 5, 0])
def test_multi_token_matches_oracle(q_len, kind, S):
    if kind == "contig_bf16":
        case = contiguous_case(200 + q_len, 6, 16, 4, 128, LENS, 2048, BF16, pad="nan")
    elif kind == "paged_f16":
        case = paged_case(210 + q_len, 6, 16, 4, 128, LENS, 16, F16, extra_pages=3, pad="nan")
    else:
        case = paged_case(220 + q_len, 6, 16, 4, 128, LENS, 32, FP8, extra_pages=3, pad="nan")
    q = multi_query(230 + q_len, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    out, lse = run(case, q, S)
    assert out.shape == (6, q_len, 16, 128) and lse.shape == (6, 16, q_len)
    check(out, lse, ref_out, ref_lse, case.dtype, f"{kind} q_len={q_len} S={S}")


@pytest.mark.parametrize("q_len", [3, 6])
def test_multi_token_with_leftpad_and_batch_idx(q_len):
    lens, pads = [300, 40, 19, 1000], [5, 38, 17, 999]  # some tokens see only padding -> empty
    case = indexed_case(240, 4, 16, 4, 128, lens, pads, 1024, BF16, cache_rows=7)
    q = multi_query(241, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for S in (1, 4):
        out, lse = run(case, q, S)
        check(out, lse, ref_out, ref_lse, BF16, f"indexed q_len={q_len} S={S}")
    paged = pad_left(paged_case(242, 4, 16, 4, 128, lens, 16, F16, extra_pages=2, pad="nan"), pads)
    q = multi_query(243, paged, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(paged), q, paged.seq_lens, 1 / math.sqrt(128))
    out, lse = run(paged, q, 3)
    check(out, lse, ref_out, ref_lse, F16, f"paged leftpad q_len={q_len}")


@pytest.mark.parametrize("G,D,dt", [(4, 128, BF16), (1, 128, F16), (2, 128, BF16), (8, 128, BF16), (2, 64, F16),
                                    (1, 128, FP8)])
def test_one_token_equals_single_query_decode_bitwise(G, D, dt):
    # one query token runs fdec_decode's own map kernel, whichever it is for the shape
    case = paged_case(244 + G, 5, 8 * G, 8, D, [900, 1, 16, 0, 333], 16, dt, extra_pages=2, pad="nan")
    d = to_dev(case)
    kw = dict(k_descale=d["k_descale"], v_descale=d["v_descale"])
    for S in (1, 7):
        o1, l1 = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=S, **kw)
        om, lm = F.decode_multi(d["q"][:, None].contiguous(), d["k"], d["v"], d["seq_lens"],
                                page_table=d["page_table"], num_splits=S, **kw)
        torch.cuda.synchronize()
        assert torch.equal(om[:, 0], o1) and torch.equal(lm[:, :, 0], l1), f"G={G} D={D} S={S}"


@pytest.mark.parametrize("q_len", [2, 4])
def test_full_128k_request(q_len):
    case = workload("c2", pad="nan")
    q = multi_query(245, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    out, lse = run(case, q, 0)
    check(out, lse, ref_out, ref_lse, BF16, f"c2 q_len={q_len}")


@pytest.mark.parametrize("G,q_len", [(1, 1), (1, 3), (2, 2), (2, 5), (1, 11)])
def test_multi_token_few_rows_on_the_16x16x32_kernel(G, q_len):
    # fewer than 12 query rows per KV head pad the 16x16x32 kernel's row block
    case = paged_case(392 + G * 10 + q_len, 3, 4 * G, 4, 128, [700, 3, 1500], 16, F16, extra_pages=2, pad="nan")
    q = multi_query(393 + q_len, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for S in (1, 6):
        out, lse = run(case, q, S)
        check(out, lse, ref_out, ref_lse, F16, f"G={G} q_len={q_len} S={S}")
    out, lse = run_bal(case, q, 0) if q_len > 1 else (None, None)
    if out is not None:
        check(out, lse, ref_out, ref_lse, F16, f"G={G} q_len={q_len} balanced")


def test_multi_token_shapes_rejected():
    case = contiguous_case(246, 2, 16, 8, 64, [10, 20], 32, BF16)  # head_dim 64: no multi-token kernel
    q = multi_query(247, case, 2)
    with pytest.raises(F.FdecError) as e:
        run(case, q, 1)
    assert e.value.status == F.FDEC_ERR_UNSUPPORTED
    case = contiguous_case(248, 2, 16, 4, 128, [10, 20], 32, BF16)
    for bad in (17, 0):
        q = torch.zeros(2, max(bad, 1), 16, 128, dtype=BF16)
        if bad == 0:
            q = q[:, :0]
        with pytest.raises(F.FdecError) as e:
            run(case, q.contiguous(), 1)
        assert e.value.status == F.FDEC_ERR_INVALID_ARG


# ---------------------------------------------------------------- on the balanced split

def run_bal(case, q, nb):
    d = to_dev(case)
    out, lse = F.decode_multi_balanced(q.to("cuda"), d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                                       num_blocks=nb, k_descale=d["k_descale"], v_descale=d["v_descale"],
                                       cache_batch_idx=d["cache_batch_idx"], cache_leftpad=d["cache_leftpad"])
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("q_len", [1, 2, 3, 4, 6, 16])
@pytest.mark.parametrize("kind", ["contig_bf16", "paged_f16", "paged_fp8"])
def test_multi_token_balanced_matches_oracle(q_len, kind):
    if kind == "contig_bf16":
        case = contiguous_case(250 + q_len, 6, 16, 4, 128, LENS, 2048, BF16, pad="nan")
    elif kind == "paged_f16":
        case = paged_case(260 + q_len, 6, 16, 4, 128, LENS, 16, F16, extra_pages=3, pad="nan")
    else:
        case = paged_case(270 + q_len, 6, 16, 4, 128, LENS, 32, FP8, extra_pages=3, pad="nan")
    q = multi_query(280 + q_len, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for nb in (1, 3, 0):
        out, lse = run_bal(case, q, nb)
        check(out, lse, ref_out, ref_lse, case.dtype, f"balanced {kind} q_len={q_len} nb={nb}")


def test_multi_token_balanced_with_leftpad_and_batch_idx():
    lens, pads = [300, 40, 19, 1000], [5, 38, 17, 999]
    case = indexed_case(290, 4, 16, 4, 128, lens, pads, 1024, BF16, cache_rows=7)
    q = multi_query(291, case, 5)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for nb in (2, 0):
        out, lse = run_bal(case, q, nb)
        check(out, lse, ref_out, ref_lse, BF16, f"balanced indexed nb={nb}")


def test_multi_balanced_one_token_equals_balanced_bitwise():
    case = paged_case(292, 5, 32, 8, 128, [900, 1, 16, 0, 333], 16, BF16, extra_pages=2, pad="nan")
    d = to_dev(case)
    for nb in (3, 0):
        o1, l1 = F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_blocks=nb)
        om, lm = F.decode_multi_balanced(d["q"][:, None].contiguous(), d["k"], d["v"], d["seq_lens"],
                                         page_table=d["page_table"], num_blocks=nb)
        torch.cuda.synchronize()
        assert torch.equal(om[:, 0], o1) and torch.equal(lm[:, :, 0], l1), f"nb={nb}"


def test_multi_token_balanced_full_paged_batch():
    case = workload("c3", pad="nan")
    q = multi_query(293, case, 4)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    out, lse = run_bal(case, q, 0)
    check(out, lse, ref_out, ref_lse, BF16, "c3 q_len=4 balanced")


# ---------------------------------------------------------------- the 16x16x32 kernel (q_len * G >= 12)

@pytest.mark.parametrize("G,q_len", [(8, 2), (8, 5), (1, 12), (1, 16), (2, 6), (2, 16), (4, 16)])
@pytest.mark.parametrize("paged", [False, True])
def test_multi_token_any_group_size(G, q_len, paged):
    Hkv = 2 if G == 8 else 4
    lens = [700, 3, 1, 64, 65, 2000]
    if paged:
        case = paged_case(300 + G + q_len, 6, G * Hkv, Hkv, 128, lens, 32, F16, extra_pages=3, pad="nan")
    else:
        case = contiguous_case(310 + G + q_len, 6, G * Hkv, Hkv, 128, lens, 2048, BF16, pad="nan")
    q = multi_query(320 + G + q_len, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for S in (1, 5, 0):
        out, lse = run(case, q, S)
        check(out, lse, ref_out, ref_lse, case.dtype, f"G={G} q_len={q_len} paged={paged} S={S}")


@pytest.mark.parametrize("q_len", [3, 4, 8])
def test_multi_token_both_kernels_agree_with_oracle(q_len, monkeypatch):
    lens, pads = [300, 40, 19, 1000], [5, 38, 17, 999]
    case = indexed_case(330 + q_len, 4, 16, 4, 128, lens, pads, 1024, BF16, cache_rows=6)
    q = multi_query(331 + q_len, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    res = {}
    for path in ("16x16", "4x4"):
        if path == "4x4":
            monkeypatch.setenv("FDEC_MULTI_PATH", "4x4")
        out, lse = run(case, q, 3)
        check(out, lse, ref_out, ref_lse, BF16, f"{path} q_len={q_len}")
        res[path] = out
    assert (res["16x16"] - res["4x4"]).abs().max().item() < 1e-4


@pytest.mark.parametrize("G,q_len", [(8, 2), (1, 12), (2, 16), (4, 16), (4, 3)])
@pytest.mark.parametrize("paged", [False, True])
def test_multi_token_balanced_any_group_size(G, q_len, paged):
    Hkv = 2 if G == 8 else 4
    lens = [700, 3, 1, 0, 64, 65, 2000]  # an empty request between others
    if paged:
        case = paged_case(340 + G + q_len, 7, G * Hkv, Hkv, 128, lens, 32, F16, extra_pages=3, pad="nan")
    else:
        case = contiguous_case(350 + G + q_len, 7, G * Hkv, Hkv, 128, lens, 2048, BF16, pad="nan")
    q = multi_query(360 + G + q_len, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for nb in (1, 3, 40, 0):
        out, lse = run_bal(case, q, nb)
        check(out, lse, ref_out, ref_lse, case.dtype, f"balanced G={G} q_len={q_len} paged={paged} nb={nb}")


def test_multi_token_balanced_many_requests():
    # more than one wave's worth of requests in the block-range scan, many of them empty
    rng = np.random.default_rng(370)
    lens = [int(x) for x in rng.integers(0, 400, size=150)]
    for i in range(0, 150, 7):
        lens[i] = 0
    case = paged_case(371, 150, 16, 4, 128, lens, 16, BF16, extra_pages=4, pad="nan")
    q = multi_query(372, case, 4)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for nb in (5, 0):
        out, lse = run_bal(case, q, nb)
        check(out, lse, ref_out, ref_lse, BF16, f"balanced 150 requests nb={nb}")


@pytest.mark.parametrize("q_len", [3, 8])
def test_multi_token_balanced_both_kernels_agree(q_len, monkeypatch):
    lens, pads = [300, 40, 19, 1000], [5, 38, 17, 999]
    case = pad_left(paged_case(380 + q_len, 4, 16, 4, 128, lens, 16, BF16, extra_pages=2, pad="nan"), pads)
    q = multi_query(381 + q_len, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    res = {}
    for path in ("16x16", "4x4"):
        if path == "4x4":
            monkeypatch.setenv("FDEC_MULTI_PATH", "4x4")
        out, lse = run_bal(case, q, 3)
        check(out, lse, ref_out, ref_lse, BF16, f"balanced {path} q_len={q_len}")
        res[path] = out
    assert (res["16x16"] - res["4x4"]).abs().max().item() < 1e-4


@pytest.mark.parametrize("G,dt", [(1, F16), (2, BF16), (1, BF16)])
def test_one_token_balanced_at_g1_g2(G, dt):
    # one query token at G = 1, 2 on the balanced split: the 16x16x32 kernel with its
    # 16-row block padded; fdec_decode_multi_balanced with q_len = 1 is the same call
    case = paged_case(390 + G, 7, 8 * G, 8, 128, [40, 0, 3000, 1, 777, 64, 65], 16, dt, extra_pages=2, pad="nan")
    d = to_dev(case)
    q = multi_query(391 + G, case, 1)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for nb in (1, 5, 0):
        om, lm = run_bal(case, q, nb)
        check(om, lm, ref_out, ref_lse, dt, f"one-token balanced G={G} nb={nb}")
        o1, l1 = F.decode_balanced(q[:, 0].contiguous().to("cuda"), d["k"], d["v"], d["seq_lens"],
                                   page_table=d["page_table"], num_blocks=nb)
        torch.cuda.synchronize()
        assert torch.equal(om[:, 0], o1) and torch.equal(lm[:, :, 0], l1), f"G={G} nb={nb}"


# ---------------------------------------------------------------- float8 caches on the 16x16x32 kernel
# ("Inference Cookbook / 推理优化" §7.2, FP8 KV cache: e4m3 codes times a descale per
# (request, KV head), bf16 queries). The 16x16x32 kernel widens the float8 tiles to
# bf16 after each LDS read; G = 1, 2 and 8 (and G = 4 from 12 query rows) run it.

@pytest.mark.parametrize("G,q_len", [(1, 2), (1, 13), (2, 3), (2, 8), (4, 3), (4, 16), (8, 2), (8, 5)])
@pytest.mark.parametrize("kind", ["contig", "paged"])
def test_fp8_multi_token_on_the_16x16x32_kernel(G, q_len, kind):
    if kind == "contig":
        case = contiguous_case(600 + 10 * G + q_len, 6, 4 * G, 4, 128, LENS, 2048, FP8, pad="nan")
    else:
        case = paged_case(700 + 10 * G + q_len, 6, 4 * G, 4, 128, LENS, 32, FP8, extra_pages=3, pad="nan")
    q = multi_query(800 + 10 * G + q_len, case, q_len)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for S in (1, 5, 0):
        out, lse = run(case, q, S)
        check(out, lse, ref_out, ref_lse, FP8, f"float8 {kind} G={G} q_len={q_len} S={S}")
    for nb in (1, 3, 0):
        out, lse = run_bal(case, q, nb)
        check(out, lse, ref_out, ref_lse, FP8, f"float8 balanced {kind} G={G} q_len={q_len} nb={nb}")


def test_fp8_multi_token_with_leftpad_and_batch_idx():
    lens, pads = [300, 40, 19, 1000], [5, 38, 17, 999]  # some tokens see only padding -> empty
    case = indexed_case(640, 4, 8, 4, 128, lens, pads, 1024, FP8, cache_rows=7)  # G = 2
    q = multi_query(641, case, 5)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for S in (1, 4):
        out, lse = run(case, q, S)
        check(out, lse, ref_out, ref_lse, FP8, f"float8 indexed S={S}")
    for nb in (2, 0):
        out, lse = run_bal(case, q, nb)
        check(out, lse, ref_out, ref_lse, FP8, f"float8 balanced indexed nb={nb}")


def test_fp8_multi_token_both_g4_kernels_match_the_oracle(monkeypatch):
    # G = 4 with 16 query rows: the 16x16x32 kernel, and the 4x4x4 kernel when forced
    case = paged_case(660, 5, 16, 4, 128, [900, 3, 64, 1500, 0], 16, FP8, extra_pages=2, pad="nan")
    q = multi_query(661, case, 4)
    ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(128))
    for path in ("16x16", "4x4"):
        if path == "4x4":
            monkeypatch.setenv("FDEC_MULTI_PATH", "4x4")
        for S in (3, 0):
            out, lse = run(case, q, S)
            check(out, lse, ref_out, ref_lse, FP8, f"float8 G=4 {path} S={S}")
        out, lse = run_bal(case, q, 4)
        check(out, lse, ref_out, ref_lse, FP8, f"float8 G=4 balanced {path}")
