"""cache_batch_idx and cache_leftpad on the GPU against the fp64 oracle, through the C ABI.

Request b reads row cache_batch_idx[b] of a contiguous cache and attends to
rows [cache_leftpad[b], L_b); splits start at the 16-row tile holding the
first valid row (its rows above the padding are masked). Every row
a request must not read (left padding, past its length, cache rows no request
names) holds NaN, so a wrong row poisons the output. Covered: both map kernels,
fused and two-kernel merges, the balanced split, float8 caches, paged caches
with left padding, the map-stage states, and the append with its rotary
position counted from the first valid row.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import assert_parity, check_append_k, okv, oracle_decode, to_dev
from synth import BF16, F16, FP8, append_case, indexed_case, pad_left, paged_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


@pytest.fixture(params=["mfma", "vector"])
def path(request, monkeypatch):
    if request.param == "vector":
        monkeypatch.setenv("FDEC_MAP_PATH", "vector")
    else:
        monkeypatch.delenv("FDEC_MAP_PATH", raising=False)
    return request.param


def kw(d):
    return dict(page_table=d["page_table"], k_descale=d["k_descale"], v_descale=d["v_descale"],
                cache_batch_idx=d["cache_batch_idx"], cache_leftpad=d["cache_leftpad"])


LENS = [700, 16, 33, 300, 0, 1000]
PADS = [0, 16, 33, 17, 0, 999]  # whole tiles, the whole request, a ragged start, a one-row request

CASES = [
    ("contig_bf16_idx", lambda: indexed_case(91, 6, 16, 4, 128, LENS, PADS, 1024, BF16, cache_rows=9)),
    ("contig_f16_noidx", lambda: indexed_case(92, 6, 16, 4, 128, LENS, PADS, 1024, F16)),
    ("paged_bf16_lp", lambda: pad_left(paged_case(93, 6, 16, 4, 128, LENS, 16, BF16, extra_pages=3, pad="nan"),
                                       PADS)),
    ("paged48_f16_lp", lambda: pad_left(paged_case(94, 6, 16, 4, 128, LENS, 48, F16, extra_pages=2, pad="nan"),
                                        PADS)),
    # float8 caches: G = 4 (either map kernel with the path fixture) and G = 2 (the vector kernel)
    ("contig_fp8_idx", lambda: indexed_case(101, 6, 16, 4, 128, LENS, PADS, 1024, FP8, cache_rows=9)),
    ("contig_fp8_g2_idx", lambda: indexed_case(102, 6, 16, 8, 128, LENS, PADS, 1024, FP8, cache_rows=7)),
    ("paged32_fp8_g2_lp", lambda: pad_left(paged_case(103, 6, 8, 4, 64, LENS, 32, FP8, extra_pages=2, pad="nan"),
                                           PADS)),
]


@pytest.mark.parametrize("name,builder", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("num_splits", [1, 5, 0])
def test_indexed_decode_matches_oracle(path, name, builder, num_splits):
    case = builder()
    ref_out, ref_lse = oracle_decode(case)
    d = to_dev(case)
    for fused in (False, True):
        out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=num_splits, fused=fused, **kw(d))
        torch.cuda.synchronize()
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{path} {name} S={num_splits} fused={fused}")


@pytest.mark.parametrize("dtype", [BF16, FP8])
@pytest.mark.parametrize("paged", [False, True])
def test_indexed_balanced_and_float8_match_oracle(dtype, paged):
    if paged:
        case = pad_left(paged_case(95, 6, 16, 4, 128, LENS, 16, dtype, extra_pages=3, pad="nan"), PADS)
    else:
        case = indexed_case(95, 6, 16, 4, 128, LENS, PADS, 1024, dtype, cache_rows=8)
    ref_out, ref_lse = oracle_decode(case)
    d = to_dev(case)
    for nb in (1, 3, 64, 0):
        out, lse = F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], num_blocks=nb, **kw(d))
        torch.cuda.synchronize()
        assert_parity(out, lse, ref_out, ref_lse, dtype, f"balanced nb={nb} paged={paged}")
    if dtype == FP8:
        for S in (1, 7):
            out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=S, **kw(d))
            torch.cuda.synchronize()
            assert_parity(out, lse, ref_out, ref_lse, dtype, f"float8 S={S} paged={paged}")


def test_zero_leftpad_and_identity_index_equal_plain_bitwise(path):
    case = indexed_case(96, 4, 16, 4, 128, [500, 1, 64, 0], [0, 0, 0, 0], 512, BF16)
    d = to_dev(case)
    ident = torch.arange(4, dtype=torch.int32, device="cuda")
    o0, l0 = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=5)
    o1, l1 = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=5, cache_batch_idx=ident,
                      cache_leftpad=d["cache_leftpad"])
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("paged", [False, True])
def test_indexed_map_states_match_oracle_states(path, paged):
    lens, pads = [300, 40, 1000, 17], [5, 40, 100, 16]
    if paged:
        case = pad_left(paged_case(97, 4, 16, 4, 128, lens, 32, F16, max_pages=32, extra_pages=2, pad="nan"), pads)
    else:
        case = indexed_case(97, 4, 16, 4, 128, lens, pads, 1024, F16, cache_rows=6)
    S = 6
    d = to_dev(case)
    po, pm, pd = F.decode_partials(d["q"], d["k"], d["v"], d["seq_lens"], S, **kw(d))
    torch.cuda.synchronize()
    chunk = F.split_chunk(case.capacity, S)
    # splits: multiples of the chunk from the 16-row tile holding the first valid row
    bounds = np.array([[(p & ~15) + i * chunk for i in range(S + 1)] for p in pads], dtype=np.int32)
    rpo, rpm, rpd = oracle.partials(okv(case), case.q, case.seq_lens, 1 / math.sqrt(128), bounds)
    gpo, gpm, gpd = (t.cpu().double().numpy() for t in (po, pm, pd))
    fin = np.isfinite(rpm)
    assert np.array_equal(np.isfinite(gpm), fin)
    assert np.all(gpd[~fin] == 0) and np.all(gpo[~fin] == 0)
    np.testing.assert_allclose(gpm[fin], rpm[fin], rtol=0, atol=1e-5 * np.abs(rpm[fin]).max() + 1e-5)
    np.testing.assert_allclose(gpd[fin], rpd[fin], rtol=1e-4)
    err = np.abs(gpo - rpo)[fin] / rpd[fin][:, None]
    assert err.max() < 1e-3


def _bits16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("rd,S", [(128, 3), (0, 1), (64, 0)])
def test_append_with_batch_idx_and_leftpad(rd, S):
    # cache rows are a permutation of an append case's rows plus two unnamed rows of NaN
    base = append_case(98, 3, 16, 4, 128, 300, F16, rotary_dim=rd, pad="nan", cache_seqlens=[20, 150, 299])
    idx = torch.tensor([3, 0, 4], dtype=torch.int32)
    rows = 5
    for name in ("k", "v"):
        t = torch.full((rows,) + tuple(getattr(base, name).shape[1:]), float("nan"), dtype=F16)
        t[idx.long()] = getattr(base, name)
        setattr(base, name, t)
    base.cache_batch_idx = idx
    case = pad_left(base, [20, 7, 0])  # request 0: its only attended row is the appended one
    kc, vc, q_rot, after = oracle.append(okv(case), case.k_new, case.v_new, case.q, case.seq_lens,
                                         case.rotary_dim, case.rope_base)
    ref_out, ref_lse = oracle.decode(after, q_rot, case.seq_lens + 1, 1 / math.sqrt(case.D))
    d = to_dev(case)
    a = F.make_append(d["k_new"], d["v_new"], d["rope_cos"], d["rope_sin"], case.rotary_dim)
    out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=S, append=a, **kw(d))
    torch.cuda.synchronize()
    kg, vg = _bits16(d["k"].cpu()), _bits16(d["v"].cpu())
    assert np.array_equal(vg, vc)  # v rows and every untouched row, bitwise
    check_append_k(kg, kc, case, f"append rd={rd} S={S}")  # k: 1 ulp in the appended rows only
    if rd == 0:
        assert np.array_equal(kg, kc)
    assert_parity(out, lse, ref_out, ref_lse, F16, f"append rd={rd} S={S}")
