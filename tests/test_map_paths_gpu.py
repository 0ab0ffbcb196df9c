"""Both split-KV map kernels against the fp64 oracle, through the C ABI.

GQA groups of four or eight query heads at D = 128 run on the matrix-core map
kernels; FDEC_MAP_PATH=vector forces the vector kernel
for the same inputs. The cases cover every tile position of a ragged tail
(lengths around multiples of 16 and 32), empty requests, pages of 16, 32 and
48 tokens, 1, 3 and 4 KV heads per block, both element types, and a head
count that does not divide into whole blocks of four waves.
"""
import math
import os

import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import assert_parity, okv, oracle_decode, to_dev
from synth import BF16, F16, contiguous_case, paged_case

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


CASES = [
    ("contig_bf16_tail", lambda: contiguous_case(61, 4, 16, 4, 128, [1, 31, 32, 1000], 1024, BF16, pad="nan")),
    ("contig_f16_tail", lambda: contiguous_case(62, 4, 32, 8, 128, [15, 16, 17, 33], 64, F16, pad="nan")),
    ("contig_bf16_empty", lambda: contiguous_case(63, 3, 12, 3, 128, [0, 47, 0], 64, BF16, pad="nan")),
    ("contig_f16_hkv1", lambda: contiguous_case(64, 2, 4, 1, 128, [2049, 700], 2100, F16, pad="nan")),
    ("contig_bf16_hkv6", lambda: contiguous_case(65, 2, 24, 6, 128, [513, 1111], 1200, BF16, pad="nan")),
    ("paged16_f16", lambda: paged_case(66, 4, 16, 4, 128, [15, 16, 17, 777], 16, F16, extra_pages=5,
                                       pad="nan")),
    ("paged32_bf16", lambda: paged_case(67, 3, 32, 8, 128, [64, 95, 1500], 32, BF16, extra_pages=3, pad="nan")),
    ("paged48_f16", lambda: paged_case(68, 3, 8, 2, 128, [48, 49, 480], 48, F16, extra_pages=2, pad="nan")),
    # groups of eight query heads (two groups of four per wave on matrix cores)
    ("g8_contig_bf16", lambda: contiguous_case(69, 3, 64, 8, 128, [1, 33, 3000], 3072, BF16, pad="nan")),
    ("g8_paged16_f16", lambda: paged_case(70, 4, 16, 2, 128, [0, 16, 17, 1234], 16, F16, extra_pages=3,
                                          pad="nan")),
    ("g8_contig_hkv3", lambda: contiguous_case(71, 2, 24, 3, 128, [700, 65], 768, BF16, pad="nan")),
]


@pytest.mark.parametrize("name,builder", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("num_splits", [1, 5, 32, 0])
def test_map_paths_match_oracle(path, name, builder, num_splits):
    case = builder()
    ref_out, ref_lse = oracle_decode(case)
    d = to_dev(case)
    for fused in (False, True):
        out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                            num_splits=num_splits, fused=fused)
        torch.cuda.synchronize()
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{path} {name} S={num_splits} fused={fused}")


@pytest.mark.parametrize("paged", [False, True])
def test_map_path_states_match_oracle_states(path, paged):
    # split states (m_i, d_i, O~_i) of the matrix-core kernel, normalised to the
    # split's true maximum, against the oracle's
    lens = [1, 33, 300, 1000]
    if paged:
        case = paged_case(69, 4, 16, 4, 128, lens, 32, F16, max_pages=32, extra_pages=5, pad="nan")
    else:
        case = contiguous_case(69, 4, 16, 4, 128, lens, 1024, F16, pad="nan")
    S = 7
    d = to_dev(case)
    po, pm, pd = F.decode_partials(d["q"], d["k"], d["v"], d["seq_lens"], S, page_table=d["page_table"])
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


def test_map_paths_agree_closely():
    # the two kernels differ only in summation order and P's hi + lo split
    case = contiguous_case(70, 2, 32, 8, 128, [4000, 2500], 4096, BF16, pad="nan")
    d = to_dev(case)
    res = {}
    for p in ("vector", "mfma"):
        old = os.environ.pop("FDEC_MAP_PATH", None)
        if p == "vector":
            os.environ["FDEC_MAP_PATH"] = "vector"
        try:
            res[p] = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=9)
            torch.cuda.synchronize()
        finally:
            os.environ.pop("FDEC_MAP_PATH", None)
            if old is not None:
                os.environ["FDEC_MAP_PATH"] = old
    (ov, lv), (om, lm) = res["vector"], res["mfma"]
    assert (ov - om).abs().max().item() < 5e-5
    assert ((lv - lm).abs() / lv.abs().clamp(min=1)).max().item() < 2e-6
