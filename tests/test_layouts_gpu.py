"""Cache layouts and page sizes, through strides, against the NHD result and the oracle.

The cache is described by three element strides (page or request, token, KV
head) with head_dim contiguous, so other layouts need no other kernel:
  - HND pages [pages, Hkv, page, D] (each page holds one KV head's rows
    contiguously): s_token = D, s_head = page * D;
  - one pool holding K and V per block, [blocks, 2, page, Hkv, D] ([vllm-arch]
    KV cache shape): K = pool[:, 0] and V = pool[:, 1], s_outer = 2 page Hkv D;
  - the same with HND pages, [blocks, 2, Hkv, page, D];
and pages of 16 to 1024 tokens. Every layout holds the same logical values as
the NHD case, and each kernel reads them in the same order, so the output must
equal the NHD output bitwise; the NHD output meets the parity bar against the
fp64 oracle.
"""
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import assert_parity, oracle_decode, to_dev
from synth import BF16, F16, FP8, cascade_case, paged_case

pytestmark = pytest.mark.gpu

LAYOUTS = ["hnd", "pool_nhd", "pool_hnd"]


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


def relayout(k, v, layout):
    """Copies of device caches k, v [P, page, Hkv, D] in another layout, as [P, page, Hkv, D] views."""
    dt = k.dtype
    k8, v8 = k.view(torch.uint8) if dt == FP8 else k, v.view(torch.uint8) if dt == FP8 else v
    if layout == "hnd":
        ko = k8.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        vo = v8.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    elif layout == "pool_nhd":
        pool = torch.stack([k8, v8], dim=1).contiguous()  # [P, 2, page, Hkv, D]
        ko, vo = pool[:, 0], pool[:, 1]
    elif layout == "pool_hnd":
        # [P, 2, Hkv, page, D]
        pool = torch.stack([k8.permute(0, 2, 1, 3), v8.permute(0, 2, 1, 3)], dim=1).contiguous()
        ko, vo = pool[:, 0].permute(0, 2, 1, 3), pool[:, 1].permute(0, 2, 1, 3)
    else:
        raise ValueError(layout)
    bits = torch.uint8 if dt == FP8 else torch.int16  # compare bit patterns (the padding holds NaN)
    assert torch.equal(ko.view(bits), k8.view(bits)) and torch.equal(vo.view(bits), v8.view(bits))
    assert ko.stride(3) == 1
    if dt == FP8:
        ko, vo = ko.view(FP8), vo.view(FP8)
    return ko, vo


def run(d, k, v, how, S):
    if how == "balanced":
        out, lse = F.decode_balanced(d["q"], k, v, d["seq_lens"], page_table=d["page_table"], num_blocks=S,
                                     k_descale=d["k_descale"], v_descale=d["v_descale"])
    else:
        out, lse = F.decode(d["q"], k, v, d["seq_lens"], page_table=d["page_table"], num_splits=S,
                            k_descale=d["k_descale"], v_descale=d["v_descale"])
    torch.cuda.synchronize()
    return out, lse


def make_case(seed, ps, dtype, G):
    Hkv = 4
    lens = [3 * ps + 5, 1, 700, 0, ps]
    return paged_case(seed, len(lens), G * Hkv, Hkv, 128, lens, ps, dtype, extra_pages=3, pad="nan")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("ps", [16, 64, 256])
@pytest.mark.parametrize("dtype,G,how", [(BF16, 4, "split"), (F16, 4, "split"), (FP8, 4, "split"),
                                         (BF16, 4, "balanced"), (FP8, 4, "balanced"), (F16, 1, "split"),
                                         (BF16, 8, "split"), (F16, 4, "vector")])
def test_layout_equals_nhd_bitwise(layout, ps, dtype, G, how, monkeypatch):
    if how == "vector":
        monkeypatch.setenv("FDEC_MAP_PATH", "vector")
    case = make_case(81 + ps, ps, dtype, G)
    d = to_dev(case)
    S = 7 if how != "balanced" else 5
    out0, lse0 = run(d, d["k"], d["v"], how, S)
    if layout == LAYOUTS[0]:
        ref_out, ref_lse = oracle_decode(case)
        assert_parity(out0, lse0, ref_out, ref_lse, dtype, f"nhd ps={ps} {how}")
    k, v = relayout(d["k"], d["v"], layout)
    out, lse = run(d, k, v, how, S)
    assert torch.equal(out, out0) and torch.equal(lse, lse0), f"{layout} ps={ps} {dtype} G={G} {how}"


@pytest.mark.parametrize("dtype", [BF16, FP8])
def test_large_pages_against_oracle(dtype):
    # 1024-token pages: a request's tiles stay on one page for 64 tiles
    case = paged_case(88, 3, 32, 8, 128, [5000, 1024, 1], 1024, dtype, extra_pages=1, pad="nan")
    ref_out, ref_lse = oracle_decode(case)
    d = to_dev(case)
    for layout in ("nhd", "hnd"):
        k, v = (d["k"], d["v"]) if layout == "nhd" else relayout(d["k"], d["v"], layout)
        for how, S in (("split", 0), ("split", 9), ("balanced", 0)):
            out, lse = run(d, k, v, how, S)
            assert_parity(out, lse, ref_out, ref_lse, dtype, f"ps=1024 {layout} {how} S={S}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_cascade_layouts_equal_nhd_bitwise(layout):
    case = cascade_case(89, 4, 16, 4, 128, prefix_len=300, ps=64, suffix_lens=[5, 100, 0, 64], dtype=BF16,
                        pad="nan", extra_pages=2)
    d = to_dev(case)

    def casc(k, v):
        out, lse = F.cascade_decode(d["q"], k, v, d["page_table"], d["prefix_pages"], case.prefix_len,
                                    d["seq_lens"], 2, 3)
        torch.cuda.synchronize()
        return out, lse

    out0, lse0 = casc(d["k"], d["v"])
    ref_out, ref_lse = oracle_decode(case)
    assert_parity(out0, lse0, ref_out, ref_lse, BF16, "cascade nhd")
    k, v = relayout(d["k"], d["v"], layout)
    out, lse = casc(k, v)
    assert torch.equal(out, out0) and torch.equal(lse, lse0), layout
