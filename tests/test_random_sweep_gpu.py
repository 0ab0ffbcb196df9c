"""Seeded random sweep over shapes and entry points, against the fp64 oracle, through the C ABI.

Each case draws, from its own seed: the GQA group size (1, 2, 4, 8), head dim
(64 or 128), cache type (fp16, bf16; float8 where the matrix-core kernels take
it), a contiguous cache or pages of 16, 32 or 64 tokens, a batch of 1 to 6
requests whose lengths mix empty, one-token, tile-edge and long requests,
NaN in every unused row, and a split count from 0 (planned) to 40; then one of
the entry points that takes that shape: fdec_decode (two kernels or the
single-kernel merge, with or without an append + NeoX rotary),
fdec_decode_balanced, fdec_decode_multi (1 to 8 query tokens, any G). Each case
first runs the device-data check on its inputs, which must flag nothing. The
parity bar is the one every other parity test uses. The draws are fixed, so a failure
names a case that can be rerun by its id.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import LSE_RTOL, OUT_TOL, assert_parity, check_append_k, okv, oracle_decode, to_dev
from synth import BF16, F16, FP8, append_case, contiguous_case, multi_query, paged_case

pytestmark = pytest.mark.gpu

NCASES = 192


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


def draw(i):
    """The i-th case's parameters (pure function of i)."""
    r = np.random.default_rng(1000 + i)
    G = int(r.choice([1, 2, 4, 4, 8]))
    Hkv = int(r.choice([1, 2, 4, 8])) if G < 8 else int(r.choice([1, 2, 4]))
    D = 128 if G == 4 or r.random() < 0.7 else 64
    B = int(r.integers(1, 7))
    cap = int(r.choice([64, 200, 1000, 3000]))
    kinds = ["two", "fused", "append"]
    if G == 4 and D == 128:
        kinds += ["balanced", "multi", "multi"]
    elif D == 128:
        kinds += ["multi", "balanced"]
    kind = str(r.choice(kinds))
    dtypes = [F16, BF16]
    # float8: uniform splits for every shape; the balanced split and multi-token
    # decode (every G) at head_dim 128
    if kind in ("two", "fused") or (D == 128 and kind in ("balanced", "multi")):
        dtypes.append(FP8)
    dtype = dtypes[int(r.integers(0, len(dtypes)))]
    ps = int(r.choice([0, 16, 32, 64]))
    special = [0, 1, 15, 16, 17, cap]
    lens = [int(r.choice(special)) if r.random() < 0.35 else int(r.integers(1, cap + 1)) for _ in range(B)]
    S = int(r.choice([0, 1, 2, 5, 13, 40]))
    q_len = int(r.integers(1, 9)) if kind == "multi" else 1
    return dict(i=i, G=G, Hkv=Hkv, Hq=G * Hkv, D=D, B=B, cap=cap, kind=kind, dtype=dtype, ps=ps, lens=lens, S=S,
                q_len=q_len, rd=int(r.choice([0, D // 2, D])), seed=2000 + i)


def case_id(i):
    c = draw(i)
    return (f"{i}-{c['kind']}-G{c['G']}-Hkv{c['Hkv']}-D{c['D']}-{str(c['dtype']).split('.')[-1]}"
            f"-ps{c['ps']}-S{c['S']}")


def build_case(c):
    if c["kind"] == "append":
        cs = [min(L, c["cap"] - 1) for L in c["lens"]]
        return append_case(c["seed"], c["B"], c["Hq"], c["Hkv"], c["D"], c["cap"], c["dtype"], rotary_dim=c["rd"],
                           pad="nan", cache_seqlens=cs, page_size=c["ps"])
    if c["ps"]:
        return paged_case(c["seed"], c["B"], c["Hq"], c["Hkv"], c["D"], c["lens"], c["ps"], c["dtype"],
                          extra_pages=2, pad="nan")
    return contiguous_case(c["seed"], c["B"], c["Hq"], c["Hkv"], c["D"], c["lens"], c["cap"], c["dtype"], pad="nan")


def check_multi(out, lse, ref_out, ref_lse, dtype, what):
    o = out.cpu().double().numpy()
    assert np.isfinite(o).all(), f"{what}: non-finite output"
    err = np.abs(o - ref_out).max()
    assert err <= OUT_TOL[dtype], f"{what}: max-abs out error {err:.3g}"
    l = lse.cpu().double().numpy()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(l), fin), f"{what}: lse finiteness differs"
    if fin.any():
        rel = (np.abs(l[fin] - ref_lse[fin]) / np.maximum(np.abs(ref_lse[fin]), 1.0)).max()
        assert rel <= LSE_RTOL, f"{what}: lse relative error {rel:.3g}"


@pytest.mark.parametrize("i", range(NCASES), ids=[case_id(i) for i in range(NCASES)])
def test_random_case_matches_oracle(i):
    c = draw(i)
    case = build_case(c)
    what = case_id(i)
    d = to_dev(case)
    kw = dict(k_descale=d["k_descale"], v_descale=d["v_descale"])
    a = None
    if c["kind"] == "append":
        a = F.make_append(d["k_new"], d["v_new"], d["rope_cos"], d["rope_sin"], case.rotary_dim)
    flags = F.check_inputs(d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], append=a)
    assert flags == (0, -1), f"{what}: the device-data check flagged valid inputs {flags}"
    if c["kind"] == "append":
        kc, vc, q_rot, after = oracle.append(okv(case), case.k_new, case.v_new, case.q, case.seq_lens,
                                             case.rotary_dim, case.rope_base)
        ref_out, ref_lse = oracle.decode(after, q_rot, case.seq_lens + 1, 1 / math.sqrt(case.D))
        out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=c["S"],
                            append=a)
        torch.cuda.synchronize()
        # the written v rows are exact copies; k rows within one ulp of the oracle's rounding
        vg = d["v"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(vg, vc), f"{what}: v rows"
        kg = d["k"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        check_append_k(kg, kc, case, what)
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, what)
        return
    if c["kind"] == "multi":
        q = multi_query(c["seed"] + 7, case, c["q_len"])
        ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(case.D))
        out, lse = F.decode_multi(q.to("cuda"), d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                                  num_splits=c["S"], **kw)
        torch.cuda.synchronize()
        check_multi(out, lse, ref_out, ref_lse, case.dtype, what)
        return
    ref_out, ref_lse = oracle_decode(case)
    if c["kind"] == "balanced":
        out, lse = F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                                     num_blocks=min(c["S"] * 6, 256), **kw)
    else:
        out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=c["S"],
                            fused=c["kind"] == "fused", **kw)
    torch.cuda.synchronize()
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, what)
