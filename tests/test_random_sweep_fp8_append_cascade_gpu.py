"""Seeded random sweep of the float8 append and of the cascade, against the fp64 oracle, through the C ABI.

Float8 append cases draw, from their own seed: the GQA group size (1, 2, 4, 8),
head dim (64 or 128), rotary dim (0, D/2, D), a contiguous cache or pages of
16, 32 or 64 tokens, 1 to 6 requests whose cache_seqlens mix empty, tile-edge
and full caches (room for the appended row kept), NaN in every unused row, a
split count from 0 (planned) to 40 and either merge path. The bar is the float8
append bar of the fixed tests (`check_fp8_append`).

Cascade cases draw: the group size (1, 2, 4, 8), the pool's element type (fp16,
bf16, float8), pages of 16, 32, 48, 64 or 128 tokens, a shared prefix of 0 to
3000 tokens (ragged in its last page), 1 to 70 requests (up to 560 query rows
per KV head) with suffixes of 0 to 500 tokens, NaN in every unused slot, and the
prefix / suffix split counts (0 = planned). The bar is the cascade bar of the
fixed tests (`assert_cascade_parity`: float8 pools within twice the P-rounding
bound); where prefix and suffix share one launch (G = 4, Hkv 4 or 8) the result is
also compared bit for bit with the two launches. The draws are fixed, so a failure
names a case that can be rerun by its id.
"""
import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import assert_cascade_parity, check_fp8_append, oracle_decode, to_dev
from synth import BF16, F16, FP8, append_case, cascade_case

pytestmark = pytest.mark.gpu

NAPPEND, NCASCADE = 48, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


def draw_append(i):
    r = np.random.default_rng(5000 + i)
    G = int(r.choice([1, 2, 4, 8]))
    Hkv = int(r.choice([1, 2, 4])) if G == 8 else int(r.choice([1, 2, 4, 8]))
    D = int(r.choice([64, 128]))
    B = int(r.integers(1, 7))
    cap = int(r.choice([64, 200, 1000]))
    special = [0, 1, 15, 16, 17, cap - 1]
    cs = [int(r.choice(special)) if r.random() < 0.4 else int(r.integers(0, cap)) for _ in range(B)]
    return dict(i=i, G=G, Hkv=Hkv, D=D, B=B, cap=cap, cs=cs, rd=int(r.choice([0, D // 2, D])),
                ps=int(r.choice([0, 16, 32, 64])), S=int(r.choice([0, 1, 2, 5, 13, 40])),
                fused=bool(r.random() < 0.4), seed=6000 + i)


def draw_cascade(i):
    r = np.random.default_rng(7000 + i)
    G = int(r.choice([1, 2, 4, 4, 8]))
    Hkv = int(r.choice([1, 2, 4])) if G == 8 else int(r.choice([1, 2, 4, 8]))
    B = int(r.choice([1, 3, 8, 40, 70]))
    ps = int(r.choice([16, 32, 48, 64, 128]))
    prefix = int(r.choice([0, 1, 15, 64, 100, 333, 1000, 3000]))
    hi = int(r.choice([1, 40, 500]))
    sl = [int(r.integers(0, hi + 1)) for _ in range(B)]
    return dict(i=i, G=G, Hkv=Hkv, B=B, ps=ps, prefix=prefix, sl=sl,
                dtype=[F16, BF16, FP8][int(r.integers(0, 3))],
                sp=int(r.choice([0, 1, 3, 8])), ss=int(r.choice([0, 1, 2, 8])), seed=8000 + i)


def append_id(i):
    c = draw_append(i)
    return f"{i}-G{c['G']}-Hkv{c['Hkv']}-D{c['D']}-rd{c['rd']}-ps{c['ps']}-S{c['S']}-{'fused' if c['fused'] else 'two'}"


def cascade_id(i):
    c = draw_cascade(i)
    return (f"{i}-G{c['G']}-Hkv{c['Hkv']}-B{c['B']}-{str(c['dtype']).split('.')[-1]}-ps{c['ps']}"
            f"-pre{c['prefix']}-sp{c['sp']}-ss{c['ss']}")


@pytest.mark.parametrize("i", range(NAPPEND), ids=[append_id(i) for i in range(NAPPEND)])
def test_random_fp8_append_matches_oracle(i):
    c = draw_append(i)
    case = append_case(c["seed"], c["B"], c["G"] * c["Hkv"], c["Hkv"], c["D"], c["cap"], FP8, rotary_dim=c["rd"],
                       pad="nan", cache_seqlens=c["cs"], page_size=c["ps"])
    check_fp8_append(case, c["S"], c["fused"], append_id(i))


@pytest.mark.parametrize("i", range(NCASCADE), ids=[cascade_id(i) for i in range(NCASCADE)])
def test_random_cascade_matches_oracle(i, monkeypatch):
    c = draw_cascade(i)
    case = cascade_case(c["seed"], c["B"], c["G"] * c["Hkv"], c["Hkv"], 128, c["prefix"], c["ps"], suffix_lens=c["sl"],
                        dtype=c["dtype"], pad="nan", extra_pages=2)
    d = to_dev(case)
    ref_out, ref_lse = oracle_decode(case)
    monkeypatch.delenv("FDEC_CASCADE_PATH", raising=False)
    sp, ss = c["sp"], c["ss"]
    if sp == 0 or ss == 0:  # as the library plans (the planned counts depend on the launch path)
        psp, pss = F.cascade_plan(c["B"], c["G"] * c["Hkv"], c["Hkv"], case.prefix_len, case.capacity, c["ps"],
                                  kv_dtype=c["dtype"])
        sp = sp or (max(1, min(psp, F.MAX_SPLITS - ss)) if ss else psp)
        ss = ss or max(1, min(pss, F.MAX_SPLITS - sp))

    def run():
        out, lse = F.cascade_decode(d["q"], d["k"], d["v"], d["page_table"], d["prefix_pages"], case.prefix_len,
                                    d["seq_lens"], sp, ss, k_descale=d["k_descale"], v_descale=d["v_descale"])
        torch.cuda.synchronize()
        return out, lse

    out, lse = run()
    assert_cascade_parity(case, out, lse, ref_out, ref_lse, cascade_id(i))
    if c["G"] == 4 and c["Hkv"] % 4 == 0:  # the single launch: bitwise the two launches at the same counts
        monkeypatch.setenv("FDEC_CASCADE_PATH", "two")
        o2, l2 = run()
        assert torch.equal(out, o2) and torch.equal(lse, l2), f"{cascade_id(i)}: single launch differs from two"
