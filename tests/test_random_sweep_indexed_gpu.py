"""Seeded random sweep of cache_batch_idx and cache_leftpad, against the fp64 oracle, through the C ABI.

Each case draws, from its own seed: the GQA group size (1, 2, 4, 8), head dim
(64 or 128), cache type (fp16, bf16, float8 where the entry point takes it),
a contiguous cache (rows in request order, or a permutation of more rows than
requests through cache_batch_idx) or pages of 16, 32 or 64 tokens, 1 to 6
requests whose lengths mix empty, one-row, tile-edge and long requests, a left
padding per request (none, all of it, all but one row, a tile edge, or any
count up to the length), NaN in every row no request may read, a split count or
block count (0 = planned), and one entry point: fdec_decode (two kernels or the
single-kernel merge, with or without an append + NeoX rotary counted from the
first valid row), fdec_decode_balanced, fdec_decode_multi and
fdec_decode_multi_balanced (1 to 8 query tokens). Every case first runs the
device-data check on its inputs, which must flag nothing, and half of them run
with the debug mode on. The bar is the one the fixed tests use. The draws are
fixed, so a failure names a case that can be rerun by its id.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import (LSE_RTOL, OUT_TOL, assert_parity, check_append_k, check_fp8_append, okv, oracle_decode,
                     to_dev)
from synth import BF16, F16, FP8, append_case, indexed_case, multi_query, pad_left, paged_case

pytestmark = pytest.mark.gpu

NCASES = 96


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


def _fp8_ok(kind, G, q_len):
    """Entry points that take a float8 cache at this shape (head dim 128 where it matters)."""
    if kind in ("two", "fused", "append", "balanced"):
        return True
    if kind == "multi":
        return q_len == 1 or G == 4
    return G == 4 or (G == 8 and q_len == 1)  # multi_bal


def draw(i):
    """The i-th case's parameters (pure function of i)."""
    r = np.random.default_rng(9000 + i)
    G = int(r.choice([1, 2, 4, 4, 8]))
    Hkv = int(r.choice([1, 2, 4])) if G == 8 else int(r.choice([1, 2, 4, 8]))
    D = 128 if G in (4, 8) or r.random() < 0.7 else 64
    B = int(r.integers(1, 7))
    cap = int(r.choice([64, 200, 1000, 3000]))
    kinds = ["two", "fused", "append"]
    if D == 128:
        kinds += ["multi", "multi_bal"]
        if G in (4, 8):
            kinds += ["balanced"]
    kind = str(r.choice(kinds))
    q_len = 1
    if kind == "multi":
        q_len = int(r.integers(1, 9))
    elif kind == "multi_bal":  # one query token at G = 1, 2 has no balanced kernel
        q_len = int(r.integers(1 if G in (4, 8) else 2, 9))
    dtypes = [F16, BF16] + ([FP8] if _fp8_ok(kind, G, q_len) else [])
    dtype = dtypes[int(r.integers(0, len(dtypes)))]
    ps = int(r.choice([0, 0, 16, 32, 64]))
    extra_rows = int(r.choice([-1, 0, 2])) if ps == 0 else -1  # -1: no cache_batch_idx
    special = [0, 1, 15, 16, 17, cap - 1 if kind == "append" else cap]
    hi = cap - 1 if kind == "append" else cap
    lens = [int(r.choice(special)) if r.random() < 0.35 else int(r.integers(0, hi + 1)) for _ in range(B)]
    pads = []
    for L in lens:
        how = int(r.integers(0, 5))
        pads.append([0, L, max(L - 1, 0), (L // 2) & ~15, int(r.integers(0, L + 1))][how])
    return dict(i=i, G=G, Hkv=Hkv, Hq=G * Hkv, D=D, B=B, cap=cap, kind=kind, q_len=q_len, dtype=dtype, ps=ps,
                extra_rows=extra_rows, lens=lens, pads=pads, S=int(r.choice([0, 1, 2, 5, 13, 40])),
                fused=bool(r.random() < 0.5), rd=int(r.choice([0, D // 2, D])), debug=i % 2 == 1, seed=10000 + i)


def case_id(i):
    c = draw(i)
    idx = "" if c["extra_rows"] < 0 else f"-idx{c['B'] + c['extra_rows']}"
    return (f"{i}-{c['kind']}-G{c['G']}-Hkv{c['Hkv']}-D{c['D']}-{str(c['dtype']).split('.')[-1]}"
            f"-ps{c['ps']}{idx}-S{c['S']}-q{c['q_len']}")


def _scatter_rows(case, rows, seed):
    """Move a contiguous case's request rows to a seeded permutation of `rows` cache rows
    (cache_batch_idx); the rows no request names hold NaN."""
    g = torch.Generator().manual_seed(seed)
    idx = torch.randperm(rows, generator=g)[:case.B].to(torch.int32)
    for name in ("k", "v"):
        t = getattr(case, name)
        full = torch.full((rows,) + tuple(t.shape[1:]), float("nan"), dtype=torch.float32).to(t.dtype)
        full[idx.long()] = t
        setattr(case, name, full)
    case.cache_batch_idx = idx
    return case


def build_case(c):
    args = (c["seed"], c["B"], c["Hq"], c["Hkv"], c["D"])
    if c["kind"] == "append":
        case = append_case(*args, c["cap"], c["dtype"], rotary_dim=c["rd"], pad="nan", cache_seqlens=c["lens"],
                           page_size=c["ps"])
        if c["extra_rows"] >= 0:
            case = _scatter_rows(case, c["B"] + c["extra_rows"], c["seed"] + 1)
        return pad_left(case, c["pads"])
    if c["ps"]:
        return pad_left(paged_case(*args, c["lens"], c["ps"], c["dtype"], extra_pages=2, pad="nan"), c["pads"])
    rows = None if c["extra_rows"] < 0 else c["B"] + c["extra_rows"]
    return indexed_case(*args, c["lens"], c["pads"], c["cap"], c["dtype"], cache_rows=rows)


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


def _run(c, case, what):
    d = to_dev(case)
    kw = dict(page_table=d["page_table"], k_descale=d["k_descale"], v_descale=d["v_descale"],
              cache_batch_idx=d["cache_batch_idx"], cache_leftpad=d["cache_leftpad"])
    a = None
    if c["kind"] == "append":
        a = F.make_append(d["k_new"], d["v_new"], d["rope_cos"], d["rope_sin"], case.rotary_dim)
    # the device-data check passes every valid draw
    flags = F.check_inputs(d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], append=a,
                           cache_batch_idx=d["cache_batch_idx"], cache_leftpad=d["cache_leftpad"])
    assert flags == (0, -1), f"{what}: the device-data check flagged valid inputs {flags}"
    if c["kind"] == "append":
        if case.dtype == FP8:
            check_fp8_append(case, c["S"], c["fused"], what)
            return
        kc, vc, q_rot, after = oracle.append(okv(case), case.k_new, case.v_new, case.q, case.seq_lens,
                                             case.rotary_dim, case.rope_base)
        ref_out, ref_lse = oracle.decode(after, q_rot, case.seq_lens + 1, 1 / math.sqrt(case.D))
        out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=c["S"], fused=c["fused"], append=a,
                            **kw)
        torch.cuda.synchronize()
        vg = d["v"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(vg, vc), f"{what}: v cache differs"
        kg = d["k"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        check_append_k(kg, kc, case, what)
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, what)
        return
    if c["kind"] in ("multi", "multi_bal"):
        q = multi_query(c["seed"] + 7, case, c["q_len"])
        ref_out, ref_lse = oracle.decode_multi(okv(case), q, case.seq_lens, 1 / math.sqrt(case.D))
        if c["kind"] == "multi":
            out, lse = F.decode_multi(q.to("cuda"), d["k"], d["v"], d["seq_lens"], num_splits=c["S"], **kw)
        else:
            out, lse = F.decode_multi_balanced(q.to("cuda"), d["k"], d["v"], d["seq_lens"],
                                               num_blocks=min(c["S"] * 6, 256), **kw)
        torch.cuda.synchronize()
        check_multi(out, lse, ref_out, ref_lse, case.dtype, what)
        return
    ref_out, ref_lse = oracle_decode(case)
    if c["kind"] == "balanced":
        out, lse = F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], num_blocks=min(c["S"] * 6, 256), **kw)
    else:
        out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=c["S"], fused=c["kind"] == "fused",
                            **kw)
    torch.cuda.synchronize()
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, what)


@pytest.mark.parametrize("i", range(NCASES), ids=[case_id(i) for i in range(NCASES)])
def test_random_indexed_case_matches_oracle(i):
    c = draw(i)
    case = build_case(c)
    F.set_debug(c["debug"])
    try:
        _run(c, case, case_id(i))
    finally:
        F.set_debug(False)
