"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test ties the oracle to something other than itself: exhaustive comparison
with numpy/torch number formats, torch's scaled_dot_product_attention in
float64 (a library special case, including its GQA head mapping), closed forms
(constant V, zero query, single token), one-hot scores, invariances the pages
state (splitting is exact; paging and page order do not change the result),
worked examples printed on the pages (tests/golden), and rotary identities.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from synth import BF16, F16, FP8, append_case, cascade_case, contiguous_case, paged_case

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(autouse=True, scope="module")
def _built(oracle_lib):
    return oracle_lib


def okv(case):
    return oracle.KV(case.k, case.v, oracle.dtype_code(case.k), case.Hq, case.B, case.page_size,
                     case.page_table, case.prefix_pages, case.prefix_len, case.k_descale, case.v_descale)


def golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- number formats

def test_f16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.to_f64(bits, oracle.F16)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zero is kept
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.to_f64(bits, oracle.BF16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_f8_decode_exhaustive():
    # every float8 e4m3fn code against torch's own decoding of the format
    bits = np.arange(256, dtype=np.uint8)
    ours = oracle.to_f64(bits, oracle.FP8)
    ref = torch.from_numpy(bits.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9


def _torch_f8(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_f8_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = oracle.to_f64(codes, oracle.FP8).astype(np.float32)
    assert np.array_equal(oracle.f32_to_f8(vals), codes)


def test_f8_encode_matches_torch_cast_below_overflow():
    # torch's cast to float8_e4m3fn (round to nearest even) agrees wherever it
    # does not overflow: random magnitudes over the whole range, every halfway
    # point between neighbouring codes (ties), and the subnormal range
    rng = np.random.default_rng(7)
    pos = oracle.to_f64(np.arange(0, 0x7F, dtype=np.uint8), oracle.FP8)
    x = np.concatenate([
        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 9, 20000),
        _halfway_points(pos),
        rng.uniform(0, 2.0 ** -6, 4000),
        [463.99, 464.0, 447.9, 2.0 ** -10, 3 * 2.0 ** -10, 1.0 + 2.0 ** -4],
    ])
    x = x[np.abs(x) <= 464.0].astype(np.float32)
    x = np.concatenate([x, -x])
    assert np.array_equal(oracle.f32_to_f8(x), _torch_f8(x))


def test_f8_encode_saturates_and_keeps_nan():
    big = np.array([464.5, 480.0, 1e6, 3.0e38, np.inf], dtype=np.float32)
    assert set(oracle.f32_to_f8(big).tolist()) == {0x7E}
    assert set(oracle.f32_to_f8(-big).tolist()) == {0xFE}
    assert oracle.f32_to_f8(np.array([np.nan], dtype=np.float32))[0] == 0x7F
    assert oracle.f32_to_f8(np.array([-0.0, -1e-30], dtype=np.float32)).tolist() == [0x80, 0x80]


def _halfway_points(vals):
    v = np.unique(vals[np.isfinite(vals)])
    return (v[:-1] + v[1:]) / 2.0


def test_f16_encode_matches_numpy_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 5, 20000),
        _halfway_points(np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)),
        np.array([65504.0, 65519.99, 65520.0, 7e4, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0001,
                  2.0 ** -14, 0.0, 1 + 2 ** -11 + 2 ** -40]),
    ])
    x = np.concatenate([x, -x])
    ours = oracle.from_f64(x, oracle.F16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_encode_bruteforce_nearest_even():
    # all finite non-negative bf16 values, in increasing order of their bit patterns
    pos_bits = np.arange(0, 0x7F80, dtype=np.uint16)
    pos_vals = oracle.to_f64(pos_bits, oracle.BF16)
    assert np.all(np.diff(pos_vals) > 0)
    rng = np.random.default_rng(1)
    x = np.concatenate([
        np.abs(rng.standard_normal(20000)) * 10.0 ** rng.integers(-40, 38, 20000),
        (pos_vals[:-1] + pos_vals[1:])[::97] / 2.0,  # exact ties
        np.array([1.0, 3.0, 2.0 ** -133, 2.0 ** -134, 1e-45]),
    ])
    x = x[x <= pos_vals[-1]]
    ours = oracle.from_f64(x, oracle.BF16)
    # brute force: nearest of the two neighbours, ties to the even bit pattern
    hi = np.searchsorted(pos_vals, x, side="left")
    lo = np.maximum(hi - 1, 0)
    hi = np.minimum(hi, len(pos_vals) - 1)
    dlo, dhi = x - pos_vals[lo], pos_vals[hi] - x
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(pos_bits[lo] % 2 == 0, lo, hi)))
    assert np.array_equal(ours, pos_bits[pick])
    assert np.array_equal(oracle.from_f64(-x, oracle.BF16), pos_bits[pick] | 0x8000)


# ---------------------------------------------------------------- attention definition

def _tiny_cases():
    out = []
    rng = np.random.default_rng(2)
    for i in range(12):
        Hkv = int(rng.integers(1, 3))
        G = int(rng.choice([1, 2, 4]))
        D = int(rng.choice([4, 8]))
        B = int(rng.integers(1, 3))
        cap = 7
        lens = rng.integers(1, cap + 1, B)
        dtype = F16 if i % 2 == 0 else BF16
        out.append(contiguous_case(100 + i, B, Hkv * G, Hkv, D, lens, cap, dtype, pad="nan"))
    return out


@pytest.mark.parametrize("case", _tiny_cases(), ids=lambda c: f"B{c.B}H{c.Hq}/{c.Hkv}D{c.D}")
def test_decode_matches_torch_sdpa_fp64(case):
    scale = 1.0 / math.sqrt(case.D) * (1.0 if case.D == 8 else 0.7)
    out, lse = oracle.decode(okv(case), case.q, case.seq_lens, scale)
    for b in range(case.B):
        L = int(case.seq_lens[b])
        q = case.q[b].to(torch.float64)[None, :, None, :]                # [1, Hq, 1, D]
        k = case.k[b, :L].to(torch.float64).permute(1, 0, 2)[None]      # [1, Hkv, L, D]
        v = case.v[b, :L].to(torch.float64).permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(q, k.contiguous(), v.contiguous(), scale=scale,
                                             enable_gqa=True)[0, :, 0, :]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)
        # LSE through the same library routine: add a zero key (score 0) whose
        # value is 0 while every real key has value 1; the output is Z / (1 + Z).
        ones = torch.ones(1, case.Hkv, L + 1, 1, dtype=torch.float64)
        ones[:, :, L] = 0.0
        ksink = torch.cat([k, torch.zeros(1, case.Hkv, 1, case.D, dtype=torch.float64)], dim=2)
        r = F.scaled_dot_product_attention(q, ksink.contiguous(), ones, scale=scale,
                                           enable_gqa=True)[0, :, 0, 0].numpy()
        np.testing.assert_allclose(lse[b], np.log(r / (1.0 - r)), rtol=0, atol=1e-10)


def test_constant_v_gives_constant_output():
    case = contiguous_case(7, 2, 8, 2, 32, [1, 100], 100, BF16, pad="nan")
    c = torch.randn(2, 1, 2, 32).to(BF16)
    case.v[:] = c
    out, _ = oracle.decode(okv(case), case.q, case.seq_lens, 0.3)
    for b in range(2):
        for h in range(8):
            np.testing.assert_allclose(out[b, h], c[b, 0, h // 4].to(torch.float64).numpy(),
                                       rtol=1e-13, atol=1e-13)


def test_zero_query_gives_mean_and_log_length():
    case = contiguous_case(8, 2, 4, 4, 16, [5, 33], 40, F16, pad="nan")
    case.q.zero_()
    out, lse = oracle.decode(okv(case), case.q, case.seq_lens, 0.25)
    for b in range(2):
        L = int(case.seq_lens[b])
        mean = case.v[b, :L].to(torch.float64).mean(0).numpy()  # [Hkv, D]
        np.testing.assert_allclose(out[b], mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[b], math.log(L), rtol=0, atol=1e-13)


def test_single_token_returns_its_value_row():
    case = contiguous_case(9, 3, 4, 2, 64, [1, 1, 1], 4, F16, pad="nan")
    out, lse = oracle.decode(okv(case), case.q, case.seq_lens, 0.125)
    for b in range(3):
        for h in range(4):
            g = h // 2
            assert np.array_equal(out[b, h], case.v[b, 0, g].to(torch.float64).numpy())
            s = 0.125 * np.dot(case.q[b, h].to(torch.float64).numpy(),
                               case.k[b, 0, g].to(torch.float64).numpy())
            assert abs(lse[b, h] - s) <= 1e-13 * max(1.0, abs(s))


def test_one_hot_scores_pick_one_row():
    D, L = 128, 300
    case = contiguous_case(10, 1, 4, 1, D, [L], L, F16, pad="zero")
    case.q.zero_()
    case.q[0, :, 0] = 40.0
    case.k[0, :, 0, 0] = 0.0
    jstar = 217
    case.k[0, jstar, 0, 0] = 40.0
    scale = 1.0 / math.sqrt(D)
    out, lse = oracle.decode(okv(case), case.q, case.seq_lens, scale)
    for h in range(4):
        np.testing.assert_allclose(out[0, h], case.v[0, jstar, 0].to(torch.float64).numpy(),
                                   rtol=0, atol=1e-12)
        assert abs(lse[0, h] - 1600.0 * scale) < 1e-9


# ---------------------------------------------------------------- paging

def _scatter_to_pages(case, ps, seed, extra_pages=3):
    """Copy a contiguous case into a NaN-poisoned paged pool under a random page order."""
    g = torch.Generator().manual_seed(seed)
    B, cap, Hkv, D = case.k.shape
    npages = [math.ceil(int(L) / ps) for L in case.seq_lens]
    pool = sum(npages) + extra_pages
    perm = torch.randperm(pool, generator=g)
    kp = torch.full((pool, ps, Hkv, D), float("nan"), dtype=case.k.dtype)
    vp = kp.clone()
    table = torch.full((B, max(npages)), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        L = int(case.seq_lens[b])
        for i in range(npages[b]):
            p = int(perm[off + i])
            table[b, i] = p
            n = min(ps, L - i * ps)
            kp[p, :n] = case.k[b, i * ps:i * ps + n]
            vp[p, :n] = case.v[b, i * ps:i * ps + n]
        off += npages[b]
    return kp, vp, table


@pytest.mark.parametrize("ps", [16, 32, 64])
def test_paged_equals_contiguous(ps):
    case = contiguous_case(11, 3, 8, 4, 32, [1, 77, 200], 200, BF16, pad="nan")
    ref = oracle.decode(okv(case), case.q, case.seq_lens, 0.2)
    kp, vp, table = _scatter_to_pages(case, ps, seed=ps)
    pk = oracle.KV(kp, vp, oracle.BF16, 8, 3, ps, table)
    got = oracle.decode(pk, case.q, case.seq_lens, 0.2)
    assert np.array_equal(ref[0], got[0]) and np.array_equal(ref[1], got[1])


def test_page_table_example_from_the_pages():
    rows = [[int(x) for x in r] for r in golden_rows("page_table_example.txt")]
    table = torch.tensor(rows, dtype=torch.int32)
    ps, D, Hkv = 16, 16, 2
    lens = torch.tensor([40, 20], dtype=torch.int32)  # 3 pages and 2 pages
    g = torch.Generator().manual_seed(12)
    pool_k = torch.randn(8, ps, Hkv, D, generator=g).to(F16)
    pool_v = torch.randn(8, ps, Hkv, D, generator=g).to(F16)
    pool_k[5:] = float("nan")  # pages no request uses
    pool_v[5:] = float("nan")
    pool_k[2, 8:] = float("nan")  # past sequence 0's length inside its last page
    pool_v[4, 4:] = float("nan")
    q = torch.randn(2, 4, D, generator=g).to(F16)
    got_out, got_lse = oracle.decode(oracle.KV(pool_k, pool_v, oracle.F16, 4, 2, ps, table), q,
                                     lens, 0.25)
    assert np.isfinite(got_out).all() and np.isfinite(got_lse).all()
    # the same logical sequences laid out contiguously, by hand from the table rows
    kc = torch.zeros(2, 48, Hkv, D, dtype=F16)
    vc = torch.zeros(2, 48, Hkv, D, dtype=F16)
    kc[0, :40] = torch.cat([pool_k[0], pool_k[1], pool_k[2, :8]])
    vc[0, :40] = torch.cat([pool_v[0], pool_v[1], pool_v[2, :8]])
    kc[1, :20] = torch.cat([pool_k[3], pool_k[4, :4]])
    vc[1, :20] = torch.cat([pool_v[3], pool_v[4, :4]])
    ref_out, ref_lse = oracle.decode(oracle.KV(kc, vc, oracle.F16, 4, 2), q, lens, 0.25)
    assert np.array_equal(got_out, ref_out) and np.array_equal(got_lse, ref_lse)


def test_gqa_equals_mha_with_repeated_kv_heads():
    case = contiguous_case(13, 2, 8, 2, 16, [9, 30], 30, F16, pad="nan")
    gqa = oracle.decode(okv(case), case.q, case.seq_lens, 0.3)
    rep = oracle.KV(case.k.repeat_interleave(4, dim=2), case.v.repeat_interleave(4, dim=2),
                    oracle.F16, 8, 2)
    mha = oracle.decode(rep, case.q, case.seq_lens, 0.3)
    assert np.array_equal(gqa[0], mha[0]) and np.array_equal(gqa[1], mha[1])


# ---------------------------------------------------------------- split / merge exactness

def _random_bounds(rng, lens, S, cap):
    out = np.zeros((len(lens), S + 1), dtype=np.int32)
    for b in range(len(lens)):
        cuts = np.sort(rng.integers(0, cap + 1, S - 1))
        out[b, 1:S] = cuts
        out[b, S] = cap
    return out


@pytest.mark.parametrize("S", [1, 2, 5, 16])
def test_merging_partials_at_any_split_points_is_exact(S):
    rng = np.random.default_rng(S)
    case = contiguous_case(14 + S, 2, 8, 2, 32, [1, 150], 150, BF16, pad="nan")
    kv = okv(case)
    ref_out, ref_lse = oracle.decode(kv, case.q, case.seq_lens, 0.2)
    bounds = _random_bounds(rng, case.seq_lens.numpy(), S, 150)
    if S >= 5:  # force an empty split and a one-token split
        bounds[1, 1] = bounds[1, 2] = 10
        bounds[1, 3] = 11
    po, pm, pd = oracle.partials(kv, case.q, case.seq_lens, 0.2, bounds)
    out, lse = oracle.merge(po, pm, pd)
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)
    # the merge order does not matter (max and sum are associative)
    perm = rng.permutation(S)
    out2, lse2 = oracle.merge(po[:, :, perm], pm[:, :, perm], pd[:, :, perm])
    np.testing.assert_allclose(out2, ref_out, rtol=0, atol=1e-12)
    # normalised states (o, lse) with d = 1 merge to the same result
    with np.errstate(invalid="ignore", divide="ignore"):
        o_n = np.where(pd[..., None] > 0, po / pd[..., None], 0.0)
        l_n = np.where(pd > 0, pm + np.log(pd), -np.inf)
    out3, lse3 = oracle.merge(o_n, l_n, np.where(pd > 0, 1.0, 0.0))
    np.testing.assert_allclose(out3, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse3, ref_lse, rtol=1e-13, atol=1e-13)


def test_empty_inputs():
    case = contiguous_case(20, 2, 4, 4, 16, [0, 3], 8, F16, pad="nan")
    out, lse = oracle.decode(okv(case), case.q, case.seq_lens, 0.25)
    assert np.array_equal(out[0], np.zeros((4, 16))) and np.all(lse[0] == -np.inf)
    assert np.isfinite(out[1]).all()
    po = np.zeros((1, 2, 3, 16))
    pm = np.full((1, 2, 3), -np.inf)
    pd = np.zeros((1, 2, 3))
    mo, ml = oracle.merge(po, pm, pd)
    assert np.array_equal(mo, np.zeros((1, 2, 16))) and np.all(ml == -np.inf)


# ---------------------------------------------------------------- cascade

def test_cascade_equals_attention_over_prefix_then_suffix():
    case = cascade_case(21, 3, 8, 2, 32, prefix_len=64, ps=16, suffix_lens=[0, 5, 40], dtype=BF16,
                        pad="nan", extra_pages=2)
    got = oracle.decode(okv(case), case.q, case.seq_lens, 0.2)
    # a plain paged table listing the prefix pages, then each request's own pages
    n_pre = case.prefix_pages.numel()
    table = torch.full((3, n_pre + case.page_table.shape[1]), -1, dtype=torch.int32)
    for b in range(3):
        table[b, :n_pre] = case.prefix_pages
        table[b, n_pre:] = case.page_table[b]
    plain = oracle.KV(case.k, case.v, oracle.BF16, 8, 3, 16, table)
    ref = oracle.decode(plain, case.q, case.seq_lens + 64, 0.2)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_fp8_cascade_matches_sdpa_over_dequantised_prefix_then_suffix():
    # a float8 pool: request b attends to the shared prefix, then its own pages,
    # every element read as its e4m3 value times request b's descales
    case = cascade_case(24, 3, 8, 2, 32, prefix_len=50, ps=16, suffix_lens=[0, 5, 40], dtype=FP8,
                        pad="nan", extra_pages=2)
    got = oracle.decode(okv(case), case.q, case.seq_lens, 0.2)
    for b in range(3):
        toks = [(int(case.prefix_pages[j // 16]), j % 16) for j in range(50)]
        toks += [(int(case.page_table[b, j // 16]), j % 16) for j in range(int(case.seq_lens[b]))]
        kd, vd = case.k_descale[b].double(), case.v_descale[b].double()
        kr = torch.stack([case.k[p_, s_].double() * kd[:, None] for p_, s_ in toks])  # [L, Hkv, D]
        vr = torch.stack([case.v[p_, s_].double() * vd[:, None] for p_, s_ in toks])
        ro, rl = _sdpa_rows(case.q[b], kr, vr, 0.2)
        np.testing.assert_allclose(got[0][b], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(got[1][b], rl, rtol=0, atol=1e-12)


def test_cascade_with_ragged_prefix_matches_gathered_rows():
    case = cascade_case(22, 2, 4, 2, 16, prefix_len=37, ps=16, suffix_lens=[3, 19], dtype=F16,
                        pad="nan")
    got = oracle.decode(okv(case), case.q, case.seq_lens, 0.3)
    # gather the logical rows by hand: prefix tokens, then the request's suffix tokens
    kc = torch.zeros(2, 37 + 19, 2, 16, dtype=F16)
    vc = torch.zeros_like(kc)
    for b in range(2):
        rows_k, rows_v = [], []
        for j in range(37):
            p = int(case.prefix_pages[j // 16])
            rows_k.append(case.k[p, j % 16])
            rows_v.append(case.v[p, j % 16])
        for j in range(int(case.seq_lens[b])):
            p = int(case.page_table[b, j // 16])
            rows_k.append(case.k[p, j % 16])
            rows_v.append(case.v[p, j % 16])
        n = len(rows_k)
        kc[b, :n] = torch.stack(rows_k)
        vc[b, :n] = torch.stack(rows_v)
    ref = oracle.decode(oracle.KV(kc, vc, oracle.F16, 4, 2), case.q, case.seq_lens + 37, 0.3)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


# ---------------------------------------------------------------- rotary and append

def test_rope_identities():
    rng = np.random.default_rng(5)
    D, rd = 128, 128
    x = rng.standard_normal(D)
    assert np.array_equal(oracle.rope_neox(x, 0, rd), x)
    y = oracle.rope_neox(x, 1234, rd)
    h = rd // 2
    np.testing.assert_allclose(np.hypot(y[:h], y[h:]), np.hypot(x[:h], x[h:]), rtol=1e-13)
    # <rope(q, m), rope(k, n)> depends only on m - n
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    a = np.dot(oracle.rope_neox(q, 700, rd), oracle.rope_neox(k, 300, rd))
    b = np.dot(oracle.rope_neox(q, 1400, rd), oracle.rope_neox(k, 1000, rd))
    assert abs(a - b) < 1e-10
    # complex-number form: z_i = x_i + i x_{i+rd/2} times exp(i * pos * base^(-2i/rd))
    pos = 77
    z = (x[:h] + 1j * x[h:]) * np.exp(1j * pos * 10000.0 ** (-2.0 * np.arange(h) / rd))
    y = oracle.rope_neox(x, pos, rd)
    np.testing.assert_allclose(y[:h], z.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[h:], z.imag, rtol=0, atol=1e-12)


def test_rope_partial_dim_and_neox_pairing():
    D, rd = 128, 64
    x = np.zeros(D)
    x[0] = 1.0  # pairs with x[32] in NeoX, with x[1] in the interleaved form
    y = oracle.rope_neox(x, 1, rd)
    assert y[1] == 0.0 and y[32] != 0.0
    assert abs(y[0] - math.cos(1.0)) < 1e-15 and abs(y[32] - math.sin(1.0)) < 1e-15
    x = np.random.default_rng(6).standard_normal(D)
    y = oracle.rope_neox(x, 999, rd)
    assert np.array_equal(y[rd:], x[rd:])


@pytest.mark.parametrize("rd", [128, 64, 0])
def test_append_writes_one_row_per_head_and_rotates(rd):
    case = append_case(23, 3, 8, 2, 128, 64, F16, rotary_dim=rd, pad="zero")
    kv = okv(case)
    kc, vc, q_rot, after = oracle.append(kv, case.k_new, case.v_new, case.q, case.seq_lens, rd)
    k0 = oracle._bits(case.k)
    v0 = oracle._bits(case.v)
    kn = oracle._bits(case.k_new)
    vn = oracle._bits(case.v_new)
    for b in range(3):
        c = int(case.seq_lens[b])
        for g in range(2):
            assert np.array_equal(vc[b, c, g], vn[b, g])
            if rd:
                want = oracle.from_f64(oracle.rope_neox(oracle.to_f64(kn[b, g], 0), c, rd), 0)
            else:
                want = kn[b, g]
            assert np.array_equal(kc[b, c, g], want)
        keep = np.ones(64, dtype=bool)
        keep[c] = False
        assert np.array_equal(kc[b, keep], k0[b, keep]) and np.array_equal(vc[b, keep], v0[b, keep])
        for h in range(8):
            qd = oracle.to_f64(oracle._bits(case.q)[b, h], 0)
            np.testing.assert_array_equal(q_rot[b, h], oracle.rope_neox(qd, c, rd) if rd else qd)
    # cache_seqlens is an input only
    assert case.seq_lens.dtype == torch.int32


# ---------------------------------------------------------------- worked examples on the pages

def test_golden_split_picture_and_slices():
    (row,) = golden_rows("split_picture_1024.txt")
    n, S, bounds = int(row[0]), int(row[1]), [int(x) for x in row[2:]]
    assert bounds == [n * i // S for i in range(S + 1)]
    (row,) = golden_rows("lpnh_128k_slices.txt")
    n, S, slice_len, B, H, tasks = map(int, row)
    assert n // S == slice_len and B * H * S == tasks


# ---------------------------------------------------------------- float8 caches

def _dequant(case, b, L):
    """K, V of request b as float64 [1, Hkv, L, D], each element times its descale."""
    k = case.k[b, :L].to(torch.float64) * case.k_descale[b].double()[None, :, None]
    v = case.v[b, :L].to(torch.float64) * case.v_descale[b].double()[None, :, None]
    return k.permute(1, 0, 2)[None].contiguous(), v.permute(1, 0, 2)[None].contiguous()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_fp8_cache_matches_torch_sdpa_on_dequantised_values(seed):
    # descales differ per (request, KV head), with B != Hkv so a swapped index shows
    case = contiguous_case(140 + seed, 3, 8, 2, 16, [1, 9, 16], 16, FP8, pad="nan")
    scale = 0.3
    out, lse = oracle.decode(okv(case), case.q, case.seq_lens, scale)
    for b in range(case.B):
        L = int(case.seq_lens[b])
        q = case.q[b].to(torch.float64)[None, :, None, :]
        k, v = _dequant(case, b, L)
        ref = F.scaled_dot_product_attention(q, k, v, scale=scale, enable_gqa=True)[0, :, 0, :]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)
        ones = torch.ones(1, case.Hkv, L + 1, 1, dtype=torch.float64)
        ones[:, :, L] = 0.0
        ksink = torch.cat([k, torch.zeros(1, case.Hkv, 1, case.D, dtype=torch.float64)], dim=2)
        r = F.scaled_dot_product_attention(q, ksink, ones, scale=scale, enable_gqa=True)[0, :, 0, 0].numpy()
        np.testing.assert_allclose(lse[b], np.log(r / (1.0 - r)), rtol=0, atol=1e-10)


def test_fp8_descales_act_as_their_definition():
    case = contiguous_case(150, 2, 8, 2, 16, [12, 5], 16, FP8, pad="nan")
    out, lse = oracle.decode(okv(case), case.q, case.seq_lens, 0.25)
    # V's descale scales the output and leaves the weights alone
    vd = case.v_descale.clone()
    case.v_descale = vd * 4.0
    out4, lse4 = oracle.decode(okv(case), case.q, case.seq_lens, 0.25)
    np.testing.assert_allclose(out4, out * 4.0, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(lse4, lse)
    # K's descale 0 flattens the scores: the mean of the dequantised V, lse = ln L
    case.v_descale = vd
    case.k_descale = torch.zeros_like(case.k_descale)
    out0, lse0 = oracle.decode(okv(case), case.q, case.seq_lens, 0.25)
    for b in range(2):
        L = int(case.seq_lens[b])
        mean = (case.v[b, :L].to(torch.float64) * vd[b].double()[None, :, None]).mean(0).numpy()
        for h in range(8):
            np.testing.assert_allclose(out0[b, h], mean[h // 4], rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse0[b], math.log(L), rtol=0, atol=1e-13)


def test_fp8_cache_equals_bf16_cache_holding_the_same_values():
    # every e4m3 value is a bf16 value: with unit descales the two caches are
    # the same keys and values, so the oracle gives bitwise equal results
    case = paged_case(151, 3, 8, 2, 32, [40, 1, 17], 16, FP8, extra_pages=2, pad="nan")
    case.k_descale = torch.ones_like(case.k_descale)
    case.v_descale = torch.ones_like(case.v_descale)
    o8, l8 = oracle.decode(okv(case), case.q, case.seq_lens, 0.2)
    kb = oracle.KV(case.k.to(BF16), case.v.to(BF16), oracle.BF16, case.Hq, case.B, case.page_size,
                   case.page_table)
    ob, lb = oracle.decode(kb, case.q, case.seq_lens, 0.2)
    np.testing.assert_array_equal(o8, ob)
    np.testing.assert_array_equal(l8, lb)


# ---------------------------------------------------------------- cache_batch_idx and cache_leftpad

def _sdpa_rows(q, k, v, scale):
    """float64 attention of q [Hq, D] over rows k, v [L, Hkv, D] (torch), and its LSE."""
    qq = q.to(torch.float64)[None, :, None, :]
    kk = k.to(torch.float64).permute(1, 0, 2)[None].contiguous()
    vv = v.to(torch.float64).permute(1, 0, 2)[None].contiguous()
    out = F.scaled_dot_product_attention(qq, kk, vv, scale=scale, enable_gqa=True)[0, :, 0, :]
    s = torch.einsum("hd,hld->hl", qq[0, :, 0, :],
                     kk[0].repeat_interleave(q.shape[0] // k.shape[1], dim=0)) * scale
    return out.numpy(), torch.logsumexp(s, dim=-1).numpy()


def test_cache_batch_idx_reads_the_indexed_rows():
    # 3 requests over a 5-row cache; rows no request names hold NaN
    g = torch.Generator().manual_seed(160)
    Bc, cap, Hkv, D, Hq = 5, 24, 2, 16, 8
    k = torch.randn(Bc, cap, Hkv, D, generator=g).to(BF16)
    v = torch.randn(Bc, cap, Hkv, D, generator=g).to(BF16)
    idx = torch.tensor([4, 0, 2], dtype=torch.int32)
    lens = torch.tensor([24, 7, 1], dtype=torch.int32)
    for r in (1, 3):
        k[r] = float("nan")
        v[r] = float("nan")
    q = torch.randn(3, Hq, D, generator=g).to(BF16)
    kv = oracle.KV(k, v, oracle.BF16, Hq, 3, batch_idx=idx)
    out, lse = oracle.decode(kv, q, lens, 0.3)
    for b in range(3):
        L, r = int(lens[b]), int(idx[b])
        ro, rl = _sdpa_rows(q[b], k[r, :L], v[r, :L], 0.3)
        np.testing.assert_allclose(out[b], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("paged", [False, True])
def test_cache_leftpad_attends_to_the_rows_after_the_padding(paged):
    lens, pads = [40, 9, 17, 30], [0, 5, 17, 29]  # request 2: all rows padding -> empty
    if paged:
        case = paged_case(161, 4, 8, 2, 16, lens, 16, BF16, extra_pages=2, pad="nan")
    else:
        case = contiguous_case(161, 4, 8, 2, 16, lens, 40, BF16, pad="nan")
    lp = torch.tensor(pads, dtype=torch.int32)
    for b, p in enumerate(pads):  # the padding rows hold NaN: reading one poisons the result
        for j in range(p):
            if paged:
                case.k[int(case.page_table[b, j // 16]), j % 16] = float("nan")
            else:
                case.k[b, j] = float("nan")
    kv = oracle.KV(case.k, case.v, oracle.BF16, 8, 4, case.page_size, case.page_table, leftpad=lp)
    out, lse = oracle.decode(kv, case.q, case.seq_lens, 0.25)
    for b in range(4):
        rows = range(pads[b], lens[b])
        if not len(rows):
            assert np.all(out[b] == 0) and np.all(lse[b] == -np.inf)
            continue
        if paged:
            kr = torch.stack([case.k[int(case.page_table[b, j // 16]), j % 16] for j in rows])
            vr = torch.stack([case.v[int(case.page_table[b, j // 16]), j % 16] for j in rows])
        else:
            kr, vr = case.k[b, pads[b]:lens[b]], case.v[b, pads[b]:lens[b]]
        ro, rl = _sdpa_rows(case.q[b], kr, vr, 0.25)
        np.testing.assert_allclose(out[b], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl, rtol=0, atol=1e-12)
    # split states clipped at the padding merge to the same result
    S = 3
    bounds = np.array([[p + i * 8 for i in range(S)] + [64] for p in pads], dtype=np.int32)
    bounds[:, 0] = 0  # a first bound inside the padding is clipped to it
    po, pm, pd = oracle.partials(kv, case.q, case.seq_lens, 0.25, bounds)
    mo, ml = oracle.merge(po, pm, pd)
    np.testing.assert_allclose(mo, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(ml[np.isfinite(lse)], lse[np.isfinite(lse)], rtol=0, atol=1e-13)


def test_append_with_leftpad_and_batch_idx():
    # the new row goes to row c of cache row batch_idx[b], rotated at its
    # position among the valid rows, c - leftpad[b]; q is rotated alike
    case = append_case(162, 3, 8, 2, 128, 64, F16, rotary_dim=128, pad="zero")
    idx = torch.tensor([2, 0, 1], dtype=torch.int32)
    c = case.seq_lens
    lp = torch.minimum(torch.tensor([3, 0, 11], dtype=torch.int32), c)
    kv = oracle.KV(case.k, case.v, oracle.F16, 8, 3, batch_idx=idx, leftpad=lp)
    kc, vc, q_rot, after = oracle.append(kv, case.k_new, case.v_new, case.q, c, 128)
    kn, vn = oracle._bits(case.k_new), oracle._bits(case.v_new)
    for b in range(3):
        r, cb, pos = int(idx[b]), int(c[b]), int(c[b]) - int(lp[b])
        for g in range(2):
            want = oracle.from_f64(oracle.rope_neox(oracle.to_f64(kn[b, g], 0), pos, 128), 0)
            assert np.array_equal(kc[r, cb, g], want) and np.array_equal(vc[r, cb, g], vn[b, g])
        qd = oracle.to_f64(oracle._bits(case.q)[b], 0)
        for h in range(8):
            np.testing.assert_array_equal(q_rot[b, h], oracle.rope_neox(qd[h], pos, 128))
    # attention after the append covers rows [leftpad, c] of the indexed cache row
    out, lse = oracle.decode(after, q_rot, c + 1, 1 / math.sqrt(128))
    for b in range(3):
        r = int(idx[b])
        kr = torch.from_numpy(oracle.to_f64(kc[r, int(lp[b]):int(c[b]) + 1], 0))
        vr = torch.from_numpy(oracle.to_f64(vc[r, int(lp[b]):int(c[b]) + 1], 0))
        ro, rl = _sdpa_rows(torch.from_numpy(q_rot[b]), kr, vr, 1 / math.sqrt(128))
        np.testing.assert_allclose(out[b], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl, rtol=0, atol=1e-12)


@pytest.mark.parametrize("rd,paged", [(0, False), (128, False), (64, True)])
def test_fp8_append_stores_quantised_rows(rd, paged):
    # a float8 cache stores code(value / descale): for v and an unrotated k that
    # is torch's cast of the bf16 input divided in float32; a rotated k is the
    # rotated value (rounded to float32) divided alike; nothing else changes
    case = append_case(171 + rd, 3, 8, 2, 128, 64, FP8, rotary_dim=rd, pad="zero", page_size=16 if paged else 0)
    kv = okv(case)
    kc, vc, q_rot, after = oracle.append(kv, case.k_new, case.v_new, case.q, case.seq_lens, rd)
    k0, v0 = oracle._bits(case.k), oracle._bits(case.v)
    kn = case.k_new.to(torch.float32).numpy()
    vn = case.v_new.to(torch.float32).numpy()
    kd, vd = case.k_descale.numpy(), case.v_descale.numpy()
    changed = np.zeros(k0.shape[:2], dtype=bool)
    for b in range(3):
        c = int(case.seq_lens[b])
        if paged:
            pg, sl = int(case.page_table[b, c // 16]), c % 16
        else:
            pg, sl = b, c
        changed[pg, sl] = True
        for g in range(2):
            assert np.array_equal(vc[pg, sl, g], _torch_f8(vn[b, g] / np.float32(vd[b, g])))
            kval = oracle.rope_neox(kn[b, g].astype(np.float64), c, rd).astype(np.float32) if rd else kn[b, g]
            assert np.array_equal(kc[pg, sl, g], _torch_f8(kval / np.float32(kd[b, g])))
    assert np.array_equal(kc[~changed], k0[~changed]) and np.array_equal(vc[~changed], v0[~changed])
    # decode after the append reads the written codes times the descales
    scale = 1 / math.sqrt(128)
    out, lse = oracle.decode(after, q_rot, case.seq_lens + 1, scale)
    for b in range(3):
        L = int(case.seq_lens[b]) + 1
        rows = [(int(case.page_table[b, j // 16]), j % 16) if paged else (b, j) for j in range(L)]
        kr = np.stack([oracle.to_f64(kc[p_, s_], oracle.FP8) for p_, s_ in rows], axis=1)  # [Hkv, L, D]
        vr = np.stack([oracle.to_f64(vc[p_, s_], oracle.FP8) for p_, s_ in rows], axis=1)
        kr = torch.from_numpy(kr * kd[b][:, None, None])
        vr = torch.from_numpy(vr * vd[b][:, None, None])
        qb = torch.from_numpy(q_rot[b])[None, :, None, :]
        ref = F.scaled_dot_product_attention(qb, kr[None], vr[None], scale=scale, enable_gqa=True)[0, :, 0, :]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- multi-token (speculative) decode

@pytest.mark.parametrize("paged", [False, True])
def test_multi_token_decode_matches_sdpa_with_causal_mask(paged):
    # token i of request b is row L_b - q_len + i and sees rows [leftpad, that row];
    # request 2 is shorter than q_len, so its first token sees nothing
    q_len, lens, pads = 3, [20, 5, 2], [0, 1, 0]
    if paged:
        case = paged_case(170, 3, 8, 2, 16, lens, 16, BF16, extra_pages=2, pad="nan")
    else:
        case = contiguous_case(170, 3, 8, 2, 16, lens, 20, BF16, pad="nan")
    g = torch.Generator().manual_seed(171)
    q = torch.randn(3, q_len, 8, 16, generator=g).to(BF16)
    lp = torch.tensor(pads, dtype=torch.int32)
    kv = oracle.KV(case.k, case.v, oracle.BF16, 8, 3, case.page_size, case.page_table, leftpad=lp)
    out, lse = oracle.decode_multi(kv, q, case.seq_lens, 0.3)
    assert out.shape == (3, q_len, 8, 16) and lse.shape == (3, 8, q_len)
    for b in range(3):
        L = lens[b]
        if paged:
            rows = [(int(case.page_table[b, j // 16]), j % 16) for j in range(L)]
            kb = torch.stack([case.k[p, s] for p, s in rows]) if L else case.k[:0, 0]
            vb = torch.stack([case.v[p, s] for p, s in rows]) if L else case.v[:0, 0]
        else:
            kb, vb = case.k[b, :L], case.v[b, :L]
        kk = kb.to(torch.float64).permute(1, 0, 2)[None].contiguous()
        vv = vb.to(torch.float64).permute(1, 0, 2)[None].contiguous()
        qq = q[b].to(torch.float64).permute(1, 0, 2)[None].contiguous()  # [1, Hq, q_len, D]
        j = torch.arange(L)
        mask = torch.stack([(j >= pads[b]) & (j <= L - q_len + i) for i in range(q_len)])  # [q_len, L]
        for i in range(q_len):
            if not bool(mask[i].any()):
                assert np.all(out[b, i] == 0) and np.all(lse[b, :, i] == -np.inf)
                continue
            kk_i = torch.nan_to_num(kk[:, :, mask[i]])  # only the rows token i sees
            vv_i = vv[:, :, mask[i]]
            ref = F.scaled_dot_product_attention(qq[:, :, i:i + 1], kk_i, vv_i, scale=0.3, enable_gqa=True)
            np.testing.assert_allclose(out[b, i], ref[0, :, 0].numpy(), rtol=0, atol=1e-12)
            s = torch.einsum("hd,hld->hl", qq[0, :, i], kk_i[0].repeat_interleave(4, dim=0)) * 0.3
            np.testing.assert_allclose(lse[b, :, i], torch.logsumexp(s, dim=-1).numpy(), rtol=0, atol=1e-12)


def test_multi_token_with_one_token_is_single_query_decode():
    case = paged_case(172, 3, 8, 2, 32, [40, 1, 17], 16, F16, extra_pages=1, pad="nan")
    kv = okv(case)
    out1, lse1 = oracle.decode(kv, case.q, case.seq_lens, 0.2)
    outm, lsem = oracle.decode_multi(kv, case.q[:, None], case.seq_lens, 0.2)
    np.testing.assert_array_equal(outm[:, 0], out1)
    np.testing.assert_array_equal(lsem[:, :, 0], lse1)
