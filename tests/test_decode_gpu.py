"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Sizes here span several 16-token tiles, several splits and ragged tails; the
full workload sizes are at the end. Padding rows and unused pages hold NaN, so
any read past a request's length shows up as a non-finite output.
"""
import math

import numpy as np
import pytest
import torch

import decode_attention_fdec_amd as F
import oracle
from helpers import LSE_RTOL, OUT_TOL, assert_parity, check_append_k, okv, oracle_decode, to_dev
from synth import BF16, F16, FP8, append_case, contiguous_case, paged_case, workload

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    oracle.build(force=False)
    torch.cuda.init()


def run(case, num_splits=0, fused=False, scale=0.0):
    d = to_dev(case)
    out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                        num_splits=num_splits, fused=fused, softmax_scale=scale)
    torch.cuda.synchronize()
    return out, lse


# ---------------------------------------------------------------- merge stage alone

@pytest.mark.parametrize("S", [1, 2, 7, 64, 256])
def test_merge_kernel_matches_oracle_merge(S):
    rng = np.random.default_rng(S)
    B, Hq, D = 3, 8, 128
    pm = rng.standard_normal((B, Hq, S)) * 5
    pd = rng.uniform(0.5, 50, (B, Hq, S))
    po = rng.standard_normal((B, Hq, S, D)) * pd[..., None]
    if S > 2:
        pm[0, 0, 1] = -np.inf  # empty states
        pd[0, 0, 1] = 0.0
        po[0, 0, 1] = 0.0
    pm[2, 3, :] = -np.inf  # every state empty
    pd[2, 3, :] = 0.0
    po[2, 3] = 0.0
    po32, pm32, pd32 = (torch.tensor(x, dtype=torch.float32) for x in (po, pm, pd))
    ref_out, ref_lse = oracle.merge(po32.double().numpy(), pm32.double().numpy(), pd32.double().numpy())
    out, lse = F.merge_states(po32.to(DEV), pm32.to(DEV), pd32.to(DEV))
    torch.cuda.synchronize()
    o, l = out.cpu().double().numpy(), lse.cpu().double().numpy()
    np.testing.assert_allclose(o, ref_out, rtol=1e-5, atol=1e-5)
    fin = np.isfinite(ref_lse)
    np.testing.assert_allclose(l[fin], ref_lse[fin], rtol=1e-6, atol=1e-6)
    assert np.all(l[~fin] == -np.inf) and np.all(o[2, 3] == 0.0)


# ---------------------------------------------------------------- map stage alone

@pytest.mark.parametrize("paged", [False, True])
def test_map_stage_states_match_oracle_states(paged):
    lens = [1, 33, 300, 1000]
    if paged:
        case = paged_case(31, 4, 32, 8, 128, lens, 16, BF16, max_pages=64, extra_pages=5, pad="nan")
    else:
        case = contiguous_case(31, 4, 32, 8, 128, lens, 1024, BF16, pad="nan")
    S = 5
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
    assert err.max() < 3e-3


# ---------------------------------------------------------------- full decode, small shapes

SMALL = [
    # (name, builder)
    ("mha_f16", lambda: contiguous_case(41, 2, 8, 8, 128, [1000, 77], 1000, F16, pad="nan")),
    ("gqa4_bf16", lambda: contiguous_case(42, 3, 32, 8, 128, [513, 1, 2000], 2048, BF16, pad="nan")),
    ("gqa2_f16", lambda: contiguous_case(43, 2, 8, 4, 128, [129, 400], 400, F16, pad="nan")),
    ("gqa8_bf16", lambda: contiguous_case(44, 2, 16, 2, 128, [700, 31], 768, BF16, pad="nan")),
    ("d64_f16", lambda: contiguous_case(45, 2, 16, 4, 64, [999, 64], 1000, F16, pad="nan")),
    ("d64_bf16_g8", lambda: contiguous_case(46, 1, 16, 2, 64, [333], 333, BF16, pad="nan")),
    ("paged16_bf16", lambda: paged_case(47, 4, 32, 8, 128, [17, 500, 1024, 3], 16, BF16, extra_pages=7,
                                        pad="nan")),
    ("paged32_f16", lambda: paged_case(48, 3, 16, 4, 128, [31, 250, 1000], 32, F16, extra_pages=3, pad="nan")),
    ("paged64_bf16_g1", lambda: paged_case(49, 2, 8, 8, 128, [64, 640], 64, BF16, extra_pages=2, pad="nan")),
    ("paged48_f16", lambda: paged_case(50, 2, 8, 2, 128, [100, 47], 48, F16, extra_pages=2, pad="nan")),
]


@pytest.mark.parametrize("name,builder", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("num_splits", [1, 3, 16, 0])
def test_decode_matches_oracle(name, builder, num_splits):
    case = builder()
    ref_out, ref_lse = oracle_decode(case)
    out, lse = run(case, num_splits=num_splits)
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{name} S={num_splits}")


@pytest.mark.parametrize("name,builder", SMALL[:2] + SMALL[6:7], ids=["mha_f16", "gqa4_bf16", "paged16"])
def test_fused_single_kernel_is_bitwise_equal_to_two_kernels(name, builder):
    case = builder()
    for S in (1, 4, 13, 64):
        o1, l1 = run(case, num_splits=S, fused=False)
        o2, l2 = run(case, num_splits=S, fused=True)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"{name} S={S}"


def test_fused_counters_return_to_zero_and_runs_repeat_bitwise():
    case = contiguous_case(51, 2, 32, 8, 128, [3000, 1500], 4096, BF16, pad="nan")
    d = to_dev(case)
    S = 24
    ws = F.Workspace(F.workspace_size(2, 32, 8, 128, S), DEV)
    outs = []
    for _ in range(5):
        o, l = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=S, fused=True, workspace=ws)
        outs.append((o.clone(), l.clone()))
    torch.cuda.synchronize()
    cnt = ws.buf[: 2 * 8 * 4].view(torch.int32)
    assert torch.count_nonzero(cnt).item() == 0
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_empty_and_single_token_requests():
    case = contiguous_case(52, 3, 8, 2, 128, [0, 1, 16], 64, F16, pad="nan")
    ref_out, ref_lse = oracle_decode(case)
    for fused in (False, True):
        out, lse = run(case, num_splits=4, fused=fused)
        o = out.cpu()
        assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse.cpu()[0]))
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"fused={fused}")


def test_custom_softmax_scale():
    case = contiguous_case(53, 1, 8, 8, 128, [600], 600, F16, pad="nan")
    ref_out, ref_lse = oracle_decode(case, scale=0.05)
    out, lse = run(case, num_splits=5, scale=0.05)
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, "scale 0.05")


def test_strided_cache_view():
    # a [B, cap, 2, Hkv, D] cache (K and V interleaved per token), addressed through strides
    g = torch.Generator().manual_seed(54)
    B, cap, Hkv, D = 2, 300, 4, 128
    kv = torch.randn(B, cap, 2, Hkv, D, generator=g).to(F16)
    q = torch.randn(B, 16, D, generator=g).to(F16)
    lens = torch.tensor([300, 123], dtype=torch.int32)
    k, v = kv[:, :, 0], kv[:, :, 1]
    ref = oracle.decode(oracle.KV(k.contiguous(), v.contiguous(), oracle.F16, 16, B), q, lens, 1 / math.sqrt(D))
    kd = kv.to(DEV)
    out, lse = F.decode(q.to(DEV), kd[:, :, 0], kd[:, :, 1], lens.to(DEV), num_splits=3)
    torch.cuda.synchronize()
    assert_parity(out, lse, ref[0], ref[1], F16, "strided")


# ---------------------------------------------------------------- gather is exact

@pytest.mark.parametrize("paged", [False, True])
def test_one_hot_scores_return_the_value_row_bitwise(paged):
    B, Hq, Hkv, D, L = 2, 8, 2, 128, 700
    if paged:
        case = paged_case(55, B, Hq, Hkv, D, [L, L - 13], 16, F16, extra_pages=4, pad="nan")
    else:
        case = contiguous_case(55, B, Hq, Hkv, D, [L, L - 13], L, F16, pad="nan")
    case.q.zero_()
    case.q[:, :, 0] = 40.0
    jstar = [[611, 5], [0, 686]]  # per (request, KV head)
    for b in range(B):
        for g in range(Hkv):
            for j in range(int(case.seq_lens[b])):
                if paged:
                    p, s = int(case.page_table[b, j // 16]), j % 16
                    case.k[p, s, g, 0] = 40.0 if j == jstar[b][g] else 0.0
                else:
                    case.k[b, j, g, 0] = 40.0 if j == jstar[b][g] else 0.0
    for S in (1, 7):
        out, lse = run(case, num_splits=S)
        o = out.cpu()
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                j = jstar[b][g]
                if paged:
                    row = case.v[int(case.page_table[b, j // 16]), j % 16, g]
                else:
                    row = case.v[b, j, g]
                assert torch.equal(o[b, h], row.float()), f"b={b} h={h} S={S}"
                assert abs(float(lse[b, h]) - 1600 / math.sqrt(D)) < 1e-4


def test_paged_output_is_bitwise_equal_to_contiguous():
    B, Hq, Hkv, D, ps = 3, 32, 8, 128, 16
    cont = contiguous_case(56, B, Hq, Hkv, D, [1024, 77, 500], 1024, BF16, pad="nan")
    # same logical rows in a permuted page pool of equal capacity
    g = torch.Generator().manual_seed(57)
    npg = 1024 // ps
    perm = torch.randperm(B * npg, generator=g).to(torch.int32)
    table = perm.view(B, npg).contiguous()
    kp = torch.full((B * npg, ps, Hkv, D), float("nan"), dtype=BF16)
    vp = kp.clone()
    for b in range(B):
        for i in range(npg):
            kp[int(table[b, i])] = cont.k[b, i * ps:(i + 1) * ps]
            vp[int(table[b, i])] = cont.v[b, i * ps:(i + 1) * ps]
    d = to_dev(cont)
    for S in (1, 5, 32):
        o1, l1 = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], num_splits=S)
        o2, l2 = F.decode(d["q"], kp.to(DEV), vp.to(DEV), d["seq_lens"], page_table=table.to(DEV), num_splits=S)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), f"S={S}"


# ---------------------------------------------------------------- append + rotary

def _append_run(case, num_splits, fused=False):
    d = to_dev(case)
    a = F.make_append(d["k_new"], d["v_new"], d["rope_cos"], d["rope_sin"], case.rotary_dim)
    out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"],
                        num_splits=num_splits, append=a, fused=fused)
    torch.cuda.synchronize()
    return out, lse, d["k"].cpu(), d["v"].cpu(), d["seq_lens"].cpu()


def _append_oracle(case):
    kc, vc, q_rot, after = oracle.append(okv(case), case.k_new, case.v_new, case.q, case.seq_lens,
                                         case.rotary_dim, case.rope_base)
    ref_out, ref_lse = oracle.decode(after, q_rot, case.seq_lens + 1, 1 / math.sqrt(case.D))
    return kc, vc, ref_out, ref_lse


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("rd,paged,S", [(128, False, 4), (64, False, 1), (0, False, 7), (128, True, 3),
                                        (0, True, 2)])
def test_append_writes_rows_and_attends(rd, paged, S):
    case = append_case(61, 3, 16, 4, 128, 300, F16, rotary_dim=rd, pad="nan", page_size=16 if paged else 0,
                       cache_seqlens=[0, 150, 299])
    kc, vc, ref_out, ref_lse = _append_oracle(case)
    k0 = _bits(case.k)
    out, lse, kg, vg, lens_after = _append_run(case, S)
    assert torch.equal(lens_after, case.seq_lens)  # lengths are never advanced
    kg, vg = _bits(kg), _bits(vg)
    # v rows and every untouched k row are bit-exact; the rotated k row within 1 fp16 ulp
    assert np.array_equal(vg, vc)
    check_append_k(kg, kc, case, f"append rd={rd}")
    if rd == 0:
        assert np.array_equal(kg, kc)
    assert not np.array_equal(kg, k0)  # the rows were written
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"append rd={rd}")


@pytest.mark.parametrize("rd,paged,S,fused", [(128, False, 4, False), (64, True, 3, False), (0, False, 1, True),
                                              (128, True, 7, True)])
def test_append_groups_of_eight(rd, paged, S, fused):
    # eight query heads per KV head: two groups of four through the matrix-core append kernel
    case = append_case(63, 3, 32, 4, 128, 300, BF16, rotary_dim=rd, pad="nan", page_size=16 if paged else 0,
                       cache_seqlens=[0, 150, 299])
    kc, vc, ref_out, ref_lse = _append_oracle(case)
    out, lse, kg, vg, _ = _append_run(case, S, fused=fused)
    kg, vg = _bits(kg), _bits(vg)
    assert np.array_equal(vg, vc)
    check_append_k(kg, kc, case, f"append G=8 rd={rd}")
    if rd == 0:
        assert np.array_equal(kg, kc)
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"append G=8 rd={rd}")


def test_append_rotated_rows_mostly_bit_exact():
    case = workload("c4", pad="nan")
    kc, vc, ref_out, ref_lse = _append_oracle(case)
    out, lse, kg, vg, _ = _append_run(case, 0)
    kg = _bits(kg)
    n1 = check_append_k(kg, kc, case, "c4")
    n_rows = case.B * case.Hkv * case.D  # elements of the appended rows
    assert n1 <= max(4, n_rows // 100), f"{n1} of {n_rows} appended elements differ by 1 ulp"
    assert np.array_equal(_bits(vg), vc)
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, "c4")


# ---------------------------------------------------------------- full-size workloads

@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c2g8"])
def test_full_size_workload_matches_oracle(name):
    case = workload(name, pad="nan")
    ref_out, ref_lse = oracle_decode(case)
    S = case.num_splits
    for fused in (False, True):
        out, lse = run(case, num_splits=S, fused=fused)
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"{name} fused={fused}")


def test_c2_fixed_16_splits_equals_planned_splits():
    # the explainer's 128k context in 16 slices of 8k versus the planner's choice
    case = workload("c2")
    S_plan = F.plan(1, 32, 8, None, 131072)
    o16, l16 = run(case, num_splits=16)
    op, lp = run(case, num_splits=S_plan)
    assert (o16 - op).abs().max().item() < 1e-4
    assert ((l16 - lp).abs() / l16.abs().clamp(min=1)).max().item() < 1e-6


# ---------------------------------------------------------------- graph capture

@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", ["gqa4_paged", "gqa2_contig", "append_rope", "fp8_gqa2_paged"])
def test_graph_replays_match_eager_bitwise(name, fused):
    # one step captured as a HIP graph and replayed several times, with eager
    # work and synchronisations between the replays; every replay must give
    # the eager result bit for bit (no memset nodes: the fused path's counters
    # return to zero by themselves)
    append = None
    if name == "gqa4_paged":
        case = paged_case(58, 3, 32, 8, 128, [700, 33, 1500], 16, BF16, extra_pages=3, pad="nan")
    elif name == "gqa2_contig":
        case = contiguous_case(59, 2, 16, 8, 128, [999, 250], 1024, F16, pad="nan")
    elif name == "fp8_gqa2_paged":  # float8 on the vector kernel, unit descales
        case = paged_case(61, 3, 16, 8, 128, [700, 33, 1500], 16, FP8, extra_pages=3, pad="nan")
    else:
        case = append_case(60, 2, 32, 8, 128, 512, F16, rotary_dim=128, base=10000.0, pad="nan")
    d = to_dev(case)
    B, Hq, D = case.q.shape
    S = 7
    if case.k_new is not None:
        append = F.make_append(d["k_new"], d["v_new"], d["rope_cos"], d["rope_sin"], case.rotary_dim)
    k0, v0 = d["k"].clone(), d["v"].clone()
    ws = F.Workspace(F.workspace_size(B, Hq, case.Hkv, D, S), DEV)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)

    def step():
        F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=S,
                 append=append, fused=fused, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for i in range(4):
        out.zero_()
        lse.zero_()
        if append is not None:  # the append rewrites the same rows each replay
            d["k"].copy_(k0)
            d["v"].copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        step()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o)
    if fused:
        assert torch.count_nonzero(ws.buf[: B * case.Hkv * 4].view(torch.int32)).item() == 0


# ---------------------------------------------------------------- num_splits = 0 through the C ABI

@pytest.mark.parametrize("kind", ["paged_bf16", "contig_f16_mha"])
def test_num_splits_zero_plans_inside_the_library(kind):
    """fdec_decode with num_splits = 0 plans from the capacity alone ("Inference
    Cookbook" §6.2: 0 = automatic) without reading device memory. A C caller sizes
    the workspace with fdec_plan_kv then fdec_workspace_size; the call equals the
    binding's call at that split count bitwise, and one byte less of workspace is
    rejected before any launch."""
    import ctypes

    if kind == "paged_bf16":
        case = paged_case(71, 5, 32, 8, 128, [3000, 17, 0, 900, 2048], 16, BF16, extra_pages=3, pad="nan")
    else:
        case = contiguous_case(72, 2, 32, 32, 128, [4000, 1300], 4096, F16, pad="nan")
    lib = F.load_library()
    d = to_dev(case)
    kv = F.make_kv(d["k"], d["v"], d["page_table"])
    S = ctypes.c_int(0)
    assert lib.fdec_plan_kv(case.B, case.Hq, case.Hkv, None, kv.capacity, kv.page_size, kv.dtype, 256,
                            ctypes.byref(S)) == 0
    assert S.value >= 1
    n = lib.fdec_workspace_size(case.B, case.Hq, case.Hkv, case.D, S.value)
    ws = F.Workspace(n)
    out = torch.empty(case.B, case.Hq, case.D, dtype=torch.float32, device="cuda")
    lse = torch.empty(case.B, case.Hq, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    short = lib.fdec_decode(d["q"].data_ptr(), case.B, case.Hq, ctypes.byref(kv), d["seq_lens"].data_ptr(), 0, 0.0,
                            None, 0, out.data_ptr(), lse.data_ptr(), ws.buf.data_ptr(), n - 1, stream)
    assert short == F.FDEC_ERR_WORKSPACE
    rc = lib.fdec_decode(d["q"].data_ptr(), case.B, case.Hq, ctypes.byref(kv), d["seq_lens"].data_ptr(), 0, 0.0,
                         None, 0, out.data_ptr(), lse.data_ptr(), ws.buf.data_ptr(), n, stream)
    assert rc == 0, lib.fdec_last_error()
    o2, l2 = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=S.value)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    ref_out, ref_lse = oracle_decode(case)
    assert_parity(out, lse, ref_out, ref_lse, case.dtype, f"num_splits=0 {kind}")
