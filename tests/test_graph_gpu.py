"""The other entry points captured in a HIP graph, through the C ABI.

Each case captures one call (the shared-prefix cascade on either merge path and
with a float8 pool, multi-token decode on both matrix-core kernels, its balanced
split, the balanced split on a float8 cache, and the float8 append) and replays
it four times, with eager work and synchronisations between the replays. Every
replay and every eager call in between must give the first eager result bit for
bit: nothing a call leaves in its workspace may change the next one, and no call
records a memset node.
"""
import pytest
import torch

import decode_attention_fdec_amd as F
from synth import BF16, F16, FP8, append_case, cascade_case, multi_query, paged_case
from helpers import to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


@pytest.fixture(scope="module", autouse=True)
def _gpu(fdec):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()


def _cascade(seed, G, dtype):
    case = cascade_case(seed, 6, 4 * G, 4, 128, 700, 64, suffix_lens=[0, 5, 130, 64, 1, 300], dtype=dtype,
                        pad="nan", extra_pages=2)
    d = to_dev(case)
    B, Hq, D = case.q.shape
    sp, ss = 5, 7
    ws = F.Workspace(F.cascade_workspace_size(B, Hq, case.Hkv, D, sp, ss), DEV)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)

    def step():
        F.cascade_decode(d["q"], d["k"], d["v"], d["page_table"], d["prefix_pages"], case.prefix_len,
                         d["seq_lens"], sp, ss, out=out, lse=lse, workspace=ws, k_descale=d["k_descale"],
                         v_descale=d["v_descale"])
    return step, (out, lse), None


def _multi(seed, G, q_len, dtype, balanced):
    case = paged_case(seed, 4, 8 * G, 8, 128, [900, 3, 64, 1500], 16, dtype, extra_pages=2, pad="nan")
    d = to_dev(case)
    q = multi_query(seed + 1, case, q_len).to(DEV)
    B, Hq, D = case.q.shape
    out = torch.empty(B, q_len, Hq, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, Hq, q_len, dtype=torch.float32, device=DEV)
    kw = dict(page_table=d["page_table"], out=out, lse=lse, k_descale=d["k_descale"], v_descale=d["v_descale"])
    if balanced:
        nb = 40
        ws = F.Workspace(F.balanced_workspace_size(B, q_len * Hq, case.Hkv, D, nb), DEV)

        def step():
            F.decode_multi_balanced(q, d["k"], d["v"], d["seq_lens"], num_blocks=nb, workspace=ws, **kw)
    else:
        S = 9
        ws = F.Workspace(F.workspace_size(B * q_len, Hq, case.Hkv, D, S), DEV)

        def step():
            F.decode_multi(q, d["k"], d["v"], d["seq_lens"], num_splits=S, workspace=ws, **kw)
    return step, (out, lse), None


def _balanced_fp8():
    case = paged_case(331, 5, 32, 8, 128, [2000, 1, 16, 700, 0], 16, FP8, extra_pages=2, pad="nan")
    d = to_dev(case)
    B, Hq, D = case.q.shape
    nb = 48
    ws = F.Workspace(F.balanced_workspace_size(B, Hq, case.Hkv, D, nb), DEV)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)

    def step():
        F.decode_balanced(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_blocks=nb,
                          out=out, lse=lse, workspace=ws, k_descale=d["k_descale"], v_descale=d["v_descale"])
    return step, (out, lse), None


def _append_fp8(G, fused):
    case = append_case(341 + G, 3, 8 * G, 8, 128, 400, FP8, rotary_dim=64, pad="nan", cache_seqlens=[0, 150, 399],
                       page_size=16)
    d = to_dev(case)
    B, Hq, D = case.q.shape
    S = 5
    a = F.make_append(d["k_new"], d["v_new"], d["rope_cos"], d["rope_sin"], case.rotary_dim)
    ws = F.Workspace(F.workspace_size(B, Hq, case.Hkv, D, S), DEV)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, Hq, dtype=torch.float32, device=DEV)
    k0, v0 = d["k"].clone(), d["v"].clone()

    def step():
        F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=S, append=a,
                 fused=fused, out=out, lse=lse, workspace=ws, k_descale=d["k_descale"], v_descale=d["v_descale"])

    def restore():  # the append rewrites the same rows each call
        d["k"].copy_(k0)
        d["v"].copy_(v0)
    return step, (out, lse, d["k"], d["v"]), restore


CASES = {
    "cascade_g4_bf16": lambda: _cascade(301, 4, BF16),
    "cascade_g4_fp8": lambda: _cascade(302, 4, FP8),
    "cascade_g2_f16": lambda: _cascade(303, 2, F16),      # uniform merge path
    "multi_q3_g4_bf16": lambda: _multi(311, 4, 3, BF16, False),   # 16x16x32 kernel
    "multi_q2_g4_fp8": lambda: _multi(312, 4, 2, FP8, False),     # 4x4x4 kernel
    "multi_bal_q4_g2_f16": lambda: _multi(313, 2, 4, F16, True),
    "balanced_g4_fp8": _balanced_fp8,
    "append_fp8_g4_two": lambda: _append_fp8(4, False),
    "append_fp8_g2_fused": lambda: _append_fp8(2, True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_match_eager_bitwise(name):
    step, outs, restore = CASES[name]()
    if restore:
        restore()
    step()
    torch.cuda.synchronize()
    bits = lambda t: t.contiguous().view(torch.uint8)  # NaN padding in the caches compares by bits
    ref = [bits(t).clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    if restore:
        restore()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    for i in range(4):
        for t in outs[:2]:
            t.zero_()
        if restore:
            restore()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(bits(t), r), f"{name}: replay {i}, output {j}"
        if restore:
            restore()
        step()  # eager work between replays
        torch.cuda.synchronize()
        for j, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(bits(t), r), f"{name}: eager call after replay {i}, output {j}"
