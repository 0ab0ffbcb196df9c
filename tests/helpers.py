"""Shared test helpers: oracle views of synthetic cases and the parity bar.

The tolerances are the parity bar for floating point: max-abs error of the
output <= 1e-3 with fp16 KV and <= 3e-3 with bf16 KV; LSE within 1e-4
relative, with the relative error taken against max(|lse|, 1) so that an LSE
near zero (a single token, tiny tests) is not held to an absolute 1e-12.
"""
import math

import numpy as np
import torch

import oracle
from synth import FP8

OUT_TOL = {torch.float16: 1e-3, torch.bfloat16: 3e-3, torch.float8_e4m3fn: 3e-3}  # float8 caches: bf16 queries
LSE_RTOL = 1e-4


def okv(case, k=None, v=None):
    return oracle.KV(case.k if k is None else k, case.v if v is None else v, oracle.dtype_code(case.k),
                     case.Hq, case.B, case.page_size, case.page_table, case.prefix_pages, case.prefix_len,
                     case.k_descale, case.v_descale, case.cache_batch_idx, case.cache_leftpad)


def oracle_decode(case, scale=None, nthreads=0):
    scale = 1.0 / math.sqrt(case.D) if scale is None else scale
    return oracle.decode(okv(case), case.q, case.seq_lens, scale, nthreads)


def assert_parity(out, lse, ref_out, ref_lse, dtype, what=""):
    out = out.detach().cpu().double().numpy()
    err = np.abs(out - ref_out)
    tol = OUT_TOL[dtype]
    assert np.isfinite(out).all(), f"{what}: non-finite output"
    assert err.max() <= tol, f"{what}: max-abs out error {err.max():.3g} > {tol}"
    if lse is not None:
        lse = lse.detach().cpu().double().numpy()
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(lse), fin), f"{what}: lse finiteness differs"
        assert np.all(lse[~fin] == ref_lse[~fin])
        rel = np.abs(lse[fin] - ref_lse[fin]) / np.maximum(np.abs(ref_lse[fin]), 1.0)
        if rel.size:
            assert rel.max() <= LSE_RTOL, f"{what}: lse relative error {rel.max():.3g} > {LSE_RTOL}"
    return float(err.max())


def to_dev(case, device="cuda"):
    """Copy every tensor of a case to the device (returns a dict of device tensors)."""
    d = {}
    for name in ("q", "k", "v", "seq_lens", "page_table", "k_new", "v_new", "rope_cos", "rope_sin",
                 "prefix_pages", "k_descale", "v_descale", "cache_batch_idx", "cache_leftpad"):
        t = getattr(case, name)
        d[name] = None if t is None else t.to(device).contiguous()
    return d


def appended_row_mask(case):
    """Boolean mask over the K cache: the row each append writes ("Inference Cookbook"
    §3.3: the new token goes to row cache_seqlens[b]), for every KV head and d.
    Paged caches: slot c % page of page page_table[b, c // page]; contiguous caches:
    row c of cache row cache_batch_idx[b] (b without one)."""
    mask = np.zeros(tuple(case.k.shape), dtype=bool)
    for b in range(case.B):
        c = int(case.seq_lens[b])
        if case.page_size:
            mask[int(case.page_table[b, c // case.page_size]), c % case.page_size] = True
        else:
            row = int(case.cache_batch_idx[b]) if case.cache_batch_idx is not None else b
            mask[row, c] = True
    return mask


def check_append_k(kg, kc, case, what=""):
    """The K cache after an append (kg: GPU, kc: oracle, both as uint16 bit patterns).
    Every element outside the appended rows is bitwise equal; an appended (rotated)
    element may differ from the oracle's single rounding by one unit in the last place
    (the kernel rotates in fp32, the oracle in double). Returns the number of appended
    elements that differ by that one ulp."""
    m = appended_row_mask(case)
    assert kg.shape == kc.shape == m.shape
    assert np.array_equal(kg[~m], kc[~m]), f"{what}: a K element outside the appended rows differs"
    diff = np.abs(kg[m].astype(np.int32) - kc[m].astype(np.int32))
    assert diff.size == 0 or diff.max() <= 1, f"{what}: an appended K element is off by more than 1 ulp"
    return int((diff > 0).sum())


# ---------------------------------------------------------------- float8 append

def _f8_order(c):
    """Position of e4m3fn codes on the number line (the two zeros coincide)."""
    c = c.astype(np.int32)
    return np.where(c & 0x80, -(c & 0x7F), c & 0x7F)


def _fp8_append_run(case, S, fused=False):
    import decode_attention_fdec_amd as F

    d = to_dev(case)
    a = F.make_append(d["k_new"], d["v_new"], d["rope_cos"], d["rope_sin"], case.rotary_dim)
    out, lse = F.decode(d["q"], d["k"], d["v"], d["seq_lens"], page_table=d["page_table"], num_splits=S,
                        append=a, fused=fused, k_descale=d["k_descale"], v_descale=d["v_descale"],
                        cache_batch_idx=d["cache_batch_idx"], cache_leftpad=d["cache_leftpad"])
    torch.cuda.synchronize()
    kg = d["k"].cpu().view(torch.uint8).numpy()
    vg = d["v"].cpu().view(torch.uint8).numpy()
    return out, lse, kg, vg


def check_fp8_append(case, S, fused, what):
    kc, vc, q_rot, after = oracle.append(okv(case), case.k_new, case.v_new, case.q, case.seq_lens,
                                         case.rotary_dim, case.rope_base)
    ref_out, ref_lse = oracle.decode(after, q_rot, case.seq_lens + 1, 1 / math.sqrt(case.D))
    out, lse, kg, vg = _fp8_append_run(case, S, fused)
    # v, the k rows not written and the k dims not rotated are bitwise the oracle's
    assert np.array_equal(vg, vc), f"{what}: v cache differs"
    m = appended_row_mask(case)
    assert np.array_equal(kg[~m], kc[~m]), f"{what}: a k element outside the appended rows differs"
    rd = case.rotary_dim
    kg_r, kc_r = kg[m].reshape(-1, case.D), kc[m].reshape(-1, case.D)
    assert np.array_equal(kg_r[:, rd:], kc_r[:, rd:]), f"{what}: an unrotated appended k element differs"
    # a rotated element: the kernel rotates in fp32, the oracle in double; the
    # code may then sit one step away when the value lies at a rounding midpoint
    step = np.abs(_f8_order(kg_r[:, :rd]) - _f8_order(kc_r[:, :rd]))
    assert step.size == 0 or step.max() <= 1, f"{what}: a rotated k code is off by more than one step"
    n_off = int((step > 0).sum())
    assert n_off <= max(2, step.size // 1000), f"{what}: {n_off} rotated codes off by one step"
    if n_off == 0:
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, what)
    else:  # outputs of the (request, KV head) groups whose row differs move by that step only
        assert torch.isfinite(out).all()
        err = np.abs(out.cpu().double().numpy() - ref_out).max()
        assert err <= 0.05, f"{what}: output error {err:.3g} with {n_off} codes one step off"
    return n_off


# ---------------------------------------------------------------- cascade parity

def _request_rows(case, t, b):
    """Rows [L, Hkv, D] (float64, dequantised) request b attends to: prefix, then suffix."""
    ps = case.page_size
    pre = t[case.prefix_pages.long()].reshape(-1, case.Hkv, case.D)[:case.prefix_len]
    n = int(case.seq_lens[b])
    suf = t[case.page_table[b, :(n + ps - 1) // ps].long()].reshape(-1, case.Hkv, case.D)[:n]
    return torch.cat([pre, suf]).double()


def p_rounding_bound(case):
    """Per output element, the most that rounding P to bf16 for the P V matrix-core
    operand (relative error at most 2^-9 per weight) can move it:
    2^-9 sum_j p_j |v_jd| / sum_j p_j, with the exact weights p_j (float64, from the
    dequantised rows). Test-side arithmetic for the tolerance only."""
    G = case.Hq // case.Hkv
    scale = 1.0 / math.sqrt(case.D)
    out = np.zeros((case.B, case.Hq, case.D))
    for b in range(case.B):
        k, v = _request_rows(case, case.k, b), _request_rows(case, case.v, b)
        if k.shape[0] == 0:
            continue
        if case.k_descale is not None:
            k = k * case.k_descale[b].double()[None, :, None]
            v = v * case.v_descale[b].double()[None, :, None]
        q = case.q[b].double().view(case.Hkv, G, case.D)
        s = torch.einsum("gid,lgd->gil", q, k) * scale
        p = torch.exp(s - s.amax(dim=-1, keepdim=True))
        wv = torch.einsum("gil,lgd->gid", p, v.abs()) / p.sum(-1, keepdim=True)
        out[b] = (2.0 ** -9 * wv).reshape(case.Hq, case.D).numpy()
    return out


def assert_cascade_parity(case, out, lse, ref_out, ref_lse, what):
    """16-bit pools: the usual tolerance. Float8 pools: the shared prefix pages hold
    codes of value * 32 read at descales up to 1/16, so values reach twice N(0, 1) and
    one key can hold much of a softmax; each output element is held to twice its
    P-rounding bound (plus fp32 noise), the LSE to the usual tolerance."""
    if case.dtype != FP8:
        assert_parity(out, lse, ref_out, ref_lse, case.dtype, what)
        return
    err = np.abs(out.cpu().double().numpy() - ref_out)
    assert np.isfinite(err).all(), f"{what}: non-finite output"
    tol = 2.0 * p_rounding_bound(case) + 2e-5
    r = err / tol
    assert r.max() <= 1.0, f"{what}: error {err.max():.3g}, {r.max():.3g} x its bound at {np.unravel_index(r.argmax(), r.shape)}"
    assert_parity(out * 0, lse, ref_out * 0, ref_lse, case.dtype, what)  # the LSE
