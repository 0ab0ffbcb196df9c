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
