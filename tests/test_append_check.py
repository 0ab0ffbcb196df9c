"""CPU checks of the append comparison the GPU tests use (check_append_k).

The oracle's own cache after an append stands in for the GPU's: the check
accepts it, accepts a one-ulp change inside an appended row, and rejects a
one-bit change of any other K element and a two-ulp change inside an
appended row ("Inference Cookbook" §3.3: only row cache_seqlens[b] is written).
"""
import numpy as np
import pytest

import oracle
from helpers import appended_row_mask, check_append_k, okv
from synth import F16, append_case


def _bits(t):
    return t.contiguous().view(np.uint16) if isinstance(t, np.ndarray) else t.contiguous().numpy().view(np.uint16)


@pytest.mark.parametrize("paged", [False, True])
def test_check_append_k_is_strict_outside_the_appended_rows(paged):
    case = append_case(5, 3, 8, 2, 64, 64, F16, rotary_dim=64, pad="nan", page_size=16 if paged else 0,
                       cache_seqlens=[0, 17, 63])
    kc, _, _, _ = oracle.append(okv(case), case.k_new, case.v_new, case.q, case.seq_lens, case.rotary_dim,
                                case.rope_base)
    kc = np.asarray(kc)
    m = appended_row_mask(case)
    assert m.sum() == case.B * case.Hkv * case.D
    # the oracle's appended rows are exactly the masked elements that changed
    k0 = _bits(case.k)
    assert np.all((kc == k0) | m)
    assert check_append_k(kc.copy(), kc, case) == 0
    # one ulp inside an appended row passes and is counted
    kg = kc.copy()
    idx = np.argwhere(m)[5]
    kg[tuple(idx)] ^= 1
    assert check_append_k(kg, kc, case) == 1
    # two ulps there fail
    kg = kc.copy()
    kg[tuple(idx)] = (int(kg[tuple(idx)]) + 2) & 0xFFFF
    with pytest.raises(AssertionError):
        check_append_k(kg, kc, case)
    # one bit anywhere outside the appended rows fails
    rng = np.random.default_rng(0)
    outside = np.argwhere(~m)
    for j in rng.choice(len(outside), 8, replace=False):
        kg = kc.copy()
        kg[tuple(outside[j])] ^= 1
        with pytest.raises(AssertionError):
            check_append_k(kg, kc, case)
