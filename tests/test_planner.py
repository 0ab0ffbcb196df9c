"""Split planners (host only).

fdec_plan_rules restates the flash-attn cookbook's four rules (§6.3) and must
reproduce the page's own H100 examples (§8.2, tests/golden). fdec_plan is the
MI355X cost model: no parity, pinned by constraints.
"""
import os

import pytest

import decode_attention_fdec_amd as F

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            out.append(line.split())
    return out


@pytest.mark.parametrize("row", rows("split_examples_h100.txt"), ids=lambda r: f"B{r[1]}H{r[2]}")
def test_rules_mode_reproduces_page_examples(fdec, row):
    sm, B, H, _page_says, expected = int(row[0]), int(row[1]), int(row[2]), row[3], int(row[4])
    assert F.plan_rules(B, H, sm) == expected


def test_rules_mode_no_split_at_80_percent(fdec):
    assert F.plan_rules(1, 205, 256) == 1  # 205 >= 0.8 * 256
    assert F.plan_rules(1, 200, 256) > 1


def test_split_picture_from_the_pages(fdec):
    (row,) = rows("split_picture_1024.txt")
    n, S, bounds = int(row[0]), int(row[1]), [int(x) for x in row[2:]]
    c = F.split_chunk(n, S)
    assert [min(i * c, n) for i in range(S + 1)] == bounds
    (row,) = rows("lpnh_128k_slices.txt")
    n, S, slice_len = int(row[0]), int(row[1]), int(row[2])
    assert F.split_chunk(n, S) == slice_len


def test_plan_constraints(fdec):
    for B, Hq, Hkv, cap in [(1, 32, 8, 131072), (1, 32, 32, 4096), (4, 32, 8, 2048), (32, 32, 8, 8192),
                            (64, 32, 8, 2048), (1, 8, 8, 16), (3, 4, 1, 100)]:
        S = F.plan(B, Hq, Hkv, None, cap)
        assert 1 <= S <= F.MAX_SPLITS
        assert F.split_chunk(cap, S) >= 16
        assert F.plan(B, Hq, Hkv, None, cap) == S  # deterministic


def test_plan_fills_the_chip_for_long_contexts(fdec):
    # one request, 8 KV heads, 128k tokens: a map block sustains at most ~35 GB/s,
    # so the aggregate rate needs well over a hundred concurrent blocks
    S = F.plan(1, 32, 8, None, 131072)
    assert 8 * S * 35e9 >= 5.0e12
    # a batch that already has >= 2 blocks per CU of equal long work does not split much
    assert F.plan(64, 32, 8, [8192] * 64, 8192) <= 2


def test_plan_short_sequences_split_little(fdec):
    assert F.plan(32, 32, 8, [64] * 32, 64) == 1
    assert F.plan(1, 32, 8, [128], 131072) == 1 or F.split_chunk(131072, F.plan(1, 32, 8, [128], 131072)) >= 128


def test_plan_rejects_bad_lengths(fdec):
    with pytest.raises(F.FdecError):
        F.plan(2, 32, 8, [10, 9999], 4096)
    with pytest.raises(F.FdecError):
        F.plan(2, 32, 8, None, 4096, page_size=8)


def test_plan_kv_by_cache_type(fdec):
    shapes = [(1, 8, 8, 131072), (1, 16, 8, 131072), (1, 32, 8, 131072), (1, 64, 8, 131072), (1, 32, 32, 4096),
              (8, 16, 8, 8192), (32, 8, 8, 4096), (4, 16, 8, 2048), (3, 4, 1, 100)]
    for B, Hq, Hkv, cap in shapes:
        S16 = F.plan(B, Hq, Hkv, None, cap)
        # fdec_plan is fdec_plan_kv with a 16-bit cache
        assert F.plan(B, Hq, Hkv, None, cap, kv_dtype=F.FDEC_F16) == S16
        assert F.plan(B, Hq, Hkv, None, cap, kv_dtype=F.FDEC_BF16) == S16
        S8 = F.plan(B, Hq, Hkv, None, cap, kv_dtype=F.FDEC_FP8_E4M3)
        assert 1 <= S8 <= F.MAX_SPLITS and F.split_chunk(cap, S8) >= 16
        if Hq in (4 * Hkv, 8 * Hkv):
            assert S8 == S16  # the matrix-core kernel plans the same for float8
        else:
            assert S8 >= S16  # a float8 wave streams half the bytes: at least as many splits
    # one 128k-token request on the vector kernel: four (KV head, split) pairs per CU
    assert 8 * F.plan(1, 16, 8, None, 131072, kv_dtype=F.FDEC_FP8_E4M3) >= 4 * 256
    with pytest.raises(F.FdecError):
        F.plan(1, 16, 8, None, 4096, kv_dtype=7)
    # the binding takes torch dtypes as well as fdec_dtype codes
    import torch
    assert F.plan(1, 16, 8, None, 131072, kv_dtype=torch.float8_e4m3fn) == \
        F.plan(1, 16, 8, None, 131072, kv_dtype=F.FDEC_FP8_E4M3)
    assert F.plan(1, 16, 8, None, 131072, kv_dtype=torch.float16) == F.plan(1, 16, 8, None, 131072)
