"""The balanced split's partition rule, checked on the CPU.

fdec_decode_balanced cuts the request-ordered sequence of 16-token tiles into
nb equal ranges (block i takes tiles [i*NT/nbe, (i+1)*NT/nbe) with
nbe = min(nb, NT)), writes a request's piece from block i into slot i + b, and
has the block holding a request's first tile record (first slot, count). This
restates that rule and checks, over random length mixes, the properties the
merge relies on: every tile is covered exactly once, a request's pieces take
consecutive slots that match its record, slots stay below nb + B, and pieces
start on tile boundaries (so a paged tile never straddles a page).
"""
import random

import pytest

TILE = 16


def partition(lens, nb):
    T = [(L + TILE - 1) // TILE for L in lens]
    NT = sum(T)
    nbe = min(nb, NT)

    def block_of(x):
        return nbe - 1 if x >= NT else ((x + 1) * nbe - 1) // NT

    P = [sum(T[:j]) for j in range(len(lens))]
    meta, pieces = {}, {}
    for blk in range(nb):
        working = blk < nbe
        start = blk * NT // nbe if working else 0
        end = (blk + 1) * NT // nbe if working else 0
        for j, L in enumerate(lens):
            first = block_of(P[j]) if NT > 0 else 0
            if first == blk:
                assert j not in meta, "two blocks record one request"
                meta[j] = (first + j, block_of(P[j] + T[j] - 1) - first + 1 if T[j] > 0 else 0)
            if working and T[j] > 0 and P[j] < end and P[j] + T[j] > start:
                ts, te = max(start, P[j]) - P[j], min(end, P[j] + T[j]) - P[j]
                pieces.setdefault(j, []).append((blk + j, ts * TILE, min(te * TILE, L)))
    return meta, pieces


@pytest.mark.parametrize("seed", range(4))
def test_partition_covers_every_tile_once(seed):
    rng = random.Random(seed)
    for _ in range(600):
        B = rng.choice([1, 2, 3, 5, 17, 64, 65, 130])
        hi = rng.choice([1, 16, 17, 100, 5000])
        lens = [rng.choice([0, rng.randint(0, hi)]) for _ in range(B)]
        nb = rng.choice([1, 2, 3, 7, 64, 255, 256])
        meta, pieces = partition(lens, nb)
        assert set(meta) == set(range(B))
        slots = []
        for j, L in enumerate(lens):
            s0, cnt = meta[j]
            w = sorted(pieces.get(j, []))
            assert [x[0] for x in w] == list(range(s0, s0 + cnt))
            assert cnt <= nb
            pos = 0
            for slot, t0, t1 in w:
                assert slot < nb + B and t0 == pos and t0 % TILE == 0 and t0 < t1 <= L
                pos = t1
            assert pos == L
            slots += [x[0] for x in w]
        assert len(slots) == len(set(slots))


def test_partition_balances_work():
    # the c3 length mix: block ranges differ by at most one tile
    rng = random.Random(3)
    lens = [rng.randint(512, 8192) for _ in range(32)]
    nb = 128
    meta, pieces = partition(lens, nb)
    per_block = {}
    for j, ps in pieces.items():
        for slot, t0, t1 in ps:
            per_block[slot - j] = per_block.get(slot - j, 0) + (t1 - t0 + TILE - 1) // TILE
    counts = sorted(per_block.values())
    assert len(counts) == nb and counts[-1] - counts[0] <= 1 + sum(1 for _ in lens)  # partial last tiles
