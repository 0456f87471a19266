"""The work items of the 129-256-row decode reduction, from the segments (CPU).

That kernel cuts every segment tile (LORA_TILE_ROWS positions of one adapter) into items of
four positions, numbers them densely in tile order, and appends the base-only positions in
fours; its grid holds floor((M + 3 (min(M, n) + 2)) / 4) items, a bound the host computes
from M and n alone.  Here the item list is rebuilt from the oracle's segments for random and
adversarial id vectors: every row is covered exactly once, every item's rows share its
tile's adapter, and the count never exceeds the bound (and reaches it for the worst cases).
"""

import numpy as np

import oracle

TILE, SUB = 16, 4


def items_of(ids: np.ndarray, n: int):
    s = oracle.build_segments(ids, n, TILE)
    perm, tiles, meta = (np.asarray(s[k]).reshape(-1) for k in ("perm", "tiles", "meta"))
    M = len(ids)
    n_tiles, lora_rows = int(meta[3]), int(meta[1])
    firsts = [int(tiles[2 * t]) for t in range(n_tiles)] + [lora_rows]
    items = []
    for t in range(n_tiles):
        for p0 in range(firsts[t], firsts[t + 1], SUB):
            items.append((p0, min(SUB, firsts[t + 1] - p0), int(tiles[2 * t + 1])))
    for p0 in range(lora_rows, M, SUB):
        items.append((p0, min(SUB, M - p0), -1))
    return perm, items


def bound(M: int, n: int) -> int:
    return (M + 3 * min(M, n) + 6) // SUB


def check(ids: np.ndarray, n: int) -> int:
    perm, items = items_of(ids.astype(np.int32), n)
    seen = np.zeros(len(ids), int)
    for p0, nr, a in items:
        rows = perm[p0:p0 + nr]
        assert 1 <= nr <= SUB
        assert np.all(ids[rows] == a) if a >= 0 else np.all(ids[rows] == -1)
        seen[rows] += 1
    assert np.all(seen == 1)
    assert len(items) <= bound(len(ids), n), (len(items), bound(len(ids), n))
    return len(items)


def test_items_cover_rows_and_respect_the_bound():
    rng = np.random.default_rng(20)
    for trial in range(400):
        M = int(rng.integers(129, 257))
        n = int(rng.integers(1, 700))
        kind = trial % 4
        if kind == 0:
            ids = rng.integers(-1, n, size=M)
        elif kind == 1:
            ids = rng.integers(0, min(n, 3), size=M)
        elif kind == 2:
            ids = np.sort(rng.integers(0, n, size=M))
        else:
            c = int(rng.integers(1, 6))
            ids = np.repeat(np.arange(M // c + 1), c)[:M] % n
            ids[rng.random(M) < 0.3] = -1
        check(ids, n)


def test_bound_is_reached():
    # every adapter with 5 rows (one full item + a 1-row item), the base rows a 1-row item:
    # as many partial items as there can be
    n = 51
    ids = np.repeat(np.arange(n), 5)
    ids = np.concatenate([ids, [-1]])  # 256 rows
    got = check(ids, n)
    assert got == 2 * n + 1
    assert bound(len(ids), n) - got <= 1
