"""CPU model of the grouped GEMMs' tile list and gang scheduling (no GPU).

The device code (gemm_common.h: build_tile_map, tile_at, for_each_tile) builds a tile list
from expert_offset and hands it out to gangs of 8 workgroups through one atomic item
counter and per-gang claim slots. This test restates those rules in Python and runs them
under random interleavings of the workgroups, on random and skewed expert loads, checking:

- every (group, row, output-column tile) is computed exactly once;
- no tile is empty and no tile is taller than the kernel's tile height (320 rows in both
  phases of the bf16 and the FP8 kernels, 128 rows in the bf16 kernels for batches of at most
  128 tokens; 256-row blocks are checked as well);
- the tile count stays within the bound the workspace is sized for (ffn_max_tiles in
  abi.cpp, counted in 256-row blocks, so it also bounds the taller tiles) and no gang
  reads past its row of slots (slot stride ceil(max/G) + 2);
- the list order: shared groups first, then routed experts with an even number of row
  blocks, then those with an odd number, each pass by row count (most first, ties to the
  lower id) in the gate/up launch and in id order in the down-projection.

It is a model: it checks the protocol's design, and the GPU parity tests check the
kernels that implement it.
"""
import random

import numpy as np

BM = 256   # the row-block size the workspace bound counts in
GANGS = 8
SMALL_BATCH = 128  # batches of at most this many tokens: bf16 tiles of 128 rows


def tile_map(rows, n_r, rb=BM, sort=True):
    """Row blocks of at most rb rows per group, rows per block, and the list order (shared,
    even, odd; the routed experts of each pass by row count, most first, when sort -- the
    gate/up launch -- else in id order -- the down-projection)."""
    mt, rpb = [], []
    for r in rows:
        mt0 = (r + rb - 1) // rb
        p = (r + mt0 - 1) // mt0 if mt0 else 0
        rpb.append(p)
        mt.append((r + p - 1) // p if p else 0)
    # routed experts by row count, most first, ties to the lower id
    by_rows = sorted(range(n_r), key=lambda g: (-rows[g], g)) if sort else list(range(n_r))
    order = [g for g in range(n_r, len(rows)) if mt[g]]
    order += [g for g in by_rows if mt[g] and mt[g] % 2 == 0]
    order += [g for g in by_rows if mt[g] and mt[g] % 2 == 1]
    return mt, rpb, order


def tiles_of(rows, n_r, ntn, rb=BM, sort=True):
    mt, rpb, order = tile_map(rows, n_r, rb, sort)
    out = []
    for g in order:
        if g < n_r:  # column-major: the row blocks of one column tile are neighbours
            pairs = [(m, n) for n in range(ntn) for m in range(mt[g])]
        else:  # blocks of 4 row blocks x 8 column tiles, row-major inside a block
            pairs = [(m, n) for r0 in range(0, mt[g], 4) for c0 in range(0, ntn, 8)
                     for m in range(r0, min(r0 + 4, mt[g])) for n in range(c0, min(c0 + 8, ntn))]
        for m, n in pairs:
            m0 = m * rpb[g]
            out.append((g, m0, n, min(rpb[g], rows[g] - m0)))
    return out


def max_tiles(T, top_k, n_r, n_shared, d, d_ff, phase):
    P = T * top_k
    routed_blocks = P // BM + n_r + 1
    tb = (T + BM - 1) // BM
    if phase == 1:
        return (routed_blocks + n_shared * tb) * (d_ff // 128)
    return (routed_blocks + (tb if n_shared else 0)) * (d // 256)


def run_gangs(tiles, grid, stride, rng):
    """Random interleaving of the claim protocol; returns the tiles each workgroup ran."""
    total = len(tiles)
    G = grid // GANGS
    n_items = (total + G - 1) // G
    counter = 0
    slots = np.zeros((GANGS, stride), np.int64)
    step = {b: 0 for b in range(GANGS * G)}  # workgroups past G * 8 idle at once
    ran = []
    active = list(step)
    while active:
        b = rng.choice(active)
        gang, rank = b % GANGS, b // GANGS
        k = step[b]
        assert k < stride, "a gang read past its slots"
        if slots[gang, k] == 0:  # first member at step k claims the next item
            counter += 1
            slots[gang, k] = counter
        item = slots[gang, k] - 1
        if item >= n_items:
            active.remove(b)
            continue
        L = item * G + rank
        if L < total:
            ran.append(tiles[L])
        step[b] = k + 1
    return ran


def check(T, top_k, n_r, n_shared, d, d_ff, counts, grid, rng):
    heights = [(1, 256), (2, 256), (1, 320), (2, 320)]
    if T <= SMALL_BATCH:
        heights += [(1, SMALL_BATCH), (2, SMALL_BATCH)]
    for phase, rb in heights:
        ns_groups = n_shared if phase == 1 else min(n_shared, 1)
        ntn = d_ff // 128 if phase == 1 else d // 256
        rows = list(counts) + [T] * ns_groups
        tiles = tiles_of(rows, n_r, ntn, rb, sort=phase == 1)
        bound = max_tiles(T, top_k, n_r, n_shared, d, d_ff, phase)
        assert len(tiles) <= bound
        G = grid // GANGS
        stride = (bound + G - 1) // G + 2
        ran = run_gangs(tiles, grid, stride, rng)
        seen = set()
        for g, m0, n, r in ran:
            assert 1 <= r <= rb
            for row in range(m0, m0 + r):
                key = (g, row, n)
                assert key not in seen, key
                seen.add(key)
        assert len(seen) == sum(rows) * ntn


def _counts(rng, T, top_k, n_r, skew):
    p = rng.dirichlet(np.ones(n_r) * skew)
    return rng.multinomial(T * top_k, p)


def test_schedule_v3_prefill_shape():
    rng = np.random.default_rng(1)
    r = random.Random(1)
    counts = _counts(rng, 8192, 8, 256, 20.0)
    check(8192, 8, 256, 1, 7168, 2048, counts, 256, r)


def test_schedule_random_shapes():
    rng = np.random.default_rng(2)
    r = random.Random(2)
    for _ in range(40):
        n_r = int(rng.choice([1, 2, 16, 64, 256]))
        T = int(rng.choice([1, 7, 64, 300, 2048]))
        top_k = int(rng.integers(1, min(8, n_r) + 1))
        counts = _counts(rng, T, top_k, n_r, float(rng.choice([0.1, 1.0, 10.0])))
        n_shared = int(rng.choice([0, 1, 2, 8]))
        d = int(rng.choice([256, 512, 2816]))
        d_ff = int(rng.choice([128, 1408, 2048]))
        grid = int(rng.choice([64, 256, 264]))
        check(T, top_k, n_r, n_shared, d, d_ff, counts, grid, r)


def test_schedule_v3_decode_shape():
    """128 tokens (the small-batch tiles), 8 hot experts: every group is one 128-row block."""
    rng = np.random.default_rng(5)
    r = random.Random(5)
    p = rng.dirichlet(np.ones(256) * 0.3)  # skewed, but each token picks 8 distinct experts
    picks = np.concatenate([rng.choice(256, 8, replace=False, p=p) for _ in range(128)])
    counts = np.bincount(picks, minlength=256)
    assert counts.max() > 32
    check(128, 8, 256, 1, 7168, 2048, counts, 256, r)
    mt, _, _ = tile_map(list(counts) + [128], 256, SMALL_BATCH)
    assert max(mt) == 1


def test_schedule_all_rows_on_few_experts():
    r = random.Random(3)
    check(4096, 4, 4, 1, 512, 256, np.array([4096] * 4), 64, r)  # 16 blocks per expert
    check(3000, 1, 2, 2, 256, 128, np.array([2999, 1]), 64, r)   # a one-row expert


def test_tile_order():
    rows = [300, 0, 600, 256, 513, 9000, 70]  # n_r = 5, two shared groups
    mt, rpb, order = tile_map(rows, 5)
    assert mt == [2, 0, 3, 1, 3, 36, 1]
    assert rpb == [150, 0, 200, 256, 171, 250, 70]
    assert order == [5, 6, 0, 2, 4, 3]  # odd pass: 600, 513, 256 rows
    assert tile_map(rows, 5, sort=False)[2] == [5, 6, 0, 2, 3, 4]  # the down-projection: id order
    mt, rpb, order = tile_map(rows, 5, 320)  # the bf16 kernel's phase-1 tiles
    assert mt == [1, 0, 2, 1, 2, 29, 1]
    assert rpb == [300, 0, 300, 256, 257, 311, 70]
    assert order == [5, 6, 2, 4, 0, 3]


def test_taller_tiles_split_fewer_v3_experts():
    """At V3 prefill (65536 pairs over 256 experts, 256 on average) 320-row blocks leave
    less than half as many experts in two blocks as 256-row blocks do, so fewer experts'
    weights are read twice."""
    rng = np.random.default_rng(4)
    counts = _counts(rng, 8192, 8, 256, 20.0)
    split = lambda rb: sum(1 for m in tile_map(list(counts), 256, rb)[0] if m > 1)
    assert split(320) * 2 < split(256)


def test_k_segment_reciprocal():
    """b_offset's segment index: floor(2 kt * ceil(2^31 / d) / 2^32) equals kt // d for
    every segment length d the kernels use (one step included) and every step index up
    to the longest K loop (8 shared experts of d_ff 2048 in 64-wide bf16 steps: 256)."""
    kt = np.arange(0, 4096, dtype=np.uint64)
    for d in range(1, 2049):
        inv = np.uint64(((1 << 31) + d - 1) // d)
        seg = ((np.uint64(2) * kt) * inv) >> np.uint64(32)
        assert np.array_equal(seg, kt // np.uint64(d)), d


def _shared_tile_at(local, mt, ntn, br_full=4, bc_full=8):
    """tile_at's closed form for a shared group (gemm_common.h), restated: row groups of 4 row
    blocks (the last may be shorter), inside one column groups of 8 tiles (the last may be
    narrower), row-major inside a block."""
    rg = local // (br_full * ntn)
    rem = local - rg * br_full * ntn
    br = min(br_full, mt - rg * br_full)
    cg = rem // (br * bc_full)
    rem2 = rem - cg * br * bc_full
    bc = min(bc_full, ntn - cg * bc_full)
    return rg * br_full + rem2 // bc, cg * bc_full + rem2 % bc


def test_shared_block_order_closed_form():
    """The device's index arithmetic for shared groups gives, position by position, the
    blocked order the list model enumerates, and so covers every (row block, column tile)
    exactly once, including short last row groups and narrow last column groups."""
    for mt in (1, 2, 3, 4, 5, 7, 8, 13, 26, 33):
        for ntn in (1, 3, 8, 11, 16, 28):
            want = [(m, n) for _, m0, n, _ in tiles_of([mt * 100], 0, ntn, 100) for m in [m0 // 100]]
            got = [_shared_tile_at(L, mt, ntn) for L in range(mt * ntn)]
            assert got == want, (mt, ntn)
            assert len(set(got)) == mt * ntn


def test_tile_order_by_rows():
    """Each routed pass runs from the expert with the most rows to the one with the fewest;
    equal counts keep ascending ids, and the shared groups stay first in id order."""
    rows = [100, 250, 100, 600, 0, 250, 700, 640, 8192]  # n_r = 8, one shared group
    mt, _, order = tile_map(rows, 8, 320)
    assert mt[:8] == [1, 1, 1, 2, 0, 1, 3, 2]
    assert order == [8, 7, 3, 6, 1, 5, 0, 2]
    rng = np.random.default_rng(6)
    counts = list(_counts(rng, 8192, 8, 256, 20.0))
    mt, _, order = tile_map(counts + [8192], 256, 320)
    routed = [g for g in order if g < 256]
    for par in (0, 1):
        seq = [g for g in routed if mt[g] % 2 == par]
        assert all((counts[a], -a) > (counts[b], -b) for a, b in zip(seq, seq[1:]))
    assert sorted(routed) == [g for g in range(256) if mt[g]]
