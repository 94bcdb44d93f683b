"""Host logic of the 2D-grid emulation: block splits, ring arrival orders,
tile plans and the per-step compute/transfer model (no GPU needed)."""

import itertools

import numpy as np
import pytest

import pair_representation_amd as pra
from pair_representation_amd import grid


@pytest.mark.parametrize("n,parts", [(1, 1), (10, 3), (300, 2), (300, 3), (10000, 2), (7, 7)])
def test_split_partitions_the_range(n, parts):
    blocks = grid.split(n, parts)
    assert len(blocks) == parts
    covered = np.concatenate([np.arange(o, o + l) for o, l in blocks])
    assert np.array_equal(covered, np.arange(n))
    lens = [l for _, l in blocks]
    assert max(lens) - min(lens) <= 1


def test_split_rejects_impossible():
    with pytest.raises(ValueError):
        grid.split(3, 4)
    with pytest.raises(ValueError):
        grid.split(5, 0)


@pytest.mark.parametrize("s", [1, 2, 3, 5])
def test_ring_order_starts_at_own_block_and_visits_all(s):
    for own in range(s):
        order = grid.ring_order(own, s)
        assert order[0] == own and sorted(order) == list(range(s))
        # consecutive arrivals are ring neighbours
        assert all((b - a) % s == 1 for a, b in zip(order, order[1:]))


@pytest.mark.parametrize("direction", [pra.OUTGOING, pra.INCOMING])
@pytest.mark.parametrize("s_rows,s_cols", [(1, 1), (2, 2), (3, 3), (3, 1), (1, 3), (2, 3)])
def test_plan_covers_grid_and_k_once(direction, s_rows, s_cols):
    n = 31
    tiles = grid.plan(n, direction, s_rows, s_cols)
    assert len(tiles) == s_rows * s_cols
    hits = np.zeros((n, n), int)
    for t in tiles:
        hits[t.row_off:t.row_off + t.n_rows, t.col_off:t.col_off + t.n_cols] += 1
        ks = np.concatenate([np.arange(o, o + l) for o, l in t.k_blocks])
        assert np.array_equal(np.sort(ks), np.arange(n))            # every k exactly once
        own = (t.col_off, t.n_cols) if direction == pra.OUTGOING else (t.row_off, t.n_rows)
        assert t.k_blocks[0] == own                                 # own block first
    assert (hits == 1).all()


def test_plan_k_blocks_follow_the_ring():
    # 3x3 outgoing: tile (1, 2) receives column blocks 2, 0, 1
    cols = grid.split(30, 3)
    t = [t for t in grid.plan(30, pra.OUTGOING, 3) if (t.p, t.q) == (1, 2)][0]
    assert t.k_blocks == [cols[2], cols[0], cols[1]]
    # incoming: tile (2, 0) receives row blocks 2, 0, 1
    t = [t for t in grid.plan(30, pra.INCOMING, 3) if (t.p, t.q) == (2, 0)][0]
    assert t.k_blocks == [cols[2], cols[0], cols[1]]


def test_step_model_crossover():
    # at the crossover tile size compute and transfer times are equal
    m = grid.step_model(10000, 2, tflops=1250.0, link_gbs=153.0)
    assert m["crossover_tile"] == pytest.approx(1250e12 * 2 / (2 * 153e9))
    n_eq = m["crossover_tile"] * 2
    e = grid.step_model(n_eq, 2, tflops=1250.0, link_gbs=153.0)
    assert e["compute_s"] == pytest.approx(e["transfer_s"])
    # the 10,000-residue 2x2 grid: 5000-wide tiles, below the crossover
    assert m["tile"] == 5000 and m["bound"] == "transfer"
    assert m["compute_s"] == pytest.approx(2 * 5000 ** 3 * 128 / 1250e12)
    assert m["transfer_s"] == pytest.approx(5000 ** 2 * 128 * 2 / 153e9)
    for s_, big in itertools.product([2, 4], [False, True]):
        r = grid.step_model(40000 if big else 4000, s_, 1250.0, 153.0)
        assert r["bound"] == ("compute" if r["tile"] >= r["crossover_tile"] else "transfer")
