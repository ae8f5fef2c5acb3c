"""Pins of the oracle's routing (expert histogram + stable grouping by expert).

Masked indexing per expert ("MoE training token repeat and expert
computation", description) is checked by brute force: scan every slot and
keep those whose id equals e.
"""
import numpy as np
import pytest

from oracle import route


def brute_force_groups(ids, E):
    f = np.asarray(ids).reshape(-1)
    return [[s for s in range(f.size) if f[s] == e] for e in range(E)]


def check_route(ids, E):
    ids = np.asarray(ids, dtype=np.int32)
    counts, offsets, sorted_slot, inv_pos = route(ids, E)
    groups = brute_force_groups(ids, E)
    S = ids.size
    assert counts.tolist() == [len(g) for g in groups]
    assert offsets[0] == 0 and offsets[-1] == S and len(offsets) == E + 1
    for e in range(E):
        assert sorted_slot[offsets[e]:offsets[e + 1]].tolist() == groups[e]
    assert sorted(sorted_slot.tolist()) == list(range(S))
    for p in range(S):
        assert inv_pos[sorted_slot[p]] == p
    f = ids.reshape(-1)
    assert np.all(np.diff(f[sorted_slot]) >= 0)


@pytest.mark.parametrize("seed", range(6))
def test_random(seed):
    rng = np.random.default_rng(seed)
    T, K, E = rng.integers(1, 40), rng.integers(1, 5), rng.integers(1, 9)
    check_route(rng.integers(0, E, size=(T, K)), E)


def test_edge_cases():
    check_route(np.zeros((7, 3)), 5)                     # all slots to one expert, 4 empty
    check_route(np.array([[2, 2], [2, 0], [1, 1]]), 4)   # duplicates inside a token, expert 3 empty
    check_route(np.array([[3]]), 4)                       # T=1, K=1
    check_route(np.arange(12).reshape(4, 3) % 5, 5)
    counts, offsets, sorted_slot, inv_pos = route(np.zeros((0, 4), dtype=np.int32), 3)
    assert counts.tolist() == [0, 0, 0] and offsets.tolist() == [0, 0, 0, 0]
    assert sorted_slot.size == 0 and inv_pos.size == 0


def test_known_small_example():
    # ids [[1,0],[0,1],[1,1]]: expert 0 holds slots 1,2; expert 1 holds 0,3,4,5
    counts, offsets, sorted_slot, inv_pos = route(np.array([[1, 0], [0, 1], [1, 1]]), 2)
    assert counts.tolist() == [2, 4]
    assert offsets.tolist() == [0, 2, 6]
    assert sorted_slot.tolist() == [1, 2, 0, 3, 4, 5]
    assert inv_pos.tolist() == [2, 0, 1, 3, 4, 5]


def test_bad_ids_raise():
    with pytest.raises(ValueError):
        route(np.array([[0, 4]]), 4)
    with pytest.raises(ValueError):
        route(np.array([[-1, 0]]), 4)
