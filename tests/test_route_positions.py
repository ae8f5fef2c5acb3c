"""Host emulation of the device routing passes' position assignment.

The three routing kernels (per-chunk histogram, one-workgroup scan,
ballot-ranked scatter) decide where every slot lands in the expert-sorted
order.  This test replays those index computations on the CPU, chunk by
chunk, round by round and wavefront by wavefront, with the kernels' constants
(512-slot chunks, 256-slot rounds, 64-lane waves), and checks what the rest
of the library relies on:

* valid slots get the oracle's stable grouping by expert;
* slots with an id outside [0, E) fill the positions after the valid ones,
  in ascending slot order, with inv_pos -1;
* every position in [0, S) is written exactly once, so the token of every
  position is a real token (the backward gathers rows for all S positions).

It replays the scheme, not the compiled kernel; the GPU tests check the
kernels' outputs against the same expectations.
"""
import numpy as np
import pytest

import oracle

CHUNK, ROUND, WAVE = 512, 256, 64


def emulate_routing(ids, E, K):
    f = np.asarray(ids, dtype=np.int64).reshape(-1)
    S = f.size
    nblk = max(1, (S + CHUNK - 1) // CHUNK)
    key = np.where((f >= 0) & (f < E), f, E)              # E groups the bad ids
    # pass 1: per-chunk histogram of valid ids and count of bad ones
    hist = np.zeros((nblk, E + 1), dtype=np.int64)
    for b in range(nblk):
        hist[b] = np.bincount(key[b * CHUNK:(b + 1) * CHUNK], minlength=E + 1)
    # pass 2: expert offsets, per-chunk bases, bad slots after all valid ones
    counts = hist[:, :E].sum(axis=0)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    base = np.zeros((nblk, E + 1), dtype=np.int64)
    run = offsets[:E].copy()
    bad_run = offsets[E]
    for b in range(nblk):
        base[b, :E] = run
        run = run + hist[b, :E]
        base[b, E] = bad_run
        bad_run += hist[b, E]
    # pass 3: scatter, ranks from lane order inside a wave, wave order inside a round
    sorted_slot = np.full(S, -1, dtype=np.int64)
    tok_of_pos = np.full(S, -1, dtype=np.int64)
    written = np.zeros(S, dtype=np.int64)
    inv_pos = np.full(S, -7, dtype=np.int64)
    for b in range(nblk):
        running = base[b].copy()
        for r in range(CHUNK // ROUND):
            wcnt = np.zeros((ROUND // WAVE, E + 1), dtype=np.int64)
            ranks = {}
            for wv in range(ROUND // WAVE):
                for lane in range(WAVE):
                    s = b * CHUNK + r * ROUND + wv * WAVE + lane
                    if s >= S:
                        continue
                    k = key[s]
                    ranks[s] = (wv, k, wcnt[wv, k])
                    wcnt[wv, k] += 1
            for s, (wv, k, rank) in ranks.items():
                pos = running[k] + rank + wcnt[:wv, k].sum()
                sorted_slot[pos] = s
                tok_of_pos[pos] = s // K
                written[pos] += 1
                inv_pos[s] = pos if k < E else -1
            running += wcnt.sum(axis=0)
    return counts, offsets, sorted_slot, inv_pos, tok_of_pos, written


@pytest.mark.parametrize("T,K,E,nbad,seed", [(1, 1, 1, 0, 0), (300, 3, 7, 0, 1), (700, 4, 16, 5, 2),
                                             (129, 8, 5, 40, 3), (64, 2, 3, 128, 4), (1000, 2, 33, 1, 5)])
def test_positions_cover_every_slot_once(T, K, E, nbad, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=(T, K))
    flat = ids.reshape(-1)
    bad = rng.choice(flat.size, size=min(nbad, flat.size), replace=False)
    flat[bad] = rng.choice([-1, E, E + 5, -1000], size=bad.size)
    counts, offsets, sorted_slot, inv_pos, tok_of_pos, written = emulate_routing(ids, E, K)
    S = T * K
    assert np.all(written == 1)                          # each position written once
    assert np.all((tok_of_pos >= 0) & (tok_of_pos < T))  # a real token at every position
    good = (flat >= 0) & (flat < E)
    c, o, ss, ip = oracle.route(flat[good].reshape(-1, 1), E)   # the valid slots alone
    nvalid = int(good.sum())
    np.testing.assert_array_equal(counts, c)
    np.testing.assert_array_equal(offsets, o)
    valid_slots = np.nonzero(good)[0]
    np.testing.assert_array_equal(sorted_slot[:nvalid], valid_slots[ss])
    np.testing.assert_array_equal(sorted_slot[nvalid:], np.nonzero(~good)[0])
    assert np.all(inv_pos[~good] == -1)
    np.testing.assert_array_equal(inv_pos[valid_slots], ip)
    assert sorted(sorted_slot.tolist()) == list(range(S))
