"""Pins of the dispatch oracle: a written-out counting sort on tiny inputs and
the invariants (histogram sums to valid tokens x k, bijection, dest o perm)."""
import numpy as np
import pytest

import oracle as O


def _brute_dispatch(ids, E):
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * E
    for v in flat:
        if 0 <= v < E:
            counts[v] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    perm = []
    for e in range(E):                  # expert by expert
        for f, v in enumerate(flat):    # slots in flat order
            if v == e:
                perm.append(f)
    perm += [-1] * (len(flat) - len(perm))
    dest = [-1] * len(flat)
    for p, f in enumerate(perm):
        if f >= 0:
            dest[f] = p
    return counts, offsets, perm, dest


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (7, 3, 5, 1), (33, 4, 16, 2), (50, 8, 256, 3), (64, 22, 40, 4)])
def test_dispatch_brute_force(T, k, E, seed):
    g = np.random.default_rng(seed)
    ids = g.integers(-2, E + 2, size=(T, k)).astype(np.int32)   # includes invalid ids
    ids[g.uniform(size=T) < 0.2] = -1                            # invalid tokens
    got = O.dispatch(ids, E)
    want = _brute_dispatch(ids, E)
    for a, b in zip(got, want):
        np.testing.assert_array_equal(a, np.array(b, dtype=np.int32))


def test_dispatch_invariants_under_skew():
    g = np.random.default_rng(5)
    T, k, E = 4096, 8, 2560
    hot = g.choice(E, 16, replace=False)
    ids = np.stack([g.permutation(hot)[:k] for _ in range(T)]).astype(np.int32)
    mask = g.uniform(size=T) < 0.95
    ids[~mask] = -1
    counts, offsets, perm, dest = O.dispatch(ids, E)
    nvalid = int(mask.sum()) * k
    assert counts.sum() == nvalid and offsets[-1] == nvalid and offsets[0] == 0
    assert (np.diff(offsets) == counts).all()
    assert set(np.nonzero(counts)[0]) <= set(hot)
    placed = perm[:nvalid]
    assert (perm[nvalid:] == -1).all()
    flat = ids.reshape(-1)
    assert np.array_equal(np.sort(placed), np.nonzero(flat >= 0)[0])          # bijection onto valid slots
    assert (dest[placed] == np.arange(nvalid)).all()                          # dest o perm = id
    assert (dest[flat < 0] == -1).all()
    # grouped by expert, ascending flat index within an expert
    ex = flat[placed]
    assert (np.diff(ex) >= 0).all()
    same = np.diff(ex) == 0
    assert (np.diff(placed)[same] > 0).all()


def test_dispatch_empty_and_all_invalid():
    counts, offsets, perm, dest = O.dispatch(np.zeros((0, 4), np.int32), 8)
    assert counts.sum() == 0 and offsets.tolist() == [0] * 9 and perm.size == 0
    counts, offsets, perm, dest = O.dispatch(np.full((5, 2), -1, np.int32), 3)
    assert (perm == -1).all() and (dest == -1).all() and offsets[-1] == 0
