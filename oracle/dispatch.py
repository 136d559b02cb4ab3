"""Oracle for the dispatch: expert histogram, exclusive prefix scan, stable
permutation of the routed slots by expert.

Source: lmdeploy PR #4835, "Intern-S2-Mobius meta-MoE support, MoE gate v2, CP
attention fixes" — commit notes of "MoE gate v2" (shared-memory expert
histogram, hierarchical multi-block scan over tiles for large E) and of the
per-token validity mask (invalid tokens get no entry; the slot-to-position map
en2f is cleared to -1 so nothing reads compacted-out rows).

A routed slot is the flat index f = t * k + j of topk_ids[t, j]. It is valid
when its id lies in [0, E); ids outside that range (-1 from an invalid token)
produce no entry.

Test infrastructure only.
"""
from __future__ import annotations

import numpy as np


def dispatch(topk_ids: np.ndarray, E: int):
    """Returns (counts [E], offsets [E+1], perm [T*k], dest [T*k]), all int32.

      counts[e]   number of valid slots routed to expert e
      offsets     exclusive prefix sum of counts; offsets[E] = valid slots
      perm[p]     for p < offsets[E]: the flat slot placed at position p. Slots
                  are grouped by expert in ascending expert order, and within
                  an expert by ascending flat index (a stable counting sort,
                  which is what a tile-ordered scan produces). perm[p] = -1
                  for p >= offsets[E].
      dest[f]     position of slot f, or -1 when slot f is not valid;
                  dest[perm[p]] = p.
    """
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    n = ids.size
    valid = (ids >= 0) & (ids < E)
    counts = np.bincount(ids[valid], minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    slots = np.nonzero(valid)[0]                       # ascending flat index
    order = np.argsort(ids[slots], kind="stable")      # stable: keeps flat order per expert
    perm = np.full(n, -1, dtype=np.int64)
    perm[: slots.size] = slots[order]
    dest = np.full(n, -1, dtype=np.int64)
    dest[perm[: slots.size]] = np.arange(slots.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm.astype(np.int32), dest.astype(np.int32))
