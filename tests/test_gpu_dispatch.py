"""moe_dispatch against the oracle: counts, offsets, perm and dest bit-exact on
every workload's routing shape (incl. invalid tokens, the skewed large-E
case, out-of-range ids), ragged slot counts, the maximum expert count, and
run-to-run determinism."""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_helpers import dev, host, note, require_gpu

pytestmark = pytest.mark.gpu

m = pytest.importorskip("moe_token_routing_amd")


def _check(ids: np.ndarray, E: int, what: str):
    require_gpu()
    note("dispatch %s T=%d k=%d E=%d" % (what, ids.shape[0], ids.shape[1], E))
    got = m.dispatch(dev(ids.astype(np.int32)), E)
    torch.cuda.synchronize()
    ref = O.dispatch(ids, E)
    for name, g, r in zip(("counts", "offsets", "perm", "dest"), got, ref):
        np.testing.assert_array_equal(host(g), r, err_msg="%s: %s" % (what, name))
    return got


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "large_e", "wide_k"])
def test_dispatch_workloads(name):
    w = wl.WORKLOADS[name]
    mask = wl.token_mask(w)
    ids = wl.synthetic_topk_ids(w, mask=mask)
    got = _check(ids, w.E, name)
    if name == "large_e":
        counts = host(got[0])
        hot = wl.hot_expert_ids(w)
        assert counts[hot].sum() == w.T * w.k        # every pick on the 16 hot experts


# up to 1024 slots are one tile, which the place kernel counts itself
@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (3, 2, 5, 1), (100, 7, 33, 2), (200, 5, 4096, 7),
                                         (32, 32, 3, 8), (205, 5, 17, 9), (1000, 8, 256, 3),
                                         (4099, 5, 4096, 4), (2047, 32, 64, 5), (70001, 3, 1000, 6)])
def test_dispatch_random_ids(T, k, E, seed):
    g = np.random.default_rng(seed)
    ids = g.integers(-3, E + 3, size=(T, k)).astype(np.int32)
    ids[g.uniform(size=T) < 0.1] = -1
    _check(ids, E, "random")


def test_dispatch_all_one_expert_and_all_invalid():
    T, k, E = 5000, 8, 4096
    _check(np.full((T, k), E - 1, np.int32), E, "one expert")
    _check(np.full((T, k), -1, np.int32), E, "all invalid")
    _check(np.zeros((T, 1), np.int32), 1, "E=1")
    _check(np.full((100, 8), -1, np.int32), 64, "all invalid, one tile")


def test_dispatch_zero_tokens():
    require_gpu()
    counts, offsets, perm, dest = m.dispatch(torch.empty((0, 4), dtype=torch.int32, device="cuda:0"), 10)
    assert (host(counts) == 0).all() and (host(offsets) == 0).all() and perm.numel() == 0


def test_dispatch_is_deterministic():
    require_gpu()
    w = wl.WORKLOADS["wide_k"]
    ids = dev(wl.synthetic_topk_ids(w, T=4096))
    first = [host(t) for t in m.dispatch(ids, w.E)]
    for _ in range(5):
        again = [host(t) for t in m.dispatch(ids, w.E)]
        for a, b in zip(first, again):
            np.testing.assert_array_equal(a, b)
