"""moe_dispatch_noalloc (the dispatch with the library's static device
scratch, for callers that cannot allocate) against moe_dispatch with a
workspace, through the C ABI: bit for bit on two calls in a row, the second
with a smaller input, so the second reads a scratch array that still holds
the first call's larger histograms; and on the shapes that take each of the
dispatch's launch sequences (one tile, fused tile sums, separate scan)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle as O
import workloads as wl
from gpu_helpers import DEV, dev, host, note, require_gpu

pytestmark = pytest.mark.gpu

m = pytest.importorskip("moe_token_routing_amd")


def _both(ids, E):
    """(noalloc outputs, workspace outputs) for the same ids, both via the C ABI."""
    lib = m.lib()
    T, k = ids.shape
    ids_d = dev(ids)
    outs = []
    for use_ws in (False, True):
        counts = torch.full((E,), -7, dtype=torch.int32, device=DEV)
        offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
        perm = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
        dest = torch.full((T * k,), -7, dtype=torch.int32, device=DEV)
        ptr = lambda t: ctypes.c_void_p(t.data_ptr())
        stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        if use_ws:
            nbytes = lib.moe_dispatch_workspace_bytes(T, k, E)
            ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device=DEV)
            rc = lib.moe_dispatch(ptr(ids_d), T, k, E, ptr(counts), ptr(offsets), ptr(perm), ptr(dest),
                                  ptr(ws), nbytes, stream)
        else:
            rc = lib.moe_dispatch_noalloc(ptr(ids_d), T, k, E, ptr(counts), ptr(offsets), ptr(perm), ptr(dest),
                                          stream)
        assert rc == 0, m.status_string(rc)
        torch.cuda.synchronize()
        outs.append([host(t) for t in (counts, offsets, perm, dest)])
    return outs


def _ids(g, T, k, E, invalid=0.05):
    ids = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[g.uniform(size=(T, k)) < invalid] = -1
    return ids


def test_noalloc_matches_workspace_call_twice_shrinking():
    require_gpu()
    g = np.random.default_rng(90)
    # first the prefill batch (64 tiles, fused tile sums), then a smaller one
    # over more experts: the scratch holds the first call's histograms
    w = wl.WORKLOADS["prefill"]
    for T, k, E in [(w.T, w.k, w.E), (3000, 6, 1000)]:
        note("dispatch noalloc T=%d k=%d E=%d" % (T, k, E))
        ids = _ids(g, T, k, E)
        (a, b) = _both(ids, E)
        for name, x, y in zip(("counts", "offsets", "perm", "dest"), a, b):
            np.testing.assert_array_equal(x, y, err_msg=name)
        for name, x, r in zip(("counts", "offsets", "perm", "dest"), a, O.dispatch(ids, E)):
            np.testing.assert_array_equal(x, r, err_msg=name + " vs oracle")


@pytest.mark.parametrize("T,k,E", [(100, 8, 256), (4096, 8, 2560), (70001, 3, 1000), (0, 4, 16)])
def test_noalloc_each_launch_sequence(T, k, E):
    """One tile (place only), the separate column scan (tiles^2 E large),
    many tiles with fused sums, and no slots at all."""
    require_gpu()
    g = np.random.default_rng(T + E)
    note("dispatch noalloc T=%d k=%d E=%d" % (T, k, E))
    ids = _ids(g, T, k, E) if T else np.zeros((0, k), np.int32)
    (a, b) = _both(ids, E)
    for name, x, y in zip(("counts", "offsets", "perm", "dest"), a, b):
        np.testing.assert_array_equal(x, y, err_msg=name)
