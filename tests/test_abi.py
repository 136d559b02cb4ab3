"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_routing.h")

m = pytest.importorskip("moe_token_routing_amd")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m.LIB_PATH):
        pytest.fail("libmoe_routing.so is not built (run __graft_entry__.build())")
    return m.lib()


def test_every_declared_function_is_exported(lib):
    names = _declared_functions()
    assert set(names) == {"moe_status_string", "moe_route_workspace_bytes", "moe_route",
                          "moe_dispatch_workspace_bytes", "moe_dispatch", "moe_dispatch_noalloc",
                          "moe_route_dispatch_workspace_bytes", "moe_route_dispatch", "moe_route_dispatch_quant",
                          "moe_norm_quant_nvfp4",
                          "moe_norm_quant_nvfp4_rank_block", "moe_combine",
                          "moe_expert_fc1_workspace_bytes", "moe_expert_fc1_nvfp4",
                          "moe_expert_fc1_swiglu_nvfp4"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(m._SIGNATURES)


def test_status_strings(lib):
    for code in range(0, -8, -1):
        assert m.status_string(code) != "unknown status"
    assert m.status_string(-99) == "unknown status"


def test_workspace_queries():
    assert m.route_workspace_bytes(0, 64, 16, 4, m.MOE_DTYPE_BF16) == 0
    assert m.route_workspace_bytes(16, 64, 16, 4, m.MOE_DTYPE_BF16, logits_in=True) == 0
    bf = m.route_workspace_bytes(8192, 8192, 256, 8, m.MOE_DTYPE_BF16)
    f32 = m.route_workspace_bytes(8192, 8192, 256, 8, m.MOE_DTYPE_F32)
    assert bf >= 3 * 256 * 8192 * 2 + 8192 * 256 * 4 and f32 > bf
    assert bf % 256 == 0
    assert m.dispatch_workspace_bytes(0, 8, 256) == 0
    assert m.dispatch_workspace_bytes(8192, 8, 256) % 256 == 0
    assert m.dispatch_workspace_bytes(8192, 8, 256) >= 64 * 256 * 4
    assert m.dispatch_workspace_bytes(4, 33, 16) == 0            # k out of range


V = ctypes.c_void_p
FAKE = V(1 << 20)   # a non-NULL, 16-byte aligned address that is never dereferenced


def test_combine_rejects_before_launch(lib):
    f = lib.moe_combine
    args = dict(eo=FAKE, R=8, slots=FAKE, w=FAKE, nw=FAKE, gc=0.0, eps=1e-6, T=4, H=64, k=2, out=FAKE)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["eo"], a["R"], a["slots"], a["w"], a["nw"], a["gc"], a["eps"], a["T"], a["H"], a["k"], a["out"], None)

    assert call(H=63) == -2 and call(H=0) == -2 and call(k=0) == -2 and call(k=33) == -2
    assert call(T=-1) == -2 and call(R=-1) == -2 and call(H=16392) == -2
    assert call(eps=-1.0) == -5 and call(eps=float("nan")) == -5 and call(gc=float("inf")) == -5
    assert call(slots=None) == -1 and call(out=None) == -1 and call(eo=None) == -1
    assert call(eo=None, R=0, T=0) == 0           # nothing to do
    assert call(T=0) == 0
    assert call(out=V((1 << 20) + 4)) == -7


def test_norm_quant_rejects_before_launch(lib):
    f = lib.moe_norm_quant_nvfp4
    assert f(FAKE, FAKE, 1.0, 1e-6, FAKE, 4, 40, FAKE, FAKE, None) == -2      # H % 16
    assert f(FAKE, FAKE, 1.0, 1e-6, FAKE, 4, 0, FAKE, FAKE, None) == -2
    assert f(FAKE, FAKE, 1.0, -1e-6, FAKE, 4, 64, FAKE, FAKE, None) == -5
    assert f(FAKE, FAKE, 1.0, 1e-6, None, 4, 64, FAKE, FAKE, None) == -1
    assert f(None, FAKE, 1.0, 1e-6, FAKE, 4, 64, FAKE, FAKE, None) == -1
    assert f(FAKE, FAKE, 1.0, 1e-6, FAKE, 0, 64, None, None, None) == 0


def test_norm_quant_rank_block_rejects_before_launch(lib):
    f = lib.moe_norm_quant_nvfp4_rank_block
    assert f(FAKE, 24, FAKE, 1.0, 1e-6, FAKE, 4, 96, FAKE, FAKE, None) == -2    # shard % 16
    assert f(FAKE, 64, FAKE, 1.0, 1e-6, FAKE, 4, 96, FAKE, FAKE, None) == -2    # H % shard
    assert f(FAKE, 192, FAKE, 1.0, 1e-6, FAKE, 4, 96, FAKE, FAKE, None) == -2   # shard > H
    assert f(FAKE, 0, FAKE, 1.0, 1e-6, FAKE, 4, 96, FAKE, FAKE, None) == -2
    assert f(FAKE, 48, FAKE, 1.0, -1.0, FAKE, 4, 96, FAKE, FAKE, None) == -5
    assert f(None, 48, FAKE, 1.0, 1e-6, FAKE, 4, 96, FAKE, FAKE, None) == -1
    assert f(FAKE, 48, FAKE, 1.0, 1e-6, FAKE, 0, 96, None, None, None) == 0


def test_route_rejects_before_launch(lib):
    f = lib.moe_route

    def call(hidden=FAKE, dtype=1, W=FAKE, bias=FAKE, mask=FAKE, scale=1.0, T=4, H=64, E=16, k=4,
             logits=FAKE, ids=FAKE, w=FAKE, ws=FAKE, wsb=1 << 30):
        return f(hidden, dtype, W, bias, mask, scale, T, H, E, k, logits, ids, w, ws, wsb, None)

    assert call(dtype=7) == -3
    assert call(k=17) == -2 and call(k=0) == -2 and call(k=33, E=64) == -2
    assert call(E=4097, k=4) == -2 and call(H=24) == -2 and call(T=-2) == -2
    assert call(scale=float("nan")) == -5
    assert call(bias=None) == -1 and call(mask=None) == -1 and call(W=None) == -1
    assert call(ws=None) == -4 and call(wsb=16) == -4
    assert call(T=0) == 0
    assert call(ids=V((1 << 20) + 8)) == -7


def test_route_dispatch_rejects_before_launch(lib):
    f = lib.moe_route_dispatch

    def call(hidden=FAKE, dtype=1, W=FAKE, bias=FAKE, mask=FAKE, scale=1.0, T=4, H=64, E=16, k=4,
             logits=FAKE, ids=FAKE, w=FAKE, counts=FAKE, offsets=FAKE, perm=FAKE, dest=FAKE, ws=FAKE,
             wsb=1 << 30):
        return f(hidden, dtype, W, bias, mask, scale, T, H, E, k, logits, ids, w, counts, offsets, perm, dest,
                 ws, wsb, None)

    # the route's checks
    assert call(dtype=7) == -3
    assert call(k=17) == -2 and call(k=0) == -2 and call(E=4097, k=4) == -2 and call(H=24) == -2
    assert call(T=-2) == -2 and call(scale=float("inf")) == -5
    assert call(bias=None) == -1 and call(W=None) == -1 and call(ids=V((1 << 20) + 8)) == -7
    # the dispatch's
    assert call(counts=None) == -1 and call(perm=None) == -1 and call(dest=V((1 << 20) + 4)) == -7
    # the workspace: the route's part and the tile histograms
    assert call(ws=None) == -4 and call(wsb=16) == -4
    need = m.route_dispatch_workspace_bytes(4096, 64, 16, 4, m.MOE_DTYPE_BF16)
    assert call(T=4096, wsb=need - 1) == -4
    assert need == m.route_workspace_bytes(4096, 64, 16, 4, m.MOE_DTYPE_BF16) + m.dispatch_workspace_bytes(4096, 4, 16)
    assert need % 256 == 0
    # logits-in needs only the tile histograms, and one tile of slots none
    assert m.route_dispatch_workspace_bytes(200, 16, 16, 4, m.MOE_DTYPE_BF16, logits_in=True) == 0
    assert m.route_dispatch_workspace_bytes(2000, 16, 16, 4, m.MOE_DTYPE_BF16, logits_in=True) == \
        m.dispatch_workspace_bytes(2000, 4, 16) > 0


def test_route_dispatch_quant_rejects_before_launch(lib):
    f = lib.moe_route_dispatch_quant

    def call(hidden=FAKE, W=FAKE, T=4, H=64, E=16, k=4, counts=FAKE, x=FAKE, Hq=32, nw=FAKE, gc=1.0, eps=1e-6,
             gs=FAKE, packed=FAKE, scales=FAKE, ws=FAKE, wsb=1 << 30):
        return f(hidden, 1, W, FAKE, FAKE, 1.0, T, H, E, k, FAKE, FAKE, FAKE, counts, FAKE, FAKE, FAKE,
                 x, Hq, nw, gc, eps, gs, packed, scales, ws, wsb, None)

    assert call(k=17) == -2 and call(H=24) == -2 and call(counts=None) == -1     # route, dispatch
    assert call(x=None) == -1 and call(gs=None) == -1 and call(packed=None) == -1  # norm + quant
    assert call(Hq=24) == -2 and call(Hq=0) == -2 and call(Hq=(1 << 20)) == -2    # the expert input's width
    assert call(eps=-1.0) == -5 and call(gc=float("nan")) == -5
    assert call(x=V((1 << 20) + 2)) == -7
    assert call(ws=None) == -4


def test_dispatch_rejects_before_launch(lib):
    f = lib.moe_dispatch
    assert f(FAKE, 4, 0, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -2
    assert f(FAKE, 4, 2, 4097, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -2
    assert f(FAKE, 4, 2, 16, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == -1
    assert f(FAKE, 4, 2, 16, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -4
    assert f(FAKE, 4, 2, 16, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == -4


def test_dispatch_noalloc_rejects_before_launch(lib):
    f = lib.moe_dispatch_noalloc
    assert f(FAKE, 4, 0, 16, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert f(FAKE, 4, 33, 64, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert f(FAKE, 4, 2, 4097, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert f(FAKE, -1, 2, 16, FAKE, FAKE, FAKE, FAKE, None) == -2
    assert f(FAKE, 4, 2, 16, None, FAKE, FAKE, FAKE, None) == -1
    assert f(None, 4, 2, 16, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert f(FAKE, 4, 2, 16, FAKE, FAKE, V((1 << 20) + 4), FAKE, None) == -7


def test_expert_fc1_rejects_before_launch(lib):
    f = lib.moe_expert_fc1_nvfp4
    ws = lib.moe_expert_fc1_workspace_bytes(4, 2, 8)
    # tile starts (9 int32, padded to 256 bytes) + one record per possible row tile
    assert ws == 256 + 16 * (1 + 8)   # tiles of 256 rows
    assert lib.moe_expert_fc1_workspace_bytes(4, 2, 0) == 0
    assert lib.moe_expert_fc1_workspace_bytes(-1, 2, 8) == 0
    assert lib.moe_expert_fc1_workspace_bytes(4, 0, 8) == 0
    assert lib.moe_expert_fc1_workspace_bytes(1 << 30, 2, 8) == 0
    assert lib.moe_expert_fc1_workspace_bytes(0, 2, 8) == 256 + 16 * 8
    args = lambda T=4, k=2, K=128, N=256, E=8, ws_b=ws, x=FAKE: (
        x, FAKE, FAKE, FAKE, FAKE, T, k, FAKE, FAKE, FAKE, FAKE, K, N, E, FAKE, FAKE, FAKE, ws_b, None)
    assert f(*args(K=96)) == -2        # K % 64
    assert f(*args(N=200)) == -2       # N % 128
    assert f(*args(E=0)) == -2
    assert f(*args(k=33)) == -2
    assert f(*args(T=-1)) == -2
    assert f(*args(x=None)) == -1
    assert f(*args(ws_b=ws - 1)) == -4
    assert f(*args(T=0)) == 0
    g = lib.moe_expert_fc1_swiglu_nvfp4   # N output columns over 2N weight rows
    assert g(*args(N=96)) == -2        # N % 64
    assert g(*args(N=0)) == -2
    assert g(*args(K=96)) == -2
    assert g(*args(x=None)) == -1
    assert g(*args(ws_b=ws - 1)) == -4
    assert g(*args(T=0)) == 0
    assert g(*args(T=0, N=64)) == 0    # 64 columns: allowed here, not with Relu2
    assert f(*args(T=0, N=64)) == -2
