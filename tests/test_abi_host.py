"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, validates arguments before touching the GPU, and sizes its
workspaces without any [S*k, D] term. No kernel is launched here."""
import ctypes
import json
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    import sparse_mixture_experts_gemv_amd as smoe
    return smoe.load()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    import sparse_mixture_experts_gemv_amd._lib as b
    names = header_functions()
    assert len(names) == 22, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(b.SIGNATURES)


def test_status_strings(lib):
    import sparse_mixture_experts_gemv_amd as smoe
    assert smoe.status_str(0) == "MOE_OK"
    assert smoe.status_str(1) == "MOE_ERR_INVALID_ARGUMENT"
    assert smoe.status_str(2) == "MOE_ERR_UNSUPPORTED"
    assert smoe.status_str(3) == "MOE_ERR_WORKSPACE_TOO_SMALL"
    assert smoe.status_str(4) == "MOE_ERR_LAUNCH"
    assert smoe.status_str(5) == "MOE_ERR_SCRATCH_LIMIT"
    assert smoe.status_str(99) == "MOE_ERR_UNKNOWN"
    assert lib.moe_version() >= 100


# a non-NULL, 16-byte aligned host address: never dereferenced, because every
# call below fails validation before anything is enqueued
FAKE = ctypes.c_void_p(0x100000)
MISALIGNED = ctypes.c_void_p(0x100008)


def test_route_validation(lib):
    r = lib.moe_route_topk
    assert r(FAKE, FAKE, 16, 64, 8, 0, FAKE, FAKE, FAKE, 1 << 20, None) == 1  # k < 1
    assert r(FAKE, FAKE, 16, 64, 8, 9, FAKE, FAKE, FAKE, 1 << 20, None) == 1  # k > E
    assert r(FAKE, FAKE, -1, 64, 8, 2, FAKE, FAKE, FAKE, 1 << 20, None) == 1  # S < 0
    assert r(None, FAKE, 16, 64, 8, 2, FAKE, FAKE, FAKE, 1 << 20, None) == 1  # NULL
    assert r(MISALIGNED, FAKE, 16, 64, 8, 2, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert r(FAKE, FAKE, 16, 96, 8, 2, FAKE, FAKE, FAKE, 1 << 20, None) == 2  # D % 64
    assert r(FAKE, FAKE, 16, 64, 12, 2, FAKE, FAKE, FAKE, 1 << 20, None) == 2  # E % 8
    assert r(FAKE, FAKE, 16, 64, 512, 2, FAKE, FAKE, FAKE, 1 << 20, None) == 2  # E > 256
    assert r(FAKE, FAKE, 16, 64, 64, 2, FAKE, FAKE, FAKE, 16, None) == 3  # workspace (E > 16 needs partial logits)
    assert r(None, None, 0, 64, 8, 2, None, None, None, 0, None) == 0  # S == 0: no-op


def test_sparse_map_validation(lib):
    m = lib.moe_sparse_map
    assert m(FAKE, 16, 2, 0, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 1  # E < 1
    assert m(FAKE, 16, 3, 2, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 1  # k > E
    assert m(FAKE, 16, 2, 8, None, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert m(FAKE, 16, 2, 8, FAKE, FAKE, FAKE, MISALIGNED, FAKE, 1 << 20, None) == 1
    assert m(FAKE, 16, 2, 2048, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, None) == 2  # E > 1024
    assert m(FAKE, 1 << 30, 4, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == 2  # S*k >= 2^31
    assert m(FAKE, 4096, 2, 8, FAKE, FAKE, FAKE, FAKE, FAKE, 4, None) == 3


def test_ffn_validation(lib):
    f = lib.moe_scatter_ffn_fwd
    args = lambda S=16, D=64, F=128, E=8, k=2, ws=1 << 30, x=FAKE: (
        x, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, S, D, F, E, k, FAKE, FAKE, ws, None)
    assert f(*args(k=9)) == 1
    assert f(*args(x=None)) == 1
    assert f(*args(x=MISALIGNED)) == 1
    assert f(*args(D=80)) == 2
    assert f(*args(F=100)) == 2
    assert f(*args(E=2048, k=2)) == 2
    assert f(*args(ws=1024)) == 3
    assert f(*args(S=1, D=1 << 20, F=64)) == 2  # 8192 column tiles of the down GEMM exceed the order table
    assert f(None, None, None, None, None, None, None, 0, 64, 128, 8, 2, None, None, 0, None) == 0


def test_parallel_linear_validation(lib):
    fwd, bwd = lib.moe_parallel_linear_fwd, lib.moe_parallel_linear_bwd
    fa = lambda S=16, k=2, Di=64, Do=128, E=8, gi=0, go=0, ws=1 << 30, x=FAKE, y=FAKE: (
        x, FAKE, None, FAKE, FAKE, S, k, Di, Do, E, gi, go, y, FAKE, ws, None)
    assert fwd(*fa(k=9)) == 1                 # k > E
    assert fwd(*fa(gi=2)) == 1                # grouping flag not 0/1
    assert fwd(*fa(x=None)) == 1
    assert fwd(*fa(y=MISALIGNED)) == 1
    assert fwd(*fa(Di=96)) == 2               # D_in % 64
    assert fwd(*fa(Do=80)) == 2               # D_out % 64
    assert fwd(*fa(E=2048)) == 2
    assert fwd(*fa(ws=1024)) == 3
    assert fwd(*fa(S=1 << 20, Di=1024)) == 2  # S*k*D >= 2^30
    assert fwd(*fa(S=0, x=None, y=None)) == 0
    ba = lambda dx=FAKE, dw=FAKE, dg=FAKE, S=16, ws=1 << 30, dy=FAKE: (
        FAKE, FAKE, None, FAKE, FAKE, dy, S, 2, 64, 128, 8, 0, 0, dx, dw, dg, FAKE, ws, None)
    assert bwd(*ba(dx=None, dw=None, dg=None)) == 1  # nothing requested
    assert bwd(*ba(dy=None)) == 1
    assert bwd(*ba(dw=MISALIGNED)) == 1
    assert bwd(*ba(ws=4096)) == 3
    assert bwd(*ba(S=0, dw=None)) == 0              # nothing to write
    bb = lib.moe_parallel_linear_bwd_bf16w
    assert bb(*ba(dx=None, dw=None, dg=None)) == 1
    assert bb(*ba(dw=MISALIGNED)) == 1
    assert bb(*ba(ws=4096)) == 3
    n = lib.moe_parallel_linear_workspace_bytes(4096, 2, 4096, 14336, 8)
    # fp32 rows [S*k, max(D_in, D_out)] + bf16 slot-order copies of x and g*dy + small tables
    base = 8192 * 14336 * 4 + 8192 * 4096 * 2 + 8192 * 14336 * 2
    assert base <= n <= base + (1 << 20)


def test_ffn_bwd_validation(lib):
    b = lib.moe_scatter_ffn_bwd
    args = lambda S=16, D=64, F=128, E=8, k=2, ws=1 << 30, dx=FAKE, dg=FAKE, x=FAKE, tw=FAKE, sv=None: (
        x, FAKE, FAKE, FAKE, tw, FAKE, FAKE, FAKE, S, D, F, E, k, sv, dx, FAKE, FAKE, FAKE, dg, FAKE, ws, None)
    assert b(*args(k=9)) == 1
    assert b(*args(x=None)) == 1
    assert b(*args(tw=None)) == 1                 # the router weights are required
    assert b(*args(dx=MISALIGNED)) == 1
    assert b(*args(D=96)) == 2
    assert b(*args(F=80)) == 2
    assert b(*args(E=2048)) == 2
    assert b(*args(ws=4096)) == 3
    assert b(*args(sv=MISALIGNED)) == 1
    # the bf16-weight-gradient form shares every check
    bb = lib.moe_scatter_ffn_bwd_bf16w
    assert bb(*args(k=9)) == 1
    assert bb(*args(tw=None)) == 1
    assert bb(*args(F=80)) == 2
    assert bb(*args(ws=4096)) == 3
    t = lib.moe_scatter_ffn_fwd_train
    targs = lambda S=16, D=64, F=128, E=8, k=2, ws=1 << 30, sv=FAKE: (
        FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, S, D, F, E, k, FAKE, sv, FAKE, ws, None)
    assert t(*targs(sv=None)) == 1               # the saved-activations buffer is required
    assert t(*targs(F=80)) == 2
    assert t(*targs(ws=4096)) == 3
    assert t(*targs(S=0, sv=None)) == 0
    n = lib.moe_scatter_ffn_bwd_workspace_bytes(4096, 4096, 14336, 8, 2)
    N = 8192
    base = N * 2 * 14336 * 2 + N * 14336 * 2 + 2 * N * 4096 * 2 + N * 4096 * 4
    assert base <= n <= base + N * 4 * 56 * 4 + (1 << 20)


def test_workspace_has_no_token_replication(lib):
    """Closed form on the ScatterMoE guide's pipeline figure: replicating the
    tokens costs S*k*D*2 bytes (67.1 MB at S=D=4096, k=2, fp16; 2.15 GB over
    32 layers). The atomic-combine workspace grows with D only through the
    fp32 [S, D] accumulator, never through an [S*k, D] term; the default
    workspace adds exactly the fp32 per-route output rows [S*k, D] of the
    ordered combine (outputs of the down projection, not copies of x)."""
    fig = json.load(open(os.path.join(ROOT, "tests", "golden", "page_figures.json")))
    rep = fig["replication_bytes_per_layer"]
    nbytes = rep["S"] * rep["k"] * rep["D"] * rep["bytes_per_element"]
    assert round(nbytes / 1e6, 1) == rep["value_MB"]
    assert round(32 * nbytes / 1e9, 2) == fig["replication_bytes_32_layers"]["value_GB"]
    oh = fig["one_hot_register_elements"]
    assert oh["block_size"] * oh["num_experts"] == oh["value"]
    ws = lambda S, D, F, E, k: lib.moe_scatter_ffn_workspace_bytes_atomic(S, D, F, E, k)
    rows = lambda S, D, F, E, k: lib.moe_scatter_ffn_workspace_bytes(S, D, F, E, k)
    for (S, F, E, k) in [(4096, 14336, 8, 2), (4096, 2048, 256, 8), (8192, 2880, 128, 4)]:
        for D in (4096, 8192):
            # y [S*k, D] fp32 replaces acc [S, D] fp32 (plus a block-order table of at most a few KB)
            assert 0 <= rows(S, D, F, E, k) - ws(S, D, F, E, k) - (S * k - S) * D * 4 < (1 << 20)
        d1, d2 = ws(S, 4096, F, E, k), ws(S, 8192, F, E, k)
        # growth with D: the fp32 accumulator plus a block-order table of a few KB,
        # nowhere near the S*k*D*2 bytes a token copy would add
        extra = (d2 - d1) - S * 4096 * 4
        assert 0 <= extra < (1 << 20) and (d2 - d1) < S * 4096 * 4 + S * k * 4096 * 2 // 16
        # h [S*k, F] bf16 + acc [S, D] fp32 + tile and order tables (small)
        base = S * k * F * 2 + S * 4096 * 4
        assert base <= d1 <= base + (1 << 20)
    # the router and map workspaces do not scale with D at all
    assert lib.moe_route_workspace_bytes(4096, 256) == 8 * 4096 * 256 * 4  # 8 K-splits of partial logits
    assert lib.moe_route_workspace_bytes(4096, 8) == 0  # small-E router keeps logits in registers
    assert lib.moe_sparse_map_workspace_bytes(4096, 8, 256) < 1 << 20


def test_noalloc_scratch_coverage(lib):
    """The no-allocation map serves exactly the maps whose workspace fits its 4 MiB + 4 KiB array:
    every map with E <= 512, every map of fewer than 2^20 routes, and E = 1024 up to 2^22 routes."""
    limit = (4 << 20) + (4 << 10)
    ws = lib.moe_sparse_map_workspace_bytes
    for E in (2, 8, 64, 128, 256, 384, 512):
        for S, k in ((1 << 21, 4), (1 << 22, 8), (1 << 23, 8), ((1 << 27) - 1, 8), (3000, 7)):
            assert ws(S, k, E) <= limit, (S, k, E)
    for E in (513, 600, 777, 1000, 1024):
        for N in (8193, 100_000, (1 << 20) - 1):
            assert ws(N, 1, E) <= limit, (N, E)
    assert ws(1 << 22, 1, 1024) == limit
    assert ws((1 << 22) + 1, 1, 1024) > limit
    assert ws(1 << 23, 1, 1024) > limit


def test_product_path_does_not_use_oracle():
    """The package must not import or load the oracle or fall back to the CPU."""
    pkg = os.path.join(ROOT, "sparse_mixture_experts_gemv_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), f"{fn} mentions the oracle"
