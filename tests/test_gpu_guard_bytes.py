"""Out-of-bounds write check: every output and workspace buffer of the C-ABI
calls is placed between guard regions of a known byte pattern, and the
pattern is checked after each call. The outputs themselves start filled with
all-ones bytes (NaN for bf16 and fp32, -1 for int32), so the check also
shows that each output is written in full.

The shapes are ragged on purpose: D and F that are not multiples of the
128- or 256-column tiles, expert row counts that leave partial last M tiles,
and maps on both sides of the one-workgroup limit. These calls are ordinary
in-bounds calls; the test expects no fault, it checks that the masked
stores at the ragged edges stay inside their buffers."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

GUARD = 4096      # bytes on each side (keeps the 16-byte alignment of the inner view)
PATTERN = 0x5A    # guard bytes
FILL = 0xFF       # initial content of the outputs


class Guarded:
    """A device buffer of `nbytes` between two guard regions."""

    def __init__(self, nbytes: int, fill: int = FILL):
        self.nbytes = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), PATTERN, dtype=torch.uint8, device=DEV)
        self.buf[GUARD:GUARD + nbytes] = fill

    def view(self, dtype, shape):
        inner = self.buf[GUARD:GUARD + self.nbytes]
        return inner.view(dtype).view(shape)

    def check(self, what: str):
        head = self.buf[:GUARD]
        tail = self.buf[GUARD + self.nbytes:]
        assert bool(torch.all(head == PATTERN)), f"{what}: bytes before the buffer were written"
        assert bool(torch.all(tail == PATTERN)), f"{what}: bytes after the buffer were written"


def guarded(shape, dtype):
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    g = Guarded(n)
    return g, g.view(dtype, shape)


def fully_written(t: torch.Tensor, what: str):
    """No element still holds the all-ones fill."""
    raw = t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)
    assert not bool(torch.any(raw == -1)), f"{what}: some elements were not written"


FFN_SHAPES = [  # (S, D, F, E, k): ragged columns and partial tiles at several tile heights
    (1000, 320, 192, 4, 2),    # 500 rows per expert: 256-row tiles, D and F ragged against 256 / 128
    (600, 192, 320, 8, 2),     # 150: 192-row tiles
    (300, 320, 192, 8, 2),     # 75: 64-row tiles
    (37, 192, 192, 16, 4),     # ~9: 32-row tiles
    (2000, 128, 192, 4, 2),    # 1000: 256-row tiles on the 3-deep weight ring
]


def problem(S, D, F, E, k, seed):
    cfg = wl.MoEConfig("guard", 40 + seed % 30, S, D, F, E, k, None)
    p = wl.make_problem(cfg, device=DEV)
    ids = wl.gen_random_ids(S, k, E, seed=seed)
    w = np.random.default_rng(seed).dirichlet(np.ones(k), size=S).astype(np.float32)
    return p, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)


@pytest.mark.parametrize("S,E,k", [(37, 8, 2), (129, 256, 16), (3000, 64, 8), (5000, 128, 4)])
def test_guard_route_and_map(S, E, k):
    """Router outputs and workspace; map outputs and workspace (one-workgroup form up to 8192
    routes, the three-pass form above)."""
    import sparse_mixture_experts_gemv_amd as smoe
    D = 192
    cfg = wl.MoEConfig("guard-route", 33, S, D, 64, E, k, None)
    x, wg = wl.gen_x(cfg).to(DEV), wl.gen_w_gate(cfg).to(DEV)
    gi, ids = guarded((S, k), torch.int32)
    gw, w = guarded((S, k), torch.float32)
    gws_r = Guarded(max(smoe.route_workspace_bytes(S, E), 16), fill=0)
    smoe.moe_route_topk(x, wg, k, ids, w, gws_r.view(torch.uint8, (gws_r.nbytes,)))
    gc, counts = guarded((E,), torch.int32)
    go, offsets = guarded((E + 1,), torch.int32)
    gr, rows = guarded((S * k,), torch.int32)
    gs, src = guarded((S * k,), torch.int32)
    gws_m = Guarded(max(smoe.sparse_map_workspace_bytes(S, k, E), 16), fill=0)
    smoe.moe_sparse_map(ids, E, (counts, offsets, rows, src), gws_m.view(torch.uint8, (gws_m.nbytes,)))
    torch.cuda.synchronize()
    for g, what in ((gi, "topk_ids"), (gw, "topk_weights"), (gws_r, "route workspace"), (gc, "expert_counts"),
                    (go, "expert_offsets"), (gr, "sparse_rows"), (gs, "slot_src"), (gws_m, "map workspace")):
        g.check(what)
    for t, what in ((ids, "topk_ids"), (w, "topk_weights"), (counts, "expert_counts"), (offsets, "expert_offsets"),
                    (rows, "sparse_rows"), (src, "slot_src")):
        fully_written(t, what)
    say(f"  guards intact: route + map S={S} E={E} k={k}")


@pytest.mark.parametrize("atomic", [False, True], ids=["rows", "atomic"])
@pytest.mark.parametrize("S,D,F,E,k", FFN_SHAPES)
def test_guard_ffn_forward(S, D, F, E, k, atomic):
    import sparse_mixture_experts_gemv_amd as smoe
    p, ids, w = problem(S, D, F, E, k, seed=S + D)
    _, offsets, _, src = smoe.moe_sparse_map(ids, E)
    go, out = guarded((S, D), torch.bfloat16)
    gws = Guarded(smoe.scatter_ffn_workspace_bytes(S, D, F, E, k, atomic), fill=0)
    smoe.moe_scatter_ffn_fwd(p["x"], p["w1"], p["w3"], p["w2"], w, offsets, src, out,
                             gws.view(torch.uint8, (gws.nbytes,)), atomic=atomic)
    torch.cuda.synchronize()
    go.check("out")
    gws.check("workspace")
    fully_written(out, "out")
    say(f"  guards intact: forward {S}x{D}x{F} E={E} k={k} {'atomic' if atomic else 'rows'}")


@pytest.mark.parametrize("S,D,F,E,k", FFN_SHAPES)
def test_guard_ffn_training_and_backward(S, D, F, E, k):
    """Training-mode forward (a | b and h land in the caller's buffer) and the backward with every
    output guarded."""
    import sparse_mixture_experts_gemv_amd as smoe
    p, ids, w = problem(S, D, F, E, k, seed=S + F)
    _, offsets, _, src = smoe.moe_sparse_map(ids, E)
    g = torch.Generator(device=DEV).manual_seed(3)
    dout = (torch.randn((S, D), generator=g, device=DEV) * 0.1).to(torch.bfloat16)
    gsv, saved = guarded((smoe.saved_activations_numel(S, F, k),), torch.bfloat16)
    out = smoe.moe_scatter_ffn_fwd(p["x"], p["w1"], p["w3"], p["w2"], w, offsets, src, saved=saved)
    torch.cuda.synchronize()
    gsv.check("saved activations")
    fully_written(saved, "saved activations")
    assert out.shape == (S, D)
    lib = smoe.load()
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    for dw16 in (False, True):
        dt = torch.bfloat16 if dw16 else torch.float32
        gdx, dx = guarded((S, D), torch.bfloat16)
        gw1, dw1 = guarded((E, D, F), dt)
        gw3, dw3 = guarded((E, D, F), dt)
        gw2, dw2 = guarded((E, F, D), dt)
        gdg, dg = guarded((S, k), torch.float32)
        gws = Guarded(smoe.scatter_ffn_bwd_workspace_bytes(S, D, F, E, k), fill=0)
        fn = lib.moe_scatter_ffn_bwd_bf16w if dw16 else lib.moe_scatter_ffn_bwd
        st = fn(P(p["x"]), P(p["w1"]), P(p["w3"]), P(p["w2"]), P(w), P(offsets), P(src), P(dout), S, D, F, E, k,
                None, P(dx), P(dw1), P(dw3), P(dw2), P(dg), P(gws.view(torch.uint8, (gws.nbytes,))),
                gws.nbytes, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        assert st == 0, smoe.status_str(st)
        for gg, t, what in ((gdx, dx, "dx"), (gw1, dw1, "dw1"), (gw3, dw3, "dw3"), (gw2, dw2, "dw2"), (gdg, dg, "dg")):
            gg.check(f"{what} ({'bf16' if dw16 else 'fp32'} dW)")
            fully_written(t, what)
        gws.check("backward workspace")
    say(f"  guards intact: training forward + backward {S}x{D}x{F} E={E} k={k}")


@pytest.mark.parametrize("grouped_in,grouped_out", [(False, False), (False, True), (True, False), (True, True)])
def test_guard_parallel_linear(grouped_in, grouped_out):
    import sparse_mixture_experts_gemv_amd as smoe
    S, D_in, D_out, E, k = 300, 320, 192, 8, 2
    p, ids, w = problem(S, D_in, D_out, E, k, seed=11)
    _, offsets, _, src = smoe.moe_sparse_map(ids, E)
    x = p["x"] if not grouped_in else torch.randn((S * k, D_in), device=DEV).to(torch.bfloat16)
    W = p["w1"]
    rows_out = S * k if grouped_out else S
    gy, y = guarded((rows_out, D_out), torch.bfloat16)
    gws = Guarded(smoe.parallel_linear_workspace_bytes(S, k, D_in, D_out, E), fill=0)
    ws = gws.view(torch.uint8, (gws.nbytes,))
    smoe.moe_parallel_linear_fwd(x, W, w, offsets, src, k, grouped_in, grouped_out, y, ws)
    torch.cuda.synchronize()
    gy.check("y")
    fully_written(y, "y")
    dy = torch.randn((rows_out, D_out), device=DEV).to(torch.bfloat16)
    lib = smoe.load()
    import ctypes
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    gdx, dx = guarded(tuple(x.shape), torch.bfloat16)
    gdw, dw = guarded((E, D_in, D_out), torch.float32)
    gdg, dg = guarded((S, k), torch.float32)
    st = lib.moe_parallel_linear_bwd(P(x), P(W), P(w), P(offsets), P(src), P(dy), S, k, D_in, D_out, E,
                                     int(grouped_in), int(grouped_out), P(dx), P(dw), P(dg), P(ws), gws.nbytes,
                                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, smoe.status_str(st)
    for gg, t, what in ((gdx, dx, "dx"), (gdw, dw, "dw"), (gdg, dg, "dgates")):
        gg.check(what)
        fully_written(t, what)
    gws.check("workspace")
