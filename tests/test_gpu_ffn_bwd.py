"""moe_scatter_ffn_bwd on the GPU against the fp64 oracle.

Small shapes are compared element by element (every gradient, every
element); they cover each tile height of the recompute GEMM (256, 192, 64 and
32 rows) and of the backward GEMMs (192, 128, 64, 32), ragged tiles (D or F not a
multiple of 256), k = 1, empty experts (zero weight gradients) and skewed
routing. Full-size configurations are checked on samples the oracle can
compute: dx and the router-weight gradient of sampled tokens, and 64-column
slices of the weight gradients of sampled experts (a slice of F is exact: the
SwiGLU acts column by column).

Tolerance (derived from the arithmetic): the kernels keep a and b of the
recomputed forward, da and db, and g*dout in bf16 (relative rounding 2^-9
each) and sum in fp32, so a gradient element carries a few bf16 roundings of
its inputs on top of its own rounding: normwise max-rel <= 2e-2 and, per
row, relative L2 <= 2e-2, and MAE within 6x the error of a perfect bf16
answer (dx) or of bf16-rounding the fp32 weight gradient (measured: about
2x). The router-weight gradient is the fp32 dot product <h, c> with h
recomputed from the bf16 a and b, so each h element carries up to ~2 bf16
roundings (~4e-3 relative): max-rel <= 1e-2 (measured: <= 3.3e-3).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, bf16_floor_mae, say

pytestmark = pytest.mark.gpu

SMALL = [  # (S, D, F, E, k, skew): recompute tile from S*k/E (256/192/64/32), dh / dx tiles (192/128/64/32)
    (2000, 128, 192, 4, 2, None),   # 1000 rows per expert: 256-row recompute on the 3-deep weight ring / 192
    (1000, 128, 192, 4, 2, None),   # 500 rows per expert: 256 / 128 (dh) and 192 (dx)
    (1000, 192, 320, 8, 2, None),   # 250 rows per expert: 256 / 128; F and D ragged against 256
    (600, 128, 192, 8, 2, None),    # 150: 192 / 128
    (300, 128, 192, 8, 2, None),    # 75: 64 / 64
    (200, 128, 256, 16, 2, 1.2),    # 25: 32 / 32, skewed
    (40, 256, 128, 64, 8, None),    # 5: most experts empty
    (33, 320, 192, 4, 1, None),     # k = 1
    (300, 64, 128, 1024, 16, None),  # E = 1024, k = 16: the largest expert count, most experts with 0-10 rows
]
ROW_L2_BAR = 2e-2
MAXREL_BAR = 2e-2
FLOOR_FACTOR = 6.0
DG_BAR = 1e-2


def bits(t):
    return wl.bf16_bits(t.cpu())


def grad_close(got, ref, what):
    got = got.astype(np.float64).reshape(ref.shape[0] if ref.ndim == 2 else -1, ref.shape[-1])
    ref = ref.reshape(got.shape)
    d = np.abs(got - ref)
    mae = float(d.mean())
    maxrel = float(d.max() / max(np.abs(ref).max(), 1e-300))
    nz = np.linalg.norm(ref, axis=1) > 0
    row = float((np.linalg.norm(got - ref, axis=1)[nz] / np.linalg.norm(ref, axis=1)[nz]).max()) if nz.any() else 0.0
    floor = bf16_floor_mae(ref)
    say(f"  {what}: MAE {mae:.3e} (bf16 floor {floor:.3e})  max-rel {maxrel:.3e}  worst row L2 {row:.3e}")
    assert np.all(got[~nz] == 0), f"{what}: rows with a zero reference must be exactly zero"
    assert maxrel <= MAXREL_BAR and row <= ROW_L2_BAR and mae <= FLOOR_FACTOR * floor, (what, mae, floor, maxrel, row)


def dg_close(got, ref, what):
    rel = float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))
    say(f"  {what}: max-rel {rel:.3e}")
    assert rel <= DG_BAR, (what, rel)


def problem(S, D, F, E, k, skew, seed):
    cfg = wl.MoEConfig("bwd", 70 + seed % 20, S, D, F, E, k, None)
    p = wl.make_problem(cfg, device=DEV)
    ids = wl.gen_random_ids(S, k, E, seed=seed, skew=skew)
    w = np.random.default_rng(seed).dirichlet(np.ones(k), size=S).astype(np.float32)
    g = torch.Generator(device=DEV).manual_seed(seed)
    dout = (torch.randn((S, D), generator=g, device=DEV) * 0.1).to(torch.bfloat16)
    return p, ids, w, dout


def gpu_bwd(p, ids, w, dout, need=("dx", "dw1", "dw3", "dw2", "dg")):
    import sparse_mixture_experts_gemv_amd as smoe
    E = p["w1"].shape[0]
    _, offsets, _, src = smoe.moe_sparse_map(torch.from_numpy(ids).to(DEV), E)
    out = smoe.moe_scatter_ffn_bwd(p["x"], p["w1"], p["w3"], p["w2"], torch.from_numpy(w).to(DEV), offsets, src,
                                   dout, need=need)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("S,D,F,E,k,skew", SMALL)
def test_ffn_bwd_small_all_elements(oracle_lib, S, D, F, E, k, skew):
    p, ids, w, dout = problem(S, D, F, E, k, skew, seed=S + D + F)
    got = gpu_bwd(p, ids, w, dout)
    ref = oracle_lib.ffn_bwd(bits(p["x"]), bits(p["w1"]), bits(p["w3"]), bits(p["w2"]), ids, w.astype(np.float64),
                             bits(dout))
    tag = f"{S}x{D}x{F} E={E} k={k}"
    grad_close(got["dx"].float().cpu().numpy(), ref["dx"], f"dx {tag}")
    for n in ("dw1", "dw3", "dw2"):
        grad_close(got[n].cpu().numpy(), ref[n], f"{n} {tag}")
    dg_close(got["dg"].cpu().numpy().astype(np.float64), ref["dg"], f"dg {tag}")


@pytest.mark.parametrize("idx", [1, 3, 5, 6])
def test_ffn_bwd_bf16_weight_gradients(oracle_lib, idx):
    """moe_scatter_ffn_bwd_bf16w: dw1, dw3, dw2 are the fp32 call's rounded to bf16 (RNE), bit for
    bit; dx and dg are the fp32 call's; the bf16 gradients are within the bar of the fp64 oracle."""
    import sparse_mixture_experts_gemv_amd as smoe
    S, D, F, E, k, skew = SMALL[idx]
    p, ids, w, dout = problem(S, D, F, E, k, skew, seed=S + D + F)
    _, offsets, _, src = smoe.moe_sparse_map(torch.from_numpy(ids).to(DEV), E)
    args = (p["x"], p["w1"], p["w3"], p["w2"], torch.from_numpy(w).to(DEV), offsets, src, dout)
    g32 = smoe.moe_scatter_ffn_bwd(*args)
    g16 = smoe.moe_scatter_ffn_bwd(*args, dw_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    for n in ("dw1", "dw3", "dw2"):
        assert g16[n].dtype == torch.bfloat16
        assert torch.equal(g16[n], g32[n].to(torch.bfloat16)), n
    assert torch.equal(g16["dx"], g32["dx"]) and torch.equal(g16["dg"], g32["dg"])
    ref = oracle_lib.ffn_bwd(bits(p["x"]), bits(p["w1"]), bits(p["w3"]), bits(p["w2"]), ids, w.astype(np.float64),
                             bits(dout), want=("dw1", "dw3", "dw2"))
    for n in ("dw1", "dw3", "dw2"):
        grad_close(g16[n].float().cpu().numpy(), ref[n], f"{n} bf16 {S}x{D}x{F} E={E} k={k}")


def test_ffn_bwd_subsets_and_reproducible(oracle_lib):
    """Any subset of the outputs equals the full call bit for bit, and calls repeat exactly."""
    p, ids, w, dout = problem(600, 128, 192, 8, 2, None, seed=9)
    full = gpu_bwd(p, ids, w, dout)
    again = gpu_bwd(p, ids, w, dout)
    for n in full:
        assert torch.equal(full[n], again[n]), n
    for need in (("dx",), ("dw1",), ("dw3",), ("dw2",), ("dg",), ("dw1", "dg")):
        part = gpu_bwd(p, ids, w, dout, need=need)
        for n in need:
            assert torch.equal(part[n], full[n]), (need, n)


@pytest.mark.parametrize("dw_dtype", [torch.float32, torch.bfloat16])
def test_ffn_bwd_no_tokens(dw_dtype):
    """S = 0 with weight gradients requested: they are written as zeros (fp32 or bf16)."""
    import sparse_mixture_experts_gemv_amd as smoe
    E, D, F, k = 4, 64, 128, 2
    w1 = torch.randn(E, D, F, device=DEV).to(torch.bfloat16)
    w2 = torch.randn(E, F, D, device=DEV).to(torch.bfloat16)
    z = lambda *s, dt=torch.bfloat16: torch.empty(s, dtype=dt, device=DEV)
    offsets = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    out = smoe.moe_scatter_ffn_bwd(z(0, D), w1, w1, w2, z(0, k, dt=torch.float32), offsets, z(0, dt=torch.int32),
                                   z(0, D), need=("dw1", "dw3", "dw2"), dw_dtype=dw_dtype)
    torch.cuda.synchronize()
    for n in ("dw1", "dw3", "dw2"):
        assert out[n].dtype == dw_dtype
        assert torch.count_nonzero(out[n]).item() == 0


def test_ffn_bwd_no_tokens_with_router_gradient_pointer():
    """S = 0 through the C ABI with weight gradients and a non-NULL router-weight gradient: the call
    writes zero weight gradients and launches nothing over the empty route range."""
    import ctypes

    import sparse_mixture_experts_gemv_amd as smoe
    lib = smoe.load()
    E, D, F, k = 4, 64, 128, 2
    w1 = torch.randn(E, D, F, device=DEV).to(torch.bfloat16)
    w2 = torch.randn(E, F, D, device=DEV).to(torch.bfloat16)
    offsets = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    dw = [torch.full(s, 7.0, dtype=torch.float32, device=DEV) for s in ((E, D, F), (E, D, F), (E, F, D))]
    dg = torch.full((16,), 3.0, dtype=torch.float32, device=DEV)  # a real, aligned pointer; nothing to write
    ws_bytes = smoe.scatter_ffn_bwd_workspace_bytes(0, D, F, E, k)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.moe_scatter_ffn_bwd(None, P(w1), P(w1), P(w2), None, P(offsets), None, None, 0, D, F, E, k, None,
                                 None, P(dw[0]), P(dw[1]), P(dw[2]), P(dg), P(ws), ws.numel(),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0, smoe.status_str(st)
    for t in dw:
        assert torch.count_nonzero(t).item() == 0
    assert torch.all(dg == 3.0)


@pytest.mark.parametrize("name,ntok", [("mixtral", 12), ("gptoss", 8), ("dsv3", 6)])
def test_ffn_bwd_full_size_sampled(oracle_lib, name, ntok):
    """Full-size backward with the router's routing: dx and dg of sampled tokens (the oracle on
    those tokens with only their experts), and 64-column slices of the weight gradients of two
    sampled experts (the oracle on the tokens routed to them, F restricted to the slice)."""
    import sparse_mixture_experts_gemv_amd as smoe
    cfg = wl.CONFIGS[name]
    S, D, F, E, k = cfg.S, cfg.D, cfg.F, cfg.E, cfg.k
    p = wl.make_problem(cfg, device=DEV)
    ids_d, w_d = smoe.moe_route_topk(p["x"], p["wg"], k)
    ids, w = ids_d.cpu().numpy(), w_d.cpu().numpy()
    g = torch.Generator(device=DEV).manual_seed(5)
    dout = (torch.randn((S, D), generator=g, device=DEV) * 0.1).to(torch.bfloat16)
    got = gpu_bwd(p, ids, w, dout)
    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([[0, S - 1], rng.choice(S, ntok - 2, replace=False)]))
    sel = lambda t, idx: t.index_select(0, torch.from_numpy(np.asarray(idx, np.int64)).to(DEV))
    uniq = np.unique(ids[toks])
    remap = np.full(E, -1, np.int32)
    remap[uniq] = np.arange(uniq.size, dtype=np.int32)
    ref = oracle_lib.ffn_bwd(bits(sel(p["x"], toks)), bits(sel(p["w1"], uniq)), bits(sel(p["w3"], uniq)),
                             bits(sel(p["w2"], uniq)), remap[ids[toks]], w[toks].astype(np.float64),
                             bits(sel(dout, toks)), want=("dx", "dg"))
    grad_close(sel(got["dx"], toks).float().cpu().numpy(), ref["dx"], f"{name} dx (sampled tokens)")
    dg_close(got["dg"].cpu().numpy()[toks].astype(np.float64), ref["dg"], f"{name} dg (sampled tokens)")
    counts = np.bincount(ids.reshape(-1), minlength=E)
    experts = [int(np.argmax(counts)), int(rng.choice(np.nonzero(counts)[0]))]
    c0 = (F // 3) // 64 * 64
    for e in experts:
        et = np.nonzero(np.any(ids == e, axis=1))[0]  # tokens routed to e (all their routes kept)
        uq = np.unique(ids[et])
        rm = np.full(E, -1, np.int32)
        rm[uq] = np.arange(uq.size, dtype=np.int32)
        w1s = bits(sel(p["w1"], uq)[:, :, c0:c0 + 64])
        w3s = bits(sel(p["w3"], uq)[:, :, c0:c0 + 64])
        w2s = bits(sel(p["w2"], uq)[:, c0:c0 + 64, :])
        r = oracle_lib.ffn_bwd(bits(sel(p["x"], et)), w1s, w3s, w2s, rm[ids[et]], w[et].astype(np.float64),
                               bits(sel(dout, et)), want=("dw1", "dw3", "dw2"))
        le = rm[e]
        grad_close(got["dw1"][e, :, c0:c0 + 64].cpu().numpy(), r["dw1"][le], f"{name} dw1[{e}] cols {c0}+64")
        grad_close(got["dw3"][e, :, c0:c0 + 64].cpu().numpy(), r["dw3"][le], f"{name} dw3[{e}] cols {c0}+64")
        grad_close(got["dw2"][e, c0:c0 + 64, :].cpu().numpy(), r["dw2"][le], f"{name} dw2[{e}] rows {c0}+64")


@pytest.mark.parametrize("S,D,F,E,k", [(2000, 128, 192, 4, 2), (1000, 128, 192, 4, 2), (600, 128, 192, 8, 2),
                                       (200, 128, 256, 16, 2)])
def test_ffn_training_forward_and_saved_backward(S, D, F, E, k):
    """The training-mode forward returns the same output bit for bit and keeps a, b and h (a and b
    checked against an fp64 product); a backward fed those saved activations skips the
    recomputation and gives bit-identical gradients."""
    import sparse_mixture_experts_gemv_amd as smoe
    p, ids, w, dout = problem(S, D, F, E, k, None, seed=S + 3 * E)
    ids_d, w_d = torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV)
    _, offsets, _, src = smoe.moe_sparse_map(ids_d, E)
    out = smoe.moe_scatter_ffn_fwd(p["x"], p["w1"], p["w3"], p["w2"], w_d, offsets, src)
    saved = torch.empty(smoe.saved_activations_numel(S, F, k), dtype=torch.bfloat16, device=DEV)
    out_t = smoe.moe_scatter_ffn_fwd(p["x"], p["w1"], p["w3"], p["w2"], w_d, offsets, src, saved=saved)
    torch.cuda.synchronize()
    assert torch.equal(out, out_t)
    N = S * k
    ab = saved[:N * 2 * F].view(N, 2 * F).double().cpu()
    srcs = src.cpu().numpy()
    tok = torch.from_numpy(srcs // k)
    exp = torch.from_numpy(ids.reshape(-1)[srcs].astype(np.int64))
    x64 = p["x"].double().cpu()[tok]
    a_ref = torch.einsum("nd,ndf->nf", x64, p["w1"].double().cpu()[exp])
    b_ref = torch.einsum("nd,ndf->nf", x64, p["w3"].double().cpu()[exp])
    for got, ref, name in ((ab[:, :F], a_ref, "a"), (ab[:, F:], b_ref, "b")):
        rel = float((got - ref).abs().max() / ref.abs().max())
        say(f"  saved {name}: max-rel {rel:.3e}")
        assert rel < 1e-2, (name, rel)
    recompute = smoe.moe_scatter_ffn_bwd(p["x"], p["w1"], p["w3"], p["w2"], w_d, offsets, src, dout)
    from_saved = smoe.moe_scatter_ffn_bwd(p["x"], p["w1"], p["w3"], p["w2"], w_d, offsets, src, dout, saved=saved)
    torch.cuda.synchronize()
    for n in recompute:
        assert torch.equal(recompute[n], from_saved[n]), n
