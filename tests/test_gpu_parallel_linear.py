"""moe_parallel_linear_fwd / moe_parallel_linear_bwd on the GPU against the fp64 oracle.

Every grouping mode (grouped or scattered input and output), with and
without router gates, on shapes that cover each M-tile height (192 full
and short, 128, 64 and 32 rows), ragged N tiles (D_in or D_out not a multiple of 256), k = 1, many
empty experts (whose weight gradient must be exactly zero) and skewed
routing. Outputs are compared element by element with the tolerance bar of
the forward pass; the weight gradient is fp32 and is compared the same way
per expert row.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, assert_close, say

pytestmark = pytest.mark.gpu

MODES = [(False, False), (False, True), (True, False), (True, True)]
SHAPES = [  # (S, k, D_in, D_out, E, skew)
    (2000, 2, 128, 320, 4, None),  # 1000 rows per expert: 256-row tiles, D_out ragged
    (1000, 2, 128, 192, 4, None),  # 500 rows per expert: 192-row tiles
    (1000, 2, 128, 256, 8, None),  # 250: 128-row tiles
    (700, 2, 256, 320, 8, None),   # 175: 192-row tiles on the short-tile path; D_out ragged against 256 columns
    (300, 2, 192, 128, 8, None),   # 75: 64-row tiles; D_in ragged
    (120, 2, 128, 192, 16, 1.2),   # 15: 32-row tiles, skewed routing
    (65, 1, 64, 64, 4, None),      # k = 1
    (40, 4, 128, 256, 64, None),   # 2.5 rows per expert: most experts empty
    (30, 20, 64, 128, 24, None),   # k = 20: the finalize pass takes the routes in two chunks
    (300, 16, 64, 128, 1024, None),  # E = 1024, k = 16: ~5 rows per expert, the largest expert count
]


def bits(t):
    return wl.bf16_bits(t.cpu())


def pl_problem(S, k, D_in, D_out, E, skew, gi, go, seed):
    g = torch.Generator().manual_seed(seed)
    ids = wl.gen_random_ids(S, k, E, seed=seed, skew=skew)
    x = (torch.randn((S * k if gi else S), D_in, generator=g)).to(torch.bfloat16)
    w = (torch.randn(E, D_in, D_out, generator=g) * D_in ** -0.5).to(torch.bfloat16)
    gates = torch.from_numpy(np.random.default_rng(seed).dirichlet(np.ones(k), size=S).astype(np.float32))
    dy = torch.randn((S * k if go else S), D_out, generator=g).to(torch.bfloat16)
    return dict(ids=ids, x=x, w=w, gates=gates, dy=dy)


def gpu_map(ids, E):
    import sparse_mixture_experts_gemv_amd as smoe
    _, offsets, _, src = smoe.moe_sparse_map(torch.from_numpy(ids).to(DEV), E)
    return offsets, src


def case_id(shape, mode, gated):
    S, k, D_in, D_out, E, skew = shape
    return f"S{S}k{k}_{D_in}x{D_out}_E{E}{'_zipf' if skew else ''}_{'G' if mode[0] else 'S'}{'G' if mode[1] else 'S'}" \
           f"{'_gated' if gated else ''}"


CASES = [(s, m, g) for s in SHAPES for m in MODES for g in (True, False)]


@pytest.mark.parametrize("shape,mode,gated", CASES, ids=[case_id(*c) for c in CASES])
def test_parallel_linear_fwd(oracle_lib, shape, mode, gated):
    import sparse_mixture_experts_gemv_amd as smoe
    S, k, D_in, D_out, E, skew = shape
    gi, go = mode
    p = pl_problem(S, k, D_in, D_out, E, skew, gi, go, seed=S + D_in + 7 * E)
    offsets, src = gpu_map(p["ids"], E)
    gates = p["gates"].to(DEV) if gated else None
    y = smoe.moe_parallel_linear_fwd(p["x"].to(DEV), p["w"].to(DEV), gates, offsets, src, k, gi, go)
    torch.cuda.synchronize()
    ref = oracle_lib.parallel_linear(bits(p["x"]), bits(p["w"]), p["ids"],
                                     p["gates"].double().numpy() if gated else None, gi, go)
    assert_close(y.float().cpu().numpy(), ref, "y " + case_id(shape, mode, gated), configured=False)


@pytest.mark.parametrize("shape,mode,gated", CASES, ids=[case_id(*c) for c in CASES])
def test_parallel_linear_bwd(oracle_lib, shape, mode, gated):
    import sparse_mixture_experts_gemv_amd as smoe
    S, k, D_in, D_out, E, skew = shape
    gi, go = mode
    p = pl_problem(S, k, D_in, D_out, E, skew, gi, go, seed=3 * S + D_out + E)
    offsets, src = gpu_map(p["ids"], E)
    gates = p["gates"].to(DEV) if gated else None
    dx, dw, dg = smoe.moe_parallel_linear_bwd(p["x"].to(DEV), p["w"].to(DEV), gates, offsets, src, p["dy"].to(DEV),
                                              k, gi, go)
    torch.cuda.synchronize()
    rdx, rdw, rdg = oracle_lib.parallel_linear_bwd(bits(p["x"]), bits(p["w"]), p["ids"], bits(p["dy"]),
                                                   p["gates"].double().numpy() if gated else None, gi, go)
    cid = case_id(shape, mode, gated)
    assert_close(dx.float().cpu().numpy(), rdx, "dx " + cid, configured=False)
    got_dw = dw.cpu().numpy().astype(np.float64)
    used = np.unique(p["ids"])
    empty = np.setdiff1d(np.arange(E), used)
    assert np.all(got_dw[empty] == 0.0), "experts without routes must get a zero weight gradient"
    assert_close(got_dw[used].reshape(-1, D_out), rdw[used].reshape(-1, D_out), "dw " + cid, configured=False)
    m = np.abs(dg.cpu().numpy().astype(np.float64) - rdg)
    rel = float(m.max() / max(np.abs(rdg).max(), 1e-300))
    say(f"  dgates {cid}: max-rel {rel:.3e}")
    assert rel < 2e-3, rel


def test_parallel_linear_bwd_partial_outputs_and_reproducible(oracle_lib):
    """Each gradient alone equals its value from the full call, bit for bit, and repeats exactly."""
    import sparse_mixture_experts_gemv_amd as smoe
    S, k, D_in, D_out, E = 300, 2, 192, 128, 8
    p = pl_problem(S, k, D_in, D_out, E, None, False, False, seed=5)
    offsets, src = gpu_map(p["ids"], E)
    args = (p["x"].to(DEV), p["w"].to(DEV), p["gates"].to(DEV), offsets, src, p["dy"].to(DEV), k)
    full = smoe.moe_parallel_linear_bwd(*args)
    again = smoe.moe_parallel_linear_bwd(*args)
    only_dx = smoe.moe_parallel_linear_bwd(*args, need_dw=False, need_dgates=False)[0]
    only_dw = smoe.moe_parallel_linear_bwd(*args, need_dx=False, need_dgates=False)[1]
    only_dg = smoe.moe_parallel_linear_bwd(*args, need_dx=False, need_dw=False)[2]
    torch.cuda.synchronize()
    for a, b in zip(full, again):
        assert torch.equal(a, b)
    assert torch.equal(full[0], only_dx) and torch.equal(full[1], only_dw) and torch.equal(full[2], only_dg)


@pytest.mark.parametrize("shape", [SHAPES[2], SHAPES[5], SHAPES[7]], ids=["128rows", "32rows_zipf", "empty_experts"])
def test_parallel_linear_bwd_bf16_dw(oracle_lib, shape):
    """moe_parallel_linear_bwd_bf16w: dw is the fp32 call's dw rounded to bf16 (RNE), bit for bit;
    dx and dgates are the fp32 call's; dw is also within the bar of the fp64 oracle."""
    import sparse_mixture_experts_gemv_amd as smoe
    S, k, D_in, D_out, E, skew = shape
    p = pl_problem(S, k, D_in, D_out, E, skew, False, True, seed=11 * S + E)
    offsets, src = gpu_map(p["ids"], E)
    args = (p["x"].to(DEV), p["w"].to(DEV), p["gates"].to(DEV), offsets, src, p["dy"].to(DEV), k, False, True)
    dx32, dw32, dg32 = smoe.moe_parallel_linear_bwd(*args)
    dx16, dw16, dg16 = smoe.moe_parallel_linear_bwd(*args, dw_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert dw16.dtype == torch.bfloat16
    assert torch.equal(dw16, dw32.to(torch.bfloat16))
    assert torch.equal(dx16, dx32) and torch.equal(dg16, dg32)
    _, rdw, _ = oracle_lib.parallel_linear_bwd(bits(p["x"]), bits(p["w"]), p["ids"], bits(p["dy"]),
                                               p["gates"].double().numpy(), False, True)
    used = np.unique(p["ids"])
    got = dw16.float().cpu().numpy().astype(np.float64)
    assert np.all(np.delete(got, used, axis=0) == 0.0)
    assert_close(got[used].reshape(-1, D_out), rdw[used].reshape(-1, D_out), f"dw bf16 {shape}", configured=False)


@pytest.mark.parametrize("dw_dtype", [torch.float32, torch.bfloat16])
def test_parallel_linear_bwd_no_tokens_zeroes_dw(dw_dtype):
    """S = 0: the weight gradient is written as zeros (fp32 or bf16)."""
    import sparse_mixture_experts_gemv_amd as smoe
    E, D_in, D_out, k = 4, 64, 128, 2
    w = torch.randn(E, D_in, D_out, device=DEV).to(torch.bfloat16)
    x = torch.empty((0, D_in), dtype=torch.bfloat16, device=DEV)
    dy = torch.empty((0, D_out), dtype=torch.bfloat16, device=DEV)
    offsets = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    src = torch.empty(0, dtype=torch.int32, device=DEV)
    _, dw, _ = smoe.moe_parallel_linear_bwd(x, w, None, offsets, src, dy, k, need_dx=False, need_dgates=False,
                                            dw_dtype=dw_dtype)
    torch.cuda.synchronize()
    assert dw.dtype == dw_dtype
    assert dw.shape == (E, D_in, D_out) and torch.count_nonzero(dw).item() == 0


@pytest.mark.parametrize("name,ntok", [("mixtral", 16), ("dsv3", 6)])
def test_parallel_linear_full_size_sampled(oracle_lib, name, ntok):
    """The benchmark's configuration (up-projection x [S, D] by index -> grouped [S*k, F], router
    gates) at full size, checked against the oracle on samples it can compute: forward rows,
    input-gradient rows and router-gate gradients of sampled tokens (the oracle run on those tokens
    alone, with only the experts they use), and 64 x 64 blocks of every expert's weight gradient
    (the oracle on the matching column slices of x and dy, over all tokens)."""
    import sparse_mixture_experts_gemv_amd as smoe
    cfg = wl.CONFIGS[name]
    S, D, F, E, k = cfg.S, cfg.D, cfg.F, cfg.E, cfg.k
    p = wl.make_problem(cfg, device=DEV)
    x, w = p["x"], p["w1"]
    ids, gates = smoe.moe_route_topk(x, p["wg"], k)
    _, offsets, rows, src = smoe.moe_sparse_map(ids, E)
    g = torch.Generator(device=DEV).manual_seed(11)
    dy = torch.randn((S * k, F), generator=g, device=DEV).to(torch.bfloat16)
    y = smoe.moe_parallel_linear_fwd(x, w, gates, offsets, src, k, False, True)
    dx, dw, dg = smoe.moe_parallel_linear_bwd(x, w, gates, offsets, src, dy, k, False, True)
    torch.cuda.synchronize()
    ids_h, gates_h, rows_h = ids.cpu().numpy(), gates.cpu().numpy().astype(np.float64), rows.cpu().numpy()
    toks = np.unique(np.concatenate([[0, S - 1], np.random.default_rng(3).choice(S, ntok - 2, replace=False)]))
    tsel = torch.from_numpy(toks).to(DEV)
    # sub-problem: the sampled tokens, their experts relabelled 0..U-1 (same order, so the stable
    # slot order of the sub-problem is the full one restricted to these routes)
    uniq = np.unique(ids_h[toks])
    remap = np.full(E, -1, np.int32)
    remap[uniq] = np.arange(uniq.size, dtype=np.int32)
    sub_ids, sub_g = remap[ids_h[toks]], gates_h[toks]
    w_sub = bits(w.index_select(0, torch.from_numpy(uniq.astype(np.int64)).to(DEV)))
    full_slots = rows_h.reshape(S, k)[toks].reshape(-1)            # route order of the sampled tokens
    sub_rows = oracle_lib.sparse_map(sub_ids, uniq.size)[2]         # their slots in the sub-problem
    y_ref = oracle_lib.parallel_linear(bits(x[tsel]), w_sub, sub_ids, sub_g, False, True)
    assert_close(y[torch.from_numpy(full_slots).to(DEV)].float().cpu().numpy(), y_ref[sub_rows],
                 f"{name} y (sampled routes)", configured=False)
    dy_sub = np.zeros((sub_ids.size, F), dtype=np.uint16)
    dy_sub[sub_rows] = bits(dy[torch.from_numpy(full_slots).to(DEV)])
    rdx, _, rdg = oracle_lib.parallel_linear_bwd(bits(x[tsel]), w_sub, sub_ids, dy_sub, sub_g, False, True,
                                                 want=("dx", "dg"))
    assert_close(dx[tsel].float().cpu().numpy(), rdx, f"{name} dx (sampled tokens)", configured=False)
    got_dg = dg.cpu().numpy()[toks].astype(np.float64)
    rel = float(np.max(np.abs(got_dg - rdg)) / np.max(np.abs(rdg)))
    say(f"  {name} dgates (sampled tokens): max-rel {rel:.3e}")
    assert rel < 2e-3, rel
    for (r0, c0) in [(0, 0), (D - 64, F - 64), (D // 2, F // 3 // 64 * 64)]:
        _, rdw, _ = oracle_lib.parallel_linear_bwd(bits(x[:, r0:r0 + 64]), bits(w[:, r0:r0 + 64, c0:c0 + 64]),
                                                   ids_h, bits(dy[:, c0:c0 + 64]), gates_h, False, True,
                                                   want=("dw",))
        got = dw[:, r0:r0 + 64, c0:c0 + 64].cpu().numpy().astype(np.float64)
        assert_close(got.reshape(-1, 64), rdw.reshape(-1, 64), f"{name} dw block ({r0}, {c0})", configured=False)
