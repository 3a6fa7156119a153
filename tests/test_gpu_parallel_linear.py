"""moe_parallel_linear_fwd / moe_parallel_linear_bwd on the GPU against the fp64 oracle.

Every grouping mode (grouped or scattered input and output), with and
without router gates, on shapes that cover each M-tile height (128, 64 and
32 rows), ragged N tiles (D_in or D_out not a multiple of 256), k = 1, many
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
    (700, 2, 256, 320, 8, None),   # 175 rows per expert: 128-row tiles; D_out ragged against 256 columns
    (300, 2, 192, 128, 8, None),   # 75: 64-row tiles; D_in ragged
    (120, 2, 128, 192, 16, 1.2),   # 15: 32-row tiles, skewed routing
    (65, 1, 64, 64, 4, None),      # k = 1
    (40, 4, 128, 256, 64, None),   # 2.5 rows per expert: most experts empty
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


def test_parallel_linear_bwd_no_tokens_zeroes_dw():
    """S = 0: the weight gradient is written as zeros."""
    import sparse_mixture_experts_gemv_amd as smoe
    E, D_in, D_out, k = 4, 64, 128, 2
    w = torch.randn(E, D_in, D_out, device=DEV).to(torch.bfloat16)
    x = torch.empty((0, D_in), dtype=torch.bfloat16, device=DEV)
    dy = torch.empty((0, D_out), dtype=torch.bfloat16, device=DEV)
    offsets = torch.zeros(E + 1, dtype=torch.int32, device=DEV)
    src = torch.empty(0, dtype=torch.int32, device=DEV)
    _, dw, _ = smoe.moe_parallel_linear_bwd(x, w, None, offsets, src, dy, k, need_dx=False, need_dgates=False)
    torch.cuda.synchronize()
    assert dw.shape == (E, D_in, D_out) and torch.count_nonzero(dw).item() == 0
