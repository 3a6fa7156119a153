"""Seeded random shapes against the fp64 oracle: forward (both combines),
FFN backward (fp32 and bf16 weight gradients) and ParallelLinear (a random
grouping mode each).

The hand-picked shapes of the other test files cover each tile height and
edge on purpose; these draw D and F (multiples of 64), E, k, S and the load
skew at random, so combinations nobody picked (ragged column tiles with
short experts, many empty experts next to a hot one, k close to E) are
exercised too. Every element is compared with the bars of the hand-picked
tests. The list is fixed by its seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, assert_close, oracle_ffn_rows

pytestmark = pytest.mark.gpu


def random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 4, 6, 8, 16, 24, 64, 128]))
        k = int(rng.integers(1, min(E, 8) + 1))
        S = int(rng.choice([1, 2, 5, 9, 17, 64, 100, 300, 700]))
        D = 64 * int(rng.integers(1, 9))
        F = 64 * int(rng.integers(1, 9))
        skew = None if rng.random() < 0.5 else float(rng.choice([0.8, 1.2, 2.0]))
        out.append((S, D, F, E, k, skew, 1000 + i))
    return out


FWD = random_shapes(20, 7)
BWD = random_shapes(12, 8)
PL = random_shapes(12, 9)


def shape_id(c):
    S, D, F, E, k, skew, seed = c
    return f"S{S}_D{D}_F{F}_E{E}_k{k}" + (f"_zipf{skew}" if skew else "")


def routing(S, k, E, skew, seed):
    ids = wl.gen_random_ids(S, k, E, seed=seed, skew=skew)
    w = np.random.default_rng(seed).dirichlet(np.ones(k), size=S).astype(np.float32)
    return ids, w


@pytest.mark.parametrize("atomic", [False, True], ids=["rows", "atomic"])
@pytest.mark.parametrize("case", FWD, ids=[shape_id(c) for c in FWD])
def test_random_forward(oracle_lib, case, atomic):
    import sparse_mixture_experts_gemv_amd as smoe
    S, D, F, E, k, skew, seed = case
    cfg = wl.MoEConfig("rand", seed % 50 + 20, S, D, F, E, k, None)
    p = wl.make_problem(cfg, device=DEV)
    ids, w = routing(S, k, E, skew, seed)
    _, offsets, _, src = smoe.moe_sparse_map(torch.from_numpy(ids).to(DEV), E)
    out = smoe.moe_scatter_ffn_fwd(p["x"], p["w1"], p["w3"], p["w2"], torch.from_numpy(w).to(DEV), offsets, src,
                                   atomic=atomic)
    torch.cuda.synchronize()
    ref = oracle_ffn_rows(oracle_lib, p, ids, w, np.arange(S))
    assert_close(out.float().cpu().numpy().astype(np.float64), ref, f"random fwd {shape_id(case)}", configured=False)


@pytest.mark.parametrize("case", BWD, ids=[shape_id(c) for c in BWD])
def test_random_backward(oracle_lib, case):
    import sparse_mixture_experts_gemv_amd as smoe
    from test_gpu_ffn_bwd import bits, dg_close, grad_close
    S, D, F, E, k, skew, seed = case
    cfg = wl.MoEConfig("randb", seed % 50 + 20, S, D, F, E, k, None)
    p = wl.make_problem(cfg, device=DEV)
    ids, w = routing(S, k, E, skew, seed)
    g = torch.Generator(device=DEV).manual_seed(seed)
    dout = (torch.randn((S, D), generator=g, device=DEV) * 0.1).to(torch.bfloat16)
    _, offsets, _, src = smoe.moe_sparse_map(torch.from_numpy(ids).to(DEV), E)
    args = (p["x"], p["w1"], p["w3"], p["w2"], torch.from_numpy(w).to(DEV), offsets, src, dout)
    got = smoe.moe_scatter_ffn_bwd(*args)
    got16 = smoe.moe_scatter_ffn_bwd(*args, dw_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle_lib.ffn_bwd(bits(p["x"]), bits(p["w1"]), bits(p["w3"]), bits(p["w2"]), ids, w.astype(np.float64),
                             bits(dout))
    tag = shape_id(case)
    grad_close(got["dx"].float().cpu().numpy(), ref["dx"], f"dx {tag}")
    for n in ("dw1", "dw3", "dw2"):
        grad_close(got[n].cpu().numpy(), ref[n], f"{n} {tag}")
        assert torch.equal(got16[n], got[n].to(torch.bfloat16)), n
    dg_close(got["dg"].cpu().numpy().astype(np.float64), ref["dg"], f"dg {tag}")


@pytest.mark.parametrize("case", PL, ids=[shape_id(c) for c in PL])
def test_random_parallel_linear(oracle_lib, case):
    import sparse_mixture_experts_gemv_amd as smoe
    from test_gpu_parallel_linear import bits, pl_problem
    S, D_in, D_out, E, k, skew, seed = case
    gi, go, gated = (seed % 2 == 0), (seed % 3 == 0), (seed % 5 != 0)
    p = pl_problem(S, k, D_in, D_out, E, skew, gi, go, seed)
    _, offsets, _, src = smoe.moe_sparse_map(torch.from_numpy(p["ids"]).to(DEV), E)
    gates = p["gates"].to(DEV) if gated else None
    y = smoe.moe_parallel_linear_fwd(p["x"].to(DEV), p["w"].to(DEV), gates, offsets, src, k, gi, go)
    dx, dw, dg = smoe.moe_parallel_linear_bwd(p["x"].to(DEV), p["w"].to(DEV), gates, offsets, src, p["dy"].to(DEV),
                                              k, gi, go)
    torch.cuda.synchronize()
    g64 = p["gates"].double().numpy() if gated else None
    ry = oracle_lib.parallel_linear(bits(p["x"]), bits(p["w"]), p["ids"], g64, gi, go)
    rdx, rdw, rdg = oracle_lib.parallel_linear_bwd(bits(p["x"]), bits(p["w"]), p["ids"], bits(p["dy"]), g64, gi, go)
    tag = f"{shape_id(case)} {'G' if gi else 'S'}{'G' if go else 'S'}{' gated' if gated else ''}"
    assert_close(y.float().cpu().numpy(), ry, "y " + tag, configured=False)
    assert_close(dx.float().cpu().numpy(), rdx, "dx " + tag, configured=False)
    used = np.unique(p["ids"])
    got_dw = dw.cpu().numpy().astype(np.float64)
    assert np.all(np.delete(got_dw, used, axis=0) == 0.0)
    assert_close(got_dw[used].reshape(-1, D_out), rdw[used].reshape(-1, D_out), "dw " + tag, configured=False)
    rel = float(np.max(np.abs(dg.cpu().numpy().astype(np.float64) - rdg)) / max(np.max(np.abs(rdg)), 1e-300))
    assert rel < 2e-3, (tag, rel)
