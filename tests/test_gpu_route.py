"""moe_route_topk on the GPU against the oracle router H(X) = Softmax(TopK(X W_gate, k)).

The GPU sums logits in fp32 and the oracle in fp64, so tokens whose fp64
logits hold a near-tie (two of the top k+1 within 1e-4) may legally rank
differently; every other token must match exactly. Gates are compared to
the oracle's fp64 softmax over the experts the GPU chose."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, host_bits, near_tie_tokens, say

pytestmark = pytest.mark.gpu


def check_route(o, x, wg, k, what, tokens=None):
    import sparse_mixture_experts_gemv_amd as smoe
    S = x.shape[0]
    ids, w = smoe.moe_route_topk(x, wg, k)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    tokens = np.arange(S) if tokens is None else tokens
    xs = host_bits(x[torch.from_numpy(tokens).to(x.device)])
    ref_ids, _, logits = o.route(xs, host_bits(wg), k)
    _, ref_w, _ = o.route(xs, host_bits(wg), k, ids_in=ids[tokens])
    ties = set(near_tie_tokens(logits, k).tolist())
    mism = [i for i in range(len(tokens)) if not np.array_equal(ids[tokens[i]], ref_ids[i])]
    bad = [i for i in mism if i not in ties]
    say(f"  route {what}: S={S} E={wg.shape[1]} k={k} checked={len(tokens)} near-ties={len(ties)} "
        f"differing={len(mism)}")
    assert not bad, f"{what}: ids differ on non-tied tokens {bad[:5]}"
    for i in mism:  # a legal flip only swaps experts whose fp64 logits are within the tie band
        chosen = np.sort(logits[i, ids[tokens[i]]])
        best = np.sort(logits[i, ref_ids[i]])
        assert np.all(np.abs(chosen - best) < 1e-4)
    assert np.all(ids >= 0) and np.all(ids < wg.shape[1])
    assert all(len(set(r)) == k for r in ids.tolist())
    err = np.abs(w[tokens] - ref_w).max()
    assert err < 1e-5, (what, err)
    assert np.allclose(w.sum(1), 1.0, atol=1e-5)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["tiny", "mixtral", "gptoss", "dsv3"])
def test_route_configs(oracle_lib, name):
    cfg = wl.CONFIGS[name]
    x = wl.gen_x(cfg).to(DEV)
    wg = wl.gen_w_gate(cfg).to(DEV)
    check_route(oracle_lib, x, wg, cfg.k, name)  # every token


@pytest.mark.parametrize("S,D,E,k", [(1, 64, 8, 1), (37, 128, 16, 3), (300, 192, 64, 8), (129, 256, 256, 16),
                                     (1000, 512, 96, 6), (65, 64, 8, 8),
                                     (50, 640, 16, 4), (19, 4096, 8, 2), (2053, 1152, 128, 4),
                                     (333, 192, 24, 5), (77, 256, 200, 16), (40, 128, 248, 11)])
def test_route_shapes(oracle_lib, S, D, E, k):
    cfg = wl.MoEConfig("route", 90 + E, S, D, 64, E, k, None)
    check_route(oracle_lib, wl.gen_x(cfg).to(DEV), wl.gen_w_gate(cfg).to(DEV), k, f"shape {S}x{D}x{E}")


@pytest.mark.parametrize("E", [8, 64])
def test_route_exact_ties(oracle_lib, E):
    """Duplicated router columns tie exactly: the lower expert id ranks first
    (E = 8 runs the register router, E = 64 the MFMA logits + top-k pass)."""
    import sparse_mixture_experts_gemv_amd as smoe
    h = E // 2
    cfg = wl.MoEConfig("ties", 77, 200, 128, 64, E, 2, 0.05)
    half = wl.gen_w_gate(cfg)[:, :h]
    wg = torch.cat([half, half], dim=1).contiguous().to(DEV)
    ids, w = smoe.moe_route_topk(wl.gen_x(cfg).to(DEV), wg, 2)
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    assert np.all(ids[:, 0] < h) and np.all(ids[:, 1] == ids[:, 0] + h)
    assert np.allclose(w, 0.5, atol=1e-7)
