"""The whole forward (route, map, experts, combine), and a training step of the
experts (training-mode forward + backward), captured as HIP graphs.

Replays run with eager work and host synchronisations between them and each
replay must equal the eager forward bit for bit (the default path is
deterministic), including after the input is refilled in place. The atomic
combine (its accumulator cleared by a kernel inside the graph) is compared
within bf16 rounding, since its fp32 adds land in any order."""
import pytest
import torch

import workloads as wl
from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,S,atomic", [("tiny", None, False), ("qwen2", 8, False), ("qwen2", 64, False),
                                           ("mixtral", 512, False), ("tiny", None, True), ("qwen2", 64, True)])
def test_graph_replays_match_eager(name, S, atomic):
    import sparse_mixture_experts_gemv_amd as smoe
    cfg = wl.CONFIGS[name]
    p = wl.make_problem(cfg, S=S, device=DEV)
    S = p["x"].shape[0]
    topk = (p["ids"], p["weights"]) if "ids" in p else None
    layer = smoe.MoELayer(p["wg"], p["w1"], p["w3"], p["w2"], cfg.k, S, atomic=atomic)
    x = p["x"].clone()
    eager = layer.forward(x, topk).clone()
    layer.capture(x, topk)
    for rep in range(3):
        torch.cuda.synchronize()
        noise = torch.randn(1024, device=DEV).sum()  # eager work between replays
        out = layer.replay()
        torch.cuda.synchronize()
        if atomic:
            torch.testing.assert_close(out.float(), eager.float(), rtol=2e-2, atol=2e-2, msg=f"replay {rep}")
        else:
            assert torch.equal(out, eager), f"replay {rep}"
        del noise
    # new input written in place: the replay follows it
    x.copy_(wl.gen_x(cfg, S=S, tag_index=1).to(DEV))
    fresh = smoe.MoELayer(p["wg"], p["w1"], p["w3"], p["w2"], cfg.k, S, atomic=atomic).forward(x, topk).clone()
    out = layer.replay()
    torch.cuda.synchronize()
    if atomic:  # fp32 atomics: the order of the adds may differ between runs
        torch.testing.assert_close(out.float(), fresh.float(), rtol=2e-2, atol=2e-2)
    else:
        assert torch.equal(out, fresh)


@pytest.mark.parametrize("dw_dtype", [torch.float32, torch.bfloat16])
def test_graph_training_step_replays_match_eager(dw_dtype):
    """A training step of the experts (training-mode forward keeping a|b and h, then the backward on
    them) captured as one HIP graph: every replay gives the eager step's output and gradients bit
    for bit (the path is deterministic)."""
    import numpy as np
    import sparse_mixture_experts_gemv_amd as smoe
    S, D, F, E, k = 600, 128, 192, 8, 2
    cfg = wl.MoEConfig("graph_train", 66, S, D, F, E, k, None)
    p = wl.make_problem(cfg, device=DEV)
    ids = torch.from_numpy(wl.gen_random_ids(S, k, E, seed=3)).to(DEV)
    w = torch.from_numpy(np.random.default_rng(3).dirichlet(np.ones(k), size=S).astype(np.float32)).to(DEV)
    _, offsets, _, src = smoe.moe_sparse_map(ids, E)
    g = torch.Generator(device=DEV).manual_seed(4)
    dout = (torch.randn((S, D), generator=g, device=DEV) * 0.1).to(torch.bfloat16)
    saved = torch.empty(smoe.saved_activations_numel(S, F, k), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((S, D), dtype=torch.bfloat16, device=DEV)
    fws = torch.empty(smoe.scatter_ffn_workspace_bytes(S, D, F, E, k), dtype=torch.uint8, device=DEV)
    bws = torch.empty(smoe.scatter_ffn_bwd_workspace_bytes(S, D, F, E, k), dtype=torch.uint8, device=DEV)

    def step():
        smoe.moe_scatter_ffn_fwd(p["x"], p["w1"], p["w3"], p["w2"], w, offsets, src, out, fws, saved=saved)
        return smoe.moe_scatter_ffn_bwd(p["x"], p["w1"], p["w3"], p["w2"], w, offsets, src, dout, workspace=bws,
                                        saved=saved, dw_dtype=dw_dtype)

    eager = {n: t.clone() for n, t in step().items()}
    out_eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        grads = step()
    for rep in range(3):
        torch.cuda.synchronize()
        torch.randn(1024, device=DEV).sum()  # eager work between replays
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_eager), f"out, replay {rep}"
        for n in eager:
            assert torch.equal(grads[n], eager[n]), f"{n}, replay {rep}"
