"""The whole forward (route, map, experts, combine) captured as a HIP graph.

Replays run with eager work and host synchronisations between them and each
replay must equal the eager forward bit for bit (the default path is
deterministic), including after the input is refilled in place."""
import pytest
import torch

import workloads as wl
from gpu_util import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,S", [("tiny", None), ("qwen2", 8), ("qwen2", 64), ("mixtral", 512)])
def test_graph_replays_match_eager(name, S):
    import sparse_mixture_experts_gemv_amd as smoe
    cfg = wl.CONFIGS[name]
    p = wl.make_problem(cfg, S=S, device=DEV)
    S = p["x"].shape[0]
    topk = (p["ids"], p["weights"]) if "ids" in p else None
    layer = smoe.MoELayer(p["wg"], p["w1"], p["w3"], p["w2"], cfg.k, S)
    x = p["x"].clone()
    eager = layer.forward(x, topk).clone()
    layer.capture(x, topk)
    for rep in range(3):
        torch.cuda.synchronize()
        noise = torch.randn(1024, device=DEV).sum()  # eager work between replays
        out = layer.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep}"
        del noise
    # new input written in place: the replay follows it
    x.copy_(wl.gen_x(cfg, S=S, tag_index=1).to(DEV))
    fresh = smoe.MoELayer(p["wg"], p["w1"], p["w3"], p["w2"], cfg.k, S).forward(x, topk).clone()
    out = layer.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, fresh)
