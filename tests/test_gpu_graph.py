"""The whole forward (route, map, experts, combine) captured as a HIP graph.

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
