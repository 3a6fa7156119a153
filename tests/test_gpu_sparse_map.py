"""moe_sparse_map on the GPU: bit-exact against the oracle's stable counting
sort, on the configurations' expert counts, the Fast-LLM expert-count sweeps
(4..32 and 64..256), both map forms (one workgroup up to 8192 routes, three
passes above), large route counts and the degenerate cases."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def run_map(ids_np, E):
    import sparse_mixture_experts_gemv_amd as smoe
    ids = torch.from_numpy(np.ascontiguousarray(ids_np, dtype=np.int32)).to(DEV)
    out = smoe.moe_sparse_map(ids, E)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def check_exact(oracle_lib, ids, E, what):
    say(f"  map {what}: S={ids.shape[0]} k={ids.shape[1]} E={E}")
    got = run_map(ids, E)
    ref = oracle_lib.sparse_map(ids, E)
    for name, g, r in zip(("counts", "offsets", "sparse_rows", "slot_src"), got, ref):
        assert np.array_equal(g, r), f"{what}: {name} differs at {np.nonzero(g != r)[0][:8]}"
    return got


@pytest.mark.parametrize("E", [4, 8, 16, 32, 64, 96, 128, 256, 1024])
@pytest.mark.parametrize("skew", [None, 1.2])
def test_expert_sweep(oracle_lib, E, skew):
    for S, k in [(1, 1), (7, 2), (1000, min(4, E)), (8192, min(8, E))]:
        ids = wl.gen_random_ids(S, k, E, seed=E * 31 + S, skew=skew)
        check_exact(oracle_lib, ids, E, f"sweep skew={skew}")


@pytest.mark.parametrize("E", [8, 1024])
def test_small_and_general_paths(oracle_lib, E):
    """Maps of up to 8192 routes run in one workgroup, larger ones in three
    passes: both sides of that edge, and chunk edges of the one-workgroup
    form (16 waves of whole 256-route groups)."""
    for S, k in [(4096, 2), (8192, 1), (8193, 1), (4097, 2), (257, 1), (4095, 2), (4111, 2)]:
        ids = wl.gen_random_ids(S, k, E, seed=S * 7 + E, skew=1.2)
        check_exact(oracle_lib, ids, E, "path edge")


@pytest.mark.parametrize("E", [8, 1024])
def test_round_size_edge(oracle_lib, E):
    """From 2^18 routes the three-pass map switches from rounds of 512 routes
    (one per chunk) to rounds of 4096: both sides of that edge, ragged."""
    for S, k in [((1 << 18) - 1, 1), (1 << 18, 1), ((1 << 17) + 1, 2), ((1 << 16) + 3, 4)]:
        ids = np.random.default_rng(S + E).integers(0, E, size=(S, k), dtype=np.int32)
        check_exact(oracle_lib, ids, E, "round-size edge")


@pytest.mark.parametrize("E,skewed", [(1024, False), (600, True)])
def test_chunks_of_several_rounds(oracle_lib, E, skewed):
    """Past 2^23 routes with E >= 512 the count matrix would need more than
    2048 chunks, so each chunk holds two rounds of 4096 routes (the second
    round's ids load while the first is ranked) and the last chunk is
    ragged: 2^20 + 777 tokens x 9 routes."""
    S, k = (1 << 20) + 777, 9
    rng = np.random.default_rng(E)
    if skewed:  # a few hot experts
        ids = np.minimum((E * rng.power(4.0, size=(S, k))).astype(np.int32), E - 1)
    else:
        ids = rng.integers(0, E, size=(S, k), dtype=np.int32)
    check_exact(oracle_lib, ids, E, "two rounds per chunk")


@pytest.mark.parametrize("name", ["tiny", "mixtral", "gptoss", "dsv3", "qwen2"])
def test_config_shapes(oracle_lib, name):
    cfg = wl.CONFIGS[name]
    if cfg.routing == "zipf":
        for S in wl.QWEN2_BATCHES:
            ids, _ = wl.gen_zipf_routing(cfg, S)
            check_exact(oracle_lib, ids, cfg.E, f"{name} S={S}")
    else:
        ids = wl.gen_random_ids(cfg.S, cfg.k, cfg.E, seed=cfg.cfg_id)
        check_exact(oracle_lib, ids, cfg.E, name)


def test_gptoss_router_ids(oracle_lib):
    """GPT-OSS shape: ids from the softmax of random router logits, map bit-exact."""
    import sparse_mixture_experts_gemv_amd as smoe
    cfg = wl.CONFIGS["gptoss"]
    x = wl.gen_x(cfg).to(DEV)
    wg = wl.gen_w_gate(cfg).to(DEV)
    ids, _ = smoe.moe_route_topk(x, wg, cfg.k)
    torch.cuda.synchronize()
    check_exact(oracle_lib, ids.cpu().numpy(), cfg.E, "gptoss router ids")


@pytest.mark.parametrize("S", [1 << 16, 1 << 19, 1 << 21])
def test_large(oracle_lib, S):
    ids = wl.gen_random_ids(S, 4, 128, seed=S)
    check_exact(oracle_lib, ids, 128, "large")


def test_degenerate(oracle_lib):
    check_exact(oracle_lib, np.full((5000, 1), 3, np.int32), 8, "all on one expert")
    check_exact(oracle_lib, np.tile(np.arange(8, dtype=np.int32), (333, 1)), 8, "k = E")
    check_exact(oracle_lib, np.array([[5, 2]], np.int32), 8, "one token")
    check_exact(oracle_lib, np.array([[0]], np.int32), 1, "E = 1")
    ids = wl.gen_random_ids(777, 2, 4, seed=1)
    check_exact(oracle_lib, (ids * 37 + 5).astype(np.int32), 160, "sparse expert set")
    counts, offsets, _, _ = run_map(np.zeros((0, 2), np.int32), 8)
    assert not counts.any() and not offsets.any()


@pytest.mark.parametrize("S,E", [(300, 8), (20000, 64), (300000, 128)])
def test_invalid_ids_get_no_slot(oracle_lib, S, E):
    """Ids outside [0, E) (a precondition violation) get sparse_rows = -1 and
    no slot; the other routes keep the stable order (one-workgroup map, and
    both round sizes of the three-pass map)."""
    bad = wl.gen_random_ids(S, 2, E, seed=3).ravel()
    rng = np.random.default_rng(S)
    pos = rng.choice(bad.size, size=max(2, bad.size // 97), replace=False)
    bad[pos[::2]] = E + rng.integers(0, 5, size=pos[::2].size)
    bad[pos[1::2]] = -1 - rng.integers(0, 5, size=pos[1::2].size)
    counts, offsets, rows, src = run_map(bad.reshape(S, 2), E)
    keep = np.ones(bad.size, bool)
    keep[pos] = False
    assert np.all(rows[pos] == -1)
    ref_src = np.nonzero(keep)[0][np.argsort(bad[keep], kind="stable")]
    n = int(keep.sum())
    assert offsets[-1] == n and np.array_equal(src[:n], ref_src)
    ref_rows = np.full(bad.size, -1, np.int64)
    ref_rows[ref_src] = np.arange(n)
    assert np.array_equal(rows, ref_rows)
    assert np.array_equal(counts, np.bincount(bad[keep], minlength=E))


def test_deterministic():
    ids = wl.gen_random_ids(32768, 8, 256, seed=11)
    a = run_map(ids, 256)
    for _ in range(3):
        b = run_map(ids, 256)
        assert all(np.array_equal(u, v) for u, v in zip(a, b))
