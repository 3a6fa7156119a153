"""moe_sparse_map_noalloc (the sparse map on the library's static per-GPU
scratch) against moe_sparse_map with a caller workspace, through the C ABI:
two calls in a row, the second with a smaller input, both bit-exact against
the workspace call and against the oracle's stable counting sort; the
largest maps the scratch covers; and the host-side rejection of a map that
needs more scratch than the array holds."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def ids_for(S, k, E, seed, skew=False):
    g = torch.Generator(device=DEV).manual_seed(seed)
    logits = torch.randn((S, E), generator=g, device=DEV)
    if skew:  # a few hot experts
        logits[:, : max(1, E // 16)] += 2.0
    return logits.topk(k, dim=1).indices.to(torch.int32).contiguous()


def outputs(S, k, E, fill):
    return tuple(torch.full((n,), fill, dtype=torch.int32, device=DEV) for n in (E, E + 1, S * k, S * k))


def call_noalloc(ids, E, out):
    import sparse_mixture_experts_gemv_amd as smoe
    S, k = ids.shape
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    return smoe.load().moe_sparse_map_noalloc(P(ids), S, k, E, *(P(t) for t in out),
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def check_against_workspace_call(oracle_lib, ids, E, what):
    import sparse_mixture_experts_gemv_amd as smoe
    S, k = ids.shape
    got = outputs(S, k, E, -7)
    st = call_noalloc(ids, E, got)
    assert st == 0, smoe.status_str(st)
    ref = smoe.moe_sparse_map(ids, E)  # caller workspace
    torch.cuda.synchronize()
    for g, r, n in zip(got, ref, ("expert_counts", "expert_offsets", "sparse_rows", "slot_src")):
        assert torch.equal(g, r), (what, n)
    o = oracle_lib.sparse_map(ids.cpu().numpy(), E)
    for g, r, n in zip(got, o, ("expert_counts", "expert_offsets", "sparse_rows", "slot_src")):
        assert np.array_equal(g.cpu().numpy(), r), (what, n, "oracle")
    say(f"  no-alloc map {what}: S={S} k={k} E={E} bit-exact (workspace call and oracle)")


def test_noalloc_two_calls_second_smaller(oracle_lib):
    """The first call fills the scratch with a large map's counts; the second, smaller call (still
    the multi-pass form, which reads the scratch) must not see any of them; a third stays below the
    one-workgroup limit (no scratch)."""
    check_against_workspace_call(oracle_lib, ids_for(1 << 18, 4, 128, seed=1), 128, "large (2^20 routes)")
    check_against_workspace_call(oracle_lib, ids_for(5000, 4, 128, seed=2, skew=True), 128, "smaller (20000 routes)")
    check_against_workspace_call(oracle_lib, ids_for(700, 8, 64, seed=3), 64, "one workgroup (5600 routes)")


@pytest.mark.parametrize("S,k,E", [(1 << 21, 4, 128), (1 << 16, 8, 512), (32768, 8, 1024), (1 << 18, 16, 1024)])
def test_noalloc_largest_covered_maps(oracle_lib, S, k, E):
    """Maps at the scratch's limits: every map with E <= 512 fits, and E = 1024 up to 2^22 routes
    (1024 chunks of 4096 routes: a 4 MiB count matrix, the whole array)."""
    check_against_workspace_call(oracle_lib, ids_for(S, k, E, seed=S + E), E, "at the scratch limit")


def test_noalloc_rejects_maps_beyond_the_scratch():
    """E = 1024 with 2^23 routes needs an 8 MiB count matrix: MOE_ERR_SCRATCH_LIMIT, before anything
    is enqueued (the outputs keep their fill)."""
    import sparse_mixture_experts_gemv_amd as smoe
    S, k, E = 1 << 19, 16, 1024
    g = torch.Generator(device=DEV).manual_seed(4)
    ids = torch.randint(0, E, (S, k), generator=g, device=DEV, dtype=torch.int32)
    out = outputs(S, k, E, -7)
    st = call_noalloc(ids, E, out)
    torch.cuda.synchronize()
    assert smoe.status_str(st) == "MOE_ERR_SCRATCH_LIMIT"
    assert all(bool(torch.all(t == -7)) for t in out)
    with pytest.raises(smoe.MoEError, match="MOE_ERR_SCRATCH_LIMIT"):
        smoe.moe_sparse_map_noalloc(ids, E, out)


def test_noalloc_python_binding_and_empty_map():
    import sparse_mixture_experts_gemv_amd as smoe
    ids = ids_for(300, 2, 16, seed=5)
    a = smoe.moe_sparse_map_noalloc(ids, 16, outputs(300, 2, 16, -7))
    b = smoe.moe_sparse_map(ids, 16)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    empty = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    out = outputs(0, 2, 16, -7)
    smoe.moe_sparse_map_noalloc(empty, 16, out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[0]).item() == 0 and torch.count_nonzero(out[1]).item() == 0
