"""Seeded input generators: determinism, shapes and the routing statistics they promise."""
import numpy as np
import torch

import workloads as wl


def test_seeded_and_bf16():
    cfg = wl.CONFIGS["tiny"]
    a, b = wl.gen_x(cfg), wl.gen_x(cfg)
    assert a.dtype == torch.bfloat16 and a.shape == (cfg.S, cfg.D)
    assert torch.equal(a, b)
    w1, w3, w2 = wl.gen_expert_weights(cfg)
    assert w1.shape == (8, 256, 512) and w2.shape == (8, 512, 256)
    assert not torch.equal(w1, w3)
    # an expert slice can be redrawn alone
    w1b, _, _ = wl.gen_expert_weights(cfg, experts=[3])
    assert torch.equal(w1b[3], w1[3]) and not torch.any(w1b[2] != 0)
    # std of the fan-in reading
    assert abs(float(w1.float().std()) - 256 ** -0.5) < 3e-3
    assert abs(float(wl.gen_w_gate(cfg).float().std()) - 0.02) < 2e-3


def test_zipf_routing_skew():
    cfg = wl.CONFIGS["qwen2"]
    ids, w = wl.gen_zipf_routing(cfg, S=4096)
    assert ids.shape == (4096, 8) and ids.dtype == np.int32
    assert all(len(set(r)) == 8 for r in ids[:500].tolist())
    assert np.allclose(w.sum(1), 1.0, atol=1e-6) and np.all(w > 0)
    load = np.bincount(ids.ravel(), minlength=64)
    ratio = load.max() / load.mean()
    assert 5.0 < ratio < 10.0, ratio  # heavy skew (about 7.8)
    ids2, w2 = wl.gen_zipf_routing(cfg, S=4096)
    assert np.array_equal(ids, ids2) and np.array_equal(w, w2)
    ids8, _ = wl.gen_zipf_routing(cfg, S=8)
    assert len(np.unique(ids8)) < 64


def test_random_ids_distinct():
    ids = wl.gen_random_ids(1000, 8, 256, seed=1)
    assert ids.min() >= 0 and ids.max() < 256
    assert all(len(set(r)) == 8 for r in ids.tolist())
