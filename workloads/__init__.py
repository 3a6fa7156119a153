"""Seeded synthetic workloads for the dropless sparse-MoE forward path.

This module only draws inputs. It holds none of the method's arithmetic: no
routing, no sparse map, no expert math. Both the fp64 oracle (tests only) and
the HIP path receive exactly the tensors drawn here.

Shapes follow the model families the ScatterMoE guide and the TritonMoE
abstract benchmark (Mixtral-8x7B layer, DeepSeek-V3, Qwen2-MoE) plus the
GPT-OSS expert count of the Fast-LLM sparse-map pull request (128 experts,
4 per token). No dataset is involved: every tensor is random and seeded.

Recipe:
  * x ~ N(0, 1); W1, W3 ~ N(0, D^-1/2 std); W2 ~ N(0, F^-1/2 std)
    ("1/sqrt(fan_in)" read as a standard deviation).
  * W_gate ~ N(0, 0.02 std) for the tiny and Mixtral shapes, N(0, D^-1/2 std)
    for GPT-OSS and DeepSeek-V3 (router logits close to N(0, 1)).
  * Qwen2-MoE shape: the router is bypassed; each token draws k distinct
    experts, sequentially without replacement, with p(rank r) ~ r^-1.2 over a
    seeded permutation of the experts (Zipf skew). Its gate weights are a flat
    Dirichlet draw (normalised Exp(1) variates), stored as fp32.
  * Every tensor is drawn in fp32 from its own generator, seeded by
    (config, tensor, expert), and rounded once to bf16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np
import torch

TAG_X, TAG_WGATE, TAG_W1, TAG_W3, TAG_W2, TAG_ROUTE = 1, 2, 3, 4, 5, 6


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    cfg_id: int
    S: int
    D: int
    F: int
    E: int
    k: int
    gate_std: Optional[float]  # None -> D ** -0.5
    routing: str = "router"  # "router" | "zipf"
    zipf_s: float = 1.2

    @property
    def wgate_std(self) -> float:
        return self.D ** -0.5 if self.gate_std is None else self.gate_std

    def with_S(self, S: int) -> "MoEConfig":
        return dataclasses.replace(self, S=S)

    def describe(self) -> str:
        return (f"{self.name} S={self.S} D={self.D} F={self.F} E={self.E} "
                f"k={self.k} routing={self.routing}")


CONFIGS = {
    "tiny": MoEConfig("tiny", 1, 128, 256, 512, 8, 2, 0.02),
    "mixtral": MoEConfig("mixtral", 2, 4096, 4096, 14336, 8, 2, 0.02),
    "gptoss": MoEConfig("gptoss", 3, 8192, 2880, 2880, 128, 4, None),
    "dsv3": MoEConfig("dsv3", 4, 4096, 7168, 2048, 256, 8, None),
    "qwen2": MoEConfig("qwen2", 5, 4096, 3584, 2560, 64, 8, None, routing="zipf"),
}
QWEN2_BATCHES = (8, 64, 512, 4096)


def seed_of(cfg_id: int, tag: int, index: int = 0) -> int:
    return cfg_id * 1_000_003 + tag * 10_007 + index


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn_bf16(shape, std: float, seed: int, device) -> torch.Tensor:
    g = _gen(seed, device)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


def gen_x(cfg: MoEConfig, device="cpu", S: Optional[int] = None, tag_index: int = 0) -> torch.Tensor:
    """Token activations [S, D] bf16."""
    S = cfg.S if S is None else S
    return _randn_bf16((S, cfg.D), 1.0, seed_of(cfg.cfg_id, TAG_X, tag_index), device)


def gen_w_gate(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """Router weight [D, E] bf16."""
    return _randn_bf16((cfg.D, cfg.E), cfg.wgate_std, seed_of(cfg.cfg_id, TAG_WGATE), device)


def gen_expert_weights(cfg: MoEConfig, device="cpu", experts=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Stacked expert weights W1, W3 [E, D, F] and W2 [E, F, D], bf16.

    Each expert slice has its own generator, so a slice can be redrawn alone.
    `experts` (optional) restricts the draw to those experts (others stay zero).
    """
    E, D, F = cfg.E, cfg.D, cfg.F
    w1 = torch.zeros((E, D, F), dtype=torch.bfloat16, device=device)
    w3 = torch.zeros((E, D, F), dtype=torch.bfloat16, device=device)
    w2 = torch.zeros((E, F, D), dtype=torch.bfloat16, device=device)
    sd_in, sd_f = D ** -0.5, F ** -0.5
    for e in (range(E) if experts is None else experts):
        w1[e] = _randn_bf16((D, F), sd_in, seed_of(cfg.cfg_id, TAG_W1, e), device)
        w3[e] = _randn_bf16((D, F), sd_in, seed_of(cfg.cfg_id, TAG_W3, e), device)
        w2[e] = _randn_bf16((F, D), sd_f, seed_of(cfg.cfg_id, TAG_W2, e), device)
    return w1, w3, w2


def gen_zipf_routing(cfg: MoEConfig, S: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Skewed expert choices [S, k] int32 and gate weights [S, k] fp32.

    Sequential draws without replacement from p(r) ~ r^-s over ranks r = 1..E
    are taken with Gumbel keys: the k largest of log p + Gumbel noise, in
    descending key order, have the law of k sequential draws without
    replacement. Rank r maps to expert perm[r - 1].
    """
    S = cfg.S if S is None else S
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg.cfg_id, TAG_ROUTE, S)))
    perm = rng.permutation(cfg.E)
    logp = -cfg.zipf_s * np.log(np.arange(1, cfg.E + 1, dtype=np.float64))
    keys = logp[None, :] + rng.gumbel(size=(S, cfg.E))
    ranks = np.argsort(-keys, axis=1, kind="stable")[:, : cfg.k]
    ids = perm[ranks].astype(np.int32)
    ex = rng.exponential(size=(S, cfg.k))
    weights = (ex / ex.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(weights)


def gen_random_ids(S: int, k: int, E: int, seed: int, skew: Optional[float] = None) -> np.ndarray:
    """Distinct expert ids per token [S, k] int32 for sparse-map tests.

    Uniform when skew is None, else Zipf(skew) ranks over the identity order.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    logp = np.zeros(E) if skew is None else -skew * np.log(np.arange(1, E + 1, dtype=np.float64))
    out = np.empty((S, k), dtype=np.int32)
    chunk = max(1, (1 << 22) // max(E, 1))
    for s0 in range(0, S, chunk):
        s1 = min(S, s0 + chunk)
        keys = logp[None, :] + rng.gumbel(size=(s1 - s0, E))
        out[s0:s1] = np.argpartition(-keys, k - 1, axis=1)[:, :k] if k < E else np.argsort(-keys, axis=1)
    return out


def make_problem(cfg: MoEConfig, S: Optional[int] = None, device="cuda", gen_device=None) -> dict:
    """All inputs of `cfg` (optionally with another token count) on `device`.

    Small problems are drawn on the CPU; large ones are drawn on `device`
    (the values then differ from a CPU draw, but every consumer -- the HIP
    path and, through host copies, the oracle -- reads the same tensors).
    """
    S = cfg.S if S is None else S
    if gen_device is None:
        big = cfg.E * cfg.D * cfg.F > (1 << 26)
        gen_device = device if big else "cpu"
    x = gen_x(cfg, gen_device, S=S).to(device)
    wg = gen_w_gate(cfg, gen_device).to(device)
    w1, w3, w2 = (t.to(device) for t in gen_expert_weights(cfg, gen_device))
    p = dict(cfg=cfg, S=S, x=x, wg=wg, w1=w1, w3=w3, w2=w2)
    if cfg.routing == "zipf":
        ids, w = gen_zipf_routing(cfg, S)
        p["ids"] = torch.from_numpy(ids).to(device)
        p["weights"] = torch.from_numpy(w).to(device)
    return p


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a (CPU) bf16 tensor as a uint16 numpy array."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a bf16 tensor."""
    return t.detach().cpu().to(torch.float64).numpy()
