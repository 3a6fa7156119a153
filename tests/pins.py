"""Pins of the fp64 oracle to things other than itself.

Each pin takes an `oracle.Oracle` instance and raises AssertionError when the
oracle disagrees with what the pages or the mathematics fix:

  * brute force: every expert on every token in fp64 numpy (dense matmuls),
    masked by the gate matrix (ScatterMoE guide, "1. The Anatomy of
    ParallelLinear" and "2. The Hidden Cost of Activation Materialization");
  * a library routine: the sparse map equals numpy's stable argsort by expert,
    and offsets equal the exclusive cumulative sum of numpy's bincount (guide,
    "2. Grouped Coordinate Indexing Without Padding", Histogram/Offsets
    equations); the Fast-LLM correctness list (unique rows, rows inside
    disjoint expert ranges, histogram counts, determinism);
  * the router H(X) = Softmax(TopK(X W_gate, k)) against numpy argsort of
    numpy logits and scipy's softmax; k = E gives the full softmax; exact
    ties go to the lower expert id;
  * closed forms: E = 1, k = 1 is the dense SwiGLU FFN; experts that share
    their weights give the dense SwiGLU FFN for any routing whose gates sum
    to one;
  * exact invariances: token permutation, expert relabelling, scaling of W2
    and of the gates by two.

The module is also run against deliberately broken copies of the oracle
(tests/test_oracle_mutants.py) to show that each plausible mistake fails
at least one pin.
"""
from __future__ import annotations

import numpy as np
import scipy.special
import torch

import workloads as wl


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    return wl.bf16_bits(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16))


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def small_problem(S=48, D=64, F=96, E=8, k=2, seed=0, gate_std=None, shared_experts=False):
    """Random bf16 problem (bit arrays) small enough for brute force."""
    rng = np.random.default_rng(seed)
    x = bf16_bits_from_f32(rng.standard_normal((S, D)))
    wg = bf16_bits_from_f32(rng.standard_normal((D, E)) * (gate_std or D ** -0.5))
    if shared_experts:
        w1 = np.broadcast_to(bf16_bits_from_f32(rng.standard_normal((D, F)) * D ** -0.5), (E, D, F)).copy()
        w3 = np.broadcast_to(bf16_bits_from_f32(rng.standard_normal((D, F)) * D ** -0.5), (E, D, F)).copy()
        w2 = np.broadcast_to(bf16_bits_from_f32(rng.standard_normal((F, D)) * F ** -0.5), (E, F, D)).copy()
    else:
        w1 = bf16_bits_from_f32(rng.standard_normal((E, D, F)) * D ** -0.5)
        w3 = bf16_bits_from_f32(rng.standard_normal((E, D, F)) * D ** -0.5)
        w2 = bf16_bits_from_f32(rng.standard_normal((E, F, D)) * F ** -0.5)
    return dict(x=x, wg=wg, w1=w1, w3=w3, w2=w2, k=k, E=E)


def dense_swiglu(x, w1, w3, w2):
    """Textbook SwiGLU FFN in fp64 numpy: (SiLU(x W1) * (x W3)) W2."""
    a = x @ w1
    b = x @ w3
    return (a * scipy.special.expit(a) * b) @ w2


def brute_force_layer(p, ids, weights):
    """Run every expert on every token and mask by the dense gate matrix."""
    x = bits_to_f64(p["x"])
    S = x.shape[0]
    E = p["E"]
    G = np.zeros((S, E))
    for j in range(ids.shape[1]):
        G[np.arange(S), ids[:, j]] += weights[:, j]
    out = np.zeros((S, x.shape[1]))
    for e in range(E):
        ye = dense_swiglu(x, bits_to_f64(p["w1"][e]), bits_to_f64(p["w3"][e]), bits_to_f64(p["w2"][e]))
        out += G[:, e:e + 1] * ye
    return out


def rel_err(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------- pins --

def pin_router_library(o, seed=1):
    """ids = stable argsort of -logits (library), gates = scipy softmax of the chosen logits."""
    for (S, D, E, k) in [(64, 96, 8, 2), (40, 64, 16, 4), (30, 32, 64, 8)]:
        p = small_problem(S=S, D=D, F=32, E=E, k=k, seed=seed + E)
        ids, w, logits = o.route(p["x"], p["wg"], k)
        ref_logits = bits_to_f64(p["x"]) @ bits_to_f64(p["wg"])
        assert np.allclose(logits, ref_logits, rtol=1e-12, atol=1e-12), "router logits"
        ref_ids = np.argsort(-ref_logits, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref_ids), "router top-k ids"
        ref_w = scipy.special.softmax(np.take_along_axis(ref_logits, ref_ids, 1), axis=1)
        assert np.allclose(w, ref_w, rtol=1e-12, atol=1e-14), "router gates"
        assert np.allclose(w.sum(1), 1.0, atol=1e-14), "gates sum to one"
        assert np.all(np.diff(w, axis=1) <= 0), "gates descending"
        assert all(len(set(r)) == k for r in ids.tolist()), "distinct experts per token"


def pin_router_full_softmax(o, seed=2):
    """k = E: the gates are the full softmax over all experts, sorted descending."""
    p = small_problem(S=20, D=48, F=16, E=6, k=6, seed=seed)
    ids, w, logits = o.route(p["x"], p["wg"], 6)
    full = scipy.special.softmax(bits_to_f64(p["x"]) @ bits_to_f64(p["wg"]), axis=1)
    assert np.allclose(np.take_along_axis(full, ids, 1), w, rtol=1e-12, atol=1e-15)
    assert np.allclose(np.sort(full, axis=1)[:, ::-1], w, rtol=1e-12, atol=1e-15)


def pin_router_ties(o, seed=3):
    """Exactly tied logits (duplicated W_gate columns) go to the lower expert id."""
    rng = np.random.default_rng(seed)
    D, E = 32, 8
    base = rng.standard_normal((D, 4)) * 0.2
    wg = bf16_bits_from_f32(np.concatenate([base, base], axis=1))  # expert e and e+4 tie
    x = bf16_bits_from_f32(rng.standard_normal((16, D)))
    ids, w, _ = o.route(x, wg, 2)
    for r, wr in zip(ids, w):
        assert r[0] < 4 and r[1] == r[0] + 4, "tie must rank the lower id first"
        assert abs(wr[0] - 0.5) < 1e-15 and abs(wr[1] - 0.5) < 1e-15


def pin_router_given_ids(o, seed=4):
    """With ids supplied, the gates are the softmax of exactly those logits."""
    p = small_problem(S=24, D=40, F=16, E=8, k=3, seed=seed)
    ids_in = wl.gen_random_ids(24, 3, 8, seed=seed)
    ids, w, logits = o.route(p["x"], p["wg"], 3, ids_in=ids_in)
    assert np.array_equal(ids, ids_in)
    ref_w = scipy.special.softmax(np.take_along_axis(logits, ids_in, 1), axis=1)
    assert np.allclose(w, ref_w, rtol=1e-12, atol=1e-15)


def check_map(ids, E, counts, offsets, rows, src):
    flat = np.ascontiguousarray(ids).reshape(-1)
    n = flat.size
    ref_src = np.argsort(flat, kind="stable").astype(np.int32)
    assert np.array_equal(src, ref_src), "slot_src = stable argsort by expert"
    ref_counts = np.bincount(flat, minlength=E).astype(np.int32)
    assert np.array_equal(counts, ref_counts), "histogram"
    assert offsets[0] == 0 and np.array_equal(offsets[1:], np.cumsum(ref_counts)), "offsets"
    assert np.array_equal(np.sort(rows), np.arange(n)), "sparse rows unique (a permutation)"
    assert np.array_equal(rows[src], np.arange(n)), "sparse_rows and slot_src are inverse"
    assert np.all(rows >= offsets[flat]) and np.all(rows < offsets[flat + 1]), "rows inside expert range"
    assert np.all(np.diff(offsets) >= 0) and offsets[-1] == n, "ranges disjoint and covering"


def pin_sparse_map(o, seed=5):
    """Stable counting sort = numpy stable argsort; Fast-LLM invariants; E sweeps; edge cases."""
    cases = []
    for E in (4, 8, 16, 32, 64, 96, 128, 256):
        k = min(4, E)
        cases.append((wl.gen_random_ids(257, k, E, seed=seed + E), E))
        cases.append((wl.gen_random_ids(301, k, E, seed=seed + 7 * E, skew=1.2), E))
    cases.append((wl.gen_random_ids(128, 4, 128, seed=9), 128))  # GPT-OSS: 128 experts, 4 per token
    cases.append((np.zeros((0, 2), np.int32), 8))  # no tokens
    cases.append((np.array([[3, 1]], np.int32), 8))  # one token
    cases.append((np.full((50, 1), 5, np.int32), 8))  # all on one expert, others empty
    cases.append((np.tile(np.arange(6, dtype=np.int32), (9, 1)), 6))  # k = E
    for ids, E in cases:
        a = o.sparse_map(ids, E)
        check_map(ids, E, *a)
        b = o.sparse_map(ids, E)
        assert all(np.array_equal(u, v) for u, v in zip(a, b)), "deterministic"


def pin_brute_force(o, seed=6):
    """Per-token oracle = every expert on every token, masked by the gate matrix."""
    for (E, k) in [(8, 2), (4, 4), (16, 3)]:
        p = small_problem(S=40, D=64, F=96, E=E, k=k, seed=seed + E)
        ids, w, _ = o.route(p["x"], p["wg"], k)
        out = o.ffn(p["x"], p["w1"], p["w3"], p["w2"], ids, w, nthreads=3)
        ref = brute_force_layer(p, ids, w)
        assert rel_err(out, ref) < 1e-12, f"brute force E={E} k={k}: {rel_err(out, ref)}"


def pin_dense_single_expert(o, seed=7):
    """E = 1, k = 1: the layer is the dense SwiGLU FFN."""
    p = small_problem(S=33, D=64, F=80, E=1, k=1, seed=seed)
    ids, w, _ = o.route(p["x"], p["wg"], 1)
    assert np.all(ids == 0) and np.all(w == 1.0)
    out = o.ffn(p["x"], p["w1"], p["w3"], p["w2"], ids, w)
    ref = dense_swiglu(bits_to_f64(p["x"]), bits_to_f64(p["w1"][0]), bits_to_f64(p["w3"][0]),
                       bits_to_f64(p["w2"][0]))
    assert rel_err(out, ref) < 1e-12


def pin_shared_experts(o, seed=8):
    """Experts sharing their weights give the dense FFN for any routing (gates sum to one)."""
    p = small_problem(S=36, D=48, F=64, E=8, k=3, seed=seed, shared_experts=True)
    dense = dense_swiglu(bits_to_f64(p["x"]), bits_to_f64(p["w1"][0]), bits_to_f64(p["w3"][0]),
                         bits_to_f64(p["w2"][0]))
    ids, w, _ = o.route(p["x"], p["wg"], 3)
    assert rel_err(o.ffn(p["x"], p["w1"], p["w3"], p["w2"], ids, w), dense) < 1e-12
    zid = wl.gen_random_ids(36, 3, 8, seed=seed, skew=1.2)
    zw = np.random.default_rng(seed).dirichlet(np.ones(3), size=36)
    assert rel_err(o.ffn(p["x"], p["w1"], p["w3"], p["w2"], zid, zw), dense) < 1e-12


def pin_invariances(o, seed=9):
    """Exact invariances: token permutation, expert relabelling, x2 scaling of W2 and of the gates."""
    p = small_problem(S=32, D=64, F=64, E=8, k=2, seed=seed)
    ids, w, _ = o.route(p["x"], p["wg"], 2)
    base = o.ffn(p["x"], p["w1"], p["w3"], p["w2"], ids, w)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(32)
    out = o.ffn(p["x"][perm], p["w1"], p["w3"], p["w2"], ids[perm], w[perm])
    assert np.array_equal(out, base[perm]), "token permutation"
    sigma = rng.permutation(8)  # new expert sigma[e] holds old expert e
    inv = np.argsort(sigma)
    out = o.ffn(p["x"], p["w1"][inv], p["w3"][inv], p["w2"][inv], sigma[ids].astype(np.int32), w)
    assert np.array_equal(out, base), "expert relabelling"
    w2x2 = bf16_bits_from_f32(bits_to_f64(p["w2"]).astype(np.float32) * 2.0)
    assert np.array_equal(o.ffn(p["x"], p["w1"], p["w3"], w2x2, ids, w), 2.0 * base), "linear in W2"
    assert np.array_equal(o.ffn(p["x"], p["w1"], p["w3"], p["w2"], ids, 2.0 * w), 2.0 * base), "linear in g"
    tok = np.array([5, 0, 31, 5], dtype=np.int64)
    assert np.array_equal(o.ffn(p["x"], p["w1"], p["w3"], p["w2"], ids, w, tokens=tok), base[tok]), "token subset"


# ------------------------------------------------------- parallel linear --

PL_MODES = [(False, False), (False, True), (True, False), (True, True)]  # (grouped_in, grouped_out)


def pl_problem(S=40, k=2, D_in=48, D_out=40, E=8, seed=0, grouped_in=False, grouped_out=False, skew=None):
    """Random ParallelLinear problem (bf16 bit arrays); x / dy hold S*k slot rows when grouped."""
    rng = np.random.default_rng(seed)
    ids = wl.gen_random_ids(S, k, E, seed=seed + 11, skew=skew)
    x = bf16_bits_from_f32(rng.standard_normal(((S * k if grouped_in else S), D_in)))
    w = bf16_bits_from_f32(rng.standard_normal((E, D_in, D_out)) * D_in ** -0.5)
    g = rng.dirichlet(np.ones(k), size=S)
    dy = bf16_bits_from_f32(rng.standard_normal(((S * k if grouped_out else S), D_out)))
    return dict(x=x, w=w, ids=ids, g=g, dy=dy)


def dense_gate_matrix(ids, g, E):
    G = np.zeros((ids.shape[0], E))
    for j in range(ids.shape[1]):
        G[np.arange(ids.shape[0]), ids[:, j]] += g[:, j]
    return G


def library_slots(ids):
    """(slot_src, sparse_rows) from numpy's stable argsort of the flat expert ids."""
    src = np.argsort(ids.reshape(-1), kind="stable")
    rows = np.empty_like(src)
    rows[src] = np.arange(src.size)
    return src, rows


def pin_parallel_linear_dense_mask(o, seed=20):
    """Scattered in and out: y = sum_e G[:, e] * (X W_e), every expert on every token masked by the
    dense gate matrix (gates given, and gates absent = indicator matrix)."""
    for (S, k, E) in [(40, 2, 8), (24, 4, 4), (30, 1, 16)]:
        p = pl_problem(S=S, k=k, E=E, seed=seed + E)
        X, W = bits_to_f64(p["x"]), bits_to_f64(p["w"])
        for gates in (p["g"], None):
            y = o.parallel_linear(p["x"], p["w"], p["ids"], gates)
            G = dense_gate_matrix(p["ids"], p["g"] if gates is not None else np.ones_like(p["g"]), E)
            ref = sum(G[:, e:e + 1] * (X @ W[e]) for e in range(E))
            assert rel_err(y, ref) < 1e-12, f"dense mask S={S} k={k} E={E}"


def pin_parallel_linear_modes(o, seed=21):
    """Grouped layouts are slot-order permutations (library argsort) of the scattered ones: grouped
    output rows taken back to route order and summed over j give the scattered output; grouped
    input rows gathered by slot give the scattered-input result bit for bit."""
    p = pl_problem(S=36, k=3, E=8, seed=seed, skew=1.2)
    src, rows = library_slots(p["ids"])
    S, k = p["ids"].shape
    ys = o.parallel_linear(p["x"], p["w"], p["ids"], p["g"])
    yg = o.parallel_linear(p["x"], p["w"], p["ids"], p["g"], grouped_out=True)
    assert rel_err(yg[rows].reshape(S, k, -1).sum(1), ys) < 1e-13, "grouped output = permuted routes"
    xg = p["x"][src // k]  # slot r holds its token's row
    assert np.array_equal(o.parallel_linear(xg, p["w"], p["ids"], p["g"], grouped_in=True), ys), "grouped input"
    assert np.array_equal(o.parallel_linear(xg, p["w"], p["ids"], p["g"], grouped_in=True, grouped_out=True), yg)


def pin_parallel_linear_single_expert(o, seed=22):
    """E = 1, k = 1, no gates: every mode is the plain product X W (numpy matmul)."""
    for gi, go in PL_MODES:
        p = pl_problem(S=33, k=1, D_in=40, D_out=56, E=1, seed=seed, grouped_in=gi, grouped_out=go)
        y = o.parallel_linear(p["x"], p["w"], p["ids"], None, gi, go)
        assert rel_err(y, bits_to_f64(p["x"]) @ bits_to_f64(p["w"][0])) < 1e-13


def pin_parallel_linear_bwd_adjoint(o, seed=23):
    """y is linear in x, in W and in g, so with s = <dy, y>: <dx, x> = s, sum_e <dw_e, W_e> = s and
    sum_f g_f dg_f = s (the adjoint identities), in every grouping mode, skewed routing included."""
    for gi, go in PL_MODES:
        for skew in (None, 1.2):
            p = pl_problem(S=30, k=2, E=8, seed=seed + 2 * gi + go, grouped_in=gi, grouped_out=go, skew=skew)
            y = o.parallel_linear(p["x"], p["w"], p["ids"], p["g"], gi, go)
            dx, dw, dg = o.parallel_linear_bwd(p["x"], p["w"], p["ids"], p["dy"], p["g"], gi, go)
            s = float(np.sum(bits_to_f64(p["dy"]) * y))
            tol = 1e-10 * float(np.sum(np.abs(bits_to_f64(p["dy"]) * y)))
            assert abs(float(np.sum(dx * bits_to_f64(p["x"]))) - s) < tol, f"<dx, x> mode {gi}{go}"
            assert abs(float(np.sum(dw * bits_to_f64(p["w"]))) - s) < tol, f"<dw, W> mode {gi}{go}"
            assert abs(float(np.sum(dg * p["g"])) - s) < tol, f"<dg, g> mode {gi}{go}"


def pin_parallel_linear_bwd_dense(o, seed=24):
    """Scattered in and out: dx = sum_e G[:, e] * (dY W_e^T), dw_e = (G[:, e] * X)^T dY and
    dg[t, j] = <dY[t], X[t] W_{ids[t, j]}> by dense numpy products; E = 1, k = 1 reduces to
    dx = dY W^T, dw = X^T dY in every mode; an expert with no routes gets dw = 0."""
    p = pl_problem(S=40, k=2, E=8, seed=seed)
    X, W, dY = bits_to_f64(p["x"]), bits_to_f64(p["w"]), bits_to_f64(p["dy"])
    ids = p["ids"].copy()
    ids[ids == 5] = 6  # expert 5 gets no routes (ids stay distinct per token unless 5 and 6 met)
    ids[:, 1] = np.where(ids[:, 1] == ids[:, 0], (ids[:, 0] + 1) % 5, ids[:, 1])
    assert np.all(ids[:, 0] != ids[:, 1]) and not np.any(ids == 5)
    dx, dw, dg = o.parallel_linear_bwd(p["x"], p["w"], ids, p["dy"], p["g"])
    G = dense_gate_matrix(ids, p["g"], 8)
    assert rel_err(dx, sum(G[:, e:e + 1] * (dY @ W[e].T) for e in range(8))) < 1e-12, "dense dx"
    for e in range(8):
        ref = (G[:, e:e + 1] * X).T @ dY
        assert (np.all(dw[e] == 0) if e == 5 else rel_err(dw[e], ref) < 1e-12), f"dense dw[{e}]"
    P = np.stack([X @ W[e] for e in range(8)])  # every expert on every token [E, S, D_out]
    ref_dg = np.stack([np.sum(dY * P[ids[:, j], np.arange(40)], axis=1) for j in range(2)], axis=1)
    assert rel_err(dg, ref_dg) < 1e-12, "dense dg"
    for gi, go in PL_MODES:
        q = pl_problem(S=27, k=1, D_in=40, D_out=32, E=1, seed=seed + 1, grouped_in=gi, grouped_out=go)
        dx1, dw1, _ = o.parallel_linear_bwd(q["x"], q["w"], q["ids"], q["dy"], None, gi, go)
        assert rel_err(dx1, bits_to_f64(q["dy"]) @ bits_to_f64(q["w"][0]).T) < 1e-13, f"E=1 dx {gi}{go}"
        assert rel_err(dw1[0], bits_to_f64(q["x"]).T @ bits_to_f64(q["dy"])) < 1e-13, f"E=1 dw {gi}{go}"


# ----------------------------------------------------------------- ffn bwd --

def numpy_moe_forward(x, w1, w3, w2, ids, g):
    """Dense fp64 numpy forward of the routed SwiGLU layer at real-valued inputs:
    out = sum_e G[:, e] * (SiLU(x W1_e) * (x W3_e)) W2_e with the dense gate matrix G."""
    S, k = ids.shape
    E = w1.shape[0]
    G = np.zeros((S, E))
    for j in range(k):
        G[np.arange(S), ids[:, j]] += g[:, j]
    return sum(G[:, e:e + 1] * dense_swiglu(x, w1[e], w3[e], w2[e]) for e in range(E))


def pin_ffn_bwd_finite_differences(o, seed=30):
    """Every gradient of the backward equals the derivative of the dense numpy forward: along random
    directions V, <grad, V> = (L(p + eps V) - L(p - eps V)) / (2 eps) with L = <dout, out>, for x, W1,
    W3, W2 and the gates; includes an expert with no routes (zero weight gradient)."""
    rng = np.random.default_rng(seed)
    S, D, F, E, k = 7, 16, 24, 5, 2
    x = bf16_bits_from_f32(rng.standard_normal((S, D)))
    w1 = bf16_bits_from_f32(rng.standard_normal((E, D, F)) * D ** -0.5)
    w3 = bf16_bits_from_f32(rng.standard_normal((E, D, F)) * D ** -0.5)
    w2 = bf16_bits_from_f32(rng.standard_normal((E, F, D)) * F ** -0.5)
    ids = np.stack([rng.choice(4, size=2, replace=False) for _ in range(S)]).astype(np.int32)  # expert 4 unused
    g = rng.dirichlet(np.ones(k), size=S)
    dout = bf16_bits_from_f32(rng.standard_normal((S, D)))
    grads = o.ffn_bwd(x, w1, w3, w2, ids, g, dout)
    P = dict(x=bits_to_f64(x), w1=bits_to_f64(w1), w3=bits_to_f64(w3), w2=bits_to_f64(w2), g=g)
    G = bits_to_f64(dout)
    L = lambda q: float(np.sum(G * numpy_moe_forward(q["x"], q["w1"], q["w3"], q["w2"], ids, q["g"])))
    for name, gname in [("x", "dx"), ("w1", "dw1"), ("w3", "dw3"), ("w2", "dw2"), ("g", "dg")]:
        for _ in range(2):
            V = rng.standard_normal(P[name].shape)
            eps = 1e-5
            qp = dict(P); qp[name] = P[name] + eps * V
            qm = dict(P); qm[name] = P[name] - eps * V
            fd = (L(qp) - L(qm)) / (2 * eps)
            an = float(np.sum(grads[gname] * V))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), f"{gname}: analytic {an} vs finite difference {fd}"
    assert np.all(grads["dw1"][4] == 0) and np.all(grads["dw3"][4] == 0) and np.all(grads["dw2"][4] == 0)


def pin_ffn_bwd_linear_in_dout(o, seed=31):
    """The backward is linear in dout: doubling dout (exact in bf16) doubles every gradient exactly;
    token permutation permutes dx and dg and leaves the weight gradients unchanged up to the order of
    their sums."""
    p = small_problem(S=12, D=32, F=40, E=4, k=2, seed=seed)
    ids, w, _ = o.route(p["x"], p["wg"], 2)
    rng = np.random.default_rng(seed)
    d1 = bf16_bits_from_f32(rng.standard_normal((12, 32)))
    d2 = bf16_bits_from_f32(bits_to_f64(d1).astype(np.float32) * 2.0)
    a = o.ffn_bwd(p["x"], p["w1"], p["w3"], p["w2"], ids, w, d1)
    b = o.ffn_bwd(p["x"], p["w1"], p["w3"], p["w2"], ids, w, d2)
    for n in a:
        assert np.array_equal(2.0 * a[n], b[n]), n
    perm = rng.permutation(12)
    c = o.ffn_bwd(p["x"][perm], p["w1"], p["w3"], p["w2"], ids[perm], w[perm], d1[perm])
    assert np.array_equal(c["dx"], a["dx"][perm]) and np.array_equal(c["dg"], a["dg"][perm])
    for n in ("dw1", "dw3", "dw2"):
        assert rel_err(c[n], a[n]) < 1e-13, n


ALL_PINS = [pin_router_library, pin_router_full_softmax, pin_router_ties, pin_router_given_ids,
            pin_sparse_map, pin_brute_force, pin_dense_single_expert, pin_shared_experts, pin_invariances,
            pin_parallel_linear_dense_mask, pin_parallel_linear_modes, pin_parallel_linear_single_expert,
            pin_parallel_linear_bwd_adjoint, pin_parallel_linear_bwd_dense, pin_ffn_bwd_finite_differences,
            pin_ffn_bwd_linear_in_dout]
