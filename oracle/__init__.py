"""ctypes wrapper of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use it; the product path never does. It does not import
the HIP package and shares no code with it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c99", "-Wall"]


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (no FMA contraction, IEEE semantics)."""
    cmd = ["gcc", *CFLAGS, src, "-o", out, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


_P = ctypes.c_void_p
_I64 = ctypes.c_int64


class Oracle:
    def __init__(self, path: str = LIB):
        if not os.path.exists(path) and path == LIB:
            build(out=path)
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.oracle_route.argtypes = [_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P]
        L.oracle_route.restype = ctypes.c_int
        L.oracle_sparse_map.argtypes = [_P, _I64, _I64, _I64, _P, _P, _P, _P]
        L.oracle_sparse_map.restype = ctypes.c_int
        L.oracle_ffn_tokens.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _I64, _P,
                                        ctypes.c_int]
        L.oracle_ffn_tokens.restype = ctypes.c_int
        L.oracle_parallel_linear.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, ctypes.c_int,
                                             ctypes.c_int, _P]
        L.oracle_parallel_linear.restype = ctypes.c_int
        L.oracle_parallel_linear_bwd.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, ctypes.c_int,
                                                 ctypes.c_int, _P, _P, _P]
        L.oracle_parallel_linear_bwd.restype = ctypes.c_int
        L.oracle_ffn_bwd.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]
        L.oracle_ffn_bwd.restype = ctypes.c_int

    @staticmethod
    def _ptr(a: Optional[np.ndarray]):
        return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

    def route(self, x_bits: np.ndarray, wg_bits: np.ndarray, k: int, ids_in: Optional[np.ndarray] = None):
        """H(X) = Softmax(TopK(X W_gate, k)) -> (ids int32 [S,k], weights f64 [S,k], logits f64 [S,E])."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        wg_bits = np.ascontiguousarray(wg_bits, dtype=np.uint16)
        S, D = x_bits.shape
        D2, E = wg_bits.shape
        assert D == D2
        ids = np.zeros((S, k), dtype=np.int32)
        w = np.zeros((S, k), dtype=np.float64)
        logits = np.zeros((S, E), dtype=np.float64)
        if ids_in is not None:
            ids_in = np.ascontiguousarray(ids_in, dtype=np.int32)
            assert ids_in.shape == (S, k)
        st = self.lib.oracle_route(self._ptr(x_bits), self._ptr(wg_bits), S, D, E, k, self._ptr(ids_in),
                                   self._ptr(ids), self._ptr(w), self._ptr(logits))
        if st:
            raise ValueError(f"oracle_route status {st}")
        return ids, w, logits

    def sparse_map(self, ids: np.ndarray, E: int):
        """Stable counting-sort map -> (counts [E], offsets [E+1], sparse_rows [S*k], slot_src [S*k])."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        n = ids.size
        S, k = (ids.shape if ids.ndim == 2 else (n, 1))
        counts = np.zeros(E, dtype=np.int32)
        offsets = np.zeros(E + 1, dtype=np.int32)
        rows = np.zeros(n, dtype=np.int32)
        src = np.zeros(n, dtype=np.int32)
        st = self.lib.oracle_sparse_map(self._ptr(ids), S, k, E, self._ptr(counts), self._ptr(offsets),
                                        self._ptr(rows), self._ptr(src))
        if st:
            raise ValueError(f"oracle_sparse_map status {st}")
        return counts, offsets, rows, src

    def ffn(self, x_bits, w1_bits, w3_bits, w2_bits, ids, weights, tokens=None, nthreads: Optional[int] = None):
        """out[i] = sum_j weights[s,j] * SwiGLU_{ids[s,j]}(x[s]) for s = tokens[i] -> f64 [ntok, D]."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        S, D = x_bits.shape
        E, D2, F = w1_bits.shape
        assert D2 == D and w3_bits.shape == (E, D, F) and w2_bits.shape == (E, F, D)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        k = ids.shape[1]
        weights = np.ascontiguousarray(weights, dtype=np.float64)
        assert ids.shape == (S, k) and weights.shape == (S, k)
        tokens = np.arange(S, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int64)
        out = np.zeros((tokens.size, D), dtype=np.float64)
        nthreads = nthreads or min(16, os.cpu_count() or 1)
        st = self.lib.oracle_ffn_tokens(self._ptr(x_bits), self._ptr(w1_bits), self._ptr(w3_bits),
                                        self._ptr(w2_bits), self._ptr(ids), self._ptr(weights), D, F, E, k,
                                        self._ptr(tokens), tokens.size, self._ptr(out), int(nthreads))
        if st:
            raise ValueError(f"oracle_ffn_tokens status {st}")
        return out

    @staticmethod
    def _pl_args(x_bits, w_bits, ids, gates, grouped_in):
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        S, k = ids.shape
        E, D_in, D_out = w_bits.shape
        assert x_bits.shape == ((S * k if grouped_in else S), D_in)
        if gates is not None:
            gates = np.ascontiguousarray(gates, dtype=np.float64).reshape(S * k)
        return x_bits, w_bits, ids, gates, S, k, E, D_in, D_out

    def parallel_linear(self, x_bits, w_bits, ids, gates=None, grouped_in=False, grouped_out=False):
        """ParallelLinear(X, W, I, G) -> f64 [S*k or S, D_out] (grouped rows are in slot order)."""
        x_bits, w_bits, ids, gates, S, k, E, D_in, D_out = self._pl_args(x_bits, w_bits, ids, gates, grouped_in)
        y = np.zeros(((S * k if grouped_out else S), D_out), dtype=np.float64)
        st = self.lib.oracle_parallel_linear(self._ptr(x_bits), self._ptr(w_bits), self._ptr(gates), self._ptr(ids),
                                             S, k, D_in, D_out, E, int(grouped_in), int(grouped_out), self._ptr(y))
        if st:
            raise ValueError(f"oracle_parallel_linear status {st}")
        return y

    def parallel_linear_bwd(self, x_bits, w_bits, ids, dy_bits, gates=None, grouped_in=False, grouped_out=False,
                            want=("dx", "dw", "dg")):
        """Backward of ParallelLinear -> (dx f64, dw f64 [E, D_in, D_out], dg f64 [S, k]); outputs not
        named in `want` are not computed and come back as None."""
        x_bits, w_bits, ids, gates, S, k, E, D_in, D_out = self._pl_args(x_bits, w_bits, ids, gates, grouped_in)
        dy_bits = np.ascontiguousarray(dy_bits, dtype=np.uint16)
        assert dy_bits.shape == ((S * k if grouped_out else S), D_out)
        dx = np.zeros(((S * k if grouped_in else S), D_in), dtype=np.float64) if "dx" in want else None
        dw = np.zeros((E, D_in, D_out), dtype=np.float64) if "dw" in want else None
        dg = np.zeros((S, k), dtype=np.float64) if "dg" in want else None
        st = self.lib.oracle_parallel_linear_bwd(self._ptr(x_bits), self._ptr(w_bits), self._ptr(gates),
                                                 self._ptr(ids), self._ptr(dy_bits), S, k, D_in, D_out, E,
                                                 int(grouped_in), int(grouped_out), self._ptr(dx), self._ptr(dw),
                                                 self._ptr(dg))
        if st:
            raise ValueError(f"oracle_parallel_linear_bwd status {st}")
        return dx, dw, dg

    def ffn_bwd(self, x_bits, w1_bits, w3_bits, w2_bits, ids, weights, dout_bits,
                want=("dx", "dw1", "dw3", "dw2", "dg")):
        """Backward of the SwiGLU expert FFN with weighted combine -> dict of f64 arrays
        dx [S, D], dw1 / dw3 [E, D, F], dw2 [E, F, D], dg [S, k] (only those in `want`)."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        S, D = x_bits.shape
        E, D2, F = w1_bits.shape
        assert D2 == D and w3_bits.shape == (E, D, F) and w2_bits.shape == (E, F, D)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        k = ids.shape[1]
        weights = np.ascontiguousarray(weights, dtype=np.float64)
        dout_bits = np.ascontiguousarray(dout_bits, dtype=np.uint16)
        assert ids.shape == (S, k) and weights.shape == (S, k) and dout_bits.shape == (S, D)
        shapes = dict(dx=(S, D), dw1=(E, D, F), dw3=(E, D, F), dw2=(E, F, D), dg=(S, k))
        out = {n: np.zeros(shapes[n], dtype=np.float64) for n in want}
        st = self.lib.oracle_ffn_bwd(self._ptr(x_bits), self._ptr(np.ascontiguousarray(w1_bits, dtype=np.uint16)),
                                     self._ptr(np.ascontiguousarray(w3_bits, dtype=np.uint16)),
                                     self._ptr(np.ascontiguousarray(w2_bits, dtype=np.uint16)), self._ptr(ids),
                                     self._ptr(weights), self._ptr(dout_bits), S, D, F, E, k,
                                     *(self._ptr(out.get(n)) for n in ("dx", "dw1", "dw3", "dw2", "dg")))
        if st:
            raise ValueError(f"oracle_ffn_bwd status {st}")
        return out

    def layer(self, x_bits, wg_bits, w1_bits, w3_bits, w2_bits, k, tokens=None, nthreads=None):
        """Route, map and FFN of the whole forward (map returned for inspection)."""
        E = wg_bits.shape[1]
        ids, w, logits = self.route(x_bits, wg_bits, k)
        smap = self.sparse_map(ids, E)
        out = self.ffn(x_bits, w1_bits, w3_bits, w2_bits, ids, w, tokens=tokens, nthreads=nthreads)
        return dict(ids=ids, weights=w, logits=logits, map=smap, out=out)


_default: Optional[Oracle] = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(LIB)
    return _default
