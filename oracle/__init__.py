"""ctypes binding of the fp64 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It never touches the HIP library and the HIP library never
touches it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")

F32, BF16 = 0, 1


def build(source: str = SOURCE, out: str = LIB_PATH, verbose: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math: IEEE double and float)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-ffp-contract=off", "-I", HERE, source, "-lm", "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _p(a):
    return None if a is None else a.ctypes.data


class Oracle:
    """Thin numpy-facing wrapper over liboracle.so (or a rebuilt variant of it)."""

    def __init__(self, lib_path: str = LIB_PATH):
        if not os.path.exists(lib_path):
            build(out=lib_path)
        lib = ctypes.CDLL(lib_path)
        i64, vp, i32, f32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.oracle_router_logits.argtypes = [i64, i64, i64, i32, vp, vp, vp]
        lib.oracle_route.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
        lib.oracle_dispatch.argtypes = [i64, i64, i64, i64, vp, vp, vp, vp, vp, vp]
        lib.oracle_expert.argtypes = [i64, i64, i32, vp, vp, vp, vp, vp]
        lib.oracle_layer_output.argtypes = [i64, i64, i64, i64, i64, i32, vp, vp, vp, vp,
                                            vp, vp, vp, i64, vp, vp]
        lib.oracle_aux_loss.argtypes = [i64, i64, i64, vp, vp]
        lib.oracle_aux_loss.restype = ctypes.c_double
        lib.oracle_bias_update.argtypes = [i64, i64, i64, vp, f32, vp]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_z_loss.argtypes = [i64, i64, vp]
        lib.oracle_z_loss.restype = ctypes.c_double
        lib.oracle_aux_topk.argtypes = [i64, i64, i64, vp, vp, vp]
        lib.oracle_aux_topk.restype = ctypes.c_double
        lib.oracle_combine_concat.argtypes = [i64, i64, i64, i64, i32, vp, vp, vp, vp]
        for name in ("oracle_router_logits", "oracle_route", "oracle_dispatch",
                     "oracle_expert", "oracle_layer_output", "oracle_bias_update"):
            getattr(lib, name).restype = None
        self.lib = lib

    @staticmethod
    def _dtype_code(a: np.ndarray) -> int:
        if a.dtype == np.float32:
            return F32
        if a.dtype == np.uint16:
            return BF16
        raise TypeError(f"oracle inputs are float32 or bf16 bits (uint16), got {a.dtype}")

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def router_logits(self, x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x)
        w_router = np.ascontiguousarray(w_router)
        T, d = x.shape
        d2, E = w_router.shape
        assert d == d2 and x.dtype == w_router.dtype
        out = np.empty((T, E), np.float64)
        self.lib.oracle_router_logits(T, d, E, self._dtype_code(x), _p(x), _p(w_router), _p(out))
        return out

    def route(self, logits: np.ndarray, K: int, bias: np.ndarray | None = None,
              want_probs: bool = True, select_only: bool = False, mean: bool = False):
        """Routing of fp32 scores (see oracle.h).  Two variants:
        select_only: the bias decides which K experts are chosen, and the
            weights and probabilities come from the softmax of the unbiased
            scores (the other reading of the engineering page's §1.2, where
            the balancing bias only steers the selection);
        mean: the K outputs are averaged without weights (MoE notes §2.3,
            third combine form), i.e. every weight is 1/K."""
        logits = np.ascontiguousarray(logits, np.float32)
        T, E = logits.shape
        if not (1 <= K <= E):
            raise ValueError("need 1 <= K <= E")
        b = None if bias is None else np.ascontiguousarray(bias, np.float32)
        ids = np.empty((T, K), np.int32)
        w = np.empty((T, K), np.float64)
        probs = np.empty((T, E), np.float64) if (want_probs or select_only) else None
        self.lib.oracle_route(T, E, K, _p(logits), _p(b), _p(ids), _p(w), _p(probs))
        if select_only:
            _, _, probs = self.route(logits, K, None)
            chosen = np.take_along_axis(probs, ids.astype(np.int64), axis=1)
            w = chosen / chosen.sum(axis=1, keepdims=True)
        if mean:
            w = np.full((T, K), 1.0 / K)
        return ids, w, probs

    def dispatch(self, ids: np.ndarray, E: int, capacity: int = -1) -> dict:
        ids = np.ascontiguousarray(ids, np.int32)
        T, K = ids.shape
        counts = np.empty(E, np.int32)
        kept = np.empty(E, np.int32)
        offsets = np.empty(E + 1, np.int32)
        assign_row = np.empty(T * K, np.int32)
        row_assign = np.empty(T * K, np.int32)
        self.lib.oracle_dispatch(T, E, K, capacity, _p(ids), _p(counts), _p(kept), _p(offsets),
                                 _p(assign_row), _p(row_assign))
        return {"counts": counts, "kept": kept, "offsets": offsets,
                "assign_row": assign_row, "row_assign": row_assign}

    def expert(self, x_row: np.ndarray, w1e: np.ndarray, w3e: np.ndarray,
               w2e: np.ndarray) -> np.ndarray:
        x_row = np.ascontiguousarray(x_row)
        F, d = w1e.shape
        h = np.empty(d, np.float64)
        self.lib.oracle_expert(d, F, self._dtype_code(x_row), _p(x_row),
                               _p(np.ascontiguousarray(w1e)), _p(np.ascontiguousarray(w3e)),
                               _p(np.ascontiguousarray(w2e)), _p(h))
        return h

    def layer_output(self, x, w1, w3, w2, ids, w, assign_row=None, tokens=None) -> np.ndarray:
        x = np.ascontiguousarray(x)
        T, d = x.shape
        E, F, _ = w1.shape
        K = ids.shape[1]
        ids = np.ascontiguousarray(ids, np.int32)
        w = np.ascontiguousarray(w, np.float64)
        ar = None if assign_row is None else np.ascontiguousarray(assign_row, np.int32)
        toks = np.arange(T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
        y = np.empty((len(toks), d), np.float64)
        for a in (w1, w3, w2):
            assert a.flags.c_contiguous and a.dtype == x.dtype
        self.lib.oracle_layer_output(T, d, E, K, F, self._dtype_code(x), _p(x), _p(w1), _p(w3),
                                     _p(w2), _p(ids), _p(w), _p(ar), len(toks), _p(toks), _p(y))
        return y

    def aux_loss(self, counts: np.ndarray, probs: np.ndarray, K: int) -> float:
        counts = np.ascontiguousarray(counts, np.int32)
        probs = np.ascontiguousarray(probs, np.float64)
        T, E = probs.shape
        return float(self.lib.oracle_aux_loss(T, E, K, _p(counts), _p(probs)))

    def z_loss(self, logits: np.ndarray) -> float:
        logits = np.ascontiguousarray(logits, np.float32)
        T, E = logits.shape
        return float(self.lib.oracle_z_loss(T, E, _p(logits)))

    def aux_topk(self, counts: np.ndarray, ids: np.ndarray, probs: np.ndarray) -> float:
        counts = np.ascontiguousarray(counts, np.int32)
        ids = np.ascontiguousarray(ids, np.int32)
        probs = np.ascontiguousarray(probs, np.float64)
        T, E = probs.shape
        return float(self.lib.oracle_aux_topk(T, E, ids.shape[1], _p(counts), _p(ids), _p(probs)))

    def combine_concat(self, h: np.ndarray, assign_row: np.ndarray, w_cat: np.ndarray, dtype: str = "f32") -> np.ndarray:
        """y [T, d_out] (float64) = w_cat . concat over slots of h[assign_row[t, k]];
        h [S, d] and w_cat [d_out, K*d] as float32 arrays, or uint16 bf16 bits
        with dtype="bf16"; assign_row [T, K] int32 (-1 = dropped)."""
        assign_row = np.ascontiguousarray(assign_row, np.int32)
        T, K = assign_row.shape
        dt = BF16 if dtype == "bf16" else F32
        h = np.ascontiguousarray(h, np.uint16 if dt == BF16 else np.float32)
        w_cat = np.ascontiguousarray(w_cat, np.uint16 if dt == BF16 else np.float32)
        d = h.shape[1]
        d_out = w_cat.shape[0]
        assert w_cat.shape[1] == K * d
        y = np.zeros((T, d_out), np.float64)
        self.lib.oracle_combine_concat(T, K, d, d_out, dt, _p(h), _p(assign_row), _p(w_cat), _p(y))
        return y

    def bias_update(self, counts: np.ndarray, T: int, K: int, alpha: float,
                    bias: np.ndarray) -> np.ndarray:
        counts = np.ascontiguousarray(counts, np.int32)
        out = np.array(bias, np.float32, copy=True)
        self.lib.oracle_bias_update(T, len(counts), K, _p(counts), ctypes.c_float(alpha), _p(out))
        return out

    # Standalone forward (used for the CPU baseline): fp32 logits from the
    # oracle's own fp64 router, then routing, grouping and the layer output.
    def forward(self, x, w_router, w1, w3, w2, K, bias=None, capacity=-1, tokens=None):
        logits = self.router_logits(x, w_router).astype(np.float32)
        ids, w, probs = self.route(logits, K, bias)
        disp = self.dispatch(ids, w_router.shape[1], capacity)
        y = self.layer_output(x, w1, w3, w2, ids, w, disp["assign_row"], tokens)
        return {"logits": logits, "ids": ids, "w": w, "probs": probs, "y": y, **disp}


_default = None


def get() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
