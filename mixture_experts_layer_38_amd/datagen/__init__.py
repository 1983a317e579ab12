"""Seeded synthetic inputs shared by the HIP path's callers and the CPU oracle.

The generator itself (gen.c) is a counter-based SplitMix64 + Box-Muller draw;
any element can be regenerated from (seed, tensor_id, index).  This module
holds no MoE arithmetic: it produces x, the router weight, the expert weights
and the per-expert logit offset of a workload, as numpy arrays (bf16 arrays are
returned as their uint16 bit patterns).

Recipe per tensor (tensor ids in brackets):
  x   [1]  [T, d]   ~ N(0, 1)
  W_r [2]  [d, E]   ~ N(0, 1/d)
  W1  [3]  [E, F, d] ~ N(0, 1/d)
  W3  [4]  [E, F, d] ~ N(0, 1/d)
  W2  [5]  [E, d, F] ~ N(0, 1/F)
  logit offset [6] [E]: zero, log of the normalised Zipf(s) rank law with rank
      e+1, or U(lo, hi) drawn from the generator.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

from ..configs import MoEConfig

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoegen.so")

TENSOR_X, TENSOR_WR, TENSOR_W1, TENSOR_W3, TENSOR_W2, TENSOR_BIAS = 1, 2, 3, 4, 5, 6

_lib = None


def build(verbose: bool = False) -> str:
    import subprocess
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           os.path.join(_HERE, "gen.c"), "-lm", "-o", LIB_PATH + ".tmp"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.gen_normal_f32.argtypes = [u64, u64, u64, i64, dbl, vp]
    lib.gen_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, vp]
    lib.gen_uniform_f32.argtypes = [u64, u64, u64, i64, dbl, dbl, vp]
    lib.gen_words.argtypes = [u64, u64, u64, i64, vp]
    lib.gen_splitmix64.argtypes = [u64, i64, vp]
    for f in (lib.gen_normal_f32, lib.gen_normal_bf16, lib.gen_uniform_f32, lib.gen_words,
              lib.gen_splitmix64):
        f.restype = None
    _lib = lib
    return lib


def normal(seed: int, tensor_id: int, shape, sigma: float, dtype: str,
           offset: int = 0, out: np.ndarray | None = None) -> np.ndarray:
    """N(0, sigma^2) draws; dtype "f32" -> float32, "bf16" -> uint16 bit patterns."""
    lib = _load()
    n = int(np.prod(shape))
    if dtype == "f32":
        a = out if out is not None else np.empty(shape, np.float32)
        lib.gen_normal_f32(seed, tensor_id, offset, n, float(sigma), a.ctypes.data)
    elif dtype == "bf16":
        a = out if out is not None else np.empty(shape, np.uint16)
        lib.gen_normal_bf16(seed, tensor_id, offset, n, float(sigma), a.ctypes.data)
    else:
        raise ValueError(dtype)
    return a


def uniform_f32(seed: int, tensor_id: int, n: int, lo: float, hi: float) -> np.ndarray:
    lib = _load()
    a = np.empty(n, np.float32)
    lib.gen_uniform_f32(seed, tensor_id, 0, n, float(lo), float(hi), a.ctypes.data)
    return a


def words(seed: int, tensor_id: int, n: int, offset: int = 0) -> np.ndarray:
    lib = _load()
    a = np.empty(n, np.uint64)
    lib.gen_words(seed, tensor_id, offset, n, a.ctypes.data)
    return a


def splitmix64(state: int, n: int) -> np.ndarray:
    lib = _load()
    a = np.empty(n, np.uint64)
    lib.gen_splitmix64(state, n, a.ctypes.data)
    return a


def logit_offset(cfg: MoEConfig) -> np.ndarray | None:
    """Per-expert additive logit offset of the workload (float32 [E]) or None."""
    if cfg.skew == "none":
        return None
    if cfg.skew == "zipf":
        r = np.arange(1, cfg.E + 1, dtype=np.float64)
        p = r ** (-cfg.zipf_s)
        return np.log(p / p.sum()).astype(np.float32)
    if cfg.skew == "uniform":
        return uniform_f32(cfg.seed, TENSOR_BIAS, cfg.E, cfg.bias_lo, cfg.bias_hi)
    raise ValueError(cfg.skew)


def make_inputs(cfg: MoEConfig, with_experts: bool = True) -> dict:
    """All inputs of one workload as host arrays (bf16 as uint16 bits)."""
    dt = cfg.dtype
    out = {
        "x": normal(cfg.seed, TENSOR_X, (cfg.T, cfg.d), 1.0, dt),
        "w_router": normal(cfg.seed, TENSOR_WR, (cfg.d, cfg.E), 1.0 / math.sqrt(cfg.d), dt),
        "logit_bias": logit_offset(cfg),
    }
    if with_experts:
        out["w1"] = normal(cfg.seed, TENSOR_W1, (cfg.E, cfg.F, cfg.d), 1.0 / math.sqrt(cfg.d), dt)
        out["w3"] = normal(cfg.seed, TENSOR_W3, (cfg.E, cfg.F, cfg.d), 1.0 / math.sqrt(cfg.d), dt)
        out["w2"] = normal(cfg.seed, TENSOR_W2, (cfg.E, cfg.d, cfg.F), 1.0 / math.sqrt(cfg.F), dt)
    return out


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (for printing / tests)."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits with round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)
