"""Seeded synthetic inputs shared by the CPU oracle and the GPU library.

Everything here is input generation only: random weights, hidden states,
router logits and routing traces. None of the MoE layer's arithmetic
(quantisation, routing, packing, FFN) lives in this module.

The generator is SplitMix64 used counter-style (see ``synth.c``), with
Box-Muller normals; every array is a pure function of (seed, stream, index),
so the same call always returns the same bytes, in any process.

Stream ids name what an array is for, so two arrays never share a stream:
``stream_id(kind, layer, expert, matrix)``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lock = threading.Lock()
_lib = None

# stream kinds
K_EXPERT_W = 1      # expert weight matrices (matrix 0 gate, 1 up, 2 down)
K_ROUTER_W = 2      # router weight [E][H]
K_ROUTER_BIAS = 3   # router selection bias [E]
K_HIDDEN = 4        # hidden states x [T][H]
K_ZIPF_RANK = 5     # popularity rank permutation of the experts
K_ZIPF_GUMBEL = 6   # Gumbel noise of Zipf logits
K_SHARED_W = 7      # shared expert matrices
K_TRACE = 8         # correlated routing traces
K_MISC = 9


def stream_id(kind: int, layer: int = 0, expert: int = 0, matrix: int = 0) -> int:
    return (kind << 56) | (layer << 32) | (expert << 8) | matrix


def build(force: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(src):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_SO):
                build()
            lib = ctypes.CDLL(_SO)
            u64, i64, i32, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32, ctypes.c_double
            vp = ctypes.c_void_p
            lib.synth_stream_key.restype = u64
            lib.synth_stream_key.argtypes = [u64, u64]
            lib.synth_u64_at.restype = u64
            lib.synth_u64_at.argtypes = [u64, u64, u64]
            lib.synth_normal_f32.argtypes = [u64, u64, i64, dbl, dbl, vp]
            lib.synth_uniform_f64.argtypes = [u64, u64, i64, vp]
            lib.synth_gumbel_f64.argtypes = [u64, u64, i64, vp]
            lib.synth_permutation.argtypes = [u64, u64, i32, vp]
            lib.synth_zipf_logits.argtypes = [u64, u64, i32, i32, dbl, vp, vp]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def normal(seed: int, stream: int, shape, std: float = 1.0, mean: float = 0.0, out: np.ndarray | None = None):
    """float32 array of N(mean, std^2) values."""
    n = int(np.prod(shape))
    if out is None:
        out = np.empty(shape, dtype=np.float32)
    assert out.dtype == np.float32 and out.size == n
    _load().synth_normal_f32(seed, stream, n, float(mean), float(std), _ptr(out))
    return out


def uniform(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_uniform_f64(seed, stream, n, _ptr(out))
    return out


def gumbel(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_gumbel_f64(seed, stream, n, _ptr(out))
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_permutation(seed, stream, n, _ptr(out))
    return out


def u64_at(seed: int, stream: int, n: int) -> int:
    return int(_load().synth_u64_at(seed, stream, n))


# ----------------------------------------------------------------------------
# Workload-level helpers (shapes and distributions of the layer's inputs)
# ----------------------------------------------------------------------------

def expert_weights(seed: int, layer: int, expert: int, H: int, I: int, std: float = 0.02, shared: bool = False):
    """fp32 (gate [I][H], up [I][H], down [H][I]) of one expert, N(0, std^2)."""
    kind = K_SHARED_W if shared else K_EXPERT_W
    g = normal(seed, stream_id(kind, layer, expert, 0), (I, H), std)
    u = normal(seed, stream_id(kind, layer, expert, 1), (I, H), std)
    d = normal(seed, stream_id(kind, layer, expert, 2), (H, I), std)
    return g, u, d


def router_weights(seed: int, layer: int, E: int, H: int, std: float = 0.02) -> np.ndarray:
    return normal(seed, stream_id(K_ROUTER_W, layer), (E, H), std)


def router_bias(seed: int, layer: int, E: int, std: float = 0.1) -> np.ndarray:
    return normal(seed, stream_id(K_ROUTER_BIAS, layer), (E,), std)


def hidden(seed: int, T: int, H: int, batch: int = 0) -> np.ndarray:
    return normal(seed, stream_id(K_HIDDEN, 0, batch), (T, H), 1.0)


def zipf_rank(seed: int, layer: int, E: int) -> np.ndarray:
    """rank_of[e] in 1..E: popularity rank of expert e (1 = most popular)."""
    perm = permutation(seed, stream_id(K_ZIPF_RANK, layer), E)
    rank_of = np.empty(E, dtype=np.int32)
    rank_of[perm] = np.arange(1, E + 1, dtype=np.int32)
    return rank_of


def zipf_logits(seed: int, layer: int, T: int, E: int, s: float = 1.1, batch: int = 0) -> np.ndarray:
    """fp32 logits [T][E] whose top-k follows Zipf(s) expert popularity."""
    rank_of = zipf_rank(seed, layer, E)
    z = np.empty((T, E), dtype=np.float32)
    _load().synth_zipf_logits(seed, stream_id(K_ZIPF_GUMBEL, layer, batch), T, E, float(s), _ptr(rank_of), _ptr(z))
    return z
