"""CPU oracle of the routed-expert MoE layer (numpy front end of moe_oracle.c).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
and its Python binding never import, link or call it, and share no code with
it.

Every function wraps one stage of the scalar C oracle; see ``moe_oracle.h``
for the definition each stage follows and the passage of the pages it cites.

Parity status (what pins each stage) is listed in the test files
``tests/test_oracle_*.py``; no stage is unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_ORACLE_LIB: another build of the same source (the sanitizer build)
_SO = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "libmoe_oracle.so")
SANITIZED_SO = os.path.join(_HERE, "libmoe_oracle_asan.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]
_SRC = os.path.join(_HERE, "moe_oracle.c")
_HDR = os.path.join(_HERE, "moe_oracle.h")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11"]
_lock = threading.Lock()
_lib = None


def build(force: bool = False, sanitize: bool = False) -> str:
    """Compile libmoe_oracle.so with gcc (no fast-math, no FP contraction);
    sanitize: the AddressSanitizer + UndefinedBehaviorSanitizer build
    (libmoe_oracle_asan.so, loaded through MOE_ORACLE_LIB with libasan
    preloaded)."""
    sanitize = sanitize or os.path.abspath(_SO) == SANITIZED_SO
    so = SANITIZED_SO if sanitize else _SO
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(so) or os.path.getmtime(so) < newest:
        tmp = so + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, *(SANITIZE_FLAGS if sanitize else []), _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, so)
    return so


class _Expert(ctypes.Structure):
    _fields_ = [
        ("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
        ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p),
    ]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_SO):
                build()
            lib = ctypes.CDLL(_SO)
            vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
            lib.orc_quantize_rows.argtypes = [i32, vp, i64, i32, vp, vp]
            lib.orc_unpack_rows.argtypes = [i32, vp, i64, i32, vp]
            lib.orc_quantize_act.argtypes = [vp, i32, i32, vp, vp]
            lib.orc_exp_f32.argtypes = [ctypes.c_float]
            lib.orc_exp_f32.restype = ctypes.c_float
            lib.orc_silu_f32.argtypes = [ctypes.c_float]
            lib.orc_silu_f32.restype = ctypes.c_float
            lib.orc_router.argtypes = [i32, vp, vp, vp, i32, i32, i32, i32, dbl, vp, vp, vp, vp]
            lib.orc_bucket.argtypes = [vp, i32, i32, i32, vp, vp, vp]
            lib.orc_expert_token.argtypes = [i32, ctypes.POINTER(_Expert), vp, ctypes.c_float, i32, i32,
                                             vp, vp, vp, vp, vp, vp, vp]
            lib.orc_combine.argtypes = [vp, vp, i32, i32, i32, i32, vp]
            lib.orc_layer.argtypes = [vp, vp, vp, vp, dbl, vp, vp, ctypes.POINTER(_Expert), i32,
                                      i32, i32, i32, i32, i32, dbl, vp, vp, vp, vp, vp, vp]
            lib.orc_topp.argtypes = [i32, i32, i32, vp, dbl, dbl, vp, vp, vp]
            lib.orc_swiglu_f64.argtypes = [vp, vp, vp, vp, i32, i32, vp]
            lib.orc_set_threads.argtypes = [i32]
            lib.orc_set_threads.restype = i32
            _lib = lib
    return _lib


def _p(a):
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous numpy"
    return a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


QMAX = {8: 127, 4: 7, 2: 1}


def row_bytes(bits: int, cols: int) -> int:
    return cols * bits // 8


# --- O1 / O2 -----------------------------------------------------------------

def quantize_rows(bits: int, w: np.ndarray):
    """fp32 [R][C] -> (packed uint8 [R][C*bits/8], scales fp32 [R])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    R, C = w.shape
    packed = np.empty((R, row_bytes(bits, C)), dtype=np.uint8)
    scales = np.empty(R, dtype=np.float32)
    _check(_load().orc_quantize_rows(bits, _p(w), R, C, _p(packed), _p(scales)), "quantize_rows")
    return packed, scales


def unpack_rows(bits: int, packed: np.ndarray, cols: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    R = packed.shape[0]
    q = np.empty((R, cols), dtype=np.int8)
    _check(_load().orc_unpack_rows(bits, _p(packed), R, cols, _p(q)), "unpack_rows")
    return q


def quantize_act(x: np.ndarray):
    """fp32 [T][H] -> (xq int8 [T][H], sx fp32 [T])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H = x.shape
    xq = np.empty((T, H), dtype=np.int8)
    sx = np.empty(T, dtype=np.float32)
    _check(_load().orc_quantize_act(_p(x), T, H, _p(xq), _p(sx)), "quantize_act")
    return xq, sx


def exp_f32(x: float) -> float:
    return float(_load().orc_exp_f32(ctypes.c_float(x)))


def silu_f32(x: float) -> float:
    return float(_load().orc_silu_f32(ctypes.c_float(x)))


# --- O3 ----------------------------------------------------------------------

def router(x: np.ndarray, wr: np.ndarray | None, bias: np.ndarray | None, k: int, logits_in: bool = False,
           routed_scale: float = 1.0, want_keys: bool = False):
    """Returns (idx int32 [T][k], w fp32 [T][k]) and, if want_keys, (keys, sig) fp64 [T][E]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T = x.shape[0]
    if logits_in:
        E, H = x.shape[1], 0
    else:
        wr = np.ascontiguousarray(wr, dtype=np.float32)
        E, H = wr.shape
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    keys = np.empty((T, E), dtype=np.float64) if want_keys else None
    sig = np.empty((T, E), dtype=np.float64) if want_keys else None
    _check(_load().orc_router(1 if logits_in else 0, _p(x), _p(wr) if not logits_in else None, _p(bias), T, H, E, k,
                              float(routed_scale), _p(idx), _p(w), _p(keys), _p(sig)), "router")
    if want_keys:
        return idx, w, keys, sig
    return idx, w


def topp(idx: np.ndarray, sig: np.ndarray, top_p: float, routed_scale: float = 1.0):
    """Top-p truncation of a top-k selection (orc_topp): returns (idx with -1
    for dropped slots, w, cumulative normalised weights fp64 [T][k])."""
    idx = np.array(idx, dtype=np.int32, order="C")
    sig = np.ascontiguousarray(sig, dtype=np.float64)
    T, k = idx.shape
    E = sig.shape[1]
    w = np.zeros((T, k), dtype=np.float32)
    cum = np.empty((T, k), dtype=np.float64)
    _check(_load().orc_topp(T, E, k, _p(sig), float(routed_scale), float(top_p), _p(idx), _p(w), _p(cum)), "topp")
    return idx, w, cum


# --- O4 ----------------------------------------------------------------------

def bucket(idx: np.ndarray, E: int):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    _check(_load().orc_bucket(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm)), "bucket")
    return counts, offsets, perm


# --- experts -----------------------------------------------------------------

@dataclass
class Expert:
    """One expert's packed weights (host numpy arrays)."""
    bits: int
    gate: np.ndarray   # uint8 [I][H*bits/8]
    up: np.ndarray     # uint8 [I][H*bits/8]
    down: np.ndarray   # uint8 [H][I*bits/8]
    s_gate: np.ndarray  # fp32 [I]
    s_up: np.ndarray    # fp32 [I]
    s_down: np.ndarray  # fp32 [H]

    @property
    def H(self):
        return self.down.shape[0]

    @property
    def I(self):
        return self.gate.shape[0]

    def struct(self) -> _Expert:
        return _Expert(_p(self.gate), _p(self.up), _p(self.down), _p(self.s_gate), _p(self.s_up), _p(self.s_down))


def pack_expert(bits: int, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> Expert:
    g, sg = quantize_rows(bits, wg)
    u, su = quantize_rows(bits, wu)
    d, sd = quantize_rows(bits, wd)
    return Expert(bits, g, u, d, sg, su, sd)


def expert_token(ex: Expert, xq_t: np.ndarray, sx_t: float):
    """O5 on one token. Returns dict of accg, accu, a, aq, sa, accd, y."""
    H, I = ex.H, ex.I
    xq_t = np.ascontiguousarray(xq_t, dtype=np.int8)
    out = dict(accg=np.empty(I, np.int32), accu=np.empty(I, np.int32), a=np.empty(I, np.float32),
               aq=np.empty(I, np.int8), sa=np.empty(1, np.float32), accd=np.empty(H, np.int32),
               y=np.empty(H, np.float32))
    st = ex.struct()
    _check(_load().orc_expert_token(ex.bits, ctypes.byref(st), _p(xq_t), ctypes.c_float(sx_t), H, I,
                                    _p(out["accg"]), _p(out["accu"]), _p(out["a"]), _p(out["aq"]), _p(out["sa"]),
                                    _p(out["accd"]), _p(out["y"])), "expert_token")
    out["sa"] = float(out["sa"][0])
    return out


# --- O7 ----------------------------------------------------------------------

def combine(y_slots: np.ndarray, w: np.ndarray, has_shared: bool) -> np.ndarray:
    y_slots = np.ascontiguousarray(y_slots, dtype=np.float32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, S, H = y_slots.shape
    k = w.shape[1]
    assert S == k + (1 if has_shared else 0)
    out = np.empty((T, H), dtype=np.float32)
    _check(_load().orc_combine(_p(y_slots), _p(w), T, k, H, 1 if has_shared else 0, _p(out)), "combine")
    return out


# --- full layer ---------------------------------------------------------------

class ExpertTable:
    """Holds E host experts (entries may be None when never routed to)."""

    def __init__(self, experts: list):
        self.experts = experts
        E = len(experts)
        self._arr = (_Expert * E)()
        self.bits = np.zeros(E, dtype=np.uint8)
        for e, ex in enumerate(experts):
            if ex is not None:
                self._arr[e] = ex.struct()
                self.bits[e] = ex.bits


def layer(x: np.ndarray, table: ExpertTable, shared: Expert | None, k: int, wr: np.ndarray | None = None,
          bias: np.ndarray | None = None, logits: np.ndarray | None = None, routed_scale: float = 1.0,
          top_p: float = 0.0):
    """Full layer. Returns dict xq, sx, idx, w, y_slots, out. top_p > 0 applies
    the top-p truncation (orc_topp); dropped slots have id -1 and zero y.

    Experts referenced by the routing must be present in ``table``; the call
    raises if one is missing.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, H = x.shape
    E = len(table.experts)
    I = next(ex for ex in table.experts + [shared] if ex is not None).I
    S = k + (1 if shared is not None else 0)
    res = dict(xq=np.empty((T, H), np.int8), sx=np.empty(T, np.float32), idx=np.empty((T, k), np.int32),
               w=np.empty((T, k), np.float32), y_slots=np.empty((T, S, H), np.float32),
               out=np.empty((T, H), np.float32))
    # check routing covers only present experts: run the router first
    if logits is not None:
        idx, _ = router(logits, None, bias, k, logits_in=True, routed_scale=routed_scale)
    else:
        idx, _ = router(x, wr, bias, k, routed_scale=routed_scale)
    missing = sorted({int(e) for e in idx.ravel() if table.experts[int(e)] is None})
    if missing:
        raise KeyError(f"oracle layer: experts {missing[:8]} routed to but not provided")
    sh = shared.struct() if shared is not None else None
    lg = None if logits is None else np.ascontiguousarray(logits, dtype=np.float32)
    wr_ = None if wr is None else np.ascontiguousarray(wr, dtype=np.float32)
    b_ = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    _check(_load().orc_layer(_p(x), _p(lg), _p(wr_), _p(b_), float(routed_scale), ctypes.addressof(table._arr),
                             _p(table.bits), ctypes.byref(sh) if sh is not None else None,
                             shared.bits if shared is not None else 0, T, H, I, E, k, float(top_p),
                             _p(res["xq"]), _p(res["sx"]), _p(res["idx"]), _p(res["w"]), _p(res["y_slots"]),
                             _p(res["out"])), "layer")
    return res


def set_threads(n: int) -> int:
    """Threads the layer's (token, slot) loop uses (n <= 0: unchanged); returns
    the count now in use."""
    return int(_load().orc_set_threads(int(n)))


def swiglu_f64(wg, wu, wd, x):
    wg, wu, wd = (np.ascontiguousarray(a, dtype=np.float32) for a in (wg, wu, wd))
    x = np.ascontiguousarray(x, dtype=np.float32)
    I, H = wg.shape
    y = np.empty(H, dtype=np.float64)
    _check(_load().orc_swiglu_f64(_p(wg), _p(wu), _p(wd), _p(x), H, I, _p(y)), "swiglu_f64")
    return y
