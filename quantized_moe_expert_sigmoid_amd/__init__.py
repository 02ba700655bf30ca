"""Python binding of libmoe.so, the MI355X (gfx950) routed-expert MoE layer.

Argument marshalling only: every function here takes torch CUDA tensors,
checks dtypes/shapes/devices, and calls the C entry point of the same name in
``libmoe.so`` (declared in ``include/moe.h``). All arithmetic runs in the HIP
kernels. If the library is missing or the device is not a gfx950 GPU the
calls raise; there is no CPU fallback.

PyTorch provides device memory and the stream: calls are enqueued on the
torch current stream of the tensors' device at context creation (or on the
stream passed to :class:`MoeCtx`).
"""
from __future__ import annotations

import ctypes
import os
import sys
_sys = sys  # read by the destructors
import threading
import weakref

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIBRARY: another build of the same sources (the sanitizer build of the
# host code); by default the in-tree libmoe.so
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_HERE, "libmoe.so")
_lock = threading.Lock()
_lib = None

MOE_OK, MOE_EINVAL, MOE_ENOMEM, MOE_EHIP, MOE_EUNSUPPORTED, MOE_EPOOL, MOE_ETIMEOUT = 0, -1, -2, -3, -4, -5, -6
MOE_FFN_AUTO, MOE_FFN_DOT4, MOE_FFN_MFMA = 0, 1, 2
_STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ENOMEM", -3: "MOE_EHIP", -4: "MOE_EUNSUPPORTED",
           -5: "MOE_EPOOL", -6: "MOE_ETIMEOUT"}


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class ExpertW(ctypes.Structure):
    """moe_expert_w: six device pointers."""
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


class RouterCfg(ctypes.Structure):
    _fields_ = [("n_experts", ctypes.c_int), ("top_k", ctypes.c_int), ("routed_scale", ctypes.c_float),
                ("logits_in", ctypes.c_int), ("top_p", ctypes.c_float)]


class DebugBufs(ctypes.Structure):
    _fields_ = [("accg", ctypes.c_void_p), ("accu", ctypes.c_void_p), ("a", ctypes.c_void_p),
                ("aq", ctypes.c_void_p), ("sa", ctypes.c_void_p), ("accd", ctypes.c_void_p)]


# name -> (restype, argtypes)
_vp, _i32, _i64, _sz, _f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_SIGS = {
    "moe_ctx_create": (_i32, [_i32, _vp, ctypes.POINTER(_vp)]),
    "moe_ctx_destroy": (None, [_vp]),
    "moe_ctx_set_stream": (_i32, [_vp, _vp]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (_i32, []),
    "moe_ctx_check": (_i32, [_vp]),
    "moe_expert_block_layout": (_sz, [_i32, _i32, _i32, ctypes.POINTER(_sz)]),
    "moe_quantize_rows": (_i32, [_vp, _i32, _vp, _i64, _i32, _vp, _vp]),
    "moe_quantize_act_i8": (_i32, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "moe_router_topk": (_i32, [_vp, ctypes.POINTER(RouterCfg), _vp, _vp, _vp, _i32, _i32, _vp, _vp]),
    "moe_bucket_tokens": (_i32, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_expert_ffn_q4": (_i32, [_vp, _vp, ctypes.POINTER(ExpertW), _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                 _i32, _vp]),
    "moe_expert_ffn_q8": (_i32, [_vp, _vp, ctypes.POINTER(ExpertW), _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                 _i32, _vp]),
    "moe_expert_ffn_q2": (_i32, [_vp, _vp, ctypes.POINTER(ExpertW), _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                 _i32, _vp]),
    "moe_combine": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp]),
    "moe_ctx_set_debug": (_i32, [_vp, ctypes.POINTER(DebugBufs)]),
    "moe_ctx_enable_timing": (_i32, [_vp, _i32]),
    "moe_ctx_set_ffn_kernels": (_i32, [_vp, _i32]),
    "moe_ctx_read_timing": (_i32, [_vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)]),
    "moe_layer_forward": (_i32, [_vp, _i32, ctypes.POINTER(RouterCfg), _vp, _vp, _vp, _vp, _vp,
                                 ctypes.POINTER(ExpertW), _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_pool_create": (_i32, [_vp, _sz, _i32, _i32, _i32, _i32, ctypes.POINTER(_vp)]),
    "moe_pool_destroy": (None, [_vp]),
    "moe_pool_register": (_i32, [_vp, _i32, _i32, _i32, _vp, _sz, _i32]),
    "moe_pool_prepare": (_i32, [_vp, _i32, _vp, _i32, _i32, _vp, _vp, ctypes.POINTER(ctypes.c_int)]),
    "moe_pool_stats": (_i32, [_vp, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64),
                              ctypes.POINTER(ctypes.c_uint64)]),
    "moe_pool_resident": (_i32, [_vp, _i32, _i32]),
    "moe_pool_prefetch": (_i32, [_vp, _i32, _vp, _i32, ctypes.POINTER(ctypes.c_int)]),
    "moe_pool_usage": (_i32, [_vp, _vp]),
    "moe_pool_pin_hot": (_i32, [_vp, _vp, _sz, ctypes.POINTER(ctypes.c_int)]),
    "moe_pool_prefetch_stats": (_i32, [_vp, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_uint64)]),
    "moe_probe_stream_read": (_i32, [_vp, _vp, _sz, _sz, _i32, _i32, ctypes.POINTER(ctypes.c_uint32),
                                     ctypes.POINTER(ctypes.c_double)]),
    "moe_pool_register_alt": (_i32, [_vp, _i32, _i32, _i32, _vp, _sz]),
    "moe_pool_set_demotion": (_i32, [_vp, _i32]),
    "moe_pool_tier_stats": (_i32, [_vp] + [ctypes.POINTER(ctypes.c_uint64)] * 3),
    "moe_pool_resident_bits": (_i32, [_vp, _i32, _i32]),
    "moe_expert_ffn_mixed": (_i32, [_vp, _vp, ctypes.POINTER(ExpertW), _i32, _vp, _i32, _vp, _vp, _vp, _vp]
                             + [_i32] * 5 + [_vp, _vp]),
    "moe_expert_ffn_mixed_x": (_i32, [_vp, _vp, ctypes.POINTER(ExpertW), _i32, _vp, _i32, _vp, _vp, _vp]
                               + [_i32] * 5 + [_vp, _vp]),
    "moe_pool_call_widths": (_i32, [_vp, ctypes.POINTER(_i32)]),
    "moe_pool_table_stats": (_i32, [_vp] + [ctypes.POINTER(ctypes.c_uint64)] * 2),
    "moe_pool_layer_table": (_i32, [_vp, _i32, ctypes.POINTER(_vp), ctypes.POINTER(_vp)]),
    "moe_layer_forward_noalloc": (_i32, [_vp, _i32, ctypes.POINTER(RouterCfg), _vp, _vp, _vp, _vp, _vp,
                                         ctypes.POINTER(ExpertW), _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
}


def exported_names():
    return list(_SIGS)


def lib():
    """Load libmoe.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                                   "`python -m quantized_moe_expert_sigmoid_amd.build` (no CPU fallback exists)")
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGS.items():
                f = getattr(L, name)
                f.restype = res
                f.argtypes = args
            _lib = L
    return _lib


def _ck(st: int):
    if st != MOE_OK:
        raise MoeError(st, lib().moe_last_error().decode(errors="replace"))


def _ptr(t):
    if t is None:
        return None
    return t.data_ptr()


def _dev(t: torch.Tensor, dtype, name, shape=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) torch tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")
    return t.data_ptr()


class MoeCtx:
    """moe_ctx bound to one device and one stream."""

    def __init__(self, device: int = 0, stream: torch.cuda.Stream | None = None):
        self.device = device
        s = stream if stream is not None else torch.cuda.current_stream(device)
        self.stream = s
        h = ctypes.c_void_p()
        _ck(lib().moe_ctx_create(device, ctypes.c_void_p(s.cuda_stream), ctypes.byref(h)))
        self.handle = h
        self._dbg_keep = None
        self._pools = weakref.WeakSet()  # pools on this context: closed before it

    def close(self):
        if self.handle:
            for p in list(self._pools):
                p.close()
            lib().moe_ctx_destroy(self.handle)
            self.handle = None

    def __del__(self):
        # at interpreter teardown the HIP runtime (and this module's globals)
        # may already be gone
        if _sys is None or _sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def set_stream(self, stream: torch.cuda.Stream):
        _ck(lib().moe_ctx_set_stream(self.handle, ctypes.c_void_p(stream.cuda_stream)))
        self.stream = stream

    def check(self):
        _ck(lib().moe_ctx_check(self.handle))

    STAGES = ("router", "bucket", "gateup", "requant", "down", "combine")

    def set_ffn_kernels(self, which):
        """"auto", "dot4" or "mfma" (or MOE_FFN_*): kernels of the expert FFN."""
        if isinstance(which, str):
            which = {"auto": MOE_FFN_AUTO, "dot4": MOE_FFN_DOT4, "mfma": MOE_FFN_MFMA}[which]
        _ck(lib().moe_ctx_set_ffn_kernels(self.handle, int(which)))

    def enable_timing(self, on: bool = True):
        _ck(lib().moe_ctx_enable_timing(self.handle, 1 if on else 0))

    def read_timing(self) -> dict:
        """{stage: (total_ms, launches)} since the last read (waits for the events)."""
        ms = (ctypes.c_double * len(self.STAGES))()
        n = (ctypes.c_int * len(self.STAGES))()
        _ck(lib().moe_ctx_read_timing(self.handle, ms, n))
        return {name: (ms[i], n[i]) for i, name in enumerate(self.STAGES)}

    def set_debug(self, bufs: dict | None):
        """bufs: dict with any of accg, accu, a, aq, sa, accd (device tensors) or None."""
        if bufs is None:
            _ck(lib().moe_ctx_set_debug(self.handle, None))
            self._dbg_keep = None
            return
        d = DebugBufs(*[_ptr(bufs.get(n)) for n in ("accg", "accu", "a", "aq", "sa", "accd")])
        self._dbg_keep = bufs
        _ck(lib().moe_ctx_set_debug(self.handle, ctypes.byref(d)))


# ---------------------------------------------------------------------------
# Entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def moe_expert_block_layout(bits: int, H: int, I: int):
    offs = (ctypes.c_size_t * 6)()
    n = lib().moe_expert_block_layout(bits, H, I, offs)
    if n == 0:
        raise MoeError(MOE_EINVAL, f"moe_expert_block_layout: bits {bits} H {H} I {I}")
    return int(n), [int(o) for o in offs]


def moe_quantize_rows(ctx: MoeCtx, bits: int, w: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor):
    R, C = w.shape
    _dev(w, torch.float32, "w")
    _dev(packed, torch.uint8, "packed", (R, C * bits // 8))
    _dev(scales, torch.float32, "scales", (R,))
    _ck(lib().moe_quantize_rows(ctx.handle, bits, w.data_ptr(), R, C, packed.data_ptr(), scales.data_ptr()))
    return packed, scales


def moe_quantize_act_i8(ctx: MoeCtx, x: torch.Tensor, xq: torch.Tensor, sx: torch.Tensor):
    T, H = x.shape
    _dev(x, torch.float32, "x")
    _dev(xq, torch.int8, "xq", (T, H))
    _dev(sx, torch.float32, "sx", (T,))
    _ck(lib().moe_quantize_act_i8(ctx.handle, x.data_ptr(), T, H, xq.data_ptr(), sx.data_ptr()))
    return xq, sx


def moe_router_topk(ctx: MoeCtx, x: torch.Tensor, w_router: torch.Tensor | None, bias: torch.Tensor | None, k: int,
                    topk_idx: torch.Tensor, topk_w: torch.Tensor, routed_scale: float = 1.0,
                    logits_in: bool = False, n_experts: int | None = None, top_p: float = 0.0):
    T = x.shape[0]
    _dev(x, torch.float32, "x")
    if logits_in:
        E, H = x.shape[1], 0
    else:
        E, H = w_router.shape
        _dev(w_router, torch.float32, "w_router", (E, x.shape[1]))
    if n_experts is not None and n_experts != E:
        raise ValueError("n_experts does not match the logits/router width")
    if bias is not None:
        _dev(bias, torch.float32, "bias", (E,))
    _dev(topk_idx, torch.int32, "topk_idx", (T, k))
    _dev(topk_w, torch.float32, "topk_w", (T, k))
    cfg = RouterCfg(E, k, float(routed_scale), 1 if logits_in else 0, float(top_p))
    _ck(lib().moe_router_topk(ctx.handle, ctypes.byref(cfg), x.data_ptr(),
                              None if logits_in else w_router.data_ptr(), _ptr(bias), T, H,
                              topk_idx.data_ptr(), topk_w.data_ptr()))
    return topk_idx, topk_w


def moe_bucket_tokens(ctx: MoeCtx, topk_idx: torch.Tensor, E: int, counts: torch.Tensor, offsets: torch.Tensor,
                      perm: torch.Tensor):
    T, k = topk_idx.shape
    _dev(topk_idx, torch.int32, "topk_idx")
    _dev(counts, torch.int32, "counts", (E,))
    _dev(offsets, torch.int32, "offsets", (E + 1,))
    _dev(perm, torch.int32, "perm", (T * k,))
    _ck(lib().moe_bucket_tokens(ctx.handle, topk_idx.data_ptr(), T, k, E, counts.data_ptr(), offsets.data_ptr(),
                                perm.data_ptr()))
    return counts, offsets, perm


def _ffn(name, ctx, table, shared, expert_bits, xq, sx, topk_idx, H, I, E, y_slots):
    T, k = topk_idx.shape
    _dev(table, torch.int64, "experts table", (E, 6))
    _dev(xq, torch.int8, "xq", (T, H))
    _dev(sx, torch.float32, "sx", (T,))
    _dev(topk_idx, torch.int32, "topk_idx")
    _dev(y_slots, torch.float32, "y_slots", (T, k + 1, H))
    if expert_bits is not None:
        _dev(expert_bits, torch.uint8, "expert_bits", (E,))
    sh = ctypes.byref(shared) if shared is not None else None
    _ck(getattr(lib(), name)(ctx.handle, table.data_ptr(), sh, _ptr(expert_bits), xq.data_ptr(), sx.data_ptr(),
                             topk_idx.data_ptr(), T, H, I, E, k, y_slots.data_ptr()))
    return y_slots


def moe_expert_ffn_q4(ctx, table, shared, expert_bits, xq, sx, topk_idx, H, I, E, y_slots):
    return _ffn("moe_expert_ffn_q4", ctx, table, shared, expert_bits, xq, sx, topk_idx, H, I, E, y_slots)


def moe_expert_ffn_q8(ctx, table, shared, expert_bits, xq, sx, topk_idx, H, I, E, y_slots):
    return _ffn("moe_expert_ffn_q8", ctx, table, shared, expert_bits, xq, sx, topk_idx, H, I, E, y_slots)


def moe_expert_ffn_q2(ctx, table, shared, expert_bits, xq, sx, topk_idx, H, I, E, y_slots):
    return _ffn("moe_expert_ffn_q2", ctx, table, shared, expert_bits, xq, sx, topk_idx, H, I, E, y_slots)


FFN_BY_BITS = {4: moe_expert_ffn_q4, 8: moe_expert_ffn_q8, 2: moe_expert_ffn_q2}


def _widths_mask(widths):
    if isinstance(widths, int):
        return widths
    mask = 0
    for b in widths:
        mask |= 1 << int(b)
    return mask


def moe_expert_ffn_mixed(ctx, table, shared, shared_bits, expert_bits, widths, xq, sx, topk_idx, H, I, E, y_slots,
                         topk_w=None, out=None, x=None):
    """Every slot at its expert's width (expert_bits, device uint8 [E]);
    widths: the widths the layer has (iterable of 8, 4, 2), or the mask
    itself (an int, as moe_pool_call_widths gives it). With out (and
    topk_w): also the combine of the slots. table and expert_bits may be raw
    device addresses (a pool's own table, MoePool.layer_table). With x (fp32
    hidden states [T][H]) in place of xq and sx (both None): the call
    quantises them itself (moe_expert_ffn_mixed_x)."""
    T, k = topk_idx.shape
    if not isinstance(table, int):
        _dev(table, torch.int64, "experts table", (E, 6))
    if x is not None:
        if xq is not None or sx is not None:
            raise ValueError("pass either x or (xq, sx)")
        _dev(x, torch.float32, "x", (T, H))
    else:
        _dev(xq, torch.int8, "xq", (T, H))
        _dev(sx, torch.float32, "sx", (T,))
    _dev(topk_idx, torch.int32, "topk_idx")
    _dev(y_slots, torch.float32, "y_slots", (T, k + 1, H))
    if not isinstance(expert_bits, int):
        _dev(expert_bits, torch.uint8, "expert_bits", (E,))
    if out is not None:
        _dev(out, torch.float32, "out", (T, H))
        _dev(topk_w, torch.float32, "topk_w", (T, k))
    mask = _widths_mask(widths)
    sh = ctypes.byref(shared) if shared is not None else None
    tp = table if isinstance(table, int) else table.data_ptr()
    bp = expert_bits if isinstance(expert_bits, int) else expert_bits.data_ptr()
    if x is not None:
        _ck(lib().moe_expert_ffn_mixed_x(ctx.handle, tp, sh, int(shared_bits), bp, mask, x.data_ptr(),
                                         topk_idx.data_ptr(), _ptr(topk_w), T, H, I, E, k, y_slots.data_ptr(),
                                         _ptr(out)))
    else:
        _ck(lib().moe_expert_ffn_mixed(ctx.handle, tp, sh, int(shared_bits), bp, mask,
                                       xq.data_ptr(), sx.data_ptr(), topk_idx.data_ptr(), _ptr(topk_w), T, H, I, E, k,
                                       y_slots.data_ptr(), _ptr(out)))
    return y_slots


def moe_combine(ctx: MoeCtx, y_slots: torch.Tensor, topk_w: torch.Tensor, has_shared: bool, out: torch.Tensor):
    T, S, H = y_slots.shape
    k = topk_w.shape[1]
    if S != k + 1:
        raise ValueError("y_slots must be [T][k+1][H]")
    _dev(y_slots, torch.float32, "y_slots")
    _dev(topk_w, torch.float32, "topk_w", (T, k))
    _dev(out, torch.float32, "out", (T, H))
    _ck(lib().moe_combine(ctx.handle, y_slots.data_ptr(), topk_w.data_ptr(), T, k, H, 1 if has_shared else 0,
                          out.data_ptr()))
    return out


def moe_probe_stream_read(ctx: MoeCtx, buf: torch.Tensor, bytes_per_launch: int, wg_per_cu: int = 4,
                          reps: int = 20):
    """Streaming-read probe over a device uint8 buffer (see include/moe.h).
    Returns (xor of the last window's 32-bit words, average launch us)."""
    _dev(buf, torch.uint8, "buf")
    x, us = ctypes.c_uint32(), ctypes.c_double()
    _ck(lib().moe_probe_stream_read(ctx.handle, buf.data_ptr(), buf.numel(), int(bytes_per_launch), int(wg_per_cu),
                                    int(reps), ctypes.byref(x), ctypes.byref(us)))
    return x.value, us.value


def moe_layer_forward(ctx: MoeCtx, bits: int, x: torch.Tensor, table: torch.Tensor, shared: ExpertW | None,
                      k: int, I: int, out: torch.Tensor, w_router: torch.Tensor | None = None,
                      bias: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                      routed_scale: float = 1.0, topk_idx=None, topk_w=None, xq=None, sx=None, y_slots=None,
                      top_p: float = 0.0):
    """Whole layer in one call (see include/moe.h). Optional outputs may be None."""
    return _layer("moe_layer_forward", ctx, bits, x, table, shared, k, I, out, w_router, bias, logits, routed_scale,
                  topk_idx, topk_w, xq, sx, y_slots, top_p)


def moe_layer_forward_noalloc(ctx: MoeCtx, bits: int, x: torch.Tensor, table: torch.Tensor, shared: ExpertW | None,
                              k: int, I: int, out: torch.Tensor, w_router: torch.Tensor | None = None,
                              bias: torch.Tensor | None = None, logits: torch.Tensor | None = None,
                              routed_scale: float = 1.0, topk_idx=None, topk_w=None, xq=None, sx=None,
                              y_slots=None, top_p: float = 0.0):
    """moe_layer_forward with the library's static scratch: allocates nothing
    (see include/moe.h for its size limit and sharing rule)."""
    return _layer("moe_layer_forward_noalloc", ctx, bits, x, table, shared, k, I, out, w_router, bias, logits,
                  routed_scale, topk_idx, topk_w, xq, sx, y_slots, top_p)


def _layer(name, ctx, bits, x, table, shared, k, I, out, w_router, bias, logits, routed_scale, topk_idx, topk_w, xq,
           sx, y_slots, top_p):
    T, H = x.shape
    E = table.shape[0]
    _dev(x, torch.float32, "x")
    _dev(table, torch.int64, "experts table", (E, 6))
    _dev(out, torch.float32, "out", (T, H))
    if logits is not None:
        _dev(logits, torch.float32, "logits", (T, E))
    else:
        _dev(w_router, torch.float32, "w_router", (E, H))
    if bias is not None:
        _dev(bias, torch.float32, "bias", (E,))
    for t, dt, shp, nm in ((topk_idx, torch.int32, (T, k), "topk_idx"), (topk_w, torch.float32, (T, k), "topk_w"),
                           (xq, torch.int8, (T, H), "xq"), (sx, torch.float32, (T,), "sx"),
                           (y_slots, torch.float32, (T, k + 1, H), "y_slots")):
        if t is not None:
            _dev(t, dt, nm, shp)
    cfg = RouterCfg(E, k, float(routed_scale), 1 if logits is not None else 0, float(top_p))
    sh = ctypes.byref(shared) if shared is not None else None
    _ck(getattr(lib(), name)(ctx.handle, bits, ctypes.byref(cfg), x.data_ptr(), _ptr(logits),
                             None if logits is not None else w_router.data_ptr(), _ptr(bias), table.data_ptr(), sh,
                             T, H, I, out.data_ptr(), _ptr(topk_idx), _ptr(topk_w), _ptr(xq), _ptr(sx),
                             _ptr(y_slots)))
    return out


# ---------------------------------------------------------------------------
# Expert storage helpers (device memory via torch, layout from the library)
# ---------------------------------------------------------------------------

class ExpertBlocks:
    """n experts stored as contiguous blocks (moe_expert_block_layout) in one
    device tensor, plus the device table of moe_expert_w pointers."""

    def __init__(self, n: int, bits: int, H: int, I: int, device="cuda"):
        self.n, self.bits, self.H, self.I = n, bits, H, I
        self.block_bytes, self.offsets = moe_expert_block_layout(bits, H, I)
        self.data = torch.empty((n, self.block_bytes), dtype=torch.uint8, device=device)
        base = self.data.data_ptr()
        rows = [[base + e * self.block_bytes + o for o in self.offsets] for e in range(n)]
        self.table = torch.tensor(rows, dtype=torch.int64, device=device)

    def views(self, e: int):
        """(gate, up, down, s_gate, s_up, s_down) tensor views of expert e."""
        H, I, b = self.H, self.I, self.bits
        blk = self.data[e]
        o = self.offsets
        g = blk[o[0]:o[0] + I * H * b // 8].view(I, H * b // 8)
        u = blk[o[1]:o[1] + I * H * b // 8].view(I, H * b // 8)
        d = blk[o[2]:o[2] + H * I * b // 8].view(H, I * b // 8)
        sg = blk[o[3]:o[3] + 4 * I].view(torch.float32)
        su = blk[o[4]:o[4] + 4 * I].view(torch.float32)
        sd = blk[o[5]:o[5] + 4 * H].view(torch.float32)
        return g, u, d, sg, su, sd

    def struct(self, e: int) -> ExpertW:
        return ExpertW(*[self.data.data_ptr() + e * self.block_bytes + o for o in self.offsets])

    def pack_from_fp32(self, ctx: MoeCtx, e: int, wg: torch.Tensor, wu: torch.Tensor, wd: torch.Tensor):
        """Quantise fp32 gate/up/down on the GPU straight into expert e's block."""
        g, u, d, sg, su, sd = self.views(e)
        moe_quantize_rows(ctx, self.bits, wg, g, sg)
        moe_quantize_rows(ctx, self.bits, wu, u, su)
        moe_quantize_rows(ctx, self.bits, wd, d, sd)


# ---------------------------------------------------------------------------
# Expert pool
# ---------------------------------------------------------------------------

class MoePool:
    """moe_pool: HBM cache of expert blocks refilled from pinned host memory.
    ctx=None gives a bookkeeping-only pool (no device memory, no copies)."""

    def __init__(self, ctx: MoeCtx | None, capacity_bytes: int, n_layers: int, n_experts: int, H: int, I: int):
        self.ctx, self.n_layers, self.n_experts, self.H, self.I = ctx, n_layers, n_experts, H, I
        h = ctypes.c_void_p()
        _ck(lib().moe_pool_create(ctx.handle if ctx is not None else None, capacity_bytes, n_layers, n_experts,
                                  H, I, ctypes.byref(h)))
        self.handle = h.value
        self._blocks = {}  # keeps the registered host blocks alive
        if ctx is not None:
            ctx._pools.add(self)

    def close(self):
        if self.handle:
            lib().moe_pool_destroy(self.handle)
            self.handle = None
            self._blocks.clear()

    def __del__(self):
        # at interpreter teardown the HIP runtime (and this module's globals)
        # may already be gone
        if _sys is None or _sys.is_finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    def register(self, layer: int, expert: int, bits: int, block_host: torch.Tensor | None, pin: bool = False,
                 nbytes: int | None = None):
        """block_host: CPU uint8 tensor holding the block (pinned for an
        asynchronous refill); None only for a bookkeeping-only pool."""
        if block_host is not None:
            if block_host.is_cuda or block_host.dtype != torch.uint8 or not block_host.is_contiguous():
                raise TypeError("block_host must be a contiguous CPU uint8 tensor")
            nbytes = block_host.numel()
            ptr = block_host.data_ptr()
        else:
            nbytes = moe_expert_block_layout(bits, self.H, self.I)[0] if nbytes is None else nbytes
            ptr = None
        _ck(lib().moe_pool_register(self.handle, layer, expert, bits, ptr, nbytes, 1 if pin else 0))
        if block_host is not None:
            self._blocks[(layer, expert)] = block_host

    def prepare(self, layer: int, topk_idx_host, table: torch.Tensor | None = None,
                bits: torch.Tensor | None = None) -> int:
        """topk_idx_host: int32 [T][k] on the host (numpy array or CPU tensor).
        table: device int64 [E][6] (moe_expert_w rows), bits: device uint8 [E];
        or the raw addresses from layer_table(layer). Returns the number of
        misses."""
        import numpy as np
        idx = np.ascontiguousarray(topk_idx_host if not isinstance(topk_idx_host, torch.Tensor)
                                   else topk_idx_host.cpu().numpy(), dtype=np.int32)
        if idx.ndim != 2:
            raise ValueError("topk_idx_host must be [T][k]")
        T, k = idx.shape
        if table is not None and not isinstance(table, int):
            _dev(table, torch.int64, "table", (self.n_experts, 6))
        if bits is not None and not isinstance(bits, int):
            _dev(bits, torch.uint8, "bits", (self.n_experts,))
        tp = table if isinstance(table, int) else _ptr(table)
        bp = bits if isinstance(bits, int) else _ptr(bits)
        n = ctypes.c_int(0)
        _ck(lib().moe_pool_prepare(self.handle, layer, idx.ctypes.data if idx.size else None, T, k,
                                   tp, bp, ctypes.byref(n)))
        return n.value

    def stats(self):
        h, m, b = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
        _ck(lib().moe_pool_stats(self.handle, ctypes.byref(h), ctypes.byref(m), ctypes.byref(b)))
        return {"hits": h.value, "misses": m.value, "bytes_h2d": b.value}

    def prefetch(self, layer: int, ids_host) -> int:
        """Start refills of the given experts of `layer` (best effort); returns
        how many were started."""
        import numpy as np
        ids = np.ascontiguousarray(ids_host, dtype=np.int32).ravel()
        n = ctypes.c_int(0)
        _ck(lib().moe_pool_prefetch(self.handle, layer, ids.ctypes.data if ids.size else None, ids.size,
                                    ctypes.byref(n)))
        return n.value

    def usage(self):
        """Requests per (layer, expert): uint64 numpy array [n_layers][E]."""
        import numpy as np
        c = np.zeros((self.n_layers, self.n_experts), dtype=np.uint64)
        _ck(lib().moe_pool_usage(self.handle, c.ctypes.data))
        return c

    def pin_hot(self, budget_bytes: int, counts=None) -> int:
        """Pin the most requested experts within budget_bytes (counts: the
        usage array of an earlier run, or None for this pool's own)."""
        import numpy as np
        c = None if counts is None else np.ascontiguousarray(counts, dtype=np.uint64)
        if c is not None and c.shape != (self.n_layers, self.n_experts):
            raise ValueError("counts must be [n_layers][n_experts]")
        n = ctypes.c_int(0)
        _ck(lib().moe_pool_pin_hot(self.handle, c.ctypes.data if c is not None else None, int(budget_bytes),
                                   ctypes.byref(n)))
        return n.value

    def save_usage(self, path: str):
        """Write the usage counts (the engine's usage file): numpy .npy."""
        import numpy as np
        np.save(path, self.usage(), allow_pickle=False)

    @staticmethod
    def load_usage(path: str):
        import numpy as np
        return np.load(path, allow_pickle=False)

    def prefetch_stats(self):
        i, u = ctypes.c_uint64(), ctypes.c_uint64()
        _ck(lib().moe_pool_prefetch_stats(self.handle, ctypes.byref(i), ctypes.byref(u)))
        return {"issued": i.value, "used": u.value}

    def register_alt(self, layer: int, expert: int, bits: int, block_host: torch.Tensor | None,
                     nbytes: int | None = None):
        """A narrower block of an already registered expert (int4 under int8,
        int2 under int4), loaded instead of the full one under pressure when
        demotion is on."""
        if block_host is not None:
            if block_host.is_cuda or block_host.dtype != torch.uint8 or not block_host.is_contiguous():
                raise TypeError("block_host must be a contiguous CPU uint8 tensor")
            nbytes = block_host.numel()
            ptr = block_host.data_ptr()
        else:
            nbytes = moe_expert_block_layout(bits, self.H, self.I)[0] if nbytes is None else nbytes
            ptr = None
        _ck(lib().moe_pool_register_alt(self.handle, layer, expert, bits, ptr, nbytes))
        if block_host is not None:
            self._blocks[(layer, expert, "alt")] = block_host

    def set_demotion(self, enable: bool):
        _ck(lib().moe_pool_set_demotion(self.handle, 1 if enable else 0))

    def tier_stats(self):
        v = [ctypes.c_uint64() for _ in range(3)]
        _ck(lib().moe_pool_tier_stats(self.handle, *(ctypes.byref(x) for x in v)))
        return {"demoted_loads": v[0].value, "demoted_uses": v[1].value, "bytes_saved": v[2].value}

    def table_stats(self):
        v = [ctypes.c_uint64() for _ in range(2)]
        _ck(lib().moe_pool_table_stats(self.handle, *(ctypes.byref(x) for x in v)))
        return {"copies": v[0].value, "skipped": v[1].value}

    def call_widths(self) -> int:
        """Bit b set when an expert of the latest prepare call is resident at width b."""
        m = ctypes.c_int()
        _ck(lib().moe_pool_call_widths(self.handle, ctypes.byref(m)))
        return m.value

    def layer_table(self, layer: int):
        """The pool's own device table of `layer`: (table address, widths
        address), raw device pointers (the widths follow the table). Passing
        them to prepare lets it skip copies of an unchanged table."""
        t, b = _vp(), _vp()
        _ck(lib().moe_pool_layer_table(self.handle, layer, ctypes.byref(t), ctypes.byref(b)))
        return t.value, b.value

    def resident_bits(self, layer: int, expert: int) -> int:
        """Width of the resident copy (8, 4, 2), 0 when not resident."""
        r = lib().moe_pool_resident_bits(self.handle, layer, expert)
        if r < 0:
            raise MoeError(MOE_EINVAL, "moe_pool_resident_bits: invalid arguments")
        return r

    def resident(self, layer: int, expert: int) -> bool:
        r = lib().moe_pool_resident(self.handle, layer, expert)
        if r < 0:
            raise MoeError(MOE_EINVAL, "moe_pool_resident: invalid arguments")
        return bool(r)
