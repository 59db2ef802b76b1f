"""Python binding of the MI355X quantized-recurrent-state decode library.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libstq.so`` (built in-tree by ``build.py``).  PyTorch supplies device memory
and the stream.  Importing this package fails loudly when the library is not
built; there is no fallback.

Names follow the C ABI in ``include/stq.h``: ``Layout`` (stq_pack_layout),
``Pool`` (stq_alloc_pool), ``decode_step``, ``unpack``, ``pack``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# STQ_LIBRARY selects another build of this library (libstq_debug.so,
# libstq_san.so); the default is the release build next to this file
LIB_PATH = os.environ.get("STQ_LIBRARY") or os.path.join(HERE, "libstq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

_lib = C.CDLL(LIB_PATH)

STQ_OK, STQ_ERR_INVALID, STQ_ERR_UNSUPPORTED, STQ_ERR_TOO_SMALL, STQ_ERR_ALIGN, STQ_ERR_DEVICE = range(6)
UNIT_HEAD, UNIT_KEYROW = 0, 1
GATE_SCALAR, GATE_KEYVEC = 0, 1
NONE, F32, F16, BF16 = 0, 1, 2, 3
FIT_STEP, FIT_LAGGED = 0, 1

SYMBOLS = ["stq_status_string", "stq_last_error", "stq_pack_layout", "stq_layout_query",
           "stq_layout_head", "stq_layout_free", "stq_alloc_pool", "stq_decode_step",
           "stq_unpack", "stq_pack", "stq_fit_scales", "stq_check_slot_ids", "stq_allocate_bits"]


class StqConfig(C.Structure):
    _fields_ = [("H", C.c_int32), ("d_k", C.c_int32), ("d_v", C.c_int32),
                ("unit", C.c_int32), ("gate", C.c_int32), ("row_scale", C.c_int32),
                ("col_scale", C.c_int32), ("io_dtype", C.c_int32), ("window", C.c_int32),
                ("comps", C.c_int32), ("scale_fit", C.c_int32), ("unit_bits", C.POINTER(C.c_uint8)),
                ("row_impact", C.POINTER(C.c_float))]


class StqPool(C.Structure):
    _fields_ = [("base", C.c_void_p), ("bytes", C.c_size_t), ("slots", C.c_int32),
                ("layout", C.c_void_p)]


_P = C.c_void_p
_lib.stq_status_string.restype = C.c_char_p
_lib.stq_status_string.argtypes = [C.c_int]
_lib.stq_last_error.restype = C.c_char_p
_lib.stq_last_error.argtypes = []
_lib.stq_pack_layout.argtypes = [C.POINTER(StqConfig), C.POINTER(_P)]
_lib.stq_layout_query.argtypes = [_P, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]
_lib.stq_layout_head.argtypes = [_P, C.c_int32, C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]
_lib.stq_layout_free.argtypes = [_P]
_lib.stq_layout_free.restype = None
_lib.stq_alloc_pool.argtypes = [_P, C.c_int32, _P, C.c_size_t, _P, C.POINTER(StqPool)]
_lib.stq_decode_step.argtypes = [C.POINTER(StqPool), C.c_int32, _P, _P, _P, _P, _P, _P, _P, _P]
_lib.stq_unpack.argtypes = [C.POINTER(StqPool), C.c_int32, _P, _P, _P]
_lib.stq_pack.argtypes = [C.POINTER(StqPool), C.c_int32, _P, _P, _P]
_lib.stq_allocate_bits.argtypes = [C.c_int32, _P, _P, C.c_double, C.c_int32, _P]
_lib.stq_check_slot_ids.argtypes = [C.POINTER(StqPool), C.c_int32, _P]
_lib.stq_fit_scales.argtypes = [C.POINTER(StqPool), C.c_int32, _P, _P]
for _f in ("stq_pack_layout", "stq_layout_query", "stq_layout_head", "stq_alloc_pool",
           "stq_decode_step", "stq_unpack", "stq_pack", "stq_fit_scales", "stq_check_slot_ids",
           "stq_allocate_bits"):
    getattr(_lib, _f).restype = C.c_int


class StqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.stq_status_string(status).decode()
        detail = _lib.stq_last_error().decode()
        super().__init__(f"{where}: {msg} ({detail})")


def _check(status: int, where: str) -> None:
    if status != STQ_OK:
        raise StqError(status, where)


def library():
    """The loaded ctypes handle (for symbol checks and direct C-ABI calls)."""
    return _lib


class Layout:
    """stq_pack_layout: validated configuration + slot layout (host object)."""

    def __init__(self, H, d_k, d_v, unit_bits, *, unit=UNIT_HEAD, gate=GATE_SCALAR,
                 row_scale=F16, col_scale=F16, io_dtype=BF16, window=1, comps=0,
                 scale_fit=FIT_STEP, row_impact=None):
        self.unit_bits = np.ascontiguousarray(unit_bits, dtype=np.uint8)
        self.row_impact = None if row_impact is None else np.ascontiguousarray(row_impact, dtype=np.float32)
        self.cfg = StqConfig(H, d_k, d_v, unit, gate, row_scale, col_scale, io_dtype, window,
                             comps, scale_fit, self.unit_bits.ctypes.data_as(C.POINTER(C.c_uint8)),
                             None if self.row_impact is None
                             else self.row_impact.ctypes.data_as(C.POINTER(C.c_float)))
        h = _P()
        _check(_lib.stq_pack_layout(C.byref(self.cfg), C.byref(h)), "stq_pack_layout")
        self.handle = h
        sb, hb = C.c_size_t(), C.c_size_t()
        _check(_lib.stq_layout_query(h, C.byref(sb), C.byref(hb)), "stq_layout_query")
        self.slot_bytes, self.header_bytes = sb.value, hb.value
        self.H, self.d_k, self.d_v = H, d_k, d_v
        self.io_dtype, self.gate, self.window = io_dtype, gate, window
        self.scale_fit = scale_fit

    @classmethod
    def from_workload(cls, w, unit_bits, row_impact=None):
        """Layout of a ``synth.Workload`` (any object with the same fields)."""
        return cls(w.H, w.dk, w.dv, unit_bits,
                   unit=UNIT_KEYROW if w.unit == "keyrow" else UNIT_HEAD,
                   gate=GATE_KEYVEC if w.gate == "keyvec" else GATE_SCALAR,
                   row_scale=F16 if w.row_scale == "f16" else F32,
                   col_scale=F16 if w.col_scale == "f16" else NONE,
                   io_dtype=BF16 if w.io == "bf16" else F32,
                   window=w.window, comps=w.comps,
                   scale_fit=FIT_LAGGED if getattr(w, "scale_fit", "step") == "lagged" else FIT_STEP,
                   row_impact=row_impact)

    def head(self, h: int):
        off, nb = C.c_size_t(), C.c_size_t()
        _check(_lib.stq_layout_head(self.handle, h, C.byref(off), C.byref(nb)), "stq_layout_head")
        return off.value, nb.value

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            _lib.stq_layout_free(h)
            self.handle = None


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _dptr(t, what, dtype=None):
    import torch
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what} must be {dtype}, got {t.dtype}")
    return C.c_void_p(t.data_ptr())


class Pool:
    """stq_alloc_pool over a torch uint8 device buffer owned by this object."""

    def __init__(self, layout: Layout, slots: int, device="cuda", stream=None):
        import torch
        self.layout = layout
        q = StqPool()
        _check(_lib.stq_alloc_pool(layout.handle, slots, None, 0, None, C.byref(q)), "stq_alloc_pool")
        self.buffer = torch.empty(q.bytes, dtype=torch.uint8, device=device)
        self.pool = StqPool()
        _check(_lib.stq_alloc_pool(layout.handle, slots, C.c_void_p(self.buffer.data_ptr()),
                                   q.bytes, _stream_ptr(stream), C.byref(self.pool)),
               "stq_alloc_pool")
        self.slots = slots

    def slot_bytes_view(self, s: int):
        """uint8 view of slot s (device)."""
        lo = self.layout.header_bytes + s * self.layout.slot_bytes
        return self.buffer[lo: lo + self.layout.slot_bytes]

    def slots_view(self):
        """[slots, slot_bytes] uint8 view of every slot (device)."""
        lo = self.layout.header_bytes
        return self.buffer[lo: lo + self.slots * self.layout.slot_bytes].view(
            self.slots, self.layout.slot_bytes)


def decode_step(pool: Pool, slot_ids, q, k, v, a, beta, o, stream=None) -> None:
    """stq_decode_step on torch device tensors (shapes as in include/stq.h)."""
    import torch
    L = pool.layout
    B = slot_ids.numel()
    io = torch.bfloat16 if L.io_dtype == BF16 else torch.float32
    if q.shape != (B, L.H, L.d_k) or k.shape != (B, L.H, L.d_k) or v.shape != (B, L.H, L.d_v):
        raise ValueError("q, k must be [B,H,d_k] and v [B,H,d_v]")
    want_a = (B, L.H, L.d_k) if L.gate == GATE_KEYVEC else (B, L.H)
    if tuple(a.shape) != want_a or tuple(beta.shape) != (B, L.H) or tuple(o.shape) != (B, L.H, L.d_v):
        raise ValueError(f"a must be {want_a}, beta [B,H], o [B,H,d_v]")
    _check(_lib.stq_decode_step(
        C.byref(pool.pool), B, _dptr(slot_ids, "slot_ids", torch.int32),
        _dptr(q, "q", io), _dptr(k, "k", io), _dptr(v, "v", io),
        _dptr(a, "a", torch.float32), _dptr(beta, "beta", torch.float32),
        _dptr(o, "o", torch.float32), _stream_ptr(stream)), "stq_decode_step")


def unpack(pool: Pool, slot_ids, out, stream=None) -> None:
    """stq_unpack into out [B,H,d_k,d_v] fp32."""
    import torch
    L = pool.layout
    B = slot_ids.numel()
    if tuple(out.shape) != (B, L.H, L.d_k, L.d_v):
        raise ValueError("out must be [B,H,d_k,d_v]")
    _check(_lib.stq_unpack(C.byref(pool.pool), B, _dptr(slot_ids, "slot_ids", torch.int32),
                           _dptr(out, "out", torch.float32), _stream_ptr(stream)), "stq_unpack")


def pack(pool: Pool, slot_ids, state, stream=None) -> None:
    """stq_pack of state [B,H,d_k,d_v] fp32 into the slots."""
    import torch
    L = pool.layout
    B = slot_ids.numel()
    if tuple(state.shape) != (B, L.H, L.d_k, L.d_v):
        raise ValueError("state must be [B,H,d_k,d_v]")
    _check(_lib.stq_pack(C.byref(pool.pool), B, _dptr(slot_ids, "slot_ids", torch.int32),
                         _dptr(state, "state", torch.float32), _stream_ptr(stream)), "stq_pack")


def fit_scales(pool: Pool, slot_ids, stream=None) -> None:
    """stq_fit_scales: next scales of the slots from their last step's
    statistics (lagged-scale layouts; run it on a side stream between steps)."""
    import torch
    _check(_lib.stq_fit_scales(C.byref(pool.pool), slot_ids.numel(),
                               _dptr(slot_ids, "slot_ids", torch.int32), _stream_ptr(stream)),
           "stq_fit_scales")


def check_slot_ids(pool: "Pool", slot_ids) -> None:
    """stq_check_slot_ids on host ids (numpy, list, or a tensor copied to the
    host): raises StqError naming the first out-of-range or repeated id."""
    ids = np.ascontiguousarray(
        slot_ids.cpu().numpy() if hasattr(slot_ids, "cpu") else slot_ids, dtype=np.int32)
    _check(_lib.stq_check_slot_ids(C.byref(pool.pool), int(ids.size), C.c_void_p(ids.ctypes.data)),
           "stq_check_slot_ids")


def allocate_bits(gate_mean, state_msq, avg_bits: float, n_pivots: int):
    """stq_allocate_bits on host arrays (one entry per unit); returns the
    uint8 unit widths (4/6/8, 16 for pivots) for Layout / stq_config."""
    import numpy as np
    g = np.ascontiguousarray(gate_mean, dtype=np.float32)
    m = np.ascontiguousarray(state_msq, dtype=np.float32)
    if g.ndim != 1 or g.shape != m.shape:
        raise ValueError("gate_mean and state_msq must be 1-D of one length")
    out = np.zeros(g.shape[0], np.uint8)
    _check(_lib.stq_allocate_bits(int(g.shape[0]), C.c_void_p(g.ctypes.data), C.c_void_p(m.ctypes.data),
                                  float(avg_bits), int(n_pivots), C.c_void_p(out.ctypes.data)),
           "stq_allocate_bits")
    return out


def calibrate(H, d_k, d_v, *, B, steps, inputs, unit=UNIT_HEAD, gate=GATE_SCALAR,
              io_dtype=BF16, warmup=None, device="cuda"):
    """Calibration statistics for the lifetime-aware bit allocation (STEPQuant
    essay, temporal-axis paragraphs: widths and pivots are chosen offline from
    how long each unit holds memory and how large its state is).

    Runs the unquantized recurrence -- a layout of fp32 units (width 32) --
    through stq_decode_step for `steps` steps of B requests, from the zero
    state, with ``inputs(t) -> (q, k, v, a, beta)`` device tensors shaped as
    for decode_step.  Returns float32 arrays over the units (H for
    STQ_UNIT_HEAD, H*d_k for STQ_UNIT_KEYROW, head-major):
      gate_mean  the unit's gate averaged over requests and steps (a head's
                 key-vector gates averaged over its rows);
      state_msq  the unit's mean squared state entry, averaged over requests
                 and the steps from `warmup` on (default steps // 2).
    Offline tooling: the reductions are torch operations on the device; the
    recurrence runs in the library's kernels."""
    import torch
    keyrow = unit == UNIT_KEYROW
    keyvec = gate == GATE_KEYVEC
    warmup = steps // 2 if warmup is None else warmup
    bits = np.full(H * d_k if keyrow else H, 32, np.uint8)
    L = Layout(H, d_k, d_v, bits, unit=unit, gate=gate, io_dtype=io_dtype)
    pool = Pool(L, B, device=device)
    ids = torch.arange(B, dtype=torch.int32, device=device)
    o = torch.empty(B, H, d_v, dtype=torch.float32, device=device)
    state = torch.empty(B, H, d_k, d_v, dtype=torch.float32, device=device)
    gsum = torch.zeros(H, d_k if keyvec else 1, dtype=torch.float64, device=device)
    ssum = torch.zeros(H, d_k, dtype=torch.float64, device=device)
    n_state = 0
    for t in range(steps):
        q, k, v, a, beta = inputs(t)
        decode_step(pool, ids, q, k, v, a, beta, o)
        gsum += (a.double() if keyvec else a.double()[..., None]).sum(dim=0)
        if t >= warmup:
            unpack(pool, ids, state)
            ssum += state.double().square().sum(dim=(0, 3))
            n_state += 1
    if n_state == 0:
        raise ValueError("calibrate: no step at or after warmup")
    g = (gsum / (steps * B)).cpu().numpy()               # [H, d_k] or [H, 1]
    m = (ssum / (n_state * B * d_v)).cpu().numpy()       # [H, d_k]: per key row
    if keyrow:
        gate_mean = np.broadcast_to(g, (H, d_k)).reshape(-1)
        state_msq = m.reshape(-1)
    else:
        gate_mean = g.mean(axis=1)
        state_msq = m.mean(axis=1)
    return gate_mean.astype(np.float32), state_msq.astype(np.float32)
