"""ctypes wrapper of the CPU oracle (``stq_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  The oracle
is plain single-threaded C; this file only marshals numpy arrays.  Every call
below releases the GIL (ctypes does), so independent units can be driven from
a thread pool while the oracle itself stays single-threaded per unit.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "stq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
LIB_SAN = os.path.join(HERE, "liboracle_san.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]
SANFLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
            "-shared-libasan"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no contraction of a*b+c into fma, no fast math)."""
    if os.environ.get("ORACLE_LIBRARY"):
        return os.environ["ORACLE_LIBRARY"]   # a prebuilt build (the sanitizer run)
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def build_sanitized() -> str:
    """The oracle with AddressSanitizer + UndefinedBehaviorSanitizer, built with
    clang so that it shares clang's ASan runtime with the library's sanitizer
    build (tests/sanitize.sh)."""
    tmp = LIB_SAN + ".tmp%d" % os.getpid()
    subprocess.check_call(["/opt/rocm/llvm/bin/clang", *CFLAGS, *SANFLAGS, SRC, "-o", tmp, "-lm"])
    os.replace(tmp, LIB_SAN)
    return LIB_SAN


class _Cfg(C.Structure):
    _fields_ = [("H", C.c_int32), ("dk", C.c_int32), ("dv", C.c_int32),
                ("unit_keyrow", C.c_int32), ("gate_vec", C.c_int32),
                ("rscale_f16", C.c_int32), ("cscale_f16", C.c_int32),
                ("window", C.c_int32), ("comps", C.c_int32), ("scale_fit", C.c_int32),
                ("bits", C.POINTER(C.c_uint8)), ("impact", C.POINTER(C.c_float))]


_lib = None


def lib():
    global _lib
    if _lib is None:
        L = C.CDLL(build())
        P = C.c_void_p
        L.ora_slot_bytes.restype = C.c_size_t
        L.ora_slot_bytes.argtypes = [P]
        L.ora_head_layout.argtypes = [P, C.c_int, P]
        L.ora_slot_init.argtypes = [P, P]
        L.ora_unpack_head.argtypes = [P, C.c_int, P, P]
        L.ora_pack_head.argtypes = [P, C.c_int, P, P]
        L.ora_step_head.argtypes = [P, C.c_int, P, P, P, P, P, C.c_float, P]
        L.ora_fit_head.argtypes = [P, C.c_int, P]
        L.ora_step_f32.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, P, C.c_float, P]
        L.ora_step_f64.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, P, C.c_double, P]
        L.ora_f32_to_f16.argtypes = [P, P, C.c_size_t]
        L.ora_f16_to_f32.argtypes = [P, P, C.c_size_t]
        L.ora_csum.restype = C.c_float
        L.ora_csum.argtypes = [P, P, C.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags.c_contiguous
    return a.ctypes.data_as(C.c_void_p)


class Cfg:
    """Oracle view of a layer: shape, storage options and per-unit widths."""

    def __init__(self, H, dk, dv, unit_keyrow, gate_vec, rscale_f16, cscale_f16,
                 window, comps, bits, scale_fit=0, row_impact=None):
        self.H, self.dk, self.dv = H, dk, dv
        self.unit_keyrow, self.gate_vec = bool(unit_keyrow), bool(gate_vec)
        self.window, self.comps = int(window), int(comps)
        self.scale_fit = int(scale_fit)
        self.bits = np.ascontiguousarray(bits, dtype=np.uint8)
        assert self.bits.size == (H * dk if unit_keyrow else H)
        self.row_impact = None if row_impact is None else np.ascontiguousarray(row_impact, dtype=np.float32)
        assert self.row_impact is None or self.row_impact.size == H * dk
        self._c = _Cfg(H, dk, dv, int(unit_keyrow), int(gate_vec), int(rscale_f16),
                       int(cscale_f16), int(window), int(comps), int(scale_fit),
                       self.bits.ctypes.data_as(C.POINTER(C.c_uint8)),
                       None if self.row_impact is None
                       else self.row_impact.ctypes.data_as(C.POINTER(C.c_float)))
        self.ptr = C.cast(C.pointer(self._c), C.c_void_p)
        self.slot_bytes = int(lib().ora_slot_bytes(self.ptr))

    @classmethod
    def from_workload(cls, w, bits, row_impact=None):
        return cls(w.H, w.dk, w.dv, w.unit == "keyrow", w.gate == "keyvec",
                   w.row_scale == "f16", w.col_scale == "f16", w.window, w.comps, bits,
                   scale_fit=1 if getattr(w, "scale_fit", "step") == "lagged" else 0,
                   row_impact=row_impact)

    def head_layout(self, h: int) -> dict:
        out = np.zeros(16, dtype=np.uint64)
        lib().ora_head_layout(self.ptr, h, _p(out))
        keys = ["base", "codes", "rs", "cs", "wn", "g", "cidx", "cval", "du", "dkap",
                "bytes", "nquant", "nrs", "ncs", "sr", "sc"]
        return {k: int(v) for k, v in zip(keys, out)}

    def new_slot(self) -> np.ndarray:
        s = np.zeros(self.slot_bytes, dtype=np.uint8)
        lib().ora_slot_init(self.ptr, _p(s))
        return s

    def unpack_head(self, slot: np.ndarray, h: int) -> np.ndarray:
        M = np.zeros((self.dk, self.dv), dtype=np.float32)
        lib().ora_unpack_head(self.ptr, h, _p(slot), _p(M))
        return M

    def pack_head(self, slot: np.ndarray, h: int, M: np.ndarray) -> None:
        M = np.ascontiguousarray(M, dtype=np.float32)
        assert M.shape == (self.dk, self.dv)
        lib().ora_pack_head(self.ptr, h, _p(slot), _p(M))

    def step_head(self, slot: np.ndarray, h: int, q, k, v, a, beta) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.float32)
        k = np.ascontiguousarray(k, dtype=np.float32)
        v = np.ascontiguousarray(v, dtype=np.float32)
        a = np.ascontiguousarray(np.atleast_1d(a), dtype=np.float32)
        assert q.shape == (self.dk,) and k.shape == (self.dk,) and v.shape == (self.dv,)
        assert a.size == (self.dk if self.gate_vec else 1)
        o = np.zeros(self.dv, dtype=np.float32)
        lib().ora_step_head(self.ptr, h, _p(slot), _p(q), _p(k), _p(v), _p(a),
                            float(np.float32(beta)), _p(o))
        return o


    def fit_head(self, slot: np.ndarray, h: int) -> None:
        """Lagged scales: the next scales of head h from its statistics."""
        lib().ora_fit_head(self.ptr, h, _p(slot))


def step_f32(M: np.ndarray, q, k, v, a, beta, gate_vec: bool) -> np.ndarray:
    """Unquantized fp32 step, M [dk, dv] updated in place; returns o."""
    assert M.dtype == np.float32 and M.flags.c_contiguous
    dk, dv = M.shape
    q, k, v = (np.ascontiguousarray(x, dtype=np.float32) for x in (q, k, v))
    a = np.ascontiguousarray(np.atleast_1d(a), dtype=np.float32)
    o = np.zeros(dv, dtype=np.float32)
    lib().ora_step_f32(dk, dv, int(gate_vec), _p(M), _p(q), _p(k), _p(v), _p(a),
                       float(np.float32(beta)), _p(o))
    return o


def step_f64(M: np.ndarray, q, k, v, a, beta, gate_vec: bool) -> np.ndarray:
    """Unquantized fp64 step, M [dk, dv] updated in place; returns o."""
    assert M.dtype == np.float64 and M.flags.c_contiguous
    dk, dv = M.shape
    q, k, v = (np.ascontiguousarray(x, dtype=np.float64) for x in (q, k, v))
    a = np.ascontiguousarray(np.atleast_1d(a), dtype=np.float64)
    o = np.zeros(dv, dtype=np.float64)
    lib().ora_step_f64(dk, dv, int(gate_vec), _p(M), _p(q), _p(k), _p(v), _p(a),
                       float(beta), _p(o))
    return o


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.zeros(x.shape, dtype=np.uint16)
    lib().ora_f32_to_f16(_p(x), _p(y), x.size)
    return y


def f16_to_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    y = np.zeros(x.shape, dtype=np.float32)
    lib().ora_f16_to_f32(_p(x), _p(y), x.size)
    return y


def csum(x, y) -> np.float32:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.ascontiguousarray(y, dtype=np.float32)
    return np.float32(lib().ora_csum(_p(x), _p(y), x.size))
