"""Seeded synthetic workloads for the quantized-state decode step.

This module is shared by the oracle driver and the HIP path, and by nothing
else of the method: it draws inputs and layer metadata and holds none of the
step's arithmetic (no dequantization, update, scale fitting or packing).

Random numbers come from SplitMix64 evaluated at a counter (Steele, Lea and
Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014; output
function "Mix13" by D. Stafford): element ``n`` of the stream with key ``s``
is ``mix(s + (n + 1) * 0x9E3779B97F4A7C15)``.  A unit's key is derived from
(seed, config, tensor, layer, step, request, head) by chaining ``mix``, so any
unit's inputs can be regenerated alone, without generating the batch.

Workloads follow the five decode settings of the state-quantization pages:
a tiny GDN check, a Qwen-like GDN layer with mixed 4/6/8-bit heads, a
Kimi-like KDA layer with per-key-row widths and heavy-tailed row/column
outliers, a B=512 serving pool over four layers, and the windowed 8-bit
variant (STEPQuant essay, results and kernel paragraphs; LeapQuant article,
"研究の概要").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# tensor ids of the stream keys
T_Q, T_K, T_V, T_GATE, T_BETA, T_INIT, T_LAYOUT, T_GATE_OFFSET, T_Q_SCALE = 1, 2, 3, 4, 5, 6, 7, 8, 9


def _mix(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def stream_key(*fields) -> np.ndarray:
    """Key of one stream; fields may be ints or broadcastable integer arrays."""
    k = np.zeros((), dtype=np.uint64)
    for f in fields:
        with np.errstate(over="ignore"):
            k = _mix((k ^ np.asarray(f, dtype=np.uint64)) + _GAMMA)
    return k


def raw(key: np.ndarray, n: int) -> np.ndarray:
    """First ``n`` SplitMix64 outputs of every key: shape key.shape + (n,)."""
    key = np.asarray(key, dtype=np.uint64)[..., None]
    ctr = np.arange(1, n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + ctr * _GAMMA)


def uniform(key, n: int) -> np.ndarray:
    """Doubles in (0, 1]: top 53 bits of each output, plus one ulp."""
    return ((raw(key, n) >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53


def normal(key, n: int) -> np.ndarray:
    """Standard normals by Box-Muller (cosine branch) on output pairs."""
    u = uniform(key, 2 * n)
    u1, u2 = u[..., 0::2], u[..., 1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16, nearest-even; returns the uint16 patterns."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = ((b >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return ((b + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- configs

@dataclass(frozen=True)
class Workload:
    name: str
    cid: int                 # config id in stream keys
    B: int
    H: int
    dk: int
    dv: int
    T: int
    unit: str                # "head" (GDN) | "keyrow" (KDA)
    gate: str                # "scalar" | "keyvec"
    row_scale: str           # "f32" | "f16"
    col_scale: str           # "none" | "f16"
    io: str                  # "f32" | "bf16"
    bits: str                # "uniform6" | "uniform8" | "avg4" | "avg6"
    pivot_frac: float
    init: str                # "zero" | "outlier"
    window: int = 1
    comps: int = 0
    layers: int = 1
    seed: int = 0
    desc: str = ""
    scale_fit: str = "step"  # "step" (refit inside each step) | "lagged" (fitted apart)
    gate_spread: float = 0.0  # KDA: per key row fixed offset U(-spread, spread) of the gate's N(2, 1)
    query_spread: float = 0.0  # per key channel fixed query scale exp(spread N(0,1)) before normalizing
    impact: str = "none"       # "none" | "queries": row-impact scores E[q_i^2] from calibration queries

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny_gdn": Workload(
        "tiny_gdn", 1, B=4, H=2, dk=64, dv=64, T=16, unit="head", gate="scalar",
        row_scale="f32", col_scale="none", io="f32", bits="uniform6", pivot_frac=0.0,
        init="zero", desc="GDN B=4 H=2 d=64 T=16, uniform 6-bit, fp32 row scale"),
    "qwen_gdn": Workload(
        "qwen_gdn", 2, B=64, H=32, dk=128, dv=128, T=256, unit="head", gate="scalar",
        row_scale="f16", col_scale="f16", io="bf16", bits="avg6", pivot_frac=0.02,
        init="zero", desc="GDN B=64 H=32 d=128 T=256, per-head {4,6,8} avg 6, 2% fp16 pivots"),
    "kimi_kda": Workload(
        "kimi_kda", 3, B=256, H=32, dk=128, dv=128, T=256, unit="keyrow", gate="keyvec",
        row_scale="f16", col_scale="f16", io="bf16", bits="avg4", pivot_frac=0.01,
        init="outlier", desc="KDA B=256 H=32 d=128 T=256, per-key-row avg 4 bit, 1% pivot rows"),
    "serving_gdn": Workload(
        "serving_gdn", 4, B=512, H=32, dk=128, dv=128, T=2048, unit="head", gate="scalar",
        row_scale="f16", col_scale="f16", io="bf16", bits="avg4", pivot_frac=0.02,
        init="zero", layers=4, desc="GDN pool B=512 H=32 d=128 L=4, avg 4 bit, 2% fp16 pivot heads"),
    "serving_fp32": Workload(
        "serving_fp32", 6, B=512, H=32, dk=128, dv=128, T=2048, unit="head", gate="scalar",
        row_scale="f16", col_scale="f16", io="bf16", bits="fp32", pivot_frac=0.0,
        init="zero", layers=4,
        desc="the serving shape with fp32 (unquantized) state: the comparison point"),
    "serving_int8": Workload(
        "serving_int8", 7, B=512, H=32, dk=128, dv=128, T=2048, unit="head", gate="scalar",
        row_scale="f16", col_scale="f16", io="bf16", bits="uniform8", pivot_frac=0.0,
        init="zero", layers=4, desc="the serving shape with uniform 8-bit heads"),
    "serving_int6": Workload(
        "serving_int6", 8, B=512, H=32, dk=128, dv=128, T=2048, unit="head", gate="scalar",
        row_scale="f16", col_scale="f16", io="bf16", bits="uniform6", pivot_frac=0.0,
        init="zero", layers=4, desc="the serving shape with uniform 6-bit heads"),
    "serving_lagged": Workload(
        "serving_lagged", 9, B=512, H=32, dk=128, dv=128, T=2048, unit="head", gate="scalar",
        row_scale="f16", col_scale="f16", io="bf16", bits="avg4", pivot_frac=0.02,
        init="zero", layers=4, scale_fit="lagged",
        desc="the serving pool with lagged scales (written with the previous state's fit)"),
    "kimi_serving": Workload(
        "kimi_serving", 12, B=512, H=32, dk=128, dv=128, T=256, unit="keyrow", gate="keyvec",
        row_scale="f16", col_scale="f16", io="bf16", bits="avg4", pivot_frac=0.01,
        init="outlier", layers=4,
        desc="the KDA layer at serving scale: B=512, four layers (1.3 GB of state, beyond the "
             "256 MB last-level cache), per-key-row avg 4 bit, 1% pivot rows"),
    "kda_lifetimes": Workload(
        "kda_lifetimes", 10, B=256, H=32, dk=128, dv=128, T=256, unit="keyrow", gate="keyvec",
        row_scale="f16", col_scale="f16", io="bf16", bits="allocated", pivot_frac=0.01,
        init="outlier", gate_spread=3.0,
        desc="KDA B=256 H=32 d=128 T=256, key rows of different lifetimes (fixed per-row "
             "gate offsets), widths from a calibration pass and the lifetime-aware allocation "
             "(mean 6 bits, 1% pivot rows)"),
    "kimi_impact": Workload(
        "kimi_impact", 11, B=256, H=32, dk=128, dv=128, T=256, unit="keyrow", gate="keyvec",
        row_scale="f16", col_scale="f16", io="bf16", bits="avg4", pivot_frac=0.01,
        init="outlier", query_spread=1.0, impact="queries",
        desc="the KDA layer with queries of unequal weight per key channel and row-impact "
             "scores E[q_i^2] from calibration queries (impact-weighted column scales)"),
    "windowed_kda": Workload(
        "windowed_kda", 5, B=512, H=32, dk=128, dv=128, T=1024, unit="keyrow", gate="keyvec",
        row_scale="f16", col_scale="f16", io="bf16", bits="uniform8", pivot_frac=0.0,
        init="outlier", window=16, comps=82,
        desc="KDA B=512 H=32 d=128 T=1024, uniform 8 bit, requantize every 16 tokens, 82 fp32 comps"),
}


# --------------------------------------------------------- layer metadata

def _perm(key, n: int) -> np.ndarray:
    """Seeded permutation of range(n): order of n stream outputs."""
    return np.argsort(raw(key, n), kind="stable")


def unit_bits(w: Workload, layer: int = 0) -> np.ndarray:
    """Per-unit widths in {4,6,8,16,32}: one per head (GDN) or per (head, key row) (KDA).

    16 marks an FP16 pivot unit, 32 an fp32 (unquantized) unit.  The pivot count is max(1, round(frac * units))
    when frac > 0.  Non-pivot widths follow the maximum-entropy split over
    {4,6,8} with the stated mean: mean 6 gives equal thirds (remainder to 6),
    mean 4 can only be met by all-4.
    """
    n = w.H if w.unit == "head" else w.H * w.dk
    bits = np.zeros(n, dtype=np.uint8)
    order = _perm(stream_key(w.seed, w.cid, T_LAYOUT, layer, 0), n)
    npiv = max(1, int(round(w.pivot_frac * n))) if w.pivot_frac > 0 else 0
    piv, rest = order[:npiv], order[npiv:]
    bits[piv] = 16
    m = len(rest)
    if w.bits == "uniform6":
        bits[rest] = 6
    elif w.bits in ("uniform8",):
        bits[rest] = 8
    elif w.bits == "fp32":
        bits[rest] = 32
    elif w.bits == "avg4":
        bits[rest] = 4
    elif w.bits == "allocated":
        raise ValueError(f"{w.name}: widths come from a calibration pass and the bit allocation, "
                         "not from the workload")
    elif w.bits == "avg6":
        n4 = n8 = m // 3
        n6 = m - n4 - n8
        wid = np.array([4] * n4 + [6] * n6 + [8] * n8, dtype=np.uint8)
        shuf = _perm(stream_key(w.seed, w.cid, T_LAYOUT, layer, 1), m)
        bits[rest] = wid[shuf]
    else:
        raise ValueError(w.bits)
    return bits


# ----------------------------------------------------------- step inputs

@dataclass
class StepInputs:
    """Inputs of one decode step for a set of units, as fp32 values.

    For bf16 workloads the fp32 values are exactly the bf16 values, and
    ``*_bits`` hold the bf16 patterns the device consumes.
    """
    q: np.ndarray        # [..., dk]
    k: np.ndarray        # [..., dk]
    v: np.ndarray        # [..., dv]
    a: np.ndarray        # [...] (scalar gate) or [..., dk]
    beta: np.ndarray     # [...]
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None


def _softplus(x):
    return np.where(x > 30, x, np.log1p(np.exp(np.minimum(x, 30))))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def step_inputs(w: Workload, layer: int, t: int, b, h) -> StepInputs:
    """Inputs at step ``t`` for request(s) ``b`` and head(s) ``h`` (broadcast)."""
    b = np.asarray(b, dtype=np.int64)
    h = np.asarray(h, dtype=np.int64)
    b, h = np.broadcast_arrays(b, h)
    key = lambda tensor: stream_key(w.seed, w.cid, tensor, layer, t, b, h)
    q = normal(key(T_Q), w.dk)
    if w.query_spread:
        q = q * query_scales(w, layer, h)
    k = normal(key(T_K), w.dk)
    v = normal(key(T_V), w.dv)
    q = q / np.linalg.norm(q, axis=-1, keepdims=True)
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    if w.gate == "scalar":
        x = normal(key(T_GATE), 1)[..., 0]
        a = np.exp(-_softplus(x) * 0.1).astype(np.float32)
    else:
        y = normal(key(T_GATE), w.dk) + 2.0 + gate_offsets(w, layer, h)
        a = (0.8 + 0.2 * _sigmoid(y)).astype(np.float32)
    beta = _sigmoid(normal(key(T_BETA), 1)[..., 0]).astype(np.float32)
    q32, k32, v32 = (x.astype(np.float32) for x in (q, k, v))
    if w.io == "bf16":
        qb, kb, vb = to_bf16_bits(q32), to_bf16_bits(k32), to_bf16_bits(v32)
        return StepInputs(bf16_bits_to_f32(qb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb),
                          a, beta, qb, kb, vb)
    return StepInputs(q32, k32, v32, a, beta)


def query_scales(w: Workload, layer: int, h) -> np.ndarray:
    """Fixed per-key-channel query scale exp(spread * N(0,1)), one per
    (layer, head, channel), applied before the query is normalized: some key
    rows are read far more than others.  [..., d_k]"""
    h = np.asarray(h, dtype=np.int64)
    return np.exp(w.query_spread * normal(stream_key(w.seed, w.cid, T_Q_SCALE, layer, 0, h), w.dk))


def gate_offsets(w: Workload, layer: int, h) -> np.ndarray:
    """Fixed per-key-row offset of the KDA gate's normal, U(-spread, spread),
    one per (layer, head, row): rows with a large offset forget slowly (long
    lifetime), rows with a negative one quickly.  [..., d_k] (zeros when the
    workload has no spread)."""
    h = np.asarray(h, dtype=np.int64)
    if w.gate_spread == 0.0:
        return np.zeros(h.shape + (w.dk,))
    u = uniform(stream_key(w.seed, w.cid, T_GATE_OFFSET, layer, 0, h), w.dk)
    return w.gate_spread * (2.0 * u - 1.0)


def batch_inputs(w: Workload, layer: int, t: int) -> StepInputs:
    """Inputs of all B x H units at step t (arrays [B, H, ...])."""
    bb, hh = np.meshgrid(np.arange(w.B), np.arange(w.H), indexing="ij")
    return step_inputs(w, layer, t, bb, hh)


def initial_state(w: Workload, layer: int, b, h) -> np.ndarray:
    """fp32 initial state M = S^T [..., dk, dv] for the given units.

    "zero": all zeros.  "outlier": base entries N(0, 0.1^2); five seeded key
    rows and five value columns are replaced by heavy-tailed outliers of
    magnitude 20 x median|base| x |t3| / median|t3| with random sign, drawn
    once per entry (row/column intersections are not doubled).
    """
    b = np.asarray(b, dtype=np.int64)
    h = np.asarray(h, dtype=np.int64)
    b, h = np.broadcast_arrays(b, h)
    shape = b.shape + (w.dk, w.dv)
    if w.init == "zero":
        return np.zeros(shape, dtype=np.float32)
    n = w.dk * w.dv
    key = stream_key(w.seed, w.cid, T_INIT, layer, 0, b, h)
    base = 0.1 * normal(key, n)
    med = np.median(np.abs(base), axis=-1, keepdims=True)
    # Student-t(3): Z / sqrt(chi2_3 / 3); four normals per entry
    z = normal(stream_key(key, 1), 4 * n).reshape(b.shape + (n, 4))
    t3 = z[..., 0] / np.sqrt((z[..., 1:] ** 2).sum(-1) / 3.0)
    med_t3 = 0.7648923284  # median of |t_3|
    sign = np.where(uniform(stream_key(key, 2), n) < 0.5, -1.0, 1.0)
    out_val = 20.0 * med * (np.abs(t3) / med_t3) * sign
    sel = raw(stream_key(key, 3), w.dk + w.dv)
    rows = np.argsort(sel[..., : w.dk], axis=-1, kind="stable")[..., :5]
    cols = np.argsort(sel[..., w.dk:], axis=-1, kind="stable")[..., :5]
    mask = np.zeros(b.shape + (w.dk, w.dv), dtype=bool)
    flat_mask = mask.reshape(-1, w.dk, w.dv)
    r2 = rows.reshape(-1, 5)
    c2 = cols.reshape(-1, 5)
    for u in range(flat_mask.shape[0]):
        flat_mask[u, r2[u], :] = True
        flat_mask[u, :, c2[u]] = True
    M = np.where(mask.reshape(b.shape + (n,)), out_val, base)
    return M.reshape(shape).astype(np.float32)
