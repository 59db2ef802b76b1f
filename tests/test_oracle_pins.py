"""Pins of the CPU oracle against facts fixed outside it: IEEE fp16 rounding,
exact arithmetic, textbook closed forms of the delta rule, Proposition 1 of
the STEPQuant essay, brute-force quantization, the storage accounting the
essay prints, and brute-force top-K.  None of these re-types the oracle's
formulas; each is chosen so that a plausible mistake (a dropped term, a wrong
sign, a transposed operand, a wrong bit position) fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import synth
from tests import slotcodec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")


def _cfg(ora, H=1, dk=16, dv=16, keyrow=False, gate_vec=False, rf16=True, cf16=True,
         window=1, comps=0, bits=None, width=8):
    if bits is None:
        bits = np.full(H * dk if keyrow else H, width, dtype=np.uint8)
    return ora.Cfg(H, dk, dv, keyrow, gate_vec, rf16, cf16, window, comps, bits)


# ------------------------------------------------------------ fp16 rounding

def test_fp16_matches_ieee_nearest_even(ora):
    """Strided sweep of all float32 patterns plus every pattern next to an fp16
    rounding boundary, against numpy's IEEE half conversion."""
    rng = np.random.default_rng(0)
    pats = [np.arange(0, 2 ** 32, 9973, dtype=np.uint64).astype(np.uint32)]
    # patterns whose low 13 mantissa bits sit at / beside the half-way point
    hi = rng.integers(0, 2 ** 19, size=200_000, dtype=np.uint64) << np.uint64(13)
    for low in (0x0FFF, 0x1000, 0x1001, 0x0000, 0x1FFF):
        pats.append((hi | np.uint64(low)).astype(np.uint32))
    # subnormal fp16 region and overflow edge
    pats.append(np.arange(0x33000000, 0x38900000, 37, dtype=np.uint32))
    pats.append(np.arange(0x477FE000, 0x47800100, 1, dtype=np.uint32))
    x = np.concatenate(pats).view(np.float32)
    x = x[np.isfinite(x)]
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = ora.f32_to_f16(x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (x[bad[:5]], got[bad[:5]], want[bad[:5]])
    back = ora.f16_to_f32(np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16))
    ref = np.arange(0, 2 ** 16, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)
    same = (back == ref) | (np.isnan(back) & np.isnan(ref))
    assert same.all()


# ------------------------------------------------------------ canonical sum

def test_csum_exact_on_integers(ora):
    """With small integer terms every partial sum is exact, so the canonical sum
    must equal the exact dot product (a dropped or doubled term fails)."""
    rng = np.random.default_rng(1)
    for n in (8, 16, 64, 128):
        for _ in range(50):
            x = rng.integers(-300, 300, n).astype(np.float32)
            y = rng.integers(-300, 300, n).astype(np.float32)
            assert float(ora.csum(x, y)) == float(np.dot(x.astype(np.int64), y.astype(np.int64)))


def test_csum_error_bound(ora):
    """|csum - exact| <= n * 2^-24 * sum|x y| (standard dot-product bound)."""
    rng = np.random.default_rng(2)
    for n in (64, 128):
        for _ in range(200):
            x = rng.standard_normal(n).astype(np.float32)
            y = rng.standard_normal(n).astype(np.float32)
            exact = np.dot(x.astype(np.float64), y.astype(np.float64))
            bound = n * 2.0 ** -24 * np.sum(np.abs(x.astype(np.float64) * y))
            assert abs(float(ora.csum(x, y)) - exact) <= bound


# ------------------------------------------------- unquantized closed forms

def _orthonormal(rng, d, n):
    q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return q[:, :n].T  # n orthonormal rows


@pytest.mark.parametrize("prec", ["f64", "f32"])
def test_delta_rule_retrieval_closed_form(ora, prec):
    """a = 1, beta = 1, orthonormal keys: after writing (k_m, v_m), reading with
    q = k_m returns v_m exactly (delta-rule associative memory)."""
    rng = np.random.default_rng(3)
    dk, dv, n = 32, 24, 12
    keys = _orthonormal(rng, dk, n)
    vals = rng.standard_normal((n, dv))
    dt = np.float64 if prec == "f64" else np.float32
    step = ora.step_f64 if prec == "f64" else ora.step_f32
    M = np.zeros((dk, dv), dtype=dt)
    for m in range(n):
        step(M, keys[m].astype(dt), keys[m].astype(dt), vals[m].astype(dt), np.ones(1), 1.0, False)
    tol = 1e-12 if prec == "f64" else 2e-5
    for m in range(n):
        o = step(M.copy(), keys[m].astype(dt), np.zeros(dk, dt), np.zeros(dv, dt), np.ones(1), 0.0, False)
        np.testing.assert_allclose(o, vals[m], atol=tol, rtol=0)


def test_gated_retrieval_closed_form(ora):
    """Scalar gates a_t: reading key k_m after step T gives prod_{s>m} a_s * v_m."""
    rng = np.random.default_rng(4)
    dk, dv, n = 16, 8, 10
    keys = _orthonormal(rng, dk, n)
    vals = rng.standard_normal((n, dv))
    gates = rng.uniform(0.7, 1.0, n)
    M = np.zeros((dk, dv))
    for m in range(n):
        ora.step_f64(M, keys[m], keys[m], vals[m], gates[m:m + 1], 1.0, False)
    for m in range(n):
        o = ora.step_f64(M.copy(), keys[m], np.zeros(dk), np.zeros(dv), np.ones(1), 0.0, False)
        np.testing.assert_allclose(o, np.prod(gates[m + 1:]) * vals[m], atol=1e-12, rtol=0)


def test_keyvec_gate_one_hot_keys(ora):
    """KDA gate on one-hot keys: each key row decays by its own gate product,
    and a repeated key overwrites (beta = 1)."""
    rng = np.random.default_rng(5)
    dk, dv = 8, 6
    seq = [3, 5, 1, 3]
    vals = rng.standard_normal((len(seq), dv))
    gates = rng.uniform(0.8, 1.0, (len(seq), dk))
    M = np.zeros((dk, dv))
    for t, i in enumerate(seq):
        e = np.eye(dk)[i]
        ora.step_f64(M, e, e, vals[t], gates[t], 1.0, True)
    # row 3 was overwritten at the last step; rows 5 and 1 decayed since written
    np.testing.assert_allclose(M[3], vals[3], atol=1e-12)
    np.testing.assert_allclose(M[5], vals[1] * gates[2, 5] * gates[3, 5], atol=1e-12)
    np.testing.assert_allclose(M[1], vals[2] * gates[3, 1], atol=1e-12)
    assert np.all(M[[0, 2, 4, 6, 7]] == 0)


def test_f32_path_tracks_f64(ora):
    rng = np.random.default_rng(6)
    dk = dv = 64
    M32 = np.zeros((dk, dv), np.float32)
    M64 = np.zeros((dk, dv))
    for t in range(64):
        k = rng.standard_normal(dk); k /= np.linalg.norm(k)
        q = rng.standard_normal(dk); q /= np.linalg.norm(q)
        v = rng.standard_normal(dv)
        a = rng.uniform(0.8, 1.0, dk)
        b = rng.uniform(0.2, 0.9)
        k, q, v, a = (x.astype(np.float32).astype(np.float64) for x in (k, q, v, a))
        b = float(np.float32(b))
        o32 = ora.step_f32(M32, q, k, v, a, b, True)
        o64 = ora.step_f64(M64, q, k, v, a, b, True)
        assert np.max(np.abs(o32 - o64)) <= 1e-5 * max(1.0, np.max(np.abs(o64)))


# ------------------------------------------------------------ Proposition 1

@pytest.mark.parametrize("gate_vec", [False, True])
def test_prop1_misaligned_error_decays_by_gates_only(ora, gate_vec):
    """Error in rows orthogonal to every key is only scaled by the gates:
    E_T = diag(prod a) E_0 (the state update is linear in M)."""
    rng = np.random.default_rng(7)
    dk, dv, T = 16, 12, 20
    M = rng.standard_normal((dk, dv))
    E0 = np.zeros((dk, dv))
    E0[12:] = rng.standard_normal((4, dv))      # rows 12..15
    Me = M + E0
    gprod = np.ones(dk)
    for t in range(T):
        k = np.zeros(dk); k[:12] = rng.standard_normal(12); k /= np.linalg.norm(k)
        q = rng.standard_normal(dk)
        v = rng.standard_normal(dv)
        a = rng.uniform(0.8, 1.0, dk if gate_vec else 1)
        beta = rng.uniform(0.1, 1.0)
        ora.step_f64(M, q, k, v, a, beta, gate_vec)
        ora.step_f64(Me, q, k, v, a, beta, gate_vec)
        gprod *= a if gate_vec else a[0]
    np.testing.assert_allclose(Me - M, gprod[:, None] * E0, atol=1e-12, rtol=0)


def test_prop1_aligned_error_removed(ora):
    """Error aligned with the incoming key (E = k e^T) is scaled by
    a(1 - beta |k|^2): removed for beta = 1, kept otherwise."""
    rng = np.random.default_rng(8)
    dk, dv = 16, 8
    for beta in (1.0, 0.3):
        M = rng.standard_normal((dk, dv))
        k = rng.standard_normal(dk); k /= np.linalg.norm(k)
        e = rng.standard_normal(dv)
        Me = M + np.outer(k, e)
        q, v = rng.standard_normal(dk), rng.standard_normal(dv)
        a = np.array([0.9])
        ora.step_f64(M, q, k, v, a, beta, False)
        ora.step_f64(Me, q, k, v, a, beta, False)
        np.testing.assert_allclose(Me - M, 0.9 * (1 - beta) * np.outer(k, e), atol=1e-12)


# ------------------------------------------------------ storage and quantizer

def _random_head(rng, widths, dv, rf16=True):
    dk = len(widths)
    n = np.zeros((dk, dv), np.int64)
    hv = np.zeros((dk, dv), np.uint16)
    for i, b in enumerate(int(x) for x in widths):
        if b == 16:
            hv[i] = rng.standard_normal(dv).astype(np.float16).view(np.uint16)
        else:
            qm = (1 << (b - 1)) - 1
            n[i] = rng.integers(-qm, qm + 1, dv)
    r = rng.uniform(0.01, 2.0, dk)
    r = r.astype(np.float16).astype(np.float32) if rf16 else r.astype(np.float32)
    r[np.asarray(widths) == 16] = 0
    c = rng.uniform(0.05, 3.0, dv).astype(np.float16).astype(np.float32)
    return n, hv, r, c


@pytest.mark.parametrize("keyrow", [False, True])
def test_unpack_reads_the_stated_format(ora, keyrow):
    """A head written by the test's own bit packer must dequantize to
    RN(n r c) (exact product in fp64, then one rounding) and pivots to their
    fp16 values: pins bit order, offset-binary codes and section offsets."""
    rng = np.random.default_rng(9)
    dk, dv, H = 16, 16, 3
    if keyrow:
        bits = rng.choice(np.array([4, 6, 8, 16], np.uint8), H * dk)
    else:
        bits = np.array([4, 6, 8], np.uint8)
    cfg = _cfg(ora, H=H, dk=dk, dv=dv, keyrow=keyrow, bits=bits)
    slot = cfg.new_slot()
    for h in range(H):
        widths = bits[h * dk:(h + 1) * dk] if keyrow else np.full(dk, bits[h])
        n, hv, r, c = _random_head(rng, widths, dv)
        lay = cfg.head_layout(h)
        slotcodec.write_head(slot, lay, widths, n, hv, r, c, True, True)
        M = cfg.unpack_head(slot, h)
        want = (n * r[:, None].astype(np.float64) * c[None, :].astype(np.float64)).astype(np.float32)
        piv = widths == 16
        want[piv] = hv[piv].view(np.float16).astype(np.float32)
        assert np.array_equal(M, want)


# The two scale kinds: fp16 row and column scales (the dual-axis fit), and an
# fp32 row scale with no column scale (the tiny GDN configuration).
SCALES = {"f16": (True, True), "f32_rows_only": (False, False)}


@pytest.mark.parametrize("scales", list(SCALES))
@pytest.mark.parametrize("width", [4, 6, 8])
def test_pack_matches_bruteforce_quantizer(ora, width, scales):
    """For the scales the oracle fits, each code is the nearest level
    argmin_n |M - n r c| except where M/(r c) sits within 1e-5 of a half level;
    no error exceeds half a step; every row reaches +-qmax (normal fp16 scales,
    or fp32 row scales); every column's scale bounds its largest entry; with
    fp32 row scales and no column scale the step of row i is max_j |M_ij| /
    qmax to fp32 rounding."""
    rf16, cf16 = SCALES[scales]
    rng = np.random.default_rng(10 + width)
    dk = dv = 32
    cfg = _cfg(ora, dk=dk, dv=dv, width=width, rf16=rf16, cf16=cf16)
    qm = (1 << (width - 1)) - 1
    for trial in range(10):
        M = (rng.standard_normal((dk, dv)) * rng.uniform(0.1, 3, dk)[:, None]
             * rng.uniform(0.1, 3, dv)[None, :]).astype(np.float32)
        slot = cfg.new_slot()
        cfg.pack_head(slot, 0, M)
        n, _, r, c = slotcodec.read_head(slot, cfg.head_layout(0), np.full(dk, width), dk, dv, rf16, cf16)
        if not cf16:
            assert np.all(c == 1.0)
            want = np.abs(M.astype(np.float64)).max(axis=1) / qm
            assert np.all(np.abs(r / want - 1) <= 2.0 ** -23)
        step = r[:, None].astype(np.float64) * c[None, :]
        x = M / step
        levels = np.arange(-qm, qm + 1)
        brute = levels[np.argmin(np.abs(x[..., None] - levels), axis=-1)]
        near_half = np.abs(np.abs(x - np.floor(x)) - 0.5) < 1e-5
        assert np.all((n == brute) | near_half)
        assert np.all(np.abs(M - n * step) <= 0.5 * step * (1 + 1e-5))
        assert np.all(np.abs(n).max(axis=1) == qm)
        if cf16:
            assert np.all(c >= np.abs(M).max(axis=0) * (1 - 2 ** -10))


@pytest.mark.parametrize("width", [4, 6, 8])
def test_requantize_of_dequantize_is_idempotent(ora, width):
    """pack(unpack(Q)) keeps every code; scales move by at most 2 fp16 ulp."""
    rng = np.random.default_rng(20 + width)
    dk = dv = 32
    cfg = _cfg(ora, dk=dk, dv=dv, width=width)
    for trial in range(10):
        M = rng.standard_normal((dk, dv)).astype(np.float32)
        s1 = cfg.new_slot()
        cfg.pack_head(s1, 0, M)
        s2 = cfg.new_slot()
        cfg.pack_head(s2, 0, cfg.unpack_head(s1, 0))
        lay = cfg.head_layout(0)
        n1, _, r1, c1 = slotcodec.read_head(s1, lay, np.full(dk, width), dk, dv, True, True)
        n2, _, r2, c2 = slotcodec.read_head(s2, lay, np.full(dk, width), dk, dv, True, True)
        assert np.array_equal(n1, n2)
        ulp = lambda x: np.abs(x.astype(np.float16).view(np.int16).astype(np.int64))
        assert np.max(np.abs(ulp(r1) - ulp(r2))) <= 2
        assert np.max(np.abs(ulp(c1) - ulp(c2))) <= 2


def test_pivot_rows_do_not_set_column_scales(ora):
    """FP16 pivot key rows are stored raw, so their (here 100x larger) entries
    must not widen the column scales of the quantized rows."""
    rng = np.random.default_rng(11)
    dk = dv = 16
    bits = np.full(dk, 8, np.uint8)
    bits[[2, 9]] = 16
    cfg = _cfg(ora, dk=dk, dv=dv, keyrow=True, bits=bits)
    M = rng.standard_normal((dk, dv)).astype(np.float32)
    M[[2, 9]] *= 100
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, M)
    n, hv, r, c = slotcodec.read_head(slot, cfg.head_layout(0), bits, dk, dv, True, True)
    cmax = np.abs(np.delete(M, [2, 9], axis=0)).max(axis=0)
    assert np.all(np.abs(c / cmax - 1) <= 2 ** -11)
    assert np.array_equal(hv[[2, 9]], M[[2, 9]].astype(np.float16).view(np.uint16))
    assert np.all(r[[2, 9]] == 0)


def test_row_step_rounds_up_and_never_clips(ora):
    """The row step is the smallest fp16 not below absmax/qmax, so every
    |M/(r c)| stays within qmax + 1/2 and no code clips (checked against
    numpy's half rounding); this also pins the step to absmax/qmax."""
    rng = np.random.default_rng(12)
    dk = dv = 32
    for width in (4, 6, 8):
        qm = (1 << (width - 1)) - 1
        cfg = _cfg(ora, dk=dk, dv=dv, width=width)
        for trial in range(10):
            M = (rng.standard_normal((dk, dv)) * rng.uniform(1e-3, 10, dk)[:, None]).astype(np.float32)
            slot = cfg.new_slot()
            cfg.pack_head(slot, 0, M)
            n, _, r, c = slotcodec.read_head(slot, cfg.head_layout(0), np.full(dk, width), dk, dv, True, True)
            Z = (M.astype(np.float64) / c[None, :].astype(np.float64))
            need = np.abs(Z).max(axis=1) / qm
            assert np.all(r >= need * (1 - 2 ** -22))                  # not below absmax/qmax
            below = np.nextafter(r.astype(np.float16), np.float16(0)).astype(np.float64)
            assert np.all((below < need * (1 + 2 ** -22)) | (r == 0))   # the smallest such fp16
            assert np.all(np.abs(M / (r[:, None].astype(np.float64) * c[None, :])) <= qm + 0.5)


def test_zero_state_gives_zero_codes_and_scales(ora):
    cfg = _cfg(ora, dk=16, dv=16, width=4)
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, np.zeros((16, 16), np.float32))
    n, _, r, c = slotcodec.read_head(slot, cfg.head_layout(0), np.full(16, 4), 16, 16, True, True)
    assert np.all(n == 0) and np.all(r == 0) and np.all(c == 0)


def test_fp16_scale_saturates(ora):
    """Entries beyond the fp16 range give a finite column scale of 65504."""
    cfg = _cfg(ora, dk=8, dv=8, width=8)
    M = np.ones((8, 8), np.float32)
    M[0, 0] = 1e6
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, M)
    _, _, _, c = slotcodec.read_head(slot, cfg.head_layout(0), np.full(8, 8), 8, 8, True, True)
    assert c[0] == 65504.0 and np.all(np.isfinite(c))


# --------------------------------------------------------- storage accounting

def test_storage_accounting_matches_pages(ora):
    """6-bit STEPQuant with fp16 row+column scales at d=128 and 1.39% FP16 pivot
    heads compresses the fp32 state about 5.03x (essay); the layout must land
    within 1% of that (appendix D with the exact format is not on the pages)."""
    g = json.load(open(GOLDEN))
    H = 72  # 1 pivot head of 72 = 1.39%
    bits = np.full(H, 6, np.uint8)
    bits[0] = 16
    assert abs(1 / H - g["pivot_head_fraction_qwen"]["value"]) < 1e-4
    cfg = _cfg(ora, H=H, dk=128, dv=128, bits=bits)
    ratio = H * 128 * 128 * 4 / cfg.slot_bytes
    assert abs(ratio / g["compression_6bit_qwen"]["value"] - 1) < 0.01
    # KDA: 6-bit key rows, about 1% pivot rows
    Hk = 32
    kb = np.full(Hk * 128, 6, np.uint8)
    kb[np.arange(0, Hk * 128, 100)] = 16
    cfgk = _cfg(ora, H=Hk, dk=128, dv=128, keyrow=True, bits=kb)
    rk = Hk * 128 * 128 * 4 / cfgk.slot_bytes
    assert abs(rk / g["compression_6bit_kimi"]["value"] - 1) < 0.02


def test_serving_pool_size(ora):
    """B=512, H=32, d=128, 31 four-bit heads and one fp16 pivot head, four
    layers: 4 x 512 x (31 x (8192+256+256) + 32768) bytes, against fp32."""
    w = synth.WORKLOADS["serving_gdn"]
    cfg = ora.Cfg.from_workload(w, synth.unit_bits(w))
    assert cfg.slot_bytes == 31 * 8704 + 32768
    pool = w.layers * w.B * cfg.slot_bytes
    fp32 = w.layers * w.B * w.H * 128 * 128 * 4
    assert abs(pool / 1e9 - 0.62) < 0.01 and abs(fp32 / 1e9 - 4.29) < 0.01


# --------------------------------------------------- quantized vs unquantized

@pytest.mark.parametrize("width,tol", [(16, 2e-3), (8, 3e-2)])
def test_quantized_step_tracks_fp64(ora, width, tol):
    """Every-step requantization at 8 bits (and fp16 pivots) stays close to the
    exact recurrence over 32 steps: catches misplaced scales or gates."""
    rng = np.random.default_rng(30 + width)
    dk = dv = 32
    for gate_vec in (False, True):
        cfg = _cfg(ora, dk=dk, dv=dv, keyrow=gate_vec, gate_vec=gate_vec, width=width)
        slot = cfg.new_slot()
        M = np.zeros((dk, dv))
        for t in range(32):
            k = rng.standard_normal(dk); k /= np.linalg.norm(k)
            q = rng.standard_normal(dk); q /= np.linalg.norm(q)
            v = rng.standard_normal(dv)
            a = rng.uniform(0.85, 1.0, dk if gate_vec else 1)
            b = rng.uniform(0.3, 1.0)
            k, q, v, a = (x.astype(np.float32) for x in (k, q, v, a))
            o = cfg.step_head(slot, 0, q, k, v, a, b)
            o64 = ora.step_f64(M, q, k, v, a, float(np.float32(b)), gate_vec)
            assert np.max(np.abs(o - o64)) <= tol * np.max(np.abs(o64))


@pytest.mark.parametrize("scales", list(SCALES))
@pytest.mark.parametrize("width", [4, 6, 8])
@pytest.mark.parametrize("kda", [False, True])
def test_quantized_step_injects_at_most_half_a_step(ora, width, kda, scales):
    """Each quantized step is the exact (fp64) gated delta-rule step of the
    previously stored state plus a quantization injection of at most half a
    step r'_i c'_j per entry (half an fp16 ulp on pivot rows), and o is the
    exact output of the updated state before requantization, to fp32
    rounding.  Element by element this pins the update (sign, orientation,
    gate placement), the dequantization scales, that o uses the updated state,
    and rounding to nearest."""
    rf16, cf16 = SCALES[scales]
    rng = np.random.default_rng(40 + width + 7 * kda)
    dk = dv = 32
    if kda:
        bits = np.full(dk, width, np.uint8)
        bits[[3, 20]] = 16
        cfg = _cfg(ora, dk=dk, dv=dv, keyrow=True, gate_vec=True, bits=bits, rf16=rf16, cf16=cf16)
    else:
        bits = np.full(dk, width, np.uint8)
        cfg = _cfg(ora, dk=dk, dv=dv, width=width, rf16=rf16, cf16=cf16)
    piv = bits == 16
    lay = cfg.head_layout(0)
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, (rng.standard_normal((dk, dv)) * 0.5).astype(np.float32))
    for t in range(24):
        prev = cfg.unpack_head(slot, 0).astype(np.float64)
        k = rng.standard_normal(dk); k /= np.linalg.norm(k)
        q = rng.standard_normal(dk); q /= np.linalg.norm(q)
        v = rng.standard_normal(dv)
        a = rng.uniform(0.85, 1.0, dk if kda else 1)
        b = rng.uniform(0.3, 1.0)
        k, q, v, a = (x.astype(np.float32) for x in (k, q, v, a))
        o = cfg.step_head(slot, 0, q, k, v, a, b)
        exact = prev.copy()
        o64 = ora.step_f64(exact, q, k, v, a, float(np.float32(b)), kda)
        assert np.max(np.abs(o - o64)) <= 1e-5 * np.max(np.abs(o64)) + 1e-7, t
        new = cfg.unpack_head(slot, 0).astype(np.float64)
        _, _, r, c = slotcodec.read_head(slot, lay, bits, dk, dv, rf16, cf16)
        half = 0.5 * np.outer(r.astype(np.float64), c.astype(np.float64))
        bound = np.where(piv[:, None], 2.0 ** -11 * np.abs(exact), half * (1 + 1e-5)) \
            + 1e-6 * np.abs(exact) + 1e-30
        assert np.all(np.abs(new - exact) <= bound), t


def test_fp32_units_are_the_fp32_recurrence(ora):
    """Heads of fp32 units (width 32) step exactly like the unquantized fp32
    step (itself pinned by the closed forms above), bit for bit, next to a
    quantized head and a pivot head that do not affect them; pack and unpack
    of an fp32 head are the identity."""
    rng = np.random.default_rng(77)
    dk = dv = 16
    for gate_vec in (False, True):
        bits = np.array([32, 4, 16, 32], np.uint8)
        cfg = _cfg(ora, H=4, dk=dk, dv=dv, gate_vec=gate_vec, bits=bits)
        lay = cfg.head_layout(0)
        assert lay["nquant"] == 0 and lay["bytes"] == (dk * dv * 4 + 255) // 256 * 256
        slot = cfg.new_slot()
        M0 = (rng.standard_normal((dk, dv)) * 0.3).astype(np.float32)
        cfg.pack_head(slot, 0, M0)
        cfg.pack_head(slot, 3, M0)
        assert np.array_equal(cfg.unpack_head(slot, 0), M0)
        M = M0.copy()
        for t in range(12):
            k = rng.standard_normal(dk).astype(np.float32)
            q = rng.standard_normal(dk).astype(np.float32)
            v = rng.standard_normal(dv).astype(np.float32)
            a = rng.uniform(0.8, 1.0, dk if gate_vec else 1).astype(np.float32)
            b = np.float32(rng.uniform(0.2, 1.0))
            want = ora.step_f32(M, q, k, v, a, b, gate_vec)
            for h in range(4):
                o = cfg.step_head(slot, h, q, k, v, a, b)
                if bits[h] == 32:
                    assert np.array_equal(o, want), (t, h)
                    assert np.array_equal(cfg.unpack_head(slot, h), M), (t, h)


def test_all_pivot_is_fp16_recurrence(ora):
    """All units FP16 pivots: the state after each step is the fp16 rounding of
    the fp32 step applied to the previous fp16 state (numpy half casts)."""
    rng = np.random.default_rng(40)
    dk = dv = 16
    cfg = _cfg(ora, dk=dk, dv=dv, width=16)
    slot = cfg.new_slot()
    M = np.zeros((dk, dv), np.float32)
    for t in range(10):
        k = rng.standard_normal(dk).astype(np.float32)
        q = rng.standard_normal(dk).astype(np.float32)
        v = rng.standard_normal(dv).astype(np.float32)
        a = np.float32(rng.uniform(0.8, 1.0))
        cfg.step_head(slot, 0, q, k, v, a, 0.5)
        ora.step_f32(M, q, k, v, np.array([a]), 0.5, False)
        M = M.astype(np.float16).astype(np.float32)
        assert np.array_equal(cfg.unpack_head(slot, 0), M)


# ------------------------------------------------------------ windowed mode

def _window_cfg(ora, W=4, K=5, dk=16, dv=16):
    return _cfg(ora, dk=dk, dv=dv, keyrow=True, gate_vec=True, width=8, window=W, comps=K)


def test_window_pack_selects_topk_by_bruteforce(ora):
    """Compensation entries are the K largest |M| (ties to the lower
    column-major index j*d_k + i), stored in index order with their exact fp32
    values; the rest is quantized with those positions at code 0."""
    rng = np.random.default_rng(50)
    W, K = 4, 7
    cfg = _window_cfg(ora, W, K)
    M = rng.standard_normal((16, 16)).astype(np.float32)
    M[3, 4] = M[9, 1] = -5.0          # a tie in magnitude
    M.flat[200] = 5.0
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, M)
    lay = cfg.head_layout(0)
    idx = slot[lay["cidx"]:lay["cidx"] + 2 * K].view(np.uint16)
    val = slot[lay["cval"]:lay["cval"] + 4 * K].view(np.float32)
    flat = M.T.reshape(-1)                     # column-major: p = j*16 + i
    order = np.lexsort((np.arange(flat.size), -np.abs(flat)))
    want = np.sort(order[:K])
    assert np.array_equal(idx, want)
    assert np.array_equal(val, flat[want])
    n, _, r, c = slotcodec.read_head(slot, lay, np.full(16, 8), 16, 16, True, True)
    assert np.all(n.T.reshape(-1)[want] == 0)
    rest = np.ones(flat.size, bool); rest[want] = False
    assert np.all(c >= np.where(rest.reshape(16, 16).T, np.abs(M), 0).max(axis=0) * (1 - 2 ** -10))
    back = cfg.unpack_head(slot, 0).T.reshape(-1)
    assert np.array_equal(back[want], flat[want])


def test_window_topk_ties_at_the_cut(ora):
    """Many equal magnitudes across the K-th place: the lower column-major
    indices j*d_k + i win."""
    W, K = 4, 6
    cfg = _window_cfg(ora, W, K)
    M = np.zeros((16, 16), np.float32)
    tied = [17, 40, 41, 90, 130, 200, 201, 250]     # eight entries of |3|, by p
    for t, p in enumerate(tied):
        M[p % 16, p // 16] = 3.0 if t % 2 else -3.0
    M[5, 0] = 7.0
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, M)
    lay = cfg.head_layout(0)
    idx = slot[lay["cidx"]:lay["cidx"] + 2 * K].view(np.uint16)
    assert idx.tolist() == sorted([5] + tied[:5])


def test_window_in_window_matches_dense_recurrence(ora):
    """Inside a window the outputs come from the fixed base plus fp32 deltas:
    they match the exact recurrence started from the dequantized base, and
    the materialized state before the window end matches it too."""
    rng = np.random.default_rng(51)
    W, K, dk, dv = 6, 4, 16, 16
    cfg = _window_cfg(ora, W, K, dk, dv)
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, rng.standard_normal((dk, dv)).astype(np.float32))
    M = cfg.unpack_head(slot, 0).astype(np.float64)
    for t in range(W - 1):
        k = rng.standard_normal(dk); k /= np.linalg.norm(k)
        q = rng.standard_normal(dk); q /= np.linalg.norm(q)
        v = rng.standard_normal(dv)
        a = rng.uniform(0.8, 1.0, dk)
        k, q, v, a = (x.astype(np.float32) for x in (k, q, v, a))
        o = cfg.step_head(slot, 0, q, k, v, a, 0.7)
        o64 = ora.step_f64(M, q, k, v, a, float(np.float32(0.7)), True)
        np.testing.assert_allclose(o, o64, atol=2e-5 * np.abs(o64).max(), rtol=0)
        np.testing.assert_allclose(cfg.unpack_head(slot, 0), M, atol=2e-5 * np.abs(M).max(), rtol=0)
    # the W-th step closes the window: deltas cleared, gates reset
    k = np.eye(dk, dtype=np.float32)[0]
    cfg.step_head(slot, 0, k, k, np.zeros(dv, np.float32), np.ones(dk, np.float32), 0.5)
    lay = cfg.head_layout(0)
    assert slot[lay["wn"]:lay["wn"] + 4].view(np.int32)[0] == 0
    assert np.all(slot[lay["g"]:lay["g"] + 4 * dk].view(np.float32) == 1.0)


def test_first_window_step_tracks_per_step(ora):
    """The first step of a window (W = 2, no compensation entries) applies the
    same update to the same stored state as the every-step mode, in another
    rounding order: the two outputs agree to 1e-5 relative.  (Later steps are
    not comparable: the every-step mode has requantized by then.)"""
    rng = np.random.default_rng(52)
    dk = dv = 16
    per = _cfg(ora, dk=dk, dv=dv, keyrow=True, gate_vec=True, width=8)
    win = _cfg(ora, dk=dk, dv=dv, keyrow=True, gate_vec=True, width=8, window=2, comps=0)
    s1, s2 = per.new_slot(), win.new_slot()
    for t in range(2):
        k = rng.standard_normal(dk).astype(np.float32)
        q = rng.standard_normal(dk).astype(np.float32)
        v = rng.standard_normal(dv).astype(np.float32)
        a = rng.uniform(0.8, 1, dk).astype(np.float32)
        o1 = per.step_head(s1, 0, q, k, v, a, 0.5)
        o2 = win.step_head(s2, 0, q, k, v, a, 0.5)
        if t == 0:
            np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-5 * np.abs(o1).max())


def _comps(slot, lay, K, dk):
    idx = slot[lay["cidx"]:lay["cidx"] + 2 * K].view(np.uint16).astype(np.int64)
    val = slot[lay["cval"]:lay["cval"] + 4 * K].view(np.float32).astype(np.float64)
    return idx % dk, idx // dk, idx, val


def _f16_at_most_one_apart(c, lo, hi):
    """c is the fp16 nearest-even of some value in [lo, hi] (numpy casts)."""
    lo16 = np.asarray(lo, np.float32).astype(np.float16).astype(np.float64)
    hi16 = np.asarray(hi, np.float32).astype(np.float16).astype(np.float64)
    return (c >= lo16) & (c <= hi16)


@pytest.mark.parametrize("W,K,mixed", [(4, 5, False), (2, 9, False), (5, 12, True)])
def test_window_end_matches_exact_recurrence(ora, W, K, mixed):
    """Three windows from a packed random state.  At every window end the
    stored state is checked against the exact (fp64) gated delta-rule
    recurrence run over the window from the dequantized base (compensation
    entries included):
      - the new compensation entries hold that state's values at their
        positions (to the fp32 rounding of the in-window arithmetic), are
        stored by ascending column-major index, and are its K largest |M|
        among non-pivot rows (to the same slack);
      - every other quantized entry is within half a step r'_i c'_j of it,
        and FP16 pivot rows within half an fp16 ulp;
      - each column scale is the fp16 of the largest |M| over that column's
        non-entry quantized rows, up to the slack;
      - the cumulative gate is back to 1 and no delta is pending.
    Outputs inside the window are checked against the same recurrence.
    Pins the window end's materialization (base with entries, every delta,
    the cumulative gate), the top-K choice and its exclusion from the scales."""
    rng = np.random.default_rng(60 + W + K)
    dk = dv = 16
    bits = np.full(dk, 8, np.uint8)
    if mixed:
        bits[[1, 6]] = 4
        bits[11] = 16
    cfg = _cfg(ora, dk=dk, dv=dv, keyrow=True, gate_vec=True, bits=bits, window=W, comps=K)
    lay = cfg.head_layout(0)
    piv = bits == 16
    slot = cfg.new_slot()
    M0 = rng.standard_normal((dk, dv)).astype(np.float32)
    M0[rng.integers(0, dk, 3), rng.integers(0, dv, 3)] *= 8.0
    cfg.pack_head(slot, 0, M0)
    for window in range(3):
        M = cfg.unpack_head(slot, 0).astype(np.float64)
        assert slot[lay["wn"]:lay["wn"] + 4].view(np.int32)[0] == 0
        for t in range(W):
            k = rng.standard_normal(dk); k /= np.linalg.norm(k)
            q = rng.standard_normal(dk); q /= np.linalg.norm(q)
            v = rng.standard_normal(dv)
            a = rng.uniform(0.8, 1.0, dk)
            b = rng.uniform(0.3, 1.0)
            k, q, v, a = (x.astype(np.float32) for x in (k, q, v, a))
            o = cfg.step_head(slot, 0, q, k, v, a, b)
            o64 = ora.step_f64(M, q, k, v, a, float(np.float32(b)), True)
            assert np.max(np.abs(o - o64)) <= 2e-5 * np.abs(o64).max(), (window, t)
        slack = 2e-5 * np.abs(M).max()
        assert slot[lay["wn"]:lay["wn"] + 4].view(np.int32)[0] == 0
        assert np.all(slot[lay["g"]:lay["g"] + 4 * dk].view(np.float32) == 1.0)
        ri, cj, idx, val = _comps(slot, lay, K, dk)
        assert np.all(np.diff(idx) > 0), "entries stored by ascending column-major index"
        assert not piv[ri].any(), "no entry on a pivot row"
        assert np.all(np.abs(val - M[ri, cj]) <= slack), window
        chosen = np.zeros((dk, dv), bool)
        chosen[ri, cj] = True
        others = ~chosen & ~piv[:, None]
        assert np.abs(M[chosen]).min() >= np.abs(M[others]).max() - slack, window
        n, hv, r, c = slotcodec.read_head(slot, lay, bits, dk, dv, True, True)
        new = cfg.unpack_head(slot, 0).astype(np.float64)
        half = 0.5 * np.outer(r.astype(np.float64), c.astype(np.float64))
        q_ok = np.abs(new - M) <= half * (1 + 1e-5) + slack
        p_ok = np.abs(new - M) <= 2.0 ** -11 * np.abs(M) + slack
        assert np.all(np.where(piv[:, None], p_ok, q_ok | chosen)), window
        assert np.all(n[chosen] == 0)
        C = np.where(others, np.abs(M), 0.0).max(axis=0)
        assert np.all(_f16_at_most_one_apart(c, C - slack, C + slack)), window


@pytest.mark.parametrize("K", [3, 17])
def test_entries_are_left_out_of_both_scale_maxima(ora, K):
    """A state whose K largest entries are far above the rest: after pack,
    each column scale is exactly the fp16 (numpy cast) of the largest |M| over
    the column's non-entry entries, and each row step is the smallest fp16 not
    below the largest non-entry |M_ij / c_j| over qmax; the entries keep their
    exact values and hold code 0."""
    rng = np.random.default_rng(70 + K)
    dk = dv = 16
    cfg = _window_cfg(ora, 4, K)
    lay = cfg.head_layout(0)
    for trial in range(6):
        M = rng.standard_normal((dk, dv)).astype(np.float32)
        flat = rng.choice(dk * dv, K, replace=False)
        M.flat[flat] = (rng.uniform(20, 50, K) * rng.choice([-1, 1], K)).astype(np.float32)
        slot = cfg.new_slot()
        cfg.pack_head(slot, 0, M)
        ri, cj, idx, val = _comps(slot, lay, K, dk)
        chosen = np.zeros((dk, dv), bool)
        chosen[ri, cj] = True
        assert np.array_equal(np.sort(np.ravel_multi_index((ri, cj), (dk, dv))), np.sort(flat))
        assert np.array_equal(val, M[ri, cj].astype(np.float64))
        n, _, r, c = slotcodec.read_head(slot, lay, np.full(dk, 8), dk, dv, True, True)
        assert np.all(n[chosen] == 0)
        rest = np.where(chosen, 0.0, np.abs(M))
        want_c = rest.max(axis=0).astype(np.float16).astype(np.float32)
        assert np.array_equal(c, want_c)
        need = (rest / c[None, :].astype(np.float64)).max(axis=1) / 127
        assert np.all(r >= need * (1 - 2 ** -22))
        below = np.nextafter(r.astype(np.float16), np.float16(0)).astype(np.float64)
        assert np.all((below < need * (1 + 2 ** -22)) | (r == 0))


# ------------------------------------------------------------- workloads

def test_workload_metadata():
    w = synth.WORKLOADS["qwen_gdn"]
    b = synth.unit_bits(w)
    assert sorted(np.unique(b, return_counts=True)[1].tolist()) == [1, 10, 10, 11]
    assert np.mean(b[b != 16]) == 6.0
    k = synth.unit_bits(synth.WORKLOADS["kimi_kda"])
    assert (k == 16).sum() == 41 and set(np.unique(k)) == {4, 16}
    s = synth.unit_bits(synth.WORKLOADS["serving_gdn"])
    assert (s == 16).sum() == 1 and (s == 4).sum() == 31


def test_inputs_regenerate_per_unit():
    w = synth.WORKLOADS["kimi_kda"].with_(B=8)
    full = synth.batch_inputs(w, 0, 3)
    one = synth.step_inputs(w, 0, 3, 5, 7)
    assert np.array_equal(full.q[5, 7], one.q) and np.array_equal(full.a[5, 7], one.a)
    assert np.all((one.a > 0.8) & (one.a < 1.0))
    assert abs(np.linalg.norm(one.k) - 1) < 1e-2
    M0 = synth.initial_state(w, 0, 2, 3)
    med = np.median(np.abs(M0))
    big = np.abs(M0) > 5 * med
    assert 5 <= big.any(axis=1).sum() <= 128 and big.sum() < 0.2 * M0.size


# ------------------------------------------------------------ lagged scales

def _lagged_cfg(ora, width, kda, scales, dk=32, dv=32):
    rf16, cf16 = SCALES[scales]
    bits = np.full(dk, width, np.uint8)
    if kda:
        bits[[3, 20]] = 16
        return ora.Cfg(1, dk, dv, True, True, rf16, cf16, 1, 0, bits, scale_fit=1), bits
    return ora.Cfg(1, dk, dv, False, False, rf16, cf16, 1, 0, bits[:1], scale_fit=1), bits


def _read_lagged(slot, lay, dk, dv, rf16, cf16):
    b = lay["base"]
    nr = (slot[b + lay["nrs"]:b + lay["nrs"] + 2 * dk].view(np.float16).astype(np.float64) if rf16
          else slot[b + lay["nrs"]:b + lay["nrs"] + 4 * dk].view(np.float32).astype(np.float64))
    nc = (slot[b + lay["ncs"]:b + lay["ncs"] + 2 * dv].view(np.float16).astype(np.float64) if cf16
          else np.ones(dv))
    sr = slot[b + lay["sr"]:b + lay["sr"] + 4 * dk].view(np.float32).astype(np.float64)
    sc = (slot[b + lay["sc"]:b + lay["sc"] + 4 * dv].view(np.float32).astype(np.float64) if cf16
          else None)
    return nr, nc, sr, sc


def _smallest_f16_not_below(x):
    h = np.asarray(x, np.float32).astype(np.float16)
    up = h.astype(np.float64) < x
    h[up] = np.nextafter(h[up], np.float16(np.inf))
    return h.astype(np.float64)


@pytest.mark.parametrize("scales", list(SCALES))
@pytest.mark.parametrize("width", [4, 6, 8])
@pytest.mark.parametrize("kda", [False, True])
def test_lagged_step_against_the_exact_step(ora, width, kda, scales):
    """Lagged scales, element by element against the exact (fp64) step of the
    stored state: the step writes with the scales fitted from the previous
    state's statistics (they become the stored scales); each quantized entry
    is within half a step of the exact value, or, where the exact value lies
    beyond qmax + 1/2 steps, stored at +-qmax with its sign (clipped); pivot
    rows within half an fp16 ulp; o is the exact output.  The statistics are
    the exact state's column absmax and its row absmax in the fp16 of that
    column absmax (the every-step refit of the state); the fit gives the numpy
    fp16 of the column statistic
    and the smallest fp16 (or the fp32, for fp32 row scales) not below the
    row statistic over qmax."""
    rf16, cf16 = SCALES[scales]
    rng = np.random.default_rng(80 + width + 3 * kda + 7 * rf16)
    dk = dv = 32
    cfg, bits = _lagged_cfg(ora, width, kda, scales, dk, dv)
    qm = (1 << (width - 1)) - 1
    piv = bits == 16
    lay = cfg.head_layout(0)
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, (rng.standard_normal((dk, dv)) * 0.5).astype(np.float32))
    clipped_seen = 0
    for t in range(16):
        prev = cfg.unpack_head(slot, 0).astype(np.float64)
        nr0, nc0, _, _ = _read_lagged(slot, lay, dk, dv, rf16, cf16)
        k = rng.standard_normal(dk); k /= np.linalg.norm(k)
        q = rng.standard_normal(dk); q /= np.linalg.norm(q)
        v = rng.standard_normal(dv) * (3.0 if t % 5 == 4 else 1.0)   # now and then a jump
        a = rng.uniform(0.85, 1.0, dk if kda else 1)
        b = rng.uniform(0.3, 1.0)
        k, q, v, a = (x.astype(np.float32) for x in (k, q, v, a))
        o = cfg.step_head(slot, 0, q, k, v, a, b)
        exact = prev.copy()
        o64 = ora.step_f64(exact, q, k, v, a, float(np.float32(b)), kda)
        assert np.max(np.abs(o - o64)) <= 1e-5 * np.max(np.abs(o64)) + 1e-7, t
        n, hv, r, c = slotcodec.read_head(slot, lay, bits, dk, dv, rf16, cf16)
        new = cfg.unpack_head(slot, 0).astype(np.float64)
        nr, nc, sr, sc = _read_lagged(slot, lay, dk, dv, rf16, cf16)
        if t > 0:
            # written with the scales fitted before the step
            assert np.array_equal(r[~piv].astype(np.float64), nr0[~piv]), t
            if cf16:
                assert np.array_equal(c.astype(np.float64), nc0), t
        step = np.outer(r.astype(np.float64), c.astype(np.float64))
        slack = 1e-6 * np.abs(exact).max() + 1e-30
        inside = np.abs(exact) <= (qm + 0.5) * step
        q_ok = np.where(inside, np.abs(new - exact) <= 0.5 * step * (1 + 1e-5) + slack,
                        (np.abs(n) == qm) & (np.sign(n) == np.sign(exact)))
        p_ok = np.abs(new - exact) <= 2.0 ** -11 * np.abs(exact) + slack
        assert np.all(np.where(piv[:, None], p_ok, q_ok)), t
        clipped_seen += int((~inside & ~piv[:, None]).sum())
        # statistics of the exact state
        qrows = ~piv
        if cf16:
            want_c = np.abs(exact[qrows]).max(axis=0)
            assert np.all(np.abs(sc - want_c) <= 1e-5 * want_c.max() + 1e-30), t
            cfit = sc.astype(np.float32).astype(np.float16).astype(np.float64)
            Zx = exact / np.where(cfit > 0, cfit, np.inf)[None, :]
        else:
            Zx = exact
        want_r = np.where(qrows, np.abs(Zx).max(axis=1), 0.0)
        assert np.all(np.abs(sr - want_r) <= 1e-5 * want_r.max() + 1e-30), t
        # the fit
        cfg.fit_head(slot, 0)
        nr, nc, sr2, sc2 = _read_lagged(slot, lay, dk, dv, rf16, cf16)
        assert np.array_equal(sr2, sr)
        if cf16:
            assert np.array_equal(nc, sc.astype(np.float32).astype(np.float16).astype(np.float64)), t
        if rf16:
            assert np.array_equal(nr[qrows], _smallest_f16_not_below(sr[qrows] / qm)), t
        else:
            assert np.all(np.abs(nr[qrows] - sr[qrows] / qm) <= 2.0 ** -24 * nr[qrows]), t
        assert np.all(nr[piv] == 0)
    assert clipped_seen > 0, "the jumps should make the lagged scales clip somewhere"


@pytest.mark.parametrize("kda", [False, True])
def test_lagged_first_step_is_the_every_step_refit(ora, kda):
    """A state without fitted next scales (fresh, or just packed) is refitted
    in the step: its first step is bit for bit the every-step mode's."""
    rng = np.random.default_rng(90 + kda)
    dk = dv = 32
    lag, bits = _lagged_cfg(ora, 4, kda, "f16", dk, dv)
    per = ora.Cfg(1, dk, dv, kda, kda, True, True, 1, 0, bits if kda else bits[:1])
    for packed in (False, True):
        s1, s2 = lag.new_slot(), per.new_slot()
        if packed:
            M0 = (rng.standard_normal((dk, dv)) * 0.5).astype(np.float32)
            lag.pack_head(s1, 0, M0)
            per.pack_head(s2, 0, M0)
        k = rng.standard_normal(dk).astype(np.float32)
        q = rng.standard_normal(dk).astype(np.float32)
        v = rng.standard_normal(dv).astype(np.float32)
        a = rng.uniform(0.8, 1.0, dk if kda else 1).astype(np.float32)
        o1 = lag.step_head(s1, 0, q, k, v, a, 0.6)
        o2 = per.step_head(s2, 0, q, k, v, a, 0.6)
        assert np.array_equal(o1, o2)
        h1 = slotcodec.read_head(s1, lag.head_layout(0), bits, dk, dv, True, True)
        h2 = slotcodec.read_head(s2, per.head_layout(0), bits, dk, dv, True, True)
        for x, y in zip(h1, h2):
            assert np.array_equal(x, y)


def test_lagged_scales_catch_up(ora):
    """A state that stops changing (gate 1, write strength 0) after a jump:
    the step of the jump clips (its scales were fitted before the jump) far
    beyond the range, and so does the next step (it writes the clipped state
    with scales fitted to the unclipped one); from the third step after it,
    entries exceed the range by less than one step (a row maximum that lands
    on the other side of a rounding boundary of the new grid) and every row
    again spans at least 90 % of its code range."""
    rng = np.random.default_rng(95)
    dk = dv = 32
    qm = 127
    cfg, bits = _lagged_cfg(ora, 8, False, "f16", dk, dv)
    lay = cfg.head_layout(0)
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, (rng.standard_normal((dk, dv)) * 0.1).astype(np.float32))
    ones = np.ones(1, np.float32)
    k = np.eye(dk, dtype=np.float32)[5]
    z = np.zeros(dv, np.float32)
    cfg.step_head(slot, 0, k, k, z, ones, 0.0)   # refit in the step
    cfg.fit_head(slot, 0)
    # the jump: a large value row written along key 5
    prev = cfg.unpack_head(slot, 0).astype(np.float64)
    v = (rng.standard_normal(dv) * 20).astype(np.float32)
    cfg.step_head(slot, 0, k, k, v, ones, 1.0)
    exact = prev.copy()
    ora.step_f64(exact, k, k, v, ones, 1.0, False)
    n, _, r, c = slotcodec.read_head(slot, lay, bits, dk, dv, True, True)
    assert (np.abs(exact) > (qm + 0.5) * np.outer(r, c)).sum() > dv // 2   # the jump clipped
    cfg.fit_head(slot, 0)
    for t in range(6):
        prev = cfg.unpack_head(slot, 0).astype(np.float64)
        cfg.step_head(slot, 0, k, k, z, ones, 0.0)
        cfg.fit_head(slot, 0)
        if t >= 2:
            n, _, r, c = slotcodec.read_head(slot, lay, bits, dk, dv, True, True)
            assert np.all(np.abs(prev) <= (qm + 1.0) * np.outer(r, c) * (1 + 1e-6)), t
            assert np.all(np.abs(n).max(axis=1) >= 0.9 * qm), t


# ------------------------------------------------------------ row impact

def _imp_cfg(ora, impact, width=8, dk=32, dv=32, H=1, keyrow=False):
    bits = np.full(H * dk if keyrow else H, width, np.uint8)
    return ora.Cfg(H, dk, dv, keyrow, keyrow, True, True, 1, 0, bits, row_impact=impact)


def test_impact_equal_scores_are_the_plain_fit(ora):
    """Equal impact scores (any positive value, or all zero) leave the fit as
    it is without scores, bit for bit, in pack and in every step; and
    multiplying every score of a head by a constant changes nothing."""
    rng = np.random.default_rng(100)
    dk = dv = 32
    plain = _imp_cfg(ora, None)
    imp = rng.uniform(0.1, 2.0, dk).astype(np.float32)
    variants = [(np.full(dk, 3.5, np.float32), plain), (np.zeros(dk, np.float32), plain),
                (imp * 7.0, _imp_cfg(ora, imp))]
    for scores, ref in variants:
        cfg = _imp_cfg(ora, scores)
        s1, s2 = cfg.new_slot(), ref.new_slot()
        M0 = (rng.standard_normal((dk, dv)) * 0.5).astype(np.float32)
        cfg.pack_head(s1, 0, M0)
        ref.pack_head(s2, 0, M0)
        assert np.array_equal(s1, s2)
        for t in range(6):
            k, q = rng.standard_normal(dk).astype(np.float32), rng.standard_normal(dk).astype(np.float32)
            v = rng.standard_normal(dv).astype(np.float32)
            a = np.float32(rng.uniform(0.8, 1.0))
            o1 = cfg.step_head(s1, 0, q, k, v, a, 0.5)
            o2 = ref.step_head(s2, 0, q, k, v, a, 0.5)
            assert np.array_equal(o1, o2) and np.array_equal(s1, s2), t


def test_column_scale_follows_the_largest_rms_output_contribution(ora):
    """An entry M_ij reaches o_j as q_i M_ij, whose RMS over queries with
    E[q_i^2] = iota_i is sqrt(iota_i) |M_ij|.  The column scale is set by the
    entry with the largest such contribution: with row A (impact 1, value 1)
    and row B (impact 1/4) in one column, B sets the scale once its value
    exceeds 2 (its contribution exceeds A's), and not before."""
    dk = dv = 8
    imp = np.ones(dk, np.float32)
    imp[1] = 0.25
    cfg = _imp_cfg(ora, imp, dk=dk, dv=dv)
    lay = cfg.head_layout(0)
    for yb, want in ((1.5, 1.0), (1.9, 1.0), (2.5, 1.25), (3.0, 1.5)):
        M = np.full((dk, dv), 0.01, np.float32)
        M[0, 3] = 1.0
        M[1, 3] = yb
        slot = cfg.new_slot()
        cfg.pack_head(slot, 0, M)
        _, _, _, c = slotcodec.read_head(slot, lay, np.full(dk, 8), dk, dv, True, True)
        assert c[3] == np.float16(want), (yb, c[3])


def test_zero_impact_rows_leave_the_column_scales(ora):
    """Rows of impact 0 do not set the column scales: each column scale is
    the numpy fp16 of the largest |M| over the other rows, however large the
    zero-impact rows are; those rows still get their full range (no code
    clips, every entry within half a step)."""
    rng = np.random.default_rng(101)
    dk = dv = 32
    quiet = {0: [2, 9, 30], 1: [0, 17]}          # per head
    imp = np.ones((2, dk), np.float32)
    imp[1] *= 4.0                                 # scores are relative within a head
    for h, rows in quiet.items():
        imp[h, rows] = 0.0
    cfg = _imp_cfg(ora, imp.ravel(), H=2)
    for trial in range(5):
        slot = cfg.new_slot()
        Ms = []
        for h in range(2):
            M = rng.standard_normal((dk, dv)).astype(np.float32)
            M[quiet[h]] *= 50.0
            cfg.pack_head(slot, h, M)
            Ms.append(M)
        for h in range(2):
            M, rows = Ms[h], quiet[h]
            n, _, r, c = slotcodec.read_head(slot, cfg.head_layout(h), np.full(dk, 8), dk, dv, True, True)
            rest = np.abs(np.delete(M, rows, axis=0)).max(axis=0)
            assert np.array_equal(c, rest.astype(np.float16).astype(np.float32)), (trial, h)
            step = np.outer(r.astype(np.float64), c.astype(np.float64))
            assert np.all(np.abs(M) <= (127 + 0.5) * step)
            assert np.all(np.abs(M - n * step) <= 0.5 * step * (1 + 1e-5))
            assert np.all(np.abs(n[rows]).max(axis=1) == 127)


def test_impact_weighted_fit_lowers_the_output_error(ora):
    """The purpose of the weighting: when a few large entries sit in rows
    whose query weight is small (each widens its whole column under the plain
    absmax fit, which no row scale can undo), fitting the column scales to the
    high-impact rows at least halves the output error
    E|sum_i q_i (M_ij - stored_ij)|^2 for queries drawn with that impact
    profile (E[q_i^2] = iota_i), against the plain fit of the same states; at
    4, 6 and 8 bits."""
    rng = np.random.default_rng(102)
    dk = dv = 32
    iota = np.where(np.arange(dk) < 8, 0.02, 1.0).astype(np.float32)  # 8 low-impact rows
    for width in (4, 6, 8):
        plain, weighted = _imp_cfg(ora, None, width), _imp_cfg(ora, iota, width)
        err = {0: 0.0, 1: 0.0}
        for trial in range(20):
            M = (rng.standard_normal((dk, dv)) * 0.3).astype(np.float32)
            for i in range(8):   # three large entries in each low-impact row
                M[i, rng.choice(dv, 3, replace=False)] *= 50.0
            for key, cfg in ((0, plain), (1, weighted)):
                slot = cfg.new_slot()
                cfg.pack_head(slot, 0, M)
                E = cfg.unpack_head(slot, 0).astype(np.float64) - M
                # E over q with E[q_i q_k] = iota_i delta_ik
                err[key] += float((iota[:, None] * E ** 2).sum())
        assert err[1] < 0.5 * err[0], (width, err)


@pytest.mark.parametrize("width", [4, 8])
def test_impact_weighted_step_injects_at_most_half_a_step(ora, width):
    """With row-impact weights the step is still the exact step of the stored
    state plus at most half a step r'_i c'_j per entry, and o is exact."""
    rng = np.random.default_rng(103 + width)
    dk = dv = 32
    iota = rng.uniform(0.0, 1.0, dk).astype(np.float32) ** 3
    cfg = _imp_cfg(ora, iota, width)
    lay = cfg.head_layout(0)
    slot = cfg.new_slot()
    cfg.pack_head(slot, 0, (rng.standard_normal((dk, dv)) * 0.5).astype(np.float32))
    for t in range(16):
        prev = cfg.unpack_head(slot, 0).astype(np.float64)
        k = rng.standard_normal(dk); k /= np.linalg.norm(k)
        q = rng.standard_normal(dk); q /= np.linalg.norm(q)
        v = rng.standard_normal(dv)
        a = rng.uniform(0.85, 1.0, 1)
        b = rng.uniform(0.3, 1.0)
        k, q, v, a = (x.astype(np.float32) for x in (k, q, v, a))
        o = cfg.step_head(slot, 0, q, k, v, a, b)
        exact = prev.copy()
        o64 = ora.step_f64(exact, q, k, v, a, float(np.float32(b)), False)
        assert np.max(np.abs(o - o64)) <= 1e-5 * np.max(np.abs(o64)) + 1e-7, t
        new = cfg.unpack_head(slot, 0).astype(np.float64)
        _, _, r, c = slotcodec.read_head(slot, lay, np.full(dk, width), dk, dv, True, True)
        half = 0.5 * np.outer(r.astype(np.float64), c.astype(np.float64))
        assert np.all(np.abs(new - exact) <= half * (1 + 1e-5) + 1e-6 * np.abs(exact) + 1e-30), t
