"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every function declared in include/stq.h, computes the same slot layout as the
oracle, and rejects bad arguments before launching anything."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def stq():
    import linear_attention_recurrent_stq_amd as m
    return m


def test_exports_every_declared_symbol(stq):
    hdr = open(os.path.join(ROOT, "include", "stq.h")).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(stq_\w+)\s*\(", hdr, re.M))
    assert {"stq_pack_layout", "stq_alloc_pool", "stq_decode_step", "stq_unpack"} <= declared
    lib = stq.library()
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert set(stq.SYMBOLS) == declared


@pytest.mark.parametrize("name", [n for n, w in synth.WORKLOADS.items() if w.bits != "allocated"])
def test_layout_matches_oracle(stq, ora, name):
    w = synth.WORKLOADS[name]
    bits = synth.unit_bits(w)
    L = stq.Layout.from_workload(w, bits)
    o = ora.Cfg.from_workload(w, bits)
    assert L.slot_bytes == o.slot_bytes
    for h in range(w.H):
        off, nb = L.head(h)
        lay = o.head_layout(h)
        assert (off, nb) == (lay["base"], lay["bytes"])


def test_layout_mixed_rows_matches_oracle(stq, ora):
    rng = np.random.default_rng(0)
    for d in (64, 128):
        bits = rng.choice(np.array([4, 6, 8, 16], np.uint8), 5 * d)
        L = stq.Layout(5, d, d, bits, unit=stq.UNIT_KEYROW, gate=stq.GATE_KEYVEC, window=8, comps=20)
        o = ora.Cfg(5, d, d, True, True, True, True, 8, 20, bits)
        assert L.slot_bytes == o.slot_bytes
        for h in range(5):
            assert L.head(h) == (o.head_layout(h)["base"], o.head_layout(h)["bytes"])


def _header_bytes(H, dk, widths):
    """Device table: head descriptors (64 B each), the row table (4 B per key
    row), then the step kernel's head groups (4 B each: 4-bit heads in pairs,
    every other head alone), padded to 256 B."""
    four = sum(1 for x in widths if x == 4)
    groups = (four + 1) // 2 + sum(1 for x in widths if x != 4)
    n = 64 * H + 4 * H * dk + 4 * groups
    return (n + 255) // 256 * 256


def test_pool_size_query_without_device(stq):
    w = synth.WORKLOADS["serving_gdn"]
    bits = synth.unit_bits(w)
    L = stq.Layout.from_workload(w, bits)
    q = stq.StqPool()
    assert stq.library().stq_alloc_pool(L.handle, 512, None, 0, None, C.byref(q)) == stq.STQ_OK
    assert q.bytes == L.header_bytes + 512 * 302592
    assert L.header_bytes == _header_bytes(32, 128, bits)


@pytest.mark.parametrize("name", [n for n, w in synth.WORKLOADS.items() if w.bits != "allocated"])
def test_header_holds_the_head_groups(stq, name):
    w = synth.WORKLOADS[name]
    bits = synth.unit_bits(w)
    L = stq.Layout.from_workload(w, bits)
    # per-key-row layouts have no uniform 4-bit heads unless every row is 4-bit
    per_head = bits if w.unit == "head" else [
        int(bits[h * w.dk]) if (bits[h * w.dk:(h + 1) * w.dk] == bits[h * w.dk]).all() else 0
        for h in range(w.H)]
    assert L.header_bytes == _header_bytes(w.H, w.dk, per_head)


@pytest.mark.parametrize("H,d", [(32, 128), (64, 64)])
def test_windowed_header_holds_the_window_end_flag(stq, H, d):
    """Windowed layouts keep an 8-byte window-end flag after the tables (at
    an 8-byte boundary), inside the header: at H = 64, d = 64 the tables fill
    whole 256-byte blocks, so the flag takes one more block."""
    w = synth.WORKLOADS["windowed_kda"].with_(H=H, dk=d, dv=d, comps=20, name=f"win_hdr_{H}_{d}")
    bits = synth.unit_bits(w)
    L = stq.Layout.from_workload(w, bits)
    n = 64 * H + 4 * H * d + 4 * H          # descriptors, row table, one group per 8-bit head
    want = ((n + 7) // 8 * 8 + 8 + 255) // 256 * 256
    assert L.header_bytes == want
    plain = stq.Layout.from_workload(w.with_(window=1, comps=0, name=f"step_hdr_{H}_{d}"), bits)
    assert plain.header_bytes == (n + 255) // 256 * 256
    if n % 256 == 0:
        assert L.header_bytes == plain.header_bytes + 256


@pytest.mark.parametrize("field,value,status", [
    ("H", 0, 1), ("d_k", 96, 2), ("d_v", 32, 2), ("unit", 5, 1), ("gate", 2, 1),
    ("row_scale", 0, 1), ("col_scale", 1, 1), ("io_dtype", 2, 1), ("window", 0, 1),
    ("window", 17, 2), ("comps", 3, 1), ("comps", -1, 1),
])
def test_config_rejected(stq, field, value, status):
    bits = np.full(4, 4, np.uint8)
    cfg = stq.StqConfig(4, 64, 64, 0, 0, stq.F16, stq.F16, stq.BF16, 1, 0, stq.FIT_STEP,
                        bits.ctypes.data_as(C.POINTER(C.c_uint8)))
    setattr(cfg, field, value)
    h = C.c_void_p()
    assert stq.library().stq_pack_layout(C.byref(cfg), C.byref(h)) == status
    assert not h.value
    assert stq.library().stq_last_error().decode()


def test_fp32_units(stq, ora):
    """Width 32 (fp32, unquantized units) is a whole-head width of the
    every-step mode: accepted there, with the oracle's layout; rejected in the
    windowed mode and on part of a KDA head's key rows."""
    bits = np.array([32, 4, 16, 32], np.uint8)
    L = stq.Layout(4, 128, 128, bits)
    o = ora.Cfg(4, 128, 128, False, False, True, True, 1, 0, bits)
    assert L.slot_bytes == o.slot_bytes
    assert L.head(0) == (0, 128 * 128 * 4)
    kda = np.full(2 * 64, 4, np.uint8)
    kda[:64] = 32                          # head 0 all fp32, head 1 4-bit
    stq.Layout(2, 64, 64, kda, unit=stq.UNIT_KEYROW, gate=stq.GATE_KEYVEC)
    kda[64] = 32                           # one fp32 row in head 1
    with pytest.raises(stq.StqError) as e:
        stq.Layout(2, 64, 64, kda, unit=stq.UNIT_KEYROW, gate=stq.GATE_KEYVEC)
    assert "whole heads" in str(e.value)
    with pytest.raises(stq.StqError) as e:
        stq.Layout(4, 128, 128, bits, window=4, comps=8)
    assert "window" in str(e.value)


def test_bad_widths_and_too_many_comps(stq):
    with pytest.raises(stq.StqError) as e:
        stq.Layout(2, 64, 64, np.array([4, 5], np.uint8))
    assert "unit_bits[1]" in str(e.value)
    with pytest.raises(stq.StqError):
        # a head of pivot rows only leaves no entry for compensation
        bits = np.full(2 * 64, 16, np.uint8)
        stq.Layout(2, 64, 64, bits, unit=stq.UNIT_KEYROW, window=4, comps=1)
    with pytest.raises(stq.StqError):
        stq.Layout(2, 64, 64, np.array([4, 4], np.uint8), window=1, comps=2)


def test_calls_validate_before_launch(stq):
    lib = stq.library()
    w = synth.WORKLOADS["tiny_gdn"]
    L = stq.Layout.from_workload(w, synth.unit_bits(w))
    pool = stq.StqPool()
    assert lib.stq_decode_step(C.byref(pool), 1, None, None, None, None, None, None, None, None) \
        == stq.STQ_ERR_INVALID
    fake = stq.StqPool(C.c_void_p(0x100000), 1 << 20, 4, L.handle)
    P = C.c_void_p
    assert lib.stq_decode_step(C.byref(fake), -1, P(16), P(16), P(16), P(16), P(16), P(16), P(16), None) \
        == stq.STQ_ERR_INVALID
    assert lib.stq_decode_step(C.byref(fake), 5, P(16), P(16), P(16), P(16), P(16), P(16), P(16), None) \
        == stq.STQ_ERR_INVALID  # B > slots
    assert lib.stq_decode_step(C.byref(fake), 2, P(16), P(24), P(16), P(16), P(16), P(16), P(16), None) \
        == stq.STQ_ERR_ALIGN
    assert lib.stq_decode_step(C.byref(fake), 2, P(18), P(16), P(16), P(16), P(16), P(16), P(16), None) \
        == stq.STQ_ERR_ALIGN
    assert lib.stq_decode_step(C.byref(fake), 2, P(16), None, P(16), P(16), P(16), P(16), P(16), None) \
        == stq.STQ_ERR_INVALID
    assert lib.stq_decode_step(C.byref(fake), 0, None, None, None, None, None, None, None, None) \
        == stq.STQ_OK
    assert lib.stq_unpack(C.byref(fake), 2, P(16), None, None) == stq.STQ_ERR_INVALID
    assert lib.stq_pack(C.byref(fake), 2, P(16), P(8), None) == stq.STQ_ERR_ALIGN
    small = C.c_size_t(0)
    out = stq.StqPool()
    assert lib.stq_alloc_pool(L.handle, 4, P(0x100000), 100, None, C.byref(out)) == stq.STQ_ERR_TOO_SMALL
    assert lib.stq_alloc_pool(L.handle, 4, P(0x100008), 1 << 20, None, C.byref(out)) == stq.STQ_ERR_ALIGN
    assert lib.stq_layout_head(L.handle, 7, C.byref(small), None) == stq.STQ_ERR_INVALID


def test_check_slot_ids_on_host(stq):
    """stq_check_slot_ids: distinct ids in range pass; a repeated id, a
    negative id and an id past the slot count are rejected, naming the
    first bad position."""
    w = synth.WORKLOADS["qwen_gdn"]
    L = stq.Layout.from_workload(w, synth.unit_bits(w))
    pool = stq.StqPool(None, 0, 8, L.handle)
    lib = stq.library()

    def check(ids):
        a = np.ascontiguousarray(ids, dtype=np.int32)
        return lib.stq_check_slot_ids(C.byref(pool), a.size, C.c_void_p(a.ctypes.data))

    assert check([3, 0, 7, 1]) == stq.STQ_OK
    assert check(np.arange(8)[::-1]) == stq.STQ_OK
    assert check([]) == stq.STQ_OK
    assert check([2, 5, 2]) == stq.STQ_ERR_INVALID
    assert b"position 2" in lib.stq_last_error() and b"twice" in lib.stq_last_error()
    assert check([1, -1]) == stq.STQ_ERR_INVALID
    assert b"position 1" in lib.stq_last_error()
    assert check([0, 8]) == stq.STQ_ERR_INVALID
    assert b"outside [0, 8)" in lib.stq_last_error()
    # more ids than slots is a bad batch before any id is read
    assert lib.stq_check_slot_ids(C.byref(pool), 9, None) == stq.STQ_ERR_INVALID
    # the binding raises with the library's text
    with pytest.raises(stq.StqError, match="twice"):
        class _P:  # a pool-like object over the same view
            pass
        p = _P()
        p.pool = pool
        stq.check_slot_ids(p, [4, 4])


def test_debug_validate_library_loads_and_exports(stq):
    """The STQ_DEBUG_VALIDATE build (the same kernels, a host side that
    checks slot ids before every launch) loads and exports every declared
    function."""
    path = os.path.join(ROOT, "linear_attention_recurrent_stq_amd", "libstq_debug.so")
    lib = C.CDLL(path)
    for name in stq.SYMBOLS:
        assert hasattr(lib, name), name


def test_lagged_scale_validation(stq):
    """Lagged scales need the every-step mode and heads whose key rows share a
    width; stq_fit_scales rejects a layout without lagged scales before
    launching anything."""
    bits = np.full(4, 4, np.uint8)
    with pytest.raises(stq.StqError, match="every-step"):
        stq.Layout(4, 128, 128, bits, window=4, scale_fit=stq.FIT_LAGGED)
    kb = np.full(4 * 128, 4, np.uint8)
    kb[7] = 16
    with pytest.raises(stq.StqError, match="one width"):
        stq.Layout(4, 128, 128, kb, unit=stq.UNIT_KEYROW, gate=stq.GATE_KEYVEC, scale_fit=stq.FIT_LAGGED)
    with pytest.raises(stq.StqError, match="scale_fit"):
        stq.Layout(4, 128, 128, bits, scale_fit=7)
    # uniform key rows per head (different widths across heads) are accepted
    kb = np.repeat(np.array([4, 6, 8, 16], np.uint8), 128)
    L = stq.Layout(4, 128, 128, kb, unit=stq.UNIT_KEYROW, gate=stq.GATE_KEYVEC, scale_fit=stq.FIT_LAGGED)
    assert L.slot_bytes > 0
    plain = stq.Layout(4, 128, 128, bits)
    fake = stq.StqPool(C.c_void_p(1 << 20), 0, 4, plain.handle)
    ids = np.zeros(1, np.int32)
    lib = stq.library()
    assert lib.stq_fit_scales(C.byref(fake), 0, C.c_void_p(ids.ctypes.data), None) == stq.STQ_ERR_INVALID
    assert b"no lagged scales" in lib.stq_last_error()


def test_lagged_layout_matches_oracle(stq, ora):
    """Slot layout of lagged-scale heads (next scales and statistics after the
    column scales) equals the oracle's, for fp16 and fp32 row scales, with and
    without column scales."""
    for rs, cs in ((stq.F16, stq.F16), (stq.F32, stq.NONE)):
        bits = np.array([4, 6, 8, 16, 32], np.uint8)
        L = stq.Layout(5, 128, 64, bits, row_scale=rs, col_scale=cs, scale_fit=stq.FIT_LAGGED)
        o = ora.Cfg(5, 128, 64, False, False, rs == stq.F16, cs == stq.F16, 1, 0, bits, scale_fit=1)
        assert L.slot_bytes == o.slot_bytes
        for h in range(5):
            assert L.head(h) == (o.head_layout(h)["base"], o.head_layout(h)["bytes"])


def test_row_impact_validation(stq):
    """Row-impact scores: negative or non-finite scores are rejected; the
    windowed mode and lagged scales take none; the weights add H*d_k floats
    to the pool's table header."""
    bits = np.full(4, 4, np.uint8)
    good = np.ones(4 * 128, np.float32)
    plain = stq.Layout(4, 128, 128, bits)
    L = stq.Layout(4, 128, 128, bits, row_impact=good)
    assert L.slot_bytes == plain.slot_bytes
    groups = 2  # four 4-bit heads in two pairs
    assert plain.header_bytes == (64 * 4 + 4 * 4 * 128 + 4 * groups + 255) // 256 * 256
    assert L.header_bytes == (64 * 4 + 4 * 4 * 128 + 4 * groups + 4 * 4 * 128 + 255) // 256 * 256
    for bad in (-1.0, np.nan, np.inf):
        b = good.copy()
        b[17] = bad
        with pytest.raises(stq.StqError, match="row_impact"):
            stq.Layout(4, 128, 128, bits, row_impact=b)
    with pytest.raises(stq.StqError, match="row-impact"):
        stq.Layout(4, 128, 128, np.full(4, 8, np.uint8), window=4, row_impact=good)
    with pytest.raises(stq.StqError, match="row-impact"):
        stq.Layout(4, 128, 128, bits, scale_fit=stq.FIT_LAGGED, row_impact=good)
