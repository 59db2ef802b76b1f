"""HIP path vs the CPU oracle through the C ABI, on seeded inputs.

Bar: slot bytes (codes, scales, pivots) identical to the oracle's, and every
output vector within max relative error 1e-4 (the arithmetic is specified to
the rounding, so both are expected to be exact; the bar is what is asserted).
"""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

O_TOL = 1e-4


def _harness(*a, **k):
    from tests.parity import Harness
    return Harness(*a, **k)


def _check_step(o_gpu, o_ref, follow, t, tag):
    """Every output element within relative error O_TOL of the oracle's,
    element by element (|x - y| <= O_TOL |y|; exact where y = 0)."""
    x = np.asarray(o_gpu, np.float64)
    y = np.asarray(np.stack(o_ref) if len(o_ref) else np.zeros_like(x), np.float64)
    bad = np.abs(x - y) > O_TOL * np.abs(y)
    if bad.any():
        n = int(np.nonzero(bad.any(axis=1))[0][0])
        b, h = follow[n]
        e = float(np.max(np.abs(x[n] - y[n]) / np.maximum(np.abs(y[n]), 1e-300)))
        raise AssertionError(f"{tag}: o mismatch at step {t}, unit (b={b}, h={h}): rel err {e:.3g}")
    return 0.0


def _run(w, T, follow=None, bits=None, check_slots_every=0, tag="", row_impact=None):
    print(f"[{tag}] {w.name} B={w.B} H={w.H} d={w.dk} T={T}", flush=True)
    hs = _harness(w, follow=follow, bits=bits, row_impact=row_impact)
    try:
        hs.init_state()
        if w.init != "zero":
            bad = hs.compare_slots()
            assert not bad, f"{tag}: packed initial state differs: {bad[:4]}"
        for t in range(T):
            if follow is None:
                x = hs.load_full(t)
                o_gpu, o_ref = hs.step(x)
            else:
                x = hs.load_followed(t)
                o_gpu, o_ref = hs.step(x, idx_in_x=True)
            _check_step(o_gpu, o_ref, hs.follow, t, tag)
            if check_slots_every and (t + 1) % check_slots_every == 0:
                bad = hs.compare_slots()
                assert not bad, f"{tag}: slot bytes differ after step {t}: {bad[:4]}"
        bad = hs.compare_slots()
        assert not bad, f"{tag}: slot bytes differ after {T} steps: {bad[:4]}"
        return hs
    finally:
        hs.close()


def test_tiny_gdn_every_step():
    """B=4, H=2, d=64, uniform 6-bit, fp32 row scales, fp32 io: all units, all 16 steps."""
    _run(synth.WORKLOADS["tiny_gdn"], 16, check_slots_every=1, tag="tiny")


def test_qwen_gdn_mixed_widths_small_batch():
    """Per-head 4/6/8-bit and an FP16 pivot head, bf16 io, B=8, 24 steps, all units."""
    w = synth.WORKLOADS["qwen_gdn"].with_(B=8)
    _run(w, 24, check_slots_every=8, tag="qwen-small")


def test_kimi_kda_outliers_small_batch():
    """Per-key-row widths (4-bit + FP16 pivot rows), vector gate, outlier start."""
    w = synth.WORKLOADS["kimi_kda"].with_(B=4)
    _run(w, 24, check_slots_every=8, tag="kimi-small")


def test_mixed_row_widths_d64():
    """KDA rows of every width {4,6,8,16} in one state, d=64: the per-row path."""
    w = synth.WORKLOADS["kimi_kda"].with_(B=3, H=4, dk=64, dv=64, name="kda_mixed_d64")
    rng = np.random.default_rng(0)
    bits = rng.choice(np.array([4, 6, 8, 16], np.uint8), w.H * w.dk, p=[0.4, 0.25, 0.25, 0.1])
    _run(w, 20, bits=bits, check_slots_every=5, tag="kda-mixed")


def test_allocated_row_widths_d128():
    """KDA key-row widths from stq_allocate_bits (seeded gate means and state
    magnitudes, mean 6 bits, 1 % pivots): rows of 4, 6, 8 and 16 bits mixed
    within each d = 128 head; every unit over 12 steps from the outlier
    start, slot bytes compared every 4 steps."""
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS["kimi_kda"].with_(B=6, name="kda_allocated")
    rng = np.random.default_rng(7)
    n = w.H * w.dk
    gate = (0.8 + 0.2 / (1 + np.exp(-rng.normal(2, 1, n)))).astype(np.float32)
    msq = rng.lognormal(-2.0, 1.5, n).astype(np.float32)
    bits = stq.allocate_bits(gate, msq, 6.0, n // 100)
    per_head = bits.reshape(w.H, w.dk)
    assert sum(len(set(r.tolist())) > 2 for r in per_head) > w.H // 2  # mixed heads
    _run(w, 12, bits=bits, check_slots_every=4, tag="kda-allocated")


def _run_sampled(w, T, n_units, seed, layer=0, track=False, tag="", follow=None, bits=None,
                 row_impact=None):
    """Full batch on the GPU; n_units seeded (request, head) units (or the
    given list) followed by the oracle over T steps (the others keep their
    first inputs)."""
    if follow is None:
        rng = np.random.default_rng(seed)
        follow = set()
        while len(follow) < n_units:
            follow.add((int(rng.integers(0, w.B)), int(rng.integers(0, w.H))))
    follow = sorted(follow)
    print(f"[{tag}] {w.name} layer {layer}: {len(follow)} followed units of B={w.B} x H={w.H}, "
          f"T={T}", flush=True)
    hs = _harness(w, layer=layer, follow=follow, bits=bits, row_impact=row_impact)
    try:
        if track:
            hs.track_fp32()
        hs.init_state()
        hs.load_full(0)
        for t in range(T):
            x = hs.load_followed(t)
            o_gpu, o_ref = hs.step(x, idx_in_x=True)
            _check_step(o_gpu, o_ref, hs.follow, t, tag)
            if (t + 1) % 64 == 0:
                print(f"[{tag}] step {t + 1} ok", flush=True)
        bad = hs.compare_slots()
        assert not bad, f"{tag}: slot bytes differ after {T} steps: {bad[:4]}"
        return hs
    finally:
        hs.close()


def test_kda_4bit_rows_with_pivot_rows():
    """KDA heads whose rows are 4-bit or FP16 pivots, with 8-row blocks holding
    0, 1, 2 and 3 pivot rows (a thread owns one such block), a head without
    pivot rows and an all-pivot head; d=128 and d=64."""
    for d in (128, 64):
        w = synth.WORKLOADS["kimi_kda"].with_(B=3, H=4, dk=d, dv=d, name=f"kda_4p_d{d}")
        bits = np.full((w.H, d), 4, np.uint8)
        bits[0, [0, 1, 9, 12, 13, 14, 40, d - 1]] = 16
        bits[1, 5] = 16
        bits[3, :] = 16
        _run(w, 12, bits=bits.ravel(), check_slots_every=4, tag=f"kda-4p-d{d}")


def test_fp32_heads():
    """fp32 (unquantized) heads: the serving shape with every head fp32, and a
    layout mixing fp32, 4/6/8-bit and FP16 pivot heads; all units, slot bytes
    compared every few steps; stq_unpack of the mixed layout, and of a
    key-row layout whose units are all fp32 rows, equals the oracle's (a
    width of 32 in the row table once read back as 0)."""
    _run(synth.WORKLOADS["serving_fp32"].with_(B=16), 8, check_slots_every=4, tag="fp32")
    w = synth.WORKLOADS["qwen_gdn"].with_(B=6, H=6, name="qwen_mixed_fp32")
    bits = np.array([32, 4, 16, 6, 32, 8], np.uint8)
    hs = _run(w, 10, bits=bits, check_slots_every=5, tag="fp32-mixed")
    wk = synth.WORKLOADS["kimi_kda"].with_(B=3, H=4, init="zero", name="kda_fp32")
    bk = np.full(wk.H * wk.dk, 32, np.uint8)
    bk[wk.dk:2 * wk.dk] = 4
    for w_, b_, steps in ((w, bits, 10), (wk, bk, 6)):
        h2 = _harness(w_, bits=b_)
        try:
            for t in range(steps):
                h2.step(h2.load_full(t))
            got = h2.unpack_gpu()
            for b, h in h2.follow:
                assert np.array_equal(got[b, h], h2.ocfg.unpack_head(h2.oslots[b], h)), (w_.name, b, h)
        finally:
            h2.close()


def test_qwen_gdn_all_units_all_steps():
    """B=64 x H=32, heads of 4/6/8 bits and an FP16 pivot head: every unit, all 256 steps."""
    _run(synth.WORKLOADS["qwen_gdn"], 256, check_slots_every=64, tag="qwen-all")


def test_serving_gdn_all_units_16_steps():
    """B=512 x H=32 (16,384 states, 31 four-bit heads + 1 pivot head): all units, 16 steps."""
    _run(synth.WORKLOADS["serving_gdn"], 16, check_slots_every=8, tag="serving-all")


def test_serving_gdn_sampled_units_all_2048_steps():
    """Full serving batch, 64 followed units of layer 1 over all 2048 steps; the
    distance of the quantized output from the unquantized fp32 recurrence is
    tracked (reported, not a parity bar: it is the method's quantization error)."""
    w = synth.WORKLOADS["serving_gdn"]
    hs = _run_sampled(w, w.T, 64, seed=11, layer=1, track=True, tag="serving-long")
    e = np.array(hs.shadow_err)
    print(f"[serving-long] quantized vs fp32 output, max over units per step: "
          f"median {np.median(e):.3g}, p90 {np.percentile(e, 90):.3g}, max {e.max():.3g}", flush=True)
    assert np.isfinite(e).all()


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64), (64, 64)])
def test_paired_heads_other_head_sizes(dk, dv):
    """4-bit GDN heads in pairs (batch of 256 x 32 states) at the other head
    sizes: 64 followed units over 12 steps, slot bytes compared at the end."""
    w = synth.WORKLOADS["serving_gdn"].with_(B=256, dk=dk, dv=dv, name=f"serving_{dk}x{dv}")
    _run_sampled(w, 12, 64, seed=20 + dk + dv, tag=f"pairs-{dk}x{dv}")


def _both_kinds_bits(d):
    """Eight KDA heads: 4-bit rows with FP16 pivot rows (blocks of 8 rows
    holding 0 to 8 pivots), heads of 4-bit rows only, and an all-pivot head."""
    bits = np.full((8, d), 4, np.uint8)
    bits[0, [0, 1, 9, 12, 13, 14, 40, d - 1]] = 16
    bits[1, 5] = 16
    bits[3, :] = 16
    bits[4, [2, 3, 4, d // 2, d - 3]] = 16
    bits[5, d - 1] = 16
    bits[7, 8:16] = 16
    return bits


def _expected_groups(bits):
    """Heads whose rows are all 4-bit in pairs, in head order, first; then
    every other head alone, in head order; an unpaired 4-bit head last."""
    pairs, singles, pending = [], [], None
    for h, r in enumerate(bits):
        if not (r == 4).all():
            singles.append((h, 0xFFFF))
        elif pending is None:
            pending = h
        else:
            pairs.append((pending, h))
            pending = None
    if pending is not None:
        singles.append((pending, 0xFFFF))
    return pairs + singles


@pytest.mark.parametrize("d", [128, 64])
def test_pivot_row_heads_in_a_paired_batch(d):
    """A batch large enough for paired heads (1024 x 8 states) of KDA heads
    with 4-bit and FP16 pivot rows (pivot masks and head groups read back from
    the pool header), 4-bit heads (paired) and an all-pivot head: every head
    of 3 requests followed over 12 steps from the outlier start, slot bytes
    compared."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS["kimi_kda"].with_(B=1024, H=8, dk=d, dv=d, name=f"kda_pairs_d{d}")
    bits = _both_kinds_bits(d)
    L = stq.Layout.from_workload(w, bits.ravel())
    pool = stq.Pool(L, 1)
    hdr = pool.buffer[:L.header_bytes].cpu().numpy()
    desc = hdr[:64 * w.H].view(np.uint32).reshape(w.H, 16)
    for h in range(w.H):
        r = bits[h]
        w4p = np.isin(r, (4, 16)).all() and (r == 4).any() and (r == 16).any()
        want = np.zeros(4, np.uint32)
        if w4p:
            for i in np.nonzero(r == 16)[0]:
                want[i // 32] |= np.uint32(1 << (i % 32))
        assert (desc[h, 12:16] == want).all(), f"pivot mask of head {h}"
    want = _expected_groups(bits)
    g0 = 64 * w.H + 4 * w.H * d
    got = hdr[g0:g0 + 4 * len(want)].view(np.uint32)
    assert [(int(x) & 0xFFFF, int(x) >> 16) for x in got] == want
    del pool
    follow = [(b, h) for b in (0, 517, 1023) for h in range(w.H)]
    _run_sampled(w, 12, 0, seed=0, follow=follow, bits=bits.ravel(), tag=f"pairs-4p-d{d}")


def test_paired_heads_fp32_inputs_and_scales():
    """Paired 4-bit heads (256 x 32 states) with fp32 q/k/v, fp32 row scales
    and no column scales: the other input and scale types on the prefetch
    path; 64 followed units over 10 steps, slot bytes compared."""
    w = synth.WORKLOADS["serving_gdn"].with_(B=256, io="f32", row_scale="f32", col_scale="none",
                                             name="serving_f32_io")
    _run_sampled(w, 10, 64, seed=41, tag="pairs-f32")


def test_largest_head_count():
    """H = 4096 (the largest the layout accepts), d = 64, B = 2: 8192 states,
    so 4-bit heads are paired across a 2,000-group table with head indices up
    to 4095; 96 followed units over 6 steps, slot bytes compared."""
    w = synth.WORKLOADS["serving_gdn"].with_(B=2, H=4096, dk=64, dv=64, name="serving_h4096")
    _run_sampled(w, 6, 96, seed=31, tag="h4096")


@pytest.mark.parametrize("half", [0, 1])
def test_kimi_kda_all_units_all_256_steps(half):
    """B=256 x H=32 KDA (4-bit rows + 41 FP16 pivot rows), outlier start:
    every unit over all 256 steps (each half of the requests in its own test,
    the whole batch on the GPU), slot bytes compared at the end."""
    w = synth.WORKLOADS["kimi_kda"]
    reqs = range(half * w.B // 2, (half + 1) * w.B // 2)
    _run_sampled(w, w.T, 0, 0, follow=[(b, h) for b in reqs for h in range(w.H)],
                 tag=f"kimi-all-{half}")


def test_kimi_kda_sampled_units_all_256_steps():
    """Full KDA batch, 256 followed units over all 256 steps."""
    w = synth.WORKLOADS["kimi_kda"]
    _run_sampled(w, w.T, 256, seed=12, tag="kimi-long")


def test_kimi_serving_sampled_units():
    """The KDA layer at serving scale (B=512, 4-bit rows with FP16 pivot
    rows, layers 0 and 3 of four, whose pivot maps differ): 128 followed units
    over 64 steps each, slot bytes compared at the end."""
    w = synth.WORKLOADS["kimi_serving"]
    for layer in (0, 3):
        _run_sampled(w, 64, 128, seed=71 + layer, layer=layer, tag=f"kimi-serving-{layer}")


def test_unpack_and_pack_match_oracle():
    """stq_unpack equals the oracle's dequantization; stq_pack of a random fp32
    state gives the oracle's bytes (mixed widths, pivots, outliers)."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS["kimi_kda"].with_(B=4)
    hs = _harness(w)
    try:
        hs.init_state()
        for t in range(3):
            hs.step(hs.load_full(t))
        got = hs.unpack_gpu()
        for b, h in hs.follow:
            want = hs.ocfg.unpack_head(hs.oslots[b], h)
            assert np.array_equal(got[b, h], want), (b, h)
        rng = np.random.default_rng(3)
        M = (rng.standard_normal((w.B, w.H, w.dk, w.dv)) * 0.3).astype(np.float32)
        stq.pack(hs.pool, hs.slot_ids, torch.from_numpy(M).cuda())
        for b, h in hs.follow:
            hs.ocfg.pack_head(hs.oslots[b], h, M[b, h])
        assert not hs.compare_slots()
    finally:
        hs.close()


def _saturated_rows(hs) -> int:
    """Quantized rows of the followed units (oracle side) whose fp16 row scale
    is 65504, the largest fp16."""
    n = 0
    for b, h in hs.follow:
        lay = hs.ocfg.head_layout(h)
        if lay["nquant"] == 0:
            continue
        lo = lay["base"] + lay["rs"]
        n += int((hs.oslots[b][lo:lo + 2 * hs.w.dk].view(np.uint16) == 0x7BFF).sum())
    return n


@pytest.mark.parametrize("name", ["serving_gdn", "qwen_gdn", "kimi_kda"])
def test_saturated_rows_clamp_codes(name):
    """Rows beyond the fp16 range: a packed state with rows of ~1e11 and steps
    whose v are scaled by 2^40 push row scales to 65504, where codes are
    clamped to +-qmax.  Every unit's slot bytes after pack and after every
    step, and every output, equal the oracle's (4-bit pairs and a pivot head;
    4/6/8-bit heads; 4-bit rows with FP16 pivot rows)."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS[name].with_(B=4, layers=1)
    print(f"[saturated] {w.name} B={w.B}", flush=True)
    hs = _harness(w)
    try:
        rng = np.random.default_rng(7)
        M = (rng.standard_normal((w.B, w.H, w.dk, w.dv)) * 0.3).astype(np.float32)
        big = np.float32(2.0 ** 40)
        M[:, :, 3] *= big
        M[:, :, 77] *= big
        stq.pack(hs.pool, hs.slot_ids, torch.from_numpy(M).cuda())
        for b, h in hs.follow:
            hs.ocfg.pack_head(hs.oslots[b], h, M[b, h])
        assert not hs.compare_slots()
        assert _saturated_rows(hs) > 0
        sat_steps = 0
        for t in range(6):
            x = hs.load_full(t)
            if t in (1, 3):
                # v of requests 0 and 2 times 2^40 (exact: a power of two)
                x.v[[0, 2]] *= big
                if x.v_bits is not None:
                    x.v_bits[[0, 2]] = (x.v[[0, 2]].view(np.uint32) >> 16).astype(np.uint16)
                _, _, v = hs._to_dev(x)
                hs.v.copy_(v)
            o_gpu, o_ref = hs.step(x)
            _check_step(o_gpu, o_ref, hs.follow, t, "saturated")
            bad = hs.compare_slots()
            assert not bad, f"slot bytes differ after step {t}: {bad[:4]}"
            sat_steps += _saturated_rows(hs) > 0
        assert sat_steps >= 2
    finally:
        hs.close()


def test_invalid_slot_id_touches_nothing():
    """An out-of-range slot id yields a NaN output and leaves every slot unchanged."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS["qwen_gdn"].with_(B=4)
    hs = _harness(w)
    try:
        hs.load_full(0)
        hs.step(hs.load_full(0))
        before = hs.slot_bytes_gpu()
        ids = hs.slot_ids.clone()
        ids[2] = 1000
        stq.decode_step(hs.pool, ids, hs.q, hs.k, hs.v, hs.a, hs.beta, hs.o)
        torch.cuda.synchronize()
        o = hs.o.cpu().numpy()
        assert np.isnan(o[2]).all() and np.isfinite(o[[0, 1, 3]]).all()
        after = hs.slot_bytes_gpu()
        assert np.array_equal(before[hs.slot_of[2]], after[hs.slot_of[2]])
        assert np.array_equal(before[np.setdiff1d(np.arange(4), hs.slot_of[[0, 1, 3]])],
                              after[np.setdiff1d(np.arange(4), hs.slot_of[[0, 1, 3]])])
    finally:
        hs.close()


def test_invalid_slot_id_in_paired_heads():
    """A batch large enough for paired 4-bit heads (256 x 32 states): an
    invalid slot id gives NaN outputs for every head of that request (paired
    or not) and leaves the pool unchanged; the other requests match the
    oracle."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS["serving_gdn"].with_(B=256)
    follow = [(b, h) for b in (0, 7, 255) for h in range(w.H)]
    hs = _harness(w, follow=follow)
    try:
        hs.load_full(0)
        o_gpu, o_ref = hs.step(hs.load_followed(0), idx_in_x=True)
        _check_step(o_gpu, o_ref, hs.follow, 0, "paired-invalid")
        before = hs.slot_bytes_gpu()
        ids = hs.slot_ids.clone()
        ids[7] = -3
        stq.decode_step(hs.pool, ids, hs.q, hs.k, hs.v, hs.a, hs.beta, hs.o)
        torch.cuda.synchronize()
        o = hs.o.cpu().numpy()
        assert np.isnan(o[7]).all()
        assert np.isfinite(o[[0, 255]]).all()
        after = hs.slot_bytes_gpu()
        assert np.array_equal(before[hs.slot_of[7]], after[hs.slot_of[7]])
    finally:
        hs.close()


def test_deterministic_and_batch_independent():
    """Same inputs twice give identical bytes; a request's result does not
    depend on which other requests share the call (B=1 vs B=5)."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS["qwen_gdn"].with_(B=5)
    outs = []
    for rep in range(2):
        hs = _harness(w)
        try:
            for t in range(4):
                hs.step(hs.load_full(t))
            outs.append(hs.slot_bytes_gpu())
            if rep == 1:
                # replay request 3 alone into a fresh 1-slot pool
                L = hs.L
                p1 = stq.Pool(L, 1)
                ids = torch.zeros(1, dtype=torch.int32, device="cuda")
                o1 = torch.empty(1, w.H, w.dv, device="cuda")
                for t in range(4):
                    x = synth.batch_inputs(w, 0, t)
                    q, k, v = (hs._to_dev(x))
                    stq.decode_step(p1, ids, q[3:4].cuda().contiguous(), k[3:4].cuda().contiguous(),
                                    v[3:4].cuda().contiguous(), torch.from_numpy(x.a[3:4]).cuda(),
                                    torch.from_numpy(x.beta[3:4]).cuda(), o1)
                alone = p1.slots_view().cpu().numpy()[0]
                assert np.array_equal(alone, outs[1][hs.slot_of[3]])
        finally:
            hs.close()
    assert np.array_equal(outs[0], outs[1])


def test_empty_batch_is_a_noop():
    import torch
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS["tiny_gdn"]
    hs = _harness(w)
    try:
        before = hs.slot_bytes_gpu()
        e = torch.empty(0, dtype=torch.int32, device="cuda")
        z = lambda *s, dt=torch.float32: torch.empty(*s, dtype=dt, device="cuda")
        stq.decode_step(hs.pool, e, z(0, 2, 64), z(0, 2, 64), z(0, 2, 64), z(0, 2), z(0, 2), z(0, 2, 64))
        torch.cuda.synchronize()
        assert np.array_equal(before, hs.slot_bytes_gpu())
    finally:
        hs.close()


# ------------------------------------------------------------ windowed mode

def test_windowed_kda_all_units_two_and_a_half_windows():
    """8-bit KDA state requantized every 16 tokens with 82 fp32 compensation
    entries per state: every unit of B=4 x H=32 over 40 steps (two window ends),
    slot bytes compared after each window end."""
    w = synth.WORKLOADS["windowed_kda"].with_(B=4)
    _run(w, 40, check_slots_every=8, tag="win-kda")


def test_windowed_mixed_rows_d64():
    """Windowed mode with key rows of every width (and pivot rows), d=64, W=4."""
    w = synth.WORKLOADS["windowed_kda"].with_(B=3, H=4, dk=64, dv=64, window=4, comps=10,
                                              name="win_mixed_d64")
    rng = np.random.default_rng(5)
    bits = rng.choice(np.array([4, 6, 8, 16], np.uint8), w.H * w.dk, p=[0.4, 0.25, 0.25, 0.1])
    _run(w, 13, bits=bits, check_slots_every=1, tag="win-mixed")


def test_windowed_mixed_rows_d128():
    """Windowed mode with key rows of every width {4,6,8,16} in each d = 128
    head (the per-row in-window and window-end kernels), W = 16, K = 82:
    every unit of 4 x 4 states over 40 steps (two window ends), slot bytes
    compared every 8 steps."""
    w = synth.WORKLOADS["windowed_kda"].with_(B=4, H=4, name="win_mixed_d128")
    rng = np.random.default_rng(6)
    bits = rng.choice(np.array([4, 6, 8, 16], np.uint8), w.H * w.dk, p=[0.4, 0.25, 0.25, 0.1])
    _run(w, 40, bits=bits, check_slots_every=8, tag="win-mixed-d128")


@pytest.mark.parametrize("d,W", [(64, 4), (128, 16)])
def test_windowed_staggered_windows(d, W):
    """Requests whose windows close at different calls: call c steps only the
    requests b with (b + c) % 3 != 0, so within one call some states fill
    their window and others do not, and many calls end no window at all (the
    window-end kernel is told by the pool's flag which calls to skip).  Every
    unit of 6 x 4 states, outputs at every call and slot bytes every 5 calls,
    against the oracle."""
    import torch
    import oracle
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS["windowed_kda"].with_(B=6, H=4, dk=d, dv=d, window=W, comps=10 if d == 64 else 82,
                                              name=f"win_staggered_d{d}")
    bits = synth.unit_bits(w)
    L = stq.Layout.from_workload(w, bits)
    ocfg = oracle.Cfg.from_workload(w, bits)
    pool = stq.Pool(L, w.B)
    slot_of = np.array([3, 0, 5, 1, 4, 2], np.int32)
    oslots = [ocfg.new_slot() for _ in range(w.B)]
    bb, hh = np.meshgrid(np.arange(w.B), np.arange(w.H), indexing="ij")
    M0 = synth.initial_state(w, 0, bb, hh)
    stq.pack(pool, torch.from_numpy(slot_of).cuda(), torch.from_numpy(M0).cuda())
    for b in range(w.B):
        for h in range(w.H):
            ocfg.pack_head(oslots[b], h, M0[b, h])
    cv = lambda bits_: torch.from_numpy(np.ascontiguousarray(bits_).view(np.int16)).view(torch.bfloat16).cuda()
    calls = 3 * W + 6
    ends = 0
    for c in range(calls):
        sub = np.array([b for b in range(w.B) if (b + c) % 3 != 0], np.int64)
        x = synth.batch_inputs(w, 0, c)
        ids = torch.from_numpy(slot_of[sub]).cuda()
        o = torch.empty(len(sub), w.H, w.dv, device="cuda")
        stq.decode_step(pool, ids, cv(x.q_bits[sub]), cv(x.k_bits[sub]), cv(x.v_bits[sub]),
                        torch.from_numpy(np.ascontiguousarray(x.a[sub])).cuda(),
                        torch.from_numpy(np.ascontiguousarray(x.beta[sub])).cuda(), o)
        got = o.cpu().numpy()
        ref = []
        for n, b in enumerate(sub):
            for h in range(w.H):
                ref.append(ocfg.step_head(oslots[b], h, x.q[b, h], x.k[b, h], x.v[b, h], x.a[b, h],
                                          x.beta[b, h]))
        follow = [(int(b), h) for b in sub for h in range(w.H)]
        _check_step(got.reshape(-1, w.dv), ref, follow, c, f"staggered-d{d}")
        ends += sum(1 for b in sub if sum(1 for cc in range(c + 1) if (b + cc) % 3 != 0) % W == 0)
        if (c + 1) % 5 == 0 or c == calls - 1:
            allb = pool.slots_view().cpu().numpy()
            for b in range(w.B):
                assert np.array_equal(allb[slot_of[b]], oslots[b]), f"slot bytes of request {b} after call {c}"
    assert ends >= w.B  # every request closed at least one window, at differing calls


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_windowed_unequal_head_sizes(dk, dv):
    """Windowed mode at d_k != d_v (uniform 8-bit rows, and rows of mixed
    widths), W = 8, K = 41: every unit over 20 steps, slot bytes compared
    every 4 steps."""
    w = synth.WORKLOADS["windowed_kda"].with_(B=3, H=4, dk=dk, dv=dv, window=8, comps=41,
                                              name=f"win_{dk}x{dv}")
    _run(w, 20, check_slots_every=4, tag=f"win-{dk}x{dv}")
    rng = np.random.default_rng(dk + dv)
    bits = rng.choice(np.array([4, 6, 8, 16], np.uint8), w.H * w.dk, p=[0.4, 0.25, 0.25, 0.1])
    _run(w.with_(name=f"win_{dk}x{dv}_mixed"), 20, bits=bits, check_slots_every=4,
         tag=f"win-{dk}x{dv}-mixed")


@pytest.mark.parametrize("K", [300, 1024])
def test_windowed_many_entries(K):
    """More compensation entries than threads of a workgroup (K > 256 at
    d = 128: the whole-state selection path and several entries per thread),
    up to the 1024 the layout accepts: every unit of 2 x 4 states over 36
    steps from the outlier start (two window ends), slot bytes compared every
    4 steps."""
    w = synth.WORKLOADS["windowed_kda"].with_(B=2, H=4, comps=K, name=f"win_k{K}")
    _run(w, 36, check_slots_every=4, tag=f"win-k{K}")


@pytest.mark.parametrize("dk,dv", [(128, 64), (64, 128)])
def test_mixed_row_widths_unequal_head_sizes(dk, dv):
    """Every-step mode with rows of every width {4,6,8,16} at d_k != d_v (the
    generic per-row path), and 4-bit rows with FP16 pivot rows (the pivot-row
    class): every unit over 12 steps, slot bytes compared every 4 steps."""
    w = synth.WORKLOADS["kimi_kda"].with_(B=3, H=4, dk=dk, dv=dv, name=f"kda_mixed_{dk}x{dv}")
    rng = np.random.default_rng(3 * dk + dv)
    bits = rng.choice(np.array([4, 6, 8, 16], np.uint8), w.H * w.dk, p=[0.4, 0.25, 0.25, 0.1])
    _run(w, 12, bits=bits, check_slots_every=4, tag=f"kda-mixed-{dk}x{dv}")
    bits = np.where(rng.random(w.H * w.dk) < 0.1, 16, 4).astype(np.uint8)
    _run(w.with_(name=f"kda_4p_{dk}x{dv}"), 12, bits=bits, check_slots_every=4, tag=f"kda-4p-{dk}x{dv}")


def test_windowed_zero_state_ties():
    """From the empty state every |M| ties at 0 in the first window's selection
    (and in pack): the lowest indices must win, exactly as in the oracle."""
    w = synth.WORKLOADS["windowed_kda"].with_(B=2, H=4, window=2, comps=40, init="zero",
                                              name="win_zero")
    hs = _harness(w)
    try:
        import torch
        import linear_attention_recurrent_stq_amd as stq
        zero = np.zeros((w.B, w.H, w.dk, w.dv), np.float32)
        stq.pack(hs.pool, hs.slot_ids, torch.from_numpy(zero).cuda())
        for b, h in hs.follow:
            hs.ocfg.pack_head(hs.oslots[b], h, zero[b, h])
        assert not hs.compare_slots()
        for t in range(5):
            o_gpu, o_ref = hs.step(hs.load_full(t))
            _check_step(o_gpu, o_ref, hs.follow, t, "win-zero")
            assert not hs.compare_slots(), t
    finally:
        hs.close()


@pytest.mark.parametrize("d", [128, 64])
def test_windowed_tied_outliers(d):
    """Selections whose K-th magnitude is tied among candidates: per state,
    N(0, 0.1^2) entries plus 30 entries of magnitude 5 and 200 of magnitude
    3 (random signs and places), so the 82 entries (40 at d = 64) take the
    30 largest and, of the 200 ties, those of lowest index.  Pack, then
    steps across two window ends (W = 4); slot bytes and outputs equal the
    oracle's after every step."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    K = 82 if d == 128 else 40
    w = synth.WORKLOADS["windowed_kda"].with_(B=3, H=4, dk=d, dv=d, window=4, comps=K,
                                              name=f"win_ties_d{d}")
    print(f"[win-ties] d={d} K={K}", flush=True)
    hs = _harness(w)
    try:
        rng = np.random.default_rng(11 + d)
        M = (rng.standard_normal((w.B, w.H, d, d)) * 0.1).astype(np.float32)
        for b in range(w.B):
            for h in range(w.H):
                pos = rng.choice(d * d, 230, replace=False)
                mag = np.where(np.arange(230) < 30, 5.0, 3.0).astype(np.float32)
                sign = np.where(rng.random(230) < 0.5, -1.0, 1.0).astype(np.float32)
                M[b, h].reshape(-1)[pos] = mag * sign
        stq.pack(hs.pool, hs.slot_ids, torch.from_numpy(M).cuda())
        for b, h in hs.follow:
            hs.ocfg.pack_head(hs.oslots[b], h, M[b, h])
        assert not hs.compare_slots()
        for t in range(9):
            o_gpu, o_ref = hs.step(hs.load_full(t))
            _check_step(o_gpu, o_ref, hs.follow, t, "win-ties")
            assert not hs.compare_slots(), t
    finally:
        hs.close()


def test_windowed_unpack_mid_window():
    """stq_unpack of a windowed state with pending deltas materializes
    fma(g, B, D) exactly as the oracle."""
    w = synth.WORKLOADS["windowed_kda"].with_(B=2, H=8)
    hs = _harness(w)
    try:
        hs.init_state()
        for t in range(7):
            hs.step(hs.load_full(t))
        got = hs.unpack_gpu()
        for b, h in hs.follow:
            assert np.array_equal(got[b, h], hs.ocfg.unpack_head(hs.oslots[b], h)), (b, h)
    finally:
        hs.close()


@pytest.mark.parametrize("half", [0, 1])
def test_windowed_all_units_two_windows(half):
    """B=512 x H=32 windowed KDA pool: every unit over the first two windows
    (each half of the requests in its own test, the whole batch on the GPU)."""
    w = synth.WORKLOADS["windowed_kda"]
    reqs = range(half * w.B // 2, (half + 1) * w.B // 2)
    _run_sampled(w, 32, 0, 0, follow=[(b, h) for b in reqs for h in range(w.H)],
                 tag=f"win-all-{half}")


def test_windowed_sampled_units_all_1024_steps():
    """Full windowed batch, 256 followed units over all 1024 steps (64 window ends)."""
    w = synth.WORKLOADS["windowed_kda"]
    _run_sampled(w, w.T, 256, seed=13, tag="win-long")


def test_debug_validate_build_rejects_bad_batches():
    """The STQ_DEBUG_VALIDATE library checks the device slot ids on the host
    before launching: a batch with a repeated id or an id out of range is
    rejected with STQ_ERR_INVALID and the pool is left as it was; a good batch
    steps exactly like the release library."""
    import ctypes as C
    import os
    import torch
    import linear_attention_recurrent_stq_amd as stq
    path = os.path.join(os.path.dirname(stq.__file__), "libstq_debug.so")
    dbg = C.CDLL(path)
    P = C.c_void_p
    dbg.stq_pack_layout.argtypes = [C.POINTER(stq.StqConfig), C.POINTER(P)]
    dbg.stq_alloc_pool.argtypes = [P, C.c_int32, P, C.c_size_t, P, C.POINTER(stq.StqPool)]
    dbg.stq_decode_step.argtypes = [C.POINTER(stq.StqPool), C.c_int32, P, P, P, P, P, P, P, P]
    dbg.stq_last_error.restype = C.c_char_p
    dbg.stq_layout_free.argtypes = [P]
    w = synth.WORKLOADS["qwen_gdn"].with_(B=6)
    hs = _harness(w)
    try:
        x = hs.load_full(0)
        cfg = hs.L.cfg
        h = P()
        assert dbg.stq_pack_layout(C.byref(cfg), C.byref(h)) == stq.STQ_OK
        q = stq.StqPool()
        assert dbg.stq_alloc_pool(h, w.B, None, 0, None, C.byref(q)) == stq.STQ_OK
        buf = torch.empty(q.bytes, dtype=torch.uint8, device="cuda")
        pool = stq.StqPool()
        s = P(torch.cuda.current_stream().cuda_stream)
        assert dbg.stq_alloc_pool(h, w.B, P(buf.data_ptr()), q.bytes, s, C.byref(pool)) == stq.STQ_OK
        ptr = lambda t: P(t.data_ptr())

        def step(ids):
            return dbg.stq_decode_step(C.byref(pool), w.B, ptr(ids), ptr(hs.q), ptr(hs.k), ptr(hs.v),
                                       ptr(hs.a), ptr(hs.beta), ptr(hs.o), s)

        torch.cuda.synchronize()
        before = buf.cpu()
        for bad in ([0, 1, 2, 3, 1, 5], [0, 1, 2, 3, 4, 6], [0, -1, 2, 3, 4, 5]):
            ids = torch.tensor(bad, dtype=torch.int32, device="cuda")
            assert step(ids) == stq.STQ_ERR_INVALID, bad
            print(f"[debug-validate] {bad}: {dbg.stq_last_error().decode()}", flush=True)
            torch.cuda.synchronize()
            assert torch.equal(buf.cpu(), before)
        assert step(hs.slot_ids) == stq.STQ_OK
        hs.step(x)  # the release library on the harness's own pool
        torch.cuda.synchronize()
        hdr = hs.L.header_bytes
        assert torch.equal(buf[hdr:].cpu(), hs.pool.buffer[hdr:].cpu())
        dbg.stq_layout_free(h)
    finally:
        hs.close()


# ------------------------------------------------------------ lagged scales

def test_lagged_scales_small_batches():
    """Lagged scales (the step writes with scales fitted to the previous
    state, stq_fit_scales fits the next ones): every unit, slot bytes (codes,
    scales, next scales, statistics) compared after every step, for 4-bit
    heads with an FP16 pivot head (serving shape, 8 requests), heads of 4, 6
    and 8 bits from a packed outlier state, and fp32 row scales without
    column scales at d = 64 with fp32 inputs."""
    w = synth.WORKLOADS["serving_lagged"].with_(B=8, layers=1)
    _run(w, 20, check_slots_every=1, tag="lagged-serving")
    w = synth.WORKLOADS["qwen_gdn"].with_(B=6, scale_fit="lagged", init="outlier", name="qwen_lagged")
    _run(w, 20, check_slots_every=1, tag="lagged-qwen")
    w = synth.WORKLOADS["tiny_gdn"].with_(scale_fit="lagged", name="tiny_lagged")
    _run(w, 16, check_slots_every=1, tag="lagged-tiny")


def test_lagged_scales_paired_heads():
    """Lagged scales on the paired 4-bit path (512 x 32 states, the serving
    batch): 64 followed units over 48 steps, slot bytes compared at the end;
    and head sizes 128 x 64 and 64 x 128 (256 x 32 states)."""
    w = synth.WORKLOADS["serving_lagged"].with_(layers=1)
    _run_sampled(w, 48, 64, seed=51, tag="lagged-pairs")
    for dk, dv in ((128, 64), (64, 128)):
        w2 = w.with_(B=256, dk=dk, dv=dv, name=f"lagged_{dk}x{dv}")
        _run_sampled(w2, 12, 48, seed=52, tag=f"lagged-{dk}x{dv}")


# ------------------------------------------- calibration and allocated widths

def test_calibration_matches_oracle_and_allocated_widths_step_exactly():
    """The library's calibration pass (the fp32-unit recurrence through the C
    ABI, statistics reduced on the device) gives the oracle's per-row gate
    means and mean squared state entries on the KDA workload whose key rows
    have different lifetimes (8 requests, 48 steps).  The widths the
    allocation oracle gives for them (mean 6 bits, 1 % pivot rows) mix 4, 6,
    8 and 16 bits in every head and favour long-lived rows; the library's
    allocation of the same statistics is identical; and the HIP path steps
    those widths bit for bit like the oracle: every unit of 8 requests over 24
    steps from the outlier start, slot bytes compared every 8 steps."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    from tests.calibration import allocated_bits
    w = synth.WORKLOADS["kda_lifetimes"]
    B, T = 8, 48

    def inputs(t):
        x = synth.step_inputs(w, 0, t, np.arange(B)[:, None], np.arange(w.H)[None, :])
        bf = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
        return (bf(x.q_bits), bf(x.k_bits), bf(x.v_bits), torch.from_numpy(x.a).cuda(),
                torch.from_numpy(x.beta).cuda())

    g_lib, m_lib = stq.calibrate(w.H, w.dk, w.dv, B=B, steps=T, inputs=inputs, unit=stq.UNIT_KEYROW,
                                 gate=stq.GATE_KEYVEC)
    bits, g, m = allocated_bits(w, 0, B, T)
    np.testing.assert_allclose(g_lib, g, rtol=1e-6, atol=0)
    np.testing.assert_allclose(m_lib, m, rtol=1e-5, atol=0)
    assert np.array_equal(stq.allocate_bits(g, m, 6.0, int((bits == 16).sum())), bits)
    per_head = bits.reshape(w.H, w.dk)
    assert sum(len(set(r.tolist())) >= 3 for r in per_head) > w.H // 2
    lt = 1.0 / (1.0 - np.minimum(g.astype(np.float64), 1 - 2 ** -20))
    assert np.median(lt[bits == 8]) > np.median(lt[bits == 4])
    print(f"[allocated] widths {dict(zip(*np.unique(bits, return_counts=True)))}", flush=True)
    _run(w.with_(B=8), 24, bits=bits, check_slots_every=8, tag="allocated")


# ------------------------------------------------------------ row impact

def test_row_impact_weighted_fit():
    """Row-impact-weighted column scales (scores E[q_i^2] from calibration
    queries on the KDA layer whose queries weigh key channels unequally):
    every unit of 4 requests over 24 steps from the outlier start, slot bytes
    compared every 4 steps (4-bit rows with FP16 pivot rows); every unit of a
    6-bit GDN layer with the same scores per head; and the full 256 x 32
    batch with 64 followed units over 64 steps."""
    from tests.calibration import query_impact
    w = synth.WORKLOADS["kimi_impact"]
    iota = query_impact(w, 0, 16, 16)
    assert iota.max() > 20 * iota.min()   # the scores do differ
    _run(w.with_(B=4), 24, check_slots_every=4, tag="impact", row_impact=iota)
    g = synth.WORKLOADS["qwen_gdn"].with_(B=4, bits="uniform6", init="outlier", query_spread=1.0,
                                          name="qwen_impact")
    _run(g, 16, check_slots_every=4, tag="impact-gdn", row_impact=iota)
    _run_sampled(w, 64, 64, seed=61, tag="impact-full", row_impact=iota)


# ------------------------------------------------------------ snapshot / resume

@pytest.mark.parametrize("name,T", [("qwen_gdn", 24), ("windowed_kda", 40), ("serving_lagged", 24)])
def test_snapshot_and_resume(name, T):
    """A slot is the whole state of a request: stepping T steps straight
    through equals stepping T/2, copying the slots' bytes into a fresh pool at
    other slot positions, and stepping T/2 more there (outputs and final
    bytes identical).  Every-step layout; windowed layout resumed in the
    middle of a window; lagged scales (next scales and statistics travel with
    the slot)."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    w = synth.WORKLOADS[name].with_(B=6, layers=1)
    bits = synth.unit_bits(w)
    L = stq.Layout.from_workload(w, bits)
    lagged = getattr(w, "scale_fit", "step") == "lagged"
    io = torch.bfloat16 if w.io == "bf16" else torch.float32

    def inputs(t):
        x = synth.batch_inputs(w, 0, t)
        cv = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).cuda()
        return cv(x.q_bits), cv(x.k_bits), cv(x.v_bits), torch.from_numpy(x.a).cuda(), \
            torch.from_numpy(x.beta).cuda()

    def run(pool, ids, t0, t1, outs):
        o = torch.empty(w.B, w.H, w.dv, device="cuda")
        for t in range(t0, t1):
            stq.decode_step(pool, ids, *inputs(t), o)
            if lagged:
                stq.fit_scales(pool, ids)
            outs.append(o.cpu().numpy().copy())

    def seed(pool, ids):
        if w.init != "zero":
            bb, hh = np.meshgrid(np.arange(w.B), np.arange(w.H), indexing="ij")
            stq.pack(pool, ids, torch.from_numpy(synth.initial_state(w, 0, bb, hh)).cuda())

    ids_a = torch.arange(w.B, dtype=torch.int32, device="cuda")
    straight = stq.Pool(L, w.B)
    seed(straight, ids_a)
    out_a = []
    run(straight, ids_a, 0, T, out_a)

    first = stq.Pool(L, w.B)
    seed(first, ids_a)
    out_b = []
    run(first, ids_a, 0, T // 2, out_b)
    snap = first.slots_view().cpu()                      # request b lives in slot b
    second = stq.Pool(L, w.B + 3)                        # a larger pool, other positions
    where = np.array([7, 0, 4, 2, 8, 5], np.int32)[:w.B]
    view = second.slots_view()
    for b in range(w.B):
        view[int(where[b])].copy_(snap[b].cuda())
    ids_c = torch.from_numpy(where).cuda()
    run(second, ids_c, T // 2, T, out_b)
    torch.cuda.synchronize()
    for t in range(T):
        assert np.array_equal(out_a[t], out_b[t]), (name, t)
    fa, fc = straight.slots_view().cpu().numpy(), second.slots_view().cpu().numpy()
    for b in range(w.B):
        assert np.array_equal(fa[b], fc[int(where[b])]), (name, b)


# ------------------------------------------------------------ graph replay

@pytest.mark.parametrize("name", ["qwen_gdn", "windowed_kda"])
def test_decode_step_in_a_replayed_graph(name):
    """stq_decode_step captured once in a HIP graph and replayed step after
    step (fresh inputs copied in between, eager work and a synchronization
    between replays) gives, at every replay, the same outputs as the same
    call made eagerly on a twin pool, and the same slot bytes at the end.
    Windowed layout (W = 4): the captured call keeps one token, so after its
    first window end the pool's flag holds that token at every replay and
    every window-end workgroup checks its state's count."""
    import torch
    import linear_attention_recurrent_stq_amd as stq
    over = dict(B=4, H=4, layers=1, name=f"graph_{name}")
    if name == "windowed_kda":
        over.update(dk=64, dv=64, window=4, comps=10)
    w = synth.WORKLOADS[name].with_(**over)
    bits = synth.unit_bits(w)
    L = stq.Layout.from_workload(w, bits)
    eager, graphed = stq.Pool(L, w.B), stq.Pool(L, w.B)
    ids = torch.tensor([2, 0, 3, 1], dtype=torch.int32, device="cuda")
    if w.init != "zero":
        bb, hh = np.meshgrid(np.arange(w.B), np.arange(w.H), indexing="ij")
        M0 = torch.from_numpy(synth.initial_state(w, 0, bb, hh)).cuda()
        stq.pack(eager, ids, M0)
        stq.pack(graphed, ids, M0)
    io = torch.bfloat16 if w.io == "bf16" else torch.float32
    q = torch.empty(w.B, w.H, w.dk, dtype=io, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty(w.B, w.H, w.dv, dtype=io, device="cuda")
    a = torch.empty((w.B, w.H, w.dk) if w.gate == "keyvec" else (w.B, w.H), device="cuda")
    beta = torch.empty(w.B, w.H, device="cuda")
    o_e = torch.empty(w.B, w.H, w.dv, device="cuda")
    o_g = torch.empty_like(o_e)

    def load(t):
        x = synth.batch_inputs(w, 0, t)
        cv = lambda b: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
        q.copy_(cv(x.q_bits)); k.copy_(cv(x.k_bits)); v.copy_(cv(x.v_bits))
        a.copy_(torch.from_numpy(x.a)); beta.copy_(torch.from_numpy(x.beta))

    load(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stq.decode_step(graphed, ids, q, k, v, a, beta, o_g)
    torch.cuda.synchronize()
    steps = 3 * w.window + 2 if w.window > 1 else 12
    for t in range(steps):
        load(t)
        stq.decode_step(eager, ids, q, k, v, a, beta, o_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_e, o_g), f"{name}: replay {t} differs from the eager call"
    assert torch.equal(eager.slots_view(), graphed.slots_view()), f"{name}: slot bytes differ"
    print(f"[graph] {name}: {steps} replays identical to the eager calls", flush=True)
