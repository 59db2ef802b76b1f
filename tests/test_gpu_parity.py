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
    from tests.parity import rel_err
    worst = 0.0
    for n, (b, h) in enumerate(follow):
        e = rel_err(o_gpu[n], o_ref[n])
        worst = max(worst, e)
        assert e <= O_TOL, f"{tag}: o mismatch at step {t}, unit (b={b}, h={h}): rel err {e:.3g}"
    return worst


def _run(w, T, follow=None, bits=None, check_slots_every=0, tag=""):
    print(f"[{tag}] {w.name} B={w.B} H={w.H} d={w.dk} T={T}", flush=True)
    hs = _harness(w, follow=follow, bits=bits)
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


def _run_sampled(w, T, n_units, seed, layer=0, track=False, tag="", follow=None, bits=None):
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
    hs = _harness(w, layer=layer, follow=follow, bits=bits)
    try:
        if track:
            hs.track_fp32()
        hs.init_state()
        hs.load_full(0)
        for t in range(T):
            x = hs.load_followed(t)
            o_gpu, o_ref = hs.step(x, idx_in_x=True)
            _check_step(o_gpu, o_ref, hs.follow, t, tag)
            if (t + 1) % 256 == 0:
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
    compared every few steps."""
    _run(synth.WORKLOADS["serving_fp32"].with_(B=16), 8, check_slots_every=4, tag="fp32")
    w = synth.WORKLOADS["qwen_gdn"].with_(B=6, H=6, name="qwen_mixed_fp32")
    bits = np.array([32, 4, 16, 6, 32, 8], np.uint8)
    _run(w, 10, bits=bits, check_slots_every=5, tag="fp32-mixed")


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
    """Heads whose rows are all 4-bit in pairs, in head order; every other
    head alone; an unpaired 4-bit head last."""
    groups, pending = [], None
    for h, r in enumerate(bits):
        if not (r == 4).all():
            groups.append((h, 0xFFFF))
        elif pending is None:
            pending = h
        else:
            groups.append((pending, h))
            pending = None
    if pending is not None:
        groups.append((pending, 0xFFFF))
    return groups


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


def test_kimi_kda_all_units_32_steps():
    """B=256 x H=32 KDA (4-bit rows + 41 FP16 pivot rows), outlier start: every unit, 32 steps."""
    _run(synth.WORKLOADS["kimi_kda"], 32, check_slots_every=16, tag="kimi-all")


def test_kimi_kda_sampled_units_all_256_steps():
    """Full KDA batch, 256 followed units over all 256 steps."""
    w = synth.WORKLOADS["kimi_kda"]
    _run_sampled(w, w.T, 256, seed=12, tag="kimi-long")


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
