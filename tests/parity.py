"""GPU-vs-oracle parity harness (test side).

Runs the HIP path through the C ABI on a whole batch and the CPU oracle on the
same seeded inputs for a chosen set of (request, head) units, comparing every
output vector and the final slot bytes.  Units are independent, so units the
oracle does not follow may be fed cheaper inputs (a ring of pre-generated
steps) without affecting the followed ones.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


class Harness:
    def __init__(self, w: synth.Workload, layer: int = 0, follow=None, seed_perm: int = 1,
                 bits=None, row_impact=None):
        import torch
        import linear_attention_recurrent_stq_amd as stq
        self.torch, self.stq = torch, stq
        self.w, self.layer = w, layer
        self.bits = synth.unit_bits(w, layer) if bits is None else np.asarray(bits, np.uint8)
        self.L = stq.Layout.from_workload(w, self.bits, row_impact=row_impact)
        self.ocfg = oracle.Cfg.from_workload(w, self.bits, row_impact=row_impact)
        assert self.L.slot_bytes == self.ocfg.slot_bytes
        self.pool = stq.Pool(self.L, w.B)
        # requests are mapped to a seeded permutation of the slots
        perm = np.argsort(synth.raw(synth.stream_key(seed_perm, w.cid, 99), w.B)[:w.B], kind="stable")
        self.slot_of = perm.astype(np.int32)
        self.slot_ids = torch.from_numpy(self.slot_of).cuda()
        if follow is None:
            follow = [(b, h) for b in range(w.B) for h in range(w.H)]
        self.follow = list(follow)
        self.fb = np.array([u[0] for u in self.follow], np.int64)
        self.fh = np.array([u[1] for u in self.follow], np.int64)
        self.fb_dev = torch.from_numpy(self.fb).cuda()
        self.fh_dev = torch.from_numpy(self.fh).cuda()
        self.everything = len(self.follow) == w.B * w.H
        self.shadow = None  # unquantized fp32 states of the followed units
        self.shadow_err = []
        reqs = sorted(set(self.fb.tolist()))
        self.oslots = {b: self.ocfg.new_slot() for b in reqs}
        self.exec = ThreadPoolExecutor(THREADS)
        dev = "cuda"
        B, H, dk, dv = w.B, w.H, w.dk, w.dv
        io = torch.bfloat16 if w.io == "bf16" else torch.float32
        self.q = torch.empty(B, H, dk, dtype=io, device=dev)
        self.k = torch.empty(B, H, dk, dtype=io, device=dev)
        self.v = torch.empty(B, H, dv, dtype=io, device=dev)
        self.a = torch.empty((B, H, dk) if w.gate == "keyvec" else (B, H), dtype=torch.float32, device=dev)
        self.beta = torch.empty(B, H, dtype=torch.float32, device=dev)
        self.o = torch.empty(B, H, dv, dtype=torch.float32, device=dev)
        self.t = 0

    # ------------------------------------------------------------- inputs
    def _to_dev(self, x: synth.StepInputs):
        torch = self.torch
        if self.w.io == "bf16":
            conv = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
            return conv(x.q_bits), conv(x.k_bits), conv(x.v_bits)
        return torch.from_numpy(x.q), torch.from_numpy(x.k), torch.from_numpy(x.v)

    def load_full(self, t: int):
        x = synth.batch_inputs(self.w, self.layer, t)
        q, k, v = self._to_dev(x)
        self.q.copy_(q); self.k.copy_(k); self.v.copy_(v)
        self.a.copy_(self.torch.from_numpy(x.a)); self.beta.copy_(self.torch.from_numpy(x.beta))
        return x

    def load_followed(self, t: int):
        """Overwrite only the followed units' inputs (others keep what they had)."""
        x = synth.step_inputs(self.w, self.layer, t, self.fb, self.fh)
        q, k, v = self._to_dev(x)
        bi, hi = self.fb_dev, self.fh_dev
        self.q[bi, hi] = q.cuda(); self.k[bi, hi] = k.cuda(); self.v[bi, hi] = v.cuda()
        self.a[bi, hi] = self.torch.from_numpy(x.a).cuda()
        self.beta[bi, hi] = self.torch.from_numpy(x.beta).cuda()
        return x

    # -------------------------------------------------------------- state
    def init_state(self):
        """Seed the initial state (outlier workloads) on both sides with pack."""
        if self.w.init == "zero":
            return
        torch = self.torch
        B, H = self.w.B, self.w.H
        bb, hh = np.meshgrid(np.arange(B), np.arange(H), indexing="ij")
        M0 = synth.initial_state(self.w, self.layer, bb, hh)
        self.stq.pack(self.pool, self.slot_ids, torch.from_numpy(M0).cuda())
        for b, h in self.follow:
            self.ocfg.pack_head(self.oslots[b], h, M0[b, h])
        if self.shadow is not None:
            self.shadow = [np.ascontiguousarray(M0[b, h]) for b, h in self.follow]

    def track_fp32(self):
        """Also run the unquantized fp32 recurrence for every followed unit
        (from the same initial state) and record, per step, the largest
        relative distance of the quantized output from it."""
        self.shadow = [np.zeros((self.w.dk, self.w.dv), np.float32) for _ in self.follow]

    # --------------------------------------------------------------- step
    def step(self, x_followed: synth.StepInputs, idx_in_x=None):
        """One GPU step on the whole batch, one oracle step per followed unit.
        Returns the GPU o of the followed units [n, dv] (gathered on the
        device) and the oracle o per followed unit."""
        self.stq.decode_step(self.pool, self.slot_ids, self.q, self.k, self.v, self.a,
                             self.beta, self.o)
        lagged = self.ocfg.scale_fit == 1
        if lagged:
            self.stq.fit_scales(self.pool, self.slot_ids)
        gate_vec = self.w.gate == "keyvec"

        def one(n):
            b, h = self.follow[n]
            j = (b, h) if idx_in_x is None else (n,)
            a = x_followed.a[j]
            a = a if gate_vec else np.float32(a)
            o = self.ocfg.step_head(self.oslots[b], h, x_followed.q[j], x_followed.k[j],
                                    x_followed.v[j], a, x_followed.beta[j])
            if lagged:
                self.ocfg.fit_head(self.oslots[b], h)
            e = 0.0
            if self.shadow is not None:
                o32 = oracle.step_f32(self.shadow[n], x_followed.q[j], x_followed.k[j],
                                      x_followed.v[j], a, x_followed.beta[j], gate_vec)
                e = float(np.max(np.abs(o - o32)) / max(float(np.max(np.abs(o32))), 1e-30))
            return o, e

        res = list(self.exec.map(one, range(len(self.follow))))
        o_ref = [r[0] for r in res]
        if self.shadow is not None:
            self.shadow_err.append(max(r[1] for r in res))
        if self.everything:
            o_gpu = self.o.cpu().numpy()[self.fb, self.fh]
        else:
            o_gpu = self.o[self.fb_dev, self.fh_dev].cpu().numpy()
        self.t += 1
        return o_gpu, o_ref

    def slot_bytes_gpu(self) -> np.ndarray:
        return self.pool.slots_view().cpu().numpy()

    def compare_slots(self):
        """Byte comparison of every followed head region; returns mismatch list."""
        allb = self.slot_bytes_gpu()
        bad = []
        for b, h in self.follow:
            lay = self.ocfg.head_layout(h)
            lo, hi = lay["base"], lay["base"] + lay["bytes"]
            g = allb[self.slot_of[b], lo:hi]
            r = self.oslots[b][lo:hi]
            if not np.array_equal(g, r):
                bad.append((b, h, int(np.nonzero(g != r)[0][0])))
        return bad

    def unpack_gpu(self):
        torch = self.torch
        out = torch.empty(self.w.B, self.w.H, self.w.dk, self.w.dv, dtype=torch.float32, device="cuda")
        self.stq.unpack(self.pool, self.slot_ids, out)
        return out.cpu().numpy()

    def close(self):
        self.exec.shutdown()
