"""Test-side reader and writer of one head region, written with numpy bit
arrays (independent of the oracle's bit loops), used to pin the storage format.

Format: row i holds d_v codes of b_i bits as a little-endian, LSB-first bit
stream; a stored code is offset binary u = n + 2^(b-1); width 16 rows hold
fp16 patterns.  Section offsets come from a layout dict (see oracle.Cfg).
"""
import numpy as np


def _bits_of(buf: np.ndarray) -> np.ndarray:
    return np.unpackbits(buf, bitorder="little")


def read_head(slot: np.ndarray, lay: dict, widths, dk: int, dv: int, rscale_f16: bool,
              cscale_f16: bool):
    """Returns (codes n [dk,dv] int, pivot fp16 patterns [dk,dv] uint16, r [dk], c [dv])."""
    base = lay["base"]
    n = np.zeros((dk, dv), dtype=np.int64)
    hv = np.zeros((dk, dv), dtype=np.uint16)
    off = base + lay["codes"]
    for i in range(dk):
        b = int(widths[i])
        nbytes = dv * b // 8
        bits = _bits_of(slot[off:off + nbytes]).reshape(dv, b).astype(np.int64)
        raw = (bits << np.arange(b)).sum(axis=1)
        if b == 16:
            hv[i] = raw.astype(np.uint16)
        else:
            n[i] = raw - (1 << (b - 1))
        off += nbytes
    if lay["nquant"] > 0:
        if rscale_f16:
            r = slot[base + lay["rs"]: base + lay["rs"] + 2 * dk].view(np.float16).astype(np.float32)
        else:
            r = slot[base + lay["rs"]: base + lay["rs"] + 4 * dk].view(np.float32).copy()
        if cscale_f16:
            c = slot[base + lay["cs"]: base + lay["cs"] + 2 * dv].view(np.float16).astype(np.float32)
        else:
            c = np.ones(dv, dtype=np.float32)
    else:
        r = np.zeros(dk, dtype=np.float32)
        c = np.ones(dv, dtype=np.float32)
    return n, hv, r, c


def write_head(slot: np.ndarray, lay: dict, widths, n, hv, r, c, rscale_f16: bool,
               cscale_f16: bool):
    dk, dv = n.shape
    base = lay["base"]
    off = base + lay["codes"]
    for i in range(dk):
        b = int(widths[i])
        raw = hv[i].astype(np.int64) if b == 16 else n[i].astype(np.int64) + (1 << (b - 1))
        bits = ((raw[:, None] >> np.arange(b)) & 1).astype(np.uint8).reshape(-1)
        nbytes = dv * b // 8
        slot[off:off + nbytes] = np.packbits(bits, bitorder="little")
        off += nbytes
    if lay["nquant"] > 0:
        if rscale_f16:
            slot[base + lay["rs"]: base + lay["rs"] + 2 * dk] = \
                np.asarray(r, dtype=np.float16).view(np.uint8)
        else:
            slot[base + lay["rs"]: base + lay["rs"] + 4 * dk] = \
                np.asarray(r, dtype=np.float32).view(np.uint8)
        if cscale_f16:
            slot[base + lay["cs"]: base + lay["cs"] + 2 * dv] = \
                np.asarray(c, dtype=np.float16).view(np.uint8)
