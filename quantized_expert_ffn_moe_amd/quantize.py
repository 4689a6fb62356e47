"""Host-side quantisers from float weights to the library's expert formats
(numpy, no GPU).  Their outputs are the canonical inputs of
``moe_pack_expert`` and ``moe_pack_expert_q4k`` (``binding.py``).

* Symmetric groups (browser demo page "A 3-billion-parameter OCR model. In
  this tab.", section "Four bits, one shared scale": a two's-complement code
  per weight and one f32 scale per group along K): round to nearest with the
  group's absolute maximum mapped to the largest positive code.
* The two-level 4-bit format of the community K-quant decoder (Unlimited-OCR
  DeepEncoder ONNX model card, "The rest of the pipeline"):
  ``W = d * sc * q - dmin * m`` with super-blocks of 256 columns (f16 d,
  dmin) and sub-blocks of 32 (6-bit sc, m).  Each sub-block's range
  [min(w, 0), max(w)] is spread over the 16 codes; the super-block factors
  are the largest sub-block scale and minimum over 63, rounded to f16, and
  the 6-bit fields and the codes are rounded to nearest against the
  quantised factors.  (A plain round-to-nearest quantiser: no search over
  scales.)
"""
from __future__ import annotations

import numpy as np

SUB, SUPER = 32, 256


def quantize_symmetric(W, bits: int, group: int):
    """W [N][K] float -> (codes int8 [N][K], scales f32 [N][K/group])."""
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    if bits not in (4, 8) or K % group:
        raise ValueError("bits must be 4 or 8 and the group must divide K")
    qmax = 7 if bits == 4 else 127
    qmin = -8 if bits == 4 else -128
    blocks = W.reshape(N, K // group, group)
    s = (np.abs(blocks).max(axis=2) / qmax).astype(np.float32)
    s64 = s.astype(np.float64)[:, :, None]
    q = np.where(s64 > 0, np.rint(blocks / np.where(s64 > 0, s64, 1.0)), 0.0)
    return np.clip(q, qmin, qmax).astype(np.int8).reshape(N, K), s


def quantize_two_level(W) -> dict:
    """W [N][K] float (K a multiple of 32) -> {q, d, dmin, sc, m} as taken by
    ``moe_pack_expert_q4k``: q uint8 [N][K], d and dmin f16 bit patterns
    [N][ceil(K/256)], sc and m uint8 [N][K/32]."""
    W = np.asarray(W, dtype=np.float64)
    N, K = W.shape
    if K % SUB:
        raise ValueError("K must be a multiple of 32")
    nsub, nsb = K // SUB, -(-K // SUPER)
    blocks = W.reshape(N, nsub, SUB)
    lo = np.minimum(blocks.min(axis=2), 0.0)
    hi = np.maximum(blocks.max(axis=2), lo)
    scale = (hi - lo) / 15.0                    # per sub-block step
    mins = -lo                                  # per sub-block minimum, >= 0
    pad = nsb * (SUPER // SUB) - nsub           # the last super-block may be partial
    sp = np.pad(scale, ((0, 0), (0, pad))).reshape(N, nsb, SUPER // SUB)
    mp = np.pad(mins, ((0, 0), (0, pad))).reshape(N, nsb, SUPER // SUB)
    d = (sp.max(axis=2) / 63.0).astype(np.float16)
    dmin = (mp.max(axis=2) / 63.0).astype(np.float16)
    d64 = np.repeat(d.astype(np.float64), SUPER // SUB, axis=1)[:, :nsub]
    dm64 = np.repeat(dmin.astype(np.float64), SUPER // SUB, axis=1)[:, :nsub]
    sc = np.clip(np.rint(np.where(d64 > 0, scale / np.where(d64 > 0, d64, 1.0), 0.0)), 0, 63)
    m = np.clip(np.rint(np.where(dm64 > 0, mins / np.where(dm64 > 0, dm64, 1.0), 0.0)), 0, 63)
    step = (d64 * sc)[:, :, None]
    off = (dm64 * m)[:, :, None]
    q = np.where(step > 0, np.rint((blocks + off) / np.where(step > 0, step, 1.0)), 0.0)
    return {"q": np.clip(q, 0, 15).astype(np.uint8).reshape(N, K),
            "d": d.view(np.uint16), "dmin": dmin.view(np.uint16),
            "sc": sc.astype(np.uint8), "m": m.astype(np.uint8)}


def bits_per_weight(fmt_group: int, bits: int, K: int) -> float:
    """Stored bits per weight of a row of K weights: codes plus metadata (f32
    group scales; or, for the two-level format, a 16-byte record per 256
    columns, the layout of the gate and up matrices)."""
    if fmt_group == SUPER and bits == 4:
        return 4.0 + 128.0 * -(-K // SUPER) / K
    return bits + 32.0 / fmt_group
