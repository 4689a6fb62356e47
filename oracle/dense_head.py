"""Float64 CPU oracle for the decoder's two dense ends: the layer-0 SwiGLU MLP
and the lm_head projection with greedy token selection.

TEST INFRASTRUCTURE ONLY.  Like ``moe_oracle``, this module is the plain, slow
definition the GPU library is checked against.  Only the test suite, the
smoke check in ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the library under ``quantized_expert_ffn_moe_amd/``
never does, and this module imports nothing from that package.

What it computes, and where the pages say so
--------------------------------------------
* Layer 0 of the decoder is a dense SwiGLU MLP rather than a mixture of
  experts (franken_ocr README, section "Architecture"; browser demo page,
  "One forward pass, left to right", step 6).  Its weights belong to the quantised
  set next to the expert matrices (README, "CPU Backend and Optimizations",
  quantisation policy).
* The final RMSNorm feeds an lm_head GEMV from 1,280 to 129,280 logits, and
  decoding is greedy (demo page, step 7 of the forward pass; README,
  "Architecture").  lm_head is kept at source precision (bf16) by the
  conservative recipe and may be int8 in the experimental all-int8 recipe
  (README, "focr convert" and the environment-variable table).

Readings where the pages are silent:
* The dense MLP's intermediate size is 6,848: the pages' int8 GEMM checks
  carry a model-specific K = 6848 case for the i32 accumulation bound
  (README, "CPU Backend and Optimizations" and "Conformance and Release
  Evidence"), and with hidden 1280 the only FFN product that reduces over
  6,848 is the dense MLP's down projection.
* Its codes use the experts' symmetric group format (W = s * q, one f32 scale
  per group along K); 6,848 = 107 * 64, so the group size is 32 or 64, not 128.
* Greedy decoding picks the largest logit; among equal logits the lowest
  token id (the same tie rule as the router).
* A bf16 weight is the value of its 16-bit pattern read as the top half of an
  IEEE binary32 (sign, 8-bit exponent, 7 stored mantissa bits).

Parity pins: ``tests/test_dense_head_oracle.py`` (closed forms, brute force,
one-hot cases, exact bf16 decoding against ``fractions.Fraction``).
"""
from __future__ import annotations

import numpy as np

from oracle.moe_oracle import dequantize, rmsnorm, swiglu_ffn

f64 = np.float64

__all__ = ["bf16_bits_value", "lm_head_logits", "greedy_token", "dense_ffn", "dense_weights",
           "dequantize", "rmsnorm"]


def bf16_bits_value(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns, decoded field by field in f64.

    sign = bit 15, exponent = bits 14..7 (bias 127), fraction = bits 6..0.
    Normal numbers: (-1)^s * (1 + f / 128) * 2^(e - 127); exponent 0 holds
    zeros and subnormals (f / 128) * 2^-126; exponent 255 holds inf / NaN.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    s = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    f = (b & 0x7F).astype(f64)
    normal = np.ldexp(1.0 + f / 128.0, (e - 127).astype(np.int64))
    sub = np.ldexp(f / 128.0, -126)
    special = np.where(f == 0, np.inf, np.nan)
    v = np.where(e == 0, sub, np.where(e == 255, special, normal))
    return s * v


def lm_head_logits(H, W, norm: bool, eps: float) -> np.ndarray:
    """logits[t, v] = sum_k W[v, k] * z[t, k], z = RMSNorm(h_t) (or h_t without the norm)."""
    H = np.atleast_2d(np.asarray(H, dtype=f64))
    Z = rmsnorm(H, eps) if norm else H
    return Z @ np.asarray(W, dtype=f64).T


def greedy_token(logits):
    """The largest logit per token and its id; ties go to the lowest id
    (``np.argmax`` returns the first of equal maxima)."""
    L = np.atleast_2d(np.asarray(logits, dtype=f64))
    ids = np.argmax(L, axis=1).astype(np.int32)
    return ids, L[np.arange(L.shape[0]), ids]


def dense_weights(ffn: dict):
    """Dequantised (W_g, W_u, W_d) of a dense FFN given as codes + scales."""
    g = ffn["group"]
    return (dequantize(ffn["gate_q"], ffn["gate_s"], g),
            dequantize(ffn["up_q"], ffn["up_s"], g),
            dequantize(ffn["down_q"], ffn["down_s"], g))


def dense_ffn(X, ffn: dict, norm: bool, eps: float) -> np.ndarray:
    """y = W_d (SiLU(W_g z) * (W_u z)), z = RMSNorm(x) (or x without the norm)."""
    X = np.atleast_2d(np.asarray(X, dtype=f64))
    Z = rmsnorm(X, eps) if norm else X
    Wg, Wu, Wd = dense_weights(ffn)
    return swiglu_ffn(Wg, Wu, Wd, Z)
