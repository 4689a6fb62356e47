"""Float64 CPU oracle for one decoder layer step of the MoE decoder.

TEST INFRASTRUCTURE ONLY.  Like ``moe_oracle`` and ``rswa``, this module is
the plain, slow definition the GPU library is checked against.  Only the test
suite, the smoke check in ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import it; the library under ``quantized_expert_ffn_moe_amd/``
never does, and this module imports nothing from that package.

What it computes, and where the pages say so
--------------------------------------------
A decoder layer of the MoE decoder is an attention block followed by the MoE
FFN, each behind an RMSNorm and each added to the residual stream (browser demo
page "A 3-billion-parameter OCR model. In this tab.", "One forward pass, left
to right", step 6: the R-SWA attention of ten heads of 128 and the MoE FFN;
franken_ocr README "Architecture"; the model card's "The rest of the pipeline"
calls the attention plain Llama-style multi-head attention).

  z  = RMSNorm(h)                               (no gain, eps inside the root)
  q  = W_q z,  k = W_k z,  v = W_v z            (1280 -> 1280 each, ten heads of 128)
  a  = R-SWA(q, k, v; frozen reference KV, 128-slot ring of generated tokens)
  h' = h + W_o a
  h''= h' + MoE(RMSNorm(h'))

Readings where the pages are silent:
* The projection weights are bf16 (the conservative recipe keeps attention at
  source precision, README "focr convert"); there are no projection biases
  (Llama-style attention has none).
* No positional transform is applied: the pages name none, so q and k are the
  projections' outputs as they are.
* The new key and value enter the ring rounded to bf16 (``rswa``).
"""
from __future__ import annotations

import numpy as np

from oracle.moe_oracle import moe_chain, rmsnorm
from oracle.rswa import rswa_decode

f64 = np.float64
HEADS, HEAD_DIM = 10, 128


def attn_block(h, w_q, w_k, w_v, w_o, ref_k, ref_v, ring_k, ring_v, n_gen, eps: float,
               heads: int = HEADS):
    """The attention half of a decoder layer for S independent streams.

    h [S][D] residual rows; w_q, w_k, w_v, w_o [D][D] (values, e.g. of bf16
    weights); ref_k, ref_v [S][heads][n_ref][d]; ring_k, ring_v
    [S][heads][128][d]; n_gen [S].  Returns (h' [S][D], rings after the
    write: list of (ring_k, ring_v) per stream)."""
    h = np.atleast_2d(np.asarray(h, dtype=f64))
    S, D = h.shape
    d = D // heads
    z = rmsnorm(h, eps)
    q = z @ np.asarray(w_q, dtype=f64).T
    k = z @ np.asarray(w_k, dtype=f64).T
    v = z @ np.asarray(w_v, dtype=f64).T
    out = np.empty((S, D), dtype=f64)
    rings = []
    for s in range(S):
        a, rk, rv = rswa_decode(q[s].reshape(heads, d), k[s].reshape(heads, d), v[s].reshape(heads, d),
                                ref_k[s], ref_v[s], ring_k[s], ring_v[s], int(n_gen[s]))
        out[s] = a.reshape(D)
        rings.append((rk, rv))
    return h + out @ np.asarray(w_o, dtype=f64).T, rings


def decoder_layer(h, attn: dict, kv: dict, moe_layer_weights: dict, eps: float, heads: int = HEADS,
                  top_k: int = 6):
    """One whole decoder layer: the attention block, then the MoE FFN on the
    updated residual (RMSNorm before it, residual add after it).

    attn: w_q, w_k, w_v, w_o; kv: ref_k, ref_v, ring_k, ring_v, n_gen.
    Returns (h'' [S][D], h' [S][D] (after attention), (ids, w, z) of the MoE
    layer, rings)."""
    h1, rings = attn_block(h, attn["w_q"], attn["w_k"], attn["w_v"], attn["w_o"], kv["ref_k"], kv["ref_v"],
                           kv["ring_k"], kv["ring_v"], kv["n_gen"], eps, heads=heads)
    h2, trace = moe_chain(h1, [moe_layer_weights], eps, False, top_k=top_k)
    return h2, h1, trace[0], rings
