"""Float64 CPU oracle for one decode step of R-SWA attention (Reference
Sliding Window Attention), the decoder's attention.

TEST INFRASTRUCTURE ONLY.  Like ``moe_oracle``, this module is the plain,
slow definition the GPU library is checked against.  Only the test suite, the
smoke check in ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the library under ``quantized_expert_ffn_moe_amd/``
never does, and this module imports nothing from that package.

What it computes, and where the pages say so
--------------------------------------------
* Ten attention heads of dimension 128 (browser demo page "A
  3-billion-parameter OCR model. In this tab.", "One forward pass, left to
  right", step 6; franken_ocr README "Architecture" and "Design Philosophy").
* Every decoder attention layer is R-SWA: a generated token attends to all
  reference tokens (the visual prefill plus the prompt prefix, kept as a
  frozen global KV that is never evicted) and to the previous generated
  tokens through a ring buffer of 128 slots, so the generated-token KV stays
  constant in size (README "Design Philosophy", "Bounded generated-token KV";
  the "Bounded long-doc memory" row of the table under "Why focr?"; demo page
  step 6).
* Attention weights and the KV stay at source precision (bf16) in the
  conservative recipe (README "CPU Backend and Optimizations", quantisation
  policy; "focr convert").

Readings where the pages are silent:
* The new token's key and value are written into ring slot n_gen mod 128
  (n_gen = generated tokens before it) before it attends, so the ring holds
  the newest min(n_gen + 1, 128) generated tokens, the new one included.
* Plain softmax attention per head over the union of the reference keys and
  the live ring slots, scores q.k / sqrt(128); the query, key and value
  arrive after whatever positional transform the model applies (the pages do
  not describe one), so none is applied here.
* The KV is stored as bf16 (nearest, ties to even); q and the output are f32.
"""
from __future__ import annotations

import numpy as np

from oracle.moe_oracle import bf16_round

f64 = np.float64
WINDOW = 128


def ring_write(ring_k, ring_v, k_new, v_new, n_gen: int):
    """Copies of the ring [heads][WINDOW][d] with the new token's bf16-rounded
    key and value in slot n_gen mod WINDOW."""
    rk = np.array(ring_k, dtype=f64, copy=True)
    rv = np.array(ring_v, dtype=f64, copy=True)
    slot = n_gen % WINDOW
    rk[:, slot, :] = bf16_round(k_new)
    rv[:, slot, :] = bf16_round(v_new)
    return rk, rv


def live_slots(n_gen: int):
    """Ring slots that hold generated tokens after the new one is written."""
    return np.arange(min(n_gen + 1, WINDOW))


def attend(q, keys, values):
    """softmax(q.k_j / sqrt(d)) weighted sum of v_j, for one head (keys [n][d])."""
    q = np.asarray(q, dtype=f64)
    keys = np.asarray(keys, dtype=f64)
    values = np.asarray(values, dtype=f64)
    s = keys @ q / np.sqrt(q.shape[-1])
    m = s.max()
    p = np.exp(s - m)
    return (p / p.sum()) @ values


def rswa_decode(q, k_new, v_new, ref_k, ref_v, ring_k, ring_v, n_gen: int):
    """One generated token of one stream.

    q, k_new, v_new: [heads][d]; ref_k, ref_v: [heads][n_ref][d] (bf16
    values); ring_k, ring_v: [heads][WINDOW][d], the ring before this token.
    Returns (out [heads][d], ring_k, ring_v after the write)."""
    rk, rv = ring_write(ring_k, ring_v, k_new, v_new, n_gen)
    live = live_slots(n_gen)
    heads = np.asarray(q).shape[0]
    out = np.empty((heads, np.asarray(q).shape[1]), dtype=f64)
    for h in range(heads):
        keys = np.concatenate([np.asarray(ref_k[h], dtype=f64), rk[h, live]])
        vals = np.concatenate([np.asarray(ref_v[h], dtype=f64), rv[h, live]])
        out[h] = attend(q[h], keys, vals)
    return out, rk, rv
