"""Pins for the decoder-layer oracle (oracle/decoder_layer.py): closed forms of
the attention block on small shapes (one key, two keys, uniform attention),
planted wiring mistakes they reject, and the layer as attention block then MoE
layer.  The closed forms are written out here with torch's bf16 rounding and
explicit softmaxes, not with the oracle's functions."""
import math

import numpy as np
import pytest
import torch

from oracle import decoder_layer as DL
from oracle import moe_oracle as O
from synth import QFmt, make_tiny_layer

D, HEADS, DH, WIN = 8, 2, 4, 128
EPS = 1e-6


def bf16(a):
    return torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def case(seed, n_ref, n_gen, zero_q=False):
    r = np.random.default_rng(seed)
    w = {k: bf16(r.normal(0, 0.5, (D, D))) for k in ("w_q", "w_k", "w_v", "w_o")}
    if zero_q:
        w["w_q"] = np.zeros((D, D))
    h = r.normal(0, 1, (1, D))
    kv = {"ref_k": bf16(r.normal(0, 1, (1, HEADS, n_ref, DH))), "ref_v": bf16(r.normal(0, 1, (1, HEADS, n_ref, DH))),
          "ring_k": bf16(r.normal(0, 1, (1, HEADS, WIN, DH))), "ring_v": bf16(r.normal(0, 1, (1, HEADS, WIN, DH))),
          "n_gen": np.array([n_gen])}
    return h, w, kv


def run(fn, h, w, kv):
    return fn(h, w["w_q"], w["w_k"], w["w_v"], w["w_o"], kv["ref_k"], kv["ref_v"], kv["ring_k"], kv["ring_v"],
              kv["n_gen"], EPS, heads=HEADS)[0]


def znorm(h):
    return h / np.sqrt(np.mean(h * h) + EPS)


def closed_single_key(h, w, kv):
    """No reference keys, first generated token: its own bf16 value is the output."""
    z = znorm(h[0])
    a = bf16(w["w_v"] @ z)
    return h[0] + w["w_o"] @ a


def closed_two_keys(h, w, kv):
    """One reference key and the new token's: a two-way softmax per head."""
    z = znorm(h[0])
    q, k, v = w["w_q"] @ z, bf16(w["w_k"] @ z), bf16(w["w_v"] @ z)
    a = np.empty(D)
    for hd in range(HEADS):
        sl = slice(DH * hd, DH * hd + DH)
        s_ref = float(q[sl] @ kv["ref_k"][0, hd, 0]) / math.sqrt(DH)
        s_new = float(q[sl] @ k[sl]) / math.sqrt(DH)
        m = max(s_ref, s_new)
        e_ref, e_new = math.exp(s_ref - m), math.exp(s_new - m)
        a[sl] = (e_ref * kv["ref_v"][0, hd, 0] + e_new * v[sl]) / (e_ref + e_new)
    return h[0] + w["w_o"] @ a


def closed_uniform(h, w, kv):
    """q = 0: every live key weighs the same, so each head outputs the mean value."""
    z = znorm(h[0])
    v = bf16(w["w_v"] @ z)
    n_gen = int(kv["n_gen"][0])
    a = np.empty(D)
    for hd in range(HEADS):
        ring = kv["ring_v"][0, hd].copy()
        ring[n_gen % WIN] = v[DH * hd:DH * hd + DH]
        vals = np.concatenate([kv["ref_v"][0, hd], ring[:min(n_gen + 1, WIN)]])
        a[DH * hd:DH * hd + DH] = vals.mean(axis=0)
    return h[0] + w["w_o"] @ a


CASES = [(closed_single_key, dict(n_ref=0, n_gen=0)), (closed_two_keys, dict(n_ref=1, n_gen=0)),
         (closed_uniform, dict(n_ref=3, n_gen=5, zero_q=True)), (closed_uniform, dict(n_ref=2, n_gen=300, zero_q=True))]


@pytest.mark.parametrize("closed,kw", CASES, ids=lambda c: getattr(c, "__name__", str(c)))
def test_attn_block_closed_forms(closed, kw):
    for seed in range(3):
        h, w, kv = case(seed, **kw)
        np.testing.assert_allclose(run(DL.attn_block, h, w, kv)[0], closed(h, w, kv), rtol=1e-12, atol=1e-12)


def _planted():
    from oracle.rswa import rswa_decode

    def make(norm=True, k_from_h=False, residual=True, o_transposed=False, v_unrounded=False):
        def fn(h, w_q, w_k, w_v, w_o, ref_k, ref_v, ring_k, ring_v, n_gen, eps, heads):
            h = np.atleast_2d(h)
            z = O.rmsnorm(h, eps) if norm else h
            q, k, v = z @ w_q.T, (h if k_from_h else z) @ w_k.T, z @ w_v.T
            a, _, _ = rswa_decode(q[0].reshape(heads, -1), k[0].reshape(heads, -1), v[0].reshape(heads, -1),
                                  ref_k[0], ref_v[0], ring_k[0], ring_v[0], int(n_gen[0]))
            if v_unrounded and int(n_gen[0]) == 0 and ref_k.shape[2] == 0:
                a = v[0].reshape(heads, -1)
            o = a.reshape(-1) @ (w_o if o_transposed else w_o.T)
            return ((h + o) if residual else o[None]), None
        return fn
    return {"no_norm": make(norm=False), "k_from_h": make(k_from_h=True), "no_residual": make(residual=False),
            "o_transposed": make(o_transposed=True), "v_unrounded": make(v_unrounded=True)}


@pytest.mark.parametrize("name", sorted(_planted()))
def test_closed_forms_catch_planted_mistakes(name):
    fn = _planted()[name]
    caught = False
    for closed, kw in CASES:
        h, w, kv = case(7, **kw)
        h = h * 3.0   # a norm that is not 1: skipping RMSNorm shows
        if not np.allclose(run(fn, h, w, kv)[0], closed(h, w, kv), rtol=1e-9, atol=1e-9):
            caught = True
    assert caught, name


def test_decoder_layer_is_attention_then_moe():
    """The whole layer: its attention half equals attn_block, and what the MoE
    half adds equals one MoE layer on the RMSNorm of the updated residual."""
    layer = make_tiny_layer(3, 4, D, 4, 4, QFmt(4, 4))
    h, w, kv = case(11, n_ref=2, n_gen=9)
    h2, h1, (ids, wt, z), _ = DL.decoder_layer(h, w, kv, layer, EPS, heads=HEADS, top_k=2)
    np.testing.assert_array_equal(h1, run(DL.attn_block, h, w, kv))
    ids2, w2, y2, _ = O.moe_layer(O.rmsnorm(h1, EPS), layer, top_k=2)
    np.testing.assert_allclose(h2 - h1, y2, rtol=1e-12, atol=1e-12)
    assert ids.tolist() == ids2.tolist()
