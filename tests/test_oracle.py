"""Pins for the float64 oracle: every function is checked against something
other than itself (hand-worked values, closed forms, brute force, library
routines on special cases, invariants)."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

from oracle import moe_oracle as O
from synth import QFmt, make_tiny_layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_layer.json")


def _fixture_layer():
    d = json.load(open(GOLDEN))
    fmt = QFmt(d["bits"], d["group"])
    layer = {k: np.asarray(d[k], dtype=np.float64 if k == "router_w" else None)
             for k in ("router_w", "gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s",
                       "shared_gate_q", "shared_gate_s", "shared_up_q", "shared_up_s",
                       "shared_down_q", "shared_down_s")}
    for k in list(layer):
        if k.endswith("_q"):
            layer[k] = layer[k].astype(np.int8)
        elif k.endswith("_s"):
            layer[k] = layer[k].astype(np.float32)
    layer.update(router_b=None, routed_fmt=fmt, shared_fmt=fmt)
    return d, layer


# ---------------------------------------------------------------- hand-worked case
def test_tiny_fixture_top2():
    d, layer = _fixture_layer()
    x = np.asarray(d["x"], dtype=np.float64)[None]
    ids, w, y, P = O.moe_layer(x, layer, top_k=2)
    ex = d["expected"]
    np.testing.assert_allclose(P[0], ex["P"], rtol=0, atol=1e-15)
    assert ids[0].tolist() == ex["ids_top2"]
    np.testing.assert_allclose(w[0], ex["w_top2"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(y[0], ex["y"], rtol=1e-13, atol=1e-14)


def test_tiny_fixture_top3_tie_goes_to_lower_index():
    d, layer = _fixture_layer()
    x = np.asarray(d["x"], dtype=np.float64)[None]
    ids, w, _, _ = O.moe_layer(x, layer, top_k=3)
    assert ids[0].tolist() == d["expected"]["ids_top3"]
    np.testing.assert_allclose(w[0], d["expected"]["w_top3"], rtol=0, atol=1e-15)


def test_silu_constants_of_fixture():
    d, _ = _fixture_layer()
    s = d["expected"]["silu"]
    got = O.silu(np.array([1.0, -1.0, 2.0]))
    np.testing.assert_allclose(got, [s["S1"], s["Sm1"], s["S2"]], rtol=1e-15)


# ---------------------------------------------------------------- softmax / routing
def test_softmax_matches_scipy_and_sums_to_one():
    rng = np.random.default_rng(1)
    L = rng.normal(0, 3, (50, 64))
    P = O.softmax(L)
    np.testing.assert_allclose(P, scipy.special.softmax(L, axis=1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-15)


def test_equal_logits_closed_form():
    P = O.softmax(np.zeros((1, 64)))
    assert np.all(P == 1.0 / 64)
    ids, w = O.greedy_topk(P, 6)
    assert ids[0].tolist() == [0, 1, 2, 3, 4, 5]
    assert np.all(w == 1.0 / 64)


def _brute_topk(p, k):
    order = sorted(range(len(p)), key=lambda e: (-p[e], e))
    return order[:k]


def test_topk_against_full_sort_with_ties():
    rng = np.random.default_rng(2)
    for _ in range(300):
        # coarse values force many exact ties
        p = rng.integers(0, 9, 64).astype(np.float64)
        p /= p.sum() if p.sum() else 1.0
        ids, w = O.greedy_topk(p[None], 6)
        assert ids[0].tolist() == _brute_topk(p.tolist(), 6)
        np.testing.assert_array_equal(w[0], p[ids[0]])


def test_routing_weights_bounds():
    rng = np.random.default_rng(3)
    L = rng.normal(0, 2, (400, 64))
    ids, w = O.greedy_topk(O.softmax(L), 6)
    s = w.sum(axis=1)
    assert np.all(s <= 1.0 + 1e-15) and np.all(s >= 6 / 64 - 1e-15)
    assert np.all(np.diff(w, axis=1) <= 0)  # pick order = descending weight


def test_duplicate_router_rows_lower_index_first():
    layer = make_tiny_layer(5, E=16, H=32, I=16, Is=16, fmt=QFmt(4, 16))
    Wr = np.zeros((16, 32))
    Wr[11] = Wr[4] = 1.0  # the two best experts have identical rows
    Wr[7] = 0.5
    x = np.ones((1, 32))
    P = O.softmax(O.router_logits(x, Wr))
    ids, _ = O.greedy_topk(P, 3)
    assert ids[0].tolist() == [4, 11, 7]


def test_router_bias_adds_to_logits():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(3, 8)); Wr = rng.normal(size=(5, 8)); b = rng.normal(size=5)
    np.testing.assert_allclose(O.router_logits(x, Wr, b) - O.router_logits(x, Wr), np.tile(b, (3, 1)),
                               rtol=0, atol=1e-12)


# ---------------------------------------------------------------- dequantisation
@pytest.mark.parametrize("bits,lo,hi", [(4, -8, 7), (8, -128, 127)])
def test_dequant_exact_against_fractions(bits, lo, hi):
    rng = np.random.default_rng(bits)
    codes = np.arange(lo, hi + 1, dtype=np.int8)
    K = 32 * ((len(codes) + 31) // 32)
    Q = np.zeros((4, K), np.int8)
    Q[:, :len(codes)] = codes
    S = rng.uniform(0.002, 0.02, (4, K // 32)).astype(np.float32)
    W = O.dequantize(Q, S, 32)
    for r in range(4):
        for c in range(K):
            assert Fraction(W[r, c]) == Fraction(float(S[r, c // 32])) * int(Q[r, c])


def test_dequant_group_runs_along_k():
    Q = np.ones((2, 12), np.int8)
    S = np.array([[1, 2, 4], [8, 16, 32]], np.float32)
    W = O.dequantize(Q, S, 4)
    np.testing.assert_array_equal(W[0], [1] * 4 + [2] * 4 + [4] * 4)
    np.testing.assert_array_equal(W[1], [8] * 4 + [16] * 4 + [32] * 4)


# ---------------------------------------------------------------- expert FFN
def test_silu_identities_and_torch():
    v = np.linspace(-30, 30, 601)
    s = O.silu(v)
    assert O.silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(s - O.silu(-v), v, rtol=1e-14, atol=1e-13)
    np.testing.assert_allclose(s, torch.nn.functional.silu(torch.tensor(v, dtype=torch.float64)).numpy(),
                               rtol=1e-14, atol=1e-300)


def test_one_hot_positions_catch_transposes():
    # gate/up only see x[5] through row 2; down maps intermediate 2 to output 9 only
    H, I = 16, 8
    Wg = np.zeros((I, H)); Wu = np.zeros((I, H)); Wd = np.zeros((H, I))
    Wg[2, 5] = 1.5; Wu[2, 5] = -2.0; Wd[9, 2] = 0.25
    x = np.zeros((1, H)); x[0, 5] = 2.0
    y = O.swiglu_ffn(Wg, Wu, Wd, x)[0]
    g, u = 3.0, -4.0
    expect = np.zeros(H); expect[9] = 0.25 * (g / (1 + math.exp(-g))) * u
    np.testing.assert_allclose(y, expect, rtol=1e-15, atol=0)


def test_fused_shared_equals_sum_of_two_experts():
    layer = make_tiny_layer(6, E=4, H=32, I=8, Is=16, fmt=QFmt(4, 8))
    Wg, Wu, Wd = O.shared_weights(layer)
    x = np.random.default_rng(6).normal(size=(5, 32))
    full = O.swiglu_ffn(Wg, Wu, Wd, x)
    a = O.swiglu_ffn(Wg[:8], Wu[:8], Wd[:, :8], x)
    b = O.swiglu_ffn(Wg[8:], Wu[8:], Wd[:, 8:], x)
    np.testing.assert_allclose(full, a + b, rtol=1e-12, atol=1e-12)


def test_all_experts_identical_k_equals_e_reduces_to_dense_mlp():
    E, H, I = 4, 32, 8
    layer = make_tiny_layer(7, E=E, H=H, I=I, Is=8, fmt=QFmt(8, 8))
    for k in ("gate", "up", "down"):
        layer[f"{k}_q"][:] = layer[f"{k}_q"][0]
        layer[f"{k}_s"][:] = layer[f"{k}_s"][0]
        layer[f"shared_{k}_q"][:] = 0
    x = np.random.default_rng(7).normal(size=(3, H))
    _, w, y, _ = O.moe_layer(x, layer, top_k=E)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, atol=1e-15)
    # textbook SwiGLU MLP in torch, f64
    t = lambda a: torch.tensor(np.asarray(a, np.float64))
    deq = lambda q, s, G: t(q.astype(np.float64) * np.repeat(s.astype(np.float64), G, axis=1))
    Wg, Wu, Wd = (deq(layer[f"{k}_q"][0], layer[f"{k}_s"][0], 8) for k in ("gate", "up", "down"))
    ref = (torch.nn.functional.silu(t(x) @ Wg.T) * (t(x) @ Wu.T)) @ Wd.T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- whole-layer invariants
def _layer_and_x(seed=8, T=9):
    layer = make_tiny_layer(seed, E=8, H=64, I=32, Is=64, fmt=QFmt(4, 16), shared_fmt=QFmt(8, 32))
    x = np.random.default_rng(seed).normal(size=(T, 64))
    return layer, x


def test_zero_gate_codes_leave_only_shared():
    layer, x = _layer_and_x()
    layer["gate_q"][:] = 0
    _, _, y, _ = O.moe_layer(x, layer, top_k=3)
    ys = O.swiglu_ffn(*O.shared_weights(layer), x)
    np.testing.assert_array_equal(y, ys)


def test_zero_shared_codes_leave_weighted_routed_sum():
    layer, x = _layer_and_x()
    layer["shared_down_q"][:] = 0
    ids, w, y, _ = O.moe_layer(x, layer, top_k=3)
    for t in range(x.shape[0]):
        acc = np.zeros(64)
        for i in range(3):
            acc += w[t, i] * O.swiglu_ffn(*O.expert_weights(layer, int(ids[t, i])), x[t:t + 1])[0]
        np.testing.assert_allclose(y[t], acc, rtol=1e-12, atol=1e-13)


def test_doubling_down_scales_adds_one_more_copy_of_that_expert():
    layer, x = _layer_and_x()
    ids, w, y, _ = O.moe_layer(x, layer, top_k=3)
    e = int(ids[0, 0])
    layer2 = dict(layer); layer2["down_s"] = layer["down_s"].copy(); layer2["down_s"][e] *= 2
    ids2, w2, y2, _ = O.moe_layer(x, layer2, top_k=3)
    assert np.array_equal(ids, ids2)
    for t in range(x.shape[0]):
        extra = np.zeros(64)
        for i in range(3):
            if ids[t, i] == e:
                extra += w[t, i] * O.swiglu_ffn(*O.expert_weights(layer, e), x[t:t + 1])[0]
        np.testing.assert_allclose(y2[t] - y[t], extra, rtol=1e-10, atol=1e-12)


def test_relabelling_experts_permutes_ids_only():
    layer, x = _layer_and_x()
    perm = np.random.default_rng(9).permutation(8)  # new expert j = old expert perm[j]
    lay2 = dict(layer)
    lay2["router_w"] = layer["router_w"][perm]
    for k in ("gate_q", "gate_s", "up_q", "up_s", "down_q", "down_s"):
        lay2[k] = layer[k][perm]
    ids, w, y, _ = O.moe_layer(x, layer, top_k=3)
    ids2, w2, y2, _ = O.moe_layer(x, lay2, top_k=3)
    np.testing.assert_array_equal(perm[ids2], ids)
    np.testing.assert_allclose(w2, w, rtol=1e-14)
    np.testing.assert_allclose(y2, y, rtol=1e-12, atol=1e-13)


def test_tokens_are_independent():
    layer, x = _layer_and_x()
    _, _, y, _ = O.moe_layer(x, layer, top_k=3)
    for t in range(x.shape[0]):
        _, _, yt, _ = O.moe_layer(x[t:t + 1], layer, top_k=3)
        # BLAS may block a batched product differently from a single row
        np.testing.assert_allclose(yt[0], y[t], rtol=1e-13, atol=1e-12)


def test_forced_ids_reproduce_free_routing():
    layer, x = _layer_and_x()
    ids, w, y, _ = O.moe_layer(x, layer, top_k=3)
    ids2, w2, y2, _ = O.moe_layer(x, layer, top_k=3, forced_ids=ids)
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(w2, w)


# ---------------------------------------------------------------- norm, rounding, chain
def test_rmsnorm_closed_forms():
    eps = 1e-6
    z = O.rmsnorm(np.array([[3.0, 4.0]]), eps)
    np.testing.assert_allclose(z, [[3 / math.sqrt(12.5 + eps), 4 / math.sqrt(12.5 + eps)]], rtol=1e-15)
    c = O.rmsnorm(np.full((1, 1280), 0.5), eps)
    np.testing.assert_allclose(c, 0.5 / math.sqrt(0.25 + eps), rtol=1e-15)
    h = np.random.default_rng(10).normal(size=(4, 1280))
    np.testing.assert_allclose(np.sqrt(np.mean(O.rmsnorm(h, 0.0) ** 2, axis=1)), 1.0, rtol=1e-14)


def test_bf16_round_ties_and_torch():
    one = 1.0
    assert O.bf16_round(one + 2 ** -8) == 1.0                      # tie -> even
    assert O.bf16_round(one + 3 * 2 ** -8) == one + 2 ** -6        # tie -> even (up)
    assert O.bf16_round(one + 2 ** -8 + 2 ** -30) == one + 2 ** -7  # no double rounding
    assert O.bf16_round(-(one + 2 ** -8 + 2 ** -30)) == -(one + 2 ** -7)
    v = np.random.default_rng(11).normal(0, 10, 20000).astype(np.float32)
    ref = torch.tensor(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(v.astype(np.float64)), ref)


def test_chain_with_zero_weights_is_identity():
    layer, x = _layer_and_x()
    for k in ("down_q", "shared_down_q"):
        layer[k] = np.zeros_like(layer[k])
    h, _ = O.moe_chain(x, [layer, layer], 1e-6, False, top_k=3)
    np.testing.assert_array_equal(h, x)


def test_chain_single_layer_is_norm_then_residual():
    layer, x = _layer_and_x()
    h, trace = O.moe_chain(x, [layer], 1e-6, True, top_k=3)
    z = O.bf16_round(O.rmsnorm(x, 1e-6))
    _, _, y, _ = O.moe_layer(z, layer, top_k=3)
    np.testing.assert_array_equal(h, x + y)
    np.testing.assert_array_equal(trace[0][2], z)


# ---------------------------------------------------------------- hand-worked chain
CHAIN_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_chain.json")


def _chain_fixture():
    d = json.load(open(CHAIN_GOLDEN))
    fmt = QFmt(d["bits"], d["group"])
    layers = []
    for raw in d["layers"]:
        lay = {}
        for k, v in raw.items():
            if k == "router_w":
                lay[k] = np.asarray(v, dtype=np.float64)
            elif k.endswith("_q"):
                lay[k] = np.asarray(v, dtype=np.int8)
            else:
                lay[k] = np.asarray(v, dtype=np.float32)
        lay.update(router_b=None, routed_fmt=fmt, shared_fmt=fmt)
        layers.append(lay)
    return d, layers


def test_tiny_chain_two_layers_hand_worked():
    d, layers = _chain_fixture()
    ex = d["expected"]
    x = np.asarray(d["x"], dtype=np.float64)[None]
    h, trace = O.moe_chain(x, layers, d["eps"], False, top_k=d["top_k"])
    np.testing.assert_allclose(trace[0][2][0], ex["z0"], rtol=1e-15)
    assert trace[0][0][0].tolist() == ex["ids1"]
    np.testing.assert_allclose(trace[0][1][0], ex["w1"], rtol=1e-14)
    np.testing.assert_allclose(trace[1][2][0], ex["z1"], rtol=1e-13)
    assert trace[1][0][0].tolist() == ex["ids2"]
    np.testing.assert_allclose(trace[1][1][0], ex["w2"], rtol=1e-13)
    np.testing.assert_allclose(h[0], ex["h2"], rtol=1e-13, atol=1e-14)
    h1, _ = O.moe_chain(x, layers[:1], d["eps"], False, top_k=d["top_k"])
    np.testing.assert_allclose(h1[0], ex["h1"], rtol=1e-13, atol=1e-14)


def test_tiny_chain_bf16_norm_hand_worked():
    d, layers = _chain_fixture()
    ex = d["expected"]["bf16_one_layer"]
    x = np.asarray(d["x"], dtype=np.float64)[None]
    h, trace = O.moe_chain(x, layers[:1], d["eps"], True, top_k=d["top_k"])
    np.testing.assert_array_equal(trace[0][2][0], ex["z0"])
    assert trace[0][0][0].tolist() == ex["ids1"]
    np.testing.assert_allclose(trace[0][1][0], ex["w1"], rtol=1e-14)
    np.testing.assert_allclose(h[0], ex["h1"], rtol=1e-13, atol=1e-14)


def _planted_chains():
    """Copies of the chain, each with one plausible wiring mistake."""
    def norm_of_x_every_layer(x, layers, eps, bf16, k):
        h = x.copy()
        for lay in layers:
            z = O.rmsnorm(x, eps)
            z = O.bf16_round(z) if bf16 else z
            h = h + O.moe_layer(z, lay, k)[2]
        return h

    def residual_onto_x(x, layers, eps, bf16, k):
        h = x.copy()
        for lay in layers:
            z = O.rmsnorm(h, eps)
            z = O.bf16_round(z) if bf16 else z
            h = x + O.moe_layer(z, lay, k)[2]
        return h

    def norm_after_residual(x, layers, eps, bf16, k):
        h = x.copy()
        for lay in layers:
            z = O.bf16_round(h) if bf16 else h
            h = O.rmsnorm(h + O.moe_layer(z, lay, k)[2], eps)
        return h

    def residual_onto_z(x, layers, eps, bf16, k):
        h = x.copy()
        for lay in layers:
            z = O.rmsnorm(h, eps)
            z = O.bf16_round(z) if bf16 else z
            h = z + O.moe_layer(z, lay, k)[2]
        return h

    def eps_outside_sqrt(x, layers, eps, bf16, k):
        h = x.copy()
        for lay in layers:
            z = h / (np.sqrt(np.mean(h * h, axis=-1, keepdims=True)) + eps)
            z = O.bf16_round(z) if bf16 else z
            h = h + O.moe_layer(z, lay, k)[2]
        return h

    def no_residual(x, layers, eps, bf16, k):
        h = x.copy()
        for lay in layers:
            z = O.rmsnorm(h, eps)
            z = O.bf16_round(z) if bf16 else z
            h = O.moe_layer(z, lay, k)[2]
        return h

    def rounding_before_norm(x, layers, eps, bf16, k):
        h = x.copy()
        for lay in layers:
            z = O.rmsnorm(O.bf16_round(h) if bf16 else h, eps)
            h = h + O.moe_layer(z, lay, k)[2]
        return h

    def layers_reversed(x, layers, eps, bf16, k):
        return O.moe_chain(x, layers[::-1], eps, bf16, top_k=k)[0]

    return [norm_of_x_every_layer, residual_onto_x, norm_after_residual, residual_onto_z,
            eps_outside_sqrt, no_residual, rounding_before_norm, layers_reversed]


@pytest.mark.parametrize("planted", _planted_chains(), ids=lambda f: f.__name__)
def test_tiny_chain_catches_planted_wiring_mistakes(planted):
    d, layers = _chain_fixture()
    x = np.asarray(d["x"], dtype=np.float64)[None]
    ex = d["expected"]
    wrong2 = planted(x, layers, d["eps"], False, d["top_k"])[0]
    wrong1b = planted(x, layers[:1], d["eps"], True, d["top_k"])[0]
    caught = (not np.allclose(wrong2, ex["h2"], rtol=1e-9, atol=1e-9)
              or not np.allclose(wrong1b, ex["bf16_one_layer"]["h1"], rtol=1e-9, atol=1e-9))
    assert caught, planted.__name__
