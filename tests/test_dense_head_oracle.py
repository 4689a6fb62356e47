"""Pins for the dense-ends oracle (layer-0 SwiGLU MLP, lm_head + greedy
token): hand-worked values, closed forms, brute force and an independent
decoding of every bf16 pattern."""
import math
import struct

import numpy as np
import pytest

from oracle import dense_head as D
from synth import QFmt, make_dense_ffn, make_hidden, make_lm_head


# ---------------------------------------------------------------- bf16 decoding
def test_bf16_every_pattern_matches_ieee_binary32_top_half():
    bits = np.arange(1 << 16, dtype=np.uint32)
    got = D.bf16_bits_value(bits.astype(np.uint16))
    ref = np.array([struct.unpack("<f", struct.pack("<I", int(b) << 16))[0] for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_hand_values():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x3FC0 = 1.5, 0x0001 = smallest subnormal 2^-133
    got = D.bf16_bits_value(np.array([0x3F80, 0xC000, 0x3FC0, 0x0001, 0x8000], dtype=np.uint16))
    assert got.tolist()[:4] == [1.0, -2.0, 1.5, 2.0 ** -133]
    assert got[4] == 0.0 and math.copysign(1.0, got[4]) == -1.0


# ---------------------------------------------------------------- greedy token
def test_greedy_token_hand_cases():
    ids, v = D.greedy_token(np.array([[1.0, 3.0, 3.0, 2.0], [5.0, 5.0, 5.0, 5.0], [-np.inf, -1.0, -2.0, -1.0]]))
    assert ids.tolist() == [1, 0, 1]
    assert v.tolist() == [3.0, 5.0, -1.0]


def test_greedy_token_brute_force_with_many_ties():
    rng = np.random.default_rng(3)
    L = rng.integers(0, 4, size=(200, 37)).astype(np.float64)   # small range: ties everywhere
    ids, v = D.greedy_token(L)
    for t in range(L.shape[0]):
        best = 0
        for j in range(1, L.shape[1]):
            if L[t, j] > L[t, best]:
                best = j
        assert ids[t] == best and v[t] == L[t, best]


# ---------------------------------------------------------------- lm_head
def test_lm_head_hand_worked():
    # h = (3, 4): mean of squares 12.5, z = h / sqrt(12.5) (eps = 0)
    h = np.array([[3.0, 4.0]])
    W = np.array([[1, 0], [0, 1], [1, 1], [2, -1]], dtype=np.float64)
    z0, z1 = 3 / math.sqrt(12.5), 4 / math.sqrt(12.5)
    got = D.lm_head_logits(h, W, norm=True, eps=0.0)
    np.testing.assert_allclose(got[0], [z0, z1, z0 + z1, 2 * z0 - z1], rtol=1e-15)
    assert D.greedy_token(got)[0].tolist() == [2]
    raw = D.lm_head_logits(h, W, norm=False, eps=0.0)
    assert raw[0].tolist() == [3.0, 4.0, 7.0, 2.0]


def test_lm_head_one_hot_rows_pick_features():
    rng = np.random.default_rng(5)
    h = rng.standard_normal((3, 16))
    cols = rng.integers(0, 16, size=40)
    W = np.zeros((40, 16))
    W[np.arange(40), cols] = 1.0
    z = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(D.lm_head_logits(h, W, True, 1e-6), z[:, cols], rtol=1e-14)


def test_lm_head_constant_row_closed_form():
    # h = c * ones: z = c / sqrt(c^2 + eps) in every feature; logits = row sums * that
    c, eps = 0.5, 1e-6
    h = np.full((1, 8), c)
    W = np.arange(24, dtype=np.float64).reshape(3, 8) - 10.0
    zc = c / math.sqrt(c * c + eps)
    np.testing.assert_allclose(D.lm_head_logits(h, W, True, eps)[0], W.sum(axis=1) * zc, rtol=1e-14)


def test_lm_head_generators_shapes():
    hb = make_lm_head("bf16", vocab=1000)
    assert hb["w"].shape == (1000, 1280) and hb["w"].dtype == np.uint16
    hi = make_lm_head("int8", group=128, vocab=1000)
    assert hi["q"].shape == (1000, 1280) and hi["s"].shape == (1000, 10)
    assert np.abs(hi["q"]).max() <= 127
    h = make_hidden(4)
    assert h.shape == (4, 1280) and h.dtype == np.float32


# ---------------------------------------------------------------- dense SwiGLU
def _tiny_dense():
    one = np.ones((2, 2), np.float32)
    return {
        "gate_q": np.array([[1, 0, 0, 0], [0, 1, 0, 0]], np.int8), "gate_s": one,
        "up_q": np.array([[0, 0, 1, 0], [0, 0, 0, 1]], np.int8), "up_s": one.copy(),
        "down_q": np.array([[1, 0], [0, 1], [1, 1], [2, -1]], np.int8), "down_s": np.ones((4, 1), np.float32),
        "bits": 8, "group": 2, "inter": 2,
    }


def test_dense_ffn_hand_worked():
    ffn = _tiny_dense()
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    s1, s2 = 1 / (1 + math.exp(-1)), 2 / (1 + math.exp(-2))   # SiLU(1), SiLU(2)
    h0, h1 = s1 * 3, s2 * 4
    got = D.dense_ffn(x, ffn, norm=False, eps=0.0)
    np.testing.assert_allclose(got[0], [h0, h1, h0 + h1, 2 * h0 - h1], rtol=1e-15)


def test_dense_ffn_hand_worked_with_norm():
    ffn = _tiny_dense()
    x = np.array([[1.0, 2.0, 3.0, 4.0]])
    z = x[0] / math.sqrt(7.5)                 # mean of squares (1 + 4 + 9 + 16) / 4
    sil = lambda v: v / (1 + math.exp(-v))
    h0, h1 = sil(z[0]) * z[2], sil(z[1]) * z[3]
    np.testing.assert_allclose(D.dense_ffn(x, ffn, True, 0.0)[0], [h0, h1, h0 + h1, 2 * h0 - h1], rtol=1e-14)


def test_dense_ffn_scale_invariants():
    ffn = make_dense_ffn(QFmt(8, 64), inter=128)
    x = make_hidden(2)
    y = D.dense_ffn(x, ffn, True, 1e-6)
    f2 = dict(ffn, down_s=ffn["down_s"] * 2)
    np.testing.assert_allclose(D.dense_ffn(x, f2, True, 1e-6), 2 * y, rtol=1e-13)
    f3 = dict(ffn, up_s=ffn["up_s"] * 2)
    np.testing.assert_allclose(D.dense_ffn(x, f3, True, 1e-6), 2 * y, rtol=1e-13)
    f4 = dict(ffn, up_q=np.zeros_like(ffn["up_q"]))
    assert np.all(D.dense_ffn(x, f4, True, 1e-6) == 0.0)


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 32)])
def test_dense_ffn_full_shape_splits_over_the_intermediate(bits, group):
    """At the real shape (I = 6848) the MLP equals the sum of the two MLPs over
    two parts of the intermediate dimension, cut on a group boundary (catches
    a wrong axis there)."""
    ffn = make_dense_ffn(QFmt(bits, group))
    assert ffn["gate_q"].shape == (6848, 1280) and ffn["down_q"].shape == (1280, 6848)
    x = make_hidden(2)
    y = D.dense_ffn(x, ffn, True, 1e-6)
    half = 53 * 64
    parts = []
    for sl in (slice(0, half), slice(half, 6848)):
        gs = slice(sl.start // group, sl.stop // group)
        parts.append(D.dense_ffn(x, {"gate_q": ffn["gate_q"][sl], "gate_s": ffn["gate_s"][sl],
                                     "up_q": ffn["up_q"][sl], "up_s": ffn["up_s"][sl],
                                     "down_q": ffn["down_q"][:, sl], "down_s": ffn["down_s"][:, gs],
                                     "group": group}, True, 1e-6))
    np.testing.assert_allclose(parts[0] + parts[1], y, rtol=1e-10, atol=1e-10 * np.abs(y).max())
