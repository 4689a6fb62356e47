"""Pins of the oracle's two-level 4-bit (Q4_K-style) format (CPU only).

The pages name the format only (Unlimited-OCR DeepEncoder ONNX model card,
"The rest of the pipeline": the community K-quant decoder and the WebGPU
engine's q4k storage); the oracle takes the K-quant definition
W = d * sc * q - dmin * m.  The pins: a super-block worked out by hand (with
a partial second super-block), the special case that is the symmetric int4
format with groups of 32, the format's affine structure in q, and a layer
whose two-level weights equal a symmetric layer's.
"""
import json
import pathlib

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import QFmt, make_tiny_layer
from synth.workloads import Q4K_GROUP

GOLDEN = pathlib.Path(__file__).parent / "golden" / "q4k_superblock.json"


def test_hand_worked_superblock():
    g = json.loads(GOLDEN.read_text())
    K = g["row_length"]
    q = (np.arange(K) % 16).astype(np.uint8)[None, :]
    d = np.array([g["d_bits"]], dtype=np.uint16)
    dmin = np.array([g["dmin_bits"]], dtype=np.uint16)
    np.testing.assert_array_equal(O.f16_value(d)[0], g["d_values"])
    np.testing.assert_array_equal(O.f16_value(dmin)[0], g["dmin_values"])
    W = O.dequantize_q4k(q, d, dmin, np.array([g["sc"]], np.uint8), np.array([g["m"]], np.uint8))
    assert W.shape == (1, K)
    for e in g["expected"]:
        assert W[0, e["k"]] == e["w"], e


def _symmetric_case(rng, N, K):
    """Fields for which d sc q - dmin m = (d sc) (q - 8): dmin = d, m = 8 sc."""
    nsb, nsub = -(-K // 256), K // 32
    q = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
    d = rng.uniform(1e-3, 1e-2, size=(N, nsb)).astype(np.float16)
    sc = rng.integers(1, 8, size=(N, nsub)).astype(np.uint8)
    return q, d.view(np.uint16), d.view(np.uint16), sc, (8 * sc).astype(np.uint8)


@pytest.mark.parametrize("K", [256, 896, 1280, 1792])
def test_reduces_to_symmetric_int4_g32(K):
    rng = np.random.default_rng(K)
    q, d, dmin, sc, m = _symmetric_case(rng, 5, K)
    W = O.dequantize_q4k(q, d, dmin, sc, m)
    dsub = np.repeat(O.f16_value(d), 8, axis=1)[:, :K // 32]
    scales = (dsub * sc).astype(np.float32)           # exact: an f16 value times a 3-bit integer
    assert np.array_equal(scales.astype(np.float64), dsub * sc)
    ref = O.dequantize((q.astype(np.int16) - 8).astype(np.int8), scales, 32)
    np.testing.assert_array_equal(W, ref)


def test_affine_in_the_code():
    """W(q = 0) = -dmin m (no d, no sc) and W(q + 1) - W(q) = d sc (no dmin, no m)."""
    rng = np.random.default_rng(3)
    N, K = 4, 896
    f = {"d": rng.uniform(1e-4, 1e-2, (N, 4)).astype(np.float16).view(np.uint16),
         "dmin": rng.uniform(1e-4, 1e-2, (N, 4)).astype(np.float16).view(np.uint16),
         "sc": rng.integers(0, 64, (N, K // 32)).astype(np.uint8),
         "m": rng.integers(0, 64, (N, K // 32)).astype(np.uint8)}
    q = rng.integers(0, 15, (N, K)).astype(np.uint8)
    W0 = O.dequantize_q4k(np.zeros_like(q), **f)
    W1 = O.dequantize_q4k(q, **f)
    W2 = O.dequantize_q4k(q + 1, **f)
    sb = np.arange(K) // 256
    sub = np.arange(K) // 32
    dmin_k = np.asarray(f["dmin"]).view(np.float16).astype(np.float64)[:, sb]
    d_k = np.asarray(f["d"]).view(np.float16).astype(np.float64)[:, sb]
    np.testing.assert_array_equal(W0, -dmin_k * f["m"][:, sub])
    np.testing.assert_allclose(W2 - W1, d_k * f["sc"][:, sub], rtol=1e-12, atol=0)


def test_fields_out_of_range_are_rejected():
    q, d, dmin, sc, m = _symmetric_case(np.random.default_rng(0), 2, 256)
    with pytest.raises(ValueError):
        O.dequantize_q4k(q + 16, d, dmin, sc, m)
    with pytest.raises(ValueError):
        O.dequantize_q4k(q, d, dmin, sc + 64, m)
    with pytest.raises(ValueError):
        O.dequantize_q4k(q, d[:, :0], dmin, sc, m)


def _pair_of_layers(layer, names):
    """(symmetric layer, two-level layer) with equal weights: each named
    matrix gets scales d * sc (d an f16 value per 256 columns, sc in 1..7) in
    the symmetric copy and the fields q = code + 8, dmin = d, m = 8 sc in the
    two-level copy."""
    sym, two = dict(layer), dict(layer)
    for n in names:
        nsub = np.asarray(layer[f"{n}_s"]).shape[-1]
        lead = np.asarray(layer[f"{n}_s"]).shape[:-1]
        rng = np.random.default_rng(len(n))
        d = rng.uniform(1e-3, 1e-2, lead + (-(-nsub // 8),)).astype(np.float16)
        sc = rng.integers(1, 8, lead + (nsub,)).astype(np.uint8)
        sym[f"{n}_s"] = (np.repeat(d.astype(np.float64), 8, axis=-1)[..., :nsub] * sc).astype(np.float32)
        del two[f"{n}_s"]
        two[f"{n}_q"] = (np.asarray(layer[f"{n}_q"]).astype(np.int16) + 8).astype(np.uint8)
        two[f"{n}_d"] = two[f"{n}_dmin"] = d.view(np.uint16)
        two[f"{n}_sc"] = sc
        two[f"{n}_m"] = (8 * sc).astype(np.uint8)
    two["routed_fmt"] = two["shared_fmt"] = QFmt(4, Q4K_GROUP)
    return sym, two


def test_layer_with_two_level_weights_matches_the_symmetric_layer():
    """A layer whose two-level weights equal symmetric int4 G32 weights gives the
    symmetric layer's output (checks the oracle's format dispatch for routed and
    shared matrices, K = 512 with two super-blocks, intermediate 288 with a
    partial one)."""
    base = make_tiny_layer(21, E=8, H=512, I=288, Is=320, fmt=QFmt(4, 32))
    sym_layer, two = _pair_of_layers(base, ["gate", "up", "down", "shared_gate", "shared_up", "shared_down"])
    X = np.random.default_rng(5).standard_normal((7, 512))
    ids_s, w_s, y_s, _ = O.moe_layer(X, sym_layer, top_k=3)
    ids_t, w_t, y_t, _ = O.moe_layer(X, two, top_k=3)
    np.testing.assert_array_equal(ids_s, ids_t)
    np.testing.assert_allclose(y_t, y_s, rtol=1e-12, atol=1e-12)


def _variant(q, d, dmin, sc, m, mistake):
    """The two-level formula with one planted mistake (CPU only; never used
    outside this test)."""
    Q = np.asarray(q).astype(np.float64)
    K = Q.shape[1]
    D = np.repeat(O.f16_value(d), 256, axis=1)[:, :K]
    Dm = np.repeat(O.f16_value(dmin), 256, axis=1)[:, :K]
    S = np.repeat(np.asarray(sc, np.float64), 32, axis=1)
    M = np.repeat(np.asarray(m, np.float64), 32, axis=1)
    if mistake == "swap_d_dmin":
        D, Dm = Dm, D
    elif mistake == "swap_sc_m":
        S, M = M, S
    elif mistake == "plus_min":
        return D * S * Q + Dm * M
    elif mistake == "signed_codes":
        Q = Q - 8
    elif mistake == "sub_by_superblock":
        S = np.repeat(np.asarray(sc, np.float64)[:, ::8], 256, axis=1)[:, :K]
    return D * S * Q - Dm * M


@pytest.mark.parametrize("mistake", ["swap_d_dmin", "swap_sc_m", "plus_min", "signed_codes", "sub_by_superblock"])
def test_the_hand_worked_superblock_catches_planted_mistakes(mistake):
    g = json.loads(GOLDEN.read_text())
    K = g["row_length"]
    args = ((np.arange(K) % 16).astype(np.uint8)[None, :], np.array([g["d_bits"]], np.uint16),
            np.array([g["dmin_bits"]], np.uint16), np.array([g["sc"]], np.uint8), np.array([g["m"]], np.uint8))
    W = _variant(*args, mistake)
    assert any(W[0, e["k"]] != e["w"] for e in g["expected"]), mistake
    # and the unmutated formula agrees with the oracle
    np.testing.assert_array_equal(_variant(*args, "none"), O.dequantize_q4k(*args))
