"""The seeded generators: determinism, ranges, shapes and the bf16 input rounding."""
import numpy as np
import torch

from synth import (HIDDEN, INTER, N_EXPERTS, SHARED_INTER, WORKLOADS, bf16_bits_to_f32,
                   f32_to_bf16_bits, make_layer, make_tokens)


def test_layers_are_deterministic_and_in_range():
    wl = WORKLOADS[2]
    a, b = make_layer(wl, 0), make_layer(wl, 0)
    for k in a:
        if isinstance(a[k], np.ndarray):
            np.testing.assert_array_equal(a[k], b[k])
    assert a["gate_q"].shape == (N_EXPERTS, INTER, HIDDEN)
    assert a["down_q"].shape == (N_EXPERTS, HIDDEN, INTER)
    assert a["shared_down_q"].shape == (HIDDEN, SHARED_INTER)
    assert a["gate_q"].min() == -8 and a["gate_q"].max() == 7
    assert a["gate_s"].shape == (N_EXPERTS, INTER, HIDDEN // 32)
    assert 0.002 <= a["gate_s"].min() and a["gate_s"].max() <= 0.02
    c = make_layer(wl, 1)
    assert not np.array_equal(a["gate_q"], c["gate_q"])


def test_int8_codes_range():
    a = make_layer(WORKLOADS[0], 0)
    assert a["gate_q"].min() == -127 and a["gate_q"].max() == 127


def test_zipf_bias():
    b = make_layer(WORKLOADS[4], 0)["router_b"]
    np.testing.assert_allclose(b, 2.0 * np.log(1.0 / np.arange(1, 65)), rtol=1e-6)


def test_bf16_tokens_round_like_torch():
    x, bits = make_tokens(WORKLOADS[3])
    assert x.shape == (273, HIDDEN) and bits.dtype == np.uint16
    raw = np.random.default_rng(0).normal(size=5000).astype(np.float32)
    ref = torch.tensor(raw).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(raw), ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ref), torch.tensor(raw).to(torch.bfloat16).float().numpy())


def test_two_level_layer_fields():
    """Workload 7: routed experts in the two-level format (fields in range, the
    stated distributions), the shared expert in int8 G128."""
    a = make_layer(WORKLOADS[7], 0)
    assert WORKLOADS[7].routed.q4k and not WORKLOADS[7].shared.q4k
    assert a["gate_q"].shape == (N_EXPERTS, INTER, HIDDEN) and a["gate_q"].dtype == np.uint8
    assert a["gate_q"].min() == 0 and a["gate_q"].max() == 15
    assert a["down_d"].shape == (N_EXPERTS, HIDDEN, 4) and a["up_d"].shape == (N_EXPERTS, INTER, 5)
    assert a["down_sc"].shape == (N_EXPERTS, HIDDEN, INTER // 32)
    d = a["gate_d"].view(np.float16).astype(np.float64)
    dmin = a["gate_dmin"].view(np.float16).astype(np.float64)
    assert 1e-4 * 0.999 <= d.min() and d.max() <= 4e-4 * 1.001
    np.testing.assert_allclose(dmin, 8 * d, rtol=2 ** -10)
    sc, m = a["gate_sc"].astype(int), a["gate_m"].astype(int)
    assert sc.min() == 8 and sc.max() == 63
    assert np.all(m <= sc) and np.all(m >= np.maximum(sc - 8, 0))
    assert "gate_s" not in a and a["shared_gate_q"].dtype == np.int8
    b = make_layer(WORKLOADS[7], 0)
    for k in ("gate_q", "down_d", "up_m"):
        np.testing.assert_array_equal(a[k], b[k])
