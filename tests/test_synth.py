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
