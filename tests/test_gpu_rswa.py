"""GPU R-SWA attention decode step vs the float64 oracle, through the C ABI
(needs an MI355X)."""
import sys

import numpy as np
import pytest

from oracle import rswa as R
from oracle.dense_head import bf16_bits_value
from synth import f32_to_bf16_bits, make_rswa
from tests.conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")


def say(*a):
    print("[rswa]", *a, flush=True)
    sys.stdout.flush()


def run(d):
    from quantized_expert_ffn_moe_amd import binding as B
    dev = B.rswa_to_device(d)
    S = d["q"].shape[0]
    out = torch.full((S, 10, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.moe_rswa_workspace_bytes(S, d["n_ref"]), dtype=torch.uint8, device="cuda")
    B.moe_rswa_decode(dev, out, ws)
    torch.cuda.synchronize()
    ring_k = dev["ring_k"].cpu().numpy().view(np.uint16)
    ring_v = dev["ring_v"].cpu().numpy().view(np.uint16)
    return out.cpu().numpy(), ring_k, ring_v


def check(d, streams=None):
    """Every checked stream: output within 1e-3 x rms of the oracle's, and the
    updated ring bit-exact (the same bf16 rounding of the same f32 values)."""
    out, ring_k, ring_v = run(d)
    worst = 0.0
    for s in (range(d["q"].shape[0]) if streams is None else streams):
        ref, rk, rv = R.rswa_decode(d["q"][s].astype(np.float64), d["k_new"][s].astype(np.float64),
                                    d["v_new"][s].astype(np.float64),
                                    bf16_bits_value(d["ref_k"][s]), bf16_bits_value(d["ref_v"][s]),
                                    bf16_bits_value(d["ring_k"][s]), bf16_bits_value(d["ring_v"][s]), int(d["n_gen"][s]))
        rms = np.sqrt(np.mean(ref ** 2))
        err = np.abs(out[s] - ref).max()
        assert err <= 1e-3 * rms, (s, err, rms)
        worst = max(worst, err / rms)
        assert np.array_equal(ring_k[s], f32_to_bf16_bits(rk.astype(np.float32)))
        assert np.array_equal(ring_v[s], f32_to_bf16_bits(rv.astype(np.float32)))
    return worst


@pytest.mark.parametrize("S", [4, 16])
@pytest.mark.parametrize("n_ref", [0, 1, 63, 64, 65, 288, 1000])
def test_rswa_reference_lengths(lib, n_ref, S):
    """4 streams take the split-KV path, 16 the one-workgroup-per-row path."""
    d = make_rswa(S, n_ref, n_gen=[0, 5, 127, 300] * (S // 4), seed=n_ref)
    worst = check(d)
    say(f"{S} streams, n_ref {n_ref}: err/rms {worst:.2e}")


@pytest.mark.parametrize("S", [3, 16])
def test_rswa_first_token_without_reference_is_its_value(lib, S):
    """n_ref = 0 and n_gen = 0: one key, so the output is the new value (as bf16)."""
    d = make_rswa(S, 0, n_gen=[0] * S, seed=5)
    out, _, _ = run(d)
    np.testing.assert_array_equal(out, bf16_bits_value(f32_to_bf16_bits(d["v_new"])).astype(np.float32))


def test_rswa_continuous_batch_128_streams(lib):
    d = make_rswa(128, 288, seed=11)
    worst = check(d, streams=range(0, 128, 9))
    say(f"128 streams, n_ref 288: err/rms {worst:.2e}")


def test_rswa_long_reference(lib):
    d = make_rswa(2, 4400, n_gen=[50, 1000], seed=13)
    check(d)


def test_rswa_deterministic(lib):
    d = make_rswa(5, 300, seed=17)
    a = run(d)
    b = run(d)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
