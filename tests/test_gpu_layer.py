"""One whole decoder layer step through the C ABI against oracle/decoder_layer.py
(needs an MI355X): the attention half (RMSNorm, q/k/v projections, R-SWA, o
projection and residual; moe_attn_block_forward), then the MoE half
(moe_decode_forward for one token, moe_layer_forward for many streams), for
1, 4, 16 and 128 streams.

Bar: what each half adds to the residual within 1e-3 x rms of the oracle's
(each half checked on the GPU's own input to it); the rings bit-identical
except the new token's slot, whose bf16 rounding both sides decide from
their own key (a value at a rounding boundary may differ by one bf16 step);
the MoE routing as in the other parity tests.
"""
import functools
import sys

import numpy as np
import pytest

from oracle import decoder_layer as DL
from oracle import moe_oracle as O
from synth import NORM_EPS, WORKLOADS, bf16_bits_to_f32, make_attn_weights, make_hidden, make_layer, make_rswa
from tests.conftest import gpu_available
from tests.parity import check_layer

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")


def say(*a):
    print("[layer]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def attn_w():
    return make_attn_weights(0)


@functools.lru_cache(maxsize=None)
def attn_w64():
    return {k: bf16_bits_to_f32(v).astype(np.float64) for k, v in attn_w().items()}


def f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def run_attn(S, n_ref, n_gen, seed):
    from quantized_expert_ffn_moe_amd import binding as B
    kvh = make_rswa(S, n_ref, n_gen=n_gen, seed=seed)
    dev = B.rswa_to_device(kvh)
    h0 = make_hidden(S, batch=300 + seed)
    h = torch.from_numpy(h0).cuda()
    ws = torch.empty(B.moe_attn_block_workspace_bytes(S, n_ref), dtype=torch.uint8, device="cuda")
    B.moe_attn_block_forward(h, B.attn_weights_to_device(**attn_w()), dev, ws)
    torch.cuda.synchronize()
    return kvh, dev, h0, h


def check_attn(kvh, dev, h0, h, sample):
    w = attn_w64()
    h1 = h.cpu().numpy().astype(np.float64)
    ref_k, ref_v = f64(kvh["ref_k"]), f64(kvh["ref_v"])
    ring_k, ring_v = f64(kvh["ring_k"]), f64(kvh["ring_v"])
    got_rk = dev["ring_k"].cpu().numpy().view(np.uint16)
    got_rv = dev["ring_v"].cpu().numpy().view(np.uint16)
    outs, refs = [], []
    for s in sample:
        ho, rings = DL.attn_block(h0[s:s + 1].astype(np.float64), w["w_q"], w["w_k"], w["w_v"], w["w_o"],
                                  ref_k[s:s + 1], ref_v[s:s + 1], ring_k[s:s + 1], ring_v[s:s + 1],
                                  kvh["n_gen"][s:s + 1], NORM_EPS)
        refs.append(ho[0] - h0[s])
        outs.append(h1[s] - h0[s])
        slot = int(kvh["n_gen"][s]) % 128
        rk_o, rv_o = rings[0]
        for got, ref_ring, old in ((got_rk[s], rk_o, kvh["ring_k"][s]), (got_rv[s], rv_o, kvh["ring_v"][s])):
            keep = np.ones(128, bool)
            keep[slot] = False
            np.testing.assert_array_equal(got[:, keep], old[:, keep])          # other slots untouched
            # the new slot: the bf16 rounding of the key and value is decided
            # by each side from its own f32 / f64 value, so a value at a
            # rounding boundary may land one bf16 step away, and a value near
            # zero may differ by the f32 projection's error (1e-4 of the
            # vector's largest element bounds it); no more than that
            new = bf16_bits_to_f32(got[:, slot]).astype(np.float64)
            ref = ref_ring[:, slot]
            step = np.ldexp(1.0, np.frexp(np.maximum(np.abs(new), np.abs(ref)))[1] - 8)   # one bf16 step
            allowed = np.maximum(step, 1e-4 * np.abs(ref).max())
            diff = np.abs(new - ref)
            assert np.all(diff <= allowed), float((diff / allowed).max())
            assert np.mean(diff > 0) < 0.02, float(np.mean(diff > 0))
    outs, refs = np.array(outs), np.array(refs)
    rms = np.sqrt(np.mean(refs ** 2))
    ratio = float(np.abs(outs - refs).max() / rms)
    assert ratio <= 1e-3, ratio
    return ratio


@pytest.mark.parametrize("S,n_ref", [(1, 288), (1, 0), (2, 0), (4, 288), (5, 288), (16, 64), (17, 288), (65, 64),
                                     (128, 288)])
def test_attn_block(lib, S, n_ref):
    n_gen = [127 + 53 * s for s in range(S)]
    say(f"attention block, {S} streams, n_ref {n_ref}")
    kvh, dev, h0, h = run_attn(S, n_ref, n_gen, seed=S)
    # every stream up to 17 (the split-row projections start at 16 streams); else 12, the last one included
    sample = np.arange(S) if S <= 17 else np.sort(np.append(np.random.default_rng(S).choice(S - 1, 11, replace=False), S - 1))
    r = check_attn(kvh, dev, h0, h, sample)
    say(f"  attention half err/rms {r:.2e} on {len(sample)} streams")


def test_decoder_layer_one_token(lib):
    """Attention half, then the persistent decode step with one layer."""
    from quantized_expert_ffn_moe_amd import binding as B
    wl = WORKLOADS[1]
    layer = make_layer(wl, 0)
    say("decoder layer step, 1 token (attention + MoE int4 G64 / int8 G128)")
    kvh, dev, h0, h = run_attn(1, 288, [200], seed=41)
    r1 = check_attn(kvh, dev, h0, h, [0])
    h1 = h.clone()
    y = torch.empty(1, 1280, dtype=torch.float32, device="cuda")
    ids = torch.empty(1, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(1, 6, dtype=torch.float32, device="cuda")
    ws = B.decode_workspace()
    B.moe_decode_forward(h1, y, [B.pack_layer(layer)], ids, w, ws, B.MOE_NORM_INPUT | B.MOE_ACCUMULATE)
    torch.cuda.synchronize()
    assert ws[8:12].view(torch.int32).item() == 0
    h1n = h1.cpu().numpy().astype(np.float64)
    r2, _ = check_layer(O.rmsnorm(h1n, NORM_EPS), layer, ids.cpu().numpy(), w.cpu().numpy(),
                        y.cpu().numpy() - h1n)
    say(f"  attention half {r1:.2e}, MoE half {r2:.2e}")


def test_decoder_layer_128_streams(lib):
    """Attention half for 128 streams, then moe_layer_forward in place."""
    from quantized_expert_ffn_moe_amd import binding as B
    S = 128
    wl = WORKLOADS[5]
    layer = make_layer(wl, 0)
    say("decoder layer step, 128 streams")
    kvh, dev, h0, h = run_attn(S, 288, None, seed=42)
    sample = np.sort(np.random.default_rng(7).choice(S, 12, replace=False))
    r1 = check_attn(kvh, dev, h0, h, sample)
    h1 = h.clone()
    ids = torch.empty(S, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(S, 6, dtype=torch.float32, device="cuda")
    B.moe_layer_forward(h, B.pack_layer(layer), h, ids, w, B.workspace(S), B.MOE_NORM_INPUT | B.MOE_ACCUMULATE)
    torch.cuda.synchronize()
    h1n = h1.cpu().numpy().astype(np.float64)[sample]
    r2, _ = check_layer(O.rmsnorm(h1n, NORM_EPS), layer, ids.cpu().numpy()[sample], w.cpu().numpy()[sample],
                        h.cpu().numpy()[sample] - h1n)
    say(f"  attention half {r1:.2e}, MoE half {r2:.2e} on {len(sample)} streams")


def test_attn_block_empty_and_errors(lib):
    from quantized_expert_ffn_moe_amd import binding as B
    ws = torch.empty(B.moe_attn_block_workspace_bytes(0, 8), dtype=torch.uint8, device="cuda")
    dev = B.rswa_to_device(make_rswa(0, 8, n_gen=[]))
    h = torch.empty(0, 1280, dtype=torch.float32, device="cuda")
    B.moe_attn_block_forward(h, B.attn_weights_to_device(**attn_w()), dev, ws)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    dev1 = B.rswa_to_device(make_rswa(1, 8, n_gen=[3]))
    with pytest.raises(B.MoeError, match="WORKSPACE"):
        B.moe_attn_block_forward(torch.zeros(1, 1280, device="cuda"), B.attn_weights_to_device(**attn_w()), dev1, small)
