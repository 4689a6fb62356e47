"""GPU two-level 4-bit (Q4_K-style) experts vs the float64 oracle, through the
C ABI (needs an MI355X): the per-token layer path, the grouped path and the
persistent decode step, with the routed experts (and in some cases the
shared expert too) in the format."""
import dataclasses
import functools
import sys

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import NORM_EPS, QFmt, WORKLOADS, make_layer, make_tokens
from synth.workloads import Q4K_GROUP
from tests.conftest import gpu_available
from tests.parity import check_layer, check_output

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")

WL = WORKLOADS[7]                                             # routed two-level, shared int8 G128
WL_BOTH = dataclasses.replace(WL, shared=QFmt(4, Q4K_GROUP))  # shared expert in the format too


def say(*a):
    print("[q4k]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def layer_of(both: bool, li: int):
    return make_layer(WL_BOTH if both else WL, li)


@functools.lru_cache(maxsize=None)
def packed_of(both: bool, li: int):
    from quantized_expert_ffn_moe_amd import binding as B
    return B.pack_layer(layer_of(both, li))


def tokens(n, batch=0):
    x, _ = make_tokens(WL, batch=batch, n_tokens=n)
    return x.astype(np.float64), torch.from_numpy(x).cuda()


@pytest.mark.parametrize("both", [False, True])
@pytest.mark.parametrize("T", [1, 4, 13, 64])
def test_q4k_layer(lib, T, both):
    """moe_layer_forward with two-level experts (always the per-token path), up
    to its 64-token limit."""
    from quantized_expert_ffn_moe_amd import binding as B
    say(f"layer T={T} shared two-level={both}")
    x, xt = tokens(T, batch=T)
    ids, w, y = B.layer(xt, packed_of(both, 0))
    torch.cuda.synchronize()
    ratio, near = check_layer(x, layer_of(both, 0), ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy())
    say(f"  err/rms {ratio:.2e} near-ties {near}")


@pytest.mark.parametrize("both", [False, True])
@pytest.mark.parametrize("T", [5, 65, 300, 1000])
def test_q4k_grouped(lib, T, both):
    """The grouped path (forced below its default token count), f32 input:
    32-row tiles over several tiles per expert and a ragged last tile."""
    from quantized_expert_ffn_moe_amd import binding as B
    say(f"grouped T={T} shared two-level={both}")
    x, xt = tokens(T, batch=100 + T)
    ids, w, y = B.layer(xt, packed_of(both, 0), B.MOE_FORCE_GROUPED)
    torch.cuda.synchronize()
    ratio, near = check_layer(x, layer_of(both, 0), ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy())
    say(f"  err/rms {ratio:.2e} near-ties {near}")


def test_q4k_grouped_bf16_and_paths_agree(lib):
    """bf16 activations on the grouped path, and the same 40 tokens through the
    per-token path: both within the bar, identical routing."""
    from quantized_expert_ffn_moe_amd import binding as B
    x, xt = tokens(40, batch=7)
    xb = xt.to(torch.bfloat16)
    xv = xb.float().cpu().numpy().astype(np.float64)
    res = []
    for flags in (B.MOE_FORCE_GROUPED, B.MOE_FORCE_DECODE):
        ids, w, y = B.layer(xb, packed_of(True, 2), flags)
        torch.cuda.synchronize()
        ratio, _ = check_layer(xv, layer_of(True, 2), ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy())
        say(f"bf16 input, flags {flags}: err/rms {ratio:.2e}")
        res.append(ids.cpu().numpy())
    np.testing.assert_array_equal(res[0], res[1])


def test_q4k_normalised_bf16_input(lib):
    """RMSNorm inside the call with the normalised input rounded to bf16."""
    from quantized_expert_ffn_moe_amd import binding as B
    x, xt = tokens(5, batch=3)
    h = (xt * 3.0).contiguous()
    ids, w, y = B.layer(h, packed_of(False, 1), B.MOE_NORM_INPUT | B.MOE_NORM_BF16)
    torch.cuda.synchronize()
    z = O.bf16_round(O.rmsnorm(3.0 * x, NORM_EPS))
    ratio, _ = check_layer(z, layer_of(False, 1), ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy())
    say(f"norm + bf16 input: err/rms {ratio:.2e}")


def _decode(both, n_layers, xt, ws):
    from quantized_expert_ffn_moe_amd import binding as B
    packed = [packed_of(both, li) for li in range(n_layers)]
    y = torch.empty(1, 1280, dtype=torch.float32, device="cuda")
    ids = torch.empty(n_layers, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(n_layers, 6, dtype=torch.float32, device="cuda")
    B.moe_decode_forward(xt, y, packed, ids, w, ws, B.MOE_NORM_INPUT | B.MOE_ACCUMULATE)
    torch.cuda.synchronize()
    assert ws[8:12].view(torch.int32).item() == 0, "a wait inside the decode kernel timed out"
    return ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("both", [False, True])
def test_q4k_decode_step_11_layers(lib, both):
    """The 11-layer decode step in one launch: each layer checked on the GPU's
    own residual stream (prefix runs), then the whole step against 11 in-place
    moe_layer_forward calls, and two repeated calls bit for bit."""
    from quantized_expert_ffn_moe_amd import binding as B
    say(f"decode step, 11 two-level layers, shared two-level={both}")
    x, xt = tokens(1)
    ws = B.decode_workspace()
    hs = [x]
    for n in range(1, 12):
        ids, w, y = _decode(both, n, xt, ws)
        z = O.rmsnorm(hs[-1], NORM_EPS)
        ratio, near = check_layer(z, layer_of(both, n - 1), ids[-1:], w[-1:], y - hs[-1])
        say(f"  layer {n}: err/rms {ratio:.2e}")
        hs.append(y.astype(np.float64))
    h = xt.clone()
    lws = B.workspace(1)
    i1 = torch.empty(1, 6, dtype=torch.int32, device="cuda")
    w1 = torch.empty(1, 6, device="cuda")
    for li in range(11):
        B.moe_layer_forward(h, packed_of(both, li), h, i1, w1, lws, B.MOE_NORM_INPUT | B.MOE_ACCUMULATE)
    check_output(hs[-1], h.cpu().numpy().astype(np.float64), tol=1e-4)
    a = _decode(both, 11, xt, ws)
    b = _decode(both, 11, xt, ws)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("both", [False, True])
def test_q4k_grouped_chain_sampled(lib, both):
    """300 tokens through 3 two-level layers in place (RMSNorm + residual inside
    each call, grouped path), every layer checked on 12 sampled tokens against
    the oracle fed the GPU's own residual stream."""
    from quantized_expert_ffn_moe_amd import binding as B
    T, L = 300, 3
    x, xt = tokens(T, batch=31)
    h = xt.clone()
    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE
    ws = B.workspace(T)
    ids = torch.empty(T, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(T, 6, dtype=torch.float32, device="cuda")
    sample = np.sort(np.random.default_rng(3).choice(T, 12, replace=False))
    for li in range(L):
        h_in = h[sample].cpu().numpy().astype(np.float64)
        B.moe_layer_forward(h, packed_of(both, li), h, ids, w, ws, flags)
        torch.cuda.synchronize()
        out = h[sample].cpu().numpy().astype(np.float64) - h_in
        ratio, near = check_layer(O.rmsnorm(h_in, NORM_EPS), layer_of(both, li), ids.cpu().numpy()[sample],
                                  w.cpu().numpy()[sample], out)
        say(f"  grouped chain layer {li + 1}: err/rms {ratio:.2e} near-ties {near}")


def test_q4k_decode_step_bf16_input(lib):
    """The decode step with a bf16 input row (the residual stream widened from
    bf16 by the reducers)."""
    from quantized_expert_ffn_moe_amd import binding as B
    x, xt = tokens(1, batch=9)
    xb = xt.to(torch.bfloat16)
    xv = xb.float().cpu().numpy().astype(np.float64)
    ws = B.decode_workspace()
    ids, w, y = _decode(False, 2, xb, ws)
    z1 = O.rmsnorm(xv, NORM_EPS)
    ids1, w1, y1 = _decode(False, 1, xb, ws)
    check_layer(z1, layer_of(False, 0), ids1, w1, y1 - xv)
    np.testing.assert_array_equal(ids[:1], ids1)
    ratio, _ = check_layer(O.rmsnorm(y1.astype(np.float64), NORM_EPS), layer_of(False, 1), ids[1:], w[1:],
                           y - y1)
    say(f"bf16 input decode, layer 2: err/rms {ratio:.2e}")


@pytest.mark.parametrize("both", [False, True])
@pytest.mark.parametrize("T", [8, 85, 86, 682, 683])
def test_q4k_grouped_switch_points(lib, T, both):
    """Token counts on both sides of the grouped path's switches with two-level
    experts: the two-pass router (8), 16- and 32-row fused tiles (512 slots)
    and fused against unfused 32-row tiles (4096 slots)."""
    from quantized_expert_ffn_moe_amd import binding as B
    say(f"switch point T={T} shared two-level={both}")
    x, xt = tokens(T, batch=200 + T)
    ids, w, y = B.layer(xt, packed_of(both, 1))
    torch.cuda.synchronize()
    ratio, near = check_layer(x, layer_of(both, 1), ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy())
    say(f"  err/rms {ratio:.2e} near-ties {near}")
