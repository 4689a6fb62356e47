"""GPU library vs the float64 oracle, through the C ABI (needs an MI355X)."""
import functools
import sys

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import NORM_EPS, WORKLOADS, make_layer, make_tokens
from tests.conftest import gpu_available
from tests.parity import check_layer, check_output

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")


def say(*a):
    print("[parity]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def layer_of(wi: int, li: int):
    return make_layer(WORKLOADS[wi], li)


@functools.lru_cache(maxsize=None)
def packed_of(wi: int, li: int):
    from quantized_expert_ffn_moe_amd import binding as B
    return B.pack_layer(layer_of(wi, li))


def tokens(wi, n=None, batch=0):
    x, bits = make_tokens(WORKLOADS[wi], batch=batch, n_tokens=n)
    if bits is not None:
        xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        xt = torch.from_numpy(x).cuda()
    return x.astype(np.float64), xt


def run(xt, packed, flags=0):
    from quantized_expert_ffn_moe_amd import binding as B
    ids, w, y = B.layer(xt, packed, flags)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("wi,path", [(0, "decode"), (0, "grouped"), (2, "grouped"), (2, "decode"),
                                     (3, "grouped")])
def test_single_layer_full_size(lib, wi, path):
    from quantized_expert_ffn_moe_amd import binding as B
    flags = B.MOE_FORCE_DECODE if path == "decode" else B.MOE_FORCE_GROUPED
    say(f"workload {WORKLOADS[wi].name} path {path}")
    x, xt = tokens(wi)
    ids, w, y = run(xt, packed_of(wi, 0), flags)
    ratio, near = check_layer(x, layer_of(wi, 0), ids, w, y)
    say(f"  err/rms {ratio:.2e} near-ties {near}")


@pytest.mark.parametrize("T", [2, 3, 5, 7, 31, 33, 64, 100])
def test_ragged_token_counts_both_paths(lib, T):
    from quantized_expert_ffn_moe_amd import binding as B
    x, xt = tokens(2, n=T, batch=7)
    say(f"T={T}")
    res = {}
    paths = (("decode", B.MOE_FORCE_DECODE), ("grouped", B.MOE_FORCE_GROUPED)) if T <= 64 else \
        (("grouped", B.MOE_FORCE_GROUPED), ("grouped-default", 0))
    for name, flags in paths:
        ids, w, y = run(xt, packed_of(2, 0), flags)
        ratio, _ = check_layer(x, layer_of(2, 0), ids, w, y)
        res[name] = (ids, y)
        say(f"  {name}: err/rms {ratio:.2e}")
    a, b = list(res.values())
    np.testing.assert_array_equal(a[0], b[0])


# the default per-token / grouped switch of each format (the last token count
# that takes the per-token path; measured crossovers of one layer call)
SWITCH = {5: 18, 2: 6, 0: 12, 3: 13, 7: 16}


@pytest.mark.parametrize("wi,T", [(wi, SWITCH[wi] + d) for wi in (5, 2, 0, 3, 7) for d in (0, 1)])
def test_default_path_switch(lib, wi, T):
    """Default flags on both sides of the per-token / grouped switch of each
    format (int4 G64 / int8 G128 f32, int4 G32 bf16, int8 G128 f32, int4 G128
    bf16, two-level / int8 G128 f32): the default call must equal the forced
    call of the path it takes, and both paths match the oracle."""
    from quantized_expert_ffn_moe_amd import binding as B
    say(f"{WORKLOADS[wi].name}: {T} tokens, default path")
    x, xt = tokens(wi, n=T, batch=17)
    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE if WORKLOADS[wi].n_layers > 1 else 0
    if flags:
        # the chained formats: the layer as a decoder calls it (norm and residual in the call)
        y0 = torch.from_numpy(x.astype(np.float32)).cuda()
        outs = []
        for f in (0, B.MOE_FORCE_DECODE if T <= SWITCH[wi] else B.MOE_FORCE_GROUPED):
            ids, w, y = B.layer(y0, packed_of(wi, 0), flags | f, y=y0.clone())
            torch.cuda.synchronize()
            outs.append((ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()))
        for u, v in zip(*outs):
            np.testing.assert_array_equal(u, v)
        z = O.rmsnorm(x, NORM_EPS)
        ids, w, y = outs[0]
        ratio, _ = check_layer(z, layer_of(wi, 0), ids, w, y - x.astype(np.float32))
    else:
        d = run(xt, packed_of(wi, 0))
        f = run(xt, packed_of(wi, 0), B.MOE_FORCE_DECODE if T <= SWITCH[wi] else B.MOE_FORCE_GROUPED)
        for u, v in zip(d, f):
            np.testing.assert_array_equal(u, v)
        ratio, _ = check_layer(x, layer_of(wi, 0), *d)
    say(f"  err/rms {ratio:.2e}")


@pytest.mark.parametrize("wi,T", [(2, 8), (2, 85), (2, 86), (2, 682), (2, 683), (5, 85), (5, 86), (5, 683)])
def test_tile_shape_boundaries(lib, wi, T):
    """Token counts on both sides of the grouped path's switches: the two-pass
    router (from 8 tokens), 16- and 32-row fused tiles (512 slots), small and
    large tiles (4096 slots, where the histogram also goes multi-workgroup
    above); one format pair (int4 G32) and the mixed one (int4 G64 routed,
    int8 G128 shared, f32 input)."""
    say(f"workload {wi} T={T}")
    x, xt = tokens(wi, n=T, batch=11)
    ids, w, y = run(xt, packed_of(wi, 0), 0)
    ratio, near = check_layer(x, layer_of(wi, 0), ids, w, y)
    say(f"  err/rms {ratio:.2e} near-ties {near}")


@pytest.mark.parametrize("bits,T", [(8, 150), (8, 700), (4, 1100)])
def test_g32_grouped_small_tiles(lib, bits, T):
    """Groups of 32 (routed and shared) on the grouped path, which keeps them on
    the 32-row fused small tiles at every token count: int8 at 150 and 700
    tokens, int4 at 1100 (6600 slots)."""
    from dataclasses import replace
    from quantized_expert_ffn_moe_amd import binding as B
    from synth import QFmt
    wl = replace(WORKLOADS[2], routed=QFmt(bits, 32), shared=QFmt(bits, 32))
    layer = make_layer(wl, 0)
    x, bits = make_tokens(wl, batch=5, n_tokens=T)
    xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    ids, w, y = run(xt, B.pack_layer(layer), B.MOE_FORCE_GROUPED)
    ratio, near = check_layer(x.astype(np.float64), layer, ids, w, y)
    say(f"int{bits} G32 T={T}: err/rms {ratio:.2e} near-ties {near}")


def test_mixed_formats_f32_input_grouped(lib):
    """int4 G64 routed + int8 G128 shared with f32 activations (hi/lo split operands)."""
    from quantized_expert_ffn_moe_amd import binding as B
    x, xt = tokens(1, n=40, batch=3)
    ids, w, y = run(xt, packed_of(1, 0), B.MOE_FORCE_GROUPED)
    ratio, _ = check_layer(x, layer_of(1, 0), ids, w, y)
    say(f"mixed formats grouped err/rms {ratio:.2e}")


def test_all_tokens_on_few_experts(lib):
    """A huge bias on experts 0..5 sends every token to them: several tiles per expert."""
    from quantized_expert_ffn_moe_amd import binding as B
    lay = dict(layer_of(3, 0))
    b = np.zeros(64, np.float32); b[:6] = 60.0 - 8.0 * np.arange(6)
    lay["router_b"] = b
    packed = dict(packed_of(3, 0)); packed["router_b"] = torch.from_numpy(b).cuda()
    x, xt = tokens(3, n=150, batch=5)
    ids, w, y = run(xt, packed, B.MOE_FORCE_GROUPED)
    assert np.all(ids == np.arange(6)[None, :])
    ratio, _ = check_layer(x, lay, ids, w, y)
    say(f"skewed err/rms {ratio:.2e}")


def test_deterministic_and_empty(lib):
    from quantized_expert_ffn_moe_amd import binding as B
    x, xt = tokens(3)
    a = run(xt, packed_of(3, 0))
    b = run(xt, packed_of(3, 0))
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)
    ids, w, y = B.layer(xt[:0], packed_of(3, 0))
    assert y.shape == (0, 1280)


@pytest.mark.parametrize("zdt", ["f32", "bf16"])
def test_rmsnorm(lib, zdt):
    from quantized_expert_ffn_moe_amd import binding as B
    h = np.random.default_rng(3).normal(0, 3, (37, 1280)).astype(np.float32)
    ht = torch.from_numpy(h).cuda()
    z = torch.empty(37, 1280, dtype=torch.float32 if zdt == "f32" else torch.bfloat16, device="cuda")
    B.moe_rmsnorm(ht, z, NORM_EPS)
    zg = z.float().cpu().numpy().astype(np.float64)
    zo = O.rmsnorm(h.astype(np.float64), NORM_EPS)
    if zdt == "f32":
        np.testing.assert_allclose(zg, zo, rtol=2e-6, atol=0)
    else:
        # the rounding decision is taken on an fp32 z: at most one bf16 ulp apart
        np.testing.assert_allclose(zg, zo, rtol=2 ** -8 + 2e-6, atol=0)
        assert np.mean(zg == O.bf16_round(zo)) > 0.999


def _chain(wi, T, sample):
    """Run the whole chain in place (RMSNorm + residual inside each call), then
    check every layer on the sampled tokens against the oracle, teacher-forced
    with the GPU's own residual stream and normalised input."""
    from quantized_expert_ffn_moe_amd import binding as B
    wl = WORKLOADS[wi]
    x, xt = tokens(wi, n=T)
    h = xt.float().contiguous()
    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE | (B.MOE_NORM_BF16 if wl.norm_bf16 else 0)
    ws = B.workspace(T)
    ids_l, w_l, h_l = [], [], [h.clone()]
    ids = torch.empty(T, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(T, 6, dtype=torch.float32, device="cuda")
    for li in range(wl.n_layers):
        B.moe_layer_forward(h, packed_of(wi, li), h, ids, w, ws, flags)
        ids_l.append(ids.cpu().numpy()); w_l.append(w.cpu().numpy()); h_l.append(h.clone())
    torch.cuda.synchronize()
    zdt = torch.bfloat16 if wl.norm_bf16 else torch.float32
    worst = 0.0
    for li in range(wl.n_layers):
        hin = h_l[li][sample].contiguous()
        z = torch.empty(len(sample), 1280, dtype=zdt, device="cuda")
        B.moe_rmsnorm(hin, z, NORM_EPS)
        zin = z.float().cpu().numpy().astype(np.float64)
        out = (h_l[li + 1][sample] - h_l[li][sample]).cpu().numpy()
        ratio, near = check_layer(zin, layer_of(wi, li), ids_l[li][sample], w_l[li][sample], out)
        worst = max(worst, ratio)
        say(f"  layer {li + 1}: err/rms {ratio:.2e} near-ties {near}")
    # end to end, from the same input, without teacher forcing
    # (only on tokens whose routing agrees at every layer: a near-tie may
    # legitimately send the two sides down different experts)
    h_o, trace = O.moe_chain(x[sample], [layer_of(wi, li) for li in range(wl.n_layers)], NORM_EPS, wl.norm_bf16)
    same = np.ones(len(sample), bool)
    for li in range(wl.n_layers):
        same &= np.all(trace[li][0] == ids_l[li][sample], axis=1)
    assert same.sum() >= len(sample) // 2
    e2e = check_output(h_l[-1][sample][same].cpu().numpy() - x[sample][same], h_o[same] - x[sample][same])
    say(f"  end-to-end err/rms {e2e:.2e} on {same.sum()}/{len(sample)} tokens (worst layer {worst:.2e})")


def test_chain_decode_11_layers(lib):
    say("11-layer decode chain, 1 token")
    _chain(1, 1, np.array([0]))


def test_chain_multipage_prefill_11_layers_sampled(lib):
    say("11-layer multi-page prefill, 2184 tokens, 24 sampled")
    sample = np.sort(np.random.default_rng(0).choice(2184, 24, replace=False))
    _chain(4, 2184, sample)


@pytest.mark.parametrize("wi", [5, 6])
def test_chain_continuous_batch_decode_sampled(lib, wi):
    """One continuous-batch decode step (128 or 256 streams, 11 chained layers)."""
    T = WORKLOADS[wi].n_tokens
    say(f"11-layer continuous-batch decode step, {T} streams, 16 sampled")
    sample = np.sort(np.random.default_rng(wi).choice(T, 16, replace=False))
    _chain(wi, T, sample)


def _decode_step(wi, n_layers, xt, flags):
    from quantized_expert_ffn_moe_amd import binding as B
    packed = [packed_of(wi, li) for li in range(n_layers)]
    y = torch.empty(1, 1280, dtype=torch.float32, device="cuda")
    ids = torch.empty(n_layers, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(n_layers, 6, dtype=torch.float32, device="cuda")
    ws = _decode_step.ws if hasattr(_decode_step, "ws") else B.decode_workspace()
    _decode_step.ws = ws
    B.moe_decode_forward(xt, y, packed, ids, w, ws, flags)
    torch.cuda.synchronize()
    err = ws[8:12].view(torch.int32).item()
    assert err == 0, "a wait inside the decode kernel timed out"
    return ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()


def test_decode_step_single_layer_int8(lib):
    """One layer, no norm, no residual (the int8 G128 single-token workload) in one launch."""
    say("persistent decode step, 1 layer int8 G128")
    x, xt = tokens(0)
    ids, w, y = _decode_step(0, 1, xt, 0)
    ratio, near = check_layer(x, layer_of(0, 0), ids, w, y)
    say(f"  err/rms {ratio:.2e}")


def test_decode_step_11_layers_per_layer(lib):
    """The 11-layer decode step: every prefix of the chain checked layer by layer."""
    from quantized_expert_ffn_moe_amd import binding as B
    say("persistent decode step, 11 layers")
    x, xt = tokens(1)
    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE
    hs = [x.astype(np.float64)]
    all_ids = None
    for n in range(1, 12):
        ids, w, y = _decode_step(1, n, xt, flags)
        if all_ids is not None:
            np.testing.assert_array_equal(ids[:-1], all_ids)   # prefixes route identically
        all_ids = ids
        z = O.rmsnorm(hs[-1], NORM_EPS)
        ratio, near = check_layer(z, layer_of(1, n - 1), ids[-1:], w[-1:], y - hs[-1])
        say(f"  layer {n}: err/rms {ratio:.2e}")
        hs.append(y.astype(np.float64))
    # same chain through moe_layer_forward, in place
    h = xt.clone()
    ws = B.workspace(1)
    i1 = torch.empty(1, 6, dtype=torch.int32, device="cuda"); w1 = torch.empty(1, 6, device="cuda")
    for li in range(11):
        B.moe_layer_forward(h, packed_of(1, li), h, i1, w1, ws, flags)
    hl = h.cpu().numpy()
    check_output(hs[-1], hl.astype(np.float64), tol=1e-4)
    # repeated calls on the same workspace (call counter) give the same bits
    a = _decode_step(1, 11, xt, flags)
    b = _decode_step(1, 11, xt, flags)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_decode_step_bf16_input_biased(lib):
    """bf16 input token, biased router, int4 G32 experts, 3 chained layers."""
    from quantized_expert_ffn_moe_amd import binding as B
    x, xt = tokens(2, n=1, batch=11)
    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE
    ids, w, y = _decode_step(2, 1, xt, flags)
    z = O.rmsnorm(x.astype(np.float64), NORM_EPS)
    ratio, _ = check_layer(z, layer_of(2, 0), ids, w, y - x)
    say(f"bf16 decode step err/rms {ratio:.2e}")
