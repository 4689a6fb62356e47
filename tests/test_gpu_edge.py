"""Edge cases of the MoE layer on the GPU, through the C ABI (needs an MI355X):

* exact router ties: equal probabilities go to the lower expert index (the
  greedy pick of the browser demo page "A 3-billion-parameter OCR model. In
  this tab.", "One forward pass, left to right", step 6, with ties read as
  lower index first), on the per-token path, the grouped path and the decode
  step, at the top of the list and at the 6th/7th boundary;
* int8 code -128, which the format allows (the README's int8 recipe stores
  signed bytes) and the workloads never draw;
* the largest call the header allows (8192 tokens) on the grouped path;
* non-finite input rows: ids stay six distinct experts in 0..63 and the
  finite tokens are unaffected.
"""
import functools
import sys

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import NORM_EPS, WORKLOADS, make_layer, make_tokens
from tests.conftest import gpu_available
from tests.parity import check_layer

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")


def say(*a):
    print("[edge]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def base_layer(wi: int, li: int = 0):
    return make_layer(WORKLOADS[wi], li)


def tokens(wi, n, batch=0):
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


def decode_step(xt, packed_layers, flags, ws=None):
    from quantized_expert_ffn_moe_amd import binding as B
    n = len(packed_layers)
    y = torch.empty(1, 1280, dtype=torch.float32, device="cuda")
    ids = torch.empty(n, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(n, 6, dtype=torch.float32, device="cuda")
    ws = B.decode_workspace() if ws is None else ws
    B.moe_decode_forward(xt, y, packed_layers, ids, w, ws, flags)
    torch.cuda.synchronize()
    assert ws[8:12].view(torch.int32).item() == 0, "a wait inside the decode kernel timed out"
    return ids.cpu().numpy(), w.cpu().numpy(), y.cpu().numpy()


# ---------------------------------------------------------------- exact ties
TIE_CASES = {
    # experts 4 and 11 share a router row and a bias far above every other
    # expert: they are picks 0 and 1, with 4 first and bitwise-equal weights
    "top": ({4: 12.0, 11: 12.0}, [4, 11]),
    # five experts far ahead (8 apart: the unnormalised logits spread with a
    # std of about 0.72), then 4 and 11 tied for the 6th place: 4 is picked,
    # 11 is the 7th and left out
    "boundary": ({0: 52.0, 1: 44.0, 2: 36.0, 3: 28.0, 5: 20.0, 4: 12.0, 11: 12.0}, [0, 1, 2, 3, 5, 4]),
}


def tie_layer(case):
    from quantized_expert_ffn_moe_amd import binding as B
    bias, _ = TIE_CASES[case]
    lay = dict(base_layer(0))
    rw = np.array(lay["router_w"], dtype=np.float32)
    rw[4] = rw[11]
    b = np.zeros(64, np.float32)
    for e, v in bias.items():
        b[e] = v
    lay["router_w"], lay["router_b"] = rw, b
    return lay, B.pack_layer(lay)


def assert_tie(ids, w, case):
    _, want = TIE_CASES[case]
    assert np.all(ids[:, :len(want)] == np.asarray(want)[None, :]), ids[:4]
    if case == "top":
        np.testing.assert_array_equal(w[:, 0], w[:, 1])


@pytest.mark.parametrize("case", sorted(TIE_CASES))
@pytest.mark.parametrize("T,path", [(1, "decode"), (40, "decode"), (1, "grouped"), (40, "grouped"),
                                    (700, "grouped"), (1100, "grouped")])
def test_exact_router_tie_goes_to_lower_index(lib, case, T, path):
    from quantized_expert_ffn_moe_amd import binding as B
    lay, packed = tie_layer(case)
    x, xt = tokens(0, T, batch=3)
    flags = B.MOE_FORCE_DECODE if path == "decode" else B.MOE_FORCE_GROUPED
    say(f"tie {case}, {T} tokens, {path} path")
    ids, w, y = run(xt, packed, flags)
    assert_tie(ids, w, case)
    ratio, _ = check_layer(x, lay, ids, w, y)
    say(f"  err/rms {ratio:.2e}")


@pytest.mark.parametrize("case", sorted(TIE_CASES))
def test_exact_router_tie_decode_step(lib, case):
    from quantized_expert_ffn_moe_amd import binding as B
    lay, packed = tie_layer(case)
    x, xt = tokens(0, 1, batch=4)
    say(f"tie {case}, decode step (3 layers, the tie in each)")
    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE
    ids, w, y = decode_step(xt, [packed] * 3, flags)
    assert_tie(ids, w, case)
    # layer 1 against the oracle
    h = x.astype(np.float64)
    ids1, w1, y1 = decode_step(xt, [packed], flags)
    ratio, _ = check_layer(O.rmsnorm(h, NORM_EPS), lay, ids1, w1, y1 - h)
    say(f"  layer 1 err/rms {ratio:.2e}")


# ---------------------------------------------------------------- int8 code -128
def minus128_layer():
    """Workload 0's int8 G128 layer with code -128 planted: every row of every
    matrix gets -128 in its first column and every 7th code becomes -128."""
    from quantized_expert_ffn_moe_amd import binding as B
    lay = dict(base_layer(0))
    for k in ("gate_q", "up_q", "down_q", "shared_gate_q", "shared_up_q", "shared_down_q"):
        q = np.array(lay[k], dtype=np.int8)
        q[..., 0] = -128
        flat = q.reshape(-1)
        flat[::7] = -128
        lay[k] = q
    assert (lay["gate_q"] == -128).any()
    return lay, B.pack_layer(lay)


@pytest.mark.parametrize("T,path", [(1, "decode"), (13, "decode"), (40, "grouped"), (700, "grouped")])
def test_int8_code_minus128(lib, T, path):
    from quantized_expert_ffn_moe_amd import binding as B
    lay, packed = minus128_layer()
    x, xt = tokens(0, T, batch=6)
    flags = B.MOE_FORCE_DECODE if path == "decode" else B.MOE_FORCE_GROUPED
    say(f"int8 -128 codes, {T} tokens, {path} path")
    ids, w, y = run(xt, packed, flags)
    ratio, _ = check_layer(x, lay, ids, w, y)
    say(f"  err/rms {ratio:.2e}")


def test_int8_code_minus128_decode_step(lib):
    lay, packed = minus128_layer()
    x, xt = tokens(0, 1, batch=7)
    say("int8 -128 codes, decode step")
    ids, w, y = decode_step(xt, [packed], 0)
    ratio, _ = check_layer(x, lay, ids, w, y)
    say(f"  err/rms {ratio:.2e}")


# ---------------------------------------------------------------- the largest call
def test_max_tokens_grouped_sampled(lib):
    """8192 tokens (the header's maximum) through one layer of the multi-page
    workload's format (int4 G64, Zipf router bias, bf16 tokens), RMSNorm and
    the residual inside the call, checked on sampled tokens: the largest
    histogram, tile list and workspace carve."""
    from quantized_expert_ffn_moe_amd import binding as B
    T = 8192
    wl = WORKLOADS[4]
    lay = base_layer(4, 0)
    packed = B.pack_layer(lay)
    x, xt = tokens(4, T, batch=9)
    h = xt.float().contiguous()
    h0 = h.clone()
    ids = torch.empty(T, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(T, 6, dtype=torch.float32, device="cuda")
    ws = B.workspace(T)
    say(f"{T} tokens, grouped path, workspace {ws.numel() / 2 ** 20:.0f} MiB")
    B.moe_layer_forward(h, packed, h, ids, w, ws, B.MOE_NORM_INPUT | B.MOE_ACCUMULATE | B.MOE_NORM_BF16)
    torch.cuda.synchronize()
    idn = ids.cpu().numpy()
    assert idn.min() >= 0 and idn.max() < 64
    counts = np.bincount(idn.reshape(-1), minlength=64)
    say(f"  experts touched {int((counts > 0).sum())}, largest count {int(counts.max())}")
    sample = np.sort(np.random.default_rng(8192).choice(T, 32, replace=False))
    sample = np.unique(np.concatenate([[0, T - 1], sample]))
    z = torch.empty(len(sample), 1280, dtype=torch.bfloat16, device="cuda")
    B.moe_rmsnorm(h0[sample].contiguous(), z, NORM_EPS)
    zin = z.float().cpu().numpy().astype(np.float64)
    out = (h[sample] - h0[sample]).cpu().numpy()
    ratio, near = check_layer(zin, lay, idn[sample], w.cpu().numpy()[sample], out)
    say(f"  sampled {len(sample)} tokens: err/rms {ratio:.2e} near-ties {near}")
    assert wl.norm_bf16


# ---------------------------------------------------------------- non-finite rows
@pytest.mark.parametrize("T,path", [(5, "decode"), (5, "grouped"), (300, "grouped"), (1100, "grouped")])
def test_non_finite_rows_keep_valid_ids(lib, T, path):
    from quantized_expert_ffn_moe_amd import binding as B
    wi = 0
    x, xt = tokens(wi, T, batch=12)
    bad = {1: float("nan"), 3: float("inf")}
    for t, v in bad.items():
        xt[t, 17] = v
    flags = B.MOE_FORCE_DECODE if path == "decode" else B.MOE_FORCE_GROUPED
    say(f"non-finite rows {sorted(bad)} of {T}, {path} path")
    ids, w, y = run(xt, base_packed(wi), flags | B.MOE_NORM_INPUT)
    for t in range(T):
        assert ids[t].min() >= 0 and ids[t].max() < 64 and len(set(ids[t].tolist())) == 6, (t, ids[t])
    good = np.array([t for t in range(T) if t not in bad])
    z = O.rmsnorm(x[good], NORM_EPS)
    ratio, _ = check_layer(z, base_layer(wi), ids[good], w[good], y[good])
    say(f"  finite tokens err/rms {ratio:.2e}")


def test_non_finite_decode_step_keeps_valid_ids(lib):
    from quantized_expert_ffn_moe_amd import binding as B
    x, xt = tokens(0, 1, batch=13)
    xt[0, 5] = float("nan")
    say("non-finite row, decode step (2 layers)")
    ws = B.decode_workspace()
    ids, w, y = decode_step(xt, [base_packed(0)] * 2, B.MOE_NORM_INPUT | B.MOE_ACCUMULATE, ws)
    for l in range(2):
        assert ids[l].min() >= 0 and ids[l].max() < 64 and len(set(ids[l].tolist())) == 6, ids[l]
    # the workspace stays usable: a finite token right after matches the oracle
    x2, xt2 = tokens(0, 1, batch=14)
    ids2, w2, y2 = decode_step(xt2, [base_packed(0)], 0, ws)
    ratio, _ = check_layer(x2, base_layer(0), ids2, w2, y2)
    say(f"  next finite token err/rms {ratio:.2e}")


@functools.lru_cache(maxsize=None)
def base_packed(wi: int):
    from quantized_expert_ffn_moe_amd import binding as B
    return B.pack_layer(base_layer(wi))
