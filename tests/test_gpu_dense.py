"""GPU dense ends (lm_head + greedy token, dense layer-0 SwiGLU MLP) vs the
float64 oracle, through the C ABI (needs an MI355X)."""
import functools
import sys

import numpy as np
import pytest

from oracle import dense_head as D
from synth import NORM_EPS, QFmt, make_dense_ffn, make_hidden, make_lm_head
from tests.conftest import gpu_available
from tests.parity import check_routing

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

torch = pytest.importorskip("torch")


def say(*a):
    print("[dense]", *a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=None)
def head_of(dtype, vocab=129280):
    return make_lm_head(dtype, vocab=vocab)


@functools.lru_cache(maxsize=None)
def head_weights_f64(dtype, vocab=129280):
    h = head_of(dtype, vocab)
    if dtype == "bf16":
        return D.bf16_bits_value(h["w"])
    return D.dequantize(h["q"], h["s"], h["group"])


def run_head(head, hx, flags, with_logits=True):
    from quantized_expert_ffn_moe_amd import binding as B
    T = hx.shape[0]
    dev = B.lm_head_to_device(head)
    h = torch.from_numpy(hx).cuda()
    tok = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    tl = torch.empty(T, dtype=torch.float32, device="cuda")
    logits = torch.empty(T, head["vocab"], dtype=torch.float32, device="cuda") if with_logits else None
    ws = torch.empty(B.moe_lm_head_workspace_bytes(T, head["vocab"]), dtype=torch.uint8, device="cuda")
    B.moe_lm_head_argmax(h, dev, tok, tl, ws, flags, logits)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), tl.cpu().numpy(), (logits.cpu().numpy() if with_logits else None)


def check_head(ref_logits, tok, tl, logits):
    """Logits within 1e-3 x rms of the oracle's; the token equal to the oracle's
    wherever its best logit leads the runner-up by more than that tolerance,
    else (a near tie) a token whose oracle logit is within it of the best."""
    tol = 1e-3 * np.sqrt(np.mean(ref_logits ** 2))
    if logits is not None:
        err = np.abs(logits - ref_logits).max()
        assert err <= tol, (err, tol)
    rid, rv = D.greedy_token(ref_logits)
    for t in range(ref_logits.shape[0]):
        second = np.partition(ref_logits[t], -2)[-2] if ref_logits.shape[1] > 1 else -np.inf
        if rv[t] - second > tol:
            assert tok[t] == rid[t], (t, tok[t], rid[t])
        else:
            assert ref_logits[t, tok[t]] >= rv[t] - tol
        assert abs(tl[t] - ref_logits[t, tok[t]]) <= tol
    return tol


@pytest.mark.parametrize("dtype,T", [("bf16", 1), ("bf16", 4), ("int8", 1), ("int8", 3)])
def test_lm_head_full_vocab(lib, dtype, T):
    from quantized_expert_ffn_moe_amd import binding as B
    say(f"lm_head {dtype} vocab 129280, {T} tokens, final norm")
    hx = make_hidden(T, batch=T)
    tok, tl, logits = run_head(head_of(dtype), hx, B.MOE_NORM_INPUT)
    ref = D.lm_head_logits(hx, head_weights_f64(dtype), True, NORM_EPS)
    tol = check_head(ref, tok, tl, logits)
    say(f"  tokens {tok.tolist()} max|err| {np.abs(logits - ref).max():.2e} (tol {tol:.2e})")


@pytest.mark.parametrize("vocab", [1, 129, 1000])
def test_lm_head_ragged_vocab_no_norm(lib, vocab):
    say(f"lm_head bf16 vocab {vocab}, no norm, 2 tokens")
    hx = make_hidden(2, batch=7)
    head = head_of("bf16", vocab)
    tok, tl, logits = run_head(head, hx, 0)
    ref = D.lm_head_logits(hx, head_weights_f64("bf16", vocab), False, 0.0)
    check_head(ref, tok, tl, logits)
    # without the logits buffer the token is the same
    tok2, tl2, _ = run_head(head, hx, 0, with_logits=False)
    assert np.array_equal(tok, tok2) and np.array_equal(tl, tl2)


def test_lm_head_tie_goes_to_lowest_id(lib):
    """Two identical best rows (ids 5 and 1033, different workgroups and lanes
    of the same piece layout) and a third copy at id 1034: the lowest id wins."""
    from quantized_expert_ffn_moe_amd import binding as B
    vocab = 4000
    base = head_of("bf16", vocab)
    w = base["w"].copy()
    w[[5, 1033, 1034]] = 0x3F80                    # rows of 1.0: logit = sum of z
    hx = np.abs(make_hidden(1, batch=9)) + 0.5     # positive: those rows win
    head = {"dtype": "bf16", "w": w, "vocab": vocab}
    tok, tl, logits = run_head(head, hx, B.MOE_NORM_INPUT)
    assert tok[0] == 5
    assert logits[0, 5] == logits[0, 1033] == logits[0, 1034] == tl[0]


def test_lm_head_deterministic(lib):
    from quantized_expert_ffn_moe_amd import binding as B
    hx = make_hidden(3, batch=11)
    a = run_head(head_of("int8"), hx, B.MOE_NORM_INPUT)
    b = run_head(head_of("int8"), hx, B.MOE_NORM_INPUT)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def run_dense(ffn, x, flags, y0=None):
    from quantized_expert_ffn_moe_amd import binding as B
    T = x.shape[0]
    dev = B.dense_ffn_to_device(ffn)
    xt = torch.from_numpy(x).cuda()
    if y0 is None:
        y = torch.full((T, 1280), float("nan"), dtype=torch.float32, device="cuda")
    else:
        y = torch.from_numpy(y0).cuda()
    ws = torch.empty(B.moe_dense_ffn_workspace_bytes(T, ffn["inter"]), dtype=torch.uint8, device="cuda")
    B.moe_dense_ffn_forward(xt, dev, y, ws, flags)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check_ffn(got, ref):
    tol = 1e-3 * np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref).max()
    assert err <= tol, (err, tol)
    return err / np.sqrt(np.mean(ref ** 2))


@functools.lru_cache(maxsize=None)
def dense_of(bits, group, inter=6848):
    return make_dense_ffn(QFmt(bits, group), inter)


@pytest.mark.parametrize("bits,group,T", [(8, 64, 1), (8, 64, 4), (4, 32, 2), (8, 32, 3)])
def test_dense_ffn_full_size(lib, bits, group, T):
    from quantized_expert_ffn_moe_amd import binding as B
    say(f"dense MLP int{bits} G{group} inter 6848, {T} tokens, norm")
    ffn = dense_of(bits, group)
    x = make_hidden(T, batch=20 + T)
    y = run_dense(ffn, x, B.MOE_NORM_INPUT)
    r = check_ffn(y, D.dense_ffn(x, ffn, True, NORM_EPS))
    say(f"  err/rms {r:.2e}")


def test_dense_ffn_in_place_residual(lib):
    """x and y the same buffer with MOE_ACCUMULATE: y = x + MLP(RMSNorm(x))."""
    from quantized_expert_ffn_moe_amd import binding as B
    ffn = dense_of(8, 64)
    x = make_hidden(2, batch=31)
    dev = B.dense_ffn_to_device(ffn)
    h = torch.from_numpy(x).cuda()
    ws = torch.empty(B.moe_dense_ffn_workspace_bytes(2, 6848), dtype=torch.uint8, device="cuda")
    B.moe_dense_ffn_forward(h, dev, h, ws, B.MOE_NORM_INPUT | B.MOE_ACCUMULATE)
    torch.cuda.synchronize()
    out = h.cpu().numpy().astype(np.float64) - x
    check_ffn(out, D.dense_ffn(x, ffn, True, NORM_EPS))


@pytest.mark.parametrize("bits,group,inter", [(8, 64, 64), (4, 128, 1792), (8, 128, 8192)])
def test_dense_ffn_other_intermediates(lib, bits, group, inter):
    say(f"dense MLP int{bits} G{group} inter {inter}, 1 token, no norm")
    ffn = dense_of(bits, group, inter)
    x = make_hidden(1, batch=40)
    check_ffn(run_dense(ffn, x, 0), D.dense_ffn(x, ffn, False, 0.0))


def test_decoder_ffn_stack_one_token(lib):
    """One decode token through the decoder's FFN stack and head, all on the GPU
    through the C ABI: layer-0 dense MLP (residual), the 11 chained MoE layers
    (one persistent launch), final norm + lm_head + greedy token.  Checked
    layer by layer against the oracle, teacher-forced with the GPU's own
    residual stream, and the token against the oracle's greedy pick."""
    from oracle import moe_oracle as MO
    from quantized_expert_ffn_moe_amd import binding as B
    from synth import WORKLOADS, make_layer
    say("decoder FFN stack: dense MLP + 11 MoE layers + lm_head, 1 token")
    wl = WORKLOADS[1]
    layers = [make_layer(wl, li) for li in range(wl.n_layers)]
    packed = [B.pack_layer(layer) for layer in layers]
    ffn = dense_of(8, 64)
    head = head_of("bf16")
    x = make_hidden(1, batch=77)
    h = torch.from_numpy(x).cuda()
    # layer 0: dense MLP with its input norm, added to the residual in place
    ws_d = torch.empty(B.moe_dense_ffn_workspace_bytes(1, 6848), dtype=torch.uint8, device="cuda")
    B.moe_dense_ffn_forward(h, B.dense_ffn_to_device(ffn), h, ws_d, B.MOE_NORM_INPUT | B.MOE_ACCUMULATE)
    h1 = h.clone()
    # layers 1-11: the persistent decode step
    ids = torch.empty(wl.n_layers, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(wl.n_layers, 6, dtype=torch.float32, device="cuda")
    ws = B.decode_workspace()
    y = torch.empty(1, 1280, dtype=torch.float32, device="cuda")
    B.moe_decode_forward(h1, y, packed, ids, w, ws, B.MOE_NORM_INPUT | B.MOE_ACCUMULATE)
    # head
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    tl = torch.empty(1, dtype=torch.float32, device="cuda")
    logits = torch.empty(1, head["vocab"], dtype=torch.float32, device="cuda")
    ws_h = torch.empty(B.moe_lm_head_workspace_bytes(1, head["vocab"]), dtype=torch.uint8, device="cuda")
    B.moe_lm_head_argmax(y, B.lm_head_to_device(head), tok, tl, ws_h, B.MOE_NORM_INPUT, logits)
    torch.cuda.synchronize()
    # dense layer
    h1n = h1.cpu().numpy().astype(np.float64)
    check_ffn(h1n - x, D.dense_ffn(x, ffn, True, NORM_EPS))
    # MoE layers: the whole chain from the GPU's layer-0 output, prefix by prefix
    h_prev = h1n
    ids_n, w_n = ids.cpu().numpy(), w.cpu().numpy()
    yn = y.cpu().numpy().astype(np.float64)
    _, free = MO.moe_chain(h1n, layers, NORM_EPS, False)
    same = all(np.array_equal(free[li][0][0], ids_n[li]) for li in range(wl.n_layers))
    # the chain is checked whatever the routing: the oracle takes the GPU's ids
    # (a near-tie admits both answers), and each layer's ids and weights must be
    # a valid greedy pick of the oracle's own probabilities at that layer
    out_o, trace = MO.moe_chain(h1n, layers, NORM_EPS, False,
                                forced_ids=[ids_n[li][None] for li in range(wl.n_layers)])
    for li in range(wl.n_layers):
        P = MO.softmax(MO.router_logits(trace[li][2], layers[li]["router_w"], layers[li].get("router_b")))
        check_routing(ids_n[li][None], w_n[li][None], P)
    check_ffn(yn - h1n, out_o - h1n)
    # head on the GPU's final residual
    ref = D.lm_head_logits(yn, head_weights_f64("bf16"), True, NORM_EPS)
    check_head(ref, tok.cpu().numpy(), tl.cpu().numpy(), logits.cpu().numpy())
    say(f"  token {int(tok.item())}, routing identical to the oracle's at every layer: {same}")
