"""The benchmark's same-run parity gate, on the CPU: fed the oracle's own
outputs it passes, and each planted mistake in the "GPU" outputs (an output
error above the 1e-3 x rms bar, a swapped pick, a wrong weight, a wrong greedy
token) makes it raise.  Tiny layers keep it fast; the gate is the code every
bench leg runs before it prints."""
import numpy as np
import pytest

import bench
from oracle import dense_head as D
from oracle import moe_oracle as O
from synth import NORM_EPS, QFmt, make_tiny_layer

E, H, I, IS = 16, 64, 64, 128


def layers(n):
    return [make_tiny_layer(100 + l, E, H, I, IS, QFmt(4, 32)) for l in range(n)]


def tokens(T, seed=5):
    return np.random.default_rng(seed).standard_normal((T, H))


def run_gate(lays, x, ids, w, out, chained):
    return bench.moe_oracle_leg(lays, x, np.arange(x.shape[0]), ids, w, out, chained=chained, norm_bf16=False,
                                block=4, what="tiny", budget_s=1e9)


def oracle_outputs(lays, x, chained):
    if chained:
        h, trace = O.moe_chain(x, lays, NORM_EPS, False)
        return h, [t[0] for t in trace], [t[1] for t in trace]
    ids, w, y, _ = O.moe_layer(x, lays[0])
    return y, [ids], [w]


@pytest.mark.parametrize("chained", [False, True])
def test_gate_passes_the_oracle_itself(chained):
    lays = layers(3 if chained else 1)
    x = tokens(12)
    out, ids, w = oracle_outputs(lays, x, chained)
    base, gate = run_gate(lays, x, ids, w, out, chained)
    assert gate["tokens"] == 12 and gate["max_err_over_rms"] < 1e-12
    assert base["kind"] == "oracle" and base["value"] > 0


@pytest.mark.parametrize("chained", [False, True])
def test_gate_rejects_an_output_error_above_the_bar(chained):
    lays = layers(3 if chained else 1)
    x = tokens(12)
    out, ids, w = oracle_outputs(lays, x, chained)
    ref = out - (x if chained else 0.0)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    ok = out.copy()
    ok[3, 7] += 0.5e-3 * rms                  # inside the bar: passes
    run_gate(lays, x, ids, w, ok, chained)
    bad = out.copy()
    bad[3, 7] += 2e-3 * rms                   # above it: rejected
    with pytest.raises(bench.GateError, match="max\\|err\\|"):
        run_gate(lays, x, ids, w, bad, chained)


def test_gate_rejects_a_wrong_pick_and_a_wrong_weight():
    lays = layers(1)
    x = tokens(12)
    out, ids, w = oracle_outputs(lays, x, False)
    P = O.softmax(O.router_logits(x, lays[0]["router_w"], lays[0].get("router_b")))
    # a token whose 6th and 7th probabilities are well apart: swapping in the
    # 7th expert is a routing mistake, not a near-tie
    order = np.argsort(-P, axis=1, kind="stable")
    gaps = P[np.arange(12), order[:, 5]] - P[np.arange(12), order[:, 6]]
    t = int(np.argmax(gaps))
    assert gaps[t] > 1e-6
    bad_ids = [ids[0].copy()]
    bad_ids[0][t, 5] = order[t, 6]
    with pytest.raises(bench.GateError, match="routing"):
        run_gate(lays, x, bad_ids, w, out, False)
    bad_w = [w[0].copy()]
    bad_w[0][t, 0] *= 1 + 1e-4                # beyond the 1e-5 relative bar
    with pytest.raises(bench.GateError, match="routing"):
        run_gate(lays, x, ids, bad_w, out, False)


def test_head_gate_rejects_a_wrong_token():
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((2, 1000))
    tok, val = D.greedy_token(logits)
    bench.head_gate(logits, np.asarray(tok), np.asarray(val))
    wrong = np.asarray(tok).copy()
    wrong[1] = int(np.argsort(logits[1])[-2])  # the runner-up, well below the best
    assert logits[1, tok[1]] - logits[1, wrong[1]] > 1e-3 * np.sqrt(np.mean(logits ** 2))
    with pytest.raises(bench.GateError):
        bench.head_gate(logits, wrong, logits[np.arange(2), wrong])
    with pytest.raises(bench.GateError):
        bench.head_gate(logits, np.asarray(tok), np.asarray(val) + 1.0)
