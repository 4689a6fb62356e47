"""Comparison protocol between the GPU library and the float64 oracle.

* Routing: the GPU ids must be a valid greedy top-k of the oracle's
  probabilities.  Where the oracle's 6th/7th gap (and the gap between two
  adjacent picks) exceeds 1e-6 the ids are unique, so they must match exactly;
  inside a near-tie either answer is correct.
* Weights: |w_gpu - P_oracle[id]| <= 1e-5 * P_oracle[id] (fp32 softmax).
* Output: the oracle is re-run with the GPU's ids (forced) and
  max |y_gpu - y_oracle| <= 1e-3 * rms(y_oracle) over the call's output.
"""
import numpy as np

from oracle import moe_oracle as O

GAP = 1e-6
W_RTOL = 1e-5
Y_TOL = 1e-3


def check_routing(ids, w, P, k=6):
    ids = np.asarray(ids); w = np.asarray(w, np.float64); P = np.asarray(P, np.float64)
    T, E = P.shape
    exact_mismatch = 0
    near_ties = 0
    for t in range(T):
        p = P[t]
        pick = ids[t].astype(np.int64)
        assert len(set(pick.tolist())) == k and pick.min() >= 0 and pick.max() < E, (t, pick)
        pp = p[pick]
        assert np.all(pp[:-1] >= pp[1:] - GAP), (t, pick, pp)
        rest = np.ones(E, bool); rest[pick] = False
        assert p[rest].max() <= pp.min() + GAP, (t, pick)
        order = sorted(range(E), key=lambda e: (-p[e], e))
        ps = p[order]
        if ps[k - 1] - ps[k] > GAP and np.all(ps[:k - 1] - ps[1:k] > GAP):
            if pick.tolist() != order[:k]:
                exact_mismatch += 1
        else:
            near_ties += 1
        err = np.abs(w[t] - pp)
        assert np.all(err <= W_RTOL * pp + 1e-12), (t, pick, w[t], pp)
    assert exact_mismatch == 0
    return near_ties


def check_output(y_gpu, y_oracle, tol=Y_TOL):
    y_gpu = np.asarray(y_gpu, np.float64); y_oracle = np.asarray(y_oracle, np.float64)
    rms = float(np.sqrt(np.mean(y_oracle ** 2)))
    err = float(np.abs(y_gpu - y_oracle).max())
    assert err <= tol * rms, f"max|err| {err:.3e} > {tol} * rms {rms:.3e} (ratio {err / rms:.3e})"
    return err / rms


def check_layer(x_in, layer, ids, w, y, k=6):
    """x_in: the layer input the GPU used (f64 values).  Returns (err/rms, near_ties)."""
    x_in = np.atleast_2d(np.asarray(x_in, np.float64))
    P = O.softmax(O.router_logits(x_in, layer["router_w"], layer.get("router_b")))
    near = check_routing(ids, w, P, k)
    _, _, y_o, _ = O.moe_layer(x_in, layer, top_k=k, forced_ids=np.asarray(ids))
    return check_output(y, y_o), near
