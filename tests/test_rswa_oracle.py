"""Pins for the R-SWA decode oracle: ring-buffer bookkeeping against brute
force over the whole generated history, softmax closed forms, and the
library's scaled-dot-product attention on the reduced case."""
import math

import numpy as np
import torch

from oracle import rswa as R
from oracle.moe_oracle import bf16_round


def _rng(seed):
    return np.random.default_rng(seed)


def test_single_key_returns_its_value():
    v = np.array([[1.5, -2.0, 0.25, 4.0]])
    out = R.attend(np.array([0.3, 0.1, -0.2, 0.9]), np.array([[1.0, 2.0, 3.0, 4.0]]), v)
    assert out.tolist() == v[0].tolist()


def test_equal_scores_average_the_values():
    keys = np.ones((5, 4))
    vals = np.arange(20, dtype=np.float64).reshape(5, 4)
    np.testing.assert_allclose(R.attend(np.array([1.0, -1.0, 2.0, 0.5]), keys, vals), vals.mean(axis=0), rtol=1e-15)


def test_two_keys_closed_form():
    q = np.array([1.0, 0.0, 0.0, 0.0])
    keys = np.array([[2.0, 0, 0, 0], [0.0, 0, 0, 0]])   # scores 2 / sqrt(4) = 1 and 0
    vals = np.array([[1.0, 0, 0, 0], [0.0, 1, 0, 0]])
    e = math.e
    np.testing.assert_allclose(R.attend(q, keys, vals), [e / (e + 1), 1 / (e + 1), 0, 0], rtol=1e-15)


def test_matches_library_attention_on_one_head():
    rng = _rng(1)
    q = rng.standard_normal(128)
    k = rng.standard_normal((37, 128))
    v = rng.standard_normal((37, 128))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(k)[None, None], torch.from_numpy(v)[None, None])
    np.testing.assert_allclose(R.attend(q, k, v), ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-13)


def _history_case(n_gen, heads=3, d=8, n_ref=5, seed=0):
    """Generate n_gen + 1 tokens one by one through the ring, and the same
    attention computed by brute force from the full history."""
    rng = _rng(seed)
    ref_k = bf16_round(rng.standard_normal((heads, n_ref, d)))
    ref_v = bf16_round(rng.standard_normal((heads, n_ref, d)))
    ring_k = np.zeros((heads, R.WINDOW, d))
    ring_v = np.zeros((heads, R.WINDOW, d))
    hist_k, hist_v = [], []
    for g in range(n_gen + 1):
        q = rng.standard_normal((heads, d))
        kn = rng.standard_normal((heads, d))
        vn = rng.standard_normal((heads, d))
        out, ring_k, ring_v = R.rswa_decode(q, kn, vn, ref_k, ref_v, ring_k, ring_v, g)
        hist_k.append(bf16_round(kn))
        hist_v.append(bf16_round(vn))
    # brute force: reference block + the newest min(n_gen + 1, 128) generated tokens
    last_k = np.stack(hist_k[-R.WINDOW:], axis=1)
    last_v = np.stack(hist_v[-R.WINDOW:], axis=1)
    brute = np.stack([R.attend(q[h], np.concatenate([ref_k[h], last_k[h]]), np.concatenate([ref_v[h], last_v[h]]))
                      for h in range(heads)])
    return out, brute


def test_ring_before_the_window_fills():
    out, brute = _history_case(n_gen=40)
    np.testing.assert_allclose(out, brute, rtol=1e-13, atol=1e-14)


def test_ring_after_it_wraps():
    # 300 generated tokens: slots have been overwritten twice; only the newest 128 count
    out, brute = _history_case(n_gen=300, seed=2)
    np.testing.assert_allclose(out, brute, rtol=1e-13, atol=1e-14)


def test_ring_exactly_full():
    out, brute = _history_case(n_gen=127, seed=3)
    np.testing.assert_allclose(out, brute, rtol=1e-13, atol=1e-14)


def test_write_rounds_to_bf16_in_the_right_slot():
    rk = np.zeros((2, R.WINDOW, 4))
    rv = np.zeros((2, R.WINDOW, 4))
    kn = np.full((2, 4), 1.0 + 2 ** -9)          # halfway between two bf16 values: ties to even -> 1.0
    vn = np.full((2, 4), 1.0 + 3 * 2 ** -9)      # rounds up to 1 + 2^-7
    k2, v2 = R.ring_write(rk, rv, kn, vn, n_gen=130)
    assert np.all(k2[:, 2] == 1.0) and np.all(v2[:, 2] == 1.0 + 2 ** -7)
    assert np.count_nonzero(k2) == 8 and np.count_nonzero(v2) == 8
    assert np.all(rk == 0)                        # the input ring is not modified
