"""The host quantisers (CPU): their outputs dequantise (by the oracle) to
within each format's step of the float weights, pack through the C ABI, and
the group-size trade of the demo page's "Four bits, one shared scale"
section shows on heavy-tailed weights: smaller groups cost more metadata and
follow the weights more closely."""
import numpy as np
import pytest

from oracle import moe_oracle as O
from quantized_expert_ffn_moe_amd import quantize as Qz


def heavy_tailed(rows, K, seed):
    """Student-t (3 degrees of freedom) weights with a per-row spread: a stand-in
    for trained weights with outliers."""
    rng = np.random.default_rng(seed)
    return rng.standard_t(3, size=(rows, K)) * rng.uniform(0.005, 0.02, size=(rows, 1))


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 64), (4, 128), (8, 128)])
def test_symmetric_round_trip_within_half_a_step(bits, group):
    W = heavy_tailed(64, 1280, bits * group)
    codes, s = Qz.quantize_symmetric(W, bits, group)
    R = O.dequantize(codes, s, group)
    step = np.repeat(s.astype(np.float64), group, axis=1)
    assert np.all(np.abs(R - W) <= 0.5 * step * (1 + 1e-6) + 1e-12)
    # the largest weight of every group is hit exactly (up to the f32 scale)
    blocks = np.abs(W).reshape(64, -1, group).max(axis=2)
    np.testing.assert_allclose(np.abs(R).reshape(64, -1, group).max(axis=2), blocks, rtol=1e-6)


@pytest.mark.parametrize("K", [896, 1280, 1792])
def test_two_level_round_trip(K):
    W = heavy_tailed(48, K, K)
    f = Qz.quantize_two_level(W)
    assert f["q"].max() <= 15 and f["sc"].max() <= 63 and f["m"].max() <= 63
    R = O.dequantize_q4k(f["q"], f["d"], f["dmin"], f["sc"], f["m"])
    # each sub-block: at most half a quantised step, plus the rounding of the
    # minimum (half a dmin) and of the step (q <= 15 times half a d)
    d = np.repeat(O.f16_value(f["d"]), 256, axis=1)[:, :K]
    dmin = np.repeat(O.f16_value(f["dmin"]), 256, axis=1)[:, :K]
    step = d * np.repeat(f["sc"].astype(np.float64), 32, axis=1)
    bound = 0.5 * step + 0.5 * dmin + 7.5 * d + 1e-12
    assert np.all(np.abs(R - W) <= bound)
    rel = np.sqrt(np.mean((R - W) ** 2) / np.mean(W ** 2))
    assert rel < 0.2


def test_group_size_trade():
    """Relative RMS reconstruction error rises with the group size while the
    metadata falls; the two-level format sits at G = 64's byte cost."""
    W = heavy_tailed(128, 1280, 7)
    err, bpw = {}, {}
    for g in (32, 64, 128):
        c, s = Qz.quantize_symmetric(W, 4, g)
        R = O.dequantize(c, s, g)
        err[g] = np.sqrt(np.mean((R - W) ** 2) / np.mean(W ** 2))
        bpw[g] = Qz.bits_per_weight(g, 4, 1280)
    f = Qz.quantize_two_level(W)
    R = O.dequantize_q4k(f["q"], f["d"], f["dmin"], f["sc"], f["m"])
    err["q4k"] = np.sqrt(np.mean((R - W) ** 2) / np.mean(W ** 2))
    bpw["q4k"] = Qz.bits_per_weight(256, 4, 1280)
    assert err[32] < err[64] < err[128]
    assert bpw[32] > bpw[64] > bpw[128]
    assert bpw["q4k"] == bpw[64] == 4.5
    print({k: (round(float(v), 4), bpw[k]) for k, v in err.items()})


def test_quantised_weights_pack(lib):
    from quantized_expert_ffn_moe_amd import binding as B
    g, u = heavy_tailed(896, 1280, 2), heavy_tailed(896, 1280, 3)
    dn = heavy_tailed(1280, 896, 4)
    codes, meta = B.moe_pack_expert_q4k(Qz.quantize_two_level(g), Qz.quantize_two_level(u),
                                        Qz.quantize_two_level(dn))
    assert codes.size == B.moe_expert_code_bytes(4, 896) and meta.size == B.moe_expert_scale_count(256, 896)
    qs = [Qz.quantize_symmetric(m, 4, 64) for m in (g, u, dn)]
    c2, s2 = B.moe_pack_expert(qs[0][0], qs[1][0], qs[2][0], qs[0][1], qs[1][1], qs[2][1], 4, 64)
    assert c2.size == codes.size
