"""Host-side checks of the C ABI: exports, packing layout, argument validation.
Nothing here launches a kernel, so it runs without a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

from quantized_expert_ffn_moe_amd import binding as B
from synth import QFmt, make_tiny_layer

INCLUDE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")


def test_every_declared_symbol_is_exported(lib):
    text = "".join(open(os.path.join(INCLUDE, f)).read() for f in sorted(os.listdir(INCLUDE)) if f.endswith(".h"))
    names = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(moe_[a-z_0-9]+)\s*\(", text, re.M))
    assert names == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n) and getattr(lib, n) is not None


def test_status_strings(lib):
    for s in range(8):
        assert lib.moe_status_str(s)
    assert b"unknown" in lib.moe_status_str(99)


def _s4(v):
    return v - 16 if v >= 8 else v


def _s8(v):
    return v - 256 if v >= 128 else v


def _unpack_rows(buf, N, K, bits):
    """Decode the gate/up tile layout described in include/moe.h (independent of the packer)."""
    KB = 128 if bits == 4 else 64
    out = np.zeros((N, K), np.int64)
    words = np.frombuffer(buf, dtype="<u4")
    for nt in range(N // 16):
        for kb in range(K // KB):
            base = (nt * (K // KB) + kb) * 256
            for lane in range(64):
                row, q = nt * 16 + lane % 16, lane // 16
                for j in range(4):
                    w = int(words[base + lane * 4 + j])
                    if bits == 4:
                        for i in range(8):
                            out[row, kb * KB + 32 * j + 8 * q + i] = _s4((w >> (4 * i)) & 15)
                    else:
                        for i in range(4):
                            out[row, kb * KB + 32 * (j // 2) + 8 * q + 4 * (j % 2) + i] = _s8((w >> (8 * i)) & 255)
    return out


def _unpack_slabs(buf, K, bits, n_kc):
    """Decode the first n_kc 32-column slabs of a down matrix ([1280][K])."""
    DR = 64 if bits == 4 else 32
    nrt = 1280 // DR
    out = np.zeros((1280, 32 * n_kc), np.int64)
    words = np.frombuffer(buf, dtype="<u4")
    for kc in range(n_kc):
        for rt in range(nrt):
            base = (kc * nrt + rt) * 256
            for lane in range(64):
                r, q = lane % 16, lane // 16
                for j in range(4):
                    w = int(words[base + lane * 4 + j])
                    if bits == 4:
                        for i in range(8):
                            out[DR * rt + 16 * j + r, 32 * kc + 8 * q + i] = _s4((w >> (4 * i)) & 15)
                    else:
                        for i in range(4):
                            out[DR * rt + 16 * (j // 2) + r, 32 * kc + 8 * q + 4 * (j % 2) + i] = \
                                _s8((w >> (8 * i)) & 255)
    return out


@pytest.mark.parametrize("bits,group", [(4, 32), (8, 128)])
def test_pack_round_trip(lib, bits, group):
    rng = np.random.default_rng(bits)
    lo, hi = QFmt(bits, group).code_range
    inter = 896
    gate = rng.integers(lo, hi, (inter, 1280), endpoint=True, dtype=np.int8)
    up = rng.integers(lo, hi, (inter, 1280), endpoint=True, dtype=np.int8)
    down = rng.integers(lo, hi, (1280, inter), endpoint=True, dtype=np.int8)
    if bits == 8:
        gate[0, :5] = [-128, -127, 0, 126, 127]
    gs = rng.uniform(0.002, 0.02, (inter, 1280 // group)).astype(np.float32)
    us = rng.uniform(0.002, 0.02, (inter, 1280 // group)).astype(np.float32)
    ds = rng.uniform(0.002, 0.02, (1280, inter // group)).astype(np.float32)
    codes, scales = B.moe_pack_expert(gate, up, down, gs, us, ds, bits, group)
    mb = inter * 1280 * bits // 8
    assert codes.size == 3 * mb
    # decode only the first tiles of each matrix to keep the pure-Python decoder fast
    np.testing.assert_array_equal(_unpack_rows(codes[:mb][: 16 * 1280 * bits // 8 * 2], 32, 1280, bits), gate[:32])
    np.testing.assert_array_equal(_unpack_rows(codes[mb:2 * mb][: 16 * 1280 * bits // 8], 16, 1280, bits), up[:16])
    np.testing.assert_array_equal(_unpack_slabs(codes[2 * mb:], inter, bits, 2), down[:, :64])
    ng = 1280 // group
    np.testing.assert_array_equal(scales[: inter * ng].reshape(inter, ng), gs)
    np.testing.assert_array_equal(scales[inter * ng: 2 * inter * ng].reshape(inter, ng), us)
    DR = 64 if bits == 4 else 32
    sd = scales[2 * inter * ng:].reshape(inter // group, 1280 // DR, 16, DR // 16)
    # entry (g, rt, r, j) is row DR*rt + 16j + r
    np.testing.assert_array_equal(sd.transpose(1, 3, 2, 0).reshape(1280, inter // group), ds)


def test_pack_rejects_bad_codes_and_formats(lib):
    lay = make_tiny_layer(1, E=1, H=1280, I=896, Is=896, fmt=QFmt(4, 64))
    args = [lay["gate_q"][0], lay["up_q"][0], lay["down_q"][0], lay["gate_s"][0], lay["up_s"][0], lay["down_s"][0]]
    bad = args[0].copy(); bad[3, 7] = 8
    with pytest.raises(B.MoeError, match="FORMAT"):
        B.moe_pack_expert(bad, *args[1:], 4, 64)
    with pytest.raises(B.MoeError, match="FORMAT"):
        B.moe_pack_expert(*args, 4, 48)
    assert B.moe_expert_code_bytes(5, 896) == 0 and B.moe_expert_scale_count(16, 896) == 0


def _q4k_matrix(rng, N, K):
    return {"q": rng.integers(0, 16, (N, K)).astype(np.uint8),
            "d": rng.uniform(1e-4, 1e-2, (N, -(-K // 256))).astype(np.float16).view(np.uint16),
            "dmin": rng.uniform(1e-4, 1e-2, (N, -(-K // 256))).astype(np.float16).view(np.uint16),
            "sc": rng.integers(0, 64, (N, K // 32)).astype(np.uint8),
            "m": rng.integers(0, 64, (N, K // 32)).astype(np.uint8)}


def _record_fields(w):
    """(d bits, dmin bits, sc[8], m[8]) of one 16-byte record, decoded from the
    layout in include/moe.h (independent of the packer)."""
    w = [int(v) for v in w]
    byte = lambda x, k: (x >> (8 * k)) & 255
    sc = [byte(w[1 + j // 4], j % 4) & 63 for j in range(8)]
    m = [((byte(w[3], j % 4) >> (4 * (j // 4))) & 15) | ((byte(w[1 + j // 4], j % 4) >> 6) << 4) for j in range(8)]
    return w[0] & 0xFFFF, w[0] >> 16, sc, m


@pytest.mark.parametrize("inter", [896, 1792])
def test_pack_q4k_layout(lib, inter):
    rng = np.random.default_rng(inter)
    g, u, d = _q4k_matrix(rng, inter, 1280), _q4k_matrix(rng, inter, 1280), _q4k_matrix(rng, 1280, inter)
    codes, meta = B.moe_pack_expert_q4k(g, u, d)
    mb = inter * 1280 // 2
    assert codes.size == 3 * mb
    nsbd = -(-inter // 256)
    assert meta.size * 4 == 16 * 2 * inter * 5 + 4 * nsbd * 1280 + 2 * (inter // 32) * 1280 \
        == 4 * B.moe_expert_scale_count(B.MOE_Q4K, inter)
    # codes: the int4 tiles of q - 8
    np.testing.assert_array_equal(_unpack_rows(codes[:mb][: 16 * 1280], 32, 1280, 4), g["q"][:32].astype(int) - 8)
    np.testing.assert_array_equal(_unpack_rows(codes[mb:2 * mb][: 8 * 1280], 16, 1280, 4), u["q"][:16].astype(int) - 8)
    np.testing.assert_array_equal(_unpack_slabs(codes[2 * mb:], inter, 4, 2), d["q"][:, :64].astype(int) - 8)
    rec = meta.view(np.uint32)[: 2 * inter * 5 * 4].reshape(-1, 4)
    for mat, base in ((g, 0), (u, inter * 5)):
        for r in (0, 7, inter - 1):
            for b in range(5):
                db, dmb, sc, m = _record_fields(rec[base + r * 5 + b])
                assert (db, dmb) == (mat["d"][r, b], mat["dmin"][r, b])
                assert sc == mat["sc"][r, 8 * b:8 * b + 8].tolist() and m == mat["m"][r, 8 * b:8 * b + 8].tolist()
    # down: slot rt * 64 + r * 4 + j holds row 64 rt + 16 j + r
    raw = meta.view(np.uint8)[16 * 2 * inter * 5:]
    dd = raw[: 4 * nsbd * 1280].view(np.uint32).reshape(nsbd, 1280)
    sm = raw[4 * nsbd * 1280:].view(np.uint16).reshape(inter // 32, 1280)
    slot = np.arange(1280)
    row = 64 * (slot // 64) + 16 * (slot % 4) + (slot // 4) % 16
    assert sorted(row.tolist()) == list(range(1280))
    np.testing.assert_array_equal(dd & 0xFFFF, d["d"][row].T)
    np.testing.assert_array_equal(dd >> 16, d["dmin"][row].T)
    np.testing.assert_array_equal(sm & 255, d["sc"][row].T)
    np.testing.assert_array_equal(sm >> 8, d["m"][row].T)


def test_pack_q4k_rejects_bad_fields(lib):
    rng = np.random.default_rng(0)
    mats = [_q4k_matrix(rng, 896, 1280), _q4k_matrix(rng, 896, 1280), _q4k_matrix(rng, 1280, 896)]
    for key, idx, val in (("q", (3, 9), 16), ("sc", (5, 2), 64), ("m", (0, 0), 200), ("d", (1, 1), 0x7C00),
                          ("dmin", (2, 3), 0xFE00)):
        bad = [dict(x) for x in mats]
        bad[2] = {k: v.copy() for k, v in mats[2].items()}
        bad[2][key][idx] = val
        with pytest.raises(B.MoeError, match="FORMAT"):
            B.moe_pack_expert_q4k(*bad)
    q = B.Q4kMatrix(None, None, None, None, None)
    assert lib.moe_pack_expert_q4k(ctypes.byref(q), ctypes.byref(q), ctypes.byref(q), 896, 0x100, 0x100) == 1
    assert lib.moe_pack_expert_q4k(ctypes.byref(q), ctypes.byref(q), ctypes.byref(q), 100, 0x100, 0x100) == 2
    # the symmetric packer does not take the two-level group
    lay = make_tiny_layer(1, E=1, H=1280, I=896, Is=896, fmt=QFmt(4, 32))
    with pytest.raises(B.MoeError, match="FORMAT"):
        B.moe_pack_expert(lay["gate_q"][0], lay["up_q"][0], lay["down_q"][0], lay["gate_s"][0], lay["up_s"][0],
                          lay["down_s"][0], 4, B.MOE_Q4K)


def _fwd(lib, **kw):
    A = 0x10000  # fake, aligned device addresses: validation never dereferences them
    a = dict(x=A, x_dtype=0, T=4, rw=A, rb=None, eq=A, es=A, eb=4, eg=64, sq=A, ss=A, sb=8, sg=128,
             y=A * 2, ids=A, w=A, ws=A, wsb=1 << 40, flags=0, stream=None)
    a.update(kw)
    return lib.moe_layer_forward(a["x"], a["x_dtype"], a["T"], a["rw"], a["rb"], a["eq"], a["es"], a["eb"], a["eg"],
                                 a["sq"], a["ss"], a["sb"], a["sg"], a["y"], a["ids"], a["w"], a["ws"], a["wsb"],
                                 a["flags"], a["stream"])


def test_forward_validation_codes(lib):
    assert _fwd(lib, x=None) == 1
    assert _fwd(lib, ws=None) == 1
    assert _fwd(lib, T=-1) == 2
    assert _fwd(lib, T=8193) == 2
    assert _fwd(lib, eb=5) == 3
    assert _fwd(lib, sg=16) == 3
    assert _fwd(lib, y=0x10008) == 4
    assert _fwd(lib, rb=0x10002) == 4
    assert _fwd(lib, T=0, ids=0x10004, w=0x10008) == 0   # 4-byte aligned ids/weights are accepted
    assert _fwd(lib, eq=0x10004) == 4
    assert _fwd(lib, wsb=16) == 5
    assert _fwd(lib, flags=1 << 9) == 7
    assert _fwd(lib, flags=B.MOE_FORCE_DECODE | B.MOE_FORCE_GROUPED) == 7
    assert _fwd(lib, flags=B.MOE_NORM_BF16) == 7
    assert _fwd(lib, flags=B.MOE_NORM_INPUT, x_dtype=1) == 7
    assert _fwd(lib, x_dtype=2) == 7
    assert _fwd(lib, y=0x10000) == 7                        # aliasing without accumulate
    assert _fwd(lib, T=0) == 0                               # empty call: nothing enqueued
    assert _fwd(lib, T=0, x=None, y=None, ids=None, w=None) == 0
    assert _fwd(lib, T=0, ws=None) == 1
    # the two-level format has 4-bit codes
    assert _fwd(lib, eb=8, eg=B.MOE_Q4K) == 3
    assert _fwd(lib, sg=B.MOE_Q4K) == 3                     # shared codes are int8 here
    assert _fwd(lib, eg=B.MOE_Q4K, T=0) == 0


def test_workspace_bytes(lib):
    assert B.moe_workspace_bytes(-1) == 0 and B.moe_workspace_bytes(8193) == 0
    small, big = B.moe_workspace_bytes(1), B.moe_workspace_bytes(2184)
    assert 0 < small < big
    # ysorted + h_routed dominate: T*6*(1280+896)*4
    assert big >= 2184 * 6 * (1280 + 896) * 4


def test_rmsnorm_validation(lib):
    assert lib.moe_rmsnorm(None, 0x100, 0, 1, 1e-6, None) == 1
    assert lib.moe_rmsnorm(0x100, 0x104, 0, 1, 1e-6, None) == 4
    assert lib.moe_rmsnorm(0x100, 0x200, 3, 1, 1e-6, None) == 7
    assert lib.moe_rmsnorm(0x100, 0x200, 0, 0, 1e-6, None) == 0


def test_hbm_read_probe_validation(lib):
    # argument checks come before any HIP call, so they run without a GPU
    assert lib.moe_hbm_read_probe(None, 16, 0x100, None) == 1
    assert lib.moe_hbm_read_probe(0x100, 16, None, None) == 1
    assert lib.moe_hbm_read_probe(0x108, 16, 0x100, None) == 4
    assert lib.moe_hbm_read_probe(0x100, 24, 0x100, None) == 4
    assert lib.moe_hbm_read_probe(0x100, 16, 0x102, None) == 4
    assert lib.moe_hbm_read_probe(0x100, 0, 0x100, None) == 0


def test_decode_forward_validation(lib):
    A = 0x10000
    L = (B.LayerWeights * 2)(B.LayerWeights(A, None, A, A, A, A), B.LayerWeights(A, None, A, A, A, A))
    def fwd(**kw):
        a = dict(x=A, xd=0, y=A, n=2, layers=L, eb=4, eg=64, sb=8, sg=128, ids=A, w=A, ws=A, wsb=1 << 30,
                 flags=0, stream=None)
        a.update(kw)
        return lib.moe_decode_forward(a["x"], a["xd"], a["y"], a["n"], a["layers"], a["eb"], a["eg"], a["sb"],
                                      a["sg"], a["ids"], a["w"], a["ws"], a["wsb"], a["flags"], a["stream"])
    assert fwd(x=None) == 1
    assert fwd(n=0) == 2 and fwd(n=17) == 2
    assert fwd(eg=16) == 3
    assert fwd(eb=8, eg=B.MOE_Q4K) == 3 and fwd(sg=B.MOE_Q4K) == 3
    assert fwd(flags=B.MOE_NORM_BF16 | B.MOE_NORM_INPUT) == 7
    assert fwd(flags=B.MOE_FORCE_DECODE) == 7
    assert fwd(xd=1) == 7                    # bf16 input cannot alias the f32 output
    assert fwd(ws=0x10008) == 4
    assert fwd(wsb=100) == 5
    bad = (B.LayerWeights * 2)(B.LayerWeights(A, None, A, A, A, A), B.LayerWeights(A, None, 0x10008, A, A, A))
    assert fwd(layers=bad) == 4
    nul = (B.LayerWeights * 2)(B.LayerWeights(A, None, A, A, A, A), B.LayerWeights(None, None, A, A, A, A))
    assert fwd(layers=nul) == 1
    assert lib.moe_decode_workspace_init(None, 0, None) == 1
    assert lib.moe_decode_workspace_init(A, 16, None) == 5
    assert B.moe_decode_workspace_bytes() > 224 * 1280 * 4


# ----------------------------------------------------------------- dense ends: validation only
def test_lm_head_validation(lib):
    A = 0x10000                                  # aligned fake device addresses: nothing is launched
    ok = dict(h=A, T=1, flags=0, w=A, bits=16, s=None, g=0, vocab=129280, logits=None, tok=A, tl=A, ws=A,
              wsb=B.moe_lm_head_workspace_bytes(1, 129280))

    def call(**kw):
        a = dict(ok, **kw)
        return lib.moe_lm_head_argmax(a["h"], a["T"], a["flags"], a["w"], a["bits"], a["s"], a["g"], a["vocab"],
                                      a["logits"], a["tok"], a["tl"], a["ws"], a["wsb"], None)
    assert call(h=None) == 1 and call(tok=None) == 1
    assert call(bits=4) == 3 and call(bits=8, s=A, g=48) == 3 and call(bits=8, s=None, g=128) == 1
    assert call(T=5) == 2 and call(vocab=0) == 2 and call(T=-1) == 2
    assert call(flags=4) == 7
    assert call(h=A + 4) == 4 and call(tl=A + 2) == 4
    assert call(wsb=16) == 5
    assert call(T=0) == 0                        # nothing to do
    assert B.moe_lm_head_workspace_bytes(5, 10) == 0 and B.moe_lm_head_workspace_bytes(1, 0) == 0
    assert B.moe_lm_head_workspace_bytes(4, 129280) >= (129280 // 256) * 4 * 8


def test_dense_ffn_validation(lib):
    A = 0x10000
    ok = dict(x=A, T=2, q=A, s=A, bits=8, g=64, inter=6848, y=A, flags=0, ws=A,
              wsb=B.moe_dense_ffn_workspace_bytes(2, 6848))

    def call(**kw):
        a = dict(ok, **kw)
        return lib.moe_dense_ffn_forward(a["x"], a["T"], a["q"], a["s"], a["bits"], a["g"], a["inter"], a["y"],
                                         a["flags"], a["ws"], a["wsb"], None)
    assert call(x=None) == 1 and call(s=None) == 1
    assert call(bits=2) == 3 and call(g=16) == 3
    assert call(inter=6848 + 32) == 2 and call(g=128) == 2      # 6848 is not a multiple of 128
    assert call(T=5) == 2 and call(inter=8192 + 64) == 2
    assert call(flags=8) == 7
    assert call(y=A + 8) == 4 and call(s=A + 2) == 4
    assert call(wsb=100) == 5
    assert call(T=0) == 0
    assert B.moe_dense_ffn_workspace_bytes(2, 6848) >= 2 * 6848 * 4
    assert B.moe_dense_ffn_workspace_bytes(1, 100) == 0


def test_rswa_validation(lib):
    A = 0x10000
    ok = dict(S=2, n_ref=288, q=A, k=A, v=A, rk=A, rv=A, gk=A, gv=A, ng=A, out=A, ws=A,
              wsb=B.moe_rswa_workspace_bytes(2, 288))

    def call(**kw):
        a = dict(ok, **kw)
        return lib.moe_rswa_decode(a["S"], a["n_ref"], a["q"], a["k"], a["v"], a["rk"], a["rv"], a["gk"], a["gv"],
                                   a["ng"], a["out"], a["ws"], a["wsb"], None)
    assert call(q=None) == 1 and call(ng=None) == 1 and call(rk=None) == 1
    assert call(S=-1) == 2 and call(S=4097) == 2 and call(n_ref=65537) == 2
    assert call(q=A + 4) == 4 and call(ng=A + 2) == 4 and call(rk=A + 8) == 4
    assert call(wsb=64) == 5
    assert call(S=0) == 0
    assert B.moe_rswa_workspace_bytes(1, 0) >= 10 * 2 * 132 * 4       # ring only: two chunks of 64
    assert B.moe_rswa_workspace_bytes(2, 288) >= 2 * 10 * 7 * 132 * 4


@pytest.mark.parametrize("bits", [4, 8])
def test_pack_dense_ffn_layout(lib, bits):
    """The dense MLP code buffer as include/moe_dense.h describes it: gate | up
    | down rows, int8 one code per byte, int4 element 2j in the low nibble."""
    rng = np.random.default_rng(7 + bits)
    inter = 128
    lo, hi = (-8, 8) if bits == 4 else (-128, 128)
    g = rng.integers(lo, hi, (inter, 1280), dtype=np.int8)
    u = rng.integers(lo, hi, (inter, 1280), dtype=np.int8)
    d = rng.integers(lo, hi, (1280, inter), dtype=np.int8)
    g[0, :4] = [lo, hi - 1, 0, -1]
    out = B.moe_pack_dense_ffn(g, u, d, bits)
    assert out.size == B.load().moe_dense_ffn_code_bytes(bits, inter) == 3 * inter * 1280 * bits // 8
    parts = np.split(out, 3)
    for part, m in zip(parts, (g, u, d)):
        flat = m.reshape(-1).astype(np.int64)
        if bits == 8:
            got = part.view(np.int8).astype(np.int64)
        else:
            low, high = part & 0x0F, part >> 4
            dec = np.empty(flat.size, np.int64)
            dec[0::2] = np.where(low >= 8, low.astype(np.int64) - 16, low)
            dec[1::2] = np.where(high >= 8, high.astype(np.int64) - 16, high)
            got = dec
        np.testing.assert_array_equal(got, flat)


def test_pack_dense_ffn_rejects(lib):
    inter = 64
    g = np.zeros((inter, 1280), np.int8)
    u = np.zeros((inter, 1280), np.int8)
    d = np.zeros((1280, inter), np.int8)
    out = np.zeros(3 * inter * 1280, np.uint8)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    assert lib.moe_pack_dense_ffn(p(g), p(u), p(d), 4, inter, p(out)) == 0
    g[3, 5] = 8                                   # out of the int4 range
    assert lib.moe_pack_dense_ffn(p(g), p(u), p(d), 4, inter, p(out)) == 3
    assert lib.moe_pack_dense_ffn(p(g), p(u), p(d), 8, inter, p(out)) == 0
    assert lib.moe_pack_dense_ffn(p(g), p(u), p(d), 2, inter, p(out)) == 3
    assert lib.moe_pack_dense_ffn(p(g), p(u), p(d), 8, 96, p(out)) == 2
    assert lib.moe_pack_dense_ffn(None, p(u), p(d), 8, inter, p(out)) == 1
    assert lib.moe_dense_ffn_code_bytes(4, 6848) == 3 * 6848 * 640 and lib.moe_dense_ffn_code_bytes(3, 64) == 0
