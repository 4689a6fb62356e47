"""Workload definitions and seeded generators.

Shapes follow the decoder described on the franken_ocr pages: hidden 1280,
64 routed experts with top-6 routing, expert intermediate 896 and the two
shared experts fused into one SwiGLU of intermediate 1792 ("DeepSeek-V2 MoE
decoder" in the Architecture section of the franken_ocr README; "One forward
pass, left to right", step 6, of the browser demo page).  The workloads
are the synthetic stand-ins for the pages' workloads: one decode token, the
11-layer decode step, 32 concurrent pages, the 273-row visual prefill
(splice layout in the I/O contract of the Unlimited-OCR DeepEncoder ONNX
model card) and an 8-page multi-page prefill.  Two more are decode steps of
the continuous-batch spine at its default of 128 active streams and its
clamp of 256 (the batch-size setting under "focr ocr-batch" in the franken_ocr
README's command reference): every stream adds one token per step.

Every tensor comes from its own numpy ``SeedSequence(0, spawn_key=(w, l, t))``
stream (w = workload index, l = layer, t = tensor id), so any layer can be
regenerated alone and a smaller token count is a prefix of nothing: tokens
are drawn from their own stream keyed by the batch index.

Codes are returned unpacked, one signed code per int8 byte, row-major
``[rows][K]`` with K the reduction axis; scales are float32 ``[rows][K/G]``.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

HIDDEN = 1280
N_EXPERTS = 64
TOP_K = 6
INTER = 896
SHARED_INTER = 1792
NORM_EPS = 1e-6

# tensor ids inside one layer's seed space
_T_ROUTER, _T_BIAS = 0, 1
_T_GATE, _T_UP, _T_DOWN = 2, 3, 4
_T_GATE_S, _T_UP_S, _T_DOWN_S = 5, 6, 7
_T_SGATE, _T_SUP, _T_SDOWN = 8, 9, 10
_T_SGATE_S, _T_SUP_S, _T_SDOWN_S = 11, 12, 13
_TOKEN_LAYER = 0xFFFF  # "layer" slot used for token batches


# group value that selects the two-level 4-bit format (see ``_q4k``)
Q4K_GROUP = 256
Q4K_SUB = 32


@dataclass(frozen=True)
class QFmt:
    bits: int   # 4 or 8
    group: int  # consecutive K elements that share one f32 scale (Q4K_GROUP: the two-level format)

    @property
    def code_range(self):
        return (-8, 7) if self.bits == 4 else (-127, 127)

    @property
    def q4k(self) -> bool:
        return self.bits == 4 and self.group == Q4K_GROUP


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    n_tokens: int
    n_layers: int
    x_dtype: str            # "f32" or "bf16"
    routed: QFmt
    shared: QFmt
    bias: str               # "none", "normal1.5" or "zipf2"
    chained: bool           # RMSNorm before each layer + residual add
    norm_bf16: bool         # layer input rounded to bf16 after the norm

    def with_tokens(self, n: int) -> "Workload":
        return replace(self, n_tokens=n)

    def with_layers(self, n: int) -> "Workload":
        return replace(self, n_layers=n)


WORKLOADS = [
    Workload(0, "decode_1tok_1layer_int8g128", 1, 1, "f32",
             QFmt(8, 128), QFmt(8, 128), "none", False, False),
    Workload(1, "decode_1tok_11layers_int4g64_shared_int8g128", 1, 11, "f32",
             QFmt(4, 64), QFmt(8, 128), "none", True, False),
    Workload(2, "batched_decode_32tok_int4g32_biased", 32, 1, "bf16",
             QFmt(4, 32), QFmt(4, 32), "normal1.5", False, False),
    Workload(3, "visual_prefill_273tok_int4g128", 273, 1, "bf16",
             QFmt(4, 128), QFmt(4, 128), "none", False, False),
    Workload(4, "multipage_prefill_2184tok_11layers_int4g64_zipf", 2184, 11, "bf16",
             QFmt(4, 64), QFmt(4, 64), "zipf2", True, True),
    # continuous-batch decode: one step advances every active stream by one
    # token; 128 streams is the batch spine's default, 256 its clamp
    Workload(5, "continuous_batch_decode_128streams_11layers_int4g64_shared_int8g128", 128, 11, "f32",
             QFmt(4, 64), QFmt(8, 128), "none", True, False),
    Workload(6, "continuous_batch_decode_256streams_11layers_int4g64_shared_int8g128", 256, 11, "f32",
             QFmt(4, 64), QFmt(8, 128), "none", True, False),
    # the decode step with the routed experts in the two-level (Q4_K-style)
    # 4-bit format and the shared expert in int8: the q4k/q8 storage of the
    # WebGPU engine the model card pairs with the community K-quant GGUF
    Workload(7, "decode_1tok_11layers_q4k_shared_int8g128", 1, 11, "f32",
             QFmt(4, Q4K_GROUP), QFmt(8, 128), "none", True, False),
]


def workload(i: int) -> Workload:
    return WORKLOADS[i]


def _rng(w: int, layer: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(0, spawn_key=(w, layer, tensor)))


def _codes(rng, shape, fmt: QFmt) -> np.ndarray:
    lo, hi = fmt.code_range
    return rng.integers(lo, hi, size=shape, endpoint=True, dtype=np.int8)


def _scales(rng, shape) -> np.ndarray:
    return rng.uniform(0.002, 0.02, size=shape).astype(np.float32)


def _q4k(rng, lead: tuple, K: int) -> dict:
    """One stack of matrices ``[*lead][K]`` in the two-level 4-bit format.

    Fields: unsigned 4-bit codes q in [0, 15]; per 32 columns (a sub-block) a
    6-bit scale sc and a 6-bit minimum m; per 256 columns (a super-block; the
    last one of a row is partial when K is not a multiple of 256) the f16
    factors d and dmin, returned as their 16-bit patterns.  Distribution: d
    uniform in [1e-4, 4e-4], dmin = 8 d (rounded to f16), sc uniform in
    [8, 63] and m = sc - U{0..8} clipped at 0, so that a sub-block's weights
    d sc q - dmin m straddle zero with magnitudes like the symmetric formats'.
    """
    nsb, nsub = -(-K // Q4K_GROUP), K // Q4K_SUB
    q = rng.integers(0, 15, size=lead + (K,), endpoint=True, dtype=np.uint8)
    d = rng.uniform(1e-4, 4e-4, size=lead + (nsb,)).astype(np.float16)
    dmin = (d.astype(np.float32) * 8.0).astype(np.float16)
    sc = rng.integers(8, 63, size=lead + (nsub,), endpoint=True).astype(np.uint8)
    m = np.clip(sc.astype(np.int16) - rng.integers(0, 8, size=lead + (nsub,), endpoint=True), 0, 63).astype(np.uint8)
    return {"q": q, "d": d.view(np.uint16), "dmin": dmin.view(np.uint16), "sc": sc, "m": m}


def _matrix(out: dict, name: str, rng_q, rng_s, lead: tuple, rows: int, K: int, fmt: QFmt):
    """Codes and scales of one matrix stack into ``out`` under ``name``_*:
    symmetric formats give ``_q`` (int8 codes) and ``_s`` (f32 scales); the
    two-level format gives ``_q`` (uint8 codes 0..15), ``_d``, ``_dmin``,
    ``_sc`` and ``_m``."""
    if fmt.q4k:
        for k, v in _q4k(rng_q, lead + (rows,), K).items():
            out[f"{name}_{k}"] = v
    else:
        out[f"{name}_q"] = _codes(rng_q, lead + (rows, K), fmt)
        out[f"{name}_s"] = _scales(rng_s, lead + (rows, K // fmt.group))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_tokens(wl: Workload, batch: int = 0, n_tokens: int | None = None):
    """Input activations of one batch: (values f32 [T,H], bf16 bits or None)."""
    T = wl.n_tokens if n_tokens is None else n_tokens
    x = _rng(wl.index, _TOKEN_LAYER, batch).standard_normal((T, HIDDEN)).astype(np.float32)
    if wl.x_dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bf16_bits_to_f32(bits), bits
    return x, None


def _bias(wl: Workload, layer: int):
    if wl.bias == "none":
        return None
    if wl.bias == "normal1.5":
        return _rng(wl.index, layer, _T_BIAS).normal(0.0, 1.5, N_EXPERTS).astype(np.float32)
    if wl.bias == "zipf2":
        rank = np.arange(1, N_EXPERTS + 1, dtype=np.float64)
        return (2.0 * np.log(1.0 / rank)).astype(np.float32)
    raise ValueError(wl.bias)


def make_layer(wl: Workload, layer: int) -> dict:
    """All tensors of one MoE layer (layer counts from 0 within the workload)."""
    w, l = wl.index, layer
    E, H, I, Is = N_EXPERTS, HIDDEN, INTER, SHARED_INTER
    rf, sf = wl.routed, wl.shared
    d = {
        "router_w": (_rng(w, l, _T_ROUTER).standard_normal((E, H)) * 0.02).astype(np.float32),
        "router_b": _bias(wl, l),
        "routed_fmt": rf,
        "shared_fmt": sf,
    }
    _matrix(d, "gate", _rng(w, l, _T_GATE), _rng(w, l, _T_GATE_S), (E,), I, H, rf)
    _matrix(d, "up", _rng(w, l, _T_UP), _rng(w, l, _T_UP_S), (E,), I, H, rf)
    _matrix(d, "down", _rng(w, l, _T_DOWN), _rng(w, l, _T_DOWN_S), (E,), H, I, rf)
    _matrix(d, "shared_gate", _rng(w, l, _T_SGATE), _rng(w, l, _T_SGATE_S), (), Is, H, sf)
    _matrix(d, "shared_up", _rng(w, l, _T_SUP), _rng(w, l, _T_SUP_S), (), Is, H, sf)
    _matrix(d, "shared_down", _rng(w, l, _T_SDOWN), _rng(w, l, _T_SDOWN_S), (), H, Is, sf)
    return d


def make_tiny_layer(seed: int, E: int, H: int, I: int, Is: int, fmt: QFmt,
                    shared_fmt: QFmt | None = None, bias_std: float = 0.0) -> dict:
    """A small layer of arbitrary shape for oracle tests (same tensor names)."""
    sf = shared_fmt or fmt
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(99,)))
    return {
        "router_w": (rng.standard_normal((E, H)) * 0.5).astype(np.float32),
        "router_b": (rng.normal(0, bias_std, E).astype(np.float32) if bias_std else None),
        "gate_q": _codes(rng, (E, I, H), fmt),
        "up_q": _codes(rng, (E, I, H), fmt),
        "down_q": _codes(rng, (E, H, I), fmt),
        "gate_s": _scales(rng, (E, I, H // fmt.group)),
        "up_s": _scales(rng, (E, I, H // fmt.group)),
        "down_s": _scales(rng, (E, H, I // fmt.group)),
        "shared_gate_q": _codes(rng, (Is, H), sf),
        "shared_up_q": _codes(rng, (Is, H), sf),
        "shared_down_q": _codes(rng, (H, Is), sf),
        "shared_gate_s": _scales(rng, (Is, H // sf.group)),
        "shared_up_s": _scales(rng, (Is, H // sf.group)),
        "shared_down_s": _scales(rng, (H, Is // sf.group)),
        "routed_fmt": fmt,
        "shared_fmt": sf,
    }


# --------------------------------------------------------------------------
# the decoder's dense ends: layer-0 SwiGLU MLP and lm_head (seed space 7)
# --------------------------------------------------------------------------
VOCAB = 129280
DENSE_INTER = 6848
_W_DENSE_HEAD = 7
_T_HEAD_W, _T_HEAD_S = 20, 21
_T_DG, _T_DU, _T_DD, _T_DGS, _T_DUS, _T_DDS = 22, 23, 24, 25, 26, 27
_T_HIDDEN = 28


def make_lm_head(dtype: str, group: int = 128, vocab: int = VOCAB) -> dict:
    """lm_head weights [vocab][1280]: "bf16" (N(0, 0.02) rounded to bf16, as
    16-bit patterns) or "int8" (codes in [-127, 127], f32 scales per group of
    K).  Smaller vocabularies are prefixes of the full one."""
    if dtype == "bf16":
        w = (_rng(_W_DENSE_HEAD, 0, _T_HEAD_W).standard_normal((VOCAB, HIDDEN)) * 0.02).astype(np.float32)
        return {"dtype": "bf16", "w": f32_to_bf16_bits(w[:vocab]), "vocab": vocab}
    if dtype == "int8":
        q = _codes(_rng(_W_DENSE_HEAD, 0, _T_HEAD_W), (VOCAB, HIDDEN), QFmt(8, group))
        s = _scales(_rng(_W_DENSE_HEAD, 0, _T_HEAD_S), (VOCAB, HIDDEN // group))
        return {"dtype": "int8", "q": q[:vocab], "s": s[:vocab], "group": group, "vocab": vocab}
    raise ValueError(dtype)


def make_dense_ffn(fmt: QFmt, inter: int = DENSE_INTER) -> dict:
    """Codes and scales of a dense SwiGLU MLP 1280 -> inter -> 1280 (gate and
    up [inter][1280], down [1280][inter]; scales per group of K)."""
    H, g = HIDDEN, fmt.group
    return {
        "gate_q": _codes(_rng(_W_DENSE_HEAD, 1, _T_DG), (inter, H), fmt),
        "up_q": _codes(_rng(_W_DENSE_HEAD, 1, _T_DU), (inter, H), fmt),
        "down_q": _codes(_rng(_W_DENSE_HEAD, 1, _T_DD), (H, inter), fmt),
        "gate_s": _scales(_rng(_W_DENSE_HEAD, 1, _T_DGS), (inter, H // g)),
        "up_s": _scales(_rng(_W_DENSE_HEAD, 1, _T_DUS), (inter, H // g)),
        "down_s": _scales(_rng(_W_DENSE_HEAD, 1, _T_DDS), (H, inter // g)),
        "bits": fmt.bits, "group": g, "inter": inter,
    }


def make_hidden(n: int, batch: int = 0) -> np.ndarray:
    """Residual-stream stand-in rows h ~ N(0, 1), f32 [n][1280]."""
    return _rng(_W_DENSE_HEAD, _TOKEN_LAYER, _T_HIDDEN + 16 * batch).standard_normal((n, HIDDEN)).astype(np.float32)


# --------------------------------------------------------------------------
# R-SWA attention decode inputs (seed space 8)
# --------------------------------------------------------------------------
HEADS = 10
HEAD_DIM = 128
RSWA_WINDOW = 128
_W_RSWA = 8


def make_rswa(n_streams: int, n_ref: int, n_gen=None, seed: int = 0) -> dict:
    """One decode step of n_streams independent streams: q, the new key and
    value [S][10][128] f32 ~ N(0, 1); the frozen reference block and the ring
    [S][10][n][128] as bf16 bit patterns of N(0, 1) draws (the ring as left by
    earlier steps); n_gen [S] int32, generated tokens before this one (by
    default a spread from 0 to past several ring wraps)."""
    r = _rng(_W_RSWA, seed, 0)
    S, Hh, D, W = n_streams, HEADS, HEAD_DIM, RSWA_WINDOW
    d = {
        "q": r.standard_normal((S, Hh, D)).astype(np.float32),
        "k_new": r.standard_normal((S, Hh, D)).astype(np.float32),
        "v_new": r.standard_normal((S, Hh, D)).astype(np.float32),
        "ref_k": f32_to_bf16_bits(r.standard_normal((S, Hh, n_ref, D)).astype(np.float32)),
        "ref_v": f32_to_bf16_bits(r.standard_normal((S, Hh, n_ref, D)).astype(np.float32)),
        "ring_k": f32_to_bf16_bits(r.standard_normal((S, Hh, W, D)).astype(np.float32)),
        "ring_v": f32_to_bf16_bits(r.standard_normal((S, Hh, W, D)).astype(np.float32)),
    }
    if n_gen is None:
        n_gen = r.integers(0, 4 * W, size=S)
    d["n_gen"] = np.asarray(n_gen, dtype=np.int32).reshape(S)
    d["n_ref"] = n_ref
    return d


# --------------------------------------------------------------------------
# attention projections of a decoder layer (seed space 9)
# --------------------------------------------------------------------------
_W_ATTN = 9


def make_attn_weights(seed: int = 0) -> dict:
    """W_q, W_k, W_v, W_o [1280][1280] as bf16 bit patterns of N(0, 0.02)
    draws (the router's draw; y = W x, row n gives output n)."""
    return {k: f32_to_bf16_bits((_rng(_W_ATTN, seed, t).standard_normal((HIDDEN, HIDDEN)) * 0.02).astype(np.float32))
            for t, k in enumerate(("w_q", "w_k", "w_v", "w_o"))}
