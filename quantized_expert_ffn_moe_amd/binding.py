"""Thin ctypes binding of libmoe.so (the C ABI in include/moe.h,
include/moe_dense.h and include/moe_attn.h).

Argument marshalling only: torch tensors become device addresses and the
current HIP stream, numpy arrays become host addresses.  Every step of the
layer runs in the library's own kernels; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HIDDEN, EXPERTS, TOPK, INTER, SHARED_INTER = 1280, 64, 6, 896, 1792
MOE_F32, MOE_BF16 = 0, 1
MOE_ACCUMULATE, MOE_NORM_INPUT, MOE_NORM_BF16 = 1, 2, 4
MOE_FORCE_DECODE, MOE_FORCE_GROUPED = 8, 16

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
EXPORTS = ("moe_status_str", "moe_expert_code_bytes", "moe_expert_scale_count", "moe_pack_expert",
           "moe_pack_expert_q4k",
           "moe_workspace_bytes", "moe_layer_forward", "moe_rmsnorm", "moe_decode_workspace_bytes",
           "moe_decode_workspace_init", "moe_decode_forward", "moe_lm_head_workspace_bytes",
           "moe_lm_head_argmax", "moe_dense_ffn_workspace_bytes", "moe_dense_ffn_forward",
           "moe_dense_ffn_code_bytes", "moe_pack_dense_ffn",
           "moe_rswa_workspace_bytes", "moe_rswa_decode", "moe_layer_forward_static",
           "moe_attn_block_workspace_bytes", "moe_attn_block_forward", "moe_hbm_read_probe")
MOE_HEAD_INT8, MOE_HEAD_BF16 = 8, 16
MOE_Q4K = 256   # group value of the two-level 4-bit format
DECODE_MAX_LAYERS = 16


class LayerWeights(ctypes.Structure):
    """moe_layer_weights_t: device pointers of one layer."""
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("expert_q", ctypes.c_void_p), ("expert_scales", ctypes.c_void_p),
                ("shared_q", ctypes.c_void_p), ("shared_scales", ctypes.c_void_p)]



class Q4kMatrix(ctypes.Structure):
    """moe_q4k_matrix_t: host pointers of one two-level matrix."""
    _fields_ = [("q", ctypes.c_void_p), ("d", ctypes.c_void_p), ("dmin", ctypes.c_void_p),
                ("sc", ctypes.c_void_p), ("m", ctypes.c_void_p)]


_lib = None


class MoeError(RuntimeError):
    pass


def load():
    """Load the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [i32]
    L.moe_expert_code_bytes.restype = sz
    L.moe_expert_code_bytes.argtypes = [i32, i32]
    L.moe_expert_scale_count.restype = sz
    L.moe_expert_scale_count.argtypes = [i32, i32]
    L.moe_pack_expert.restype = i32
    L.moe_pack_expert.argtypes = [vp] * 6 + [i32, i32, i32, vp, vp]
    L.moe_pack_expert_q4k.restype = i32
    L.moe_pack_expert_q4k.argtypes = [ctypes.POINTER(Q4kMatrix)] * 3 + [i32, vp, vp]
    L.moe_workspace_bytes.restype = sz
    L.moe_workspace_bytes.argtypes = [i32]
    L.moe_layer_forward.restype = i32
    L.moe_layer_forward.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, i32, i32,
                                    vp, vp, vp, vp, sz, u32, vp]
    L.moe_layer_forward_static.restype = i32
    L.moe_layer_forward_static.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, i32, i32,
                                           vp, vp, vp, u32, vp]
    L.moe_rmsnorm.restype = i32
    L.moe_rmsnorm.argtypes = [vp, vp, i32, i32, ctypes.c_float, vp]
    L.moe_decode_workspace_bytes.restype = sz
    L.moe_decode_workspace_bytes.argtypes = []
    L.moe_decode_workspace_init.restype = i32
    L.moe_decode_workspace_init.argtypes = [vp, sz, vp]
    L.moe_decode_forward.restype = i32
    L.moe_decode_forward.argtypes = [vp, i32, vp, i32, ctypes.POINTER(LayerWeights), i32, i32, i32, i32,
                                     vp, vp, vp, sz, u32, vp]
    L.moe_lm_head_workspace_bytes.restype = sz
    L.moe_lm_head_workspace_bytes.argtypes = [i32, i32]
    L.moe_lm_head_argmax.restype = i32
    L.moe_lm_head_argmax.argtypes = [vp, i32, u32, vp, i32, vp, i32, i32, vp, vp, vp, vp, sz, vp]
    L.moe_dense_ffn_workspace_bytes.restype = sz
    L.moe_dense_ffn_workspace_bytes.argtypes = [i32, i32]
    L.moe_dense_ffn_forward.restype = i32
    L.moe_dense_ffn_forward.argtypes = [vp, i32, vp, vp, i32, i32, i32, vp, u32, vp, sz, vp]
    L.moe_dense_ffn_code_bytes.restype = sz
    L.moe_dense_ffn_code_bytes.argtypes = [i32, i32]
    L.moe_pack_dense_ffn.restype = i32
    L.moe_pack_dense_ffn.argtypes = [vp, vp, vp, i32, i32, vp]
    L.moe_rswa_workspace_bytes.restype = sz
    L.moe_rswa_workspace_bytes.argtypes = [i32, i32]
    L.moe_attn_block_workspace_bytes.restype = sz
    L.moe_attn_block_workspace_bytes.argtypes = [i32, i32]
    L.moe_attn_block_forward.restype = i32
    L.moe_attn_block_forward.argtypes = [i32, i32] + [vp] * 8 + [vp, sz, vp]
    L.moe_rswa_decode.restype = i32
    L.moe_rswa_decode.argtypes = [i32, i32] + [vp] * 9 + [vp, sz, vp]
    L.moe_hbm_read_probe.restype = i32
    L.moe_hbm_read_probe.argtypes = [vp, sz, vp, vp]
    _lib = L
    return L


def check(status: int):
    if status != 0:
        raise MoeError(load().moe_status_str(status).decode())


def _np_ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ----------------------------------------------------------------- packing (host)
def moe_expert_code_bytes(bits: int, inter: int) -> int:
    return load().moe_expert_code_bytes(bits, inter)


def moe_expert_scale_count(group: int, inter: int) -> int:
    return load().moe_expert_scale_count(group, inter)


def moe_pack_expert(gate, up, down, gate_s, up_s, down_s, bits: int, group: int):
    """Pack one expert (host numpy in, host numpy out)."""
    inter = gate.shape[0]
    arrs = [np.ascontiguousarray(a, dtype=np.int8) for a in (gate, up, down)]
    scs = [np.ascontiguousarray(a, dtype=np.float32) for a in (gate_s, up_s, down_s)]
    codes = np.empty(moe_expert_code_bytes(bits, inter), np.uint8)
    scales = np.empty(moe_expert_scale_count(group, inter), np.float32)
    check(load().moe_pack_expert(*[_np_ptr(a) for a in arrs], *[_np_ptr(a) for a in scs],
                                 inter, bits, group, _np_ptr(codes), _np_ptr(scales)))
    return codes, scales


def moe_pack_expert_q4k(gate: dict, up: dict, down: dict):
    """Pack one two-level expert: dicts with q, d, dmin, sc, m (host numpy) ->
    (codes uint8, records as float32 words)."""
    inter = gate["q"].shape[0]
    keep, mats = [], []
    for f in (gate, up, down):
        arrs = {k: np.ascontiguousarray(f[k], dtype=np.uint16 if k in ("d", "dmin") else np.uint8)
                for k in ("q", "d", "dmin", "sc", "m")}
        keep.append(arrs)
        mats.append(Q4kMatrix(*[_np_ptr(arrs[k]) for k in ("q", "d", "dmin", "sc", "m")]))
    codes = np.empty(moe_expert_code_bytes(4, inter), np.uint8)
    meta = np.empty(moe_expert_scale_count(MOE_Q4K, inter), np.float32)
    check(load().moe_pack_expert_q4k(*[ctypes.byref(m) for m in mats], inter, _np_ptr(codes), _np_ptr(meta)))
    return codes, meta


def _pack_one(layer: dict, prefix: str, fmt, e=None):
    get = (lambda k: layer[f"{prefix}{k}"]) if e is None else (lambda k: layer[f"{prefix}{k}"][e])
    if fmt.bits == 4 and fmt.group == MOE_Q4K:
        return moe_pack_expert_q4k(*[{k: get(f"{n}_{k}") for k in ("q", "d", "dmin", "sc", "m")}
                                     for n in ("gate", "up", "down")])
    return moe_pack_expert(get("gate_q"), get("up_q"), get("down_q"), get("gate_s"), get("up_s"), get("down_s"),
                           fmt.bits, fmt.group)


def pack_layer(layer: dict, device="cuda"):
    """Pack one layer's codes/scales on the host and move them to the device."""
    import torch
    rf, sf = layer["routed_fmt"], layer["shared_fmt"]
    E = layer["gate_q"].shape[0]
    cb, sc = moe_expert_code_bytes(rf.bits, INTER), moe_expert_scale_count(rf.group, INTER)
    codes = np.empty(E * cb, np.uint8)
    scales = np.empty(E * sc, np.float32)
    for e in range(E):
        c, s = _pack_one(layer, "", rf, e)
        codes[e * cb:(e + 1) * cb] = c
        scales[e * sc:(e + 1) * sc] = s
    scodes, sscales = _pack_one(layer, "shared_", sf)
    t = lambda a: torch.from_numpy(a).to(device)
    return {
        "router_w": t(np.ascontiguousarray(layer["router_w"], np.float32)),
        "router_b": None if layer.get("router_b") is None else t(np.ascontiguousarray(layer["router_b"], np.float32)),
        "expert_q": t(codes), "expert_s": t(scales), "expert_bits": rf.bits, "expert_group": rf.group,
        "shared_q": t(scodes), "shared_s": t(sscales), "shared_bits": sf.bits, "shared_group": sf.group,
    }


# ----------------------------------------------------------------- GPU entry points
def moe_workspace_bytes(n_tokens: int) -> int:
    return load().moe_workspace_bytes(n_tokens)


def workspace(n_tokens: int, device="cuda"):
    import torch
    return torch.empty(max(moe_workspace_bytes(n_tokens), 256), dtype=torch.uint8, device=device)


def moe_layer_forward(x, packed: dict, y, topk_ids, topk_w, ws, flags: int = 0, stream=None):
    """Enqueue one layer: x [T,1280] f32/bf16 -> y [T,1280] f32, ids/weights [T,6]."""
    import torch
    T = x.shape[0] if x.dim() == 2 else 0
    x_dtype = MOE_BF16 if x.dtype == torch.bfloat16 else MOE_F32
    check(load().moe_layer_forward(
        _ptr(x), x_dtype, T, _ptr(packed["router_w"]), _ptr(packed["router_b"]),
        _ptr(packed["expert_q"]), _ptr(packed["expert_s"]), packed["expert_bits"], packed["expert_group"],
        _ptr(packed["shared_q"]), _ptr(packed["shared_s"]), packed["shared_bits"], packed["shared_group"],
        _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(), flags, _stream(stream)))


STATIC_MAX_TOKENS = 256


def moe_layer_forward_static(x, packed: dict, y, topk_ids, topk_w, flags: int = 0, stream=None):
    """moe_layer_forward without a workspace: the library's own per-GPU scratch
    (at most STATIC_MAX_TOKENS tokens; calls that overlap on one GPU race)."""
    import torch
    T = x.shape[0] if x.dim() == 2 else 0
    x_dtype = MOE_BF16 if x.dtype == torch.bfloat16 else MOE_F32
    check(load().moe_layer_forward_static(
        _ptr(x), x_dtype, T, _ptr(packed["router_w"]), _ptr(packed["router_b"]),
        _ptr(packed["expert_q"]), _ptr(packed["expert_s"]), packed["expert_bits"], packed["expert_group"],
        _ptr(packed["shared_q"]), _ptr(packed["shared_s"]), packed["shared_bits"], packed["shared_group"],
        _ptr(y), _ptr(topk_ids), _ptr(topk_w), flags, _stream(stream)))


def moe_rmsnorm(h, z, eps: float = 1e-6, stream=None):
    import torch
    z_dtype = MOE_BF16 if z.dtype == torch.bfloat16 else MOE_F32
    check(load().moe_rmsnorm(_ptr(h), _ptr(z), z_dtype, h.shape[0], eps, _stream(stream)))


def layer(x, packed: dict, flags: int = 0, y=None, ws=None):
    """Convenience: allocate outputs (torch) and run one layer; returns (ids, w, y)."""
    import torch
    T = x.shape[0]
    dev = x.device
    y = torch.empty(T, HIDDEN, dtype=torch.float32, device=dev) if y is None else y
    ids = torch.empty(T, TOPK, dtype=torch.int32, device=dev)
    w = torch.empty(T, TOPK, dtype=torch.float32, device=dev)
    ws = workspace(T, dev) if ws is None else ws
    moe_layer_forward(x, packed, y, ids, w, ws, flags)
    return ids, w, y


# ----------------------------------------------------------------- decode step
def moe_decode_workspace_bytes() -> int:
    return load().moe_decode_workspace_bytes()


def decode_workspace(device="cuda", stream=None):
    """Allocate and initialise a decode-step workspace."""
    import torch
    ws = torch.empty(moe_decode_workspace_bytes(), dtype=torch.uint8, device=device)
    check(load().moe_decode_workspace_init(_ptr(ws), ws.numel(), _stream(stream)))
    return ws


def layer_weights(packed_layers):
    arr = (LayerWeights * len(packed_layers))()
    for i, p in enumerate(packed_layers):
        arr[i] = LayerWeights(p["router_w"].data_ptr(),
                              None if p["router_b"] is None else p["router_b"].data_ptr(),
                              p["expert_q"].data_ptr(), p["expert_s"].data_ptr(),
                              p["shared_q"].data_ptr(), p["shared_s"].data_ptr())
    return arr


def moe_decode_forward(x, y, packed_layers, topk_ids, topk_w, ws, flags=0, weights=None, stream=None):
    """Enqueue one token through len(packed_layers) chained layers (one launch)."""
    import torch
    p0 = packed_layers[0]
    arr = layer_weights(packed_layers) if weights is None else weights
    x_dtype = MOE_BF16 if x.dtype == torch.bfloat16 else MOE_F32
    check(load().moe_decode_forward(_ptr(x), x_dtype, _ptr(y), len(packed_layers), arr,
                                    p0["expert_bits"], p0["expert_group"], p0["shared_bits"], p0["shared_group"],
                                    _ptr(topk_ids), _ptr(topk_w), _ptr(ws), ws.numel(), flags, _stream(stream)))


def _want(t, dtype, shape, name):
    """The C ABI cannot see dtypes or strides: check them here."""
    if t is None:
        raise MoeError(f"{name} is required")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise MoeError(f"{name}: expected a contiguous {dtype} tensor of shape {tuple(shape)}, "
                       f"got {t.dtype} {tuple(t.shape)}")


# ----------------------------------------------------------------- dense ends (include/moe_dense.h)
def moe_pack_dense_ffn(gate, up, down, bits: int) -> np.ndarray:
    """Dense MLP codes (one signed code per int8) -> the code buffer of moe_dense_ffn_forward."""
    inter = int(np.shape(gate)[0])
    g, u, d = (np.ascontiguousarray(c, dtype=np.int8) for c in (gate, up, down))
    if g.shape != (inter, HIDDEN) or u.shape != (inter, HIDDEN) or d.shape != (HIDDEN, inter):
        raise MoeError(f"dense codes: expected [inter][1280], [inter][1280], [1280][inter], "
                       f"got {g.shape} {u.shape} {d.shape}")
    L = load()
    out = np.empty(L.moe_dense_ffn_code_bytes(bits, inter), dtype=np.uint8)
    check(L.moe_pack_dense_ffn(_np_ptr(g), _np_ptr(u), _np_ptr(d), bits, inter, _np_ptr(out)))
    return out


def lm_head_to_device(head: dict, device="cuda"):
    """lm_head weights as moe_lm_head_argmax takes them (row-major, no repacking)."""
    import torch
    if head["dtype"] == "bf16":
        w = torch.from_numpy(np.ascontiguousarray(head["w"]).view(np.int16)).to(device)
        return {"w": w, "bits": MOE_HEAD_BF16, "s": None, "group": 0, "vocab": head["vocab"]}
    w = torch.from_numpy(np.ascontiguousarray(head["q"])).to(device)
    s = torch.from_numpy(np.ascontiguousarray(head["s"], dtype=np.float32)).to(device)
    return {"w": w, "bits": MOE_HEAD_INT8, "s": s, "group": head["group"], "vocab": head["vocab"]}


def dense_ffn_to_device(ffn: dict, device="cuda"):
    """Dense MLP codes (gate | up | down rows, int4 two per byte) and scales as
    moe_dense_ffn_forward takes them."""
    import torch
    b = ffn["bits"]
    codes = moe_pack_dense_ffn(ffn["gate_q"], ffn["up_q"], ffn["down_q"], b)
    scales = np.concatenate([np.asarray(ffn[k], dtype=np.float32).reshape(-1) for k in ("gate_s", "up_s", "down_s")])
    return {"q": torch.from_numpy(codes).to(device), "s": torch.from_numpy(scales).to(device),
            "bits": b, "group": ffn["group"], "inter": ffn["inter"]}


def moe_lm_head_workspace_bytes(n_tokens: int, vocab: int) -> int:
    return load().moe_lm_head_workspace_bytes(n_tokens, vocab)


def moe_lm_head_argmax(h, head: dict, token, token_logit, ws, flags: int = 0, logits=None, stream=None):
    """Enqueue lm_head + greedy token for h [T,1280] f32."""
    import torch
    T = h.shape[0]
    _want(h, torch.float32, (T, HIDDEN), "h")
    _want(token, torch.int32, (T,), "token")
    _want(token_logit, torch.float32, (T,), "token_logit")
    if logits is not None:
        _want(logits, torch.float32, (T, head["vocab"]), "logits")
    check(load().moe_lm_head_argmax(_ptr(h), h.shape[0], flags, _ptr(head["w"]), head["bits"], _ptr(head["s"]),
                                    head["group"], head["vocab"], _ptr(logits), _ptr(token), _ptr(token_logit),
                                    _ptr(ws), ws.numel(), _stream(stream)))


def moe_dense_ffn_workspace_bytes(n_tokens: int, inter: int) -> int:
    return load().moe_dense_ffn_workspace_bytes(n_tokens, inter)


def moe_dense_ffn_forward(x, dense: dict, y, ws, flags: int = 0, stream=None):
    """Enqueue the dense SwiGLU MLP for x [T,1280] f32 into y [T,1280] f32."""
    import torch
    _want(x, torch.float32, (x.shape[0], HIDDEN), "x")
    _want(y, torch.float32, (x.shape[0], HIDDEN), "y")
    check(load().moe_dense_ffn_forward(_ptr(x), x.shape[0], _ptr(dense["q"]), _ptr(dense["s"]), dense["bits"],
                                       dense["group"], dense["inter"], _ptr(y), flags, _ptr(ws), ws.numel(),
                                       _stream(stream)))


# ----------------------------------------------------------------- R-SWA decode step (include/moe_attn.h)
def rswa_to_device(d: dict, device="cuda"):
    """Inputs of one R-SWA decode step as device tensors (bf16 KV as int16 bit patterns)."""
    import torch
    out = {k: torch.from_numpy(np.ascontiguousarray(d[k])).to(device) for k in ("q", "k_new", "v_new", "n_gen")}
    for k in ("ref_k", "ref_v", "ring_k", "ring_v"):
        out[k] = torch.from_numpy(np.ascontiguousarray(d[k]).view(np.int16)).to(device)
    out["n_ref"] = d["n_ref"]
    return out


def moe_attn_block_workspace_bytes(n_streams: int, n_ref: int) -> int:
    return load().moe_attn_block_workspace_bytes(n_streams, n_ref)


def attn_weights_to_device(w_q, w_k, w_v, w_o, device="cuda"):
    """bf16 bit patterns (uint16) of the projections as moe_attn_block_forward
    takes them: W_q | W_k | W_v stacked [3840][1280], W_o [1280][1280]."""
    import torch
    qkv = np.ascontiguousarray(np.concatenate([w_q, w_k, w_v]).view(np.int16))
    return {"w_qkv": torch.from_numpy(qkv).to(device),
            "w_o": torch.from_numpy(np.ascontiguousarray(np.asarray(w_o).view(np.int16))).to(device)}


def moe_attn_block_forward(h, attn: dict, kv: dict, ws, stream=None):
    """Enqueue the attention half of a decoder layer: h [S,1280] f32 updated in
    place; kv as for moe_rswa_decode (its rings updated in place)."""
    import torch
    S, n_ref = h.shape[0], kv["n_ref"]
    _want(h, torch.float32, (S, HIDDEN), "h")
    _want(attn["w_qkv"], torch.int16, (3 * HIDDEN, HIDDEN), "w_qkv")
    _want(attn["w_o"], torch.int16, (HIDDEN, HIDDEN), "w_o")
    for k in ("ref_k", "ref_v"):
        _want(kv[k], torch.int16, (S, 10, n_ref, 128), k)
    for k in ("ring_k", "ring_v"):
        _want(kv[k], torch.int16, (S, 10, 128, 128), k)
    _want(kv["n_gen"], torch.int32, (S,), "n_gen")
    check(load().moe_attn_block_forward(S, n_ref, _ptr(h), _ptr(attn["w_qkv"]), _ptr(attn["w_o"]), _ptr(kv["ref_k"]),
                                        _ptr(kv["ref_v"]), _ptr(kv["ring_k"]), _ptr(kv["ring_v"]), _ptr(kv["n_gen"]),
                                        _ptr(ws), ws.numel(), _stream(stream)))


def moe_rswa_workspace_bytes(n_streams: int, n_ref: int) -> int:
    return load().moe_rswa_workspace_bytes(n_streams, n_ref)


def moe_rswa_decode(dev: dict, out, ws, stream=None):
    """Enqueue one R-SWA decode step (updates dev["ring_k"], dev["ring_v"] in place)."""
    import torch
    S, n_ref = dev["q"].shape[0], dev["n_ref"]
    for k in ("q", "k_new", "v_new"):
        _want(dev[k], torch.float32, (S, 10, 128), k)
    for k in ("ref_k", "ref_v"):
        _want(dev[k], torch.int16, (S, 10, n_ref, 128), k)
    for k in ("ring_k", "ring_v"):
        _want(dev[k], torch.int16, (S, 10, 128, 128), k)
    _want(dev["n_gen"], torch.int32, (S,), "n_gen")
    _want(out, torch.float32, (S, 10, 128), "out")
    check(load().moe_rswa_decode(S, dev["n_ref"], _ptr(dev["q"]), _ptr(dev["k_new"]), _ptr(dev["v_new"]),
                                 _ptr(dev["ref_k"]), _ptr(dev["ref_v"]), _ptr(dev["ring_k"]), _ptr(dev["ring_v"]),
                                 _ptr(dev["n_gen"]), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))


# ----------------------------------------------------------------- measurement
def moe_hbm_read_probe(buf, sink, stream=None):
    """Enqueue one streaming read of the device tensor `buf` (its bytes, 16-byte
    multiple); sink: a cleared int32 device tensor of one element, XORed with
    the buffer's 32-bit words."""
    import torch
    _want(sink, torch.int32, (1,), "sink")
    check(load().moe_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)))
