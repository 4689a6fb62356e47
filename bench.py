"""Benchmark: MoE-layer decode tokens/s and achieved HBM bandwidth on one MI355X.

Workload (one step = one token through the 11 chained MoE layers of the
decoder: RMSNorm, router, top-6 routed int4 G64 experts, int8 G128 fused shared
expert, weighted combine, residual add; all kernels of the library):
synthetic seeded weights and tokens, distinct token every step, R replicas of
the 11-layer weight set rotated step by step so that the 256 MiB last-level
cache cannot serve a step's weights from the previous visit.

Prints one JSON line.  The CPU baseline is the float64 oracle, timed on the
host on a bounded sample of tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer decode tokens/s + achieved HBM GB/s (% peak), int4 G=64, 1 GPU"
HBM_PEAK_GBS = 8000.0


def expert_bytes(fmt, inter):
    """Packed bytes of one expert (gate, up, down): codes plus f32 group scales,
    or, for the two-level 4-bit format (group 256), codes plus one 16-byte
    record per gate/up row and 256-column super-block, and for down one
    4-byte d/dmin word per row and super-block (the routed down rows, 896
    columns, end in a half super-block) and one 2-byte sc/m entry per row and
    32-column sub-block."""
    H = 1280
    if fmt.bits == 4 and fmt.group == 256:
        return 3 * H * inter // 2 + 16 * 2 * inter * (H // 256) + 4 * -(-inter // 256) * H + 2 * (inter // 32) * H
    return 3 * H * inter * fmt.bits // 8 + 3 * H * inter // fmt.group * 4


def layer_bytes(layer_ids, routed_fmt, shared_fmt):
    """Algorithmic bytes of one decode layer for one token: the packed codes and
    scales of the 6 picked experts, the shared expert and the router, plus the
    token's activations in and out."""
    H, I, IS, E = 1280, 896, 1792, 64
    per_expert = expert_bytes(routed_fmt, I)
    shared = expert_bytes(shared_fmt, IS)
    router = E * H * 4
    acts = H * 4 * 3 + 6 * 8  # h read, y read-modify-write, ids/w out
    return len(set(layer_ids)) * per_expert + shared + router + acts


KERNEL_SOURCES = ("quantized_expert_ffn_moe_amd/csrc/moe_kernels.hip", "quantized_expert_ffn_moe_amd/csrc/moe_internal.h")
# HBM counter summaries of the decode kernel, per routed group size
TRAFFIC_FILES = {64: os.path.join(ROOT, "profiles", "decode_chain_kernel_11layers_traffic.json"),
                 256: os.path.join(ROOT, "profiles", "decode_chain_kernel_11layers_q4k_traffic.json")}


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(group=64):
    """HBM bytes per dispatch of the decode kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (scaled by the copy-kernel calibration), or
    None when there are none for this routed format or the kernel sources have
    changed since those counters were taken."""
    if group not in TRAFFIC_FILES:
        return None
    try:
        with open(TRAFFIC_FILES[group]) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    return rec["hbm_bytes_per_dispatch"]


def cpu_baseline(layers, tokens, budget_s=20.0):
    """The oracle as it is, on the host cores, over as many tokens as fit the budget."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O
    from synth import NORM_EPS
    done, t0 = 0, time.perf_counter()
    while done < len(tokens):
        O.moe_chain(tokens[done:done + 1].astype(np.float64), layers, NORM_EPS, False)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": done / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} decode tokens through the 11 layers (float64 numpy oracle), {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--path", choices=["chain", "layers"], default="chain")
    ap.add_argument("--workload", choices=["decode", "batched32", "prefill273", "multipage2184", "batch128", "batch256",
                                           "lmhead_bf16", "lmhead_int8", "dense0", "rswa128", "ffnstack"],
                    default="decode",
                    help="decode = the headline 11-layer decode step; the prefill workloads report MFMA "
                         "figures; batchN = one continuous-batch decode step of N streams (HBM figures)")
    ap.add_argument("--group", type=int, default=64, choices=[32, 64, 128, 256],
                    help="decode: group size of the routed int4 experts (64 is the headline; 32 and 128 sweep "
                         "the group-size trade of metadata bytes against time; 256 = the two-level "
                         "Q4_K-style format); grouped workloads: 256 puts every expert in the two-level format")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU layout is a design note.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe_mib:
        # a plain copy kernel of known size: HBM counters read on it calibrate the
        # FETCH_SIZE / WRITE_SIZE figures of the MoE kernels
        n = args.copy_probe_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": args.steps}))
        return

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import WORKLOADS, make_layer, make_tokens

    if args.workload.startswith("lmhead") or args.workload == "dense0":
        return bench_dense(args)
    if args.workload == "rswa128":
        return bench_rswa(args)
    if args.workload == "ffnstack":
        return bench_ffnstack(args)
    if args.workload != "decode":
        return bench_prefill(args)

    wl = WORKLOADS[1]
    if args.group == 256:
        wl = WORKLOADS[7]      # routed experts in the two-level 4-bit format, shared int8 G128
    elif args.group != wl.routed.group:
        from dataclasses import replace
        from synth import QFmt
        wl = replace(wl, routed=QFmt(4, args.group), name=f"decode_1tok_11layers_int4g{args.group}_shared_int8g128")
    L = wl.n_layers
    layers = [make_layer(wl, li) for li in range(L)]
    base = [B.pack_layer(layer) for layer in layers]
    sets = [base]
    for _ in range(args.replicas - 1):
        sets.append([{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in p.items()} for p in base])
    n_tok = args.warmup + args.steps
    xs = np.concatenate([make_tokens(wl, batch=i)[0] for i in range(n_tok)])
    x_dev = torch.from_numpy(xs).cuda()

    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE
    h = torch.empty(1, 1280, dtype=torch.float32, device="cuda")
    ids = torch.empty(L, 1, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(L, 1, 6, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()

    if args.path == "chain":
        ws = B.decode_workspace(stream=stream)
        warr = [B.layer_weights(sset) for sset in sets]

        def step(i):
            B.moe_decode_forward(x_dev[i:i + 1], h, sets[i % args.replicas], ids, w, ws, flags,
                                 weights=warr[i % args.replicas], stream=stream)
        kernel_name = "chain_kernel (persistent decode step, one launch per token)"
    else:
        ws = B.workspace(1)

        def step(i):
            h.copy_(x_dev[i:i + 1])
            for li in range(L):
                B.moe_layer_forward(h, sets[i % args.replicas][li], h, ids[li], w[li], ws, flags, stream=stream)
        kernel_name = "per-layer kernels (router, decode items, reduce) x 11"

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.warmup, n_tok):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps

    # per-launch kernel duration: an event pair around each launch, on the launch stream
    with torch.cuda.stream(stream):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for k, i in enumerate(range(args.warmup, n_tok)):
            evs[k][0].record(stream)
            step(i)
            evs[k][1].record(stream)
        torch.cuda.synchronize()
    ms_kernel = sum(a.elapsed_time(b) for a, b in evs) / args.steps

    ids_last = ids.cpu().numpy()
    step_bytes = sum(layer_bytes(ids_last[li, 0].tolist(), wl.routed, wl.shared) for li in range(L))
    achieved = step_bytes / (ms_kernel * 1e-3) / 1e9

    out = {
        "metric": METRIC if args.group == 64 else METRIC.replace(
            "int4 G=64", "two-level 4-bit (Q4_K-style)" if args.group == 256 else f"int4 G={args.group}"),
        "value": 1000.0 / ms_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded weights and tokens)",
        "config": {"workload": wl.name, "tokens_per_step": 1, "layers": L,
                   "routed": "q4k (two-level)" if wl.routed.q4k else f"int{wl.routed.bits} g{wl.routed.group}",
                   "shared": f"int{wl.shared.bits} g{wl.shared.group}",
                   "weight_replicas": args.replicas, "path": args.path},
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counted_traffic(args.group),
                     "bytes_per_launch": step_bytes, "ms_per_launch": ms_kernel},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers, xs[: args.warmup + args.steps])
    print(json.dumps(out), flush=True)


def prefill_flops(T, ids, routed_fmt):
    """Algorithmic FLOPs of one prefill layer: 2 per multiply-add of the
    routed gate/up/down products over all (token, pick) pairs and of the shared
    expert over all tokens, plus the router."""
    H, I, IS, E = 1280, 896, 1792, 64
    return 2 * (T * 6 * 3 * H * I + T * 3 * H * IS + T * E * H)


def grouped_step_bytes(wl, ids_per_layer):
    """Algorithmic bytes of one step of a many-token workload: every routed
    expert the step touches once per layer (codes and scales), the shared
    expert and the router, plus the activations (residual in, layer output
    read-modify-write, ids and weights out)."""
    H, I, IS, E = 1280, 896, 1792, 64
    rf, sf = wl.routed, wl.shared
    per_expert = expert_bytes(rf, I)
    shared = expert_bytes(sf, IS)
    T = wl.n_tokens
    total = 0
    for ids in ids_per_layer:
        u = len(set(ids.reshape(-1).tolist()))
        total += u * per_expert + shared + E * H * 4 + T * (H * 4 * 3 + 6 * 8)
    return total


def bench_prefill(args):
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import WORKLOADS, make_layer, make_tokens

    wl = WORKLOADS[{"batched32": 2, "prefill273": 3, "multipage2184": 4, "batch128": 5, "batch256": 6}[args.workload]]
    if args.group == 256:
        # the same workload with every expert (routed and shared) in the two-level format
        from dataclasses import replace
        from synth import QFmt
        wl = replace(wl, routed=QFmt(4, 256), shared=QFmt(4, 256), name=wl.name + "_all_q4k")
    L = wl.n_layers
    layers = [make_layer(wl, li) for li in range(L)]
    packed = [B.pack_layer(layer) for layer in layers]
    T = wl.n_tokens
    x, bits = make_tokens(wl)
    if bits is not None:
        xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    else:
        xt = torch.from_numpy(x).cuda()
    h = torch.empty(T, 1280, dtype=torch.float32, device="cuda")
    ids = torch.empty(L, T, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(L, T, 6, dtype=torch.float32, device="cuda")
    ws = B.workspace(T)
    stream = torch.cuda.Stream()
    if wl.chained:
        flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE | (B.MOE_NORM_BF16 if wl.norm_bf16 else 0)

        def step(i):
            h.copy_(xt.float())
            for li in range(L):
                B.moe_layer_forward(h, packed[li], h, ids[li], w[li], ws, flags, stream=stream)
    else:
        # one layer fits the 256 MiB last-level cache: rotate weight replicas
        # so that no step finds its weights there
        packed += [B.pack_layer(layers[0]) for _ in range(3)]

        def step(i):
            B.moe_layer_forward(xt, packed[i % 4], h, ids[0], w[0], ws, 0, stream=stream)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = L * prefill_flops(T, None, wl.routed)
    tflops = flops / (ms * 1e-3) / 1e12
    out = {"metric": f"{wl.name}: tokens/s", "value": T / (ms * 1e-3), "unit": "tokens/s",
           "ms_per_step": ms, "steps": args.steps, "warmup": args.warmup, "dtype": "f16 MFMA, fp32 acc",
           "config": {"workload": wl.name, "tokens": T, "layers": L},
           "achieved_tflops": tflops, "bf16_peak_tflops": 2500.0, "mfma_frac": tflops / 2500.0}
    if args.workload.startswith("batch") or args.workload == "prefill273":
        # a decode step of many streams, 32 concurrent pages or the visual
        # prefill read the experts their tokens touch once per layer: the HBM
        # roofline bounds them
        nbytes = grouped_step_bytes(wl, list(ids[:L].cpu().numpy()))
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_step": nbytes}
    print(json.dumps(out), flush=True)


def bench_dense(args):
    """The decoder's dense ends for one decode token: lm_head (bf16 or int8 G128,
    129,280 rows) with the final norm and the greedy token, or the layer-0
    SwiGLU MLP (int8 G64, intermediate 6848) with its input norm and residual
    add.  Weight replicas rotate so that the 256 MiB last-level cache cannot
    hold a call's weights."""
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import QFmt, make_dense_ffn, make_hidden, make_lm_head

    H = 1280
    stream = torch.cuda.Stream()
    h = torch.from_numpy(make_hidden(1)).cuda()
    if args.workload.startswith("lmhead"):
        dtype = args.workload.split("_")[1]
        head = make_lm_head(dtype)
        reps = [B.lm_head_to_device(head) for _ in range(2)]
        V = head["vocab"]
        wbytes = V * H * (2 if dtype == "bf16" else 1) + (0 if dtype == "bf16" else V * (H // 128) * 4)
        nbytes = wbytes + H * 4 + 8
        tok = torch.empty(1, dtype=torch.int32, device="cuda")
        tl = torch.empty(1, dtype=torch.float32, device="cuda")
        ws = torch.empty(B.moe_lm_head_workspace_bytes(1, V), dtype=torch.uint8, device="cuda")
        name = f"lm_head_{dtype}_129280_greedy_1tok"

        def step(i):
            B.moe_lm_head_argmax(h, reps[i % len(reps)], tok, tl, ws, B.MOE_NORM_INPUT, None, stream=stream)
    else:
        ffn = make_dense_ffn(QFmt(8, 64))
        reps = [B.dense_ffn_to_device(ffn) for _ in range(12)]
        I = ffn["inter"]
        nbytes = 3 * I * H + 3 * I * (H // 64) * 4 + H * 4 * 3
        ws = torch.empty(B.moe_dense_ffn_workspace_bytes(1, I), dtype=torch.uint8, device="cuda")
        name = "dense_layer0_swiglu_int8g64_6848_1tok"

        def step(i):
            B.moe_dense_ffn_forward(h, reps[i % len(reps)], h, ws, B.MOE_NORM_INPUT | B.MOE_ACCUMULATE,
                                    stream=stream)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    print(json.dumps({"metric": f"{name}: calls/s", "value": 1e3 / ms, "unit": "calls/s", "ms_per_step": ms,
                      "steps": args.steps, "warmup": args.warmup, "dtype": "f32 FMA on decoded weights",
                      "config": {"workload": name, "tokens": 1},
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_call": nbytes}}),
          flush=True)


def bench_ffnstack(args):
    """One decode token through the decoder's FFN stack and head: the layer-0
    dense MLP (int8 G64, residual in place), the 11 MoE layers in one
    persistent launch, the final norm + lm_head (bf16) + greedy token; weight
    replicas rotated.  Attention is not part of it."""
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import QFmt, WORKLOADS, make_dense_ffn, make_hidden, make_layer, make_lm_head

    wl = WORKLOADS[1]
    L = wl.n_layers
    H = 1280
    R = 2
    layers = [make_layer(wl, li) for li in range(L)]
    moe_sets = [[B.pack_layer(layer) for layer in layers] for _ in range(R)]
    warr = [B.layer_weights(ms) for ms in moe_sets]
    ffn = make_dense_ffn(QFmt(8, 64))
    dense_sets = [B.dense_ffn_to_device(ffn) for _ in range(R)]
    head = make_lm_head("bf16")
    head_sets = [B.lm_head_to_device(head) for _ in range(R)]
    stream = torch.cuda.Stream()
    xs = torch.from_numpy(make_hidden(args.warmup + args.steps)).cuda()
    h = torch.empty(1, H, dtype=torch.float32, device="cuda")
    y = torch.empty(1, H, dtype=torch.float32, device="cuda")
    ids = torch.empty(L, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(L, 6, dtype=torch.float32, device="cuda")
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    tl = torch.empty(1, dtype=torch.float32, device="cuda")
    ws_d = torch.empty(B.moe_dense_ffn_workspace_bytes(1, ffn["inter"]), dtype=torch.uint8, device="cuda")
    ws_m = B.decode_workspace(stream=stream)
    ws_h = torch.empty(B.moe_lm_head_workspace_bytes(1, head["vocab"]), dtype=torch.uint8, device="cuda")
    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE

    def step(i):
        r = i % R
        h.copy_(xs[i:i + 1])
        B.moe_dense_ffn_forward(h, dense_sets[r], h, ws_d, flags, stream=stream)
        B.moe_decode_forward(h, y, moe_sets[r], ids, w, ws_m, flags, weights=warr[r], stream=stream)
        B.moe_lm_head_argmax(y, head_sets[r], tok, tl, ws_h, B.MOE_NORM_INPUT, None, stream=stream)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.warmup, args.warmup + args.steps):
            step(i)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ids_last = ids.cpu().numpy()
    moe_bytes = sum(layer_bytes(ids_last[li].tolist(), wl.routed, wl.shared) for li in range(L))
    dense_bytes = 3 * ffn["inter"] * H + 3 * ffn["inter"] * (H // 64) * 4 + H * 4 * 3
    head_bytes = head["vocab"] * H * 2 + H * 4 + 8
    nbytes = moe_bytes + dense_bytes + head_bytes
    gbs = nbytes / (ms * 1e-3) / 1e9
    name = "decoder_ffn_stack_dense0_11moe_lmhead_bf16_1tok"
    print(json.dumps({"metric": f"{name}: tokens/s", "value": 1e3 / ms, "unit": "tokens/s", "ms_per_step": ms,
                      "steps": args.steps, "warmup": args.warmup, "dtype": "f32",
                      "config": {"workload": name, "tokens": 1, "moe_layers": L},
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_step": nbytes}}),
          flush=True)


def bench_rswa(args):
    """One R-SWA attention decode step of 128 streams (reference block 288 =
    the 273-row visual prefill plus a 15-token prompt, ring full), three KV
    replicas rotated so that the last-level cache cannot hold a step's KV."""
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import make_rswa

    S, n_ref = 128, 288
    reps = [B.rswa_to_device(make_rswa(S, n_ref, n_gen=[127 + 37 * s for s in range(S)], seed=r)) for r in range(3)]
    out = torch.empty(S, 10, 128, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.moe_rswa_workspace_bytes(S, n_ref), dtype=torch.uint8, device="cuda")
    kv = S * 10 * (n_ref + 128) * 128 * 2 * 2
    nbytes = kv + S * 10 * 128 * 4 * 4 + S * 10 * 128 * 2 * 2 + S * 4
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            B.moe_rswa_decode(reps[i % 3], out, ws, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            B.moe_rswa_decode(reps[i % 3], out, ws, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    name = "rswa_decode_128streams_ref288_ring128"
    print(json.dumps({"metric": f"{name}: tokens/s", "value": S / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
                      "steps": args.steps, "warmup": args.warmup, "dtype": "f32 on bf16 KV",
                      "config": {"workload": name, "streams": S, "n_ref": n_ref},
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_step": nbytes}}),
          flush=True)


if __name__ == "__main__":
    main()
