"""Benchmark: MoE-layer decode tokens/s and achieved HBM bandwidth on one MI355X.

Workload (one step = one token through the 11 chained MoE layers of the
decoder: RMSNorm, router, top-6 routed int4 G64 experts, int8 G128 fused shared
expert, weighted combine, residual add; all kernels of the library):
synthetic seeded weights and tokens, distinct token every step, R replicas of
the 11-layer weight set rotated step by step so that the 256 MiB last-level
cache cannot serve a step's weights from the previous visit.

Every leg keeps the outputs of its timed calls.  After timing, the float64
oracle runs on the host cores over a bounded sample of the same tokens: its
time is the CPU baseline, and its outputs check the GPU's outputs of those
tokens (the same-run parity gate).  A leg whose gate fails, or whose decode
kernel reports a wait that gave up, prints no result and exits with status 3.

Prints one JSON line.
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
MFMA_F16_PEAK_TFLOPS = 2500.0
BUDGET_S = 20.0          # host seconds of oracle work per leg (baseline + gate)
DTYPE_DECODE = "i8 MFMA on 3 digit planes of 22-bit block-float activations x exact codes, f32 acc"
DTYPE_GROUPED = "f16 MFMA (exact codes; f32 inputs as f16 hi/lo pairs), f32 acc"


class GateError(Exception):
    pass


def gate_exit(leg: str, msg: str):
    print(f"bench.py [{leg}]: no result: {msg}", file=sys.stderr, flush=True)
    sys.exit(3)


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


def host_threads():
    from threadpoolctl import threadpool_info
    return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])


# ----------------------------------------------------------------------------
# the oracle leg: CPU baseline and same-run parity gate
# ----------------------------------------------------------------------------
def moe_oracle_leg(layers, x64, rows, gpu_ids, gpu_w, gpu_out, *, chained, norm_bf16, block, what,
                   budget_s=BUDGET_S):
    """The float64 oracle on the host cores over the tokens ``rows`` of the
    timed GPU work, ``block`` tokens per oracle call, until ``budget_s`` is
    spent (at least one block):

    * its time is the CPU baseline (the oracle as it stands);
    * its outputs gate the GPU's outputs of the same tokens: per layer the
      GPU's ids and weights must be a valid greedy top-6 of the oracle's
      probabilities (ids exact wherever the gaps exceed 1e-6, weights within
      1e-5 relative), and the output within 1e-3 x rms of the oracle's (for a
      chain, of what the layers add to the residual).  Where a near-tie routed
      a token differently, the oracle is re-run (untimed) with the GPU's ids.

    x64 [T,1280] f64 inputs; gpu_ids, gpu_w: [L][T,6]; gpu_out [T,1280] (the
    residual after the last layer for a chain, y for one layer).
    Returns (baseline dict, gate dict); raises GateError on a mismatch."""
    import numpy as np

    from oracle import moe_oracle as O
    from synth import NORM_EPS
    from tests.parity import check_routing

    def run(x, forced=None):
        if chained:
            return O.moe_chain(x, layers, NORM_EPS, norm_bf16, forced_ids=forced)
        ids, w, y, _ = O.moe_layer(x, layers[0], forced_ids=None if forced is None else forced[0])
        return y, [(ids, w, x)]

    L = len(layers)
    used, done, near = 0.0, [], 0
    errs, refs = [], []
    for b0 in range(0, len(rows), block):
        r = np.asarray(rows[b0:b0 + block])
        t0 = time.perf_counter()
        out_o, trace = run(x64[r])
        used += time.perf_counter() - t0
        done.extend(r.tolist())
        gi = [np.asarray(gpu_ids[li])[r] for li in range(L)]
        if not all(np.array_equal(trace[li][0], gi[li]) for li in range(L)):
            out_o, trace = run(x64[r], forced=gi)
        try:
            for li in range(L):
                lay = layers[li]
                P = O.softmax(O.router_logits(trace[li][2], lay["router_w"], lay.get("router_b")))
                near += check_routing(gi[li], np.asarray(gpu_w[li])[r], P)
        except AssertionError as e:
            raise GateError(f"{what}: routing differs from the oracle's on tokens {r[:8].tolist()}: {e}")
        base = x64[r] if chained else 0.0
        refs.append(out_o - base)
        errs.append(np.asarray(gpu_out, np.float64)[r] - base - (out_o - base))
        if used > budget_s:
            break
    ref = np.concatenate(refs)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    ratio = float(np.abs(np.concatenate(errs)).max() / rms)
    if not ratio <= 1e-3:
        raise GateError(f"{what}: max|err| / rms = {ratio:.3e} > 1e-3 over {len(done)} tokens")
    base = {"value": len(done) / used, "unit": "tokens/s", "cores": host_threads(), "kind": "oracle",
            "sample": f"{len(done)} of the timed tokens through {L} layer{'s' if L > 1 else ''} "
                      f"(float64 numpy oracle, {block} token{'s' if block > 1 else ''} per call), {used:.1f} s"}
    gate = {"tokens": len(done), "layers": L, "max_err_over_rms": ratio, "near_ties": int(near),
            "bar": "ids exact where gaps > 1e-6, w rtol 1e-5, max|err| <= 1e-3 rms"}
    return base, gate


def decode_prefix_gate(x_tok, xt, layers, sset, warr, ids_t, w_t, y_t, flags, ws, stream, chained):
    """Per-layer check of one timed decode token: the same launch with 1..L
    layers on the same weights and workspace.  The L-layer launch must repeat
    the timed launch's outputs bit for bit; each layer's output, given the
    GPU's residual before it, must match the oracle's layer to 1e-3 x rms."""
    import numpy as np
    import torch

    from oracle import moe_oracle as O
    from quantized_expert_ffn_moe_amd import binding as B
    from synth import NORM_EPS
    from tests.parity import check_layer

    L = len(layers)
    h_prev = x_tok.astype(np.float64)
    worst = 0.0
    for n in range(1, L + 1):
        y = torch.empty(1, 1280, dtype=torch.float32, device="cuda")
        ids = torch.empty(n, 6, dtype=torch.int32, device="cuda")
        w = torch.empty(n, 6, dtype=torch.float32, device="cuda")
        with torch.cuda.stream(stream):
            B.moe_decode_forward(xt, y, sset[:n], ids, w, ws, flags, weights=warr if n == L else None,
                                 stream=stream)
        torch.cuda.synchronize()
        yn, idn, wn = y.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
        if n == L:
            if not (np.array_equal(yn, y_t) and np.array_equal(idn, ids_t) and np.array_equal(wn, w_t)):
                raise GateError("the repeated decode launch differs from the timed launch")
        z = O.rmsnorm(h_prev, NORM_EPS) if chained else h_prev
        try:
            r, _ = check_layer(z, layers[n - 1], idn[-1:], wn[-1:], yn - (h_prev if chained else 0.0))
        except AssertionError as e:
            raise GateError(f"decode layer {n}: {e}")
        worst = max(worst, r)
        h_prev = yn.astype(np.float64)
    return worst


def check_error_word(ws, leg):
    err = int(ws[8:12].view(__import__("torch").int32).item())
    if err != 0:
        gate_exit(leg, f"a bounded wait inside the decode kernel gave up (error word {err:#x}); results invalid")


# ----------------------------------------------------------------------------
# headline: the decode step (and the one-layer int8 decode of the first config)
# ----------------------------------------------------------------------------
def bench_decode(args):
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import WORKLOADS, make_layer, make_tokens

    one_layer = args.workload == "decode1"
    if one_layer:
        wl = WORKLOADS[0]      # one layer, one token, int8 G128 routed and shared, no norm, no residual
    else:
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
    # one layer (28.7 MB) would sit in the 256 MiB last-level cache: rotate enough replicas
    R = args.replicas if not one_layer else max(args.replicas, 16)
    sets = [base]
    for _ in range(R - 1):
        sets.append([{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in p.items()} for p in base])
    n_tok = args.warmup + args.steps
    xs = np.concatenate([make_tokens(wl, batch=i)[0] for i in range(n_tok)])
    x_dev = torch.from_numpy(xs).cuda()

    flags = 0 if one_layer else B.MOE_NORM_INPUT | B.MOE_ACCUMULATE
    y_all = torch.empty(n_tok, 1280, dtype=torch.float32, device="cuda")
    ids_all = torch.empty(n_tok, L, 6, dtype=torch.int32, device="cuda")
    w_all = torch.empty(n_tok, L, 6, dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    ws = B.decode_workspace(stream=stream)
    warr = [B.layer_weights(sset) for sset in sets]

    def step(i):
        B.moe_decode_forward(x_dev[i:i + 1], y_all[i:i + 1], sets[i % R], ids_all[i], w_all[i], ws, flags,
                             weights=warr[i % R], stream=stream)
    kernel_name = "chain_kernel (persistent decode step, one launch per token)"

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
    y_timed = y_all.cpu().numpy()
    ids_timed = ids_all.cpu().numpy()
    w_timed = w_all.cpu().numpy()

    # the step is one kernel launch, so the timed region's average (events on
    # the launch stream around all K launches, divided by K) is the average
    # launch duration, back-to-back dispatch gap included.  An event pair
    # around each launch, reported beside it, also counts the events' own
    # processing and overstates the kernel.
    ms_kernel = ms_step
    with torch.cuda.stream(stream):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for k, i in enumerate(range(args.warmup, n_tok)):
            evs[k][0].record(stream)
            step(i)
            evs[k][1].record(stream)
        torch.cuda.synchronize()
    pair_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_isolated = float(pair_ms.mean())
    pair_pct = [float(v) for v in np.percentile(pair_ms, [10, 50, 90])]
    leg = wl.name
    check_error_word(ws, leg)
    # every launch is deterministic: the second pass must reproduce the first
    if not (np.array_equal(y_all.cpu().numpy(), y_timed) and np.array_equal(ids_all.cpu().numpy(), ids_timed)):
        gate_exit(leg, "two passes over the same tokens gave different outputs")

    step_bytes = np.mean([sum(layer_bytes(ids_timed[i, li].tolist(), wl.routed, wl.shared) for li in range(L))
                          for i in range(args.warmup, n_tok)])
    practical = practical_read_gbs(stream)
    achieved = step_bytes / (ms_kernel * 1e-3) / 1e9

    # same-run parity gate and CPU baseline on the timed tokens
    timed = list(range(args.warmup, n_tok))
    try:
        worst = decode_prefix_gate(xs[timed[0]:timed[0] + 1], x_dev[timed[0]:timed[0] + 1], layers,
                                   sets[timed[0] % R], warr[timed[0] % R], ids_timed[timed[0]], w_timed[timed[0]],
                                   y_timed[timed[0]:timed[0] + 1], flags, ws, stream, not one_layer)
        check_error_word(ws, leg)
        cpu, gate = moe_oracle_leg(layers, xs.astype(np.float64), timed,
                                   [ids_timed[:, li] for li in range(L)], [w_timed[:, li] for li in range(L)],
                                   y_timed, chained=not one_layer, norm_bf16=False, block=1, what=leg,
                                   budget_s=0.0 if args.no_cpu_baseline else BUDGET_S)
    except GateError as e:
        gate_exit(leg, str(e))
    gate["per_layer_worst_err_over_rms"] = worst

    if one_layer:
        metric = "MoE-layer decode tokens/s + achieved HBM GB/s (% peak), int8 G=128, 1 layer, 1 GPU"
    elif args.group == 64:
        metric = METRIC
    else:
        metric = METRIC.replace("int4 G=64", "two-level 4-bit (Q4_K-style)" if args.group == 256
                                else f"int4 G={args.group}")
    out = {
        "metric": metric,
        "value": 1000.0 / ms_step,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_DECODE,
        "data": "synthetic (seeded weights and tokens)",
        "config": {"workload": wl.name, "tokens_per_step": 1, "layers": L,
                   "routed": "q4k (two-level)" if wl.routed.q4k else f"int{wl.routed.bits} g{wl.routed.group}",
                   "shared": f"int{wl.shared.bits} g{wl.shared.group}",
                   "weight_replicas": R, "path": "chain"},
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counted_traffic(args.group) if not one_layer else None,
                     "bytes_per_launch": step_bytes, "ms_per_launch": ms_kernel,
                     "ms_per_launch_event_pair": ms_isolated,
                     "ms_per_launch_event_pair_p10_p50_p90": pair_pct,
                     "practical_read_gbs": practical, "frac_of_practical": achieved / practical},
        "parity_gate": gate,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------------------
# grouped-path workloads
# ----------------------------------------------------------------------------
def prefill_flops(T):
    """Algorithmic FLOPs of one layer over T tokens: 2 per multiply-add of the
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


def chain_gate(args, wl, layers, packed, xt, ws, stream, h_last, ids_last, w_last, rows):
    """Gate and CPU baseline of a chained many-token step, layer by layer on the
    GPU's own residual stream (a bf16-rounded layer input turns tiny residual
    differences into whole bf16 steps, so the chain is compared teacher-forced,
    as the GPU tests do): the step is run once more keeping every layer's
    residual, which must reproduce the timed step bit for bit; then, on sampled
    tokens, each layer's ids, weights and output against the oracle at the
    input the GPU used (the GPU's RMSNorm of its residual).  The oracle's time
    over the sample (all layers) is the baseline."""
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import NORM_EPS

    L, T = wl.n_layers, wl.n_tokens
    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE | (B.MOE_NORM_BF16 if wl.norm_bf16 else 0)
    h = xt.float().contiguous()
    hs = [h.clone()]
    ids = torch.empty(L, T, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(L, T, 6, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(stream):
        for li in range(L):
            B.moe_layer_forward(h, packed[li], h, ids[li], w[li], ws, flags, stream=stream)
            hs.append(h.clone())
    torch.cuda.synchronize()
    if not (np.array_equal(hs[-1].cpu().numpy(), h_last) and np.array_equal(ids.cpu().numpy(), ids_last[:L])):
        raise GateError("the repeated step differs from the timed step")
    sample = np.sort(rows[:(4 if args.no_cpu_baseline else min(T, 64))])
    zdt = torch.bfloat16 if wl.norm_bf16 else torch.float32
    used, worst, near = 0.0, 0.0, 0
    for li in range(L):
        z = torch.empty(len(sample), 1280, dtype=zdt, device="cuda")
        B.moe_rmsnorm(hs[li][sample].contiguous(), z, NORM_EPS)
        zin = z.float().cpu().numpy().astype(np.float64)
        out = (hs[li + 1][sample] - hs[li][sample]).cpu().numpy()
        x64 = np.zeros((T, 1280)); x64[sample] = zin
        y64 = np.zeros((T, 1280), np.float32); y64[sample] = out
        cpu, g = moe_oracle_leg([layers[li]], x64, sample, [ids_last[li]], [w_last[li]], y64, chained=False,
                                norm_bf16=False, block=len(sample), what=f"{wl.name} layer {li + 1}")
        used += len(sample) / cpu["value"]
        worst = max(worst, g["max_err_over_rms"])
        near += g["near_ties"]
    base = {"value": len(sample) / used, "unit": "tokens/s", "cores": host_threads(), "kind": "oracle",
            "sample": f"{len(sample)} of the timed tokens through the {L} layers, each layer on the GPU's own "
                      f"residual (float64 numpy oracle), {used:.1f} s"}
    gate = {"tokens": len(sample), "layers": L, "max_err_over_rms": worst, "near_ties": near,
            "bar": "per layer on the GPU's residual: ids exact where gaps > 1e-6, w rtol 1e-5, max|err| <= 1e-3 rms",
            "repeat_bitwise": True}
    return base, gate


def bench_grouped(args):
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
    # the outputs of the last timed step (every step computes the same values)
    h_last = h.cpu().numpy()
    ids_last = ids.cpu().numpy()
    w_last = w.cpu().numpy()

    flops = L * prefill_flops(T)
    tflops = flops / (ms * 1e-3) / 1e12
    rows = np.random.default_rng(T).permutation(T)
    try:
        if wl.chained:
            cpu, gate = chain_gate(args, wl, layers, packed, xt, ws, stream, h_last, ids_last, w_last, rows)
        else:
            cpu, gate = moe_oracle_leg(layers, x.astype(np.float64), rows, [ids_last[0]], [w_last[0]], h_last,
                                       chained=False, norm_bf16=False, block=T if T <= 300 else 8, what=wl.name,
                                       budget_s=0.0 if args.no_cpu_baseline else BUDGET_S)
    except GateError as e:
        gate_exit(wl.name, str(e))
    out = {"metric": f"{wl.name}: tokens/s", "value": T / (ms * 1e-3), "unit": "tokens/s",
           "ms_per_step": ms, "steps": args.steps, "warmup": args.warmup, "dtype": DTYPE_GROUPED,
           "data": "synthetic (seeded weights and tokens)",
           "config": {"workload": wl.name, "tokens": T, "layers": L},
           "achieved_tflops": tflops, "f16_mfma_peak_tflops": MFMA_F16_PEAK_TFLOPS,
           "mfma_frac": tflops / MFMA_F16_PEAK_TFLOPS, "parity_gate": gate}
    if args.workload == "multipage2184":
        out["roofline"] = {"bound": "mfma", "achieved": tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": tflops / MFMA_F16_PEAK_TFLOPS, "traffic": None, "flops_per_step": flops}
    else:
        # a decode step of many streams, 32 concurrent pages or the visual
        # prefill read the experts their tokens touch once per layer: the HBM
        # roofline bounds them
        nbytes = grouped_step_bytes(wl, list(ids_last[:L]))
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_step": nbytes}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu
    print(json.dumps(add_practical(out)), flush=True)


# ----------------------------------------------------------------------------
# the decoder's dense ends, the R-SWA step and the FFN stack
# ----------------------------------------------------------------------------
def practical_read_gbs(stream, mib=1024, reps=20):
    """The device's practical streaming-read rate in GB/s: the library's
    read probe over a 1 GiB buffer (four times the last-level cache), events
    on the launch stream around `reps` reads after 3 untimed ones."""
    import torch
    from quantized_expert_ffn_moe_amd import binding as B
    buf = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    buf.fill_(0x5A)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(3):
            B.moe_hbm_read_probe(buf, sink, stream=stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            B.moe_hbm_read_probe(buf, sink, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    return (mib << 20) / (ms * 1e-3) / 1e9


def add_practical(out):
    """An HBM-bound line also carries the practical read rate measured in the
    same run, and its achieved bandwidth as a fraction of it."""
    import torch
    r = out.get("roofline")
    if r and r.get("bound") == "hbm":
        p = practical_read_gbs(torch.cuda.current_stream())
        r["practical_read_gbs"] = p
        r["frac_of_practical"] = r["achieved"] / p
    return out


def timed_loop(step, stream, warmup, steps, first=0):
    import torch
    with torch.cuda.stream(stream):
        for i in range(warmup):
            step(first + i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(steps):
            step(first + warmup + i)
        e1.record(stream)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def head_gate(ref_logits, tok, tl):
    """The greedy token equals the oracle's wherever its best logit leads the
    runner-up by more than 1e-3 x rms(logits), else its oracle logit is within
    that of the best; the token's logit within the same bound."""
    import numpy as np
    from oracle import dense_head as D
    tol = 1e-3 * np.sqrt(np.mean(ref_logits ** 2))
    rid, rv = D.greedy_token(ref_logits)
    for t in range(ref_logits.shape[0]):
        second = np.partition(ref_logits[t], -2)[-2]
        if rv[t] - second > tol and tok[t] != rid[t]:
            raise GateError(f"token {t}: greedy id {tok[t]} != oracle {rid[t]}")
        if ref_logits[t, tok[t]] < rv[t] - tol or abs(tl[t] - ref_logits[t, tok[t]]) > tol:
            raise GateError(f"token {t}: logit {tl[t]} vs oracle {ref_logits[t, tok[t]]} (best {rv[t]})")
    return float(np.max(np.abs(np.asarray(tl, np.float64) - ref_logits[np.arange(len(tok)), tok])) / tol * 1e-3)


def bench_dense(args):
    """The decoder's dense ends for one decode token: lm_head (bf16 or int8 G128,
    129,280 rows) with the final norm and the greedy token, or the layer-0
    SwiGLU MLP (int8 G64, intermediate 6848) with its input norm and residual
    add.  Weight replicas rotate so that the 256 MiB last-level cache cannot
    hold a call's weights."""
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import NORM_EPS, QFmt, make_dense_ffn, make_hidden, make_lm_head

    H = 1280
    stream = torch.cuda.Stream()
    x0 = make_hidden(1)
    h = torch.from_numpy(x0).cuda()
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
    ms = timed_loop(step, stream, args.warmup, args.steps)
    gbs = nbytes / (ms * 1e-3) / 1e9

    # gate and baseline: the lm_head's input never changes, so the last timed
    # call's token is checked; the dense MLP updates its input in place, so the
    # same call is made once more from a saved input
    from oracle import dense_head as D
    try:
        if args.workload.startswith("lmhead"):
            tok_n, tl_n = tok.cpu().numpy(), tl.cpu().numpy()
            t0 = time.perf_counter()
            W = D.bf16_bits_value(head["w"]) if dtype == "bf16" else D.dequantize(head["q"], head["s"], head["group"])
            ref = D.lm_head_logits(x0.astype(np.float64), W, True, NORM_EPS)
            used = time.perf_counter() - t0
            err = head_gate(ref, tok_n, tl_n)
            gate = {"tokens": 1, "token": int(tok_n[0]), "logit_err_over_rms": err,
                    "bar": "greedy id exact unless a near tie; logit within 1e-3 rms"}
        else:
            hin = h.clone()
            with torch.cuda.stream(stream):
                step(0)
            torch.cuda.synchronize()
            xin = hin.cpu().numpy().astype(np.float64)
            t0 = time.perf_counter()
            ref = D.dense_ffn(xin, ffn, True, NORM_EPS)
            used = time.perf_counter() - t0
            got = h.cpu().numpy().astype(np.float64) - xin
            err = float(np.abs(got - ref).max() / np.sqrt(np.mean(ref ** 2)))
            if not err <= 1e-3:
                raise GateError(f"dense MLP max|err|/rms {err:.3e}")
            gate = {"tokens": 1, "max_err_over_rms": err, "bar": "max|err| <= 1e-3 rms"}
    except GateError as e:
        gate_exit(name, str(e))
    out = {"metric": f"{name}: calls/s", "value": 1e3 / ms, "unit": "calls/s", "ms_per_step": ms,
           "steps": args.steps, "warmup": args.warmup, "dtype": "f32 FMA on decoded weights",
           "data": "synthetic (seeded weights and rows)",
           "config": {"workload": name, "tokens": 1},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_call": nbytes},
           "parity_gate": gate}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = {"value": 1.0 / used, "unit": "calls/s", "cores": host_threads(), "kind": "oracle",
                               "sample": f"one call (float64 numpy oracle, dequantisation included), {used:.1f} s"}
    print(json.dumps(add_practical(out)), flush=True)


def bench_ffnstack(args):
    """One decode token through the decoder's FFN stack and head: the layer-0
    dense MLP (int8 G64, residual in place), the 11 MoE layers in one
    persistent launch, the final norm + lm_head (bf16) + greedy token; weight
    replicas rotated.  Attention is not part of it."""
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import NORM_EPS, QFmt, WORKLOADS, make_dense_ffn, make_hidden, make_layer, make_lm_head

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
    x_host = make_hidden(args.warmup + args.steps)
    xs = torch.from_numpy(x_host).cuda()
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
    ms = timed_loop(step, stream, args.warmup, args.steps)
    name = "decoder_ffn_stack_dense0_11moe_lmhead_bf16_1tok"
    check_error_word(ws_m, name)
    ids_last = ids.cpu().numpy()
    w_last = w.cpu().numpy()
    h1, y_last, tok_n, tl_n = h.cpu().numpy(), y.cpu().numpy(), tok.cpu().numpy(), tl.cpu().numpy()
    moe_bytes = sum(layer_bytes(ids_last[li].tolist(), wl.routed, wl.shared) for li in range(L))
    dense_bytes = 3 * ffn["inter"] * H + 3 * ffn["inter"] * (H // 64) * 4 + H * 4 * 3
    head_bytes = head["vocab"] * H * 2 + H * 4 + 8
    nbytes = moe_bytes + dense_bytes + head_bytes
    gbs = nbytes / (ms * 1e-3) / 1e9

    # gate and baseline on the last timed token: dense layer, the 11 MoE layers
    # from the GPU's dense output, the head on the GPU's final residual
    from oracle import dense_head as D
    try:
        x_last = x_host[-1:].astype(np.float64)
        t0 = time.perf_counter()
        ref_d = D.dense_ffn(x_last, ffn, True, NORM_EPS)
        used = time.perf_counter() - t0
        err_d = float(np.abs(h1 - x_last - ref_d).max() / np.sqrt(np.mean(ref_d ** 2)))
        if not err_d <= 1e-3:
            raise GateError(f"dense layer max|err|/rms {err_d:.3e}")
        t1 = time.perf_counter()
        _, gate = moe_oracle_leg(layers, h1.astype(np.float64), [0], [ids_last[li][None] for li in range(L)],
                                 [w_last[li][None] for li in range(L)], y_last, chained=True, norm_bf16=False,
                                 block=1, what=name)
        W = D.bf16_bits_value(head["w"])
        ref_h = D.lm_head_logits(y_last.astype(np.float64), W, True, NORM_EPS)
        used += time.perf_counter() - t1
        head_gate(ref_h, tok_n, tl_n)
    except GateError as e:
        gate_exit(name, str(e))
    gate.update(dense_err_over_rms=err_d, token=int(tok_n[0]))
    out = {"metric": f"{name}: tokens/s", "value": 1e3 / ms, "unit": "tokens/s", "ms_per_step": ms,
           "steps": args.steps, "warmup": args.warmup, "dtype": DTYPE_DECODE + " (MoE); f32 FMA (dense ends)",
           "data": "synthetic (seeded weights and rows)",
           "config": {"workload": name, "tokens": 1, "moe_layers": L},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_step": nbytes},
           "parity_gate": gate}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = {"value": 1.0 / used, "unit": "tokens/s", "cores": host_threads(), "kind": "oracle",
                               "sample": f"the last timed token (float64 numpy oracle: dense MLP, 11 MoE layers, "
                                         f"lm_head), {used:.1f} s"}
    print(json.dumps(add_practical(out)), flush=True)


def bench_rswa(args):
    """One R-SWA attention decode step of 128 streams (reference block 288 =
    the 273-row visual prefill plus a 15-token prompt, ring full), three KV
    replicas rotated so that the last-level cache cannot hold a step's KV."""
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import make_rswa

    S, n_ref = 128, 288
    n_gen = [127 + 37 * s for s in range(S)]
    reps = [B.rswa_to_device(make_rswa(S, n_ref, n_gen=n_gen, seed=r)) for r in range(3)]
    out_t = torch.empty(S, 10, 128, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.moe_rswa_workspace_bytes(S, n_ref), dtype=torch.uint8, device="cuda")
    kv = S * 10 * (n_ref + 128) * 128 * 2 * 2
    nbytes = kv + S * 10 * 128 * 4 * 4 + S * 10 * 128 * 2 * 2 + S * 4
    stream = torch.cuda.Stream()
    ms = timed_loop(lambda i: B.moe_rswa_decode(reps[i % 3], out_t, ws, stream=stream), stream,
                    args.warmup, args.steps)
    gbs = nbytes / (ms * 1e-3) / 1e9
    name = "rswa_decode_128streams_ref288_ring128"

    # gate and baseline: the timed steps advanced the rings in place, so the
    # step is made once more on fresh inputs and checked on sampled streams
    from oracle import rswa as RO
    from synth import bf16_bits_to_f32
    d = make_rswa(S, n_ref, n_gen=n_gen, seed=0)
    dev = B.rswa_to_device(d)
    with torch.cuda.stream(stream):
        B.moe_rswa_decode(dev, out_t, ws, stream=stream)
    torch.cuda.synchronize()
    got = out_t.cpu().numpy()
    sample = np.random.default_rng(S).permutation(S)
    used, done, worst = 0.0, 0, 0.0
    for s in sample:
        t0 = time.perf_counter()
        ref, _, _ = RO.rswa_decode(d["q"][s], d["k_new"][s], d["v_new"][s], bf16_bits_to_f32(d["ref_k"][s]),
                                   bf16_bits_to_f32(d["ref_v"][s]), bf16_bits_to_f32(d["ring_k"][s]),
                                   bf16_bits_to_f32(d["ring_v"][s]), int(d["n_gen"][s]))
        used += time.perf_counter() - t0
        done += 1
        worst = max(worst, float(np.abs(got[s] - ref).max() / np.sqrt(np.mean(ref ** 2))))
        if used > (0.0 if args.no_cpu_baseline else BUDGET_S / 4) or done >= 32:
            break
    if not worst <= 1e-3:
        gate_exit(name, f"R-SWA output max|err|/rms {worst:.3e} on {done} streams")
    out = {"metric": f"{name}: tokens/s", "value": S / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
           "steps": args.steps, "warmup": args.warmup, "dtype": "f32 on bf16 KV",
           "data": "synthetic (seeded q, k, v and KV)",
           "config": {"workload": name, "streams": S, "n_ref": n_ref},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_step": nbytes},
           "parity_gate": {"streams": done, "max_err_over_rms": worst, "bar": "max|err| <= 1e-3 rms per stream"}}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = {"value": done / used, "unit": "tokens/s", "cores": host_threads(), "kind": "oracle",
                               "sample": f"{done} of the 128 streams (float64 numpy oracle), {used:.1f} s"}
    print(json.dumps(add_practical(out)), flush=True)


def bench_layer(args):
    """One whole decoder layer step: the attention half (RMSNorm, q/k/v
    projections, R-SWA over a 288-row reference block and the 128-slot ring, o
    projection and residual) and the MoE half (int4 G64 routed, int8 G128
    shared; the persistent decode step for one token, moe_layer_forward for
    128 streams).  Weight and KV replicas rotate so that the last-level cache
    cannot hold a step's bytes; the rings advance in place every step."""
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import (NORM_EPS, WORKLOADS, bf16_bits_to_f32, make_attn_weights, make_hidden, make_layer,
                       make_rswa)

    S = 1 if args.workload == "layer1" else 128
    n_ref, H = 288, 1280
    wl = WORKLOADS[1] if S == 1 else WORKLOADS[5]
    R = 8 if S == 1 else 2
    layer = make_layer(wl, 0)
    aw = make_attn_weights(0)
    attn = [B.attn_weights_to_device(**aw) for _ in range(R)]
    moe = [B.pack_layer(layer) for _ in range(R)]
    n_gen = [127 + 37 * s for s in range(S)]
    kvs = [B.rswa_to_device(make_rswa(S, n_ref, n_gen=n_gen, seed=r)) for r in range(R)]
    xs = torch.from_numpy(make_hidden(S * (args.warmup + args.steps + 1), batch=500)).cuda()
    h = torch.empty(S, H, dtype=torch.float32, device="cuda")
    ids = torch.empty(S, 6, dtype=torch.int32, device="cuda")
    w = torch.empty(S, 6, dtype=torch.float32, device="cuda")
    y = torch.empty(S, H, dtype=torch.float32, device="cuda")
    ws_a = torch.empty(B.moe_attn_block_workspace_bytes(S, n_ref), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    ws_m = B.decode_workspace(stream=stream) if S == 1 else B.workspace(S)
    flags = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE
    warr = [B.layer_weights([m]) for m in moe]

    def step(i):
        r = i % R
        h.copy_(xs[S * i:S * i + S])
        B.moe_attn_block_forward(h, attn[r], kvs[r], ws_a, stream=stream)
        if S == 1:
            B.moe_decode_forward(h, y, [moe[r]], ids, w, ws_m, flags, weights=warr[r], stream=stream)
        else:
            B.moe_layer_forward(h, moe[r], h, ids, w, ws_m, flags, stream=stream)
    ms = timed_loop(step, stream, args.warmup, args.steps)
    name = f"decoder_layer_step_{S}stream{'s' if S > 1 else ''}_ref288_attn_bf16_moe_int4g64_int8g128"
    if S == 1:
        check_error_word(ws_m, name)
    ids_last = ids.cpu().numpy()
    live = [min(g + 1, 128) for g in n_gen]
    kv_bytes = sum(10 * (n_ref + lv) * 128 * 2 * 2 + 10 * 128 * 2 * 2 for lv in live)
    attn_bytes = 4 * H * H * 2
    moe_bytes = (layer_bytes(ids_last[0].tolist(), wl.routed, wl.shared) if S == 1
                 else grouped_step_bytes(wl, [ids_last]))
    nbytes = kv_bytes + attn_bytes + moe_bytes + S * H * 4 * 2
    gbs = nbytes / (ms * 1e-3) / 1e9

    # gate and baseline: one more step on fresh inputs, each half checked on
    # sampled streams against the oracle on the GPU's own input to it
    from oracle import decoder_layer as DL
    from oracle import moe_oracle as O
    from tests.parity import check_layer
    kvh = make_rswa(S, n_ref, n_gen=n_gen, seed=99)
    dev = B.rswa_to_device(kvh)
    h0 = make_hidden(S, batch=777)
    hg = torch.from_numpy(h0).cuda()
    with torch.cuda.stream(stream):
        B.moe_attn_block_forward(hg, attn[0], dev, ws_a, stream=stream)
    torch.cuda.synchronize()
    h1 = hg.cpu().numpy().astype(np.float64)
    with torch.cuda.stream(stream):
        if S == 1:
            B.moe_decode_forward(hg, y, [moe[0]], ids, w, ws_m, flags, weights=warr[0], stream=stream)
        else:
            B.moe_layer_forward(hg, moe[0], hg, ids, w, ws_m, flags, stream=stream)
    torch.cuda.synchronize()
    h2 = (y if S == 1 else hg).cpu().numpy().astype(np.float64)
    w64 = {k: bf16_bits_to_f32(v).astype(np.float64) for k, v in aw.items()}
    f64 = lambda b: bf16_bits_to_f32(b).astype(np.float64)
    sample = np.arange(S) if S == 1 else np.sort(np.random.default_rng(5).choice(S, 4 if args.no_cpu_baseline else 12,
                                                                                   replace=False))
    t0 = time.perf_counter()
    refs, outs = [], []
    for s_ in sample:
        ho, _ = DL.attn_block(h0[s_:s_ + 1].astype(np.float64), w64["w_q"], w64["w_k"], w64["w_v"], w64["w_o"],
                              f64(kvh["ref_k"][s_:s_ + 1]), f64(kvh["ref_v"][s_:s_ + 1]),
                              f64(kvh["ring_k"][s_:s_ + 1]), f64(kvh["ring_v"][s_:s_ + 1]),
                              kvh["n_gen"][s_:s_ + 1], NORM_EPS)
        refs.append(ho[0] - h0[s_])
        outs.append(h1[s_] - h0[s_])
    refs, outs = np.array(refs), np.array(outs)
    r_attn = float(np.abs(outs - refs).max() / np.sqrt(np.mean(refs ** 2)))
    try:
        if not r_attn <= 1e-3:
            raise GateError(f"attention half max|err|/rms {r_attn:.3e}")
        r_moe, _ = check_layer(O.rmsnorm(h1[sample], NORM_EPS), layer, ids.cpu().numpy()[sample],
                               w.cpu().numpy()[sample], h2[sample] - h1[sample])
    except (AssertionError, GateError) as e:
        gate_exit(name, str(e))
    used = time.perf_counter() - t0
    out = {"metric": f"{name}: tokens/s", "value": S / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
           "steps": args.steps, "warmup": args.warmup,
           "dtype": "bf16 MFMA on bf16 weights x f32 activations as bf16 hi/lo (projections); f32 on bf16 KV "
                    "(attention); " + (DTYPE_DECODE if S == 1 else DTYPE_GROUPED) + " (MoE)",
           "data": "synthetic (seeded weights, KV and rows)",
           "config": {"workload": name, "streams": S, "n_ref": n_ref, "replicas": R},
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None, "bytes_per_step": nbytes},
           "parity_gate": {"streams": int(len(sample)), "attention_err_over_rms": r_attn, "moe_err_over_rms": r_moe,
                           "bar": "each half on the GPU's input to it: max|err| <= 1e-3 rms; routing as the tests"}}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = {"value": len(sample) / used, "unit": "tokens/s", "cores": host_threads(),
                               "kind": "oracle",
                               "sample": f"{len(sample)} stream{'s' if len(sample) > 1 else ''} of one step (float64 "
                                         f"numpy oracle: attention half and MoE layer), {used:.2f} s"}
    print(json.dumps(add_practical(out)), flush=True)


def bench_crossover(args):
    """Where the per-token (GEMV) path and the grouped (MFMA) path of
    moe_layer_forward cross: one layer at T tokens through each path (forced),
    for the continuous-batch decode formats (int4 G64 routed, int8 G128
    shared, f32 input with the norm and residual in the call), for int4 G32
    (bf16 input, biased router), int8 G128 routed and shared (f32 input),
    int4 G128 (bf16 input) and the two-level routed format with int8 G128
    shared (f32 input, norm and residual); 4 weight replicas rotated.  Prints
    one JSON line with the table (microseconds per layer call)."""
    import numpy as np
    import torch

    from quantized_expert_ffn_moe_amd import binding as B
    from synth import WORKLOADS, make_layer, make_tokens

    counts = [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16, 17, 18, 20, 22, 24, 32, 48, 64]
    table = {}
    stream = torch.cuda.Stream()
    def fmt(q):
        return "q4k" if q.group == 256 else f"int{q.bits}g{q.group}"

    for wi in (5, 2, 0, 3, 7):
        wl = WORKLOADS[wi]
        lay = make_layer(wl, 0)
        reps = [B.pack_layer(lay) for _ in range(4)]
        flags0 = B.MOE_NORM_INPUT | B.MOE_ACCUMULATE if wl.x_dtype == "f32" and wl.n_layers > 1 else 0
        rows = {}
        for T in counts:
            x, bits = make_tokens(wl, n_tokens=T, batch=60)
            xt = (torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16) if bits is not None
                  else torch.from_numpy(x)).cuda()
            xin = xt.float().contiguous() if wl.x_dtype == "f32" else xt
            y = torch.zeros(T, 1280, dtype=torch.float32, device="cuda")
            ids = torch.empty(T, 6, dtype=torch.int32, device="cuda")
            w = torch.empty(T, 6, dtype=torch.float32, device="cuda")
            ws = B.workspace(T)
            row = {}
            for name, f in (("per_token", B.MOE_FORCE_DECODE), ("grouped", B.MOE_FORCE_GROUPED), ("default", 0)):
                ms = timed_loop(lambda i: B.moe_layer_forward(xin, reps[i % 4], y, ids, w, ws, flags0 | f,
                                                              stream=stream), stream, args.warmup, args.steps)
                row[name] = round(ms * 1e3, 2)
            rows[T] = row
        key = f"{wl.name.split('_')[0]}_{fmt(wl.routed)}_{fmt(wl.shared)}_{wl.x_dtype}" + ("_biased" if wi == 2 else "")
        table[key] = rows
    print(json.dumps({"metric": "moe_layer_forward per-token vs grouped path: us per layer call",
                      "unit": "us", "steps": args.steps, "warmup": args.warmup, "table": table}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--workload", choices=["decode", "decode1", "batched32", "prefill273", "multipage2184", "batch128",
                                           "batch256", "lmhead_bf16", "lmhead_int8", "dense0", "rswa128", "ffnstack",
                                           "crossover", "layer1", "layer128"],
                    default="decode",
                    help="decode = the headline 11-layer decode step; decode1 = one token through one int8 G128 "
                         "layer; the prefill workloads report MFMA figures; batchN = one continuous-batch decode "
                         "step of N streams (HBM figures)")
    ap.add_argument("--group", type=int, default=64, choices=[32, 64, 128, 256],
                    help="decode: group size of the routed int4 experts (64 is the headline; 32 and 128 sweep "
                         "the group-size trade of metadata bytes against time; 256 = the two-level "
                         "Q4_K-style format); grouped workloads: 256 puts every expert in the two-level format")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="leave the CPU baseline out of the line (the parity gate still runs, on one oracle call)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the multi-GPU layout is a design note.",
              file=sys.stderr)
        sys.exit(2)

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

    if args.workload.startswith("lmhead") or args.workload == "dense0":
        return bench_dense(args)
    if args.workload == "rswa128":
        return bench_rswa(args)
    if args.workload == "ffnstack":
        return bench_ffnstack(args)
    if args.workload in ("decode", "decode1"):
        return bench_decode(args)
    if args.workload == "crossover":
        return bench_crossover(args)
    if args.workload in ("layer1", "layer128"):
        return bench_layer(args)
    return bench_grouped(args)


if __name__ == "__main__":
    main()
