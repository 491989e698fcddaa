"""Benchmark of the routed int4 MoE expert layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Workloads (seeded synthetic inputs, shapes of the pages' model: hidden 2048,
256 routed experts, top-8, SwiGLU inter 512, int4 experts):
  frame         (default) the full-depth decode frame: 40 sequential MoE
                layers x 16 tokens (own RTN g64 weights and router per
                layer), residual bf16(x + y) between layers; value is frame
                tokens/s (16 tokens through all 40 layers per step).
  decode        one decode step of one MoE layer for 1 token:
                router GEMV + top-k, grouping, gate/up GEMV + SwiGLU, down
                GEMV, combine; asym g64 clip-searched weights.  Steps rotate
                over 40 address-distinct copies of the layer, as successive
                layers of a 40-layer model would, so experts are read from HBM
                and not from the 256 MB last-level cache.
  prefill       512 tokens, Zipf(1.1)-popular experts (logits given), asym g64.
  long_prefill  4096 tokens, N(0,1) logits given, sym g128.
  tiny          4 tokens, 16 experts, top-2 (correctness size).
  decode_shared, frame_shared
                decode / frame with each layer's shared expert (int8
                symmetric g128, inter 512) in the same forward call.
  decode_fp8, frame_fp8, prefill_fp8, long_prefill_fp8
                decode / frame / prefill / long prefill with block-FP8 experts
                (E4M3, float32 scale per 128 x 128 block; the released
                experts' format) of the same Gaussian weights.
  decode_nvfp4, frame_nvfp4, prefill_nvfp4, long_prefill_nvfp4
                the same with NVFP4 experts (E2M1, E4M3 scale per 16 inputs,
                float32 global per matrix).
  shared        the shared expert alone (moe_q4_shared) for the frame's 16
                tokens; steps rotate over 200 address-distinct copies (3 MB
                each) so its codes are read from HBM.
  shared_prefill
                the shared expert alone for the long prompt's 4096 tokens
                (matrix-core GEMMs).

With --lanes N the frame workloads run as one moe_q4_frame call per step:
the 16 tokens split into N token lanes, each through all 40 layers on its own
stream over 1/N of the expert kernels' resident grid, so one lane's layers
overlap the other's (cross-layer pipelining); the roofline is then per lane
launch.

The prefill workloads give the layer its prefill copy of the weights
(moe_q4_prefill_pack, made once before timing, as at weight load); with
--no-pack the grouped GEMMs read the canonical arrays.

One JSON line on stdout: value = tokens/s of whole steps (inputs resident in
HBM), roofline of the dominant kernel measured with HIP events recorded on the
launch stream at its stage boundaries, and the CPU oracle timed on a bounded
sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/f16 matrix (the prefill GEMMs run f16)
METRIC = "MoE layer tokens/s; decode HBM GB/s, prefill MFMA TFLOPs (% of peak)"

WORKLOADS = {
    "tiny": 1, "decode": 2, "prefill": 3, "frame": 4, "long_prefill": 5,
    "decode_shared": 2, "frame_shared": 4, "shared": 4, "decode_fp8": 2, "frame_fp8": 4,
    "prefill_fp8": 3, "long_prefill_fp8": 5,
    "decode_nvfp4": 2, "frame_nvfp4": 4, "prefill_nvfp4": 3, "long_prefill_nvfp4": 5,
    "shared_prefill": 5,
}
SHARED_INTER = 512   # the shared expert's inner size (that of a routed expert)
SHARED_COPIES = 200  # address-distinct shared experts of the "shared" workload


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=None)
    p.add_argument("--warmup", type=int, default=None)
    p.add_argument("--workload", default="frame", choices=sorted(WORKLOADS))
    p.add_argument("--copies", type=int, default=40, help="address-distinct weight copies (decode)")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="budget of each CPU oracle sample (one at all cores, one at one thread)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-pack", action="store_true",
                   help="prefill GEMMs read the canonical weight arrays instead of the prefill copy")
    p.add_argument("--deterministic", action="store_true",
                   help="moe_q4_forward_det: decode y summed per token in slot order (run-to-run identical)")
    p.add_argument("--lanes", type=int, default=None,
                   help="frame workloads: run the frame as this many token lanes on their own streams (moe_q4_frame)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 256 MiB device copy 3 times (HBM counter calibration) and exit")
    return p.parse_args()


CSRC = os.path.join(ROOT, "quantized_moe_expert_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def source_digest(unit: str) -> str:
    """sha256 over a kernel source file and the local headers it includes
    (recursively), so a recorded counter figure can be matched to the code."""
    import hashlib
    import re
    seen, todo = set(), [unit]
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.add(f)
        text = open(os.path.join(CSRC, f), encoding="utf-8").read()
        todo += [h for h in re.findall(r'#include "([^"]+)"', text) if os.path.exists(os.path.join(CSRC, h))]
    h = hashlib.sha256()
    for f in sorted(seen):
        h.update(f.encode())
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def recorded_traffic(kernel: str, workload: str, unit: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    profiles/<kernel>.<workload>.traffic.md (FETCH_SIZE and WRITE_SIZE runs,
    each scaled by the copy calibration), or None when there is none or the
    kernel's source has changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}.{workload}.traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and line.startswith("- "):
            key, val = line[2:].split(":", 1)
            rec[key.strip()] = val.strip().strip("`")
    if rec.get("source_digest") != source_digest(unit):
        return None
    try:
        return int(float(rec["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device copy of known size: what FETCH_SIZE / WRITE_SIZE report
    for it gives the scale of those counters on this GPU."""
    import torch
    n = 256 * 1024 * 1024
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def clone_layer(lay):
    import synth
    return synth.Layer(fmt=lay.fmt, num_experts=lay.num_experts, hidden=lay.hidden, inter=lay.inter,
                       gate_q=lay.gate_q.clone(), up_q=lay.up_q.clone(), down_q=lay.down_q.clone(),
                       gate_sm=lay.gate_sm.clone(), up_sm=lay.up_sm.clone(), down_sm=lay.down_sm.clone(),
                       global_scale=lay.global_scale.clone() if lay.global_scale is not None else None)


def expert_bytes(lay) -> int:
    return lay.nbytes() // lay.num_experts


def clone_shared(sx):
    import synth
    return synth.SharedExpert(hidden=sx.hidden, inter=sx.inter, **{n: getattr(sx, n).clone() for n in (
        "gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")})


def shared_gateup_bytes(sx) -> int:
    """Codes and scales of the shared expert's gate and up projections."""
    return sum(t.numel() * t.element_size() for t in (sx.gate_q, sx.up_q, sx.gate_s, sx.up_s))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import numpy as np
    import torch

    import quantized_moe_expert_amd as m
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    m.lib()
    dev = torch.device("cuda")
    cfg = WORKLOADS[args.workload]
    defaults = {"tiny": (200, 20), "decode": (400, 40), "prefill": (50, 5), "frame": (10, 2),
                "long_prefill": (20, 3), "decode_shared": (400, 40), "frame_shared": (10, 2), "shared": (400, 40),
                "decode_fp8": (400, 40), "frame_fp8": (10, 2), "prefill_fp8": (50, 5), "long_prefill_fp8": (20, 3),
                "decode_nvfp4": (400, 40), "frame_nvfp4": (10, 2), "prefill_nvfp4": (50, 5),
                "long_prefill_nvfp4": (20, 3), "shared_prefill": (50, 5)}
    K = args.steps if args.steps is not None else defaults[args.workload][0]
    W = args.warmup if args.warmup is not None else defaults[args.workload][1]

    t0 = time.time()
    only_shared = args.workload in ("shared", "shared_prefill")
    with_shared = args.workload in ("decode_shared", "frame_shared", "shared", "shared_prefill")
    fp8 = args.workload.endswith("_fp8")
    nvfp4 = args.workload.endswith("_nvfp4")
    case = synth.make_case(cfg, device="cuda", layers=1 if only_shared else None,
                           fmt=synth.FMT_FP8_B128 if fp8 else synth.FMT_NVFP4 if nvfp4 else None)
    torch.cuda.synchronize()
    T, H, E, k, I = case.T, case.H, case.E, case.k, case.I
    base_wl = {"decode_shared": "decode", "frame_shared": "frame", "decode_fp8": "decode",
               "frame_fp8": "frame", "prefill_fp8": "prefill",
               "long_prefill_fp8": "long_prefill", "decode_nvfp4": "decode", "frame_nvfp4": "frame",
               "prefill_nvfp4": "prefill", "long_prefill_nvfp4": "long_prefill"}.get(args.workload, args.workload)
    decode_path = base_wl in ("tiny", "decode", "frame", "shared")
    shared_gemm = args.workload == "shared_prefill"
    mode = "decode" if decode_path else "prefill"

    # ---- per-step units of work ------------------------------------------------
    if base_wl == "decode":
        copies = max(1, args.copies)
        base = case.layers[0]
        layers = [base] + [clone_layer(base) for _ in range(copies - 1)]
        routers = [case.router_w] + [case.router_w.clone() for _ in range(copies - 1)]
        nl_per_step = 1
    elif base_wl == "frame":
        layers = case.layers
        routers = case.router_ws
        nl_per_step = len(layers)
    else:
        layers = case.layers
        routers = case.router_ws or [None]
        nl_per_step = 1
    shareds = None
    if with_shared:
        if base_wl == "frame":  # one shared expert per layer
            shareds = [synth.make_shared(H, SHARED_INTER, 0, f"{case.name}/L{l}/shared", device="cuda")
                       for l in range(len(layers))]
        else:
            s0 = synth.make_shared(H, SHARED_INTER, 0, f"{case.name}/shared", device="cuda")
            n_sx = SHARED_COPIES if only_shared else len(layers)
            shareds = [s0] + [clone_shared(s0) for _ in range(n_sx - 1)]
    torch.cuda.synchronize()
    log(f"[bench] generated {args.workload} inputs in {time.time() - t0:.1f}s")
    # the prefill path reads the prefill copy of the weights, made once here
    # like any load-time weight conversion, outside the timing
    use_pack = mode == "prefill" and not shared_gemm and not args.no_pack
    packs = [m.prefill_pack(l) for l in layers] if use_pack else [None] * len(layers)
    structs = [m.layer_struct(l, pack=p) for l, p in zip(layers, packs)]
    sstructs = [m.shared_struct(sx) for sx in shareds] if shareds else None
    ws_bytes = m.workspace_size(m.WS_FORWARD_DET if args.deterministic else m.WS_FORWARD, T, E, k, H, I)
    if with_shared:
        ws_bytes += m.workspace_size(m.WS_SHARED, T, 1, 1, H, SHARED_INTER)
    wsf = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    m.moe_q4_workspace_init(wsf)
    lg = torch.empty((T, E), dtype=torch.int16, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    gate = torch.empty((T, k), dtype=torch.float32, device=dev)
    ybuf = [torch.empty((T, H), dtype=torch.float32, device=dev) for _ in range(2)]
    xbuf = [torch.empty_like(case.x), torch.empty_like(case.x)]
    state = {"i": 0}
    lanes = args.lanes
    if lanes is not None and (base_wl != "frame" or args.deterministic):
        raise SystemExit("--lanes applies to the frame workloads (without --deterministic)")
    if lanes is not None:
        # the frame as token lanes: one moe_q4_frame call per step
        nlay = len(layers)
        fr = {"xc": torch.empty((nlay - 1, T, H), dtype=case.x.dtype, device=dev),
              "yc": torch.empty((nlay, T, H), dtype=torch.float32, device=dev),
              "lg": torch.empty((nlay, T, E), dtype=torch.int16, device=dev),
              "idx": torch.empty((nlay, T, k), dtype=torch.int32, device=dev),
              "gate": torch.empty((nlay, T, k), dtype=torch.float32, device=dev)}
        fr["ws"] = torch.empty(max(m.frame_workspace_size(T, E, k, H, I, SHARED_INTER if with_shared else 0, lanes),
                                   256), dtype=torch.uint8, device=dev)
        lane_streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(lanes - 1)]

        def frame_call(evs=None):
            m.moe_q4_frame(case.x, T, k, structs, routers, sstructs, fr["xc"], fr["yc"], fr["lg"], fr["idx"],
                           fr["gate"], lanes, lane_streams, fr["ws"], events=evs)

        def lanes_fork():
            for s_ in lane_streams[1:]:
                s_.wait_stream(torch.cuda.current_stream())

        def lanes_join():
            for s_ in lane_streams[1:]:
                torch.cuda.current_stream().wait_stream(s_)

    def layer_ids():
        if base_wl == "decode":
            return [state["i"] % len(layers)]
        if only_shared:
            return [state["i"] % len(shareds)]
        return list(range(nl_per_step))

    def call(j, li, evs):
        """One layer: moe_q4_forward_ex (routing, grouping, experts, the
        shared expert when present; the residual of a chain fused in), or
        the shared expert alone.  evs: None or the 4 stage events."""
        if only_shared:
            if evs is None:
                m.moe_q4_shared(case.x, T, sstructs[li], ybuf[0], 0, wsf)
            else:
                m.moe_q4_shared_timed(case.x, T, sstructs[li], ybuf[0], 0, wsf, evs)
            return
        rw = routers[li] if routers[0] is not None else None
        logits_in = lg if rw is not None else case.logits
        sx = sstructs[li] if sstructs else None
        fwd = m.moe_q4_forward_det if args.deterministic else m.moe_q4_forward_ex
        if base_wl == "frame" and j > 0:
            x_prev = case.x if j == 1 else xbuf[(j - 1) & 1]
            fwd(x_prev, ybuf[(j - 1) & 1], xbuf[j & 1], rw, None, logits_in, T, k, structs[li], sx,
                idx, gate, ybuf[j & 1], wsf, events=evs)
        else:
            fwd(case.x, None, None, rw, None, logits_in, T, k, structs[li], sx, idx, gate,
                ybuf[j & 1], wsf, events=evs)

    def step():
        """One step: every layer of the workload once."""
        if lanes is not None:
            frame_call()
            return
        for j, li in enumerate(layer_ids()):
            call(j, li, None)
        state["i"] += 1

    def step_profiled(evsets):
        """The calls of step() with stage events: the runtime records them at
        the start and end of the call's two main kernels (gate/up and routing
        launches for decode, the two grouped GEMMs for prefill, gate/up and
        down launches of the shared expert alone) on the launch stream."""
        if lanes is not None:  # per (layer, lane): events[(j * lanes + i) * 4 ...]
            frame_call([e.cuda_event for evs in evsets for e in evs])
            for j in range(len(layers)):
                for i in range(lanes):
                    routed.append(fr["idx"][j, T * i // lanes:T * (i + 1) // lanes].clone())
            return
        for j, li in enumerate(layer_ids()):
            call(j, li, [e.cuda_event for e in evsets[j]])
            if not only_shared:
                routed.append(idx.clone())
        state["i"] += 1

    routed = []

    # ---- warmup + timed steps ------------------------------------------------
    if lanes is not None:
        lanes_fork()
    for _ in range(W):
        step()
    if lanes is not None:
        lanes_join()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    if lanes is not None:  # the lane streams start after `start` and `stop` follows them all
        lanes_fork()
    for _ in range(K):
        step()
    if lanes is not None:
        lanes_join()
    stop.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / K
    tokens_per_step = T
    value = tokens_per_step * K / (total_ms / 1e3)
    log(f"[bench] {args.workload}: {ms_per_step * 1e3:.2f} us/step, {value:.1f} tokens/s")

    # ---- stage timing of the dominant kernel (same work, events on the stream)
    nev = m.STAGE_EVENTS
    prof_steps = max(1, min(K, 50 if nl_per_step == 1 else 2))
    per_call = nl_per_step * (lanes or 1)  # event sets per step: one per layer (and lane)
    ev_sets = [[[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(per_call)]
               for _ in range(prof_steps)]
    for per_step in ev_sets:  # materialise the event handles
        for evs in per_step:
            for e in evs:
                e.record()
    torch.cuda.synchronize()
    if lanes is not None:
        lanes_fork()
    for per_step in ev_sets:
        step_profiled(per_step)
    if lanes is not None:
        lanes_join()
    torch.cuda.synchronize()
    # [0]: the dominant kernel (decode gate/up GEMV / prefill gate-up GEMM),
    # [1]: the second kernel (decode routing launch / prefill down GEMM); each is the span
    # between the events the runtime recorded at that kernel's start and end
    stage_ms = np.array([[evs[0].elapsed_time(evs[1]), evs[2].elapsed_time(evs[3])]
                         for per_step in ev_sets for evs in per_step])
    stage_avg = stage_ms.mean(axis=0)
    log(f"[bench] kernel times (us): {', '.join(f'{v * 1e3:.2f}' for v in stage_avg)}")

    # work actually routed in the profiled layer (outside timed regions)
    # active experts per profiled layer call, averaged (the frame's layers differ)
    act = float(np.mean([torch.unique(r).numel() for r in routed])) if routed else 0.0
    lay0 = layers[0]
    proj_bytes = expert_bytes(lay0) // 3        # one projection of one expert (codes + scales)
    nlanes = lanes or 1
    Tl = T // nlanes  # tokens per launch (per lane with --lanes)
    P = Tl * k
    sx_bytes = shared_gateup_bytes(shareds[0]) + Tl * SHARED_INTER * 4 if with_shared else 0  # + h (fp32) out
    if shared_gemm:
        # dominant kernel: the shared gate/up GEMM + SwiGLU on the matrix cores
        dom = "shared_gemm_kernel<1> (gate/up f16 GEMM + SwiGLU)"
        flops = 2.0 * T * H * (2 * SHARED_INTER)
        achieved = flops / (stage_avg[0] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None, "kernel": dom,
                "avg_us": round(float(stage_avg[0]) * 1e3, 3), "algorithmic_flops": flops}
    elif only_shared:
        # dominant kernel: the shared gate/up GEMV + SwiGLU: its int8 codes and
        # scales once, the activations, h (fp32) out
        dom = "shared_gateup_kernel"
        alg_bytes = sx_bytes + T * H * 2
        achieved = alg_bytes / (stage_avg[0] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic(dom, args.workload, "shared.hip"), "kernel": dom,
                "avg_us": round(float(stage_avg[0]) * 1e3, 3), "algorithmic_bytes": int(alg_bytes)}
    elif decode_path:
        # dominant kernel: gate/up GEMV + SwiGLU: reads the gate and up codes and
        # scales of every active expert once and the activations, writes h (fp32)
        dom = "decode_gateup_kernel"
        alg_bytes = act * 2 * proj_bytes + Tl * H * 2 + P * I * 4 + sx_bytes
        achieved = alg_bytes / (stage_avg[0] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if lanes else recorded_traffic(dom, args.workload, "decode.hip"), "kernel": dom + (
                    " (routed and shared items)" if with_shared else "") + (
                    f" (one lane's launch, {lanes} lanes side by side)" if lanes else ""),
                "avg_us": round(float(stage_avg[0]) * 1e3, 3), "algorithmic_bytes": int(alg_bytes),
                "active_experts": int(act)}
    else:
        dom = ("grouped_gemm_fp8_kernel<1> (gate/up bf16 GEMM + SwiGLU)" if fp8
               else "grouped_gemm_kernel<FMT,1> (gate/up GEMM + SwiGLU)")
        gemm_key = "grouped_gemm_fp8_kernel_1" if fp8 else "grouped_gemm_kernel_1"
        flops = 2.0 * P * H * (2 * I)
        achieved = flops / (stage_avg[0] * 1e-3) / 1e12
        wbytes = act * 2 * proj_bytes
        if base_wl == "prefill":
            # weight-bandwidth-bound case: report against HBM
            gbs = (wbytes + T * H * 2 + P * I * 2) / (stage_avg[0] * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "traffic": recorded_traffic(gemm_key, args.workload, "prefill.hip"), "kernel": dom,
                    "avg_us": round(float(stage_avg[0]) * 1e3, 3), "tflops": round(achieved, 2),
                    "active_experts": int(act)}
        else:
            roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                    "traffic": recorded_traffic(gemm_key, args.workload, "prefill.hip"),
                    "kernel": dom, "avg_us": round(float(stage_avg[0]) * 1e3, 3),
                    "algorithmic_flops": flops, "active_experts": int(act)}
    roof["second_kernel_us"] = round(float(stage_avg[1]) * 1e3, 3)
    if decode_path and not only_shared:
        # the whole step's algorithmic HBM bytes: per layer the router rows
        # (when the GEMV runs), every active expert's three projections once,
        # x in, y out (the shared expert's codes when present)
        router_bytes = E * H * 2 if routers[0] is not None else 0
        shared_all = shared_gateup_bytes(shareds[0]) * 3 // 2 if with_shared else 0  # gate, up, down
        layer_bytes = nlanes * (router_bytes + act * 3 * proj_bytes + Tl * H * 2 + Tl * H * 4 + shared_all)
        step_bytes = layer_bytes * nl_per_step
        step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
        roof["step"] = {"algorithmic_bytes": int(step_bytes), "achieved": round(step_gbs, 1), "unit": "GB/s",
                        "frac": round(step_gbs / HBM_PEAK_GBS, 4), "layers": nl_per_step}

    # ---- CPU oracle on a bounded sample ------------------------------------------
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, args, decode_path, args.cpu_seconds, shareds[0] if with_shared else None,
                           only_shared, nl_per_step)

    names = {"tiny": "tiny layer: 4 tokens, H=256, 16 experts, top-2, I=128, int4 asym g64",
             "decode": "decode step, 1 MoE layer: 1 token, H=2048, 256 experts, top-8, I=512, int4 asym g64 "
                       "(clip search); 40 address-distinct layer copies rotated",
             "prefill": "prefill, 1 MoE layer: 512 tokens, Zipf(1.1) expert popularity, H=2048, 256 experts, "
                        "top-8, I=512, int4 asym g64",
             "frame": "full-depth decode frame: 40 MoE layers x 16 tokens, H=2048, 256 experts, top-8, I=512, "
                      "int4 asym g64 (RTN), residual chain",
             "long_prefill": "long prefill, 1 MoE layer: 4096 tokens, N(0,1) logits, H=2048, 256 experts, top-8, "
                             "I=512, int4 sym g128"}
    sx_note = f" + shared expert int8 sym g128 I={SHARED_INTER} per layer"
    names["decode_shared"] = names["decode"] + sx_note
    names["frame_shared"] = names["frame"] + sx_note
    names["decode_fp8"] = names["decode"].replace("int4 asym g64 (clip search)", "block-FP8 E4M3, 128x128 scales")
    names["frame_fp8"] = names["frame"].replace("int4 asym g64 (RTN)", "block-FP8 E4M3, 128x128 scales")
    names["prefill_fp8"] = names["prefill"].replace("int4 asym g64", "block-FP8 E4M3, 128x128 scales")
    names["long_prefill_fp8"] = names["long_prefill"].replace("int4 sym g128", "block-FP8 E4M3, 128x128 scales")
    nv = "NVFP4 (E2M1, E4M3 scale per 16, fp32 global)"
    names["decode_nvfp4"] = names["decode"].replace("int4 asym g64 (clip search)", nv)
    names["frame_nvfp4"] = names["frame"].replace("int4 asym g64 (RTN)", nv)
    names["prefill_nvfp4"] = names["prefill"].replace("int4 asym g64", nv)
    names["long_prefill_nvfp4"] = names["long_prefill"].replace("int4 sym g128", nv)
    names["shared_prefill"] = (f"shared expert alone: 4096 tokens, H=2048, I={SHARED_INTER}, int8 sym g128, "
                               "matrix-core GEMMs")
    names["shared"] = (f"shared expert alone: 16 tokens, H=2048, I={SHARED_INTER}, int8 sym g128; "
                       f"{SHARED_COPIES} address-distinct copies rotated")
    out = {"metric": METRIC, "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
           "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16" if decode_path or fp8 else "f16", "data": "synthetic",
           "config": {"workload": names[args.workload], "tokens": T, "hidden": H, "experts": 0 if only_shared else E,
                      "top_k": 0 if only_shared else k, "inter": SHARED_INTER if only_shared else I,
                      "layers_per_step": nl_per_step, "path": mode,
                      "format": "int8_sym_g128" if only_shared else {
                          synth.FMT_ASYM_G64: "asym_g64", synth.FMT_SYM_G128: "sym_g128",
                          synth.FMT_FP8_B128: "fp8_e4m3_b128", synth.FMT_NVFP4: "nvfp4"}[case.fmt],
                      "shared_expert": with_shared, "deterministic": bool(args.deterministic),
                      "weights": "prefill copy" if use_pack else "canonical", "lanes": nlanes},
           "roofline": roof, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_sample(case, budget_s, shared, only_shared):
    """Tokens of layer 0 through the oracle, a few per call, until budget_s
    of wall time is spent; returns (tokens, seconds, calls, tokens per call)."""
    import numpy as np

    import oracle
    T, H, E, k = case.T, case.H, case.E, case.k
    lay = case.layers[0]
    host_layer = oracle.layer_np(lay)
    host_sx = [t.cpu().numpy() for t in shared.tensors()] if shared is not None else None
    x_np = case.x.cpu().numpy().view(np.uint16)
    rw = case.router_ws[0].cpu().numpy().view(np.uint16) if case.router_ws else None
    lg_all = case.logits.cpu().numpy().view(np.uint16) if case.logits is not None else None
    per = 1 if T == 1 else min(T, 16)
    done_tokens, t_total, reps = 0, 0.0, 0
    while t_total < budget_s and reps < 10000:
        sel = np.arange(T)[(reps * per) % T:(reps * per) % T + per]
        t1 = time.perf_counter()
        xs = np.ascontiguousarray(x_np[sel])
        y = None
        if not only_shared:
            lg = oracle.router(xs, rw, len(sel), H, E) if rw is not None else np.ascontiguousarray(lg_all[sel])
            idx, gate = oracle.topk(lg, len(sel), E, k)
            y = oracle.experts(lay.fmt, E, H, lay.inter, *host_layer, xs, idx, gate, len(sel), k,
                               global_scale=oracle.layer_global(lay))
        if host_sx is not None:
            oracle.shared(H, shared.inter, *host_sx, xs, len(sel), y_in=y)
        t_total += time.perf_counter() - t1
        done_tokens += len(sel)
        reps += 1
    return done_tokens, t_total, reps, per


def cpu_baseline(case, args, decode_path, budget_s, shared=None, only_shared=False, layers_per_step=1):
    """The oracle as it stands, on this host's cores, over a bounded sample of
    the same workload: once with every core (OMP_NUM_THREADS, else all), once
    with one thread.  value is in the bench line's unit: tokens/s through all
    layers of one step (the per-layer rate divided by the layers per step)."""
    import oracle
    oracle.build(force=False)
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    oracle.set_threads(threads)
    n_all, t_all, reps_all, per = oracle_sample(case, budget_s, shared, only_shared)
    oracle.set_threads(1)
    n_one, t_one, reps_one, _ = oracle_sample(case, budget_s, shared, only_shared)
    oracle.set_threads(threads)
    layer_all, layer_one = n_all / t_all, n_one / t_one
    what = "shared expert" if only_shared else (
        "route + experts + combine" + (" + shared expert" if shared is not None else ""))
    unit = "tokens/s" if layers_per_step == 1 else f"tokens/s through {layers_per_step} layers"
    return {"value": round(layer_all / layers_per_step, 4), "unit": unit, "cores": threads, "kind": "oracle",
            "single_thread_value": round(layer_one / layers_per_step, 4),
            "per_layer_tokens_s": {"all_cores": round(layer_all, 3), "one_thread": round(layer_one, 3)},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"layer 0 of the workload, {per} token(s) per call: {n_all} tokens in {t_all:.1f} s at "
                      f"{threads} threads, {n_one} tokens in {t_one:.1f} s at 1 thread ({what}, fp64); "
                      f"the other layers cost the same per token"}


if __name__ == "__main__":
    main()
