#!/usr/bin/env python3
"""Forward + backward throughput of the RAWINT4 routed-expert LoRA layer on one MI355X.

A step is one forward and one backward of the layer (grouping, gate/up GEMM with
SwiGLU, down GEMM with the route-weighted combine, down and gate/up transpose-
free dX, LoRA side products and the six LoRA gradient reductions) over one
synthetic batch already resident in HBM.  Prints ONE JSON line on stdout;
progress goes to stderr.

``--infer lora|base`` times the inference forward instead (kt_rawint4_moe_infer:
with the LoRA, or the frozen base alone); ``--recompute`` times the training step
in its checkpointed form (an inference forward that keeps nothing, then
kt_rawint4_moe_bwd_recompute).  The default line is the training step.

Default workload: 384 experts, top-8, hidden 7168, intermediate 2048, LoRA rank 64
(alpha 128), 16384 tokens, SwiGLU clamp 7, uniform routing.  ``--config`` picks
another of the five workloads of ``int4_quantized_moe_amd.workloads.CONFIGS``;
``--format mxfp4`` gives it an MXFP4 base (E2M1 codes, power-of-two scales).
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-expert fwd+bwd tokens/sec per layer; % MFMA peak / % HBM BW"
METRIC_INFER = "routed-expert inference forward tokens/sec per layer; % MFMA peak / % HBM BW"
FWD_PHASES = ("gemm_gate_up", "gemm_down", "lora_a_gate_up", "lora_a_down")
PEAK_MFMA_FP16 = 2.5e15  # dense fp16/bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12  # bytes/s


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def phase_work(cfg, slots):
    """Algorithmic flops and packed-weight bytes per launch of each phase.

    Flops per token-slot: gate/up 4HI + 4rI, down 2IH + 2rH, down dX 2HI + 2rI,
    gate/up dX 4IH + 4rH (each with its in-GEMM LoRA term); LoRA side products
    4rH, 2rI, 2rH, 4rI; LoRA gradients 6rH + 6rI; in all 12HI + 18r(H+I).
    Packed-weight bytes: codes (N*K/2) plus bf16 scales (N*K/16) of each active
    expert's projection(s) the phase streams.
    """
    H, I, r = cfg.hidden, cfg.intermediate, cfg.rank
    proj = H * I // 2 + H * I // 16  # one projection of one expert
    return {
        "gemm_gate_up": (slots * (4 * H * I + 4 * r * I), 2 * proj),
        "gemm_down": (slots * (2 * I * H + 2 * r * H), proj),
        "gemm_down_dx": (slots * (2 * H * I + 2 * r * I), proj),
        "gemm_gate_up_dx": (slots * (4 * I * H + 4 * r * H), 2 * proj),
        "lora_a_gate_up": (slots * 4 * r * H, 0),
        "lora_a_down": (slots * 2 * r * I, 0),
        "lora_b_down_bwd": (slots * 2 * r * H, 0),
        "lora_b_gate_up_bwd": (slots * 4 * r * I, 0),
        "lora_grads": (slots * (6 * r * H + 6 * r * I), 0),
    }


def cpu_baseline(cfg, weights, batch, target_s, infer=None):
    """The oracle, as it stands, on whole experts of the same batch: every slot routed
    to the first n experts (other slots dropped), so that each expert's dequantisation
    is shared by as many rows as at the full batch.  The oracle's time is linear in
    the slots at a fixed rows-per-expert mix, so the workload's rate is the sample's
    slots per second over the workload's slots per token.  Forward only for an
    inference run; zero LoRA for the base alone."""
    import numpy as np

    import oracle as O

    lora = None
    if infer == "base":
        lora = {n: np.zeros(s) for n, s in cfg.lora_shapes().items()}
    ids_all = batch.expert_ids
    total_slots = int(np.count_nonzero((ids_all >= 0) & (ids_all < cfg.num_experts)))
    order = [int(e) for e in np.unique(ids_all[(ids_all >= 0) & (ids_all < cfg.num_experts)])]

    def run(n):
        keep = order[:n]
        rows = np.flatnonzero(np.isin(ids_all, keep).any(axis=1))
        ids = np.where(np.isin(ids_all[rows], keep), ids_all[rows], -1).astype(np.int64)
        slots = int(np.count_nonzero(ids >= 0))
        t0 = time.perf_counter()
        O.moe(cfg, weights, batch.inputs[rows], ids, batch.route_weights[rows],
              None if infer else batch.grad_output[rows], lora=lora)
        return time.perf_counter() - t0, slots

    n = 1
    t, slots = run(n)
    log(f"cpu oracle pilot: 1 expert ({slots} slots) in {t:.2f}s")
    if t < target_s / 3 and n < len(order):
        n = int(min(len(order), max(1, target_s / max(t, 1e-3))))
        t, slots = run(n)
        log(f"cpu oracle sample: {n} experts ({slots} slots) in {t:.2f}s")
    return {
        "value": slots / t * cfg.qlen / total_slots,
        "unit": "tokens/s",
        "cores": O.num_threads(),
        "kind": "oracle",
        "sample": f"every slot of {n} of {len(order)} active experts ({slots} of {total_slots} token-slots), "
                  f"{'forward' if infer else 'fwd+bwd'}, fp64 accumulation, {t:.1f} s wall; tokens/s = "
                  f"sample slots per second x qlen / all slots",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=4, help="index into workloads.CONFIGS")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--infer", choices=("lora", "base"), default=None,
                    help="time the inference forward (with the LoRA, or the frozen base alone) instead of the "
                         "training step")
    ap.add_argument("--format", choices=("rawint4", "mxfp4"), default="rawint4",
                    help="weight format of the frozen base (the workload's shapes and seeds either way)")
    ap.add_argument("--recompute", action="store_true",
                    help="training step with an inference forward and the checkpoint-recompute backward")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after timing, run one plain elementwise copy (torch.neg, fp32) of this many MiB: "
                         "the calibration kernel for hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (expert parallelism is designed, "
              "not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from int4_quantized_moe_amd import _lib, device, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    cfg = workloads.CONFIGS[args.config]
    if args.format != cfg.weight_format:
        cfg = dataclasses.replace(cfg, name=f"{cfg.name}_{args.format}", weight_format=args.format)
    seed = workloads.config_seed(args.config)
    log(f"workload {cfg.name}: generating (seed {seed})")
    t0 = time.perf_counter()
    weights = workloads.make_weights(cfg, seed)
    batch = workloads.make_batch(cfg, seed)
    log(f"generated in {time.perf_counter() - t0:.1f}s; uploading")
    dl = device.DeviceLayer(cfg, weights, "cuda:0", base_only=args.infer == "base")
    db = device.DeviceBatch(batch, "cuda:0")
    out = torch.empty((db.qlen, cfg.hidden), dtype=torch.bfloat16, device="cuda:0")
    stream = torch.cuda.current_stream()
    if args.infer and args.recompute:
        print("--infer and --recompute exclude each other", file=sys.stderr)
        sys.exit(2)
    if args.infer:
        ws = dl.infer_workspace(db.qlen)

        def step(mid=None):
            dl.infer(db.inputs, db.expert_ids, db.route_weights, ws, output=out, stream=stream)
    else:
        ws = dl.workspace(db.qlen)
        grads = dl.grad_buffers(fill=0.0)
        dx = torch.empty_like(out)
        droute = torch.empty((db.qlen, cfg.top_k), dtype=torch.float32, device="cuda:0")

        ws_fwd = dl.infer_workspace(db.qlen) if args.recompute else ws

        def step(mid=None):
            if args.recompute:
                dl.infer(db.inputs, db.expert_ids, db.route_weights, ws_fwd, output=out, stream=stream)
            else:
                dl.forward(db.inputs, db.expert_ids, db.route_weights, ws, output=out, stream=stream)
            if mid is not None:
                mid.record(stream)
            dl.backward(db.inputs, db.expert_ids, db.route_weights, db.grad_output, ws, grads, accumulate=False,
                        grad_scale=1.0, grad_input=dx, grad_route=droute, stream=stream, recompute=args.recompute)
    log(f"workspace {ws.numel() / 2**30:.2f} GiB")

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.kt_rawint4_profile_read()  # drop anything recorded before
    _lib.kt_rawint4_profile_enable(True)
    log(f"timing {args.steps} steps")
    # one event at each step boundary and one between its forward and its backward
    # (all on the stream every kernel is launched on)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    mids = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    start, stop = marks[0], marks[-1]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(None if args.infer else mids[i])
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    _lib.kt_rawint4_profile_enable(False)
    phases = _lib.kt_rawint4_profile_read()
    gpu_ms = start.elapsed_time(stop)
    ms_per_step = gpu_ms / args.steps
    value = db.qlen * args.steps / (gpu_ms / 1e3)
    log(f"{ms_per_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}), {value:.1f} tokens/s")
    if args.infer:
        t_fwd, t_bwd = ms_per_step, 0.0
    else:
        t_fwd = sum(marks[i].elapsed_time(mids[i]) for i in range(args.steps)) / args.steps
        t_bwd = sum(mids[i].elapsed_time(marks[i + 1]) for i in range(args.steps)) / args.steps
        log(f"forward {t_fwd:.3f} ms, backward {t_bwd:.3f} ms per step")

    slots = int(np.count_nonzero((batch.expert_ids >= 0) & (batch.expert_ids < cfg.num_experts)))
    active = int(np.unique(batch.expert_ids).size)
    work = phase_work(cfg if args.infer != "base" else dataclasses.replace(cfg, rank=0), slots)
    per_step = {}
    for name, (ms, n) in phases.items():
        if n:
            per_step[name] = round(ms / args.steps, 4)
            log(f"  {name:22s} {ms / n:9.3f} ms/launch x {n / args.steps:.0f}/step")
    gemms = [p for p in work if p.startswith("gemm") and phases.get(p, (0, 0))[1]]
    dom = max(gemms, key=lambda p: phases[p][0])
    dom_ms = phases[dom][0] / phases[dom][1]
    flops, wbytes = work[dom]
    wbytes *= active
    if flops / max(wbytes, 1) > PEAK_MFMA_FP16 / PEAK_HBM:
        achieved, peak = flops / (dom_ms / 1e3) / 1e12, PEAK_MFMA_FP16 / 1e12
        roof = {"bound": "mfma", "unit": "TFLOP/s"}
    else:
        achieved, peak = wbytes / (dom_ms / 1e3) / 1e9, PEAK_HBM / 1e9
        roof = {"bound": "hbm", "unit": "GB/s"}
    # HBM bytes per launch of the dominant kernel, from the committed counter summary
    # (profiles/hbm_traffic_<phase>_<workload>.txt), only while it was taken from these sources
    from int4_quantized_moe_amd import profsum

    mode = f"_infer_{args.infer}" if args.infer else ("_recompute" if args.recompute else "")
    measured = profsum.read_traffic(os.path.join(ROOT, "profiles", f"hbm_traffic_{dom}_{cfg.name}{mode}.txt"))
    traffic = None if measured is None else int(round(measured["read"] + measured["write"]))
    roof.update({"scope": f"one kernel: {dom}, the phase with the largest time per launch (the step as a whole "
                          "is under roofline_step)",
                 "kernel": dom, "achieved": round(achieved, 2), "peak": peak, "frac": round(achieved / peak, 4),
                 "traffic": traffic, "avg_ms": round(dom_ms, 4)})
    if args.infer:  # the forward alone: gate/up and down, with their LoRA terms unless the base runs alone
        r = cfg.rank if args.infer == "lora" else 0
        total_flops = sum(work[p][0] for p in FWD_PHASES) if r else slots * 6 * cfg.hidden * cfg.intermediate
        total_wbytes = 3 * active * (cfg.hidden * cfg.intermediate // 2 + cfg.hidden * cfg.intermediate // 16)
    else:
        total_flops = slots * (12 * cfg.hidden * cfg.intermediate + 18 * cfg.rank * (cfg.hidden + cfg.intermediate))
        total_wbytes = 2 * 3 * active * (cfg.hidden * cfg.intermediate // 2 + cfg.hidden * cfg.intermediate // 16)
    # the step against the roofline that bounds it (the same flop-per-byte test as for one kernel)
    if total_flops / max(total_wbytes, 1) > PEAK_MFMA_FP16 / PEAK_HBM:
        step_bound, step_achieved = "mfma", total_flops / (ms_per_step / 1e3) / 1e12
        step_frac = step_achieved * 1e12 / PEAK_MFMA_FP16
    else:
        step_bound, step_achieved = "hbm", total_wbytes / (ms_per_step / 1e3) / 1e9
        step_frac = step_achieved * 1e9 / PEAK_HBM
    log(f"step: {total_flops / (ms_per_step / 1e3) / 1e12:.1f} TFLOP/s "
        f"({100 * total_flops / (ms_per_step / 1e3) / PEAK_MFMA_FP16:.2f}% MFMA), packed weights "
        f"{total_wbytes / (ms_per_step / 1e3) / 1e9:.1f} GB/s ({100 * total_wbytes / (ms_per_step / 1e3) / PEAK_HBM:.2f}% HBM)")

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy calibration: {args.copy_mib} MiB read, {args.copy_mib} MiB written")
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, weights, batch, args.cpu_seconds, args.infer)
        log(f"cpu baseline {cpu['value']:.2f} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC_INFER if args.infer else METRIC,
        "value": round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "experts": cfg.num_experts, "top_k": cfg.top_k, "hidden": cfg.hidden,
                   "intermediate": cfg.intermediate, "rank": cfg.rank, "alpha": cfg.alpha, "qlen": cfg.qlen,
                   "swiglu_limit": cfg.swiglu_limit, "routing": cfg.routing, "active_experts": active,
                   "weight_format": cfg.weight_format,
                   **({"mode": f"inference ({'LoRA' if args.infer == 'lora' else 'frozen base alone'})"}
                      if args.infer else {}),
                   **({"mode": "checkpoint recompute (inference forward + recompute backward)"}
                      if args.recompute else {})},
        "t_fwd_ms": round(t_fwd, 4),
        "t_bwd_ms": round(t_bwd, 4),
        "mfma_frac_step": round(total_flops / (ms_per_step / 1e3) / PEAK_MFMA_FP16, 4),
        "hbm_frac_step": round(total_wbytes / (ms_per_step / 1e3) / PEAK_HBM, 4),
        "roofline_step": {"bound": step_bound, "unit": "TFLOP/s" if step_bound == "mfma" else "GB/s",
                          "achieved": round(step_achieved, 2),
                          "peak": PEAK_MFMA_FP16 / 1e12 if step_bound == "mfma" else PEAK_HBM / 1e9,
                          "frac": round(step_frac, 4),
                          "work": "algorithmic flops of the whole step" if step_bound == "mfma"
                                  else "packed weights and scales of the active experts, once per pass"},
        "phase_ms_per_step": per_step,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
