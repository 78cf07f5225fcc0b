"""Benchmark of the low-latency MoE dispatch + combine step on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--workload decode]

A step is one dispatch(q) + one combine(q) over one decode micro-batch, with
the parity q alternating step by step, all inputs resident in HBM. The
default workload is the decode micro-batch (128 tokens, hidden 7168, 256
experts, top-8, bf16). Prints one JSON line on stdout:

  value      effective HBM GB/s of the whole step: algorithmic bytes per step
             (what the method must move, see algorithmic_bytes()) over the
             measured time per step;
  roofline   the dominant kernel's algorithmic bytes per launch over its
             average launch time (HIP events on its stream), against the
             8 TB/s HBM peak;
  cpu_baseline  the CPU oracle on the same workload, single-threaded.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(w, md: int, routed: int) -> dict:
    """Bytes the method must move per step.
    dispatch: read x (bf16) and the routing; write the send rows and the
      routed receive rows; publish and clean the signal words.
    combine: read the routing and weights, the routed expert-output rows
      (bf16) and write the fp32 output; clean the signal words."""
    n, h, e, k = w.num_tokens, w.hidden, w.num_experts, w.topk
    dispatch = n * h * 2 + 4 * n * k + n * md + routed * md + 8 * e + 8 * e
    combine = 8 * n * k + routed * h * 2 + 4 * n * h + 8 * e
    return {"dispatch": dispatch, "combine": combine, "total": dispatch + combine}


def cpu_baseline(w, budget_s: float) -> dict:
    import oracle
    import workloads as W
    x, idx, wt = W.tokens(w), W.routing(w), W.weights(w)
    y = W.expert_outputs(w)
    img = oracle.new_image(w.capacity, w.hidden, w.num_experts, w.dtype)
    for q in (0, 1):
        oracle.clean(img, w.capacity, w.hidden, w.num_experts, w.dtype, q)
    md, _ = oracle.message_bytes(w.hidden, w.dtype)
    _, cnt = oracle.route(idx, w.num_experts, w.capacity)
    nbytes = algorithmic_bytes(w, md, int(cnt.sum()))["total"]
    steps, t0 = 0, time.perf_counter()
    while True:
        q = steps & 1
        oracle.dispatch(img, w.capacity, w.hidden, w.num_experts, w.dtype, q, x, idx)
        oracle.combine(img, w.capacity, w.hidden, w.num_experts, w.dtype, q, y, idx, wt)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s and steps >= 3:
            break
    return {"value": round(nbytes * steps / el / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{steps} full {w.name} steps (dispatch+combine) on one host core, "
                      f"{el * 1e6 / steps:.0f} us/step",
            "us_per_step": round(el * 1e6 / steps, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode")
    ap.add_argument("--batches", type=int, default=4,
                    help="distinct input batches cycled over the steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the step has no multi-GPU path in this build)", file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_ll_moe_amd as ll
    import workloads as W

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    md = ll.ll_moe_layout_offsets(w.capacity, w.hidden, w.num_experts, w.dtype, 0)["msg_bytes"]

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    batches = []
    routed = []
    for b in range(args.batches):
        wb = w.with_(seed=w.seed + b)
        idx = W.routing(wb)
        batches.append((dev_t(W.tokens(wb)), dev_t(idx), dev_t(W.weights(wb))))
        valid = (idx >= 0) & (idx < w.num_experts)
        routed.append(int(valid.sum()))
    # distinct experts per token: every pick is routed
    assert all(r == w.num_tokens * w.topk for r in routed)
    y = dev_t(W.expert_outputs(w))
    out = torch.empty((w.num_tokens, w.hidden), dtype=torch.float32, device=dev)
    total = ll.ll_moe_layout_bytes(w.capacity, w.hidden, w.num_experts, w.dtype)
    lay = torch.empty(total, dtype=torch.uint8, device=dev)
    for q in (0, 1):
        ll.ll_moe_clean_signals(lay, w.capacity, w.hidden, w.num_experts, w.dtype, q)

    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    def dispatch(s):
        x, idx, _ = batches[s % len(batches)]
        ll.ll_moe_dispatch(lay, w.capacity, w.num_tokens, w.hidden, w.num_experts, w.topk,
                           w.dtype, s & 1, x, idx, sptr)

    def combine(s):
        _, idx, wt = batches[s % len(batches)]
        ll.ll_moe_combine(lay, w.capacity, w.num_tokens, w.hidden, w.num_experts, w.topk,
                          w.dtype, s & 1, y, idx, wt, out, sptr)

    for s in range(args.warmup):
        dispatch(s)
        combine(s)
    torch.cuda.synchronize()

    # timed region: K back-to-back steps, nothing else on the stream
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for s in range(args.steps):
        dispatch(s)
        combine(s)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    print(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.2f} us/step", file=sys.stderr,
          flush=True)

    # per-kernel launch times: the same steps with an event pair around each
    # launch, on the stream the kernels run on
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        e = ev[s]
        e[0].record(stream)
        dispatch(s)
        e[1].record(stream)
        e[2].record(stream)
        combine(s)
        e[3].record(stream)
    torch.cuda.synchronize()
    d_us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    c_us = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) * 1e3
    print(f"[bench] dispatch {d_us:.2f} us/launch, combine {c_us:.2f} us/launch",
          file=sys.stderr, flush=True)

    ab = algorithmic_bytes(w, md, routed[0])
    value = ab["total"] / (ms_per_step * 1e-3) / 1e9
    dom = "dispatch" if d_us >= c_us else "combine"
    dom_us = d_us if dom == "dispatch" else c_us
    achieved = ab[dom] / (dom_us * 1e-6) / 1e9

    result = {
        "metric": "dispatch+combine effective HBM GB/s (us/step alongside)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_step": round(ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == W.BF16 else "fp8_e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "num_tokens": w.num_tokens, "hidden": w.hidden,
                   "num_experts": w.num_experts, "topk": w.topk,
                   "payload": "bf16" if w.dtype == W.BF16 else "fp8_e4m3",
                   "max_tokens": w.capacity, "parity": "alternating",
                   "algorithmic_bytes_per_step": ab["total"]},
        "fraction_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "kernels_us": {"dispatch": round(d_us, 3), "combine": round(c_us, 3)},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes_per_launch": ab[dom]},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
