"""Benchmark of the low-latency MoE dispatch + combine step on one MI355X.

    python bench.py [--gpus 1] [--steps 100] [--warmup 10] [--workload NAME]

A step is one dispatch(q) + one combine(q) over one decode micro-batch, with
the parity q alternating step by step, all inputs resident in HBM. Before the
W warm-up steps each workload runs its step untimed for --settle-ms (25 ms)
so that the part's clocks have settled: after a short warm-up alone the first
timed region of 1024 tokens ran 2-3% slower than every later one.

With no --workload the run times three workloads in one process, one after
the other, each layout freed before the next is allocated:

  worst_fill   1024 tokens, hidden 7168, 256 experts, top-8, bf16, half the
               tokens on a hot set of 8 experts: the worst-case decode batch
               the layout is sized for, and the headline;
  decode       128 tokens, hidden 7168, 256 experts, top-8, bf16;
  decode_fp8   as decode with the fp8 e4m3 dispatch payload.

It prints one JSON line on stdout. The top-level figures are the headline
workload's; "configs" holds the same block for every workload timed:

  value      effective HBM GB/s of the whole step: algorithmic bytes per step
             (what the method must move, see algorithmic_bytes()) over the
             measured time per step;
  roofline   the dominant kernel's algorithmic bytes per launch over its
             average launch time (HIP events on its stream), against the
             8 TB/s HBM peak;
  cold       the same launches after a 1 GiB read pass has evicted L2 and
             the MALL (clean lines only: no write-back overlaps them);
  floors     hand-written probes timed like the step: the dispatch's stores
             alone over its exact destination rows and the combine's gather
             alone over its exact rows, neither with routing or publish;
  ceilings   contiguous 1 GiB write / read / copy by hand-written kernels,
             and a fold reading 4 bytes per byte written (the combine's mix);
  kernel_vs_ceilings  each kernel's rate over the ceiling of its kind of
             traffic (the dispatch against write, the combine against fold);
  cpu_baseline  the CPU oracle on the headline workload, one host core.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
HOLD_CYCLES = 5_000_000
# read (not written) before every cold step: four times the 256 MB MALL
COLD_EVICT_BYTES = 1 << 30
CEILING_BYTES = 1 << 30
HEADLINE = "worst_fill"
DEFAULT_WORKLOADS = ("worst_fill", "decode", "decode_fp8")


def algorithmic_bytes(w, md: int, routed: int) -> dict:
    """Bytes the method must move per step.
    dispatch: read x (bf16) and the routing; write the send rows and the
      routed receive rows; publish and clean the signal words.
    combine: read the routing and weights, the routed expert-output rows
      (bf16) and write the fp32 output; clean the signal words."""
    n, h, e, k = w.num_tokens, w.hidden, w.num_experts, w.topk
    dispatch = n * h * 2 + 4 * n * k + n * md + routed * md + 8 * e + 8 * e
    combine = 8 * n * k + routed * h * 2 + 4 * n * h + 8 * e
    return {"dispatch": dispatch, "combine": combine, "total": dispatch + combine,
            "dispatch_writes": n * md + routed * md}


def two_phase_bytes(w, md: int, routed: int) -> dict:
    """Bytes the two-phase combine must move per step.
    send (expert side): read the counts, each routed receive row's header
      and its expert-output row (bf16); write the staging rows (combine
      messages) and raise the flags; clean the other set's words.
    recv (token side): read the routing, weights and flags, the staged
      payloads (bf16), and write the fp32 output; clean the other set."""
    n, h, e, k = w.num_tokens, w.hidden, w.num_experts, w.topk
    mc = 4 + 2 * h
    send = 8 * e + routed * 4 + routed * h * 2 + routed * mc + 8 * e + 8 * e
    recv = 8 * n * k + 8 * routed + routed * h * 2 + 4 * n * h + 8 * e
    return {"send": send, "recv": recv}


def unpack_bytes(w, md: int, routed: int) -> int:
    """Bytes the dispatch's expert side must move per launch: read the
    counts and every received message; write the header-free payload rows
    (and fp8 scale rows), the source tokens and the counts; clean the other
    set's words."""
    h, e = w.hidden, w.num_experts
    row = 2 * h if w.dtype == 0 else h + 4 * (h // 128)
    return 8 * e + routed * md + routed * (row + 4) + 4 * e + 8 * e


# kernel names in the traces (a launch matches any of its role's names): the
# dispatch runs as dispatch_direct_kernel below 64 MiB, dispatch_kernel above
KERNEL_NAMES = {"dispatch": ("dispatch_kernel<", "dispatch_direct_kernel<"),
                "combine": ("combine_kernel<",), "send": ("combine_send_kernel",),
                "recv": ("combine_recv_kernel<",), "unpack": ("dispatch_recv_kernel",)}
COUNTERS_JSON = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                             "hbm_counters.json")
# the hand-written copy that calibrates the counters: the stream probe's
# copy mode (the source is first filled by its write mode)
COPY_KERNEL = "stream_kernel<2,"


# The sources of the dispatch / combine path (launch shapes included); the
# diagnostic kernels are not part of it.
PATH_SOURCES = ("api.hip", "combine.hip", "dispatch.hip", "expert.h", "gather.h", "kernels.h",
                "layout.h", "message.h", "receive.hip", "route.h", "two_phase.hip")


def kernel_source_hash(root: str = None) -> str:
    """Hash of the path's HIP sources with comments and blank space taken
    out; stored counters apply only to the same code."""
    import hashlib
    import re
    if root is None:
        root = os.path.join(os.path.dirname(os.path.abspath(__file__)), "combine_ll_moe_amd", "csrc")
    h = hashlib.sha256()
    for name in PATH_SOURCES:
        f = os.path.join(root, name)
        h.update(name.encode())
        with open(f, encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch from the stored FETCH_SIZE / WRITE_SIZE counters,
    each scaled by what the counter read for a plain copy of known size; None
    when there are none for this workload or the kernels changed since."""
    try:
        with open(COUNTERS_JSON) as f:
            c = json.load(f)
    except OSError:
        return None
    if c.get("source_sha256") != kernel_source_hash():
        return None
    k = c.get("workloads", {}).get(workload, {}).get(kernel)
    if not k:
        return None
    cp = c["copy"]
    f_fetch = cp["fetch_kib"] * 1024.0 / cp["bytes"]
    f_write = cp["write_kib"] * 1024.0 / cp["bytes"]
    return round(k["fetch_kib"] * 1024.0 / f_fetch + k["write_kib"] * 1024.0 / f_write)


def _counter_means(path: str, counter: str) -> dict:
    import csv
    import collections
    acc = collections.defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _bench_line(log_path: str) -> dict:
    """The JSON line a bench run printed (its log)."""
    with open(log_path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                return json.loads(line)
    raise ValueError(f"{log_path}: no bench line")


def _refusals(block: dict) -> list:
    """Names of the waiting legs of a bench block that reported a refusal."""
    bad = []
    for leg in ("two_phase_combine", "expert_side"):
        if (block.get(leg) or {}).get("refusals"):
            bad.append(leg)
    return bad


def summarize_profiles(args) -> None:
    """Turn rocprofv3 CSV output into the committed summaries under profiles/:
    a markdown table per workload and the counters file bench.py reads.
    Counter runs whose bench line reported a refusal (a waiting kernel that
    gave up moves none of its bytes) are not written."""
    import csv
    prof = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")
    os.makedirs(prof, exist_ok=True)
    for log in (args.fetch_log, args.write_log):
        if log:
            bad = _refusals(_bench_line(log))
            if bad:
                raise SystemExit(f"{log}: the counter run reported refusals in {bad}; "
                                 "its counters would average launches that moved nothing")
    stats = list(csv.DictReader(open(args.trace)))
    fetch = _counter_means(args.fetch, "FETCH_SIZE")
    write = _counter_means(args.write, "WRITE_SIZE")
    cfetch = _counter_means(args.copy_fetch, "FETCH_SIZE")
    cwrite = _counter_means(args.copy_write, "WRITE_SIZE")
    copies = [k for k in cwrite if COPY_KERNEL in k]
    copy_name = max(copies, key=lambda k: cwrite[k])
    copy = {"bytes": args.copy_bytes, "kernel": copy_name,
            "fetch_kib": round(cfetch[copy_name], 1), "write_kib": round(cwrite[copy_name], 1)}
    per = {}
    for short, names in KERNEL_NAMES.items():
        fk = [k for k in fetch if any(n in k for n in names) and "probe" not in k]
        wk = [k for k in write if any(n in k for n in names) and "probe" not in k]
        if fk and wk:
            per[short] = {"kernel": fk[0], "fetch_kib": round(fetch[fk[0]], 1),
                          "write_kib": round(write[wk[0]], 1)}
    try:
        with open(COUNTERS_JSON) as f:
            c = json.load(f)
    except OSError:
        c = {}
    if c.get("source_sha256") != kernel_source_hash():
        c = {"workloads": {}}
    c["source_sha256"] = kernel_source_hash()
    c["copy"] = copy
    c.setdefault("workloads", {})[args.workload] = per
    with open(COUNTERS_JSON, "w") as f:
        json.dump(c, f, indent=1, sort_keys=True)

    import workloads as W
    w = W.WORKLOADS[args.workload]
    md = (4 + 2 * w.hidden) if w.dtype == W.BF16 else (4 + w.hidden + w.hidden // 32)
    ab = algorithmic_bytes(w, md, w.num_tokens * w.topk)
    ab.update(two_phase_bytes(w, md, w.num_tokens * w.topk))
    ab["unpack"] = unpack_bytes(w, md, w.num_tokens * w.topk)
    f_fetch = copy["fetch_kib"] * 1024.0 / copy["bytes"]
    f_write = copy["write_kib"] * 1024.0 / copy["bytes"]
    lines = [f"# {args.workload}: dispatch, combine, two-phase combine and expert-side kernels (rocprofv3)", "",
             f"Workload: {w.name}, N={w.num_tokens}, hidden={w.hidden}, experts={w.num_experts}, "
             f"top-k={w.topk}, payload {'bf16' if w.dtype == W.BF16 else 'fp8 e4m3'}.", "",
             "## Kernel durations (`--kernel-trace --stats`)", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    # the same launches split by bench.py's timed regions: each region starts
    # with the stream hold (a spin kernel); the bench line of the traced run
    # lists the regions in order
    titles = _bench_line(args.trace_log).get("profile_regions", [])
    trace = list(csv.DictReader(open(args.trace.replace("kernel_stats", "kernel_trace"))))
    segs, cur = [], None
    for r in trace:
        d_ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        # a hold spins for HOLD_CYCLES (hundreds of microseconds); the empty
        # launches of the floors are spin kernels of no length
        if "spin_kernel" in r["Kernel_Name"] and d_ns > 50_000:
            cur = {}
            segs.append(cur)
        elif cur is not None:
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            cur.setdefault(r["Kernel_Name"], []).append(d)
    if len(titles) != len(segs):
        raise SystemExit(f"{len(segs)} holds in the trace but {len(titles)} regions in the bench "
                         "line: not the same run")
    merged = {}
    for title, seg in zip(titles, segs):
        for name, ds in seg.items():
            merged.setdefault(title, {}).setdefault(name, []).extend(ds)
    lines += ["", "## The same launches by timed region of bench.py", "",
              "Each region starts after a stream hold (a spin kernel), queued behind two "
              "signal-word cleans (not listed), and runs to the next hold: the timed launches "
              "are the region's own kernel, but untimed work queued after them (warm-up "
              "steps, status checks, output fills) is listed under the same region. A receiver "
              "launched on a second stream before the hold ends waits out the hold, and its "
              "duration includes that wait. The tracer adds about 3 us to every launch (an "
              "empty launch back to back: 4.7 us traced, 1.6 us not), so launches of a few "
              "microseconds run launch-bound here; the kernel durations of the long and the "
              "dominant kernels agree with bench.py's event timings.", "",
              "| region | kernel | calls | average us |", "|---|---|---|---|"]
    for title, seg in merged.items():
        for name, ds in seg.items():
            if "clean_kernel" in name:  # the set resets queued before each hold
                continue
            lines.append(f"| {title} | `{name[:60]}` | {len(ds)} | {sum(ds) / len(ds):.2f} |")
    lines += ["", "## HBM bytes per launch (`--pmc FETCH_SIZE`, `--pmc WRITE_SIZE`)", "",
              f"Calibration: a hand-written {copy['bytes']} B device copy (`{copy_name[:60]}`) read "
              f"FETCH_SIZE {copy['fetch_kib']} KiB and WRITE_SIZE {copy['write_kib']} KiB, "
              f"factors {f_fetch:.3f} and {f_write:.3f}. The counter runs skip the "
              "overlapped-latency legs and reported no refusal, so every launch averaged "
              "moved its bytes.", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | algorithmic bytes | ratio |",
              "|---|---|---|---|---|---|"]
    for short, k in per.items():
        hbm = k["fetch_kib"] * 1024 / f_fetch + k["write_kib"] * 1024 / f_write
        lines.append(f"| {short} | {k['fetch_kib']} | {k['write_kib']} | {hbm:.0f} | {ab[short]} | "
                     f"{hbm / ab[short]:.3f} |")
    lines += ["", "## Commands", "", "```"] + args.commands + ["```", ""]
    out = os.path.join(prof, f"ll_moe_{args.workload}.md")
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print(out)


def slot_rows(idx: np.ndarray, num_experts: int, capacity: int) -> np.ndarray:
    """Expert-output / receive row e * capacity + slot of every pick, for the
    floor probes only (every pick routed, at most capacity per expert): slots
    in ascending (token, k) order per expert, by a stable sort."""
    flat = idx.ravel().astype(np.int64)
    assert ((flat >= 0) & (flat < num_experts)).all()
    order = np.argsort(flat, kind="stable")
    se = flat[order]
    start = np.searchsorted(se, se, side="left")
    slot = np.empty_like(flat)
    slot[order] = np.arange(flat.size) - start
    assert slot.max(initial=0) < capacity
    return (flat * capacity + slot).reshape(idx.shape)


class Clock:
    """Times GPU work on one stream. A short spin kernel first holds the
    stream while the timed launches are queued behind it, so the events time
    the GPU running them back to back, not the host's launch rate. Every
    hold is preceded by `reset` (the signal-word cleans) and recorded under
    a region name, in order, for the profile summaries."""

    def __init__(self, torch, stream, reset):
        self.torch, self.stream, self.reset = torch, stream, reset
        self.regions = []

    def hold(self, region: str, prepare=None):
        self.reset()
        if prepare is not None:
            prepare()
        self.torch.cuda._sleep(HOLD_CYCLES)
        self.regions.append(region)

    def per_call(self, region: str, fn, count: int, prepare=None) -> float:
        """Average microseconds of fn(s), s = 0..count-1, back to back."""
        torch = self.torch
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        self.hold(region, prepare)
        a.record(self.stream)
        for s in range(count):
            fn(s)
        b.record(self.stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / count


def ceilings(torch, ll, clock: Clock) -> dict:
    """Contiguous 1 GiB write, read and copy by the hand-written stream
    probe, and its fold of 1 GiB read into 256 MiB written (4:1, the
    combine's mix), best over a few grid sizes and both load/store hints:
    the part's practical HBM rates for this kind of access."""
    dev = torch.device("cuda:0")
    a = torch.empty(CEILING_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty(CEILING_BYTES, dtype=torch.uint8, device=dev)
    ll.ll_moe_diag_stream(ll.PROBE_WRITE, False, a, None, CEILING_BYTES, 4096)
    torch.cuda.synchronize()
    res = {}
    # (mode, name, bytes written or read, bytes moved per byte of that):
    # fold4 reads the whole 1 GiB into a quarter of it, the combine's mix
    for mode, name, nbytes, moved in (
            (ll.PROBE_WRITE, "write", CEILING_BYTES, 1), (ll.PROBE_READ, "read", CEILING_BYTES, 1),
            (ll.PROBE_COPY, "copy", CEILING_BYTES, 2),
            (ll.PROBE_FOLD4, "fold4", CEILING_BYTES // 4, 5)):
        best = None
        for nt in (False, True):
            for blocks in (4096, 16384, 65536):
                us = clock.per_call(f"ceiling {name} nt={int(nt)} blocks={blocks}",
                                    lambda s: ll.ll_moe_diag_stream(mode, nt, b, a, nbytes,
                                                                    blocks), 5)
                gbs = moved * nbytes / (us * 1e-6) / 1e9
                if best is None or gbs > best["gbs"]:
                    best = {"gbs": round(gbs, 1), "us": round(us, 2), "non_temporal": nt,
                            "blocks": blocks}
        res[name] = best
    res["bytes"] = CEILING_BYTES
    del a, b
    torch.cuda.empty_cache()
    return res


def measure(name: str, args, torch, ll, W) -> dict:
    """Every figure of one workload; frees its device memory before
    returning."""
    w = W.WORKLOADS[name]
    dev = torch.device("cuda:0")
    md = ll.ll_moe_layout_offsets(w.capacity, w.hidden, w.num_experts, w.dtype, 0)["msg_bytes"]

    def dev_t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(dev)

    batches, routed, idx_host = [], [], []
    most = np.zeros(w.num_experts, np.int64)
    for b in range(args.batches):
        wb = w.with_(seed=w.seed + b)
        idx = W.routing(wb)
        batches.append((dev_t(W.tokens(wb)), dev_t(idx), dev_t(W.weights(wb))))
        idx_host.append(idx)
        valid = (idx >= 0) & (idx < w.num_experts)
        routed.append(int(valid.sum()))
        most = np.maximum(most, np.bincount(idx[valid].ravel(), minlength=w.num_experts))
    # distinct experts per token: every pick is routed
    assert all(r == w.num_tokens * w.topk for r in routed)
    # expert outputs on the rows some batch fills, the NaN poison elsewhere
    filled = np.zeros(w.num_experts * w.capacity, bool)
    for e in range(w.num_experts):
        filled[e * w.capacity:e * w.capacity + min(int(most[e]), w.capacity)] = True
    y = dev_t(W.expert_outputs(w, filled))
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

    def step(s):
        dispatch(s)
        combine(s)

    def reset_sets():
        # every timed region starts from clean signal words (a dispatch of
        # set q needs set q's words at zero) and runs parity 0, 1, ...
        for q in (0, 1):
            ll.ll_moe_clean_signals(lay, w.capacity, w.hidden, w.num_experts, w.dtype, q, sptr)

    clock = Clock(torch, stream, reset_sets)
    say = lambda msg: print(f"[bench {name}] {msg}", file=sys.stderr, flush=True)

    # untimed: steps for settle_ms of wall time (whole pairs of parities),
    # then the W warm-up steps
    t_settle = time.perf_counter() + args.settle_ms * 1e-3
    settle_steps = 0
    while time.perf_counter() < t_settle:
        for s in range(20):
            step(s)
        torch.cuda.synchronize()
        settle_steps += 20
    reset_sets()
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    # K back-to-back steps, nothing else between them
    step_us = clock.per_call("dispatch + combine steps", step, args.steps)
    say(f"{args.steps} steps: {step_us:.2f} us/step")

    # per-kernel launch times: K launches of one kernel back to back (parity
    # alternating, as in the step), timed on the stream they run on
    d_us = clock.per_call("dispatch back to back (roofline timing)", dispatch, args.steps)
    c_us = clock.per_call("combine back to back (roofline timing)", combine, args.steps)
    say(f"dispatch {d_us:.2f} us/launch, combine {c_us:.2f} us/launch")

    # the same steps captured once as a HIP graph and replayed back to back
    # (an even number of them, so that every replay starts on a clean set 0)
    graph_us = None
    if not args.no_graph:
        gsteps = args.steps + (args.steps & 1)
        reset_sets()
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                gs = torch.cuda.current_stream().cuda_stream
                for s in range(gsteps):
                    x, idx, wt = batches[s % len(batches)]
                    ll.ll_moe_dispatch(lay, w.capacity, w.num_tokens, w.hidden, w.num_experts,
                                       w.topk, w.dtype, s & 1, x, idx, gs)
                    ll.ll_moe_combine(lay, w.capacity, w.num_tokens, w.hidden, w.num_experts,
                                      w.topk, w.dtype, s & 1, y, idx, wt, out, gs)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / gsteps
            best = us if best is None else min(best, us)
        graph_us = best
        del g
        say(f"graph replay: {graph_us:.2f} us/step")

    # repeated trials of the same K steps: spread of the step time
    trials = [clock.per_call("dispatch + combine steps (trial)", step, args.steps)
              for _ in range(args.trials)]

    # the two-phase combine on the same batches: a step is dispatch(q),
    # combine_send(q), combine_recv(q); then each side alone, K launches
    # back to back on one set (the expert side re-stages the same rows, its
    # flags counting past the counts; the token side re-folds raised flags)
    two_phase = None
    if not args.no_two_phase:
        # one caller-zeroed status word per token-side call
        nwords = max(args.steps, args.warmup) + 1
        tp_status = torch.zeros(nwords, dtype=torch.int32, device=dev)
        spins = 1 << 20

        def send(s):
            ll.ll_moe_combine_send(lay, w.capacity, w.hidden, w.num_experts, w.dtype, s & 1, y,
                                   sptr)

        def recv(s, word):
            _, idx, wt = batches[s % len(batches)]
            ll.ll_moe_combine_recv(lay, w.capacity, w.num_tokens, w.hidden, w.num_experts,
                                   w.topk, w.dtype, s & 1, idx, wt, out, spins,
                                   tp_status[word:word + 1], sptr)

        def tp_step(s, word=None):
            dispatch(s)
            send(s)
            recv(s, s if word is None else word)

        def prepared_set0():
            tp_status.zero_()
            tp_step(0, nwords - 1)  # set 0: one step's counts and flags

        def all_ready(n):
            torch.cuda.synchronize()
            return bool(((tp_status[:n] & ~ll.RECV_WAITED) == ll.RECV_READY).all().item())

        reset_sets()
        tp_status.zero_()
        for s in range(args.warmup):
            tp_step(s)
        tp_ok = all_ready(args.warmup)
        tp_us = clock.per_call("two-phase steps (dispatch, combine_send, combine_recv)", tp_step,
                               args.steps, prepare=tp_status.zero_)
        tp_ok = tp_ok and all_ready(args.steps)
        send_us = clock.per_call("combine_send back to back on one set (after one step "
                                 "preparing set 0)", lambda s: send(0), args.steps,
                                 prepare=prepared_set0)
        recv_us = clock.per_call("combine_recv back to back on one set (after one step "
                                 "preparing set 0)", lambda s: recv(0, s), args.steps,
                                 prepare=prepared_set0)
        tp_ok = tp_ok and all_ready(args.steps)
        reset_sets()
        torch.cuda.synchronize()
        tb = two_phase_bytes(w, md, routed[0])
        two_phase = {
            "us_per_step": round(tp_us, 3),
            "fused_us_per_step": round(step_us, 3),
            "send_us": round(send_us, 3), "recv_us": round(recv_us, 3),
            "send_gbs": round(tb["send"] / (send_us * 1e-6) / 1e9, 2),
            "recv_gbs": round(tb["recv"] / (recv_us * 1e-6) / 1e9, 2),
            "bytes_per_launch": tb, "refusals": not tp_ok,
            "traffic": {"send": stored_traffic(w.name, "send"),
                        "recv": stored_traffic(w.name, "recv")}}
        say(f"two-phase: {tp_us:.2f} us/step (send {send_us:.2f}, recv {recv_us:.2f}); "
            f"fused {step_us:.2f}")

    # the dispatch's expert side (ll_moe_dispatch_recv): alone, K launches on
    # one prepared set; then (unless --no-latency) the latency from the
    # dispatch's start to the unpacked expert inputs, with the receiver
    # queued after the dispatch on the same stream, or already waiting on a
    # second stream (overlapped)
    expert_side = None
    if not args.no_expert_side:
        rows = w.num_experts * w.capacity
        pb = 2 * w.hidden if w.dtype == W.BF16 else w.hidden
        u_payload = torch.empty((rows, pb), dtype=torch.uint8, device=dev)
        u_scales = (torch.empty((rows, w.hidden // 128), dtype=torch.float32, device=dev)
                    if w.dtype == W.FP8_E4M3 else None)
        u_src = torch.empty(rows, dtype=torch.int32, device=dev)
        u_counts = torch.empty(w.num_experts, dtype=torch.int32, device=dev)
        # one caller-zeroed status word per call
        u_nwords = max(args.steps, args.warmup) + 1
        u_status = torch.zeros(u_nwords, dtype=torch.int32, device=dev)
        side = torch.cuda.Stream()
        u_ok = True

        def unpack(s, word, st=None):
            ll.ll_moe_dispatch_recv(lay, w.capacity, w.hidden, w.num_experts, w.dtype, s & 1,
                                    routed[s % len(batches)], u_payload, u_scales, u_src,
                                    u_counts, 1 << 20, u_status[word:word + 1],
                                    sptr if st is None else st)

        def u_ready(n):
            torch.cuda.synchronize()
            return bool(((u_status[:n] & ~ll.RECV_WAITED) == ll.RECV_READY).all().item())

        def u_prepare():
            u_status.zero_()
            dispatch(0)

        reset_sets()
        u_status.zero_()
        for s in range(args.warmup):
            dispatch(s)
            unpack(s, s)
        u_ok = u_ready(args.warmup)
        unpack_us = clock.per_call("dispatch_recv back to back on one prepared set",
                                   lambda s: unpack(0, s), args.steps, prepare=u_prepare)
        u_ok = u_ok and u_ready(args.steps)
        seq_step_us = clock.per_call("dispatch + dispatch_recv steps on one stream",
                                     lambda s: (dispatch(s), unpack(s, s)), args.steps,
                                     prepare=u_status.zero_)
        u_ok = u_ok and u_ready(args.steps)

        waited = {"same_stream": 0, "overlapped": 0}

        def latency(overlapped: bool, trials: int = 20):
            nonlocal u_ok
            res = []
            for i in range(trials):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                reset_sets()
                u_status.zero_()
                side.wait_stream(stream)  # after the reset and the zeroing, before the hold
                torch.cuda._sleep(HOLD_CYCLES)
                clock.regions.append("dispatch start to expert inputs: dispatch_recv "
                                     + ("already waiting on a second stream"
                                        if overlapped else "queued after the dispatch"))
                a.record(stream)
                dispatch(i)
                if overlapped:
                    unpack(i, 0, side.cuda_stream)
                    b.record(side)
                else:
                    unpack(i, 0)
                    b.record(stream)
                torch.cuda.synchronize()
                u_ok = u_ok and u_ready(1)
                if int(u_status[0].item()) & ll.RECV_WAITED:
                    waited["overlapped" if overlapped else "same_stream"] += 1
                res.append(a.elapsed_time(b) * 1e3)
            return float(np.median(res))

        lat = None
        if not args.no_latency:
            lat = {"same_stream": round(latency(False), 3), "overlapped": round(latency(True), 3),
                   "trials": 20, "receiver_waited": waited}
        torch.cuda.synchronize()
        ub = unpack_bytes(w, md, routed[0])
        expert_side = {
            "unpack_us": round(unpack_us, 3),
            "unpack_gbs": round(ub / (unpack_us * 1e-6) / 1e9, 2),
            "bytes_per_launch": ub,
            "sequential_steps_us": round(seq_step_us, 3),
            "dispatch_to_inputs_us": lat,
            "refusals": not u_ok,
            "traffic": stored_traffic(w.name, "unpack")}
        say(f"expert side: unpack {unpack_us:.2f} us; dispatch start to expert inputs {lat}")
        del u_payload, u_scales, u_src, u_counts

    # cold launches: before every step a 1 GiB read pass evicts L2 and the
    # 256 MB MALL. A read leaves only clean lines behind, so no write-back of
    # its own overlaps the timed launches (the dirty lines of the step before
    # are written back while it reads). Event pairs time each launch; the
    # same event pairs without the eviction give this method's warm figure
    # (event pairs add a little to each launch, so compare the two).
    cold = None
    if args.cold_steps > 0:
        scratch = torch.empty(COLD_EVICT_BYTES, dtype=torch.uint8, device=dev)
        sink = torch.zeros(16, dtype=torch.uint8, device=dev)
        ll.ll_moe_diag_stream(ll.PROBE_WRITE, False, scratch, None, COLD_EVICT_BYTES, 4096)
        torch.cuda.synchronize()

        def per_launch(evict):
            # every step queued behind the stream hold, so the GPU runs
            # eviction, events and launches back to back, without host gaps
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                  for _ in range(args.cold_steps)]
            torch.cuda.synchronize()
            clock.hold("cold: after a 1 GiB read pass, event pairs between launches" if evict
                       else "warm: the same event pairs between launches")
            for s in range(args.cold_steps):
                if evict:
                    ll.ll_moe_diag_stream(ll.PROBE_READ, False, sink, scratch, COLD_EVICT_BYTES,
                                          4096)
                ev[s][0].record(stream)
                dispatch(s)
                ev[s][1].record(stream)
                combine(s)
                ev[s][2].record(stream)
            torch.cuda.synchronize()
            ds = [e[0].elapsed_time(e[1]) * 1e3 for e in ev]
            cs = [e[1].elapsed_time(e[2]) * 1e3 for e in ev]
            return float(np.median(ds)), float(np.median(cs))

        cd, cc = per_launch(True)
        wd, wc = per_launch(False)
        ab0 = algorithmic_bytes(w, md, routed[0])
        cold = {"method": f"{COLD_EVICT_BYTES >> 20} MiB read pass (clean lines only) before "
                          "every step; median of per-launch event pairs",
                "evict_bytes": COLD_EVICT_BYTES, "steps": args.cold_steps,
                "us_per_step": round(cd + cc, 3), "dispatch_us": round(cd, 3),
                "combine_us": round(cc, 3),
                "fraction_of_hbm_peak": round(ab0["total"] / ((cd + cc) * 1e-6) / 1e9 /
                                              HBM_PEAK_GBS, 4),
                "warm_same_method": {"us_per_step": round(wd + wc, 3),
                                     "dispatch_us": round(wd, 3), "combine_us": round(wc, 3)}}
        say(f"cold (after a {COLD_EVICT_BYTES >> 20} MiB read pass): dispatch {cd:.2f} us, "
            f"combine {cc:.2f} us; warm with the same event pairs: {wd:.2f} / {wc:.2f} us")
        del scratch, sink

    ab = algorithmic_bytes(w, md, routed[0])

    # floors: the dispatch's stores alone over its exact destination rows
    # and the combine's gather alone over its exact rows (hand-written
    # probes built on the kernels' own store and gather code), and an empty
    # launch, each timed like the step
    floors = None
    if not args.no_floors:
        rows_q = []
        for q in (0, 1):
            o = ll.ll_moe_layout_offsets(w.capacity, w.hidden, w.num_experts, w.dtype, q)
            per_tok = []
            for b in range(len(batches)):
                r = slot_rows(idx_host[b], w.num_experts, w.capacity)
                offs = np.empty((w.num_tokens, w.topk + 1), np.int64)
                offs[:, 0] = o["send"] + np.arange(w.num_tokens) * md
                offs[:, 1:] = o["recv"] + r * md
                per_tok.append(torch.from_numpy(offs.ravel().copy()).to(dev))
            rows_q.append(per_tok)
        gather_rows = [torch.from_numpy(slot_rows(i, w.num_experts, w.capacity)
                                        .astype(np.int32)).to(dev) for i in idx_host]
        nrows = w.num_tokens * (w.topk + 1)
        per = max(1, min(w.topk + 1, nrows // 512))
        line = nrows * md >= 64 << 20  # the dispatch's whole-line rule

        def store_rows(s, rows_mode, policy=ll.PROBE_SC1):
            ll.ll_moe_diag_store_rows(lay, rows_q[s & 1][s % len(batches)], nrows, md, per,
                                      line, rows_mode, policy, sptr)

        def gather(s):
            _, _, wt = batches[s % len(batches)]
            ll.ll_moe_diag_gather_rows(y, w.num_experts * w.capacity, w.hidden,
                                       gather_rows[s % len(batches)], wt, w.num_tokens, w.topk,
                                       out, sptr)

        # the dispatch's store routines: from LDS by workgroup or by
        # wavefront, and straight from registers
        st_group = clock.per_call("floor: dispatch's stores alone, rows by workgroup "
                                  "(store_rows probe)",
                                  lambda s: store_rows(s, ll.PROBE_ROWS_GROUP), args.steps)
        st_wave = clock.per_call("floor: dispatch's stores alone, rows by wavefront "
                                 "(store_rows probe)",
                                 lambda s: store_rows(s, ll.PROBE_ROWS_WAVE), args.steps)
        st_direct = clock.per_call("floor: dispatch's stores alone, rows from registers "
                                   "(store_rows probe)",
                                   lambda s: store_rows(s, ll.PROBE_ROWS_DIRECT), args.steps)
        st_us, best_rows = min((st_group, ll.PROBE_ROWS_GROUP), (st_wave, ll.PROBE_ROWS_WAVE),
                               (st_direct, ll.PROBE_ROWS_DIRECT))
        ga_us = clock.per_call("floor: combine's gather alone (gather_rows probe)", gather,
                               args.steps)
        both_us = clock.per_call("floor: store_rows + gather_rows steps",
                                 lambda s: (store_rows(s, best_rows), gather(s)), args.steps)
        empty_us = clock.per_call("floor: empty launches", lambda s: torch.cuda._sleep(0),
                                  args.steps)
        # the same stores with other cache policies (context for the
        # write-through choice)
        policies = {}
        for pname, pol in (("write_back", ll.PROBE_WRITE_BACK), ("nt", ll.PROBE_NT),
                           ("sc1_nt", ll.PROBE_SC1_NT)):
            policies[pname] = round(clock.per_call(
                f"floor: dispatch's stores alone, {pname} stores",
                lambda s: store_rows(s, best_rows, pol), args.steps), 3)
        floors = {
            "store_rows_us": round(st_us, 3), "store_rows_bytes": ab["dispatch_writes"],
            "store_rows_by_workgroup_us": round(st_group, 3),
            "store_rows_by_wavefront_us": round(st_wave, 3),
            "store_rows_from_registers_us": round(st_direct, 3),
            "store_rows_per_workgroup": per,
            "gather_us": round(ga_us, 3), "gather_bytes": ab["combine"],
            "store_then_gather_us_per_step": round(both_us, 3),
            "empty_launch_us": round(empty_us, 3),
            "store_rows_other_policies_us": policies,
            "step_us_at_60pct": round(ab["total"] / (0.6 * HBM_PEAK_GBS * 1e9) * 1e6, 3)}
        say(f"floors: stores alone {st_group:.2f} (rows by workgroup) / {st_wave:.2f} "
            f"(by wavefront) / {st_direct:.2f} (from registers) us, gather alone {ga_us:.2f} us, both as steps "
            f"{both_us:.2f} us/step, empty launch {empty_us:.2f} us; other store policies "
            f"{policies}")
        del rows_q, gather_rows

    dom = "dispatch" if d_us >= c_us else "combine"
    dom_us = d_us if dom == "dispatch" else c_us
    achieved = ab[dom] / (dom_us * 1e-6) / 1e9
    gbs = ab["total"] / (step_us * 1e-6) / 1e9
    res = {
        "config": {"workload": w.name, "num_tokens": w.num_tokens, "hidden": w.hidden,
                   "num_experts": w.num_experts, "topk": w.topk,
                   "payload": "bf16" if w.dtype == W.BF16 else "fp8_e4m3",
                   "max_tokens": w.capacity, "parity": "alternating",
                   "algorithmic_bytes_per_step": ab["total"]},
        "dtype": "bf16" if w.dtype == W.BF16 else "fp8_e4m3+bf16",
        "us_per_step": round(step_us, 3),
        "value": round(gbs, 2),
        "fraction_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "kernels_us": {"dispatch": round(d_us, 3), "combine": round(c_us, 3)},
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "graph_us_per_step": None if graph_us is None else round(graph_us, 3),
        "step_trials_us": {"n": len(trials),
                           "median": round(float(np.median(trials)), 3) if trials else None,
                           "min": round(min(trials), 3) if trials else None},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(w.name, dom),
                     "bytes_per_launch": ab[dom], "us_per_launch": round(dom_us, 3)},
        "kernel_fracs": {k: round(ab[k] / (u * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
                         for k, u in (("dispatch", d_us), ("combine", c_us))},
        "cold": cold,
        "floors": floors,
        "two_phase_combine": two_phase,
        "expert_side": expert_side,
    }
    if args.regions:
        res["profile_regions"] = list(clock.regions)
    del batches, y, out, lay
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


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
            "sample": f"{steps} full {w.name} steps (dispatch+combine) on one host core "
                      f"(of {os.cpu_count()} host threads), {el * 1e6 / steps:.0f} us/step",
            "us_per_step": round(el * 1e6 / steps, 1),
            "host_cpu": _host_cpu(), "host_threads": os.cpu_count()}


def _host_cpu() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=25.0,
                    help="untimed steps for this long before the warm-up steps (clocks settle)")
    ap.add_argument("--workload", default=None,
                    help="time one workload only (default: worst_fill, decode and decode_fp8, "
                         "worst_fill the headline)")
    ap.add_argument("--batches", type=int, default=4,
                    help="distinct input batches cycled over the steps")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--trials", type=int, default=7,
                    help="further timed repetitions of the K steps (median and min reported)")
    ap.add_argument("--no-floors", action="store_true",
                    help="skip the hand-written floor probes (stores alone, gather alone)")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the contiguous write / read / copy ceilings")
    ap.add_argument("--no-two-phase", action="store_true",
                    help="skip the two-phase combine timings")
    ap.add_argument("--no-expert-side", action="store_true",
                    help="skip the expert-side receive timings")
    ap.add_argument("--no-latency", action="store_true",
                    help="skip the dispatch-to-expert-inputs latency legs (their waiting "
                         "receivers refuse when a profiler serializes kernels)")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="steps timed after evicting L2 and MALL (0: skip)")
    ap.add_argument("--regions", action="store_true",
                    help="list the timed regions in the JSON line (for profile summaries)")
    ap.add_argument("--summarize-profiles", action="store_true",
                    help="write profiles/ summaries from rocprofv3 CSV files (no GPU)")
    ap.add_argument("--trace")
    ap.add_argument("--trace-log")
    ap.add_argument("--fetch")
    ap.add_argument("--fetch-log")
    ap.add_argument("--write")
    ap.add_argument("--write-log")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-bytes", type=int, default=0)
    ap.add_argument("--commands", nargs="*", default=[])
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run the hand-written device copy of BYTES five times "
                         "(calibrates the HBM byte counters against a known size)")
    args = ap.parse_args()

    if args.summarize_profiles:
        summarize_profiles(args)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the step has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    import combine_ll_moe_amd as ll
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_probe:
        nbytes = args.copy_probe - args.copy_probe % 16
        a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        ll.ll_moe_diag_stream(ll.PROBE_WRITE, False, a, None, nbytes, 4096)
        torch.cuda.synchronize()
        for _ in range(5):
            ll.ll_moe_diag_stream(ll.PROBE_COPY, False, b, a, nbytes, 4096)
        torch.cuda.synchronize()
        print(f"[copy-probe] copied {nbytes} bytes 5 times", file=sys.stderr)
        return

    names = [args.workload] if args.workload else list(DEFAULT_WORKLOADS)
    for n in names:
        if n not in W.WORKLOADS:
            raise SystemExit(f"unknown workload {n}; known: {sorted(W.WORKLOADS)}")
    headline = names[0] if args.workload else HEADLINE

    results = {}
    for n in names:
        results[n] = measure(n, args, torch, ll, W)

    ceil = None
    if not args.no_ceilings:
        reset = lambda: None
        clock = Clock(torch, torch.cuda.current_stream(), reset)
        ceil = ceilings(torch, ll, clock)
        print(f"[bench] ceilings: {ceil}", file=sys.stderr, flush=True)
        # each kernel's algorithmic rate against the practical ceiling of
        # its kind of traffic: the dispatch mostly writes (for 1024 tokens of
        # 7168 columns, 14.7 of its 146.9 MB are reads of x); the combine
        # reads 4 bytes per byte written at top-k 8, as the fold does
        for r in results.values():
            f = r["kernel_fracs"]
            r["kernel_vs_ceilings"] = {
                "dispatch_vs_write": round(f["dispatch"] * HBM_PEAK_GBS / ceil["write"]["gbs"], 4),
                "combine_vs_fold4": round(f["combine"] * HBM_PEAK_GBS / ceil["fold4"]["gbs"], 4)}

    h = results[headline]
    result = {
        "metric": "dispatch+combine effective HBM GB/s (us/step alongside)",
        "value": h["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": h["settle"],
        "ms_per_step": round(h["us_per_step"] * 1e-3, 6),
        "us_per_step": h["us_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic",
        "config": h["config"],
        "fraction_of_hbm_peak": h["fraction_of_hbm_peak"],
        "kernels_us": h["kernels_us"],
        "graph_us_per_step": h["graph_us_per_step"],
        "step_trials_us": h["step_trials_us"],
        "cold": h["cold"],
        "floors": h["floors"],
        "two_phase_combine": h["two_phase_combine"],
        "expert_side": h["expert_side"],
        "roofline": h["roofline"],
        "kernel_vs_ceilings": h.get("kernel_vs_ceilings"),
        "cpu_baseline": None,
        "configs": {n: {k: v for k, v in r.items() if k != "profile_regions"}
                    for n, r in results.items()},
        "ceilings": ceil,
    }
    if args.regions:
        result["profile_regions"] = h.get("profile_regions", [])
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(W.WORKLOADS[headline], args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
