"""Benchmark of the ZeRO partitioned mixed-precision Adam shard step on one
MI355X.

A step is the whole hot path on one data-parallel rank's shard:
flatten (per-layer fp16 grads -> flat partition) -> exact norm/overflow +
decision -> fused unscale/clip/AdamW/fp16-copy.  By default the flatten
computes the exact-norm partials while it copies and a decide-only pass
folds them (--path fused); --path separate runs the standalone norm pass
over the partition instead.  Both take bit-identical decisions.
--path accum32 runs the gradient-accumulation form: --micro-batches K
per-layer fp16 gradient sets added into an fp32 partition (the last one with
the exact-norm partials), decide, and the update reading the fp32 gradient
(30 bytes per parameter); a step is then one optimizer step over K
micro-batches.  Default workload: the largest shard that fits one GPU, the
1T-parameter model over Nd = 1024 (ZeRO paper card, "Evidence": about 16 GB
of model state per GPU), rank 512: 976,562,500 parameters from 17 per-layer
gradient segments, flattened in 40 bucket calls of 25,000,000 elements
(--workload gpt2 / 100b / tiny select the smaller shards).
Inputs (fp32 masters, per-layer fp16 gradients) are synthetic, seeded, and
resident in HBM before the timed region; four gradient sets are generated up
front and used in turn.

stdout: one JSON line.  Progress goes to stderr.
  value            whole-step parameters per second
  roofline         the Adam kernel (the dominant one): algorithmic bytes per
                   launch (28 per parameter) / its mean duration, measured with
                   HIP events on the launch stream inside the timed region,
                   against the 8 TB/s HBM peak; `traffic` is the measured HBM
                   bytes per launch from the committed rocprofv3 counter
                   summary when it was taken on the current kernel source
  cpu_baseline     the CPU oracle (single thread) on at least 3 full steps of
                   the same shard (more while --cpu-seconds lasts)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "shard Adam-step params/sec + achieved HBM GB/s (% of peak) at 1 MI355X"
HBM_PEAK_GBPS = 8000.0
ADAM_BYTES = 28          # read fp16 g + fp32 p,m,v; write fp32 p,m,v + fp16 p
ADAM32_BYTES = 30        # the same with an fp32 g
NORM_BYTES = 2           # read fp16 g
FLATTEN_BYTES = 4        # read fp16 source, write fp16 partition
WIDEN_BYTES = 6          # read fp16 source, write fp32 partition
ACCUM_BYTES = 10         # read fp16 source and fp32 partition, write fp32 partition
# 1-bit Adam compression stage, per parameter: momentum (with the worker window
# sums) 14, worker compression (with the server window sums) 16 + 1/8, server
# compression + update 26 + 1/4; the two folds read a few bytes per 4096
ONEBIT_BYTES = 14 + 16.125 + 26.25
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "zero_partitioned_mixed_flatten_amd", "csrc")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def code_text(text):
    """C/C++/HIP source with its comments removed and every run of blank space
    collapsed to one space (string and character literals kept as written), so
    that editing a comment does not count as changing a kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def code_hash(path):
    with open(path, encoding="utf-8") as f:
        return hashlib.sha256(code_text(f.read()).encode()).hexdigest()[:16]


def pmc_summary(workload):
    """The committed counter summary of a workload's shard."""
    return os.path.join(PROFILES, f"step_kernels_{workload}_shard_pmc.json")


def measured_traffic(path, n, workload):
    """HBM bytes per step of the path's roofline kernel(s) from the committed
    counter summary of the workload, or None when it is missing, for another
    shard size, for another path, or taken on other kernel sources."""
    try:
        with open(pmc_summary(workload)) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if path is None or s.get("n") != n:
        return None
    for src in s.get("sources_for", {}).get(path, []):
        if s.get("code_sha256_16", {}).get(src) != code_hash(os.path.join(CSRC, src)):
            return None
    return s.get("hbm_bytes_per_launch", {}).get(path)


CPUS_AVAILABLE = None          # set before the oracle is pinned to one core


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model, CPUS_AVAILABLE or len(os.sched_getaffinity(0))


class one_core:
    """Run the oracle pinned to one core (the process's first allowed CPU),
    then restore the affinity."""

    def __enter__(self):
        self.saved = os.sched_getaffinity(0)
        global CPUS_AVAILABLE
        CPUS_AVAILABLE = len(self.saved)
        os.sched_setaffinity(0, {min(self.saved)})
        return self

    def __exit__(self, *exc):
        os.sched_setaffinity(0, self.saved)
        return False


def cpu_baseline(w, p32, grads_host, budget_s, micro=0, min_steps=3):
    """The oracle on whole steps of the same shard: at least min_steps, then
    more until budget_s has passed (at most 20 steps).  micro > 0: the
    gradient-accumulation step over that many micro-batches."""
    import numpy as np
    import oracle as O
    import shardgen
    hp = O.hparams()
    st = O.new_state(w.scale0)
    p = p32.copy()
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    p16 = shardgen.to_f16_bits(p)
    grad = np.empty(w.n, np.float32 if micro else np.uint16)
    steps, t0 = 0, time.perf_counter()
    while True:
        if micro:
            for j in range(micro):
                O.flatten(grads_host[j], w.layout.segments, grad, accumulate=(j > 0))
            O.decide(st, hp, *O.norm_overflow_f32(grad))
            O.adam_update_f32(st, p16, p, m, v, grad)
        else:
            srcs = grads_host[steps % len(grads_host)]
            O.step(hp, st, srcs, w.layout.segments, grad, p16, p, m, v)
        steps += 1
        el = time.perf_counter() - t0
        if (el >= budget_s and steps >= min_steps) or steps >= 20:
            break
    what = (f"{micro} fp16 micro-batches accumulated in fp32 + exact fp32 norm + decision + fp32 AdamW + "
            f"fp16 copy" if micro else "flatten + exact norm + decision + fp32 AdamW + fp16 copy")
    bpp = (WIDEN_BYTES + ACCUM_BYTES * (micro - 1) + ADAM32_BYTES) if micro else (FLATTEN_BYTES + NORM_BYTES +
                                                                                   ADAM_BYTES)
    model, ncpu = cpu_info()
    return {"value": w.n * steps / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "gbps": bpp * w.n * steps / el / 1e9, "bytes_per_param": bpp, "cpu_model": model,
            "cpus_available": ncpu,
            "sample": f"{steps} full step(s) of the same {w.n:,}-parameter shard ({what}), "
                      f"single-threaded C pinned to one core, {el:.1f} s"}


def run_offload(args, w, p32, grads_host, dev_sets, hp):
    """The ZeRO-Offload form: device flatten, then the gradient down, the CPU's
    exact norm, decision and AdamW on host-resident fp32 state, the fp16
    parameters up.  Its roofline is the host update against the host's own
    streaming-copy bandwidth (measured here: the pages and the host publish no
    DRAM figure)."""
    import numpy as np
    import torch
    import zero_partitioned_mixed_flatten_amd as Z
    from zero_partitioned_mixed_flatten_amd.stepper import host_f32
    n = w.n
    huge = args.host_pages == "huge"
    dev = Z.OffloadStep(n, threads=args.threads, chunk_elems=args.chunk,
                        device_decides=(args.offload_decide == "device"), huge_pages=huge)
    dev.p32.copy_(torch.from_numpy(p32))
    dev.p16.copy_(dev.p32.half().cuda())
    dev.init_state(w.scale0)
    plans = []
    for d in dev_sets:
        dev.set_segments(d, w.layout.segments, w.bucket_elems)     # same partial plan for every set
        plans.append(dev.buckets)
    threads = dev.ctx.threads

    def one_step(k):
        dev.buckets = plans[k % len(plans)]
        dev.flatten(hp)
        dev.offload(hp)

    log(f"offload: {threads} host threads, chunk {args.chunk}; warmup {args.warmup} steps")
    for k in range(args.warmup):
        one_step(k)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_step(args.warmup + k)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    st = dev.read_state()

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps

    # the host phases alone, on the same host arrays (the state is not advanced: a copy decides)
    probe = dev.read_state()
    norm_s = timed(lambda: Z.zero_host_norm_overflow(dev.ctx.ptr, dev.host_grad16, n, hp, probe))
    adam_s = timed(lambda: Z.zero_host_adam_step(dev.ctx.ptr, dev.host_p16, dev.p32, dev.m32, dev.v32,
                                                 dev.host_grad16, n, probe))
    nbytes = (ADAM_BYTES // 2) * n // 64 * 64
    # the reference copy runs on the same kind of pages as the fp32 state
    hsrc = host_f32(nbytes // 4 + 16, huge).view(torch.uint8)
    hdst = host_f32(nbytes // 4 + 16, huge).view(torch.uint8)
    a_src = hsrc[(-hsrc.data_ptr()) % 64:][:nbytes]
    a_dst = hdst[(-hdst.data_ptr()) % 64:][:nbytes]
    copy_s = timed(lambda: Z.zero_host_stream_copy(dev.ctx.ptr, a_dst, a_src, nbytes))
    del hsrc, hdst
    d2h_s = timed(lambda: dev.host_grad16.copy_(dev.grad16, non_blocking=True))
    h2d_s = timed(lambda: dev.p16.copy_(dev.host_p16, non_blocking=True))
    host_copy_gbps = 2 * nbytes / copy_s / 1e9
    achieved = ADAM_BYTES * n / adam_s / 1e9
    log(f"step {1e3 * el / args.steps:.3f} ms; host adam {1e3 * adam_s:.2f} ms ({achieved:.0f} GB/s), host norm "
        f"{1e3 * norm_s:.2f} ms, host copy {host_copy_gbps:.0f} GB/s, D2H {2 * n / d2h_s / 1e9:.1f} GB/s, "
        f"H2D {2 * n / h2d_s / 1e9:.1f} GB/s; skipped={st.skipped_total}")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        with one_core():
            cpu = cpu_baseline(w, p32, grads_host, args.cpu_seconds)
    out = {
        "metric": METRIC,
        "value": n * args.steps / el,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * el / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.layout.model} Nd={w.layout.nd} rank {w.layout.rank} shard, offloaded step",
                   "params": n, "segments": len(w.layout.segments), "path": "offload", "host_threads": threads,
                   "chunk_elems": args.chunk, "decides": args.offload_decide, "host_pages": args.host_pages,
                   "state": "device: fp16 p, g; host: fp32 p, m, v (+ pinned fp16 g, p staging)"},
        "roofline": {"bound": "host-dram", "kernel": "host_adam_step", "achieved": achieved,
                     "peak": host_copy_gbps, "unit": "GB/s", "frac": achieved / host_copy_gbps, "traffic": None,
                     "algorithmic_bytes": ADAM_BYTES * n,
                     "peak_source": "measured host streaming copy (zero_host_stream_copy, 14 B/param, on the "
                                    "same kind of pages as the fp32 state)"},
        "phases_ms": {"host_norm_decide": 1e3 * norm_s, "host_adam": 1e3 * adam_s, "d2h_grad16": 1e3 * d2h_s,
                      "h2d_p16": 1e3 * h2d_s},
        "pcie_gbps": {"d2h": 2 * n / d2h_s / 1e9, "h2d": 2 * n / h2d_s / 1e9},
        "host_copy_gbps": host_copy_gbps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def run_onebit(args, w, p32, grads_host, dev_sets, hp):
    """1-bit Adam: two untimed warm-up steps of the ordinary fused step, then
    the timed steps of the compression stage (flatten with exact-norm
    partials, decide, zero_onebit_step).  The roofline object is the whole
    compression stage (three streaming kernels and two folds, 56.375
    algorithmic bytes per parameter); rocprofv3 gives the split."""
    import torch
    import zero_partitioned_mixed_flatten_amd as Z
    n = w.n
    stream = torch.cuda.current_stream()
    dev = Z.OneBitStep(n, warmup=2)
    dev.any_order = args.bucket_launch == "any-order"
    dev.p32.copy_(torch.from_numpy(p32))
    dev.p16.copy_(dev.p32.half())
    dev.init_state(w.scale0)
    plans = []
    for d in dev_sets:
        dev.set_segments(d, w.layout.segments, w.bucket_elems)
        plans.append(dev.buckets)
    k = 0
    while not dev.compressing():                      # the warm-up (compressing() reads the state back)
        dev.buckets = plans[k % len(plans)]
        dev.step(hp)
        k += 1
    log(f"onebit: warm-up done after {k} steps; warmup {args.warmup} compression steps")

    def one_step(i, ev=None):
        rec = (lambda j: ev[j].record(stream)) if ev is not None else (lambda j: None)
        dev.buckets = plans[i % len(plans)]
        rec(0)
        dev.flatten_norm()
        dev.decide(hp)
        rec(1)
        dev.update()                                  # the compression stage (the device chooses it)
        rec(2)

    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    st = dev.read_state()
    mean = lambda xs: sum(xs) / len(xs)
    front_ms = mean([e[0].elapsed_time(e[1]) for e in events])
    comp_ms = mean([e[1].elapsed_time(e[2]) for e in events])
    achieved = ONEBIT_BYTES * n / (comp_ms / 1e3) / 1e9
    ob = dev.read_onebit()
    log(f"step {1e3 * el / args.steps:.3f} ms; flatten+decide {1e3 * front_ms:.1f} us, compression stage "
        f"{1e3 * comp_ms:.1f} us ({achieved:.0f} GB/s); scales {ob.scale_w:.4g}/{ob.scale_s:.4g}; "
        f"skipped={st.skipped_total}")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        with one_core():
            cpu = cpu_baseline_onebit(w, p32, grads_host, args.cpu_seconds)
    out = {
        "metric": METRIC,
        "value": n * args.steps / el,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * el / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.layout.model} Nd={w.layout.nd} rank {w.layout.rank} shard, 1-bit Adam "
                               f"compression stage", "params": n, "path": "onebit", "warmup_steps": 2,
                   "state": "fp16 p, g + fp32 p, m, v (frozen) + fp32 worker/server errors + 2 x 1 bit",
                   "step_bytes_per_param": FLATTEN_BYTES + ONEBIT_BYTES},
        "roofline": {"bound": "hbm", "kernel": "onebit_step (5 kernels)", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": measured_traffic("onebit", n, args.workload),
                     "algorithmic_bytes": ONEBIT_BYTES * n},
        "kernels_us": {"flatten_norm+decide": 1e3 * front_ms, "onebit_step": 1e3 * comp_ms},
        "scales": {"worker": ob.scale_w, "server": ob.scale_s},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline_onebit(w, p32, grads_host, budget_s):
    """The oracle's compression-stage steps (after two warm-up steps, untimed)."""
    import numpy as np
    import oracle as O
    import shardgen
    hp = O.hparams()
    st = O.new_state(w.scale0)
    p = p32.copy()
    m, v, ew, es = (np.zeros_like(p) for _ in range(4))
    p16 = shardgen.to_f16_bits(p)
    grad = np.empty(w.n, np.uint16)
    for k in range(2):
        O.step(hp, st, grads_host[k % len(grads_host)], w.layout.segments, grad, p16, p, m, v)
    steps, t0 = 0, time.perf_counter()
    while True:
        O.flatten(grads_host[steps % len(grads_host)], w.layout.segments, grad)
        O.decide(st, hp, *O.norm_overflow(grad))
        O.onebit_step(st, p16, p, m, v, ew, es, grad)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 20:
            break
    model, ncpu = cpu_info()
    return {"value": w.n * steps / el, "unit": "params/s", "cores": 1, "kind": "oracle",
            "cpu_model": model, "cpus_available": ncpu,
            "sample": f"{steps} compression-stage step(s) of the same {w.n:,}-parameter shard (flatten + exact "
                      f"norm + decision + 1-bit Adam), single-threaded C pinned to one core, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="1t", choices=["tiny", "gpt2", "100b", "1t"])
    ap.add_argument("--path", default="fused", choices=["fused", "separate", "accum32", "offload", "onebit"])
    ap.add_argument("--threads", type=int, default=None,
                    help="host workers for --path offload (default: all CPUs but one)")
    ap.add_argument("--chunk", type=int, default=1 << 24, help="elements per transfer chunk for --path offload")
    ap.add_argument("--host-pages", default="huge", choices=["huge", "4k"],
                    help="--path offload: host fp32 state on transparent huge pages or on 4 KiB pages")
    ap.add_argument("--offload-decide", default="device", choices=["device", "host"],
                    help="--path offload: who reduces and decides (bit-identical either way)")
    ap.add_argument("--micro-batches", type=int, default=4,
                    help="micro-batches per optimizer step for --path accum32")
    ap.add_argument("--graph", action="store_true",
                    help="fused/separate paths: replay each step as a captured HIP graph (one per gradient set)")
    ap.add_argument("--cpu-seconds", type=float, default=30.0,
                    help="CPU-baseline budget; at least 3 whole oracle steps run whatever it is")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bucket-launch", default="any-order", choices=["any-order", "ordered"],
                    help="a bucketed partition's flattens: one call for all buckets, consecutive buckets "
                         "overlapping (any-order), or one ordered call per bucket")
    ap.add_argument("--copy-only", action="store_true",
                    help="run only the streaming-copy reference (for counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one rank's shard step on one GPU; there is no multi-GPU path (the "
              "cross-rank exchange of the step is not implemented). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import shardgen
    import zero_partitioned_mixed_flatten_amd as Z

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    w = shardgen.workload(args.workload)
    n = w.n
    stream = torch.cuda.current_stream()

    if args.copy_only:
        nbytes = (ADAM_BYTES // 2) * n // 16 * 16
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        src.view(torch.int32).random_()
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            Z.zero_stream_copy(dst, src, nbytes)
        torch.cuda.synchronize()
        log(f"copy-only: {args.warmup + args.steps} copies of {nbytes} bytes done")
        return

    log(f"workload {shardgen.layout_summary(w.layout)}")
    t = time.time()
    p32 = shardgen.master_params(w)
    nsets = 4
    grads_host = []
    for k in range(nsets):
        gpart = shardgen.grad_partition(w, k + 1, w.scale0)
        grads_host.append(shardgen.source_tensors(w.layout, gpart))
        del gpart
    log(f"inputs generated in {time.time() - t:.1f} s")

    hp = Z.hparams(w.hp.lr, w.hp.beta1, w.hp.beta2, w.hp.eps, w.hp.weight_decay, w.hp.max_grad_norm,
                   w.hp.backoff, w.hp.growth, w.hp.min_scale, w.hp.growth_interval)
    dev_sets = [[torch.from_numpy(s.view(np.float16)).cuda() for s in srcs] for srcs in grads_host]
    if args.path == "offload":
        run_offload(args, w, p32, grads_host, dev_sets, hp)
        return
    if args.path == "onebit":
        run_onebit(args, w, p32, grads_host, dev_sets, hp)
        return
    accum = args.path == "accum32"
    fused = args.path in ("fused", "accum32")
    K = args.micro_batches if accum else 1
    if accum:
        if not 1 <= K <= nsets:
            sys.exit(f"--micro-batches must be 1..{nsets}")
        dev = Z.AccumStep(n, fused=True, any_order=(args.bucket_launch == "any-order"))
        plans = [dev.plan(d, w.layout.segments, w.bucket_elems)[1] for d in dev_sets[:K]]
    else:
        dev = Z.ShardStep(n, fused=fused, any_order=(args.bucket_launch == "any-order"))
        plans = []
        for d in dev_sets:
            dev.set_segments(d, w.layout.segments, w.bucket_elems)
            plans.append(dev.buckets)
    dev.p32.copy_(torch.from_numpy(p32))
    dev.p16.copy_(dev.p32.half())
    dev.init_state(w.scale0)
    torch.cuda.synchronize()

    # events: [start, after each flatten ..., after decide/norm, after adam]
    nev = K + 3

    def one_step(k, ev=None):
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        rec(0)
        if accum:
            for j in range(K):
                if j == K - 1:
                    dev.accumulate_norm(plans[j], first=(j == 0))
                else:
                    dev.accumulate(plans[j], first=(j == 0))
                rec(1 + j)
            dev.decide(hp)
        else:
            dev.buckets = plans[k % nsets]
            if fused:
                dev.flatten_norm()
            else:
                dev.flatten()
            rec(1)
            if fused:
                dev.decide(hp)
            else:
                dev.norm_overflow(hp)
        rec(nev - 2)
        dev.adam()
        rec(nev - 1)

    graphs = None
    if args.graph and not accum:
        # one graph per gradient set, each capturing flatten(+partials), decide/norm and Adam;
        # the per-kernel split is timed afterwards on eager steps
        one_step(0)
        torch.cuda.synchronize()
        graphs = []
        side = torch.cuda.Stream()
        for k in range(nsets):
            g = torch.cuda.CUDAGraph()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    one_step(k)
            torch.cuda.current_stream().wait_stream(side)
            graphs.append(g)
        torch.cuda.synchronize()
        log(f"captured {len(graphs)} step graphs")

    log(f"warmup {args.warmup} steps")
    for k in range(args.warmup):
        if graphs:
            graphs[k % nsets].replay()
        else:
            one_step(k)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if graphs:
            graphs[(args.warmup + k) % nsets].replay()
        else:
            one_step(args.warmup + k, events[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    el = t1 - t0
    st = dev.read_state()
    mean = lambda xs: sum(xs) / len(xs)
    if graphs:                     # the split, from eager steps after the timed replays
        for k in range(args.steps):
            one_step(k, events[k])
        torch.cuda.synchronize()
    seg_all = [[e[i].elapsed_time(e[i + 1]) for e in events] for i in range(nev - 1)]
    seg_ms = [mean(x) for x in seg_all]
    median = lambda xs: sorted(xs)[len(xs) // 2]
    seg_med = [median(x) for x in seg_all]
    step_med_ms = median([e[0].elapsed_time(e[nev - 1]) for e in events])
    adam_s = seg_ms[-1] / 1e3
    adam_bpp = ADAM32_BYTES if accum else ADAM_BYTES
    achieved = adam_bpp * n / adam_s / 1e9
    if accum:
        names = [("widen" if j == 0 else "accumulate") + ("_norm" if j == K - 1 else "") for j in range(K)]
        flat_bpp = [WIDEN_BYTES if j == 0 else ACCUM_BYTES for j in range(K)]
        names += ["decide", "adam_step_f32"]
    else:
        names = ["flatten_norm" if fused else "flatten", "decide" if fused else "norm_overflow", "adam_step"]
        flat_bpp = [FLATTEN_BYTES]
    kernels_us = {}
    kernels_us_median = {}
    kernels_gbps = {}
    for i, name in enumerate(names):
        key = name if name not in kernels_us else f"{name}_{i}"
        kernels_us[key] = 1e3 * seg_ms[i]
        kernels_us_median[key] = 1e3 * seg_med[i]
        if i < len(flat_bpp):
            kernels_gbps[key] = flat_bpp[i] * n / (seg_ms[i] / 1e3) / 1e9
    if not fused:
        kernels_gbps["norm_overflow"] = NORM_BYTES * n / (seg_ms[1] / 1e3) / 1e9
    kernels_gbps[names[-1]] = achieved
    log(f"step {1e3 * el / args.steps:.3f} ms; " + ", ".join(f"{k} {v:.1f} us" for k, v in kernels_us.items())
        + f"; adam {achieved:.0f} GB/s; skipped={st.skipped_total} scale={st.loss_scale:g}")

    # streaming-copy reference on the same byte count as one Adam launch; it
    # copies random bits (a copy of zero pages measured 1.3-2% faster)
    nbytes = (ADAM_BYTES // 2) * n // 16 * 16
    csrc = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    csrc.view(torch.int32).random_()
    cdst = torch.empty_like(csrc)
    for _ in range(3):
        Z.zero_stream_copy(cdst, csrc, nbytes)
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record(stream)
    reps = 20
    for _ in range(reps):
        Z.zero_stream_copy(cdst, csrc, nbytes)
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_gbps = 2 * nbytes / (ce[0].elapsed_time(ce[1]) / 1e3 / reps) / 1e9
    del csrc, cdst

    cpu = None
    if not args.no_cpu_baseline:
        log(f"cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        with one_core():
            cpu = cpu_baseline(w, p32, grads_host, args.cpu_seconds, K if accum else 0)

    traffic = measured_traffic(args.path if (not accum or K == 4) else None, n, args.workload)
    if accum:
        step_bpp = WIDEN_BYTES + ACCUM_BYTES * (K - 1) + ADAM32_BYTES
    else:
        step_bpp = ADAM_BYTES + FLATTEN_BYTES + (0 if fused else NORM_BYTES)
    step_bytes = step_bpp * n
    workload = f"{w.layout.model} Nd={w.layout.nd} rank {w.layout.rank} shard"
    if accum:
        workload += f", {K} fp16 micro-batches accumulated in fp32"
    out = {
        "metric": METRIC,
        "value": n * args.steps / el,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * el / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": workload,
                   "params": n, "segments": len(w.layout.segments), "bucket_elems": w.bucket_elems,
                   "state": "fp16 p,g + fp32 p,m,v (16 B/param)" if not accum else
                            "fp16 p + fp32 g,p,m,v (18 B/param)", "loss_scale0": w.scale0,
                   "path": args.path, "micro_batches": K, "step_bytes_per_param": step_bpp,
                   "hip_graph": bool(graphs), "bucket_launch": args.bucket_launch},
        "roofline": {"bound": "hbm", "kernel": names[-1], "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic, "algorithmic_bytes": adam_bpp * n},
        "step_gbps": step_bytes / (el / args.steps) / 1e9,
        "step_frac": step_bytes / (el / args.steps) / 1e9 / HBM_PEAK_GBPS,
        "step_ms_median_events": step_med_ms,
        "kernels_us": kernels_us,
        "kernels_us_median": kernels_us_median,
        "kernels_gbps": kernels_gbps,
        "kernels_frac": {k: v / HBM_PEAK_GBPS for k, v in kernels_gbps.items()},
        "copy_reference_gbps": copy_gbps,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
