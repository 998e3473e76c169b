#!/usr/bin/env python3
"""Benchmark: one ZeRO rank's partitioned mixed-precision AdamW shard step on
one MI355X.

A step is the whole hot path on this rank's shard, through the C ABI:
  unscale + inf/NaN detection + squared norm (two kernels; the second also
  forms the step's coefficients and advances the loss scaler and step counter
  kept in device memory), then the fused AdamW update with clipping and
  16-bit parameter writeback (one kernel).  No step waits for the host.
  --host-scaler instead reads the 4-byte overflow flag back every step and
  updates the loss scale and step counter on the host.
Inputs are seeded synthetic values uploaded to HBM before timing.

Prints one JSON line.  `value` is params/s of the whole step; `roofline`
reports the fused AdamW kernel (the dominant one) against MI355X's 8 TB/s HBM
peak, from HIP events recorded on the stream it runs on.  On the default
path the 100B model's 250M-parameter rank shard is timed afterwards the same
way and reported under `extra_workload`; `value` stays the first shard's.
"""
import argparse
import contextlib
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0              # MI355X HBM3E, published
ADAM_BYTES_PER_PARAM = 28           # 2 grad + 3x4 read + 3x4 write + 2 param
NORM_BYTES_PER_PARAM = 2            # gradient read once
STEP_BYTES_PER_PARAM = ADAM_BYTES_PER_PARAM + NORM_BYTES_PER_PARAM
# fp32 gradient-accumulation path: the step reads the 4-byte fp32 copy
ADAM_F32_BYTES_PER_PARAM = 30
NORM_F32_BYTES_PER_PARAM = 4
ACC_FIRST_BYTES_PER_PARAM = 6       # 2 read + 4 written
ACC_BYTES_PER_PARAM = 10            # 2 + 4 read, 4 written
METRIC = "shard optimizer-step params/sec and achieved HBM GB/s (% of peak), 1 MI355X"
KERNEL_SRC = os.path.join(ROOT, "zero_sharded_mixed_partition_amd", "csrc", "shard_step.hip")
COUNTERS = os.path.join(ROOT, "profiles", "hbm_counters.json")


def code_hash(text: str) -> str:
    """sha256[:16] of C/HIP source with its comments and blank lines removed,
    so that the counter summaries stay tied to the code, not to its comments."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, encoding="utf-8") as f:
        return code_hash(f.read())


def measured_traffic(key: str, kernel: str = "adam_update"):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary for run `key`, or None if absent or taken on a different kernel
    source."""
    try:
        with open(COUNTERS) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(kernel, {}).get(key)
    if not rec or rec.get("kernel_code_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def upload_inputs(w, begin, S, grad_dtype, block_chunks=16):
    """Generate the shard's seeded inputs block by block and copy them to HBM."""
    import numpy as np
    import torch

    import workloads as W
    dev = "cuda"
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[grad_dtype]
    P = torch.empty(S, dtype=torch.float32, device=dev)
    M = torch.empty(S, dtype=torch.float32, device=dev)
    V = torch.empty(S, dtype=torch.float32, device=dev)
    G = torch.empty(S, dtype=tdt, device=dev)
    blk = block_chunks * W.CHUNK
    for lo in range(0, S, blk):
        cnt = min(blk, S - lo)
        for name, dst in (("master", P), ("exp_avg", M), ("exp_avg_sq", V)):
            dst[lo:lo + cnt].copy_(torch.from_numpy(W.fill(w, name, begin + lo, cnt)))
        g = W.fill(w, "grad", begin + lo, cnt, step=w.step)
        G[lo:lo + cnt].copy_(torch.from_numpy(g.view(np.int16)).view(tdt))
        print(f"# uploaded {lo + cnt}/{S} elements", file=sys.stderr, flush=True)
    return P, M, V, G


def _oracle_block(w, lo, n, accum, threads=0, reduce=0):
    """Seconds of oracle time for one full step (exact norm + AdamW; with
    `accum` > 0, that many micro-batch accumulations into the fp32 copy
    first; with `reduce` > 0, the reduction of that many ranks' slices into
    it) on flat parameters [lo, lo+n); input generation excluded."""
    import oracle
    import workloads as W

    p, m, v, g = W.shard_inputs(w, lo, n, threads=threads)
    t0 = time.perf_counter()
    gfmt, ginv = w.grad_dtype, 1.0 / w.loss_scale
    if accum:
        acc = None
        for _ in range(accum):
            acc, _ovf = oracle.grad_accumulate(acc, g, w.grad_dtype, ginv)
        g, gfmt, ginv = acc, "f32", 1.0
    elif reduce:
        acc, _ovf = oracle.grad_reduce([g] * reduce, w.grad_dtype, ginv)
        g, gfmt, ginv = acc, "f32", 1.0
    sq, ovf = oracle.shard_sqnorm_overflow(g, gfmt, ginv)
    oracle.shard_step(p, m, v, g, gfmt, w.param_dtype, global_sq=sq, global_overflow=ovf,
                      inv_loss_scale=ginv, max_grad_norm=w.max_grad_norm, lr=w.lr, beta1=w.beta1,
                      beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay, step=w.step)
    return time.perf_counter() - t0


def _oracle_worker(job):
    """One process of the all-cores leg: its blocks one after another, one thread."""
    w, blocks, accum, reduce = job
    if w.grad_dtype == "bf16":          # the bf16 input cast goes through torch's CPU kernels
        import torch
        torch.set_num_threads(1)
    spent = 0.0
    for lo, n in blocks:
        spent += _oracle_block(w, lo, n, accum, threads=1, reduce=reduce)
    return sum(n for _, n in blocks), spent


def cpu_baseline(w, begin, S, accum=0, target_s=10.0, block=1 << 24, par_block=1 << 22, reduce=0, per_proc=6):
    """The CPU oracle timed on a bounded sample of the same shard, blocks of
    consecutive parameters from its start, one step per block:
      all cores  one process per host core this process may run on (its
                 affinity set), `per_proc` blocks of `par_block` each (about
                 a second of oracle time per process); rate = sampled params /
                 the busiest process's oracle time;
      one core   one process, blocks of `block` until `target_s` seconds of
                 oracle time.
    Runs before the GPU is touched (workers are forked)."""
    import multiprocessing

    affinity = len(os.sched_getaffinity(0))
    cores = max(1, affinity)
    nblk = min(per_proc * cores, -(-S // par_block))
    blocks = [(begin + k * par_block, min(par_block, S - k * par_block)) for k in range(nblk)]
    jobs = [(w, blocks[j::cores], accum, reduce) for j in range(cores) if blocks[j::cores]]
    with multiprocessing.get_context("fork").Pool(len(jobs)) as pool:
        res = pool.map(_oracle_worker, jobs)
    par_done, par_time = sum(r[0] for r in res), max(r[1] for r in res)

    done, spent = 0, 0.0
    while spent < target_s and done < S:
        n = min(block, S - done)
        spent += _oracle_block(w, begin + done, n, accum, reduce=reduce)
        done += n
    what = f"{accum} accumulations + " if accum else f"reduction of {reduce} slices + " if reduce else ""
    return {"value": par_done / par_time, "unit": "params/s", "cores": len(jobs), "kind": "oracle",
            "host_cores_affinity": affinity, "host_cpu_count": os.cpu_count(),
            "sample": f"first {par_done} of the shard's {S} params in blocks of {par_block}, one step each "
                      f"({what}exact norm + AdamW, float64 NumPy), {len(jobs)} processes of one thread "
                      f"each, one per host core of the {affinity} this process may run on "
                      f"(os.cpu_count() {os.cpu_count()}); busiest process {par_time:.1f} s of oracle time, "
                      f"{sum(r[1] for r in res):.1f} s in all, "
                      f"input generation excluded",
            "one_core": {"value": done / spent, "cores": 1,
                         "sample": f"first {done} params in blocks of {block}, one process, {spent:.1f} s of "
                                   f"oracle time"}}


def bench_offload(w, args):
    """The offloaded step: fp32 state in pinned host memory, the 16-bit
    gradient on the device; per step D2H gradient, host norm + AdamW, H2D
    parameters.  Prints one JSON line."""
    import numpy as np
    import torch

    import workloads as W
    import zero_sharded_mixed_partition_amd as Z
    torch.cuda.set_device(0)
    _, S, _ = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}
    host = [torch.empty(S, dtype=torch.float32, pin_memory=True) for _ in range(3)]
    G = torch.empty(S, dtype=tdt[w.grad_dtype], device="cuda")
    blk = 16 * W.CHUNK
    for lo in range(0, S, blk):
        cnt = min(blk, S - lo)
        for name, dst in zip(("master", "exp_avg", "exp_avg_sq"), host):
            dst[lo:lo + cnt].copy_(torch.from_numpy(W.fill(w, name, begin + lo, cnt)))
        g = W.fill(w, "grad", begin + lo, cnt, step=w.step)
        G[lo:lo + cnt].copy_(torch.from_numpy(g.view(np.int16)).view(G.dtype))
        print(f"# prepared {lo + cnt}/{S} elements", file=sys.stderr, flush=True)
    par = torch.empty(S, dtype=tdt[w.param_dtype], device="cuda")
    opt = Z.OffloadShardAdam(*host, grad_dtype=tdt[w.grad_dtype], param_dtype=tdt[w.param_dtype], lr=w.lr,
                             beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                             max_grad_norm=w.max_grad_norm,
                             scaler=(Z.LossScaler(scale=w.loss_scale) if w.loss_scale != 1.0
                                     else Z.LossScaler.static(1.0)), applied_steps=w.step - 1)
    for _ in range(args.warmup):
        opt.step(G, par)
    torch.cuda.synchronize()
    phases = {"norm": [], "pipeline": []}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        opt.step(G, par)
        for k, v in opt.last_times.items():
            phases[k].append(v)
        print("# step done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    avg = {k: sum(v) / len(v) * 1e3 for k, v in phases.items()}
    pcie_bytes = 2 * S

    # host ceilings, after the timed region: the host step alone over the
    # whole shard (no PCIe; 2 + 12 bytes read, 12 + 2 written per parameter)
    # and the library's host copy of the master's bytes (the step's chunks,
    # threads and store style: one read and one write stream)
    g_host = torch.empty(S, dtype=tdt[w.grad_dtype], pin_memory=True)
    g_host.copy_(G)
    p_host = torch.empty(S, dtype=tdt[w.param_dtype], pin_memory=True)
    sq_h, _ = Z.zero_cpu_shard_unscale_norm_overflow(g_host, 1.0 / opt.scaler.scale)
    hp_h = Z.AdamHyper(lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                       step=opt.t + 1, inv_loss_scale=1.0 / opt.scaler.scale, max_grad_norm=w.max_grad_norm)
    host_ms = []
    for _ in range(3):
        h0 = time.perf_counter()
        Z.zero_cpu_shard_adam_step(host[0], host[1], host[2], g_host, p_host, hp_h, sq_h, False)
        host_ms.append((time.perf_counter() - h0) * 1e3)
    scratch = torch.empty_like(host[0])
    copy_ms = []
    for _ in range(3):
        h0 = time.perf_counter()
        Z.zero_cpu_copy_reference(scratch, host[0])
        copy_ms.append((time.perf_counter() - h0) * 1e3)
    host_step_ms, host_copy_ms = min(host_ms), min(copy_ms)
    # host memory traffic: plain stores to a line not yet in a cache read it
    # first (write-allocate), so the copy moves 4 + 4 + 4 bytes per float; the
    # step moves 28 per parameter (its fp32 streams are updated in place and
    # the 16-bit copy goes out with streaming stores, which read nothing)
    host_step_gbps = 28 * S / (host_step_ms * 1e-3) / 1e9
    host_copy_gbps = 8 * S / (host_copy_ms * 1e-3) / 1e9
    host_copy_wa = 12 * S / (host_copy_ms * 1e-3) / 1e9
    del g_host, p_host, scratch
    out = {
        "metric": METRIC, "value": S / (ms_step * 1e-3), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "shard_params": S, "path": "CPU offload (fp32 state in pinned host memory)",
                   "grad_dtype": w.grad_dtype, "param_dtype": w.param_dtype, "host_threads": os.cpu_count()},
        "offload": {"phase_ms": avg, "chunk": opt.chunk, "norm_on": "device",
                    "pcie_gbps_each_way": pcie_bytes / (avg["pipeline"] * 1e-3) / 1e9,
                    "host_state_gbps": 24 * S / (avg["pipeline"] * 1e-3) / 1e9,
                    "host_step_alone": {"ms": host_step_ms, "gbps": host_step_gbps, "bytes_per_param": 28,
                                        "threads": os.cpu_count()},
                    "host_copy": {"ms": host_copy_ms, "gbps": host_copy_gbps, "gbps_with_write_allocate": host_copy_wa,
                                  "what": "zero_cpu_copy_reference over the fp32 master's bytes: one read and one "
                                          "write stream on the host step's threads"},
                    "host_step_frac_of_copy": host_step_gbps / host_copy_wa},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt1t",
                    help="tiny | gpt2 | llama7b | gpt100b | gpt1t (default: one rank's shard of a 1T model)")
    ap.add_argument("--accum", type=int, default=0,
                    help="micro-batches accumulated into an fp32 gradient copy per step (0: step the 16-bit "
                         "gradient directly)")
    ap.add_argument("--reduce", type=int, default=0,
                    help="K: the step's gradient is the reduction of K ranks' 16-bit slices of this partition "
                         "into the fp32 copy (the local half of the gradient reduce-scatter)")
    ap.add_argument("--separate-norm", action="store_true",
                    help="with --accum/--reduce: run the norm pass over the fp32 copy on its own instead of in the "
                         "pass that writes the copy")
    ap.add_argument("--offload", action="store_true",
                    help="keep the fp32 state in pinned host memory and step on host cores (CPU offload)")
    ap.add_argument("--graph", action="store_true",
                    help="replay one recorded step graph per step (the step's kernels as a single launch; pays off "
                         "on small shards where launches dominate)")
    ap.add_argument("--host-scaler", action="store_true",
                    help="keep the loss scaler and step counter on the host, reading the 4-byte overflow flag back "
                         "every step (default: both live in device memory and no step waits for the host)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-workload", default="gpt100b",
                    help="a second workload timed after the headline one on the default path and reported under "
                         "extra_workload ('' to skip; ignored with --accum/--reduce/--graph/--host-scaler)")
    ap.add_argument("--alloc", choices=["contiguous", "torch"], default="contiguous",
                    help="where the shard's buffers come from: physically contiguous HBM through the library's "
                         "allocator in a torch memory pool (default), or torch's default allocator")
    args = ap.parse_args()
    if args.graph and (args.accum or args.offload or args.reduce):
        print("--graph records the 16-bit-gradient step on the GPU; it does not combine with --accum, "
              "--reduce or --offload", file=sys.stderr)
        sys.exit(2)
    if args.reduce and (args.accum or args.offload or not 1 <= args.reduce <= 16):
        print("--reduce K takes 1 <= K <= 16 and does not combine with --accum or --offload", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py measures one rank's shard step on ONE GPU; --gpus {args.gpus} is not supported "
              "(the data-parallel collectives around the step are outside this benchmark).", file=sys.stderr)
        sys.exit(2)

    import workloads as W
    w = W.get(args.workload)

    if args.offload:
        return bench_offload(w, args)

    cpu = None
    if not args.no_cpu_baseline:
        # first, before torch or the GPU is touched: the oracle is host-only
        # and its all-cores leg forks worker processes
        import oracle
        _, S0, _ = oracle.partition_plan(w.shapes, w.n_d, w.align)
        cpu = cpu_baseline(w, w.rank * S0, S0, accum=args.accum, reduce=args.reduce)
        print(f"# cpu baseline {cpu['value']:.4g} params/s on {cpu['cores']} cores, "
              f"{cpu['one_core']['value']:.4g} on one", file=sys.stderr, flush=True)

    import torch

    import zero_sharded_mixed_partition_amd as Z
    torch.cuda.set_device(0)
    K = args.accum
    R = args.reduce
    res = run_shard(w, args, K, R, args.steps, args.warmup)
    S, ms_step = res["S"], res["ms_step"]

    # the achievable rate of one read + one write stream over the same 14 B/param
    # each way (at most 16 GiB): the library's reference copy kernel, and
    # torch's device-to-device copy (the runtime's blit kernel, also the
    # known-size copy that scales the HBM byte counters)
    cbytes = min(S * 14, 16 << 30) // 16 * 16
    src = torch.empty(cbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    # HBM moves all-zero data faster than varied data (the same access pattern
    # ran about 3 points faster on zeros): the copy moves normal floats, like
    # the shard's streams
    src.normal_(0.0, 0.02)
    dst.normal_(0.0, 0.02)

    def time_copy(fn):
        for _ in range(3):
            fn()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            fn()
        c1.record()
        torch.cuda.synchronize()
        return 2 * cbytes / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9

    ref_gbps = time_copy(lambda: Z.zero_copy_reference(dst, src, cbytes))
    copy_gbps = time_copy(lambda: dst.copy_(src))
    del src, dst

    # the second workload at the target shard sizes, as extra keys: one rank's
    # 250M-parameter shard of a 100B model, applied and skipped steps timed
    # on the same path (default run only; the headline value stays the one above)
    extra = None
    if args.extra_workload and not (K or R or args.graph or args.host_scaler):
        w2 = W.get(args.extra_workload)
        if w2.name != w.name:
            r2 = run_shard(w2, args, 0, 0, args.steps, args.warmup)
            extra = {"workload": w2.name, "shard_params": r2["S"], "n_d": w2.n_d, "rank": w2.rank,
                     "grad_dtype": w2.grad_dtype, "param_dtype": w2.param_dtype, "steps": args.steps,
                     "ms_per_step": r2["ms_step"], "params_per_s": r2["S"] / (r2["ms_step"] * 1e-3),
                     "hbm_gbps": r2["step_gbps"], "hbm_frac_of_peak": r2["step_gbps"] / PEAK_HBM_GBPS,
                     "step_ms": r2["step_ms"], "buffers": r2["buffers"],
                     "update": {"kernel": r2["roofline"]["kernel"], "avg_ms": r2["roofline"]["avg_ms"],
                                "gbps": r2["roofline"]["achieved"], "frac": r2["roofline"]["frac"],
                                "traffic": r2["roofline"]["traffic"]},
                     "norm_pass": r2["norm_pass"], "skipped_step": r2["skipped_step"]}

    out = {
        "metric": METRIC,
        "value": S / (ms_step * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "shard_params": S, "n_d": w.n_d, "rank": w.rank,
                   "flat_offset": res["begin"], "grad_dtype": w.grad_dtype, "param_dtype": w.param_dtype,
                   "state_dtype": "f32", "step_t": w.step, "clip_max_norm": w.max_grad_norm,
                   "weight_decay": w.weight_decay, "param_layout": w.param_layout,
                   "path": res["path"], "algorithmic_bytes_per_param": res["step_bpp"],
                   "buffers": res["buffers"]},
        "hbm_gbps": res["step_gbps"],
        "hbm_frac_of_peak": res["step_gbps"] / PEAK_HBM_GBPS,
        "roofline": res["roofline"],
        "step_ms": res["step_ms"],
        "norm_pass": res["norm_pass"],
        "skipped_step": res["skipped_step"],
        "copy_reference": {"kernel": "copy16 (zero_copy_reference)", "bytes_each_way": cbytes, "gbps": ref_gbps,
                           "frac_of_peak": ref_gbps / PEAK_HBM_GBPS,
                           "adam_update_frac_of_copy": res["roofline"]["achieved"] / ref_gbps,
                           "step_frac_of_copy": res["step_gbps"] / ref_gbps},
        "accumulate": res["accumulate"],
        "reduce": res["reduce"],
        "torch_copy_gbps": copy_gbps,
        "skipped_steps": res["skipped"],
        "extra_workload": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


class StepMarks:
    """Named timing points of one step on the current stream.  A HIP event is
    recorded only where work was enqueued since the last recorded one;
    otherwise the name stands for that event.  Every recorded event costs the
    GPU a few microseconds (about 4 us each on MI355X: a small shard's step
    ran 24% longer with five per step than with none), so the timed steps
    record two, around the update kernel, and each step starts at the
    previous step's last event when nothing was enqueued in between."""

    def __init__(self, pool, start=None):
        self._pool, self.ev = pool, {}
        self._last, self._dirty = start, start is None

    def mark(self, name):
        if self._dirty:
            self._last = self._pool.pop()
            self._last.record()
            self._dirty = False
        self.ev[name] = self._last

    def enqueued(self):
        self._dirty = True

    def ms(self, a, b):
        return self.ev[a].elapsed_time(self.ev[b])


def run_shard(w, args, K, R, steps, warmup):
    """Uploads workload w's shard, runs `warmup` untimed and `steps` timed
    steps (a synchronize on both sides of the timed region), then 10 skipped
    steps timed apart; frees the shard and returns the measurements."""
    import torch

    import zero_sharded_mixed_partition_amd as Z
    offsets, S, padded = Z.zero_partition_plan(w.shapes, w.n_d, w.align)
    begin = w.rank * S
    print(f"# workload {w.name}: shard {S} params at flat offset {begin}", file=sys.stderr, flush=True)
    # the shard's streams: physically contiguous HBM by default (the update
    # kernel's rate depends on where its eight streams' pages land); the
    # library counts the segments it hands out, so the label says what they got
    pool_ctx = torch.cuda.use_mem_pool(Z.contiguous_pool()) if args.alloc == "contiguous" else contextlib.nullcontext()
    pool0 = Z.zero_pool_counts()
    with pool_ctx:
        P, M, V, G = upload_inputs(w, begin, S, w.grad_dtype)
        pdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.param_dtype]
        par = torch.empty(S, dtype=pdt, device="cuda")
        A = torch.empty(S, dtype=torch.float32, device="cuda") if (K or R) else None
        # the other ranks' slices: copies of this rank's gradient (distinct buffers, same values)
        slices = [G] + [G.clone() for _ in range(R - 1)] if R else None
    pool1 = Z.zero_pool_counts()
    n_contig, n_fallback = pool1[0] - pool0[0], pool1[1] - pool0[1]
    if args.alloc != "contiguous":
        buffers = "torch default allocator"
    elif pool1[1] == 0:
        buffers = (f"physically contiguous HBM (library allocator behind a torch memory pool: {pool1[0]} segments "
                   f"so far, {n_contig} new for this shard, none fell back to ordinary memory)")
    else:
        buffers = (f"library allocator behind a torch memory pool: {pool1[1]} of its {pool1[0] + pool1[1]} segments "
                   f"({n_fallback} of {n_contig + n_fallback} new for this shard) fell back to ordinary device "
                   f"memory, the rest physically contiguous")
    opt = Z.ShardAdam(P, M, V, lr=w.lr, beta1=w.beta1, beta2=w.beta2, eps=w.eps, weight_decay=w.weight_decay,
                      max_grad_norm=w.max_grad_norm,
                      scaler=(Z.LossScaler(scale=w.loss_scale) if w.loss_scale != 1.0 else Z.LossScaler.static(1.0)),
                      applied_steps=w.step - 1, graph=args.graph,
                      device_state=not args.host_scaler)
    DS = opt.state is not None
    FUSED = bool(K or R) and not args.separate_norm
    torch.cuda.synchronize()

    def step(m=None):
        if args.graph and m is None:
            return opt.step(G, par)
        mark = m.mark if m is not None else (lambda name: None)
        done = m.enqueued if m is not None else (lambda: None)
        mark("start")
        if K:
            for k in range(K):
                if k == K - 1:
                    mark("copy0")                # the last micro-batch (with the norm when fused)
                if k == 0 and K > 1:
                    mark("first0")
                opt.accumulate(A, G, first=(k == 0), last=FUSED and k == K - 1)
                done()
                if k == 0 and K > 1:
                    mark("first1")
            mark("copy1")
        if R:
            mark("copy0")
            opt.reduce(A, slices, with_norm=FUSED)
            done()
            mark("copy1")
        grad = A if (K or R) else G
        mark("norm0")
        if FUSED:
            pass                               # the copy's norm and flag came with the pass that wrote it
        elif DS:
            opt.norm_decide(grad)              # the decision (coefficients, scaler, counts) in the norm's last kernel
            done()
        else:
            opt.unscale_norm(grad)
            done()
        mark("norm1")
        if FUSED and DS:
            opt.decide(grad)                   # one thread: coefficients, scaler, counts
            done()
        mark("upd0")
        if DS:
            opt.update(grad, par)
        else:
            opt.apply(grad, par)
        done()
        mark("upd1")
        r = opt.finish()                       # device_state: None, nothing waits
        if not DS:
            done()                             # the host scaler enqueued the flag's copy
        return r

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    n_skip = min(10, steps)
    pool = [torch.cuda.Event(enable_timing=True) for _ in range(9 * (2 * steps + n_skip) + 9)]
    marks = []
    skipped = 0
    wall = []
    skipped0 = opt.read_state().skipped if DS else 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ts = time.perf_counter()
        # device state: nothing is enqueued between steps, so a step starts at
        # the previous one's last event
        m = StepMarks(pool, marks[-1].ev["upd1"] if (marks and DS) else None)
        if args.graph:
            m.mark("start")
            r = step(None)
            m.enqueued()
            m.mark("upd1")
        else:
            r = step(m)
        marks.append(m)
        skipped += bool(r)                                     # host scaler: the step ended with the flag read
        wall.append(time.perf_counter() - ts)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if DS:
        # nothing waited inside the loop: per-step times from the events, start to next start
        starts = [m.ev["start"] for m in marks]
        wall = [starts[k].elapsed_time(starts[k + 1]) * 1e-3 for k in range(steps - 1)]
        wall.append(marks[-1].ms("start", "upd1") * 1e-3)
        skipped = opt.read_state().skipped - skipped0
    print(f"# timed {steps} steps", file=sys.stderr, flush=True)
    if args.graph:
        # a replayed graph has no events between its kernels: the per-kernel
        # times come from the same kernels launched one by one, after the
        # timed region
        marks = []
        for k in range(steps):
            m = StepMarks(pool)
            step(m)
            marks.append(m)
        torch.cuda.synchronize()

    # skipped steps, timed apart: +inf in one gradient element makes the norm
    # pass raise the flag and the update exit without touching the state
    keep = G[S // 2].clone()
    G[S // 2] = float("inf")
    sev = []
    skipped1 = opt.read_state().skipped if DS else 0
    torch.cuda.synchronize()
    skip_wall = []
    for k in range(n_skip):
        ts = time.perf_counter()
        sev.append(StepMarks(pool))
        r = step(sev[-1])
        if DS:
            torch.cuda.synchronize()
        else:
            assert r, "a gradient holding +inf must skip the step"
        skip_wall.append(time.perf_counter() - ts)
    if DS:
        assert opt.read_state().skipped - skipped1 == n_skip, "a gradient holding +inf must skip the step"
    G[S // 2] = keep
    torch.cuda.synchronize()

    ms_step = (t1 - t0) * 1e3 / steps
    norm_ms = sorted(m.ms("norm0", "norm1") for m in marks)
    adam_ms = sorted(m.ms("upd0", "upd1") for m in marks)
    mean = lambda xs: sum(xs) / len(xs)  # noqa: E731
    pct = lambda xs, q: xs[min(len(xs) - 1, int(q * len(xs)))]  # noqa: E731
    adam_bpp = ADAM_F32_BYTES_PER_PARAM if (K or R) else ADAM_BYTES_PER_PARAM
    norm_bpp = 0 if FUSED else (NORM_F32_BYTES_PER_PARAM if (K or R) else NORM_BYTES_PER_PARAM)
    acc_bpp = (ACC_FIRST_BYTES_PER_PARAM + ACC_BYTES_PER_PARAM * (K - 1)) if K else 0
    red_bpp = 2 * R + 4 if R else 0
    step_bpp = adam_bpp + norm_bpp + acc_bpp + red_bpp
    adam_avg = mean(adam_ms)
    adam_gbps = adam_bpp * S / (adam_avg * 1e-3) / 1e9
    step_gbps = step_bpp * S / (ms_step * 1e-3) / 1e9
    run_key = w.name + (f"+accum{K}" if K else "") + (f"+reduce{R}" if R else "") + ("+graph" if args.graph else "") \
        + ("+separate-norm" if (K or R) and not FUSED else "")
    traffic = measured_traffic(run_key)
    accum_stats = None
    if K:
        acc_ms = mean([m.ms("copy0", "copy1") for m in marks])     # the last (non-first) accumulation
        accum_stats = {"micro_batches": K, "kernel": "grad_sum_norm (with the norm)" if FUSED else "grad_accumulate",
                       "avg_ms": acc_ms,
                       "algorithmic_bytes": ACC_BYTES_PER_PARAM * S if K > 1 else ACC_FIRST_BYTES_PER_PARAM * S,
                       "gbps": (ACC_BYTES_PER_PARAM if K > 1 else ACC_FIRST_BYTES_PER_PARAM) * S / (acc_ms * 1e-3) / 1e9,
                       "traffic": measured_traffic(run_key, "grad_sum_norm" if FUSED else "grad_accumulate")}
        if K > 1:
            # the first micro-batch (2 B read, 4 B written per element) against
            # the widening copy over the same bytes: G (2 B/param) into A (4 B/param)
            first_ms = mean([m.ms("first0", "first1") for m in marks])
            first_gbps = ACC_FIRST_BYTES_PER_PARAM * S / (first_ms * 1e-3) / 1e9
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            for _ in range(3):
                Z.zero_copy_widen_reference(A, G, 2 * S)
            c0.record()
            for _ in range(10):
                Z.zero_copy_widen_reference(A, G, 2 * S)
            c1.record()
            torch.cuda.synchronize()
            widen_gbps = ACC_FIRST_BYTES_PER_PARAM * S / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9
            accum_stats["first"] = {"kernel": "grad_accumulate (first micro-batch)", "avg_ms": first_ms,
                                    "algorithmic_bytes": ACC_FIRST_BYTES_PER_PARAM * S, "gbps": first_gbps,
                                    "frac_of_peak": first_gbps / PEAK_HBM_GBPS,
                                    "traffic": measured_traffic(run_key, "grad_accumulate_first"),
                                    "widening_copy_gbps": widen_gbps, "frac_of_widening_copy": first_gbps / widen_gbps}
    reduce_stats = None
    if R:
        red_ms = mean([m.ms("copy0", "copy1") for m in marks])
        reduce_stats = {"slices": R, "kernel": "grad_sum_norm (with the norm)" if FUSED else "grad_reduce",
                        "avg_ms": red_ms, "algorithmic_bytes": red_bpp * S,
                        "gbps": red_bpp * S / (red_ms * 1e-3) / 1e9,
                        "traffic": measured_traffic(run_key, "grad_sum_norm" if FUSED else "grad_reduce")}
    path = ((f"fp32 gradient accumulation, {K} micro-batches" if K else
             f"reduction of {R} ranks' 16-bit slices into the fp32 copy" if R else "16-bit gradient")
            + ((", norm in the pass that writes the copy" if FUSED else ", separate norm pass") if (K or R) else "")
            + (", recorded step graph" if args.graph else "")
            + (", scaler and step counter in device memory" if DS else ", host loss scaler (4-byte flag read per step)"))
    out = {
        "S": S, "begin": begin, "ms_step": ms_step, "step_bpp": step_bpp, "step_gbps": step_gbps,
        "path": path, "buffers": buffers, "skipped": skipped,
        "roofline": {"bound": "hbm", "kernel": "adam_update_devcoef" if DS else "adam_update", "achieved": adam_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": adam_gbps / PEAK_HBM_GBPS, "traffic": traffic,
                     "traffic_source": ("rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, profiles/hbm_counters.json, "
                                        "taken on the same kernel code (hash match)") if traffic else None,
                     "algorithmic_bytes": adam_bpp * S, "avg_ms": adam_avg,
                     "p10_ms": pct(adam_ms, 0.1), "p90_ms": pct(adam_ms, 0.9),
                     "timed_on": "eager launches after the timed region" if args.graph else "the timed steps"},
        "step_ms": {"median": pct(sorted(wall), 0.5) * 1e3, "p10": pct(sorted(wall), 0.1) * 1e3,
                    "p90": pct(sorted(wall), 0.9) * 1e3},
        "norm_pass": ({"fused_into": "grad_sum_norm"} if FUSED else
                      {"avg_ms": mean(norm_ms), "gbps": norm_bpp * S / (mean(norm_ms) * 1e-3) / 1e9}),
        "skipped_step": {"steps": n_skip, "ms_per_step": mean(skip_wall) * 1e3,
                         "norm_ms": mean([m.ms("norm0", "norm1") for m in sev]),
                         "update_ms": mean([m.ms("upd0", "upd1") for m in sev])},
        "accumulate": accum_stats,
        "reduce": reduce_stats,
    }
    del opt, P, M, V, G, par, A, slices
    torch.cuda.synchronize()
    return out


if __name__ == "__main__":
    main()
