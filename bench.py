#!/usr/bin/env python3
"""Benchmark one rank's ZeRO shard step on one MI355X.

A step is one pass of the whole hot path over resident synthetic inputs:
for the default workload (Psi = 7.5e9 flat buffer, N_d = 64, rank 0's
117,187,500-element partition) that is zero_reduce_grad_shard over the 64
fp16 gradient slices followed by zero_adam_step (fp32 master, m, v in place,
fresh fp16 params), with the reduce's non-finite flag as the step's skip
input.  Other workloads (--workload) run the Adam step alone (N_d = 1 or a
single rank's shard).

Prints one JSON line: params updated per second (value), the per-kernel
HIP-event durations measured inside the timed region on the launch stream,
the dominant kernel's roofline against MI355X's 8 TB/s HBM peak, and the CPU
oracle timed on a bounded sample on this host.  The default run also times,
in the same process and after the headline, the Adam step of the other
7B-scale workloads and of GPT-2-XL (`per_config`: the N_d = 8 rank-3 shard
with its infinities, the Llama-7B list, the GPT-2-XL list, each over its
own resident state, freed before the next) and the N_d = 64 shard's Adam
step with the fp16 parameter view at ranks 1 and 63, and one element past
rank 0's, out of the other arrays' phase (`adam_by_rank`).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "params updated/sec and achieved HBM GB/s (% of roofline) per Adam shard step"
# the sources that decide what the kernels do and how they are launched
KERNEL_SRCS = [os.path.join(ROOT, "zero_partitioned_mixed_layout_amd", "csrc", f)
               for f in ("zs_kernels.hip", "zs_internal.h", "zs_host.cpp")]
# committed rocprofv3 counter summaries, one per workload (lines "traffic: ...")
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "hbm_traffic_*.md")


def code_tokens(text: str) -> str:
    """C/C++/HIP source with comments removed and every run of whitespace
    made one space (string and character literals kept whole), so that the
    hash below changes with the code, not with its comments or layout."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_src_sha(read=None) -> str:
    """Hash of the code (not the comments) of the kernel sources; `read`
    maps a path to its text (default: the working tree)."""
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        if read is None:
            with open(p, encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(p)
        h.update(code_tokens(text).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summaries,
    if they were taken on the current kernel sources (kernels, launch
    constants, plan builder); else None."""
    pat = re.compile(r"^traffic:\s+(.*)$")
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        for line in open(path):
            m = pat.match(line.strip())
            if not m:
                continue
            kv = dict(x.split("=", 1) for x in m.group(1).split())
            if kv.get("kernel") == kernel and kv.get("workload") == workload:
                if kv.get("src_sha256") != kernel_src_sha():
                    return None
                return float(kv["hbm_bytes_per_launch"])
    return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="flat_7p5b_nd64",
                    choices=["flat_7p5b_nd64", "flat_7p5b_nd8", "gpt2_xl", "llama_7b", "tiny_flat"])
    ap.add_argument("--slices", action="store_true",
                    help="flat workloads without gradient slices (flat_7p5b_nd8): give the step "
                         "the reduce of N_d simulated fp16 slices too, as flat_7p5b_nd64 has")
    ap.add_argument("--inject-inf", action="store_true",
                    help="flat workloads without slices: set the workload's fraction of the "
                         "gradients (0.01%% if it names none) to +inf or -inf at seeded positions "
                         "and clear the non-finite flag before every step, so that each Adam "
                         "launch raises it afresh (for counting the flag's atomics; the clear "
                         "is timed with the step)")
    ap.add_argument("--loss-scale", type=int, default=None, metavar="LOG2",
                    help="the Adam step reads the gradients as carrying a loss scale of 2^LOG2 "
                         "(zero_adam_step_scaled) and each step ends with the scale's update "
                         "(zero_loss_scale_update), which consumes the step's flag")
    ap.add_argument("--fused", action="store_true",
                    help="workloads with gradient slices: one zero_reduce_adam_step launch per "
                         "step instead of zero_reduce_grad_shard + zero_adam_step")
    ap.add_argument("--gather", action="store_true",
                    help="workloads with gradient slices: end the step with zero_gather_shards "
                         "of the N_d fp16 shards into the full parameter buffer (this rank's "
                         "shard in place; the other ranks' shards stood in for by the slices)")
    ap.add_argument("--offload", action="store_true",
                    help="ZeRO-Offload: fp32 master, m, v in host memory and the Adam update "
                         "on the host CPU (zero_offload_step); the fp16 gradient and "
                         "parameters stay on the GPU")
    ap.add_argument("--offload-chunk", type=int, default=0,
                    help="elements per offload pipeline chunk (0: library default)")
    ap.add_argument("--offload-threads", type=int, default=0,
                    help="host threads of the offload update (0: min(16, hardware threads))")
    ap.add_argument("--bf16", action="store_true",
                    help="the bfloat16 variant: bfloat16 parameters, gradients and slices "
                         "(fp32 master, m, v as before)")
    ap.add_argument("--list-layout", choices=["flat", "separate"], default="flat",
                    help="tensor-list workloads: views into five flattened buffers (the "
                         "state a ZeRO rank holds) or five allocations per tensor")
    ap.add_argument("--chunk-elems", type=int, default=0,
                    help="elements per chunk of the Adam plan (0: library default)")
    ap.add_argument("--cpu-sample", type=int, default=1 << 26,
                    help="elements of the shard the CPU oracle is timed on")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="keep stepping the CPU oracle over its sample until this much "
                         "wall time has passed (at most 8 steps)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="time only the headline workload (no per_config, no adam_by_rank)")
    ap.add_argument("--per-config-steps", type=int, default=0,
                    help="timed Adam steps per extra workload (0: max(10, --steps))")
    ap.add_argument("--param-rank", type=int, default=None,
                    help="flat workloads: place the fp16 parameter view of the shard at this "
                         "rank's offset in the full buffer (the other arrays unchanged)")
    ap.add_argument("--param-shift", type=int, default=0, metavar="ELEMS",
                    help="flat workloads: move the fp16 parameter view this many elements "
                         "further into the full buffer (1-3: out of the other arrays' 8-byte "
                         "phase, as a rank's view is when the shard length is not a multiple "
                         "of four)")
    ap.add_argument("--slices-back-to-back", action="store_true",
                    help="workloads with gradient slices: lay the N_d slices back to back in "
                         "one buffer (slice r at r times the shard length) instead of rows of a "
                         "128-byte-aligned pitch; with a shard length of 4 mod 8 every other "
                         "slice sits 8 bytes off and the reduce takes its 8-byte path")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="instead of the step: copy a BYTES-byte device buffer into another "
                         "with torch, --steps times (the plain copy kernel that scales the "
                         "HBM byte counters), print one JSON line and exit")
    return ap.parse_args()


def copy_calibration(nbytes: int, reps: int) -> None:
    """A plain device-to-device copy of known size, for scaling rocprofv3's
    FETCH_SIZE / WRITE_SIZE counters: each launch reads and writes nbytes."""
    import torch
    n = nbytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"copy_bytes_read_per_launch": 4 * n, "copy_bytes_written_per_launch": 4 * n,
                      "launches": reps, "avg_ms": dt * 1e3, "gbps_rw": 8 * n / dt / 1e9}),
          flush=True)


def plain_copy(stream, nbytes: int = 4 << 30, reps: int = 10) -> dict:
    """A plain stream for context: torch's device-to-device copy of nbytes
    (read nbytes, write nbytes; the runtime's copy kernel), timed with HIP
    events on `stream` after the timed region.  Not the roofline's
    denominator, which is the published 8 TB/s."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    b.record(stream)
    b.synchronize()
    s = a.elapsed_time(b) / reps / 1e3
    del src, dst
    torch.cuda.empty_cache()
    gbps = 2 * nbytes / s / 1e9
    return {"kernel": "torch device-to-device copy (__amd_rocclr_copyBuffer)", "bytes_per_launch": 2 * nbytes,
            "avg_us": s * 1e6, "gbps": gbps, "frac": gbps / HBM_PEAK_GBPS}


def reduce_kernel_name(rows, out):
    """The name of the reduce kernel zero_reduce_grad_shard launches over
    these slices and output, to label its timed launch: zs_reduce_kernel
    when all share a 16-byte phase (zs_reduce_few_kernel at 1-3 slices),
    zs_reduce_vec4_kernel when they share an 8-byte one, else
    zs_reduce_single_kernel (outputs alone out of phase are not told
    apart: the bench's outputs are aligned)."""
    ptrs = [r.data_ptr() for r in rows] + [out.data_ptr()]
    if len({p % 16 for p in ptrs}) == 1:
        return "zs_reduce_kernel" if len(rows) > 3 else "zs_reduce_few_kernel"
    if len({p % 8 for p in ptrs}) == 1:
        return "zs_reduce_vec4_kernel"
    return "zs_reduce_single_kernel"


class Step:
    """Device state and the launches of one step for a workload."""

    def __init__(self, zs, W, name, chunk_elems=0, fused=False, gather=False, offload=False,
                 offload_threads=0, bf16=False, list_layout="flat", offload_chunk=0,
                 slices=False, inject_inf=False, loss_scale=None, param_rank=None,
                 param_shift=0, slices_back_to_back=False):
        import numpy as np
        import torch
        self.zs, self.W, self.torch = zs, W, torch
        half = torch.bfloat16 if bf16 else torch.float16
        wl = W.WORKLOADS[name]
        self.wl = wl
        self.hp = zs.AdamHParams(**W.ADAM_HP)
        self.flag = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.rflag = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.rows = None
        self.reduce_name = "zs_reduce_kernel"
        if len(wl.tensors) == 1:
            lay = zs.zero_shard_layout(wl.psi, wl.nd, wl.rank, wl.align)
            self.layout = lay
            self.full, sh = W.device_flat_state(wl, lay.offset, lay.real_len, lay.padded_total,
                                                half=half)
            if param_rank is not None or param_shift:
                # the same shard state, its fp16 parameter view at another
                # rank's place in the full buffer (a view off its lines for
                # most ranks when the shard length is not a multiple of 64),
                # param_shift elements further
                r = wl.rank if param_rank is None else param_rank
                off = r * lay.shard_len + param_shift
                if not 0 <= r < wl.nd or off < 0 or off + lay.real_len > lay.padded_total:
                    raise SystemExit(f"--param-rank {param_rank} --param-shift {param_shift}: "
                                     "outside the layout")
                sh.p = self.full[off:off + lay.real_len]
            self.tensors = [sh]
            if wl.reduce_slices or slices:
                self.slice_buf, self.rows = W.device_slices(wl, lay.real_len, half=half,
                                                            back_to_back=slices_back_to_back)
                self.reduce_name = reduce_kernel_name(self.rows, sh.g)
            else:
                W.device_fill_grads(wl, self.tensors, 1)
                if inject_inf:
                    pos, sign = W.inf_positions(lay.real_len, wl.inf_frac or 1e-4, wl.seed)
                    W.device_inject_inf(sh.g, pos, sign)
                    self.n_inf = int(pos.size)
        else:
            self.layout = None
            self.tensors = W.device_list_state(wl, half=half, layout=list_layout)
            W.device_fill_grads(wl, self.tensors, 1)
        self.inject_inf = inject_inf and self.rows is None and len(self.tensors) == 1
        self.plan = zs.zero_plan_create([t.arrays() for t in self.tensors], chunk_elems)
        self.n_params = self.plan.stats()["n_params"]
        self.t = 0
        self.fused = fused and self.rows is not None
        self.offload = None
        if offload:
            if len(self.tensors) != 1:
                raise SystemExit("--offload runs on the flat workloads")
            sh = self.tensors[0]
            self.host = [x.cpu().numpy().copy() for x in (sh.w, sh.m, sh.v)]
            self.hflag = np.zeros(1, dtype=np.int32)
            self.offload = zs.zero_offload_create(offload_chunk, offload_threads)
            self.fused = False
        self.loss_scale = None
        if loss_scale is not None and self.offload is None and not self.fused:
            self.loss_scale = zs.LossScale(log2_scale=loss_scale, interval=2000,
                                           min_log2=min(0, loss_scale),
                                           max_log2=max(24, loss_scale))
        self.gather = gather and self.rows is not None
        if self.gather:
            # this rank's fp16 shard is the view of the full buffer at its
            # offset; the other ranks' updated shards are stood in for by
            # the gradient slices of the same length
            r0 = self.wl.rank
            self.shards = [self.tensors[0].p if r == r0 else self.rows[r] for r in range(self.wl.nd)]

    def reduce(self):
        self.zs.zero_reduce_grad_shard(self.rows, self.tensors[0].g, self.rflag)

    def adam(self):
        self.t += 1
        if self.inject_inf:
            self.flag.zero_()
        skip = self.rflag if self.rows is not None else None
        self.zs.zero_adam_step(self.plan, self.hp, self.t, self.flag, skip,
                               loss_scale=self.loss_scale)

    def scale_update(self):
        # the reduce's flag when there is a reduce (the step's skip input),
        # else the Adam step's own
        self.loss_scale.update(self.rflag if self.rows is not None else self.flag)

    def offload_step(self):
        self.t += 1
        sh = self.tensors[0]
        self.offload.step(sh.g, sh.p, *self.host, self.hp, self.t, nonfinite_flag=self.hflag)

    def reduce_adam(self):
        self.t += 1
        sh = self.tensors[0]
        self.zs.zero_reduce_adam_step(self.rows, sh.p, sh.w, sh.m, sh.v, self.hp, self.t,
                                      nonfinite_flag=self.flag)

    def gather_full(self):
        self.zs.zero_gather_shards(self.shards, self.full)

    def kernels(self):
        if self.fused:
            # the entry point: one fused kernel below zs.ZERO_FUSED_SPLIT_SLICES
            # slices, the reduce and then the Adam kernel from there on; its
            # algorithmic bytes are the fused minimum either way
            ks = [("zero_reduce_adam_step", self.reduce_adam,
                   (2 * self.wl.nd + 26) * self.n_params)]
        else:
            ks = []
            if self.rows is not None:
                ks.append((self.reduce_name, self.reduce, (2 * self.wl.nd + 2) * self.n_params))
            if self.offload is not None:
                ks.append(("zero_offload_step", self.offload_step, 4 * self.n_params))
            else:
                ks.append(("zs_adam_kernel", self.adam, 28 * self.n_params))
            if self.loss_scale is not None:
                ks.append(("zs_loss_scale_kernel", self.scale_update, 20))
        if self.gather:
            ks.append(("zs_gather_kernel", self.gather_full,
                       4 * self.layout.shard_len * (self.wl.nd - 1)))
        return ks


def cpu_baseline(step, sample_n: int, min_seconds: float):
    """The oracle as it stands, on contiguous partitions of the first
    sample_n elements of the shard (first tensor of a list), one host thread
    per partition: whole steps (the reduce of the N_d slices where the
    workload has one, then Adam at t = 1, 2, ...) until min_seconds of wall
    time have passed."""
    import concurrent.futures as cf
    import numpy as np
    import torch
    import oracle

    T = host_cpus()["usable"]
    sh = step.tensors[0]
    n = min(sample_n, sh.n)
    hp = dict(step.W.ADAM_HP)
    w = sh.w[:n].cpu().numpy().copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p = np.zeros(n, np.uint16)
    if step.rows is not None:
        sl = [r[:n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16) for r in step.rows]
        g = np.empty(n, np.uint16)
    else:
        g = sh.g[:n].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        sl = None
    bounds = [(n * i // T, n * (i + 1) // T) for i in range(T)]

    def part(b, t):
        lo, hi = b
        if sl is not None:
            oracle.reduce_grad([s[lo:hi] for s in sl], g[lo:hi])
        oracle.adam_step(g[lo:hi], p[lo:hi], w[lo:hi], m[lo:hi], v[lo:hi], t=t, **hp)

    oracle.lib()
    steps = 0
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(T) as ex:
        while True:
            steps += 1
            list(ex.map(part, bounds, [steps] * T))
            dt = time.perf_counter() - t0
            if dt >= min_seconds or steps >= 8:
                break
    # one more step over the first partition alone, on this thread
    t1 = time.perf_counter()
    part(bounds[0], steps + 1)
    dt1 = time.perf_counter() - t1
    n1 = bounds[0][1] - bounds[0][0]
    what = ("reduce of %d fp16 slices + Adam step" % step.wl.nd) if sl is not None else "Adam step"
    per_param = 28 + ((2 * step.wl.nd + 2) if sl is not None else 0)
    hc = host_cpus()
    return {"value": n * steps / dt, "unit": "params/s", "cores": T, "kind": "oracle",
            "affinity_cpus": hc["affinity"], "cgroup_cpu_quota": hc["quota"],
            "gbps": per_param * n * steps / dt / 1e9, "alg_bytes_per_param": per_param,
            "single_thread_value": n1 / dt1, "cpu_model": cpu_model(),
            "sample": f"first {n} elements of the shard: {steps} x ({what}), {T} host threads, "
                      f"{dt:.2f} s wall; then one step over the first {n1} elements on one "
                      f"thread, {dt1:.2f} s"}


def host_cpus() -> dict:
    """CPUs this process may use: its affinity mask, capped by the cgroup's
    CPU quota where one is set (cpu.max), which is the share a machine
    shared between GPUs gives the jobs of one GPU."""
    aff = len(os.sched_getaffinity(0))
    quota = None
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = int(q) / int(per)
    except (OSError, ValueError):
        pass
    usable = aff if quota is None else max(1, min(aff, int(quota)))
    return {"affinity": aff, "quota": quota, "usable": usable}


def host_rmw_bandwidth(threads: int, nbytes: int = 4 << 30, reps: int = 4) -> dict:
    """Host memory bandwidth of an in-place read-modify-write stream (one
    read and one write of every byte, as the offload update does to the fp32
    master, m and v), on `threads` threads, each touching its own part of
    the array first.  Host only: numpy releases the interpreter lock in its
    loops, so the threads run in parallel."""
    import concurrent.futures as cf
    import numpy as np
    n = nbytes // 4
    a = np.empty(n, np.float32)
    parts = [(n * i // threads, n * (i + 1) // threads) for i in range(threads)]
    one = np.float32(1.0)

    def touch(r):
        a[r[0]:r[1]] = 1.0

    def work(r):
        x = a[r[0]:r[1]]
        for _ in range(reps):
            np.multiply(x, one, out=x)

    with cf.ThreadPoolExecutor(threads) as ex:
        list(ex.map(touch, parts))
        list(ex.map(work, parts))                     # warm
        t0 = time.perf_counter()
        list(ex.map(work, parts))
        dt = time.perf_counter() - t0
    del a
    return {"gbps": 2 * nbytes * reps / dt / 1e9, "threads": threads, "bytes": nbytes,
            "pattern": "in-place multiply of fp32 (1 read + 1 write per byte), numpy, "
                       "first touch in the threads"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


PCIE_PEAK_GBPS = 128.0  # PCIe Gen5 x16 host link, both directions together


def pcie_copy_rates(nbytes: int = 1 << 30, reps: int = 5) -> dict:
    """Pinned host <-> device copy rates (GB/s): each direction alone and
    both at once on two streams."""
    import torch
    n = nbytes // 2
    dev = torch.empty(n, dtype=torch.float16, device="cuda")
    dev2 = torch.empty(n, dtype=torch.float16, device="cuda")
    hin = torch.empty(n, dtype=torch.float16, pin_memory=True)
    hout = torch.empty(n, dtype=torch.float16, pin_memory=True)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps

    t_d2h = timed(lambda: hout.copy_(dev, non_blocking=True))
    t_h2d = timed(lambda: dev.copy_(hin, non_blocking=True))

    def both():
        with torch.cuda.stream(s1):
            hout.copy_(dev, non_blocking=True)
        with torch.cuda.stream(s2):
            dev2.copy_(hin, non_blocking=True)

    t_both = timed(both)
    return {"d2h_gbps": nbytes / t_d2h / 1e9, "h2d_gbps": nbytes / t_h2d / 1e9,
            "both_gbps": 2 * nbytes / t_both / 1e9, "bytes": nbytes}


def time_steps(torch, stream, ks, steps):
    """Run `steps` steps of the launches ks = [(name, launch, alg_bytes)],
    each launch between two HIP events on `stream`; returns (wall seconds
    between two synchronisations, per-kernel statistics)."""
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in ks] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        for (a, b), (_, launch, _) in zip(ev[k], ks):
            a.record(stream)
            launch()
            b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kstats = {}
    for j, (name, _, alg_bytes) in enumerate(ks):
        ms = [ev[k][j][0].elapsed_time(ev[k][j][1]) for k in range(steps)]
        avg_s = sum(ms) / len(ms) / 1e3
        gbps = alg_bytes / avg_s / 1e9
        kstats[name] = {"avg_us": avg_s * 1e6, "min_us": min(ms) * 1e3,
                        "median_us": sorted(ms)[len(ms) // 2] * 1e3,
                        "alg_bytes_per_launch": alg_bytes, "gbps": gbps,
                        "frac": gbps / HBM_PEAK_GBPS, "total_s": sum(ms) / 1e3}
    return wall, kstats


def rounded(d: dict) -> dict:
    return {k: (round(v, 3) if isinstance(v, float) else v) for k, v in d.items() if k != "total_s"}


def adam_by_rank(zs, torch, stream, step, ranks, steps, align=None, shift=0):
    """The flat shard's Adam step with its fp16 parameter view placed at
    each rank's offset in the full buffer (gradient, master, m, v the same
    arrays): where the shard length is not a multiple of 64 elements, most
    ranks' views start off a 128-byte line.  align: the layout's unit
    (default the workload's); a rank whose shard is shorter than this one's
    under it updates the first elements only.  shift: elements added to the
    view's offset (1: the parameter out of the other arrays' 8-byte phase,
    as a rank's view is under a layout whose shard length is odd); the
    entry is then keyed "rank+shift"."""
    sh = step.tensors[0]
    wl = step.wl
    lays = {r: zs.zero_shard_layout(wl.psi, wl.nd, r, align or wl.align) for r in ranks}
    out = {}
    for r in ranks:
        off = lays[r].offset + shift
        n = min(sh.n, lays[r].real_len, step.full.numel() - off)
        view = step.full[off:off + n]
        plan = zs.zero_plan_create([(view, sh.g[:n], sh.w[:n], sh.m[:n], sh.v[:n])])

        def adam():
            step.t += 1
            zs.zero_adam_step(plan, step.hp, step.t)

        for _ in range(3):
            adam()
        _, ks = time_steps(torch, stream, [("zs_adam_kernel", adam, 28 * n)], steps)
        k = ks["zs_adam_kernel"]
        out[f"{r}+{shift}" if shift else str(r)] = {
            "byte_offset_in_line": (view.data_ptr() % 128), "params": n,
            "avg_us": round(k["avg_us"], 3), "gbps": round(k["gbps"], 3),
            "frac": round(k["frac"], 4)}
        plan.destroy()
    return out


def per_config_leg(zs, W, torch, stream, name, warmup, steps):
    """The Adam step of one more workload over its own resident state: warm
    steps with finite gradients, then (the N_d = 8 shard) the workload's
    infinities injected, then `steps` timed Adam launches.  The state is
    freed before returning."""
    import gc
    print(f"[bench] per_config: setting up {name}", file=sys.stderr, flush=True)
    st = Step(zs, W, name)
    ks = st.kernels()
    for _ in range(warmup):
        for _, launch, _ in ks:
            launch()
    n_inf = None
    if st.wl.inf_frac and st.layout is not None:
        pos, sign = W.inf_positions(st.layout.real_len, st.wl.inf_frac, st.wl.seed)
        W.device_inject_inf(st.tensors[0].g, pos, sign)
        n_inf = int(pos.size)
    _, kstats = time_steps(torch, stream, ks, steps)
    k = kstats["zs_adam_kernel"]
    entry = {"workload": name, "params": st.n_params, "kernel": "zs_adam_kernel",
             "steps": steps, "warmup": warmup, **rounded(k),
             "params_per_s": st.n_params / (k["avg_us"] / 1e6),
             "traffic": measured_traffic("zs_adam_kernel", name),
             "chunk_elems": st.plan.stats()["chunk_elems"],
             "adam_tile_elems": st.plan.stats()["tile_elems"],
             "tensors": len(st.wl.tensors)}
    if n_inf is not None:
        torch.cuda.synchronize()
        entry["injected_inf"] = n_inf
        entry["flag"] = int(st.flag.item())
    if len(st.wl.tensors) > 1:
        entry["list_layout"] = "flat"
    st.plan.destroy()
    del st, ks
    gc.collect()
    torch.cuda.empty_cache()
    return entry


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the shard step "
              "has no cross-GPU exchange to time here.", file=sys.stderr)
        sys.exit(2)
    import gc
    import torch
    from zero_partitioned_mixed_layout_amd import workloads as W
    from zero_partitioned_mixed_layout_amd import zero_shard as zs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    print(f"[bench] setting up {args.workload}", file=sys.stderr, flush=True)
    step = Step(zs, W, args.workload, args.chunk_elems, args.fused, args.gather, args.offload,
                args.offload_threads, args.bf16, args.list_layout, args.offload_chunk,
                args.slices, args.inject_inf, args.loss_scale, args.param_rank,
                args.param_shift, args.slices_back_to_back)
    ks = step.kernels()
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        for _, launch, _ in ks:
            launch()
    torch.cuda.synchronize()
    print(f"[bench] warm-up done ({args.warmup} steps); timing {args.steps}", file=sys.stderr,
          flush=True)
    wall, kstats = time_steps(torch, stream, ks, args.steps)
    dom = max(kstats, key=lambda k: kstats[k]["total_s"])
    d = kstats[dom]
    traffic = (measured_traffic(dom, args.workload)
               if args.param_rank is None and not args.param_shift and not args.bf16 else None)
    if traffic is None:
        print(f"[bench] no HBM counters for {dom} on {args.workload} taken on the current kernel "
              f"code ({kernel_src_sha()}): traffic is null", file=sys.stderr, flush=True)
    value = step.n_params * args.steps / wall
    bytes_per_step = sum(b for _, _, b in ks)
    # the headline configuration's other extras, while its state is resident
    headline_plain = (not args.no_per_config and args.workload == "flat_7p5b_nd64" and
                      not (args.fused or args.gather or args.offload or args.bf16 or
                           args.loss_scale is not None or args.param_rank is not None or
                           args.param_shift or args.slices_back_to_back))
    pc_steps = args.per_config_steps or max(10, args.steps)
    by_rank = None
    if headline_plain:
        print("[bench] Adam step by rank of the parameter view", file=sys.stderr, flush=True)
        by_rank = {"0": {"byte_offset_in_line": step.tensors[0].p.data_ptr() % 128,
                         "avg_us": round(kstats["zs_adam_kernel"]["avg_us"], 3),
                         "gbps": round(kstats["zs_adam_kernel"]["gbps"], 3),
                         "frac": round(kstats["zs_adam_kernel"]["frac"], 4)}}
        by_rank.update(adam_by_rank(zs, torch, stream, step, (1, step.wl.nd - 1), pc_steps))
        slow = min(by_rank, key=lambda r: by_rank[r]["frac"])
        # rank 0's view one element further: the parameter's stores shifted
        shifted = adam_by_rank(zs, torch, stream, step, (0,), pc_steps, shift=1)
        # the same ranks under a layout whose unit is 64 elements: every
        # rank's view on a 128-byte line (the workload itself has unit 1)
        a64 = adam_by_rank(zs, torch, stream, step, (1, step.wl.nd - 1), pc_steps, align=64)
        by_rank = {"ranks": by_rank, "slowest_rank": int(slow),
                   "slowest_frac": by_rank[slow]["frac"], "steps": pc_steps,
                   "layout_align_64": {"ranks": a64, "slowest_frac":
                                       min(v["frac"] for v in a64.values())},
                   "param_one_element_off": shifted["0+1"]}
    copy = plain_copy(stream)
    cpu = (None if args.no_cpu_baseline
           else cpu_baseline(step, args.cpu_sample, args.cpu_seconds))
    cfg = {"workload": args.workload +
           ("+slices" if args.slices and not step.wl.reduce_slices and step.rows is not None else "") +
           ("+inf" if step.inject_inf else "") +
           (f"+loss_scale_2^{args.loss_scale}" if step.loss_scale is not None else "") +
           ("+fused" if step.fused else "") +
           ("+gather" if step.gather else "") + ("+offload" if step.offload else "") +
           ("+bf16" if args.bf16 else "") +
           (f"+param_rank_{args.param_rank}" if args.param_rank is not None else "") +
           (f"+param_shift_{args.param_shift}" if args.param_shift else "") +
           ("+slices_back_to_back" if args.slices_back_to_back and step.rows is not None else ""),
           "psi": step.wl.psi, "nd": step.wl.nd,
           "rank": step.wl.rank, "align": step.wl.align, "shard_params": step.n_params,
           "tensors": len(step.wl.tensors),
           "injected_inf": step.n_inf if step.inject_inf else None,
           "list_layout": args.list_layout if len(step.wl.tensors) > 1 else None,
           "chunk_elems": step.plan.stats()["chunk_elems"],
           "adam_tile_elems": step.plan.stats()["tile_elems"],
           "kernels_per_step": [k for k, _, _ in ks],
           "alg_bytes_per_step": bytes_per_step,
           "step_hbm_gbps": bytes_per_step * args.steps / wall / 1e9}
    fused_vs = None
    if step.fused:
        cfg["fused_route"] = ("one fused kernel" if step.wl.nd < zs.ZERO_FUSED_SPLIT_SLICES
                              else "reduce kernel, then Adam kernel")
        # the two separate entry points over the same buffers in the same
        # process, each step interleaved with the fused one: placement of
        # the buffers in physical memory differs between processes by a few
        # percent, so only a comparison within one process is meaningful
        print("[bench] fused against reduce + Adam, interleaved", file=sys.stderr, flush=True)
        rn = step.reduce_name
        both = [ks[0], (rn, step.reduce, (2 * step.wl.nd + 2) * step.n_params),
                ("zs_adam_kernel", step.adam, 28 * step.n_params)]
        _, kb = time_steps(torch, stream, both, args.steps)
        sep_us = kb[rn]["avg_us"] + kb["zs_adam_kernel"]["avg_us"]
        fused_vs = {"steps": args.steps, "fused_us": round(kb[ks[0][0]]["avg_us"], 3),
                    "reduce_us": round(kb[rn]["avg_us"], 3),
                    "adam_us": round(kb["zs_adam_kernel"]["avg_us"], 3),
                    "separate_us": round(sep_us, 3),
                    "fused_over_separate": round(kb[ks[0][0]]["avg_us"] / sep_us, 4)}
    roofline = {"bound": "hbm", "kernel": dom, "achieved": d["gbps"], "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": d["frac"], "traffic": traffic}
    offload = None
    if step.offload is not None:
        rates = pcie_copy_rates()
        info = step.offload.info()
        host_bw = host_rmw_bandwidth(info["threads"])
        o = kstats["zero_offload_step"]
        t_s = o["avg_us"] / 1e6
        # host memory bytes per parameter the algorithm moves: the fp32
        # master, m and v read and written back (24).  The fp16 staging adds
        # up to 8 more (the CPU reads the gradient and writes the parameter,
        # the copy engines write and read them), some of it served from the
        # host's caches, so it is reported beside the roofline, not in it
        alg_bytes = 24 * step.n_params
        offload = {"avg_ms": t_s * 1e3, "params_per_s": step.n_params / t_s,
                   "pcie_bytes_per_param": 4, "pcie_gbps": o["gbps"],
                   "host_state_bytes_per_param": 24,
                   "host_state_gbps": alg_bytes / t_s / 1e9,
                   "host_gbps_with_staging": 32 * step.n_params / t_s / 1e9,
                   "host_rmw_probe": host_bw, "pipeline": info,
                   "pinned_copy": rates}
        if dom == "zero_offload_step":
            roofline = {"bound": "host-memory", "kernel": dom,
                        "achieved": alg_bytes / t_s / 1e9, "peak": host_bw["gbps"],
                        "unit": "GB/s", "frac": alg_bytes / t_s / 1e9 / host_bw["gbps"],
                        "traffic": None,
                        "peak_source": "host_rmw_probe, measured in this run (the host's memory "
                                       "bandwidth varies between runs on a shared host)"}
    headline_params = step.n_params
    step.plan.destroy()
    del step, ks
    gc.collect()
    torch.cuda.empty_cache()
    per_config = None
    if headline_plain:
        per_config = {"flat_7p5b_nd64": {
            "workload": "flat_7p5b_nd64", "params": headline_params, "kernel": "zs_adam_kernel",
            "steps": args.steps, "warmup": args.warmup, **rounded(kstats["zs_adam_kernel"]),
            "params_per_s": headline_params / (kstats["zs_adam_kernel"]["avg_us"] / 1e6),
            "traffic": measured_traffic("zs_adam_kernel", "flat_7p5b_nd64"),
            "note": "the headline run's Adam launches"}}
        for name in ("flat_7p5b_nd8", "llama_7b", "gpt2_xl"):
            wl = W.WORKLOADS[name]
            per_config[name] = per_config_leg(zs, W, torch, stream, name,
                                              max(args.warmup, wl.warm_steps), pc_steps)
    out = {
        "metric": METRIC, "value": value, "unit": "params/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic", "config": cfg,
        "roofline": roofline,
        "kernels": {k: rounded(v) for k, v in kstats.items()},
        "cpu_baseline": cpu,
        "plain_copy": copy,
    }
    if fused_vs is not None:
        out["fused_vs_separate"] = fused_vs
    if by_rank is not None:
        out["adam_by_rank"] = by_rank
    if per_config is not None:
        out["per_config"] = per_config
    if offload is not None:
        out["offload"] = offload
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
