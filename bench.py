"""Throughput of the Gated DeltaNet record / replay / GQA-expand path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--capture separate|fused]

One step is one pass of the whole path over one batch of seeded synthetic
input already resident in HBM:

    large_batch_decode (default): gqa_expand(k -> k_log, block map)
                                  + gdn_record + gdn_replay(accepted=1) on the fresh tape
    spec_decode:      the same at B=8, T=4 with a drawn accepted count
    chunk_prefill:    gqa_expand of fp32 q and k (tiled map) + the record over 4096 steps,
                      by gdn_prefill (chunks of 64 steps; --prefill sequential: gdn_record)
    long_tape_replay: gdn_replay of a 64-step fp16 tape for accepted in {0,1,16,63,64}
    tiny:             gdn_record + gdn_replay
    cell_d192_128, cell_d64_32: the page's other two head-shape cells as decode
                      steps (B=1024 / 16384), same launches as large_batch_decode
    prefill_d192_128: the record over 4096 steps at the Dk=192, Dv=128, Hk=Hv=4 cell,
                      by gdn_prefill (--prefill sequential: gdn_record)
    rms_norm_prefill: rms_norm_bf16 of 4096 fp32 hidden states of width 2048

With --capture fused (decode workloads) the record writes k_log and g_log
itself and the separate gqa_expand launch goes away.

`value` is effective HBM bandwidth: the algorithmic bytes of the step (what
the method must read and write, defined below) divided by the measured step
time.  `roofline` describes the dominant kernel, timed with HIP events on the
stream it runs on; `cpu_baseline` times the CPU oracle on a bounded sample of
the same workload on this host.

Algorithmic bytes (e = I/O element size, state float32, U = active (b,t) steps,
A = taken tape positions, a' = min(accepted, T)):
    record  8*B*Hv*Dv*Dk + 4*B*T [mask] + U*e*(2*Hk*Dk + 3*Hv*Dv + 2*Hv)
    replay  8*B*Hv*Dv*Dk + 4*B*a' [mask] + A*e*Hv*(Dv + Dk + 1)
    expand  e*seq*K*(Hg + H)
    capture U*e*Hv*(Dk + 1) on top of the record (k_log and g_log writes)
    rms_norm 8*n*dim + 2*dim (x in, out out, the bf16 weight)
The replay's "touched" bytes count every position below a' (the select reads
masked positions too): A is replaced by B*a'.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
METRIC = "GDN record+replay effective HBM GB/s (% of peak) and head-steps/sec"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "gdn_record": ["gdn_record.hip", "gdn_record_mfma.hip", "gdn_device.hpp"],
    "gdn_replay": ["gdn_replay.hip", "gdn_replay_mfma.hip", "gdn_device.hpp"],
    "gqa_expand": ["gqa_expand.hip", "gdn_device.hpp"],
    "rms_norm_bf16": ["rms_norm.hip", "gdn_device.hpp"],
    "gdn_prefill": ["gdn_prefill.hip", "gdn_device.hpp"],
}


# ----------------------------------------------------------- byte accounting

def record_bytes(B, T, Hk, Hv, Dk, Dv, e, active_steps, has_mask):
    return (8 * B * Hv * Dv * Dk + (4 * B * T if has_mask else 0)
            + active_steps * e * (2 * Hk * Dk + 3 * Hv * Dv + 2 * Hv))


def replay_bytes(B, T, Hv, Dk, Dv, e, accepted, taken_steps, has_mask):
    a = min(accepted, T)
    return 8 * B * Hv * Dv * Dk + (4 * B * a if has_mask else 0) + taken_steps * e * Hv * (Dv + Dk + 1)


def expand_bytes(seq, hg, h, k, e):
    return e * seq * k * (hg + h)


def rms_norm_bytes(n, dim):
    return 8 * n * dim + 2 * dim


def capture_bytes(Hv, Dk, e, active_steps):
    return active_steps * e * Hv * (Dk + 1)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "linear_attention_recurrence_step_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str, label: str = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none for this kernel, workload and launch label (an
    entry without a label stands for every launch of the kernel) or the
    kernel's source changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            entries = json.load(f)
    except (OSError, ValueError):
        return None
    for ent in entries.get("entries", []):
        if ent.get("kernel") == kernel and ent.get("workload") == workload and \
                ent.get("label", label) == label:
            if ent.get("source_sha256") == kernel_source_hash(kernel):
                return ent.get("traffic_bytes")
    return None


# ------------------------------------------------------------------ workloads

def _active(mask, B, T, upto=None):
    upto = T if upto is None else min(upto, T)
    if mask is None:
        return B * upto
    return int((mask[:, :upto] > 0).sum().item())


class Step:
    """Device buffers and launch sequence of one step of a workload."""

    def __init__(self, name, dev, seed=0, capture="separate", prefill="chunked"):
        import torch
        import gdn_inputs as gi
        import linear_attention_recurrence_step_amd as gdn
        self.gdn = gdn
        self.name = name
        self.gi_norm = gi.NORM_WORKLOADS
        self.fused = capture == "fused"
        self.prefill_step = name in gi.PREFILL_WORKLOADS
        self.chunked = prefill == "chunked" and self.prefill_step
        self.kernels = []            # (label, kernel, algorithmic bytes, head-steps)
        self.touched = {}
        if name in gi.NORM_WORKLOADS:
            if self.fused:
                raise SystemExit("--capture fused applies to workloads with a record and a replay")
            self.w = w = gi.NORM_WORKLOADS[name]
            x, wt = gi.norm_inputs(w["n_tokens"], w["dim"], seed)
            self.cpu = (x, wt)
            self.x, self.wt = x.to(dev), wt.to(dev)
            self.out = torch.empty_like(self.x)
            self.kernels.append(("rms_norm", "rms_norm_bf16", rms_norm_bytes(w["n_tokens"], w["dim"]), 0))
            return
        self.w = w = gi.WORKLOADS[name]
        if self.fused and (name == "long_tape_replay" or self.prefill_step):
            raise SystemExit("--capture fused applies to workloads with a record and a replay")
        self.e = 4 if w.io == "f32" else 2
        self.kernels = []            # (label, kernel, algorithmic bytes, head-steps)
        T = w.T
        if name == "long_tape_replay":
            tape = gi.tape_inputs(w.B, T, w.Hv, w.Dk, w.Dv, w.io, seed=seed, mask=w.mask, mask_p=w.mask_p)
            self.cpu = tape
            self.d = {k: (v.to(dev) if v is not None else None) for k, v in tape.items()}
            self.out = torch.empty_like(self.d["state_in"])
            self.touched = {}
            for a in w.accepted:
                taken = _active(tape["mask"], w.B, T, a)
                self.kernels.append(("replay[a=%d]" % a, "gdn_replay",
                                     replay_bytes(w.B, T, w.Hv, w.Dk, w.Dv, self.e, a, taken, True),
                                     taken * w.Hv))
                self.touched["replay[a=%d]" % a] = replay_bytes(w.B, T, w.Hv, w.Dk, w.Dv, self.e, a,
                                                                w.B * min(a, T), True)
            return
        inp = gi.workload_inputs(name, seed)
        self.cpu = inp
        self.touched = {}
        self.d = d = {k: (v.to(dev) if v is not None else None) for k, v in inp.items()}
        io = d["q"].dtype
        self.y = torch.empty(d["v"].shape, dtype=io, device=dev)
        self.dl = torch.empty(d["v"].shape, dtype=io, device=dev)
        self.s_rec = torch.empty_like(d["state_in"])
        self.s_rep = torch.empty_like(d["state_in"])
        U = _active(inp["mask"], w.B, T)
        has_mask = inp["mask"] is not None
        if name == "chunk_prefill":
            self.src = [gi.expand_source(w.B * T, w.Hk, w.Dk, w.expand_io, seed=seed + 1 + i).to(dev)
                        for i in range(2)]
            self.dst = [torch.empty((w.B * T, w.Hv, w.Dk), dtype=self.src[0].dtype, device=dev)
                        for _ in range(2)]
            eb = 4 if w.expand_io == "f32" else 2
            for i, what in enumerate(("q", "k")):
                self.kernels.append(("expand_%s" % what, "gqa_expand",
                                     expand_bytes(w.B * T, w.Hk, w.Hv, w.Dk, eb), 0))
        elif not self.prefill_step:
            self.k_log = torch.empty((w.B, T, w.Hv, w.Dk), dtype=io, device=dev)
            self.g_log = torch.empty((w.B, T, w.Hv), dtype=io, device=dev) if self.fused else None
            if not self.fused:
                self.kernels.append(("expand_k", "gqa_expand",
                                     expand_bytes(w.B * T, w.Hk, w.Hv, w.Dk, self.e), 0))
        rb = record_bytes(w.B, T, w.Hk, w.Hv, w.Dk, w.Dv, self.e, U, has_mask)
        if self.fused:
            self.kernels.append(("record+capture", "gdn_record",
                                 rb + capture_bytes(w.Hv, w.Dk, self.e, U), U * w.Hv))
        elif self.chunked:
            # the chunked record: same outputs, same algorithmic bytes; its
            # workspace is allocated once, outside the timed steps
            self.ws = torch.empty(gdn.gdn_prefill_workspace_size(w.B, T, w.Hv), dtype=torch.uint8,
                                  device=dev)
            self.kernels.append(("prefill", "gdn_prefill", rb, U * w.Hv))
        else:
            self.kernels.append(("record", "gdn_record", rb, U * w.Hv))
        if not self.prefill_step:
            if name == "spec_decode":
                import numpy as np
                self.accepted = int(np.random.Generator(np.random.PCG64(seed + 77)).integers(0, w.T + 1))
            else:
                self.accepted = w.accepted[0]
            taken = _active(inp["mask"], w.B, T, self.accepted)
            self.kernels.append(("replay", "gdn_replay",
                                 replay_bytes(w.B, T, w.Hv, w.Dk, w.Dv, self.e, self.accepted, taken, has_mask),
                                 taken * w.Hv))
            self.touched = {"replay": replay_bytes(w.B, T, w.Hv, w.Dk, w.Dv, self.e, self.accepted,
                                                   w.B * min(self.accepted, T), has_mask)}

    def launches(self):
        """Callables, one per kernel launch, in step order."""
        if self.name in self.gi_norm:
            return [lambda: self.gdn.rms_norm_bf16(self.x, self.wt, self.w["eps"], out=self.out)]
        gdn, d, w = self.gdn, self.d, self.w
        if self.name == "long_tape_replay":
            return [(lambda a=a: gdn.gdn_replay(d["delta_log"], d["k_log"], d["g_log"], d["state_in"],
                                                d["mask"], a, state_out=self.out))
                    for a in w.accepted]
        out = []
        if self.name == "chunk_prefill":
            for i in range(2):
                out.append(lambda i=i: gdn.gqa_expand(self.src[i], w.Hv, w.gqa_map, dst=self.dst[i]))
        elif not self.fused and not self.prefill_step:
            out.append(lambda: gdn.gqa_expand(d["k"], w.Hv, w.gqa_map, dst=self.k_log))
        if self.chunked:
            out.append(lambda: gdn.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"],
                                               d["mask"], gqa_map=w.gqa_map, y=self.y,
                                               state_out=self.s_rec, delta_log=self.dl,
                                               workspace=self.ws))
        elif self.fused:
            out.append(lambda: gdn.gdn_record(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"],
                                              d["mask"], gqa_map=w.gqa_map, y=self.y,
                                              state_out=self.s_rec, delta_log=self.dl,
                                              k_log=self.k_log, g_log=self.g_log))
        else:
            out.append(lambda: gdn.gdn_record(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state_in"],
                                              d["mask"], gqa_map=w.gqa_map, y=self.y,
                                              state_out=self.s_rec, delta_log=self.dl))
        if not self.prefill_step:
            g_log = self.g_log if self.fused else d["g"]
            out.append(lambda: gdn.gdn_replay(self.dl, self.k_log, g_log, d["state_in"], d["mask"],
                                              self.accepted, state_out=self.s_rep))
        return out


# ------------------------------------------------------------ CPU baseline

CPU_THREADS_MAX = 16


def _host_threads(requested=None):
    """(cores in this process's affinity mask, threads the oracle timing uses):
    every core of the mask, at most CPU_THREADS_MAX, unless requested."""
    aff = len(os.sched_getaffinity(0))
    if requested:
        return aff, max(1, int(requested))
    return aff, max(1, min(aff, CPU_THREADS_MAX))


def _timed_threads(work_lists, budget_s):
    """Run each list of prepared oracle calls in its own thread, over and over
    until the budget is spent; returns (bytes done, seconds).  A list is
    [(callable, algorithmic bytes of one call), ...].  Only the oracle's C
    calls run inside the loops (ctypes releases the GIL around them)."""
    import threading
    done = [0] * len(work_lists)
    ends = [0.0] * len(work_lists)
    start = threading.Barrier(len(work_lists) + 1)
    holder = {}

    def loop(i):
        calls = work_lists[i]
        for f, _ in calls:                       # one untimed pass
            f()
        start.wait()
        deadline = holder["t0"] + budget_s
        n = 0
        while True:
            for f, nb in calls:
                f()
                n += nb
            if time.perf_counter() >= deadline:
                break
        done[i] = n
        ends[i] = time.perf_counter()

    threads = [threading.Thread(target=loop, args=(i,)) for i in range(len(work_lists))]
    for t in threads:
        t.start()
    holder["t0"] = time.perf_counter()
    start.wait()
    for t in threads:
        t.join()
    return sum(done), max(ends) - holder["t0"]


def _unit_calls(name, w, sl, e):
    """Prepared oracle calls for one slice of the sample (dict of CPU tensors)
    and their algorithmic bytes, in the order a step runs them."""
    import torch
    import gdn_inputs as gi
    import oracle
    calls = []
    if name == "long_tape_replay":
        nb = sl["delta_log"].shape[0]
        for a in w.accepted:
            f, _ = oracle.prepare_replay(sl["delta_log"], sl["k_log"], sl["g_log"], sl["state_in"],
                                         sl["mask"], a)
            taken = _active(sl["mask"], nb, w.T, a)
            calls.append((f, replay_bytes(nb, w.T, w.Hv, w.Dk, w.Dv, e, a, taken, True)))
        return calls
    if name in gi.PREFILL_WORKLOADS:
        heads = sl["v"].shape[2]
        f, _ = oracle.prepare_record(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], sl["state_in"],
                                     None, gqa_map="block")
        return [(f, record_bytes(1, w.T, heads, heads, w.Dk, w.Dv, e, w.T, False))]
    nb = sl["q"].shape[0]
    bits = torch.int32 if e == 4 else torch.int16
    kbits = sl["k"].contiguous().view(bits).numpy().reshape(nb * w.T, w.Hk, w.Dk)
    fx, k_log_bits = oracle.prepare_expand(kbits, w.Hv, w.gqa_map)
    fx()
    fr, (_, _, dlt) = oracle.prepare_record(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                            sl["state_in"], sl["mask"], gqa_map=w.gqa_map)
    fr()
    # the replay's tape: the record's delta in the I/O dtype, the expanded keys, g
    tape_d = torch.from_numpy(dlt).to(sl["q"].dtype)
    k_log = torch.from_numpy(k_log_bits).view(sl["k"].dtype).reshape(nb, w.T, w.Hv, w.Dk)
    a = w.accepted[0] if name != "spec_decode" else w.T
    fp, _ = oracle.prepare_replay(tape_d, k_log, sl["g"], sl["state_in"], sl["mask"], a)
    U = _active(sl["mask"], nb, w.T)
    taken = _active(sl["mask"], nb, w.T, a)
    has_mask = sl["mask"] is not None
    return [(fx, expand_bytes(nb * w.T, w.Hk, w.Hv, w.Dk, e)),
            (fr, record_bytes(nb, w.T, w.Hk, w.Hv, w.Dk, w.Dv, e, U, has_mask)),
            (fp, replay_bytes(nb, w.T, w.Hv, w.Dk, w.Dv, e, a, taken, has_mask))]


def cpu_baseline(name: str, budget_s: float, threads_req=None):
    """Time the CPU oracle on a bounded sample of the workload on this host.

    The sample (batch rows, or value heads of the one-sequence prefill, or
    tokens) is split into one contiguous slice per thread; each thread runs
    its slice's oracle calls (prepared once: inputs widened to float64 and
    outputs allocated outside the timed loop) until the budget is spent.
    Then one slice of one unit runs alone on one thread for the per-core
    figure.  Bytes are the same algorithmic bytes as the GPU figures."""
    import gdn_inputs as gi

    if name in gi.NORM_WORKLOADS:
        return _cpu_baseline_norm(name, budget_s, threads_req)
    w = gi.WORKLOADS[name]
    aff, threads = _host_threads(threads_req)
    e = 4 if w.io == "f32" else 2
    seed = 123
    if name in gi.PREFILL_WORKLOADS:
        units = min(w.Hv, threads)                     # value heads of the single batch row
        inp = gi.record_inputs(1, w.T, w.Hk, w.Hv, w.Dk, w.Dv, w.io, seed, w.mask, w.mask_p)

        def slice_of(lo, hi):
            hk = [hv % w.Hk for hv in range(lo, hi)]   # the tiled map, as keys pre-expanded
            return dict(q=inp["q"][:, :, hk], k=inp["k"][:, :, hk], v=inp["v"][:, :, lo:hi],
                        g=inp["g"][:, :, lo:hi], beta=inp["beta"][:, :, lo:hi],
                        state_in=inp["state_in"][:, lo:hi])
    else:
        # batch rows: at least one per thread, and about 32 MiB of state
        per_row = w.Hv * w.Dv * w.Dk * 4
        units = min(w.B, max(threads, (32 << 20) // per_row))
        if name == "long_tape_replay":
            inp = gi.tape_inputs(units, w.T, w.Hv, w.Dk, w.Dv, w.io, seed=seed, mask=w.mask,
                                 mask_p=w.mask_p)
        else:
            inp = gi.record_inputs(units, w.T, w.Hk, w.Hv, w.Dk, w.Dv, w.io, seed, w.mask, w.mask_p)

        def slice_of(lo, hi):
            return {k: (v[lo:hi] if v is not None else None) for k, v in inp.items()}
    threads = min(threads, units)
    bounds = [(i * units // threads, (i + 1) * units // threads) for i in range(threads)]
    work = [_unit_calls(name, w, slice_of(lo, hi), e) for lo, hi in bounds]
    total, dt = _timed_threads(work, budget_s)
    one_total, dt1 = _timed_threads([_unit_calls(name, w, slice_of(0, 1), e)], budget_s / 4)
    unit_name = "value heads" if name in gi.PREFILL_WORKLOADS else "batch rows"
    return {"value": round(total / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "%d of %d %s of %s, one slice per thread, %.1f s"
                      % (units, w.Hv if name in gi.PREFILL_WORKLOADS else w.B, unit_name, name, dt),
            "single_thread_value": round(one_total / dt1 / 1e9, 4),
            "affinity_cores": aff, "cpu_model": _cpu_model(),
            "label": "CPU baseline, not the target"}


def _cpu_baseline_norm(name: str, budget_s: float, threads_req=None):
    """The RMSNorm oracle on a sample of 1024 tokens, one token slice per thread."""
    import gdn_inputs as gi
    import oracle

    w = gi.NORM_WORKLOADS[name]
    aff, threads = _host_threads(threads_req)
    n = min(w["n_tokens"], 1024)
    x, wt = gi.norm_inputs(n, w["dim"], 123)
    xn = x.numpy()

    def calls(lo, hi):
        f, _ = oracle.prepare_rms_norm_bf16(xn[lo:hi], wt, w["eps"])
        return [(f, rms_norm_bytes(hi - lo, w["dim"]))]

    bounds = [(i * n // threads, (i + 1) * n // threads) for i in range(threads)]
    total, dt = _timed_threads([calls(lo, hi) for lo, hi in bounds], budget_s)
    one, dt1 = _timed_threads([calls(0, n // threads)], budget_s / 4)
    return {"value": round(total / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d tokens of %s, one slice per thread, %.1f s" % (n, w["n_tokens"], name, dt),
            "single_thread_value": round(one / dt1 / 1e9, 4), "affinity_cores": aff,
            "cpu_model": _cpu_model(), "label": "CPU baseline, not the target"}


def _cpu_model() -> str:
    """The host CPU's model name as lscpu prints it (the longer of its
    "Model name" and "BIOS Model name" lines), else /proc/cpuinfo's."""
    import subprocess
    names = []
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            key, _, val = line.partition(":")
            if key.strip() in ("Model name", "BIOS Model name") and val.strip():
                names.append(val.strip())
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    names.append(line.split(":", 1)[1].strip())
                    break
    except OSError:
        pass
    return max(names, key=len) if names else "unknown"


# ------------------------------------------------------- counter calibration

COPY_BYTES = 512 << 20


def calibrate_copy(dev, launches: int) -> None:
    """A plain device copy of COPY_BYTES (read once, written once): gqa_expand
    with one source and one destination head is exactly a copy.  Its byte
    counters, divided by COPY_BYTES, give the scale of each counter."""
    import torch
    import linear_attention_recurrence_step_amd as gdn
    k = 32768
    seq = COPY_BYTES // (4 * k)
    src = torch.randn(seq, 1, k, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(launches):
        gdn.gqa_expand(src, 1, "tiled", dst=dst)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / launches
    assert torch.equal(src, dst)
    print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES,
                      "launches": launches, "us_per_launch": round(dt * 1e6, 1),
                      "GB/s": round(2 * COPY_BYTES / dt / 1e9, 1)}), flush=True)


def copy_bandwidth(dev, launches: int = 20) -> float:
    """GB/s of a plain 512 MiB device copy (gqa_expand with one head each
    side), timed with HIP events: the practical HBM peak beside the published one."""
    import torch
    import linear_attention_recurrence_step_amd as gdn
    k = 32768
    seq = COPY_BYTES // (4 * k)
    src = torch.randn(seq, 1, k, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        gdn.gqa_expand(src, 1, "tiled", dst=dst)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(launches):
        gdn.gqa_expand(src, 1, "tiled", dst=dst)
    b.record()
    torch.cuda.synchronize()
    return 2 * COPY_BYTES * launches / (a.elapsed_time(b) * 1e-3) / 1e9


def copy_same_size(dev, nbytes: int, launches: int, scrub_buf, scrub_sum, stream) -> dict:
    """A plain device copy of nbytes each way (gqa_expand with one head), each
    launch timed with HIP events after the same cache scrub as the step's
    launches: the practical ceiling for a kernel that moves that many bytes."""
    import torch
    import linear_attention_recurrence_step_amd as gdn
    k = 1024
    seq = max(1, nbytes // (4 * k))
    src = torch.randn(seq, 1, k, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        gdn.gqa_expand(src, 1, "tiled", dst=dst)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for i in range(launches):
        if scrub_buf is not None:
            scrub_buf.fill_(float(i))
            torch.sum(scrub_buf, dim=0, out=scrub_sum)
        ev[i][0].record(stream)
        gdn.gqa_expand(src, 1, "tiled", dst=dst)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    us = _pct([a.elapsed_time(b) for a, b in ev], 50) * 1e3
    moved = seq * k * 4
    return {"bytes_each_way": moved, "us": round(us, 2), "GB/s": round(2 * moved / (us * 1e-6) / 1e9, 1)}


def reported_hbm_figure():
    """Memory bus width (bits) and clock (kHz) as the HIP runtime reports
    them, and clock x width / 8 in GB/s (None if unavailable).  HBM3E moves
    several bits per pin per reported clock, so this product is a fraction of
    the published peak, not a peak itself."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return None
    vals = []
    # hipDeviceAttributeMemoryBusWidth = 59, hipDeviceAttributeMemoryClockRate = 60 (ROCm 7 headers)
    for attr in (59, 60):
        v = ctypes.c_int()
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, 0) != 0:
            return None
        vals.append(v.value)
    return {"bus_width_bits": vals[0], "memory_clock_khz": vals[1],
            "clock_x_width_GBps": round(vals[1] * 1e3 * vals[0] / 8 / 1e9, 1),
            "published_GBps": HBM_PEAK_GBPS}


def _pct(xs, p):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(round(p / 100.0 * (len(xs) - 1))))]


# ----------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_batch_decode")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing")
    ap.add_argument("--scrub", choices=("on", "off"), default="on",
                    help="before every timed launch, write and then read back a 1 GiB buffer, so "
                         "that no input is left in the L2 / 256 MB MALL (not even one an earlier "
                         "launch of the step read) and no dirty line of the scrub is left to "
                         "write back during the launch")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="threads of the CPU baseline (default: the affinity mask's cores, at most %d)"
                         % CPU_THREADS_MAX)
    ap.add_argument("--capture", choices=("separate", "fused"), default="separate",
                    help="separate: k_log by a gqa_expand launch and g_log = g; fused: the record "
                         "writes k_log and g_log itself")
    ap.add_argument("--prefill", choices=("chunked", "sequential"), default="chunked",
                    help="chunk_prefill's record step: gdn_prefill (chunks of 64 steps on the "
                         "matrix cores) or gdn_record (one step after another)")
    ap.add_argument("--no-peak-probe", action="store_true",
                    help="skip the 512 MiB copy that measures the practical HBM peak")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain copy of known size (gqa_expand with hg == h) for "
                         "scaling the HBM byte counters, and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this path runs on a single MI355X and its "
              "multi-GPU sharding is a design, not a build; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    dev = torch.device("cuda", 0)
    if args.calibrate_copy:
        calibrate_copy(dev, args.steps)
        return
    step = Step(args.workload, dev, args.seed, args.capture, args.prefill)
    launches = step.launches()
    w = step.w

    for _ in range(args.warmup):
        for f in launches:
            f()
    torch.cuda.synchronize()

    step_bytes = sum(k[2] for k in step.kernels)
    scrub = args.scrub == "on"
    scrub_buf = torch.empty(1 << 28, dtype=torch.float32, device=dev) if scrub else None
    scrub_sum = torch.empty((), dtype=torch.float32, device=dev) if scrub else None

    stream = torch.cuda.current_stream(dev)
    # events around every launch: ev[s][i] = (start, end) of launch i of step s
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, f in enumerate(launches):
            if scrub:
                # outside the events: the write evicts the L2 and the MALL, the
                # read back leaves them holding clean lines of the scrub buffer only
                scrub_buf.fill_(float(s * len(launches) + i))
                torch.sum(scrub_buf, dim=0, out=scrub_sum)
            ev[s][i][0].record(stream)
            f()
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if scrub:
        # the wall clock includes the scrubs: a step is the sum of its launches' event intervals
        elapsed = sum(a.elapsed_time(b) for s in range(args.steps) for a, b in ev[s]) * 1e-3

    samples = [[ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]
               for i in range(len(launches))]
    per_kernel_ms = [sum(x) / args.steps for x in samples]

    head_steps = sum(k[3] for k in step.kernels)
    ms_per_step = elapsed * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    kernels = []
    for (label, kern, nbytes, hs), ms, xs in zip(step.kernels, per_kernel_ms, samples):
        ent = {"name": label, "kernel": kern, "us": round(ms * 1e3, 2),
               "us_p10_p50_p90": [round(_pct(xs, p) * 1e3, 2) for p in (10, 50, 90)],
               "algorithmic_bytes": nbytes, "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "frac_of_peak": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        if label in step.touched:
            ent["touched_bytes"] = step.touched[label]
            ent["touched_GB/s"] = round(step.touched[label] / (ms * 1e-3) / 1e9, 1)
        kernels.append(ent)
    dom = max(range(len(kernels)), key=lambda i: per_kernel_ms[i])
    dk = kernels[dom]
    roofline = {"bound": "hbm", "achieved": dk["GB/s"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dk["GB/s"] / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(dk["kernel"], args.workload, dk["name"]),
                "kernel": dk["name"], "bytes_per_launch": dk["algorithmic_bytes"],
                "us_per_launch": dk["us"]}
    if not args.no_peak_probe and not step.prefill_step:
        # the same bytes moved by a plain copy, timed the same way: the ceiling
        # at this size (small launches do not reach the large-copy rate)
        cp = copy_same_size(dev, dk["algorithmic_bytes"] // 2, max(args.steps, 10), scrub_buf, scrub_sum, stream)
        cp["kernel_frac_of_copy"] = round(dk["GB/s"] / cp["GB/s"], 4)
        roofline["copy_same_bytes"] = cp
    if step.prefill_step:
        # the long record is a chain of dependent steps, not an HBM stream
        roofline["note"] = ("latency-bound: 64 dependent chunk steps per 16-row block (gdn_prefill)"
                            if step.chunked else
                            "issue-bound: 4096 dependent steps per state row (gdn_record)")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "cache_scrub": scrub,
        "config": ({"workload": args.workload, "n_tokens": w["n_tokens"], "dim": w["dim"],
                    "eps": w["eps"], "x_dtype": "f32", "weight_dtype": "bf16",
                    "step": "rms_norm"} if isinstance(w, dict) else
                   {"workload": args.workload, "B": w.B, "T": w.T, "Hk": w.Hk, "Hv": w.Hv,
                    "Dk": w.Dk, "Dv": w.Dv, "io_dtype": w.io, "state_dtype": "f32",
                    "gqa_map": w.gqa_map, "mask": w.mask, "capture": args.capture,
                    **({"prefill": args.prefill} if step.prefill_step else {}),
                    "step": " + ".join(k[0] for k in step.kernels)}),
        "frac_of_peak": round(value / HBM_PEAK_GBPS, 4),
        "head_steps_per_s": round(head_steps / (ms_per_step * 1e-3), 1),
        "head_steps_per_step": head_steps,
        "algorithmic_bytes_per_step": step_bytes,
        "kernels": kernels,
        "roofline": roofline,
    }
    if isinstance(w, dict):
        out["tokens_per_s"] = round(w["n_tokens"] / (ms_per_step * 1e-3), 1)
    if step.prefill_step:
        out["tokens_per_s"] = round(w.B * w.T / (ms_per_step * 1e-3), 1)
    if not args.no_peak_probe:
        out["practical_peak"] = {"copy_GB/s": round(copy_bandwidth(dev), 1),
                                 "copy_bytes_each_way": COPY_BYTES,
                                 "reported": reported_hbm_figure()}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_budget, args.cpu_threads or None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
