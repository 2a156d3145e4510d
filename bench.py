"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the path over one layer's batch: pa_plan (host), then the
append of the new K/V and attention -- pa_append_kv -> pa_attention_batch, or in the
fused form the bench times, pa_decode_step (decode rows) / pa_attention_step (any
batch), which do the append inside the attention launches.  The headline workload is the Qwen3-8B
single-layer decode step (32 requests, kv_len = 2048 + U[0,255], 32 query / 8 KV
heads, head_dim 128, 16-token blocks, bf16); its value is algorithmic HBM bytes per
second of the whole step.  The mixed continuous batch (one 512-token prefill chunk at
offset 4096 plus 31 decode rows, 543 new tokens) is timed the same way and reported
in tokens/s, and the prefill chunk alone is reported against the bf16 MFMA peak.

Each step reads a different copy of the KV pools (the copies stand for different
layers), so no step finds the previous step's KV in the 256 MB last-level cache.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --kernel-only decode|decode_q8|decode_fp8|mixed|mixed_fused|mixed_q8|mixed_fp8|shared|
                                  shared_q8|shared_fp8|prefill|spec
                                                   # attention launches only, for rocprofv3
    python bench.py --summarize DIR [--title T]          # rocprofv3 CSV output -> profile text
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time
from typing import Optional

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-step attention HBM GB/s (% of peak) + mixed-batch tokens/s, Qwen3-8B layer"
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_attention_04_amd", "csrc", "pa_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_qwen3_8b_traffic.json")
CALIBRATION_COPY_BYTES = 256 << 20
KERNEL_AVG_LAUNCHES = 200       # back-to-back launches behind the roofline's average duration


def algorithmic_bytes(wl) -> dict:
    """Bytes the method itself must move for one layer step: every KV slot read once
    (a block shared by several rows counts once), Q, O, LSE, table entries and lengths,
    and the appended K / V rows (read from the new-token buffers, written to the pool)."""
    B = wl.block_size
    table = sum(-(-int(L) // B) * 4 for L in wl.kv_len)
    slots = {}
    for r in range(wl.num_reqs):
        nb = -(-int(wl.kv_len[r]) // B)
        for b in range(nb):
            blk = int(wl.block_tables[r, b])
            n = min(B, int(wl.kv_len[r]) - b * B)
            slots[blk] = max(slots.get(blk, 0), n)
    new_tok = 2 * wl.num_kv_heads * wl.head_dim * 2          # one token's bf16 K and V rows
    if getattr(wl, "kv_format", "bf16") == "q8_0":            # codes plus a 2-byte scale per 32 values
        per_tok = 2 * wl.num_kv_heads * (wl.head_dim + 2 * (wl.head_dim // 32))
    elif getattr(wl, "kv_format", "bf16") == "fp8":           # one E4M3 code per value
        per_tok = 2 * wl.num_kv_heads * wl.head_dim
    else:
        per_tok = new_tok
    kv_unique = sum(slots.values()) * per_tok
    kv_logical = int(wl.kv_len.sum()) * per_tok
    q = wl.total_q * wl.num_q_heads * wl.head_dim * 2
    o = q
    lse = wl.total_q * wl.num_q_heads * 4
    meta = table + 8 * wl.num_reqs
    append = wl.total_q * (new_tok + per_tok) + wl.total_q * 4
    return dict(kv_unique=kv_unique, kv_logical=kv_logical, attention=kv_unique + q + o + lse + meta,
                append=append, step=kv_unique + q + o + lse + meta + append)


def prefill_flops(wl) -> int:
    """4 * head_dim * Hq FLOPs per visible (query, key) pair of the prefill rows."""
    pairs = 0
    for r in range(wl.num_reqs):
        c, kv = int(wl.qo_len[r]), int(wl.kv_len[r])
        if c > 1:
            h = kv - c
            pairs += c * h + c * (c + 1) // 2
    return pairs * 4 * wl.head_dim * wl.num_q_heads


def prefill_only_workload(poison=False):
    import synthetic
    return synthetic.build("prefill_512_at_4096", 4, 32, 8, qo_len=[512], kv_len=[4608],
                           num_blocks=synthetic.POOL_BLOCKS_12GIB, poison=poison)


def spec_verify_workload(poison=False):
    """Speculative verification rows: 16 requests x 8 new tokens (causal) at 8192 tokens of context."""
    import synthetic
    return synthetic.build("spec_verify", 91, 32, 8, qo_len=[8] * 16, kv_len=[8192 + 8] * 16,
                           num_blocks=16 * (8192 // 16 + 2) + 64, poison=poison)


class Stepper:
    """Device copies of a workload, with `copies` KV-pool replicas rotated per step."""

    def __init__(self, wl, copies: int, device="cuda", cascade: bool = False, fused: bool = False,
                 one_launch: Optional[int] = None):
        import torch

        import paged_kv_attention_04_amd as pa

        self.pa, self.wl = pa, wl
        self.g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
        self.num_cus = pa.num_cus(0)
        if getattr(wl, "kv_format", "bf16") == "q8_0":
            kvp = pa.to_device(wl.kv_pool, device)      # one pool: K and V tiles side by side
            self.pools = [(kvp, None)] + [(kvp.clone(), None) for _ in range(copies - 1)]
        else:
            kp, vp = pa.to_device(wl.k_pool, device), pa.to_device(wl.v_pool, device)
            self.pools = [(kp, vp)] + [(kp.clone(), vp.clone()) for _ in range(copies - 1)]
        self.q = pa.to_device(wl.q, device)
        self.bt = pa.to_device(wl.block_tables, device)
        self.qo_indptr = pa.to_device(wl.qo_indptr, device)
        self.kv = pa.to_device(wl.kv_len, device)
        self.sm = pa.to_device(wl.slot_mapping, device)
        self.kn, self.vn = pa.to_device(wl.k_new, device), pa.to_device(wl.v_new, device)
        self.out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device=device)
        self.lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device=device)
        self.cascade = cascade
        self.fused = fused               # decode-only batches: append fused into the attention launch
        self.q8 = getattr(wl, "kv_format", "bf16") == "q8_0"
        self.fp8 = getattr(wl, "kv_format", "bf16") == "fp8"
        self.one_launch = one_launch     # None: the planner's choice of one or two launches
        self.plan = self.make_plan()
        self.ws = pa.workspace_for(self.plan, device)
        self.i = 0

    def make_plan(self):
        wl = self.wl
        plan = self.pa.pa_plan(self.g, wl.qo_len, wl.kv_len, self.num_cus)
        if self.cascade:
            self.pa.pa_plan_shared_prefix(self.g, plan, wl.qo_len, wl.kv_len, wl.block_tables, self.num_cus,
                                          q8=getattr(wl, "kv_format", "bf16") == "q8_0")
        if self.one_launch is not None:
            plan.one_launch = self.one_launch
        return plan

    def step(self, attention_only: bool = False):
        pa, wl = self.pa, self.wl
        kp, vp = self.pools[self.i % len(self.pools)]
        self.i += 1
        if self.fused:
            if not attention_only:
                self.plan = self.make_plan()
            if self.q8:
                step = pa.pa_attention_step_q8 if self.plan.num_prefill_rows > 0 else pa.pa_decode_step_q8
                step(self.g, self.plan, self.q, kp, self.kn, self.vn, self.bt, self.qo_indptr, self.kv,
                     self.out, self.lse, self.ws)
                return
            if self.fp8:
                step = pa.pa_attention_step_fp8 if self.plan.num_prefill_rows > 0 else pa.pa_decode_step_fp8
                step(self.g, self.plan, self.q, kp, vp, self.kn, self.vn, self.bt, self.qo_indptr, self.kv,
                     self.out, self.lse, self.ws, wl.k_scale, wl.v_scale)
                return
            step = pa.pa_attention_step if self.plan.num_prefill_rows > 0 else pa.pa_decode_step
            step(self.g, self.plan, self.q, kp, vp, self.kn, self.vn, self.bt, self.qo_indptr, self.kv,
                 self.out, self.lse, self.ws)
            return
        if not attention_only:
            self.plan = self.make_plan()
            if self.q8:
                pa.pa_append_kv_q8(self.g, kp, self.kn, self.vn, self.sm)
            elif self.fp8:
                pa.pa_append_kv_fp8(self.g, kp, vp, self.kn, self.vn, self.sm, wl.k_scale, wl.v_scale)
            else:
                pa.pa_append_kv(self.g, kp, vp, self.kn, self.vn, self.sm)
        if self.q8:
            pa.pa_attention_batch_q8(self.g, self.plan, self.q, kp, self.bt, self.qo_indptr, self.kv, self.out,
                                     self.lse, self.ws)
        elif self.fp8:
            pa.pa_attention_batch_fp8(self.g, self.plan, self.q, kp, vp, self.bt, self.qo_indptr, self.kv, self.out,
                                      self.lse, self.ws, wl.k_scale, wl.v_scale)
        else:
            pa.pa_attention_batch(self.g, self.plan, self.q, kp, vp, self.bt, self.qo_indptr, self.kv, self.out,
                                  self.lse, self.ws)


def time_steps(stepper, steps: int, warmup: int, attention_only: bool = False, events: bool = False):
    """Seconds per step over exactly `steps` steps, bracketed by synchronisations.  Python's
    garbage collector runs before the warmup steps and is paused until the timed steps
    end, so the device goes from the warmup straight into the timed steps.  With
    `events`, also the device time per step from HIP events recorded on the current
    stream (the one the library launches on) before the first and after the last timed
    step: returns (wall seconds per step, event seconds per step)."""
    import gc

    import torch
    gc.collect()
    gc.disable()
    try:
        for _ in range(warmup):
            stepper.step(attention_only)
        stream = torch.cuda.current_stream()
        ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if events else None
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if ev:
            ev[0].record(stream)
        for _ in range(steps):
            stepper.step(attention_only)
        if ev:
            ev[1].record(stream)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps
    finally:
        gc.enable()
    if ev:
        return wall, ev[0].elapsed_time(ev[1]) * 1e-3 / steps
    return wall


def event_time(stepper, reps: int) -> float:
    """Average device time of one attention call (the plan fixed): HIP events on the
    current stream -- the stream the library launches on -- around `reps` back-to-back
    calls, divided by `reps`."""
    import gc

    import torch
    stream = torch.cuda.current_stream()
    gc.collect()
    gc.disable()
    try:
        for _ in range(5):
            stepper.step(attention_only=True)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            stepper.step(attention_only=True)
        b.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    return a.elapsed_time(b) * 1e-3 / reps


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch", {}).get("total")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _sampled_rows(wl, every: int):
    """Every `every`-th query row of a workload as its own one-token row at the same
    position: the same keys through the same table row, so the oracle does exactly that
    row's share of the work.  Returns (q, block_tables, qo_len, kv_len)."""
    rows, bts, kvs = [], [], []
    for r in range(wl.num_reqs):
        q0, ql, kv = int(wl.qo_indptr[r]), int(wl.qo_len[r]), int(wl.kv_len[r])
        for i in range(ql):
            if (q0 + i) % every == 0:
                rows.append(q0 + i)
                bts.append(r)
                kvs.append(kv - ql + i + 1)
    n = len(rows)
    return (np.ascontiguousarray(wl.q[rows]), np.ascontiguousarray(wl.block_tables[bts]), np.ones(n, np.int32),
            np.asarray(kvs, np.int32))


def _oracle_rate(wl, kp, vp, every: int, min_seconds: float) -> dict:
    """Attention passes of the oracle over a workload (every `every`-th query row when
    every > 1) until `min_seconds` have passed, at least one: seconds per pass and
    (query, key) pairs per second, pairs counted per query head as the oracle counts them."""
    import oracle
    fmt = getattr(wl, "kv_format", "bf16")
    q, bt, qo, kv = (wl.q, wl.block_tables, wl.qo_len, wl.kv_len) if every == 1 else _sampled_rows(wl, every)
    reps, pairs = 0, 0
    t0 = time.perf_counter()
    while True:
        res = oracle.attention(q, kp, vp, bt, qo, kv, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_size,
                               wl.num_blocks, wl.scale, kv_format=fmt)
        reps += 1
        pairs += res["pairs"]
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"pass_s": el / reps, "pairs_per_s": pairs / el, "passes": reps}


def _full_pairs(wl) -> int:
    """Visible (query, key) pairs of a whole workload (per query head)."""
    return int(sum(int(q) * (int(kv) - int(q)) + int(q) * (int(q) + 1) // 2 for q, kv in zip(wl.qo_len, wl.kv_len)))


def cpu_baseline(min_seconds: float = 0.5, pair_budget: int = 40_000, built: Optional[dict] = None) -> dict:
    """The oracle as it stands (fp64 C, OpenMP over rows and heads), timed on the host on
    every workload, with all host threads and with one thread.  Each timing covers at
    most about `pair_budget` (query, key) pairs per thread: a workload with more is timed
    on every k-th query row and its whole pass extrapolated from the pairs per second
    (the oracle's cost is linear in the pairs).  The 36-layer workload is timed for one
    layer and multiplied by 36, and says so.  The headline value is the decode-step
    workload at all threads, in the headline's unit.  `built` may hold workloads the caller
    already made ("decode", "shared", "mixed"; unpoisoned)."""
    import oracle
    import synthetic

    built = built or {}
    nproc = oracle.num_threads()
    out = {"cpu_model": cpu_model(), "threads_all": nproc, "configs": []}
    _, chunks = synthetic.prompt_chunks(seed=5, prompt_len=2048, chunk=512, num_blocks=256, poison=False)
    cases = [("tiny: 4 decode rows, kv_len 17/64/100/250, 8 q / 2 kv heads", synthetic.config_tiny(poison=False), 1),
             ("qwen3_8b_decode_step: 32 x (2048 + U[0,255])",
              built.get("decode") or synthetic.config_decode(poison=False), 1),
             ("shared_prefix: 16 x (8192 + U[0,255]), 6144 shared",
              built.get("shared") or synthetic.config_shared_prefix(poison=False), 1),
             ("mixed: 512-token chunk at 4096 + 31 decode rows", built.get("mixed") or synthetic.config_mixed(poison=False), 1),
             ("36-layer sweep, batch-32 decode layer (x 36 layers)",
              synthetic.config_sweep_decode(32, 0, poison=False), 36)]
    cases += [(f"36-layer sweep, 2048-token prompt, chunk {i} of 4 x 512 (x 36 layers)", c, 36)
              for i, c in enumerate(chunks)]
    head = None
    for name, wl, layers in cases:
        kp, vp = oracle.append(wl.k_pool, wl.v_pool, wl.k_new, wl.v_new, wl.slot_mapping, wl.num_kv_heads,
                               wl.head_dim, wl.block_size, wl.num_blocks)
        full = _full_pairs(wl)
        for threads in (nproc, 1):
            oracle.set_num_threads(threads)
            every = max(1, -(-full // (pair_budget * threads)))
            rate = _oracle_rate(wl, kp, vp, every, min_seconds if every == 1 else 0.0)
            pass_s = full / rate["pairs_per_s"] if every > 1 else rate["pass_s"]
            sample = (f"every {every}th query row, whole pass extrapolated from pairs/s" if every > 1
                      else f"{rate['passes']} whole passes")
            out["configs"].append({
                "workload": name, "threads": threads, "pass_s": round(pass_s * layers, 5),
                "new_tokens_per_s": round(wl.total_q / pass_s, 2), "pairs_per_s": round(rate["pairs_per_s"], 1),
                "sample": sample + (f"; one layer timed, pass_s x {layers} layers" if layers > 1 else "")})
            if name.startswith("qwen3_8b_decode_step") and threads == nproc:
                head = (wl, pass_s, sample)
    oracle.set_num_threads(nproc)
    wl, pass_s, sample = head
    ab = algorithmic_bytes(wl)
    out.update({"value": round(ab["attention"] / pass_s / 1e9, 4), "unit": "GB/s", "cores": nproc,
                "kind": "oracle",
                "sample": f"decode-step workload (32 requests, {int(wl.kv_len.sum())} KV tokens): {sample}, fp64 C "
                          f"oracle, {nproc} threads; every workload at {nproc} threads and at 1 thread under configs"})
    return out


SWEEP_LAYERS = 36


class LayerStack:
    """One workload's tables, lengths, slots, Q and new K/V, with a separate device KV
    pool per layer (the same block ids index every layer's pool: a block is one page per
    layer); pool values are random bf16 drawn on the device."""

    def __init__(self, wl, layers: int = SWEEP_LAYERS, cascade: bool = False, device="cuda"):
        import torch

        import paged_kv_attention_04_amd as pa

        self.pa, self.wl, self.layers = pa, wl, layers
        self.g = pa.Geometry.make(wl.num_q_heads, wl.num_kv_heads, wl.num_blocks, wl.scale)
        self.num_cus = pa.num_cus(0)
        shape = (wl.num_blocks, wl.num_kv_heads, wl.block_size, wl.head_dim)
        gen = torch.Generator(device=device).manual_seed(5)
        self.pools = [tuple(torch.randn(shape, generator=gen, dtype=torch.bfloat16, device=device).view(torch.int16)
                            for _ in range(2)) for _ in range(layers)]
        self.q = pa.to_device(wl.q, device)
        self.bt = pa.to_device(wl.block_tables, device)
        self.qo_indptr = pa.to_device(wl.qo_indptr, device)
        self.kv = pa.to_device(wl.kv_len, device)
        self.sm = pa.to_device(wl.slot_mapping, device)
        self.kn, self.vn = pa.to_device(wl.k_new, device), pa.to_device(wl.v_new, device)
        self.out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.int16, device=device)
        self.lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device=device)
        self.cascade = cascade
        self.plan = self.make_plan()
        self.ws = pa.workspace_for(self.plan, device)

    def make_plan(self):
        wl = self.wl
        plan = self.pa.pa_plan(self.g, wl.qo_len, wl.kv_len, self.num_cus)
        if self.cascade:
            self.pa.pa_plan_shared_prefix(self.g, plan, wl.qo_len, wl.kv_len, wl.block_tables, self.num_cus,
                                          q8=getattr(wl, "kv_format", "bf16") == "q8_0")
        return plan

    def step(self, replan: bool = True, fused: bool = False):
        """One model step: the plan once, then per layer the append and the attention
        (one launch per layer with `fused`: pa_decode_step, decode-only batches)."""
        pa = self.pa
        if replan:
            self.plan = self.make_plan()
        for kp, vp in self.pools:
            if fused:
                step = pa.pa_attention_step if self.plan.num_prefill_rows > 0 else pa.pa_decode_step
                step(self.g, self.plan, self.q, kp, vp, self.kn, self.vn, self.bt, self.qo_indptr, self.kv, self.out,
                     self.lse, self.ws)
                continue
            pa.pa_append_kv(self.g, kp, vp, self.kn, self.vn, self.sm)
            pa.pa_attention_batch(self.g, self.plan, self.q, kp, vp, self.bt, self.qo_indptr, self.kv, self.out,
                                  self.lse, self.ws)


def median_step_seconds(fn, steps: int, warmup: int) -> float:
    """Median over `steps` runs of fn, each bracketed by HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev])) * 1e-3


def sweep36(steps: int = 20, warmup: int = 5) -> dict:
    """36-layer decode steps at batch 1 (short, long), 8, 32, 64, eager and replayed from a
    captured graph, and a 2048-token prompt in four 512-token chunks over 36 layers."""
    import torch

    import synthetic

    res = {"layers": SWEEP_LAYERS, "decode": []}
    for batch, long_only in ((1, False), (1, True), (8, False), (32, False), (64, False)):
        wl = synthetic.config_sweep_decode(batch, 0, long_only=long_only, poison=False, fill_pools=False)
        ab = algorithmic_bytes(wl)
        stack = LayerStack(wl, cascade=True)
        t = median_step_seconds(stack.step, steps, warmup)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            stack.step(replan=False)                    # warm up on the capture stream's side
        torch.cuda.current_stream().wait_stream(side)
        with torch.cuda.graph(graph):
            stack.step(replan=False)
        tg = median_step_seconds(graph.replay, steps, warmup)
        graph_f = torch.cuda.CUDAGraph()             # append fused into the attention launch
        with torch.cuda.graph(graph_f):
            stack.step(replan=False, fused=True)
        tf = median_step_seconds(graph_f.replay, steps, warmup)
        unique = ab["step"] * SWEEP_LAYERS
        logical = (ab["kv_logical"] - ab["kv_unique"] + ab["step"]) * SWEEP_LAYERS
        res["decode"].append({
            "batch": batch, "context": "8192 (6144 shared)" if long_only else ("2048" if batch == 1 else "half 2048, half 8192 sharing 6144"),
            "step_ms": round(t * 1e3, 4), "graph_step_ms": round(tg * 1e3, 4),
            "graph_fused_step_ms": round(tf * 1e3, 4),
            "unique_gb_per_step": round(unique / 1e9, 4), "unique_gbs": round(unique / tg / 1e9, 1),
            "logical_gbs": round(logical / tg / 1e9, 1), "frac_of_hbm_peak": round(unique / tg / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s": round(batch / tg, 1), "prefix_groups": stack.plan.num_prefix_groups,
            "pool_blocks_per_layer": wl.num_blocks,
            "pool": ("12 GiB / 36 layers" if wl.num_blocks <= synthetic.POOL_BLOCKS_12GIB else
                     f"enlarged past 12 GiB / 36 layers ({synthetic.POOL_BLOCKS_12GIB} blocks per layer): "
                     f"the batch's tables need {wl.num_blocks}")})
        del stack, graph, graph_f
        torch.cuda.empty_cache()
    # 2048-token prompt, four 512-token chunks, 36 layers each
    _, chunks = synthetic.prompt_chunks(seed=5, prompt_len=2048, chunk=512, num_blocks=256, poison=False)
    stacks = [LayerStack(c) for c in chunks]
    flops = sum(prefill_flops(c) for c in chunks) * SWEEP_LAYERS

    def prompt(fused):
        for st in stacks:
            st.step(replan=True, fused=fused)
    t_sep = median_step_seconds(lambda: prompt(False), max(steps // 2, 5), 2)
    t = median_step_seconds(lambda: prompt(True), max(steps // 2, 5), 2)
    res["prefill_2k_in_4x512"] = {"ms": round(t * 1e3, 4), "tflops": round(flops / t / 1e12, 1),
                                  "frac_of_bf16_mfma_peak": round(flops / t / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                                  "tokens_per_s": round(2048 / t, 1),
                                  "step": "per chunk and layer: pa_plan + pa_attention_step (a short append launch, then the chunk tiles)",
                                  "ms_append_then_attention": round(t_sep * 1e3, 4)}
    return res


def kernel_only(which: str, reps: int):
    """Attention launches only (plus one calibration copy of known size), for counters."""
    import torch

    import paged_kv_attention_04_amd as pa
    import synthetic

    torch.cuda.set_device(0)
    pa.lib()
    wl = {"decode": lambda: synthetic.config_decode(poison=False),
          "decode_q8": lambda: synthetic.config_decode_q8(poison=False),
          "decode_fp8": lambda: synthetic.config_decode_fp8(poison=False),
          "mixed_fp8": lambda: synthetic.config_mixed_fp8(poison=False),
          "shared_fp8": lambda: synthetic.config_shared_prefix_fp8(poison=False),
          "mixed": lambda: synthetic.config_mixed(poison=False),
          "mixed_fused": lambda: synthetic.config_mixed(poison=False),
          "mixed_q8": lambda: synthetic.config_mixed_q8(poison=False),
          "shared_q8": lambda: synthetic.config_shared_prefix_q8(poison=False),
          "shared": lambda: synthetic.config_shared_prefix(poison=False),
          "prefill": prefill_only_workload,
          "spec": spec_verify_workload}[which]()
    st = Stepper(wl, 4, cascade=which in ("shared", "shared_q8", "shared_fp8"), fused=which in ("decode", "mixed_fused"))
    src = torch.empty(CALIBRATION_COPY_BYTES // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)                                           # calibration: reads and writes 256 MiB
    for _ in range(reps):
        st.step(attention_only=True)
    torch.cuda.synchronize()
    print(json.dumps({"kernel_only": which, "launches": reps, "attention_bytes": algorithmic_bytes(wl)["attention"],
                      "calibration_copy_bytes": CALIBRATION_COPY_BYTES}), flush=True)


def summarize(directory: str, title: str):
    """Turn rocprofv3 CSV output (kernel trace and / or counter collection) into text."""
    import csv
    from collections import defaultdict
    lines = [f"### {title}", ""]
    for f in sorted(glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True)):
        lines += ["| kernel | calls | avg us | min us | max us | total us |", "|---|---|---|---|---|---|"]
        for r in csv.DictReader(open(f)):
            name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0]
            lines.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | {float(r['MinNs']) / 1e3:.3f} | "
                         f"{float(r['MaxNs']) / 1e3:.3f} | {float(r['TotalDurationNs']) / 1e3:.1f} |")
        lines.append("")
    for f in sorted(glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)):
        per = defaultdict(list)
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
            grid = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0)
            wg = int(r.get("Workgroup_Size_X", r.get("Workgroup_Size", 1)) or 1)
            per[(name, grid // max(wg, 1))].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += ["| kernel | workgroups | calls | avg us | median us | min us |", "|---|---|---|---|---|---|"]
        for (name, wgs), d in sorted(per.items()):
            lines.append(f"| {name} | {wgs} | {len(d)} | {np.mean(d):.3f} | {np.median(d):.3f} | {min(d):.3f} |")
        lines.append("")
    for f in sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)):
        agg = defaultdict(list)
        for r in csv.DictReader(open(f)):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0]
            agg[(name, r["Counter_Name"])].append(float(r["Counter_Value"]))
        lines += ["| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
        for (name, c), v in sorted(agg.items()):
            lines.append(f"| {name} | {c} | {len(v)} | {sum(v) / len(v):.1f} |")
        lines.append("")
    print("\n".join(lines))


def write_traffic(fetch_dir: str, write_dir: str):
    """HBM bytes per decode launch from two counter runs of `--kernel-only decode`
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by what the same counter
    reads for the calibration copy of known size; written next to the kernel-source hash."""
    import csv

    def per_kernel(directory, counter):
        vals = {}
        for f in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = "decode" if "pa_decode_split" in r["Kernel_Name"] else (
                    "copy" if "pa_" not in r["Kernel_Name"] else "other")
                vals.setdefault(key, []).append(float(r["Counter_Value"]))
        return vals

    f, w = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")
    kib_true = CALIBRATION_COPY_BYTES / 1024
    read_scale = kib_true / max(f["copy"])       # the largest non-library dispatch is the 256 MiB copy
    write_scale = kib_true / max(w["copy"])
    read = float(np.mean(f["decode"])) * 1024 * read_scale
    write = float(np.mean(w["decode"])) * 1024 * write_scale
    out = {"kernel": "pa_decode_split", "workload": "qwen3_8b_decode_step",
           "kernel_source_sha256_16": kernel_source_hash(),
           "fetch_kib_per_dispatch": float(np.mean(f["decode"])), "write_kib_per_dispatch": float(np.mean(w["decode"])),
           "calibration": {"copy_bytes": CALIBRATION_COPY_BYTES, "fetch_kib": max(f["copy"]), "write_kib": max(w["copy"]),
                           "read_scale": read_scale, "write_scale": write_scale},
           "bytes_per_launch": {"read": round(read), "write": round(write), "total": round(read + write)}}
    json.dump(out, open(TRAFFIC_FILE, "w"), indent=1)
    print(json.dumps(out))


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=8, help="KV pool replicas rotated over the steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 36-layer sweep")
    ap.add_argument("--cpu-seconds", type=float, default=0.5, help="least seconds per whole-pass CPU timing")
    ap.add_argument("--only", choices=["headline"], help="run the headline step only (for rocprofv3)")
    ap.add_argument("--kernel-only", choices=["decode", "decode_q8", "decode_fp8", "mixed", "mixed_fused", "mixed_q8",
                                              "mixed_fp8", "shared", "shared_q8", "shared_fp8", "prefill", "spec"])
    ap.add_argument("--reps", type=int, default=20)
    ap.add_argument("--summarize")
    ap.add_argument("--title", default="rocprofv3 summary")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args(argv)
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.summarize:
        summarize(args.summarize, args.title)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    if args.kernel_only:
        kernel_only(args.kernel_only, args.reps)
        return

    import torch

    import paged_kv_attention_04_amd as pa
    import synthetic

    torch.cuda.set_device(0)
    pa.lib()

    # headline: Qwen3-8B single-layer decode step (plan + append + attention)
    wl = synthetic.config_decode(poison=False)
    ab = algorithmic_bytes(wl)
    st = Stepper(wl, args.copies, fused=True)      # plan + pa_decode_step (append fused into attention)
    sec, sec_ev = time_steps(st, args.steps, args.warmup, events=True)
    t_attn = event_time(st, KERNEL_AVG_LAUNCHES)   # the one launch of a step, back to back
    value = ab["step"] / sec / 1e9
    achieved = ab["step"] / t_attn / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                "kernel": "pa_decode_split<false, true> (bf16 pool, append fused: the one launch of a step)",
                "avg_us": round(t_attn * 1e6, 3),
                "avg_us_from": f"HIP events on the launch stream around {KERNEL_AVG_LAUNCHES} back-to-back launches",
                "avg_us_timed_region": round(sec_ev * 1e6, 3),
                "bytes_per_launch": ab["step"]}
    config = {"workload": "qwen3_8b_decode_step: 32 requests, kv_len 2048+U[0,255], 32 q / 8 kv heads, "
                          "head_dim 128, 16-token blocks, bf16 KV pool of 5461 blocks, 1 layer; "
                          "step = pa_plan + pa_decode_step (the append fused into the attention launch)",
              "kv_bytes_unique": ab["kv_unique"], "step_bytes": ab["step"],
              "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
              "plan": {"split_blocks": st.plan.split_blocks, "max_splits": st.plan.max_splits,
                       "decode_workgroups": st.plan.decode_items}}
    line = {"metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": config, "roofline": roofline}
    if args.only == "headline":
        print(json.dumps(line), flush=True)
        return

    # mixed continuous batch: tokens per second of a whole step
    wm = synthetic.config_mixed(poison=False)
    sm = Stepper(wm, args.copies, fused=True)
    sec_m = float(np.median([time_steps(sm, args.steps, args.warmup) for _ in range(3)]))   # median of 3 runs
    t_m = event_time(sm, max(args.steps, 50))
    del sm
    sm2 = Stepper(wm, args.copies)                 # the same step as pa_append_kv + pa_attention_batch
    sec_m2 = float(np.median([time_steps(sm2, args.steps, args.warmup) for _ in range(3)]))
    del sm2

    # shared-prefix decode (16 requests share 6144 tokens), plain and with the cascade plan
    ws3 = synthetic.config_shared_prefix(poison=False)
    ab3 = algorithmic_bytes(ws3)
    shared = {"workload": "16 requests, kv_len 8192+U[0,255], first 384 blocks (6144 tokens) shared",
              "kv_bytes_unique": ab3["kv_unique"], "kv_bytes_logical": ab3["kv_logical"]}
    for cascade in (False, True):
        s3 = Stepper(ws3, 4, cascade=cascade)
        time_steps(s3, 10, 5, attention_only=True)
        t3 = event_time(s3, max(args.steps // 2, 50))
        shared["cascade" if cascade else "plain"] = {
            "attention_us": round(t3 * 1e6, 3), "unique_gbs": round(ab3["attention"] / t3 / 1e9, 1),
            "frac_of_hbm_peak": round(ab3["attention"] / t3 / 1e9 / HBM_PEAK_GBS, 4),
            "prefix_groups": s3.plan.num_prefix_groups, "prefix_splits": s3.plan.prefix_splits}
        del s3

    # the same decode step on a q8_0 pool (same lengths and tables): the saving against
    # the pages' model, saving = fewer bytes / bandwidth - conversion time
    del st
    # the saving model's three attention times (bf16, q8_0, FP8: attention alone, append
    # separate), each after a warm-up of its own and the least of three timed runs (the
    # shorter quantised launches are the likelier to catch a slow stretch of the box)
    def least_time(st):
        return min(event_time(st, max(args.steps // 2, 50)) for _ in range(3))
    st_plain = Stepper(wl, args.copies)            # bf16 attention alone, the q8_0 line's reference
    time_steps(st_plain, 10, 5, attention_only=True)
    t_plain = least_time(st_plain)
    del st_plain
    wq = synthetic.config_decode_q8(poison=False)
    abq = algorithmic_bytes(wq)
    sq = Stepper(wq, args.copies)                  # attention alone (append separate): the saving model
    time_steps(sq, 10, 5, attention_only=True)
    t_q = least_time(sq)
    del sq
    sq = Stepper(wq, args.copies, fused=True)      # the step: plan + pa_decode_step_q8 (append fused)
    sec_q = time_steps(sq, args.steps, args.warmup)
    del sq
    fewer = ab["attention"] - abq["attention"]
    predicted = fewer / (ab["attention"] / t_plain)
    q8 = {"workload": "qwen3_8b_decode_step on a q8_0 pool (32-value groups, int8 codes, binary16 scales; "
                      "each (block, KV head) K tile then V tile), same lengths and block tables",
          "attention_us": round(t_q * 1e6, 3), "bytes_per_launch": abq["attention"],
          "gbs": round(abq["attention"] / t_q / 1e9, 1),
          "frac_of_hbm_peak": round(abq["attention"] / t_q / 1e9 / HBM_PEAK_GBS, 4),
          "step_ms": round(sec_q * 1e3, 5), "step": "pa_plan + pa_decode_step_q8 (append fused)",
          "bf16_attention_us": round(t_plain * 1e6, 3),
          "fewer_bytes": fewer, "bf16_gbs": round(ab["attention"] / t_plain / 1e9, 1),
          "predicted_saving_us": round(predicted * 1e6, 3),
          "measured_saving_us": round((t_plain - t_q) * 1e6, 3),
          "implied_conversion_us": round((predicted - (t_plain - t_q)) * 1e6, 3)}
    # the mixed batch on a q8_0 pool: the append quantises in its own launch, then the chunk
    # row runs the matrix-unit tile over codes and the decode rows the q8_0 decode kernel
    wmq = synthetic.config_mixed_q8(poison=False)
    smq = Stepper(wmq, args.copies, fused=True)
    sec_mq = time_steps(smq, args.steps, args.warmup)
    t_mq = event_time(smq, max(args.steps // 2, 50))
    del smq
    q8["mixed_batch"] = {"workload": "1 prefill row (512 tokens at offset 4096) + 31 decode rows on a q8_0 pool",
                         "step": "pa_plan + pa_attention_step_q8 (all appends inside the decode launch, then the chunk tiles)",
                         "tokens_per_s": round(wmq.total_q / sec_mq, 1), "ms_per_step": round(sec_mq * 1e3, 5),
                         "attention_launches_us": round(t_mq * 1e6, 3)}
    wsq = synthetic.config_shared_prefix_q8(poison=False)
    ssq = Stepper(wsq, 2, cascade=True)
    time_steps(ssq, 10, 5, attention_only=True)
    t_sq = event_time(ssq, max(args.steps // 2, 50))
    q8["shared_prefix_cascade"] = {"workload": "the shared-prefix decode (16 rows, 384 shared blocks) on a q8_0 pool",
                                   "attention_us": round(t_sq * 1e6, 3), "prefix_splits": ssq.plan.prefix_splits}
    del ssq

    # the same three on FP8 pools (E4M3 codes, per-pool scales): half the KV bytes of bf16,
    # the codes widened to bf16 in registers (decode) or on their way into LDS (tiles)
    wf = synthetic.config_decode_fp8(poison=False)
    abf = algorithmic_bytes(wf)
    sf = Stepper(wf, args.copies)                  # attention alone (append separate): the saving model
    time_steps(sf, 10, 5, attention_only=True)
    t_f = least_time(sf)
    del sf
    sf = Stepper(wf, args.copies, fused=True)      # the step: plan + pa_decode_step_fp8 (append fused)
    sec_f = time_steps(sf, args.steps, args.warmup)
    del sf
    fewer_f = ab["attention"] - abf["attention"]
    predicted_f = fewer_f / (ab["attention"] / t_plain)
    fp8 = {"workload": "qwen3_8b_decode_step on FP8 pools (OCP E4M3 codes, one K and one V scale, the bf16 "
                       "layout), same lengths and block tables",
           "attention_us": round(t_f * 1e6, 3), "bytes_per_launch": abf["attention"],
           "gbs": round(abf["attention"] / t_f / 1e9, 1),
           "frac_of_hbm_peak": round(abf["attention"] / t_f / 1e9 / HBM_PEAK_GBS, 4),
           "step_ms": round(sec_f * 1e3, 5), "step": "pa_plan + pa_decode_step_fp8 (append fused)",
           "bf16_attention_us": round(t_plain * 1e6, 3), "fewer_bytes": fewer_f,
           "predicted_saving_us": round(predicted_f * 1e6, 3),
           "measured_saving_us": round((t_plain - t_f) * 1e6, 3),
           "implied_conversion_us": round((predicted_f - (t_plain - t_f)) * 1e6, 3)}
    wmf = synthetic.config_mixed_fp8(poison=False)
    smf = Stepper(wmf, args.copies, fused=True)
    sec_mf = time_steps(smf, args.steps, args.warmup)
    t_mf = event_time(smf, max(args.steps // 2, 50))
    del smf
    fp8["mixed_batch"] = {"workload": "1 prefill row (512 tokens at offset 4096) + 31 decode rows on FP8 pools",
                          "step": "pa_plan + pa_attention_step_fp8 (all appends inside the decode launch, then the chunk tiles)",
                          "tokens_per_s": round(wmf.total_q / sec_mf, 1), "ms_per_step": round(sec_mf * 1e3, 5),
                          "attention_launches_us": round(t_mf * 1e6, 3)}
    wsf = synthetic.config_shared_prefix_fp8(poison=False)
    ssf = Stepper(wsf, 2, cascade=True)
    time_steps(ssf, 10, 5, attention_only=True)
    t_sf = event_time(ssf, max(args.steps // 2, 50))
    fp8["shared_prefix_cascade"] = {"workload": "the shared-prefix decode (16 rows, 384 shared blocks) on FP8 pools",
                                    "attention_us": round(t_sf * 1e6, 3), "prefix_splits": ssf.plan.prefix_splits}
    del ssf

    # speculative verification: 16 requests, 8 new tokens each at 8192 tokens of context
    # (small qo_len rows, served by the chunked-prefill path; K / V streaming dominates)
    wv = spec_verify_workload()
    abv = algorithmic_bytes(wv)
    sv = Stepper(wv, 2)
    time_steps(sv, 10, 5, attention_only=True)
    t_v = event_time(sv, max(args.steps // 4, 30))
    spec = {"workload": "16 requests x 8 new tokens (causal) at kv_len 8200, 32 q / 8 kv heads",
            "attention_us": round(t_v * 1e6, 3), "bytes_per_launch": abv["attention"],
            "gbs": round(abv["attention"] / t_v / 1e9, 1),
            "frac_of_hbm_peak": round(abv["attention"] / t_v / 1e9 / HBM_PEAK_GBS, 4),
            "prefill_splits": sv.plan.prefill_splits}
    del sv

    # the prefill chunk alone, against the bf16 matrix peak
    wp = prefill_only_workload()
    sp = Stepper(wp, 2)
    time_steps(sp, 10, 5, attention_only=True)
    t_p = event_time(sp, max(args.steps // 2, 30))
    del sp
    pflops = prefill_flops(wp)

    line.update({
        "mixed_batch": {"workload": "1 prefill row (512 tokens at offset 4096) + 31 decode rows, 543 new tokens",
                        "step": "pa_plan + pa_attention_step (decode and chunk rows' appends inside the decode launch, then the chunk tiles)",
                        "tokens_per_s": round(wm.total_q / sec_m, 1), "ms_per_step": round(sec_m * 1e3, 5),
                        "launches_us": round(t_m * 1e6, 3),
                        "append_then_attention_ms_per_step": round(sec_m2 * 1e3, 5)},
        "shared_prefix": shared,
        "q8_0_decode": q8,
        "fp8_decode": fp8,
        "spec_verify": spec,
        "prefill_chunk": {"workload": "512 new tokens at kv offset 4096, 32 q / 8 kv heads, causal",
                          "us": round(t_p * 1e6, 3), "tflops": round(pflops / t_p / 1e12, 1),
                          "frac_of_bf16_mfma_peak": round(pflops / t_p / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4)},
    })
    if not args.no_sweep:
        line["sweep_36_layers"] = sweep36()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds, built={"decode": wl, "shared": ws3, "mixed": wm})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
