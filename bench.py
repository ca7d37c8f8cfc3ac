#!/usr/bin/env python3
"""Benchmark of the paged decode-attention path on one MI355X.

One step = the whole path over one batch: the store of the batch's new
tokens and pa_decode, fused in one pa_decode_append launch (or pa_cache_write
then pa_decode, for the fp8 and tree layers and with --separate-write), and
pa_reduce when the context is split.  The inputs are
the seeded synthetic Llama-3-8B-shaped decode layer (64 sequences, 32 query
heads / 8 KV heads, head_dim 128, bf16, contexts uniform in [512, 4096], a
20,000-block pool), resident in HBM before timing starts.  Before the W
warm-up steps the step runs untimed for --settle-ms (100 ms) so that the
GPU has left its idle clocks.

Prints one JSON line:
  value          tokens/s of whole steps (num_seqs * q_len tokens per step),
                 timed by wall clock over K steps with no timing event inside
  roofline       the decode kernel: algorithmic KV + Q bytes per launch over its
                 average launch time (HIP events on the launch stream; for a
                 split context the event pair spans pa_decode and pa_reduce)
                 against the 8 TB/s HBM peak; traffic from the committed counter
                 summary.  Where the K bytes are under twice the 256 MB MALL (the
                 kernels load V non-temporally, so K is what can stay cached;
                 the 8B layers), warm launches are partly served from the MALL,
                 so the figure is taken over cold launches instead.  Shared
                 prefix blocks count once; achieved_logical / frac_logical
                 count every sequence's context in full.
  roofline_cold  (roofline_warm) the same figure over the other kind of launch:
                 cold launches each follow a 512 MiB read; their time is that of
                 N (read, launch) pairs less that of N reads, one event pair each
  cpu_baseline   the fp64 oracle on a bounded sample of the same workload

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--partition P]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBPS = 8000.0
DEFAULT_CONFIG = "llama3-8b-decode"
METRIC = "decode tokens/s and achieved KV HBM GB/s (% of MI355X peak) per pa_decode call"
PREFILL_METRIC = "prefill tokens/s and attention TFLOP/s (% of MI355X bf16 matrix peak) per pa_prefill call"
KERNEL_SOURCES = ("decode_valu.hip", "decode_mfma.hip", "pa_schedule.h", "pa_kernels.h", "pa_device.h")
PREFILL_SOURCES = ("prefill.hip", "pa_prefill.h", "pa_device.h")
COPY_SOURCES = ("copy_blocks.hip", "pa_kernels.h")
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MALL_BYTES = 256 * 1024 * 1024  # MI355X Infinity Cache (memory-side, in front of HBM)

# Context split per workload, the fastest measured on MI355X (kernel trace):
# one pass where every (sequence, KV head) already gives two workgroups per CU
# (on the 8B layer the whole grid is resident at once and each CU pairs a long
# sequence with a short one: 113 us against 124 us balanced; the fp8 layer
# 70 us against 80 us, cold),
# the balanced split where ragged contexts leave CUs idle, and the workload's
# own partition size where it names one (the FlashDecoding-style split + reduce).
LAUNCH = {
    "tiny-f32": 0,
    "llama3-8b-decode": 0,
    "llama3-70b-decode": -1,
    "spec-verify": 0,
    "llama3-8b-decode-fp8kv": 0,
    "tree-verify": 0,
}


def partition_for(p: wl.Problem) -> int:
    """Launch configuration: the context split used for each workload."""
    if p.partition_size:
        return p.partition_size
    return LAUNCH.get(p.spec.name, 0)


def decode_kernel_name(p: wl.Problem, partition: int) -> str:
    if p.query_start is not None:
        return (f"prefill_kernel (bf16, head_dim {p.head_dim}, {p.spec.group} query heads per KV head, "
                f"up to {int(p.q_counts.max())} new tokens per sequence, 256 query rows per workgroup)")
    rows = p.spec.group * p.q_len
    fp8 = p.spec.kv == "fp8"
    kind = "decode_mfma_kernel" if fp8 or (p.dtype == "bf16" and rows >= 8) else "decode_valu_kernel"
    mode = "balanced" if partition < 0 else ("partitions" if partition > 0 else "one pass")
    kv = "fp8 E4M3 KV, bf16 q" if fp8 else p.dtype
    mask = f", tree mask over {p.q_len} nodes" if p.parents is not None else ""
    return f"{kind} ({kv}, head_dim {p.head_dim}, {rows} rows per KV head{mask}, {mode})"


def code_only(text: str) -> str:
    """Source text without comments and blank space: what the compiler sees of it, so that
    editing a comment does not retire counter figures taken on the same kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "paged_kv_attention_decode_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def to_dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def appended_slots(p: wl.Problem):
    """Slots of the new tokens under the append rule pa_decode_append follows (new token
    j of sequence b at position L_b - q_len + j of b's blocks), -1 where none."""
    slots = []
    for b in range(p.num_seqs):
        L = int(p.context_lens[b])
        for j in range(p.q_len):
            pos = L - p.q_len + j
            phys = int(p.block_tables[b, pos // 16]) if pos >= 0 else -1
            slots.append(phys * 16 + pos % 16 if 0 <= phys < p.num_blocks else -1)
    return np.array(slots, dtype=np.int64)


class Resident:
    """The workload in HBM and the calls of one step."""

    def __init__(self, p: wl.Problem, partition: int, torch, separate_write: bool = False):
        import paged_kv_attention_decode_amd as pa

        self.pa, self.p, self.partition, self.torch = pa, p, partition, torch
        self.q = to_dev(p.q, torch)
        # one allocation per layer, V placed by pa_kv_cache_layout (one head slice off K's offsets)
        tk = to_dev(p.k_cache, torch)
        self.k_cache, self.v_cache = pa.allocate_kv_cache(tk.shape[0], tk.shape[2], tk.shape[3], tk.dtype, "cuda")
        self.k_cache.copy_(tk)
        del tk
        self.v_cache.copy_(to_dev(p.v_cache, torch))
        self.tables = torch.from_numpy(p.block_tables).cuda()
        self.lens = torch.from_numpy(p.context_lens).cuda()
        self.new_k = to_dev(p.new_k, torch) if p.new_k is not None else None
        self.new_v = to_dev(p.new_v, torch) if p.new_v is not None else None
        self.slots = torch.from_numpy(p.slot_mapping).cuda() if p.slot_mapping is not None else None
        self.fp8 = p.spec.kv == "fp8"
        if self.fp8:
            self.k_scale = torch.from_numpy(p.k_scale).cuda()
            self.v_scale = torch.from_numpy(p.v_scale).cuda()
        self.parents = torch.from_numpy(p.parents).cuda() if p.parents is not None else None
        self.query_start = torch.from_numpy(p.query_start).cuda() if p.query_start is not None else None
        self.max_q_len = int(p.q_counts.max())
        self.out = torch.empty_like(self.q)
        self.ws = None
        if partition:
            self.ws = pa.new_workspace(self.q, self.k_cache, self.tables, p.q_len, partition)
        # the new tokens' store fused into the decode launch, where the workload's slots
        # are the appended positions (always, for the synthetic layers)
        self.fused = (not separate_write and self.new_k is not None and not self.fp8 and self.parents is None
                      and self.query_start is None and np.array_equal(appended_slots(p), p.slot_mapping))

    def write(self):
        if self.fused:
            return
        if self.new_k is not None:
            if self.fp8:
                self.pa.cache_write_fp8(self.new_k, self.new_v, self.k_cache, self.v_cache, self.slots, self.k_scale,
                                        self.v_scale)
            else:
                self.pa.cache_write(self.new_k, self.new_v, self.k_cache, self.v_cache, self.slots)

    def decode(self):
        p = self.p
        if self.query_start is not None:
            self.pa.prefill(self.q, self.k_cache, self.v_cache, self.tables, self.lens, self.query_start,
                            float(p.scale), self.max_q_len, out=self.out)
            return
        if self.parents is not None:
            self.pa.decode_tree(self.q, self.k_cache, self.v_cache, self.tables, self.lens, self.parents,
                                float(p.scale), self.partition, out=self.out, workspace=self.ws)
            return
        if self.fp8:
            self.pa.decode_fp8(self.q, self.k_cache, self.v_cache, self.k_scale, self.v_scale, self.tables, self.lens,
                               float(p.scale), p.q_len, self.partition, out=self.out, workspace=self.ws)
            return
        if self.fused:
            self.pa.decode_append(self.q, self.new_k, self.new_v, self.k_cache, self.v_cache, self.tables, self.lens,
                                  float(p.scale), p.q_len, self.partition, out=self.out if self.partition <= 0
                                  else None, workspace=self.ws)
            return
        self.pa.decode(self.q, self.k_cache, self.v_cache, self.tables, self.lens, float(p.scale), p.q_len,
                       self.partition, out=self.out, workspace=self.ws)

    def reduce(self):
        if self.partition > 0:
            p = self.p
            self.pa.reduce(self.out, self.ws, self.lens, p.q_len, p.max_blocks_per_seq, self.partition)

    def step(self):
        self.write()
        self.decode()
        self.reduce()


def calibration_copies(torch):
    """Five 1 GiB device-to-device copies in a row: rocprof_summary.py scales the
    FETCH_SIZE and WRITE_SIZE counters of the same run by what they read for these."""
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(2.0)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def load_traffic(workload: str, decode_s: float, sources=KERNEL_SOURCES):
    """HBM traffic of the attention kernel from the committed counter summary, if it
    was taken on the current kernel sources."""
    kind = {id(PREFILL_SOURCES): "prefill", id(COPY_SOURCES): "copy"}.get(id(sources), "decode")
    path = os.path.join(ROOT, "profiles", f"{kind}_traffic_{workload}.json")
    if not os.path.exists(path):
        return None, None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash(sources):
        return None, "kernel changed since the counters were taken"
    per_launch = float(t["fetch_bytes_per_launch"]) + float(t["write_bytes_per_launch"])
    return per_launch / decode_s / 1e9, per_launch


def cpu_baseline(p: wl.Problem, gpu_out, budget_s: float = 10.0):
    """The oracle, untuned, on the same workload: the cache write of the batch's
    new tokens once, then attention sequence by sequence (cycling over the batch)
    until the time budget is spent; scaled to tokens/s of whole steps."""
    import oracle
    from threadpoolctl import threadpool_info

    t0 = time.perf_counter()
    fp8 = p.spec.kv == "fp8"
    if p.new_k is None:
        kc, vc = p.k_cache, p.v_cache
    elif fp8:
        kc, vc = oracle.cache_write_fp8(p.k_cache, p.v_cache, p.new_k, p.new_v, p.slot_mapping, p.k_scale, p.v_scale,
                                        p.dtype)
    else:
        kc, vc = oracle.cache_write(p.k_cache, p.v_cache, p.new_k, p.new_v, p.slot_mapping)
    t_write = time.perf_counter() - t0
    n = 0
    worst = 0.0
    t0 = time.perf_counter()
    while n < p.num_seqs or time.perf_counter() - t0 < budget_s:
        b = n % p.num_seqs
        rows = [(b, j, h) for j in range(int(p.q_counts[b])) for h in range(p.num_q_heads)]
        if p.query_start is not None:
            ref = oracle.paged_prefill_rows(p.q, kc, vc, p.block_tables, p.context_lens, p.query_start, p.scale,
                                            p.dtype, rows)
        elif p.parents is not None:
            ref = oracle.paged_tree_decode_rows(p.q, kc, vc, p.block_tables, p.context_lens, p.parents, p.scale,
                                                p.dtype, rows)
        elif fp8:
            ref = oracle.paged_decode_fp8_rows(p.q, kc, vc, p.k_scale, p.v_scale, p.block_tables, p.context_lens,
                                               p.scale, p.q_len, p.dtype, rows)
        else:
            ref = oracle.paged_decode_rows(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, p.q_len, p.dtype,
                                           rows)
        if gpu_out is not None and n < p.num_seqs and rows:
            r0 = int(p.query_start[b]) if p.query_start is not None else b * p.q_len
            got = np.stack([gpu_out[r0 + j, h] for (_, j, h) in rows])
            worst = max(worst, float(np.max(np.abs(got - ref))))
        n += 1
        if n >= p.num_seqs and time.perf_counter() - t0 >= budget_s:
            break
    t_attn = time.perf_counter() - t0
    est = t_write + t_attn * p.num_seqs / n
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": int(p.q_counts.sum()) / est,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"fp64 NumPy oracle on the same workload: cache write of all "
                   f"{len(p.slot_mapping) if p.slot_mapping is not None else 0} new tokens ({t_write:.2f} s), then "
                   f"attention of {n} sequences x {p.num_q_heads} heads x their new tokens "
                   f"({int(p.q_counts.sum())} in the batch), cycling over the "
                   f"batch of {p.num_seqs} ({t_attn:.2f} s); tokens/s of whole steps"),
        "max_abs_vs_gpu": worst,
    }


PCIE_PEAK_GBPS = 64.0  # host link: PCIe 5.0 x16, one direction


def bench_copy_blocks(args, torch) -> int:
    """pa_copy_blocks of 2048 distinct random blocks (K and V) of the workload's pool.

    copy-blocks: within the pool (copy-on-write); every call reads and writes
    2 x 2048 blocks of HBM, rated against the HBM peak.  swap-out / swap-in: the
    same blocks to / from a pinned host pool of 2048 blocks, rated by the bytes
    crossing the host link against its one-direction peak."""
    import paged_kv_attention_decode_amd as pa

    spec = wl.CONFIGS[args.config]
    p = wl.make_problem(spec)
    kc, vc = to_dev(p.k_cache, torch), to_dev(p.v_cache, torch)
    n = min(2048, p.num_blocks // 2)
    ids = np.random.default_rng(spec.seed).permutation(p.num_blocks)
    block_bytes = kc[0].numel() * kc.element_size()
    if args.op == "copy-blocks":
        pairs = np.stack([ids[:n], ids[n:2 * n]], axis=1)
        src, dst = (kc, vc), (kc, vc)
        moved, bound, peak = 2 * 2 * n * block_bytes, "hbm", HBM_PEAK_GBPS  # K and V, read and written
    else:
        hk = torch.empty((n,) + tuple(kc.shape[1:]), dtype=kc.dtype).pin_memory()
        hv = torch.empty_like(hk).pin_memory()
        host = np.random.default_rng(spec.seed + 1).permutation(n)
        if args.op == "swap-out":
            pairs = np.stack([ids[:n], host], axis=1)
            src, dst = (kc, vc), (hk, hv)
        else:
            pairs = np.stack([host, ids[:n]], axis=1)
            src, dst = (hk, hv), (kc, vc)
        moved, bound, peak = 2 * n * block_bytes, "pcie", PCIE_PEAK_GBPS  # K and V across the link
    mapping = torch.from_numpy(pairs.astype(np.int64)).cuda()
    settle_ms, settle_steps = settle(lambda: pa.copy_blocks(*src, *dst, mapping), args.settle_ms, torch)
    for _ in range(max(0, args.warmup)):
        pa.copy_blocks(*src, *dst, mapping)
    torch.cuda.synchronize()
    K = args.steps
    # K calls back to back: wall clock for the step, one event pair around all K for the launches
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for k in range(K):
        pa.copy_blocks(*src, *dst, mapping)
    e1.record()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K
    launch_ms = e0.elapsed_time(e1) / K
    achieved = moved / (launch_ms / 1e3) / 1e9
    if args.calibrate_copy:
        calibration_copies(torch)
    # HBM traffic from the committed counter summary (the copy within the pool only)
    traffic, traffic_bytes = load_traffic(args.op, launch_ms / 1e3, COPY_SOURCES) if args.op == "copy-blocks" else (None, None)
    what = "HBM GB/s (read + written)" if bound == "hbm" else "host-link GB/s"
    print(json.dumps({
        "metric": f"pa_copy_blocks {what} per call", "value": round(achieved, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "settle_ms": round(settle_ms, 1), "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": p.dtype, "data": "synthetic",
        "config": {"workload": args.config, "op": args.op, "blocks_copied": n, "block_bytes": block_bytes},
        "roofline": {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": round(traffic, 1) if isinstance(traffic, float) else None,
                     "kernel": "copy_blocks_kernel",
                     "algorithmic_bytes_per_launch": moved, "avg_launch_us": round(launch_ms * 1e3, 2),
                     **({"traffic_bytes_per_launch": traffic_bytes} if isinstance(traffic_bytes, (int, float))
                        else {"traffic_note": traffic_bytes} if traffic_bytes else {})},
    }), flush=True)
    return 0


COLD_ROUNDS = 9  # rounds of the cold-launch timing (each times args.cold launches)


def settle(step, ms: float, torch) -> tuple:
    """Run the step, untimed, until ms of wall clock have passed; returns the time spent.

    An idle MI355X starts a burst of work at lower clocks and takes tens of
    milliseconds to reach its steady ones: launches in the first ~30 ms of a
    process ran 6-12% slower.  The settle runs before the W warm-up steps so
    that the timed steps see the steady state, as a continuously busy server's
    GPU would, whatever W the caller picks.  Returns (milliseconds, steps run)."""
    t0 = time.perf_counter()
    steps = 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            step()
        steps += 8
        torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3, steps


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="before the warm-up steps, run the step untimed for this long so the GPU leaves its "
                         "idle clocks (0 skips it)")
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=list(wl.CONFIGS))
    ap.add_argument("--partition", type=int, default=None, help="override the context split (0 = one pass)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the cpu_baseline leg")
    ap.add_argument("--cold", type=int, default=8,
                    help="also time this many decode launches one by one, each after reading 512 MiB "
                         "(evicts L2 and MALL); 0 skips them")
    ap.add_argument("--op", default="decode", choices=["decode", "copy-blocks", "swap-out", "swap-in"],
                    help="decode: the whole path (default); copy-blocks: pa_copy_blocks of 2048 blocks within "
                         "the pool; swap-out / swap-in: the same 2048 blocks to / from pinned host memory")
    ap.add_argument("--separate-write", action="store_true",
                    help="store the new tokens with pa_cache_write before pa_decode instead of the fused "
                         "pa_decode_append")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (for scaling memory counters)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; every figure is for one MI355X",
                          "n_gpus_requested": args.gpus}))
        return 2

    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    torch.cuda.set_device(0)

    if args.op != "decode":
        return bench_copy_blocks(args, torch)

    spec = wl.CONFIGS[args.config]
    p = wl.make_problem(spec)
    partition = partition_for(p) if args.partition is None else args.partition
    r = Resident(p, partition, torch, args.separate_write)

    settle_ms, settle_steps = settle(r.step, args.settle_ms, torch)
    for _ in range(max(0, args.warmup)):
        r.step()
    torch.cuda.synchronize()

    # Timed regions.  (A) K whole steps with no timing event inside (an event
    # pair costs about 5 us of GPU time, which would be charged to every step):
    # their wall clock gives ms_per_step and value.  (B) K attention launches
    # back to back (pa_decode, and pa_reduce for a split context: the two make
    # the attention), one HIP-event pair on the launch stream around all K:
    # the average launch duration the roofline is rated on.  (C) the same
    # launches with an event pair around each, for their spread.
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        r.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(K):
        r.decode()
        r.reduce()
    e1.record()
    torch.cuda.synchronize()
    decode_ms = e0.elapsed_time(e1) / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for k in range(K):
        ev[k][0].record()
        r.decode()
        r.reduce()
        ev[k][1].record()
    torch.cuda.synchronize()
    launch_ms = np.array([a.elapsed_time(b) for a, b in ev])
    spread_us = {f"p{q}": round(float(np.percentile(launch_ms, q)) * 1e3, 2) for q in (10, 50, 90)}
    single_pair_us = round(float(np.mean(launch_ms)) * 1e3, 2)

    # breakdown of the other two calls, from a separate untimed pass of whole
    # steps (event-bracketed, so each figure includes one timing event's cost)
    nb = min(K, 20)
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nb)]
    for k in range(nb):
        bev[k][0].record()
        r.write()
        bev[k][1].record()
        r.decode()
        bev[k][2].record()
        r.reduce()
        bev[k][3].record()
    torch.cuda.synchronize()
    write_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in bev]))
    decode_only_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in bev]))
    reduce_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in bev])) if partition > 0 else 0.0

    # cold-cache decode launches: a 512 MiB read between launches (twice the 256 MB MALL and
    # the 8 x 4 MB of L2) evicts both.  A read,
    # not a write: the lines a write leaves dirty would be written back during the timed
    # launch (measured: +45-60 us on every workload), which times the flush, not the decode.
    # Timed by difference, so that no event pair sits around a single launch (a pair costs
    # about 5 us of GPU time, most of a fp8 launch's 8%): one event pair around N (read, launch)
    # pairs and one around N reads alone, nine rounds, the median of the differences / N.
    cold_ms = None
    if args.cold > 0:
        scratch = torch.ones(1 << 27, dtype=torch.float32, device="cuda")
        scratch.sum()
        torch.cuda.synchronize()

        def timed(with_launch: bool) -> float:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.cold):
                scratch.sum()
                if with_launch:
                    r.decode()
                    r.reduce()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b)

        diffs = []
        for _ in range(COLD_ROUNDS):
            reads = timed(False)
            diffs.append((timed(True) - reads) / args.cold)
        cold_ms = float(np.median(diffs))
        del scratch

    if args.calibrate_copy:
        calibration_copies(torch)

    out = r.out.float().cpu().numpy().astype(np.float64)
    finite = bool(np.isfinite(out).all())

    ab = wl.algorithmic_bytes(p)
    kv_bytes = ab["kv_unique"] + ab["q"]
    tokens = ab["tokens"]
    decode_s = decode_ms / 1e3
    if p.query_start is not None:  # chunked prefill: dense products, rated on the matrix cores
        flops = wl.attention_flops(p)
        achieved = flops / decode_s / 1e12
        traffic, traffic_bytes = load_traffic(args.config, decode_s, PREFILL_SOURCES)
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": round(traffic, 1) if isinstance(traffic, float) else None,
                "traffic_unit": "GB/s",
                "kernel": decode_kernel_name(p, partition),
                "algorithmic_flops_per_launch": flops,
                "algorithmic_bytes_per_launch": kv_bytes + ab["out"],
                "avg_launch_us": round(decode_ms * 1e3, 2), "launch_us_percentiles": spread_us,
                "avg_launch_us_event_pair_each": single_pair_us}
    else:
        # rated over warm launches (the timed region), or over cold ones where the
        # MALL could serve a large part of the working set between warm launches.
        # The kernels load V non-temporally, so what can stay cached is K: half
        # the KV bytes.
        cold_basis = kv_bytes / 2 < 2 * MALL_BYTES and cold_ms is not None
        basis_s = cold_ms / 1e3 if cold_basis else decode_s
        achieved = kv_bytes / basis_s / 1e9
        traffic, traffic_bytes = load_traffic(args.config, basis_s)
        kernel = decode_kernel_name(p, partition)
        if r.fused:
            kernel += ", storing the new tokens first (pa_decode_append)"
        if partition > 0:
            kernel += " + reduce_kernel (pa_reduce)"
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": round(traffic, 1) if isinstance(traffic, float) else None,
                "kernel": kernel,
                "timing": ("cold launches (each after a 512 MiB read; the K bytes are under twice the "
                           "256 MB MALL, which serves part of them between warm launches): one event pair around "
                           f"{args.cold} (read, launch) pairs minus one around {args.cold} reads") if cold_basis
                else f"warm launches: {K} back to back, one event pair around them",
                "algorithmic_bytes_per_launch": kv_bytes,
                "avg_launch_us": round(basis_s * 1e6, 2)}
        if ab["kv_logical"] != ab["kv_unique"]:
            # shared prefix blocks: the headline counts them once; every sequence's
            # context read in full, as the kernel streams it, is reported beside it
            logical = (ab["kv_logical"] + ab["q"]) / basis_s / 1e9
            roof["achieved_logical"] = round(logical, 1)
            roof["frac_logical"] = round(logical / HBM_PEAK_GBPS, 4)
            roof["logical_bytes_per_launch"] = ab["kv_logical"] + ab["q"]
        if not cold_basis:
            roof["launch_us_percentiles"] = spread_us
            roof["avg_launch_us_event_pair_each"] = single_pair_us
        other_ms = decode_ms if cold_basis else cold_ms
        if other_ms is not None:
            other = kv_bytes / (other_ms / 1e3) / 1e9
            res_other = {"achieved": round(other, 1), "frac": round(other / HBM_PEAK_GBPS, 4),
                         "avg_launch_us": round(other_ms * 1e3, 2)}
            roof_other_key = "roofline_warm" if cold_basis else "roofline_cold"
        else:
            res_other, roof_other_key = None, None
    if isinstance(traffic_bytes, str):
        roof["traffic_note"] = traffic_bytes
    elif traffic_bytes is not None:
        roof["traffic_bytes_per_launch"] = traffic_bytes

    res = {
        "metric": METRIC if p.query_start is None else PREFILL_METRIC,
        "value": round(tokens / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "settle_ms": round(settle_ms, 1),
        "settle_steps": settle_steps,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": p.dtype,
        "data": "synthetic",
        "config": {
            "workload": args.config, "num_seqs": p.num_seqs, "num_q_heads": p.num_q_heads,
            "num_kv_heads": p.num_kv_heads, "head_dim": p.head_dim, "block_size": 16,
            "q_len": p.q_len if p.query_start is None else "per sequence",
            **({"new_tokens_per_seq": [int(x) for x in p.q_counts]} if p.query_start is not None else {}),
            "context_tokens": int(p.context_lens.sum()), "num_blocks": p.num_blocks,
            "new_tokens_written": 0 if p.slot_mapping is None else int(len(p.slot_mapping)),
            "partition_size": partition, "seed": spec.seed,
            "kv_cache": "fp8 E4M3, per-head scales" if p.spec.kv == "fp8" else p.dtype,
            "mask": "tree (" + p.spec.tree + f", {p.q_len} nodes)" if p.parents is not None
            else ("causal" if int(p.q_counts.max()) > 1 else "none"),
        },
        "kv_hbm_gbps_step": round(kv_bytes / (ms_per_step / 1e3) / 1e9, 1),
        "breakdown_us": {"cache_write": "fused into the decode launch" if r.fused else round(write_ms * 1e3, 2),
                         "decode": round(decode_only_ms * 1e3, 2),
                         "reduce": round(reduce_ms * 1e3, 2),
                         "decode_plus_reduce_timed": round(decode_ms * 1e3, 2),
                         "decode_plus_reduce_cold": None if cold_ms is None else round(cold_ms * 1e3, 2),
                         "cold_launches": args.cold * COLD_ROUNDS if args.cold > 0 else 0},
        "roofline": roof,
        "outputs_finite": finite,
    }
    if p.query_start is None and roof_other_key is not None:
        res[roof_other_key] = res_other
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(p, out)
    print(json.dumps(res), flush=True)
    return 0 if finite else 1


if __name__ == "__main__":
    sys.exit(main())
