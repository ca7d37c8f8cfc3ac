"""Helpers shared by the GPU tests and bench.py: move a workload to the GPU,
run the library's path on it, bring results back, and the parity gates."""

from __future__ import annotations

import numpy as np

import workloads as wl

# parity gates: the stated tolerances plus a relative-L2 gate on the whole output
TOL = {
    "f32": dict(atol=2e-3, rtol=0.0, rel_l2=1e-5),
    "bf16": dict(atol=2e-2, rtol=1e-2, rel_l2=5e-3),
}


# Every output row (one query token and head, head_dim values) on its own: relative L2
# against the oracle's row.  The whole-output gates above can hide one wrong row among
# thousands; a lost or doubled piece of a cut sequence, or one lost block of 16 tokens,
# moves its rows by 2e-2 to 1 in this measure, while bf16 rounding of the weights and of
# the output stays near 2e-3 (tests/test_gates.py shows both).  Rows whose reference is
# zero (nothing visible) are held to an absolute norm of the same size.
ROW_REL_L2 = 1e-2


def row_rel_l2(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def parity(got: np.ndarray, ref: np.ndarray, dtype: str, atol=None, rtol=None, rel_l2=None,
           rows: bool = False) -> dict:
    """The stated elementwise tolerance plus relative L2 over the whole output; with
    rows=True also ROW_REL_L2 on every row (last axis) for bf16 outputs."""
    t = dict(TOL[dtype])
    if atol is not None:
        t["atol"] = atol
    if rtol is not None:
        t["rtol"] = rtol
    if rel_l2 is not None:
        t["rel_l2"] = rel_l2
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    bound = t["atol"] + t["rtol"] * np.abs(ref)
    finite = bool(np.isfinite(got).all())
    excess = float(np.max(err - bound)) if err.size else 0.0
    denom = float(np.linalg.norm(ref))
    rl2 = float(np.linalg.norm(got - ref) / denom) if denom > 0 else float(np.linalg.norm(got))
    ok = finite and excess <= 0.0 and rl2 <= t["rel_l2"]
    r = dict(ok=ok, finite=finite, max_abs=float(err.max()) if err.size else 0.0, excess=excess, rel_l2=rl2, tol=t)
    if rows:
        worst = float(row_rel_l2(got, ref).max()) if err.size else 0.0
        r["row_rel_l2"] = worst
        r["ok"] = r["ok"] and worst <= ROW_REL_L2
    return r


class OracleJob:
    """The oracle's full output for a named workload, computed by tests/_oracle_full.py in a
    child process (its worker pool never shares state with the process driving the GPU)
    while the caller runs the GPU side; result() waits for it."""

    def __init__(self, name: str, workers: int = 0):
        import os
        import subprocess
        import sys
        import tempfile

        if workers <= 0:
            try:
                workers = min(16, len(os.sched_getaffinity(0)))
            except AttributeError:  # pragma: no cover
                workers = min(16, os.cpu_count() or 1)
        fd, self.path = tempfile.mkstemp(suffix=".npy")
        os.close(fd)
        here = os.path.dirname(os.path.abspath(__file__))
        self.proc = subprocess.Popen([sys.executable, os.path.join(here, "_oracle_full.py"), name, self.path,
                                      str(workers)])

    def result(self, timeout: float = 600.0) -> np.ndarray:
        import os

        try:
            rc = self.proc.wait(timeout=timeout)
            assert rc == 0, f"the oracle's child process failed ({rc})"
            return np.load(self.path)
        finally:
            if self.proc.poll() is None:
                self.proc.kill()
            os.unlink(self.path)


def to_dev(a: np.ndarray, dtype: str, device="cuda"):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def to_dev_pools(k: np.ndarray, v: np.ndarray, dtype: str, device="cuda"):
    """A layer's K and V pools in one allocation, placed by the library's layout query."""
    import paged_kv_attention_decode_amd as pa

    tk = to_dev(k, dtype, device)
    kc, vc = pa.allocate_kv_cache(k.shape[0], k.shape[2], k.shape[3], tk.dtype, device)
    kc.copy_(tk)
    del tk
    vc.copy_(to_dev(v, dtype, device))
    return kc, vc


def to_host(t) -> np.ndarray:
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    return (wl.bf16_bits_to_f32(a) if dtype == "bf16" else np.asarray(a, np.float32)).astype(np.float64)


class DeviceProblem:
    """A workload resident in HBM, ready for the path."""

    def __init__(self, p: wl.Problem, device="cuda"):
        import torch

        self.p = p
        dt = p.dtype
        self.q = to_dev(p.q, dt, device)
        self.k_cache, self.v_cache = to_dev_pools(p.k_cache, p.v_cache, dt, device)
        self.block_tables = torch.from_numpy(p.block_tables).to(device)
        self.context_lens = torch.from_numpy(p.context_lens).to(device)
        self.new_k = self.new_v = self.slots = None
        if p.new_k is not None:
            self.new_k = to_dev(p.new_k, dt, device)
            self.new_v = to_dev(p.new_v, dt, device)
            self.slots = torch.from_numpy(p.slot_mapping).to(device)
        self.fp8 = p.spec.kv == "fp8"
        if self.fp8:
            self.k_scale = torch.from_numpy(p.k_scale).to(device)
            self.v_scale = torch.from_numpy(p.v_scale).to(device)
        self.parents = None if p.parents is None else torch.from_numpy(p.parents).to(device)
        self.out = torch.empty_like(self.q)
        self.workspace = None

    def step(self, partition_size: int, write: bool = True):
        """One pass of the path: cache write of the new tokens, decode, reduce."""
        import paged_kv_attention_decode_amd as pa

        p = self.p
        if write and self.new_k is not None:
            if self.fp8:
                pa.cache_write_fp8(self.new_k, self.new_v, self.k_cache, self.v_cache, self.slots, self.k_scale,
                                   self.v_scale)
            else:
                pa.cache_write(self.new_k, self.new_v, self.k_cache, self.v_cache, self.slots)

        def dec(ps, out=None, workspace=None):
            if self.parents is not None:
                return pa.decode_tree(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens,
                                      self.parents, float(p.scale), ps, out=out, workspace=workspace)
            if self.fp8:
                return pa.decode_fp8(self.q, self.k_cache, self.v_cache, self.k_scale, self.v_scale, self.block_tables,
                                     self.context_lens, float(p.scale), p.q_len, ps, out=out, workspace=workspace)
            return pa.decode(self.q, self.k_cache, self.v_cache, self.block_tables, self.context_lens, float(p.scale),
                             p.q_len, ps, out=out, workspace=workspace)

        if partition_size <= 0:  # one pass or balanced
            if partition_size < 0 and self.workspace is None:
                self.workspace = pa.new_workspace(self.q, self.k_cache, self.block_tables, p.q_len, partition_size)
            dec(partition_size, out=self.out, workspace=self.workspace)
        else:
            self.workspace = dec(partition_size, workspace=self.workspace)
            pa.reduce(self.out, self.workspace, self.context_lens, p.q_len, p.max_blocks_per_seq, partition_size)
        return self.out


def host_caches_after_write(p: wl.Problem):
    """The caches as the oracle sees them after the new tokens are stored."""
    import oracle

    if p.new_k is None:
        return p.k_cache, p.v_cache
    if p.spec.kv == "fp8":
        return oracle.cache_write_fp8(p.k_cache, p.v_cache, p.new_k, p.new_v, p.slot_mapping, p.k_scale, p.v_scale,
                                      p.dtype)
    return oracle.cache_write(p.k_cache, p.v_cache, p.new_k, p.new_v, p.slot_mapping)


def reference_rows(p: wl.Problem, rows, kc=None, vc=None):
    """The oracle on the listed (b, j, h) rows over the caches after the write."""
    import oracle

    if kc is None:
        kc, vc = host_caches_after_write(p)
    if p.parents is not None:
        return oracle.paged_tree_decode_rows(p.q, kc, vc, p.block_tables, p.context_lens, p.parents, p.scale, p.dtype,
                                             rows)
    if p.spec.kv == "fp8":
        return oracle.paged_decode_fp8_rows(p.q, kc, vc, p.k_scale, p.v_scale, p.block_tables, p.context_lens,
                                            p.scale, p.q_len, p.dtype, rows)
    return oracle.paged_decode_rows(p.q, kc, vc, p.block_tables, p.context_lens, p.scale, p.q_len, p.dtype, rows)


def reference_full(p: wl.Problem):
    rows = [(b, j, h) for b in range(p.num_seqs) for j in range(p.q_len) for h in range(p.num_q_heads)]
    return reference_rows(p, rows).reshape(p.num_seqs * p.q_len, p.num_q_heads, p.head_dim)


def sample_rows(p: wl.Problem, n: int, seed: int = 0):
    """(b, j, h) rows to check one by one: the shortest and the longest sequence,
    then random ones; sorted by sequence so the oracle gathers each once."""
    rng = np.random.default_rng(seed)
    lens = p.context_lens
    bs = {int(np.argmin(lens)), int(np.argmax(lens))}
    while len(bs) < min(p.num_seqs, max(2, n // 4)):
        bs.add(int(rng.integers(0, p.num_seqs)))
    rows = set()
    for b in sorted(bs):
        rows.add((b, p.q_len - 1, 0))
        rows.add((b, 0, p.num_q_heads - 1))
    while len(rows) < n:
        b = sorted(bs)[int(rng.integers(0, len(bs)))]
        rows.add((b, int(rng.integers(0, p.q_len)), int(rng.integers(0, p.num_q_heads))))
    return sorted(rows)


def check_full_size_every_row(name: str, say=print) -> dict:
    """A full-size workload on the GPU in the schedule bench.py times and in the other
    schedules (one pass, 512-token partitions + pa_reduce, balanced), every output row
    against the oracle (parity with rows=True), and the cache write's rows bit for bit."""
    import bench

    job = OracleJob(name)  # the oracle runs beside the GPU work
    p = wl.make_problem(name)
    d = DeviceProblem(p)
    schedules = [bench.partition_for(p)] + [ps for ps in (0, 512, -1) if ps != bench.partition_for(p)]
    outs = {}
    for ps in schedules:
        say(f"{name}: partition {ps}")
        d.workspace = None  # a fresh workspace per schedule (a split one must not serve a balanced call)
        outs[ps] = widen(to_host(d.step(ps).clone()), p.dtype)
        assert np.isfinite(outs[ps]).all(), (name, ps)
    if p.new_k is not None:  # the cache write, on the rows it touched
        kc, _ = host_caches_after_write(p)
        flat = to_host(d.k_cache).reshape(-1, p.num_kv_heads, p.head_dim)
        want = kc.reshape(-1, p.num_kv_heads, p.head_dim)
        assert np.array_equal(flat[p.slot_mapping], want[p.slot_mapping]), name
    say(f"{name}: waiting for the oracle")
    ref = job.result()
    results = {}
    for ps in schedules:
        r = parity(outs[ps], ref, p.dtype, rows=True)
        say(f"{name}: partition {ps} against the oracle on every row: {r}")
        assert r["ok"], (name, ps, r)
        results[ps] = r
    return results
