"""Benchmark of the attention forward on one MI355X.

One step is one call of the prefill path on the long causal workload
(q_seq = kv_len = 16384, 32 query heads over 8 KV heads, head_dim 128, f32,
with the (max, log-sum) side output). The same JSON line also carries the
decode path measured on its cache workload (32/8 heads, head_dim 128, cache
8192 rows) with the KV cache rotated through 8 copies so the 256 MB
Infinity Cache cannot serve it. Reported beside them: the smaller prefill
workloads; the long causal workload read from a fused QKV buffer with row
strides, with the rotary embedding fused in, and through the backward pass;
and the decode over a paged cache (16- and 256-row pages).

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--only prefill|decode] [--no-cpu-baseline]
                    [--copy-calibration] [--mfma-valu-probe]

Timed region: barrier-free at one GPU; torch.cuda.synchronize() on both
sides, wall clock around exactly K steps. Kernel durations come from HIP
events recorded on the stream the kernels run on (torch's current stream).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from tiled_attention_03_amd import inputs  # noqa: E402

MFMA_F32_PEAK_TFLOPS = 157.3   # MI355X dense f32 matrix peak
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E peak
BOUNDED_BWD_BYTES = 2_000_000_000  # workspace of the bounded stored backward (2 GB)
METRIC = "prefill attention TFLOP/s and decode KV-read GB/s on 1 MI355X (% roofline)"
PREFILL_TRAFFIC = (os.path.join(ROOT, "profiles", "prefill_causal16k_traffic.md"),
                   os.path.join(ROOT, "tiled_attention_03_amd", "csrc", "prefill.hip"))
DECODE_TRAFFIC = (os.path.join(ROOT, "profiles", "decode_cache8192_traffic.md"),
                  os.path.join(ROOT, "tiled_attention_03_amd", "csrc", "decode.hip"))


# ------------------------------------------------------------ accounting

def window(w, i):
    if w.mode == inputs.CAUSAL:
        return min(w.start_pos + i + 1, w.kv_len)
    return w.kv_len


def unmasked_pairs(w, rows=None):
    rows = range(w.q_seq) if rows is None else rows
    return sum(window(w, int(i)) for i in rows)


def prefill_flops(w, rows=None, heads=None):
    """Q.K^T plus P.V over unmasked (row, key) pairs only."""
    heads = w.num_heads if heads is None else heads
    return 4 * w.head_dim * heads * unmasked_pairs(w, rows)


def decode_bytes(w, kv_pos, with_lse=False):
    """K and V rows [0, kv_len) of one KV layout (each read once, shared by
    the GQA group) plus Q in and out (and lse)."""
    kv_len = min(kv_pos + 1, w.max_seq)
    b = 2 * kv_len * w.num_kv_heads * w.head_dim * 4 + 2 * w.num_heads * w.head_dim * 4
    if with_lse:
        b += w.num_heads * 2 * 4
    return b


# ------------------------------------------------------------ clocks

class ClockSampler:
    """Samples the graphics clock the driver reports (the level marked
    current in pp_dpm_sclk) every `period` seconds while the block runs.
    Reading sysfs needs no privileges; without the file it reports None."""

    def __init__(self, period=0.02):
        import glob
        import threading
        paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = paths[0] if paths else None
        self.period = period
        self.samples = []
        self._threading = threading
        self._stop = None
        self._thread = None

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return int(re.search(r"(\d+)\s*[Mm]hz", line).group(1))
        except (OSError, AttributeError, ValueError):
            return None
        return None

    def _run(self):
        stop = self._stop
        while not stop.is_set():
            mhz = self._read()
            if mhz is not None:
                self.samples.append(mhz)
            stop.wait(self.period)

    def __enter__(self):
        if self.path is not None:
            self._stop = self._threading.Event()
            self._thread = self._threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None

    def summary(self):
        if not self.samples:
            return None
        return {"min": min(self.samples), "median": int(np.median(self.samples)),
                "max": max(self.samples), "samples": len(self.samples)}


# ------------------------------------------------------------ GPU timing

def time_calls(fn, n, torch, clock=None):
    """Average per-call duration (s) from events around each call, on the
    current stream, plus the wall time of the n calls. `clock` (a
    ClockSampler) samples the graphics clock over the timed calls only."""
    import contextlib
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    torch.cuda.synchronize()
    with clock if clock is not None else contextlib.nullcontext():
        t0 = time.perf_counter()
        for i in range(n):
            starts[i].record()
            fn(i)
            ends[i].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    durs = [s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends)]
    return float(np.mean(durs)), float(np.min(durs)), wall


def warm_replays(graph, torch, seconds=0.15):
    """Replay a captured graph back to back for about `seconds` of wall time
    before a short timed region, so that the GPU runs at its steady clock
    (a few milliseconds of timed work after an idle gap otherwise catch the
    clock still rising; the long prefill steps do not need this)."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(4):
            graph.replay()
        torch.cuda.synchronize()


def bench_prefill(w, steps, warmup, torch, ta, graph_replays=0, rope_theta=None,
                  fused_qkv=False, clock=None, rope_keys_once=False):
    """Prefill timing. With graph_replays > 0 the call is captured once in a
    HIP graph and replayed back to back (for kernels shorter than a Python
    launch); otherwise each call is launched eagerly between events. With
    rope_theta the rotary entry point runs (table built once, outside the
    timed calls; the rotation is not counted in the FLOPs). With fused_qkv,
    q, k and v are column slices of one [rows, (H + 2 Hkv) d] buffer and out
    is written into a buffer with 64 floats of padding per row
    (attn_fwd_ex with row strides). With rope_keys_once each timed call
    turns the keys once into a scratch copy (attn_rope_apply) and then runs
    attn_fwd_rope_q, which turns only the queries (both in the time)."""
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_prefill(w)
    qdim = w.num_heads * w.head_dim
    kvdim = w.num_kv_heads * w.head_dim
    if fused_qkv:
        assert w.q_seq == w.rows and w.start_pos == 0
        fused = torch.empty((w.q_seq, qdim + 2 * kvdim), device=dev)
        for lo, x in ((0, q), (qdim, k), (qdim + kvdim, v)):
            fused[:, lo:lo + x.shape[1]].copy_(torch.from_numpy(x))
        qd, kd, vd = fused[:, :qdim], fused[:, qdim:qdim + kvdim], fused[:, qdim + kvdim:]
        out_wide = torch.empty((w.q_seq, qdim + 64), device=dev)
        out = out_wide[:, :qdim]
    else:
        qd, kd, vd = (torch.from_numpy(x).to(dev) for x in (q, k, v))
        out = torch.empty((w.q_seq, qdim), device=dev)
    del q, k, v
    lse = torch.empty((w.q_seq, w.num_heads, 2), device=dev) if w.with_lse else None

    if fused_qkv:
        def call(_i):
            ta.attn_fwd_ex(qd, qd.stride(0), kd, kd.stride(0), vd, vd.stride(0), out,
                           out.stride(0), lse, 0, w.q_seq, w.kv_len, w.num_heads,
                           w.num_kv_heads, w.head_dim, w.mode, w.start_pos, w.scale)
    elif rope_theta is None:
        def call(_i):
            ta.attn_fwd(qd, kd, vd, out, lse, w.q_seq, w.kv_len, w.num_heads, w.num_kv_heads,
                        w.head_dim, w.mode, w.start_pos, w.scale)
    else:
        rows = max(w.start_pos + w.q_seq, w.kv_len)
        table = torch.empty((rows, w.head_dim // 2, 2), device=dev)
        ta.attn_rope_table(table, rows, w.head_dim, rope_theta)

        if rope_keys_once:
            k_rot = torch.empty_like(kd)

            def call(_i):
                ta.attn_rope_apply(kd, kvdim, k_rot, kvdim, w.kv_len, w.num_kv_heads,
                                   w.head_dim, 0, table, rows)
                ta.attn_fwd_rope_q(qd, qdim, k_rot, kvdim, vd, kvdim, out, qdim, lse, 0,
                                   w.q_seq, w.kv_len, w.num_heads, w.num_kv_heads, w.head_dim,
                                   w.mode, w.start_pos, w.scale, table, rows)
        else:
            def call(_i):
                ta.attn_fwd_rope(qd, qdim, kd, kvdim, vd, kvdim, out, qdim, lse, 0, w.q_seq,
                                 w.kv_len, w.num_heads, w.num_kv_heads, w.head_dim, w.mode,
                                 w.start_pos, w.scale, table, rows)

    flops = prefill_flops(w)
    if graph_replays > 0:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(warmup):
                call(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                call(i)
        warm_replays(graph, torch)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(graph_replays):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        mean_s = start.elapsed_time(end) * 1e-3 / (graph_replays * steps)
        return {"flops": flops, "mean_s": mean_s, "min_s": mean_s, "wall_s": None,
                "tflops_kernel": flops / mean_s / 1e12, "tflops_wall": None}
    for i in range(warmup):
        call(i)
    mean_s, min_s, wall = time_calls(call, steps, torch, clock)
    return {"flops": flops, "mean_s": mean_s, "min_s": min_s, "wall_s": wall,
            "tflops_kernel": flops / mean_s / 1e12, "tflops_wall": flops * steps / wall / 1e12}


def bench_backward(w, steps, warmup, torch, ta, stored=True, ws_bytes=None):
    """attn_bwd on the workload, fed by one forward pass; FLOPs are the
    algorithmic five products per unmasked pair (scores, dP, dV, dK, dQ):
    2.5x the forward's. stored: workspace for the stored-dS path (three
    launches); else the minimal one (dq recomputes scores and dP)."""
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_prefill(w)
    g = inputs.normal(q.shape, w.seed_base + 7)
    qd, kd, vd, gd = (torch.from_numpy(x).to(dev) for x in (q, k, v, g))
    del q, k, v, g
    H, Hkv, d = w.num_heads, w.num_kv_heads, w.head_dim
    out = torch.empty((w.q_seq, H * d), device=dev)
    lse = torch.empty((w.q_seq, H, 2), device=dev)
    ta.attn_fwd(qd, kd, vd, out, lse, w.q_seq, w.kv_len, H, Hkv, d, w.mode, w.start_pos, w.scale)
    dq = torch.empty_like(out)
    dk = torch.empty((w.kv_len, Hkv * d), device=dev)
    dv = torch.empty_like(dk)
    nbytes = (ta.attn_bwd_workspace_bytes_stored(w.q_seq, w.kv_len, H, w.mode, w.start_pos)
              if stored else ta.attn_bwd_workspace_bytes(w.q_seq, H))
    if ws_bytes is not None:
        nbytes = ws_bytes
    ws = torch.empty((nbytes // 4,), device=dev)

    def call(_i):
        ta.attn_bwd(qd, kd, vd, out, gd, lse, dq, dk, dv, w.q_seq, w.kv_len, H, Hkv, d, w.mode,
                    w.start_pos, w.scale, ws, nbytes)

    for i in range(warmup):
        call(i)
    mean_s, min_s, wall = time_calls(call, steps, torch)
    flops = 2.5 * prefill_flops(w)
    return {"flops": flops, "mean_s": mean_s, "min_s": min_s,
            "tflops_kernel": flops / mean_s / 1e12, "workspace_bytes": nbytes}


def bench_decode(w, kv_pos_values, replays, torch, ta, copies=8, page_size=None, clock=None):
    """Decode device time. The cache is rotated over `copies` independent
    allocations (copies x 64 MiB > the 256 MB Infinity Cache), and the
    `copies` calls are captured once in a HIP graph and replayed, so the
    GPU runs the calls back to back instead of waiting on Python launches.
    kv_pos lives in device memory: the same graph serves every kv_pos.
    With page_size, the cache is a pool of shuffled pages (64 unused pages
    mixed in) read through a page table (attn_decode_paged). `clock`
    samples the graphics clock over the timed replays only."""
    import contextlib
    dev = torch.device("cuda:0")
    q, k, v = inputs.make_decode(w)
    qd = torch.from_numpy(q).to(dev)
    if page_size is None:
        k0, v0 = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
        table, num_pages = None, 0
    else:
        kp, vp, tbl, num_pages = inputs.paged_pool(k, v, page_size, 64, w.seed_base + 9,
                                                   fill=0.0)
        k0, v0 = torch.from_numpy(kp).to(dev), torch.from_numpy(vp).to(dev)
        table = torch.from_numpy(tbl).to(dev)
        del kp, vp
    del k, v
    caches = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    out = torch.empty((1, w.num_heads * w.head_dim), device=dev)
    nbytes = ta.attn_decode_workspace_bytes(w.num_heads, w.num_kv_heads, w.head_dim,
                                            w.max_seq)
    ws = torch.zeros(max(nbytes // 4, 1), device=dev)  # zero-filled before first use
    pos = torch.zeros(1, dtype=torch.int32, device=dev)

    def call(i):
        kc, vc = caches[i % copies]
        if page_size is None:
            ta.attn_decode(qd, kc, vc, pos, out, None, w.num_heads, w.num_kv_heads,
                           w.head_dim, w.max_seq, w.scale, ws, nbytes)
        else:
            ta.attn_decode_paged(qd, kc, vc, num_pages, page_size, table, pos, out, None,
                                 w.num_heads, w.num_kv_heads, w.head_dim, w.max_seq, w.scale,
                                 ws, nbytes)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(copies):
            call(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(copies):
            call(i)
    res = {}
    for kv_pos in kv_pos_values:
        pos.fill_(kv_pos)
        warm_replays(graph, torch, 0.05)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        with clock if clock is not None else contextlib.nullcontext():
            start.record()
            for _ in range(replays):
                graph.replay()
            end.record()
            torch.cuda.synchronize()
        per_call = start.elapsed_time(end) * 1e-3 / (replays * copies)
        b = decode_bytes(w, kv_pos)
        res[str(kv_pos)] = {"us": round(per_call * 1e6, 2),
                            "GB/s": round(b / per_call / 1e9, 1),
                            "frac": round(b / per_call / 1e9 / HBM_PEAK_GBPS, 4)}
    return res


def bench_decode_read(w, kv_pos_values, replays, torch, copies=8, device_pos=False):
    """Read ceiling of the decode's access pattern, measured the way the
    decode is: the read-only probe kernel (libta03_probe.so: the decode's
    grid, 64-key units, per-lane load shapes and two register sets, no math,
    no merge) over the same 8 rotated caches, captured in one graph and
    replayed. Same algorithmic bytes as the decode. The cache length is
    passed from the host, or with device_pos read from device memory first,
    as the decode reads kv_pos."""
    import ctypes
    from tiled_attention_03_amd import binding
    binding.lib()  # torch's HIP runtime and libta03.so first
    probe = ctypes.CDLL(os.path.join(ROOT, "tiled_attention_03_amd", "libta03_probe.so"))
    P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    probe.ta03_probe_decode_read_sink_floats.argtypes = [I, I, I, I]
    probe.ta03_probe_decode_read_sink_floats.restype = S
    probe.ta03_probe_decode_read.argtypes = [P, P, P, I, I, I, I, I, I, P, S, P]
    probe.ta03_probe_decode_read.restype = I
    dev = torch.device("cuda:0")
    _, k, v = inputs.make_decode(w)
    k0, v0 = torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev)
    del k, v
    caches = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    nsink = probe.ta03_probe_decode_read_sink_floats(w.num_heads, w.num_kv_heads, w.head_dim,
                                                     w.max_seq)
    sink = torch.empty(max(int(nsink), 1), device=dev)
    res = {}
    pos = torch.zeros(1, dtype=torch.int32, device=dev)
    for kv_pos in kv_pos_values:
        kv_len = min(kv_pos + 1, w.max_seq)
        pos.fill_(kv_pos)

        def call(i):
            kc, vc = caches[i % copies]
            st = probe.ta03_probe_decode_read(
                kc.data_ptr(), vc.data_ptr(), pos.data_ptr() if device_pos else None, kv_len,
                w.num_heads, w.num_kv_heads, w.head_dim, w.max_seq, 0, sink.data_ptr(),
                int(nsink), torch.cuda.current_stream().cuda_stream)
            assert st == 0, f"read probe status {st}"

        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(copies):
                call(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(copies):
                call(i)
        warm_replays(graph, torch, 0.05)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for _ in range(replays):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        per_call = start.elapsed_time(end) * 1e-3 / (replays * copies)
        b = decode_bytes(w, kv_pos)
        res[str(kv_pos)] = {"us": round(per_call * 1e6, 2),
                            "GB/s": round(b / per_call / 1e9, 1)}
        del graph
    return res


def mfma_valu_probe(torch, iters=4000):
    """Issue-rate probe (libta03_probe.so): one block per compute unit, one or
    two waves per SIMD, f32 matrix instructions only, vector FMAs only, and
    both in one loop; cycles per iteration per SIMD from the launch time at
    2.4 GHz (the clock the 16K workload's busy-cycle counters show)."""
    import ctypes
    from tiled_attention_03_amd import binding
    binding.lib()
    probe = ctypes.CDLL(os.path.join(ROOT, "tiled_attention_03_amd", "libta03_probe.so"))
    probe.ta03_probe_mfma_valu.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    probe.ta03_probe_mfma_valu.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(cus * 512, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    res = {}
    for threads in (256, 512):
        for mode, name in ((1, "matrix"), (2, "vector"), (3, "both")):
            for _ in range(3):
                assert probe.ta03_probe_mfma_valu(out.data_ptr(), cus, threads, iters, mode, st) == 0
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            assert probe.ta03_probe_mfma_valu(out.data_ptr(), cus, threads, iters, mode, st) == 0
            e1.record()
            torch.cuda.synchronize()
            s = e0.elapsed_time(e1) * 1e-3
            res[f"{threads // 256}_waves_per_simd_{name}"] = {
                "ms": round(s * 1e3, 3), "cycles_per_iter_at_2.4GHz": round(s * 2.4e9 / iters)}
    res["work_per_iter_per_wave"] = {"matrix": "32 v_mfma_f32_16x16x4_f32 (32 cycles each at "
                                     "the f32 matrix peak)", "vector": "128 v_fma_f32"}
    print(json.dumps({"mfma_valu_probe": res}), flush=True)


def copy_calibration(torch, mib=1024, reps=3):
    """A plain device copy of known size, for scaling FETCH_SIZE/WRITE_SIZE."""
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    a = torch.randn(n, device=dev)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "reps": reps}), flush=True)


# ------------------------------------------------------------ CPU baseline

def cpu_baseline(w, wd, budget_s=10.0, block=256, max_blocks=8, decode_budget_s=2.0):
    """The float64 checker on the host cores, on the heaviest row blocks of
    the same workload (all heads), walked from the last row backwards until
    `budget_s` of CPU work or `max_blocks` blocks; beside it, the checker's
    decode at the largest kv_pos of the decode workload, repeated for about
    `decode_budget_s`."""
    import oracle
    blas = None
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in info]
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    q, k, v = inputs.make_prefill(w)
    total_s, flops, done = 0.0, 0, 0
    hi = w.q_seq
    while done < max_blocks and hi > 0 and total_s < budget_s:
        rows = np.arange(max(0, hi - block), hi)
        t0 = time.perf_counter()
        oracle.attention_forward(q, k, v, num_heads=w.num_heads, num_kv_heads=w.num_kv_heads,
                                 head_dim=w.head_dim, mode=w.mode, kv_len=w.kv_len,
                                 start_pos=w.start_pos, scale=w.scale, rows=rows)
        total_s += time.perf_counter() - t0
        flops += prefill_flops(w, rows)
        hi -= block
        done += 1
    del q, k, v
    qd, kd, vd = inputs.make_decode(wd)
    kv_pos = wd.kv_pos_values[-1]
    dec_s, calls = 0.0, 0
    while dec_s < decode_budget_s and calls < 100:
        t0 = time.perf_counter()
        oracle.decode_forward(qd, kd, vd, kv_pos=kv_pos, num_heads=wd.num_heads,
                              num_kv_heads=wd.num_kv_heads, head_dim=wd.head_dim,
                              max_seq=wd.max_seq, scale=wd.scale)
        dec_s += time.perf_counter() - t0
        calls += 1
    dec_bytes = decode_bytes(wd, kv_pos)
    return {"value": flops / total_s / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"rows [{hi}, {w.q_seq}) x {w.num_heads} heads of {w.name}, "
                      f"float64 numpy, {total_s:.1f} s, {flops / 1e9:.1f} GFLOP",
            "seconds": round(total_s, 3),
            "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas": blas,
            "decode": {"workload": wd.name, "kv_pos": kv_pos, "calls": calls,
                       "ms_per_call": round(dec_s / calls * 1e3, 3),
                       "GB/s": round(dec_bytes * calls / dec_s / 1e9, 3)}}


# ------------------------------------------------------------ traffic

def stored_traffic(files):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; otherwise None."""
    summary, src = files
    if not os.path.exists(summary):
        return None
    text = open(summary).read()
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_h = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    if not m_b or not m_h:
        return None
    cur = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return float(m_b.group(1)) if m_h.group(1) == cur else None


def copy_ceiling(torch, mib=64, copies=8, reps=48):
    """Measured context for the decode roofline: torch's device copy of a
    `mib` MiB buffer (the decode cache size) over `copies` rotated buffers,
    launched back to back; GB/s counts bytes read plus bytes written. Not part
    of the library path."""
    dev = torch.device("cuda:0")
    n = mib * (1 << 20) // 4
    src = [torch.ones(n, device=dev) for _ in range(copies)]
    dst = [torch.empty(n, device=dev) for _ in range(copies)]
    for i in range(copies):
        dst[i].copy_(src[i])
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(reps):
        dst[i % copies].copy_(src[i % copies])
    end.record()
    torch.cuda.synchronize()
    per = start.elapsed_time(end) * 1e-3 / reps
    return round(2 * n * 4 / per / 1e9, 1)


def backward_legs(w, torch, ta):
    """The backward on the 16K workload: stored-dS path with every tile, with
    a 2 GB workspace (windows), and the recompute path."""
    r = bench_backward(w, 3, 1, torch, ta)
    rb = bench_backward(w, 3, 1, torch, ta, ws_bytes=BOUNDED_BWD_BYTES)
    rr = bench_backward(w, 3, 1, torch, ta, stored=False)
    return {
        "workload": w.name, "ms": round(r["mean_s"] * 1e3, 3),
        "flops_per_call": r["flops"], "TFLOP/s": round(r["tflops_kernel"], 3),
        "frac": round(r["tflops_kernel"] / MFMA_F32_PEAK_TFLOPS, 4),
        "workspace_bytes": r["workspace_bytes"],
        "kernels": "bwd_delta_kernel<128> + bwd_dkdv16_kernel<128, 4, true> + "
                   "bwd_dq_ds_kernel<128, 4, 1>",
        "bounded": {"ms": round(rb["mean_s"] * 1e3, 3),
                    "TFLOP/s": round(rb["tflops_kernel"], 3),
                    "frac": round(rb["tflops_kernel"] / MFMA_F32_PEAK_TFLOPS, 4),
                    "workspace_bytes": rb["workspace_bytes"],
                    "kernels": "stored-dS path in windows of query tiles: "
                               "bwd_delta_kernel<128>, then per window "
                               "bwd_dkdv16_kernel<128, 4, true> + bwd_dq_ds_kernel<128, 1, 1>"},
        "recompute_path": {"ms": round(rr["mean_s"] * 1e3, 3),
                           "TFLOP/s": round(rr["tflops_kernel"], 3),
                           "frac": round(rr["tflops_kernel"] / MFMA_F32_PEAK_TFLOPS, 4),
                           "workspace_bytes": rr["workspace_bytes"],
                           "kernels": "bwd_dq_kernel<128> + "
                                      "bwd_dkdv16_kernel<128, 4, false>"}}


# ------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", choices=["prefill", "decode", "reported", "backward"], default=None,
                    help="one part of the line; 'reported' = the smaller prefill workloads only, "
                         "'backward' = the backward legs only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-reported", action="store_true",
                    help="skip the smaller prefill workloads")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--mfma-valu-probe", action="store_true",
                    help="only the matrix / vector-ALU issue-overlap probe")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); multi-GPU runs are not part of this build.",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import tiled_attention_03_amd as ta
    ta.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.mfma_valu_probe:
        mfma_valu_probe(torch)
        return

    w = inputs.CAUSAL_16K
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "f32", "data": "synthetic"}
    clocks = {}

    if args.only == "backward":
        result["backward"] = backward_legs(w, torch, ta)
        print(json.dumps(result), flush=True)
        return

    if args.only == "reported":
        rep = {}
        for wr in (inputs.FULL_1K, inputs.CROSS_512x2K, inputs.CONTINUE_512):
            r = bench_prefill(wr, 10, 3, torch, ta, graph_replays=10)
            rep[wr.name] = {"us": round(r["mean_s"] * 1e6, 2),
                            "TFLOP/s": round(r["tflops_kernel"], 3),
                            "frac": round(r["tflops_kernel"] / MFMA_F32_PEAK_TFLOPS, 4)}
        result["prefill_reported"] = rep
        print(json.dumps(result), flush=True)
        return

    if args.only != "decode":
        print(f"[bench] prefill {w.name}: {args.warmup} warmup + {args.steps} timed",
              flush=True)
        clk_prefill = ClockSampler()
        p = bench_prefill(w, args.steps, args.warmup, torch, ta, clock=clk_prefill)
        clocks["prefill"] = clk_prefill.summary()
        result.update({
            "value": round(p["tflops_wall"], 3), "unit": "TFLOP/s",
            "ms_per_step": round(p["wall_s"] / args.steps * 1e3, 3),
            "config": {"workload": w.name, "mode": "causal", "q_seq": w.q_seq,
                       "kv_len": w.kv_len, "num_heads": w.num_heads,
                       "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                       "lse": True, "heavy_k_rows": "1% x8",
                       "flops_per_step": p["flops"]},
            "roofline": {"bound": "mfma", "achieved": round(p["tflops_kernel"], 3),
                         "peak": MFMA_F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(p["tflops_kernel"] / MFMA_F32_PEAK_TFLOPS, 4),
                         "traffic": stored_traffic(PREFILL_TRAFFIC),
                         "kernel": "prefill_kernel<128, 0, 1>",
                         "kernel_ms_mean": round(p["mean_s"] * 1e3, 3),
                         "kernel_ms_min": round(p["min_s"] * 1e3, 3)},
        })
        print(f"[bench] prefill {p['tflops_kernel']:.2f} TFLOP/s "
              f"({p['mean_s'] * 1e3:.2f} ms/launch)", flush=True)
        if not args.no_reported:
            rep = {}
            for wr in (inputs.FULL_1K, inputs.CROSS_512x2K, inputs.CONTINUE_512):
                r = bench_prefill(wr, 10, 3, torch, ta, graph_replays=10)
                rep[wr.name] = {"us": round(r["mean_s"] * 1e6, 2),
                                "TFLOP/s": round(r["tflops_kernel"], 3),
                                "frac": round(r["tflops_kernel"] / MFMA_F32_PEAK_TFLOPS, 4)}
                print(f"[bench] {wr.name}: {rep[wr.name]}", flush=True)
            result["prefill_reported"] = rep
            r = bench_prefill(w, 3, 1, torch, ta, fused_qkv=True)
            result["prefill_strided"] = {
                "workload": w.name + "_fused_qkv",
                "layout": "q, k, v column slices of one [16384, 6144] buffer; out row stride 4160",
                "ms": round(r["mean_s"] * 1e3, 3), "TFLOP/s": round(r["tflops_kernel"], 3),
                "frac": round(r["tflops_kernel"] / MFMA_F32_PEAK_TFLOPS, 4),
                "kernel": "prefill_kernel<128, 0, 1>"}
            print(f"[bench] strided {result['prefill_strided']}", flush=True)
            r = bench_prefill(w, 3, 1, torch, ta, rope_theta=10000.0)
            result["prefill_rope"] = {
                "workload": w.name + "_rope_theta10000",
                "ms": round(r["mean_s"] * 1e3, 3), "TFLOP/s": round(r["tflops_kernel"], 3),
                "frac": round(r["tflops_kernel"] / MFMA_F32_PEAK_TFLOPS, 4),
                "kernel": "prefill_kernel<128, 1, 1> (keys turned as loaded)"}
            r = bench_prefill(w, 3, 1, torch, ta, rope_theta=10000.0, rope_keys_once=True)
            result["prefill_rope"]["keys_turned_once"] = {
                "ms": round(r["mean_s"] * 1e3, 3), "TFLOP/s": round(r["tflops_kernel"], 3),
                "frac": round(r["tflops_kernel"] / MFMA_F32_PEAK_TFLOPS, 4),
                "kernels": "rope_apply_kernel (keys, once per call) + prefill_kernel<128, 2, 1> "
                           "(queries turned as loaded), both timed"}
            print(f"[bench] rotary {result['prefill_rope']}", flush=True)
            result["backward"] = backward_legs(w, torch, ta)
            print(f"[bench] backward {result['backward']}", flush=True)

    if args.only != "prefill":
        wd = inputs.DECODE_8K
        print(f"[bench] decode {wd.name}", flush=True)
        clk_decode = ClockSampler(period=0.005)
        d = bench_decode(wd, wd.kv_pos_values, 25, torch, ta, clock=clk_decode)
        clocks["decode"] = clk_decode.summary()
        rd = bench_decode_read(wd, wd.kv_pos_values, 25, torch)
        rdp = bench_decode_read(wd, wd.kv_pos_values, 25, torch, device_pos=True)
        for key, r in rd.items():
            d[key]["read_probe_us"] = r["us"]
            d[key]["vs_read_probe"] = round(d[key]["us"] / r["us"], 3)
            d[key]["read_probe_device_pos_us"] = rdp[key]["us"]
        head = d[str(wd.kv_pos_values[-1])]
        head_read = rd[str(wd.kv_pos_values[-1])]
        result["decode"] = {
            "workload": wd.name, "unit": "GB/s", "kv_pos": d,
            "roofline": {"bound": "hbm", "achieved": head["GB/s"], "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": head["frac"],
                         "traffic": stored_traffic(DECODE_TRAFFIC),
                         "kernel": "decode_kernel<128>",
                         "kv_pos": wd.kv_pos_values[-1],
                         "read_ceiling_GBps": head_read["GB/s"],
                         "read_ceiling_us": head_read["us"],
                         "read_ceiling_kernel": "decode_read_kernel<128> (libta03_probe.so), "
                                                "cache length from the host",
                         "read_ceiling_device_pos_us": rdp[str(wd.kv_pos_values[-1])]["us"],
                         "vs_read_ceiling": round(head["us"] / head_read["us"], 3),
                         "measured_copy_GBps": copy_ceiling(torch)}}
        print(f"[bench] decode {d}", flush=True)
        if not args.no_reported:
            paged = {}
            for P in (16, 256):
                paged[str(P)] = bench_decode(wd, wd.kv_pos_values, 25, torch, ta, page_size=P)
                print(f"[bench] decode paged {P}: {paged[str(P)]}", flush=True)
            result["decode_paged"] = {"workload": wd.name + "_paged", "extra_pages": 64,
                                      "unit": "GB/s", "page_size": paged,
                                      "kernel": "decode_kernel<128>"}
        if args.only == "decode":
            result.update({"value": head["GB/s"], "unit": "GB/s",
                           "ms_per_step": head["us"] / 1e3,
                           "config": {"workload": wd.name,
                                      "kv_pos": wd.kv_pos_values[-1]}})

    if not args.no_cpu_baseline and args.only is None:
        print("[bench] cpu baseline (float64 checker on host cores)", flush=True)
        result["cpu_baseline"] = cpu_baseline(w, inputs.DECODE_8K)

    props = torch.cuda.get_device_properties(0)
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "sclk_mhz_seen": clocks}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
