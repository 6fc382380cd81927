"""Prefill parity: the HIP path through the C ABI against the float64 checker
on the same seeded inputs, element by element."""

import json
import os

import numpy as np
import pytest

from tests.gpu_util import (check_lse, check_out, device, gpu_prefill, log,
                            oracle_prefill, to_dev)
import tiled_attention_03_amd as ta
from tiled_attention_03_amd import inputs

pytestmark = pytest.mark.gpu

CAUSAL, FULL, CROSS = inputs.CAUSAL, inputs.FULL, inputs.CROSS


def _run_both(w, q, k, v, rows=None, with_lse=True):
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              mode=w.mode, kv_len=w.kv_len, start_pos=w.start_pos, scale=w.scale)
    got_o, got_l = gpu_prefill(q, k, v, with_lse=with_lse, **kw)
    ref_o, ref_l = oracle_prefill(q, k, v, rows=rows, **kw)
    if rows is not None:
        got_o = got_o[rows]
        got_l = got_l[rows] if got_l is not None else None
    return got_o, got_l, ref_o, ref_l


@pytest.mark.parametrize("rows", ["auto", "16", "32"])
@pytest.mark.parametrize("w", [inputs.CAUSAL_SMALL, inputs.FULL_1K, inputs.CROSS_512x2K,
                               inputs.CONTINUE_512], ids=lambda w: w.name)
def test_pages_workloads_full_parity(w, rows, kernel_override):
    if rows != "auto":
        kernel_override(ta.OVERRIDE_PREFILL_ROWS, int(rows))
    log(f"prefill parity {w.name} rows={rows}")
    q, k, v = inputs.make_prefill(w)
    go, gl, ro, rl = _run_both(w, q, k, v)
    e_o = check_out(go, ro, w.name)
    e_l = check_lse(gl, rl, w.name)
    log(f"  max|dout|={e_o:.2e} max|dlse|={e_l:.2e}")


@pytest.mark.timeout(900)
def test_long_causal_every_row():
    """The 16384-row causal workload with heavy K rows, in the launch the
    benchmark times: every row and head of out and lse against the checker,
    compared in chunks of 1024 rows."""
    w = inputs.CAUSAL_16K
    log(f"prefill parity (every row) {w.name}")
    q, k, v = inputs.make_prefill(w)
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              mode=w.mode, kv_len=w.kv_len, start_pos=w.start_pos, scale=w.scale)
    go, gl = gpu_prefill(q, k, v, **kw)
    e_o = e_l = 0.0
    for r0 in range(0, w.q_seq, 1024):
        rows = np.arange(r0, min(r0 + 1024, w.q_seq))
        ro, rl = oracle_prefill(q, k, v, rows=rows, **kw)
        e_o = max(e_o, check_out(go[rows], ro, f"{w.name} rows {r0}+"))
        e_l = max(e_l, check_lse(gl[rows], rl, f"{w.name} rows {r0}+"))
        log(f"  rows [{r0}, {rows[-1] + 1}) max|dout|={e_o:.2e} max|dlse|={e_l:.2e}")


def test_long_causal_sampled_rows_16row_kernel(kernel_override):
    """The same workload forced through the 16-row kernel: sampled rows."""
    kernel_override(ta.OVERRIDE_PREFILL_ROWS, 16)
    w = inputs.CAUSAL_16K
    log(f"prefill parity (sampled rows, 16-row kernel) {w.name}")
    q, k, v = inputs.make_prefill(w)
    rng = np.random.default_rng(5099)
    rows = np.unique(np.concatenate([
        [0, 1, 2, 31, 32, 33, 127, 128, 4095, 8191, 8192, 16351, 16352, 16383],
        rng.choice(w.q_seq, 18, replace=False)]))
    go, gl, ro, rl = _run_both(w, q, k, v, rows=rows)
    e_o = check_out(go, ro, w.name)
    e_l = check_lse(gl, rl, w.name)
    log(f"  rows={len(rows)} max|dout|={e_o:.2e} max|dlse|={e_l:.2e}")


def test_golden_small_causal():
    """The stored checker values for the small causal GQA workload."""
    from tests.test_golden import load_golden
    doc, out_g, lse_g = load_golden()
    w = inputs.CAUSAL_SMALL
    q, k, v = inputs.make_prefill(w)
    go, gl = gpu_prefill(q, k, v, num_heads=w.num_heads, num_kv_heads=w.num_kv_heads,
                         head_dim=w.head_dim, mode=w.mode, kv_len=w.kv_len, scale=w.scale)
    check_out(go[doc["out_rows"]], out_g, "golden out")
    check_lse(gl, lse_g, "golden lse")


SWEEP = [
    # mode, q_seq, kv_len, H, Hkv, d, start_pos
    (CAUSAL, 1, 1, 1, 1, 64, 0),
    (CAUSAL, 5, 5, 2, 1, 64, 0),
    (CAUSAL, 33, 33, 4, 4, 64, 0),
    (CAUSAL, 70, 70, 8, 2, 128, 0),
    (CAUSAL, 129, 129, 6, 3, 128, 0),
    (CAUSAL, 31, 100, 4, 1, 128, 69),
    (CAUSAL, 65, 300, 8, 1, 64, 200),
    (CAUSAL, 40, 97, 16, 2, 128, 57),    # group 8: two head blocks per KV head
    (CAUSAL, 3, 1000, 4, 2, 128, 997),
    (FULL, 1, 1, 2, 2, 128, 0),
    (FULL, 47, 47, 4, 2, 64, 0),
    (FULL, 96, 96, 3, 1, 128, 0),
    (CROSS, 7, 1, 4, 2, 64, 0),
    (CROSS, 33, 31, 2, 2, 128, 0),
    (CROSS, 64, 257, 4, 4, 128, 0),
    (CROSS, 100, 45, 12, 4, 64, 0),
    # >= 32 key tiles over few row strips: four key splits per block (32-row kernel)
    (CAUSAL, 40, 1100, 4, 2, 64, 1060),
    (CROSS, 70, 1500, 8, 8, 64, 0),
]


@pytest.mark.parametrize("rows", ["auto", "16", "32"])
@pytest.mark.parametrize("case", SWEEP, ids=[f"m{c[0]}_q{c[1]}_kv{c[2]}_h{c[3]}x{c[4]}_d{c[5]}_sp{c[6]}"
                                             for c in SWEEP])
def test_ragged_sweep(case, rows, kernel_override):
    """Every shape through the launch's own choice and through each of the
    two prefill kernels (16-row and 32-row waves), forced by the library's
    kernel-choice override."""
    if rows != "auto":
        kernel_override(ta.OVERRIDE_PREFILL_ROWS, int(rows))
    mode, n, kv, H, Hkv, d, sp = case
    log(f"prefill sweep {case} rows={rows}")
    w, q, k, v = inputs.random_case(700 + SWEEP.index(case), mode, n, kv, H, Hkv, d,
                                    start_pos=sp)
    go, gl, ro, rl = _run_both(w, q, k, v)
    check_out(go, ro, str(case))
    check_lse(gl, rl, str(case))


def test_empty_query_batch_is_a_noop():
    import torch
    dev = device()
    q = torch.zeros((0, 256), device=dev)
    out = torch.full((4, 256), 7.0, device=dev)
    ta.attn_fwd(q, None, None, out, None, 0, 0, 4, 2, 64, CROSS, 0, 0.125)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_cross_over_zero_keys_writes_zeros_and_sentinel():
    import torch
    dev = device()
    n, H, d = 37, 4, 64
    q = to_dev(inputs.normal((n, H * d), 42))
    out = torch.full((n, H * d), float("nan"), device=dev)
    lse = torch.full((n, H, 2), float("nan"), device=dev)
    ta.attn_fwd(q, None, None, out, lse, n, 0, H, 2, d, CROSS, 0, 0.125)
    torch.cuda.synchronize()
    assert torch.all(out == 0.0)
    assert torch.all(lse == -1e30)


def test_poisoned_cache_and_outputs():
    """Cache rows outside every window hold NaN and must not be read; out and
    lse start as NaN and must be fully overwritten."""
    import torch
    H, Hkv, d, n, sp, rows = 8, 2, 128, 77, 150, 400
    w, q, k, v = inputs.random_case(801, CAUSAL, n, sp + n, H, Hkv, d, start_pos=sp,
                                    kv_rows=rows)
    k[sp + n:] = np.nan
    v[sp + n:] = np.nan
    dev = device()
    out = torch.full((n, H * d), float("nan"), device=dev)
    lse = torch.full((n, H, 2), float("nan"), device=dev)
    ta.attn_fwd(to_dev(q), to_dev(k), to_dev(v), out, lse, n, sp + n, H, Hkv, d, CAUSAL, sp,
                w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle_prefill(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=CAUSAL,
                            kv_len=sp + n, start_pos=sp, scale=w.scale)
    check_out(out.cpu().numpy(), ro, "poison out")
    check_lse(lse.cpu().numpy(), rl, "poison lse")


def test_run_to_run_bitwise_deterministic():
    w = inputs.CONTINUE_512
    q, k, v = inputs.make_prefill(w)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              mode=w.mode, kv_len=w.kv_len, start_pos=w.start_pos, scale=w.scale,
              q_dev=qd, k_dev=kd, v_dev=vd)
    a = gpu_prefill(q, k, v, **kw)
    b = gpu_prefill(q, k, v, **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_continuation_matches_whole_pass_rows():
    """Rows [s, s+n) of a whole causal pass equal a pass starting at s (both
    on the GPU, within tolerance: different tilings of the same rows)."""
    H, Hkv, d, total, s = 8, 2, 128, 300, 173
    w, q, k, v = inputs.random_case(802, CAUSAL, total, total, H, Hkv, d)
    scale = w.scale
    a_o, a_l = gpu_prefill(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=CAUSAL,
                           kv_len=total, scale=scale)
    b_o, b_l = gpu_prefill(q[s:], k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d,
                           mode=CAUSAL, kv_len=total, start_pos=s, scale=scale)
    check_out(b_o, a_o[s:].astype(np.float64), "continuation")
    check_lse(b_l, a_l[s:].astype(np.float64), "continuation lse")


def test_graph_replay_matches_checker():
    """attn_fwd captured once in a HIP graph and replayed after the inputs
    change in place (eager work and synchronisation between replays): every
    replay matches the checker on that replay's inputs."""
    import torch
    w = inputs.FULL_1K
    dev = device()
    q0, k0, v0 = inputs.make_prefill(w)
    qd, kd, vd = to_dev(q0), to_dev(k0), to_dev(v0)
    out = torch.empty((w.q_seq, w.num_heads * w.head_dim), device=dev)
    lse = torch.empty((w.q_seq, w.num_heads, 2), device=dev)

    def call():
        ta.attn_fwd(qd, kd, vd, out, lse, w.q_seq, w.kv_len, w.num_heads, w.num_kv_heads,
                    w.head_dim, w.mode, 0, w.scale)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              mode=w.mode, kv_len=w.kv_len, scale=w.scale)
    for rep in range(3):
        q = inputs.normal(q0.shape, 6000 + rep)
        qd.copy_(torch.from_numpy(q).to(dev))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ro, rl = oracle_prefill(q, k0, v0, **kw)
        check_out(out.cpu().numpy(), ro, f"graph replay {rep}")
        check_lse(lse.cpu().numpy(), rl, f"graph replay lse {rep}")


def test_strided_fused_qkv_and_padded_out():
    """Q, K and V as column slices of one fused [n, (H+2Hkv)*d] buffer, out
    with padded rows: matches the checker on dense copies, and the padding
    columns are left untouched."""
    import torch
    H, Hkv, d, n, sp = 8, 2, 128, 300, 0
    dev = device()
    width = (H + 2 * Hkv) * d
    qkv = inputs.normal((n, width), 811)
    q = np.ascontiguousarray(qkv[:, :H * d])
    k = np.ascontiguousarray(qkv[:, H * d:(H + Hkv) * d])
    v = np.ascontiguousarray(qkv[:, (H + Hkv) * d:])
    qkv_d = to_dev(qkv)
    ostride = H * d + 64
    out = torch.full((n, ostride), float("nan"), device=dev)
    lse = torch.full((n, H, 2), float("nan"), device=dev)
    scale = d ** -0.5
    ta.attn_fwd_ex(qkv_d[:, :H * d], width, qkv_d[:, H * d:], width, qkv_d[:, (H + Hkv) * d:],
                   width, out, ostride, lse, 0, n, n, H, Hkv, d, CAUSAL, sp, scale)
    torch.cuda.synchronize()
    ro, rl = oracle_prefill(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=CAUSAL,
                            kv_len=n, scale=scale)
    got = out.cpu().numpy()
    check_out(got[:, :H * d], ro, "strided out")
    check_lse(lse.cpu().numpy(), rl, "strided lse")
    assert np.all(np.isnan(got[:, H * d:])), "padding columns were written"


def test_long_causal_fused_qkv_sampled_rows():
    """The 16384-row causal workload read from one fused [16384, 6144] QKV
    buffer with out written at a 4160-float row stride (the strided launch
    the benchmark times): sampled rows against the checker, and the whole
    output and lse bit for bit equal to the contiguous call (row strides
    change addresses only)."""
    import torch
    w = inputs.CAUSAL_16K
    log(f"prefill parity fused QKV (sampled rows) {w.name}")
    H, Hkv, d, n = w.num_heads, w.num_kv_heads, w.head_dim, w.q_seq
    qd_, kvd = H * d, Hkv * d
    q, k, v = inputs.make_prefill(w)
    dev = device()
    fused = torch.empty((n, qd_ + 2 * kvd), device=dev)
    for lo, x in ((0, q), (qd_, k), (qd_ + kvd, v)):
        fused[:, lo:lo + x.shape[1]].copy_(torch.from_numpy(x))
    out_wide = torch.full((n, qd_ + 64), float("nan"), device=dev)
    lse = torch.empty((n, H, 2), device=dev)
    width = qd_ + 2 * kvd
    ta.attn_fwd_ex(fused[:, :qd_], width, fused[:, qd_:qd_ + kvd], width,
                   fused[:, qd_ + kvd:], width, out_wide, qd_ + 64, lse, 0, n, n, H, Hkv, d,
                   CAUSAL, 0, w.scale)
    torch.cuda.synchronize()
    got_o = out_wide[:, :qd_].cpu().numpy()
    assert torch.isnan(out_wide[:, qd_:]).all().item(), "padding columns were written"
    got_l = lse.cpu().numpy()
    del fused, out_wide
    dense_o, dense_l = gpu_prefill(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d,
                                   mode=CAUSAL, kv_len=n, start_pos=0, scale=w.scale)
    assert np.array_equal(got_o, dense_o), "strided out differs from the contiguous call"
    assert np.array_equal(got_l, dense_l), "strided lse differs from the contiguous call"
    rng = np.random.default_rng(5098)
    rows = np.unique(np.concatenate([[0, 31, 32, 8191, 16383],
                                     rng.choice(n, 11, replace=False)]))
    ro, rl = oracle_prefill(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=CAUSAL,
                            kv_len=n, start_pos=0, scale=w.scale, rows=rows)
    e_o = check_out(got_o[rows], ro, "fused qkv 16K")
    e_l = check_lse(got_l[rows], rl, "fused qkv 16K")
    log(f"  rows={len(rows)} max|dout|={e_o:.2e} max|dlse|={e_l:.2e}")


@pytest.mark.parametrize("mode,sp", [(CAUSAL, 37), (CROSS, 0), (FULL, 0)])
def test_sub_batches_with_q_base(mode, sp):
    """Splitting the query batch into sub-batch calls with q_base (the
    prefill page's sub-batched dispatch) reproduces the whole batch."""
    import torch
    H, Hkv, d, n = 4, 2, 64, 170
    kv = n + sp if mode != CROSS else 211
    w, q, k, v = inputs.random_case(820 + mode, mode, n, kv, H, Hkv, d, start_pos=sp)
    dev = device()
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    out = torch.full((n, H * d), float("nan"), device=dev)
    lse = torch.full((n, H, 2), float("nan"), device=dev)
    for base, cnt in ((0, 61), (61, 64), (125, 45)):
        ta.attn_fwd_ex(qd, H * d, kd, Hkv * d, vd, Hkv * d, out, H * d, lse, base, cnt, kv, H, Hkv,
                       d, mode, sp, w.scale)
    torch.cuda.synchronize()
    ro, rl = oracle_prefill(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=mode,
                            kv_len=kv, start_pos=sp, scale=w.scale)
    check_out(out.cpu().numpy(), ro, f"sub-batches mode={mode}")
    check_lse(lse.cpu().numpy(), rl, f"sub-batches lse mode={mode}")


@pytest.mark.parametrize("rope", [False, True, "keys_once"],
                         ids=["plain", "rotary", "rotary_keys_once"])
@pytest.mark.parametrize("rows", ["auto", "16", "32"])
@pytest.mark.parametrize("stride", [(1 << 24) + 64, (1 << 25) + 64], ids=["2^24", "2^25"])
def test_row_strides_past_32bit_tile_offsets(stride, rows, rope, kernel_override):
    """Q, K and V rows 2^24 + 64 or 2^25 + 64 floats apart (column slices of
    one fused buffer of 40 such rows, 2.7 or 5.4 GB): the buffer-resource
    tile copies need 32-bit tile offsets, so these launches take the general
    copy path (and the 16-row kernel, which takes strides below 2^25, hands
    the wider one to the 32-row kernel). Rotary: keys turned as loaded, or
    turned once in place in the fused buffer (attn_rope_apply on the strided
    K columns) before attn_fwd_rope_q. Out and lse match the checker."""
    import torch
    import oracle
    H, Hkv, d, n, sp = 4, 2, 64, 35, 5
    kv = n + sp
    if rows != "auto":
        kernel_override(ta.OVERRIDE_PREFILL_ROWS, int(rows))
    width = (H + 2 * Hkv) * d
    qkv = inputs.normal((kv, width), 1300 + (stride >> 24))
    q = np.ascontiguousarray(qkv[sp:, :H * d])
    k = np.ascontiguousarray(qkv[:, H * d:(H + Hkv) * d])
    v = np.ascontiguousarray(qkv[:, (H + Hkv) * d:])
    dev = device()
    log(f"row stride {stride} floats, {kv} rows: {kv * stride * 4 / 1e9:.1f} GB")
    big = torch.empty((kv, stride), dtype=torch.float32, device=dev)
    big[:, :width] = torch.from_numpy(qkv).to(dev)
    out = torch.full((n, H * d), float("nan"), device=dev)
    lse = torch.full((n, H, 2), float("nan"), device=dev)
    scale = d ** -0.5
    qv, kvv, vv = big[sp:, :H * d], big[:, H * d:(H + Hkv) * d], big[:, (H + Hkv) * d:]
    table_ref = None
    if rope:
        table = torch.full((kv, d // 2, 2), float("nan"), dtype=torch.float32, device=dev)
        ta.attn_rope_table(table, kv, d, 10000.0)
        if rope == "keys_once":
            ta.attn_rope_apply(kvv, stride, kvv, stride, kv, Hkv, d, 0, table, kv)
            ta.attn_fwd_rope_q(qv, stride, kvv, stride, vv, stride, out, H * d, lse, 0, n, kv, H,
                               Hkv, d, CAUSAL, sp, scale, table, kv)
        else:
            ta.attn_fwd_rope(qv, stride, kvv, stride, vv, stride, out, H * d, lse, 0, n, kv, H,
                             Hkv, d, CAUSAL, sp, scale, table, kv)
        table_ref = oracle.rope_table(kv, d, 10000.0)
    else:
        ta.attn_fwd_ex(qv, stride, kvv, stride, vv, stride, out, H * d, lse, 0, n, kv, H, Hkv, d,
                       CAUSAL, sp, scale)
    torch.cuda.synchronize()
    del big
    ro, rl = oracle.attention_forward(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d,
                                      mode=CAUSAL, kv_len=kv, start_pos=sp, scale=scale,
                                      rope=table_ref)
    check_out(out.cpu().numpy(), ro, f"stride {stride} rows {rows} rope {rope}")
    check_lse(lse.cpu().numpy(), rl, f"stride {stride} rows {rows} rope {rope} lse")


def _profile_case(profile, seed, mode, n, kv, H, Hkv, d, sp):
    """Seeded inputs whose scores move a running max a lot: keys scaled up
    (ramp_up) or down (ramp_down) along the sequence by up to 12x, a few
    keys scaled 12x (spikes), or every score near -150 in log2 units
    (far_below: queries along one direction, keys opposite to it). The
    magnitudes stay where f32 dot products keep the scores within the lse
    tolerance (|s| below ~110 in natural units)."""
    w, q, k, v = inputs.random_case(seed, mode, n, kv, H, Hkv, d, start_pos=sp)
    rows = k.shape[0]
    ramp = (0.2 + 12.0 * np.arange(rows) / max(rows - 1, 1)).astype(np.float32)[:, None]
    if profile == "ramp_up":
        k = k * ramp
    elif profile == "ramp_down":
        k = k * ramp[::-1]
    elif profile == "spikes":
        idx = np.random.default_rng(seed).choice(rows, size=max(1, rows // 50), replace=False)
        k = k.copy()
        k[idx] *= np.float32(12.0)
    elif profile == "far_below":
        u = np.zeros(d, np.float32)
        u[:: 3] = 1.0
        u /= np.linalg.norm(u)
        qh = q.reshape(q.shape[0], H, d)
        kh = k.reshape(rows, Hkv, d)
        q = (29.0 * u + 0.05 * qh).reshape(q.shape).astype(np.float32)
        k = (-29.0 * u + 0.05 * kh).reshape(k.shape).astype(np.float32)
    return w, np.ascontiguousarray(q), np.ascontiguousarray(k, dtype=np.float32), v


@pytest.mark.parametrize("rows", ["auto", "16", "32"])
@pytest.mark.parametrize("case", [(CAUSAL, 300, 300, 4, 2, 64, 0), (CAUSAL, 70, 400, 8, 2, 128, 330),
                                  (CROSS, 70, 1500, 8, 8, 64, 0)],
                         ids=["causal", "continuation", "cross_splits"])
@pytest.mark.parametrize("profile", ["ramp_up", "ramp_down", "spikes", "far_below"])
def test_score_profiles_that_move_the_running_max(profile, case, rows, kernel_override):
    """Scores that climb by far more than 2^8 along the keys, fall, jump on a
    few keys, or sit near -150 (log2 units) for every key: the 32-row
    kernel's reference max moves many times, never, or from its first tile,
    and out and lse (the true max and log-sum) still match the checker; the
    cross case runs four key splits per block (their partial pairs are
    merged after each is restored)."""
    if rows != "auto":
        kernel_override(ta.OVERRIDE_PREFILL_ROWS, int(rows))
    mode, n, kv, H, Hkv, d, sp = case
    w, q, k, v = _profile_case(profile, 1400 + 7 * ["ramp_up", "ramp_down", "spikes",
                                                     "far_below"].index(profile),
                               mode, n, kv, H, Hkv, d, sp)
    go, gl, ro, rl = _run_both(w, q, k, v)
    what = f"{profile} {case} rows={rows}"
    log(f"{what}: lse max range {float(np.abs(rl[..., 0]).max()):.1f}")
    check_out(go, ro, what)
    check_lse(gl, rl, what)
