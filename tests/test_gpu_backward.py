"""Backward parity: attn_bwd through the C ABI (fed by the GPU forward's out
and lse) against the float64 checker's exact gradients on the same seeded
inputs, element by element. The bound is the forward's out tolerance plus
the rounding of a float32 sum of the gradient's terms (check_grad): dq sums
over a row's keys, dk and dv over the rows of every head of a group."""

import numpy as np
import pytest

import oracle
import tiled_attention_03_amd as ta
from tests.gpu_util import check_grad, check_out, device, log, to_dev
from tiled_attention_03_amd import inputs

pytestmark = pytest.mark.gpu

CAUSAL, FULL, CROSS = inputs.CAUSAL, inputs.FULL, inputs.CROSS


def windowed_bytes(n, kv_len, H, mode, start_pos, parts=3):
    """Workspace for the stored path in windows: the D_i scratch plus about
    1/parts of the call's dS tiles, and at least the tiles of its longest
    query tile (16 x 16 tiles of 1 KiB per head; query tile t of a causal call
    spans the keys of its last row's window)."""
    per_qt = []
    for t in range((n + 15) // 16):
        hi = min(16 * t + 16, n)
        w = min(start_pos + hi, kv_len) if mode == CAUSAL else kv_len
        per_qt.append((w + 15) // 16)
    cap = max(max(per_qt), -(-sum(per_qt) // parts))
    return ta.attn_bwd_workspace_bytes(n, H) + cap * H * 1024


def gpu_fwd_bwd(q, k, v, g, *, num_heads, num_kv_heads, head_dim, mode, kv_len, start_pos,
                scale, poison=True, stored=True, ws_short=0, ws_bytes=None):
    """GPU forward (out, lse), then attn_bwd; outputs and workspace pre-filled
    with NaN so that an element the kernels skip (or a tile they never write)
    shows. stored: workspace for the stored-dS path, else the minimal one;
    ws_short: bytes taken off the stored size; ws_bytes: this many bytes."""
    import torch
    dev = device()
    H, Hkv, d = num_heads, num_kv_heads, head_dim
    n = q.shape[0]
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    out, lse = ta.attention(qd, kd, vd, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=mode,
                            kv_len=kv_len, start_pos=start_pos, scale=scale)
    fill = float("nan") if poison else 0.0
    dq = torch.full((n, H * d), fill, device=dev)
    dk = torch.full((kv_len, Hkv * d), fill, device=dev)
    dv = torch.full((kv_len, Hkv * d), fill, device=dev)
    nbytes = ta.attn_bwd_workspace_bytes(n, H)
    if stored:
        nbytes = max(nbytes, ta.attn_bwd_workspace_bytes_stored(n, kv_len, H, mode, start_pos)
                     - ws_short)
    if ws_bytes is not None:
        nbytes = ws_bytes
    ws = torch.full((max(nbytes, 4) // 4,), fill, device=dev)
    ta.attn_bwd(qd, kd, vd, out, gd, lse, dq, dk, dv, n, kv_len, H, Hkv, d, mode, start_pos,
                scale, ws, nbytes)
    torch.cuda.synchronize()
    return dq.cpu().numpy(), dk.cpu().numpy(), dv.cpu().numpy()


def _kw(w):
    return dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
                mode=w.mode, kv_len=w.kv_len, start_pos=w.start_pos, scale=w.scale)


# Backward paths: "stored" (workspace for every dS tile, the stored path
# forced by the library's kernel-choice override even where its size rule
# would recompute; dq from the tiles), "windows" (the same with a workspace
# for about a third of the tiles: the stored path in windows of query tiles)
# and "recompute" (minimal workspace; dq recomputes the scores, 16-key dk/dv
# kernel).
PATHS = ["stored", "windows", "recompute"]


def _use_path(path, kernel_override):
    if path in ("stored", "windows"):
        kernel_override(ta.OVERRIDE_BWD_PATH, 1)
    return path != "recompute"


def _ws_for(path, w):
    return (windowed_bytes(w.q_seq, w.kv_len, w.num_heads, w.mode, w.start_pos)
            if path == "windows" else None)


def _check_all(got, ref, w, what):
    """ref: the checker's (dq, dk, dv, dq_m, dk_m, dv_m)."""
    terms = (w.kv_len, w.q_seq * w.group, w.q_seq * w.group)
    return [check_grad(a, b, m, n, f"{what} {name}")
            for name, a, b, m, n in zip(("dq", "dk", "dv"), got, ref[:3], ref[3:], terms)]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("w", [inputs.CAUSAL_SMALL, inputs.FULL_1K, inputs.CROSS_512x2K,
                               inputs.CONTINUE_512], ids=lambda w: w.name)
def test_backward_pages_workloads(w, path, kernel_override):
    """The pages' prefill workloads through each backward path."""
    stored = _use_path(path, kernel_override)
    log(f"backward parity {w.name} path={path}")
    q, k, v = inputs.make_prefill(w)
    g = inputs.normal(q.shape, w.seed_base + 7)
    got = gpu_fwd_bwd(q, k, v, g, stored=stored, ws_bytes=_ws_for(path, w), **_kw(w))
    ref = oracle.attention_backward(q, k, v, g, magnitudes=True, **_kw(w))
    e = _check_all(got, ref, w, w.name)
    log("  max|d| dq={:.2e} dk={:.2e} dv={:.2e}".format(*e))


_LONG_REF = {}


def _long_causal_reference(w, q, k, v, g):
    """The checker's gradients of the 16K workload on sampled rows and keys,
    every KV head (computed once, shared by the paths)."""
    if "ref" not in _LONG_REF:
        rng = np.random.default_rng(7099)
        rows = np.unique(np.concatenate([[0, 1, 15, 16, 31, 32, 8191, 16383],
                                         rng.choice(w.q_seq, 10, replace=False)]))
        heavy = inputs.heavy_rows(w.kv_len, w.heavy_frac, w.seed_base + 4)
        keys = np.unique(np.concatenate([[0, 1, 15, 16, 127, 128, 8192, 16352, 16383],
                                         heavy[:3], rng.choice(w.kv_len, 8, replace=False)]))
        log(f"  checker gradients: {len(rows)} rows, {len(keys)} keys, all KV heads")
        _LONG_REF["ref"] = (rows, keys, oracle.attention_backward(
            q, k, v, g, rows=rows, keys=keys, magnitudes=True, **_kw(w)))
    return _LONG_REF["ref"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", PATHS)
def test_backward_long_causal_sampled(path, kernel_override):
    """The 16384-row causal pass with heavy K rows: dq on sampled rows and
    dk, dv on sampled keys, every head and KV head. The stored path is the
    launch the benchmark times (17.2 GB of dS tiles)."""
    stored = _use_path(path, kernel_override)
    w = inputs.CAUSAL_16K
    log(f"backward parity (sampled) {w.name} path={path}")
    q, k, v = inputs.make_prefill(w)
    g = inputs.normal(q.shape, w.seed_base + 7)
    # windows: the benchmark's bounded workspace (2 GB, about 9 windows)
    ws = 2_000_000_000 if path == "windows" else None
    dq, dk, dv = gpu_fwd_bwd(q, k, v, g, stored=stored, ws_bytes=ws, **_kw(w))
    assert np.all(np.isfinite(dq)) and np.all(np.isfinite(dk)) and np.all(np.isfinite(dv))
    rows, keys, (rq, rk, rv, mq, mk, mv) = _long_causal_reference(w, q, k, v, g)
    n_rows = w.q_seq * w.group
    e_q = check_grad(dq[rows], rq, mq, w.kv_len, "dq sampled")
    e_k = check_grad(dk[keys], rk, mk, n_rows, "dk sampled")
    e_v = check_grad(dv[keys], rv, mv, n_rows, "dv sampled")
    log(f"  rows={len(rows)} keys={len(keys)} max|d| dq={e_q:.2e} dk={e_k:.2e} dv={e_v:.2e}")


@pytest.mark.timeout(600)
def test_backward_two_windows_four_tiles_per_wave():
    """An 8192-row causal pass, 32 heads (MHA), head_dim 64, with the
    smallest workspace that holds two interleaved windows: each window's dq
    grid (32 head blocks x 16 row blocks of four 16-row query tiles per
    wave) fills the compute units, so it takes four query tiles per wave, as
    the single launch does; dq on sampled rows, dk, dv on sampled keys, of 8
    of the 32 heads spread over the head blocks (the checker's cost)."""
    n, H, d = 8192, 32, 64
    w, q, k, v = inputs.random_case(1300, CAUSAL, n, n, H, H, d)
    g = inputs.normal(q.shape, 1301)
    per_qt = [-(-min(16 * t + 16, n) // 16) for t in range((n + 15) // 16)]  # causal
    cap = max(sum(per_qt[0::2]), sum(per_qt[1::2]))
    ws = ta.attn_bwd_workspace_bytes(n, H) + cap * H * 1024
    assert ta.attn_bwd_windows(n, n, H, CAUSAL, 0, ws) == 2
    log(f"backward two windows {n} rows H={H} d={d}, workspace {ws / 1e9:.2f} GB")
    dq, dk, dv = gpu_fwd_bwd(q, k, v, g, ws_bytes=ws, **_kw(w))
    rng = np.random.default_rng(1302)
    rows = np.unique(np.concatenate([[0, 15, 16, 17, 4095, 4096, n - 1],
                                     rng.choice(n, 8, replace=False)]))
    keys = np.unique(np.concatenate([[0, 1, 16, 4096, n - 17, n - 1],
                                     rng.choice(n, 8, replace=False)]))
    heads = [0, 5, 10, 15, 16, 21, 26, 31]  # MHA: KV head h is head h
    rq, rk, rv, mq, mk, mv = oracle.attention_backward(q, k, v, g, rows=rows, keys=keys,
                                                       kv_heads=heads, magnitudes=True, **_kw(w))
    c = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    e_q = check_grad(dq[rows][:, c], rq[:, c], mq[:, c], n, "dq sampled")
    e_k = check_grad(dk[keys][:, c], rk[:, c], mk[:, c], n, "dk sampled")
    e_v = check_grad(dv[keys][:, c], rv[:, c], mv[:, c], n, "dv sampled")
    log(f"  rows={len(rows)} keys={len(keys)} max|d| dq={e_q:.2e} dk={e_k:.2e} dv={e_v:.2e}")


@pytest.mark.timeout(600)
def test_backward_windows_mid_size_dq_grids():
    """An 8192-row causal pass, 32 / 8 heads, head_dim 128, in eleven
    interleaved windows: each window's dq grid (8 head blocks x 47 query
    tiles, one per wave) is between one and two blocks per compute unit,
    the range where the dq kernel splits each block's keys two ways; dq on
    sampled rows, dk, dv on sampled keys, of two of the eight KV heads (the
    checker's cost)."""
    n, H, Hkv, d = 8192, 32, 8, 128
    w, q, k, v = inputs.random_case(1310, CAUSAL, n, n, H, Hkv, d)
    g = inputs.normal(q.shape, 1311)
    ws = windowed_bytes(n, n, H, CAUSAL, 0, parts=10)
    assert ta.attn_bwd_windows(n, n, H, CAUSAL, 0, ws) == 11
    log(f"backward 11 windows {n} rows H={H}/{Hkv} d={d}, workspace {ws / 1e9:.2f} GB")
    dq, dk, dv = gpu_fwd_bwd(q, k, v, g, ws_bytes=ws, **_kw(w))
    rng = np.random.default_rng(1312)
    rows = np.unique(np.concatenate([[0, 15, 16, 175, 176, 4095, n - 1],
                                     rng.choice(n, 8, replace=False)]))
    keys = np.unique(np.concatenate([[0, 1, 16, 4096, n - 17, n - 1],
                                     rng.choice(n, 8, replace=False)]))
    kvh = [2, 7]
    rq, rk, rv, mq, mk, mv = oracle.attention_backward(q, k, v, g, rows=rows, keys=keys,
                                                       kv_heads=kvh, magnitudes=True, **_kw(w))
    cq = np.concatenate([np.arange(h * d, (h + 1) * d)
                         for c in kvh for h in range(c * (H // Hkv), (c + 1) * (H // Hkv))])
    ck = np.concatenate([np.arange(c * d, (c + 1) * d) for c in kvh])
    n_rows = n * (H // Hkv)
    e_q = check_grad(dq[rows][:, cq], rq[:, cq], mq[:, cq], n, "dq sampled")
    e_k = check_grad(dk[keys][:, ck], rk[:, ck], mk[:, ck], n_rows, "dk sampled")
    e_v = check_grad(dv[keys][:, ck], rv[:, ck], mv[:, ck], n_rows, "dv sampled")
    log(f"  rows={len(rows)} keys={len(keys)} max|d| dq={e_q:.2e} dk={e_k:.2e} dv={e_v:.2e}")


BWD_SWEEP = [
    # mode, q_seq, kv_len, H, Hkv, d, start_pos
    (CAUSAL, 1, 1, 1, 1, 64, 0),
    (CAUSAL, 5, 5, 2, 1, 64, 0),
    (CAUSAL, 70, 70, 8, 2, 128, 0),
    (CAUSAL, 129, 129, 6, 3, 128, 0),
    (CAUSAL, 31, 100, 4, 1, 128, 69),
    (CAUSAL, 65, 300, 8, 1, 64, 200),
    (CAUSAL, 3, 1000, 4, 2, 128, 997),
    (CAUSAL, 200, 330, 16, 2, 64, 130),
    (FULL, 47, 47, 4, 2, 64, 0),
    (FULL, 96, 96, 3, 1, 128, 0),
    (CROSS, 7, 1, 4, 2, 64, 0),
    (CROSS, 33, 31, 2, 2, 128, 0),
    (CROSS, 64, 257, 4, 4, 128, 0),
    (CROSS, 100, 45, 12, 4, 64, 0),
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("case", BWD_SWEEP, ids=lambda c: "m{}_q{}_kv{}_h{}x{}_d{}_sp{}".format(*c))
def test_backward_ragged_sweep(case, path, kernel_override):
    """Ragged shapes: partial query and key tiles, GQA groups of 1 to 8,
    continuation windows, single-key windows; through each backward path."""
    stored = _use_path(path, kernel_override)
    mode, n, kv, H, Hkv, d, sp = case
    w, q, k, v = inputs.random_case(1100 + n * 7 + kv, mode, n, kv, H, Hkv, d, start_pos=sp,
                                    kv_rows=kv + 5)
    k[kv:] = np.nan  # rows past kv_len must never be read into a result
    v[kv:] = np.nan
    g = inputs.normal(q.shape, 1101 + n)
    got = gpu_fwd_bwd(q, k, v, g, stored=stored, ws_bytes=_ws_for(path, w), **_kw(w))
    ref = oracle.attention_backward(q, k, v, g, magnitudes=True, **_kw(w))
    _check_all(got, ref, w, str(case))


def test_backward_workspace_short_of_stored_runs_windows(kernel_override):
    """A workspace one tile short of the stored size runs the stored path in
    windows (checked against the checker); one too small for the tiles of the
    longest query tile recomputes: same gradients as the minimal workspace,
    bit for bit."""
    kernel_override(ta.OVERRIDE_BWD_PATH, 1)
    w, q, k, v = inputs.random_case(1120, CAUSAL, 90, 120, 4, 2, 64, start_pos=30)
    g = inputs.normal(q.shape, 1121)
    a = gpu_fwd_bwd(q, k, v, g, stored=True, ws_short=1024, **_kw(w))
    ref = oracle.attention_backward(q, k, v, g, magnitudes=True, **_kw(w))
    _check_all(a, ref, w, "one tile short")
    base = ta.attn_bwd_workspace_bytes(w.q_seq, w.num_heads)
    longest = (min(w.start_pos + w.q_seq, w.kv_len) + 15) // 16  # tiles of the last query tile
    b = gpu_fwd_bwd(q, k, v, g, ws_bytes=base + (longest - 1) * w.num_heads * 1024, **_kw(w))
    c = gpu_fwd_bwd(q, k, v, g, stored=False, **_kw(w))
    for x, y in zip(b, c):
        assert np.array_equal(x, y)


def test_attention_backward_capped_workspace(kernel_override):
    """attention_backward with max_workspace_bytes runs attn_bwd with that
    scratch (here a third of the tiles, the stored path forced: it runs in
    windows): the gradients equal those of attn_bwd called with the same
    workspace, bit for bit, and match the checker."""
    import torch
    kernel_override(ta.OVERRIDE_BWD_PATH, 1)
    H, Hkv, d, n = 8, 2, 128, 300
    w, q, k, v = inputs.random_case(1320, CAUSAL, n, n, H, Hkv, d)
    g = inputs.normal(q.shape, 1321)
    ws = windowed_bytes(n, n, H, CAUSAL, 0)
    assert ta.attn_bwd_windows(n, n, H, CAUSAL, 0, ws) > 1
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    kw = dict(num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=CAUSAL, scale=w.scale)
    out, lse = ta.attention(qd, kd, vd, **kw)
    got = [x.cpu().numpy() for x in ta.attention_backward(qd, kd, vd, out, gd, lse,
                                                          max_workspace_bytes=ws, **kw)]
    torch.cuda.synchronize()
    want = gpu_fwd_bwd(q, k, v, g, ws_bytes=ws, **_kw(w))
    for a, b in zip(got, want):
        assert np.array_equal(a, b)
    ref = oracle.attention_backward(q, k, v, g, magnitudes=True, **_kw(w))
    _check_all(got, ref, w, "capped workspace")


def test_backward_single_key_windows():
    """CROSS over one key: dq = dk = 0 and dv is the sum of dout over rows and
    the group's heads."""
    H, Hkv, d, n = 8, 2, 128, 40
    w, q, k, v = inputs.random_case(1150, CROSS, n, 1, H, Hkv, d)
    g = inputs.normal(q.shape, 1151)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, g, **_kw(w))
    assert np.abs(dq).max() <= 1e-5 and np.abs(dk).max() <= 1e-5
    want = g.astype(np.float64).reshape(n, Hkv, H // Hkv, d).sum(axis=(0, 2)).reshape(1, -1)
    check_out(dv, want, "single key dv")


def test_backward_empty_query_batch_zeroes_key_gradients():
    import torch
    H, Hkv, d, kv = 4, 2, 64, 50
    dev = device()
    k = to_dev(inputs.normal((kv, Hkv * d), 1160))
    dk = torch.full((kv, Hkv * d), float("nan"), device=dev)
    dv = torch.full((kv, Hkv * d), float("nan"), device=dev)
    empty = torch.empty((0, H * d), device=dev)
    lse = torch.empty((0, H, 2), device=dev)
    ws = torch.empty((4,), device=dev)
    ta.attn_bwd(empty, k, k, empty, empty, lse, empty, dk, dv, 0, kv, H, Hkv, d, CROSS, 0,
                0.125, ws, 0)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


def test_backward_zero_keys():
    """CROSS with kv_len = 0: every window empty, dq = 0."""
    H, Hkv, d, n = 4, 2, 64, 9
    q = inputs.normal((n, H * d), 1170)
    k = np.zeros((1, Hkv * d), np.float32)
    g = inputs.normal((n, H * d), 1171)
    dq, dk, dv = gpu_fwd_bwd(q, k, k, g, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=CROSS,
                             kv_len=0, start_pos=0, scale=0.125)
    assert np.array_equal(dq, np.zeros_like(dq)) and dk.size == 0 and dv.size == 0


@pytest.mark.parametrize("path", PATHS)
def test_backward_deterministic(path, kernel_override):
    stored = _use_path(path, kernel_override)
    w, q, k, v = inputs.random_case(1180, CAUSAL, 300, 300, 8, 2, 128)
    g = inputs.normal(q.shape, 1181)
    a = gpu_fwd_bwd(q, k, v, g, stored=stored, ws_bytes=_ws_for(path, w), **_kw(w))
    b = gpu_fwd_bwd(q, k, v, g, stored=stored, ws_bytes=_ws_for(path, w), **_kw(w))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("path", PATHS)
def test_backward_graph_replay(path, kernel_override):
    """Forward and backward captured in one graph, replayed with the
    program's own work in between: every replay matches the eager result."""
    stored = _use_path(path, kernel_override)
    import torch
    H, Hkv, d, n = 8, 2, 64, 160
    w, q, k, v = inputs.random_case(1190, CAUSAL, n, n, H, Hkv, d)
    g = inputs.normal(q.shape, 1191)
    dev = device()
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    out = torch.empty((n, H * d), device=dev)
    lse = torch.empty((n, H, 2), device=dev)
    dq = torch.empty((n, H * d), device=dev)
    dk = torch.empty((n, Hkv * d), device=dev)
    dv = torch.empty((n, Hkv * d), device=dev)
    nbytes = (ta.attn_bwd_workspace_bytes_stored(n, n, H, CAUSAL, 0) if stored
              else ta.attn_bwd_workspace_bytes(n, H))
    if path == "windows":
        nbytes = windowed_bytes(n, n, H, CAUSAL, 0)
    ws = torch.empty((nbytes // 4,), device=dev)

    def step():
        ta.attn_fwd(qd, kd, vd, out, lse, n, n, H, Hkv, d, CAUSAL, 0, w.scale)
        ta.attn_bwd(qd, kd, vd, out, gd, lse, dq, dk, dv, n, n, H, Hkv, d, CAUSAL, 0, w.scale,
                    ws, nbytes)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [x.clone() for x in (dq, dk, dv)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        for x in (dq, dk, dv):
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for x, y in zip((dq, dk, dv), eager):
            assert torch.equal(x, y), f"replay {rep} differs"


@pytest.mark.parametrize("w", [inputs.FULL_1K, inputs.CAUSAL_16K], ids=lambda w: w.name)
def test_backward_path_choice_by_size(w, kernel_override):
    """Without an override the library picks the path by size, given the
    stored workspace: full 1024^2 (32 dq blocks from the tiles) recomputes,
    bitwise equal to the minimal workspace; the 16K causal pass takes the
    stored path, bitwise equal to forcing it."""
    q, k, v = inputs.make_prefill(w)
    g = inputs.normal(q.shape, w.seed_base + 7)
    auto = gpu_fwd_bwd(q, k, v, g, stored=True, **_kw(w))
    if w is inputs.FULL_1K:
        other = gpu_fwd_bwd(q, k, v, g, stored=False, **_kw(w))
    else:
        kernel_override(ta.OVERRIDE_BWD_PATH, 1)
        other = gpu_fwd_bwd(q, k, v, g, stored=True, **_kw(w))
    for x, y in zip(auto, other):
        assert np.array_equal(x, y)


def test_backward_on_a_side_stream_that_is_not_current():
    """attention() and attention_backward() given stream=side while another
    stream is current: their outputs and scratch belong to side, so work
    allocated on the current stream meanwhile cannot take their memory; the
    results equal those of the calls on the current stream, bit for bit."""
    import torch
    H, Hkv, d, n = 8, 2, 128, 300
    w, q, k, v = inputs.random_case(1200, CAUSAL, n, n, H, Hkv, d)
    g = inputs.normal(q.shape, 1201)
    qd, kd, vd, gd = to_dev(q), to_dev(k), to_dev(v), to_dev(g)
    kw = dict(num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=CAUSAL, scale=w.scale)
    out0, lse0 = ta.attention(qd, kd, vd, **kw)
    ref = ta.attention_backward(qd, kd, vd, out0, gd, lse0, **kw)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out1, lse1 = ta.attention(qd, kd, vd, stream=side, **kw)
    got = ta.attention_backward(qd, kd, vd, out1, gd, lse1, stream=side, **kw)
    # Allocations and writes on the current stream while side may still run.
    junk = [torch.full((1 << 22,), float("nan"), device=device()) for _ in range(8)]
    torch.cuda.synchronize()
    del junk
    assert torch.equal(out0, out1) and torch.equal(lse0, lse1)
    for x, y in zip(ref, got):
        assert torch.equal(x, y)
