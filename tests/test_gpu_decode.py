"""Decode parity: split-KV decode through the C ABI against the float64
checker, at the cache shapes of the pages' workload and on ragged caches."""

import numpy as np
import pytest

import oracle
from tests.gpu_util import check_lse, check_out, device, gpu_prefill, log, to_dev
from tiled_attention_03_amd import inputs

pytestmark = pytest.mark.gpu


def gpu_decode(q, k, v, kv_pos, *, num_heads, num_kv_heads, head_dim, max_seq, scale,
               with_lse=True, k_dev=None, v_dev=None, poison_outputs=True, ws=None):
    import torch
    import tiled_attention_03_amd as ta
    dev = device()
    kd = to_dev(k) if k_dev is None else k_dev
    vd = to_dev(v) if v_dev is None else v_dev
    fill = float("nan") if poison_outputs else 0.0
    out = torch.full((1, num_heads * head_dim), fill, device=dev)
    lse = torch.full((1, num_heads, 2), fill, device=dev) if with_lse else None
    pos = torch.tensor([kv_pos], dtype=torch.int32, device=dev)
    nbytes = ta.attn_decode_workspace_bytes(num_heads, num_kv_heads, head_dim, max_seq)
    if ws is None:
        # garbage everywhere, then the documented initialisation of the counters
        ws = torch.full((nbytes // 4,), float("nan"), device=dev)
        ta.attn_decode_workspace_init(ws, nbytes, num_heads, num_kv_heads, head_dim, max_seq)
    ta.attn_decode(to_dev(q), kd, vd, pos, out, lse, num_heads, num_kv_heads, head_dim,
                   max_seq, scale, ws, nbytes)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if lse is not None else None)


def ref_decode(q, k, v, kv_pos, *, num_heads, num_kv_heads, head_dim, max_seq, scale):
    return oracle.decode_forward(q, k, v, kv_pos=kv_pos, num_heads=num_heads,
                                 num_kv_heads=num_kv_heads, head_dim=head_dim,
                                 max_seq=max_seq, scale=scale)


@pytest.fixture(scope="module")
def decode_8k():
    w = inputs.DECODE_8K
    q, k, v = inputs.make_decode(w)
    return w, q, k, v, to_dev(k), to_dev(v)


@pytest.mark.parametrize("kv_pos", inputs.DECODE_8K.kv_pos_values)
def test_decode_pages_workload(decode_8k, kv_pos):
    w, q, k, v, kd, vd = decode_8k
    log(f"decode parity {w.name} kv_pos={kv_pos}")
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              max_seq=w.max_seq, scale=w.scale)
    go, gl = gpu_decode(q, k, v, kv_pos, k_dev=kd, v_dev=vd, **kw)
    ro, rl = ref_decode(q, k, v, kv_pos, **kw)
    e_o = check_out(go, ro, f"decode kv_pos={kv_pos}")
    e_l = check_lse(gl, rl, f"decode lse kv_pos={kv_pos}")
    log(f"  max|dout|={e_o:.2e} max|dlse|={e_l:.2e}")


def test_decode_position_past_cache_is_clamped(decode_8k):
    w, q, k, v, kd, vd = decode_8k
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              max_seq=w.max_seq, scale=w.scale)
    go, gl = gpu_decode(q, k, v, 20000, k_dev=kd, v_dev=vd, **kw)
    ro, rl = ref_decode(q, k, v, w.max_seq - 1, **kw)
    check_out(go, ro, "clamped")
    check_lse(gl, rl, "clamped lse")


DEC_SWEEP = [
    # H, Hkv, d, max_seq, kv_pos
    (1, 1, 64, 1, 0),
    (2, 1, 64, 70, 69),
    (4, 4, 128, 100, 37),
    (8, 2, 128, 513, 512),
    (12, 4, 64, 1000, 999),
    (16, 2, 128, 300, 64),      # group 8: two head blocks per KV head
    (32, 8, 128, 4096, 1),
    (6, 3, 128, 2049, 2000),
    (8, 8, 64, 9000, 8999),
    (32, 8, 128, 8192, 6000),   # 94 units over 32 splits: most blocks take 3
    (16, 4, 64, 700, 650),      # group 4 at head_dim 64: every matrix column a head
    (16, 2, 64, 333, 332),      # group 8 at head_dim 64: two head blocks per KV head
    (12, 2, 128, 500, 450),     # group 6: a second head block of 2 heads
    (10, 2, 64, 257, 256),      # group 5: a second head block of 1 head
]


@pytest.mark.parametrize("case", DEC_SWEEP, ids=[f"h{c[0]}x{c[1]}_d{c[2]}_max{c[3]}_pos{c[4]}"
                                                 for c in DEC_SWEEP])
def test_decode_ragged_sweep(case):
    H, Hkv, d, max_seq, pos = case
    log(f"decode sweep {case}")
    seed = 900 + DEC_SWEEP.index(case)
    q = inputs.normal((1, H * d), seed * 10 + 1)
    k = inputs.normal((max_seq, Hkv * d), seed * 10 + 2)
    v = inputs.normal((max_seq, Hkv * d), seed * 10 + 3)
    # rows past the window are poison: they must never be read
    k[pos + 1:] = np.nan
    v[pos + 1:] = np.nan
    kw = dict(num_heads=H, num_kv_heads=Hkv, head_dim=d, max_seq=max_seq, scale=d ** -0.5)
    go, gl = gpu_decode(q, k, v, pos, **kw)
    ro, rl = ref_decode(q, k, v, pos, **kw)
    check_out(go, ro, str(case))
    check_lse(gl, rl, str(case))


def test_decode_without_lse(decode_8k):
    w, q, k, v, kd, vd = decode_8k
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              max_seq=w.max_seq, scale=w.scale)
    go, gl = gpu_decode(q, k, v, 3000, k_dev=kd, v_dev=vd, with_lse=False, **kw)
    assert gl is None
    ro, _ = ref_decode(q, k, v, 3000, **kw)
    check_out(go, ro, "no lse")


def test_decode_equals_prefill_row(decode_8k):
    """attn_decode at kv_pos p equals attn_fwd(causal, one row, start_pos p)."""
    w, q, k, v, kd, vd = decode_8k
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim)
    for p in (0, 511, 5000):
        do, dl = gpu_decode(q, k, v, p, max_seq=w.max_seq, scale=w.scale, k_dev=kd,
                            v_dev=vd, **kw)
        po, pl = gpu_prefill(q, k, v, mode=inputs.CAUSAL, kv_len=p + 1, start_pos=p,
                             scale=w.scale, k_dev=kd, v_dev=vd, **kw)
        check_out(do, po.astype(np.float64), f"decode vs prefill p={p}")
        check_lse(dl, pl.astype(np.float64), f"decode vs prefill lse p={p}")


def test_decode_deterministic(decode_8k):
    w, q, k, v, kd, vd = decode_8k
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              max_seq=w.max_seq, scale=w.scale, k_dev=kd, v_dev=vd)
    a = gpu_decode(q, k, v, 8191, **kw)
    b = gpu_decode(q, k, v, 8191, **kw)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_workspace_reused_across_calls(decode_8k):
    """One workspace, many calls with changing kv_pos: the completion
    counters return to zero after every call and no stale partial of an
    earlier call leaks into a later one."""
    import torch
    import tiled_attention_03_amd as ta
    w, q, k, v, kd, vd = decode_8k
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              max_seq=w.max_seq, scale=w.scale)
    nbytes = ta.attn_decode_workspace_bytes(w.num_heads, w.num_kv_heads, w.head_dim, w.max_seq)
    ws = torch.full((nbytes // 4,), float("nan"), device=device())
    ta.attn_decode_workspace_init(ws, nbytes, w.num_heads, w.num_kv_heads, w.head_dim, w.max_seq)
    # the words the init zero-filled are the counter region (the rest stays NaN)
    counter_words = (ws == 0).cpu().numpy()
    assert counter_words.sum() >= w.num_kv_heads
    for p in (8191, 5, 700, 8191, 64, 63, 4096):
        go, gl = gpu_decode(q, k, v, p, k_dev=kd, v_dev=vd, ws=ws, **kw)
        ro, rl = ref_decode(q, k, v, p, **kw)
        check_out(go, ro, f"reuse p={p}")
        check_lse(gl, rl, f"reuse lse p={p}")
    counters = ws.view(torch.int32).cpu().numpy()[counter_words]
    assert np.all(counters == 0)


def test_graph_replay_follows_device_kv_pos(decode_8k):
    """A decode captured once in a HIP graph, replayed after the device-side
    kv_pos changes (with eager work and synchronisation between replays):
    every replay matches the checker."""
    import torch
    import tiled_attention_03_amd as ta
    w, q, k, v, kd, vd = decode_8k
    dev = device()
    nbytes = ta.attn_decode_workspace_bytes(w.num_heads, w.num_kv_heads, w.head_dim, w.max_seq)
    ws = torch.zeros(nbytes // 4, device=dev)
    qd = to_dev(q)
    out = torch.empty((1, w.num_heads * w.head_dim), device=dev)
    lse = torch.empty((1, w.num_heads, 2), device=dev)
    pos = torch.zeros(1, dtype=torch.int32, device=dev)

    def call():
        ta.attn_decode(qd, kd, vd, pos, out, lse, w.num_heads, w.num_kv_heads, w.head_dim,
                       w.max_seq, w.scale, ws, nbytes)

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
              max_seq=w.max_seq, scale=w.scale)
    for p in (100, 8191, 2047, 0, 5555):
        pos.fill_(p)
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        ro, rl = ref_decode(q, k, v, p, **kw)
        check_out(out.cpu().numpy(), ro, f"graph replay p={p}")
        check_lse(lse.cpu().numpy(), rl, f"graph replay lse p={p}")


@pytest.mark.parametrize("page_size", [16, 64, 256])
def test_paged_decode_matches_dense(decode_8k, page_size):
    """Paged cache with shuffled pages and unused NaN pages: matches the
    checker on the dense cache, and equals the dense decode bit for bit (same
    arithmetic, only row addresses differ)."""
    import torch
    import tiled_attention_03_amd as ta
    w, q, k, v, kd, vd = decode_8k
    dev = device()
    kp, vp, table, num_pages = inputs.paged_pool(k, v, page_size, 37, 870 + page_size)
    kpd, vpd, tbd = to_dev(kp), to_dev(vp), to_dev(table)
    nbytes = ta.attn_decode_workspace_bytes(w.num_heads, w.num_kv_heads, w.head_dim, w.max_seq)
    ws = torch.zeros(nbytes // 4, device=dev)
    qd = to_dev(q)
    kw = dict(num_heads=w.num_heads, num_kv_heads=w.num_kv_heads, head_dim=w.head_dim,
              max_seq=w.max_seq, scale=w.scale)
    for p in (0, 15, 16, 1000, 4095, 8191):
        out = torch.full((1, w.num_heads * w.head_dim), float("nan"), device=dev)
        lse = torch.full((1, w.num_heads, 2), float("nan"), device=dev)
        pos = torch.tensor([p], dtype=torch.int32, device=dev)
        ta.attn_decode_paged(qd, kpd, vpd, num_pages, page_size, tbd, pos, out, lse,
                             w.num_heads, w.num_kv_heads, w.head_dim, w.max_seq, w.scale, ws,
                             nbytes)
        torch.cuda.synchronize()
        ro, rl = ref_decode(q, k, v, p, **kw)
        go, gl = out.cpu().numpy(), lse.cpu().numpy()
        check_out(go, ro, f"paged P={page_size} p={p}")
        check_lse(gl, rl, f"paged lse P={page_size} p={p}")
        do, dl = gpu_decode(q, k, v, p, k_dev=kd, v_dev=vd, **kw)
        assert np.array_equal(go, do) and np.array_equal(gl, dl), f"paged != dense at p={p}"


def test_paged_decode_ragged_small():
    """A small cache whose last page is partly used, group 3, head_dim 64."""
    import torch
    import tiled_attention_03_amd as ta
    H, Hkv, d, max_seq, P = 6, 2, 64, 200, 32
    q = inputs.normal((1, H * d), 881)
    k = inputs.normal((max_seq, Hkv * d), 882)
    v = inputs.normal((max_seq, Hkv * d), 883)
    kp, vp, table, num_pages = inputs.paged_pool(k, v, P, 3, 884)
    dev = device()
    nbytes = ta.attn_decode_workspace_bytes(H, Hkv, d, max_seq)
    ws = torch.zeros(nbytes // 4, device=dev)
    for p in (0, 31, 32, 130, 199, 500):
        out = torch.empty((1, H * d), device=dev)
        lse = torch.empty((1, H, 2), device=dev)
        pos = torch.tensor([p], dtype=torch.int32, device=dev)
        ta.attn_decode_paged(to_dev(q), to_dev(kp), to_dev(vp), num_pages, P, to_dev(table), pos,
                             out, lse, H, Hkv, d, max_seq, d ** -0.5, ws, nbytes)
        torch.cuda.synchronize()
        ro, rl = ref_decode(q, k, v, p, num_heads=H, num_kv_heads=Hkv, head_dim=d,
                            max_seq=max_seq, scale=d ** -0.5)
        check_out(out.cpu().numpy(), ro, f"paged small p={p}")
        check_lse(lse.cpu().numpy(), rl, f"paged small lse p={p}")


def test_paged_decode_clamps_bad_table_entries():
    """Table entries outside [0, num_pages) are clamped on the device: the
    call completes with finite output (the value itself is meaningless)."""
    import torch
    import tiled_attention_03_amd as ta
    H, Hkv, d, max_seq, P, num_pages = 8, 2, 128, 256, 16, 16
    dev = device()
    q = to_dev(inputs.normal((1, H * d), 891))
    kp = to_dev(inputs.normal((num_pages, P, Hkv * d), 892))
    vp = to_dev(inputs.normal((num_pages, P, Hkv * d), 893))
    table = torch.tensor([-5, 3, 10 ** 6, 2 ** 31 - 1] * 4, dtype=torch.int32, device=dev)
    nbytes = ta.attn_decode_workspace_bytes(H, Hkv, d, max_seq)
    ws = torch.zeros(nbytes // 4, device=dev)
    out = torch.empty((1, H * d), device=dev)
    pos = torch.tensor([max_seq - 1], dtype=torch.int32, device=dev)
    ta.attn_decode_paged(q, kp, vp, num_pages, P, table, pos, out, None, H, Hkv, d, max_seq,
                         d ** -0.5, ws, nbytes)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out))
