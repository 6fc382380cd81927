"""Checks that pin the float64 checker (``oracle``) to facts that do not come
from the checker itself: closed forms, brute-force scalar loops, the page's
own sequential online-softmax update, torch's library attention, and
invariants of softmax attention.

Each ``pin_*`` takes the checker module as its argument and raises
AssertionError on a mismatch, so the same pins run against the real checker
(test_oracle.py) and against deliberately broken copies of it
(test_oracle_mutants.py).
"""

from __future__ import annotations

import math

import numpy as np

CAUSAL, FULL, CROSS = 0, 1, 2
SENT = -1e30


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _close(a, b, tol=1e-10, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _fwd(orc, q, k, v, H, Hkv, d, mode, kv_len, start_pos=0, scale=None, rows=None):
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return orc.attention_forward(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d,
                                 mode=mode, kv_len=kv_len, start_pos=start_pos,
                                 scale=scale, rows=rows)


# ---------------------------------------------------------------- closed forms

def pin_single_key_returns_that_v_row(orc):
    """A window of one key: the weight is 1, so out is that V row, the max is
    that key's score and log(sum) = log 1 = 0."""
    H, Hkv, d = 4, 2, 8
    q = _rand((3, H * d), 1)
    k = _rand((1, Hkv * d), 2)
    v = _rand((1, Hkv * d), 3)
    scale = 0.37
    out, lse = _fwd(orc, q, k, v, H, Hkv, d, CROSS, 1, scale=scale)
    for i in range(3):
        for h in range(H):
            kvh = h // (H // Hkv)
            _close(out[i, h * d:(h + 1) * d], v[0, kvh * d:(kvh + 1) * d], 1e-12, "out")
            s = scale * math.fsum(float(q[i, h * d + t]) * float(k[0, kvh * d + t])
                                  for t in range(d))
            _close(lse[i, h, 0], s, 1e-12, "max")
            _close(lse[i, h, 1], 0.0, 1e-12, "logsum")


def pin_identical_keys_give_mean_of_v(orc):
    """All keys equal: every weight is 1/w, out is the mean of V over the
    window, the max is the common score and log(sum) = log w."""
    H, Hkv, d, n = 2, 1, 4, 6
    q = _rand((n, H * d), 4)
    k = np.repeat(_rand((1, Hkv * d), 5), n, axis=0)
    v = _rand((n, Hkv * d), 6)
    out, lse = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, n)
    scale = 1.0 / math.sqrt(d)
    for i in range(n):
        w = i + 1
        for h in range(H):
            _close(out[i, h * d:(h + 1) * d], v[:w, :d].astype(np.float64).mean(axis=0),
                   1e-12, "mean")
            s = scale * math.fsum(float(q[i, h * d + t]) * float(k[0, t]) for t in range(d))
            _close(lse[i, h, 0], s, 1e-12, "max")
            _close(lse[i, h, 1], math.log(w), 1e-12, "log w")


def pin_zero_query_gives_mean(orc):
    """Q = 0: all scores are 0, max 0, log(sum) = log w, out = mean of V."""
    H, Hkv, d, n = 2, 2, 4, 5
    q = np.zeros((n, H * d), np.float32)
    k = _rand((n, Hkv * d), 7)
    v = _rand((n, Hkv * d), 8)
    out, lse = _fwd(orc, q, k, v, H, Hkv, d, FULL, n)
    for h in range(H):
        _close(out[:, h * d:(h + 1) * d],
               np.broadcast_to(v[:, h * d:(h + 1) * d].astype(np.float64).mean(0), (n, d)),
               1e-12, "mean")
    _close(lse[..., 0], np.zeros((n, H)), 0.0, "max")
    _close(lse[..., 1], np.full((n, H), math.log(n)), 1e-12, "log n")


def pin_causal_row0_returns_v0(orc):
    """Causal, start_pos 0: row 0 sees only key 0."""
    H, Hkv, d, n = 4, 2, 8, 7
    q, k, v = _rand((n, H * d), 9), _rand((n, Hkv * d), 10), _rand((n, Hkv * d), 11)
    out, lse = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, n)
    for h in range(H):
        kvh = h // 2
        _close(out[0, h * d:(h + 1) * d], v[0, kvh * d:(kvh + 1) * d], 1e-12, "row0")
        _close(lse[0, h, 1], 0.0, 1e-12, "row0 logsum")


def pin_two_keys_logistic(orc):
    """Two keys, d=1: weights are logistic functions of the score gap, and
    log(sum) = log(1 + exp(-|s0 - s1|))."""
    q = np.array([[1.5], [-0.5]], np.float32)
    k = np.array([[2.0], [-1.0]], np.float32)
    v = np.array([[3.0], [-7.0]], np.float32)
    scale = 0.75
    out, lse = _fwd(orc, q, k, v, 1, 1, 1, CROSS, 2, scale=scale)
    for i in range(2):
        s0 = scale * float(q[i, 0]) * 2.0
        s1 = scale * float(q[i, 0]) * -1.0
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        _close(out[i, 0], w0 * 3.0 + (1.0 - w0) * -7.0, 1e-12, "logistic out")
        _close(lse[i, 0, 0], max(s0, s1), 1e-12, "max")
        _close(lse[i, 0, 1], math.log1p(math.exp(-abs(s0 - s1))), 1e-12, "softplus")


def pin_zero_scale_is_uniform(orc):
    """scale = 0: uniform weights over each row's own window."""
    H, Hkv, d, n, sp = 2, 1, 4, 4, 3
    q = _rand((n, H * d), 12)
    k, v = _rand((sp + n, Hkv * d), 13), _rand((sp + n, Hkv * d), 14)
    out, lse = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, sp + n, start_pos=sp, scale=0.0)
    for i in range(n):
        w = sp + i + 1
        for h in range(H):
            _close(out[i, h * d:(h + 1) * d], v[:w].astype(np.float64).mean(0), 1e-12,
                   "uniform")
            _close(lse[i, h, 1], math.log(w), 1e-12, "log w")


def pin_empty_window_sentinel(orc):
    """Cross attention over zero keys: the shaders' safe sum gives out = 0, and
    the side output keeps the -1e30 start max and writes -1e30 for log(0)."""
    H, Hkv, d = 2, 1, 4
    q = _rand((3, H * d), 15)
    k = np.zeros((0, Hkv * d), np.float32)
    v = np.zeros((0, Hkv * d), np.float32)
    out, lse = _fwd(orc, q, k, v, H, Hkv, d, CROSS, 0)
    _close(out, np.zeros((3, H * d)), 0.0, "empty out")
    _close(lse, np.full((3, H, 2), SENT), 0.0, "empty lse")


# ------------------------------------------------------------- brute force

def _window(mode, i, q_seq, kv_len, start_pos):
    if mode == CAUSAL:
        return min(start_pos + i + 1, kv_len)
    return q_seq if mode == FULL else kv_len


def _brute(q, k, v, H, Hkv, d, mode, kv_len, start_pos, scale):
    """Scalar loops with math.fsum: the definition, one number at a time."""
    n = q.shape[0]
    g = H // Hkv
    out = [[0.0] * (H * d) for _ in range(n)]
    lse = [[[SENT, SENT] for _ in range(H)] for _ in range(n)]
    for i in range(n):
        w = _window(mode, i, n, kv_len, start_pos)
        for h in range(H):
            c = h // g
            if w == 0:
                continue
            s = [scale * math.fsum(float(q[i][h * d + t]) * float(k[j][c * d + t])
                                   for t in range(d)) for j in range(w)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            z = math.fsum(e)
            for t in range(d):
                out[i][h * d + t] = math.fsum(e[j] * float(v[j][c * d + t])
                                              for j in range(w)) / z
            lse[i][h] = [m, math.log(z)]
    return np.array(out), np.array(lse)


def pin_brute_force_tiny(orc):
    """Every mode, start_pos in {0, 2}, GQA groups 1/2/4, d up to 4."""
    seed = 100
    for mode in (CAUSAL, FULL, CROSS):
        for (H, Hkv) in ((1, 1), (2, 1), (4, 2), (4, 1)):
            for d in (1, 3, 4):
                for sp in ((0, 2) if mode == CAUSAL else (0,)):
                    n = 5
                    kv = n if mode == FULL else (sp + n if mode == CAUSAL else 7)
                    seed += 1
                    q = _rand((n, H * d), seed)
                    k = _rand((kv, Hkv * d), seed + 1000)
                    v = _rand((kv, Hkv * d), seed + 2000)
                    scale = 0.6
                    bo, bl = _brute(q, k, v, H, Hkv, d, mode, kv, sp, scale)
                    oo, ol = _fwd(orc, q, k, v, H, Hkv, d, mode, kv, sp, scale)
                    tag = f"mode={mode} H={H} Hkv={Hkv} d={d} sp={sp}"
                    _close(oo, bo, 1e-12, "brute out " + tag)
                    _close(ol, bl, 1e-12, "brute lse " + tag)


def pin_page_online_update(orc):
    """The pages' per-score online update (running max, running sum rescaled
    by exp(old max - new max), accumulator rescaled the same way), run
    sequentially in float64 with a -1e30 start max, reaches the checker's
    (out, max, log sum) for every row, including heavy-tailed scores."""
    H, Hkv, d, n, sp = 4, 2, 8, 6, 5
    q = _rand((n, H * d), 20)
    k = _rand((sp + n, Hkv * d), 21)
    k[[1, 7]] *= 8.0  # a few heavy keys force rescaling
    v = _rand((sp + n, Hkv * d), 22)
    scale = 1.0 / math.sqrt(d)
    out, lse = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, sp + n, sp, scale)
    for i in range(n):
        w = sp + i + 1
        for h in range(H):
            c = h // (H // Hkv)
            mx, sm = -1e30, 0.0
            acc = np.zeros(d)
            for t in range(w):
                s = scale * float(np.dot(q[i, h * d:(h + 1) * d].astype(np.float64),
                                         k[t, c * d:(c + 1) * d].astype(np.float64)))
                nm = max(mx, s)
                corr = math.exp(mx - nm)
                wt = math.exp(s - nm)
                sm = sm * corr + wt
                acc = acc * corr + wt * v[t, c * d:(c + 1) * d].astype(np.float64)
                mx = nm
            _close(out[i, h * d:(h + 1) * d], acc / sm, 1e-12, "online out")
            _close(lse[i, h, 0], mx, 1e-12, "online max")
            _close(lse[i, h, 1], math.log(sm), 1e-12, "online log sum")


# ---------------------------------------------------------- library routines

def pin_matches_torch_sdpa(orc):
    """torch's CPU scaled_dot_product_attention in float64 with GQA and an
    explicit boolean window mask (causal with start_pos, full, cross)."""
    import torch
    import torch.nn.functional as F
    cases = [(CAUSAL, 9, 9, 0), (CAUSAL, 7, 12, 5), (FULL, 10, 10, 0), (CROSS, 6, 13, 0)]
    for idx, (mode, n, kv, sp) in enumerate(cases):
        H, Hkv, d = 8, 2, 16
        q = _rand((n, H * d), 30 + idx)
        k = _rand((kv, Hkv * d), 40 + idx)
        v = _rand((kv, Hkv * d), 50 + idx)
        scale = 1.0 / math.sqrt(d)
        out, lse = _fwd(orc, q, k, v, H, Hkv, d, mode, kv, sp, scale)
        qt = torch.from_numpy(q.astype(np.float64)).view(n, H, d).transpose(0, 1)[None]
        kt = torch.from_numpy(k.astype(np.float64)).view(kv, Hkv, d).transpose(0, 1)[None]
        vt = torch.from_numpy(v.astype(np.float64)).view(kv, Hkv, d).transpose(0, 1)[None]
        mask = torch.zeros(n, kv, dtype=torch.bool)
        for i in range(n):
            mask[i, :_window(mode, i, n, kv, sp)] = True
        ref = F.scaled_dot_product_attention(qt.contiguous(), kt.contiguous(),
                                             vt.contiguous(), attn_mask=mask,
                                             scale=scale, enable_gqa=True)
        ref = ref[0].transpose(0, 1).reshape(n, H * d).numpy()
        _close(out, ref, 1e-12, f"sdpa mode={mode}")
        # m + log sum is the full log-sum-exp of the window's scores
        kr = torch.repeat_interleave(kt[0], H // Hkv, dim=0)
        s = scale * torch.matmul(qt[0], kr.transpose(1, 2).contiguous())
        s = s.masked_fill(~mask[None], float("-inf"))
        ref_lse = torch.logsumexp(s, dim=-1).transpose(0, 1).numpy()
        _close(lse[..., 0] + lse[..., 1], ref_lse, 1e-11, f"logsumexp mode={mode}")


def pin_logsumexp_scipy(orc):
    """m + log(sum) equals scipy's logsumexp over brute-force scores."""
    from scipy.special import logsumexp
    H, Hkv, d, n = 2, 2, 5, 4
    q, k = _rand((n, H * d), 60, 3.0), _rand((9, Hkv * d), 61, 3.0)
    v = _rand((9, Hkv * d), 62)
    _, lse = _fwd(orc, q, k, v, H, Hkv, d, CROSS, 9, scale=0.9)
    for i in range(n):
        for h in range(H):
            s = [0.9 * math.fsum(float(q[i, h * d + t]) * float(k[j, h * d + t])
                                 for t in range(d)) for j in range(9)]
            _close(lse[i, h, 0], max(s), 1e-12, "max")
            _close(lse[i, h, 0] + lse[i, h, 1], logsumexp(s), 1e-11, "lse")


# -------------------------------------------------------------- invariants

def pin_gqa_equals_repeated_heads(orc):
    """GQA with group g equals MHA on K/V whose heads are repeated g times."""
    H, Hkv, d, n = 8, 2, 4, 6
    q, k, v = _rand((n, H * d), 70), _rand((n, Hkv * d), 71), _rand((n, Hkv * d), 72)
    g = H // Hkv
    kr = np.repeat(k.reshape(n, Hkv, d), g, axis=1).reshape(n, H * d)
    vr = np.repeat(v.reshape(n, Hkv, d), g, axis=1).reshape(n, H * d)
    a = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, n)
    b = _fwd(orc, q, kr, vr, H, H, d, CAUSAL, n)
    _close(a[0], b[0], 1e-12, "gqa out")
    _close(a[1], b[1], 1e-12, "gqa lse")


def pin_linear_in_v(orc):
    """Weights sum to one: out(alpha*V + beta) = alpha*out(V) + beta."""
    H, Hkv, d, n = 2, 1, 4, 5
    q, k, v = _rand((n, H * d), 73), _rand((n, Hkv * d), 74), _rand((n, Hkv * d), 75)
    o1, _ = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, n)
    o2, _ = _fwd(orc, q, k, (2.5 * v.astype(np.float64) - 1.25), H, Hkv, d, CAUSAL, n)
    _close(o2, 2.5 * o1 - 1.25, 1e-12, "linearity")


def pin_kv_permutation_invariance(orc):
    """Full/cross attention is a set function of the (K, V) rows."""
    H, Hkv, d, n, kv = 2, 1, 4, 4, 8
    q, k, v = _rand((n, H * d), 76), _rand((kv, Hkv * d), 77), _rand((kv, Hkv * d), 78)
    perm = np.random.default_rng(79).permutation(kv)
    a = _fwd(orc, q, k, v, H, Hkv, d, CROSS, kv)
    b = _fwd(orc, q, k[perm], v[perm], H, Hkv, d, CROSS, kv)
    _close(a[0], b[0], 1e-12, "perm out")
    _close(a[1], b[1], 1e-12, "perm lse")


def pin_cache_continuation(orc):
    """Rows [s, s+n) of a whole causal pass equal a pass that starts at s."""
    H, Hkv, d, total, s = 4, 2, 4, 11, 6
    q, k, v = _rand((total, H * d), 80), _rand((total, Hkv * d), 81), _rand((total, Hkv * d), 82)
    a = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, total)
    b = _fwd(orc, q[s:], k, v, H, Hkv, d, CAUSAL, total, start_pos=s)
    _close(a[0][s:], b[0], 1e-12, "continuation out")
    _close(a[1][s:], b[1], 1e-12, "continuation lse")


def pin_decode_is_prefill_row(orc):
    """Decode at kv_pos p equals one causal row at start_pos p; the window is
    clamped to the cache length."""
    H, Hkv, d, max_seq = 4, 2, 8, 10
    q = _rand((1, H * d), 83)
    k, v = _rand((max_seq, Hkv * d), 84), _rand((max_seq, Hkv * d), 85)
    scale = 1.0 / math.sqrt(d)
    for p in (0, 3, 9, 15):
        kv_len = min(p + 1, max_seq)
        a = orc.decode_forward(q, k, v, kv_pos=p, num_heads=H, num_kv_heads=Hkv,
                               head_dim=d, max_seq=max_seq, scale=scale)
        b = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, kv_len, start_pos=min(p, kv_len - 1))
        _close(a[0], b[0], 1e-12, f"decode out p={p}")
        _close(a[1], b[1], 1e-12, f"decode lse p={p}")
        bo, bl = _brute(q, k, v, H, Hkv, d, CROSS, kv_len, 0, scale)
        _close(a[0], bo, 1e-12, f"decode brute p={p}")
        _close(a[1], bl, 1e-12, f"decode brute lse p={p}")


def pin_row_subset(orc):
    """Computing a subset of rows gives those rows of the whole pass."""
    H, Hkv, d, n = 2, 1, 4, 9
    q, k, v = _rand((n, H * d), 86), _rand((n, Hkv * d), 87), _rand((n, Hkv * d), 88)
    a = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, n)
    rows = np.array([8, 0, 3])
    b = _fwd(orc, q, k, v, H, Hkv, d, CAUSAL, n, rows=rows)
    _close(a[0][rows], b[0], 0.0, "subset out")
    _close(a[1][rows], b[1], 0.0, "subset lse")


# ------------------------------------------------------ rotary embedding (RoPE)
# The rotation the checker reads into the pages' rotary hooks: rotate-half
# pairing (e with e + d/2), angle p * theta^(-2e/d). The pins below restate it
# in other forms: complex multiplication, unit-vector probes, the 2-D rotation
# matrix, scalar loops, and the relative-position property of rotary scores.

def _complex_rotate(x, positions, H, d, theta):
    """x [n, H*d] rotated as complex numbers z_e = x_e + i x_{e+d/2} times
    exp(i p w_e), w_e = 1 / theta^(2e/d)."""
    half = d // 2
    w = 1.0 / np.power(float(theta), np.arange(0, d, 2, dtype=np.float64) / d)
    xh = np.asarray(x, dtype=np.float64).reshape(len(positions), H, d)
    z = xh[..., :half] + 1j * xh[..., half:]
    z = z * np.exp(1j * np.asarray(positions, dtype=np.float64)[:, None, None] * w[None, None, :])
    return np.concatenate([z.real, z.imag], axis=-1).reshape(len(positions), H * d)


def pin_rope_complex_form(orc):
    """The table-driven rotation equals multiplication by exp(i p w_e)."""
    for theta, d in ((10000.0, 8), (500.0, 16), (1e6, 4)):
        H, n = 3, 11
        x = _rand((n, H * d), 301)
        pos = np.random.default_rng(302).integers(0, 70, size=n)
        got = orc.apply_rope(x, pos, orc.rope_table(70, d, theta), H, d)
        _close(got, _complex_rotate(x, pos, H, d, theta), 1e-12, f"rope complex theta={theta}")


def pin_rope_unit_vectors(orc):
    """Basis vector e_k (k < d/2) at position p turns into cos(a) e_k +
    sin(a) e_{k+d/2}; e_{k+d/2} into -sin(a) e_k + cos(a) e_{k+d/2};
    a = p * theta^(-2k/d)."""
    d, theta, p = 8, 10000.0, 37
    table = orc.rope_table(p + 1, d, theta)
    for k in range(d // 2):
        a = p * math.pow(theta, -2.0 * k / d)
        lo = np.zeros((1, d))
        lo[0, k] = 1.0
        want = np.zeros((1, d))
        want[0, k], want[0, k + d // 2] = math.cos(a), math.sin(a)
        _close(orc.apply_rope(lo, [p], table, 1, d), want, 1e-14, f"e_{k}")
        hi = np.zeros((1, d))
        hi[0, k + d // 2] = 1.0
        want = np.zeros((1, d))
        want[0, k], want[0, k + d // 2] = -math.sin(a), math.cos(a)
        _close(orc.apply_rope(hi, [p], table, 1, d), want, 1e-14, f"e_{k + d // 2}")


def pin_rope_position_zero_is_identity(orc):
    x = _rand((4, 2 * 8), 303)
    t = orc.rope_table(1, 8, 10000.0)
    _close(t[0, :, 0], np.ones(4), 0.0, "cos at 0")
    _close(t[0, :, 1], np.zeros(4), 0.0, "sin at 0")
    _close(orc.apply_rope(x, [0, 0, 0, 0], t, 2, 8), x, 0.0, "rotation at 0")


def pin_rope_head_dim_two_is_plane_rotation(orc):
    """d = 2: one pair with frequency theta^0 = 1, i.e. the plane rotation by
    p radians."""
    x = _rand((5, 2), 304).astype(np.float64)
    pos = np.array([0, 1, 2, 7, 100])
    got = orc.apply_rope(x, pos, orc.rope_table(101, 2, 123.0), 1, 2)
    for r, p in enumerate(pos):
        c, s_ = math.cos(p), math.sin(p)
        want = [c * x[r, 0] - s_ * x[r, 1], s_ * x[r, 0] + c * x[r, 1]]
        _close(got[r], want, 1e-14, f"plane rotation p={p}")


def pin_rope_relative_position(orc):
    """Rotary scores depend on positions only through their difference, and
    <R(m) q, R(n) k> = <q, R(n - m) k>; each pair keeps its norm."""
    d, H, theta = 16, 2, 10000.0
    table = orc.rope_table(200, d, theta)
    q, k = _rand((1, H * d), 305), _rand((1, H * d), 306)
    def dot(m, n, qq=q):
        a = orc.apply_rope(qq, [m], table, H, d).reshape(H, d)
        b = orc.apply_rope(k, [n], table, H, d).reshape(H, d)
        return (a * b).sum(axis=1)
    for m, n, c in ((3, 10, 50), (0, 0, 120), (40, 5, 7)):
        _close(dot(m, n), dot(m + c, n + c), 1e-11, f"shift m={m} n={n}")
    for m, n in ((3, 10), (20, 20), (2, 150)):
        _close(dot(m, n), dot(0, n - m), 1e-11, f"difference m={m} n={n}")
    r = orc.apply_rope(q, [77], table, H, d).reshape(H, 2, d // 2)
    x = np.asarray(q, np.float64).reshape(H, 2, d // 2)
    _close((r ** 2).sum(axis=1), (x ** 2).sum(axis=1), 1e-12, "pair norms")


def pin_rope_attention_positions(orc):
    """Attention with rotation equals plain attention on inputs turned by the
    complex form: query row i at start_pos + i, key row j at j, every head
    (GQA) rotated, for a causal continuation and a cross pass over a subset of
    rows."""
    H, Hkv, d, theta = 4, 2, 8, 10000.0
    q_seq, kv_len, start = 5, 9, 4
    q, k, v = _rand((q_seq, H * d), 307), _rand((kv_len + 2, Hkv * d), 308), _rand((kv_len + 2, Hkv * d), 309)
    table = orc.rope_table(kv_len + 2, d, theta)
    qr = _complex_rotate(q, start + np.arange(q_seq), H, d, theta)
    kr = _complex_rotate(k, np.arange(kv_len + 2), Hkv, d, theta)
    for mode, sp, rows in ((CAUSAL, start, None), (CROSS, 0, np.array([4, 1]))):
        a = orc.attention_forward(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=mode,
                                  kv_len=kv_len, start_pos=sp, scale=0.3, rows=rows, rope=table)
        qq = qr if mode == CAUSAL else _complex_rotate(q, np.arange(q_seq), H, d, theta)
        b = orc.attention_forward(qq, kr, v, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=mode,
                                  kv_len=kv_len, start_pos=sp, scale=0.3, rows=rows)
        _close(a[0], b[0], 1e-12, f"rope attention out mode={mode}")
        _close(a[1], b[1], 1e-12, f"rope attention lse mode={mode}")


def pin_rope_brute_force_tiny(orc):
    """Scalar loops: rotate with math.cos / math.sin of p * theta^(-2e/d),
    then the brute-force attention."""
    H, Hkv, d, theta, q_seq, kv_len, start = 2, 1, 4, 50.0, 3, 5, 2
    q, k, v = _rand((q_seq, H * d), 310), _rand((kv_len, Hkv * d), 311), _rand((kv_len, Hkv * d), 312)
    def rot(x, nheads, pos_of):
        y = np.array(x, dtype=np.float64)
        for r in range(x.shape[0]):
            p = pos_of(r)
            for h in range(nheads):
                for e in range(d // 2):
                    a = p * math.pow(theta, -2.0 * e / d)
                    x0, x1 = float(x[r, h * d + e]), float(x[r, h * d + e + d // 2])
                    y[r, h * d + e] = x0 * math.cos(a) - x1 * math.sin(a)
                    y[r, h * d + e + d // 2] = x1 * math.cos(a) + x0 * math.sin(a)
        return y
    qr = rot(q, H, lambda r: start + r)
    kr = rot(k, Hkv, lambda r: r)
    want = _brute(qr, kr, v, H, Hkv, d, CAUSAL, kv_len, start, 0.5)
    got = orc.attention_forward(q, k, v, num_heads=H, num_kv_heads=Hkv, head_dim=d, mode=CAUSAL,
                                kv_len=kv_len, start_pos=start, scale=0.5,
                                rope=orc.rope_table(kv_len, d, theta))
    _close(got[0], want[0], 1e-12, "rope brute out")
    _close(got[1], want[1], 1e-12, "rope brute lse")


# --------------------------------------------------------------- backward
# The checker's gradients are pinned to the forward itself (central finite
# differences of L = sum(dout * out)), to torch's autograd through a plain
# masked-softmax attention, and to identities of the softmax Jacobian.

def _bwd(orc, q, k, v, g, H, Hkv, d, mode, kv_len, start_pos=0, scale=0.4, **kw):
    return orc.attention_backward(q, k, v, g, num_heads=H, num_kv_heads=Hkv, head_dim=d,
                                  mode=mode, kv_len=kv_len, start_pos=start_pos, scale=scale,
                                  **kw)


def pin_backward_finite_differences(orc):
    """Each gradient entry against (L(x + h) - L(x - h)) / 2h of the
    checker's own forward, L = sum(dout * out)."""
    H, Hkv, d, hstep = 2, 1, 3, 1e-6
    for mode, n, kv_len, sp in ((CAUSAL, 4, 5, 1), (CROSS, 3, 4, 0), (FULL, 3, 3, 0)):
        rng = np.random.default_rng(400 + mode)
        q = rng.standard_normal((n, H * d))
        k = rng.standard_normal((kv_len, Hkv * d))
        v = rng.standard_normal((kv_len, Hkv * d))
        g = rng.standard_normal((n, H * d))
        def loss(qq, kk, vv):
            o, _ = orc.attention_forward(qq, kk, vv, num_heads=H, num_kv_heads=Hkv, head_dim=d,
                                         mode=mode, kv_len=kv_len, start_pos=sp, scale=0.4)
            return float((o * g).sum())
        dq, dk, dv = _bwd(orc, q, k, v, g, H, Hkv, d, mode, kv_len, sp)
        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += hstep
                xm[idx] -= hstep
                args = {"q": (q, k, v), "k": (q, k, v), "v": (q, k, v)}[name]
                ap = [xp if a is x else a for a in args]
                am = [xm if a is x else a for a in args]
                num[idx] = (loss(*ap) - loss(*am)) / (2 * hstep)
            _close(grad, num, 2e-7, f"finite differences d{name} mode={mode}")


def pin_backward_torch_autograd(orc):
    """torch autograd (float64, CPU) through a masked softmax attention."""
    import torch
    H, Hkv, d = 4, 2, 8
    for mode, n, kv_len, sp in ((CAUSAL, 7, 9, 2), (FULL, 6, 6, 0), (CROSS, 5, 11, 0)):
        q, k, v = _rand((n, H * d), 410), _rand((kv_len, Hkv * d), 411), _rand((kv_len, Hkv * d), 412)
        g = _rand((n, H * d), 413)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        g_ = H // Hkv
        qh = tq.view(n, H, d).transpose(0, 1)
        kh = tk.view(kv_len, Hkv, d).transpose(0, 1).repeat_interleave(g_, dim=0)
        vh = tv.view(kv_len, Hkv, d).transpose(0, 1).repeat_interleave(g_, dim=0)
        s = 0.4 * qh @ kh.transpose(1, 2)
        w = torch.tensor([_window(mode, i, n, kv_len, sp) for i in range(n)])
        mask = torch.arange(kv_len)[None, :] < w[:, None]
        p = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1)
        out = (p @ vh).transpose(0, 1).reshape(n, H * d)
        (out * torch.tensor(g, dtype=torch.float64)).sum().backward()
        dq, dk, dv = _bwd(orc, q, k, v, g, H, Hkv, d, mode, kv_len, sp)
        _close(dq, tq.grad.numpy(), 1e-12, f"autograd dq mode={mode}")
        _close(dk, tk.grad.numpy(), 1e-12, f"autograd dk mode={mode}")
        _close(dv, tv.grad.numpy(), 1e-12, f"autograd dv mode={mode}")


def pin_backward_single_key(orc):
    """One key in every window: softmax is the constant 1, so dq = dk = 0 and
    dv is the sum of dout over the rows and the group's heads."""
    H, Hkv, d, n = 4, 2, 5, 6
    q, k, v, g = _rand((n, H * d), 420), _rand((1, Hkv * d), 421), _rand((1, Hkv * d), 422), \
        _rand((n, H * d), 423)
    dq, dk, dv = _bwd(orc, q, k, v, g, H, Hkv, d, CROSS, 1)
    _close(dq, np.zeros_like(dq), 0.0, "single key dq")
    _close(dk, np.zeros_like(dk), 0.0, "single key dk")
    gs = g.astype(np.float64).reshape(n, Hkv, H // Hkv, d).sum(axis=(0, 2)).reshape(1, Hkv * d)
    _close(dv, gs, 1e-12, "single key dv")


def pin_backward_sums(orc):
    """Every row's dS sums to 0 over its window, so the keys' dk sum to 0;
    every non-empty row's weights sum to 1, so the keys' dv sum to the
    rows' dout (per KV head, over its group)."""
    H, Hkv, d = 6, 2, 4
    for mode, n, kv_len, sp in ((CAUSAL, 9, 12, 3), (CROSS, 5, 0, 0), (CROSS, 7, 10, 0)):
        q, k, v, g = (_rand((n, H * d), 430), _rand((max(kv_len, 1), Hkv * d), 431),
                      _rand((max(kv_len, 1), Hkv * d), 432), _rand((n, H * d), 433))
        dq, dk, dv = _bwd(orc, q, k, v, g, H, Hkv, d, mode, kv_len, sp)
        _close(dk.sum(axis=0), np.zeros(Hkv * d), 1e-12, f"sum dk mode={mode}")
        live = np.array([_window(mode, i, n, kv_len, sp) > 0 for i in range(n)])
        gs = g.astype(np.float64)[live].reshape(-1, Hkv, H // Hkv, d).sum(axis=(0, 2)).reshape(-1)
        _close(dv.sum(axis=0), gs, 1e-12, f"sum dv mode={mode}")
        if kv_len == 0:
            _close(dq, np.zeros_like(dq), 0.0, "empty windows dq")


def pin_backward_linear_in_dout(orc):
    H, Hkv, d, n = 2, 1, 4, 6
    q, k, v = _rand((n, H * d), 440), _rand((n, Hkv * d), 441), _rand((n, Hkv * d), 442)
    g1, g2 = _rand((n, H * d), 443), _rand((n, H * d), 444)
    a = _bwd(orc, q, k, v, g1, H, Hkv, d, CAUSAL, n)
    b = _bwd(orc, q, k, v, g2, H, Hkv, d, CAUSAL, n)
    c = _bwd(orc, q, k, v, 2.0 * g1.astype(np.float64) - 3.0 * g2.astype(np.float64), H, Hkv, d,
             CAUSAL, n)
    for x, y, z, nm in zip(a, b, c, ("dq", "dk", "dv")):
        _close(z, 2.0 * x - 3.0 * y, 1e-12, f"linear {nm}")


def pin_backward_selection(orc):
    """rows / keys / kv_heads return exactly those parts of the whole."""
    H, Hkv, d, n = 4, 2, 4, 11
    q, k, v, g = (_rand((n, H * d), 450), _rand((n, Hkv * d), 451), _rand((n, Hkv * d), 452),
                  _rand((n, H * d), 453))
    dq, dk, dv = _bwd(orc, q, k, v, g, H, Hkv, d, CAUSAL, n, row_block=4)
    rows, keys = np.array([10, 2, 5]), np.array([0, 7, 3])
    sq, sk, sv = _bwd(orc, q, k, v, g, H, Hkv, d, CAUSAL, n, rows=rows, keys=keys, kv_heads=[1])
    cols = slice(1 * 2 * d, 2 * 2 * d)
    _close(sq[:, cols], dq[rows][:, cols], 1e-13, "selected dq")
    _close(sq[:, :2 * d], np.zeros((3, 2 * d)), 0.0, "unselected heads dq")
    _close(sk[:, d:], dk[keys][:, d:], 1e-13, "selected dk")
    _close(sv[:, d:], dv[keys][:, d:], 1e-13, "selected dv")


def pin_backward_magnitudes_bound_results(orc):
    """The magnitude sums bound the gradients (triangle inequality) and are
    returned beside the unchanged gradients."""
    H, Hkv, d, n = 4, 2, 4, 10
    q, k, v, g = (_rand((n, H * d), 460), _rand((n, Hkv * d), 461), _rand((n, Hkv * d), 462),
                  _rand((n, H * d), 463))
    plain = _bwd(orc, q, k, v, g, H, Hkv, d, CAUSAL, n)
    full = _bwd(orc, q, k, v, g, H, Hkv, d, CAUSAL, n, magnitudes=True)
    for a, b, m, nm in zip(plain, full[:3], full[3:], ("dq", "dk", "dv")):
        _close(a, b, 0.0, f"{nm} unchanged")
        assert np.all(m >= np.abs(b) - 1e-12), f"{nm} magnitudes below |gradient|"


def _brute_magnitudes(q, k, v, g, H, Hkv, d, mode, kv_len, start_pos, scale):
    """Scalar loops with math.fsum: the magnitude sums of the gradients'
    terms, one number at a time. For each head h (KV head c), row i and key
    j < w_i: P_ij, dP_ij = <dout_i, v_j>, D_i = sum_j P_ij dP_ij,
    dS_ij = P_ij (dP_ij - D_i), E_ij = |dS_ij| + P_ij (|dP_ij| + |D_i|);
    dq_m[i, h, e] = scale sum_j E_ij |K[j, c, e]|,
    dk_m[j, c, e] = scale sum_{h in c, i} E_ij |Q[i, h, e]|,
    dv_m[j, c, e] = sum_{h in c, i} P_ij |dout[i, h, e]|."""
    n = q.shape[0]
    group = H // Hkv
    qf, kf, vf, gf = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    dq_m = np.zeros((n, H * d))
    dk_terms = [[[] for _ in range(Hkv * d)] for _ in range(kv_len)]
    dv_terms = [[[] for _ in range(Hkv * d)] for _ in range(kv_len)]
    for h in range(H):
        c = h // group
        for i in range(n):
            w = _window(mode, i, n, kv_len, start_pos)
            if w == 0:
                continue
            s = [scale * math.fsum(qf[i, h * d + e] * kf[j, c * d + e] for e in range(d))
                 for j in range(w)]
            m = max(s)
            z = math.fsum(math.exp(x - m) for x in s)
            p = [math.exp(x - m) / z for x in s]
            dp = [math.fsum(gf[i, h * d + e] * vf[j, c * d + e] for e in range(d))
                  for j in range(w)]
            dd = math.fsum(p[j] * dp[j] for j in range(w))
            em = [abs(p[j] * (dp[j] - dd)) + p[j] * (abs(dp[j]) + abs(dd)) for j in range(w)]
            for e in range(d):
                dq_m[i, h * d + e] = scale * math.fsum(em[j] * abs(kf[j, c * d + e])
                                                       for j in range(w))
            for j in range(w):
                for e in range(d):
                    dk_terms[j][c * d + e].append(em[j] * abs(qf[i, h * d + e]))
                    dv_terms[j][c * d + e].append(p[j] * abs(gf[i, h * d + e]))
    dk_m = np.array([[scale * math.fsum(t) for t in row] for row in dk_terms]).reshape(
        kv_len, Hkv * d)
    dv_m = np.array([[math.fsum(t) for t in row] for row in dv_terms]).reshape(kv_len, Hkv * d)
    return dq_m, dk_m, dv_m


def pin_backward_magnitudes_scalar_loops(orc):
    """The magnitude sums that widen the gradient tolerance, exactly (to
    float64 rounding) against scalar loops over their terms: an inflated or
    dropped term moves them either way and fails here."""
    for mode, n, kv_len, sp, H, Hkv in ((CAUSAL, 5, 7, 2, 4, 2), (CROSS, 4, 6, 0, 2, 1),
                                        (FULL, 4, 4, 0, 3, 3)):
        d = 3
        q, k, v, g = (_rand((n, H * d), 470 + mode), _rand((kv_len, Hkv * d), 471 + mode),
                      _rand((kv_len, Hkv * d), 472 + mode), _rand((n, H * d), 473 + mode))
        got = _bwd(orc, q, k, v, g, H, Hkv, d, mode, kv_len, sp, magnitudes=True)[3:]
        want = _brute_magnitudes(q, k, v, g, H, Hkv, d, mode, kv_len, sp, 0.4)
        for a, b, nm in zip(got, want, ("dq_m", "dk_m", "dv_m")):
            assert np.all(b >= 0.0)
            _close(a, b, 1e-12 * max(1.0, float(np.abs(b).max())), f"{nm} mode={mode}")


def pin_backward_dv_magnitude_is_dv_of_abs_dout(orc):
    """dv = P^T dout is linear in dout with P >= 0, so its magnitude sum
    P^T |dout| is the checker's own dv for the input |dout|."""
    H, Hkv, d, n = 4, 2, 4, 9
    q, k, v, g = (_rand((n, H * d), 480), _rand((n, Hkv * d), 481), _rand((n, Hkv * d), 482),
                  _rand((n, H * d), 483))
    full = _bwd(orc, q, k, v, g, H, Hkv, d, CAUSAL, n, 0, magnitudes=True)
    dv_abs = _bwd(orc, q, k, v, np.abs(g), H, Hkv, d, CAUSAL, n, 0)[2]
    _close(full[5], dv_abs, 1e-12, "dv_m vs dv(|dout|)")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
