"""Float64 CPU checker for the fused attention forward.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never calls it and
shares no code with it.

What it computes is the plain definition that the pages' tiled online-softmax
shaders reach up to rounding order:

    s_ij = scale * <Q[i, h], K[j, kv_head(h)]>           for j < w_i
    m_i  = max_j s_ij
    Z_i  = sum_j exp(s_ij - m_i)
    out[i, h] = sum_j exp(s_ij - m_i) / Z_i * V[j, kv_head(h)]
    lse[i, h] = (m_i, log Z_i)

Sources (pages' titles and the part of each shader):
  * meganeura ``attention.wgsl`` -- header comment (the causal / full / cross
    windows), ``main`` body (GQA head map, online update, normalisation with a
    safe zero sum, and the (max, log of the running sum) pair written "for
    backward");
  * meganeura ``cached_attention.wgsl`` -- header and ``main`` (one query row,
    window [0, kv_pos] with kv_pos read from a device buffer);
  * cera ``attention_prefill.wgsl`` -- header "Constraints" and ``main`` (causal
    window continued from ``start_pos`` and clamped to the cache length; a
    zero-length window writes zeros).

Backward (``attention_backward``): the pages store the (max, log-sum) pair
for a backward pass they do not give; the checker returns the exact gradients
of the definition above for the loss sum(dout * out).

Rotary position embedding (optional, ``rope``): meganeura ``attention.wgsl``
applies a rotation hook to each loaded query element and builds each key
element through a hook expression, but the pages give no formula. The reading
taken here is the common rotary embedding with "rotate-half" pairing: in each
head, element e < d/2 pairs with element e + d/2, and the pair at position p is
turned by the angle p * theta^(-2e/d):

    x'[e]       = x[e] cos(a) - x[e + d/2] sin(a)
    x'[e + d/2] = x[e + d/2] cos(a) + x[e] sin(a)

with query row i at position start_pos + i and key row j at position j. The
rotation takes its (cos, sin) values from a table [positions, d/2, 2], so a
caller may pass any table; ``rope_table`` builds the standard one.

The scores are materialised block-of-rows by block-of-rows (rows are
independent, so this changes no arithmetic of any row); everything is float64.
Parity is pinned by the CPU tests (closed forms, brute force, torch's library
attention, invariants); no function here is "parity unpinned".
"""

from __future__ import annotations

import numpy as np

CAUSAL, FULL, CROSS = 0, 1, 2

# Initial running max and empty-window log-sum value of meganeura
# attention.wgsl (``main``: ``max_score`` start value and the ``select`` on a
# zero sum in the side-output write).
EMPTY_SENTINEL = -1e30


def window_length(mode: int, i: int, q_seq: int, kv_len: int, start_pos: int) -> int:
    """Keys [0, w) that query row i attends to.

    attention.wgsl header: causal uses pos+1, full uses q_seq, cross uses the
    kv length. attention_prefill.wgsl ``main``: the causal position is
    start_pos + i and the window is clamped to the cache length.
    """
    if mode == CAUSAL:
        return max(0, min(start_pos + i + 1, kv_len))
    if mode == FULL:
        return q_seq
    if mode == CROSS:
        return kv_len
    raise ValueError(f"unknown mode {mode}")


def rope_table(rows: int, head_dim: int, theta: float):
    """Standard rotary table [rows, head_dim/2, 2] in float64: entry (p, e) is
    (cos, sin) of p * theta^(-2e/head_dim)."""
    if head_dim % 2 != 0:
        raise ValueError("head_dim must be even")
    half = head_dim // 2
    inv_freq = float(theta) ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    ang = np.arange(rows, dtype=np.float64)[:, None] * inv_freq[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1)


def apply_rope(x, positions, table, num_heads: int, head_dim: int):
    """Rotate every head of the rows x [n, num_heads*head_dim], row r at
    position positions[r], with (cos, sin) from table [*, head_dim/2, 2]
    (rotate-half pairing). Returns float64."""
    positions = np.asarray(positions, dtype=np.int64)
    n = positions.shape[0]
    half = head_dim // 2
    xh = np.asarray(x, dtype=np.float64).reshape(n, num_heads, head_dim)
    t = np.asarray(table, dtype=np.float64)[positions]  # [n, half, 2]
    c = t[:, None, :, 0]
    s = t[:, None, :, 1]
    lo = xh[..., :half]
    hi = xh[..., half:]
    out = np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)
    return out.reshape(n, num_heads * head_dim)


def _check_shapes(q, k, v, num_heads, num_kv_heads, head_dim, kv_len):
    if num_heads % num_kv_heads != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    if q.shape[1] != num_heads * head_dim:
        raise ValueError("q must be [q_seq, num_heads*head_dim]")
    if k.shape[1] != num_kv_heads * head_dim or v.shape[1] != num_kv_heads * head_dim:
        raise ValueError("k, v must be [rows, num_kv_heads*head_dim]")
    if k.shape[0] < kv_len or v.shape[0] < kv_len:
        raise ValueError("k, v hold fewer than kv_len rows")


def attention_forward(q, k, v, *, num_heads: int, num_kv_heads: int, head_dim: int,
                      mode: int, kv_len: int, start_pos: int = 0, scale: float,
                      rows=None, row_block: int = 256, rope=None):
    """Attention forward in float64 for the query rows ``rows`` (default: all).

    q: [q_seq, num_heads*head_dim]; k, v: [>= kv_len, num_kv_heads*head_dim].
    Returns (out [n_rows, num_heads*head_dim], lse [n_rows, num_heads, 2]),
    both float64; lse[..., 0] is the row max and lse[..., 1] the log of the
    sum of exp(score - max), the pair meganeura attention.wgsl stores.
    rope: optional rotary table [positions, head_dim/2, 2]; query row i is
    rotated at position start_pos + i, key row j at position j.
    """
    _check_shapes(q, k, v, num_heads, num_kv_heads, head_dim, kv_len)
    q_seq = q.shape[0]
    if mode == FULL and kv_len != q_seq:
        raise ValueError("full attention needs kv_len == q_seq")
    if rows is None:
        rows = np.arange(q_seq)
    rows = np.asarray(rows, dtype=np.int64)
    n = rows.shape[0]
    group = num_heads // num_kv_heads
    d = head_dim

    out = np.zeros((n, num_heads * d), dtype=np.float64)
    lse = np.full((n, num_heads, 2), EMPTY_SENTINEL, dtype=np.float64)
    win = np.array([window_length(mode, int(i), q_seq, kv_len, start_pos) for i in rows],
                   dtype=np.int64)

    if rope is not None:
        q = apply_rope(q[rows], start_pos + rows, rope, num_heads, d)
        rows_in_q = np.arange(n)  # q now holds exactly the selected rows
        k = apply_rope(k[:kv_len], np.arange(kv_len), rope, num_kv_heads, d)
    else:
        rows_in_q = rows

    for h in range(num_heads):
        kvh = h // group  # GQA: contiguous groups of query heads share a KV head
        qh = q[:, h * d:(h + 1) * d]
        kh = k[:, kvh * d:(kvh + 1) * d]
        vh = v[:, kvh * d:(kvh + 1) * d]
        for b0 in range(0, n, row_block):
            sel = slice(b0, min(b0 + row_block, n))
            r = rows_in_q[sel]
            w = win[sel]
            wmax = int(w.max()) if w.size else 0
            if wmax == 0:
                continue  # every row empty: out stays 0, lse stays the sentinel
            qb = qh[r].astype(np.float64)
            kb = kh[:wmax].astype(np.float64)
            vb = vh[:wmax].astype(np.float64)
            s = scale * (qb @ kb.T)  # [rows, wmax]
            valid = np.arange(wmax)[None, :] < w[:, None]
            s = np.where(valid, s, -np.inf)
            m = s.max(axis=1)
            nonempty = w > 0
            m_safe = np.where(nonempty, m, 0.0)
            e = np.where(valid, np.exp(s - m_safe[:, None]), 0.0)
            z = e.sum(axis=1)
            z_safe = np.where(nonempty, z, 1.0)
            o = (e @ vb) / z_safe[:, None]
            out[sel, h * d:(h + 1) * d] = np.where(nonempty[:, None], o, 0.0)
            lse[sel, h, 0] = np.where(nonempty, m, EMPTY_SENTINEL)
            lse[sel, h, 1] = np.where(nonempty, np.log(z_safe), EMPTY_SENTINEL)
    return out, lse


def attention_backward(q, k, v, dout, *, num_heads: int, num_kv_heads: int, head_dim: int,
                       mode: int, kv_len: int, start_pos: int = 0, scale: float,
                       rows=None, keys=None, kv_heads=None, row_block: int = 256,
                       magnitudes: bool = False):
    """Gradients of the forward above, in float64: for the loss
    L = sum(dout * out), returns (dq, dk, dv).

    The pages keep the (max, log-sum) pair "for backward" but give no
    backward algorithm; this is the derivative of the plain definition.
    Per head h (kv head c = h // group), over the rows' windows:
        P   = softmax_j(s_ij)            (0 for an empty window)
        dP  = dout_h V_c^T
        D_i = sum_j P_ij dP_ij           (= <dout_i, out_i>)
        dS  = P * (dP - D)
        dq_h  = scale * dS K_c
        dk_c += scale * dS^T Q_h
        dv_c += P^T dout_h
    q, dout: [q_seq, num_heads*head_dim]; k, v: [>= kv_len, num_kv_heads*head_dim].
    rows / keys select the query rows of dq and the key rows of dk, dv that
    are returned (default: all rows, keys [0, kv_len)); kv_heads restricts
    the computation to the query heads of those KV heads (the other columns
    are returned as 0). Returns dq [n_rows, H*d], dk, dv [n_keys, Hkv*d].

    magnitudes=True also returns, for a rounding-error bound of a float32
    evaluation, the same sums over magnitudes (dq_m, dk_m, dv_m): with
    E_ij = |dS_ij| + P_ij (|dP_ij| + |D_i|) (dS and the rounding of its two
    terms), dq_m = scale E|K|, dk_m = scale E^T|Q|, dv_m = P^T|dout|.
    """
    _check_shapes(q, k, v, num_heads, num_kv_heads, head_dim, kv_len)
    q_seq = q.shape[0]
    if mode == FULL and kv_len != q_seq:
        raise ValueError("full attention needs kv_len == q_seq")
    rows = np.arange(q_seq) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(kv_len) if keys is None else np.asarray(keys, dtype=np.int64)
    kv_heads = range(num_kv_heads) if kv_heads is None else kv_heads
    group = num_heads // num_kv_heads
    d = head_dim
    row_pos = {int(r): n for n, r in enumerate(rows)}
    dq = np.zeros((rows.shape[0], num_heads * d), dtype=np.float64)
    dk = np.zeros((keys.shape[0], num_kv_heads * d), dtype=np.float64)
    dv = np.zeros((keys.shape[0], num_kv_heads * d), dtype=np.float64)
    if magnitudes:
        dq_m, dk_m, dv_m = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    win = np.array([window_length(mode, i, q_seq, kv_len, start_pos) for i in range(q_seq)],
                   dtype=np.int64)
    for c in kv_heads:
        kc = k[:kv_len, c * d:(c + 1) * d].astype(np.float64)
        vc = v[:kv_len, c * d:(c + 1) * d].astype(np.float64)
        for h in range(c * group, (c + 1) * group):
            for b0 in range(0, q_seq, row_block):
                r = np.arange(b0, min(b0 + row_block, q_seq))
                w = win[r]
                if w.max() == 0:
                    continue
                qb = q[r, h * d:(h + 1) * d].astype(np.float64)
                gb = dout[r, h * d:(h + 1) * d].astype(np.float64)
                s = scale * (qb @ kc.T)
                valid = np.arange(kv_len)[None, :] < w[:, None]
                s = np.where(valid, s, -np.inf)
                m = np.where(w > 0, s.max(axis=1), 0.0)
                e = np.where(valid, np.exp(s - m[:, None]), 0.0)
                z = e.sum(axis=1)
                p = e / np.where(w > 0, z, 1.0)[:, None]
                dp = gb @ vc.T
                dd = (p * dp).sum(axis=1)
                ds = p * (dp - dd[:, None])
                dk[:, c * d:(c + 1) * d] += scale * (ds[:, keys].T @ qb)
                dv[:, c * d:(c + 1) * d] += p[:, keys].T @ gb
                sel = [n for n, i in enumerate(r) if int(i) in row_pos]
                if sel:
                    dq[[row_pos[int(r[n])] for n in sel], h * d:(h + 1) * d] = \
                        scale * (ds[sel] @ kc)
                if magnitudes:
                    em = np.abs(ds) + p * (np.abs(dp) + np.abs(dd)[:, None])
                    dk_m[:, c * d:(c + 1) * d] += scale * (em[:, keys].T @ np.abs(qb))
                    dv_m[:, c * d:(c + 1) * d] += p[:, keys].T @ np.abs(gb)
                    if sel:
                        dq_m[[row_pos[int(r[n])] for n in sel], h * d:(h + 1) * d] = \
                            scale * (em[sel] @ np.abs(kc))
    if magnitudes:
        return dq, dk, dv, dq_m, dk_m, dv_m
    return dq, dk, dv


def decode_forward(q, k_cache, v_cache, *, kv_pos: int, num_heads: int,
                   num_kv_heads: int, head_dim: int, max_seq: int, scale: float):
    """One-token decode over a cache, in float64.

    cached_attention.wgsl ``main``: the window is [0, kv_pos] (kv_len =
    kv_pos + 1), one query row of num_heads heads; the length is clamped to the
    cache's max_seq rows as attention_prefill.wgsl clamps its window.
    q: [1, num_heads*head_dim]; caches: [max_seq, num_kv_heads*head_dim].
    Returns (out [1, num_heads*head_dim], lse [1, num_heads, 2]).
    """
    if num_heads % num_kv_heads != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    kv_len = max(0, min(int(kv_pos) + 1, max_seq))
    group = num_heads // num_kv_heads
    d = head_dim
    out = np.zeros((1, num_heads * d), dtype=np.float64)
    lse = np.full((1, num_heads, 2), EMPTY_SENTINEL, dtype=np.float64)
    if kv_len == 0:
        return out, lse
    for h in range(num_heads):
        kvh = h // group
        qv = q[0, h * d:(h + 1) * d].astype(np.float64)
        kw = k_cache[:kv_len, kvh * d:(kvh + 1) * d].astype(np.float64)
        vw = v_cache[:kv_len, kvh * d:(kvh + 1) * d].astype(np.float64)
        s = scale * (kw @ qv)
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        out[0, h * d:(h + 1) * d] = (e @ vw) / z
        lse[0, h, 0] = m
        lse[0, h, 1] = np.log(z)
    return out, lse
