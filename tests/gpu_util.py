"""Helpers shared by the GPU parity tests: device upload, calls through the
C ABI (via the ctypes binding) and the tolerance checks.

Tolerances: out elementwise |gpu - ref| <= 1e-4 + 1e-4*|ref|; each lse
component |gpu - ref| <= 1e-4; the empty-window sentinel -1e30 exactly.
Gradients (check_grad) add the rounding of a float32 sum of N terms to the
out bound: 4 sqrt(N) u M, u = 2^-24, with M the sum of the terms' magnitudes
(the checker's ``magnitudes``; a probabilistic form of the |error| <= N u M
bound of recursive summation).
"""

from __future__ import annotations

import sys

import numpy as np

import oracle
import tiled_attention_03_amd as ta

OUT_ATOL = 1e-4
OUT_RTOL = 1e-4
LSE_ATOL = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device())


def gpu_prefill(q, k, v, *, num_heads, num_kv_heads, head_dim, mode, kv_len,
                start_pos=0, scale, with_lse=True, q_dev=None, k_dev=None, v_dev=None):
    import torch
    qd = to_dev(q) if q_dev is None else q_dev
    kd = to_dev(k) if k_dev is None else k_dev
    vd = to_dev(v) if v_dev is None else v_dev
    out, lse = ta.attention(qd, kd, vd, num_heads=num_heads, num_kv_heads=num_kv_heads,
                            head_dim=head_dim, mode=mode, kv_len=kv_len,
                            start_pos=start_pos, scale=scale, with_lse=with_lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (lse.cpu().numpy() if lse is not None else None)


def oracle_prefill(q, k, v, *, num_heads, num_kv_heads, head_dim, mode, kv_len,
                   start_pos=0, scale, rows=None):
    return oracle.attention_forward(q, k, v, num_heads=num_heads, num_kv_heads=num_kv_heads,
                                    head_dim=head_dim, mode=mode, kv_len=kv_len,
                                    start_pos=start_pos, scale=scale, rows=rows)


def check_out(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bound = OUT_ATOL + OUT_RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} out elements off; "
                           f"worst {float((err - bound).max()):.3e} over bound, "
                           f"max abs err {float(err.max()):.3e}")
    return float(err.max()) if err.size else 0.0


def check_grad(got, ref, mag, n_terms, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    fwd_bound = OUT_ATOL + OUT_RTOL * np.abs(ref)
    bound = fwd_bound + 4.0 * np.sqrt(max(n_terms, 1)) * 2.0 ** -24 * np.asarray(
        mag, dtype=np.float64)
    if err.size:
        # How much of the bound the errors use, and how they compare with the
        # forward's bound alone (above 1: the summation term is needed).
        log(f"  {what}: max err/bound {float((err / bound).max()):.3f}, "
            f"max err/forward bound {float((err / fwd_bound).max()):.3f}")
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} gradient elements off; "
                           f"worst {float((err - bound).max()):.3e} over bound, "
                           f"max abs err {float(err.max()):.3e}")
    return float(err.max()) if err.size else 0.0


def check_lse(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: lse shape {got.shape} vs {ref.shape}"
    sent = ref == oracle.EMPTY_SENTINEL
    assert np.array_equal(got[sent], ref[sent]), f"{what}: empty-window sentinel differs"
    err = np.abs(got[~sent] - ref[~sent])
    assert np.all(np.isfinite(got[~sent])), f"{what}: non-finite lse"
    worst = float(err.max()) if err.size else 0.0
    assert worst <= LSE_ATOL, f"{what}: lse max abs err {worst:.3e} > {LSE_ATOL}"
    return worst
