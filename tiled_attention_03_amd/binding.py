"""ctypes binding of libta03.so: the C-ABI entry points under the same names.

Argument marshalling only. Tensors are torch CUDA (HIP) float32 tensors, read
through ``data_ptr()``; the stream defaults to torch's current stream. The
binding checks that each tensor is on the GPU, float32, contiguous and large
enough for the sizes passed (the C ABI sees bare pointers and cannot), then
calls the library, which validates the sizes themselves. There is no other
implementation behind these names: if the library is missing, every call
raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libta03.so")

CAUSAL, FULL, CROSS = 0, 1, 2
OVERRIDE_PREFILL_ROWS, OVERRIDE_BWD_PATH = 1, 2
STATUS_NAMES = {0: "TA03_OK", -1: "TA03_ERR_NULL", -2: "TA03_ERR_SHAPE",
                -3: "TA03_ERR_UNSUPPORTED", -4: "TA03_ERR_WORKSPACE",
                -5: "TA03_ERR_HIP", -6: "TA03_ERR_ALIGN"}

_lib = None


class Ta03Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libta03.so (built in-tree by tiled_attention_03_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run "
                               "`python -m tiled_attention_03_amd.build` first")
        # torch first: its HIP runtime (bundled, loaded under another file
        # name) must be the one the library binds to. Loaded the other way
        # round, the process holds two HIP runtimes and torch's streams and
        # memory are foreign to the library's launches.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        LL = ctypes.c_longlong
        L.attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, P]
        L.attn_fwd.restype = I
        L.attn_fwd_ex.argtypes = [P, LL, P, LL, P, LL, P, LL, P, I, I, I, I, I, I, I, I, F, P]
        L.attn_fwd_ex.restype = I
        L.attn_fwd_rope.argtypes = [P, LL, P, LL, P, LL, P, LL, P, I, I, I, I, I, I, I, I, F,
                                    P, I, P]
        L.attn_fwd_rope.restype = I
        L.attn_fwd_rope_q.argtypes = L.attn_fwd_rope.argtypes
        L.attn_fwd_rope_q.restype = I
        L.attn_rope_apply.argtypes = [P, LL, P, LL, I, I, I, I, P, I, P]
        L.attn_rope_apply.restype = I
        L.attn_rope_table.argtypes = [P, I, I, ctypes.c_double, P]
        L.attn_rope_table.restype = I
        L.attn_bwd_workspace_bytes.argtypes = [I, I]
        L.attn_bwd_workspace_bytes.restype = S
        L.attn_bwd_workspace_bytes_stored.argtypes = [I, I, I, I, I]
        L.attn_bwd_workspace_bytes_stored.restype = S
        L.attn_bwd_windows.argtypes = [I, I, I, I, I, S]
        L.attn_bwd_windows.restype = I
        L.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, P, S, P]
        L.attn_bwd.restype = I
        L.attn_decode_workspace_bytes.argtypes = [I, I, I, I]
        L.attn_decode_workspace_bytes.restype = S
        L.attn_decode_workspace_init.argtypes = [P, S, I, I, I, I, P]
        L.attn_decode_workspace_init.restype = I
        L.attn_decode.argtypes = [P, P, P, P, P, P, I, I, I, I, F, P, S, P]
        L.attn_decode.restype = I
        L.attn_decode_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, F, P]
        L.attn_decode_noalloc.restype = I
        L.attn_decode_paged.argtypes = [P, P, P, I, I, P, P, P, P, I, I, I, I, F, P, S, P]
        L.attn_decode_paged.restype = I
        L.attn_set_kernel_override.argtypes = [I, I]
        L.attn_set_kernel_override.restype = I
        L.attn_strerror.argtypes = [I]
        L.attn_strerror.restype = ctypes.c_char_p
        _lib = L
    return _lib


def attn_strerror(status: int) -> str:
    return lib().attn_strerror(int(status)).decode()


def attn_set_kernel_override(knob: int, value: int) -> None:
    """Testing hook: force a kernel choice for later calls in this process
    (0 restores the automatic choice; see include/ta03.h)."""
    _check(lib().attn_set_kernel_override(int(knob), int(value)))


def _alloc_stream(stream):
    """The torch stream that tensors allocated for a call on `stream` must
    belong to, so that the caching allocator does not hand their memory to
    other work while the call's kernels may still use it."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.ExternalStream(stream)
    return stream


def _ptr(t, min_numel: int, name: str, *, dtype_name="float32"):
    """Device pointer of tensor ``t`` (or None -> NULL), after checks."""
    if t is None:
        return None
    if isinstance(t, int):  # a raw device address
        return t
    import torch
    want = {"float32": torch.float32, "int32": torch.int32, "uint32": torch.uint32}[dtype_name]
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != want:
        raise ValueError(f"{name} must be {dtype_name}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < min_numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {min_numel}")
    return t.data_ptr() if t.numel() > 0 else None


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != 0:
        raise Ta03Error(status, attn_strerror(status))


def attn_fwd(q, k, v, out, lse, q_seq: int, kv_len: int, num_heads: int,
             num_kv_heads: int, head_dim: int, mode: int, start_pos: int,
             scale: float, stream=None) -> None:
    """Enqueue the prefill attention forward (see include/ta03.h)."""
    qd, kvd = num_heads * head_dim, num_kv_heads * head_dim
    kv_rows_needed = kv_len if mode != CAUSAL else min(kv_len, start_pos + q_seq)
    status = lib().attn_fwd(
        _ptr(q, q_seq * qd, "q"), _ptr(k, kv_rows_needed * kvd, "k"),
        _ptr(v, kv_rows_needed * kvd, "v"), _ptr(out, q_seq * qd, "out"),
        _ptr(lse, q_seq * num_heads * 2, "lse"), q_seq, kv_len, num_heads, num_kv_heads,
        head_dim, mode, start_pos, float(scale), _stream(stream))
    _check(status)


def _strided_ptr(t, extent: int, name: str):
    """Device pointer of a (possibly strided) float32 view whose first
    `extent` elements from its start must lie inside its storage."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    import torch
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32, got {t.dtype}")
    if extent <= 0:
        return t.data_ptr() if t.numel() > 0 else None
    avail = t.untyped_storage().nbytes() // 4 - t.storage_offset()
    if extent > avail:
        raise ValueError(f"{name}: {extent} elements needed from its start, storage holds {avail}")
    return t.data_ptr()


def attn_fwd_ex(q, q_stride: int, k, k_stride: int, v, v_stride: int, out, out_stride: int,
                lse, q_base: int, q_seq: int, kv_len: int, num_heads: int, num_kv_heads: int,
                head_dim: int, mode: int, start_pos: int, scale: float, stream=None) -> None:
    """Enqueue the prefill over strided rows and a sub-batch (see
    include/ta03.h). Tensors may be strided views (e.g. column slices of a
    fused QKV buffer); strides are in floats between rows."""
    qd, kvd = num_heads * head_dim, num_kv_heads * head_dim
    rows = q_base + q_seq
    kv_rows = kv_len if mode != CAUSAL else min(kv_len, start_pos + rows)
    def ext(n, stride, width):
        return (n - 1) * stride + width if n > 0 else 0
    status = lib().attn_fwd_ex(
        _strided_ptr(q, ext(rows, q_stride, qd), "q"), int(q_stride),
        _strided_ptr(k, ext(kv_rows, k_stride, kvd), "k"), int(k_stride),
        _strided_ptr(v, ext(kv_rows, v_stride, kvd), "v"), int(v_stride),
        _strided_ptr(out, ext(rows, out_stride, qd), "out"), int(out_stride),
        _ptr(lse, rows * num_heads * 2, "lse"), q_base, q_seq, kv_len, num_heads,
        num_kv_heads, head_dim, mode, start_pos, float(scale), _stream(stream))
    _check(status)


def _fwd_rope(fn, q, q_stride, k, k_stride, v, v_stride, out, out_stride, lse, q_base, q_seq,
              kv_len, num_heads, num_kv_heads, head_dim, mode, start_pos, scale, rope_cs,
              rope_rows, stream):
    qd, kvd = num_heads * head_dim, num_kv_heads * head_dim
    rows = q_base + q_seq
    kv_rows = kv_len if mode != CAUSAL else min(kv_len, start_pos + rows)
    def ext(n, stride, width):
        return (n - 1) * stride + width if n > 0 else 0
    status = fn(
        _strided_ptr(q, ext(rows, q_stride, qd), "q"), int(q_stride),
        _strided_ptr(k, ext(kv_rows, k_stride, kvd), "k"), int(k_stride),
        _strided_ptr(v, ext(kv_rows, v_stride, kvd), "v"), int(v_stride),
        _strided_ptr(out, ext(rows, out_stride, qd), "out"), int(out_stride),
        _ptr(lse, rows * num_heads * 2, "lse"), q_base, q_seq, kv_len, num_heads,
        num_kv_heads, head_dim, mode, start_pos, float(scale),
        _ptr(rope_cs, max(rope_rows, 0) * head_dim, "rope_cs"), int(rope_rows), _stream(stream))
    _check(status)


def attn_fwd_rope(q, q_stride: int, k, k_stride: int, v, v_stride: int, out, out_stride: int,
                  lse, q_base: int, q_seq: int, kv_len: int, num_heads: int, num_kv_heads: int,
                  head_dim: int, mode: int, start_pos: int, scale: float, rope_cs,
                  rope_rows: int, stream=None) -> None:
    """Enqueue attn_fwd_ex with the rotary embedding turned into q and k at
    load time (see include/ta03.h); rope_cs is a [rope_rows, head_dim/2, 2]
    float32 GPU tensor of (cos, sin) pairs."""
    _fwd_rope(lib().attn_fwd_rope, q, q_stride, k, k_stride, v, v_stride, out, out_stride, lse,
              q_base, q_seq, kv_len, num_heads, num_kv_heads, head_dim, mode, start_pos, scale,
              rope_cs, rope_rows, stream)


def attn_fwd_rope_q(q, q_stride: int, k, k_stride: int, v, v_stride: int, out, out_stride: int,
                    lse, q_base: int, q_seq: int, kv_len: int, num_heads: int, num_kv_heads: int,
                    head_dim: int, mode: int, start_pos: int, scale: float, rope_cs,
                    rope_rows: int, stream=None) -> None:
    """attn_fwd_rope for keys already turned (see include/ta03.h): only the
    queries are turned at load time."""
    _fwd_rope(lib().attn_fwd_rope_q, q, q_stride, k, k_stride, v, v_stride, out, out_stride,
              lse, q_base, q_seq, kv_len, num_heads, num_kv_heads, head_dim, mode, start_pos,
              scale, rope_cs, rope_rows, stream)


def attn_rope_apply(x, x_stride: int, y, y_stride: int, rows: int, heads: int, head_dim: int,
                    pos0: int, rope_cs, rope_rows: int, stream=None) -> None:
    """Enqueue the rotation of rows [0, rows) of x into y at positions
    pos0 + r (see include/ta03.h); x and y may be strided views, or the
    same tensor (in place)."""
    width = heads * head_dim
    def ext(n, stride):
        return (n - 1) * stride + width if n > 0 else 0
    _check(lib().attn_rope_apply(
        _strided_ptr(x, ext(rows, x_stride), "x"), int(x_stride),
        _strided_ptr(y, ext(rows, y_stride), "y"), int(y_stride), int(rows), int(heads),
        int(head_dim), int(pos0), _ptr(rope_cs, max(rope_rows, 0) * head_dim, "rope_cs"),
        int(rope_rows), _stream(stream)))


def attn_rope_table(cos_sin, rows: int, head_dim: int, theta: float, stream=None) -> None:
    """Enqueue the fill of a standard rotary table [rows, head_dim/2, 2]."""
    _check(lib().attn_rope_table(_ptr(cos_sin, max(rows, 0) * head_dim, "cos_sin"), int(rows),
                                 int(head_dim), float(theta), _stream(stream)))


def attn_bwd_workspace_bytes(q_seq: int, num_heads: int) -> int:
    return int(lib().attn_bwd_workspace_bytes(q_seq, num_heads))


def attn_bwd_workspace_bytes_stored(q_seq: int, kv_len: int, num_heads: int, mode: int,
                                    start_pos: int = 0) -> int:
    return int(lib().attn_bwd_workspace_bytes_stored(q_seq, kv_len, num_heads, mode, start_pos))


def attn_bwd_windows(q_seq: int, kv_len: int, num_heads: int, mode: int, start_pos: int,
                     workspace_bytes: int) -> int:
    return int(lib().attn_bwd_windows(q_seq, kv_len, num_heads, mode, start_pos,
                                      workspace_bytes))


def attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, q_seq: int, kv_len: int, num_heads: int,
             num_kv_heads: int, head_dim: int, mode: int, start_pos: int, scale: float,
             workspace, workspace_bytes: int, stream=None) -> None:
    """Enqueue the attention backward (see include/ta03.h): dq, dk, dv from
    the forward's inputs, its out and lse, and dout."""
    qn = q_seq * num_heads * head_dim
    kn = kv_len * num_kv_heads * head_dim
    wsp = _workspace_ptr(workspace, workspace_bytes)
    _check(lib().attn_bwd(
        _ptr(q, qn, "q"), _ptr(k, kn, "k"), _ptr(v, kn, "v"), _ptr(out, qn, "out"),
        _ptr(dout, qn, "dout"), _ptr(lse, q_seq * num_heads * 2, "lse"), _ptr(dq, qn, "dq"),
        _ptr(dk, kn, "dk"), _ptr(dv, kn, "dv"), q_seq, kv_len, num_heads, num_kv_heads,
        head_dim, mode, start_pos, float(scale), wsp, int(workspace_bytes), _stream(stream)))


def attention_backward(q, k, v, out, dout, lse, *, num_heads: int, num_kv_heads: int,
                       head_dim: int, mode: int, kv_len: Optional[int] = None,
                       start_pos: int = 0, scale: Optional[float] = None,
                       store_scores: bool = True, max_workspace_bytes: Optional[int] = None,
                       stream=None):
    """Allocate dq, dk, dv and the scratch with torch and call attn_bwd;
    returns (dq, dk, dv) with dk, dv of kv_len rows. store_scores sizes the
    scratch for the stored-dS path (4 bytes per (row, key) pair per head);
    False gives the minimal scratch (dq recomputes the scores).
    max_workspace_bytes caps the stored path's scratch (never below the
    minimal one): the library then runs it in windows of query rows, or
    recomputes when the cap is too small for that (attn_bwd_windows)."""
    import torch
    q_seq = q.shape[0]
    if kv_len is None:
        kv_len = k.shape[0]
    if scale is None:
        scale = head_dim ** -0.5
    dev = q.device
    s = _alloc_stream(stream)
    minimal = attn_bwd_workspace_bytes(q_seq, num_heads)
    nbytes = (attn_bwd_workspace_bytes_stored(q_seq, kv_len, num_heads, mode, start_pos)
              if store_scores else 0) or minimal
    if max_workspace_bytes is not None:
        nbytes = max(min(nbytes, int(max_workspace_bytes)), minimal)
    # Outputs and scratch belong to the stream the kernels run on: the scratch
    # is dropped on return while the kernels may still be running.
    with torch.cuda.stream(s):
        dq = torch.empty((q_seq, num_heads * head_dim), dtype=torch.float32, device=dev)
        dk = torch.empty((kv_len, num_kv_heads * head_dim), dtype=torch.float32, device=dev)
        dv = torch.empty((kv_len, num_kv_heads * head_dim), dtype=torch.float32, device=dev)
        ws = torch.empty((max(nbytes, 4) // 4,), dtype=torch.float32, device=dev)
    attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, q_seq, kv_len, num_heads, num_kv_heads,
             head_dim, mode, start_pos, scale, ws, nbytes, s)
    return dq, dk, dv


def attn_decode_workspace_bytes(num_heads: int, num_kv_heads: int, head_dim: int,
                                max_seq: int) -> int:
    return int(lib().attn_decode_workspace_bytes(num_heads, num_kv_heads, head_dim, max_seq))


def attn_decode_workspace_init(workspace, workspace_bytes: int, num_heads: int,
                               num_kv_heads: int, head_dim: int, max_seq: int,
                               stream=None) -> None:
    """Enqueue the zero fill of a decode workspace's completion counters."""
    wsp = _workspace_ptr(workspace, workspace_bytes)
    _check(lib().attn_decode_workspace_init(wsp, int(workspace_bytes), num_heads,
                                            num_kv_heads, head_dim, max_seq, _stream(stream)))


def _workspace_ptr(workspace, workspace_bytes):
    import torch
    if isinstance(workspace, torch.Tensor):
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")
        if workspace.numel() * workspace.element_size() < workspace_bytes:
            raise ValueError("workspace tensor smaller than workspace_bytes")
        return workspace.data_ptr()
    return workspace


def attn_decode(q, k_cache, v_cache, kv_pos, out, lse, num_heads: int, num_kv_heads: int,
                head_dim: int, max_seq: int, scale: float, workspace,
                workspace_bytes: int, stream=None) -> None:
    """Enqueue the single-token decode (see include/ta03.h). ``kv_pos`` is a
    one-element int32/uint32 GPU tensor; ``workspace`` a GPU tensor of at
    least ``workspace_bytes`` bytes, zero-filled before its first use
    (``attn_decode_workspace_init``); calls leave it reusable."""
    import torch
    qd, kvd = num_heads * head_dim, num_kv_heads * head_dim
    if isinstance(kv_pos, torch.Tensor):
        kvp = _ptr(kv_pos, 1, "kv_pos",
                   dtype_name="int32" if kv_pos.dtype == torch.int32 else "uint32")
    else:
        kvp = kv_pos
    wsp = _workspace_ptr(workspace, workspace_bytes)
    status = lib().attn_decode(
        _ptr(q, qd, "q"), _ptr(k_cache, max_seq * kvd, "k_cache"),
        _ptr(v_cache, max_seq * kvd, "v_cache"), kvp, _ptr(out, qd, "out"),
        _ptr(lse, num_heads * 2, "lse"), num_heads, num_kv_heads, head_dim, max_seq,
        float(scale), wsp, int(workspace_bytes), _stream(stream))
    _check(status)


def attn_decode_noalloc(q, k_cache, v_cache, kv_pos, out, lse, num_heads: int,
                        num_kv_heads: int, head_dim: int, max_seq: int, scale: float,
                        stream=None) -> None:
    """Enqueue the single-token decode without a workspace: the library's own
    fixed device scratch holds the split partials (see include/ta03.h)."""
    import torch
    qd, kvd = num_heads * head_dim, num_kv_heads * head_dim
    kvp = _ptr(kv_pos, 1, "kv_pos",
               dtype_name="int32" if kv_pos.dtype == torch.int32 else "uint32") \
        if isinstance(kv_pos, torch.Tensor) else kv_pos
    status = lib().attn_decode_noalloc(
        _ptr(q, qd, "q"), _ptr(k_cache, max_seq * kvd, "k_cache"),
        _ptr(v_cache, max_seq * kvd, "v_cache"), kvp, _ptr(out, qd, "out"),
        _ptr(lse, num_heads * 2, "lse"), num_heads, num_kv_heads, head_dim, max_seq,
        float(scale), _stream(stream))
    _check(status)


def attn_decode_paged(q, k_pool, v_pool, num_pages: int, page_size: int, block_table, kv_pos,
                      out, lse, num_heads: int, num_kv_heads: int, head_dim: int, max_seq: int,
                      scale: float, workspace, workspace_bytes: int, stream=None) -> None:
    """Enqueue the decode over a paged cache (see include/ta03.h).
    ``block_table`` is an int32 GPU tensor of ceil(max_seq / page_size)
    entries; the pools hold num_pages * page_size rows."""
    import torch
    qd, kvd = num_heads * head_dim, num_kv_heads * head_dim
    kvp = _ptr(kv_pos, 1, "kv_pos",
               dtype_name="int32" if kv_pos.dtype == torch.int32 else "uint32") \
        if isinstance(kv_pos, torch.Tensor) else kv_pos
    nblk = -(-max_seq // page_size) if page_size > 0 else 0
    tbl = _ptr(block_table, nblk, "block_table", dtype_name="int32") \
        if isinstance(block_table, torch.Tensor) else block_table
    wsp = _workspace_ptr(workspace, workspace_bytes)
    status = lib().attn_decode_paged(
        _ptr(q, qd, "q"), _ptr(k_pool, num_pages * page_size * kvd, "k_pool"),
        _ptr(v_pool, num_pages * page_size * kvd, "v_pool"), num_pages, page_size, tbl, kvp,
        _ptr(out, qd, "out"), _ptr(lse, num_heads * 2, "lse"), num_heads, num_kv_heads,
        head_dim, max_seq, float(scale), wsp, int(workspace_bytes), _stream(stream))
    _check(status)


def attention(q, k, v, *, num_heads: int, num_kv_heads: int, head_dim: int, mode: int,
              kv_len: Optional[int] = None, start_pos: int = 0, scale: Optional[float] = None,
              with_lse: bool = True, stream=None):
    """Allocate out (and lse) with torch and call attn_fwd; returns (out, lse)."""
    import torch
    q_seq = q.shape[0]
    if kv_len is None:
        kv_len = k.shape[0]
    if scale is None:
        scale = head_dim ** -0.5
    s = _alloc_stream(stream)
    with torch.cuda.stream(s):
        out = torch.empty((q_seq, num_heads * head_dim), dtype=torch.float32, device=q.device)
        lse = (torch.empty((q_seq, num_heads, 2), dtype=torch.float32, device=q.device)
               if with_lse else None)
    attn_fwd(q, k, v, out, lse, q_seq, kv_len, num_heads, num_kv_heads, head_dim, mode,
             start_pos, scale, s)
    return out, lse
