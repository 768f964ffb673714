"""Thin Python binding of libbb_attn.so (ctypes).

Same names as the C ABI in include/bb_attn.h.  This module only marshals
arguments (torch tensors -> device pointers, the current HIP stream, numpy
buffers for host tables) and turns nonzero status codes into RuntimeError.
Every step of the attention runs in the library's HIP kernels; there is no
fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libbb_attn.so")

BB_OK = 0
BB_FP32 = 0
BB_BF16 = 1
BB_LAUNCH_FUSED = 0
BB_LAUNCH_SPLIT = 1
BB_PHASE_UNITS = 2
BB_PHASE_MERGE = 4
STATUS_NAMES = {0: "BB_OK", 1: "BB_ERR_NULL", 2: "BB_ERR_SHAPE", 3: "BB_ERR_DTYPE",
                4: "BB_ERR_RAND_IDX", 5: "BB_ERR_WORKSPACE", 6: "BB_ERR_HIP",
                7: "BB_ERR_ALIAS", 8: "BB_ERR_ALIGN"}

# Every symbol include/bb_attn.h declares.
EXPORTS = ("bb_abi_version", "bb_status_str", "bb_rand_idx_build", "bb_rand_idx_build_capped",
           "bb_rand_idx_check",
           "bb_attn_workspace_bytes", "bb_attn_forward", "bb_attn_forward_ex",
           "bb_attn_forward_timed", "bb_attn_forward_lse", "bb_rand_idx_invert",
           "bb_attn_backward_workspace_bytes", "bb_attn_backward", "bb_layer_workspace_bytes",
           "bb_layer_forward")

_lib = None


class BBError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({bb_status_str(status)})")


def lib():
    """Load libbb_attn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m block_sparse_long_bigbird_amd.build` (hipcc, gfx950)")
    # torch ships its own HIP runtime under the same soname.  Loaded first, it
    # is the one the library binds to, so torch's streams and memory and the
    # library's launches share one runtime; loaded after the library, the
    # process would map two runtimes and the library's launches on torch's
    # streams would fail.
    import torch  # noqa: F401
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_size, c_u64, vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_uint64, ctypes.c_void_p
    L.bb_abi_version.restype = c_int
    L.bb_abi_version.argtypes = []
    L.bb_status_str.restype = ctypes.c_char_p
    L.bb_status_str.argtypes = [c_int]
    L.bb_rand_idx_build.restype = c_int
    L.bb_rand_idx_build.argtypes = [c_u64, c_int, c_int, c_int, c_int, vp]
    L.bb_rand_idx_build_capped.restype = c_int
    L.bb_rand_idx_build_capped.argtypes = [c_u64, c_int, c_int, c_int, c_int, c_int, vp]
    L.bb_rand_idx_check.restype = c_int
    L.bb_rand_idx_check.argtypes = [vp, c_int, c_int, c_int, c_int]
    L.bb_attn_workspace_bytes.restype = c_size
    L.bb_attn_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    fwd = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, vp, c_int, vp, c_size, vp]
    L.bb_attn_forward.restype = c_int
    L.bb_attn_forward.argtypes = fwd
    L.bb_attn_forward_ex.restype = c_int
    L.bb_attn_forward_ex.argtypes = fwd + [ctypes.c_uint]
    L.bb_attn_forward_timed.restype = c_int
    L.bb_attn_forward_timed.argtypes = fwd + [ctypes.c_uint, vp, vp]
    L.bb_attn_forward_lse.restype = c_int
    L.bb_attn_forward_lse.argtypes = fwd + [vp]
    L.bb_rand_idx_invert.restype = c_int
    L.bb_rand_idx_invert.argtypes = [vp, c_int, c_int, c_int, c_int, vp, vp]
    L.bb_attn_backward_workspace_bytes.restype = c_size
    L.bb_attn_backward_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    L.bb_attn_backward.restype = c_int
    L.bb_attn_backward.argtypes = ([vp, vp, vp, vp, vp, vp, vp] + [c_int] * 6 +
                                   [vp, vp, vp, vp, vp, vp, c_int, vp, c_size, vp])
    L.bb_layer_workspace_bytes.restype = c_size
    L.bb_layer_workspace_bytes.argtypes = [c_int] * 5
    L.bb_layer_forward.restype = c_int
    L.bb_layer_forward.argtypes = [vp] * 7 + [c_int] * 6 + [vp, c_int, vp, c_size, vp]
    _lib = L
    return L


def bb_abi_version() -> int:
    return lib().bb_abi_version()


def bb_status_str(status: int) -> str:
    return lib().bb_status_str(int(status)).decode()


def bb_rand_idx_build(seed: int, H: int, L: int, block: int, r: int) -> np.ndarray:
    """Host random-block table, int32 [H, L/block - 2, r]."""
    nb = L // block if block > 0 else 0
    out = np.zeros((max(H, 0), max(nb - 2, 0), max(r, 0)), dtype=np.int32)
    st = lib().bb_rand_idx_build(ctypes.c_uint64(seed & (2**64 - 1)), H, L, block, r,
                                 out.ctypes.data if out.size else None)
    if st != BB_OK:
        raise BBError(st, "bb_rand_idx_build")
    return out


def bb_rand_idx_build_capped(seed: int, H: int, L: int, block: int, r: int, last_idx: int) -> np.ndarray:
    """Host random-block table with the random range capped at token last_idx."""
    nb = L // block if block > 0 else 0
    out = np.zeros((max(H, 0), max(nb - 2, 0), max(r, 0)), dtype=np.int32)
    st = lib().bb_rand_idx_build_capped(ctypes.c_uint64(seed & (2**64 - 1)), H, L, block, r, last_idx,
                                        out.ctypes.data if out.size else None)
    if st != BB_OK:
        raise BBError(st, "bb_rand_idx_build_capped")
    return out


def bb_rand_idx_check(rand_idx, H: int, L: int, block: int, r: int) -> int:
    """Status of the C checker on a host table (BB_OK or an error code)."""
    a = np.ascontiguousarray(np.asarray(rand_idx), dtype=np.int32)
    return lib().bb_rand_idx_check(a.ctypes.data if a.size else None, H, L, block, r)


def bb_attn_workspace_bytes(B: int, H: int, L: int, d: int, block: int) -> int:
    return int(lib().bb_attn_workspace_bytes(B, H, L, d, block))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BB_BF16
    if t.dtype == torch.float32:
        return BB_FP32
    return 99  # the library reports BB_ERR_DTYPE


def _stream_handle(t, stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def alloc_workspace(B: int, H: int, L: int, d: int, block: int, device):
    """Device workspace of the size the library asks for (contents need no initialisation)."""
    import torch
    n = bb_attn_workspace_bytes(B, H, L, d, block)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _check_device_tensor(name, t):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def bb_attn_forward(q, k, v, pad_mask, rand_idx, B: int, H: int, L: int, d: int, block: int,
                    r: int, out, workspace, stream=None, flags: int = BB_LAUNCH_FUSED,
                    events=None) -> None:
    """Enqueue the forward on `stream` (default: torch's current stream).

    q, k, v, out: device tensors [B, H, L, d] (bf16 or fp32); pad_mask: uint8
    device tensor [B, L] or None; rand_idx: int32 device tensor [H, L/block-2, r]
    (or None when r == 0); workspace: uint8 device tensor from alloc_workspace.
    events: optional (start, stop) pair of timing-enabled torch.cuda.Event that
    the kernel launches themselves record (bb_attn_forward_timed); each must
    have been recorded once before, so that its HIP event exists.
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("pad_mask", pad_mask),
                    ("rand_idx", rand_idx), ("workspace", workspace)):
        _check_device_tensor(name, t)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if events is None:
        st = lib().bb_attn_forward_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(pad_mask), _ptr(rand_idx),
                                      B, H, L, d, block, r, _ptr(out), _dtype_code(q),
                                      _ptr(workspace), ws_bytes, _stream_handle(q, stream), flags)
    else:
        e0, e1 = (int(e.cuda_event) for e in events)
        if not e0 or not e1:
            raise ValueError("events must have been recorded once (their HIP events do not exist yet)")
        st = lib().bb_attn_forward_timed(_ptr(q), _ptr(k), _ptr(v), _ptr(pad_mask), _ptr(rand_idx),
                                         B, H, L, d, block, r, _ptr(out), _dtype_code(q),
                                         _ptr(workspace), ws_bytes, _stream_handle(q, stream), flags,
                                         e0, e1)
    if st != BB_OK:
        raise BBError(st, "bb_attn_forward")


def forward(q, k, v, rand_idx, pad_mask=None, block: int = 64, out=None, workspace=None,
            stream=None, flags: int = BB_LAUNCH_FUSED):
    """Convenience wrapper: sizes from q's shape, allocates out/workspace if not given."""
    import torch
    B, H, L, d = q.shape
    r = 0 if rand_idx is None else int(rand_idx.shape[-1])
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(B, H, L, d, block, q.device)
    bb_attn_forward(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, workspace,
                    stream=stream, flags=flags)
    return out


def bb_attn_forward_lse(q, k, v, pad_mask, rand_idx, B: int, H: int, L: int, d: int, block: int,
                        r: int, out, workspace, lse, stream=None) -> None:
    """The forward that also writes the row log-sum-exp: lse is a float32
    device tensor [B, H, L] (natural log)."""
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("pad_mask", pad_mask),
                    ("rand_idx", rand_idx), ("workspace", workspace), ("lse", lse)):
        _check_device_tensor(name, t)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().bb_attn_forward_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(pad_mask), _ptr(rand_idx),
                                   B, H, L, d, block, r, _ptr(out), _dtype_code(q),
                                   _ptr(workspace), ws_bytes, _stream_handle(q, stream), _ptr(lse))
    if st != BB_OK:
        raise BBError(st, "bb_attn_forward_lse")


def bb_rand_idx_invert(rand_idx, H: int, L: int, block: int, r: int):
    """Host inverse of a random-block table: (inv_off int32 [H, nb+1],
    inv_rows int32 [H * (nb-2) * r])."""
    nb = L // block if block > 0 else 0
    a = np.ascontiguousarray(np.asarray(rand_idx), dtype=np.int32)
    off = np.zeros((max(H, 0), max(nb + 1, 0)), dtype=np.int32)
    rows = np.zeros(max(H * max(nb - 2, 0) * max(r, 0), 0), dtype=np.int32)
    st = lib().bb_rand_idx_invert(a.ctypes.data if a.size else None, H, L, block, r,
                                  off.ctypes.data if off.size else None,
                                  rows.ctypes.data if rows.size else None)
    if st != BB_OK:
        raise BBError(st, "bb_rand_idx_invert")
    return off, rows


def bb_attn_backward_workspace_bytes(B: int, H: int, L: int, d: int, block: int) -> int:
    return int(lib().bb_attn_backward_workspace_bytes(B, H, L, d, block))


def bb_attn_backward(q, k, v, pad_mask, rand_idx, inv_off, inv_rows, B: int, H: int, L: int,
                     d: int, block: int, r: int, out, dout, lse, dq, dk, dv, workspace,
                     stream=None) -> None:
    """Enqueue the backward on `stream` (default: torch's current stream).
    inv_off / inv_rows: int32 device tensors from bb_rand_idx_invert."""
    for name, t in (("q", q), ("k", k), ("v", v), ("pad_mask", pad_mask), ("rand_idx", rand_idx),
                    ("inv_off", inv_off), ("inv_rows", inv_rows), ("out", out), ("dout", dout),
                    ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("workspace", workspace)):
        _check_device_tensor(name, t)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().bb_attn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(pad_mask), _ptr(rand_idx),
                                _ptr(inv_off), _ptr(inv_rows), B, H, L, d, block, r, _ptr(out),
                                _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                _dtype_code(q), _ptr(workspace), ws_bytes,
                                _stream_handle(q, stream))
    if st != BB_OK:
        raise BBError(st, "bb_attn_backward")


def bb_layer_workspace_bytes(B: int, L: int, hidden: int, H: int, block: int) -> int:
    return int(lib().bb_layer_workspace_bytes(B, L, hidden, H, block))


def bb_layer_forward(x, w_qkv, b_qkv, w_o, b_o, pad_mask, rand_idx, B: int, L: int, hidden: int, H: int,
                     block: int, r: int, y, workspace, stream=None) -> None:
    """Enqueue the attention layer (projections + block-sparse attention)."""
    for name, t in (("x", x), ("w_qkv", w_qkv), ("b_qkv", b_qkv), ("w_o", w_o), ("b_o", b_o),
                    ("pad_mask", pad_mask), ("rand_idx", rand_idx), ("y", y), ("workspace", workspace)):
        _check_device_tensor(name, t)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().bb_layer_forward(_ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_o), _ptr(b_o), _ptr(pad_mask),
                                _ptr(rand_idx), B, L, hidden, H, block, r, _ptr(y), _dtype_code(x),
                                _ptr(workspace), ws_bytes, _stream_handle(x, stream))
    if st != BB_OK:
        raise BBError(st, "bb_layer_forward")
