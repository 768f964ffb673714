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
BB_QUERY_MASK = 8
BB_ORDINARY_UNITS = 16
STATUS_NAMES = {0: "BB_OK", 1: "BB_ERR_NULL", 2: "BB_ERR_SHAPE", 3: "BB_ERR_DTYPE",
                4: "BB_ERR_RAND_IDX", 5: "BB_ERR_WORKSPACE", 6: "BB_ERR_HIP",
                7: "BB_ERR_ALIAS", 8: "BB_ERR_ALIGN"}

# Every symbol include/bb_attn.h declares.
EXPORTS = ("bb_abi_version", "bb_status_str", "bb_rand_idx_build", "bb_rand_idx_build_capped",
           "bb_rand_idx_check",
           "bb_attn_workspace_bytes", "bb_attn_forward", "bb_attn_forward_ex",
           "bb_attn_forward_timed", "bb_attn_forward_lse", "bb_rand_idx_invert",
           "bb_attn_backward_workspace_bytes", "bb_attn_backward", "bb_layer_workspace_bytes",
           "bb_layer_forward", "bb_attn_forward_noalloc", "bb_layer_stack_workspace_bytes",
           "bb_layer_stack_forward", "bb_attn_forward_plan", "bb_attn_forward_lse_ex",
           "bb_attn_backward_ex")

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
    L.bb_attn_forward_plan.restype = c_int
    L.bb_attn_forward_plan.argtypes = [c_int] * 7 + [ctypes.c_uint, ctypes.POINTER(ctypes.c_longlong),
                                                    ctypes.POINTER(c_int)]
    fwd = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, vp, c_int, vp, c_size, vp]
    L.bb_attn_forward.restype = c_int
    L.bb_attn_forward.argtypes = fwd
    L.bb_attn_forward_ex.restype = c_int
    L.bb_attn_forward_ex.argtypes = fwd + [ctypes.c_uint]
    L.bb_attn_forward_timed.restype = c_int
    L.bb_attn_forward_timed.argtypes = fwd + [ctypes.c_uint, vp, vp]
    L.bb_attn_forward_lse.restype = c_int
    L.bb_attn_forward_lse.argtypes = fwd + [vp]
    L.bb_attn_forward_lse_ex.restype = c_int
    L.bb_attn_forward_lse_ex.argtypes = fwd + [vp, ctypes.c_uint]
    L.bb_attn_forward_noalloc.restype = c_int
    L.bb_attn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, c_int, c_int, c_int, c_int, c_int, c_int, vp, c_int, vp]
    L.bb_rand_idx_invert.restype = c_int
    L.bb_rand_idx_invert.argtypes = [vp, c_int, c_int, c_int, c_int, vp, vp]
    L.bb_attn_backward_workspace_bytes.restype = c_size
    L.bb_attn_backward_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int]
    L.bb_attn_backward.restype = c_int
    L.bb_attn_backward.argtypes = ([vp, vp, vp, vp, vp, vp, vp] + [c_int] * 6 +
                                   [vp, vp, vp, vp, vp, vp, c_int, vp, c_size, vp])
    L.bb_attn_backward_ex.restype = c_int
    L.bb_attn_backward_ex.argtypes = L.bb_attn_backward.argtypes + [ctypes.c_uint]
    L.bb_layer_workspace_bytes.restype = c_size
    L.bb_layer_workspace_bytes.argtypes = [c_int] * 5
    L.bb_layer_forward.restype = c_int
    L.bb_layer_forward.argtypes = [vp] * 7 + [c_int] * 6 + [vp, c_int, vp, c_size, vp]
    L.bb_layer_stack_workspace_bytes.restype = c_size
    L.bb_layer_stack_workspace_bytes.argtypes = [c_int] * 5
    L.bb_layer_stack_forward.restype = c_int
    L.bb_layer_stack_forward.argtypes = [vp] * 7 + [c_int] * 7 + [vp, c_int, vp, c_size, vp]
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
    _check_built(out, H, L, block, r)
    return out


def _check_built(table, H, L, block, r):
    """Every table the binding builds goes through the checker too."""
    st = bb_rand_idx_check(table, H, L, block, r)
    if st != BB_OK:
        raise BBError(st, "bb_rand_idx_check")


def bb_rand_idx_build_capped(seed: int, H: int, L: int, block: int, r: int, last_idx: int) -> np.ndarray:
    """Host random-block table with the random range capped at token last_idx."""
    nb = L // block if block > 0 else 0
    out = np.zeros((max(H, 0), max(nb - 2, 0), max(r, 0)), dtype=np.int32)
    st = lib().bb_rand_idx_build_capped(ctypes.c_uint64(seed & (2**64 - 1)), H, L, block, r, last_idx,
                                        out.ctypes.data if out.size else None)
    if st != BB_OK:
        raise BBError(st, "bb_rand_idx_build_capped")
    _check_built(out, H, L, block, r)
    return out


def bb_rand_idx_check(rand_idx, H: int, L: int, block: int, r: int) -> int:
    """Status of the C checker on a host table (BB_OK or an error code)."""
    a = np.ascontiguousarray(np.asarray(rand_idx), dtype=np.int32)
    return lib().bb_rand_idx_check(a.ctypes.data if a.size else None, H, L, block, r)


def bb_attn_workspace_bytes(B: int, H: int, L: int, d: int, block: int) -> int:
    return int(lib().bb_attn_workspace_bytes(B, H, L, d, block))


def bb_attn_forward_plan(B: int, H: int, L: int, d: int, block: int, r: int, dtype: str,
                         flags: int = BB_LAUNCH_FUSED):
    """(work units, small-problem split used) of a forward call of these sizes;
    dtype "bf16" or "fp32"."""
    n, small = ctypes.c_longlong(0), ctypes.c_int(0)
    st = lib().bb_attn_forward_plan(B, H, L, d, block, r, BB_BF16 if dtype == "bf16" else BB_FP32, flags,
                                    ctypes.byref(n), ctypes.byref(small))
    if st != BB_OK:
        raise BBError(st, "bb_attn_forward_plan")
    return int(n.value), bool(small.value)


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


# ----------------------------------------------------------------- checks ---
# The C ABI takes raw pointers, so a tensor of the wrong dtype or shape would be
# read or written past its end.  Every wrapper below checks what the pointers
# stand for against the sizes it passes, before anything reaches the library:
# a mismatch raises ValueError and nothing is launched.

def _expect(name, t, shape, dtypes):
    """t must have exactly `shape` and one of `dtypes` (torch dtypes)."""
    if t is None:
        raise ValueError(f"{name} is required")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        names = " or ".join(str(d) for d in dtypes)
        raise ValueError(f"{name} has dtype {t.dtype}, expected {names}")


def _same_dtype_as(first, t_name_pairs):
    for name, t in t_name_pairs:
        if t is not None and t.dtype != first.dtype:
            raise ValueError(f"{name} has dtype {t.dtype}, but q has {first.dtype}: "
                             "q, k, v and the outputs share one dtype")


def _check_pad_and_table(pad_mask, rand_idx, B, H, L, block, r):
    """pad_mask: None or uint8/bool [B, L]; rand_idx: int32 [H, L/block - 2, r]
    (None only when r == 0).  Returns True when the table's contents are to be
    checked too (_check_table_contents, after the device checks)."""
    import torch
    if pad_mask is not None:
        _expect("pad_mask", pad_mask, (B, L), (torch.uint8, torch.bool))
    if block <= 0 or L % block != 0 or L // block < 3 or r < 0:
        return False                     # sizes the library rejects (BB_ERR_SHAPE)
    nb = L // block
    if rand_idx is None:
        if r > 0 and B * H > 0:
            raise ValueError(f"rand_idx is required when r = {r} > 0")
        return False
    _expect("rand_idx", rand_idx, (H, nb - 2, r), (torch.int32,))
    return True


def _check_rand_idx_contents(rand_idx, H, L, block, r):
    """Run the library's table checker (bb_rand_idx_check) on a device table.

    Once per table: the result is remembered on the tensor object together
    with its version counter (bumped by every in-place write through torch),
    so later calls with the same, unmodified table cost nothing.  The first
    check copies the table to the host and synchronises; inside a HIP graph
    capture that is impossible, so an unchecked table raises there (check it
    before capturing: upload_rand_idx, or one eager call).  Returns the host
    copy when it was made (the backward also checks its inverse against it).
    """
    import torch
    key = (rand_idx._version, H, L, block, r)
    if getattr(rand_idx, "_bb_checked", None) == key:
        return None
    if rand_idx.is_cuda and torch.cuda.is_current_stream_capturing():
        raise ValueError("rand_idx has not been checked yet and cannot be copied to the host "
                         "during graph capture: pass it through upload_rand_idx() or one eager "
                         "call before capturing")
    host = rand_idx.detach().to("cpu").numpy()
    st = bb_rand_idx_check(host, H, L, block, r)
    if st != BB_OK:
        raise BBError(st, "bb_rand_idx_check")
    rand_idx._bb_checked = key
    return host


def upload_rand_idx(table, H: int, L: int, block: int, r: int, device):
    """Check a host random-block table with bb_rand_idx_check and copy it to
    `device` as an int32 tensor [H, L/block - 2, r], marked as checked (the
    wrappers below then accept it without copying it back).  None when r == 0."""
    import torch
    a = np.ascontiguousarray(np.asarray(table), dtype=np.int32)
    st = bb_rand_idx_check(a, H, L, block, r)
    if st != BB_OK:
        raise BBError(st, "bb_rand_idx_check")
    if r == 0:
        return None
    t = torch.from_numpy(a).to(device)
    t._bb_checked = (t._version, H, L, block, r)
    return t


def _check_qkv_out(B, H, L, d, q, rest):
    """q, k, v and the outputs: [B, H, L, d], one dtype (q's).  An unsupported q
    dtype is left to the library (BB_ERR_DTYPE)."""
    _expect("q", q, (B, H, L, d), (q.dtype,))
    _same_dtype_as(q, rest)
    for name, t in rest:
        _expect(name, t, (B, H, L, d), (q.dtype,))


def _forward_args(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, workspace, stream):
    """Check the forward's arguments; the library call's argument tuple."""
    _check_qkv_out(B, H, L, d, q, (("k", k), ("v", v), ("out", out)))
    table = _check_pad_and_table(pad_mask, rand_idx, B, H, L, block, r)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("pad_mask", pad_mask),
                    ("rand_idx", rand_idx), ("workspace", workspace)):
        _check_device_tensor(name, t)
    if table:
        _check_rand_idx_contents(rand_idx, H, L, block, r)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(pad_mask), _ptr(rand_idx), B, H, L, d, block, r,
            _ptr(out), _dtype_code(q), _ptr(workspace), ws_bytes, _stream_handle(q, stream))


def bb_attn_forward(q, k, v, pad_mask, rand_idx, B: int, H: int, L: int, d: int, block: int,
                    r: int, out, workspace, stream=None, flags: int = BB_LAUNCH_FUSED,
                    events=None) -> None:
    """Enqueue the forward on `stream` (default: torch's current stream).

    q, k, v, out: device tensors [B, H, L, d] (bf16 or fp32, one dtype);
    pad_mask: uint8 (or bool) device tensor [B, L] or None; rand_idx: int32
    device tensor [H, L/block-2, r] (None when r == 0), checked with
    bb_rand_idx_check once per table; workspace: uint8 device tensor from
    alloc_workspace.
    With the default flags this calls the library's bb_attn_forward; other
    flags go through bb_attn_forward_ex.
    events: optional (start, stop) pair of timing-enabled torch.cuda.Event that
    the kernel launches themselves record (bb_attn_forward_timed); each must
    have been recorded once before, so that its HIP event exists.
    """
    args = _forward_args(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, workspace, stream)
    if events is not None:
        e0, e1 = (int(e.cuda_event) for e in events)
        if not e0 or not e1:
            raise ValueError("events must have been recorded once (their HIP events do not exist yet)")
        st = lib().bb_attn_forward_timed(*args, flags, e0, e1)
    elif flags == BB_LAUNCH_FUSED:
        st = lib().bb_attn_forward(*args)
    else:
        st = lib().bb_attn_forward_ex(*args, flags)
    if st != BB_OK:
        raise BBError(st, "bb_attn_forward")


class PreparedForward:
    """One bb_attn_forward call with its arguments checked once, at
    construction; each call of the object enqueues it again with one ctypes
    call and no Python-side checks.  For loops of small problems, where the
    checks of bb_attn_forward take longer on the host than the kernels on the
    device.  The object keeps its tensors alive; writing new values into them
    between calls is the intended use (a rand_idx rewritten in place is not
    checked again; the kernels clamp every table entry into the sequence)."""

    def __init__(self, q, k, v, pad_mask, rand_idx, B: int, H: int, L: int, d: int, block: int, r: int,
                 out, workspace, stream=None, flags: int = BB_LAUNCH_FUSED):
        self._keep = (q, k, v, pad_mask, rand_idx, out, workspace)
        self._args = _forward_args(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, workspace,
                                   stream)
        if flags == BB_LAUNCH_FUSED:
            self._fn = lib().bb_attn_forward
        else:
            self._args = self._args + (flags,)
            self._fn = lib().bb_attn_forward_ex

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != BB_OK:
            raise BBError(st, "bb_attn_forward")


def forward(q, k, v, rand_idx, pad_mask=None, block: int = 64, out=None, workspace=None,
            stream=None, flags: int = BB_LAUNCH_FUSED):
    """Convenience wrapper: sizes from q's shape, allocates out/workspace if not
    given.  rand_idx may be a host table (numpy, checked and uploaded here) or a
    device tensor."""
    import torch
    B, H, L, d = q.shape
    if rand_idx is not None and not isinstance(rand_idx, torch.Tensor):
        table = np.asarray(rand_idx)
        r = int(table.shape[-1]) if table.ndim == 3 else 0
        rand_idx = upload_rand_idx(table, H, L, block, r, q.device)
    r = 0 if rand_idx is None else int(rand_idx.shape[-1])
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(B, H, L, d, block, q.device)
    bb_attn_forward(q, k, v, pad_mask, rand_idx, B, H, L, d, block, r, out, workspace,
                    stream=stream, flags=flags)
    return out


# Size of the library's own scratch area per GPU (BB_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


def bb_attn_forward_noalloc(q, k, v, pad_mask, rand_idx, B: int, H: int, L: int, d: int, block: int,
                            r: int, out, stream=None) -> None:
    """The forward without a workspace argument (for callers that cannot
    allocate): the split-K partials go to the library's own scratch area on
    the device.  Calls that overlap on one GPU race on that area.  Arguments
    and checks as bb_attn_forward."""
    _check_qkv_out(B, H, L, d, q, (("k", k), ("v", v), ("out", out)))
    table = _check_pad_and_table(pad_mask, rand_idx, B, H, L, block, r)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("pad_mask", pad_mask),
                    ("rand_idx", rand_idx)):
        _check_device_tensor(name, t)
    if table:
        _check_rand_idx_contents(rand_idx, H, L, block, r)
    st = lib().bb_attn_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(pad_mask), _ptr(rand_idx),
                                       B, H, L, d, block, r, _ptr(out), _dtype_code(q),
                                       _stream_handle(q, stream))
    if st != BB_OK:
        raise BBError(st, "bb_attn_forward_noalloc")


def bb_attn_forward_lse(q, k, v, pad_mask, rand_idx, B: int, H: int, L: int, d: int, block: int,
                        r: int, out, workspace, lse, stream=None, flags: int = 0) -> None:
    """The forward that also writes the row log-sum-exp: lse is a float32
    device tensor [B, H, L] (natural log).  flags (BB_QUERY_MASK,
    BB_ORDINARY_UNITS) go through bb_attn_forward_lse_ex."""
    import torch
    _check_qkv_out(B, H, L, d, q, (("k", k), ("v", v), ("out", out)))
    _expect("lse", lse, (B, H, L), (torch.float32,))
    table = _check_pad_and_table(pad_mask, rand_idx, B, H, L, block, r)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("pad_mask", pad_mask),
                    ("rand_idx", rand_idx), ("workspace", workspace), ("lse", lse)):
        _check_device_tensor(name, t)
    if table:
        _check_rand_idx_contents(rand_idx, H, L, block, r)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(pad_mask), _ptr(rand_idx), B, H, L, d, block, r, _ptr(out),
            _dtype_code(q), _ptr(workspace), ws_bytes, _stream_handle(q, stream), _ptr(lse))
    if flags:
        st = lib().bb_attn_forward_lse_ex(*args, flags)
    else:
        st = lib().bb_attn_forward_lse(*args)
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
                     stream=None, flags: int = 0) -> None:
    """Enqueue the backward on `stream` (default: torch's current stream).
    inv_off / inv_rows: int32 device tensors from bb_rand_idx_invert of the same
    table (checked against it once per table, as rand_idx itself).  flags
    (BB_QUERY_MASK, as given to the forward; BB_ORDINARY_UNITS) go through
    bb_attn_backward_ex."""
    import torch
    _check_qkv_out(B, H, L, d, q, (("k", k), ("v", v), ("out", out), ("dout", dout), ("dq", dq),
                                   ("dk", dk), ("dv", dv)))
    _expect("lse", lse, (B, H, L), (torch.float32,))
    table = _check_pad_and_table(pad_mask, rand_idx, B, H, L, block, r)
    _check_inverse_shapes(inv_off, inv_rows, H, L, block, r)
    for name, t in (("q", q), ("k", k), ("v", v), ("pad_mask", pad_mask), ("rand_idx", rand_idx),
                    ("inv_off", inv_off), ("inv_rows", inv_rows), ("out", out), ("dout", dout),
                    ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv), ("workspace", workspace)):
        _check_device_tensor(name, t)
    host = _check_rand_idx_contents(rand_idx, H, L, block, r) if table else None
    _check_inverse(rand_idx, host, inv_off, inv_rows, H, L, block, r)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(pad_mask), _ptr(rand_idx), _ptr(inv_off), _ptr(inv_rows),
            B, H, L, d, block, r, _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
            _dtype_code(q), _ptr(workspace), ws_bytes, _stream_handle(q, stream))
    if flags:
        st = lib().bb_attn_backward_ex(*args, flags)
    else:
        st = lib().bb_attn_backward(*args)
    if st != BB_OK:
        raise BBError(st, "bb_attn_backward")


def _check_inverse_shapes(inv_off, inv_rows, H, L, block, r):
    """inv_off int32 [H, nb+1]; inv_rows int32 [H*(nb-2)*r] (may be None when r == 0)."""
    import torch
    if block <= 0 or L % block != 0 or L // block < 3 or r < 0:
        return
    nb = L // block
    _expect("inv_off", inv_off, (H, nb + 1), (torch.int32,))
    if r > 0 or inv_rows is not None:
        _expect("inv_rows", inv_rows, (H * (nb - 2) * r,), (torch.int32,))


def _check_inverse(rand_idx, host, inv_off, inv_rows, H, L, block, r):
    """inv_off / inv_rows equal to bb_rand_idx_invert of the table: checked once per
    (table, inverse) versions, like the table.  `host`: the table's host copy when
    it was just made."""
    import torch
    if rand_idx is None or inv_off is None or block <= 0 or L % block != 0 or L // block < 3:
        return
    key = (rand_idx._version, inv_off._version, None if inv_rows is None else inv_rows._version,
           H, L, block, r)
    if getattr(inv_off, "_bb_checked", None) == key:
        return
    if inv_off.is_cuda and torch.cuda.is_current_stream_capturing():
        raise ValueError("inv_off / inv_rows have not been checked yet and cannot be copied to the "
                         "host during graph capture: make one eager call before capturing")
    if host is None:
        host = rand_idx.detach().to("cpu").numpy()
    off, rows = bb_rand_idx_invert(host, H, L, block, r)
    if not np.array_equal(inv_off.detach().to("cpu").numpy(), off) or (
            inv_rows is not None and not np.array_equal(inv_rows.detach().to("cpu").numpy(), rows)):
        raise ValueError("inv_off / inv_rows are not bb_rand_idx_invert of rand_idx")
    inv_off._bb_checked = key


def bb_layer_workspace_bytes(B: int, L: int, hidden: int, H: int, block: int) -> int:
    return int(lib().bb_layer_workspace_bytes(B, L, hidden, H, block))


def bb_layer_forward(x, w_qkv, b_qkv, w_o, b_o, pad_mask, rand_idx, B: int, L: int, hidden: int, H: int,
                     block: int, r: int, y, workspace, stream=None) -> None:
    """Enqueue the attention layer (projections + block-sparse attention).
    x, y: bf16 [B, L, hidden]; w_qkv: bf16 [3*hidden, hidden]; b_qkv: float32
    [3*hidden]; w_o: bf16 [hidden, hidden]; b_o: float32 [hidden]."""
    import torch
    _expect("x", x, (B, L, hidden), (x.dtype,))
    _same_dtype_as(x, (("w_qkv", w_qkv), ("w_o", w_o), ("y", y)))
    _expect("w_qkv", w_qkv, (3 * hidden, hidden), (x.dtype,))
    _expect("b_qkv", b_qkv, (3 * hidden,), (torch.float32,))
    _expect("w_o", w_o, (hidden, hidden), (x.dtype,))
    _expect("b_o", b_o, (hidden,), (torch.float32,))
    _expect("y", y, (B, L, hidden), (x.dtype,))
    table = _check_pad_and_table(pad_mask, rand_idx, B, H, L, block, r)
    for name, t in (("x", x), ("w_qkv", w_qkv), ("b_qkv", b_qkv), ("w_o", w_o), ("b_o", b_o),
                    ("pad_mask", pad_mask), ("rand_idx", rand_idx), ("y", y), ("workspace", workspace)):
        _check_device_tensor(name, t)
    if table:
        _check_rand_idx_contents(rand_idx, H, L, block, r)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().bb_layer_forward(_ptr(x), _ptr(w_qkv), _ptr(b_qkv), _ptr(w_o), _ptr(b_o), _ptr(pad_mask),
                                _ptr(rand_idx), B, L, hidden, H, block, r, _ptr(y), _dtype_code(x),
                                _ptr(workspace), ws_bytes, _stream_handle(x, stream))
    if st != BB_OK:
        raise BBError(st, "bb_layer_forward")


def bb_layer_stack_workspace_bytes(B: int, L: int, hidden: int, H: int, block: int) -> int:
    return int(lib().bb_layer_stack_workspace_bytes(B, L, hidden, H, block))


def bb_layer_stack_forward(x, layers, pad_mask, B: int, L: int, hidden: int, H: int, block: int, r: int,
                           y, workspace, stream=None) -> None:
    """Enqueue a stack of attention layers.  layers: a sequence of
    (w_qkv, b_qkv, w_o, b_o, rand_idx) per layer, each as bb_layer_forward
    takes it (rand_idx an int32 device table, None when r == 0)."""
    import torch
    n = len(layers)
    if n < 1:
        raise ValueError("a stack needs at least one layer")
    _expect("x", x, (B, L, hidden), (x.dtype,))
    _expect("y", y, (B, L, hidden), (x.dtype,))
    tables = []
    for i, (w_qkv, b_qkv, w_o, b_o, ri) in enumerate(layers):
        _expect(f"layer {i} w_qkv", w_qkv, (3 * hidden, hidden), (x.dtype,))
        _expect(f"layer {i} b_qkv", b_qkv, (3 * hidden,), (torch.float32,))
        _expect(f"layer {i} w_o", w_o, (hidden, hidden), (x.dtype,))
        _expect(f"layer {i} b_o", b_o, (hidden,), (torch.float32,))
        tables.append(_check_pad_and_table(pad_mask, ri, B, H, L, block, r))
        for name, t in (("w_qkv", w_qkv), ("b_qkv", b_qkv), ("w_o", w_o), ("b_o", b_o), ("rand_idx", ri)):
            _check_device_tensor(f"layer {i} {name}", t)
    for name, t in (("x", x), ("pad_mask", pad_mask), ("y", y), ("workspace", workspace)):
        _check_device_tensor(name, t)
    for (w_qkv, b_qkv, w_o, b_o, ri), table in zip(layers, tables):
        if table:
            _check_rand_idx_contents(ri, H, L, block, r)

    def arr(i):
        return (ctypes.c_void_p * n)(*[layers[j][i].data_ptr() if layers[j][i] is not None else None
                                       for j in range(n)])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().bb_layer_stack_forward(_ptr(x), arr(0), arr(1), arr(2), arr(3), _ptr(pad_mask),
                                      arr(4) if r > 0 else None, n, B, L, hidden, H, block, r, _ptr(y),
                                      _dtype_code(x), _ptr(workspace), ws_bytes, _stream_handle(x, stream))
    if st != BB_OK:
        raise BBError(st, "bb_layer_stack_forward")
