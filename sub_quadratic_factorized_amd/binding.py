"""ctypes binding of the SQuad-Attention C ABI (include/squad_attn.h).

Argument marshalling only: every step of the operator runs in the HIP library.
The library is loaded from this package directory; if it has not been built,
importing the compute entry points raises instead of falling back to anything.

Tensor-level functions take torch tensors laid out [B, n, heads, d] (contiguous,
on a ROCm device, bf16 or float32) plus the latent grid (T, Hs, Ws) and window
(wt, wh, ww).  torch is used for device memory and the current stream only.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsquad_attn.so")

SQUAD_BF16 = 0
SQUAD_F32 = 1

SQUAD_OK = 0
SQUAD_ERR_NULL = 1
SQUAD_ERR_SHAPE = 2
SQUAD_ERR_UNSUPPORTED = 3
SQUAD_ERR_ALIAS = 4
SQUAD_ERR_ALIGN = 5
SQUAD_ERR_HIP = 6
SQUAD_ERR_WORKSPACE = 7
SQUAD_ERR_SCRATCH = 8
NOALLOC_SCRATCH_BYTES = 32 << 20  # SQUAD_NOALLOC_SCRATCH_BYTES

COMPUTE_ENTRY_POINTS = ("squad_attn_fwd", "squad_attn_local", "squad_attn_global", "squad_attn_fwd_reversed")
ALL_SYMBOLS = COMPUTE_ENTRY_POINTS + (
    "squad_attn_fwd_padded", "squad_attn_fwd_padded_noalloc", "squad_attn_check_padded", "squad_attn_padded_workspace_bytes",
    "squad_attn_flops_padded", "squad_attn_bytes_padded", "squad_window_solve",
    "squad_attn_bwd", "squad_attn_check_bwd", "squad_attn_bwd_workspace_bytes", "squad_attn_bwd_flops",
    "squad_attn_bwd_bytes", "squad_attn_fwd_save", "squad_attn_bwd_saved", "squad_attn_bwd_saved_workspace_bytes",
    "squad_attn_check", "squad_attn_max_len", "squad_attn_flops", "squad_attn_bytes", "squad_status_str",
    "squad_attn_last_hip_error", "squad_attn_abi_version",
)

_lib = None


class SquadError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_str(status)} (status {status})"
        if status == SQUAD_ERR_HIP:
            msg += f", hipError_t {lib().squad_attn_last_hip_error()}"
        super().__init__(msg)


def lib() -> ctypes.CDLL:
    """The loaded library with argument and result types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sub_quadratic_factorized_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    p, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    for name in COMPUTE_ENTRY_POINTS:
        f = getattr(L, name)
        f.argtypes = [p, p, p, p] + [i] * 10 + [p]
        f.restype = i
    L.squad_attn_check.argtypes = [p, p, p, p] + [i] * 10
    L.squad_attn_check.restype = i
    sz, ip = ctypes.c_size_t, ctypes.POINTER(ctypes.c_int)
    L.squad_attn_fwd_padded.argtypes = [p, p, p, p, p, sz] + [i] * 10 + [p]
    L.squad_attn_fwd_padded.restype = i
    L.squad_attn_fwd_padded_noalloc.argtypes = [p, p, p, p] + [i] * 10 + [p]
    L.squad_attn_fwd_padded_noalloc.restype = i
    L.squad_attn_check_padded.argtypes = [p, p, p, p, p, sz] + [i] * 10
    L.squad_attn_check_padded.restype = i
    L.squad_attn_padded_workspace_bytes.argtypes = [i] * 10
    L.squad_attn_padded_workspace_bytes.restype = ctypes.c_longlong
    L.squad_attn_flops_padded.argtypes = [i] * 9
    L.squad_attn_flops_padded.restype = d
    L.squad_attn_bytes_padded.argtypes = [i] * 10
    L.squad_attn_bytes_padded.restype = d
    L.squad_window_solve.argtypes = [i, i, i, ip, ip, ip]
    L.squad_window_solve.restype = i
    L.squad_attn_bwd.argtypes = [p] * 9 + [sz] + [i] * 10 + [p]
    L.squad_attn_bwd.restype = i
    L.squad_attn_check_bwd.argtypes = [p] * 9 + [sz] + [i] * 10
    L.squad_attn_check_bwd.restype = i
    L.squad_attn_bwd_workspace_bytes.argtypes = [i] * 10
    L.squad_attn_bwd_workspace_bytes.restype = ctypes.c_longlong
    L.squad_attn_fwd_save.argtypes = [p] * 6 + [i] * 10 + [p]
    L.squad_attn_fwd_save.restype = i
    L.squad_attn_bwd_saved.argtypes = [p] * 11 + [sz] + [i] * 10 + [p]
    L.squad_attn_bwd_saved.restype = i
    L.squad_attn_bwd_saved_workspace_bytes.argtypes = [i] * 10
    L.squad_attn_bwd_saved_workspace_bytes.restype = ctypes.c_longlong
    L.squad_attn_bwd_flops.argtypes = [i] * 9
    L.squad_attn_bwd_flops.restype = d
    L.squad_attn_bwd_bytes.argtypes = [i] * 10
    L.squad_attn_bwd_bytes.restype = d
    L.squad_attn_max_len.argtypes = [i, i]
    L.squad_attn_max_len.restype = i
    L.squad_attn_flops.argtypes = [i] * 9
    L.squad_attn_flops.restype = d
    L.squad_attn_bytes.argtypes = [i] * 10
    L.squad_attn_bytes.restype = d
    L.squad_status_str.argtypes = [i]
    L.squad_status_str.restype = ctypes.c_char_p
    L.squad_attn_last_hip_error.argtypes = []
    L.squad_attn_last_hip_error.restype = i
    L.squad_attn_abi_version.argtypes = []
    L.squad_attn_abi_version.restype = i
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().squad_status_str(status).decode()


def call_raw(name: str, q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, stream=None) -> int:
    """Call a compute entry point with raw integer pointers; returns the status."""
    return getattr(lib(), name)(q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype, stream)


def squad_attn_check(q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype) -> int:
    """Host-only validation status for raw pointer arguments (no HIP call)."""
    return lib().squad_attn_check(q, k, v, out, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype)


def squad_attn_max_len(d: int, dtype: int) -> int:
    return lib().squad_attn_max_len(d, dtype)


def squad_attn_flops(B, heads, T, Hs, Ws, wt, wh, ww, d) -> float:
    return lib().squad_attn_flops(B, heads, T, Hs, Ws, wt, wh, ww, d)


def squad_attn_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype) -> float:
    return lib().squad_attn_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype)


def squad_status_str(status: int) -> str:
    return status_str(status)


def squad_window_solve(grid) -> tuple:
    """(wt, wh, ww) the window rule picks for the latent grid (T, Hs, Ws)."""
    out = [ctypes.c_int(0) for _ in range(3)]
    st = lib().squad_window_solve(*grid, *(ctypes.byref(o) for o in out))
    if st != SQUAD_OK:
        raise SquadError(st, "squad_window_solve")
    return tuple(o.value for o in out)


def squad_attn_padded_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype) -> int:
    return lib().squad_attn_padded_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype)


def squad_attn_flops_padded(B, heads, T, Hs, Ws, wt, wh, ww, d) -> float:
    return lib().squad_attn_flops_padded(B, heads, T, Hs, Ws, wt, wh, ww, d)


def squad_attn_bytes_padded(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype) -> float:
    return lib().squad_attn_bytes_padded(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype)


def squad_attn_bwd_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype) -> int:
    return lib().squad_attn_bwd_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype)


def squad_attn_bwd_saved_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype) -> int:
    return lib().squad_attn_bwd_saved_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype)


def squad_attn_bwd_flops(B, heads, T, Hs, Ws, wt, wh, ww, d) -> float:
    return lib().squad_attn_bwd_flops(B, heads, T, Hs, Ws, wt, wh, ww, d)


def squad_attn_bwd_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype) -> float:
    return lib().squad_attn_bwd_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dtype)


def squad_attn_check_bwd(q, k, v, out, dout, dq, dk, dv, ws, ws_bytes, B, heads, T, Hs, Ws, wt, wh, ww, d,
                         dtype) -> int:
    """Host-only validation status of squad_attn_bwd for raw pointers."""
    return lib().squad_attn_check_bwd(q, k, v, out, dout, dq, dk, dv, ws, ws_bytes, B, heads, T, Hs, Ws, wt, wh, ww,
                                      d, dtype)


def squad_attn_check_padded(q, k, v, out, ws, ws_bytes, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype) -> int:
    """Host-only validation status of squad_attn_fwd_padded for raw pointers."""
    return lib().squad_attn_check_padded(q, k, v, out, ws, ws_bytes, B, heads, T, Hs, Ws, wt, wh, ww, d, dtype)


# ---------------------------------------------------------------------------
# torch tensor entry points
# ---------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return SQUAD_BF16
    if t.dtype == torch.float32:
        return SQUAD_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check_tensors(q, k, v, out, grid):
    import torch
    for t in (q, k, v):
        if t.dim() != 4 or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError("q, k, v must be contiguous [B, n, heads, d] tensors on a GPU")
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must share shape, dtype and device")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    T, Hs, Ws = grid
    if T * Hs * Ws != q.shape[1]:
        raise ValueError(f"grid {tuple(grid)} has {T * Hs * Ws} tokens, tensors have n = {q.shape[1]}")
    return out


def _call(name, q, k, v, out, grid, window, stream):
    import torch
    out = _check_tensors(q, k, v, out, grid)
    B, n, heads, d = q.shape
    T, Hs, Ws = grid
    wt, wh, ww = window
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = call_raw(name, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      B, heads, T, Hs, Ws, wt, wh, ww, d, _dtype_code(q), stream)
    if st != SQUAD_OK:
        raise SquadError(st, name)
    return out


def squad_attn_fwd(q, k, v, grid, window, out=None, stream=None):
    """out = Attn_G(q, k, Attn_L(q, k, v)), asynchronous on the current stream."""
    return _call("squad_attn_fwd", q, k, v, out, grid, window, stream)


def squad_attn_local(q, k, v, grid, window, out=None, stream=None):
    """out = Attn_L(q, k, v): the in-window pass alone."""
    return _call("squad_attn_local", q, k, v, out, grid, window, stream)


def squad_attn_global(q, k, v, grid, window, out=None, stream=None):
    """out = Attn_G(q, k, v): the cross-window, same-slot pass alone."""
    return _call("squad_attn_global", q, k, v, out, grid, window, stream)


def squad_attn_fwd_reversed(q, k, v, grid, window, out=None, stream=None):
    """out = Attn_L(q, k, Attn_G(q, k, v)): the reverse order."""
    return _call("squad_attn_fwd_reversed", q, k, v, out, grid, window, stream)


def squad_attn_fwd_padded(q, k, v, grid, window, out=None, workspace=None, stream=None):
    """SQuad on a grid the window need not tile (reflect padding at the bottom
    and right, outputs of the real tokens only).  `workspace` is a device
    tensor of at least squad_attn_padded_workspace_bytes bytes; if None one is
    allocated through torch for this call."""
    import torch
    out = _check_tensors(q, k, v, out, grid)
    B, n, heads, d = q.shape
    T, Hs, Ws = grid
    wt, wh, ww = window
    dt = _dtype_code(q)
    need = squad_attn_padded_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dt)
    if need < 0:
        raise SquadError(SQUAD_ERR_SHAPE, "squad_attn_fwd_padded")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    ws_bytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().squad_attn_fwd_padded(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         workspace.data_ptr(), ws_bytes, B, heads, T, Hs, Ws, wt, wh, ww, d, dt,
                                         stream)
    if st != SQUAD_OK:
        raise SquadError(st, "squad_attn_fwd_padded")
    return out


def squad_attn_fwd_padded_noalloc(q, k, v, grid, window, out=None, stream=None):
    """squad_attn_fwd_padded without a workspace: the padded positions' local
    outputs go to the library's fixed device scratch (the C call allocates
    nothing; pass `out` to keep this wrapper from allocating it).  Calls on one
    device must not overlap in time."""
    import torch
    out = _check_tensors(q, k, v, out, grid)
    B, n, heads, d = q.shape
    T, Hs, Ws = grid
    wt, wh, ww = window
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().squad_attn_fwd_padded_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, heads,
                                                 T, Hs, Ws, wt, wh, ww, d, _dtype_code(q), stream)
    if st != SQUAD_OK:
        raise SquadError(st, "squad_attn_fwd_padded_noalloc")
    return out


def squad_attn_bwd(q, k, v, out, dout, grid, window, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """(dq, dk, dv) of squad_attn_fwd at (q, k, v), given its output `out` and
    the upstream gradient `dout`.  `workspace`: a device tensor of at least
    squad_attn_bwd_workspace_bytes bytes (allocated through torch if None)."""
    import torch
    _check_tensors(q, k, v, None, grid)
    for t in (out, dout):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("out and dout must be contiguous tensors like q")
    dq, dk, dv = (torch.empty_like(q) if t is None else t for t in (dq, dk, dv))
    for t in (dq, dk, dv):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("dq, dk, dv must be contiguous tensors like q")
    B, n, heads, d = q.shape
    T, Hs, Ws = grid
    wt, wh, ww = window
    dt = _dtype_code(q)
    need = squad_attn_bwd_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dt)
    if need < 0:
        raise SquadError(SQUAD_ERR_SHAPE, "squad_attn_bwd")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    ws_bytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().squad_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                  dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), ws_bytes,
                                  B, heads, T, Hs, Ws, wt, wh, ww, d, dt, stream)
    if st != SQUAD_OK:
        raise SquadError(st, "squad_attn_bwd")
    return dq, dk, dv


def _like(t, ref, what):
    if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous tensor like q")


def _lse_like(t, q):
    import torch
    B, n, heads, _ = q.shape
    if t.shape != (B, n, heads) or t.dtype != torch.float32 or t.device != q.device or not t.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, n, heads] tensor on q's device")


def squad_attn_fwd_save(q, k, v, grid, window, out=None, y=None, lse=None, stream=None):
    """(out, y, lse): squad_attn_fwd's output, the local pass's output Y and,
    in bf16, its rows' log-sum-exp (None in float32), kept for
    squad_attn_bwd_saved."""
    import torch
    out = _check_tensors(q, k, v, out, grid)
    B, n, heads, d = q.shape
    T, Hs, Ws = grid
    wt, wh, ww = window
    dt = _dtype_code(q)
    y = torch.empty_like(q) if y is None else y
    _like(y, q, "y")
    if dt == SQUAD_BF16:
        lse = torch.empty(B, n, heads, dtype=torch.float32, device=q.device) if lse is None else lse
        _lse_like(lse, q)
    else:
        lse = None
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().squad_attn_fwd_save(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), y.data_ptr(),
                                       lse.data_ptr() if lse is not None else None, B, heads, T, Hs, Ws, wt, wh, ww,
                                       d, dt, stream)
    if st != SQUAD_OK:
        raise SquadError(st, "squad_attn_fwd_save")
    return out, y, lse


def squad_attn_bwd_saved(q, k, v, out, dout, y, lse, grid, window, dq=None, dk=None, dv=None, workspace=None,
                         stream=None):
    """(dq, dk, dv) as squad_attn_bwd, from the Y (and bf16 lse) that
    squad_attn_fwd_save kept.  `workspace`: at least
    squad_attn_bwd_saved_workspace_bytes bytes (allocated through torch if
    None)."""
    import torch
    _check_tensors(q, k, v, None, grid)
    for t, what in ((out, "out"), (dout, "dout"), (y, "y")):
        _like(t, q, what)
    dt = _dtype_code(q)
    if dt == SQUAD_BF16:
        if lse is None:
            raise ValueError("lse is required in bf16")
        _lse_like(lse, q)
    dq, dk, dv = (torch.empty_like(q) if t is None else t for t in (dq, dk, dv))
    for t, what in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _like(t, q, what)
    B, n, heads, d = q.shape
    T, Hs, Ws = grid
    wt, wh, ww = window
    need = squad_attn_bwd_saved_workspace_bytes(B, heads, T, Hs, Ws, wt, wh, ww, d, dt)
    if need < 0:
        raise SquadError(SQUAD_ERR_SHAPE, "squad_attn_bwd_saved")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    ws_bytes = workspace.numel() * workspace.element_size()
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    with torch.cuda.device(q.device):
        st = lib().squad_attn_bwd_saved(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                        y.data_ptr(), lse.data_ptr() if lse is not None else None, dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(), ws_bytes, B, heads, T,
                                        Hs, Ws, wt, wh, ww, d, dt, stream)
    if st != SQUAD_OK:
        raise SquadError(st, "squad_attn_bwd_saved")
    return dq, dk, dv


_autograd_fn = None


def squad_attention(q, k, v, grid, window):
    """Differentiable squad_attn_fwd for torch autograd: the forward runs
    squad_attn_fwd_save and keeps (q, k, v, out, Y, lse) for the backward,
    which runs squad_attn_bwd_saved (windows must tile the grid)."""
    global _autograd_fn
    if _autograd_fn is None:
        import torch

        class SquadAttention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, grid, window):
                out, y, lse = squad_attn_fwd_save(q, k, v, grid, window)
                saved = (q, k, v, out, y) + ((lse,) if lse is not None else ())
                ctx.save_for_backward(*saved)
                ctx.grid, ctx.window = grid, window
                return out

            @staticmethod
            def backward(ctx, dout):
                q, k, v, out, y, *rest = ctx.saved_tensors
                dq, dk, dv = squad_attn_bwd_saved(q, k, v, out, dout.contiguous(), y, rest[0] if rest else None,
                                                  ctx.grid, ctx.window)
                return dq, dk, dv, None, None

        _autograd_fn = SquadAttention
    return _autograd_fn.apply(q, k, v, tuple(grid), tuple(window))
