"""MI355X (gfx950) Mamba selective scan: Python binding of libmambascan.so.

The binding only marshals arguments: torch tensors are checked for device, dtype,
shape and contiguity, their device pointers and the current HIP stream are passed
to the C entry points declared in ``include/mamba_scan.h``, and the workspace is
allocated with torch.  Every step of the computation runs in the HIP kernels;
there is no CPU or PyTorch fallback -- if the library is missing, the call fails.

    y, h_last = mamba_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                               h0=None, return_last_state=False)
    y = mamba_state_update(h, u, delta, A, B, C, D=None, z=None, delta_bias=None)
    u, state = mamba_conv1d_silu_fwd(x, w, conv_bias=None, state_in=None, return_state=False)
    u = mamba_conv1d_silu_update(state, x, w, conv_bias=None)
    grads = mamba_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None,
                           h0=None, dh_last=None)
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmambascan.so")

MAMBA_DTYPE_F32 = 0
MAMBA_DTYPE_BF16 = 1

STATUS = {
    0: "MAMBA_OK", 1: "MAMBA_ERR_NULL_ARG", 2: "MAMBA_ERR_BAD_SHAPE", 3: "MAMBA_ERR_BAD_DTYPE",
    4: "MAMBA_ERR_UNSUPPORTED", 5: "MAMBA_ERR_MISALIGNED", 6: "MAMBA_ERR_ALIASING",
    7: "MAMBA_ERR_WORKSPACE", 8: "MAMBA_ERR_HIP",
}

# Every symbol include/mamba_scan.h declares.
EXPORTS = ("mamba_d_state_supported", "mamba_scan_fwd_workspace_size",
           "mamba_scan_fwd_workspace_size_ex", "mamba_scan_fwd", "mamba_scan_fwd_ex",
           "mamba_state_update", "mamba_state_update_ex", "mamba_conv1d_silu_fwd",
           "mamba_conv1d_silu_update", "mamba_scan_bwd_workspace_size", "mamba_scan_bwd",
           "mamba_scan_bwd_workspace_size_ex", "mamba_scan_bwd_ex",
           "mamba_scan_fwd_workspace_size_ext", "mamba_scan_fwd_ext", "mamba_state_update_ext",
           "mamba_ssd_supported", "mamba_ssd_fwd", "mamba_ssd_workspace_size", "mamba_ssd_fwd_ex",
           "mamba_ssd_state_update",
           "mamba_scan_ckpt_size", "mamba_scan_bwd_ckpt_workspace_size", "mamba_scan_bwd_ckpt",
           "mamba_scan_fwd_relay_faults", "mamba_ssd_relay_faults", "mamba_scan_fwd_noalloc",
           "mamba_probe_copy", "mamba_probe_issue", "mamba_scan_bwd_ext_workspace_size",
           "mamba_scan_bwd_ext", "mamba_status_string")


class MambaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


MAMBA_KERNEL_AUTO, MAMBA_KERNEL_BLOCK, MAMBA_KERNEL_ROWS, MAMBA_KERNEL_SCALAR = 0, 1, 2, 3
KERNELS = {"auto": MAMBA_KERNEL_AUTO, "block": MAMBA_KERNEL_BLOCK, "rows": MAMBA_KERNEL_ROWS,
           "scalar": MAMBA_KERNEL_SCALAR}


MAMBA_DISC_EULER, MAMBA_DISC_ZOH = 0, 1
DISCRETIZATIONS = {"euler": MAMBA_DISC_EULER, "zoh": MAMBA_DISC_ZOH}


class ScanOpts(ctypes.Structure):
    _fields_ = [("chunk_len", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("n_spans", ctypes.c_int32), ("kernel", ctypes.c_int32),
                ("relay", ctypes.c_int32), ("discretization", ctypes.c_int32)]


class SsdOpts(ctypes.Structure):
    """mamba_ssd_opts_t: relay (0 auto, 1 off, 2 force), n_spans (0 auto, 1 none, k)."""
    _fields_ = [("relay", ctypes.c_int32), ("n_spans", ctypes.c_int32)]


class ScanExt(ctypes.Structure):
    """mamba_scan_ext_t: trapezoid mixing coefficients, look-back input, rotation rates,
    checkpoint output for the backward pass, row strides of u, delta, z, B, C."""
    _fields_ = [("lambda_", ctypes.c_void_p), ("u_prev", ctypes.c_void_p),
                ("B_prev", ctypes.c_void_p), ("theta", ctypes.c_void_p),
                ("ckpt", ctypes.c_void_p), ("u_stride", ctypes.c_int64),
                ("delta_stride", ctypes.c_int64), ("z_stride", ctypes.c_int64),
                ("B_stride", ctypes.c_int64), ("C_stride", ctypes.c_int64)]


class ScanExtGrads(ctypes.Structure):
    """mamba_scan_ext_grads_t: gradients of lambda, u_prev, B_prev, theta."""
    _fields_ = [("dlam", ctypes.c_void_p), ("du_prev", ctypes.c_void_p),
                ("dB_prev", ctypes.c_void_p), ("dtheta", ctypes.c_void_p)]


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_lib = None


def load_library(path: str = LIBRARY) -> ctypes.CDLL:
    """Load libmambascan.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m selective_state_space_72_amd.build`"
            " (there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    lib.mamba_d_state_supported.restype = ctypes.c_int32
    lib.mamba_d_state_supported.argtypes = [_i64]
    lib.mamba_scan_fwd_workspace_size.restype = ctypes.c_size_t
    lib.mamba_scan_fwd_workspace_size.argtypes = [_i64] * 4
    lib.mamba_scan_fwd_workspace_size_ex.restype = ctypes.c_size_t
    lib.mamba_scan_fwd_workspace_size_ex.argtypes = [_i64] * 4 + [ctypes.POINTER(ScanOpts)]
    lib.mamba_scan_fwd.restype = ctypes.c_int
    lib.mamba_scan_fwd.argtypes = [_vp] * 11 + [_i64] * 4 + [ctypes.c_int, _vp, ctypes.c_size_t,
                                                              _vp]
    lib.mamba_scan_fwd_ex.restype = ctypes.c_int
    lib.mamba_scan_fwd_ex.argtypes = ([_vp] * 11 + [_i64] * 4 +
                                      [ctypes.c_int, _vp, ctypes.c_size_t,
                                       ctypes.POINTER(ScanOpts), _vp])
    lib.mamba_state_update.restype = ctypes.c_int
    lib.mamba_state_update.argtypes = [_vp] * 10 + [_i64] * 3 + [ctypes.c_int, _vp]
    lib.mamba_state_update_ex.restype = ctypes.c_int
    lib.mamba_state_update_ex.argtypes = ([_vp] * 10 + [_i64] * 3 +
                                          [ctypes.c_int, ctypes.c_int32, _vp])
    lib.mamba_conv1d_silu_fwd.restype = ctypes.c_int
    lib.mamba_conv1d_silu_fwd.argtypes = [_vp] * 6 + [_i64] * 4 + [ctypes.c_int, _vp]
    lib.mamba_conv1d_silu_update.restype = ctypes.c_int
    lib.mamba_conv1d_silu_update.argtypes = [_vp] * 5 + [_i64] * 3 + [ctypes.c_int, _vp]
    lib.mamba_scan_bwd_workspace_size.restype = ctypes.c_size_t
    lib.mamba_scan_bwd_workspace_size.argtypes = [_i64] * 4
    lib.mamba_scan_bwd.restype = ctypes.c_int
    lib.mamba_scan_bwd.argtypes = [_vp] * 20 + [_i64] * 4 + [ctypes.c_int, _vp, ctypes.c_size_t,
                                                              _vp]
    lib.mamba_scan_bwd_ext_workspace_size.restype = ctypes.c_size_t
    lib.mamba_scan_bwd_ext_workspace_size.argtypes = [_i64] * 4 + [ctypes.POINTER(ScanExt),
                                                                   ctypes.POINTER(ScanOpts)]
    lib.mamba_scan_bwd_ext.restype = ctypes.c_int
    lib.mamba_scan_bwd_ext.argtypes = ([_vp] * 20 + [ctypes.POINTER(ScanExt),
                                                     ctypes.POINTER(ScanExtGrads)] +
                                       [_i64] * 4 + [ctypes.c_int, _vp, ctypes.c_size_t,
                                                     ctypes.POINTER(ScanOpts), _vp])
    lib.mamba_scan_bwd_workspace_size_ex.restype = ctypes.c_size_t
    lib.mamba_scan_bwd_workspace_size_ex.argtypes = [_i64] * 4 + [ctypes.POINTER(ScanOpts)]
    lib.mamba_scan_bwd_ex.restype = ctypes.c_int
    lib.mamba_scan_bwd_ex.argtypes = ([_vp] * 20 + [_i64] * 4 +
                                      [ctypes.c_int, _vp, ctypes.c_size_t,
                                       ctypes.POINTER(ScanOpts), _vp])
    lib.mamba_scan_fwd_workspace_size_ext.restype = ctypes.c_size_t
    lib.mamba_scan_fwd_workspace_size_ext.argtypes = ([_i64] * 4 + [ctypes.POINTER(ScanExt),
                                                                    ctypes.POINTER(ScanOpts)])
    lib.mamba_scan_fwd_ext.restype = ctypes.c_int
    lib.mamba_scan_fwd_ext.argtypes = ([_vp] * 11 + [_i64] * 4 +
                                       [ctypes.c_int, _vp, ctypes.c_size_t,
                                        ctypes.POINTER(ScanOpts), ctypes.POINTER(ScanExt), _vp])
    lib.mamba_state_update_ext.restype = ctypes.c_int
    lib.mamba_state_update_ext.argtypes = ([_vp] * 10 + [_i64] * 3 +
                                           [ctypes.c_int, ctypes.c_int32,
                                            ctypes.POINTER(ScanExt), _vp])
    lib.mamba_ssd_supported.restype = ctypes.c_int32
    lib.mamba_ssd_supported.argtypes = [_i64, _i64]
    lib.mamba_ssd_fwd.restype = ctypes.c_int
    lib.mamba_ssd_fwd.argtypes = [_vp] * 11 + [_i64] * 5 + [ctypes.c_int, _vp]
    lib.mamba_ssd_state_update.restype = ctypes.c_int
    lib.mamba_ssd_state_update.argtypes = [_vp] * 10 + [_i64] * 4 + [ctypes.c_int, _vp]
    lib.mamba_ssd_workspace_size.restype = ctypes.c_size_t
    lib.mamba_ssd_workspace_size.argtypes = [_i64] * 5 + [ctypes.c_int,
                                                          ctypes.POINTER(SsdOpts)]
    lib.mamba_ssd_fwd_ex.restype = ctypes.c_int
    lib.mamba_ssd_fwd_ex.argtypes = ([_vp] * 11 + [_i64] * 5 + [ctypes.c_int, _vp,
                                     ctypes.c_size_t, ctypes.POINTER(SsdOpts), _vp])
    lib.mamba_scan_ckpt_size.restype = ctypes.c_size_t
    lib.mamba_scan_ckpt_size.argtypes = [_i64] * 4
    lib.mamba_scan_bwd_ckpt_workspace_size.restype = ctypes.c_size_t
    lib.mamba_scan_bwd_ckpt_workspace_size.argtypes = [_i64] * 4 + [ctypes.POINTER(ScanOpts)]
    lib.mamba_scan_bwd_ckpt.restype = ctypes.c_int
    lib.mamba_scan_bwd_ckpt.argtypes = ([_vp] * 21 + [_i64] * 4 + [ctypes.c_int, _vp,
                                                                     ctypes.c_size_t,
                                                                     ctypes.POINTER(ScanOpts), _vp])
    lib.mamba_scan_fwd_relay_faults.restype = ctypes.c_int
    lib.mamba_scan_fwd_relay_faults.argtypes = ([_vp, ctypes.c_size_t] + [_i64] * 4 +
                                                [ctypes.POINTER(ScanOpts), ctypes.POINTER(ScanExt),
                                                 ctypes.POINTER(ctypes.c_uint32), _vp])
    lib.mamba_ssd_relay_faults.restype = ctypes.c_int
    lib.mamba_ssd_relay_faults.argtypes = ([_vp, ctypes.c_size_t] + [_i64] * 5 +
                                           [ctypes.c_int, ctypes.POINTER(SsdOpts),
                                            ctypes.POINTER(ctypes.c_uint32), _vp])
    lib.mamba_scan_fwd_noalloc.restype = ctypes.c_int
    lib.mamba_scan_fwd_noalloc.argtypes = [_vp] * 11 + [_i64] * 4 + [ctypes.c_int, _vp]
    lib.mamba_probe_copy.restype = ctypes.c_int
    lib.mamba_probe_copy.argtypes = [_vp, _vp, ctypes.c_size_t, ctypes.c_int32, _vp]
    lib.mamba_probe_issue.restype = ctypes.c_int
    lib.mamba_probe_issue.argtypes = ([ctypes.c_int32] * 4 +
                                      [_vp, ctypes.POINTER(ctypes.c_uint64), _vp])
    lib.mamba_status_string.restype = ctypes.c_char_p
    lib.mamba_status_string.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def status_string(status: int) -> str:
    if _lib is not None:
        return _lib.mamba_status_string(int(status)).decode()
    return STATUS.get(int(status), f"status {status}")


# ----------------------------------------------------------------------------
# argument marshalling
# ----------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MAMBA_DTYPE_BF16
    if t.dtype == torch.float32:
        return MAMBA_DTYPE_F32
    raise TypeError(f"activations must be bfloat16 or float32, got {t.dtype}")


def _dtype_code_of(dtype) -> int:
    """Code of an activation dtype given as a torch dtype or a name ("bf16", "f32")."""
    if isinstance(dtype, str):
        codes = {"bf16": MAMBA_DTYPE_BF16, "bfloat16": MAMBA_DTYPE_BF16,
                 "f32": MAMBA_DTYPE_F32, "fp32": MAMBA_DTYPE_F32, "float32": MAMBA_DTYPE_F32}
        if dtype not in codes:
            raise TypeError(f"unknown activation dtype {dtype!r}")
        return codes[dtype]
    torch = _torch()
    if dtype == torch.bfloat16:
        return MAMBA_DTYPE_BF16
    if dtype == torch.float32:
        return MAMBA_DTYPE_F32
    raise TypeError(f"activations must be bfloat16 or float32, got {dtype}")


def _ptr(t, name, shape=None, dtype=None, device=None) -> Optional[int]:
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() > 0 else None


def _rows_ptr(t, name, shape, dtype, device):
    """Pointer and row stride (elements between consecutive rows: the leading dimensions
    taken together) of a tensor whose last dimension is contiguous and whose rows are
    evenly spaced -- a view such as xz.chunk(2, -1)[1] or a slice of the last dimension.
    Returns (None, 0) for None; the stride is 0 for a contiguous tensor."""
    if t is None:
        return None, 0
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.is_contiguous():
        return _ptr(t, name, shape, dtype, device), 0
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    lead = [(n, st) for n, st in zip(t.shape[:-1], t.stride()[:-1]) if n > 1]
    row = lead[-1][1] if lead else t.shape[-1]
    expect = row
    for n, st in reversed(lead):
        if st != expect:
            raise ValueError(f"{name}: rows must be evenly spaced (strides {t.stride()})")
        expect = st * n
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return (t.data_ptr() if t.numel() > 0 else None), int(row)


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _opts(chunk_len=0, waves=0, n_spans=0, kernel="auto", relay=0, discretization="euler"):
    if kernel not in KERNELS:
        raise ValueError(f"kernel must be one of {sorted(KERNELS)}")
    if discretization not in DISCRETIZATIONS:
        raise ValueError(f"discretization must be one of {sorted(DISCRETIZATIONS)}")
    return ScanOpts(int(chunk_len), int(waves), int(n_spans), KERNELS[kernel], int(relay),
                    DISCRETIZATIONS[discretization])


def mamba_scan_fwd_workspace_size(batch: int, seqlen: int, d_inner: int, d_state: int,
                                  chunk_len: int = 0, waves: int = 0, n_spans: int = 0,
                                  kernel: str = "auto", relay: int = 0,
                                  discretization: str = "euler", trapezoid: bool = False,
                                  rotation: bool = False, strides=(0, 0, 0, 0, 0)) -> int:
    """strides: row strides of (u, delta, z, B, C) in elements, 0 = contiguous."""
    lib = load_library()
    o = _opts(chunk_len, waves, n_spans, kernel, relay, discretization)
    # only the presence of the extension inputs matters for the size
    e = ScanExt(1 if trapezoid else None, None, None, 1 if rotation else None, None,
                *[int(x) for x in strides])
    n = lib.mamba_scan_fwd_workspace_size_ext(batch, seqlen, d_inner, d_state, ctypes.byref(e),
                                              ctypes.byref(o))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes or options for mamba_scan_fwd")
    return int(n)


def mamba_scan_fwd(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None,
                   return_last_state: bool = False, *, out=None, h_last_out=None,
                   chunk_len: int = 0, waves: int = 0, n_spans: int = 0,
                   kernel: str = "auto", relay: int = 0, discretization: str = "euler",
                   workspace=None, lam=None, u_prev=None, B_prev=None, theta=None,
                   ckpt=None) -> Tuple:
    """Selective scan over (batch, seqlen, d_inner); see include/mamba_scan.h.

    Returns (y, h_last) -- h_last is None unless return_last_state (or h_last_out).
    lam (batch, seqlen, d_inner): exponential-trapezoidal mixing coefficients, with the
    input before t = 0 in u_prev (batch, d_inner) and B_prev (batch, d_state); theta
    (batch, seqlen, d_state / 2): rotation rates of the state pairs (see mamba_scan_ext_t).
    ckpt: a float32 tensor of mamba_scan_ckpt_size(...) bytes that receives the states the
    backward pass needs (for mamba_scan_bwd(..., ckpt=...)).
    """
    torch = _torch()
    lib = load_library()
    if u.dim() != 3:
        raise ValueError("u must be (batch, seqlen, d_inner)")
    batch, seqlen, d_inner = u.shape
    if A.dim() != 2 or A.shape[0] != d_inner:
        raise ValueError("A must be (d_inner, d_state)")
    d_state = A.shape[1]
    dev = u.device
    act = u.dtype
    code = _dtype_code(u)
    f32 = torch.float32
    # u, delta, z, B, C may be views with evenly spaced rows (passed as row strides)
    p_u, s_u = _rows_ptr(u, "u", (batch, seqlen, d_inner), act, dev)
    p_delta, s_d = _rows_ptr(delta, "delta", (batch, seqlen, d_inner), act, dev)
    p_A = _ptr(A, "A", (d_inner, d_state), f32, dev)
    p_B, s_B = _rows_ptr(B, "B", (batch, seqlen, d_state), act, dev)
    p_C, s_C = _rows_ptr(C, "C", (batch, seqlen, d_state), act, dev)
    p_D = _ptr(D, "D", (d_inner,), f32, dev)
    p_z, s_z = _rows_ptr(z, "z", (batch, seqlen, d_inner), act, dev)
    p_bias = _ptr(delta_bias, "delta_bias", (d_inner,), f32, dev)
    p_h0 = _ptr(h0, "h0", (batch, d_inner, d_state), f32, dev)
    y = out if out is not None else torch.empty((batch, seqlen, d_inner), dtype=act, device=dev)
    p_y = _ptr(y, "out", (batch, seqlen, d_inner), act, dev)
    h_last = h_last_out
    if h_last is None and return_last_state:
        h_last = torch.empty((batch, d_inner, d_state), dtype=f32, device=dev)
    p_hl = _ptr(h_last, "h_last_out", (batch, d_inner, d_state), f32, dev)
    ext = ScanExt(_ptr(lam, "lam", (batch, seqlen, d_inner), act, dev),
                  _ptr(u_prev, "u_prev", (batch, d_inner), act, dev),
                  _ptr(B_prev, "B_prev", (batch, d_state), act, dev),
                  _ptr(theta, "theta", (batch, seqlen, d_state // 2), act, dev),
                  _ckpt_ptr(ckpt, batch, seqlen, d_inner, d_state, dev), s_u, s_d, s_z, s_B,
                  s_C)
    if seqlen == 0:
        # empty tensors have no address; only the presence of an option matters here
        ext.lambda_ = ext.lambda_ or (1 if lam is not None else None)
        ext.theta = ext.theta or (1 if theta is not None else None)
        ext.ckpt = ext.ckpt or (1 if ckpt is not None else None)

    opts = _opts(chunk_len, waves, n_spans, kernel, relay, discretization)
    need = lib.mamba_scan_fwd_workspace_size_ext(batch, seqlen, d_inner, d_state,
                                                 ctypes.byref(ext), ctypes.byref(opts))
    if need == ctypes.c_size_t(-1).value:
        raise MambaError(4, "mamba_scan_fwd_workspace_size")
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    p_ws = ws.data_ptr() if ws is not None and need > 0 else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib.mamba_scan_fwd_ext(p_u, p_delta, p_A, p_B, p_C, p_D, p_z, p_bias, p_h0, p_y,
                                p_hl, batch, seqlen, d_inner, d_state, code, p_ws, ws_bytes,
                                ctypes.byref(opts), ctypes.byref(ext), _stream(dev))
    if st != 0:
        raise MambaError(st, "mamba_scan_fwd")
    return y, h_last


def _ws_arg(workspace):
    if workspace is None:
        return None, 0
    return (workspace.data_ptr() if workspace.numel() > 0 else None,
            workspace.numel() * workspace.element_size())


def mamba_scan_fwd_relay_faults(workspace, batch: int, seqlen: int, d_inner: int, d_state: int,
                                *, chunk_len: int = 0, waves: int = 0, n_spans: int = 0,
                                kernel: str = "auto", relay: int = 0,
                                discretization: str = "euler", trapezoid: bool = False,
                                rotation: bool = False, strides=(0, 0, 0, 0, 0),
                                device=None) -> int:
    """Relay hand-offs that timed out in the last mamba_scan_fwd call given this workspace
    with the same sizes and options (0 when it planned no relay).  Synchronises the current
    stream."""
    lib = load_library()
    o = _opts(chunk_len, waves, n_spans, kernel, relay, discretization)
    e = ScanExt(1 if trapezoid else None, None, None, 1 if rotation else None, None,
                *[int(x) for x in strides])
    p_ws, ws_bytes = _ws_arg(workspace)
    dev = workspace.device if workspace is not None else device
    out = ctypes.c_uint32(0)
    st = lib.mamba_scan_fwd_relay_faults(p_ws, ws_bytes, batch, seqlen, d_inner, d_state,
                                         ctypes.byref(o), ctypes.byref(e), ctypes.byref(out),
                                         _stream(dev) if dev is not None else None)
    if st != 0:
        raise MambaError(st, "mamba_scan_fwd_relay_faults")
    return int(out.value)


NOALLOC_MAX_WORKSPACE = 64 << 20  # MAMBA_SCAN_NOALLOC_MAX_WORKSPACE


def mamba_scan_fwd_noalloc(u, delta, A, B, C, *, out, D=None, z=None, delta_bias=None,
                           h0=None, h_last_out=None):
    """mamba_scan_fwd into caller-provided outputs (out, h_last_out) through the entry point
    that allocates nothing (its workspace is the library's per-device array).  Returns
    (out, h_last_out)."""
    torch = _torch()
    lib = load_library()
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be (batch, seqlen, d_inner) and A (d_inner, d_state)")
    batch, seqlen, d_inner = u.shape
    d_state = A.shape[1]
    dev, act, f32 = u.device, u.dtype, torch.float32
    bld = (batch, seqlen, d_inner)
    st = lib.mamba_scan_fwd_noalloc(
        _ptr(u, "u", bld, act, dev), _ptr(delta, "delta", bld, act, dev),
        _ptr(A, "A", (d_inner, d_state), f32, dev),
        _ptr(B, "B", (batch, seqlen, d_state), act, dev),
        _ptr(C, "C", (batch, seqlen, d_state), act, dev), _ptr(D, "D", (d_inner,), f32, dev),
        _ptr(z, "z", bld, act, dev), _ptr(delta_bias, "delta_bias", (d_inner,), f32, dev),
        _ptr(h0, "h0", (batch, d_inner, d_state), f32, dev), _ptr(out, "out", bld, act, dev),
        _ptr(h_last_out, "h_last_out", (batch, d_inner, d_state), f32, dev),
        batch, seqlen, d_inner, d_state, _dtype_code(u), _stream(dev))
    if st != 0:
        raise MambaError(st, "mamba_scan_fwd_noalloc")
    return out, h_last_out


def mamba_state_update(h, u, delta, A, B, C, D=None, z=None, delta_bias=None, *, out=None,
                       discretization: str = "euler", lam=None, u_prev=None, B_prev=None,
                       theta=None):
    """One decode step; h (batch, d_inner, d_state) fp32 is updated in place.  Returns y.
    lam, u_prev (batch, d_inner), B_prev (batch, d_state): the trapezoid with the previous
    token's input; theta (batch, d_state / 2): rotation rates."""
    torch = _torch()
    lib = load_library()
    if u.dim() != 2:
        raise ValueError("u must be (batch, d_inner)")
    batch, d_inner = u.shape
    d_state = A.shape[1]
    dev = u.device
    act = u.dtype
    code = _dtype_code(u)
    f32 = torch.float32
    p_h = _ptr(h, "h", (batch, d_inner, d_state), f32, dev)
    # u, delta, z, B, C may be views with evenly spaced batch rows
    p_u, s_u = _rows_ptr(u, "u", (batch, d_inner), act, dev)
    p_delta, s_d = _rows_ptr(delta, "delta", (batch, d_inner), act, dev)
    p_A = _ptr(A, "A", (d_inner, d_state), f32, dev)
    p_B, s_B = _rows_ptr(B, "B", (batch, d_state), act, dev)
    p_C, s_C = _rows_ptr(C, "C", (batch, d_state), act, dev)
    p_D = _ptr(D, "D", (d_inner,), f32, dev)
    p_z, s_z = _rows_ptr(z, "z", (batch, d_inner), act, dev)
    p_bias = _ptr(delta_bias, "delta_bias", (d_inner,), f32, dev)
    y = out if out is not None else torch.empty((batch, d_inner), dtype=act, device=dev)
    p_y = _ptr(y, "out", (batch, d_inner), act, dev)
    if discretization not in DISCRETIZATIONS:
        raise ValueError(f"discretization must be one of {sorted(DISCRETIZATIONS)}")
    ext = ScanExt(_ptr(lam, "lam", (batch, d_inner), act, dev),
                  _ptr(u_prev, "u_prev", (batch, d_inner), act, dev),
                  _ptr(B_prev, "B_prev", (batch, d_state), act, dev),
                  _ptr(theta, "theta", (batch, d_state // 2), act, dev), None, s_u, s_d, s_z,
                  s_B, s_C)
    st = lib.mamba_state_update_ext(p_h, p_u, p_delta, p_A, p_B, p_C, p_D, p_z, p_bias, p_y,
                                    batch, d_inner, d_state, code,
                                    DISCRETIZATIONS[discretization], ctypes.byref(ext),
                                    _stream(dev))
    if st != 0:
        raise MambaError(st, "mamba_state_update")
    return y


def mamba_conv1d_silu_fwd(x, w, conv_bias=None, state_in=None, *, out=None, state_out=None,
                          return_state: bool = False):
    """Causal depthwise conv1d + SiLU over (batch, seqlen, d_inner); see include/mamba_scan.h.

    w: (d_inner, d_conv) fp32; conv_bias: (d_inner,) fp32; states (batch, d_inner,
    d_conv - 1) in x's dtype.  Returns (u, state_out); state_out is None unless
    return_state (or state_out is given).  state_out may be state_in itself.
    """
    torch = _torch()
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (batch, seqlen, d_inner)")
    batch, seqlen, d_inner = x.shape
    if w.dim() != 2 or w.shape[0] != d_inner:
        raise ValueError("w must be (d_inner, d_conv)")
    d_conv = w.shape[1]
    dev, act = x.device, x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    p_x = _ptr(x, "x", (batch, seqlen, d_inner), act, dev)
    p_w = _ptr(w, "w", (d_inner, d_conv), f32, dev)
    p_b = _ptr(conv_bias, "conv_bias", (d_inner,), f32, dev)
    sshape = (batch, d_inner, d_conv - 1)
    p_si = _ptr(state_in, "state_in", sshape, act, dev)
    u = out if out is not None else torch.empty((batch, seqlen, d_inner), dtype=act, device=dev)
    p_u = _ptr(u, "out", (batch, seqlen, d_inner), act, dev)
    so = state_out
    if so is None and return_state:
        so = torch.empty(sshape, dtype=act, device=dev)
    p_so = _ptr(so, "state_out", sshape, act, dev)
    st = lib.mamba_conv1d_silu_fwd(p_x, p_w, p_b, p_si, p_u, p_so, batch, seqlen, d_inner,
                                   d_conv, code, _stream(dev))
    if st != 0:
        raise MambaError(st, "mamba_conv1d_silu_fwd")
    return u, so


def mamba_conv1d_silu_update(state, x, w, conv_bias=None, *, out=None):
    """One decode token of the conv1d + SiLU; state (batch, d_inner, d_conv - 1) is
    updated in place.  Returns u (batch, d_inner)."""
    torch = _torch()
    lib = load_library()
    if x.dim() != 2:
        raise ValueError("x must be (batch, d_inner)")
    batch, d_inner = x.shape
    if w.dim() != 2 or w.shape[0] != d_inner:
        raise ValueError("w must be (d_inner, d_conv)")
    d_conv = w.shape[1]
    dev, act = x.device, x.dtype
    code = _dtype_code(x)
    p_s = _ptr(state, "state", (batch, d_inner, d_conv - 1), act, dev)
    p_x = _ptr(x, "x", (batch, d_inner), act, dev)
    p_w = _ptr(w, "w", (d_inner, d_conv), torch.float32, dev)
    p_b = _ptr(conv_bias, "conv_bias", (d_inner,), torch.float32, dev)
    u = out if out is not None else torch.empty((batch, d_inner), dtype=act, device=dev)
    p_u = _ptr(u, "out", (batch, d_inner), act, dev)
    st = lib.mamba_conv1d_silu_update(p_s, p_x, p_w, p_b, p_u, batch, d_inner, d_conv, code,
                                      _stream(dev))
    if st != 0:
        raise MambaError(st, "mamba_conv1d_silu_update")
    return u


def mamba_scan_bwd_workspace_size(batch: int, seqlen: int, d_inner: int, d_state: int,
                                  n_spans: int = 0, with_ckpt: bool = False,
                                  discretization: str = "euler") -> int:
    """Workspace bytes of mamba_scan_bwd (with_ckpt: of the variant that reads the forward
    pass's checkpoints)."""
    lib = load_library()
    o = ScanOpts(0, 0, int(n_spans), 0, 0, DISCRETIZATIONS[discretization])
    f = lib.mamba_scan_bwd_ckpt_workspace_size if with_ckpt else lib.mamba_scan_bwd_workspace_size_ex
    n = f(batch, seqlen, d_inner, d_state, ctypes.byref(o))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes for mamba_scan_bwd")
    return int(n)


def mamba_scan_ckpt_size(batch: int, seqlen: int, d_inner: int, d_state: int) -> int:
    """Bytes of the checkpoint buffer (mamba_scan_fwd(..., ckpt=) / mamba_scan_bwd(..., ckpt=))."""
    n = load_library().mamba_scan_ckpt_size(batch, seqlen, d_inner, d_state)
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("invalid sizes or d_state for checkpoints")
    return int(n)


def mamba_scan_ckpt_buffer(batch: int, seqlen: int, d_inner: int, d_state: int, device):
    """A float32 tensor of the checkpoint buffer's size."""
    torch = _torch()
    n = mamba_scan_ckpt_size(batch, seqlen, d_inner, d_state)
    return torch.empty(max(n // 4, 1), dtype=torch.float32, device=device)


def _ckpt_ptr(ckpt, batch, seqlen, d_inner, d_state, dev):
    if ckpt is None:
        return None
    torch = _torch()
    need = mamba_scan_ckpt_size(batch, seqlen, d_inner, d_state)
    if ckpt.dtype != torch.float32 or ckpt.device != dev or not ckpt.is_contiguous() or \
            ckpt.numel() * 4 < need:
        raise ValueError(f"ckpt must be a contiguous float32 tensor of at least {need} bytes "
                         f"on {dev}")
    return ckpt.data_ptr() if need > 0 else None


GRAD_NAMES = ("du", "ddelta", "dA", "dB", "dC", "dD", "dz", "dbias", "dh0")


def mamba_scan_bwd(u, delta, A, B, C, dy, D=None, z=None, delta_bias=None, h0=None,
                   dh_last=None, *, want=GRAD_NAMES, out=None, workspace=None,
                   n_spans: int = 0, ckpt=None, discretization: str = "euler", lam=None,
                   u_prev=None, B_prev=None, theta=None) -> dict:
    """Gradients of the selective scan (Euler, or discretization="zoh"); see
    include/mamba_scan.h.  With lam (u_prev, B_prev) or theta: the gradients of the scan
    with those Mamba-3 options (mamba_scan_bwd_ext), adding dlam, du_prev, dB_prev or
    dtheta to the result.

    Returns a dict with the names of ``want`` (a subset of GRAD_NAMES; du and ddelta are
    always computed): du, ddelta, dz, dB, dC in the activations' dtype, dA, dD, dbias,
    dh0 in float32.  dz is None without a gate.  ``out`` may map names to preallocated
    tensors.  n_spans: sequence split (0 = automatic; see mamba_scan_bwd_ex).  ckpt: the
    checkpoints written by mamba_scan_fwd(..., ckpt=) on the same inputs
    (mamba_scan_bwd_ckpt: no forward pass of its own).
    """
    torch = _torch()
    lib = load_library()
    if u.dim() != 3:
        raise ValueError("u must be (batch, seqlen, d_inner)")
    batch, seqlen, d_inner = u.shape
    if A.dim() != 2 or A.shape[0] != d_inner:
        raise ValueError("A must be (d_inner, d_state)")
    d_state = A.shape[1]
    dev, act = u.device, u.dtype
    code = _dtype_code(u)
    f32 = torch.float32
    bld, bln, bdn = (batch, seqlen, d_inner), (batch, seqlen, d_state), (batch, d_inner, d_state)
    p_u = _ptr(u, "u", bld, act, dev)
    p_delta = _ptr(delta, "delta", bld, act, dev)
    p_A = _ptr(A, "A", (d_inner, d_state), f32, dev)
    p_B = _ptr(B, "B", bln, act, dev)
    p_C = _ptr(C, "C", bln, act, dev)
    p_D = _ptr(D, "D", (d_inner,), f32, dev)
    p_z = _ptr(z, "z", bld, act, dev)
    p_bias = _ptr(delta_bias, "delta_bias", (d_inner,), f32, dev)
    p_h0 = _ptr(h0, "h0", bdn, f32, dev)
    p_dy = _ptr(dy, "dy", bld, act, dev)
    p_dhl = _ptr(dh_last, "dh_last", bdn, f32, dev)
    unknown = set(want) - set(GRAD_NAMES)
    if unknown:
        raise ValueError(f"unknown gradient names {sorted(unknown)}")
    shapes = {"du": (bld, act), "ddelta": (bld, act), "dz": (bld, act), "dB": (bln, act),
              "dC": (bln, act), "dA": ((d_inner, d_state), f32), "dD": ((d_inner,), f32),
              "dbias": ((d_inner,), f32), "dh0": (bdn, f32)}
    out = dict(out or {})
    res = {}
    ptrs = {}
    for name in GRAD_NAMES:
        shape, dt = shapes[name]
        # dz is always computed with a gate (the library requires it), returned if wanted
        wanted = name in ("du", "ddelta") or name in want or (name == "dz" and z is not None)
        if name == "dz" and z is None:
            wanted = False
        t = out.get(name) if wanted else None
        if wanted and t is None:
            t = torch.empty(shape, dtype=dt, device=dev)
        res[name] = t
        ptrs[name] = _ptr(t, name, shape, dt, dev)
    if discretization not in DISCRETIZATIONS:
        raise ValueError(f"discretization must be one of {sorted(DISCRETIZATIONS)}")
    opts = ScanOpts(0, 0, int(n_spans), 0, 0, DISCRETIZATIONS[discretization])
    if lam is not None or theta is not None:
        if ckpt is not None:
            raise ValueError("stored checkpoints are for the Euler rule without options")
        return _bwd_m3(lib, res, ptrs, want, opts, dev, act, code, workspace,
                       (p_u, p_delta, p_A, p_B, p_C, p_D, p_z, p_bias, p_h0, p_dy, p_dhl),
                       batch, seqlen, d_inner, d_state, lam, u_prev, B_prev, theta)
    p_ck = _ckpt_ptr(ckpt, batch, seqlen, d_inner, d_state, dev)
    size_f = (lib.mamba_scan_bwd_ckpt_workspace_size if ckpt is not None
              else lib.mamba_scan_bwd_workspace_size_ex)
    need = size_f(batch, seqlen, d_inner, d_state, ctypes.byref(opts))
    if need == ctypes.c_size_t(-1).value:
        raise MambaError(4, "mamba_scan_bwd_workspace_size")
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    p_ws = ws.data_ptr() if ws is not None and need > 0 else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    if ckpt is not None:
        st = lib.mamba_scan_bwd_ckpt(p_u, p_delta, p_A, p_B, p_C, p_D, p_z, p_bias, p_h0, p_dy,
                                     p_dhl, p_ck, ptrs["du"], ptrs["ddelta"], ptrs["dA"],
                                     ptrs["dB"], ptrs["dC"], ptrs["dD"], ptrs["dz"],
                                     ptrs["dbias"], ptrs["dh0"], batch, seqlen, d_inner,
                                     d_state, code, p_ws, ws_bytes, ctypes.byref(opts),
                                     _stream(dev))
    else:
        st = lib.mamba_scan_bwd_ex(p_u, p_delta, p_A, p_B, p_C, p_D, p_z, p_bias, p_h0, p_dy,
                                   p_dhl, ptrs["du"], ptrs["ddelta"], ptrs["dA"], ptrs["dB"],
                                   ptrs["dC"], ptrs["dD"], ptrs["dz"], ptrs["dbias"],
                                   ptrs["dh0"], batch, seqlen, d_inner, d_state, code, p_ws,
                                   ws_bytes, ctypes.byref(opts), _stream(dev))
    if st != 0:
        raise MambaError(st, "mamba_scan_bwd")
    return {k: v for k, v in res.items() if k in ("du", "ddelta") or k in want}


def _bwd_m3(lib, res, ptrs, want, opts, dev, act, code, workspace, ins, batch, seqlen, d_inner,
            d_state, lam, u_prev, B_prev, theta):
    """mamba_scan_bwd_ext for mamba_scan_bwd with lam or theta."""
    torch = _torch()
    bld = (batch, seqlen, d_inner)
    ext = ScanExt(_ptr(lam, "lam", bld, act, dev),
                  _ptr(u_prev, "u_prev", (batch, d_inner), act, dev),
                  _ptr(B_prev, "B_prev", (batch, d_state), act, dev),
                  _ptr(theta, "theta", (batch, seqlen, d_state // 2), act, dev))
    if seqlen == 0:  # (only the presence of the options matters)
        ext.lambda_ = ext.lambda_ or (1 if lam is not None else None)
        ext.theta = ext.theta or (1 if theta is not None else None)
    extra = {}
    if lam is not None:
        extra["dlam"] = torch.empty(bld, dtype=act, device=dev)
        extra["du_prev"] = torch.empty((batch, d_inner), dtype=act, device=dev)
        extra["dB_prev"] = torch.empty((batch, d_state), dtype=act, device=dev)
    if theta is not None:
        extra["dtheta"] = torch.empty((batch, seqlen, d_state // 2), dtype=act, device=dev)
    eg = ScanExtGrads(*[(extra[k].data_ptr() if k in extra and extra[k].numel() else None)
                        for k in ("dlam", "du_prev", "dB_prev", "dtheta")])
    need = lib.mamba_scan_bwd_ext_workspace_size(batch, seqlen, d_inner, d_state,
                                                 ctypes.byref(ext), ctypes.byref(opts))
    if need == ctypes.c_size_t(-1).value:
        raise MambaError(4, "mamba_scan_bwd_ext_workspace_size")
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    p_ws = ws.data_ptr() if ws is not None and need > 0 else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib.mamba_scan_bwd_ext(*ins, ptrs["du"], ptrs["ddelta"], ptrs["dA"], ptrs["dB"],
                                ptrs["dC"], ptrs["dD"], ptrs["dz"], ptrs["dbias"], ptrs["dh0"],
                                ctypes.byref(ext), ctypes.byref(eg), batch, seqlen, d_inner,
                                d_state, code, p_ws, ws_bytes, ctypes.byref(opts), _stream(dev))
    if st != 0:
        raise MambaError(st, "mamba_scan_bwd_ext")
    out = {k: v for k, v in res.items() if k in ("du", "ddelta") or k in want}
    out.update(extra)
    return out


_SSD_RELAY = {"auto": 0, "off": 1, "force": 2, "force_withheld": -2}


def _ssd_opts(relay: str, n_spans: int):
    if relay not in _SSD_RELAY:
        raise ValueError(f"relay must be one of {sorted(_SSD_RELAY)}")
    return SsdOpts(_SSD_RELAY[relay], n_spans)


def mamba_ssd_workspace_size(batch: int, seqlen: int, n_heads: int, head_dim: int,
                             d_state: int, dtype, relay: str = "auto", n_spans: int = 0) -> int:
    """Workspace bytes of mamba_ssd_fwd_ex on the current device (0: none needed)."""
    lib = load_library()
    o = _ssd_opts(relay, n_spans)
    n = lib.mamba_ssd_workspace_size(batch, seqlen, n_heads, head_dim, d_state,
                                     _dtype_code_of(dtype), ctypes.byref(o))
    if n == ctypes.c_size_t(-1).value:
        raise MambaError(4, "mamba_ssd_workspace_size")
    return n


def mamba_ssd_fwd(x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None,
                  return_last_state: bool = False, *, out=None, h_last_out=None,
                  head_dim: int = 64, relay: str = "auto", n_spans: int = 0,
                  workspace=None) -> Tuple:
    """Mamba-2 SSD scan (see include/mamba_scan.h): x (batch, seqlen, n_heads * head_dim),
    dt (batch, seqlen, n_heads), A/D/dt_bias (n_heads,) fp32, B/C (batch, seqlen, d_state),
    h0 (batch, n_heads * head_dim, d_state) fp32.  Returns (y, h_last).  relay ("auto",
    "off", "force") and n_spans (0 automatic, 1 none, k spans) as mamba_ssd_opts_t; with
    relay "off" and n_spans 1 this is mamba_ssd_fwd itself.  The workspace they need is
    allocated unless given."""
    torch = _torch()
    lib = load_library()
    if x.dim() != 3 or dt.dim() != 3:
        raise ValueError("x must be (batch, seqlen, d_inner) and dt (batch, seqlen, n_heads)")
    batch, seqlen, d_inner = x.shape
    n_heads = dt.shape[2]
    if n_heads * head_dim != d_inner:
        raise ValueError("d_inner must be n_heads * head_dim")
    d_state = B.shape[2]
    dev, act = x.device, x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    bld = (batch, seqlen, d_inner)
    p_x = _ptr(x, "x", bld, act, dev)
    p_dt = _ptr(dt, "dt", (batch, seqlen, n_heads), act, dev)
    p_A = _ptr(A, "A", (n_heads,), f32, dev)
    p_B = _ptr(B, "B", (batch, seqlen, d_state), act, dev)
    p_C = _ptr(C, "C", (batch, seqlen, d_state), act, dev)
    p_D = _ptr(D, "D", (n_heads,), f32, dev)
    p_z = _ptr(z, "z", bld, act, dev)
    p_bias = _ptr(dt_bias, "dt_bias", (n_heads,), f32, dev)
    p_h0 = _ptr(h0, "h0", (batch, d_inner, d_state), f32, dev)
    y = out if out is not None else torch.empty(bld, dtype=act, device=dev)
    p_y = _ptr(y, "out", bld, act, dev)
    h_last = h_last_out
    if h_last is None and return_last_state:
        h_last = torch.empty((batch, d_inner, d_state), dtype=f32, device=dev)
    p_hl = _ptr(h_last, "h_last_out", (batch, d_inner, d_state), f32, dev)
    opts = _ssd_opts(relay, n_spans)
    if relay == "off" and n_spans == 1 and workspace is None:
        st = lib.mamba_ssd_fwd(p_x, p_dt, p_A, p_B, p_C, p_D, p_z, p_bias, p_h0, p_y, p_hl,
                               batch, seqlen, n_heads, head_dim, d_state, code, _stream(dev))
        if st != 0:
            raise MambaError(st, "mamba_ssd_fwd")
        return y, h_last
    need = lib.mamba_ssd_workspace_size(batch, seqlen, n_heads, head_dim, d_state, code,
                                        ctypes.byref(opts))
    if need == ctypes.c_size_t(-1).value:
        need = 0  # the call itself reports what is wrong
    ws = workspace
    if need > 0 and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    p_ws = ws.data_ptr() if ws is not None and ws.numel() > 0 else None
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    st = lib.mamba_ssd_fwd_ex(p_x, p_dt, p_A, p_B, p_C, p_D, p_z, p_bias, p_h0, p_y, p_hl,
                              batch, seqlen, n_heads, head_dim, d_state, code, p_ws, ws_bytes,
                              ctypes.byref(opts), _stream(dev))
    if st != 0:
        raise MambaError(st, "mamba_ssd_fwd_ex")
    return y, h_last


def mamba_ssd_relay_faults(workspace, batch: int, seqlen: int, n_heads: int, head_dim: int,
                           d_state: int, dtype, relay: str = "auto", n_spans: int = 0,
                           device=None) -> int:
    """Relay hand-offs that timed out in the last mamba_ssd_fwd call given this workspace with
    the same arguments (0 when it planned no relay).  Synchronises the current stream."""
    lib = load_library()
    o = _ssd_opts(relay, n_spans)
    p_ws, ws_bytes = _ws_arg(workspace)
    dev = workspace.device if workspace is not None else device
    out = ctypes.c_uint32(0)
    st = lib.mamba_ssd_relay_faults(p_ws, ws_bytes, batch, seqlen, n_heads, head_dim, d_state,
                                    _dtype_code_of(dtype), ctypes.byref(o), ctypes.byref(out),
                                    _stream(dev) if dev is not None else None)
    if st != 0:
        raise MambaError(st, "mamba_ssd_relay_faults")
    return int(out.value)


def mamba_ssd_state_update(h, x, dt, A, B, C, D=None, z=None, dt_bias=None, *, out=None,
                           head_dim: int = 64):
    """One Mamba-2 SSD decode token (see include/mamba_scan.h): h (batch, n_heads * head_dim,
    d_state) fp32 is updated in place; x, z (batch, n_heads * head_dim), dt (batch, n_heads),
    B, C (batch, d_state), A/D/dt_bias (n_heads,) fp32.  Returns y (batch, n_heads *
    head_dim)."""
    torch = _torch()
    lib = load_library()
    if x.dim() != 2 or dt.dim() != 2 or h.dim() != 3:
        raise ValueError("x must be (batch, d_inner), dt (batch, n_heads), h (batch, d_inner, "
                         "d_state)")
    batch, d_inner = x.shape
    n_heads = dt.shape[1]
    if n_heads * head_dim != d_inner:
        raise ValueError("d_inner must be n_heads * head_dim")
    d_state = h.shape[2]
    dev, act = x.device, x.dtype
    code = _dtype_code(x)
    f32 = torch.float32
    p_h = _ptr(h, "h", (batch, d_inner, d_state), f32, dev)
    p_x = _ptr(x, "x", (batch, d_inner), act, dev)
    p_dt = _ptr(dt, "dt", (batch, n_heads), act, dev)
    p_A = _ptr(A, "A", (n_heads,), f32, dev)
    p_B = _ptr(B, "B", (batch, d_state), act, dev)
    p_C = _ptr(C, "C", (batch, d_state), act, dev)
    p_D = _ptr(D, "D", (n_heads,), f32, dev)
    p_z = _ptr(z, "z", (batch, d_inner), act, dev)
    p_bias = _ptr(dt_bias, "dt_bias", (n_heads,), f32, dev)
    y = out if out is not None else torch.empty((batch, d_inner), dtype=act, device=dev)
    p_y = _ptr(y, "out", (batch, d_inner), act, dev)
    st = lib.mamba_ssd_state_update(p_h, p_x, p_dt, p_A, p_B, p_C, p_D, p_z, p_bias, p_y,
                                    batch, n_heads, head_dim, d_state, code, _stream(dev))
    if st != 0:
        raise MambaError(st, "mamba_ssd_state_update")
    return y
