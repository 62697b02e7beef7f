"""Python binding of libssmscan.so, the gfx950 selective-scan forward and backward.

Argument marshalling only: every step of the scan runs in the HIP kernels behind the C
ABI of include/ssm_scan.h. PyTorch supplies device memory and the current stream.

    out, final_state = scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                            delta_softplus=False, h0=None)
    out, final_state, chunk_states = scan_train(...same arguments...)
    grads = scan_backward(u, delta, A, B, C, chunk_states, dout, D=None, z=None,
                          delta_bias=None, delta_softplus=False, dfinal=None)
    out, final_state = ssd(x, dt, A, B, C, D=None, z=None, dt_bias=None,
                           dt_softplus=False, h0=None, mask=None)      # Mamba-2, ssm_ssd.h
    out, final_state = selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                                      delta_softplus=False, h0=None, mask=None)
                       # differentiable: scan_train forward, scan_backward under autograd

Inputs may be strided views: the functions above copy them to contiguous tensors first
(outputs passed in must be contiguous). The ``ssm_scan_*`` functions are the raw C entry
points (pointers as ints). If the library has not been built this module raises on first
use; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

from .build import LIB_PATH

SSM_IO_F32 = 0
SSM_IO_BF16 = 1
SSM_DELTA_SOFTPLUS = 1 << 4
SSM_INITIAL_STATE = 1 << 5
SSM_WAVES_PER_CHANNEL_1 = 1 << 8
SSM_WAVES_PER_CHANNEL_2 = 1 << 9
SSM_BWD_UNSPLIT = 1 << 10

SSM_OK = 0
SSM_ERR_INVALID_ARG = -1
SSM_ERR_UNSUPPORTED = -2
SSM_ERR_MISALIGNED = -3
SSM_ERR_HIP = -4
SSM_ERR_SCRATCH_TOO_SMALL = -5

SSM_SSD_NOALLOC_SCRATCH_BYTES = 32 << 20

SSM_CKPT_INTERVAL = 256

EXPORTED = ("ssm_scan_fwd", "ssm_scan_strerror", "ssm_scan_abi_version",
            "ssm_scan_debug_wave_combine", "ssm_scan_ckpt_count", "ssm_scan_fwd_ckpt",
            "ssm_scan_fwd_masked", "ssm_scan_bwd", "ssm_scan_bwd_workspace_bytes",
            "ssm_ssd_workspace_bytes", "ssm_ssd_fwd", "ssm_ssd_fwd_noalloc")

_lib = None


class SsmScanError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"ssm_scan call failed ({status}): {ssm_scan_strerror(status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libssmscan.so (built in-tree by build.py). Raises if it is missing.

    torch is imported first: PyTorch for ROCm ships its own HIP runtime (SONAME
    libamdhip64.so.7), and the library must bind to that one, the runtime that owns the
    tensors and streams it is given. Loaded before torch, the library would pull in the
    system runtime of the same SONAME and torch would then load its own copy as well: two
    HIP runtimes in one process, and the library's would find no device."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python -m selective_state_space_fwd_amd.build)")
    import torch  # noqa: F401  (binds the library to torch's HIP runtime; see above)
    L = ctypes.CDLL(LIB_PATH)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.ssm_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, vp,
                               i64, i64, i64, i64, vp]
    L.ssm_scan_fwd.restype = ctypes.c_int
    L.ssm_scan_strerror.argtypes = [ctypes.c_int]
    L.ssm_scan_strerror.restype = ctypes.c_char_p
    L.ssm_scan_abi_version.argtypes = []
    L.ssm_scan_abi_version.restype = ctypes.c_int
    L.ssm_scan_debug_wave_combine.argtypes = [vp, vp, vp, vp, i64, vp]
    L.ssm_scan_debug_wave_combine.restype = ctypes.c_int
    L.ssm_scan_ckpt_count.argtypes = [i64]
    L.ssm_scan_ckpt_count.restype = i64
    L.ssm_scan_fwd_ckpt.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, vp, vp,
                                    i64, i64, i64, i64, vp]
    L.ssm_scan_fwd_ckpt.restype = ctypes.c_int
    L.ssm_scan_fwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp,
                                      vp, vp, i64, i64, i64, i64, vp]
    L.ssm_scan_fwd_masked.restype = ctypes.c_int
    L.ssm_scan_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, vp, vp,
                               vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                               vp]
    L.ssm_scan_bwd.restype = ctypes.c_int
    L.ssm_scan_bwd_workspace_bytes.argtypes = [i64, i64, i64, i64, ctypes.c_uint32]
    L.ssm_scan_bwd_workspace_bytes.restype = i64
    L.ssm_ssd_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.ssm_ssd_workspace_bytes.restype = i64
    L.ssm_ssd_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, vp, vp,
                              i64, i64, i64, i64, i64, i64, vp]
    L.ssm_ssd_fwd.restype = ctypes.c_int
    L.ssm_ssd_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp, vp,
                                      i64, i64, i64, i64, i64, vp]
    L.ssm_ssd_fwd_noalloc.restype = ctypes.c_int
    _lib = L
    return L


def ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias, flags, out, final_state,
                 batch, dim, dstate, seqlen, stream) -> int:
    """Raw C entry point; pointers and stream are ints (0/None for NULL)."""
    return lib().ssm_scan_fwd(u, delta, A, B, C, D, z, delta_bias, flags, out, final_state,
                              batch, dim, dstate, seqlen, stream)


def ssm_scan_fwd_ckpt(u, delta, A, B, C, D, z, delta_bias, flags, out, final_state,
                      chunk_states, batch, dim, dstate, seqlen, stream) -> int:
    return lib().ssm_scan_fwd_ckpt(u, delta, A, B, C, D, z, delta_bias, flags, out, final_state,
                                   chunk_states, batch, dim, dstate, seqlen, stream)


def ssm_scan_ckpt_count(seqlen: int) -> int:
    return lib().ssm_scan_ckpt_count(seqlen)


def ssm_scan_fwd_masked(u, delta, A, B, C, D, z, delta_bias, mask, flags, out, final_state,
                        chunk_states, batch, dim, dstate, seqlen, stream) -> int:
    return lib().ssm_scan_fwd_masked(u, delta, A, B, C, D, z, delta_bias, mask, flags, out,
                                     final_state, chunk_states, batch, dim, dstate, seqlen,
                                     stream)


def ssm_scan_bwd(u, delta, A, B, C, D, z, delta_bias, mask, flags, chunk_states, dout, dfinal,
                 du, ddelta, dA, dB, dC, dD, dz, dbias, dh0, workspace, workspace_bytes, batch,
                 dim, dstate, seqlen, stream) -> int:
    return lib().ssm_scan_bwd(u, delta, A, B, C, D, z, delta_bias, mask, flags, chunk_states,
                              dout, dfinal, du, ddelta, dA, dB, dC, dD, dz, dbias, dh0,
                              workspace, workspace_bytes, batch, dim, dstate, seqlen, stream)


def ssm_scan_bwd_workspace_bytes(batch, dim, dstate, seqlen, flags) -> int:
    return lib().ssm_scan_bwd_workspace_bytes(batch, dim, dstate, seqlen, flags)


def ssm_scan_strerror(status: int) -> str:
    return lib().ssm_scan_strerror(status).decode()


def ssm_scan_abi_version() -> int:
    return lib().ssm_scan_abi_version()


def ssm_scan_debug_wave_combine(a, b, a_out, b_out, groups, stream) -> int:
    return lib().ssm_scan_debug_wave_combine(a, b, a_out, b_out, groups, stream)


def ssm_ssd_workspace_bytes(batch, nheads, dstate, seqlen) -> int:
    return lib().ssm_ssd_workspace_bytes(batch, nheads, dstate, seqlen)


def ssm_ssd_fwd(x, dt, A, B, C, D, z, dt_bias, mask, flags, out, final_state, workspace,
                workspace_bytes, batch, nheads, headdim, dstate, seqlen, stream) -> int:
    return lib().ssm_ssd_fwd(x, dt, A, B, C, D, z, dt_bias, mask, flags, out, final_state,
                             workspace, workspace_bytes, batch, nheads, headdim, dstate,
                             seqlen, stream)


def ssm_ssd_fwd_noalloc(x, dt, A, B, C, D, z, dt_bias, mask, flags, out, final_state, batch,
                        nheads, headdim, dstate, seqlen, stream) -> int:
    """Raw C entry point of the allocation-free Mamba-2 forward (its workspace is the
    library's static device buffer of SSM_SSD_NOALLOC_SCRATCH_BYTES)."""
    return lib().ssm_ssd_fwd_noalloc(x, dt, A, B, C, D, z, dt_bias, mask, flags, out,
                                     final_state, batch, nheads, headdim, dstate, seqlen, stream)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream_of(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def _dense(*tensors):
    """Inputs as C-contiguous tensors (a strided view, such as a slice of a projection's
    output, is copied once here; the C ABI takes contiguous arrays only)."""
    return tuple(t if t is None or t.is_contiguous() else t.contiguous() for t in tensors)


def _check(u, delta, A, B, C, D, z, delta_bias, h0):
    """Dtype, device, contiguity and shape checks; returns (flags, batch, dim, dstate, seqlen)."""
    import torch

    io = u.dtype
    if io == torch.float32:
        flags = SSM_IO_F32
    elif io == torch.bfloat16:
        flags = SSM_IO_BF16
    else:
        raise TypeError(f"unsupported storage dtype {io}")
    streamed = [("u", u), ("delta", delta), ("B", B), ("C", C)] + ([("z", z)] if z is not None else [])
    for name, t in streamed:
        if t.dtype != io:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {io}")
    params = [("A", A)] + [(n, t) for n, t in (("D", D), ("delta_bias", delta_bias), ("h0", h0))
                           if t is not None]
    for name, t in params:
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    for name, t in streamed + params:
        if not t.is_cuda or t.device != u.device:
            raise ValueError(f"{name} must be on {u.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if u.dim() != 3 or A.dim() != 2:
        raise ValueError("u must be [batch, dim, seqlen] and A [dim, dstate]")
    batch, dim, seqlen = u.shape
    dstate = A.shape[1]
    want = {"delta": (batch, dim, seqlen), "z": (batch, dim, seqlen),
            "B": (batch, dstate, seqlen), "C": (batch, dstate, seqlen),
            "A": (dim, dstate), "D": (dim,), "delta_bias": (dim,), "h0": (batch, dim, dstate)}
    for name, t in streamed + params:
        if name in want and tuple(t.shape) != want[name]:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {want[name]}")
    return flags, batch, dim, dstate, seqlen


def _check_mask(mask, u, batch, seqlen):
    import torch

    if mask is None:
        return None
    if (tuple(mask.shape) != (batch, seqlen) or mask.dtype not in (torch.uint8, torch.bool)
            or mask.device != u.device or not mask.is_contiguous()):
        raise ValueError(f"mask must be a contiguous uint8/bool {(batch, seqlen)} tensor on "
                         f"{u.device}")
    return mask


def _hint_flags(waves_per_channel) -> int:
    if waves_per_channel is None:
        return 0
    if waves_per_channel == 1:
        return SSM_WAVES_PER_CHANNEL_1
    if waves_per_channel == 2:
        return SSM_WAVES_PER_CHANNEL_2
    raise ValueError("waves_per_channel must be None, 1 or 2")


def _forward(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, out, final_state,
             return_final_state, save_states, mask=None, waves_per_channel=None):
    import torch

    u, delta, A, B, C, D, z, delta_bias, h0, mask = _dense(u, delta, A, B, C, D, z, delta_bias,
                                                           h0, mask)
    flags, batch, dim, dstate, seqlen = _check(u, delta, A, B, C, D, z, delta_bias, h0)
    mask = _check_mask(mask, u, batch, seqlen)
    io = u.dtype
    if out is not None and (tuple(out.shape) != tuple(u.shape) or out.dtype != io
                            or out.device != u.device or not out.is_contiguous()):
        raise ValueError("out must be a contiguous tensor like u")
    if final_state is not None and (tuple(final_state.shape) != (batch, dim, dstate)
                                    or final_state.dtype != torch.float32
                                    or final_state.device != u.device
                                    or not final_state.is_contiguous()):
        raise ValueError("final_state must be a contiguous float32 [batch, dim, dstate] tensor")
    if out is None:
        out = torch.empty_like(u)
    if h0 is not None:
        flags |= SSM_INITIAL_STATE
        if final_state is None:
            final_state = h0.clone()
        elif final_state.data_ptr() != h0.data_ptr():
            final_state.copy_(h0)
    elif final_state is None and return_final_state:
        final_state = torch.empty((batch, dim, dstate), device=u.device, dtype=torch.float32)
    if delta_softplus:
        flags |= SSM_DELTA_SOFTPLUS
    flags |= _hint_flags(waves_per_channel)
    args = (_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(delta_bias),
            flags, _ptr(out), _ptr(final_state))
    sizes = (batch, dim, dstate, seqlen, _stream_of(u.device))
    states = None
    if save_states:
        states = torch.empty((batch, dim, ssm_scan_ckpt_count(seqlen), dstate), device=u.device,
                             dtype=torch.float32)
    if mask is not None:
        status = ssm_scan_fwd_masked(*args[:8], _ptr(mask), *args[8:], _ptr(states), *sizes)
    elif save_states:
        status = ssm_scan_fwd_ckpt(*args, _ptr(states), *sizes)
    else:
        status = ssm_scan_fwd(*args, *sizes)
    if status != SSM_OK:
        raise SsmScanError(status)
    return out, final_state, states


def scan(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus: bool = False,
         h0=None, out=None, final_state=None, return_final_state: bool = True, mask=None,
         waves_per_channel=None) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """Selective-scan forward on the GPU.

    u, delta, z: [batch, dim, seqlen]; B, C: [batch, dstate, seqlen] (float32 or bfloat16,
    all the same dtype); A: [dim, dstate], D and delta_bias: [dim], h0: [batch, dim,
    dstate] (float32); mask: [batch, seqlen] uint8/bool, 0 = padding step (the state is
    kept). waves_per_channel: None (the library chooses), 1 or 2 (fp32 only): the
    SSM_WAVES_PER_CHANNEL_* launch-shape hint. Returns (out, final_state); out has u's dtype.
    """
    out, fin, _ = _forward(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, out,
                           final_state, return_final_state, False, mask, waves_per_channel)
    return out, fin


def scan_train(u, delta, A, B, C, D=None, z=None, delta_bias=None, delta_softplus: bool = False,
               h0=None, mask=None, waves_per_channel=None):
    """``scan`` that also returns the states the backward pass restarts from:
    (out, final_state, chunk_states [batch, dim, ceil(seqlen / 256), dstate] float32)."""
    return _forward(u, delta, A, B, C, D, z, delta_bias, delta_softplus, h0, None, None, True,
                    True, mask, waves_per_channel)


def scan_backward(u, delta, A, B, C, chunk_states, dout, D=None, z=None, delta_bias=None,
                  delta_softplus: bool = False, dfinal=None, want_dh0: bool = True, mask=None,
                  deterministic: bool = True, workspace=None, unsplit: bool = False
                  ) -> Dict[str, Optional["torch.Tensor"]]:
    """Gradients of sum(dout * out) + sum(dfinal * final_state) for the forward on the same
    inputs. Returns du, ddelta, dz (u's dtype), dA, dB, dC, dD, dbias, dh0 (float32; None
    where the input is absent or, for dh0, not wanted).

    deterministic: sum dA, dB, dC, dD and dbias through a workspace in a fixed order
    (bitwise reproducible; ssm_scan_bwd_workspace_bytes of device memory, allocated here
    unless ``workspace``, a uint8 device tensor at least that large, is given); False: float
    atomics, no workspace. unsplit: SSM_BWD_UNSPLIT (each channel's whole sequence in one
    workgroup, no segments)."""
    import torch

    u, delta, A, B, C, D, z, delta_bias, mask, chunk_states, dout, dfinal = _dense(
        u, delta, A, B, C, D, z, delta_bias, mask, chunk_states, dout, dfinal)
    flags, batch, dim, dstate, seqlen = _check(u, delta, A, B, C, D, z, delta_bias, None)
    mask = _check_mask(mask, u, batch, seqlen)
    n_ck = ssm_scan_ckpt_count(seqlen)
    if (tuple(chunk_states.shape) != (batch, dim, n_ck, dstate)
            or chunk_states.dtype != torch.float32 or not chunk_states.is_contiguous()
            or chunk_states.device != u.device):
        raise ValueError(f"chunk_states must be float32 {(batch, dim, n_ck, dstate)}")
    if tuple(dout.shape) != tuple(u.shape) or dout.dtype != u.dtype or not dout.is_contiguous() \
            or dout.device != u.device:
        raise ValueError("dout must be a contiguous tensor like u")
    if dfinal is not None and (tuple(dfinal.shape) != (batch, dim, dstate)
                               or dfinal.dtype != torch.float32 or not dfinal.is_contiguous()
                               or dfinal.device != u.device):
        raise ValueError("dfinal must be a contiguous float32 [batch, dim, dstate] tensor")
    if delta_softplus:
        flags |= SSM_DELTA_SOFTPLUS
    if unsplit:
        flags |= SSM_BWD_UNSPLIT
    dev = u.device
    f32 = dict(device=dev, dtype=torch.float32)
    g = {"du": torch.empty_like(u), "ddelta": torch.empty_like(u),
         "dz": None if z is None else torch.empty_like(u),
         "dA": torch.empty((dim, dstate), **f32), "dB": torch.empty((batch, dstate, seqlen), **f32),
         "dC": torch.empty((batch, dstate, seqlen), **f32),
         "dD": None if D is None else torch.empty((dim,), **f32),
         "dbias": None if delta_bias is None else torch.empty((dim,), **f32),
         "dh0": torch.empty((batch, dim, dstate), **f32) if want_dh0 else None}
    ws_bytes = 0
    if deterministic:
        need = ssm_scan_bwd_workspace_bytes(batch, dim, dstate, seqlen, flags)
        if need < 0:
            raise SsmScanError(SSM_ERR_UNSUPPORTED)
        if workspace is None:
            workspace = torch.empty((max(need, 1),), device=dev, dtype=torch.uint8)
        elif (workspace.dtype != torch.uint8 or workspace.device != dev
              or not workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous uint8 tensor on u's device")
        ws_bytes = workspace.numel()
    else:
        workspace = None
    status = ssm_scan_bwd(_ptr(u), _ptr(delta), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                          _ptr(delta_bias), _ptr(mask), flags, _ptr(chunk_states), _ptr(dout),
                          _ptr(dfinal),
                          _ptr(g["du"]), _ptr(g["ddelta"]), _ptr(g["dA"]), _ptr(g["dB"]),
                          _ptr(g["dC"]), _ptr(g["dD"]), _ptr(g["dz"]), _ptr(g["dbias"]),
                          _ptr(g["dh0"]), _ptr(workspace), ws_bytes, batch, dim, dstate, seqlen,
                          _stream_of(dev))
    if status != SSM_OK:
        raise SsmScanError(status)
    return g


_autograd_fn = None


def _selective_scan_function():
    """The torch.autograd.Function behind ``selective_scan`` (built on first use, so that
    importing this module does not import torch)."""
    global _autograd_fn
    if _autograd_fn is not None:
        return _autograd_fn
    import torch

    class SelectiveScan(torch.autograd.Function):
        @staticmethod
        def forward(ctx, u, delta, A, B, C, D, z, delta_bias, h0, mask, delta_softplus):
            out, fin, states = scan_train(u, delta, A, B, C, D=D, z=z, delta_bias=delta_bias,
                                          delta_softplus=delta_softplus, h0=h0, mask=mask)
            ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, states)
            ctx.mask = mask
            ctx.delta_softplus = delta_softplus
            ctx.has_h0 = h0 is not None
            return out, fin

        @staticmethod
        def backward(ctx, dout, dfin):
            u, delta, A, B, C, D, z, delta_bias, states = ctx.saved_tensors
            dout = torch.zeros_like(u) if dout is None else dout.to(u.dtype).contiguous()
            dfin = None if dfin is None else dfin.to(torch.float32).contiguous()
            g = scan_backward(u, delta, A, B, C, states, dout, D=D, z=z, delta_bias=delta_bias,
                              delta_softplus=ctx.delta_softplus, dfinal=dfin,
                              want_dh0=ctx.has_h0 and ctx.needs_input_grad[8], mask=ctx.mask)
            cast = lambda grad, like: None if grad is None else grad.to(like.dtype)
            return (g["du"], g["ddelta"], cast(g["dA"], A), cast(g["dB"], B), cast(g["dC"], C),
                    g["dD"], g["dz"], g["dbias"], g["dh0"], None, None)

    _autograd_fn = SelectiveScan
    return SelectiveScan


def selective_scan(u, delta, A, B, C, D=None, z=None, delta_bias=None,
                   delta_softplus: bool = False, h0=None, mask=None
                   ) -> Tuple["torch.Tensor", "torch.Tensor"]:
    """Differentiable selective scan: (out, final_state) as ``scan``, with gradients for u,
    delta, A, B, C, D, z, delta_bias and h0 through autograd. The forward keeps the state
    every 256 steps (``scan_train``); the backward restarts the scan from them
    (``scan_backward``, reproducible workspace sums). mask is not differentiable."""
    return _selective_scan_function().apply(u, delta, A, B, C, D, z, delta_bias, h0, mask,
                                            bool(delta_softplus))


def ssd(x, dt, A, B, C, D=None, z=None, dt_bias=None, dt_softplus: bool = False, h0=None,
        mask=None, out=None, final_state=None, return_final_state: bool = True,
        workspace=None) -> Tuple["torch.Tensor", Optional["torch.Tensor"]]:
    """Mamba-2 (SSD) forward on the GPU: one scalar A and one step size per head.

    x, z: [batch, nheads*headdim, seqlen] bfloat16; dt: [batch, nheads, seqlen] bfloat16;
    A, dt_bias: [nheads] float32; B, C: [batch, dstate, seqlen] bfloat16; D:
    [nheads*headdim] float32; h0: [batch, nheads*headdim, dstate] float32; mask:
    [batch, seqlen] uint8/bool. dstate is 64, 128 or 256 and headdim a multiple of 16.
    workspace: a uint8 device tensor of at least ssm_ssd_workspace_bytes(...) bytes
    (allocated per call when None). Returns (out, final_state).
    """
    import torch

    x, dt, A, B, C, D, z, dt_bias, h0, mask = _dense(x, dt, A, B, C, D, z, dt_bias, h0, mask)
    if x.dtype != torch.bfloat16:
        raise TypeError("ssd takes bfloat16 x, dt, B, C and z")
    if x.dim() != 3 or A.dim() != 1:
        raise ValueError("x must be [batch, nheads*headdim, seqlen] and A [nheads]")
    batch, dim, seqlen = x.shape
    nheads = A.shape[0]
    if nheads == 0 or dim % nheads:
        raise ValueError("the channel count must be a multiple of the head count")
    headdim = dim // nheads
    dstate = B.shape[1] if B.dim() == 3 else -1
    want = {"dt": (dt, (batch, nheads, seqlen), torch.bfloat16),
            "B": (B, (batch, dstate, seqlen), torch.bfloat16),
            "C": (C, (batch, dstate, seqlen), torch.bfloat16),
            "A": (A, (nheads,), torch.float32),
            "z": (z, (batch, dim, seqlen), torch.bfloat16),
            "D": (D, (dim,), torch.float32),
            "dt_bias": (dt_bias, (nheads,), torch.float32),
            "h0": (h0, (batch, dim, dstate), torch.float32)}
    for name, (t, shape, dtype) in want.items():
        if t is None:
            continue
        if tuple(t.shape) != shape or t.dtype != dtype:
            raise ValueError(f"{name} must be {dtype} {shape}, got {t.dtype} {tuple(t.shape)}")
        if t.device != x.device or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous on {x.device}")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")
    mask = _check_mask(mask, x, batch, seqlen)
    flags = SSM_IO_BF16 | (SSM_DELTA_SOFTPLUS if dt_softplus else 0)
    if out is None:
        out = torch.empty_like(x)
    if h0 is not None:
        flags |= SSM_INITIAL_STATE
        if final_state is None:
            final_state = h0.clone()
        elif final_state.data_ptr() != h0.data_ptr():
            final_state.copy_(h0)
    elif final_state is None and return_final_state:
        final_state = torch.empty((batch, dim, dstate), device=x.device, dtype=torch.float32)
    need = ssm_ssd_workspace_bytes(batch, nheads, max(dstate, 0), seqlen)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), device=x.device, dtype=torch.uint8)
    status = ssm_ssd_fwd(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(z),
                         _ptr(dt_bias), _ptr(mask), flags, _ptr(out), _ptr(final_state),
                         _ptr(workspace), workspace.numel(), batch, nheads, headdim, dstate,
                         seqlen, _stream_of(x.device))
    if status != SSM_OK:
        raise SsmScanError(status)
    return out, final_state
