"""MI355X-native S6 selective scan (Mamba's selective SSM forward pass and single-token decode).

``scan_fwd`` and ``state_update`` call the C ABI of libssm57.so (include/ssm_scan.h) on PyTorch device tensors;
the arithmetic runs entirely in the HIP kernels.  ``inputs`` generates the seeded synthetic workloads.
"""
from __future__ import annotations

from . import _abi
from ._abi import EULER_B, ZOH, SSM_BF16, SSM_F32, SSMError, Params, make_params, workspace_bytes, plan_segments

__all__ = ["scan_fwd", "state_update", "EULER_B", "ZOH", "SSMError", "Params", "make_params", "workspace_bytes",
           "plan_segments", "io_code"]


def io_code(dtype) -> int:
    import torch
    if dtype == torch.float32:
        return SSM_F32
    if dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % (dtype,))


def _addr(t):
    return 0 if t is None else t.data_ptr()


def _stream_handle(stream, device):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def scan_fwd(x, dt, A, B, C, dt_bias=None, Dskip=None, z=None, h0=None, *, y=None, h_final=None, y_dtype=None,
             disc=EULER_B, softplus=True, segments=0, workspace=None, return_final_state=True, stream=None):
    """Selective scan over full sequences on the current HIP stream.

    x, dt, z: (b, D, L); B, C: (b, N, L) -- float32 or bfloat16 (all the same dtype); A: (D, N) float32;
    dt_bias, Dskip: (D,) float32; h0: (b, D, N) float32.  Returns (y, h_final); y has ``y_dtype`` (default: the input
    dtype).  Output and workspace tensors are allocated with torch when not given.
    """
    import torch
    b, D, L = x.shape
    N = A.shape[1]
    io = io_code(x.dtype)
    ydt = x.dtype if y_dtype is None else y_dtype
    p = make_params(b, D, L, N, io, io_code(ydt), disc, softplus, segments)
    for name, t in (("x", x), ("dt", dt), ("B", B), ("C", C), ("z", z), ("A", A), ("dt_bias", dt_bias),
                    ("Dskip", Dskip), ("h0", h0)):
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    if y is None:
        y = torch.empty((b, D, L), dtype=ydt, device=x.device)
    if h_final is None and return_final_state:
        h_final = torch.empty((b, D, N), dtype=torch.float32, device=x.device)
    need = workspace_bytes(p)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _abi.scan_fwd_raw(p, _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B), _addr(C), _addr(Dskip),
                           _addr(z), _addr(h0), _addr(y), _addr(h_final), _addr(workspace), ws_bytes,
                           _stream_handle(stream, x.device))
    _abi.check(st)
    return y, h_final


def state_update(state, x, dt, A, B, C, dt_bias=None, Dskip=None, z=None, *, y=None, y_dtype=None, disc=EULER_B,
                 softplus=True, stream=None):
    """One decode step: state (b, D, N) float32 updated in place; x, dt, z: (b, D); B, C: (b, N).  Returns y (b, D)."""
    import torch
    b, D, N = state.shape
    io = io_code(x.dtype)
    ydt = x.dtype if y_dtype is None else y_dtype
    p = make_params(b, D, 1, N, io, io_code(ydt), disc, softplus, 0)
    if y is None:
        y = torch.empty((b, D), dtype=ydt, device=x.device)
    st = _abi.state_update_raw(p, _addr(state), _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B), _addr(C),
                               _addr(Dskip), _addr(z), _addr(y), _stream_handle(stream, x.device))
    _abi.check(st)
    return y
