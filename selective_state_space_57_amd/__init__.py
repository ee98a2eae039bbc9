"""MI355X-native S6 selective scan (Mamba's selective SSM: forward pass, backward pass and single-token decode).

``scan_fwd``, ``scan_bwd`` and ``state_update`` call the C ABI of libssm57.so (include/ssm_scan.h) on PyTorch device
tensors; ``conv_scan_fwd`` and ``conv_state_update`` do the same with the block's causal depthwise convolution + SiLU
applied to x inside the kernels; ``complex_scan_fwd`` and ``complex_state_update`` run the complex-A variant;
``ssd_fwd`` and ``ssd_state_update`` run the Mamba-2 SSD layer (scalar A per head, bf16 matrix cores).  The
arithmetic runs entirely in the HIP kernels.  ``inputs`` generates the seeded
synthetic workloads.
"""
from __future__ import annotations

from . import _abi
from ._abi import (EULER_B, ZOH, SSM_BF16, SSM_F32, SSMError, Params, make_params, workspace_bytes, plan_segments,
                   bwd_workspace_bytes)

__all__ = ["scan_fwd", "scan_bwd", "state_update", "conv_scan_fwd", "conv_state_update", "complex_scan_fwd",
           "complex_state_update", "conv1d_fwd", "conv1d_bwd", "ssd_fwd", "ssd_state_update", "ssd_workspace_bytes", "EULER_B", "ZOH", "SSMError",
           "Params", "make_params", "workspace_bytes", "bwd_workspace_bytes", "plan_segments", "io_code"]


def io_code(dtype) -> int:
    import torch
    if dtype == torch.float32:
        return SSM_F32
    if dtype == torch.bfloat16:
        return SSM_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % (dtype,))


def _addr(t):
    return 0 if t is None else t.data_ptr()


def _expect(name, t, shape, dtype=None, device=None, optional=True):
    if t is None:
        if not optional:
            raise ValueError("%s is required" % name)
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s: expected dtype %s, got %s" % (name, dtype, t.dtype))
    if device is not None and t.device != device:
        raise ValueError("%s: expected device %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _out_dtype(y, y_dtype, default):
    if y is not None:
        if y_dtype is not None and y_dtype != y.dtype:
            raise TypeError("y_dtype %s does not match the given y (%s)" % (y_dtype, y.dtype))
        return y.dtype
    return default if y_dtype is None else y_dtype


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
    ydt = _out_dtype(y, y_dtype, x.dtype)
    dev = x.device
    f32 = torch.float32
    _expect("x", x, (b, D, L), x.dtype, dev, optional=False)
    _expect("dt", dt, (b, D, L), x.dtype, dev, optional=False)
    _expect("z", z, (b, D, L), x.dtype, dev)
    _expect("B", B, (b, N, L), x.dtype, dev, optional=False)
    _expect("C", C, (b, N, L), x.dtype, dev, optional=False)
    _expect("A", A, (D, N), f32, dev, optional=False)
    _expect("dt_bias", dt_bias, (D,), f32, dev)
    _expect("Dskip", Dskip, (D,), f32, dev)
    _expect("h0", h0, (b, D, N), f32, dev)
    _expect("y", y, (b, D, L), ydt, dev)
    _expect("h_final", h_final, (b, D, N), f32, dev)
    p = make_params(b, D, L, N, io, io_code(ydt), disc, softplus, segments)
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


def scan_bwd(x, dt, A, B, C, dy, dt_bias=None, Dskip=None, z=None, h0=None, dh_final=None, *, disc=EULER_B,
             softplus=True, want_dDskip=True, want_ddt_bias=True, want_dh0=True, workspace=None, out=None,
             stream=None):
    """Gradients of the scan given dy (b, D, L) and optionally dh_final (b, D, N) float32, recomputing every state.

    Inputs as for ``scan_fwd``; dy's dtype (float32 or bfloat16) is also the dtype of dx, ddt, dz.  Returns a dict with
    dx, ddt, dz (None without a gate), dA (D, N), dB, dC (b, N, L), dDskip, ddt_bias (D,), dh0 (b, D, N) -- float32
    except the per-step three.  ``out`` may pass preallocated tensors under the same keys.
    """
    import torch
    b, D, L = x.shape
    N = A.shape[1]
    io = io_code(x.dtype)
    gdt = dy.dtype
    dev = x.device
    f32 = torch.float32
    _expect("x", x, (b, D, L), x.dtype, dev, optional=False)
    _expect("dt", dt, (b, D, L), x.dtype, dev, optional=False)
    _expect("z", z, (b, D, L), x.dtype, dev)
    _expect("B", B, (b, N, L), x.dtype, dev, optional=False)
    _expect("C", C, (b, N, L), x.dtype, dev, optional=False)
    _expect("A", A, (D, N), f32, dev, optional=False)
    _expect("dt_bias", dt_bias, (D,), f32, dev)
    _expect("Dskip", Dskip, (D,), f32, dev)
    _expect("h0", h0, (b, D, N), f32, dev)
    _expect("dy", dy, (b, D, L), gdt, dev, optional=False)
    _expect("dh_final", dh_final, (b, D, N), f32, dev)
    p = make_params(b, D, L, N, io, io_code(gdt), disc, softplus, 0)
    o = dict(out or {})
    shapes = {"dx": ((b, D, L), gdt), "ddt": ((b, D, L), gdt), "dz": ((b, D, L), gdt), "dA": ((D, N), f32),
              "dB": ((b, N, L), f32), "dC": ((b, N, L), f32), "dDskip": ((D,), f32), "ddt_bias": ((D,), f32),
              "dh0": ((b, D, N), f32)}
    wanted = {"dx": True, "ddt": True, "dz": z is not None, "dA": True, "dB": True, "dC": True, "dDskip": want_dDskip,
              "ddt_bias": want_ddt_bias, "dh0": want_dh0}
    for k, (shp, dtp) in shapes.items():
        if not wanted[k]:
            o[k] = None
        elif o.get(k) is None:
            o[k] = torch.empty(shp, dtype=dtp, device=dev)
        else:
            _expect(k, o[k], shp, dtp, dev)
    need = bwd_workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    st = _abi.scan_bwd_raw(p, _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B), _addr(C), _addr(Dskip),
                           _addr(z), _addr(h0), _addr(dy), _addr(dh_final), _addr(o["dx"]), _addr(o["ddt"]),
                           _addr(o["dA"]), _addr(o["dB"]), _addr(o["dC"]), _addr(o["dDskip"]), _addr(o["dz"]),
                           _addr(o["ddt_bias"]), _addr(o["dh0"]), _addr(workspace), ws_bytes,
                           _stream_handle(stream, dev))
    _abi.check(st)
    return o


def _conv_params(conv_w, conv_bias, conv_state, conv_state_out, activation, D, b, dev):
    import torch
    f32 = torch.float32
    if conv_w is None or conv_w.dim() != 2 or conv_w.shape[0] != D:
        raise ValueError("conv_w: expected shape (%d, width)" % D)
    K = conv_w.shape[1]
    _expect("conv_w", conv_w, (D, K), f32, dev, optional=False)
    _expect("conv_bias", conv_bias, (D,), f32, dev)
    _expect("conv_state", conv_state, (b, D, K - 1), f32, dev)
    _expect("conv_state_out", conv_state_out, (b, D, K - 1), f32, dev)
    return _abi.make_conv(_addr(conv_w), K, _addr(conv_bias), _addr(conv_state), _addr(conv_state_out),
                          int(bool(activation)))


def conv_scan_fwd(x, conv_w, dt, A, B, C, dt_bias=None, Dskip=None, z=None, h0=None, *, conv_bias=None,
                  conv_state=None, conv_state_out=None, activation=True, y=None, h_final=None, y_dtype=None,
                  disc=EULER_B, softplus=True, segments=0, workspace=None, return_final_state=True, stream=None):
    """The scan of u = silu(causal_conv(x)) (activation=False: no SiLU): conv_w (D, width <= 4) float32, conv_bias
    (D,), conv_state (b, D, width-1) the inputs before step 0 (oldest first).  ``conv_state_out`` (may be conv_state)
    receives the last width-1 inputs.  Everything else as for ``scan_fwd``.  Returns (y, h_final)."""
    import torch
    b, D, L = x.shape
    N = A.shape[1]
    io = io_code(x.dtype)
    ydt = _out_dtype(y, y_dtype, x.dtype)
    dev = x.device
    f32 = torch.float32
    for name, t, shp, dtp, opt in (("x", x, (b, D, L), x.dtype, False), ("dt", dt, (b, D, L), x.dtype, False),
                                   ("z", z, (b, D, L), x.dtype, True), ("B", B, (b, N, L), x.dtype, False),
                                   ("C", C, (b, N, L), x.dtype, False), ("A", A, (D, N), f32, False),
                                   ("dt_bias", dt_bias, (D,), f32, True), ("Dskip", Dskip, (D,), f32, True),
                                   ("h0", h0, (b, D, N), f32, True), ("y", y, (b, D, L), ydt, True),
                                   ("h_final", h_final, (b, D, N), f32, True)):
        _expect(name, t, shp, dtp, dev, optional=opt)
    cp = _conv_params(conv_w, conv_bias, conv_state, conv_state_out, activation, D, b, dev)
    p = make_params(b, D, L, N, io, io_code(ydt), disc, softplus, segments)
    if y is None:
        y = torch.empty((b, D, L), dtype=ydt, device=dev)
    if h_final is None and return_final_state:
        h_final = torch.empty((b, D, N), dtype=f32, device=dev)
    need = workspace_bytes(p)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _abi.conv_scan_fwd_raw(p, cp, _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B), _addr(C),
                                _addr(Dskip), _addr(z), _addr(h0), _addr(y), _addr(h_final), _addr(workspace),
                                ws_bytes, _stream_handle(stream, dev))
    _abi.check(st)
    return y, h_final


def conv_state_update(state, conv_state, x, conv_w, dt, A, B, C, dt_bias=None, Dskip=None, z=None, *,
                      conv_bias=None, activation=True, y=None, y_dtype=None, disc=EULER_B, softplus=True,
                      stream=None):
    """One decode step through the convolution: state (b, D, N) and conv_state (b, D, width-1) float32 are both updated
    in place; x, dt, z: (b, D); B, C: (b, N).  Returns y (b, D)."""
    import torch
    b, D, N = state.shape
    io = io_code(x.dtype)
    ydt = _out_dtype(y, y_dtype, x.dtype)
    dev = x.device
    f32 = torch.float32
    for name, t, shp, dtp, opt in (("state", state, (b, D, N), f32, False), ("x", x, (b, D), x.dtype, False),
                                   ("dt", dt, (b, D), x.dtype, False), ("z", z, (b, D), x.dtype, True),
                                   ("B", B, (b, N), x.dtype, False), ("C", C, (b, N), x.dtype, False),
                                   ("A", A, (D, N), f32, False), ("dt_bias", dt_bias, (D,), f32, True),
                                   ("Dskip", Dskip, (D,), f32, True), ("y", y, (b, D), ydt, True)):
        _expect(name, t, shp, dtp, dev, optional=opt)
    cp = _conv_params(conv_w, conv_bias, conv_state, conv_state, activation, D, b, dev)
    p = make_params(b, D, 1, N, io, io_code(ydt), disc, softplus, 0)
    if y is None:
        y = torch.empty((b, D), dtype=ydt, device=dev)
    st = _abi.conv_state_update_raw(p, cp, _addr(state), _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B),
                                    _addr(C), _addr(Dskip), _addr(z), _addr(y), _stream_handle(stream, dev))
    _abi.check(st)
    return y


def conv1d_fwd(x, conv_w, conv_bias=None, conv_state=None, *, activation=True, u=None, u_dtype=None, stream=None):
    """The causal depthwise convolution (+ SiLU) alone: x (b, D, L) -> u (b, D, L) (dtype u_dtype, default x's);
    conv_w (D, width) float32, conv_bias (D,), conv_state (b, D, width-1) float32: the inputs before t = 0."""
    import torch
    b, D, L = x.shape
    io = io_code(x.dtype)
    udt = _out_dtype(u, u_dtype, x.dtype)
    dev = x.device
    _expect("x", x, (b, D, L), x.dtype, dev, optional=False)
    _expect("u", u, (b, D, L), udt, dev)
    conv = _conv_params(conv_w, conv_bias, conv_state, None, activation, D, b, dev)
    p = make_params(b, D, L, 16, io, io_code(udt))
    if u is None:
        u = torch.empty((b, D, L), dtype=udt, device=dev)
    _abi.check(_abi.conv1d_fwd_raw(p, conv, _addr(x), _addr(u), _stream_handle(stream, dev)))
    return u


def conv1d_bwd(x, conv_w, du, conv_bias=None, conv_state=None, dstate_out=None, *, activation=True, dx=None,
               stream=None):
    """Backward of conv1d_fwd for dL/du = du (b, D, L) (dtype of dx) and optionally dL/d(returned window)
    dstate_out (b, D, width-1) float32.  Returns dict dx (b, D, L), dweight (D, width), dbias (D,), dstate_in
    (b, D, width-1)."""
    import torch
    b, D, L = x.shape
    io = io_code(x.dtype)
    gdt = du.dtype
    dev = x.device
    f32 = torch.float32
    _expect("x", x, (b, D, L), x.dtype, dev, optional=False)
    _expect("du", du, (b, D, L), gdt, dev, optional=False)
    _expect("dx", dx, (b, D, L), gdt, dev)
    conv = _conv_params(conv_w, conv_bias, conv_state, None, activation, D, b, dev)
    K = conv_w.shape[1]
    _expect("dstate_out", dstate_out, (b, D, K - 1), f32, dev)
    p = make_params(b, D, L, 16, io, io_code(gdt))
    out = {"dx": dx if dx is not None else torch.empty((b, D, L), dtype=gdt, device=dev),
           "dweight": torch.empty((D, K), dtype=f32, device=dev), "dbias": torch.empty((D,), dtype=f32, device=dev),
           "dstate_in": torch.empty((b, D, K - 1), dtype=f32, device=dev)}
    _abi.check(_abi.conv1d_bwd_raw(p, conv, _addr(x), _addr(du), _addr(dstate_out), _addr(out["dx"]),
                                   _addr(out["dweight"]), _addr(out["dbias"]),
                                   _addr(out["dstate_in"]) if K > 1 else 0, _stream_handle(stream, dev)))
    return out


def complex_scan_fwd(x, dt, A, B, C, dt_bias=None, Dskip=None, z=None, h0=None, *, y=None, h_final=None,
                     y_dtype=None, disc=EULER_B, softplus=True, return_final_state=True, stream=None):
    """Complex diagonal A: A (D, N, 2) float32 and B, C (b, N, L, 2) in x's dtype hold (re, im) pairs; h0 / h_final
    (b, D, N, 2) float32.  y = Re(sum C h) + D x, gated.  Returns (y, h_final)."""
    import torch
    b, D, L = x.shape
    N = A.shape[1]
    io = io_code(x.dtype)
    ydt = _out_dtype(y, y_dtype, x.dtype)
    dev = x.device
    f32 = torch.float32
    for name, t, shp, dtp, opt in (("x", x, (b, D, L), x.dtype, False), ("dt", dt, (b, D, L), x.dtype, False),
                                   ("z", z, (b, D, L), x.dtype, True), ("B", B, (b, N, L, 2), x.dtype, False),
                                   ("C", C, (b, N, L, 2), x.dtype, False), ("A", A, (D, N, 2), f32, False),
                                   ("dt_bias", dt_bias, (D,), f32, True), ("Dskip", Dskip, (D,), f32, True),
                                   ("h0", h0, (b, D, N, 2), f32, True), ("y", y, (b, D, L), ydt, True),
                                   ("h_final", h_final, (b, D, N, 2), f32, True)):
        _expect(name, t, shp, dtp, dev, optional=opt)
    p = make_params(b, D, L, N, io, io_code(ydt), disc, softplus, 0)
    if y is None:
        y = torch.empty((b, D, L), dtype=ydt, device=dev)
    if h_final is None and return_final_state:
        h_final = torch.empty((b, D, N, 2), dtype=f32, device=dev)
    st = _abi.complex_scan_fwd_raw(p, _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B), _addr(C),
                                   _addr(Dskip), _addr(z), _addr(h0), _addr(y), _addr(h_final),
                                   _stream_handle(stream, dev))
    _abi.check(st)
    return y, h_final


def complex_state_update(state, x, dt, A, B, C, dt_bias=None, Dskip=None, z=None, *, y=None, y_dtype=None,
                         disc=EULER_B, softplus=True, stream=None):
    """One complex decode step: state (b, D, N, 2) float32 in place; x, dt, z (b, D); B, C (b, N, 2).  Returns y."""
    import torch
    b, D, N = state.shape[:3]
    io = io_code(x.dtype)
    ydt = _out_dtype(y, y_dtype, x.dtype)
    dev = x.device
    f32 = torch.float32
    for name, t, shp, dtp, opt in (("state", state, (b, D, N, 2), f32, False), ("x", x, (b, D), x.dtype, False),
                                   ("dt", dt, (b, D), x.dtype, False), ("z", z, (b, D), x.dtype, True),
                                   ("B", B, (b, N, 2), x.dtype, False), ("C", C, (b, N, 2), x.dtype, False),
                                   ("A", A, (D, N, 2), f32, False), ("dt_bias", dt_bias, (D,), f32, True),
                                   ("Dskip", Dskip, (D,), f32, True), ("y", y, (b, D), ydt, True)):
        _expect(name, t, shp, dtp, dev, optional=opt)
    p = make_params(b, D, 1, N, io, io_code(ydt), disc, softplus, 0)
    if y is None:
        y = torch.empty((b, D), dtype=ydt, device=dev)
    st = _abi.complex_state_update_raw(p, _addr(state), _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B),
                                       _addr(C), _addr(Dskip), _addr(z), _addr(y), _stream_handle(stream, dev))
    _abi.check(st)
    return y


def state_update(state, x, dt, A, B, C, dt_bias=None, Dskip=None, z=None, *, y=None, y_dtype=None, disc=EULER_B,
                 softplus=True, stream=None):
    """One decode step: state (b, D, N) float32 updated in place; x, dt, z: (b, D); B, C: (b, N).  Returns y (b, D)."""
    import torch
    b, D, N = state.shape
    io = io_code(x.dtype)
    ydt = _out_dtype(y, y_dtype, x.dtype)
    dev = x.device
    f32 = torch.float32
    _expect("state", state, (b, D, N), f32, dev, optional=False)
    _expect("x", x, (b, D), x.dtype, dev, optional=False)
    _expect("dt", dt, (b, D), x.dtype, dev, optional=False)
    _expect("z", z, (b, D), x.dtype, dev)
    _expect("B", B, (b, N), x.dtype, dev, optional=False)
    _expect("C", C, (b, N), x.dtype, dev, optional=False)
    _expect("A", A, (D, N), f32, dev, optional=False)
    _expect("dt_bias", dt_bias, (D,), f32, dev)
    _expect("Dskip", Dskip, (D,), f32, dev)
    _expect("y", y, (b, D), ydt, dev)
    p = make_params(b, D, 1, N, io, io_code(ydt), disc, softplus, 0)
    if y is None:
        y = torch.empty((b, D), dtype=ydt, device=x.device)
    st = _abi.state_update_raw(p, _addr(state), _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B), _addr(C),
                               _addr(Dskip), _addr(z), _addr(y), _stream_handle(stream, x.device))
    _abi.check(st)
    return y


def ssd_fwd(x, dt, A, B, C, dt_bias=None, Dskip=None, z=None, h0=None, *, y=None, h_final=None, y_dtype=None,
            disc=EULER_B, softplus=True, segments=0, workspace=None, return_final_state=True, stream=None):
    """Mamba-2 SSD layer.  x, z (b, L, H, P) bfloat16; dt (b, L, H) bfloat16; B, C (b, L, G, N) bfloat16; A, dt_bias,
    Dskip (H,) float32; h0 / h_final (b, H, P, N) float32.  segments: 0 = the library's choice of L-segments.
    workspace: a uint8 device tensor of at least ssd_workspace_bytes(...) bytes (allocated here when None).
    Returns (y (b, L, H, P), h_final)."""
    import torch
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    io = io_code(x.dtype)
    ydt = _out_dtype(y, y_dtype, x.dtype)
    dev = x.device
    f32 = torch.float32
    for name, t, shp, dtp, opt in (("x", x, (b, L, H, P), x.dtype, False), ("dt", dt, (b, L, H), x.dtype, False),
                                   ("z", z, (b, L, H, P), x.dtype, True), ("B", B, (b, L, G, N), x.dtype, False),
                                   ("C", C, (b, L, G, N), x.dtype, False), ("A", A, (H,), f32, False),
                                   ("dt_bias", dt_bias, (H,), f32, True), ("Dskip", Dskip, (H,), f32, True),
                                   ("h0", h0, (b, H, P, N), f32, True), ("y", y, (b, L, H, P), ydt, True),
                                   ("h_final", h_final, (b, H, P, N), f32, True)):
        _expect(name, t, shp, dtp, dev, optional=opt)
    p = _abi.make_ssd_params(b, L, H, P, G, N, io, io_code(ydt), disc, softplus, segments)
    if y is None:
        y = torch.empty((b, L, H, P), dtype=ydt, device=dev)
    if h_final is None and return_final_state:
        h_final = torch.empty((b, H, P, N), dtype=f32, device=dev)
    ws_need = _abi.ssd_workspace_bytes(p)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _abi.ssd_fwd_raw(p, _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B), _addr(C), _addr(Dskip),
                          _addr(z), _addr(h0), _addr(y), _addr(h_final), _addr(workspace), ws_bytes,
                          _stream_handle(stream, dev))
    _abi.check(st)
    return y, h_final


def ssd_workspace_bytes(b, L, H, P, G, N, segments=0) -> int:
    """Workspace bytes ssd_fwd needs for these sizes (bf16 io)."""
    return _abi.ssd_workspace_bytes(_abi.make_ssd_params(b, L, H, P, G, N, SSM_BF16, SSM_BF16, segments=segments))


def ssd_state_update(state, x, dt, A, B, C, dt_bias=None, Dskip=None, z=None, *, y=None, y_dtype=None, disc=EULER_B,
                     softplus=True, stream=None):
    """One SSD decode step: state (b, H, P, N) float32 updated in place; x, z (b, H, P); dt (b, H); B, C (b, G, N).
    Returns y (b, H, P)."""
    import torch
    b, H, P, N = state.shape
    G = B.shape[1]
    io = io_code(x.dtype)
    ydt = _out_dtype(y, y_dtype, x.dtype)
    dev = x.device
    f32 = torch.float32
    for name, t, shp, dtp, opt in (("state", state, (b, H, P, N), f32, False), ("x", x, (b, H, P), x.dtype, False),
                                   ("dt", dt, (b, H), x.dtype, False), ("z", z, (b, H, P), x.dtype, True),
                                   ("B", B, (b, G, N), x.dtype, False), ("C", C, (b, G, N), x.dtype, False),
                                   ("A", A, (H,), f32, False), ("dt_bias", dt_bias, (H,), f32, True),
                                   ("Dskip", Dskip, (H,), f32, True), ("y", y, (b, H, P), ydt, True)):
        _expect(name, t, shp, dtp, dev, optional=opt)
    p = _abi.make_ssd_params(b, 1, H, P, G, N, io, io_code(ydt), disc, softplus)
    if y is None:
        y = torch.empty((b, H, P), dtype=ydt, device=dev)
    st = _abi.ssd_state_update_raw(p, _addr(state), _addr(x), _addr(dt), _addr(dt_bias), _addr(A), _addr(B),
                                   _addr(C), _addr(Dskip), _addr(z), _addr(y), _stream_handle(stream, dev))
    _abi.check(st)
    return y
