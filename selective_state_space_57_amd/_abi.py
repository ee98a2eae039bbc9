"""ctypes binding of libssm57.so (the C ABI in include/ssm_scan.h).

Argument marshalling only: every step of the scan runs in the HIP kernels.  PyTorch supplies device memory and the
stream.  There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssm57.so")

SSM_F32, SSM_BF16 = 0, 1
EULER_B, ZOH = 0, 1
STATUS = {0: "SSM_OK", 1: "SSM_ERR_NULL", 2: "SSM_ERR_SHAPE", 3: "SSM_ERR_DTYPE", 4: "SSM_ERR_UNSUPPORTED",
          5: "SSM_ERR_ALIGN", 6: "SSM_ERR_WORKSPACE", 7: "SSM_ERR_HIP"}
EXPORTS = ["ssm_scan_fwd_workspace_bytes", "ssm_scan_fwd", "ssm_state_update", "ssm_status_str", "ssm_last_error",
           "ssm_abi_version", "ssm_scan_fwd_plan_segments", "ssm_scan_bwd_workspace_bytes", "ssm_scan_bwd",
           "ssm_conv_scan_fwd", "ssm_conv_state_update", "ssm_complex_scan_fwd", "ssm_complex_state_update",
           "ssm_ssd_fwd", "ssm_ssd_state_update", "ssm_ssd_fwd_workspace_bytes", "ssm_ssd_fwd_plan_segments",
           "ssm_conv1d_fwd", "ssm_conv1d_bwd", "ssm_scan_fwd_noalloc"]


class Params(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("dim", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("io_dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32),
                ("disc", ctypes.c_int32), ("dt_softplus", ctypes.c_int32), ("segments", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class ConvParams(ctypes.Structure):
    _fields_ = [("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("state_in", ctypes.c_void_p),
                ("state_out", ctypes.c_void_p), ("width", ctypes.c_int32), ("activation", ctypes.c_int32)]


class SsdParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32), ("disc", ctypes.c_int32),
                ("dt_softplus", ctypes.c_int32), ("segments", ctypes.c_int32)]


class SSMError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__("%s: %s" % (STATUS.get(status, str(status)), detail))
        self.status = status


_lib = None


def lib():
    """Load libssm57.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssm57.so is not built (expected at %s); run "
                               "`python -c 'import __graft_entry__ as g; g.build()'` or "
                               "`python selective_state_space_57_amd/build.py`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, S = ctypes.c_void_p, ctypes.c_size_t
        PP = ctypes.POINTER(Params)
        L.ssm_scan_fwd_workspace_bytes.argtypes = [PP]
        L.ssm_scan_fwd_workspace_bytes.restype = S
        L.ssm_scan_fwd_plan_segments.argtypes = [PP]
        L.ssm_scan_fwd_plan_segments.restype = ctypes.c_int
        L.ssm_scan_fwd.argtypes = [PP] + [P] * 11 + [P, S, P]
        L.ssm_scan_fwd.restype = ctypes.c_int
        L.ssm_scan_fwd_noalloc.argtypes = [PP] + [P] * 11 + [P]
        L.ssm_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssm_state_update.argtypes = [PP] + [P] * 11
        L.ssm_state_update.restype = ctypes.c_int
        L.ssm_scan_bwd_workspace_bytes.argtypes = [PP]
        L.ssm_scan_bwd_workspace_bytes.restype = S
        L.ssm_scan_bwd.argtypes = [PP] + [P] * 20 + [P, S, P]
        L.ssm_scan_bwd.restype = ctypes.c_int
        CP = ctypes.POINTER(ConvParams)
        L.ssm_conv_scan_fwd.argtypes = [PP, CP] + [P] * 11 + [P, S, P]
        L.ssm_conv_scan_fwd.restype = ctypes.c_int
        L.ssm_conv_state_update.argtypes = [PP, CP] + [P] * 11
        L.ssm_conv_state_update.restype = ctypes.c_int
        L.ssm_conv1d_fwd.argtypes = [PP, CP, P, P, P]
        L.ssm_conv1d_fwd.restype = ctypes.c_int
        L.ssm_conv1d_bwd.argtypes = [PP, CP] + [P] * 8
        L.ssm_conv1d_bwd.restype = ctypes.c_int
        L.ssm_complex_scan_fwd.argtypes = [PP] + [P] * 12
        L.ssm_complex_scan_fwd.restype = ctypes.c_int
        L.ssm_complex_state_update.argtypes = [PP] + [P] * 11
        L.ssm_complex_state_update.restype = ctypes.c_int
        SP = ctypes.POINTER(SsdParams)
        L.ssm_ssd_fwd.argtypes = [SP] + [P] * 11 + [P, S, P]
        L.ssm_ssd_fwd.restype = ctypes.c_int
        L.ssm_ssd_fwd_workspace_bytes.argtypes = [SP]
        L.ssm_ssd_fwd_workspace_bytes.restype = S
        L.ssm_ssd_fwd_plan_segments.argtypes = [SP]
        L.ssm_ssd_fwd_plan_segments.restype = ctypes.c_int
        L.ssm_ssd_state_update.argtypes = [SP] + [P] * 11
        L.ssm_ssd_state_update.restype = ctypes.c_int
        L.ssm_status_str.argtypes = [ctypes.c_int]
        L.ssm_status_str.restype = ctypes.c_char_p
        L.ssm_last_error.argtypes = []
        L.ssm_last_error.restype = ctypes.c_char_p
        L.ssm_abi_version.restype = ctypes.c_int
        _lib = L
    return _lib


def make_params(batch, dim, seqlen, dstate, io_dtype=SSM_BF16, y_dtype=None, disc=EULER_B, softplus=True,
                segments=0) -> Params:
    return Params(int(batch), int(dim), int(seqlen), int(dstate), int(io_dtype),
                  int(io_dtype if y_dtype is None else y_dtype), int(disc), int(bool(softplus)), int(segments), 0)


def make_ssd_params(batch, seqlen, nheads, headdim, ngroups, dstate, io_dtype=SSM_BF16, y_dtype=None, disc=EULER_B,
                    softplus=True, segments=0) -> SsdParams:
    return SsdParams(int(batch), int(seqlen), int(nheads), int(headdim), int(ngroups), int(dstate), int(io_dtype),
                     int(io_dtype if y_dtype is None else y_dtype), int(disc), int(bool(softplus)), int(segments))


def ssd_workspace_bytes(p: SsdParams) -> int:
    return int(lib().ssm_ssd_fwd_workspace_bytes(ctypes.byref(p)))


def ssd_plan_segments(p: SsdParams) -> int:
    return int(lib().ssm_ssd_fwd_plan_segments(ctypes.byref(p)))


def ssd_fwd_raw(p: SsdParams, x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, workspace, workspace_bytes_, stream):
    return lib().ssm_ssd_fwd(ctypes.byref(p), x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, workspace,
                             workspace_bytes_, stream)


def ssd_state_update_raw(p: SsdParams, state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream):
    return lib().ssm_ssd_state_update(ctypes.byref(p), state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream)


def check(status: int):
    if status != 0:
        raise SSMError(status, lib().ssm_last_error().decode())


def workspace_bytes(p: Params) -> int:
    return int(lib().ssm_scan_fwd_workspace_bytes(ctypes.byref(p)))


def plan_segments(p: Params) -> int:
    return int(lib().ssm_scan_fwd_plan_segments(ctypes.byref(p)))


def scan_fwd_raw(p: Params, x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, workspace, workspace_bytes_, stream):
    """Direct call with integer device addresses (0 = NULL)."""
    return lib().ssm_scan_fwd(ctypes.byref(p), x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, workspace,
                              workspace_bytes_, stream)


def scan_fwd_noalloc_raw(p: Params, x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, stream):
    """Direct call of the allocation-free forward (the library's static scratch as workspace)."""
    return lib().ssm_scan_fwd_noalloc(ctypes.byref(p), x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, stream)


def make_conv(weight, width, bias=0, state_in=0, state_out=0, activation=1) -> ConvParams:
    """Conv parameters from integer device addresses (0 = NULL)."""
    return ConvParams(weight, bias, state_in, state_out, int(width), int(activation))


def conv_scan_fwd_raw(p: Params, conv: ConvParams, x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, workspace,
                      workspace_bytes_, stream):
    return lib().ssm_conv_scan_fwd(ctypes.byref(p), ctypes.byref(conv), x, dt, dt_bias, A, B, C, Dskip, z, h0, y,
                                   h_final, workspace, workspace_bytes_, stream)


def conv_state_update_raw(p: Params, conv: ConvParams, state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream):
    return lib().ssm_conv_state_update(ctypes.byref(p), ctypes.byref(conv), state, x, dt, dt_bias, A, B, C, Dskip, z,
                                       y, stream)


def conv1d_fwd_raw(p: Params, conv: ConvParams, x, u, stream):
    return lib().ssm_conv1d_fwd(ctypes.byref(p), ctypes.byref(conv), x, u, stream)


def conv1d_bwd_raw(p: Params, conv: ConvParams, x, du, dstate_out, dx, dweight, dbias, dstate_in, stream):
    return lib().ssm_conv1d_bwd(ctypes.byref(p), ctypes.byref(conv), x, du, dstate_out, dx, dweight, dbias, dstate_in,
                                stream)


def complex_scan_fwd_raw(p: Params, x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, stream):
    return lib().ssm_complex_scan_fwd(ctypes.byref(p), x, dt, dt_bias, A, B, C, Dskip, z, h0, y, h_final, stream)


def complex_state_update_raw(p: Params, state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream):
    return lib().ssm_complex_state_update(ctypes.byref(p), state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream)


def bwd_workspace_bytes(p: Params) -> int:
    return int(lib().ssm_scan_bwd_workspace_bytes(ctypes.byref(p)))


def scan_bwd_raw(p: Params, x, dt, dt_bias, A, B, C, Dskip, z, h0, dy, dh_final, dx, ddt, dA, dB, dC, dDskip, dz,
                 ddt_bias, dh0, workspace, workspace_bytes_, stream):
    """Direct call with integer device addresses (0 = NULL)."""
    return lib().ssm_scan_bwd(ctypes.byref(p), x, dt, dt_bias, A, B, C, Dskip, z, h0, dy, dh_final, dx, ddt, dA, dB,
                              dC, dDskip, dz, ddt_bias, dh0, workspace, workspace_bytes_, stream)


def state_update_raw(p: Params, state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream):
    return lib().ssm_state_update(ctypes.byref(p), state, x, dt, dt_bias, A, B, C, Dskip, z, y, stream)
