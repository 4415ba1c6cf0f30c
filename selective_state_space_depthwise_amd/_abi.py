"""ctypes view of libaxonscan's C ABI (include/axonscan.h). No torch here: pointers are ints.

The library is loaded from this package directory; it is built by
``python -m selective_state_space_depthwise_amd.build``. There is no fallback: if the library is
missing or does not load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os
import re
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
# AXONSCAN_LIB selects another build of the library (the sanitizer build of build.py).
LIB_PATH = os.environ.get("AXONSCAN_LIB") or os.path.join(PKG, "libaxonscan.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "axonscan.h")

AXON_OK = 0
AXON_ERR_INVALID_ARGUMENT = 1
AXON_ERR_UNSUPPORTED = 2
AXON_ERR_WORKSPACE_TOO_SMALL = 3
AXON_ERR_HIP = 4
AXON_F32 = 0
AXON_BF16 = 1


class AxonError(RuntimeError):
    """A libaxonscan call returned a status other than AXON_OK."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_state", ctypes.c_int64),
                ("d_conv", ctypes.c_int64), ("act_dtype", ctypes.c_int)]


class Params(ctypes.Structure):
    _fields_ = [("A_log", ctypes.c_void_p), ("D", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("conv_w", ctypes.c_void_p), ("conv_b", ctypes.c_void_p),
                ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float),
                ("conv_activation", ctypes.c_int32), ("discretization", ctypes.c_int32)]

class LayerShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("d_model", ctypes.c_int64),
                ("d_inner", ctypes.c_int64), ("d_state", ctypes.c_int64),
                ("d_conv", ctypes.c_int64), ("act_dtype", ctypes.c_int)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("W_in", ctypes.c_void_p), ("W_f", ctypes.c_void_p), ("W_out", ctypes.c_void_p),
                ("ssm", Params)]


class SsdShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("n_heads", ctypes.c_int64),
                ("head_dim", ctypes.c_int64), ("d_state", ctypes.c_int64),
                ("act_dtype", ctypes.c_int)]


class SsdParams(ctypes.Structure):
    _fields_ = [("A_log", ctypes.c_void_p), ("D", ctypes.c_void_p), ("dt_bias", ctypes.c_void_p),
                ("dt_min", ctypes.c_float), ("dt_max", ctypes.c_float)]


CONV_ACTIVATIONS = {"none": 0, "silu": 1}
DISCRETIZATIONS = {"first_order": 0, "zoh": 1}


_lock = threading.Lock()
_lib = None


def load():
    """Load libaxonscan.so (once). Raises RuntimeError with a build hint when it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libaxonscan.so not found at {LIB_PATH}; build it with "
                "`python -m selective_state_space_depthwise_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.axon_version.restype = ctypes.c_int
        lib.axon_version.argtypes = []
        lib.axon_status_string.restype = ctypes.c_char_p
        lib.axon_status_string.argtypes = [ctypes.c_int]
        lib.axon_ssm_prefill_workspace_bytes.restype = ctypes.c_size_t
        lib.axon_ssm_prefill_workspace_bytes.argtypes = [ctypes.POINTER(Shape)]
        lib.axon_ssm_prefill.restype = ctypes.c_int
        lib.axon_ssm_prefill.argtypes = [
            ctypes.POINTER(Shape), ctypes.POINTER(Params), P, P, P, P, P, P, P, P, P, P, P,
            ctypes.c_size_t, P]
        lib.axon_ssm_prefill_noalloc.restype = ctypes.c_int
        lib.axon_ssm_prefill_noalloc.argtypes = [
            ctypes.POINTER(Shape), ctypes.POINTER(Params), P, P, P, P, P, P, P, P, P, P, P]
        lib.axon_ssm_decode_step.restype = ctypes.c_int
        lib.axon_ssm_decode_step.argtypes = [
            ctypes.POINTER(Shape), ctypes.POINTER(Params), P, P, P, P, P, P, P, P, P]
        lib.axon_layer_create.restype = ctypes.c_int
        lib.axon_layer_create.argtypes = [ctypes.POINTER(P)]
        lib.axon_layer_destroy.restype = None
        lib.axon_layer_destroy.argtypes = [P]
        lib.axon_layer_workspace_bytes.restype = ctypes.c_size_t
        lib.axon_layer_workspace_bytes.argtypes = [ctypes.POINTER(LayerShape)]
        lib.axon_layer_forward.restype = ctypes.c_int
        lib.axon_layer_forward.argtypes = [
            P, ctypes.POINTER(LayerShape), ctypes.POINTER(LayerWeights), P, P, P, P, P, P, P,
            ctypes.c_size_t, P]
        lib.axon_layer_forward_check.restype = ctypes.c_int
        lib.axon_layer_forward_check.argtypes = [
            ctypes.POINTER(LayerShape), ctypes.POINTER(LayerWeights), P, P, P, P, P, P, P,
            ctypes.c_size_t]
        lib.axon_ssd_scan_workspace_bytes.restype = ctypes.c_size_t
        lib.axon_ssd_scan_workspace_bytes.argtypes = [ctypes.POINTER(SsdShape)]
        lib.axon_ssd_scan.restype = ctypes.c_int
        lib.axon_ssd_scan.argtypes = [ctypes.POINTER(SsdShape), ctypes.POINTER(SsdParams),
                                      P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().axon_status_string(int(status)).decode()


def version() -> int:
    return load().axon_version()


def make_shape(batch, seqlen, d_inner, act_bf16, d_state=16, d_conv=4) -> Shape:
    return Shape(int(batch), int(seqlen), int(d_inner), int(d_state), int(d_conv),
                 AXON_BF16 if act_bf16 else AXON_F32)


def make_params(A_log, D, dt_bias, conv_w, conv_b, dt_min, dt_max, conv_activation="none",
                discretization="first_order") -> Params:
    """Parameter block; variant names as in CONV_ACTIVATIONS / DISCRETIZATIONS, or raw ints
    (passed through unchecked, so the library's own validation can be exercised)."""
    act = conv_activation if isinstance(conv_activation, int) else CONV_ACTIVATIONS[conv_activation]
    disc = discretization if isinstance(discretization, int) else DISCRETIZATIONS[discretization]
    return Params(A_log, D, dt_bias, conv_w, conv_b, float(dt_min), float(dt_max), act, disc)


def workspace_bytes(shape: Shape) -> int:
    return int(load().axon_ssm_prefill_workspace_bytes(ctypes.byref(shape)))


def raw_prefill(shape: Shape, params: Params, x, z, dt_raw, B, C, cache_in, state_in, y,
                cache_out, state_out, workspace, workspace_bytes_, stream) -> int:
    """axon_ssm_prefill with integer pointers (0 / None = NULL). Returns the status code."""
    return load().axon_ssm_prefill(ctypes.byref(shape), ctypes.byref(params), x, z, dt_raw, B, C,
                                   cache_in, state_in, y, cache_out, state_out, workspace,
                                   int(workspace_bytes_), stream)


def raw_prefill_noalloc(shape: Shape, params: Params, x, z, dt_raw, B, C, cache_in, state_in,
                        y, cache_out, state_out, stream) -> int:
    """axon_ssm_prefill_noalloc with integer pointers. Returns the status code."""
    return load().axon_ssm_prefill_noalloc(ctypes.byref(shape), ctypes.byref(params), x, z,
                                           dt_raw, B, C, cache_in, state_in, y, cache_out,
                                           state_out, stream)


def raw_decode_step(shape: Shape, params: Params, x, z, dt_raw, B, C, cache, state, y,
                    stream) -> int:
    """axon_ssm_decode_step with integer pointers. Returns the status code."""
    return load().axon_ssm_decode_step(ctypes.byref(shape), ctypes.byref(params), x, z, dt_raw,
                                       B, C, cache, state, y, stream)


def make_layer_shape(batch, seqlen, d_model, d_inner, act_bf16, d_state=16,
                     d_conv=4) -> LayerShape:
    return LayerShape(int(batch), int(seqlen), int(d_model), int(d_inner), int(d_state),
                      int(d_conv), AXON_BF16 if act_bf16 else AXON_F32)


def layer_workspace_bytes(shape: LayerShape) -> int:
    return int(load().axon_layer_workspace_bytes(ctypes.byref(shape)))


def layer_create() -> int:
    """A new layer context (an opaque pointer as int); raises AxonError on failure."""
    h = ctypes.c_void_p()
    st = load().axon_layer_create(ctypes.byref(h))
    if st != AXON_OK:
        raise AxonError(st, "axon_layer_create")
    return h.value


def layer_destroy(ctx: int) -> None:
    load().axon_layer_destroy(ctx)


def raw_layer_forward(ctx, shape: LayerShape, weights: LayerWeights, x_in, cache_in, state_in,
                      out, cache_out, state_out, workspace, workspace_bytes_, stream) -> int:
    """axon_layer_forward with integer pointers. Returns the status code."""
    return load().axon_layer_forward(ctx, ctypes.byref(shape), ctypes.byref(weights), x_in,
                                     cache_in, state_in, out, cache_out, state_out, workspace,
                                     int(workspace_bytes_), stream)


def raw_layer_forward_check(shape: LayerShape, weights: LayerWeights, x_in, cache_in, state_in,
                            out, cache_out, state_out, workspace, workspace_bytes_) -> int:
    """axon_layer_forward_check with integer pointers (compared only, never dereferenced).
    Returns the status code axon_layer_forward would give these arguments before launching."""
    return load().axon_layer_forward_check(ctypes.byref(shape), ctypes.byref(weights), x_in,
                                           cache_in, state_in, out, cache_out, state_out,
                                           workspace, int(workspace_bytes_))


def make_ssd_shape(batch, seqlen, n_heads, act_bf16, head_dim=64, d_state=128) -> SsdShape:
    return SsdShape(int(batch), int(seqlen), int(n_heads), int(head_dim), int(d_state),
                    AXON_BF16 if act_bf16 else AXON_F32)


def ssd_workspace_bytes(shape: SsdShape) -> int:
    return int(load().axon_ssd_scan_workspace_bytes(ctypes.byref(shape)))


def raw_ssd_scan(shape: SsdShape, params: SsdParams, x, dt_raw, B, C, state_in, y, state_out,
                 workspace, workspace_bytes_, stream) -> int:
    """axon_ssd_scan with integer pointers. Returns the status code."""
    return load().axon_ssd_scan(ctypes.byref(shape), ctypes.byref(params), x, dt_raw, B, C,
                                state_in, y, state_out, workspace, int(workspace_bytes_), stream)


def declared_functions() -> list[str]:
    """Names of the functions include/axonscan.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(axon_[a-z0-9_]+)\s*\(", text)))
