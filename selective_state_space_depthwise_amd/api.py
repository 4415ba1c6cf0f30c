"""Torch-tensor front end of libaxonscan: argument marshalling only.

Every step of the layer runs in the library's HIP kernels. PyTorch supplies device memory (the
output, cache and workspace tensors allocated here) and the stream (torch's current stream unless
one is given). Nothing is computed in Python and there is no CPU path.
"""
from __future__ import annotations

import torch

from . import _abi
from ._abi import AxonError

D_STATE = 16
D_CONV = 4


def _stream_handle(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _keep_for(device, stream, *tensors):
    """Tensors this binding allocated (from torch's caching allocator, on the current stream) and
    hands to kernels launched on another stream: record that stream on them, so that when they
    are freed their memory is not handed out again before the work queued on it has run."""
    if stream is None or stream == torch.cuda.current_stream(device):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _act_dtype(x: torch.Tensor) -> bool:
    if x.dtype == torch.float32:
        return False
    if x.dtype == torch.bfloat16:
        return True
    raise TypeError(f"activations must be float32 or bfloat16, got {x.dtype}")


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _params(A_log, D, dt_bias, conv_w, conv_b, dt_min, dt_max, E, device,
            conv_activation="none", discretization="first_order"):
    for t, n, shp in ((A_log, "A_log", (E, D_STATE)), (D, "D", (E,)), (dt_bias, "dt_bias", (E,)),
                      (conv_w, "conv_w", (E, D_CONV)), (conv_b, "conv_b", (E,))):
        _check(t, n, shp, torch.float32, device)
    return _abi.make_params(A_log.data_ptr(), D.data_ptr(), dt_bias.data_ptr(),
                            conv_w.data_ptr(), conv_b.data_ptr(), dt_min, dt_max,
                            conv_activation, discretization)


def prefill_workspace_bytes(batch: int, seqlen: int, d_inner: int, bf16: bool = False) -> int:
    """Device workspace bytes axon_ssm_prefill needs for this shape."""
    return _abi.workspace_bytes(_abi.make_shape(batch, seqlen, d_inner, bf16))


def prefill(x, z, dt_raw, B, C, A_log, D, dt_bias, conv_w, conv_b, *, dt_min=1e-4, dt_max=100.0,
            conv_cache_in=None, ssm_state_in=None, y=None, conv_cache_out=None,
            ssm_state_out=None, workspace=None, stream=None, conv_activation="none",
            discretization="first_order"):
    """Run the layer over x, z, dt_raw (B, L, E) and B, C (B, L, N) on the GPU.

    Activations are float32 or bfloat16 (all the same dtype); parameters float32. Optional
    ``conv_cache_in`` (B, K-1, E) and ``ssm_state_in`` (B, E, N) are float32 (None = zeros).
    Outputs may be given (``y``, ``conv_cache_out``, ``ssm_state_out``; the caches may be the
    inputs themselves for an in-place update) or are allocated. Returns (y, conv_cache, ssm_state).
    Asynchronous on ``stream`` (default: torch's current stream on x's device).
    Variants: ``conv_activation`` "none" (Axon-SSM) or "silu" (SiLU on the convolution output,
    the Mamba block); ``discretization`` "first_order" (Bbar = dt B) or "zoh" (exact zero-order
    hold, Bbar = expm1(dt A) / A B)."""
    device = x.device
    if device.type != "cuda":
        raise ValueError("prefill runs on the GPU only; x is on " + str(device))
    bf16 = _act_dtype(x)
    if x.dim() != 3:
        raise ValueError("x must be (batch, seqlen, d_inner)")
    Bsz, L, E = x.shape
    for t, n in ((x, "x"), (z, "z"), (dt_raw, "dt_raw")):
        _check(t, n, (Bsz, L, E), x.dtype, device)
    for t, n in ((B, "B"), (C, "C")):
        _check(t, n, (Bsz, L, D_STATE), x.dtype, device)
    prm = _params(A_log, D, dt_bias, conv_w, conv_b, dt_min, dt_max, E, device,
                  conv_activation, discretization)
    cache_shape, state_shape = (Bsz, D_CONV - 1, E), (Bsz, E, D_STATE)
    if conv_cache_in is not None:
        _check(conv_cache_in, "conv_cache_in", cache_shape, torch.float32, device)
    if ssm_state_in is not None:
        _check(ssm_state_in, "ssm_state_in", state_shape, torch.float32, device)
    mine = []  # tensors allocated here
    if y is None:
        y = torch.empty_like(x)
        mine.append(y)
    _check(y, "y", (Bsz, L, E), x.dtype, device)
    if conv_cache_out is None:
        conv_cache_out = torch.empty(cache_shape, dtype=torch.float32, device=device)
        mine.append(conv_cache_out)
    if ssm_state_out is None:
        ssm_state_out = torch.empty(state_shape, dtype=torch.float32, device=device)
        mine.append(ssm_state_out)
    _check(conv_cache_out, "conv_cache_out", cache_shape, torch.float32, device)
    _check(ssm_state_out, "ssm_state_out", state_shape, torch.float32, device)
    shape = _abi.make_shape(Bsz, L, E, bf16)
    need = _abi.workspace_bytes(shape)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
        mine.append(workspace)
    _keep_for(device, stream, *mine)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _abi.raw_prefill(
        shape, prm, x.data_ptr(), z.data_ptr(), dt_raw.data_ptr(), B.data_ptr(), C.data_ptr(),
        conv_cache_in.data_ptr() if conv_cache_in is not None else None,
        ssm_state_in.data_ptr() if ssm_state_in is not None else None,
        y.data_ptr(), conv_cache_out.data_ptr(), ssm_state_out.data_ptr(), ws_ptr, ws_bytes,
        _stream_handle(device, stream))
    if st != _abi.AXON_OK:
        raise AxonError(st, "axon_ssm_prefill")
    return y, conv_cache_out, ssm_state_out


def decode_step(x, z, dt_raw, B, C, A_log, D, dt_bias, conv_w, conv_b, conv_cache, ssm_state, *,
                dt_min=1e-4, dt_max=100.0, y=None, stream=None, conv_activation="none",
                discretization="first_order"):
    """One token per batch row: x, z, dt_raw (B, E), B, C (B, N); conv_cache (B, K-1, E) and
    ssm_state (B, E, N) float32 are updated in place. Returns y (B, E)."""
    device = x.device
    if device.type != "cuda":
        raise ValueError("decode_step runs on the GPU only; x is on " + str(device))
    bf16 = _act_dtype(x)
    if x.dim() != 2:
        raise ValueError("x must be (batch, d_inner)")
    Bsz, E = x.shape
    for t, n in ((x, "x"), (z, "z"), (dt_raw, "dt_raw")):
        _check(t, n, (Bsz, E), x.dtype, device)
    for t, n in ((B, "B"), (C, "C")):
        _check(t, n, (Bsz, D_STATE), x.dtype, device)
    prm = _params(A_log, D, dt_bias, conv_w, conv_b, dt_min, dt_max, E, device,
                  conv_activation, discretization)
    _check(conv_cache, "conv_cache", (Bsz, D_CONV - 1, E), torch.float32, device)
    _check(ssm_state, "ssm_state", (Bsz, E, D_STATE), torch.float32, device)
    if y is None:
        y = torch.empty_like(x)
        _keep_for(device, stream, y)
    _check(y, "y", (Bsz, E), x.dtype, device)
    st = _abi.raw_decode_step(
        _abi.make_shape(Bsz, 1, E, bf16), prm, x.data_ptr(), z.data_ptr(), dt_raw.data_ptr(),
        B.data_ptr(), C.data_ptr(), conv_cache.data_ptr(), ssm_state.data_ptr(), y.data_ptr(),
        _stream_handle(device, stream))
    if st != _abi.AXON_OK:
        raise AxonError(st, "axon_ssm_decode_step")
    return y


__all__ = ["prefill", "decode_step", "prefill_workspace_bytes", "AxonError", "Layer"]


class Layer:
    """The whole layer on the GPU: out = W_out (scan(conv(W_in_x x), f_proj(u)) * SiLU(W_in_z x)),
    as axon_layer_forward defines it. Holds a library context (GEMM handle and plans) and a
    cached workspace tensor; not safe for concurrent use."""

    def __init__(self):
        self._ctx = _abi.layer_create()
        self._ws = None

    def close(self):
        if self._ctx:
            _abi.layer_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 (interpreter shutdown)
            pass

    def forward(self, x_in, W_in, W_f, W_out, A_log, D, dt_bias, conv_w, conv_b, *,
                dt_min=1e-4, dt_max=100.0, conv_cache_in=None, ssm_state_in=None, out=None,
                conv_cache_out=None, ssm_state_out=None, stream=None, conv_activation="none",
                discretization="first_order"):
        """x_in (B, L, D) and the weights W_in (2E, D), W_f (2N + E, E), W_out (D, E) in one
        activation dtype (float32 or bfloat16); the SSM parameters as for ``prefill``.
        Returns (out, conv_cache, ssm_state)."""
        device = x_in.device
        if device.type != "cuda":
            raise ValueError("Layer.forward runs on the GPU only")
        bf16 = _act_dtype(x_in)
        if x_in.dim() != 3:
            raise ValueError("x_in must be (batch, seqlen, d_model)")
        Bsz, L, Dm = x_in.shape
        E = A_log.shape[0]
        _check(x_in, "x_in", (Bsz, L, Dm), x_in.dtype, device)
        _check(W_in, "W_in", (2 * E, Dm), x_in.dtype, device)
        _check(W_f, "W_f", (2 * D_STATE + E, E), x_in.dtype, device)
        _check(W_out, "W_out", (Dm, E), x_in.dtype, device)
        prm = _params(A_log, D, dt_bias, conv_w, conv_b, dt_min, dt_max, E, device,
                      conv_activation, discretization)
        shape = _abi.make_layer_shape(Bsz, L, Dm, E, bf16)
        weights = _abi.LayerWeights(W_in.data_ptr(), W_f.data_ptr(), W_out.data_ptr(), prm)
        mine = []
        if out is None:
            out = torch.empty_like(x_in)
            mine.append(out)
        _check(out, "out", (Bsz, L, Dm), x_in.dtype, device)
        if conv_cache_out is None:
            conv_cache_out = torch.empty((Bsz, D_CONV - 1, E), dtype=torch.float32, device=device)
            mine.append(conv_cache_out)
        if ssm_state_out is None:
            ssm_state_out = torch.empty((Bsz, E, D_STATE), dtype=torch.float32, device=device)
            mine.append(ssm_state_out)
        for t, n, shp in ((conv_cache_in, "conv_cache_in", (Bsz, D_CONV - 1, E)),
                          (ssm_state_in, "ssm_state_in", (Bsz, E, D_STATE)),
                          (conv_cache_out, "conv_cache_out", (Bsz, D_CONV - 1, E)),
                          (ssm_state_out, "ssm_state_out", (Bsz, E, D_STATE))):
            if t is not None:
                _check(t, n, shp, torch.float32, device)
        need = _abi.layer_workspace_bytes(shape)
        if self._ws is None or self._ws.numel() < need or self._ws.device != device:
            self._ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
        # the cached workspace is recorded on every stream that uses it, so that replacing it
        # later does not free memory a kernel on that stream still uses
        _keep_for(device, stream, self._ws, *mine)
        ptr = lambda t: 0 if t is None else t.data_ptr()  # noqa: E731
        st = _abi.raw_layer_forward(self._ctx, shape, weights, x_in.data_ptr(), ptr(conv_cache_in),
                                    ptr(ssm_state_in), out.data_ptr(), conv_cache_out.data_ptr(),
                                    ssm_state_out.data_ptr(), self._ws.data_ptr(), need,
                                    _stream_handle(device, stream))
        if st != _abi.AXON_OK:
            raise AxonError(st, "axon_layer_forward")
        return out, conv_cache_out, ssm_state_out


SSD_HEAD_DIM = 64
SSD_STATE = 128


def ssd_workspace_bytes(batch: int, seqlen: int, n_heads: int, bf16: bool = False) -> int:
    """Device workspace bytes axon_ssd_scan needs for this shape."""
    return _abi.ssd_workspace_bytes(_abi.make_ssd_shape(batch, seqlen, n_heads, bf16))


def ssd_scan(x, dt_raw, B, C, A_log, D, dt_bias, *, dt_min=1e-4, dt_max=100.0, state_in=None,
             y=None, state_out=None, workspace=None, stream=None):
    """Mamba-2 SSD core on the GPU: x (B, L, H, 64), dt_raw (B, L, H), B, C (B, L, 128), float32
    or bfloat16 (all the same dtype); A_log, D, dt_bias (H,) float32; optional state_in
    (B, H, 64, 128) float32 (None = zeros). Returns (y, state_out); state_out may be state_in
    (in place). Asynchronous on ``stream`` (default: torch's current stream)."""
    device = x.device
    if device.type != "cuda":
        raise ValueError("ssd_scan runs on the GPU only; x is on " + str(device))
    bf16 = _act_dtype(x)
    if x.dim() != 4:
        raise ValueError("x must be (batch, seqlen, n_heads, head_dim)")
    Bsz, L, H, P = x.shape
    _check(x, "x", (Bsz, L, H, SSD_HEAD_DIM), x.dtype, device)
    _check(dt_raw, "dt_raw", (Bsz, L, H), x.dtype, device)
    for t, n in ((B, "B"), (C, "C")):
        _check(t, n, (Bsz, L, SSD_STATE), x.dtype, device)
    for t, n in ((A_log, "A_log"), (D, "D"), (dt_bias, "dt_bias")):
        _check(t, n, (H,), torch.float32, device)
    state_shape = (Bsz, H, SSD_HEAD_DIM, SSD_STATE)
    if state_in is not None:
        _check(state_in, "state_in", state_shape, torch.float32, device)
    mine = []
    if y is None:
        y = torch.empty_like(x)
        mine.append(y)
    _check(y, "y", tuple(x.shape), x.dtype, device)
    if state_out is None:
        state_out = torch.empty(state_shape, dtype=torch.float32, device=device)
        mine.append(state_out)
    _check(state_out, "state_out", state_shape, torch.float32, device)
    shape = _abi.make_ssd_shape(Bsz, L, H, bf16)
    prm = _abi.SsdParams(A_log.data_ptr(), D.data_ptr(), dt_bias.data_ptr(), float(dt_min),
                         float(dt_max))
    need = _abi.ssd_workspace_bytes(shape)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
        mine.append(workspace)
    _keep_for(device, stream, *mine)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = _abi.raw_ssd_scan(shape, prm, x.data_ptr(), dt_raw.data_ptr(), B.data_ptr(),
                           C.data_ptr(), state_in.data_ptr() if state_in is not None else None,
                           y.data_ptr(), state_out.data_ptr(), ws_ptr, ws_bytes,
                           _stream_handle(device, stream))
    if st != _abi.AXON_OK:
        raise AxonError(st, "axon_ssd_scan")
    return y, state_out
