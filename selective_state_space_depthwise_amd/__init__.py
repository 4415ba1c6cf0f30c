"""libaxonscan: the Axon-SSM selective-scan hot path on AMD Instinct MI355X (gfx950).

The layer's hot path (causal depthwise conv, softplus/clip step size, diagonal selective scan
with readout and skip, SiLU gate, and the single-token decode step with its conv/state caches)
runs in hand-written HIP kernels behind a C ABI (include/axonscan.h). This package is the thin
Python binding over that ABI: ``prefill`` and ``decode_step`` take torch tensors on the GPU and
only marshal arguments; ``Layer`` runs the whole layer around the path (input, selection and
output projections on hipBLASLt, convolution, scan, gate); ``ssd_scan`` is the Mamba-2 SSD core
(scalar decay per head, 64-token chunks on the matrix cores).
"""
from ._abi import AxonError, LIB_PATH, load, status_string, version
from .api import Layer, decode_step, prefill, prefill_workspace_bytes, ssd_scan, ssd_workspace_bytes

__all__ = ["AxonError", "LIB_PATH", "Layer", "load", "status_string", "version", "prefill",
           "decode_step", "prefill_workspace_bytes", "ssd_scan", "ssd_workspace_bytes"]
