"""CPU oracle of the Axon-SSM selective-scan hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``. The product package never imports it.

The arithmetic lives in ``axon_oracle.c`` (plain C, double precision, one token at a time).
This module only compiles that file with gcc and marshals numpy arrays to it.

Array conventions (all numpy, C-contiguous):
  x, z, dt_raw: (B, L, E) float32   B, C: (B, L, N) float32
  A_log: (E, N) float32   D, dt_bias, conv_b: (E,) float32   conv_w: (E, K) float32
  conv_cache: (B, K-1, E) float64   ssm_state: (B, E, N) float64
Results are float64.

Variants (optional keys of the input / parameter dict): ``conv_activation`` "none" (default,
Axon-SSM) or "silu" (SiLU on the convolution output, the Mamba block); ``discretization``
"first_order" (default, Bbar = dt B) or "zoh" (Bbar = expm1(dt A) / A B).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "axon_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libaxon_oracle.so")

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE semantics: no fast-math, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH) and (
        os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC)
    ):
        return _LIB_PATH
    os.makedirs(_BUILD_DIR, exist_ok=True)
    tmp = _LIB_PATH + f".tmp{os.getpid()}"
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


CONV_ACTIVATIONS = {"none": 0, "silu": 1}
DISCRETIZATIONS = {"first_order": 0, "zoh": 1}


def _variant(d: dict):
    """(conv_act, disc) codes from the optional variant keys of an input / parameter dict."""
    return (CONV_ACTIVATIONS[d.get("conv_activation", "none")],
            DISCRETIZATIONS[d.get("discretization", "first_order")])


def _declare(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int64
    Dd = ctypes.c_double
    Ci = ctypes.c_int
    lib.oracle_ssm_channel.restype = ctypes.c_int
    lib.oracle_ssm_channel.argtypes = [
        I, I, I, P, P, P, I, P, P, I, P, Dd, Dd, P, Dd, Dd, Dd, Ci, Ci, P, P, P, I, P, P, P, P, P,
    ]
    lib.oracle_ssm_prefill.restype = ctypes.c_int
    lib.oracle_ssm_prefill.argtypes = [
        I, I, I, I, I, P, P, P, P, P, P, P, P, P, P, Dd, Dd, Ci, Ci, P, P, P, P, P, P, Ci,
    ]
    lib.oracle_ssm_decode_step.restype = ctypes.c_int
    lib.oracle_ssm_decode_step.argtypes = [
        I, I, I, I, P, P, P, P, P, P, P, P, P, P, Dd, Dd, Ci, Ci, P, P, P, Ci,
    ]
    return lib


def load_library(path: str):
    """Load an oracle shared library built from ``axon_oracle.c`` (or a variant of it)."""
    return _declare(ctypes.CDLL(path))


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    with _lock:
        if _lib is None:
            override = os.environ.get("AXON_ORACLE_LIB")  # e.g. the sanitizer build
            if override:
                _lib = load_library(override)
            else:
                build(force=False)
                _lib = load_library(_LIB_PATH)
        return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data


def prefill(inp: dict, conv_cache_in=None, ssm_state_in=None, threads: int = 1,
            lib=None, magnitude: bool = False) -> dict:
    """Run the oracle over whole (B, L, E) tensors. Returns y, conv_cache, ssm_state (float64),
    and with ``magnitude`` also ``mag``: |SiLU(z)| * (sum_n |C h_n| + |D u|) per token, the size
    of the terms each output sums (a conditioning diagnostic)."""
    lib = _load(lib)
    x, z, dtr = _f32(inp["x"]), _f32(inp["z"]), _f32(inp["dt_raw"])
    Bm, Cm = _f32(inp["B"]), _f32(inp["C"])
    A_log, D, dtb = _f32(inp["A_log"]), _f32(inp["D"]), _f32(inp["dt_bias"])
    w, cb = _f32(inp["conv_w"]), _f32(inp["conv_b"])
    Bsz, L, E = x.shape
    N = A_log.shape[1]
    K = w.shape[1]
    assert Bm.shape == (Bsz, L, N) and Cm.shape == (Bsz, L, N)
    assert z.shape == x.shape and dtr.shape == x.shape
    cin, sin = _f64(conv_cache_in), _f64(ssm_state_in)
    if cin is not None:
        assert cin.shape == (Bsz, K - 1, E)
    if sin is not None:
        assert sin.shape == (Bsz, E, N)
    y = np.empty((Bsz, L, E), np.float64)
    cout = np.empty((Bsz, K - 1, E), np.float64)
    sout = np.empty((Bsz, E, N), np.float64)
    mag = np.empty((Bsz, L, E), np.float64) if magnitude else None
    rc = lib.oracle_ssm_prefill(
        Bsz, L, E, N, K, _ptr(x), _ptr(z), _ptr(dtr), _ptr(Bm), _ptr(Cm), _ptr(A_log), _ptr(D),
        _ptr(dtb), _ptr(w), _ptr(cb), float(inp["dt_min"]), float(inp["dt_max"]), *_variant(inp),
        _ptr(cin), _ptr(sin), _ptr(y), _ptr(cout), _ptr(sout), _ptr(mag), int(threads),
    )
    if rc != 0:
        raise ValueError("oracle_ssm_prefill rejected its arguments")
    out = {"y": y, "conv_cache": cout, "ssm_state": sout}
    if magnitude:
        out["mag"] = mag
    return out


def channel(inp: dict, b: int, e: int, conv_cache_in=None, ssm_state_in=None, lib=None) -> dict:
    """Run the oracle for one (b, e) channel over all L tokens.

    Returns y (L,), u (L,), dt (L,), mag (L,), conv_cache (K-1,), ssm_state (N,) as float64.
    ``conv_cache_in`` / ``ssm_state_in`` are the whole (B, K-1, E) / (B, E, N) arrays or None.
    """
    lib = _load(lib)
    x, z, dtr = inp["x"], inp["z"], inp["dt_raw"]
    Bsz, L, E = x.shape
    A_log = _f32(inp["A_log"])
    N = A_log.shape[1]
    w = _f32(inp["conv_w"])
    K = w.shape[1]
    xc = _f32(x[b, :, e])
    zc = _f32(z[b, :, e])
    dc = _f32(dtr[b, :, e])
    Bc = _f32(inp["B"][b])
    Cc = _f32(inp["C"][b])
    win = None if conv_cache_in is None else _f64(np.asarray(conv_cache_in)[b, :, e])
    h0 = None if ssm_state_in is None else _f64(np.asarray(ssm_state_in)[b, e, :])
    y = np.empty(L, np.float64)
    u = np.empty(L, np.float64)
    dt = np.empty(L, np.float64)
    mag = np.empty(L, np.float64)
    wout = np.empty(max(K - 1, 1), np.float64)
    hout = np.empty(N, np.float64)
    rc = lib.oracle_ssm_channel(
        L, N, K, _ptr(xc), _ptr(zc), _ptr(dc), 1, _ptr(Bc), _ptr(Cc), N, _ptr(A_log[e]),
        float(inp["D"][e]), float(inp["dt_bias"][e]), _ptr(w[e]), float(inp["conv_b"][e]),
        float(inp["dt_min"]), float(inp["dt_max"]), *_variant(inp), _ptr(win), _ptr(h0),
        _ptr(y), 1,
        _ptr(wout), _ptr(hout), _ptr(u), _ptr(dt), _ptr(mag),
    )
    if rc != 0:
        raise ValueError("oracle_ssm_channel rejected its arguments")
    return {"y": y, "u": u, "dt": dt, "mag": mag, "conv_cache": wout[: K - 1], "ssm_state": hout}


def decode_step(step: dict, params: dict, conv_cache, ssm_state, threads: int = 1,
                lib=None) -> np.ndarray:
    """One decode step. ``step`` holds x, z, dt_raw (B, E) and B, C (B, N) float32; ``params``
    holds A_log, D, dt_bias, conv_w, conv_b, dt_min, dt_max. ``conv_cache`` (B, K-1, E) and
    ``ssm_state`` (B, E, N) are float64 arrays updated in place. Returns y (B, E) float64."""
    lib = _load(lib)
    x, z, dtr = _f32(step["x"]), _f32(step["z"]), _f32(step["dt_raw"])
    Bm, Cm = _f32(step["B"]), _f32(step["C"])
    A_log = _f32(params["A_log"])
    Bsz, E = x.shape
    N = A_log.shape[1]
    w = _f32(params["conv_w"])
    K = w.shape[1]
    assert conv_cache.dtype == np.float64 and conv_cache.flags.c_contiguous
    assert ssm_state.dtype == np.float64 and ssm_state.flags.c_contiguous
    assert conv_cache.shape == (Bsz, K - 1, E) and ssm_state.shape == (Bsz, E, N)
    y = np.empty((Bsz, E), np.float64)
    rc = lib.oracle_ssm_decode_step(
        Bsz, E, N, K, _ptr(x), _ptr(z), _ptr(dtr), _ptr(Bm), _ptr(Cm), _ptr(A_log),
        _ptr(_f32(params["D"])), _ptr(_f32(params["dt_bias"])), _ptr(w),
        _ptr(_f32(params["conv_b"])), float(params["dt_min"]), float(params["dt_max"]),
        *_variant(params), _ptr(conv_cache), _ptr(ssm_state), _ptr(y), int(threads),
    )
    if rc != 0:
        raise ValueError("oracle_ssm_decode_step rejected its arguments")
    return y


# ---- the layer around the path -----------------------------------------------------------------
def store_as(a, act: str) -> np.ndarray:
    """Round values to how the GPU path stores an intermediate: float32, or bfloat16 (round to
    nearest, ties to even), returned as float32."""
    a32 = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32))
    if act == "bf16":
        u = a32.view(np.uint32)
        u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
        a32 = u.view(np.float32)
    return a32


def layer_forward(x_in, W_in, W_f, W_out, params: dict, conv_cache_in=None, ssm_state_in=None,
                  act: str = "f32", threads: int = 1, lib=None) -> dict:
    """The whole layer ["Axon-SSM: ...", "Gating", "Selective mechanism", "Code mapping"]:
      (x_branch, z) = split(W_in x)
      u = conv(x_branch) with the cache (SiLU after it for the Mamba-block variant)
      (B_t, C_t, dt_raw_t) = f_proj(u_t), f_proj = W_f (2N + E, E), rows B, C, dt_raw
      y = the path's scan and gate (``prefill`` on u through an identity convolution)
      out = W_out y
    READING: f_proj is one full-rank linear map with no bias. Every product is taken in float64;
    each intermediate is then stored as the GPU path stores it (``act``: float32 or bfloat16).
    Returns out (B, L, D) float64, conv_cache (B, K-1, E), ssm_state (B, E, N), and the stored
    intermediates (x_branch, z, u, B, C, dt_raw, y)."""
    X = np.asarray(x_in, np.float64)
    Win = np.asarray(W_in, np.float64)
    Wf = np.asarray(W_f, np.float64)
    Wout = np.asarray(W_out, np.float64)
    Bsz, L, _ = X.shape
    E = Win.shape[0] // 2
    N = (Wf.shape[0] - E) // 2
    K = np.asarray(params["conv_w"]).shape[1]
    xb = store_as(X @ Win[:E].T, act)
    z = store_as(X @ Win[E:].T, act)
    cache = np.zeros((Bsz, K - 1, E)) if conv_cache_in is None else np.asarray(conv_cache_in,
                                                                               np.float64)
    full = np.concatenate([cache, xb.astype(np.float64)], axis=1)  # (B, K-1+L, E)
    w = np.asarray(params["conv_w"], np.float64)
    v = np.asarray(params["conv_b"], np.float64)[None, None, :] + sum(
        w[None, None, :, k] * full[:, k:k + L, :] for k in range(K))
    if params.get("conv_activation", "none") == "silu":
        v = v / (1.0 + np.exp(-v))
    u = store_as(v, act)
    U = u.astype(np.float64)
    Bm = store_as(U @ Wf[:N].T, act)
    Cm = store_as(U @ Wf[N:2 * N].T, act)
    dtr = store_as(U @ Wf[2 * N:].T, act)
    ident = np.zeros((E, K), np.float32)
    ident[:, K - 1] = 1.0
    scan_in = {"x": u, "z": z, "dt_raw": dtr, "B": Bm, "C": Cm, "A_log": params["A_log"],
               "D": params["D"], "dt_bias": params["dt_bias"], "conv_w": ident,
               "conv_b": np.zeros(E, np.float32), "dt_min": params["dt_min"],
               "dt_max": params["dt_max"],
               "discretization": params.get("discretization", "first_order")}
    r = prefill(scan_in, ssm_state_in=ssm_state_in, threads=threads, lib=lib)
    y = store_as(r["y"], act)
    out = y.astype(np.float64) @ Wout.T
    return {"out": out, "conv_cache": full[:, -(K - 1):, :].copy(), "ssm_state": r["ssm_state"],
            "x_branch": xb, "z": z, "u": u, "B": Bm, "C": Cm, "dt_raw": dtr, "y": y}


# ---- Mamba-2 SSD core ----------------------------------------------------------------------------
def ssd_scan(inp: dict, state_in=None, threads: int = 1, lib=None,
             magnitude: bool = False) -> dict:
    """The SSD core over x (B, L, H, P), dt_raw (B, L, H), B, C (B, L, N) float32 with A_log,
    D, dt_bias (H,) and the dt clips (see oracle_ssd_scan). Returns y (B, L, H, P) and
    ssm_state (B, H, P, N), float64, and with ``magnitude`` also ``mag`` (B, L, H, P):
    sum_n |C h| + |D x|, the size of the terms each output sums."""
    lib = _load(lib)
    if not hasattr(lib, "_ssd_declared"):
        P_, I_, D_ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_double
        lib.oracle_ssd_scan.restype = ctypes.c_int
        lib.oracle_ssd_scan.argtypes = [I_, I_, I_, I_, I_, P_, P_, P_, P_, P_, P_, P_, D_, D_,
                                        P_, P_, P_, P_, ctypes.c_int]
        lib._ssd_declared = True
    x, dtr = _f32(inp["x"]), _f32(inp["dt_raw"])
    Bm, Cm = _f32(inp["B"]), _f32(inp["C"])
    Bsz, L, H, P = x.shape
    N = Bm.shape[2]
    assert dtr.shape == (Bsz, L, H) and Bm.shape == (Bsz, L, N) and Cm.shape == (Bsz, L, N)
    sin = _f64(state_in)
    if sin is not None:
        assert sin.shape == (Bsz, H, P, N)
    y = np.empty((Bsz, L, H, P), np.float64)
    sout = np.empty((Bsz, H, P, N), np.float64)
    mag = np.empty((Bsz, L, H, P), np.float64) if magnitude else None
    rc = lib.oracle_ssd_scan(Bsz, L, H, P, N, _ptr(x), _ptr(dtr), _ptr(Bm), _ptr(Cm),
                             _ptr(_f32(inp["A_log"])), _ptr(_f32(inp["D"])),
                             _ptr(_f32(inp["dt_bias"])), float(inp["dt_min"]),
                             float(inp["dt_max"]), _ptr(sin), _ptr(y), _ptr(sout), _ptr(mag),
                             int(threads))
    if rc != 0:
        raise ValueError("oracle_ssd_scan rejected its arguments")
    out = {"y": y, "ssm_state": sout}
    if magnitude:
        out["mag"] = mag
    return out
