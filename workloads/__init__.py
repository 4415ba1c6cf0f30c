"""Seeded synthetic workloads for the Axon-SSM selective-scan hot path.

This module only draws inputs. It holds none of the layer's arithmetic, and both the oracle
(``oracle/``) and the HIP path (``selective_state_space_depthwise_amd``) consume what it returns.

Shapes follow the layer configuration of "Axon-SSM: Selective State Space Model for Apple
Silicon" (section "Layer configuration": d_inner E = 7680, d_state N = 16, conv kernel K = 4) and
the mamba-ssm block shape of "Selective State Space Models (Mamba)" (pattern "Mamba block":
d_model 1024, expand 2, so E = 2048). The pages name no dataset, so every tensor is drawn here:

  x, z, dt_raw, B, C  ~ N(0, 1)                           (tensor ids 1, 2, 3, 4, 5)
  D                   ~ N(0, 1) per channel               (id 6)
  dt_bias             = log(expm1(U)), U ~ U[1e-3, 0.1]   (id 7; the inverse of softplus, so
                        that softplus(dt_bias) = U)
  conv_w              ~ N(0, 0.5^2), shape (E, 4)         (id 8)
  conv_b              = 0
  A_log               = log(1..16) in every row, so A = -(1..16) (the initialisation on the
                        Axon-SSM page, section "Diagonal state matrix")
  long-context config: U log-uniform on [1e-4, 1], and about 1% of dt_raw set to +-50
                        (mask id 9, sign id 10)
Activation tensors of the bf16 configs are rounded to bf16 (round to nearest even) from the
fp32 draws; the fp32 arrays returned then hold exactly the bf16 values.

Randomness: numpy's PCG64 generator seeded with (0x5EED00 + config index, tensor id), so every
tensor is reproducible on its own and independent of draw order.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 0x5EED00
D_STATE = 16
D_CONV = 4
DT_MIN = 1e-4   # "Axon-SSM ...", section "Selective mechanism": eps
DT_MAX = 100.0  # same section: dt_max

TID_X, TID_Z, TID_DT, TID_B, TID_C, TID_D, TID_DTB, TID_W, TID_MASK, TID_SIGN = range(1, 11)
# Decode inputs of step s use tensor ids 1000 + 10 * s + (1..5).


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    kind: str            # "prefill" or "decode"
    batch: int
    seqlen: int          # prefill tokens (decode: tokens of the seeding prefill)
    d_inner: int
    act: str             # "f32" or "bf16"
    dt_mode: str = "axon"   # "axon": U[1e-3, 0.1]; "wide": log-uniform [1e-4, 1] + clip hits
    decode_steps: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index


WORKLOADS = [
    Workload(0, "tiny_f32_b1_l64_e32", "prefill", 1, 64, 32, "f32"),
    Workload(1, "axon_prefill_f32_b1_l2048_e7680", "prefill", 1, 2048, 7680, "f32"),
    Workload(2, "axon_prefill_bf16_b8_l4096_e7680", "prefill", 8, 4096, 7680, "bf16"),
    Workload(3, "axon_decode_f32_b64_e7680_256steps", "decode", 64, 128, 7680, "f32",
             decode_steps=256),
    Workload(4, "mamba_long_bf16_b2_l65536_e2048", "prefill", 2, 65536, 2048, "bf16",
             dt_mode="wide"),
]


def _rng(seed: int, tid: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tid])))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returned as float32.
    (Finite inputs only: the 32-bit sum below cannot overflow for them.)"""
    out = np.array(a, dtype=np.float32, copy=True, order="C")
    u = out.view(np.uint32)
    u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    u &= np.uint32(0xFFFF0000)
    return out


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The upper 16 bits of float32 values that are already bf16-exact (as uint16)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _normal(seed, tid, shape, scale=1.0):
    out = _rng(seed, tid).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def params(w: Workload, d_inner: int | None = None) -> dict:
    """Per-channel parameters: A_log, D, dt_bias, conv_w, conv_b (float32) and the dt clip."""
    E = d_inner or w.d_inner
    seed = w.seed
    A_log = np.tile(np.log(np.arange(1, D_STATE + 1, dtype=np.float64)), (E, 1)).astype(
        np.float32)
    D = _normal(seed, TID_D, (E,))
    g = _rng(seed, TID_DTB)
    if w.dt_mode == "wide":
        U = np.exp(g.uniform(np.log(1e-4), np.log(1.0), size=E))
    else:
        U = g.uniform(1e-3, 0.1, size=E)
    dt_bias = np.log(np.expm1(U)).astype(np.float32)
    conv_w = _normal(seed, TID_W, (E, D_CONV), scale=0.5)
    conv_b = np.zeros(E, np.float32)
    return {"A_log": A_log, "D": D, "dt_bias": dt_bias, "conv_w": conv_w, "conv_b": conv_b,
            "dt_min": DT_MIN, "dt_max": DT_MAX}


def prefill_inputs(w: Workload, batch: int | None = None, seqlen: int | None = None,
                   d_inner: int | None = None, seed_offset: int = 0) -> dict:
    """Activations (x, z, dt_raw, B, C) plus parameters for a prefill of workload ``w``.

    ``batch`` / ``seqlen`` / ``d_inner`` override the workload's sizes (smaller parity cases);
    ``seed_offset`` selects an independent draw of the activations with the same recipe."""
    Bsz = batch or w.batch
    L = w.seqlen if seqlen is None else seqlen
    E = d_inner or w.d_inner
    seed = w.seed + 7919 * seed_offset
    act = {
        "x": _normal(seed, TID_X, (Bsz, L, E)),
        "z": _normal(seed, TID_Z, (Bsz, L, E)),
        "dt_raw": _normal(seed, TID_DT, (Bsz, L, E)),
        "B": _normal(seed, TID_B, (Bsz, L, D_STATE)),
        "C": _normal(seed, TID_C, (Bsz, L, D_STATE)),
    }
    if w.dt_mode == "wide":
        hit = _rng(seed, TID_MASK).random(size=(Bsz, L, E), dtype=np.float32) < 0.01
        sign = _rng(seed, TID_SIGN).random(size=(Bsz, L, E), dtype=np.float32) < 0.5
        act["dt_raw"] = np.where(hit, np.where(sign, np.float32(50.0), np.float32(-50.0)),
                                 act["dt_raw"]).astype(np.float32)
    if w.act == "bf16":
        for k in act:
            act[k] = bf16_round(act[k])
    out = params(w, E)
    out.update(act)
    out["act"] = w.act
    return out


def decode_step_inputs(w: Workload, step: int, batch: int | None = None,
                       d_inner: int | None = None) -> dict:
    """Fresh per-token inputs of decode step ``step``: x, z, dt_raw (B, E), B, C (B, N)."""
    Bsz = batch or w.batch
    E = d_inner or w.d_inner
    base = 1000 + 10 * step
    out = {
        "x": _normal(w.seed, base + TID_X, (Bsz, E)),
        "z": _normal(w.seed, base + TID_Z, (Bsz, E)),
        "dt_raw": _normal(w.seed, base + TID_DT, (Bsz, E)),
        "B": _normal(w.seed, base + TID_B, (Bsz, D_STATE)),
        "C": _normal(w.seed, base + TID_C, (Bsz, D_STATE)),
    }
    if w.act == "bf16":
        for k in out:
            out[k] = bf16_round(out[k])
    return out


TID_XIN, TID_WIN, TID_WF, TID_WOUT = 21, 22, 23, 24


def layer_inputs(w: Workload, d_model: int, batch: int | None = None, seqlen: int | None = None,
                 d_inner: int | None = None) -> dict:
    """Inputs of the whole layer: x_in (B, L, D) ~ N(0, 1) and random-initialised projection
    weights W_in (2E, D) ~ N(0, 1/D), W_f (2N + E, E) ~ N(0, 1/E), W_out (D, E) ~ N(0, 1/E),
    plus the SSM parameters of ``params`` (no trained weights exist here). bf16 workloads
    round x_in and the three projections to bf16."""
    Bsz = batch or w.batch
    L = w.seqlen if seqlen is None else seqlen
    E = d_inner or w.d_inner
    seed = w.seed
    out = params(w, E)
    out["x_in"] = _normal(seed, TID_XIN, (Bsz, L, d_model))
    out["W_in"] = _normal(seed, TID_WIN, (2 * E, d_model), scale=d_model ** -0.5)
    out["W_f"] = _normal(seed, TID_WF, (2 * D_STATE + E, E), scale=E ** -0.5)
    out["W_out"] = _normal(seed, TID_WOUT, (d_model, E), scale=E ** -0.5)
    if w.act == "bf16":
        for k in ("x_in", "W_in", "W_f", "W_out"):
            out[k] = bf16_round(out[k])
    out["act"] = w.act
    return out


def workload(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[name_or_index]
    for w in WORKLOADS:
        if w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


# ---- Mamba-2 SSD core ----------------------------------------------------------------------------
# Block shape of "Selective State Space Models (Mamba)", pattern "Mamba-2 block": d_model 2048,
# expand 2 (d_inner 4096), headdim 64 -> 64 heads, d_state 128. The pages give no sequence
# length for it; the Axon-SSM headline length (2048, batch 1) is used.
SSD_HEAD_DIM = 64
SSD_STATE = 128
SSD_SEED_BASE = 0x55D000
TID_SSD_X, TID_SSD_DT, TID_SSD_B, TID_SSD_C, TID_SSD_ALOG, TID_SSD_D, TID_SSD_DTB = range(31, 38)


@dataclass(frozen=True)
class SsdWorkload:
    index: int
    name: str
    batch: int
    seqlen: int
    heads: int
    act: str
    dt_mode: str = "axon"

    @property
    def seed(self) -> int:
        return SSD_SEED_BASE + self.index


SSD_WORKLOADS = [
    SsdWorkload(0, "mamba2_ssd_f32_b1_l2048_h64", 1, 2048, 64, "f32"),
    SsdWorkload(1, "mamba2_ssd_bf16_b1_l2048_h64", 1, 2048, 64, "bf16"),
]


def ssd_inputs(w: SsdWorkload, batch: int | None = None, seqlen: int | None = None,
               heads: int | None = None, seed_offset: int = 0) -> dict:
    """Inputs of the SSD core: x (B, L, H, 64), dt_raw (B, L, H), B, C (B, L, 128) ~ N(0, 1);
    per head A_log = log(U[1, 16]) (A in [-16, -1]), D ~ N(0, 1), dt_bias = log(expm1(U)) with
    U ~ U[1e-3, 0.1] (or log-uniform on [1e-4, 1] plus about 1% of dt_raw at +-50 for
    dt_mode "wide"), dt clipped to [1e-4, 100]. bf16 workloads round the activations."""
    Bsz = batch or w.batch
    L = w.seqlen if seqlen is None else seqlen
    H = heads or w.heads
    seed = w.seed + 7919 * seed_offset
    out = {
        "x": _normal(seed, TID_SSD_X, (Bsz, L, H, SSD_HEAD_DIM)),
        "dt_raw": _normal(seed, TID_SSD_DT, (Bsz, L, H)),
        "B": _normal(seed, TID_SSD_B, (Bsz, L, SSD_STATE)),
        "C": _normal(seed, TID_SSD_C, (Bsz, L, SSD_STATE)),
    }
    if w.dt_mode == "wide":
        hit = _rng(seed, TID_MASK).random(size=(Bsz, L, H), dtype=np.float32) < 0.01
        sign = _rng(seed, TID_SIGN).random(size=(Bsz, L, H), dtype=np.float32) < 0.5
        out["dt_raw"] = np.where(hit, np.where(sign, np.float32(50.0), np.float32(-50.0)),
                                 out["dt_raw"]).astype(np.float32)
    if w.act == "bf16":
        for k in ("x", "dt_raw", "B", "C"):
            out[k] = bf16_round(out[k])
    g = _rng(w.seed, TID_SSD_DTB)
    if w.dt_mode == "wide":
        U = np.exp(g.uniform(np.log(1e-4), np.log(1.0), size=H))
    else:
        U = g.uniform(1e-3, 0.1, size=H)
    out["dt_bias"] = np.log(np.expm1(U)).astype(np.float32)
    out["A_log"] = np.log(_rng(w.seed, TID_SSD_ALOG).uniform(1.0, 16.0, size=H)).astype(
        np.float32)
    out["D"] = _normal(w.seed, TID_SSD_D, (H,))
    out["dt_min"], out["dt_max"] = DT_MIN, DT_MAX
    out["act"] = w.act
    return out
