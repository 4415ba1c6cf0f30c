"""Helpers for the GPU parity tests: move seeded inputs to the device, run the HIP path through
the binding, and compare with the oracle element by element.

Tolerances (element-wise, against the oracle run on the same rounded inputs):
  fp32 activations: |gpu - ref| <= 1e-4 * (1 + |ref|)
  bf16 activations: |gpu - ref| <= 2e-2 * (1 + |ref|)   (y is rounded to bf16; state stays fp32)
  conv cache: bit-exact (it holds copies of the inputs).
The fp32 stress cases with dt spanning [1e-4, 1] plus clip hits ("wide": states reach
thousands and an output can be the small difference of large terms) add a term for the size
of what each output sums:
  |gpu - ref| <= 1e-4 * (1 + |ref|) + MAG_TOL * mag,  mag = |SiLU(z)| (sum_n |C h_n| + |D u|)
(``mag`` from the oracle, pinned to the LTI closed form). MAG_TOL = 1e-5: with dt >= 1e-4 and
|A| >= 1 a state remembers at most 1e4 steps, each adding one fp32 rounding (2^-24) to a running
sum; independent roundings grow as the square root of their count, sqrt(1e4) * 2^-24 = 6e-6 of
the terms' size, and 1e-5 leaves a margin over that.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads

TOL = {"f32": 1e-4, "bf16": 2e-2}
MAG_TOL = 1e-5
# The state is fp32 in both cases; for bf16 runs its error is set by the same fp32 arithmetic.
STATE_TOL = {"f32": 1e-4, "bf16": 1e-4}
ACT_KEYS = ("x", "z", "dt_raw", "B", "C")
PARAM_KEYS = ("A_log", "D", "dt_bias", "conv_w", "conv_b")


def say(msg: str) -> None:
    """Print and flush a line naming the case, so a failure can be located from the log."""
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    return torch.device("cuda:0")


def act_dtype(act: str):
    return torch.bfloat16 if act == "bf16" else torch.float32


def to_device(inp: dict, act: str | None = None) -> dict:
    act = act or inp.get("act", "f32")
    dev = device()
    out = {}
    for k in ACT_KEYS:
        out[k] = torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev).to(act_dtype(act))
    for k in PARAM_KEYS:
        out[k] = torch.from_numpy(np.ascontiguousarray(inp[k], np.float32)).to(dev)
    out["dt_min"], out["dt_max"] = float(inp["dt_min"]), float(inp["dt_max"])
    return out


def gpu_prefill(d: dict, **kw):
    import selective_state_space_depthwise_amd as axon

    return axon.prefill(d["x"], d["z"], d["dt_raw"], d["B"], d["C"], d["A_log"], d["D"],
                        d["dt_bias"], d["conv_w"], d["conv_b"], dt_min=d["dt_min"],
                        dt_max=d["dt_max"], **kw)


def gpu_decode(step: dict, d: dict, cache, state, **kw):
    import selective_state_space_depthwise_amd as axon

    return axon.decode_step(step["x"], step["z"], step["dt_raw"], step["B"], step["C"],
                            d["A_log"], d["D"], d["dt_bias"], d["conv_w"], d["conv_b"], cache,
                            state, dt_min=d["dt_min"], dt_max=d["dt_max"], **kw)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, tol: float, what: str, mag=None) -> None:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values from the GPU"
    err = np.abs(got - ref)
    bound = tol * (1.0 + np.abs(ref))
    if mag is not None:
        bound = bound + MAG_TOL * np.asarray(mag, np.float64)
    bad = err > bound
    if bad.any():
        idx = np.unravel_index(np.argmax(err / bound), err.shape)
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements beyond {tol}*(1+|ref|); worst at "
            f"{idx}: gpu={got[idx]!r} ref={ref[idx]!r} err={err[idx]:.3e}")


def max_rel(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref)))) if got.size else 0.0


def make_case(B, L, E, act="f32", dt_mode="axon", seed=0, caches=False):
    """Seeded inputs with the workloads' recipe at a given size, plus optional caches."""
    w = workloads.Workload(0, "case", "prefill", B, L, E, act, dt_mode=dt_mode)
    inp = workloads.prefill_inputs(w, seed_offset=seed)
    extra = {}
    if caches:
        g = np.random.default_rng(1000 + seed)
        cache = g.standard_normal((B, 3, E)).astype(np.float32)
        if act == "bf16":
            cache = workloads.bf16_round(cache)
        extra["conv_cache_in"] = cache
        extra["ssm_state_in"] = g.standard_normal((B, E, 16)).astype(np.float32)
    return inp, extra


def run_and_compare(inp, extra, what, inplace=False, conditioned=False):
    """Run the HIP prefill through the binding and compare y, state (tolerance) and cache
    (bit-exact) with the oracle. Variant keys of ``inp`` (conv_activation, discretization) are
    passed to both."""
    act = inp["act"]
    variant = {k: inp[k] for k in ("conv_activation", "discretization") if k in inp}
    say(f"[parity] {what}: B={inp['x'].shape[0]} L={inp['x'].shape[1]} E={inp['x'].shape[2]} "
        f"act={act} caches={bool(extra)} inplace={inplace} {variant}")
    d = to_device(inp)
    kw = dict(variant)
    cin = sin = None
    if extra:
        cin = torch.from_numpy(extra["conv_cache_in"]).cuda()
        sin = torch.from_numpy(extra["ssm_state_in"]).cuda()
        kw.update(conv_cache_in=cin, ssm_state_in=sin)
        if inplace:
            kw.update(conv_cache_out=cin, ssm_state_out=sin)
    y, cache, state = gpu_prefill(d, **kw)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp, conv_cache_in=extra.get("conv_cache_in"),
                         ssm_state_in=extra.get("ssm_state_in"), threads=8,
                         magnitude=conditioned)
    assert_close(host(y), ref["y"], TOL[act], f"{what}: y",
                 mag=ref["mag"] if conditioned else None)
    assert_close(host(state), ref["ssm_state"], STATE_TOL[act], f"{what}: ssm_state")
    np.testing.assert_array_equal(host(cache), ref["conv_cache"], err_msg=f"{what}: conv_cache")
    return d, y, cache, state, ref
