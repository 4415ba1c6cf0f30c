"""Parity of the variants with the oracle: SiLU on the convolution output (the Mamba block of
"Selective State Space Models (Mamba)") and the exact zero-order hold (Bbar = expm1(dt A) / A B,
"Axon-SSM: ...", section "ZOH discretization"), alone and together, through every launch path:
one state per lane, two states per lane, time chunks, bf16 activations, decode steps, and the
Axon-SSM layer shape at full size on sampled channels."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (STATE_TOL, TOL, assert_close, gpu_decode, gpu_prefill, host, make_case,
                      run_and_compare, say, to_device)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

VARIANTS = [("silu", "first_order"), ("none", "zoh"), ("silu", "zoh")]
CASES = [
    # (B, L, E, act, dt_mode, caches)
    (1, 300, 7680, "f32", "axon", True),    # one state per lane, single pass
    (1, 200, 7700, "bf16", "axon", True),   # ragged channel groups
    (1, 289, 6200, "bf16", "wide", True),   # 10 tiles, the last of one token, clip hits
    (2, 100, 9000, "f32", "axon", False),   # two states per lane, single pass
    (1, 1000, 64, "f32", "axon", False),    # time chunks
    (2, 700, 48, "f32", "wide", True),      # chunks, dt across [1e-4, 1] with clip hits
    (3, 333, 100, "bf16", "axon", True),    # chunks, bf16, caches in
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_depthwise_amd as axon

    axon.load()
    yield
    torch.cuda.synchronize()


def _with(inp, act_name, disc):
    inp["conv_activation"], inp["discretization"] = act_name, disc
    return inp


@pytest.mark.parametrize("conv_act,disc", VARIANTS)
@pytest.mark.parametrize("B,L,E,act,dt_mode,caches", CASES)
def test_variant_prefill_matches_oracle(conv_act, disc, B, L, E, act, dt_mode, caches):
    inp, extra = make_case(B, L, E, act, dt_mode, seed=B * 11 + L, caches=caches)
    _with(inp, conv_act, disc)
    run_and_compare(inp, extra, f"variant {conv_act}/{disc} {B}x{L}x{E} {act} {dt_mode}",
                    conditioned=(act == "f32" and dt_mode == "wide"))


@pytest.mark.parametrize("disc", ["first_order", "zoh"])
def test_zoh_small_and_large_steps(disc):
    """dt pinned near both branch points of the exact hold's coefficient (|dt A| around 0.25)
    and at the clip bounds, with A = -(1..16)."""
    inp, extra = make_case(1, 400, 64, "f32", seed=77, caches=True)
    _with(inp, "none", disc)
    # softplus^-1 of a few step sizes, per token group: 0.25 / n for some n, and extremes
    targets = np.array([0.015625, 0.0244, 0.0250, 0.0256, 0.125, 0.25, 1.0, 3.0], np.float64)
    raw = np.log(np.expm1(targets)) - inp["dt_bias"][None, :].astype(np.float64).mean()
    for j, r in enumerate(raw):
        inp["dt_raw"][:, j::len(raw), :] = np.float32(r)
    inp["dt_raw"][:, 5::97, :] = np.float32(-1000.0)   # dt = 1e-4
    run_and_compare(inp, extra, f"zoh branch points ({disc})")


@pytest.mark.parametrize("conv_act,disc", VARIANTS)
@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_variant_decode_steps(conv_act, disc, act):
    B, E, L0, steps = 2, 96, 17, 8
    inp, extra = make_case(B, L0, E, act, seed=51, caches=True)
    _with(inp, conv_act, disc)
    say(f"[parity] variant decode {conv_act}/{disc} {act}")
    d = to_device(inp)
    kw = {"conv_activation": conv_act, "discretization": disc}
    _, cache, state = gpu_prefill(d, conv_cache_in=torch.from_numpy(extra["conv_cache_in"]).cuda(),
                                  ssm_state_in=torch.from_numpy(extra["ssm_state_in"]).cuda(),
                                  **kw)
    ref = oracle.prefill(inp, threads=8, **extra)
    rcache, rstate = ref["conv_cache"].copy(), ref["ssm_state"].copy()
    w = workloads.Workload(0, "dec", "decode", B, L0, E, act)
    for s in range(steps):
        st = workloads.decode_step_inputs(w, s)
        std = {k: torch.from_numpy(st[k]).cuda().to(d["x"].dtype) for k in st}
        y = gpu_decode(std, d, cache, state, **kw)
        ry = oracle.decode_step(st, inp, rcache, rstate)
        torch.cuda.synchronize()
        assert_close(host(y), ry, TOL[act], f"decode step {s} y")
    assert_close(host(state), rstate, STATE_TOL[act], "decode state")
    np.testing.assert_array_equal(host(cache), rcache)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("conv_act,disc", [("silu", "zoh")])
def test_variant_full_size_axon_shape(conv_act, disc):
    """The Axon-SSM layer shape (1 x 2048 x 7680 fp32) with both variants, in the benchmark's
    launch configuration; every output, state and cache element against the oracle."""
    w = workloads.workload(1)
    inp = _with(workloads.prefill_inputs(w), conv_act, disc)
    say(f"[parity] variant full size {conv_act}/{disc}")
    d = to_device(inp)
    y, cache, state = gpu_prefill(d, conv_activation=conv_act, discretization=disc)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp, threads=max(1, min(16, os.cpu_count() or 1)))
    assert_close(host(y), ref["y"], TOL["f32"], "variant full size y")
    assert_close(host(state), ref["ssm_state"], STATE_TOL["f32"], "variant full size state")
    np.testing.assert_array_equal(host(cache), ref["conv_cache"])


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_long_stream_in_chunks(act):
    """A long stream fed in pieces, as the streaming loop of "Selective State Space Models
    (Mamba)" (pattern "1M context inference") does: 8 prefills of 1000 tokens (the time-chunked
    path inside each), the Mamba-block variant (SiLU after the conv), caches carried in place
    between calls; every output compared with one oracle pass over all 8000 tokens."""
    B, L, E, n = 2, 8000, 192, 8
    inp, extra = make_case(B, L, E, act, seed=61, caches=True)
    _with(inp, "silu", "first_order")
    say(f"[parity] long stream {B}x{L}x{E} {act} in {n} pieces")
    d = to_device(inp)
    cache = torch.from_numpy(extra["conv_cache_in"]).cuda()
    state = torch.from_numpy(extra["ssm_state_in"]).cuda()
    ys = []
    step = L // n
    for p in range(n):
        part = {k: (v[:, p * step:(p + 1) * step].contiguous()
                    if k in ("x", "z", "dt_raw", "B", "C") else v) for k, v in d.items()}
        y, _, _ = gpu_prefill(part, conv_cache_in=cache, ssm_state_in=state,
                              conv_cache_out=cache, ssm_state_out=state, conv_activation="silu")
        ys.append(host(y))
    torch.cuda.synchronize()
    ref = oracle.prefill(inp, threads=8, **extra)
    assert_close(np.concatenate(ys, axis=1), ref["y"], TOL[act], "streamed y")
    assert_close(host(state), ref["ssm_state"], STATE_TOL[act], "streamed state")
    np.testing.assert_array_equal(host(cache), ref["conv_cache"])
