"""The whole layer around the path (projections on hipBLASLt, convolution, scan, gate) through
the C ABI, against the oracle's composition. The oracle takes every product in float64 and
stores each intermediate as the GPU path does, so the two differ by the GEMMs' fp32 accumulation
order; for that reason the conv cache (which holds x-branch projection outputs) is compared to
a tolerance here, not bit for bit: 1e-5 relative in fp32, one bf16 ulp (2^-8) in bf16."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import STATE_TOL, TOL, assert_close, host, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
CACHE_TOL = {"f32": 1e-5, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module")
def layer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_depthwise_amd as axon

    axon.load()
    lay = axon.Layer()
    yield lay
    torch.cuda.synchronize()
    lay.close()


def _dev(inp, act):
    dt = torch.bfloat16 if act == "bf16" else torch.float32
    d = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).cuda().to(dt)
         for k in ("x_in", "W_in", "W_f", "W_out")}
    d.update({k: torch.from_numpy(np.ascontiguousarray(inp[k], np.float32)).cuda()
              for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b")})
    return d


def _run(layer, inp, act, caches=None, variant=None, **kw):
    d = _dev(inp, act)
    variant = variant or {}
    cin = sin = None
    if caches is not None:
        cin = torch.from_numpy(caches[0]).cuda()
        sin = torch.from_numpy(caches[1]).cuda()
    out, cache, state = layer.forward(d["x_in"], d["W_in"], d["W_f"], d["W_out"], d["A_log"],
                                      d["D"], d["dt_bias"], d["conv_w"], d["conv_b"],
                                      dt_min=inp["dt_min"], dt_max=inp["dt_max"],
                                      conv_cache_in=cin, ssm_state_in=sin, **variant, **kw)
    torch.cuda.synchronize()
    return out, cache, state


def _ref(inp, act, caches=None, variant=None):
    prm = dict(inp)
    prm.update(variant or {})
    return oracle.layer_forward(inp["x_in"], inp["W_in"], inp["W_f"], inp["W_out"], prm,
                                conv_cache_in=None if caches is None else caches[0],
                                ssm_state_in=None if caches is None else caches[1], act=act,
                                threads=max(1, min(16, os.cpu_count() or 1)))


def _compare(out, cache, state, ref, act, what):
    assert_close(host(out), ref["out"], TOL[act], f"{what}: out")
    assert_close(host(state), ref["ssm_state"], STATE_TOL[act] if act == "f32" else 2e-2,
                 f"{what}: state")
    assert_close(host(cache), ref["conv_cache"], CACHE_TOL[act], f"{what}: cache")


def _caches(B, E, seed, act):
    g = np.random.default_rng(seed)
    c = g.standard_normal((B, 3, E)).astype(np.float32)
    if act == "bf16":
        c = workloads.bf16_round(c)
    return c, g.standard_normal((B, E, 16)).astype(np.float32)


CASES = [
    # (B, L, D, E, act, caches)
    (2, 37, 64, 96, "f32", False),
    (1, 130, 48, 160, "f32", True),      # time chunks in the scan
    (3, 20, 72, 64, "bf16", True),
    (1, 300, 128, 6400, "f32", False),   # one state per lane in the scan
]


@pytest.mark.parametrize("B,L,D,E,act,caches", CASES)
def test_layer_matches_oracle(layer, B, L, D, E, act, caches):
    w = workloads.Workload(0, "layer", "prefill", B, L, E, act)
    inp = workloads.layer_inputs(w, D)
    cc = _caches(B, E, 7 + L, act) if caches else None
    say(f"[layer] {B}x{L} D={D} E={E} {act} caches={caches}")
    out, cache, state = _run(layer, inp, act, cc)
    _compare(out, cache, state, _ref(inp, act, cc), act, f"layer {B}x{L}x{D}x{E} {act}")


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_layer_variants(layer, act):
    w = workloads.Workload(0, "layer", "prefill", 2, 45, 80, act)
    inp = workloads.layer_inputs(w, 40)
    cc = _caches(2, 80, 3, act)
    var = {"conv_activation": "silu", "discretization": "zoh"}
    say(f"[layer] variants {act}")
    out, cache, state = _run(layer, inp, act, cc, var)
    _compare(out, cache, state, _ref(inp, act, cc, var), act, f"layer variants {act}")


def test_layer_steps_equal_prefill(layer):
    """The layer one token at a time (seqlen 1, in-place caches) equals one call over all
    tokens, on the GPU."""
    B, L, D, E = 2, 11, 32, 48
    w = workloads.Workload(0, "layer", "prefill", B, L, E, "f32")
    inp = workloads.layer_inputs(w, D)
    d = _dev(inp, "f32")
    kw = dict(dt_min=inp["dt_min"], dt_max=inp["dt_max"])
    args = (d["W_in"], d["W_f"], d["W_out"], d["A_log"], d["D"], d["dt_bias"], d["conv_w"],
            d["conv_b"])
    full, c_full, s_full = layer.forward(d["x_in"], *args, **kw)
    cache = torch.zeros((B, 3, E), dtype=torch.float32, device="cuda")
    state = torch.zeros((B, E, 16), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(L):
        o, _, _ = layer.forward(d["x_in"][:, t:t + 1].contiguous(), *args, conv_cache_in=cache,
                                ssm_state_in=state, conv_cache_out=cache, ssm_state_out=state,
                                **kw)
        outs.append(o.clone())
    torch.cuda.synchronize()
    assert_close(host(torch.cat(outs, 1)), host(full), TOL["f32"], "out")
    assert_close(host(state), host(s_full), TOL["f32"], "state")
    assert_close(host(cache), host(c_full), CACHE_TOL["f32"], "cache")


@pytest.mark.timeout(600)
def test_layer_full_axon_shape(layer):
    """The Axon-SSM layer configuration: D = 2560, E = 7680, N = 16, K = 4 over 2048 tokens,
    fp32, whole output against the oracle."""
    w = workloads.workload(1)
    say("[layer] full Axon shape: drawing inputs")
    inp = workloads.layer_inputs(w, 2560)
    say("[layer] full Axon shape: GPU")
    out, cache, state = _run(layer, inp, "f32")
    say("[layer] full Axon shape: oracle")
    ref = _ref(inp, "f32")
    _compare(out, cache, state, ref, "f32", "layer full Axon shape")


@pytest.mark.timeout(900)
def test_layer_full_batch8_bf16(layer):
    """The benchmarked bf16 layer: 8 x 4096 tokens, D = 2560, E = 7680, whole output, state and
    cache against the oracle (its projections in float64, intermediates stored as bf16)."""
    w = workloads.workload(2)
    say("[layer] bf16 8 x 4096, D 2560: drawing inputs")
    inp = workloads.layer_inputs(w, 2560)
    say("[layer] bf16 8 x 4096, D 2560: GPU")
    out, cache, state = _run(layer, inp, "bf16")
    say("[layer] bf16 8 x 4096, D 2560: oracle")
    ref = _ref(inp, "bf16")
    _compare(out, cache, state, ref, "bf16", "layer bf16 batch 8")
