"""Parity of the HIP path (through the C ABI and the binding) with the CPU oracle.

Small cases are compared whole; they span several time chunks, ragged channel counts (not a
multiple of the 64-lane wave) and ragged last chunks. The full-size workloads run in the same
launch configuration as the benchmark and are compared on sampled channels (every token of each
sampled channel, plus its final state and cache) that the oracle computes one by one.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (STATE_TOL, TOL, assert_close, gpu_decode, gpu_prefill, host, make_case,
                      run_and_compare, say, sample_channels, single_channel_inputs, to_device)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_depthwise_amd as axon

    axon.load()  # fails loudly when the library is missing
    yield
    torch.cuda.synchronize()


SMALL = [
    # (B, L, E, act, dt_mode, caches)
    (1, 64, 32, "f32", "axon", False),      # the tiny workload itself
    (1, 1000, 64, "f32", "axon", False),    # 3 time chunks, ragged last chunk
    (3, 333, 100, "f32", "axon", True),     # ragged E and ragged last tile, caches in
    (2, 517, 130, "bf16", "axon", True),    # 2 chunks
    (1, 16384, 16, "f32", "axon", True),    # the maximum of 64 chunks
    (1, 300, 7680, "f32", "axon", True),    # 2 states per lane (the Axon-SSM channel count)
    (1, 200, 7700, "bf16", "axon", True),   # 2 states per lane, ragged channel groups
    (2, 100, 9000, "f32", "axon", False),   # 4 states per lane
    (2, 700, 48, "bf16", "wide", False),    # dt spanning [1e-4, 1] with +-50 clip hits
    (2, 700, 48, "f32", "wide", True),
    (1, 1, 70, "f32", "axon", True),        # L < K-1: the new cache mixes old cache and x
    (1, 2, 70, "bf16", "axon", True),
    (2, 3, 40, "f32", "axon", True),
    (4, 96, 200, "f32", "axon", False),     # single chunk, several waves per row
]


@pytest.mark.parametrize("B,L,E,act,dt_mode,caches", SMALL)
def test_small_cases_match_oracle(B, L, E, act, dt_mode, caches):
    inp, extra = make_case(B, L, E, act, dt_mode, seed=B * 7 + L, caches=caches)
    # fp32 with dt clip hits is a stress case outside the workloads (see gpu_util)
    run_and_compare(inp, extra, f"small {B}x{L}x{E} {act} {dt_mode}",
                     conditioned=(act == "f32" and dt_mode == "wide"))


@pytest.mark.parametrize("L", [3, 900])
def test_in_place_caches(L):
    inp, extra = make_case(2, L, 96, "f32", seed=5, caches=True)
    run_and_compare(inp, extra, f"in-place L={L}", inplace=True)


def test_empty_sequence_copies_caches():
    inp, extra = make_case(2, 0, 80, "f32", seed=9, caches=True)
    say("[parity] empty sequence")
    d = to_device(inp)
    cin = torch.from_numpy(extra["conv_cache_in"]).cuda()
    sin = torch.from_numpy(extra["ssm_state_in"]).cuda()
    y, cache, state = gpu_prefill(d, conv_cache_in=cin, ssm_state_in=sin)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 80)
    np.testing.assert_array_equal(cache.cpu().numpy(), extra["conv_cache_in"])
    np.testing.assert_array_equal(state.cpu().numpy(), extra["ssm_state_in"])
    y, cache, state = gpu_prefill(d)
    torch.cuda.synchronize()
    assert not cache.cpu().numpy().any() and not state.cpu().numpy().any()


@pytest.mark.parametrize("raw", [-1000.0, 1000.0, -50.0, 50.0])
def test_dt_clip_extremes(raw):
    inp, extra = make_case(1, 300, 64, "f32", seed=11, caches=True)
    inp["dt_raw"][:, ::3, :] = np.float32(raw)
    run_and_compare(inp, extra, f"dt_raw={raw}", conditioned=raw > 0)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_prefill_continuation(act):
    """Prefill L1 tokens, then L2 more from the returned caches == the oracle over L1 + L2."""
    inp, extra = make_case(2, 1200, 72, act, seed=13, caches=True)
    L1 = 700
    say(f"[parity] continuation {act}")
    d = to_device(inp)
    cin = torch.from_numpy(extra["conv_cache_in"]).cuda()
    sin = torch.from_numpy(extra["ssm_state_in"]).cuda()
    part = lambda a, b: {k: (v[:, a:b].contiguous() if k in ("x", "z", "dt_raw", "B", "C")  # noqa
                             else v) for k, v in d.items()}
    y1, c1, s1 = gpu_prefill(part(0, L1), conv_cache_in=cin, ssm_state_in=sin)
    y2, c2, s2 = gpu_prefill(part(L1, 1200), conv_cache_in=c1, ssm_state_in=s1,
                             conv_cache_out=c1, ssm_state_out=s1)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp, threads=8, **extra)
    assert_close(np.concatenate([host(y1), host(y2)], axis=1), ref["y"], TOL[act], "y")
    assert_close(host(s2), ref["ssm_state"], STATE_TOL[act], "state")
    np.testing.assert_array_equal(host(c2), ref["conv_cache"])


def test_workspace_reuse():
    """The same workspace tensor serves consecutive calls (contents need no initialisation)."""
    import selective_state_space_depthwise_amd as axon

    inp_a, _ = make_case(1, 1000, 64, "f32", seed=21)
    inp_b, _ = make_case(1, 1000, 64, "f32", seed=22)
    ws = torch.full((axon.prefill_workspace_bytes(1, 1000, 64),), 0xAB, dtype=torch.uint8,
                    device="cuda")
    for inp in (inp_a, inp_b, inp_a):
        y, _, _ = gpu_prefill(to_device(inp), workspace=ws)
        torch.cuda.synchronize()
        assert_close(host(y), oracle.prefill(inp, threads=8)["y"], TOL["f32"], "y")


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_decode_steps_match_oracle(act):
    """A prefill, then single-token decode steps with in-place caches; every step's y and the
    final caches against the oracle's decode steps."""
    B, E, L0, steps = 3, 100, 20, 12
    inp, extra = make_case(B, L0, E, act, seed=31, caches=True)
    say(f"[parity] decode {act}")
    d = to_device(inp)
    _, cache, state = gpu_prefill(d, conv_cache_in=torch.from_numpy(extra["conv_cache_in"]).cuda(),
                                  ssm_state_in=torch.from_numpy(extra["ssm_state_in"]).cuda())
    ref = oracle.prefill(inp, threads=8, **extra)
    rcache, rstate = ref["conv_cache"].copy(), ref["ssm_state"].copy()
    w = workloads.Workload(0, "dec", "decode", B, L0, E, act)
    for s in range(steps):
        st = workloads.decode_step_inputs(w, s)
        if s == 5:
            st["dt_raw"][:, :7] = np.float32(1000.0)  # hit the upper clip
        std = {k: torch.from_numpy(st[k]).cuda().to(d["x"].dtype) for k in st}
        y = gpu_decode(std, d, cache, state)
        ry = oracle.decode_step(st, inp, rcache, rstate)
        torch.cuda.synchronize()
        assert_close(host(y), ry, TOL[act], f"decode step {s} y")
    assert_close(host(state), rstate, STATE_TOL[act], "decode state")
    np.testing.assert_array_equal(host(cache), rcache)


def test_decode_equals_prefill_on_gpu():
    """GPU decode, token by token, agrees with one GPU prefill over the same tokens."""
    B, E, L = 2, 130, 9
    inp, extra = make_case(B, L, E, "f32", seed=41, caches=True)
    d = to_device(inp)
    cin = torch.from_numpy(extra["conv_cache_in"]).cuda()
    sin = torch.from_numpy(extra["ssm_state_in"]).cuda()
    y_full, c_full, s_full = gpu_prefill(d, conv_cache_in=cin, ssm_state_in=sin)
    cache, state = cin.clone(), sin.clone()
    ys = []
    for t in range(L):
        step = {k: d[k][:, t].contiguous() for k in ("x", "z", "dt_raw", "B", "C")}
        ys.append(gpu_decode(step, d, cache, state))
    torch.cuda.synchronize()
    assert_close(host(torch.stack(ys, 1)), host(y_full), TOL["f32"], "y")
    assert_close(host(state), host(s_full), TOL["f32"], "state")
    np.testing.assert_array_equal(host(cache), host(c_full))


# --------------------------------------------------------------------------- full-size workloads
def _full_size_prefill(index, n_samples):
    w = workloads.workload(index)
    say(f"[parity] full size {w.name}: drawing inputs")
    inp = workloads.prefill_inputs(w)
    d = to_device(inp)
    say(f"[parity] full size {w.name}: running the HIP path")
    y, cache, state = gpu_prefill(d)
    torch.cuda.synchronize()
    del d
    assert bool(torch.isfinite(y).all()), "non-finite outputs"
    Bsz, L, E = inp["x"].shape
    picks = sample_channels(Bsz, E, n_samples, seed=index)
    say(f"[parity] full size {w.name}: oracle on {len(picks)} channels")
    yc = y[[b for b, _ in picks], :, [e for _, e in picks]]  # (n, L)
    got_y = host(yc)
    got_state = host(state[[b for b, _ in picks], [e for _, e in picks], :])
    got_cache = host(cache[[b for b, _ in picks], :, [e for _, e in picks]])
    worst = 0.0
    for k, (b, e) in enumerate(picks):
        ref = oracle.channel(inp, b, e)
        assert_close(got_y[k], ref["y"], TOL[w.act], f"{w.name} y[{b},:,{e}]")
        assert_close(got_state[k], ref["ssm_state"], STATE_TOL[w.act], f"state[{b},{e}]")
        np.testing.assert_array_equal(got_cache[k], ref["conv_cache"])
        worst = max(worst, float(np.max(np.abs(got_y[k] - ref["y"]) / (1 + np.abs(ref["y"])))))
    say(f"[parity] full size {w.name}: worst |err|/(1+|ref|) = {worst:.3e}")


def test_full_size_axon_prefill_fp32():
    _full_size_prefill(1, 48)


def test_full_size_axon_prefill_bf16_batch8():
    _full_size_prefill(2, 40)


def test_full_size_long_context_bf16():
    _full_size_prefill(4, 24)


def test_full_size_decode_batch64():
    """128-token prefill of 64 sequences, then 256 decode steps; sampled channels are followed
    through every step by the oracle (prefill then decode of that channel alone)."""
    w = workloads.workload(3)
    say("[parity] full size decode: seeding prefill")
    pre = workloads.prefill_inputs(w)  # (64, 128, 7680)
    d = to_device(pre)
    _, cache, state = gpu_prefill(d)
    B, E = w.batch, w.d_inner
    picks = sample_channels(B, E, 24, seed=3)
    bi = [b for b, _ in picks]
    ei = [e for _, e in picks]
    seq = {k: [] for k in ("x", "z", "dt_raw", "B", "C")}
    ys = []
    say("[parity] full size decode: 256 steps")
    for s in range(w.decode_steps):
        st = workloads.decode_step_inputs(w, s)
        std = {k: torch.from_numpy(st[k]).cuda() for k in st}
        y = gpu_decode(std, d, cache, state)
        ys.append(host(y[bi, ei]))
        for k in ("x", "z", "dt_raw"):
            seq[k].append(st[k][bi, ei])
        for k in ("B", "C"):
            seq[k].append(st[k][bi])
    torch.cuda.synchronize()
    got = np.stack(ys, axis=1)  # (n, steps)
    got_state = host(state[bi, ei, :])
    got_cache = host(cache[bi, :, ei])
    say("[parity] full size decode: oracle")
    for k, (b, e) in enumerate(picks):
        ref0 = oracle.channel(pre, b, e)
        chan = single_channel_inputs(pre, e, {key: np.stack([v[k] for v in seq[key]])
                                              for key in seq})
        ref = oracle.channel(chan, 0, 0, conv_cache_in=ref0["conv_cache"].reshape(1, 3, 1),
                             ssm_state_in=ref0["ssm_state"].reshape(1, 1, 16))
        assert_close(got[k], ref["y"], TOL["f32"], f"decode y[{b},{e}]")
        assert_close(got_state[k], ref["ssm_state"], STATE_TOL["f32"], f"decode state[{b},{e}]")
        np.testing.assert_array_equal(got_cache[k], ref["conv_cache"])
