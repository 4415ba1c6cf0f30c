"""Parity of the HIP path (through the C ABI and the binding) with the CPU oracle.

Every case is compared whole (every output, state and cache element). Small cases span several
time chunks, ragged channel counts (not a multiple of the 64-lane wave) and ragged last chunks;
the full-size workloads run in the same launch configuration as the benchmark, against one
oracle pass over the whole workload.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import (STATE_TOL, TOL, assert_close, gpu_decode, gpu_prefill, host, make_case,
                      max_rel, run_and_compare, say, to_device)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
# the oracle's threads over channels (a GPU machine gives one GPU's job 16 host threads)
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_depthwise_amd as axon

    axon.load()  # fails loudly when the library is missing
    yield
    torch.cuda.synchronize()


SMALL = [
    # (B, L, E, act, dt_mode, caches). Below 6144 channels (batch x d_inner) the lane-per-channel
    # scan runs in time chunks; from there the row scan runs in one pass, 32-token tiles with one
    # state per lane up to 16384 channels, 16-token tiles with two states per lane above.
    (1, 64, 32, "f32", "axon", False),      # the tiny workload itself: one chunk
    (1, 1000, 64, "f32", "axon", False),    # 14 chunks of 72 tokens, ragged last chunk
    (3, 333, 100, "f32", "axon", True),     # 5 chunks, ragged E, caches in
    (2, 517, 130, "bf16", "axon", True),    # 8 chunks, last one 13 tokens
    (1, 16384, 16, "f32", "axon", True),    # the maximum of 256 chunks
    (2, 700, 48, "bf16", "wide", False),    # dt spanning [1e-4, 1] with +-50 clip hits
    (2, 700, 48, "f32", "wide", True),
    (1, 1, 70, "f32", "axon", True),        # L < K-1: the new cache mixes old cache and x
    (1, 2, 70, "bf16", "axon", True),
    (2, 3, 40, "f32", "axon", True),
    (4, 96, 200, "f32", "axon", False),     # one chunk, 800 channels
    (1, 300, 7680, "f32", "axon", True),    # row scan, one state per lane: 10 tiles, ragged
    (1, 200, 7700, "bf16", "axon", True),   # ragged channel groups, 7 tiles
    (2, 100, 9000, "f32", "axon", False),   # two states per lane: 7 tiles of 16
    (1, 1, 7680, "f32", "axon", True),      # row scan, one token: the cache mixes old and new
    (1, 3, 6200, "bf16", "axon", True),
    (1, 32, 7680, "f32", "axon", True),     # exactly one tile
    (1, 33, 7680, "f32", "axon", False),    # two tiles, the second of one token
    (1, 96, 6144, "f32", "axon", True),     # three tiles: one pass of the three-tile loop
    (1, 128, 7680, "bf16", "axon", False),  # four tiles: one loop pass and a tail of one
    # Longer one-state-per-lane sequences: whole passes of the three-tile loop plus tails of
    # one and two tiles, ragged last tiles.
    (1, 256, 7680, "f32", "axon", True),    # 8 tiles: two loop passes, a tail of two
    (1, 257, 6144, "bf16", "axon", True),   # 9 tiles, the last of one token, no tail
    (1, 351, 7700, "f32", "axon", False),   # 11 tiles (a tail of two), ragged channel groups
    (2, 290, 4000, "f32", "wide", True),    # 8000 channels in 2 rows, 10 tiles (a tail of one)
    (1, 225, 6144, "bf16", "wide", False),  # 8 tiles, the last of one token, clip hits
    (2, 65, 9000, "bf16", "axon", True),    # 16-token tiles, 5 tiles, the last of one token
    (1, 260, 16384, "f32", "wide", True),   # 16-token tiles, clip hits, 17 tiles
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
    run_and_compare(inp, extra, f"dt_raw={raw}")


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
# Every element of y, the state and the cache is compared with one oracle pass over the whole
# workload (threads over channels), in the launch configuration bench.py times.
def _full_size_prefill(index):
    w = workloads.workload(index)
    say(f"[parity] full size {w.name}: drawing inputs")
    inp = workloads.prefill_inputs(w)
    d = to_device(inp)
    say(f"[parity] full size {w.name}: running the HIP path")
    y, cache, state = gpu_prefill(d)
    torch.cuda.synchronize()
    del d
    got_state, got_cache = host(state), host(cache)
    got_y = [host(y[b]) for b in range(y.shape[0])]
    del y, cache, state
    say(f"[parity] full size {w.name}: oracle on every channel ({ORACLE_THREADS} threads)")
    ref = oracle.prefill(inp, threads=ORACLE_THREADS)
    worst = 0.0
    for b, gy in enumerate(got_y):
        assert_close(gy, ref["y"][b], TOL[w.act], f"{w.name} y[{b}]")
        worst = max(worst, max_rel(gy, ref["y"][b]))
    assert_close(got_state, ref["ssm_state"], STATE_TOL[w.act], f"{w.name} state")
    np.testing.assert_array_equal(got_cache, ref["conv_cache"], err_msg=f"{w.name} cache")
    say(f"[parity] full size {w.name}: {sum(g.size for g in got_y)} outputs, worst "
        f"|err|/(1+|ref|) = {worst:.3e}")


@pytest.mark.timeout(600)
def test_full_size_axon_prefill_fp32():
    _full_size_prefill(1)


@pytest.mark.timeout(600)
def test_full_size_axon_prefill_bf16_batch8():
    _full_size_prefill(2)


@pytest.mark.timeout(600)
def test_full_size_long_context_bf16():
    _full_size_prefill(4)


@pytest.mark.timeout(600)
def test_full_size_decode_batch64():
    """128-token prefill of 64 sequences, then 256 decode steps of all 64 x 7680 channels; every
    step's whole output and the final caches against the oracle stepping the same batch."""
    w = workloads.workload(3)
    say("[parity] full size decode: seeding prefill")
    pre = workloads.prefill_inputs(w)  # (64, 128, 7680)
    d = to_device(pre)
    _, cache, state = gpu_prefill(d)
    ref = oracle.prefill(pre, threads=ORACLE_THREADS)
    rcache, rstate = ref["conv_cache"], ref["ssm_state"]
    assert_close(host(state), rstate, STATE_TOL["f32"], "decode seed state")
    np.testing.assert_array_equal(host(cache), rcache)
    say(f"[parity] full size decode: {w.decode_steps} steps of {w.batch} x {w.d_inner}")
    worst = 0.0
    for s in range(w.decode_steps):
        st = workloads.decode_step_inputs(w, s)
        std = {k: torch.from_numpy(st[k]).cuda() for k in st}
        y = host(gpu_decode(std, d, cache, state))
        ry = oracle.decode_step(st, pre, rcache, rstate, threads=ORACLE_THREADS)
        assert_close(y, ry, TOL["f32"], f"decode step {s} y")
        worst = max(worst, max_rel(y, ry))
    torch.cuda.synchronize()
    assert_close(host(state), rstate, STATE_TOL["f32"], "decode state")
    np.testing.assert_array_equal(host(cache), rcache)
    say(f"[parity] full size decode: worst |err|/(1+|ref|) = {worst:.3e}")


def test_side_stream_with_implicit_workspace():
    """A time-chunked prefill (carry pass, combine, final pass through a workspace the binding
    allocates) launched on a side stream, while the current stream at once allocates blocks of
    the workspace's size and fills them: the binding records the side stream on what it
    allocated, so that memory is not handed out again before the side stream's kernels ran."""
    import selective_state_space_depthwise_amd as axon

    inp, extra = make_case(2, 1500, 96, "f32", seed=17, caches=False)
    d = to_device(inp)
    need = axon.prefill_workspace_bytes(2, 1500, 96)
    assert need > 0, "the case must use the time-chunked path"
    say(f"[parity] side stream, implicit workspace of {need} bytes")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(4):
        y, cache, state = gpu_prefill(d, stream=side)
        outs.append((y, cache, state))
        junk = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(3)]
        for j in junk:
            j.fill_(0xFF)
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    ref = oracle.prefill(inp, threads=ORACLE_THREADS)
    for y, cache, state in outs:
        assert_close(host(y), ref["y"], TOL["f32"], "side stream y")
        assert_close(host(state), ref["ssm_state"], STATE_TOL["f32"], "side stream state")
        np.testing.assert_array_equal(host(cache), ref["conv_cache"])
