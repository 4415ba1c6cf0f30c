"""The size limits the C ABI accepts, run on the GPU: d_inner at its maximum (2^23 channels) and
batch at its maximum (65535 rows), for prefill and for the decode step, compared with the oracle
(sampled channels at 2^23, every channel at 65535 rows); the SSD core at 65535 heads and at 65535
batch rows. One past each limit is rejected before any launch; that is checked on the CPU in
test_abi_cpu.py."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_util import (STATE_TOL, TOL, assert_close, gpu_decode, gpu_prefill, host, make_case,
                      say, to_device)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

MAX_D_INNER = 1 << 23
MAX_BATCH = 65535


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_depthwise_amd as axon

    axon.load()
    yield
    torch.cuda.empty_cache()


def test_max_d_inner_prefill_and_decode():
    """2^23 channels, 5 tokens then one decode step: the last channel, the channel-group
    boundaries and random channels follow the oracle."""
    E, L = MAX_D_INNER, 5
    say(f"[limits] prefill B=1 L={L} E={E}")
    inp, extra = make_case(1, L + 1, E, "f32", seed=90, caches=True)
    pre = {k: (v[:, :L] if k in ("x", "z", "dt_raw", "B", "C") else v) for k, v in inp.items()}
    d = to_device(pre)
    cin = torch.from_numpy(extra["conv_cache_in"]).cuda()
    sin = torch.from_numpy(extra["ssm_state_in"]).cuda()
    y, cache, state = gpu_prefill(d, conv_cache_in=cin, ssm_state_in=sin)
    say("[limits] decode step at E = 2^23")
    step = {k: torch.from_numpy(np.ascontiguousarray(inp[k][:, L])).cuda()
            for k in ("x", "z", "dt_raw", "B", "C")}
    y1 = gpu_decode(step, d, cache, state)
    torch.cuda.synchronize()
    picks = sorted({0, 15, 16, 31, 32, E // 2, E - 17, E - 16, E - 2, E - 1,
                    *np.random.default_rng(91).integers(0, E, 6).tolist()})
    for e in picks:
        ref = oracle.channel(inp, 0, e, conv_cache_in=extra["conv_cache_in"],
                             ssm_state_in=extra["ssm_state_in"])
        assert_close(host(y[0, :, e]), ref["y"][:L], TOL["f32"], f"y[0,:,{e}]")
        assert_close(host(y1[0, e:e + 1]), ref["y"][L:], TOL["f32"], f"decode y[0,{e}]")
        assert_close(host(state[0, e]), ref["ssm_state"], STATE_TOL["f32"], f"state[0,{e}]")
        np.testing.assert_array_equal(host(cache[0, :, e]), ref["conv_cache"])


def test_max_batch_prefill_and_decode():
    """65535 batch rows of 16 channels, 3 tokens then one decode step, every output compared."""
    B, E, L = MAX_BATCH, 16, 3
    say(f"[limits] prefill B={B} L={L} E={E}")
    inp, extra = make_case(B, L + 1, E, "bf16", seed=92, caches=True)
    pre = {k: (np.ascontiguousarray(v[:, :L]) if k in ("x", "z", "dt_raw", "B", "C") else v)
           for k, v in inp.items()}
    d = to_device(pre)
    cin = torch.from_numpy(extra["conv_cache_in"]).cuda()
    sin = torch.from_numpy(extra["ssm_state_in"]).cuda()
    y, cache, state = gpu_prefill(d, conv_cache_in=cin, ssm_state_in=sin)
    say("[limits] decode step at B = 65535")
    step = {k: torch.from_numpy(np.ascontiguousarray(inp[k][:, L])).cuda().to(torch.bfloat16)
            for k in ("x", "z", "dt_raw", "B", "C")}
    y1 = gpu_decode(step, d, cache, state)
    torch.cuda.synchronize()
    ref = oracle.prefill(inp, conv_cache_in=extra["conv_cache_in"],
                         ssm_state_in=extra["ssm_state_in"], threads=16)
    got = np.concatenate([host(y), host(y1)[:, None, :]], axis=1)
    assert_close(got, ref["y"], TOL["bf16"], "y (prefill + decode)")
    assert_close(host(state), ref["ssm_state"], STATE_TOL["bf16"], "state")
    np.testing.assert_array_equal(host(cache), ref["conv_cache"])


def _ssd_limit_case(B, L, H, seed):
    import workloads

    w = workloads.SsdWorkload(9, "limit", B, L, H, "f32")
    inp = workloads.ssd_inputs(w, seed_offset=seed)
    dev = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).cuda()
           for k in ("x", "dt_raw", "B", "C", "A_log", "D", "dt_bias")}
    return inp, dev


@pytest.mark.parametrize("B,H", [(1, MAX_BATCH), (MAX_BATCH, 1)])
def test_ssd_max_heads_and_batch(B, H):
    """The SSD core at 65535 heads, and at 65535 batch rows (3 tokens, incoming state), every
    output compared with the oracle."""
    import selective_state_space_depthwise_amd as axon

    L = 3
    say(f"[limits] ssd B={B} H={H} L={L}")
    inp, d = _ssd_limit_case(B, L, H, seed=B + H)
    sin = np.random.default_rng(93).standard_normal((B, H, 64, 128)).astype(np.float32)
    y, st = axon.ssd_scan(d["x"], d["dt_raw"], d["B"], d["C"], d["A_log"], d["D"], d["dt_bias"],
                          dt_min=inp["dt_min"], dt_max=inp["dt_max"],
                          state_in=torch.from_numpy(sin).cuda())
    torch.cuda.synchronize()
    ref = oracle.ssd_scan(inp, state_in=sin, threads=16)
    assert_close(host(y), ref["y"], TOL["f32"], "ssd y")
    assert_close(host(st), ref["ssm_state"], STATE_TOL["f32"], "ssd state")
