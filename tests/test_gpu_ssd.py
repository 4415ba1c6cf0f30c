"""Parity of the Mamba-2 SSD core (64-token chunks on the matrix cores) with the oracle's plain
sequential recurrence: ragged last chunks, one-token and empty sequences, incoming states,
continuation in place, bf16 activations, clip hits, and the Mamba-2 block shape of
"Selective State Space Models (Mamba)" (pattern "Mamba-2 block": 64 heads of 64 channels,
d_state 128) at 2048 tokens, compared in full.

Tolerances as for the Axon-SSM path: |gpu - ref| <= 1e-4 (1 + |ref|) for fp32 activations,
2e-2 (1 + |ref|) for bf16 (y is rounded to bf16), 1e-4 (1 + |ref|) for the fp32 state; stress
cases with clip hits add mag = sum_n |C h| + |D x| from the oracle to the bound. The
chunked form sums the same terms in another order (fp32 matrix products over 64 tokens and
128 states, decays as exp2 of cumulative sums over at most 64 tokens), so its rounding error is
of order 1e-6 relative to the magnitude of the summed terms."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import STATE_TOL, TOL, assert_close, host, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_depthwise_amd as axon

    axon.load()
    yield
    torch.cuda.synchronize()


def _inputs(B, L, H, act="f32", dt_mode="axon", seed=0):
    w = workloads.SsdWorkload(7, "case", B, L, H, act, dt_mode)
    return workloads.ssd_inputs(w, seed_offset=seed)


def _dev(inp):
    dt = torch.bfloat16 if inp["act"] == "bf16" else torch.float32
    out = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).cuda().to(dt)
           for k in ("x", "dt_raw", "B", "C")}
    for k in ("A_log", "D", "dt_bias"):
        out[k] = torch.from_numpy(np.ascontiguousarray(inp[k], np.float32)).cuda()
    return out


def _run(d, inp, **kw):
    import selective_state_space_depthwise_amd as axon

    return axon.ssd_scan(d["x"], d["dt_raw"], d["B"], d["C"], d["A_log"], d["D"], d["dt_bias"],
                         dt_min=inp["dt_min"], dt_max=inp["dt_max"], **kw)


def _state(B, H, seed):
    return np.random.default_rng(500 + seed).standard_normal((B, H, 64, 128)).astype(np.float32)


CASES = [
    # (B, L, H, act, dt_mode, with state_in)
    (2, 200, 32, "f32", "axon", True),    # 64 (batch, head) pairs: 4 chunks, ragged tail of 8
    (1, 1, 64, "f32", "axon", True),      # 64 heads, one token
    (4, 130, 16, "bf16", "axon", True),   # bf16, 3 chunks
    (1, 333, 64, "f32", "wide", False),   # clip hits, odd number of chunks
    (1, 64, 2, "f32", "axon", False),     # one whole chunk
    (2, 200, 3, "f32", "axon", True),     # 4 chunks, ragged tail of 8
    (1, 1, 4, "f32", "axon", True),       # one token
    (1, 63, 2, "f32", "axon", True),      # one short chunk
    (2, 65, 2, "f32", "axon", False),     # a chunk plus one token
    (1, 333, 5, "bf16", "axon", True),    # bf16 activations
    (2, 300, 3, "f32", "wide", True),     # dt across [1e-4, 1] with clip hits at 1e-4 and 100
]


@pytest.mark.parametrize("B,L,H,act,dt_mode,h0", CASES)
def test_ssd_matches_oracle(B, L, H, act, dt_mode, h0):
    say(f"[ssd] B={B} L={L} H={H} act={act} dt={dt_mode} state_in={h0}")
    inp = _inputs(B, L, H, act, dt_mode, seed=L + H)
    sin = _state(B, H, L) if h0 else None
    d = _dev(inp)
    y, st = _run(d, inp, state_in=torch.from_numpy(sin).cuda() if h0 else None)
    torch.cuda.synchronize()
    # stress inputs (dt_mode "wide": steps up to the clip) grow the states to thousands and an
    # output can be the small difference of large terms: their bound adds the terms' size
    wide = dt_mode == "wide"
    ref = oracle.ssd_scan(inp, state_in=sin, threads=8, magnitude=wide)
    assert_close(host(y), ref["y"], TOL[act], "ssd y", mag=ref["mag"] if wide else None)
    assert_close(host(st), ref["ssm_state"], STATE_TOL[act], "ssd state")


def test_ssd_empty_sequence_copies_state():
    say("[ssd] L=0")
    inp = _inputs(2, 0, 3)
    d = _dev(inp)
    sin = torch.from_numpy(_state(2, 3, 1)).cuda()
    y, st = _run(d, inp, state_in=sin)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 3, 64)
    assert torch.equal(st, sin)
    _, z = _run(d, inp)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z).item() == 0


def test_ssd_continuation_in_place():
    """L1 tokens, then L2 from the state updated in place, equals the oracle over L1 + L2."""
    say("[ssd] continuation 100 + 77, in place")
    inp = _inputs(2, 177, 3, seed=3)
    sin = _state(2, 3, 3)
    ref = oracle.ssd_scan(inp, state_in=sin, threads=8)
    state = torch.from_numpy(sin.copy()).cuda()
    ys = []
    for a, b in ((0, 100), (100, 177)):
        part = dict(inp)
        for k in ("x", "dt_raw", "B", "C"):
            part[k] = np.ascontiguousarray(inp[k][:, a:b])
        y, _ = _run(_dev(part), part, state_in=state, state_out=state)
        ys.append(host(y))
    torch.cuda.synchronize()
    assert_close(np.concatenate(ys, 1), ref["y"], TOL["f32"], "ssd y (continued)")
    assert_close(host(state), ref["ssm_state"], STATE_TOL["f32"], "ssd state (continued)")


@pytest.mark.parametrize("index", [0, 1])
def test_ssd_block_shape_full(index):
    """The Mamba-2 block shape (64 heads x 64 channels, d_state 128) at 2048 tokens, in the launch
    configuration the benchmark times, compared with the oracle on every output."""
    w = workloads.SSD_WORKLOADS[index]
    say(f"[ssd] full size {w.name}")
    inp = workloads.ssd_inputs(w)
    d = _dev(inp)
    y, st = _run(d, inp)
    torch.cuda.synchronize()
    ref = oracle.ssd_scan(inp, threads=16)
    assert_close(host(y), ref["y"], TOL[w.act], f"{w.name}: y")
    assert_close(host(st), ref["ssm_state"], STATE_TOL[w.act], f"{w.name}: state")
