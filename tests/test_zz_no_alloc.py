"""The allocation-free prefill (axon_ssm_prefill_noalloc, the library's own scratch instead of a
caller workspace) against axon_ssm_prefill through the C ABI, on two calls in a row: the first
on a time-chunked shape whose regular plan needs more workspace than the scratch holds (so the
entry point plans fewer chunks), the second on a smaller chunked input that reuses the scratch
the first call left behind."""
from __future__ import annotations

import numpy as np
import pytest

from gpu_util import STATE_TOL, TOL, assert_close, host, make_case, say, to_device

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _noalloc(d, act):
    from selective_state_space_depthwise_amd import _abi

    Bsz, L, E = d["x"].shape
    y = torch.empty_like(d["x"])
    cache = torch.empty((Bsz, 3, E), dtype=torch.float32, device="cuda")
    state = torch.empty((Bsz, E, 16), dtype=torch.float32, device="cuda")
    shape = _abi.make_shape(Bsz, L, E, act == "bf16")
    prm = _abi.make_params(d["A_log"].data_ptr(), d["D"].data_ptr(), d["dt_bias"].data_ptr(),
                           d["conv_w"].data_ptr(), d["conv_b"].data_ptr(), d["dt_min"],
                           d["dt_max"])
    st = _abi.raw_prefill_noalloc(shape, prm, d["x"].data_ptr(), d["z"].data_ptr(),
                                  d["dt_raw"].data_ptr(), d["B"].data_ptr(), d["C"].data_ptr(),
                                  None, None, y.data_ptr(), cache.data_ptr(), state.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert st == _abi.AXON_OK, _abi.status_string(st)
    return y, cache, state


@pytest.mark.timeout(300)
def test_noalloc_prefill_matches_prefill_twice():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import selective_state_space_depthwise_amd as axon

    axon.load()
    big = (1, 5632, 6000, "f32")     # regular plan: 88 chunks, about 70 MB of workspace
    small = (2, 700, 48, "bf16")     # 11 chunks
    assert axon.prefill_workspace_bytes(1, 5632, 6000) > (64 << 20)
    assert 0 < axon.prefill_workspace_bytes(2, 700, 48, True) < (64 << 20)
    for B, L, E, act in (big, small):
        say(f"[no-alloc] {B}x{L}x{E} {act}")
        inp, _ = make_case(B, L, E, act, seed=L + E)
        d = to_device(inp)
        y0, c0, s0 = axon.prefill(d["x"], d["z"], d["dt_raw"], d["B"], d["C"], d["A_log"],
                                  d["D"], d["dt_bias"], d["conv_w"], d["conv_b"],
                                  dt_min=d["dt_min"], dt_max=d["dt_max"])
        y1, c1, s1 = _noalloc(d, act)
        torch.cuda.synchronize()
        assert_close(host(y1), host(y0), TOL[act], f"no-alloc y {B}x{L}x{E}")
        assert_close(host(s1), host(s0), STATE_TOL[act], f"no-alloc state {B}x{L}x{E}")
        np.testing.assert_array_equal(host(c1), host(c0))
