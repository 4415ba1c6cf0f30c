"""libaxonscan's C ABI on the CPU: the library loads, exports what the header declares, sizes its
workspace from the shape alone, and rejects bad arguments before anything is launched. No call
here passes validation, so nothing reaches the GPU (fake pointers are never dereferenced)."""
import ctypes

import pytest

from selective_state_space_depthwise_amd import _abi

A = _abi
P = 0x7F0000000000  # a fake, 16-byte aligned device address; never dereferenced


def _shape(batch=1, seqlen=64, d_inner=32, bf16=False, d_state=16, d_conv=4):
    return A.make_shape(batch, seqlen, d_inner, bf16, d_state=d_state, d_conv=d_conv)


def _params(dt_min=1e-4, dt_max=100.0, base=P + (1 << 30)):
    return A.make_params(base, base + (1 << 20), base + (2 << 20), base + (3 << 20),
                         base + (4 << 20), dt_min, dt_max)


def _buffers():
    """Disjoint fake buffers, 64 MiB apart."""
    names = ["x", "z", "dt", "B", "C", "cin", "sin", "y", "cout", "sout", "ws"]
    return {n: P + (i + 1) * (64 << 20) for i, n in enumerate(names)}


def _prefill(shape=None, params=None, ws_bytes=1 << 30, **over):
    b = _buffers()
    b.update(over)
    return A.raw_prefill(shape or _shape(), params or _params(), b["x"], b["z"], b["dt"], b["B"],
                         b["C"], b["cin"], b["sin"], b["y"], b["cout"], b["sout"], b["ws"],
                         ws_bytes, None)


def _decode(shape=None, params=None, **over):
    b = _buffers()
    b.update(over)
    return A.raw_decode_step(shape or _shape(seqlen=1), params or _params(), b["x"], b["z"],
                             b["dt"], b["B"], b["C"], b["cin"], b["sin"], b["y"], None)


def test_library_exports_every_declared_symbol():
    lib = A.load()
    declared = A.declared_functions()
    assert set(declared) >= {"axon_ssm_prefill", "axon_ssm_decode_step",
                             "axon_ssm_prefill_workspace_bytes", "axon_status_string",
                             "axon_version"}
    for name in declared:
        assert hasattr(lib, name), f"{name} is declared in include/axonscan.h but not exported"
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings():
    assert A.version() == 300
    for st in range(5):
        assert A.status_string(st)
    assert A.status_string(99) == "unknown status"


def test_workspace_is_a_pure_function_of_shape():
    # enough channels to fill the GPU: no time chunks, no workspace
    assert A.workspace_bytes(_shape(1, 64, 32)) == 0
    assert A.workspace_bytes(_shape(64, 1, 7680)) == 0
    assert A.workspace_bytes(_shape(1, 2048, 7680)) == 0      # fills the GPU by state splitting
    assert A.workspace_bytes(_shape(8, 4096, 7680, True)) == 0
    # few channels, long sequence: chunked, workspace = carries + halo
    assert A.workspace_bytes(_shape(2, 65536, 2048, True)) > 0
    ws1 = A.workspace_bytes(_shape(1, 8192, 256))
    assert ws1 == A.workspace_bytes(_shape(1, 8192, 256))
    assert ws1 > 2 * 16 * 4 * 256  # at least two chunks of carries
    assert ws1 % 256 == 0
    # empty and one-token sequences plan a single chunk, whatever the channel count
    for bsz, e in ((1, 16), (1, 7680), (64, 7680)):
        assert A.workspace_bytes(_shape(bsz, 0, e)) == 0
        assert A.workspace_bytes(_shape(bsz, 1, e)) == 0
    # invalid shapes report 0
    assert A.workspace_bytes(_shape(d_state=8)) == 0
    assert A.workspace_bytes(_shape(batch=0)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(d_state=8), A.AXON_ERR_UNSUPPORTED),
    (dict(d_state=32), A.AXON_ERR_UNSUPPORTED),
    (dict(d_inner=(1 << 23) + 1, seqlen=1), A.AXON_ERR_UNSUPPORTED),
    (dict(batch=65536, d_inner=1, seqlen=1), A.AXON_ERR_UNSUPPORTED),
    (dict(d_conv=3), A.AXON_ERR_UNSUPPORTED),
    (dict(batch=0), A.AXON_ERR_INVALID_ARGUMENT),
    (dict(d_inner=0), A.AXON_ERR_INVALID_ARGUMENT),
    (dict(seqlen=-1), A.AXON_ERR_INVALID_ARGUMENT),
    (dict(batch=70000), A.AXON_ERR_UNSUPPORTED),
    (dict(batch=4, seqlen=1 << 30, d_inner=1 << 20), A.AXON_ERR_INVALID_ARGUMENT),
])
def test_prefill_rejects_bad_shapes(kw, status):
    assert _prefill(shape=_shape(**kw)) == status


@pytest.mark.parametrize("act,disc", [(2, 0), (-1, 0), (0, 2), (0, -1), (7, 9)])
def test_unknown_variants_are_unsupported(act, disc):
    prm = A.make_params(*([P + (1 << 30) + i * (1 << 20) for i in range(5)]), 1e-4, 100.0,
                        conv_activation=act, discretization=disc)
    assert _prefill(params=prm) == A.AXON_ERR_UNSUPPORTED
    assert _decode(params=prm) == A.AXON_ERR_UNSUPPORTED


def test_prefill_rejects_unknown_dtype():
    s = _shape()
    s.act_dtype = 7
    assert _prefill(shape=s) == A.AXON_ERR_UNSUPPORTED


def test_prefill_rejects_null_shape_and_params():
    lib = A.load()
    b = _buffers()
    st = lib.axon_ssm_prefill(None, ctypes.byref(_params()), b["x"], b["z"], b["dt"], b["B"],
                              b["C"], None, None, b["y"], b["cout"], b["sout"], b["ws"], 0, None)
    assert st == A.AXON_ERR_INVALID_ARGUMENT
    sh = _shape()
    st = lib.axon_ssm_prefill(ctypes.byref(sh), None, b["x"], b["z"], b["dt"], b["B"], b["C"],
                              None, None, b["y"], b["cout"], b["sout"], b["ws"], 0, None)
    assert st == A.AXON_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("name", ["x", "z", "dt", "B", "C", "y", "cout", "sout"])
def test_prefill_rejects_null_required_pointer(name):
    assert _prefill(**{name: None}) == A.AXON_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("name", ["x", "z", "dt", "B", "C", "y", "cout", "sout", "cin", "sin"])
def test_prefill_rejects_misaligned_pointer(name):
    b = _buffers()
    assert _prefill(**{name: b[name] + 4}) == A.AXON_ERR_INVALID_ARGUMENT


def test_prefill_rejects_bad_params():
    assert _prefill(params=_params(dt_min=1.0, dt_max=0.5)) == A.AXON_ERR_INVALID_ARGUMENT
    assert _prefill(params=_params(dt_min=float("nan"))) == A.AXON_ERR_INVALID_ARGUMENT
    assert _prefill(params=_params(dt_max=float("inf"))) == A.AXON_ERR_INVALID_ARGUMENT
    assert _prefill(params=_params(dt_min=-1.0)) == A.AXON_ERR_INVALID_ARGUMENT
    p = _params()
    p.A_log = None
    assert _prefill(params=p) == A.AXON_ERR_INVALID_ARGUMENT
    p = _params()
    p.conv_w = p.conv_w + 8
    assert _prefill(params=p) == A.AXON_ERR_INVALID_ARGUMENT


def test_prefill_workspace_checks():
    sh = _shape(1, 8192, 256)
    need = A.workspace_bytes(sh)
    assert need > 0
    assert _prefill(shape=sh, ws_bytes=need - 1) == A.AXON_ERR_WORKSPACE_TOO_SMALL
    assert _prefill(shape=sh, ws_bytes=need, ws=None) == A.AXON_ERR_INVALID_ARGUMENT
    assert _prefill(shape=sh, ws_bytes=need, ws=_buffers()["ws"] + 8) == \
        A.AXON_ERR_INVALID_ARGUMENT


def test_prefill_rejects_forbidden_aliasing():
    b = _buffers()
    # y on top of an input
    assert _prefill(y=b["x"]) == A.AXON_ERR_INVALID_ARGUMENT
    assert _prefill(y=b["B"] + 16) == A.AXON_ERR_INVALID_ARGUMENT
    # partial overlap of a cache with its input (exact equality is the allowed in-place form)
    assert _prefill(cout=b["cin"] + 16) == A.AXON_ERR_INVALID_ARGUMENT
    assert _prefill(sout=b["sin"] + 16) == A.AXON_ERR_INVALID_ARGUMENT
    # cache/state outputs over read-only inputs, or over each other
    assert _prefill(cout=b["x"]) == A.AXON_ERR_INVALID_ARGUMENT
    assert _prefill(sout=b["cout"]) == A.AXON_ERR_INVALID_ARGUMENT
    # workspace over an output
    sh = _shape(1, 8192, 256)
    assert _prefill(shape=sh, ws=b["y"]) == A.AXON_ERR_INVALID_ARGUMENT


def test_decode_rejects_bad_arguments():
    assert _decode(shape=_shape(seqlen=1, d_state=4)) == A.AXON_ERR_UNSUPPORTED
    assert _decode(shape=_shape(seqlen=1, batch=0)) == A.AXON_ERR_INVALID_ARGUMENT
    for name in ["x", "z", "dt", "B", "C", "cin", "sin", "y"]:
        assert _decode(**{name: None}) == A.AXON_ERR_INVALID_ARGUMENT
        assert _decode(**{name: _buffers()[name] + 4}) == A.AXON_ERR_INVALID_ARGUMENT
    b = _buffers()
    assert _decode(y=b["x"]) == A.AXON_ERR_INVALID_ARGUMENT
    assert _decode(y=b["cin"]) == A.AXON_ERR_INVALID_ARGUMENT
    assert _decode(sin=b["cin"]) == A.AXON_ERR_INVALID_ARGUMENT
    assert _decode(params=_params(dt_min=2.0, dt_max=1.0)) == A.AXON_ERR_INVALID_ARGUMENT


# ---- the layer entry points (no GPU calls: every case is rejected before any launch) ----------
def _lshape(**kw):
    base = dict(batch=1, seqlen=8, d_model=32, d_inner=48, act_bf16=False)
    base.update(kw)
    return A.make_layer_shape(base["batch"], base["seqlen"], base["d_model"], base["d_inner"],
                              base["act_bf16"], d_state=base.get("d_state", 16),
                              d_conv=base.get("d_conv", 4))


def test_layer_workspace_is_a_pure_function_of_shape():
    a = A.layer_workspace_bytes(_lshape())
    assert a > 0 and a % 256 == 0 and a == A.layer_workspace_bytes(_lshape())
    assert A.layer_workspace_bytes(_lshape(seqlen=64)) > a
    assert A.layer_workspace_bytes(_lshape(d_state=8)) == 0
    assert A.layer_workspace_bytes(_lshape(seqlen=0)) == 0
    assert A.layer_workspace_bytes(_lshape(batch=4, seqlen=1 << 62)) == 0  # batch * seqlen overflow


_FAKE_CTX = ctypes.create_string_buffer(4096)  # zeroed host memory: a context with no handle


def _lforward(ctx=ctypes.addressof(_FAKE_CTX), shape=None, params=None, ws_bytes=1 << 32, **over):
    b = _buffers()
    b.update(over)
    w = A.LayerWeights(P + (5 << 30), P + (6 << 30), P + (7 << 30), params or _params())
    return A.raw_layer_forward(ctx, shape or _lshape(), w, b["x"], b["cin"], b["sin"], b["y"],
                               b["cout"], b["sout"], b["ws"], ws_bytes, None)


def test_layer_forward_rejects_bad_arguments():
    assert _lforward(ctx=None) == A.AXON_ERR_INVALID_ARGUMENT
    assert _lforward(shape=_lshape(d_state=8)) == A.AXON_ERR_UNSUPPORTED
    assert _lforward(shape=_lshape(seqlen=0)) == A.AXON_ERR_INVALID_ARGUMENT
    assert _lforward(x=P + 4) == A.AXON_ERR_INVALID_ARGUMENT          # misaligned input
    assert _lforward(y=None) == A.AXON_ERR_INVALID_ARGUMENT           # no output
    assert _lforward(ws_bytes=16) == A.AXON_ERR_WORKSPACE_TOO_SMALL
    assert _lforward(y=_buffers()["x"]) == A.AXON_ERR_INVALID_ARGUMENT  # out overlaps x_in
    bad = A.make_params(*([P + (1 << 30) + i * (1 << 20) for i in range(5)]), 1e-4, 100.0,
                        conv_activation=3)
    assert _lforward(params=bad) == A.AXON_ERR_UNSUPPORTED
    assert _lforward() == A.AXON_ERR_INVALID_ARGUMENT                 # context without a handle


def _lcheck(shape=None, params=None, ws_bytes=1 << 32, weights=None, **over):
    """axon_layer_forward_check on host addresses spread far apart (compared, never read)."""
    b = _buffers()
    b.update(over)
    w = weights or A.LayerWeights(b.get("W_in", P + (5 << 30)), b.get("W_f", P + (6 << 30)),
                                  b.get("W_out", P + (7 << 30)), params or _params())
    return A.raw_layer_forward_check(shape or _lshape(), w, b["x"], b["cin"], b["sin"], b["y"],
                                     b["cout"], b["sout"], b["ws"], ws_bytes)


def test_layer_check_accepts_valid_arguments():
    assert _lcheck() == A.AXON_OK
    b = _buffers()
    assert _lcheck(cout=b["cin"], sout=b["sin"]) == A.AXON_OK    # in-place caches
    assert _lcheck(cin=None, sin=None) == A.AXON_OK               # zero initial caches
    assert _lforward() == A.AXON_ERR_INVALID_ARGUMENT              # a context without a handle


@pytest.mark.parametrize("case", [
    "out_over_x", "out_over_W_in", "out_over_W_f", "out_over_W_out", "out_over_A_log",
    "out_over_conv_w", "out_over_cache_in", "out_over_state_in", "out_over_cache_out",
    "out_over_state_out", "out_over_ws", "ws_over_x", "ws_over_W_f", "ws_over_cache_in",
    "ws_over_state_out", "ws_over_D", "cache_out_over_x", "cache_out_over_W_out",
    "cache_out_over_dt_bias", "cache_out_partly_over_cache_in", "cache_out_over_state_in",
    "cache_out_over_state_out", "state_out_over_x", "state_out_over_W_in",
    "state_out_over_conv_b", "state_out_partly_over_state_in", "state_out_over_cache_in"])
def test_layer_check_rejects_forbidden_aliasing(case):
    b = _buffers()
    prm = _params()
    win, wf, wout = P + (5 << 30), P + (6 << 30), P + (7 << 30)
    target, what = case.split("_over_") if "_partly_over_" not in case else \
        (case.split("_partly_over_")[0], case.split("_partly_over_")[1])
    addr = {"x": b["x"], "W_in": win, "W_f": wf, "W_out": wout, "A_log": prm.A_log,
            "D": prm.D, "dt_bias": prm.dt_bias, "conv_w": prm.conv_w, "conv_b": prm.conv_b,
            "cache_in": b["cin"], "state_in": b["sin"], "cache_out": b["cout"],
            "state_out": b["sout"], "ws": b["ws"]}[what]
    if "_partly_over_" in case:
        addr += 16  # a partial overlap: exact equality is the allowed in-place form
    key = {"out": "y", "ws": "ws", "cache_out": "cout", "state_out": "sout"}[target]
    assert _lcheck(**{key: addr}) == A.AXON_ERR_INVALID_ARGUMENT, case
    # the forward call rejects it the same way, before looking at the context
    assert _lforward(**{key: addr}) == A.AXON_ERR_INVALID_ARGUMENT, case


# ---- Mamba-2 SSD core ----------------------------------------------------------------------------
def _ssd_shape(batch=1, seqlen=200, heads=4, bf16=False, head_dim=64, d_state=128):
    return A.make_ssd_shape(batch, seqlen, heads, bf16, head_dim=head_dim, d_state=d_state)


def _ssd_params(dt_min=1e-4, dt_max=100.0, base=P + (1 << 30)):
    return A.SsdParams(base, base + (1 << 20), base + (2 << 20), dt_min, dt_max)


def _ssd(shape=None, params=None, ws_bytes=1 << 30, **over):
    b = _buffers()
    b.update(over)
    return A.raw_ssd_scan(shape or _ssd_shape(), params or _ssd_params(), b["x"], b["dt"],
                          b["B"], b["C"], b["sin"], b["y"], b["sout"], b["ws"], ws_bytes, None)


def test_ssd_workspace_is_a_pure_function_of_shape():
    # (B, H, chunks, 64, 128) chunk states + (B, H, chunks) decays + (B, chunks, 64, 64) C B^T
    # + (B, H, chunks, 64, 64) incoming-state products, each rounded up to 256 bytes
    n = A.ssd_workspace_bytes(_ssd_shape(batch=1, seqlen=2048, heads=64))
    assert n == 64 * 32 * 64 * 128 * 4 + 64 * 32 * 4 + 32 * 64 * 64 * 4 + 64 * 32 * 64 * 64 * 4
    n = A.ssd_workspace_bytes(_ssd_shape(batch=1, seqlen=2048, heads=63))
    assert n == (63 * 32 * 64 * 128 * 4 + 8192 + 32 * 64 * 64 * 4  # 63 * 32 * 4 rounds up
                 + 63 * 32 * 64 * 64 * 4)
    assert A.ssd_workspace_bytes(_ssd_shape(seqlen=65, heads=1)) == (2 * 8192 * 4 + 256 +
                                                                     2 * 4096 * 4 + 2 * 4096 * 4)
    assert A.ssd_workspace_bytes(_ssd_shape(seqlen=0)) == 0
    assert A.ssd_workspace_bytes(_ssd_shape(head_dim=32)) == 0
    assert A.ssd_workspace_bytes(_ssd_shape(batch=0)) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=32), A.AXON_ERR_UNSUPPORTED), (dict(d_state=64), A.AXON_ERR_UNSUPPORTED),
    (dict(batch=65536), A.AXON_ERR_UNSUPPORTED), (dict(heads=65536), A.AXON_ERR_UNSUPPORTED),
    (dict(batch=0), A.AXON_ERR_INVALID_ARGUMENT), (dict(heads=0), A.AXON_ERR_INVALID_ARGUMENT),
    (dict(seqlen=-1), A.AXON_ERR_INVALID_ARGUMENT),
    (dict(batch=1 << 20, seqlen=1 << 20, heads=1 << 10), A.AXON_ERR_UNSUPPORTED),
    (dict(batch=60000, seqlen=1 << 20, heads=60000), A.AXON_ERR_INVALID_ARGUMENT),
])
def test_ssd_rejects_bad_shapes(kw, status):
    assert _ssd(_ssd_shape(**kw)) == status


def test_ssd_rejects_bad_arguments():
    assert A.load().axon_ssd_scan(None, ctypes.byref(_ssd_params()), P, P, P, P, None, P, P, P,
                                  1 << 30, None) == A.AXON_ERR_INVALID_ARGUMENT
    assert A.load().axon_ssd_scan(ctypes.byref(_ssd_shape()), None, P, P, P, P, None, P, P, P,
                                  1 << 30, None) == A.AXON_ERR_INVALID_ARGUMENT
    bad = A.make_ssd_shape(1, 64, 2, False)
    bad.act_dtype = 7
    assert _ssd(bad) == A.AXON_ERR_UNSUPPORTED
    for name in ("x", "dt", "B", "C", "y", "sout"):
        assert _ssd(**{name: 0}) == A.AXON_ERR_INVALID_ARGUMENT, name
        assert _ssd(**{name: _buffers()[name] + 4}) == A.AXON_ERR_INVALID_ARGUMENT, name
    assert _ssd(sin=_buffers()["sin"] + 8) == A.AXON_ERR_INVALID_ARGUMENT
    assert _ssd(params=_ssd_params(dt_min=-1.0)) == A.AXON_ERR_INVALID_ARGUMENT
    assert _ssd(params=_ssd_params(dt_min=2.0, dt_max=1.0)) == A.AXON_ERR_INVALID_ARGUMENT
    assert _ssd(params=_ssd_params(dt_max=float("inf"))) == A.AXON_ERR_INVALID_ARGUMENT
    need = A.ssd_workspace_bytes(_ssd_shape())
    assert _ssd(ws_bytes=need - 1) == A.AXON_ERR_WORKSPACE_TOO_SMALL
    assert _ssd(ws=0, ws_bytes=need) == A.AXON_ERR_INVALID_ARGUMENT
    b = _buffers()
    assert _ssd(y=b["x"] + 256) == A.AXON_ERR_INVALID_ARGUMENT       # y overlaps x
    assert _ssd(ws=b["B"]) == A.AXON_ERR_INVALID_ARGUMENT             # workspace overlaps B
    assert _ssd(sout=b["sin"] + 1024) == A.AXON_ERR_INVALID_ARGUMENT  # partial state overlap
    assert _ssd(sout=b["y"]) == A.AXON_ERR_INVALID_ARGUMENT          # state out overlaps y


# ---- the allocation-free prefill: every check happens before any device call ----------------
def _noalloc(shape=None, params=None, **over):
    b = _buffers()
    b.update(over)
    return A.raw_prefill_noalloc(shape or _shape(), params or _params(), b["x"], b["z"], b["dt"],
                                 b["B"], b["C"], b["cin"], b["sin"], b["y"], b["cout"], b["sout"],
                                 None)


def test_prefill_noalloc_rejects_bad_arguments():
    assert _noalloc(shape=_shape(d_state=8)) == A.AXON_ERR_UNSUPPORTED
    assert _noalloc(shape=_shape(batch=0)) == A.AXON_ERR_INVALID_ARGUMENT
    assert _noalloc(params=_params(dt_min=2.0, dt_max=1.0)) == A.AXON_ERR_INVALID_ARGUMENT
    for name in ["x", "z", "dt", "B", "C", "y", "cout", "sout"]:
        assert _noalloc(**{name: None}) == A.AXON_ERR_INVALID_ARGUMENT, name
        assert _noalloc(**{name: _buffers()[name] + 4}) == A.AXON_ERR_INVALID_ARGUMENT, name
    b = _buffers()
    assert _noalloc(y=b["x"]) == A.AXON_ERR_INVALID_ARGUMENT
    assert _noalloc(cout=b["cin"] + 16) == A.AXON_ERR_INVALID_ARGUMENT
    assert _noalloc(sout=b["cout"]) == A.AXON_ERR_INVALID_ARGUMENT
