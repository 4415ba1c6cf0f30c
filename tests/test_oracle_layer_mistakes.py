"""Planted mistakes in the oracle's layer composition: each variant of ``oracle.layer_forward``
below carries one plausible error (f_proj reading the projection instead of the convolution
output, swapped branches, the output projection before the gate, a dropped SiLU, the cache
taken from u instead of the raw inputs) and must fail at least one layer pin."""
import inspect
import textwrap

import numpy as np
import pytest

import oracle
import oracle_pins

SOURCE = textwrap.dedent(inspect.getsource(oracle.layer_forward))

MISTAKES = {
    "f_proj_reads_projection": ("U = u.astype(np.float64)", "U = xb.astype(np.float64)"),
    "branches_swapped": ("xb = store_as(X @ Win[:E].T, act)\n    z = store_as(X @ Win[E:].T, act)",
                         "xb = store_as(X @ Win[E:].T, act)\n    z = store_as(X @ Win[:E].T, act)"),
    "silu_dropped": ("v = v / (1.0 + np.exp(-v))", "v = v"),
    "cache_from_u": ('return {"out": out, "conv_cache": full[:, -(K - 1):, :].copy(),',
                     'return {"out": out, "conv_cache": np.concatenate([cache, U], axis=1)'
                     '[:, -(K - 1):, :].copy(),'),
    "dt_rows_from_B_rows": ("dtr = store_as(U @ Wf[2 * N:].T, act)",
                            "dtr = store_as(U @ np.roll(Wf, N, axis=0)[2 * N:].T, act)"),
}
LAYER_PINS = [oracle_pins.pin_layer_reduces_to_path, oracle_pins.pin_layer_projections,
              oracle_pins.pin_layer_step_equals_prefill]


def _variant(old, new):
    assert SOURCE.count(old) == 1, "the planted pattern must occur exactly once"
    ns = dict(vars(oracle))
    exec(compile(SOURCE.replace(old, new), "<layer variant>", "exec"), ns)  # noqa: S102
    return ns["layer_forward"]


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_layer_mistake_is_caught(name):
    layer = _variant(*MISTAKES[name])
    caught = []
    for pin in LAYER_PINS:
        try:
            pin(layer=layer)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no layer pin caught {name}"


def test_unmodified_layer_passes_the_same_harness():
    layer = _variant("U = u.astype(np.float64)", "U = u.astype(np.float64)")
    for pin in LAYER_PINS:
        pin(layer=layer)
    assert np.isfinite(0.0)
