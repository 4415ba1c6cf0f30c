"""Planted mistakes: each variant of the oracle below carries one plausible error (a dropped
term, a wrong sign, a transposed operand, a wrong index). Every variant is compiled on the CPU
and must fail at least one pin, which shows the pins can see that kind of mistake."""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "axon_oracle.c")

MUTATIONS = {
    "drop_D_skip": ("acc += D * u;", "acc += 0.0 * D * u;"),
    "positive_A": ("A[n] = -exp((double)A_log[n]);", "A[n] = exp((double)A_log[n]);"),
    "A_without_exp": ("A[n] = -exp((double)A_log[n]);", "A[n] = -(double)A_log[n];"),
    "bbar_without_dt": (": dt * (double)Bm[t * bc_stride + n];",
                        ": (double)Bm[t * bc_stride + n];"),
    "B_C_swapped": (": dt * (double)Bm[t * bc_stride + n];",
                    ": dt * (double)Cm[t * bc_stride + n];"),
    "zoh_exp_not_expm1": ("? expm1(dt * A[n]) / A[n]", "? exp(dt * A[n]) / A[n]"),
    "zoh_without_divide": ("? expm1(dt * A[n]) / A[n]", "? expm1(dt * A[n])"),
    "zoh_is_first_order": ("? expm1(dt * A[n]) / A[n] * (double)Bm[t * bc_stride + n]",
                           "? dt * (double)Bm[t * bc_stride + n]"),
    "conv_silu_dropped": ("if (conv_act == ORACLE_CONV_SILU) u = silu(u);",
                          "if (conv_act == ORACLE_CONV_SILU) u = u;"),
    "conv_silu_on_current_input_only": ("if (conv_act == ORACLE_CONV_SILU) u = silu(u);",
                                        "if (conv_act == ORACLE_CONV_SILU) u = u - xt + silu(xt);"),
    "readout_before_update": (
        "h[n] = abar * h[n] + bbar * u;\n      acc += (double)Cm[t * bc_stride + n] * h[n];",
        "acc += (double)Cm[t * bc_stride + n] * h[n];\n      h[n] = abar * h[n] + bbar * u;"),
    "decay_on_input": ("h[n] = abar * h[n] + bbar * u;", "h[n] = h[n] + abar * bbar * u;"),
    "conv_taps_reversed": ("u += (double)conv_w[k] * win[k];",
                           "u += (double)conv_w[K - 2 - k] * win[k];"),
    "conv_bias_dropped": ("double u = conv_b;", "double u = 0.0 * conv_b;"),
    "cache_newest_first": ("if (K > 1) win[K - 2] = xt;", "if (K > 1) win[0] = xt;"),
    "softplus_no_linear_part": ("double pos = v > 0.0 ? v : 0.0;", "double pos = 0.0;"),
    "softplus_sign": ("return pos + log1p(exp(-fabs(v)));", "return pos + log1p(exp(fabs(v)));"),
    "dt_bias_subtracted": ("softplus((double)dt_raw[t * act_stride] + dt_bias)",
                           "softplus((double)dt_raw[t * act_stride] - dt_bias)"),
    "no_upper_clip": ("if (dt > dt_max) dt = dt_max;", ""),
    "no_lower_clip": ("if (dt < dt_min) dt = dt_min;", ""),
    "gate_sigmoid_not_silu": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "D_times_x_not_u": ("acc += D * u;", "acc += D * xt;"),
    "ssd_readout_before_update": (
        "          h[p * N + n] = a * h[p * N + n] + dt * (double)xt[p] * (double)Bt[n];\n"
        "          acc += (double)Ct[n] * h[p * N + n];",
        "          acc += (double)Ct[n] * h[p * N + n];\n"
        "          h[p * N + n] = a * h[p * N + n] + dt * (double)xt[p] * (double)Bt[n];"),
    "ssd_B_C_swapped": ("dt * (double)xt[p] * (double)Bt[n];", "dt * (double)xt[p] * (double)Ct[n];"),
    "ssd_D_dropped": ("yt[p] = acc + (double)j->D[hd] * (double)xt[p];", "yt[p] = acc;"),
    "ssd_A_of_head0": ("const double A = -exp((double)j->A_log[hd]);",
                       "const double A = -exp((double)j->A_log[0]);"),
    "ssd_dt_of_head0": ("softplus((double)j->dt_raw[(b * L + t) * H + hd]",
                        "softplus((double)j->dt_raw[(b * L + t) * H]"),
    "ssd_state_transposed": ("h[p * N + n] = a * h[p * N + n]", "h[p * N + n] = a * h[n * P + p]"),
    "ssd_decay_without_dt": ("const double a = exp(dt * A);", "const double a = exp(A);"),
    "ssd_state_in_ignored": ("h[i] = j->state_in ? j->state_in[bh * P * N + i] : 0.0;",
                             "h[i] = 0.0;"),
    "state_in_ignored": ("h[n] = h_in ? h_in[n] : 0.0;", "h[n] = 0.0;"),
    "mag_signed_sum": ("mag += fabs((double)Cm[t * bc_stride + n] * h[n]);",
                       "mag += (double)Cm[t * bc_stride + n] * h[n];"),
    "mag_drops_skip": ("mag += fabs(D * u);", ""),
    "mag_without_gate": ("mag_out[t * y_stride] = mag * fabs(gate);",
                         "mag_out[t * y_stride] = mag;"),
    "mag_before_update": (
        "      acc += (double)Cm[t * bc_stride + n] * h[n];\n"
        "      mag += fabs((double)Cm[t * bc_stride + n] * h[n]);",
        "      acc += (double)Cm[t * bc_stride + n] * h[n];\n"
        "      mag += fabs((double)Cm[t * bc_stride + n] * (h[n] - bbar * u));"),
    "ssd_mag_signed_sum": ("size += fabs((double)Ct[n] * h[p * N + n]);",
                           "size += (double)Ct[n] * h[p * N + n];"),
    "ssd_mag_drops_skip": ("if (mt) mt[p] = size + fabs((double)j->D[hd] * (double)xt[p]);",
                           "if (mt) mt[p] = size;"),
}


def _build_variant(name, old, new, tmpdir):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name}: pattern must occur exactly once"
    path_c = os.path.join(tmpdir, f"{name}.c")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    path_so = os.path.join(tmpdir, f"lib{name}.so")
    inc = os.path.dirname(SRC)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-I", inc,
                    "-o", path_so, path_c, "-lm", "-lpthread"], check=True)
    return oracle.load_library(path_so)


# Planted mistakes in the bfloat16 rounding of ``oracle.store_as`` (Python): truncation, ties away
# from zero, and rounding to 7 instead of 8 significant bits.
def _bf16_truncate(a, act):
    a32 = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32))
    return (a32.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32) if act == "bf16" else a32


def _bf16_ties_away(a, act):
    a32 = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32))
    u = (a32.view(np.uint32) + np.uint32(0x8000)) & np.uint32(0xFFFF0000)
    return u.view(np.float32) if act == "bf16" else a32


def _bf16_short_mantissa(a, act):
    a32 = np.ascontiguousarray(np.asarray(a, np.float64).astype(np.float32))
    u = a32.view(np.uint32)
    u = (u + np.uint32(0xFFFF) + ((u >> np.uint32(17)) & np.uint32(1))) & np.uint32(0xFFFE0000)
    return u.view(np.float32) if act == "bf16" else a32


@pytest.mark.parametrize("store", [_bf16_truncate, _bf16_ties_away, _bf16_short_mantissa],
                         ids=lambda f: f.__name__)
def test_planted_bf16_rounding_mistake_is_caught(store):
    with pytest.raises(AssertionError):
        oracle_pins.pin_store_as_bf16(store=store)


def test_store_as_pin_passes():
    oracle_pins.pin_store_as_bf16()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    with tempfile.TemporaryDirectory() as tmpdir:
        lib = _build_variant(name, old, new, tmpdir)
        caught = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(lib=lib)
            except (AssertionError, ValueError, FloatingPointError) as exc:  # noqa: PERF203
                caught.append(pin.__name__)
                del exc
        assert caught, f"no pin caught the planted mistake {name}"
