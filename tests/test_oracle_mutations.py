"""Plant plausible mistakes in a copy of the oracle and check the pins catch them.

Each mutation edits the C source text in a temporary directory, builds a
separate library, points the oracle wrapper at it, and runs the pin checks of
tests/test_oracle_pins.py.  At least one check must fail for every mutation.
The committed oracle is never modified.
"""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import oracle
from tests import test_oracle_backward as bwd
from tests import test_oracle_pins as pins

MUTATIONS = {
    "ties_to_higher_index": ("    return a > b;\n}", "    return a >= b;\n}"),
    "nan_ranked_by_position": ("        return !isnan(a);", "        return 0;"),
    "penalty_two_roundings": ("fmaf(-lambda, load[e], raw[i])", "raw[i] - lambda * load[e]"),
    "capacity_floor": ("ceil((double)T", "floor((double)T"),
    "queue_limit_off_by_one": ("if (fill[e] < C) {", "if (fill[e] <= C) {"),
    "token_major_order": ("    for (int r = 0; r < k; r++)\n        for (int t = 0; t < T; t++) {\n            size_t j",
                          "    for (int t = 0; t < T; t++)\n        for (int r = 0; r < k; r++) {\n            size_t j"),
    "fallback_wrong_rank": ("int f = cand[(size_t)t * K + k];", "int f = cand[(size_t)t * K + k - 1];"),
    "silu_on_w3": ("h[j] = a / (1.0 + exp(-a)) * b;", "h[j] = b / (1.0 + exp(-b)) * a;"),
    "w2_transposed": ("acc += h[j] * elem(w2, ro + j, dt);", "acc += h[j] * elem(w2, w2o + (size_t)j * d + q, dt);"),
    "gate_not_renormalised": ("            if (flag[j] != 2)\n                z += exp(", "            if (1)\n                z += exp("),
    "aux_loss_over_Tk": ("(double)demand[e] / (double)T :", "(double)demand[e] / ((double)T * k) :"),
    "bias_dropped": ("r = r + bias[e];", "r = r;"),
    "gate_uses_primary_score": ("                src_rank[j] = k;\n", ""),
    "temperature_left_out_of_numerator": ("- m) / tau) / z;", "- m)) / z;"),
    "gap_taken_below_second": ("const float gap = cs[0] - cs[1];", "const float gap = cs[1] - cs[2];"),
    "gap_swap_drops_displaced": ("            c[2] = ce;\n", ""),
    "glu_w2_transposed": ("acc += a[j] * elem(w2, (size_t)e * H + j, dt);", "acc += a[j] * elem(w2, (size_t)j * E + e, dt);"),
    "glu_silu_missing": ("a[j] = acc / (1.0 + exp(-acc));", "a[j] = acc;"),
    "router_weight_transposed": ("elem(wr, (size_t)e * d + i, dt)", "elem(wr, (size_t)i * E + e, dt)"),
    "dynamic_cf_natural_log": ("return 1.0 + 0.01 * log2((double)T);", "return 1.0 + 0.01 * log((double)T);"),
    "dynamic_cf_slope": ("return 1.0 + 0.01 * log2((double)T);", "return 1.0 + 0.1 * log2((double)T);"),
    "e4m3_bias_8": ("e - 7);", "e - 8);"),
    "e4m3_subnormal_scale": ("(double)f / 8.0, -6);", "(double)f / 8.0, -7);"),
    "e4m3_no_nan": ("if (e == 15 && f == 7)\n        return NAN;", "if (0)\n        return NAN;"),
    "dequant_scale_by_column": ("(double)scale[r] * oracle_fp8", "(double)scale[c % rows] * oracle_fp8"),
    "double_elements_as_float": ("        return ((const double *)p)[i];", "        return (double)((const float *)p)[i];"),
    "glu_bias1_after_silu": ("            if (bias1)\n                acc += bias1[j];\n            a[j] = acc / (1.0 + exp(-acc));",
                             "            a[j] = acc / (1.0 + exp(-acc));\n            if (bias1)\n                a[j] += bias1[j];"),
    "glu_bias1_dropped": ("                acc += bias1[j];", "                acc += 0.0;"),
    "load_window_decay_swapped": ("l[e] = alpha * l[e] + (1.0 - alpha) *", "l[e] = (1.0 - alpha) * l[e] + alpha *"),
    "load_window_counts_fallback": ("            for (int r = 0; r < k; r++) {\n                const int c = cand[(size_t)t * K1 + r];",
                                    "            for (int r = 0; r < K1; r++) {\n                const int c = cand[(size_t)t * K1 + r];"),
    "load_window_over_batch": ("((double)cnt[e] / ((double)k * n));", "((double)cnt[e] / ((double)k * T));"),
    "load_window_full_last": ("const int n = T - t0 < window ? T - t0 : window;", "const int n = window;"),
    "i8_codes_read_unsigned": ("(double)scale[r] * (double)q[r * cols + c];", "(double)scale[r] * (double)(uint8_t)q[r * cols + c];"),
    "i4_nibbles_swapped": ("nibble_value(q[r * (cols / 2) + c / 2], (int)(c & 1))", "nibble_value(q[r * (cols / 2) + c / 2], (int)!(c & 1))"),
    "i4_codes_read_unsigned": ("    return v >= 8 ? v - 16 : v;", "    return v;"),
    "i4_offset_binary": ("    return v >= 8 ? v - 16 : v;", "    return v - 8;"),
    # backward pass
    "bwd_silu_derivative_first_term_only": ("const double da = dh * b[j] * sg * (1.0 + a[j] * (1.0 - sg));",
                                            "const double da = dh * b[j] * sg;"),
    "bwd_units_silu_derivative_first_term_only": ("const double da = dh * b * sg * (1.0 + a * (1.0 - sg)), db",
                                                  "const double da = dh * b * sg, db"),
    "bwd_softmax_mean_left_out": ("(dg[r] - mean) / tau;", "dg[r] / tau;"),
    "bwd_temperature_left_out": ("(dg[r] - mean) / tau;", "(dg[r] - mean);"),
    "bwd_expert_grad_ungated": ("const double dh = g * u[j];", "const double dh = u[j];"),
    "bwd_db_times_b": ("const double db = dh * silu;", "const double db = dh * silu * b[j];"),
    "bwd_w2_grad_ungated": ("dw2[(size_t)q * nf + i] += g[rr] * dyt[q] * h;", "dw2[(size_t)q * nf + i] += dyt[q] * h;"),
    "bwd_router_input_term_left_out": ("dxt[q] += dlt[e] * elem(wr,", "dxt[q] += 0.0 * elem(wr,"),
    "bwd_w1_w3_swapped_in_dx": ("da * elem(w1, wo + (size_t)j * d + q, dt) + db * elem(w3, wo + (size_t)j * d + q, dt)",
                                "da * elem(w3, wo + (size_t)j * d + q, dt) + db * elem(w1, wo + (size_t)j * d + q, dt)"),
    "bwd_bias_grad_left_out": ("            sb += gl;\n", ""),
    "bwd_w2_transposed_in_u": ("su += dyt[q] * elem(w2, w2o + (size_t)q * d_ff + j, dt);",
                               "su += dyt[q] * elem(w2, w2o + (size_t)j * d + q, dt);"),
}

# (name, check) pairs, run in this order by the child process below
CHECKS = [
    ("capacity", pins.check_capacity), ("router_logits", pins.check_router_logits),
    ("scores", pins.check_scores), ("topk", pins.check_topk),
    ("dispatch_exhaustive", pins.check_dispatch_exhaustive),
    ("dispatch_invariants", pins.check_dispatch_invariants), ("aux_loss", pins.check_aux_loss),
    ("dense_equivalence", lambda o: pins.check_dense_equivalence(o, "f32")),
    ("identical_experts", pins.check_identical_experts), ("expert_relabel", pins.check_expert_relabel),
    ("gate_temperature", pins.check_gate_temperature), ("gap_swap", pins.check_gap_swap),
    ("router_glu", pins.check_router_glu), ("fp8_decode", pins.check_fp8_decode),
    ("dynamic_capacity", pins.check_dynamic_capacity),
    ("dequant_rows", pins.check_dequant_rows), ("ffn_double_elements", pins.check_ffn_double_elements),
    ("load_window", pins.check_load_window), ("dequant_rows_i8", pins.check_dequant_rows_i8),
    ("dequant_rows_i4", pins.check_dequant_rows_i4),
    ("backward_autograd", bwd.check_backward_autograd),
    ("backward_finite_differences", bwd.check_backward_finite_differences),
    ("backward_invariants", bwd.check_backward_invariants),
    ("backward_sampled_units", bwd.check_backward_sampled_units),
]


RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import test_oracle_mutations as m
oracle._LIB = {so!r}
oracle._lib = None
oracle.lib()
for name, chk in m.named_checks():
    try:
        chk(oracle)
        print("PASS", name, flush=True)
    except (AssertionError, IndexError, ValueError, RuntimeError) as exc:
        print("FAIL", name, flush=True)
"""


def named_checks():
    return list(CHECKS)


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, workdir):
    """The mutated library runs in a child process: a planted out-of-bounds
    write must not corrupt this test process."""
    old, new = MUTATIONS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "moe_oracle.c")).read()
    assert src.count(old) >= 1, f"mutation pattern not found: {name}"
    c = os.path.join(workdir, f"{name}.c")
    so = os.path.join(workdir, f"lib_{name}.so")
    open(c, "w").write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-shared",
                           "-fPIC", "-o", so, c, "-lm"])
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([sys.executable, "-c", RUNNER.format(root=root, so=so)],
                          capture_output=True, text=True, timeout=600)
    failed = [ln.split()[1] for ln in proc.stdout.splitlines() if ln.startswith("FAIL")]
    crashed = proc.returncode != 0
    assert failed or crashed, f"no pin catches mutation {name}: {proc.stdout}{proc.stderr}"
