"""Every plausible mistake planted in the oracle must trip at least one pin.

Each mutant is a copy of the oracle's C source with one textual change (a
dropped term, a flipped sign, a wrong index, a transposed or swapped operand,
a wrong tie rule or storage decode), compiled on the CPU and run through the
whole pin suite in a child process.  A mutant that passes every pin would mean
the pins cannot see that class of mistake.
"""
import json
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle.oracle import SOURCE, compile_library

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "silu_sign": ("z / (1.0 + exp(-z))", "z / (1.0 + exp(z))"),
    "sigmoid_sign": ("1.0 / (1.0 + exp(-z))", "1.0 / (1.0 + exp(z))"),
    "gate_up_swapped": ("a[i] = silu(g[i]) * u[i];", "a[i] = silu(u[i]) * g[i];"),
    "up_matrix_for_gate": ("matvec(G, g0, n_inter, x, g, nthreads)", "matvec(U, g0, n_inter, x, g, nthreads)"),
    "shared_term_dropped": ("const double joined = r[h] + s * S[h];", "const double joined = r[h];"),
    "shared_gate_dropped": ("const double joined = r[h] + s * S[h];", "const double joined = r[h] + S[h];"),
    "residual_of_normed_input": ("x0[h] + joined", "x[h] + joined"),
    "residual_ignored": ("L->residual ? x0[h] + joined : joined", "joined"),
    "norm_eps_outside_root": ("sqrt(ss / (double)H + L->norm_eps)", "sqrt(ss / (double)H) + L->norm_eps"),
    "norm_sum_not_mean": ("sqrt(ss / (double)H + L->norm_eps)", "sqrt(ss + L->norm_eps)"),
    "norm_not_inverted": ("double rho = 1.0 / sqrt(", "double rho = sqrt("),
    "norm_weight_dropped": ("(x0[h] * rho) * (double)L->norm_w[h]", "(x0[h] * rho)"),
    "norm_skipped": ("if (L->norm_w) {", "if (0) {"),
    "no_renormalisation": ("wsel[j] = p[sel[j]] / psum", "wsel[j] = p[sel[j]]"),
    "ties_to_higher_index": ("!taken[e] && (best < 0 || l[e] > l[best])", "!taken[e] && (best < 0 || l[e] >= l[best])"),
    "topk_smallest": ("!taken[e] && (best < 0 || l[e] > l[best])", "!taken[e] && (best < 0 || l[e] < l[best])"),
    # (a wrong softmax *denominator* is invisible: it cancels in the renormalisation)
    "softmax_numerator_inverted": ("p[e] = exp(l[e] - m) / z", "p[e] = exp(m - l[e]) / z"),
    "softmax_numerator_linear": ("p[e] = exp(l[e] - m) / z", "p[e] = (1.0 + l[e] - m) / z"),
    "router_transposed": ("acc += x[h] * (double)L->router[e * H + h]", "acc += x[h] * (double)L->router[h * E + e]"),
    "down_rows_of_wrong_expert": ("e * I, e * H, I, H, x, y, nthreads", "e * I, e * I, I, H, x, y, nthreads"),
    "routed_weight_index": ("r[h] += wsel[j] * y[h]", "r[h] += wsel[0] * y[h]"),
    "gate_vector_wrong_index": ("gl += (double)L->gate_vec[h] * x[h]", "gl += (double)L->gate_vec[h] * x[0]"),
    "matvec_drops_last_column": ("for (long c = 0; c < m->cols; ++c)\n            acc +=", "for (long c = 0; c < m->cols - 1; ++c)\n            acc +="),
    "q4_nibble_order": ("(col % 2 == 0) ? (byte & 0x0f) : (byte >> 4)", "(col % 2 == 0) ? (byte >> 4) : (byte & 0x0f)"),
    "q4_no_offset": ("scale * (double)(u - 8)", "scale * (double)u"),
    "q4_scale_of_first_block": ("m->scale[row * (m->cols / 32) + col / 32]", "m->scale[row * (m->cols / 32)]"),
    "bf16_shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "f16_exponent_bias": ("expo - 25", "expo - 24"),
    "f16_subnormal_scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "token_decode_transposed": ("[t * L->hidden + h]);\n}", "[h * 1 + t]);\n}"),
}


def _run(name, search, replace, tmp):
    src = open(SOURCE).read()
    assert src.count(search) == 1, f"{name}: mutation site must appear exactly once"
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(search, replace))
    lib = compile_library(path, os.path.join(tmp, f"lib_{name}.so"))
    proc = subprocess.run([sys.executable, "-m", "tests.oracle_pins", lib], cwd=ROOT,
                          capture_output=True, text=True, timeout=600)
    if proc.returncode != 0:
        return {"<process>": f"crashed rc={proc.returncode}"}
    return json.loads(proc.stdout.strip().splitlines()[-1])


@pytest.fixture(scope="module")
def verdicts():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(4) as ex:
            futs = {n: ex.submit(_run, n, s, r, tmp) for n, (s, r) in MUTANTS.items()}
            return {n: f.result() for n, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(verdicts, name):
    v = verdicts[name]
    caught = [p for p, r in v.items() if r != "pass"]
    assert caught, f"mutant {name} passed every pin"
