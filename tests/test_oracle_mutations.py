"""The oracle's pins catch plausible mistakes in the oracle itself.

Each case plants one mistake in a copy of oracle/qmv_oracle.c (on the CPU),
builds it, and runs the pin suites (tests/test_oracle_pins.py and
tests/test_golden.py) against that build in a child process: at least one
pin must fail.  An unedited copy must pass the same run, so a failure is the
planted mistake's and not the harness's."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qmv_oracle.c")
PINS = ["tests/test_oracle_pins.py", "tests/test_golden.py"]

# (name, text in the oracle source, replacement): every edit keeps all
# memory accesses in bounds, so a mutant fails by its values alone
MUTATIONS = [
    ("round_half_even", "float r = roundf(diff / scale);", "float r = rintf(diff / scale);"),
    ("q0_half_even", "float q0 = roundf(edge / scale);", "float q0 = rintf(edge / scale);"),
    ("w_max_from_minus_inf", "float w_max = 0.0f;", "float w_max = -FLT_MAX;"),
    ("scale_sign_flipped", "if (!side) scale = -scale;", "if (side) scale = -scale;"),
    ("no_q0_rescale", "scale = edge / q0;", "scale = scale;"),
    ("eps_1e-6", "const float eps = 1e-7f;", "const float eps = 1e-6f;"),
    ("no_top_clamp", "if (r > n_bins) r = n_bins;", "(void)0;"),
    ("bf16_ties_away", "(rest == 0x8000u && (keep & 1u))", "(rest == 0x8000u)"),
    ("pack_msb_first", "row[bit / 32] |= 1u << (bit % 32);", "row[bit / 32] |= 1u << (31 - bit % 32);"),
    ("unpack_msb_first", "c |= ((row[bit / 32] >> (bit % 32)) & 1u) << j;",
     "c |= ((row[bit / 32] >> (31 - bit % 32)) & 1u) << j;"),
    ("dequant_drops_bias", "out[k] = s * (double)tmp_codes[k] + b;", "out[k] = s * (double)tmp_codes[k];"),
    ("dequant_first_group_bias", "double b = oracle_f64_from_bf16(brow[k / g]);",
     "double b = oracle_f64_from_bf16(brow[0]);"),
    ("qmv_x_row_0", "for (int64_t k = 0; k < K; k++) acc += row[k] * xd[m * K + k];",
     "for (int64_t k = 0; k < K; k++) acc += row[k] * xd[k];"),
    ("qvm_x_reversed", "double xv = oracle_f64_from_bf16(x[m * K + k]);",
     "double xv = oracle_f64_from_bf16(x[m * K + (K - 1 - k)]);"),
    ("silu_sign", "h[k] = gv / (1.0 + exp(-gv)) * uv;", "h[k] = gv / (1.0 + exp(gv)) * uv;"),
    ("resid_dropped", "y[n] = (x_resid ? oracle_f64_from_bf16(x_resid[n]) : 0.0) + acc;", "y[n] = acc;"),
    ("gather_x_stride_without_M", "oracle_qmv_f64(x + (int64_t)lhs[p] * M * K,", "oracle_qmv_f64(x + (int64_t)lhs[p] * K,"),
    ("gather_y_stride_without_M", "y + p * M * N);", "y + p * N);"),
    ("gather_expert_from_lhs", "w + (int64_t)rhs[p] * wsz,", "w + (int64_t)(lhs[p] % E) * wsz,"),
]


def run_pins(tmp_path, source_text, tag):
    src = tmp_path / f"{tag}.c"
    src.write_text(source_text)
    lib = str(tmp_path / f"lib{tag}.so")
    oracle.compile_source(str(src), lib)
    env = dict(os.environ, QMV_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", *PINS, "-q", "-x", "-m", "not gpu",
                           "-p", "no:cacheprovider"], cwd=ROOT, env=env,
                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)


def test_unedited_copy_passes(tmp_path):
    r = run_pins(tmp_path, open(SRC).read(), "unedited")
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutation(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"{name}: the edited text must occur exactly once"
    r = run_pins(tmp_path, text.replace(old, new), name)
    # 1 = tests ran and at least one failed (not a collection or usage error)
    assert r.returncode == 1, f"{name} was not caught (rc {r.returncode}):\n{r.stdout[-1500:]}"
