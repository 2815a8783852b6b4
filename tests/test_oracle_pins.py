"""CPU tests: the fp64 oracle against its pins, and the pins against planted
mistakes (each mutant is a copy of oracle.c with one plausible error; the
pins must reject every one of them)."""
import os
import subprocess
import sys

import pytest

import oracle
from tests import oracle_pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.default())


# (name, text in oracle.c, replacement, which occurrence (0-based))
MUTANTS = [
    ("pad_sign", "t * stride + j * dilation - pad_left", "t * stride + j * dilation + pad_left", 0),
    ("kernel_flip", "acc += wrow[j] * xrow[u]", "acc += wrow[K - 1 - j] * xrow[u]", 0),
    ("stride_ignored", "int64_t u = t * stride", "int64_t u = t", 0),
    ("dilation_ignored", "j * dilation - pad_left;", "j - pad_left;", 0),
    ("bias_dropped", "double acc = bias ? bias[c] : 0.0;", "double acc = 0.0;", 0),
    ("weight_transposed", "w + (c * C_in + ci) * K", "w + ((c % C_in) * C_out + (ci % C_out)) * K", 0),
    ("input_off_by_one", "if (u >= 0 && u < T)", "if (u >= 0 && u <= T - 2)", 0),
    ("out_len_floor", "return span / stride + 1;", "return (span + stride - 1) / stride + 1;", 0),
    ("gn_unbiased_var", "double var = ss / cnt;", "double var = ss / (cnt - 1.0);", 0),
    ("gn_eps_outside", "double rstd = 1.0 / sqrt(var + eps);", "double rstd = 1.0 / (sqrt(var) + eps);", 0),
    ("gn_group_base", "y + (n * C + g * cpg) * L", "y + (n * C + g) * L", 0),
    ("gn_affine_swapped", "* rstd * ga + be;", "* rstd * be + ga;", 0),
    ("gn_mean_not_subtracted", "zr[l] = (yr[l] - mean) * rstd", "zr[l] = yr[l] * rstd", 0),
    ("ln_wrong_count", "double mean = s / (double)C;", "double mean = s / (double)(C + 1);", 0),
    ("ln_eps_dropped", "1.0 / sqrt(ss / (double)C + eps)", "1.0 / sqrt(ss / (double)C)", 0),
    ("ln_affine_swapped", "* rstd * ga + be;", "* rstd * be + ga;", 1),
    ("rowmin_is_max", "if (v < m || v != v) m = v;", "if (v > m || v != v) m = v;", 0),
    ("rowmin_drops_nan", "if (v < m || v != v) m = v;", "if (v < m) m = v;", 0),
    ("rowmin_bias_index", "out[(n * C + c) * L + l] = m + bias2[c];",
     "out[(n * C + c) * L + l] = m + bias2[0];", 0),
]


def _mutate(src, old, new, occ):
    pos = -1
    for _ in range(occ + 1):
        pos = src.index(old, pos + 1)
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, name, old, new, occ):
    src = open(oracle.SOURCE).read()
    assert old in src, "mutation site vanished: " + name
    mutated = _mutate(src, old, new, occ)
    assert mutated != src
    csrc = tmp_path / ("mut_%s.c" % name)
    csrc.write_text(mutated)
    lib = oracle.compile_source(str(csrc), str(tmp_path / ("libmut_%s.so" % name)))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                       capture_output=True, text=True, timeout=300, env=env)
    # a planted mistake must make at least one pin fail (a crash also counts)
    assert r.returncode != 0, "mutant %s passed every pin: %s" % (name, r.stdout[-500:])
