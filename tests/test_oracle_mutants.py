"""Every planted mistake in the oracle must make at least one pin fail.

Each mutant is a copy of oracle/kda_oracle.c with one expression replaced (a
dropped term, a wrong sign, a wrong index, a transposed operand), compiled with
gcc into a temporary library on the CPU.  The real oracle is never modified.
"""
import os
import shutil
import tempfile

import pytest

from oracle.kda_oracle import SOURCE, build_oracle
from tests.oracle_pins import ALL_CHECKS

# (name, original text, replacement) -- each original must occur exactly once.
MUTANTS = [
    ("decay dropped", "S[(size_t)d * V + j] *= alpha;", "S[(size_t)d * V + j] *= 1.0;"),
    ("delta sign", "c * (vt[j] - u[j])", "c * (vt[j] + u[j])"),
    ("delta without correction", "c * (vt[j] - u[j])", "c * (vt[j])"),
    ("output before update",
     "double *ot = J->o + ((size_t)t * HV + hv) * V;\n        for (int j = 0; j < V; ++j) ot[j] = 0.0;\n        for (int d = 0; d < K; ++d)\n            for (int j = 0; j < V; ++j) ot[j] += S[(size_t)d * V + j] * qv[d];",
     "double *ot = J->o + ((size_t)t * HV + hv) * V;\n        for (int j = 0; j < V; ++j) ot[j] = u[j] * 0.0;"),
    ("decay after the read", "u[j] += S[(size_t)d * V + j] * kv[d];", "u[j] += S[(size_t)d * V + j] * kv[d] / exp(gate_activate(J->gate_mode, gt[d], J->A_log, J->dt_bias, hv, K, d, J->lower_bound));"),
    ("gva index", "const int h = hv / (HV / H);", "const int h = hv % H;"),
    ("state transposed read", "u[j] += S[(size_t)d * V + j] * kv[d];", "u[j] += S[(size_t)(d % V) * V + (j % K)] * kv[d];"),
    ("softplus sign", "return -exp(A_log[hv]) * softplus(x);", "return exp(A_log[hv]) * softplus(x);"),
    ("softplus without exp(A_log)", "return -exp(A_log[hv]) * softplus(x);", "return -A_log[hv] * softplus(x);"),
    ("bias dropped", "double x = graw + (dt_bias ? dt_bias[(size_t)hv * K + d] : 0.0);", "double x = graw;"),
    ("bias index", "dt_bias[(size_t)hv * K + d]", "dt_bias[(size_t)d * (K > 0 ? 1 : 0) + hv]"),
    ("bounded gate ignores A_log", "double a = A_log ? exp(A_log[hv]) : 1.0;", "double a = 1.0;"),
    ("bounded gate A_log not exponentiated", "double a = A_log ? exp(A_log[hv]) : 1.0;", "double a = A_log ? A_log[hv] : 1.0;"),
    ("negative-eigenvalue beta not doubled", "return 2.0 * sigmoid(b);", "return sigmoid(b);"),
    ("sigmoid beta ignored", "if (mode == BETA_SIGMOID) return sigmoid(b);", "if (mode == BETA_SIGMOID) return b;"),
    ("no l2 normalisation", "inv = 1.0 / sqrt(ss + 1e-6);", "inv = 1.0;"),
    ("scale dropped", "load_qk(J->q + ((size_t)t * H + h) * K, K, J->qk_l2norm, J->scale, qv);", "load_qk(J->q + ((size_t)t * H + h) * K, K, J->qk_l2norm, 1.0, qv);"),
    ("chunk state one token late", "if (J->states && r % J->chunk == 0)", "if (J->states && r % J->chunk == 1 % J->chunk)"),
    ("chunk state index ignores earlier sequences", "J->chunk_first[n] + r / J->chunk", "r / J->chunk"),
    ("initial state ignored", "if (J->h0) memcpy(S, J->h0", "if (0) memcpy(S, J->h0"),
    ("cumsum not reset", "if ((t - seq_starts[n]) % chunk == 0) run = 0.0;", "if (t == seq_starts[n]) run = 0.0;"),
    ("cumsum exclusive", "run += a;\n                    if (g_act) g_act[idx] = a;\n                    g_cum[idx] = run;",
     "if (g_act) g_act[idx] = a;\n                    g_cum[idx] = run;\n                    run += a;"),
]


@pytest.fixture(scope="module")
def source():
    with open(SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,orig,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, orig, repl):
    assert source.count(orig) == 1, f"mutation anchor for '{name}' not unique in the oracle"
    tmp = tempfile.mkdtemp(prefix="kda_mutant_")
    try:
        src = os.path.join(tmp, "mutant.c")
        with open(src, "w") as f:
            f.write(source.replace(orig, repl))
        lib = build_oracle(src, os.path.join(tmp, "libmutant.so"))
        failed = []
        for check in ALL_CHECKS:
            try:
                check(lib)
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(check.__name__)
        assert failed, f"planted mistake '{name}' passed every pin"
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
