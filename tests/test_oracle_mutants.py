"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/gdn_oracle.c with one plausible slip (a step
out of order, a wrong sign, a wrong index, a wrong head map, a mask ignored,
an off-by-one).  It is compiled on the CPU into a temporary library and the pin
suite (tests/test_oracle_pins.py) is run against it in a child process; the
suite must fail for every mutant.  The real oracle is never modified.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTANTS = {
    "decay_after_readout": (
        "for (uint32_t i = 0; i < Dk; ++i) S[i] = gt * S[i];\n"
        "                    /* (2) what the decayed row predicts for this key */\n"
        "                    double kv = oracle_dot(S, kt, Dk);",
        "double kv = oracle_dot(S, kt, Dk);\n"
        "                    for (uint32_t i = 0; i < Dk; ++i) S[i] = gt * S[i];"),
    "innovation_sign": ("bet * (v[vo] - kv)", "bet * (kv - v[vo])"),
    "beta_on_value_only": ("bet * (v[vo] - kv)", "(bet * v[vo] - kv)"),
    "query_readout_before_write": (
        "for (uint32_t i = 0; i < Dk; ++i) S[i] = S[i] + delta * kt[i];\n"
        "                    /* (6) output: the corrected row read against the query */\n"
        "                    y[vo] = oracle_dot(S, qt, Dk);",
        "y[vo] = oracle_dot(S, qt, Dk);\n"
        "                    for (uint32_t i = 0; i < Dk; ++i) S[i] = S[i] + delta * kt[i];"),
    "readout_with_key": ("y[vo] = oracle_dot(S, qt, Dk);", "y[vo] = oracle_dot(S, kt, Dk);"),
    "no_decay_in_record": ("S[i] = gt * S[i];", "S[i] = S[i];"),
    "rank_one_along_query": ("S[i] = S[i] + delta * kt[i];", "S[i] = S[i] + delta * qt[i];"),
    "block_map_as_tiled": ("return hv / group;", "return hv % Hk;"),
    "tiled_map_as_block": ("    return hv % Hk;\n}", "    return hv / (Hv / Hk);\n}"),
    "mask_ignored": ("return mask[(size_t)b * T + t] > 0u;", "return 1;"),
    "mask_ignores_batch": ("return mask[(size_t)b * T + t] > 0u;", "return mask[t] > 0u;"),
    "gate_indexed_by_key_head": ("double gt = g[bt * Hv + hv];", "double gt = g[bt * Hv + hk];"),
    "key_from_first_step": ("const double* kt = k + (bt * Hk + hk) * Dk;",
                            "const double* kt = k + (((size_t)b * T) * Hk + hk) * Dk;"),
    "tape_not_written": ("if (delta_log != NULL) delta_log[vo] = delta;", "(void)0;"),
    "replay_no_decay": ("S[i] = S[i] * gt + kt[i] * d;", "S[i] = S[i] + kt[i] * d;"),
    "replay_accepted_off_by_one": ("int take = (t < accepted)", "int take = (t <= accepted)"),
    "replay_ignores_mask": ("int take = (t < accepted) && oracle_step_active(mask, T_log, b, t);",
                            "int take = (t < accepted);"),
    "replay_delta_row_dropped": ("double d = delta_log[(bt * Hv + hv) * Dv + dv];",
                                 "double d = delta_log[(bt * Hv + hv) * Dv];"),
    "replay_gate_from_next_step": ("double gt = g_log[bt * Hv + hv];",
                                   "double gt = g_log[(t + 1 < T_log ? bt + 1 : bt) * Hv + hv];"),
    "rms_sum_not_mean": ("double r = 1.0 / sqrt(ss / (double)dim + eps);",
                         "double r = 1.0 / sqrt(ss + eps);"),
    "rms_eps_outside_sqrt": ("double r = 1.0 / sqrt(ss / (double)dim + eps);",
                             "double r = 1.0 / (sqrt(ss / (double)dim) + eps);"),
    "rms_no_sqrt": ("double r = 1.0 / sqrt(ss / (double)dim + eps);",
                    "double r = 1.0 / (ss / (double)dim + eps);"),
    "rms_weight_reversed": ("uint32_t bits = (uint32_t)w[i] << 16;",
                            "uint32_t bits = (uint32_t)w[dim - 1 - i] << 16;"),
    "rms_abs_not_square": ("ss = ss + (double)xt[i] * (double)xt[i];", "ss = ss + fabs((double)xt[i]);"),
    "expand_source_head_zero": ("size_t so = (((size_t)t * hg + from) * k + e) * elem_bytes;",
                                "size_t so = (((size_t)t * hg) * k + e) * elem_bytes;"),
}


def _run_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, name + ": pattern not found in the oracle source"
    mutated = src.replace(old, new, 1)
    csrc = os.path.join(tmp_path, name + ".c")
    lib = os.path.join(tmp_path, name + ".so")
    with open(csrc, "w") as f:
        f.write(mutated)
    subprocess.run(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
                    "-o", lib, csrc, "-lm"], check=True)
    env = dict(os.environ, GDN_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    names = sorted(MUTANTS)
    with ThreadPoolExecutor(max_workers=4) as ex:
        codes = dict(zip(names, ex.map(lambda n: _run_mutant(n, str(tmp_path)), names)))
    survivors = [n for n, c in codes.items() if c == 0]
    assert not survivors, "mutants not caught by the oracle pins: %s" % survivors
    # a collection error (code 2+) would also be non-zero; require genuine test failures
    assert all(c == 1 for c in codes.values()), codes
