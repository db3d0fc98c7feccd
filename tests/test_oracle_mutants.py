"""The oracle pins must catch plausible mistakes.

Each mutant is a copy of ``oracle/moe_oracle.c`` with one planted slip (on the
CPU, in a temporary directory); the pin suite is run against it in a fresh
process and must fail.  The unmodified source must pass.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

# (name, original text, planted slip)
MUTANTS = [
    ("router_transposed", "acc += wr[(size_t)e * H + h] * x[h];", "acc += wr[(size_t)h * E + e] * x[h];"),
    ("router_drops_first_term", "for (int h = 0; h < H; ++h)\n            acc += wr",
     "for (int h = 1; h < H; ++h)\n            acc += wr"),
    ("ascending_selection", "if (a->v > b->v) return -1;\n    if (a->v < b->v) return 1;",
     "if (a->v > b->v) return 1;\n    if (a->v < b->v) return -1;"),
    ("ties_to_higher_id", "return (a->id < b->id) ? -1 : (a->id > b->id) ? 1 : 0;",
     "return (a->id > b->id) ? -1 : (a->id < b->id) ? 1 : 0;"),
    ("softmax_sign", "weights[k] = exp(s[k].v - lmax) / z;", "weights[k] = exp(lmax - s[k].v) / z;"),
    ("no_renormalisation", "if (renormalize)\n", "if (0 && renormalize)\n"),
    ("denominator_skips_expert0", "for (int e = 0; e < E; ++e) z += exp", "for (int e = 1; e < E; ++e) z += exp"),
    ("margin_off_by_one", "int last = (K < E) ? K : E - 1;", "int last = (K < E) ? K - 1 : E - 1;"),
    ("silu_is_sigmoid", "return g / (1.0 + exp(-g));", "return 1.0 / (1.0 + exp(-g));"),
    ("gate_up_swapped", "activated[j] = silu(g) * u;", "activated[j] = silu(u) * g;"),
    ("w2_transposed", "const double *row = w2k[k] + (size_t)h * I;", "const double *row = w2k[k] + (size_t)h;"),
    ("w2_row_stride", "d += row[j] * a[j];", "d += row[j * H] * a[j];"),
    ("weight_index_fixed", "acc += weights[k] * d;", "acc += weights[0] * d;"),
    ("shared_not_added", "y[h] = y[h] + s[h];", "y[h] = y[h];"),
    ("all_experts_use_first_slice", "oracle_expert_activated(x, w13sel + (size_t)k * 2 * I * H,",
     "oracle_expert_activated(x, w13sel,"),
    ("up_half_offset_wrong", "const double *urow = w13e + (size_t)(I + j) * H;",
     "const double *urow = w13e + (size_t)(I + j - 1) * H;"),
    ("route_weights_ignore_ids", "weights[k] = exp(logits[ids[k]] - lmax) / z;",
     "weights[k] = exp(logits[k] - lmax) / z;"),
    ("route_weights_not_renormalised", "if (renormalize != 0)\n", "if (0)\n"),
]


def _build(src_text, out_dir, name):
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    open(c, "w").write(src_text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-std=c11", "-shared",
                           "-fPIC", c, "-o", so, "-lm"])
    return so


def _run_pins(so):
    env = dict(os.environ)
    env["MOE_ORACLE_LIB_OVERRIDE"] = so
    env["OMP_NUM_THREADS"] = "1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_planted_slip_is_caught():
    src = open(SRC).read()
    for name, old, new in MUTANTS:
        assert src.count(old) >= 1, "mutant %s no longer applies" % name
    with tempfile.TemporaryDirectory() as d:
        jobs = [("unmodified", src)] + [(n, src.replace(o, nw, 1)) for n, o, nw in MUTANTS]
        sos = [(n, _build(t, d, n)) for n, t in jobs]
        with ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda p: (p[0],) + _run_pins(p[1]), sos))
    base = results[0]
    assert base[1] == 0, "unmodified oracle fails its pins:\n" + base[2]
    survivors = [n for n, rc, _ in results[1:] if rc == 0]
    assert not survivors, "planted slips not caught by any pin: %s" % survivors
