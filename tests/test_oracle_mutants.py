"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a temporary copy of the oracle
source (a wrong rounding mode, bias, maximum, sign, index, layout or head
mapping), builds it, and runs the pin suites against that build.  The pins
must fail for every mutant; a mutant they let through would be a hole in what
pins the oracle.  The committed oracle is never modified.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kvq_oracle.c")

# (name, original text, replacement); every original must occur in the source.
MUTANTS = [
    ("ties away from zero instead of to even",
     "return rint(a / quantum) * quantum;", "return round(a / quantum) * quantum;"),
    ("e4m3 exponent bias 8",
     "v = ldexp(1.0 + m / 8.0, e - 7);", "v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("e4m3 maximum 480", "#define KVO_E4M3_MAX 448.0f", "#define KVO_E4M3_MAX 480.0f"),
    ("q8_0 maximum 128", "#define KVO_Q8_MAX 127.0f", "#define KVO_Q8_MAX 128.0f"),
    ("scale by reciprocal", "float q = amax / M;", "float q = amax * (1.0f / M);"),
    ("element by reciprocal of the scale", "float v = xi / s;", "float v = xi * (1.0f / s);"),
    ("q8_0 ties to even", "double a = floor(fabs((double)v) + 0.5);",
     "double a = rint(fabs((double)v));"),
    ("e4m3 sign dropped", "uint8_t s = signbit(v) ? 0x80 : 0;", "uint8_t s = 0;"),
    ("pool rows transposed",
     "int64_t r = (page * c->n_heads + h) * c->page_size + off; /* row index */",
     "int64_t r = (page * c->page_size + off) * c->n_heads + h; /* row index */"),
    ("GQA head map interleaved", "int g = h / (c->n_q_heads / c->n_kv_heads);",
     "int g = h % c->n_kv_heads;"),
    ("page walk index", "t / c->page_size]", "t % c->page_size]"),
    ("softmax scale dropped", "z[t] = c->sm_scale * dot;", "z[t] = dot;"),
    ("MLA V row stride", "int v_row_dim = shared ? c->head_dim_qk : c->head_dim_v;",
     "int v_row_dim = c->head_dim_v;"),
    ("scale column index", "scales[row * nb + d / KVO_BLOCK]", "scales[row * nb + d % nb]"),
    ("fp16 subnormal step", "(uint16_t)(r * 16777216.0)", "(uint16_t)(r * 8388608.0)"),
    ("no subnormal floor", "if (e < emin) e = emin;", ";"),
    ("zero scale not special", "if (s == 0.0f) {", "if (0) {"),
    ("lse without log", "*lse_out = zmax + log(denom);", "*lse_out = zmax + denom;"),
    ("bf16 fraction bits", "double r = round_to_grid(fabs(x), 7, -126);",
     "double r = round_to_grid(fabs(x), 8, -126);"),
    ("e5m2 exponent bias 16", "v = ldexp(1.0 + m / 4.0, e - 15);", "v = ldexp(1.0 + m / 4.0, e - 16);"),
    ("e5m2 maximum 61440", "#define KVO_E5M2_MAX 57344.0f", "#define KVO_E5M2_MAX 61440.0f"),
    ("e5m2 three fraction bits", "double r = round_to_grid(fabs((double)v), 2, -14);",
     "double r = round_to_grid(fabs((double)v), 3, -14);"),
    ("cast without the clamp", "  if (x > M) x = M;\n  if (x < -M) x = -M;", ""),
    ("sparse length bound", "if (t < 0 || t >= L) continue;", "if (t < 0 || t > L) continue;"),
    ("sparse V row stride",
     "o[d] += w * kvo_pool_value(c->qtype, c->slab, c->scales, rows[j], c->head_dim_qk, d);",
     "o[d] += w * kvo_pool_value(c->qtype, c->slab, c->scales, rows[j], c->head_dim_v, d);"),
    ("sparse softmax scale dropped", "z[n] = c->sm_scale * dot;", "z[n] = dot;"),
    ("extend position off by one", "int64_t len = kvo_clamped_len(c, b) - E + i + 1;",
     "int64_t len = kvo_clamped_len(c, b) - E + i;"),
    ("extend without the causal limit", "int64_t len = kvo_clamped_len(c, b) - E + i + 1;",
     "int64_t len = kvo_clamped_len(c, b);"),
    ("656-byte row: tiles of 64", "#define KVO_DS_TILE 128", "#define KVO_DS_TILE 64"),
    ("656-byte row: scale by reciprocal", "float sc = amax / KVO_E4M3_MAX;",
     "float sc = amax * (1.0f / KVO_E4M3_MAX);"),
    ("extend token mapped to the next sequence",
     "while (b + 1 < c->batch && e->q_start[b + 1] <= j) ++b;",
     "while (b + 1 < c->batch && e->q_start[b + 1] < j) ++b;"),
    ("cast formats swapped",
     "return (qtype == KVO_FP8_E5M2_CAST) ? kvo_e5m2_encode(x) : kvo_e4m3_encode(x);",
     "return (qtype == KVO_FP8_E5M2_CAST) ? kvo_e4m3_encode(x) : kvo_e5m2_encode(x);"),
]


def _run_mutant(case):
    name, old, new = case
    src = open(SRC).read()
    assert old in src, "mutation target not found: %s" % name
    d = tempfile.mkdtemp(prefix="kvq_mutant_")
    c_path = os.path.join(d, "m.c")
    so = os.path.join(d, "m.so")
    with open(c_path, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
                    "-w", "-o", so, c_path, "-lm"], check=True)
    env = dict(os.environ, KVQ_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_attention_pins.py",
                        "tests/test_oracle_cast_pins.py", "tests/test_oracle_sparse_pins.py",
                        "tests/test_oracle_extend_pins.py", "tests/test_oracle_dsmla_pins.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin():
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(_run_mutant, MUTANTS))
    survived = [name for name, rc in results if rc == 0]
    assert not survived, "mutants not caught by any pin: %s" % survived
