"""Planted mutations of the oracle: each must fail at least one pin.

Every entry below plants one plausible mistake in a copy of
oracle/rtopk_oracle.c (a dropped term, a flipped sign, a transposed index, a
reversed order, an off-by-one, ...), builds that copy with gcc into a
temporary library and runs the pins of tests/test_oracle_pins.py and tests/test_lmhead_cpu.py against it
in a child process (tests/mutant_runner.py). The unchanged source must pass
the same run. The oracle in the repository is never modified. Only
mutations that change what the oracle computes belong here (relabelling the
threshold's groups by a constant offset, for instance, does not: the set of
group maxima is the same).
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "rtopk_oracle.c")

# (name, text in the oracle source, text planted in its place)
MUTANTS = [
    ("score drops the running score",
     "ent[n].score = a + (load_logit(J->logits, J->dtype, r * J->V + t) - lse);",
     "ent[n].score = (load_logit(J->logits, J->dtype, r * J->V + t) - lse);"),
    ("score adds lse instead of subtracting it",
     "ent[n].score = a + (load_logit(J->logits, J->dtype, r * J->V + t) - lse);",
     "ent[n].score = a + (load_logit(J->logits, J->dtype, r * J->V + t) + lse);"),
    ("log-sum-exp without the log",
     "return m + log(s);",
     "return m + s;"),
    ("log-sum-exp drops the first token",
     "    for (int64_t t = 0; t < n; t++)\n        s += exp(",
     "    for (int64_t t = 1; t < n; t++)\n        s += exp("),
    ("flat index transposed",
     "ent[n].flat = (int64_t)j * J->V + t;",
     "ent[n].flat = (int64_t)t * J->beam + j;"),
    ("tie-break by higher flat index",
     "return (a->flat > b->flat) - (a->flat < b->flat);",
     "return (a->flat < b->flat) - (a->flat > b->flat);"),
    ("scores sorted ascending",
     "    if (a->score > b->score)\n        return -1;\n    if (a->score < b->score)\n        return 1;",
     "    if (a->score > b->score)\n        return 1;\n    if (a->score < b->score)\n        return -1;"),
    ("finished beams scored like alive ones",
     "if (J->finished && J->finished[r]) {",
     "if (0) {"),
    ("finished beams offer token 0",
     "ent[n].flat = (int64_t)j * J->V + J->eos_id;",
     "ent[n].flat = (int64_t)j * J->V + 0;"),
    ("padding with beam 0",
     "            J->out_beam[o] = -1;",
     "            J->out_beam[o] = 0;"),
    ("one output too few",
     "        if (p < n) {",
     "        if (p + 1 < n) {"),
    ("fp64 scores rounded through float32",
     "J->out_score64[o] = ent[p].score;",
     "J->out_score64[o] = (double)(float)ent[p].score;"),
    ("binary16 exponent bias off by one",
     "v = ldexp((double)(1024 + f), e - 25);",
     "v = ldexp((double)(1024 + f), e - 24);"),
    ("binary16 subnormal scale off by one",
     "v = ldexp((double)f, -24);",
     "v = ldexp((double)f, -25);"),
    ("bfloat16 placed one bit low",
     "uint32_t u = (uint32_t)h << 16;",
     "uint32_t u = (uint32_t)h << 15;"),
    ("pair score ignores the finished flag",
     "    if (finished && finished[r])\n        return t == eos_id",
     "    if (0)\n        return t == eos_id"),
    ("pair score uses the previous row's lse",
     "return (double)alive[r] + (load_logit(logits, dtype, r * V + t) - lse[r]);",
     "return (double)alive[r] + (load_logit(logits, dtype, r * V + t) - lse[r > 0 ? r - 1 : r]);"),
    ("pair score drops the running score",
     "return (double)alive[r] + (load_logit(logits, dtype, r * V + t) - lse[r]);",
     "return (load_logit(logits, dtype, r * V + t) - lse[r]);"),
    ("finished pair score at any token",
     "return t == eos_id ? (double)alive[r] : -INFINITY;",
     "return (double)alive[r];"),
    ("threshold is the largest group maximum",
     "double result = gmax[k - 1];",
     "double result = gmax[0];"),
    ("threshold groups by blocks instead of residues",
     "int g = (int)(((i + offset) % ngroups + ngroups) % ngroups);",
     "int g = (int)(((i + offset) / ngroups) % ngroups);"),
    ("survivor count with a strict comparison",
     "if (load_logit(logits, dtype, base + i) >= T)",
     "if (load_logit(logits, dtype, base + i) > T)"),
    ("LM head drops the last hidden unit",
     "for (int64_t h = 0; h < H; h++)",
     "for (int64_t h = 0; h < H - 1; h++)"),
    ("LM head reads the weights transposed",
     "rtopk_oracle_decode_bf16(w[v * H + h])",
     "rtopk_oracle_decode_bf16(w[h * V + v])"),
    ("float64 logits read as float32",
     "return ((const double *)x)[i];",
     "return (double)((const float *)x)[i];"),
]


def _build(src_text, path):
    c = path + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", c, "-o", path, "-lm", "-lpthread"])


def _run_pins(lib):
    r = subprocess.run([sys.executable, os.path.join(HERE, "mutant_runner.py"), lib], capture_output=True,
                       text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr).strip().splitlines()[-1:] if (r.stdout + r.stderr).strip() else []


def test_unmutated_oracle_passes_the_runner(tmp_path):
    lib = str(tmp_path / "liboracle_control.so")
    _build(open(SRC).read(), lib)
    rc, tail = _run_pins(lib)
    assert rc == 0, tail


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0].replace(" ", "_") for m in MUTANTS])
def test_planted_mutation_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site of '{name}' not found exactly once in the oracle source"
    lib = str(tmp_path / "liboracle_mutant.so")
    _build(src.replace(old, new), lib)
    rc, tail = _run_pins(lib)
    assert rc != 0, f"no pin catches the planted mutation '{name}'"
    print(f"[mutant] {name}: {tail}")
