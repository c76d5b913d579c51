"""The oracle's pins catch plausible mistakes.

Each case below plants one mistake in a private copy of oracle/oracle.c,
compiles it with gcc on the CPU, and runs the pin suite (tests/test_oracle.py)
against it in a subprocess.  The suite must fail for every mutant.  Nothing
here touches a GPU or the HIP library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("gate_w transposed",
     "load_elem(gate_w, (int64_t)h * E + e, dtype)",
     "load_elem(gate_w, (int64_t)e * H + h, dtype)"),
    ("bias dropped",
     "for (int32_t e = 0; e < E; ++e) logit[e] += (double)bias[e];",
     "for (int32_t e = 0; e < E; ++e) logit[e] += 0.0;"),
    ("ties to higher index",
     "while (j >= 0 && logit[order[j]] < logit[cur]) {",
     "while (j >= 0 && logit[order[j]] <= logit[cur]) {"),
    ("ascending order",
     "while (j >= 0 && logit[order[j]] < logit[cur]) {",
     "while (j >= 0 && logit[order[j]] > logit[cur]) {"),
    ("no renormalisation",
     "w[n * K + k] = (float)(p[order[k]] / s);",
     "w[n * K + k] = (float)(p[order[k]]);"),
    ("margin off by one",
     "logit[order[K - 1]] - logit[order[K]];",
     "logit[order[K - 1]] - logit[order[E - 1]];"),
    ("segment order reversed",
     "for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e];",
     "for (int32_t e = 0; e < E; ++e) cursor[e] = offsets[e + 1] - 1;"),
    ("perm and inv swapped",
     "perm[r] = (int32_t)i;\n    inv[i] = r;",
     "inv[r] = (int32_t)i;\n    perm[i] = r;"),
    ("offsets inclusive",
     "offsets[e + 1] = offsets[e] + counts[e];",
     "offsets[e + 1] = offsets[e] + counts[e] + (e == 0);"),
    ("permute by slot modulo K",
     "int64_t n = perm[r] / K;",
     "int64_t n = perm[r] % N;"),
    ("combine slot transposed",
     "int64_t row = inv[n * K + k];",
     "int64_t row = inv[(k * N + n) % T];"),
    ("combine drops the weight",
     "acc += (double)w[n * K + k] * load_elem(y, row * H + h, dtype);",
     "acc += load_elem(y, row * H + h, dtype) / K;"),
    ("combine rounds twice",
     "double_to_bf16(acc);",
     "double_to_bf16((double)(float)acc);"),
    ("ep no deduplication",
     "if (ids[n * K + k2] / per_rank == r) first = 0;",
     "if (0) first = 0;"),
    ("ep tokens in descending order",
     "for (int64_t i = 0; i < T; ++i) {\n    if (!owner[i]) continue;",
     "for (int64_t i = T - 1; i >= 0; --i) {\n    if (!owner[i]) continue;"),
    ("ep shared slot off by one",
     "send_row[n * K + k] = send_row[n * K + k2];",
     "send_row[n * K + k] = send_row[n * K + k2] + 1;"),
    ("ep expand index not segment-relative",
     "expand_idx[p] = send_row[i] - send_offsets[ids[i] / per_rank];",
     "expand_idx[p] = send_row[i];"),
    ("backward: softmax Jacobian without the probability factor",
     "dl[n * E + e] = p[e] * (dp[e] - u);",
     "dl[n * E + e] = (dp[e] - u);"),
    ("backward: renormalisation term with the wrong sign",
     "(double)dw[n * K + k] / s - t / (s * s);",
     "(double)dw[n * K + k] / s + t / (s * s);"),
    ("backward: renormalisation term dropped",
     "(double)dw[n * K + k] / s - t / (s * s);",
     "(double)dw[n * K + k] / s;"),
    ("backward: gate gradient expert index reversed",
     "gacc[(int64_t)h * E + e] += xv * dl[n * E + e];",
     "gacc[(int64_t)h * E + e] += xv * dl[n * E + (E - 1 - e)];"),
    ("backward: combine gradient ignores the weight",
     "store_elem(dy, rw * H + h, dtype, (double)w[n * K + k] * g);",
     "store_elem(dy, rw * H + h, dtype, g);"),
    ("backward: weight gradient dots dout with itself",
     "acc += g * load_elem(y, rw * H + h, dtype);",
     "acc += g * g;"),
    ("backward: dispatch gradient takes one slot",
     "acc += load_elem(dx_perm, rw * H + h, dtype);",
     "acc = load_elem(dx_perm, rw * H + h, dtype);"),
    ("aggregate drops the residual",
     "acc += load_elem(residual, n * (int64_t)H + h, dtype);",
     "acc += 0.0;"),
    ("grouped linear uses the next expert",
     "while (!(offsets[e] <= p && p < offsets[e + 1])) ++e; /* the segment holding p */",
     "while (!(offsets[e] <= p && p < offsets[e + 1])) ++e; e = (e + 1) % E;"),
    ("grouped linear weight transposed",
     "load_elem(weight, ((int64_t)e * F + f) * H + h, dtype);",
     "load_elem(weight, ((int64_t)e * H + h % H) * F + f % F, dtype);"),
    ("bf16 decode shifted",
     "uint32_t u = (uint32_t)b << 16;",
     "uint32_t u = (uint32_t)b << 15;"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    str(mutant), "-lm", "-o", str(lib)], check=True)
    env = dict(os.environ, MOE_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"pins did not catch mutant '{name}':\n{r.stdout[-2000:]}"
