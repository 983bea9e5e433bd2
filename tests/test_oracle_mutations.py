"""Mutation check of the oracle's pins (CPU).

Each mutant below plants one plausible mistake in a copy of
oracle/mala_oracle.c (an index off by one, a wrong sign, a dropped term, a
transposed operand, a wrong traversal order or comparison, a wrong head
mapping, a merge without rescaling, ...). The copy is compiled into a
temporary library, and the oracle's pins (tests/test_oracle.py) run against
it in a child process through MALA_ORACLE_LIB. Every mutant must make a pin
fail, and the unmutated copy must pass them all. Nothing here touches the
in-tree oracle."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mala_oracle.c")

MUTANTS = {
    # the backward's bf16-operand model rounds dS before the dK / dQ products
    "bf16 model without dS rounding": ("double du = (p->round_flags & ORC_ROUND_DS) ? round_bf16(ds) : ds;",
                                       "double du = ds;"),
    # the kernel's rounding model: the reference moves on jumps of more than 8 log2 units
    "lazy reference at 4 log2 units": ("m_new = mx > m[r] + 8.0 * 0.69314718055994530942 ? mx : m[r];",
                                       "m_new = mx > m[r] + 4.0 * 0.69314718055994530942 ? mx : m[r];"),
    # the same model forms a 128-key tile whose upper 64 keys pass alone as two halves
    "lazy reference over whole 128-key tiles": ("if ((p->round_flags & ORC_LAZY_REF) && bk == 128) {",
                                                "if (0) {"),
    # Sec. 2.1: L_q counts the query's own key
    "L_q one short": ("return p->causal ? (double)(q + causal_offset(p) + 1) : (double)p->seqlen_k;",
                      "return p->causal ? (double)(q + causal_offset(p)) + 1e-9 : (double)p->seqlen_k;"),
    # Sec. 2.2: the causal mask admits the diagonal key, not the next one
    "mask admits k = q + 1": ("if (p->causal && k > q + causal_offset(p)) return 0;",
                              "if (p->causal && k > q + causal_offset(p) + 1) return 0;"),
    # Sec. 2.2 / Alg. 1: descending traversal from the diagonal
    "ascending traversal": ("for (int64_t j = j_hi; j >= j_lo; --j) {",
                            "for (int64_t j = j_lo; j <= j_hi; ++j) {"),
    # Eq. 3: strict comparison (a margin of exactly zero retains)
    "non-strict skip": ("int retain = !(tile_margin < 0.0);", "int retain = !(tile_margin <= 0.0);"),
    # Eq. 3: the running normaliser enters the test as m + log l
    "margin sign": ("mg = mt[r] - (m[r] + log(l[r])) - log_threshold(p, q0 + r);",
                    "mg = mt[r] - (m[r] - log(l[r])) - log_threshold(p, q0 + r);"),
    # Sec. 2.2: l = 0 means a ratio of +inf (retain)
    "empty normaliser skips": ("mg = INFINITY; /* Z = 0: ratio defined as +inf (Sec. 2.2) */",
                               "mg = -INFINITY;"),
    # Sec. 2.2: one failing row retains the tile (largest row margin)
    "smallest row margin": ("if (mg > tile_margin) tile_margin = mg;",
                            "if (mg < tile_margin || tile_margin == -INFINITY) tile_margin = mg;"),
    # online softmax: the running sum is rescaled with the maximum
    "no rescale of l": ("l[r] = alpha * l[r] + rowsum;", "l[r] = l[r] + rowsum;"),
    # Sec. 2.2: every valid row of a retained tile is updated
    "update only passing rows": (
        "    online_update(p, s, bk, vbase, k0, nrows, 0, bk, m, l, acc);\n  }\n  free(s);",
        "    for (int64_t r = 0; r < nrows; ++r)\n"
        "      if (l[r] != 0.0 && mt[r] - (m[r] + log(l[r])) - log_threshold(p, q0 + r) < 0)\n"
        "        for (int c = 0; c < bk; ++c) s[r * bk + c] = -INFINITY;\n"
        "    online_update(p, s, bk, vbase, k0, nrows, 0, bk, m, l, acc);\n  }\n  free(s);"),
    # GQA: consecutive query heads share a KV head
    "GQA head map": ("    const int64_t g = h / G;\n    const int64_t q0",
                     "    const int64_t g = h % p->heads_kv;\n    const int64_t q0"),
    # Eq. 4: s - z against the threshold
    "backward test sign": ("const double mg = sv - lse[row] - log_threshold(p, qi);",
                           "const double mg = sv + lse[row] - log_threshold(p, qi);"),
    # Alg. 2: dS = P (dP - D)
    "dS sign of D": ("const double ds = pr * (dp - D[row]);", "const double ds = pr * (dp + D[row]);"),
    # Alg. 2: dK = scale dS^T Q (Q, not dO)
    "dK operand": ("dkr[c] += du * (mag ? fabs(q[row * d + c]) : q[row * d + c]);",
                   "dkr[c] += du * (mag ? fabs(dout[row * d + c]) : dout[row * d + c]);"),
    # Alg. 2: the scale of the scores reaches dK
    "dK unscaled": ("      krows[x] *= p->scale;\n", "\n"),
    # Sec. 2.4: a split tests against L = N_k, not its own length
    "decode per-split L": ("pd.causal = 0; /* the single query sees all N_k keys: L = N_k */",
                           "pd.causal = 0; pd.tau = p->tau * num_splits;"),
    # the review's merge brings every summary to the common maximum
    "merge without rescale": ("const double w = exp(m[s] - M);", "const double w = 1.0;"),
    # bf16 conversion rounds to nearest even
    "bf16 rounds half up": ("u += 0x7fffu + ((u >> 16) & 1u);", "u += 0x8000u;"),
}


def _build(src_text, tmp_path, name):
    c = tmp_path / f"{name}.c"
    c.write_text(src_text)
    lib = tmp_path / f"{name}.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
                           str(lib), str(c), "-lm"])
    return str(lib)


def _pins(lib):
    env = dict(os.environ, MALA_ORACLE_LIB=lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle.py"),
                        "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-600:]


def test_unmutated_copy_passes_the_pins(tmp_path):
    rc, out = _pins(_build(open(SRC).read(), tmp_path, "clean"))
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_the_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site of {name!r} not found"
    rc, out = _pins(_build(src.replace(old, new, 1), tmp_path, "mutant"))
    assert rc != 0, f"the pins missed the mutant {name!r}"
