"""Mutation check of the oracle's pins (CPU only).

Each mutant is a plausible one-line mistake planted in a temporary copy of
oracle/fa_oracle.c (a dropped term, a wrong comparison, a wrong operand, a
wrong base).  The copy is compiled with gcc into a temporary directory and
every pin of tests/oracle_pins.py runs against it; at least one pin must fail
for each mutant.  The in-tree oracle is never modified.
"""
import os

import pytest

import oracle_pins as P
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "fa_oracle.c")

MUTANTS = {
    "window off by one": ("p->cs - p->window > 0 ? p->cs - p->window : 0",
                          "p->cs - p->window + 1 > 0 ? p->cs - p->window + 1 : 0"),
    "all source frames visible to target": (
        "if (kkind == FAO_SRC) return kframe == qframe;\n    return qframe >= p->ref_t0[kframe];",
        "if (kkind == FAO_SRC) return 1;\n    return qframe >= p->ref_t0[kframe];"),
    "reference gate strict": ("return qframe >= p->ref_t0[kframe];\n  }\n  if (qkind == FAO_SRC)",
                              "return qframe > p->ref_t0[kframe];\n  }\n  if (qkind == FAO_SRC)"),
    "reference never gated": ("return qframe >= p->ref_t0[kframe];\n  }\n  if (qkind == FAO_SRC)",
                              "return 1;\n  }\n  if (qkind == FAO_SRC)"),
    "source rows read target": ("    return 0;\n  }\n  /* reference rows",
                                "    return kframe == qframe;\n  }\n  /* reference rows"),
    "reference rows read everything": ("return kkind == FAO_REF;", "return 1;"),
    "scale dropped": ("return scale * acc;", "return acc;"),
    "base 2 softmax": ("const double w = exp(score(c->q, k, c->D, c->scale) - c->m);",
                       "const double w = exp2(score(c->q, k, c->D, c->scale) - c->m);"),
    "LSE without max": ("*lse = (float)(mc.m + log(sc.l));", "*lse = (float)(log(sc.l));"),
    "LSE in log2": ("*lse = (float)(mc.m + log(sc.l));", "*lse = (float)(mc.m + log2(sc.l));"),
    "keys used as values": ("c->acc[d] += w * (double)v[d];", "c->acc[d] += w * (double)k[d];"),
    "no normalisation": ("o[d] = (float)(acc[d] / sc.l);", "o[d] = (float)(acc[d]);"),
    "relative query frame": ("const int qframe = kind == FAO_REF ? -1 : p->cs + row / T;",
                             "const int qframe = kind == FAO_REF ? -1 : row / T;"),
    "rows: head and row swapped": (
        "const int rc = one_row(p, kind[i], head[i], row[i], o + (long)i * p->D, lse + i);",
        "const int rc = one_row(p, kind[i], row[i], head[i], o + (long)i * p->D, lse + i);"),
    "max not updated": ("if (c->n == 0 || s > c->m) c->m = s;", "if (c->n == 0) c->m = s;"),
    "int8 truncation": ("float r = nearbyintf(y);", "float r = truncf(y);"),
    "int8 ties away": ("float r = nearbyintf(y);", "float r = roundf(y);"),
    "int8 scale inverted": ("scale = absmax / qmax;", "scale = qmax / absmax;"),
    "e4m3 scale one power low": ("e = k - 9 + (f > 0.875f ? 1 : 0);", "e = k - 10 + (f > 0.875f ? 1 : 0);"),
    "e4m3 scale boundary": ("(f > 0.875f ? 1 : 0)", "(f >= 0.875f ? 1 : 0)"),
    "e4m3 ties odd": ("(c & 1) == 0 && (best & 1) == 1", "(c & 1) == 1 && (best & 1) == 0"),
    "e4m3 bias 8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);",
                    "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "sink ignored": ("(kframe >= history_lo(p) || kframe < p->sink)",
                     "(kframe >= history_lo(p))"),
    "sink off by one": ("(kframe >= history_lo(p) || kframe < p->sink)",
                        "(kframe >= history_lo(p) || kframe <= p->sink)"),
    "w8a8 weight scale by row block": (
        "(double)sw[(long)(j / 128) * kb + b]", "(double)sw[(long)(i / 128) * kb + b]"),
    "w8a8 activation scale dropped": ("acc += (double)sx[(long)i * kb + b] * ", "acc += "),
    "w8a8 block of 64": ("int t1 = (b + 1) * 128 < k ? (b + 1) * 128 : k;",
                         "int t1 = (b + 1) * 128 - 64 < k ? (b + 1) * 128 - 64 : k;"),
    "rope partner off by one": ("const double a = y[i], b = y[i + P];",
                                "const double a = y[i], b = y[(i + P + 1) % D];"),
    "rope frequency exponent doubled": ("pow(base, -(double)j / gsize[g])",
                                        "pow(base, -2.0 * (double)j / gsize[g])"),
    "rmsnorm eps dropped": ("const double r = sqrt(ss / D + eps);", "const double r = sqrt(ss / D);"),
    "rmsnorm gamma dropped": ("y[d] = (double)xv[d] / r * (double)gamma[d];",
                              "y[d] = (double)xv[d] / r;"),
    "rope axes swapped": ("(double)pos[n * 3 + g]", "(double)pos[n * 3 + (g + 1) % 3]"),
    "kmean off by one": ("mean[h * D + d] = n ? (float)(acc / (double)n) : 0.0f;",
                         "mean[h * D + d] = n ? (float)(acc / (double)(n + 1)) : 0.0f;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(find) == 1, "mutation site not unique or missing: %r" % find
    src = tmp_path / "fa_oracle_mutant.c"
    src.write_text(text.replace(find, repl))
    # the mutant needs the oracle header next to it
    (tmp_path / "fa_oracle.h").write_text(open(SRC.replace(".c", ".h")).read())
    lib = O.load(O.build(force=True, out=str(tmp_path / "libmutant.so"), src=str(src)))
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, "mutant '%s' passes every pin" % name
