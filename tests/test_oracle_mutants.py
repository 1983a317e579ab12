"""The oracle's pins catch plausible mistakes.

Each mutant is a one-spot edit of a copy of oracle.c (a dropped term, a wrong
sign, index or comparison, a transposed operand).  The copy is compiled into a
temporary library and the whole pin battery runs against it: at least one pin
must fail for every mutant.  The real oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle
from tests.oracle_pins import ALL_PINS

MUTANTS = [
    ("router weight transposed", "value_at(w_router, dtype, j * E + e)", "value_at(w_router, dtype, e * d + j)"),
    ("bias not added", "lp[e] = logits[t * E + e] + b;", "lp[e] = logits[t * E + e];"),
    ("bias subtracted", "lp[e] = logits[t * E + e] + b;", "lp[e] = logits[t * E + e] - b;"),
    ("higher index wins ties", "lp[e] > lp[best]) best = e;", "lp[e] >= lp[best]) best = e;"),
    ("selects the smallest", "lp[e] > lp[best]) best = e;", "lp[e] < lp[best]) best = e;"),
    ("no renormalisation", "w[t * K + k] = p[ids[t * K + k]] / sel;", "w[t * K + k] = p[ids[t * K + k]];"),
    ("softmax not normalised", "for (int64_t e = 0; e < E; ++e) p[e] /= z;", ""),
    ("softmax of the K probabilities",
     "for (int64_t k = 0; k < K; ++k) sel += p[ids[t * K + k]];",
     "for (int64_t k = 0; k < K; ++k) { p[ids[t * K + k]] = exp(p[ids[t * K + k]]); sel += p[ids[t * K + k]]; }"),
    ("rank counted after increment", "rank[i] = counts[e];\n        counts[e] += 1;", "counts[e] += 1;\n        rank[i] = counts[e];"),
    ("capacity off by one", "if (capacity < 0 || rank[i] < capacity)", "if (capacity < 0 || rank[i] <= capacity)"),
    ("offsets from routed counts", "offsets[e + 1] = offsets[e] + kept[e];", "offsets[e + 1] = offsets[e] + counts[e];"),
    ("silu sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("gate on the wrong branch", "a[f] = silu(g1) * g3;", "a[f] = silu(g3) * g1;"),
    ("no gate", "a[f] = silu(g1) * g3;", "a[f] = g1 * g3;"),
    ("down projection transposed", "value_at(w2e, dtype, i * F + f)", "value_at(w2e, dtype, f * d + i)"),
    ("combine ignores weights", "yt[i] += w[t * K + k] * h[i];", "yt[i] += h[i];"),
    ("dropped slots still combined", "if (assign_row && assign_row[t * K + k] < 0) continue; /* dropped */", ""),
    ("aux fraction over tokens only", "double f = (double)counts[e] / (double)(T * K);", "double f = (double)counts[e] / (double)T;"),
    ("aux without the N factor", "return (double)E * total;", "return total;"),
    ("bias update sign", "bias[e] = bias[e] - alpha;", "bias[e] = bias[e] + alpha;"),
    ("bias update moves at target", "else if (load < T * K)", "else if (load <= T * K)"),
    ("z-loss not squared", "total += lse * lse;", "total += lse;"),
    ("z-loss without the max", "double lse = m + log(s);", "double lse = log(s);"),
    ("z-loss not averaged", "return total / (double)T;", "return total;"),
    ("top-K aux counts every expert", "if (ids[t * K + k] == e) chosen += probs[t * E + e];",
     "chosen += probs[t * E + e] / (double)K;"),
    ("top-K aux over slots", "sum_fp += frac * (chosen / (double)T);", "sum_fp += frac * (chosen / (double)(T * K));"),
    ("top-K aux without the N factor", "return sum_fp * (double)E;", "return sum_fp;"),
    ("concat weight transposed", "value_at(w_cat, dtype, o * K * d + k * d + i)",
     "value_at(w_cat, dtype, (k * d + i) * d_out + o)"),
    ("concat dropped slot read", "if (row < 0) continue; /* dropped slot: a block of zeros */", ""),
    ("concat slots reversed", "const int32_t row = assign_row[t * K + k];",
     "const int32_t row = assign_row[t * K + (K - 1 - k)];"),
]


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, find, repl, tmp_path):
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(find) == 1, f"mutation site for '{name}' must occur exactly once"
    mutated = tmp_path / "oracle_mutant.c"
    mutated.write_text(src.replace(find, repl))
    lib = str(tmp_path / "liboracle_mutant.so")
    oracle.build(source=str(mutated), out=lib)
    # A mutant may write out of bounds, so its pins run in a child process.
    code = (
        "import sys, oracle\n"
        "from tests.oracle_pins import ALL_PINS\n"
        f"orc = oracle.Oracle({lib!r})\n"
        "for pin in ALL_PINS:\n"
        "    try:\n"
        "        pin(orc)\n"
        "    except AssertionError:\n"
        "        print('FAILED', pin.__name__, flush=True)\n"
    )
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    proc = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True,
                          text=True, timeout=120)
    failures = [ln.split()[1] for ln in proc.stdout.splitlines() if ln.startswith("FAILED")]
    assert failures, f"mutant '{name}' survived every pin (exit {proc.returncode})"
