"""The oracle's pins catch plausible mistakes.

Each case below plants one mistake in a copy of oracle/oracle.c (on the CPU,
in a temporary directory), builds it, and runs the pin suite
tests/test_oracle.py against the broken library.  The suite must fail for
every mutant; a mutant that survives means a pin is missing.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, planted mistake); each original must occur in oracle.c
MUTANTS = [
    ("mask_reversed", "if (j > i) return 0;", "if (j < i) return 0;"),
    ("mask_off_by_one", "if (j > i) return 0;", "if (j >= i) return 0;"),
    ("window_off_by_one", "return window <= 0 || j > i - window;",
     "return window <= 0 || j >= i - window;"),
    ("window_ignored", "return window <= 0 || j > i - window;", "return 1;"),
    ("gqa_fwd_heads_interleaved", "long kvh = b * Hkv + h / (H / Hkv);", "long kvh = b * Hkv + h % Hkv;"),
    ("gqa_bwd_heads_interleaved", "size_t kvoff = (size_t)(b * Hkv + h / (H / Hkv)) * n * d;",
     "size_t kvoff = (size_t)(b * Hkv + h % Hkv) * n * d;"),
    ("gqa_bwd_no_group_sum", "dk[kvoff + e] += gk[e];", "dk[kvoff + e] = gk[e];"),
    ("no_max_subtraction", "for (long i = 0; i < n; ++i) p[i] = exp(x[i] - m) / s;",
     "for (long i = 0; i < n; ++i) p[i] = exp(x[i]) / (s * exp(m));"),
    ("online_drops_rescale", "l = l * rescale + csum;", "l = l + csum;"),
    ("lse_drops_log_sum", "lse[r] = m + log(sum);", "lse[r] = m;"),
    ("score_scale_dropped", "srow[j] = scale * acc;\n    }\n  }\n  /* step 2",
     "srow[j] = acc;\n    }\n  }\n  /* step 2"),
    ("pv_transposed_index", "orow[c] += pj * v[j * d + c];", "orow[c] += pj * v[c * d + j % d];"),
    ("ds_wrong_sign", "dsrow[j] = P[i * n + j] * (dsrow[j] - di);",
     "dsrow[j] = P[i * n + j] * (dsrow[j] + di);"),
    ("dq_scale_dropped", "for (long c = 0; c < d; ++c) dq[i * d + c] *= scale;", ""),
    ("dk_transposed_ds", "double ws = dS[i * n + j], wp = P[i * n + j];",
     "double ws = dS[j * n + i], wp = P[i * n + j];"),
    ("dv_uses_ds", "double ws = dS[i * n + j], wp = P[i * n + j];",
     "double ws = dS[i * n + j], wp = dS[i * n + j];"),
    ("merge_unweighted", "double w = exp(lse_parts[c] - big);", "double w = 1.0;"),
    ("tiled_no_alpha", "for (long c = 0; c < d; ++c) o[r * d + c] *= alpha;", ""),
]


@pytest.mark.parametrize("name,orig,mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_kill_mutant(tmp_path, name, orig, mutant):
    src = open(SRC).read()
    assert orig in src, f"mutation site for {name} not found"
    bad = tmp_path / "oracle_mutant.c"
    bad.write_text(src.replace(orig, mutant, 1))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", str(bad), "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins:\n{r.stdout[-2000:]}"
