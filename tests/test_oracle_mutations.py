"""Plant plausible mistakes in a copy of the oracle source (on the CPU) and check that the pins
in test_oracle_pins.py catch every one of them."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hs_oracle.c")

# (name, exact snippet of the correct source, the planted mistake)
MUTANTS = [
    ("no_scale", "const double tau = s->scale > 0.0 ? s->scale : 1.0 / sqrt((double)d);",
     "const double tau = s->scale > 0.0 ? s->scale : 1.0;"),
    ("given_scale_ignored", "const double tau = s->scale > 0.0 ? s->scale : 1.0 / sqrt((double)d);",
     "const double tau = 1.0 / sqrt((double)d);"),
    ("head_mapping", "const int u = h / (s->n_q_heads / s->n_kv_heads);",
     "const int u = h % s->n_kv_heads;"),
    ("drops_diagonal", "const int64_t n = s->q_offset + j + 1;\n      logits_row",
     "const int64_t n = s->q_offset + j + (j > 0 ? 0 : 1);\n      logits_row"),
    ("candidates_overlap_window", "const int64_t n_cand = t - window + 1 > 0 ? t - window + 1 : 0;",
     "const int64_t n_cand = t - window + 2 > 0 ? t - window + 2 : 0;"),
    ("tie_prefers_later", "return (a->i > b->i) - (a->i < b->i);",
     "return (a->i < b->i) - (a->i > b->i);"),
    ("group_sum_not_max", "if (p > score[i]) score[i] = p;",
     "score[i] = (score[i] == -INFINITY ? 0.0 : score[i]) + p;"),
    ("unnormalized_score", "const double p = exp(tmp[i] - L);\n      if (p > score[i])",
     "const double p = tmp[i];\n      if (p > score[i])"),
    ("block_boundary_shift", "if (p > bs[i / block]) bs[i / block] = p;",
     "if (p > bs[i > 0 ? (i - 1) / block : 0]) bs[i > 0 ? (i - 1) / block : 0] = p;"),
    ("gates_swapped", "out[c] = gO * (sigmoid(zG) * og[c] + sigmoid(zL) * ol[c]);",
     "out[c] = gO * (sigmoid(zL) * og[c] + sigmoid(zG) * ol[c]);"),
    ("channel_gates_interleaved", "gate_ch[(row * 2 + 0) * d + c]",
     "gate_ch[(row * d + c) * 2 + 0]"),
    ("channel_gate_per_head", "gate_ch[(row * 2 + 1) * d + c]", "gate_ch[(row * 2 + 1) * d]"),
    ("channel_out_gate_per_head", "out_gate_ch[row * s->head_dim + c]",
     "out_gate_ch[row * s->head_dim]"),
    ("swa_window_too_wide",
     "for (int64_t i = (t - window + 1 > 0 ? t - window + 1 : 0); i <= t; i++) keep[i] = 1;\n      logits_row(s, q, k_loc",
     "for (int64_t i = (t - window > 0 ? t - window : 0); i <= t; i++) keep[i] = 1;\n      logits_row(s, q, k_loc"),
    ("mask_ignored", "if (keep && !keep[i]) continue;", "(void)keep;"),
    ("lse_log2", "return m + log(l);", "return m + log2(l);"),
    ("sink_sign", "return m + log(exp(L - m) + exp(sv - m));",
     "return m + log(exp(L - m) + exp(-sv - m));"),
    ("sink_ignored_when_empty", "if (L == -INFINITY) return sv;", "if (L == -INFINITY) return L;"),
    ("sink_local_in_global", "double L = with_sink(lse_of(a, keep, t + 1), sink, h);\n      weighted_sum(s, v, b, u, a, keep, t + 1, L, og);",
     "double L = with_sink(lse_of(a, keep, t + 1), sink_loc, h);\n      weighted_sum(s, v, b, u, a, keep, t + 1, L, og);"),
    ("out_gate_missing", "if (out_gate) return sigmoid((double)out_gate[row]);",
     "if (out_gate) return 1.0;"),
]


@pytest.mark.parametrize("name,good,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, good, bad, tmp_path):
    src = open(SRC).read()
    assert src.count(good) == 1, f"snippet for {name} not unique in the oracle source"
    mutant = tmp_path / "hs_oracle.c"
    mutant.write_text(src.replace(good, bad))
    hdr = os.path.join(ROOT, "oracle", "hs_oracle.h")
    (tmp_path / "hs_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutant), "-lm"], check=True)
    env = dict(os.environ, HS_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout[-2000:]}"
