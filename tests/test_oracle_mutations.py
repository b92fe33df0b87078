"""Each plausible mistake planted in a scratch copy of the oracle must fail a pin.

The mistakes are planted in the oracle's C source, or in its parity bar
(compare.py), on the CPU (never on a GPU); the pins in test_oracle_pins.py (or
test_compare_pins.py) are then run against the mutated copy in a subprocess. A mutation that every pin lets through would mean the pins do not
cover that part of the definition.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (description, original text, planted mistake)
MUTATIONS = [
    ("RoPE first-half sign", "v[i] = x1 * cs - x2 * sn;", "v[i] = x1 * cs + x2 * sn;"),
    ("RoPE second-half sign", "v[i + half] = x2 * cs + x1 * sn;", "v[i + half] = x2 * cs - x1 * sn;"),
    ("RoPE frequency exponent", "pow(base, -2.0 * (double)i / (double)rd)", "pow(base, -(double)i / (double)rd)"),
    ("RoPE interleaved pairs", "double x1 = v[i], x2 = v[i + half];", "double x1 = v[2 * i], x2 = v[2 * i + 1];"),
    ("RoPE global token position", "(double)(s + pos_offset)", "(double)(t + pos_offset)"),
    ("RoPE ignores pos_offset", "(double)(s + pos_offset)", "(double)(s)"),
    ("RoPE applied to v", "rope && which < 2;", "rope && which < 3;"),
    ("dropped last channel", "for (int64_t c = 0; c < C; ++c) {\n                    const double xc",
     "for (int64_t c = 0; c < C - 1; ++c) {\n                    const double xc"),
    ("[F,C] weight read as [C,F]", "return w_fc ? w[f * C + c] : w[c * F + f];",
     "return w_fc ? w[c * F + f] : w[c * F + f];"),
    ("q and k slices swapped", "            *which = 0;\n            *head = r / hd;",
     "            *which = 1;\n            *head = r / hd;"),
    ("grouped order: k and v slots swapped", "*which = slot == qpk ? 1 : 2;", "*which = slot == qpk ? 2 : 1;"),
    ("grouped order: q heads numbered across groups", "*head = g * qpk + slot;", "*head = slot * n_kv + g;"),
    ("partial RoPE rotates the whole head", "rope_rotate_half(dst[which] + h * head_dim, rd,",
     "rope_rotate_half(dst[which] + h * head_dim, head_dim,"),
    ("tanh GELU", "return 0.5 * y * (1.0 + erf(y / sqrt(2.0)));",
     "return 0.5 * y * (1.0 + tanh(0.7978845608028654 * (y + 0.044715 * y * y * y)));"),
    ("tanh GELU constant", "0.044715 * y * y * y", "0.04715 * y * y * y"),
    ("tanh GELU without the cube", "(y + 0.044715 * y * y * y)", "(y + 0.044715 * y * y)"),
    ("squared ReLU without the clamp", "const double r = (y > 0.0 || isnan(y)) ? y : 0.0;", "const double r = y;"),
    ("squared ReLU clamps NaN to 0", "const double r = (y > 0.0 || isnan(y)) ? y : 0.0;",
     "const double r = y > 0.0 ? y : 0.0;"),
    ("exact GELU of -inf taken as its limit 0", "return 0.5 * y * (1.0 + erf(y / sqrt(2.0)));",
     "return isinf(y) && y < 0.0 ? 0.0 : 0.5 * y * (1.0 + erf(y / sqrt(2.0)));"),
    ("empty contraction rejected", "nb <= 0 || C < 0 || S <= 0 || nsp < 1 || nsp > 3 || ntok < 0",
     "nb <= 0 || C <= 0 || S <= 0 || nsp < 1 || nsp > 3 || ntok < 0"),
    ("squared ReLU not squared", "    return r * r;", "    return r;"),
    ("split+RoPE transposed key indexed as untransposed", "else k[(slab * hd + j) * T + s] = head[j];",
     "else k[(slab * T + s) * hd + j] = head[j];"),
    ("split+RoPE RoPE skipped", "if (rope && which < 2) rope_rotate_half(head, rd,", "if (0) rope_rotate_half(head, rd,"),
    ("spatial dims unflattened in reverse", "int64_t idx = rem % sp_size[d];", "int64_t idx = rem % sp_size[nsp - 1 - d];"),
    ("bias skipped on the ff slice", "for (int64_t f = 0; f < F; ++f) y[f] += bias[f];",
     "for (int64_t f = 0; f < F; ++f) y[f] += (f < ff_dim ? 0.0 : bias[f]);"),
]


@pytest.mark.parametrize("desc,orig,bad", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(tmp_path, desc, orig, bad):
    src = open(os.path.join(ROOT, "oracle", "fused_proj_oracle.c")).read()
    assert src.count(orig) >= 1, f"mutation site not found: {desc}"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "*.tmp", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    (tmp_path / "oracle" / "fused_proj_oracle.c").write_text(src.replace(orig, bad, 1))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=tmp_path, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"no pin caught the planted mistake: {desc}\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:]


# Mistakes planted in the parity bar (oracle/compare.py); each must fail a test of
# test_compare_pins.py, which builds the bar by brute force from the oracle's own
# effective columns.
BAR_MUTATIONS = [
    ("token norm taken as L1", "xn = np.linalg.norm(rows, axis=1)", "xn = np.abs(rows).sum(axis=1)"),
    ("column norm over the wrong axis", "wn = np.linalg.norm(w_cf, axis=0)",
     "wn = np.linalg.norm(w_cf, axis=0)[::-1]"),
    ("RoPE cross term sign, first half", "c * c * n1 + s * s * n2 - 2 * c * s * d12",
     "c * c * n1 + s * s * n2 + 2 * c * s * d12"),
    ("RoPE cross term sign, second half", "c * c * n2 + s * s * n1 + 2 * c * s * d12",
     "c * c * n2 + s * s * n1 - 2 * c * s * d12"),
    ("RoPE bias partner swapped", "b1 = np.abs(c) * a1 + np.abs(s) * a2", "b1 = np.abs(c) * a2 + np.abs(s) * a1"),
    ("RoPE bias without its sine term", "b2 = np.abs(c) * a2 + np.abs(s) * a1", "b2 = np.abs(c) * a2"),
    ("RoPE angles over the head instead of the rotated width", "theta = rope_base ** (-2.0 * np.arange(half) / R)",
     "theta = rope_base ** (-2.0 * np.arange(half) / head_dim)"),
    ("RoPE position offset dropped", "phi = (positions.astype(np.float64) + pos_offset)",
     "phi = (positions.astype(np.float64) + 0)"),
    ("squared-ReLU factor halved", "ff = ff * (1.0 + 2.0 * np.sqrt(", "ff = ff * (1.0 + 1.0 * np.sqrt("),
    ("bias left out of the bar", "plain = xn[:, None] * wn[None, :] + np.abs(b)[None, :]",
     "plain = xn[:, None] * wn[None, :] + 0.0 * np.abs(b)[None, :]"),
    ("bar loosened by 2", "ratio = err / (rel * s + 1e-300)", "ratio = err / (2 * rel * s + 1e-300)"),
    ("non-finite outputs accepted", "finite &= bool(np.all(np.isfinite(g)))", "finite &= True"),
    ("backward bar without the second rounding", 'BACKWARD_REL = {"bf16": 8e-3', 'BACKWARD_REL = {"bf16": 4e-3'),
    ("backward bar loosened", 'BACKWARD_REL = {"bf16": 8e-3', 'BACKWARD_REL = {"bf16": 2e-2'),
    ("backward comparison with the forward bar",
     "return compare(got, ref, scl, dtype, rel=BACKWARD_REL[dtype], tight=False)",
     "return compare(got, ref, scl, dtype, tight=False)"),
    ("backward diagnostic from the forward rounding model",
     "return compare(got, ref, scl, dtype, rel=BACKWARD_REL[dtype], tight=False)",
     "return compare(got, ref, scl, dtype, rel=BACKWARD_REL[dtype], tight=True)"),
]


@pytest.mark.parametrize("desc,orig,bad", BAR_MUTATIONS, ids=[m[0] for m in BAR_MUTATIONS])
def test_planted_bar_mistake_fails_a_pin(tmp_path, desc, orig, bad):
    src = open(os.path.join(ROOT, "oracle", "compare.py")).read()
    assert src.count(orig) == 1, f"mutation site not found: {desc}"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.tmp", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    (tmp_path / "oracle" / "compare.py").write_text(src.replace(orig, bad, 1))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_compare_pins.py", "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=tmp_path, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"no pin caught the planted mistake: {desc}\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:]


# Mistakes planted in the backward oracle; each must fail a test of
# test_oracle_backward_pins.py (finite differences of the forward oracle, numpy products).
BACKWARD_MUTATIONS = [
    ("inverse RoPE first-half sign", "g[i] = g1 * cs + g2 * sn;", "g[i] = g1 * cs - g2 * sn;"),
    ("inverse RoPE second-half sign", "g[i + half] = g2 * cs - g1 * sn;", "g[i + half] = g2 * cs + g1 * sn;"),
    ("inverse RoPE ignores pos_offset", "rope_rotate_half_transposed(g, rd, (double)(s + pos_offset), rope_base)",
     "rope_rotate_half_transposed(g, rd, (double)(s), rope_base)"),
    ("inverse RoPE over the whole head", "rope_rotate_half_transposed(g, rd,", "rope_rotate_half_transposed(g, head_dim,"),
    ("GELU derivative without y phi(y)", "return 0.5 * (1.0 + erf(y / sqrt(2.0))) + y * pdf;",
     "return 0.5 * (1.0 + erf(y / sqrt(2.0)));"),
    ("tanh GELU derivative without the cube's factor 3", "du = k * (1.0 + 3.0 * 0.044715 * y * y);",
     "du = k * (1.0 + 0.044715 * y * y);"),
    ("squared ReLU derivative without the factor 2", "case 3: return y > 0.0 ? 2.0 * y : 0.0;",
     "case 3: return y > 0.0 ? y : 0.0;"),
    ("bias left out of the recomputed pre-activation", "y[f] = acc + (bias ? bias[f] : 0.0);", "y[f] = acc;"),
    ("channels-first d_ff read token-major", "const double up = ff_cf ? d_ff[(bi * ff_dim + f) * S + s]",
     "const double up = ff_cf ? d_ff[t * ff_dim + f]"),
    ("dx drops the ff columns", "for (int64_t f = 0; f < F; ++f) acc += dyt[f] * w_at(w, c, f, C, F, w_fc);",
     "for (int64_t f = ff_dim; f < F; ++f) acc += dyt[f] * w_at(w, c, f, C, F, w_fc);"),
    ("dW tokens unflattened batch-minor", "const double xv = x_at(x, t / S, t % S, c,",
     "const double xv = x_at(x, t % nb, t / nb, c,"),
    ("db misses the last token", "for (int64_t t = 0; t < M; ++t)\n            for (int64_t f = 0; f < F; ++f) db[f]",
     "for (int64_t t = 0; t < M - 1; ++t)\n            for (int64_t f = 0; f < F; ++f) db[f]"),
]


@pytest.mark.parametrize("desc,orig,bad", BACKWARD_MUTATIONS, ids=[m[0] for m in BACKWARD_MUTATIONS])
def test_planted_backward_mistake_fails_a_pin(tmp_path, desc, orig, bad):
    src = open(os.path.join(ROOT, "oracle", "fused_proj_oracle.c")).read()
    assert src.count(orig) == 1, f"mutation site not found: {desc}"
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "*.tmp", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutations.py"))
    (tmp_path / "oracle" / "fused_proj_oracle.c").write_text(src.replace(orig, bad, 1))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_backward_pins.py", "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=tmp_path, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"no pin caught the planted mistake: {desc}\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:]
