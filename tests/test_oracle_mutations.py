"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake in a copy of the oracle's C source (on the CPU,
in a temporary directory), builds it, and runs the pin suite against it in a
child process; the suite must fail.  A mistake that survives would mean the
step it touches is not pinned.
"""

import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

# (name, exact text in the oracle, replacement)
MUTANTS = [
    ("conv tap order reversed", "window[p][c][t + i]", "window[p][c][t + 3 - i]"),
    ("conv chain accumulated from the last tap", "for (int i = 0; i < TAPS; ++i) {",
     "for (int i = TAPS - 1; i >= 0; --i) {"),
    ("conv chain with a separate multiply and add", "acc = fmaf(window[p][c][t + i], w, acc);",
     "acc = window[p][c][t + i] * w + acc;"),
    ("conv bias added after the taps",
     "float acc = P->has_bias ? bf16_to_float(P->conv_b[ch]) : 0.0f;\n"
     "        for (int i = 0; i < TAPS; ++i) {\n"
     "          float w = bf16_to_float(P->conv_w[((size_t)p * TAPS + i) * dim + (size_t)h * D + c]);\n"
     "          acc = fmaf(window[p][c][t + i], w, acc);\n"
     "        }\n",
     "float acc = 0.0f;\n"
     "        for (int i = 0; i < TAPS; ++i) {\n"
     "          float w = bf16_to_float(P->conv_w[((size_t)p * TAPS + i) * dim + (size_t)h * D + c]);\n"
     "          acc = fmaf(window[p][c][t + i], w, acc);\n"
     "        }\n"
     "        acc = acc + (P->has_bias ? bf16_to_float(P->conv_b[ch]) : 0.0f);\n"),
    ("q scale folded into the norm factor", "q_hat[t][c] = (Y[0][t][c] * fq) * P->scale;",
     "q_hat[t][c] = Y[0][t][c] * (fq * P->scale);"),
    ("conv weight of wrong head",
     "((size_t)p * TAPS + i) * dim + (size_t)h * D + c]", "((size_t)p * TAPS + i) * dim + c]"),
    ("conv window starts at column 0", "size_t at = base + off + i;", "size_t at = base + i;"),
    ("FP32 conv taps rounded to BF16 on read",
     "if (P->conv_f32) window[p][c][i] = ((const float*)P->conv_state)[at];",
     "if (P->conv_f32) window[p][c][i] = round_bf16(((const float*)P->conv_state)[at]);"),
    ("FP32 conv window written rounded to BF16",
     "if (P->conv_f32) ((float*)P->conv_state)[base + j] = v;",
     "if (P->conv_f32) ((float*)P->conv_state)[base + j] = round_bf16(v);"),
    ("silu sign", "float e = (float)exp(-(double)x);", "float e = (float)exp((double)x);"),
    ("silu not rounded to bf16", "  return round_bf16(y);\n}", "  return y;\n}"),
    ("k not normalised", "k_hat[t][c] = Y[1][t][c] * fk;", "k_hat[t][c] = Y[1][t][c];"),
    ("scale on k instead of q", "q_hat[t][c] = (Y[0][t][c] * fq) * P->scale;\n      k_hat[t][c] = Y[1][t][c] * fk;",
     "q_hat[t][c] = Y[0][t][c] * fq;\n      k_hat[t][c] = (Y[1][t][c] * fk) * P->scale;"),
    ("k norm epsilon dropped",
     "float fq = rsqrt_f32((float)sq + 1.0e-6f);\n    float fk = rsqrt_f32((float)sk + 1.0e-6f);",
     "float fq = rsqrt_f32((float)sq + 1.0e-6f);\n    float fk = rsqrt_f32((float)sk);"),
    ("q norm epsilon dropped", "rsqrt_f32((float)sq + 1.0e-6f)", "rsqrt_f32((float)sq)"),
    ("gate projection transposed", "g += (double)bf16_to_float(row[j])",
     "g += (double)bf16_to_float(P->f_b[((size_t)h * D + j) * D + f])"),
    ("raw gate not rounded", "raw_g[t][f] = round_bf16((float)g);", "raw_g[t][f] = (float)g;"),
    ("gate products formed in FP32", "g += (double)bf16_to_float(row[j]) * (double)bf16_to_float(fa[j]);",
     "g += (double)(bf16_to_float(row[j]) * bf16_to_float(fa[j]));"),
    ("gate summed in FP32", "      double g = 0.0;\n      for (int j = 0; j < D; ++j) g += (double)bf16_to_float(row[j]) * (double)bf16_to_float(fa[j]);",
     "      float g = 0.0f;\n      for (int j = 0; j < D; ++j) g += bf16_to_float(row[j]) * bf16_to_float(fa[j]);"),
    ("decay without exp(A_log)", "float e = (float)exp((double)a_log);", "float e = a_log;"),
    ("decay sign", "float g = lower_bound * s;", "float g = -lower_bound * s;"),
    ("decay along value rows", "s[k] = s[k] * decay[t][k];", "s[k] = s[k] * decay[t][v];"),
    ("dt_bias of wrong channel", "P->dt_bias[(size_t)h * D + f]", "P->dt_bias[f]"),
    ("beta not a sigmoid", "beta[t] = sigmoid_f32(bf16_to_float(P->beta[(token0 + t) * H + h]));",
     "beta[t] = bf16_to_float(P->beta[(token0 + t) * H + h]);"),
    ("delta sign", "float u = (Y[2][t][v] - (float)dot) * beta[t];",
     "float u = ((float)dot - Y[2][t][v]) * beta[t];"),
    ("update with q instead of k", "s[k] = fmaf(k_hat[t][k], u, s[k]);", "s[k] = fmaf(q_hat[t][k], u, s[k]);"),
    ("output with k instead of q", "o += (double)s[k] * (double)q_hat[t][k];",
     "o += (double)s[k] * (double)k_hat[t][k];"),
    ("recurrence output not rounded", "o_bf[t][v] = round_bf16((float)o);", "o_bf[t][v] = (float)o;"),
    ("rmsnorm without 1/128", "float variance = (float)ss * (1.0f / 128.0f) + eps;",
     "float variance = (float)ss + eps;"),
    ("output gate not a sigmoid", "float sg = sigmoid_f32(bf16_to_float(gate[c]));",
     "float sg = bf16_to_float(gate[c]);"),
    ("output norm as o * (rstd * nw) * sigma", "float r = ((o_bf[c] * rstd) * bf16_to_float(norm_w[c])) * sg;",
     "float r = (o_bf[c] * (rstd * bf16_to_float(norm_w[c]))) * sg;"),
    ("output norm as (o * rstd) * (nw * sigma)", "float r = ((o_bf[c] * rstd) * bf16_to_float(norm_w[c])) * sg;",
     "float r = (o_bf[c] * rstd) * (bf16_to_float(norm_w[c]) * sg);"),
    ("norm weight of wrong channel", "* bf16_to_float(norm_w[c])) * sg;", "* bf16_to_float(norm_w[0])) * sg;"),
    ("verify reads slot 0 column", "*read_slot = P->slots[(size_t)b * P->slot_stride + *offset];",
     "*read_slot = P->slots[(size_t)b * P->slot_stride];"),
    ("verify writes every token to the read slot",
     "int target = T == 1 ? rs : P->slots[(size_t)b * P->slot_stride + t];", "int target = rs;"),
    ("window shift off by one", "float v = window[p][c][1 + j];", "float v = window[p][c][j];"),
    ("record k after the norm", "kg[c] = float_to_bf16(Y[1][t][c]);", "kg[c] = float_to_bf16(k_hat[t][c]);"),
    ("padding writes no zeros",
     "for (int c = 0; c < D; ++c) P->out[(token0 + t) * dim + (size_t)h * D + c] = 0;", ";"),
    ("slot 0 treated as live", "if (*read_slot <= 0 || *read_slot >= P->N) return 0;",
     "if (*read_slot < 0 || *read_slot >= P->N) return 0;"),
    ("record mode still writes state", "    } else {\n      /* State write-back",
     "    }\n    {\n      /* State write-back"),
    ("replay u by key instead of value row", "fmaf(k_hat[k], u[v], S[v][k] * a[k])",
     "fmaf(k_hat[k], u[k], S[v][k] * a[k])"),
    ("replay norm epsilon dropped", "const float fk = rsqrt_f32((float)sk + 1.0e-6f);",
     "const float fk = rsqrt_f32((float)sk);"),
    ("replay without decay", "fmaf(k_hat[k], u[v], S[v][k] * a[k])", "fmaf(k_hat[k], u[v], S[v][k])"),
    ("replay with the raw key", "k_hat[c] = bf16_to_float(kg[c]) * fk;", "k_hat[c] = bf16_to_float(kg[c]);"),
    ("replay reads the wrong record token", "const size_t rec = ((size_t)b * P->H + h) * P->T + t;",
     "const size_t rec = ((size_t)b * P->H + h) * P->T;"),
    ("replay applies one token too many", "for (int t = 0; t < n; ++t) {", "for (int t = 0; t <= n && t < P->T; ++t) {"),
]


def _run_mutant(case, tmp):
    name, old, new = case
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutant '{name}': anchor not found exactly once"
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    src = os.path.join(tmp, f"{tag}.c")
    lib = os.path.join(tmp, f"lib_{tag}.so")
    with open(src, "w") as f:
        f.write(text.replace(old, new))
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-o",
                    lib, src, "-lm"], check=True)
    env = dict(os.environ, KDA_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
            results = list(pool.map(lambda c: _run_mutant(c, tmp), MUTANTS))
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, f"mistakes no pin catches: {survivors}"
    assert all(rc == 1 for _, rc in results), results  # failed tests, not crashes


if __name__ == "__main__":
    pytest.main([__file__, "-q"])
