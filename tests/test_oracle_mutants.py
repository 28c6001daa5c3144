"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the oracle's pins reject every one of them.  The copy is compiled to a
temporary library; the pin suite runs in a child process pointed at it."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "q8_0_d_big_endian": ("const float d = oracle_fp16_to_f32(load_le16(blk));\n            for (int t = 0; t < Q8_0_ELEMS",
                          "const float d = oracle_fp16_to_f32((uint16_t)((blk[0] << 8) | blk[1]));\n            for (int t = 0; t < Q8_0_ELEMS"),
    "q8_0_q_unsigned": ("const int8_t q = (int8_t)blk[2 + t];", "const int q = (uint8_t)blk[2 + t];"),
    "q4k_nibbles_swapped": ("q = qs[32 * p + u] & 0x0f;", "q = qs[32 * p + u] >> 4;"),
    "q4k_nibbles_interleaved": ("const int p = e / 64, u = e % 64;", "const int p = (e / 2) / 64 * 0 + e / 64, u = (e % 2) * 32 + (e % 64) / 2;"),
    "q4k_subblock_index": ("sub = 2 * p + 1;", "sub = 2 * p;"),
    "q4k_min_sign": ("out[i * n_in + k * Q4K_ELEMS + e] = a - b;", "out[i * n_in + k * Q4K_ELEMS + e] = a + b;"),
    "q4k_min_dropped": ("out[i * n_in + k * Q4K_ELEMS + e] = a - b;", "out[i * n_in + k * Q4K_ELEMS + e] = a - 0.0f * b;"),
    "q4k_scale_high_bits_from_wrong_byte": ("((s[j - 4] >> 6) << 4)", "((s[j] >> 6) << 4)"),
    "q4k_mins_low_from_scale_bytes": ("m[j] = s[j + 4] & 63;", "m[j] = s[j] & 63;"),
    "q4k_dmin_offset": ("load_le16(blk + 2)", "load_le16(blk)"),
    "gemv_ignores_batch_row": ("(double)x[b * n_in + j];", "(double)x[j];"),
    "gemv_transposed_weight": ("(double)W[i * n_in + j]", "(double)W[(j * n_out + i) % (n_out * n_in)]"),
    "s_without_abs": ("sa += fabs(p);", "sa += p;"),
    "residual_dropped": ("out[k] += (double)residual[k];", "out[k] += 0.0 * residual[k];"),
    "silu_wrong_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "swiglu_operands_swapped": ("if (out) out[k] = oracle_silu(gg[k]) * uu[k];", "if (out) out[k] = oracle_silu(uu[k]) * gg[k];"),
    "qkv_k_reads_q": ("oracle_q8_0_gemv(wk, n_in, n_kv", "oracle_q8_0_gemv(wq, n_in, n_kv"),
    "fp16_bias": ("ldexpf((float)(1024 + f), e - 25)", "ldexpf((float)(1024 + f), e - 24)"),
    "fp16_subnormal_scale": ("ldexpf((float)f, -24)", "ldexpf((float)f, -25)"),
    "topk_ties_larger_index_first": ("return (a->i < b->i) ? -1 : (a->i > b->i);", "return (a->i > b->i) ? -1 : (a->i < b->i);"),
    "topk_smallest_first": ("if (a->v > b->v) return -1;\n    if (a->v < b->v) return 1;", "if (a->v < b->v) return -1;\n    if (a->v > b->v) return 1;"),
    "q6k_high_bits_shift": ("const int hi = (qh[32 * h + l] >> (2 * j)) & 3;", "const int hi = (qh[32 * h + l] >> j) & 3;"),
    "q6k_scale_index": ("(float)sc[8 * h + 2 * j + l / 16]", "(float)sc[8 * h + 2 * j]"),
    "q6k_no_offset": ("* (float)(q - 32);", "* (float)q;"),
    "q6k_ql_halves_swapped": ("ql[64 * h + 32 * (j % 2) + l]", "ql[64 * h + 32 * (j / 2) + l]"),
    "rope_rotation_sign": ("x[h * d + 2 * i] = a * c - b * s;", "x[h * d + 2 * i] = a * c + b * s;"),
    "rope_angle_exponent": ("pow(base, -2.0 * (double)i / (double)d)", "pow(base, -1.0 * (double)i / (double)d)"),
    "rope_pairs_split_halves": ("const double a = x[h * d + 2 * i], b = x[h * d + 2 * i + 1];", "const double a = x[h * d + i], b = x[h * d + i + d / 2];"),
    "attention_gqa_mapping": ("const int64_t kv = h / group;", "const int64_t kv = h % n_kv;"),
    "attention_scale_dropped": ("s[t] = scale * dot;", "s[t] = dot;"),
    "attention_off_by_one_context": ("for (int64_t t = 0; t < n_ctx; ++t) {\n            double dot", "for (int64_t t = 0; t + 1 < n_ctx; ++t) {\n            double dot"),
    "rmsnorm_sum_not_mean": ("const double r = 1.0 / sqrt(ss / (double)n + eps);", "const double r = 1.0 / sqrt(ss + eps);"),
    "rmsnorm_eps_outside_root": ("const double r = 1.0 / sqrt(ss / (double)n + eps);", "const double r = 1.0 / (sqrt(ss / (double)n) + eps);"),
    "rmsnorm_weight_dropped": ("out[b * n + j] = (double)x[b * n + j] * r * (double)w[j];", "out[b * n + j] = (double)x[b * n + j] * r;"),
    "topk_off_by_one": ("val[b * k + r] = it[r].v;", "val[b * k + r] = it[r + (r + 1 < n)].v;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutated = src.replace(old, new, 1)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "mutant.so"
    c_path.write_text(mutated)
    subprocess.run(["gcc", *oracle.CFLAGS, "-o", str(so_path), str(c_path), "-lm"], check=True)
    env = dict(os.environ, QDEC_ORACLE_LIB=str(so_path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the oracle pins"


# Mistakes planted in the numpy helpers of oracle/__init__.py (the f64-input
# products the chained-layer and full-size batched parity tests use).  The pins
# run in a copy of the oracle, synth and test files with the helper mutated,
# against the unmodified C library.
PY_MUTANTS = {
    "f64_gemv_s_without_abs": ("return y @ deq.T, np.abs(y) @ np.abs(deq).T",
                               "return y @ deq.T, np.abs(y @ deq.T)"),
    "f64_gemv_input_rows_reversed": ("return y @ deq.T, np.abs(y) @ np.abs(deq).T",
                                     "return y[::-1] @ deq.T, np.abs(y) @ np.abs(deq).T"),
    "f64_swiglu_operands_swapped": ("silu_g = g / (1.0 + np.exp(-g))",
                                    "silu_g = u / (1.0 + np.exp(-u)); u = g"),
    "f64_swiglu_silu_sign": ("silu_g = g / (1.0 + np.exp(-g))", "silu_g = g / (1.0 + np.exp(g))"),
    "f64_swiglu_sigmoid_only": ("silu_g = g / (1.0 + np.exp(-g))", "silu_g = 1.0 / (1.0 + np.exp(-g))"),
    "f64_swiglu_s_swapped": ('"Sg": sg, "Su": su', '"Sg": su, "Su": sg'),
    "f64_dense_transposed_weight": ("return y @ wd.T, np.abs(y) @ np.abs(wd).T",
                                    "return y @ wd.reshape(n_in, n_out), np.abs(y) @ np.abs(wd).T"),
    "f64_dense_s_without_abs": ("return y @ wd.T, np.abs(y) @ np.abs(wd).T",
                                "return y @ wd.T, np.abs(y @ wd.T)"),
}


def _run_pins_on_copy(tmp_path, helper_src):
    """Copy the oracle (with `helper_src` as its Python module), synth and the
    pin tests into tmp_path and run the pins there; returns pytest's exit code."""
    import shutil
    (tmp_path / "oracle").mkdir()
    (tmp_path / "oracle" / "__init__.py").write_text(helper_src)
    shutil.copy(SRC, tmp_path / "oracle" / "oracle.c")
    shutil.copytree(os.path.join(ROOT, "synth"), tmp_path / "synth",
                    ignore=shutil.ignore_patterns("__pycache__"))
    (tmp_path / "tests").mkdir()
    for f in ("conftest.py", "test_oracle.py", "helpers.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp_path / "pytest.ini")
    env = dict(os.environ, QDEC_ORACLE_LIB=oracle.build())
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        str(tmp_path / "tests" / "test_oracle.py")],
                       cwd=str(tmp_path), env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def test_python_helper_copy_passes_unmutated(tmp_path):
    """Control: the copied tree passes the pins, so a failure below comes from
    the planted mistake and not from the copy."""
    rc, out = _run_pins_on_copy(tmp_path, open(os.path.join(ROOT, "oracle", "__init__.py")).read())
    assert rc == 0, out


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_pins_reject_python_helper_mutant(name, tmp_path):
    old, new = PY_MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "__init__.py")).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    rc, out = _run_pins_on_copy(tmp_path, src.replace(old, new, 1))
    # exit code 1: a pin failed (2 would be a collection error, not a rejection)
    assert rc == 1, f"mutant {name} survived the oracle pins (rc {rc}):\n{out}"
