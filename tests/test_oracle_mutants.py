"""The oracle's pins against planted mistakes.

Each case copies oracle/oracle.c, plants one plausible mistake (a dropped
term, a wrong sign, index or bias, a transposed operand, an off-by-one),
builds the copy with the same gcc flags, and runs the pins of the affected
functions against it in a fresh process (ATTN_ORACLE_LIB points the oracle
package at the copy).  The pins must fail.  Nothing here touches the GPU or
the HIP library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, occurrence to replace (0 = first), pin files)
MUTANTS = [
    ("gqa_scale_dropped", "z[t] = scale * acc;", "z[t] = acc;", 0, ["test_oracle_gqa.py"]),
    ("gqa_head_map", "j = i / g;", "j = i % h_kv;", 0, ["test_oracle_gqa.py"]),
    ("gqa_lse_without_log", "if (lse) lse[r] = m + log(l);", "if (lse) lse[r] = m;", 0,
     ["test_oracle_gqa.py"]),
    ("gqa_max_not_subtracted", "p[t] = exp(z[t] - m);", "p[t] = exp(z[t]);", 0,
     ["test_oracle_gqa.py"]),
    ("mla_rope_term_dropped", "z[t] = scale * (acc + accr);", "z[t] = scale * acc;", 0,
     ["test_oracle_mla.py"]),
    ("mla_w_uv_transposed", "acc += ld(w_uv, ((size_t)i * d_v + e) * d_c + c, b) * ut[c];",
     "acc += ld(w_uv, ((size_t)i * d_c + c) * d_v + e, b) * ut[c];", 0, ["test_oracle_mla.py"]),
    ("mla_w_uk_transposed", "ld(w_uk, ((size_t)i * d_nope + e) * d_c + c, b)",
     "ld(w_uk, ((size_t)i * d_c + c) * d_nope + e, b)", 0, ["test_oracle_mla.py"]),
    ("multi_visible_off_by_one", "const int n = sb - (q_len - 1 - jq);",
     "const int n = sb - (q_len - jq);", 0, ["test_oracle_multi.py"]),
    ("mla_multi_visible_off_by_one",
     "const int n = sb - q_len + 1 + jq > 0 ? sb - q_len + 1 + jq : 0;",
     "const int n = sb - q_len + jq > 0 ? sb - q_len + jq : 0;", 0, ["test_oracle_mla_multi.py"]),
    ("mla_multi_position_index", "const int jq = (int)((r / h) % q_len), i = (int)(r % h);",
     "const int jq = (int)(r % q_len), i = (int)(r % h);", 0, ["test_oracle_mla_multi.py"]),
    ("mla_output_head_interleaved", "ld(w_o, (size_t)n * hd + (size_t)i * d_v + e, b)",
     "ld(w_o, (size_t)n * hd + (size_t)e * h + i, b)", 0, ["test_oracle_mla_output.py"]),
    ("mla_output_w_o_transposed", "ld(w_o, (size_t)n * hd + (size_t)i * d_v + e, b)",
     "ld(w_o, ((size_t)i * d_v + e) * d_model + n, b)", 0, ["test_oracle_mla_output.py"]),
    ("mla_page_scale_by_logical_block", "    return (double)scales[blk];",
     "    return (double)scales[t / block_size];", 0, ["test_oracle_mla_fp8.py"]),
    ("mla_page_append_scales_swapped",
     "const float ic = 1.0f / c_scales[blk], ir = 1.0f / r_scales[blk];",
     "const float ic = 1.0f / r_scales[blk], ir = 1.0f / c_scales[blk];", 0,
     ["test_oracle_mla_fp8.py"]),
    ("merge_weight_sign", "const double w = exp((double)lse_parts[(size_t)k * rows + r] - M);",
     "const double w = exp(M - (double)lse_parts[(size_t)k * rows + r]);", 0,
     ["test_oracle_merge.py"]),
    ("fp8_exponent_bias", "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)",
     0, ["test_oracle_fp8.py"]),
    ("fp8_encode_truncates", "double mq = rint(a / quantum);", "double mq = floor(a / quantum);", 0,
     ["test_oracle_fp8.py"]),
    ("mla_fp8_scales_swapped", "e < d_c ? c_scale : r_scale", "e < d_c ? r_scale : c_scale", 0,
     ["test_oracle_mla_fp8.py"]),
    ("append_neighbour_element", "const float xk = (float)ld(k_new, (size_t)bb * n + e, 2);",
     "const float xk = (float)ld(k_new, (size_t)bb * n + (e ^ 1), 2);", 0,
     ["test_oracle_fp8.py"]),
    ("page_scale_by_logical_block", "const double ks = (double)k_scales[(size_t)blk * h_kv + j];",
     "const double ks = (double)k_scales[(size_t)(t / block_size) * h_kv + j];", 0,
     ["test_oracle_fp8.py"]),
    ("cell_factor_two_dropped", "return 2ULL * (unsigned long long)L", "return 1ULL * (unsigned long long)L",
     0, ["test_oracle_cells.py"]),
]


def plant(text, old, new, occurrence):
    at = -1
    for _ in range(occurrence + 1):
        at = text.index(old, at + 1)
    return text[:at] + new + text[at + len(old):]


@pytest.mark.parametrize("name,old,new,occ,files", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new, occ, files):
    src = open(SRC).read()
    assert old in src, f"{name}: target text not found in oracle.c"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(plant(src, old, new, occ))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                    "-ffp-contract=off", str(mutant), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ATTN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        *[os.path.join(ROOT, "tests", f) for f in files]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1 and "failed" in r.stdout, \
        f"{name}: the pins did not catch it\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"


def test_unmodified_copy_passes(tmp_path):
    # the same route with nothing planted: the failures above are the mistakes'
    lib = tmp_path / "liboracle_copy.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
                    "-ffp-contract=off", SRC, "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ATTN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_merge.py"),
                        os.path.join(ROOT, "tests", "test_oracle_multi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
