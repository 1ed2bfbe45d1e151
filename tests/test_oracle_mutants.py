"""Plants plausible mistakes in copies of the CPU oracle (on the CPU only) and
checks that the pins in test_oracle_pins.py, test_oracle_bwd_pins.py,
test_oracle_blocksparse_pins.py, test_oracle_paged_pins.py and
test_oracle_kvcache_pins.py catch every one of them."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fa_oracle.c")

MUTANTS = {
    "scale_dropped": ("prow[j] = scale * dot;", "prow[j] = dot;"),
    "causal_off_by_one": ("if (causal && j > i) return 0;", "if (causal && j >= i) return 0;"),
    "window_left_off_by_one": ("if (wl >= 0 && i - j > wl) return 0;", "if (wl >= 0 && i - j >= wl) return 0;"),
    "window_right_mirrored": ("if (wr >= 0 && j - i > wr) return 0;", "if (wr >= 0 && i - j > wr) return 0;"),
    "k_replaced_by_v": ("dot += Q[r * D + d] * K[j * D + d];", "dot += Q[r * D + d] * V[j * D + d];"),
    "no_normalisation": ("prow[j] /= l;", "prow[j] /= 1.0;"),
    "lse_without_max": ("lse_rows[r] = m + log(l);", "lse_rows[r] = log(l);"),
    "exp_sign_flipped": ("prow[j] = exp(prow[j] - m);", "prow[j] = exp(m - prow[j]);"),
    "head_seq_strides_swapped": ("((((b) * S + (s_)) * H + (h)) * D + (d_))",
                                 "((((b) * H + (h)) * S + (s_)) * D + (d_))"),
    "fp16_bias_off": ("mag = ldexp(1024.0 + (double)f, e - 25);", "mag = ldexp(1024.0 + (double)f, e - 24);"),
    "bf16_subnormal_off": ("mag = ldexp((double)f, -133);", "mag = ldexp((double)f, -134);"),
    "max_ignores_nan": ("if (isnan(prow[j])) {", "if (0) {"),
    # backward
    "bwd_no_row_term": ("grow[j] = prow[j] * (grow[j] - Di);", "grow[j] = prow[j] * grow[j];"),
    "bwd_dk_from_p": ("ak += dS[i * S + j] * Q[i * D + d];", "ak += P[i * S + j] * Q[i * D + d];"),
    "bwd_dq_unscaled": ("dqrow[d] = scale * acc;", "dqrow[d] = acc;"),
    "bwd_dv_from_v": ("av += P[i * S + j] * dO[i * D + d];", "av += P[i * S + j] * V[i * D + d];"),
    "bwd_dp_transposed": ("for (int64_t d = 0; d < D; ++d) dot += dO[i * D + d] * V[j * D + d];",
                          "for (int64_t d = 0; d < D; ++d) dot += dO[j * D + d] * V[i * D + d];"),
    "bwd_dk_unscaled": ("dkrow[d] = scale * ak;", "dkrow[d] = ak;"),
    # block-sparse factor
    "bs_mask_ignored": ("if (!mask) return 1;", "if (1) return 1;"),
    "bs_key_block_divisor": ("return mask[(i / block_m) * n_kb + j / block_n] != 0;",
                             "return mask[(i / block_m) * n_kb + j / block_m] != 0;"),
    "bs_row_stride": ("return mask[(i / block_m) * n_kb + j / block_n] != 0;",
                      "return mask[(i / block_m) * (n_kb - 1) + j / block_n] != 0;"),
    "bs_head_index": ("hm = b * H + h;", "hm = h * B + b;"),
    "bs_per_head_ignored": ("hm = h;", "hm = 0;"),
    # paged gather
    "paged_div_mod_swapped": ("const int64_t page = block_table[b * table_stride + j / page_size];",
                              "const int64_t page = block_table[b * table_stride + j % page_size];"),
    "paged_row_in_page": ("const int64_t src_row = page * page_size + j % page_size;",
                          "const int64_t src_row = page * page_size + j / page_size;"),
    "paged_table_stride": ("const int64_t page = block_table[b * table_stride + j / page_size];",
                           "const int64_t page = block_table[b * (S + page_size - 1) / page_size + j / page_size];"),
    # KV-cache forward
    "kv_top_left_alignment": ("const int64_t p = L - S_q + r; /* the query's position in its sequence */",
                              "const int64_t p = r; /* the query's position in its sequence */"),
    "kv_position_off_by_one": ("const int64_t p = L - S_q + r; /* the query's position in its sequence */",
                               "const int64_t p = L - S_q + r + 1; /* the query's position in its sequence */"),
    "kv_cache_stride": ("Kc[j * D + d] = orc_load(k, dtype, ((b * S_k + j) * H + h) * D + d);",
                        "Kc[j * D + d] = orc_load(k, dtype, ((b * S_q + j) * H + h) * D + d);"),
    "kv_mask_on_row_index": ("if (!orc_allowed(p, j, causal, wl, wr)) {\n                        srow[j] = -INFINITY;",
                             "if (!orc_allowed(r, j, causal, wl, wr)) {\n                        srow[j] = -INFINITY;"),
    "kv_scale_dropped": ("srow[j] = scale * dot;", "srow[j] = dot;"),
    "kv_no_normalisation": ("for (int64_t j = 0; j < L; ++j) srow[j] /= l;",
                            "for (int64_t j = 0; j < L; ++j) srow[j] /= 1.0;"),
    "kv_v_row_index": ("orow[d] += srow[j] * Vc[j * D + d];", "orow[d] += srow[j] * Vc[(L - 1 - j) * D + d];"),
    "kv_lse_without_max": ("*lrow = m + log(l);", "*lrow = log(l);"),
    "bs_only_in_scores": ("!orc_block_on(bmask, i, j, block_m, block_n, n_kb))\n                continue;",
                          "0)\n                continue;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found once: {old}"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", str(mpath), "-o",
                    str(lib), "-lm"], check=True)
    env = dict(os.environ, FA_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_bwd_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_blocksparse_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_paged_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_kvcache_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
