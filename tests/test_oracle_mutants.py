"""The pins must catch plausible mistakes in the oracle.

Each case rebuilds the oracle from its source with one deliberate slip (a
dropped rescale, a wrong rounding rule, a wrong tie-break, a transposed
index, ...) into a temporary library, runs the pin suites against it in a
subprocess, and requires them to fail.  The shipped oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "thrift_oracle.c")

MUTANTS = {
    "no_rescale": ("acc[d] = alpha * acc[d] + w * pv;", "acc[d] = acc[d] + w * pv;"),
    # level 1 of the two-level P quantisation taken as an integer (a power of
    # two, which E8M0 absorbs) instead of the tile maximum
    "mx_level1_integer": ("v[c] = mask[c] ? 0.0 : top * exp2(t[c] - mt);",
                          "v[c] = mask[c] ? 0.0 : top * exp2(t[c] - (prec == THO_PATH_MX4 ? ceil(mt) : mt)) * "
                          "(prec == THO_PATH_MX4 ? exp2(ceil(mt) - mt) : 1.0);"),
    # FP16-path probabilities rounded on a power-of-two footing
    "fp16_level1_integer": ("pq[c] = mask[c] ? 0.0 : tho_round_to_half(exp2(t[c] - mt));",
                            "pq[c] = mask[c] ? 0.0 : tho_round_to_half(exp2(t[c] - ceil(mt))) * exp2(ceil(mt) - mt);"),
    "level1_weight_dropped": ("double w = exp2(mt - m_new);", "double w = exp2(ceil(mt) - m_new);"),
    "topk_ascending": ("const tho_cand* y = (const tho_cand*)b;\n  if (x->s > y->s) return -1;",
                       "const tho_cand* y = (const tho_cand*)b;\n  if (x->s > y->s) return 1;"),
    "head_budget_ascending": ("const tho_pair* y = (const tho_pair*)b;\n  if (x->s > y->s) return -1;",
                              "const tho_pair* y = (const tho_pair*)b;\n  if (x->s > y->s) return 1;"),
    "decode_start_aligned": ("int qpos = Sk - S + r; /* the query's", "int qpos = r; /* the query's"),
    "decode_valid_blocks_start_aligned": ("return (Sk - Sq + last_q) / bk + 1;", "return last_q / bk + 1;"),
    "e2m1_ties_up": ("if (a > t || (a == t && ((k + 1) & 1) == 0)) code = k + 1;",
                     "if (a >= t) code = k + 1;"),
    "rowsum_quantised": ("if (!mask[c]) psum += exp2(t[c] - m_new);", "if (!mask[c]) psum += pq[c] * w;"),
    "causal_off_by_one": ("mask[c] = a->causal && (c0 + c > qpos);", "mask[c] = a->causal && (c0 + c >= qpos);"),
    "v_transposed_index": ("e = ((size_t)bh * D + d) * Sp + s;", "e = ((size_t)bh * D + (s % D)) * Sp + d;"),
    "mean_divides_by_block": ("(float)(sum / (double)(r1 - r0));", "(float)(sum / (double)blk);"),
    "e4m3_no_saturation_tie": ("if (num > t || (num == t && ((k + 1) & 1) == 0))",
                               "if (num > t || (num == t && ((k + 1) & 1) == 1))"),
    "nvfp4_level1_scale": ("double top = prec == THO_PATH_NV4 ? 2688.0 : 1.0;",
                           "double top = prec == THO_PATH_NV4 ? 448.0 : 1.0;"),
    "head_budget_ties_late_block_first": ("if (x->i != y->i) return x->i - y->i;",
                                          "if (x->i != y->i) return y->i - x->i;"),
    "head_budget_floor": ("(P * topk_bp + 9999) / 10000", "(P * topk_bp) / 10000"),
    "gqa_head_map": ("int hk = hq / (a->Hq / a->Hkv);\n  int nq = tho_cdiv(S, a->bq);\n  int qpos",
                     "int hk = hq % a->Hkv;\n  int nq = tho_cdiv(S, a->bq);\n  int qpos"),
    # the lists of decisions that may go either way
    "eval_bound_scaled": ("return rel * (1.0 + 0x1p-10);", "return 4.0 * rel * (1.0 + 0x1p-10);"),
    "flip_sign": ("dp[c] = alt * s2 / (prec == THO_PATH_NV4 ? 2688.0 : 1.0) - pq[c];",
                  "dp[c] = pq[c] - alt * s2 / (prec == THO_PATH_NV4 ? 2688.0 : 1.0);"),
    "flips_skip_fp16": ("      dp[c] = alt[k] - pq[c];\n      nf = tho_add_flip", "      dp[c] = 0.0;\n      nf = tho_add_flip"),
    # backward (Attn-QAT)
    "bwd_dv_exact_p": ("dv[key * D + d] += pt[c] * dor[d];", "dv[key * D + d] += p[c] * dor[d];"),
    "bwd_ds_quantised_p": ("          double dS = p[c] * (dP - Dr);\n          for (int d = 0; d < D; ++d) g[d]",
                           "          double dS = pt[c] * (dP - Dr);\n          for (int d = 0; d < D; ++d) g[d]"),
    "bwd_no_row_term": ("Dr += dor[d] * ohp[row * D + d];", "Dr += 0.0 * ohp[row * D + d];"),
    "bwd_fp16_query_on_fp4_pairs": ("const double* qv = kind[c] == 1 ? q4 : qh;", "const double* qv = qh;"),
    "bwd_dk_unscaled": ("dk[key * D + d] += sm_scale * dS * qv[d];", "dk[key * D + d] += dS * qv[d];"),
    "bwd_one_head_per_key_head": ("for (int hq = hk * G; hq < (hk + 1) * G; ++hq)",
                                  "for (int hq = hk; hq < hk + 1; ++hq)"),
    # middle (FP8) tier
    "fp8_exponent_offset": ("int x = (e - 1) - 8;", "int x = (e - 1) - 7;"),
    "fp8_tier_recomputes_fp16_blocks": ("      if (in16) continue;\n      prec = THO_PATH_F8;",
                                        "      prec = THO_PATH_F8;"),
    "fp8_tier_uses_fp4_query": ("mt = tho_tile_scores(a, q8, a->k8", "mt = tho_tile_scores(a, q4, a->k8"),
    "fp8_tier_p_quantised_as_fp4": ("  if (prec == THO_PATH_F8) return tho_e4m3_value(tho_e4m3_encode_ratio(v, s2)) * s2;",
                                    "  if (prec == THO_PATH_F8) return tho_e2m1_value(tho_e2m1_encode(v, s2)) * s2;"),
    "fp4_pass_keeps_fp8_blocks": ("        ++sp2;\n        listed = 1;", "        ++sp2;\n        listed = 0;"),
    "fp8_v_not_transposed": ("e = (size_t)bh * D * Sp + (size_t)d * Sp + s;", "e = (size_t)bh * D * Sp + (size_t)s * D + d;"),
    "ohp_from_quantised_p": ("if (!mask[c]) hv += exp2(t[c] - m_new) * vt[(size_t)c * D + d];",
                             "if (!mask[c]) hv += w * pq[c] * vt[(size_t)c * D + d];"),
}


# mutant name prefix -> the pin file aimed at that part of the oracle
FIRST = [("fp8_", "tests/test_oracle_fp8.py"), ("fp4_pass_keeps_fp8", "tests/test_oracle_fp8.py"),
         ("bwd_", "tests/test_oracle_backward.py"), ("ohp_", "tests/test_oracle_backward.py"),
         ("head_budget", "tests/test_oracle_select_head.py"), ("decode_", "tests/test_oracle_decode.py"),
         ("no_rescale", "tests/test_oracle_attention.py"), ("causal_", "tests/test_oracle_attention.py"),
         ("rowsum_", "tests/test_oracle_attention.py"), ("mx_level1", "tests/test_oracle_attention.py"),
         ("nvfp4_level1", "tests/test_oracle_attention.py"), ("gqa_", "tests/test_oracle_attention.py"),
         ("fp16_level1", "tests/test_oracle_attention.py"), ("level1_", "tests/test_oracle_attention.py"),
         ("eval_", "tests/test_oracle_attention.py"), ("flip", "tests/test_oracle_attention.py")]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mut = tmp_path / "thrift_oracle.c"
    mut.write_text(src.replace(old, new))
    sys.path.insert(0, ROOT)
    from oracle import build_oracle

    lib = build_oracle.build(src=str(mut), out=str(tmp_path / "libmut.so"))
    env = dict(os.environ, THRIFT_ORACLE_LIB=lib)
    files = ["tests/test_oracle_formats.py", "tests/test_oracle_select.py", "tests/test_oracle_attention.py",
             "tests/test_oracle_decode.py", "tests/test_oracle_select_head.py", "tests/test_oracle_backward.py",
             "tests/test_oracle_fp8.py"]
    # every pin file runs; the one aimed at the mutated part first, so that -x stops early
    first = next((f for pre, f in FIRST if name.startswith(pre)), None)
    if first:
        files.remove(first)
        files.insert(0, first)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + files,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
