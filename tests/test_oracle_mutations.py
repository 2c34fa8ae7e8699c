"""Plant a plausible mistake in a copy of the oracle (CPU only) and require
that at least one pin catches it.  This checks the pins, not the oracle."""
import os
import subprocess

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, text in oracle.c, replacement)
MUTATIONS = [
    ("scale_without_sqrt", "1.0 / sqrt((double)dk)", "1.0 / (double)dk"),
    ("causal_drops_diagonal", "if (causal && j > i)", "if (causal && j >= i)"),
    ("valid_len_off_by_one", "!(j < valid_lens[b])", "!(j <= valid_lens[b])"),
    ("fill_added_not_replaced", "s[j] = ORACLE_MASK_FILL;", "s[j] += ORACLE_MASK_FILL;"),
    ("fill_too_small", "#define ORACLE_MASK_FILL (-1e9)", "#define ORACLE_MASK_FILL (-1e1)"),
    ("weight_transposed", "acc += x[m * Din + c] * w[(long)n * Din + c];",
     "acc += x[m * Din + c] * w[(long)c * Dout + n];"),
    ("bias_dropped", "acc + (b ? b[n] : 0.0)", "acc"),
    ("head_split_interleaved",
     "Qf[((long)b * R + r) * D + hd * dk + t]", "Qf[((long)b * R + r) * D + t * h + hd]"),
    ("head_merge_interleaved",
     "ocat[((long)b * R + r) * D + hd * dk + t]", "ocat[((long)b * R + r) * D + t * h + hd]"),
    ("value_index_transposed", "v[(long)j * dv + t]", "v[(long)t * Lk + j]"),
    ("softmax_not_normalised", "s[j] /= den;", "s[j] /= (den > 1.0 ? 1.0 : den);"),
    ("bf16_ties_away", "(fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0", "fl + 1.0"),
    ("bf16_merge_not_rounded", "if (bf16_stages) round_all(ocat, (long)B * R * D);",
     "if (0) round_all(ocat, (long)B * R * D);"),
    ("mha_backward_merge_not_rounded", "if (bf16_stages) round_all(ocat, Mq * D);", "if (0) round_all(ocat, Mq * D);"),
    ("mask_uses_query_length", "if (valid_lens && !(j < valid_lens[b]))",
     "if (valid_lens && !(i < valid_lens[b]))"),
    ("per_query_length_rows_reversed", "valid_lens[(long)b * Lq + i]", "valid_lens[(long)b * Lq + (Lq - 1 - i)]"),
    ("backward_dq_without_scale", "dqb[(long)i * dk_ + t] += tau * ds", "dqb[(long)i * dk_ + t] += ds"),
    ("backward_rowsum_unweighted", "rowsum += p[j] * dp[j];", "rowsum += dp[j];"),
    ("backward_dv_uses_ds", "dvb[(long)j * dv_ + t] += p[j] * gi[t];", "dvb[(long)j * dv_ + t] += dp[j] * gi[t];"),
    ("backward_masked_pairs_propagate",
     "if (!key_allowed(valid_lens, vl_per_query, Lq, causal, b, i, j)) continue;", ""),
    ("layer_norm_biased_std_for_kind0", "den = sqrt(ss / (D - 1)) + eps;", "den = sqrt(ss / D) + eps;"),
    ("layer_norm_eps_inside_root_for_kind0", "den = sqrt(ss / (D - 1)) + eps;", "den = sqrt(ss / (D - 1) + eps);"),
    ("layer_norm_eps_outside_root_for_kind1", "else den = sqrt(ss / D + eps);", "else den = sqrt(ss / D) + eps;"),
    ("per_query_length_ignores_query", "valid_lens[(long)b * Lq + i]", "valid_lens[(long)b * Lq]"),
    ("lse_drops_the_max", "lse[bh * (long)Lq + i] = mx + log(den);", "lse[bh * (long)Lq + i] = log(den);"),
    ("lse_in_log2", "lse[bh * (long)Lq + i] = mx + log(den);", "lse[bh * (long)Lq + i] = mx + log2(den);"),
    ("linear_backward_dw_wrong_output_feature", "const double a = dy[r * Dout + n];", "const double a = dy[r * Dout + (n + 1) % Dout];"),
    ("linear_backward_dx_uses_w_transposed", "acc[c] += a * w[(long)n * Din + c];",
     "acc[c] += a * w[(long)c * Dout + n];"),
    ("linear_backward_bias_first_row_only", "bsum += a;", "bsum += (r == 0) ? a : 0.0;"),
    ("mha_backward_value_path_overwrites_key_path", "linear_backward(dV, xkv, w_v, dxkv, dw_v, db_v, Mk, D, D, 1);",
     "linear_backward(dV, xkv, w_v, dxkv, dw_v, db_v, Mk, D, D, 0);"),
    ("mha_backward_heads_interleaved", "double* r = rows + ((long)b * L + l) * h * dk + hd * dk + t;",
     "double* r = rows + ((long)b * L + l) * h * dk + t * h + hd;"),
    ("mha_backward_merged_head_gradient_not_rounded", "if (bf16_stages) round_all(docat, Mq * D);",
     "if (0) round_all(docat, Mq * D);"),
    ("mha_backward_query_gradient_not_rounded", "round_all(dQ, Mq * D);", ""),
]


def _first_failing_pin():
    for pin in ALL_PINS:
        try:
            pin()
        except AssertionError:
            return pin.__name__
    return None


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique in oracle.c"
    src = tmp_path / "oracle_mut.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", str(src), "-o", str(lib), "-lm"], check=True)
    with oracle.use_library(str(lib)):
        caught = _first_failing_pin()
    assert caught is not None, f"no pin detects the planted mistake {name}"
