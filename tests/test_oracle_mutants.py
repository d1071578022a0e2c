"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's C source (a
dropped term, a wrong sign or index, a transposed operand, a wrong tie rule),
compiles it to a scratch library and runs every pin against it. The pins are
only trusted if each planted mistake makes at least one of them fail.
"""
import os

import pytest

import oracle_pins
from oracle import oracle as oracle_mod

# (name, exact text in eta_oracle.c, replacement) -- every occurrence is replaced.
MUTANTS = [
    ("gate_sign", "exp(-x)", "exp(x)"),
    ("gate_drops_beta", "double x = beta * (S - tau);", "double x = (S - tau);"),
    ("gate_threshold_sign", "double x = beta * (S - tau);", "double x = beta * (S + tau);"),
    ("gating_additive", "double Sg = S * eta_oracle_gate(", "double Sg = S + eta_oracle_gate("),
    ("gating_replaces_logit", "double Sg = S * eta_oracle_gate(", "double Sg = 0 * S + eta_oracle_gate("),
    ("hard_gate_strict", "return (S >= tau) ? 1.0 : 0.0;", "return (S > tau) ? 1.0 : 0.0;"),
    ("prob_bound_drops_scale", "double u_prob = s * (qc + z * qn * sqrt(var[blk]));",
     "double u_prob = (qc + z * qn * sqrt(var[blk]));"),
    ("prob_bound_no_sqrt", "z * qn * sqrt(var[blk])", "z * qn * var[blk]"),
    ("prob_bound_minus_z", "qc + z * qn", "qc - z * qn"),
    ("prob_bound_drops_qnorm", "z * qn * sqrt(var[blk])", "z * sqrt(var[blk])"),
    ("bound_takes_max", "(u_prob < u_geo) ? u_prob : u_geo", "(u_prob > u_geo) ? u_prob : u_geo"),
    ("geo_bound_drops_qnorm", "double u_geo = s * qn * maxnorm[blk];", "double u_geo = s * maxnorm[blk];"),
    ("centroid_index_transposed", "centroid[(long)blk * d + i]", "centroid[(long)i * nblk + blk]"),
    ("screen_strict", "if (U[blk] >= tau) idx[cnt++] = blk;", "if (U[blk] > tau) idx[cnt++] = blk;"),
    ("var_missing_dim", "var[blk] = sq / (n * (double)d);", "var[blk] = sq / n;"),
    ("var_sample_form", "var[blk] = sq / (n * (double)d);", "var[blk] = sq / ((n - 1.0) * (double)d);"),
    ("centroid_full_block_divisor", "c[i] /= n;", "c[i] /= (double)bs;"),
    ("maxnorm_squared", "double norm = sqrt(norm2);", "double norm = norm2;"),
    ("predict_transposed_W", "double wv = (double)W[row * H + h];",
     "double wv = (double)W[(long)h * H * d + row];"),
    ("predict_drops_bias", "double acc = (double)bias[h];", "double acc = 0.0;"),
    ("predict_wrong_query_head", "double qv = (double)q[((long)b * H + g) * d + i];",
     "double qv = (double)q[((long)b * H + h) * d + i];"),
    ("lse_drops_max", "*lse = mu + log(l);", "*lse = log(l);"),
    ("reads_past_T", "if (t1 > T) t1 = T;", ""),
    ("no_logit_scale", "double s = 1.0 / sqrt((double)d);", "double s = 1.0;"),
    ("bf16_wrong_shift", "((uint32_t)bits) << 16", "((uint32_t)bits) << 15"),
    ("empty_lse_zero", "*lse = -INFINITY;", "*lse = 0.0;"),
    ("value_uses_key", "out[i] += p * kv_at(V,", "out[i] += p * kv_at(K,"),
    ("no_normalisation", "for (int i = 0; i < d; ++i) out[i] /= l;", ""),
    ("union_first_list_only", "for (int j = 0; j < g && !hit; ++j)", "for (int j = 0; j < 1 && !hit; ++j)"),
    ("union_wrong_row_stride", "if (lists[(long)j * stride + a] == blk) hit = 1;",
     "if (lists[(long)j * g + a] == blk) hit = 1;"),
    ("prefill_window_short", "int n = T_k - T_q + t + 1; /* visible keys */",
     "int n = T_k - T_q + t; /* visible keys */"),
    ("prefill_window_top_left", "int n = T_k - T_q + t + 1; /* visible keys */",
     "int n = t + 1; /* visible keys */"),
    ("gate_sum_counts_keys", "gs += eta_oracle_gate(s * dot, tau[t], gate_beta, gate_hard);",
     "gs += 1.0;"),
    ("gate_sum_unscaled", "gs += eta_oracle_gate(s * dot, tau[t], gate_beta, gate_hard);",
     "gs += eta_oracle_gate(dot, tau[t], gate_beta, gate_hard);"),
    ("union_skips_first_head", "for (int j = 0; j < g && !hit; ++j)", "for (int j = 1; j < g && !hit; ++j)"),
    ("maxdev_from_origin", "double dev = kv_at(K, kv_dtype, d, t, i) - c[i];",
     "double dev = kv_at(K, kv_dtype, d, t, i);"),
    ("maxdev_squared", "double dist = sqrt(dist2);", "double dist = dist2;"),
    ("centered_drops_qnorm", "double u_cen = s * (qc + qn * maxdev[blk]);",
     "double u_cen = s * (qc + maxdev[blk]);"),
    ("centered_minus", "qc + qn * maxdev[blk]", "qc - qn * maxdev[blk]"),
    ("centered_takes_max", "(u_cen < u_geo) ? u_cen : u_geo", "(u_cen > u_geo) ? u_cen : u_geo"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle_mod.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, source, name, old, new):
    assert old in source, f"mutation anchor for {name} not found in the oracle source"
    src = tmp_path / "mutant.c"
    src.write_text(source.replace(old, new))
    lib = oracle_mod.compile_oracle(str(src), str(tmp_path / f"lib_{name}.so"))
    O = oracle_mod.OracleLib(lib)
    failed = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(O)
        except AssertionError:
            failed.append(check.__name__)
        except (ValueError, FloatingPointError, ZeroDivisionError, OverflowError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} survived every pin"
    os.remove(lib)
