"""Plant plausible mistakes in copies of the oracle; each must fail at least one pin.

This shows that the pins constrain every step of the oracle: a dropped term,
a wrong sign, a wrong index, a transposed operand or a wrong mask bound in
any of its functions is caught.  The mutants are built from the oracle's C
source by text substitution into a temporary directory; the real oracle is
untouched.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = [
    ("drop_scale", "s[j] = a->scale * acc;", "s[j] = acc;"),
    ("exp_sign", "s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    ("no_max_shift", "s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    ("no_normalise", "s[j] = s[j] / l;", "s[j] = s[j];"),
    ("lse_without_max", "a->LSE[out_idx] = m + log(l);", "a->LSE[out_idx] = log(l);"),
    ("head_map_modulo", "const int64_t g = h / (a->H / a->H_kv);", "const int64_t g = h % a->H_kv;"),
    ("causal_top_left", "int64_t last = i + a->N_k - a->N_q;", "int64_t last = i;"),
    ("causal_off_by_one", "int64_t last = i + a->N_k - a->N_q;", "int64_t last = i + a->N_k - a->N_q - 1;"),
    ("scores_use_V", "widen(a->K, a->dtype, k_off + k)", "widen(a->V, a->dtype, k_off + k)"),
    ("output_uses_K", "widen(a->V, a->dtype, v_off + k)", "widen(a->K, a->dtype, v_off + k)"),
    ("max_skips_first", "for (int64_t j = j_beg + 1; j < j_end; ++j)\n        if (s[j] > m) m = s[j];",
     "for (int64_t j = j_beg + 2; j < j_end; ++j)\n        if (s[j] > m) m = s[j];"),
    ("batch_ignored_kv", "const int64_t kv_head = (b * a->H_kv + g) * a->N_k;", "const int64_t kv_head = g * a->N_k;"),
    ("online_no_acc_rescale", "for (int64_t k = 0; k < d; ++k) acc[k] *= alpha;", ""),
    ("online_alpha_inverted", "exp(m - m_new);", "exp(m_new - m);"),
    ("online_l_not_rescaled", "l *= alpha;", ""),
    ("merge_weight_without_l", "double wb = (m_b == -INFINITY) ? 0.0 : l_b * exp(m_b - m);",
     "double wb = (m_b == -INFINITY) ? 0.0 : exp(m_b - m);"),
    ("merge_max_is_min", "double m = m_a > m_b ? m_a : m_b;", "double m = m_a < m_b ? m_a : m_b;"),
    ("combine_weight_uses_max", "double w = exp(lse_s[t] - lse);", "double w = exp(lse_s[t] - M);"),
    ("combine_lse_without_max", "double lse = M + log(sum);", "double lse = log(sum);"),
    ("bwd_drop_D", "const double ds = p[j] * (dp[j] - Di);", "const double ds = p[j] * dp[j];"),
    ("bwd_dS_sign", "const double ds = p[j] * (dp[j] - Di);", "const double ds = p[j] * (Di - dp[j]);"),
    ("bwd_dq_no_scale", "dq[k] += a->scale * ds *", "dq[k] += ds *"),
    ("bwd_dk_uses_dO", "dK[j * d + k] += a->scale * ds * widen(a->Q, a->dtype, q_off + k);",
     "dK[j * d + k] += a->scale * ds * widen(a->dO, a->dtype, q_off + k);"),
    ("bwd_dv_uses_dS", "dV[j * d + k] += p[j] * widen(a->dO", "dV[j * d + k] += ds * widen(a->dO"),
    ("bwd_dp_uses_K", "acc += widen(a->dO, a->dtype, q_off + k) * widen(a->V, a->dtype, (kv_head + j) * d + k);",
     "acc += widen(a->dO, a->dtype, q_off + k) * widen(a->K, a->dtype, (kv_head + j) * d + k);"),
    ("bwd_causal_ignored", "        if (a->causal) {\n                int64_t last = i + N_k - N_q;", "        if (0) {\n                int64_t last = i + N_k - N_q;"),
    ("bwd_no_max_shift_unnormalised", "for (int64_t j = 0; j < j_end; ++j) p[j] /= l;", ""),
    ("e4m3_ties_away", "double m8 = nearbyint(ldexp(a, 3 - e)) - 8.0;", "double m8 = round(ldexp(a, 3 - e)) - 8.0;"),
    ("e4m3_subnormal_step", "double q = nearbyint(ldexp(a, 9));", "double q = nearbyint(ldexp(a, 10));"),
    ("e4m3_saturates", "if (isnan(x) || a > 464.0) return (uint8_t)(sign | 0x7F);",
     "if (isnan(x) || a > 464.0) return (uint8_t)(sign | 0x7E);"),
    ("fwht_sign_swapped", "x[i + len] = a - b;", "x[i + len] = b - a;"),
    ("fwht_stage_skipped", "for (int64_t len = 1; len < d; len <<= 1)", "for (int64_t len = 2; len < d; len <<= 1)"),
    ("fp8_sign_hi_ignored", "(int)((sign_hi >> (j - 64)) & 1u)", "(int)((sign_lo >> (j - 64)) & 1u)"),
    ("fp8_no_post_scale", "(amax / 448.0f) * post_scale", "(amax / 448.0f)"),
    ("fp8_fnuz_max", "448.0f / amax", "240.0f / amax"),
    ("fp8_amax_first_row", "for (int64_t j = 0; j < d; ++j)\n                    if (fabsf(x[j]) > amax) amax = fabsf(x[j]);",
     "for (int64_t j = 0; j < d; ++j)\n                    if (r == r0 && fabsf(x[j]) > amax) amax = fabsf(x[j]);"),
]


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, find, repl):
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(find) >= 1, "mutation anchor not found: %r" % find
    mutated = src.replace(find, repl, 1)
    path = tmp_path / ("oracle_%s.c" % name)
    path.write_text(mutated)
    lib = oracle.compile_library(str(path), str(tmp_path / ("liboracle_%s.so" % name)))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, "mutant %s passed every pin" % name
