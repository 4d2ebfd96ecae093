"""Planted mistakes in the oracle must be caught by its pins.

Each case compiles a copy of the oracle's C source with one plausible mistake
(a dropped term, a wrong constant, a wrong index, a wrong sign), loads it in
place of the real oracle, and runs the pins expected to catch it.  At least
one of them must fail.  Everything runs on the CPU.
"""
import importlib
import os

import pytest

import oracle

# (name, text in kvq_oracle.c, replacement, [(test module, test function, kwargs)])
MUTANTS = [
    ("taylor_constant", "return tau * tau / 24.0 * b;", "return tau * tau / 12.0 * b;",
     [("test_oracle_bias", "test_taylor_exact_sandwich", {}),
      ("test_oracle_bias", "test_monte_carlo_tiny_workload", {})]),
    ("taylor_drops_tau", "return tau * tau / 24.0 * b;", "return tau / 24.0 * b;",
     [("test_oracle_bias", "test_taylor_exact_sandwich", {})]),
    ("bias_sign", "s -= (a->corr == 1)", "s += (a->corr == 1)",
     [("test_oracle_attention", "test_matches_library_sdpa", {"corr": "taylor", "wi": 0}),
      ("test_oracle_attention", "test_current_chunk_mass_never_drops", {"corr": "taylor"})]),
    ("exact_missing_half", "(double)step[c / group] / 2.0);", "(double)step[c / group]);",
     [("test_oracle_bias", "test_monte_carlo_tiny_workload", {})]),
    ("exact_wrong_group", "(double)step[c / group] / 2.0);", "(double)step[c % (d / group)] / 2.0);",
     [("test_oracle_bias", "test_monte_carlo_two_groups", {})]),
    ("taylor_wrong_group",
     "for (int32_t c = g * group; c < (g + 1) * group; ++c) qn += q[c] * q[c];",
     "for (int32_t c = g; c < d; c += d / group) qn += q[c] * q[c];",
     [("test_oracle_bias", "test_monte_carlo_two_groups", {})]),
    ("series_coefficient", "-1.0 / 180.0", "-1.0 / 120.0",
     [("test_oracle_bias", "test_logsinhc_series_and_branches", {})]),
    ("asymptote_sign", "log1p(-exp(-2.0 * a))", "log1p(exp(-2.0 * a))",
     [("test_oracle_bias", "test_logsinhc_library_routine", {})]),
    ("round_toward_zero", "float r = rintf(t);", "float r = truncf(t);",
     [("test_oracle_quantizer", "test_bruteforce_nearest_grid_point", {"bits": 2, "src": "f32"})]),
    ("step_divisor", "float step = range / (float)top;", "float step = range / (float)(top + 1);",
     [("test_oracle_quantizer", "test_error_bound_and_extreme_codes", {"wname": "tiny_d64_int2"})]),
    ("pack_msb_first", "out[bit / 8] |= (uint8_t)(c[k] << (bit % 8));",
     "out[bit / 8] |= (uint8_t)(c[k] << (8 - bits - bit % 8));",
     [("test_oracle_quantizer", "test_pack_unpack_roundtrip", {})]),
    ("zero_sign_not_canonical", "mn = mn + 0.0f; /* canonical zero sign */", "",
     [("test_oracle_quantizer", "test_adversarial_groups", {})]),
    ("dequant_offset", "out[r * d + k] = (double)zero[r * ng + g] +",
     "out[r * d + k] = (double)zero[r * ng + g] + 0.5 * (double)step[r * ng + g] +",
     [("test_oracle_quantizer", "test_error_bound_and_extreme_codes", {"wname": "h24_int4_cache16k"})]),
    ("gqa_mapping", "rc->hk = rc->h / (a->Hq / a->Hkv);", "rc->hk = rc->h % a->Hkv;",
     [("test_oracle_attention", "test_matches_library_sdpa", {"corr": "off", "wi": 1})]),
    ("default_scale", "return scale > 0.0 ? scale : 1.0 / sqrt((double)d);",
     "return scale > 0.0 ? scale : 1.0 / (double)d;",
     [("test_oracle_attention", "test_matches_library_sdpa", {"corr": "off", "wi": 0})]),
    ("online_no_rescale", "      l *= alpha;\n", "",
     [("test_oracle_attention", "test_online_matches_brute_force", {"corr": "off"})]),
    ("causal_top_left", "return t - a->Nc <= j + a->Ncur - a->Nq;", "return t - a->Nc <= j;",
     [("test_oracle_causal", "test_matches_library_lower_right", {"corr": "off", "wi": 0})]),
    ("causal_off_by_one", "return t - a->Nc <= j + a->Ncur - a->Nq;", "return t - a->Nc < j + a->Ncur - a->Nq;",
     [("test_oracle_causal", "test_matches_library_lower_right", {"corr": "off", "wi": 1})]),
    ("diag_mass_over_cache", "          if (t >= a->Nc) {\n            mr += pr;", "          if (t < a->Nc) {\n            mr += pr;",
     [("test_oracle_diagnostics", "test_matches_library_statistics", {"case": "tiny", "corr": "off", "tied": False})]),
    ("diag_kl_reversed", "kl += pr * ((sr[t] - lr) - (sq[t] - lq));", "kl += pr * ((sq[t] - lq) - (sr[t] - lr));",
     [("test_oracle_diagnostics", "test_matches_library_statistics", {"case": "int4", "corr": "taylor", "tied": False})]),
    ("diag_ties_to_last", "if (best < 0 || s[t] > s[best]) best = t;", "if (best < 0 || s[t] >= s[best]) best = t;",
     [("test_oracle_diagnostics", "test_matches_library_statistics", {"case": "tiny", "corr": "off", "tied": True})]),
    ("diag_ref_scale_dropped", "            sr[t] = s * rc.tau;", "            sr[t] = s;",
     [("test_oracle_diagnostics", "test_matches_library_statistics", {"case": "gqa_causal", "corr": "off", "tied": False})]),
    ("meta16_codes_against_raw_min", "      float num = x[k] - zero;", "      float num = x[k] - mn;",
     [("test_oracle_meta16", "test_quantizer_with_binary16_metadata", {"bits": 4, "group": 64})]),
    ("meta16_ties_away", "  const float r = rintf(a / u) * u;", "  const float r = roundf(a / u) * u;",
     [("test_oracle_meta16", "test_rounding_ties_subnormals_overflow", {})]),
    ("bf16_ties_away", "  const float r = rintf(ldexpf(a, -ue));", "  const float r = roundf(ldexpf(a, -ue));",
     [("test_oracle_metabf16", "test_rounding_ties_subnormals_overflow", {})]),
    ("bf16_fp16_spacing", "  int ue = (e - 1) - 7;       /* spacing in that binade */",
     "  int ue = (e - 1) - 10;       /* spacing in that binade */",
     [("test_oracle_metabf16", "test_rounding_matches_torch", {})]),
    ("bf16_no_subnormal_clamp", "  if (ue < -133) ue = -133;   /* subnormal spacing */", "",
     [("test_oracle_metabf16", "test_rounding_ties_subnormals_overflow", {})]),
    ("bf16_zero_not_rounded", "  zero = round_meta(mn, meta);", "  zero = mn;",
     [("test_oracle_metabf16", "test_quantizer_with_bfloat16_metadata", {"bits": 2, "group": 64})]),
    ("tokens_group_row_mod", "return (bkv * capg + t / a->group) * a->d + c;",
     "return (bkv * capg + t % a->group) * a->d + c;",
     [("test_oracle_tokens", "test_tokens_matches_library_sdpa", {"case": "int2_k_tokens", "corr": "off"})]),
    ("tokens_bias_per_group", "const int32_t gsz = a->kaxis == 0 ? a->group : 1;", "const int32_t gsz = a->group;",
     [("test_oracle_tokens", "test_tokens_matches_library_sdpa", {"case": "int4_both_tokens", "corr": "taylor"})]),
    ("tokens_read_transposed", "for (int32_t i = 0; i < cnt; ++i) vals[i] = xo[(t0 + i) * d + c];",
     "for (int32_t i = 0; i < cnt; ++i) vals[i] = xo[(t0 + i) + (int64_t)c * n];",
     [("test_oracle_tokens", "test_quantizer_is_the_transposed_head_dim_quantizer",
       {"bits": 2, "group": 32, "src": "f32", "meta": "f32"})]),
    ("value_not_dequantized_zero",
     "v[c] = (double)a->vc_zero[mv] + ", "v[c] = ",
     [("test_oracle_attention", "test_matches_library_sdpa", {"corr": "off", "wi": 2})]),
]


@pytest.mark.parametrize("name,find,repl,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(orc, tmp_path, name, find, repl, pins):
    with open(oracle._SRC) as f:
        src = f.read()
    assert src.count(find) == 1, f"mutation site for {name} not unique"
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(find, repl))
    so = oracle.compile_source(path, os.path.join(str(tmp_path), "libmutant.so"))
    good = oracle._lib
    oracle._lib = oracle._load(so)
    caught = []
    try:
        for mod, fn, kw in pins:
            try:
                getattr(importlib.import_module(mod), fn)(orc=oracle, **kw)
            except (AssertionError, ValueError):
                caught.append(fn)
    finally:
        oracle._lib = good
    assert caught, f"no pin caught the planted mistake {name}"
