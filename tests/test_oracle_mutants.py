"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of oracle/sp_oracle.c (a
dropped term, a wrong sign or index, a swapped operand, a wrong constant),
builds it with the same flags, and runs pin checks against that build: at
least one of them must fail.  The committed oracle is never modified.
"""
import os
import shutil

import pytest

import oracle
from oracle import build as obuild
from tests import test_oracle_region as R
from tests import test_oracle_rng as G

LN, RMS, F32, BF16 = oracle.LAYERNORM, oracle.RMSNORM, oracle.F32, oracle.BF16

MUTANTS = {
    # generator
    "philox_swapped_high_words": ("uint32_t n0 = hi1 ^ c1 ^ k0;", "uint32_t n0 = hi0 ^ c1 ^ k0;"),
    "philox_key_bumped_before_first_round": ("if (round > 0) {", "if (round >= 0) {"),
    "philox_wrong_multiplier": ("0xCD9E8D57u", "0xCD9E8D55u"),
    "dropout_wrong_word": ("return out[e % 4u];", "return out[(e + 1u) % 4u];"),
    "dropout_counter_ignores_high_word": ("(uint32_t)(block >> 32),", "0u,"),
    "threshold_rounds_up": ("return (uint32_t)floor((double)p * 4294967296.0);",
                            "return (uint32_t)ceil((double)p * 4294967296.0 + 0.5);"),
    "scale_is_keep_probability": ("return (float)(1.0 / (1.0 - (double)p));",
                                  "return (float)(1.0 - (double)p);"),
    "global_index_ignores_shard": ("uint64_t G = (uint64_t)d->shard_index * (uint64_t)rows_of(d) + (uint64_t)r;",
                                   "uint64_t G = (uint64_t)r;"),
    # rounding
    "bf16_truncates": ("u += 0x7fffu + kept_lsb;", "u += 0u * kept_lsb;"),
    "bf16_ties_away": ("u += 0x7fffu + kept_lsb;", "u += 0x8000u + 0u * kept_lsb;"),
    # forward
    "residual_dropped": ("float hf = load_io(d->io, residual, i) + v;", "float hf = v;"),
    "bias_after_dropout": ("float v = keep ? u * scale : 0.0f;",
                           "float v = keep ? (u - (bias ? bias[c] : 0.0f)) * scale + (bias ? bias[c] : 0.0f) : 0.0f;"),
    "norm_reads_unrounded_h": ("hrow[c] = (double)store_io(d->io, h_out, i, hf);",
                               "store_io(d->io, h_out, i, hf); hrow[c] = (double)hf;"),
    "sample_variance": ("double var = sq / (double)H;", "double var = sq / (double)(H - 1);"),
    "eps_outside_sqrt": ("*rstd = 1.0 / sqrt(var + eps);", "*rstd = 1.0 / sqrt(var) + eps;"),
    "rms_centres": ("for (int64_t c = 0; c < H; ++c) sq += hrow[c] * hrow[c];",
                    "double m0 = 0; for (int64_t c = 0; c < H; ++c) m0 += hrow[c] / H;"
                    " for (int64_t c = 0; c < H; ++c) sq += (hrow[c] - m0) * (hrow[c] - m0);"),
    "beta_scaled_by_gamma": ("yv = (hrow[c] - mu) * rs * (double)gamma[c] + (double)beta[c];",
                             "yv = ((hrow[c] - mu) * rs + (double)beta[c]) * (double)gamma[c];"),
    # backward
    "ln_bwd_drops_mean_g": ("dh[c] = rstd * (g - mean_g - xhat[c] * mean_gx);",
                            "dh[c] = rstd * (g - xhat[c] * mean_gx);"),
    "ln_bwd_wrong_sign": ("dh[c] = rstd * (g - mean_g - xhat[c] * mean_gx);",
                          "dh[c] = rstd * (g - mean_g + xhat[c] * mean_gx);"),
    "rms_bwd_drops_projection": ("dh[c] = rstd * (g - xhat[c] * mean_gx);", "dh[c] = rstd * g;"),
    "bwd_g_without_gamma": ("double g = dyrow[c] * gam[c];\n        xhat[c] = xc;",
                            "double g = dyrow[c];\n        xhat[c] = xc;"),
    "dgamma_uses_g": ("acc_dgamma[c] += dyrow[c] * xhat[c];",
                      "acc_dgamma[c] += dyrow[c] * gam[c] * xhat[c];"),
    "dbias_ignores_mask": ("acc_dbias[c] += dxu;", "acc_dbias[c] += dhv;"),
    "dx_not_scaled": ("double dxu = keep ? dhv * scale : 0.0;\n            if (dres_out)",
                      "double dxu = keep ? dhv : 0.0;\n            if (dres_out)"),
    "dh_out_ignored": ("double dhv = (dy ? dh[c] : 0.0) + (dh_out ? (double)load_io(d->io, dh_out, i) : 0.0);",
                       "double dhv = (dy ? dh[c] : 0.0);"),
    "exact_dgamma_uses_g": ("dgamma_out[c] += dy[i] * xhat[c];",
                            "dgamma_out[c] += dy[i] * gamma[c] * xhat[c];"),
    # region variants
    "entry_adds_zero": ("float hf = load_io(d->io, residual, i);\n                hrow[c]",
                        "float hf = load_io(d->io, residual, i) + 0.0f;\n                hrow[c]"),
    "exit_dres_scaled": ("if (dres_out) store_io(d->io, dres_out, i, (float)dhv);",
                         "if (dres_out) store_io(d->io, dres_out, i, (float)(dy ? dhv : dxu));"),
    # ring attention
    "attn_scale_squared": ("s[j] = (double)d->scale * dot;", "s[j] = (double)d->scale * (double)d->scale * dot;"),
    "attn_unnormalised": ("o_out[AT(qi, bi, hh, dd)] = acc / l;", "o_out[AT(qi, bi, hh, dd)] = acc;"),
    "attn_lse_without_max": ("lse_out[(qi * B + bi) * NH + hh] = m + log(l);",
                             "lse_out[(qi * B + bi) * NH + hh] = log(l);"),
    "attn_keys_ignore_head": ("(double)spo_bf16_to_f32(k[AT(j, bi, hh, dd)]);",
                              "(double)spo_bf16_to_f32(k[AT(j, bi, 0, dd)]);"),
    # reduce-scatter prologue
    "reduce_reversed_order": ("float acc = load_io(d->io, parts, i);                       /* rank 0 */\n"
                              "        for (int p = 1; p < nparts; ++p)",
                              "float acc = load_io(d->io, parts, (int64_t)(nparts - 1) * n + i);\n"
                              "        for (int p = nparts - 2; p >= 0; --p)"),
    "reduce_rounds_each_add": ("acc = acc + load_io(d->io, parts, (int64_t)p * n + i);",
                               "acc = store_io(d->io, x_out, i, acc + load_io(d->io, parts, (int64_t)p * n + i));"),
    "reduce_drops_last_part": ("for (int p = 1; p < nparts; ++p)", "for (int p = 1; p < nparts - 1; ++p)"),
    # accounting
    "mask_counted_as_bf16": ("uint64_t mask_bytes = (d->p > 0.0f) ? E : 0u;",
                             "uint64_t mask_bytes = (d->p > 0.0f) ? 2u * E : 0u;"),
    "output_not_retained": ("*retained_output = E * es;", "*retained_output = 0u;"),
}


def _checks(L, philox):
    """Pin checks, each a callable raising on failure (all run against L)."""
    from tests import test_oracle_accounting as A
    from tests import test_oracle_rs as S
    from tests import test_oracle_variants as V
    from tests import test_oracle_attention as T
    c = [
        lambda: T.test_matches_torch_sdpa_float64(L, 5, 2, 3, 16, 3, 1),
        lambda: T.test_two_keys_closed_form(L),
        lambda: V.test_entry_h_is_the_residual_bit_for_bit(L, F32),
        lambda: V.test_entry_backward_matches_torch_autograd(L, LN),
        lambda: V.test_exit_backward_matches_torch_autograd(L, 0.3),
        lambda: S.test_one_part_is_the_identity(L, BF16),
        lambda: S.test_integer_parts_sum_exactly(L, F32, 8),
        lambda: S.test_integer_parts_sum_exactly(L, BF16, 4),
        lambda: S.test_parts_are_added_in_rank_order(L, F32),
        lambda: S.test_parts_are_added_in_rank_order(L, BF16),
        lambda: S.test_bf16_final_rounding_is_one_rne(L),
        lambda: G.test_philox_block_matches_torch_engine(L, philox),
        lambda: G.test_dropout_word_selects_word_e_mod_4_of_block_e_div_4(L, philox),
        lambda: G.test_mask_matches_library_words_and_global_index(L, philox),
        lambda: G.test_threshold_is_floor_p_times_2_pow_32_exactly(L),
        lambda: G.test_scale_is_reciprocal_of_keep_probability(L),
        lambda: G.test_bf16_rounding_matches_torch(L),
        lambda: R.test_p0_is_identity_dropout(L, F32),
        lambda: R.test_dropout_drops_to_residual_and_keeps_expectation(L),
        lambda: R.test_norm_closed_forms_unit_affine(L, LN),
        lambda: R.test_norm_closed_forms_unit_affine(L, RMS),
        lambda: R.test_forward_matches_torch_float64_norm(L, LN, BF16),
        lambda: R.test_forward_matches_torch_float64_norm(L, RMS, BF16),
        lambda: R.test_shards_concatenate_to_unsharded_run(L, BF16, LN, 2),
        lambda: R.test_backward_matches_torch_autograd(L, LN),
        lambda: R.test_backward_matches_torch_autograd(L, RMS),
        lambda: A.test_region_bytes_reproduce_replicated_band(L),
    ]
    for norm in (LN, RMS):
        c.append(lambda norm=norm: R.test_backward_matches_finite_differences(
            L, norm, 0.1, 2, 1, True))
    return c


@pytest.fixture(scope="module")
def philox(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    return G.build_torch_philox(tmp_path_factory.mktemp("philox_m"))


def test_unmutated_oracle_passes_every_check(olib, philox):
    for chk in _checks(olib, philox):
        chk()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, philox, tmp_path):
    old, new = MUTANTS[name]
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mdir = tmp_path / "m"
    mdir.mkdir()
    shutil.copy(os.path.join(os.path.dirname(obuild.SRC), "sp_oracle.h"), mdir / "sp_oracle.h")
    (mdir / "sp_oracle.c").write_text(src.replace(old, new))
    lib_path = str(mdir / "libmut.so")
    import subprocess
    subprocess.run(["gcc", *[f for f in obuild.CFLAGS if f != "-Werror"], "-o", lib_path,
                    str(mdir / "sp_oracle.c"), "-lm"], check=True)
    L = oracle.load(lib_path)
    caught = []
    for i, chk in enumerate(_checks(L, philox)):
        try:
            chk()
        except (AssertionError, ValueError):
            caught.append(i)
    assert caught, f"no pin caught the planted mistake {name}"
