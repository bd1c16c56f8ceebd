"""The pins are strong enough: each plausible mistake planted in a copy of the oracle's C
source or of its Python front end (a dropped term, a wrong sign, a wrong operand or index, a
wrong tie rule, a wrong normalisation) makes at least one pin of test_oracle_pins fail.  The
mutants are built on the CPU (C ones into a temporary directory); the real oracle is
untouched and restored afterwards."""
import os
import subprocess

import numpy as np
import pytest

import test_oracle_pins as P
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "csa_oracle.c")

MUTANTS = {
    "summary score without ln c_b": ("keys, kv_off(s, b, j, nb, blk)) + log((double)c);",
                                     "keys, kv_off(s, b, j, nb, blk));"),
    "proxy logit without ln count": ("Kbar, off) + log((double)block_count(s, blk));", "Kbar, off);"),
    "group score not normalised per head": ("first[(size_t)g * nb + blk] - lse_h[g];",
                                            "first[(size_t)g * nb + blk];"),
    "ties to the higher index": ("return (a->index > b->index) - (a->index < b->index);",
                                 "return (a->index < b->index) - (a->index > b->index);"),
    "ragged block divided by L": ("sk / c);", "sk / s->block_size);"),
    "value summary taken from keys": ("sv += elem(V, s->dtype", "sv += elem(K, s->dtype"),
    "logit scale 1/d": ("1.0 / sqrt((double)s->head_dim)", "1.0 / (double)s->head_dim"),
    "log-weight subtracted": ("+ (double)tok_logw[", "- (double)tok_logw["),
    "output not normalised": ("out[t] /= denom;", "out[t] /= 1.0;"),
    "query head on the wrong KV head": ("j = h / G;", "j = h % s->n_kv_heads;"),
    "lse without the maximum": ("*lse = mx + log(denom);", "*lse = log(denom);"),
    "exact mass as the maximum logit": ("    return mx + log(sum);", "    return mx + 0.0 * log(sum);"),
    "box scored at its worst corner": ("acc += a > c ? a : c;", "acc += a < c ? a : c;"),
    "box maximum taken as the minimum": ("if (x > hi) hi = x;", "if (x < hi) hi = x;"),
    "equal distances to the higher cluster": ("if (dc < bd) {", "if (dc <= bd) {"),
    "centroid divided by count + 1": ("sum[(size_t)c * r + jj] / cnt[c];", "sum[(size_t)c * r + jj] / (cnt[c] + 1);"),
    "cluster logit without ln count": ("Kc, kv_off(s, b, j, C, c)) + log((double)m)", "Kc, kv_off(s, b, j, C, c))"),
    "cluster proxy without ln count": ("Kc, co) + log((double)m);", "Kc, co);"),
    "cluster mean divided by n": ("m > 0 ? sk / m : 0.0", "m > 0 ? sk / n : 0.0"),
    "projection with the basis transposed": ("(double)Up[(size_t)t * r + jj]", "(double)Up[(size_t)jj * d + t]"),
    "selected cluster also kept as a proxy": ("if (kept[c] || m == 0) continue;", "if (m == 0) continue;"),
    "no assignment to the final centroids": ("if (it == iters) break;", "if (it == iters) { a[0] = a[0]; }"),
}

BATTERY = [
    (P.test_summaries_are_exact_means_rounded_once, ("f32", 1000, 16)),
    (P.test_summaries_are_exact_means_rounded_once, ("bf16", 200, 64)),
    (P.test_dense_matches_library_attention, ("f32",)),
    (P.test_dense_closed_form_identical_keys, ()),
    (P.test_keeping_all_blocks_equals_dense, ("bf16", 3, 1000, 64)),
    (P.test_block_size_one_makes_proxies_exact, (3,)),
    (P.test_equal_logit_tail_proxy_is_exact, ()),
    (P.test_proxy_logit_is_mean_logit_plus_log_count, ()),
    (P.test_mha_selection_is_top_k_by_exact_mass, (12,)),
    (P.test_group_score_is_sum_of_normalised_masses, ()),
    (P.test_topk_ties_go_to_lower_index, ()),
    (P.test_jensen_mean_logit_bound, ()),
    (P.test_mixture_and_renormalised_error_identities, ()),
    (P.test_worked_example_from_the_page, ()),
    (P.test_integer_weights_equal_multiplicities, ()),
    (P.test_box_build_is_elementwise_min_and_max, ("f32", 200, 16)),
    (P.test_box_score_bounds_every_token_logit, ("f32",)),
    (P.test_box_score_is_the_best_corner, ()),
    (P.test_cluster_assignments_are_the_nearest_centroids, ()),
    (P.test_cluster_centroids_are_the_means_of_their_points_at_convergence, ()),
    (P.test_lloyd_rounds_never_increase_the_objective, ()),
    (P.test_cluster_layout_is_a_stable_partition, ()),
    (P.test_cluster_means_are_exact_means_rounded_once, ("bf16",)),
    (P.test_one_token_per_cluster_makes_the_proxies_exact, ()),
    (P.test_contiguous_clusters_are_the_block_method, (3,)),
    (P.test_equal_distances_go_to_the_lower_cluster, ()),
]


def _failures():
    failed = []
    for fn, args in BATTERY:
        try:
            fn(*args)
        except (AssertionError, ValueError):
            failed.append(fn.__name__)
    return failed


def test_unmutated_oracle_passes_the_battery():
    O.use_library(None)
    assert _failures() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    count = src.count(old)
    assert count >= 1, f"mutation site for {name!r} not found"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    (tmp_path / "csa_oracle.h").write_text(open(SRC[:-2] + ".h").read())
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                           str(mutant_c), "-o", str(lib), "-lm"])
    O.use_library(str(lib))
    try:
        failed = _failures()
    finally:
        O.use_library(None)
    assert failed, f"no pin caught the mutant {name!r}"


# The second-order descriptors and logits live in the oracle's Python front end;
# their mutants are planted in a copy of that module.
PY_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "oracle.py")
PY_MUTANTS = {
    "second-order term without the one half": ("+ 0.5 * scale * scale *", "+ 1.0 * scale * scale *"),
    "covariance with the sample divisor": ("Xc.T @ Xc / X.shape[0]", "Xc.T @ Xc / (X.shape[0] - 1)"),
    "eigenvectors not scaled by the root eigenvalue": ("math.sqrt(max(lam[d - 1 - i], 0.0)) * u",
                                                       "max(lam[d - 1 - i], 0.0) * u"),
    "smallest eigendirections kept": ("u = U[:, d - 1 - i]", "u = U[:, i]"),
    "error ranked by the logit variance, not its spread": ("shat[:, h] + 0.5 * np.log(", "shat[:, h] + 1.0 * np.log("),
    "proxy mass without the count": ("shat[:, h] = scale * mean_dot + np.log(counts)", "shat[:, h] = scale * mean_dot"),
    "group normalised by the errors instead of the masses": ("rel = lerr - _lse(shat, axis=2)", "rel = lerr - _lse(lerr, axis=2)"),
    "variance about zero instead of the block mean": ("dv = X[:, :, i] - mean", "dv = X[:, :, i]"),
    "variance with the sample divisor": ("var[:, :, blk] = s2 / c", "var[:, :, blk] = s2 / max(c - 1, 1)"),
    "spread without the logit scale": ("spread2 = scale * scale * np.einsum", "spread2 = np.einsum"),
    "FP4 ties to the odd mantissa": ("c % 2 == 0 and best % 2 == 1", "c % 2 == 1 and best % 2 == 0"),
    "FP4 scale for a largest code of 4": ("/ np.float32(6.0)", "/ np.float32(4.0)"),
    "FP4 nibbles swapped": ("codes[2 * t] | (codes[2 * t + 1] << 4)", "codes[2 * t + 1] | (codes[2 * t] << 4)"),
    "FP4 sign dropped": ("return best | (8 if (float(r) < 0 and best) else 0)", "return best"),
    "FP4 decoded without the scale": ("return mean, scales[..., None] * val", "return mean, val"),
    "subspace covariance not centred": ("Y = (X - X.mean(axis=0)) @ U[j]", "Y = X @ U[j]"),
    "subspace covariance with the sample divisor": ("Y.T @ Y / X.shape[0]", "Y.T @ Y / (X.shape[0] - 1)"),
    "subspace factors not scaled by the root eigenvalue": ("math.sqrt(max(mu[s_dim - 1 - i], 0.0)) * v",
                                                           "max(mu[s_dim - 1 - i], 0.0) * v"),
    "smallest subspace directions kept": ("v = V[:, s_dim - 1 - i]", "v = V[:, i]"),
    "query projected with another KV head's basis": ("qt = qf[:, h] @ U[h // G]", "qt = qf[:, h] @ U[(h + 1) % Hkv]"),
    "FP4 subspace padding codes not zero": ("+ [0] * (sf - s_dim)", "+ [1] * (sf - s_dim)"),
    "FP4 subspace factors decoded without the scale": ("return mean, scales[..., None] * np.where(nib & 8, -mag, mag)",
                                                       "return mean, np.where(nib & 8, -mag, mag)"),
    "subspace term without the one half": ("(m2 ** 2).sum(-1)\n    return out\n\n\ndef block_logits",
                                           "(m2 ** 2).sum(-1) * 2.0\n    return out\n\n\ndef block_logits"),
}
PY_BATTERY = [
    P.test_cov_descriptor_is_the_top_eigen_truncation,
    P.test_second_order_term_is_half_the_logit_variance_at_full_rank,
    P.test_equal_logit_block_has_no_second_order_term,
    P.test_second_order_estimate_tracks_the_exact_mass,
    P.test_variance_token_closed_forms,
    P.test_spread_is_the_std_of_the_block_logits_and_error_is_mass_times_spread,
    P.test_scaling_every_spread_shifts_every_score_by_its_log,
    P.test_exact_proxies_carry_no_error,
    P.test_e2m1_rounding_matches_its_binade_definition,
    P.test_fp4_pack_layout_by_hand,
    P.test_fp4_decode_error_is_within_half_a_grid_step,
    P.test_fp4_score_equals_bf16_score_on_grid_exact_descriptors,
    P.test_subspace_storage_is_the_pages_figure,
    P.test_subspace_factors_are_the_top_eigen_truncation_of_the_projected_covariance,
    P.test_subspace_of_full_dimension_scores_like_the_full_space_descriptor,
    P.test_subspace_score_is_exact_when_query_and_spread_live_in_the_subspace,
    P.test_subspace_term_at_full_rank_is_the_projected_quadratic_form,
    P.test_subspace_basis_of_coordinate_axes_keeps_the_leading_block,
    P.test_sub_fp4_size_and_layout_by_hand,
    P.test_sub_fp4_score_equals_bf16_score_on_grid_exact_factors,
]


def _py_failures(module):
    failed = []
    saved = P.O
    P.O = module
    try:
        for fn in PY_BATTERY:
            try:
                fn()
            except (AssertionError, ValueError):
                failed.append(fn.__name__)
    finally:
        P.O = saved
    return failed


def test_unmutated_python_oracle_passes_its_battery():
    assert _py_failures(O) == []


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_pins_catch_planted_python_mistake(name):
    import types

    old, new = PY_MUTANTS[name]
    src = open(PY_SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    import sys

    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = PY_SRC  # the compiled C library is shared with the original
    sys.modules["oracle_mutant"] = mod  # dataclasses look their module up
    try:
        exec(compile(src.replace(old, new), PY_SRC, "exec"), mod.__dict__)
        with np.errstate(invalid="ignore"):  # a mutant may subtract infinities
            assert _py_failures(mod), f"no pin caught the mutant {name!r}"
    finally:
        del sys.modules["oracle_mutant"]
