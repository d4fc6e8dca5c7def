"""The oracle's pins are sensitive: plant plausible mistakes in a copy of the
oracle (on the CPU only), rebuild it, and check that some pin fails for each.

The mutants are textual edits of oracle/fpstok_oracle.c compiled into a
temporary directory; the committed oracle is never touched.
"""
import importlib.util
import os
import shutil
import sys

import numpy as np
import pytest

import tests.test_oracle_next as nxt
import tests.test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, original text, mutated text)
MUTANTS = [
    ("drop_time_axis", "    r = r + dt * dt;\n", "    (void)dt;\n"),
    ("axis_order", "    float r = dx * dx;\n    r = r + dy * dy;\n    r = r + dz * dz;\n    r = r + dt * dt;\n",
     "    float r = dt * dt;\n    r = r + dz * dz;\n    r = r + dy * dy;\n    r = r + dx * dx;\n"),
    ("argmax_ties_to_highest", "if (best < 0 || mind[i] > bestv)", "if (best < 0 || mind[i] >= bestv)"),
    ("selected_not_excluded", "            if (taken[i]) continue;\n", ""),
    ("voronoi_ties_to_last_slot", "if (d < mind[i]) { mind[i] = d; near[i] = j; }",
     "if (d <= mind[i]) { mind[i] = d; near[i] = j; }"),
    ("assign_ties_to_last_slot", "                if (d < bd) { bd = d; best = j; }\n            }\n            assign[off + i] = best;",
     "                if (d <= bd) { bd = d; best = j; }\n            }\n            assign[off + i] = best;"),
    ("knn_ties_to_highest", "return (x->i > y->i) - (x->i < y->i);", "return (x->i < y->i) - (x->i > y->i);"),
    ("lloyd_unweighted", "acc[5 * j + 0] += w;", "acc[5 * j + 0] += 1.0;"),
    ("lloyd_empty_cell_to_origin", "                if (W > 0.0)\n                    for (int a = 0; a < 4; ++a) cen[4 * j + a] = (float)(acc[5 * j + 1 + a] / W);",
     "                for (int a = 0; a < 4; ++a) cen[4 * j + a] = W > 0.0 ? (float)(acc[5 * j + 1 + a] / W) : 0.0f;"),
    ("lloyd_float_accumulation", "for (int a = 0; a < 4; ++a) acc[5 * j + 1 + a] += w * (double)q[a];",
     "for (int a = 0; a < 4; ++a) acc[5 * j + 1 + a] = (float)(acc[5 * j + 1 + a] + (float)(w * q[a]));"),
    ("pool_ignores_weight", "    int32_t wcol = weighted ? charge_col : -1;", "    int32_t wcol = -1;"),
    ("pool_drops_last_knn_entry", "for (int32_t e = 0; e < k; ++e) {\n                    int32_t i = lst[e];",
     "for (int32_t e = 0; e + 1 < k; ++e) {\n                    int32_t i = lst[e];"),
    ("passthrough_threshold_off_by_one", "        if (n <= P) {\n            /* small events", "        if (n < P) {\n            /* small events"),
    ("pack_doc_id_shifted", "            if (doc_id) doc_id[at + j] = (int32_t)b;",
     "            if (doc_id) doc_id[at + j] = (int32_t)(b + 1 < B ? b + 1 : b);"),
    ("pack_drops_last_token", "        for (int32_t j = 0; j < T; ++j) {\n            for (int32_t d = 0; d < D; ++d)\n                packed",
     "        for (int32_t j = 0; j + 1 < T; ++j) {\n            for (int32_t d = 0; d < D; ++d)\n                packed"),
    ("unpack_no_zero_padding", "                    j < T ? packed[((int64_t)cu_seqlens[b] + j) * D + d] : 0.0f;",
     "                    j < T ? packed[((int64_t)cu_seqlens[b] + j) * D + d] : 1.0f;"),
    ("philox_key_not_advanced", "        if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }", "        (void)r;"),
    ("philox_words_swapped", "        uint32_t n1 = (uint32_t)p1;", "        uint32_t n1 = (uint32_t)p0;"),
    ("random_start_modulo", "start_idx[b] = n > 0 ? (int32_t)(((uint64_t)out[0] * (uint64_t)n) >> 32) : 0;",
     "start_idx[b] = n > 0 ? (int32_t)((uint64_t)out[0] % (uint64_t)n) : 0;"),
    ("random_start_event_and_step_swapped",
     "uint32_t in[4] = {(uint32_t)b, (uint32_t)((uint64_t)b >> 32), (uint32_t)step,\n                          (uint32_t)(step >> 32)};",
     "uint32_t in[4] = {(uint32_t)step, (uint32_t)(step >> 32), (uint32_t)b,\n                          (uint32_t)((uint64_t)b >> 32)};"),
    ("random_start_word1", "(int32_t)(((uint64_t)out[0] * (uint64_t)n) >> 32)",
     "(int32_t)(((uint64_t)out[1] * (uint64_t)n) >> 32)"),
    ("binary16_subnormals_flushed", "        v = ldexpf((float)m, -24);", "        v = 0.0f;"),
    ("bfloat16_rounded_not_upcast", "    uint32_t bits = (uint32_t)h << 16;\n    float v;",
     "    uint32_t bits = ((uint32_t)h << 16) | 0x8000u;\n    float v;"),
    ("backward_ignores_weight", "    int32_t wcol = weighted != 0 ? charge_col : -1;", "    int32_t wcol = -1;"),
    ("backward_drops_weight_term", "                    gi[wcol] += s / W[j];", "                    (void)s;"),
    ("backward_unit_weight", "for (int32_t c = 0; c < C; ++c) gi[c] += (double)g[c] * w / W[j];",
     "for (int32_t c = 0; c < C; ++c) gi[c] += (double)g[c] / W[j];"),
    ("backward_sign_of_weight_term", "s += (double)g[c] * ((double)f[c] - (double)m[c]);",
     "s += (double)g[c] * ((double)m[c] - (double)f[c]);"),
    ("backward_overwrites_instead_of_adding", "for (int32_t c = 0; c < C; ++c) gi[c] += (double)g[c] * w / W[j];",
     "for (int32_t c = 0; c < C; ++c) gi[c] = (double)g[c] * w / W[j];"),
]

PIN_CALLS = [
    lambda m: nxt.test_pack_worked_example(m),
    lambda m: [nxt.test_pack_counts_and_round_trip(m, s) for s in (0, 1)],
    lambda m: nxt.test_pack_rejects_bad_counts(m),
    lambda m: [nxt.test_pool_backward_finite_differences(m, mode, w, 0)
               for mode in (0, 1) for w in (False, True)],
    lambda m: nxt.test_pool_backward_worked_example(m),
    lambda m: nxt.test_pool_backward_plain_mean_and_passthrough(m),
    lambda m: nxt.test_pool_backward_zero_weight_token_and_linearity(m),
    lambda m: nxt.test_philox_known_answers(m),
    lambda m: nxt.test_random_start_mapping_and_spread(m),
    lambda m: nxt.test_random_start_from_the_known_answer_vector(m),
    lambda m: nxt.test_random_start_counter_layout(m),
    lambda m: nxt.test_upcast_binary16_exhaustive(m),
    lambda m: nxt.test_upcast_bfloat16_exhaustive(m),
    lambda m: [pins.test_closed_forms(m, c) for c in pins._cases()],
    lambda m: pins.test_identical_cloud_knn_pool_lloyd(m),
    lambda m: [pins.test_fps_and_assign_brute_force(m, s) for s in (1, 2, 3)],
    lambda m: [pins.test_knn_brute_force(m, s) for s in (4, 5)],
    lambda m: pins.test_knn_passthrough_rows(m),
    lambda m: pins.test_axis_summation_order_is_pinned(m),
    lambda m: pins.test_passthrough_and_counts(m),
    lambda m: pins.test_passthrough_knn_mode_pools_the_pulse(m),
    lambda m: pins.test_translation_invariance(m),
    lambda m: pins.test_lloyd_inertia_non_increasing_and_fixed_point(m),
    lambda m: pins.test_lloyd_update_is_exact_weighted_mean(m),
    lambda m: pins.test_lloyd_separated_clusters(m),
    lambda m: pins.test_pool_exact_small_integers(m),
    lambda m: pins.test_pool_knn_lists_and_charge_fallback(m),
    lambda m: pins.test_pool_zero_weight_cell_is_zero(m),
]


def _mutant_module(tmp_path, name, old, new):
    src = open(os.path.join(ROOT, "oracle", "fpstok_oracle.c")).read()
    assert src.count(old) == 1, "mutation anchor for %s not unique" % name
    d = tmp_path / ("oracle_" + name)
    d.mkdir()
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), d / "__init__.py")
    (d / "fpstok_oracle.c").write_text(src.replace(old, new))
    modname = "oracle_mutant_" + name
    spec = importlib.util.spec_from_file_location(modname, d / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mod
    spec.loader.exec_module(mod)
    mod.build(force=True)
    return mod


@pytest.mark.parametrize("mut", MUTANTS, ids=lambda m: m[0])
def test_mutant_is_caught(tmp_path, mut):
    name, old, new = mut
    mod = _mutant_module(tmp_path, name, old, new)
    failures = 0
    for call in PIN_CALLS:
        try:
            with np.errstate(all="ignore"):
                call(mod)
        except (AssertionError, RuntimeError):
            failures += 1
    assert failures > 0, "mutant %s survived every pin" % name
