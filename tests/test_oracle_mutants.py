"""The pins must be able to fail: each case plants one plausible mistake in a
temporary copy of the oracle's C source (a dropped term, a wrong sign,
index, constant or rounding), builds it, and checks that at least one of
the named pins rejects the mutant.  The real oracle is never modified."""
import importlib.util
import inspect
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")


def _load(name, path):
    spec = importlib.util.spec_from_file_location(name, path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


PIN_MODULES = [
    _load("oracle_pins_for_mutants", os.path.join(ROOT, "tests", "test_oracle_pins.py")),
    _load("oracle_pins_stochastic_for_mutants", os.path.join(ROOT, "tests", "test_oracle_pins_stochastic.py")),
    _load("oracle_pins_shared_for_mutants", os.path.join(ROOT, "tests", "test_oracle_pins_shared.py")),
    _load("oracle_pins_topk_for_mutants", os.path.join(ROOT, "tests", "test_oracle_pins_topk.py")),
]


def pin(name):
    for mod in PIN_MODULES:
        if hasattr(mod, name):
            return getattr(mod, name)
    raise KeyError(name)

# (name, text in qc_oracle.c, replacement, pins expected to catch it)
MUTANTS = [
    ("uniform_keeps_negative_zero", "    mn = mn + 0.0f; /* -0 -> +0 */\n", "",
     ["test_uniform_constant_and_signed_zero"]),
    ("uniform_rounds_down", "r = rintf(t);", "r = floorf(t);",
     ["test_uniform_brute_force_nearest"]),
    ("uniform_crumbs_msb_first", "put_word(p, i / 16, get_word(p, i / 16) | (code << (2 * (i % 16))));",
     "put_word(p, i / 16, get_word(p, i / 16) | (code << (2 * (15 - i % 16))));",
     ["test_uniform_packing_known_answer"]),
    ("stochastic_rounds_wrong_way", "< frac ? 1.0f : 0.0f", "> frac ? 1.0f : 0.0f",
     ["test_stochastic_uniform_follows_library_draws", "test_stochastic_uniform_unbiased"]),
    ("stochastic_ignores_offset", "r = fl + (uniform_draw(seed, elem_offset + (uint64_t)i)",
     "r = fl + (uniform_draw(seed, (uint64_t)i)", ["test_stochastic_uniform_follows_library_draws"]),
    ("ternary_half_probability", "float p = fabsf(v[j]) / s;", "float p = fabsf(v[j]) / (2.0f * s);",
     ["test_ternary_follows_library_draws", "test_ternary_unbiased_and_probability"]),
    ("ternary_sign_flip", "code = (v[j] < 0.0f) ? 3u : 1u;", "code = (v[j] < 0.0f) ? 1u : 3u;",
     ["test_ternary_closed_forms"]),
    ("ternary_mean_scale", "if (fabsf(v[j]) > s) s = fabsf(v[j]);", "s = s + fabsf(v[j]) / (float)cnt;",
     ["test_ternary_follows_library_draws", "test_ternary_closed_forms"]),
    ("uniform_dq_wrong_sign", "    return p + zero;", "    return p - zero;",
     ["test_uniform_error_bound_and_extremes", "test_uniform_error_feedback_invariants"]),
    ("uniform_levels_off_by_one", "const float sc = (mx - mn) / (float)L;",
     "const float sc = (mx - mn) / (float)(L + 1);", ["test_uniform_brute_force_nearest"]),
    ("uniform_nibbles_msb_first", "put_word(p, i / 8, get_word(p, i / 8) | (code << (4 * (i % 8))));",
     "put_word(p, i / 8, get_word(p, i / 8) | (code << (4 * (7 - i % 8))));",
     ["test_uniform_packing_known_answer"]),
    ("uniform_ef_not_updated", "                ef[i] = v[j] - uniform_dq(q, sc, mn);",
     "                ef[i] = v[j];", ["test_uniform_error_feedback_invariants"]),
    ("fp8_wrong_max", "const float sc = amax / 448.0f;", "const float sc = amax / 447.0f;",
     ["test_fp8_rowwise_invariants"]),
    ("fp8_mantissa_truncated", "double m = rint((s - 1.0) * 8.0);", "double m = floor((s - 1.0) * 8.0);",
     ["test_e4m3_encode_matches_torch_binades", "test_e4m3_special_values"]),
    ("fp8_subnormal_step", "double m = rint(a * 512.0);", "double m = rint(a * 256.0);",
     ["test_e4m3_encode_matches_torch_binades"]),
    ("fp8_decode_bias", "ldexp(8.0 + m, e - 10)", "ldexp(8.0 + m, e - 9)",
     ["test_e4m3_decode_closed_form"]),
    ("philox_weyl_typo", "weyl1 = 0xBB67AE85u", "weyl1 = 0xBB67AE86u", ["test_philox_matches_rocrand"]),
    ("philox_nine_rounds", "round < 10; ++round", "round < 9; ++round", ["test_philox_matches_rocrand"]),
    ("qsgd_grid_eight", "const float d = nrm / 7.0f;", "const float d = nrm / 8.0f;",
     ["test_qsgd_deterministic_on_grid", "test_qsgd_levels_bracket_value"]),
    ("qsgd_rounds_wrong_way", "(u < frac ? 1u : 0u)", "(u > frac ? 1u : 0u)",
     ["test_qsgd_unbiased"]),
    ("draw_wrong_word", "return (float)(r[g & 3u] >> 8) * 0x1p-24f;",
     "return (float)(r[(g + 1) & 3u] >> 8) * 0x1p-24f;", ["test_qsgd_draws_follow_library_philox"]),
    ("draw_fewer_bits", "return (float)(r[g & 3u] >> 8) * 0x1p-24f;",
     "return (float)(r[g & 3u] >> 16) * 0x1p-16f;", ["test_stochastic_uniform_draw_resolution"]),
    ("qsgd_ignores_offset", "float u = uniform_draw(seed, elem_offset + (uint64_t)i);",
     "float u = uniform_draw(seed, (uint64_t)i);",
     ["test_qsgd_counter_offsets_compose", "test_qsgd_draws_follow_library_philox"]),
    ("qsgd_drops_square", "sq[j] = v[j] * v[j];", "sq[j] = fabsf(v[j]);",
     ["test_qsgd_deterministic_on_grid"]),
    ("sign_zero_negative", "uint32_t b = (v[j] < 0.0f) ? 1u : 0u;", "uint32_t b = (v[j] <= 0.0f) ? 1u : 0u;",
     ["test_sign_bits_and_scale"]),
    ("sign_mean_over_full_bucket", "qco_tree_sum(av, cnt, bucket) / (float)cnt;",
     "qco_tree_sum(av, cnt, bucket) / (float)bucket;", ["test_sign_bits_and_scale"]),
    ("tree_left_to_right", "    float right = pair_sum(a + len / 2, len / 2);\n    return left + right;",
     "    float s = 0.0f;\n    for (int64_t i = 0; i < len; ++i) s = s + a[i];\n    (void)left;\n    return s;",
     ["test_tree_sum_order"]),
    ("vote_tie_goes_negative", "if (2 * c > m)", "if (2 * c >= m)", ["test_vote_brute_force_small_m"]),
    ("acc_wrong_scale_index", "scale + (int64_t)w * nb,", "scale + (int64_t)w,",
     ["test_accumulate_vs_exact_sum"]),
    ("acc_drops_last_worker", "for (int32_t w = 0; w < m; ++w) {\n            float dq",
     "for (int32_t w = 0; w < m - 1; ++w) {\n            float dq", ["test_accumulate_vs_exact_sum"]),
    ("shared_scale_128", "const float sc = amax[k] / 127.0f;", "const float sc = amax[k] / 128.0f;",
     ["test_int8_shared_on_grid_is_exact", "test_int8_shared_brute_force_nearest"]),
    ("shared_rounds_down", "float r = rintf(v / sc);", "float r = floorf(v / sc);",
     ["test_int8_shared_brute_force_nearest", "test_int8_shared_symmetric"]),
    ("shared_clamps_at_128", "if (r < -127.0f) r = -127.0f;", "if (r < -128.0f) r = -128.0f;",
     ["test_int8_shared_saturates_and_zero_scale"]),
    ("shared_absmax_ignores_ef", "const float v = ef ? ef[i] + x[i] : x[i];\n            if (fabsf(v) > m)",
     "const float v = x[i];\n            if (fabsf(v) > m)", ["test_bucket_absmax_matches_numpy"]),
    ("shared_combine_takes_min", "if (amax[(int64_t)w * nb + k] > r)", "if (amax[(int64_t)w * nb + k] < r)",
     ["test_absmax_combine_is_elementwise_max", "test_every_worker_agrees_on_the_scale"]),
    ("shared_sum_skips_first_worker", "for (int32_t w = 0; w < m; ++w)\n            t +=",
     "for (int32_t w = 1; w < m; ++w)\n            t +=", ["test_sum_int8_shared_is_the_exact_integer_sum"]),
    ("shared_sum_ignores_running_sum", "int64_t t = (accumulate && isum) ? isum[i] : 0;", "int64_t t = 0;",
     ["test_sum_int8_shared_is_the_exact_integer_sum"]),
    ("shared_decode_unsigned", "out[i] = (float)(int8_t)payload[i] * scale[i / bucket];",
     "out[i] = (float)payload[i] * scale[i / bucket];", ["test_int8_shared_on_grid_is_exact"]),
    ("shared_ef_not_updated", "ef[i] = v - (float)q * sc;", "ef[i] = v;",
     ["test_int8_shared_on_grid_is_exact", "test_int8_shared_error_bound_and_feedback"]),
    ("topk_ties_to_larger_index", "return p->idx < q->idx ? -1 : (p->idx > q->idx ? 1 : 0);",
     "return p->idx > q->idx ? -1 : (p->idx < q->idx ? 1 : 0);", ["test_brute_force_selection_tiny",
                                                                    "test_closed_forms"]),
    ("topk_smallest_first", "return p->key > q->key ? -1 : 1;", "return p->key < q->key ? -1 : 1;",
     ["test_brute_force_selection_tiny", "test_closed_forms"]),
    ("topk_key_keeps_sign", "items[j].key = f32_bits(v[j]) & 0x7FFFFFFFu;", "items[j].key = f32_bits(v[j]);",
     ["test_brute_force_selection_tiny"]),
    ("topk_one_fewer", "const int64_t kb = k < cnt ? k : cnt;", "const int64_t kb = k - 1 < cnt ? k - 1 : cnt;",
     ["test_brute_force_selection_tiny", "test_closed_forms"]),
    ("topk_ef_keeps_sent", "ef[lo + j] = v[j] - (chosen[j] ? v[j] : 0.0f);", "ef[lo + j] = v[j];",
     ["test_closed_forms", "test_error_feedback_keeps_everything"]),
    ("topk_decode_drops_bucket_offset", "                out[b * bucket + idx] = values[b * k + j];",
     "                out[idx] = values[b * k + j];", ["test_decode_places_values"]),
    ("topk_acc_skips_first_worker", "for (int32_t w = 0; w < m; ++w) {\n        const float* vw",
     "for (int32_t w = 1; w < m; ++w) {\n        const float* vw", ["test_sum_of_sparse_workers"]),
]


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def _build_mutant(mutant_dir, name, old, new):
    src = open(os.path.join(ORACLE_DIR, "qc_oracle.c")).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    d = mutant_dir / name
    d.mkdir()
    shutil.copy(os.path.join(ORACLE_DIR, "qc_oracle.h"), d / "qc_oracle.h")
    shutil.copy(os.path.join(ORACLE_DIR, "__init__.py"), d / "__init__.py")
    (d / "qc_oracle.c").write_text(src.replace(old, new))
    mod = _load(f"oracle_mutant_{name}", str(d / "__init__.py"))
    mod.build()
    mod.lib()
    return mod


def _run_pin(fn, mod, rocrand_philox):
    sig = inspect.signature(fn)
    kw = {"ora": mod}
    if "rocrand_philox" in sig.parameters:
        kw["rocrand_philox"] = rocrand_philox
    variants = [{}]
    if "bits" in sig.parameters:
        variants = [{"bits": 8}, {"bits": 4}, {"bits": 2}]
    if "fmt" in sig.parameters:
        variants = [{"fmt": f} for f in ("fp8", "qsgd", "sign", "int4")]
    if "with_ef" in sig.parameters:
        variants = [{"with_ef": False}, {"with_ef": True}]
    if "k" in sig.parameters:
        variants = [{"k": 1}, {"k": 3}, {"k": 64}]
    for v in variants:
        fn(**kw, **v)


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(mutant_dir, rocrand_philox, name, old, new, pins):
    mod = _build_mutant(mutant_dir, name, old, new)
    caught = []
    for name_ in pins:
        try:
            _run_pin(pin(name_), mod, rocrand_philox)
        except AssertionError:
            caught.append(name_)
    assert caught, f"no pin rejected mutant {name}"
