"""The oracle's pins must catch plausible mistakes in the oracle.

Each case copies oracle.cpp, plants one mistake (a dropped term, a wrong
sign, a wrong index, a transposed operand, a wrong rounding), builds the
copy with the same flags, and runs the fast pins against it: at least one
must fail. The planted mistakes live only in the temporary copies.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle as oracle_pkg
from tests import test_oracle_pins as pins

MUTANTS = {
    "drop_last_token_in_pv": ("for (int t = 0; t < L; ++t) acc +=", "for (int t = 0; t < L - 1; ++t) acc +="),
    "exp_sign_flipped": ("std::exp(s[(size_t)t] - m)", "std::exp(m - s[(size_t)t])"),
    "no_max_shift": ("std::exp(s[(size_t)t] - m)", "std::exp(s[(size_t)t])"),
    "min_instead_of_max": ("if (s[(size_t)t] > m) m", "if (s[(size_t)t] < m) m"),
    "scale_dropped": ("s[(size_t)t] = scale * dot;", "s[(size_t)t] = dot;"),
    "no_normalisation": ("o[d] = acc / l;", "o[d] = acc;"),
    "denominator_not_summed": ("l += p[(size_t)t];", "l = p[(size_t)t];"),
    "group_mapping_modulo": ("h = (int)(item % Hq), g = h / nrep;", "h = (int)(item % Hq), g = h % Hkv;"),
    "table_index_modulo": ("half_bits_to_float(k_pool[k_index(table[t / bs]", "half_bits_to_float(k_pool[k_index(table[t % bs]"),
    "k_slot_channel_swapped": ("(size_t)t * 8 +\n           (size_t)(d % 8);", "(size_t)(d % 8) * 8 +\n           (size_t)t;"),
    "v_layout_transposed": (
        "((size_t)(blk * Hkv + g) * (size_t)D + (size_t)d) * (size_t)bs + (size_t)t;",
        "((size_t)(blk * Hkv + g) * (size_t)bs + (size_t)t) * (size_t)D + (size_t)d;",
    ),
    "query_row_from_kv_head": ("q + ((size_t)b * Hq + h) * D, seq_lens[b]", "q + ((size_t)b * Hq + g) * D, seq_lens[b]"),
    "append_slot_off_by_one": ("const int slot = pos % bs;", "const int slot = (pos + 1) % bs;"),
    "append_position_is_length": ("const int pos = L - 1;\n        const int logical", "const int pos = L - 2 + (L == 1);\n        const int logical"),
    "subnormal_scale": ("5.9604644775390625e-08f", "1.1920928955078125e-07f"),
    "exponent_bias": ("((expo - 15 + 127) << 23)", "((expo - 14 + 127) << 23)"),
    "round_half_up": ("if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1;", "if (rem >= 0x1000u) h += 1;"),
    "copy_direction_swapped": (
        "k_pool[k_index(t, g, slot, d, Hkv, D, bs)] = k_pool[k_index(s, g, slot, d, Hkv, D, bs)];",
        "k_pool[k_index(s, g, slot, d, Hkv, D, bs)] = k_pool[k_index(t, g, slot, d, Hkv, D, bs)];",
    ),
    "copy_skips_last_slot": ("for (int slot = 0; slot < bs; ++slot)\n                for (int d = 0; d < D; ++d) {\n"
                             "                    k_pool[k_index(t,",
                             "for (int slot = 0; slot < bs - 1; ++slot)\n                for (int d = 0; d < D; ++d) {\n"
                             "                    k_pool[k_index(t,"),
    "scatter_keeps_left_padding": ("const size_t s = (size_t)(S - P + t);", "const size_t s = (size_t)t;"),
    "scatter_slot_off_by_one": ("k_pool[k_index(blk, g, t % bs, d, Hkv, D, bs)] = k_src[i];",
                                "k_pool[k_index(blk, g, (t + 1) % bs, d, Hkv, D, bs)] = k_src[i];"),
    "copy_first_head_only": ("for (int g = 0; g < Hkv; ++g)\n            for (int slot = 0; slot < bs; ++slot)\n"
                             "                for (int d = 0; d < D; ++d) {\n                    k_pool[k_index(t,",
                             "for (int g = 0; g < 1; ++g)\n            for (int slot = 0; slot < bs; ++slot)\n"
                             "                for (int d = 0; d < D; ++d) {\n                    k_pool[k_index(t,"),
    "fp8_exponent_bias": ("std::ldexp((float)(8 + m), e - 10)", "std::ldexp((float)(8 + m), e - 11)"),
    "fp8_subnormal_scale": ("std::ldexp((float)m, -9)", "std::ldexp((float)m, -10)"),
    "fp8_ties_away_from_zero": ("(dc == db && (c & 1) == 0)", "(dc == db)"),
    "fp8_overflow_to_nan": ("if (a >= 448.0) return sign | 0x7e;", "if (a >= 448.0) return 0x7f;"),
    "fp8_sign_dropped": ("return (uint8_t)(sign | best);", "return (uint8_t)best;"),
    "fp8_quantize_multiplies": ("half_bits_to_float(x) / s", "half_bits_to_float(x) * s"),
    "fp8_k_scale_dropped": ("k_index8(table[t / bs], g, t % bs, d, Hkv, D, bs)]) * k_scale;",
                            "k_index8(table[t / bs], g, t % bs, d, Hkv, D, bs)]);"),
    "fp8_v_scaled_by_k_scale": ("v_index(table[t / bs], g, t % bs, d, Hkv, D, bs)]) * v_scale;",
                                "v_index(table[t / bs], g, t % bs, d, Hkv, D, bs)]) * k_scale;"),
    "fp8_k_group_of_8": ("(size_t)(d / 16)) * (size_t)bs * 16 + (size_t)t * 16 +", "(size_t)(d / 16)) * (size_t)bs * 16 + (size_t)t * 8 +"),
    "fp8_scatter_keeps_left_padding": ("const size_t i = (((size_t)b * Hkv + g) * S + (size_t)(S - P + t)) * D + d;",
                                       "const size_t i = (((size_t)b * Hkv + g) * S + (size_t)t) * D + d;"),
    "fp8_scatter_v_with_k_scale": ("quantize_fp8(v_src[i], v_scale)", "quantize_fp8(v_src[i], k_scale)"),
    "fp8_copy_first_head_only": ("for (int g = 0; g < Hkv; ++g)\n            for (int slot = 0; slot < bs; ++slot)\n"
                                 "                for (int d = 0; d < D; ++d) {\n                    k_pool[k_index8(t,",
                                 "for (int g = 0; g < 1; ++g)\n            for (int slot = 0; slot < bs; ++slot)\n"
                                 "                for (int d = 0; d < D; ++d) {\n                    k_pool[k_index8(t,"),
    "fp8_copy_direction_swapped": (
        "k_pool[k_index8(t, g, slot, d, Hkv, D, bs)] = k_pool[k_index8(s, g, slot, d, Hkv, D, bs)];",
        "k_pool[k_index8(s, g, slot, d, Hkv, D, bs)] = k_pool[k_index8(t, g, slot, d, Hkv, D, bs)];",
    ),
    "fp8_append_slot_off_by_one": ("k_pool[k_index8(blk, g, pos % bs, d", "k_pool[k_index8(blk, g, (pos + 1) % bs, d"),
    "fp8_append_v_with_k_scale": ("quantize_fp8(v_new[i], v_scale)", "quantize_fp8(v_new[i], k_scale)"),
}

FAST_PINS = [
    (pins.test_half_to_float_all_patterns, {}),
    (pins.test_float_to_half_rne, {}),
    (pins.test_paged_matches_float64_dense, {"name": "tiny"}),
    (pins.test_paged_matches_float64_dense, {"name": "mixed_small"}),
    (pins.test_paged_matches_float64_dense, {"name": "bs16_small"}),
    (pins.test_single_token_returns_v0, {}),
    (pins.test_two_tokens_logistic, {}),
    (pins.test_dominant_key_without_overflow, {}),
    (pins.test_all_scores_very_negative, {}),
    (pins.test_query_head_to_kv_head_mapping, {}),
    (pins.test_block_relabelling_invariance, {}),
    (pins.test_kv_append_matches_numpy_scatter, {"cfg": "tiny"}),
    (pins.test_kv_append_then_attention_sees_new_token, {}),
    (pins.test_kv_copy_blocks_matches_numpy, {"shape": (2, 128, 64)}),
    (pins.test_kv_scatter_prefill_drops_the_left_padding, {}),
    (pins.test_fp8_to_float_all_codes, {}),
    (pins.test_float_to_fp8_matches_torch_in_range, {}),
    (pins.test_float_to_fp8_saturates, {}),
    (pins.test_fp8_quantization_error_bound, {}),
    (pins.test_kv_append_fp8_matches_numpy, {}),
    (pins.test_fp8_attention_equals_fp16_oracle_on_exact_pools, {}),
    (pins.test_fp8_attention_matches_float64_dense, {}),
    (pins.test_kv_copy_blocks_fp8_matches_numpy, {}),
    (pins.test_kv_scatter_prefill_fp8_reads_back_quantized, {}),
]


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _failing_pins(lib_path):
    """Run the fast pins against a library build in a child process (a
    mutant may also fault); returns the failing pin names, or ["crash"]."""
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from tests.test_oracle_mutants import _run_pins\n"
        "print('FAILED=' + ','.join(_run_pins(%r)))\n" % (ROOT, lib_path)
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        return ["crash"]
    line = [x for x in r.stdout.splitlines() if x.startswith("FAILED=")][-1]
    return [x for x in line[len("FAILED="):].split(",") if x]


def _run_pins(lib_path):
    orc = oracle_pkg.Oracle(lib_path)
    failed = []
    for fn, kw in FAST_PINS:
        try:
            with np.errstate(all="ignore"):
                fn(orc, **kw)
        except (AssertionError, ValueError):
            failed.append(fn.__name__)
    return failed


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Every mutant built and run against the fast pins once, in parallel
    (each in its own child process): {name: failing pin names, or exception}."""
    src = open(oracle_pkg.SRC).read()
    root = tmp_path_factory.mktemp("mutants")

    def build(name):
        old, new = MUTANTS[name]
        if src.count(old) != 1:
            return AssertionError(f"mutation anchor for {name} not unique")
        path = root / f"{name}.cpp"
        path.write_text(src.replace(old, new))
        lib = str(root / f"lib{name}.so")
        subprocess.run(["g++", *oracle_pkg.CXXFLAGS, str(path), "-o", lib], check=True)
        return _failing_pins(lib)

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return dict(zip(sorted(MUTANTS), ex.map(build, sorted(MUTANTS))))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, mutant_results):
    failed = mutant_results[name]
    if isinstance(failed, Exception):
        raise failed
    assert failed, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_fast_pins(tmp_path):
    lib = str(tmp_path / "liboracle_copy.so")
    shutil.copy(oracle_pkg.SRC, tmp_path / "oracle_copy.cpp")
    subprocess.run(["g++", *oracle_pkg.CXXFLAGS, str(tmp_path / "oracle_copy.cpp"), "-o", lib], check=True)
    assert _failing_pins(lib) == []
