"""The oracle's pins are strong enough to catch plausible mistakes.

Each case plants one mistake in a private copy of ``oracle/oracle.c`` (a
dropped term, a wrong sign, index or group map, a transposed operand, a
doubled scale, a wrong dequantisation scale, a decoder off by one, int8
codes read as unsigned bytes, a causal bound off by one, query rows taken in
the wrong order, a missing length update, a log-sum-exp without its maximum or in base 2, a
merge without its normalisation or with flipped weights), builds it with gcc in a temporary directory, routes the
oracle wrapper to it and runs the pin tests of ``test_oracle.py``. At least
one pin must fail for every mutant; the unmutated copy must pass them all.
Everything runs on the CPU.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins
from tests import test_oracle_lse as lse_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "group_map_modulo": ("const int kvh = h / g; /* the KV group this query head selects */",
                         "const int kvh = h % h_kv;"),
    "transposed_K": ("acc += q[j] * K[(size_t)l * d_k + j];", "acc += q[j] * K[(size_t)j * n + l];"),
    "scale_twice": ("s[l] = scale * acc;", "s[l] = scale * scale * acc;"),
    "exp_sign": ("e[l] = exp(s[l] - m);\n        Z +=", "e[l] = exp(m - s[l]);\n        Z +="),
    "dropped_first_row_in_step3": ("for (int l = 0; l < n; ++l) acc += a[l] * V",
                                   "for (int l = 1; l < n; ++l) acc += a[l] * V"),
    "v_uses_k_scale": ("load_elem(v_cache, kv_dtype, idx) * vs;", "load_elem(v_cache, kv_dtype, idx) * ks;"),
    "fp8_bias_8": ("v = ldexp(1.0 + mant / 8.0, expo - 7);", "v = ldexp(1.0 + mant / 8.0, expo - 8);"),
    "int8_read_unsigned": ("case ORACLE_INT8: return oracle_int8_to_f64(((const int8_t *)base)[idx]);",
                           "case ORACLE_INT8: return (double)((const uint8_t *)base)[idx];"),
    "causal_bound_off_by_one": ("const int n = lens[b] - T + 1 + t;", "const int n = lens[b] - T + t + (t > 0);"),
    "query_index_swapped": ("const int t = (int)(bth / h_q % T), h = (int)(bth % h_q);",
                            "const int t = (int)(bth % T), h = (int)(bth / T % h_q);"),
    "append_no_len_update": ("lens[b] += 1;", "lens[b] += 0;"),
    "append_wrong_row": ("(slot * cap + (size_t)lens[b]) * d_k * eb", "(slot * cap + (size_t)lens[b] / 2) * d_k * eb"),
    "lse_without_max": ("lse[bth] = m + log(Z);", "lse[bth] = log(Z);"),
    "lse_log2": ("lse[bth] = m + log(Z);", "lse[bth] = m + log2(Z);"),
    "lse_causal_bound_off_by_one": ("const int n = t + 1 + lens[b] - T;", "const int n = t + lens[b] - T + (t > 0);"),
    "merge_unnormalised": ("out[(size_t)r * d + c] = acc / W;", "out[(size_t)r * d + c] = acc;"),
    "merge_lse_without_max": ("lse_out[r] = M + log(W);", "lse_out[r] = log(W);"),
    "merge_weights_flipped": ("acc += exp(lses[(size_t)p * rows + r] - M) *", "acc += exp(M - lses[(size_t)p * rows + r]) *"),
    # a rewrite that changes nothing: the control that must pass every pin
    "control_noop": ("(slot * cap + (size_t)lens[b]) * d_k * eb", "(slot * cap + (size_t)lens[b] + 0) * d_k * eb"),
}
CONTROL = "control_noop"

PINS = [
    ("worked_example", lambda gd: pins.test_worked_example_printed_values(gd)),
    ("closed_form", lambda gd: pins.test_worked_example_closed_form(gd)),
    ("brute_f32", lambda gd: [pins.test_oracle_vs_decimal_brute_force(s, "f32") for s in range(6)]),
    ("brute_fp8", lambda gd: [pins.test_oracle_vs_decimal_brute_force(s, "fp8") for s in range(3)]),
    ("brute_int8", lambda gd: [pins.test_oracle_vs_decimal_brute_force(s, "int8") for s in range(3)]),
    ("sdpa_gqa", lambda gd: pins.test_oracle_vs_torch_sdpa_fp64("gqa4", 8, 2, 128, "bf16")),
    ("special_cases", lambda gd: pins.test_special_cases_reduce_to_rows_or_mean()),
    ("fp8_codes", lambda gd: pins.test_fp8_e4m3fn_decoder_all_codes()),
    ("mq_brute", lambda gd: [pins.test_multi_query_vs_masked_brute_force(s, "f32") for s in range(4)]),
    ("mq_sdpa", lambda gd: pins.test_multi_query_vs_torch_sdpa_with_causal_mask(4, 32, 8, 128, "bf16")),
    ("append_layout", lambda gd: pins.test_append_layout_gamma_offsets(gd)),
    ("append_bits", lambda gd: pins.test_append_is_bit_exact_and_touches_only_its_rows()),
    ("lse_brute", lambda gd: [lse_pins.test_lse_vs_decimal_brute_force(s, kv) for s in range(2) for kv in ("f32", "fp8")]),
    ("lse_scipy", lambda gd: lse_pins.test_lse_vs_scipy_logsumexp("bf16")),
    ("lse_one_row", lambda gd: lse_pins.test_lse_single_row_is_its_score()),
    ("lse_out", lambda gd: lse_pins.test_lse_outputs_equal_the_decode_functions()),
    ("merge_parts", lambda gd: [lse_pins.test_merge_of_row_parts_equals_the_whole(s, "bf16") for s in range(2)]),
    ("merge_closed", lambda gd: lse_pins.test_merge_closed_forms()),
]


def _build(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = tmp_path / f"lib{name}.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", str(path), "-o", str(so), "-lm"])
    return str(so)


def _failing_pins(so, golden_dir):
    failed = []
    with oracle.using_library(so):
        for pname, fn in PINS:
            try:
                fn(golden_dir)
            except (AssertionError, ValueError):
                failed.append(pname)
    return failed


@pytest.mark.parametrize("name", sorted(k for k in MUTANTS if k != CONTROL))
def test_planted_mistake_is_caught(name, tmp_path, golden_dir):
    old, new = MUTANTS[name]
    so = _build(tmp_path, name, old, new)
    assert _failing_pins(so, golden_dir), f"mutant {name} passed every pin"


def test_unmutated_copy_passes_all_pins(tmp_path, golden_dir):
    old, new = MUTANTS[CONTROL]
    so = _build(tmp_path, CONTROL, old, new)
    assert _failing_pins(so, golden_dir) == []
