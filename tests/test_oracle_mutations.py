"""Plants plausible mistakes in a copy of the oracle source (on the CPU) and
checks that the pins in test_oracle_pins.py reject every one of them."""
import os
import shutil
import subprocess

import pytest

import oracle as orc
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(orc.__file__), "oda_oracle.c")

# (name, original text, mutated text, pin functions expected to catch it)
MUTATIONS = [
    ("gqa_modulo", "h / group, c->dtype, scale, ks, vs, pos, nl", "h % Hkv, c->dtype, scale, ks, vs, pos, nl",
     ["test_run_gqa_head_grouping"]),
    ("window_off_by_one", "p >= max64(1, t - c->window + 1)", "p >= max64(1, t - c->window)",
     ["worked_local"]),
    ("sink_strict", "p <= min64(c->sink, t)", "p < min64(c->sink, t)", ["worked_local"]),
    ("softmax_no_shift", "Z += exp(z[i] - m);", "Z += exp(z[i]);", ["test_attention_matches_torch_sdpa_float64"]),
    ("score_sign", "z[i] = scale * dot;", "z[i] = -scale * dot;", ["worked_attention"]),
    ("lse_drop_max", "return m + log(Z);", "return log(Z);", ["worked_attention"]),
    ("gate_ge", "return (double)score > (double)theta;", "return (double)score >= (double)theta;",
     ["test_gate_strict_threshold"]),
    ("savings_swapped", "(fired ? 0 : f_full)", "(fired ? f_full : 0)", ["worked_accounting"]),
    ("bytes_drop_full", "(nl + (fired ? nf : 0))", "(nl)", ["worked_accounting"]),
    ("bf16_shift", "<< 16;", "<< 15;", ["test_attention_matches_torch_sdpa_float64"]),
    ("focus_inclusive_end", "p < fb && p >= 1", "p <= fb && p >= 1", ["worked_focus"]),
    ("value_row_from_query_head", "const int64_t row = ((pos[i] - 1) * num_kv_heads + g) * d;\n    for (int64_t j = 0; j < d; ++j) out[j]",
     "const int64_t row = ((pos[i] - 1) * num_kv_heads) * d;\n    for (int64_t j = 0; j < d; ++j) out[j]",
     ["test_attention_matches_torch_sdpa_float64"]),
    ("fp8_bias_8", "else v = ldexp(1.0 + (double)m / 8.0, e - 7);", "else v = ldexp(1.0 + (double)m / 8.0, e - 8);",
     ["worked_fp8"]),
    ("fp8_subnormal_exponent", "if (e == 0) v = ldexp((double)m / 8.0, -6);", "if (e == 0) v = ldexp((double)m / 8.0, -7);",
     ["worked_fp8"]),
    ("fp8_no_nan", "if (e == 15 && m == 7) return NAN;", "if (e == 16 && m == 7) return NAN;", ["worked_fp8"]),
    ("fp8_k_scale_dropped", "(k_scale * widen(kv_k, dtype, row + j))", "(widen(kv_k, dtype, row + j))",
     ["fp8_sdpa"]),
    ("fp8_v_scale_dropped", "(v_scale * widen(kv_v, dtype, row + j))", "(widen(kv_v, dtype, row + j))",
     ["fp8_sdpa"]),
    ("fp8_query_read_as_fp8", "const int32_t qt = q_dtype(dtype);", "const int32_t qt = dtype;", ["fp8_sdpa"]),
    ("head_no_relu", "if (u > 0.0) acc += (double)w2[j] * u;", "acc += (double)w2[j] * u;",
     ["test_recall_head_worked_example"]),
    ("head_no_b1", "double u = (double)b1[j];", "double u = 0.0;", ["test_recall_head_worked_example"]),
    ("head_no_b2", "double acc = (double)b2;", "double acc = 0.0;", ["test_recall_head_worked_example"]),
    ("head_w1_transposed", "u += widen(row, OR_BF16, i) * widen(xb, OR_BF16, i);",
     "u += widen(w1, OR_BF16, ((int64_t)i * hidden + j) % ((int64_t)hidden * in_dim)) * widen(xb, OR_BF16, i);",
     ["test_recall_head_matches_torch_float64"]),
]


def _run_pin(name):
    g = pins._load
    if name == "worked_local":
        for case in g("access_sets.json")["local"]:
            pins.test_local_set_worked_examples(case)
    elif name == "worked_focus":
        for case in g("access_sets.json")["focus"]:
            pins.test_focus_set_worked_examples(case)
    elif name == "worked_attention":
        for case in g("attention_worked.json")["cases"]:
            pins.test_attention_worked_examples(case)
    elif name == "worked_accounting":
        for case in g("accounting.json")["cases"]:
            pins.test_accounting_worked_examples(case)
    elif name == "worked_fp8":
        for case in g("fp8_e4m3.json")["codes"]:
            pins.test_fp8_e4m3_worked_codes(case)
    elif name == "fp8_sdpa":
        pins.test_fp8_attention_matches_torch_sdpa_on_dequantised_values(64)
    elif name == "test_attention_matches_torch_sdpa_float64":
        for dt in (orc.F32, orc.BF16):
            pins.test_attention_matches_torch_sdpa_float64(dt, 64)
    else:
        getattr(pins, name)()


@pytest.mark.parametrize("mut", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_planted_mistake(mut, tmp_path):
    name, old, new, catchers = mut
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in the oracle source"
    mutated = tmp_path / "oda_oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / f"liboracle_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutated), "-lm"], check=True)
    # sanity: the unmutated pins pass on the real build
    for c in catchers:
        _run_pin(c)
    with orc.using_library(str(so)):
        caught = False
        for c in catchers:
            try:
                _run_pin(c)
            except AssertionError:
                caught = True
        assert caught, f"planted mistake {name} was not caught by {catchers}"
