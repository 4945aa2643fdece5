"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks that the pins
catch every one: a dropped term, a wrong sign or index, a transposed operand, a wrong
loop order. Each mutant is a single textual replacement in moe_oracle.c, compiled with
gcc into a temporary library."""
import os

import pytest

import oracle_pins
from oracle import ORACLE_SOURCE, Oracle, build_oracle

MUTANTS = {
    "gate_from_slot0": ("const double g = gate_eff[t * k + j];", "const double g = gate_eff[t * k + 0];"),
    "overwrite_not_accumulate": ("y[i * D + d] += g * fo[d];", "y[i * D + d] = g * fo[d];"),
    "softmax_sign": ("probs[t * E + e] = exp((double)l32[e] - m) / z;", "probs[t * E + e] = exp(m - (double)l32[e]) / z;"),
    "tie_to_higher_index": ("if (!chosen[e] && (best < 0 || val[e] > val[best])) best = e;",
                            "if (!chosen[e] && (best < 0 || val[e] >= val[best])) best = e;"),
    "priority_always_token_major": ("const int64_t t = token_major ? v / k : v % N;\n    const int32_t j = token_major ? (int32_t)(v % k) : (int32_t)(v / N);",
                                    "const int64_t t = v / k;\n    const int32_t j = (int32_t)(v % k);"),
    "priority_always_slot_major": ("const int64_t t = token_major ? v / k : v % N;\n    const int32_t j = token_major ? (int32_t)(v % k) : (int32_t)(v / N);",
                                   "const int64_t t = v % N;\n    const int32_t j = (int32_t)(v / N);"),
    "no_drop_renormalisation": ("else gate_eff[t * k + j] = g * all / kept;", "else gate_eff[t * k + j] = g;"),
    "capacity_without_k": ("ceil(((cf * (double)N) * (double)k) / (double)E)", "ceil((cf * (double)N) / (double)E)"),
    "capacity_floor": ("ceil(((cf * (double)N) * (double)k) / (double)E)", "floor(((cf * (double)N) * (double)k) / (double)E)"),
    "switch_capacity_with_k": ("ceil(((double)N / (double)E) * cf)", "ceil(((double)N / (double)E) * cf * (double)k)"),
    "switch_capacity_floor": ("ceil(((double)N / (double)E) * cf)", "floor(((double)N / (double)E) * cf)"),
    "noise_all_ignored": ("if (noisy == NOISE_ALL)\n      for (int32_t e = 0; e < E; ++e) l32[e] = l32[e] + noise[t * E + e];", ";"),
    "w3_transposed": ("out[d] += u * wel(w3, s3, w_dtype, e, f, d, F, D);",
                      "out[d] += u * wel(w3, s3, w_dtype, e, d, f, D, F);"),
    "int8_scale_by_row": ("return (double)((const int8_t*)w)[i] * (double)s[e * C + c];",
                          "return (double)((const int8_t*)w)[i] * (double)s[e * C + (r % C)];"),
    "int8_unsigned": ("return (double)((const int8_t*)w)[i] * (double)s[e * C + c];",
                      "return (double)((const uint8_t*)w)[i] * (double)s[e * C + c];"),
    "int8_scale_other_expert": ("return (double)((const int8_t*)w)[i] * (double)s[e * C + c];",
                                "return (double)((const int8_t*)w)[i] * (double)s[c];"),
    "silu_sign": ("if (kind == ACT_SILU) return z / (1.0 + exp(-z));", "if (kind == ACT_SILU) return z / (1.0 + exp(z));"),
    "gelu_scale": ("return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));", "return 0.5 * z * (1.0 + erf(z));"),
    "act_on_w2_branch": ("h[f] = oracle_act(act, h1[f]) * h2[f];", "h[f] = h1[f] * oracle_act(act, h2[f]);"),
    "combine_overwrites": ("y[t * D + d] += gate_eff[t * k + j] * y_perm[r * D + d];",
                           "y[t * D + d] = gate_eff[t * k + j] * y_perm[r * D + d];"),
    "combine_gate_slot0": ("y[t * D + d] += gate_eff[t * k + j] * y_perm[r * D + d];",
                           "y[t * D + d] += gate_eff[t * k] * y_perm[r * D + d];"),
    "rows_wrong_expert": ("w3, s3, experts[i],", "w3, s3, experts[0],"),
    "noise_on_slot0": ("val[e] = (j > 0 && noisy == NOISE_SECOND) ?", "val[e] = (noisy == NOISE_SECOND) ?"),
    "noise_second_on_all": ("val[e] = (j > 0 && noisy == NOISE_SECOND) ?", "val[e] = (j > 0 && noisy) ?"),
    "balance_f_div_n": ("b += ((double)load[e] / ((double)N * (double)k)) * P[e];", "b += ((double)load[e] / (double)N) * P[e];"),
    "mode_b_uses_probs": ("for (int32_t j = 0; j < k; ++j) gate[t * k + j] = exp((double)l32[idx[t * k + j]] - ref) / s;",
                          "for (int32_t j = 0; j < k; ++j) gate[t * k + j] = probs[t * E + idx[t * k + j]];"),
    "bias_dropped": ("if (bias) s += (double)bias[e];", ";"),
    "logits_transposed_w": ("s += elem(x, x_dtype, t * D + d) * (double)w_r[d * E + e];",
                            "s += elem(x, x_dtype, t * D + d) * (double)w_r[e * D + d];"),
    "padded_offsets_ragged": ("offsets[e] = padded ? (int64_t)e * C : run;", "offsets[e] = run;"),
    "drop_case_b_keeps_gates": ("if (nk == k) gate_eff[t * k + j] = g;",
                                "if (nk == k || nk == 0) gate_eff[t * k + j] = g;"),
    "bf16_truncated_shift": ("uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;"),
    "margin_step0_only": ("if (gap < tok_margin) tok_margin = gap;", "if (j == 0 && gap < tok_margin) tok_margin = gap;"),
    "margin_on_logits": ("double gap = (q[best] - q[second]) / vz;", "double gap = (double)val[best] - (double)val[second];"),
    "margin_on_clean_values": ("q[e] = exp((double)val[e] - vm); vz += q[e];", "q[e] = exp((double)l32[e] - vm); vz += q[e];"),
    "margin_runner_up_already_chosen": ("if (!chosen[e] && e != best && (second < 0 || val[e] > val[second])) second = e;",
                                        "if (e != best && (second < 0 || val[e] > val[second])) second = e;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(ORACLE_SOURCE).read()
    assert src.count(old) == 1, f"mutation site of {name} not found exactly once"
    mpath = os.path.join(tmp_path, "moe_oracle_mut.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    lib = build_oracle(mpath, os.path.join(tmp_path, "libmut.so"))
    orc = Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
