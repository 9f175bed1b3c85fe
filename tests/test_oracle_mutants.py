"""Planted mistakes: each test builds a copy of the oracle with one plausible
error (a dropped term, a wrong sign or index, a transposed operand, a broken
tie-break) and shows that at least one pin rejects it. The real oracle source
is never modified; the copies live in a temporary directory."""
import os

import pytest

import oracle
import oracle_checks as oc

MUTANTS = {
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "tie_break_high_index": ("if (best < 0 || v[e] > v[best])", "if (best < 0 || v[e] >= v[best])"),
    "down_weight_transposed": ("wd_off + (size_t)c * d_ff + f", "wd_off + (size_t)f * d + c"),
    "sigmoid_bias_dropped": ("v[e] = sigmoidf_canon(l[e]) + bias[e];", "v[e] = sigmoidf_canon(l[e]);"),
    "weights_from_biased_values": ("w[j] = sigmoidf_canon(l[idx[j]]);", "w[j] = v[idx[j]];"),
    "logit_chain_descending": ("for (jj = 0; jj < d; jj++) {", "for (jj = d - 1; jj >= 0; jj--) {"),
    "exp_taylor_term_dropped": ("p = fmaf(p, r, C4);", "p = fmaf(p, r, 0.0f);"),
    "exp_reduction_sign": ("r = fmaf(-n, LN2_LO, r);", "r = fmaf(n, LN2_LO, r);"),
    "shared_expert_dropped": ("acc += s[(size_t)i * d + c];", "acc += 0.0;"),
    "dispatch_unstable": ("row_of[t * k + j] = offsets[e] + cursor[e]++;",
                          "row_of[t * k + j] = offsets[e + 1] - 1 - cursor[e]++;"),
    "renorm_sum_drops_slot": ("                s += w[j];\n            }\n            for (j = 0; j < k; j++)\n"
                              "                w[j] = w[j] / s;",
                              "                s += j ? w[j] : 0.0f;\n            }\n            for (j = 0; j < k; j++)\n"
                              "                w[j] = w[j] / s;"),
    "softmax_bias_on_logits": ("v[e] = oracle_cexpf(l[e] - m) / z + bias[e];", "v[e] = l[e] + bias[e];"),
    "gate_up_swapped_roles": ("double h = silu(g[b]) * u[b];", "double h = silu(u[b]) * g[b];"),
    "bias_update_starved_le": ("if (p < starved)", "if (p <= starved)"),
    "bias_update_sign": ("float err = target - p;", "float err = p - target;"),
    "bias_update_no_upper_clamp": ("        if (bias[e] > 10.0f)\n            bias[e] = 10.0f;\n", ""),
    "bias_update_boost_dropped": ("err = err + 0.5f;", "err = err + 0.0f;"),
    "metrics_cv_biased_std": ("sqrt(var / (double)(E - 1))", "sqrt(var / (double)E)"),
    "metrics_entropy_unnormalised": ("double p = (P[e] > 1e-9 ? P[e] : 1e-9) / psum;",
                                     "double p = (P[e] > 1e-9 ? P[e] : 1e-9);"),
    "metrics_aux_fraction_of_pairs": ("aux += (cnt[e] / (double)T) * P[e];",
                                      "aux += (cnt[e] / (double)(T * k)) * P[e];"),
    "metrics_z_without_max": ("lse = m + log(s);", "lse = log(s);"),
    "logit_bias_dropped": ("            v[e] = l[e] + bias[e];\n", "            v[e] = l[e];\n"),
    "noise_dropped": ("v[e] = v[e] + noise[e];", "v[e] = v[e] + 0.0f;"),
    "bwd_silu_prime_dropped": ("dg[f] = dh * u[f] * s * (1.0 + g[f] * (1.0 - s));", "dg[f] = dh * u[f] * s;"),
    "bwd_du_from_u": ("du[f] = dh * g[f] * s;", "du[f] = dh * u[f] * s;"),
    "bwd_softmax_jacobian_sign": ("dl[idx[j]] += exp((double)l[idx[j]] - mk) / zk * (dtw[j] - dot);",
                                  "dl[idx[j]] += exp((double)l[idx[j]] - mk) / zk * (dtw[j] + dot);"),
    "bwd_sigmoid_renorm_cross_term": ("dl[idx[j]] += (dtw[j] / D - dot / (D * D)) * s * (1.0 - s);",
                                      "dl[idx[j]] += (dtw[j] / D) * s * (1.0 - s);"),
    "bwd_zloss_factor": ("dl[e] += z_coef * 2.0 * lse * p[e] / (double)T;", "dl[e] += z_coef * lse * p[e] / (double)T;"),
    "bwd_router_dx_dropped": ("da[c] += dl[(size_t)t * E + j] * (double)w_router[(size_t)j * d + c];",
                              "da[c] += 0.0 * w_router[(size_t)j * d + c];"),
    "bwd_weight_grad_unweighted": ("                    wt = (double)w[tt * k + j];", "                    wt = 1.0;"),
    "count_off_by_one": ("        counts[idx[t]]++;\n    if (!logits_out)",
                         "        counts[idx[t] == 0 ? 1 : idx[t]]++;\n    if (!logits_out)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = os.path.join(tmp_path, f"oracle_{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = oracle.load(oracle.build(path, os.path.join(tmp_path, f"liboracle_{name}.so")))
    failures = []
    for check in oc.ALL_CHECKS:
        try:
            check(lib)
        except AssertionError as e:
            failures.append(f"{check.__name__}: {str(e)[:80]}")
    assert failures, f"mutant {name} passed every pin"
