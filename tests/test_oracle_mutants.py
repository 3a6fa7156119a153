"""Plausible mistakes planted in copies of the oracle must each fail a pin.

Each mutant is a text edit of oracle/oracle.c compiled into a temporary
library on the CPU; the real oracle is never modified. Every edit keeps all
memory accesses in bounds.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import pins

MUTANTS = {
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "gate_up_swapped": ("a[f] = silu(a[f]) * b[f];", "a[f] = silu(b[f]) * a[f];"),
    "gate_dropped": ("o[n] += g * y[n];", "o[n] += y[n];"),
    "gate_index_reversed": ("double g = jb->weights[s * k + j];", "double g = jb->weights[s * k + (k - 1 - j)];"),
    "tie_to_higher_id": ("if (best < 0 || l[e] > l[best]) best = e;", "if (best < 0 || l[e] >= l[best]) best = e;"),
    "topk_ascending": ("if (best < 0 || l[e] > l[best]) best = e;", "if (best < 0 || l[e] < l[best]) best = e;"),
    "softmax_unnormalised": ("for (int64_t j = 0; j < k; ++j) w[j] /= z;", "for (int64_t j = 0; j < k; ++j) w[j] /= 1.0;"),
    "softmax_missing_max_term": ("w[j] = exp(l[ids[j]] - m);", "w[j] = exp(l[ids[j]] - m) + (j == 0 ? 1e-9 : 0.0);"),
    "w1_transposed": ("a[f] += xv * bf16_to_double(r1[f]);", "a[f] += xv * bf16_to_double(w1e[f * D + d]);"),
    "w_gate_transposed": ("for (int64_t e = 0; e < E; ++e) l[e] += xv * bf16_to_double(wrow[e]);",
                          "for (int64_t e = 0; e < E; ++e) l[e] += xv * bf16_to_double(wg[(e * D + d) % (D * E)]);"),
    "down_first_term_dropped": ("for (int64_t f = 0; f < F; ++f) {\n        double hv = a[f];",
                                "for (int64_t f = 1; f < F; ++f) {\n        double hv = a[f];"),
    "wrong_expert_slab": ("jb->w2 + e * F * D", "jb->w2 + ((e + 1) % jb->E) * F * D"),
    "map_unstable": ("for (int64_t f = 0; f < n; ++f) {\n        int32_t slot = next[ids[f]]++;",
                     "for (int64_t f = n - 1; f >= 0; --f) {\n        int32_t slot = next[ids[f]]++;"),
    "offsets_off_by_one": ("offsets[e + 1] = offsets[e] + counts[e];",
                           "offsets[e + 1] = offsets[e] + counts[e] - (e == 0 && counts[0] > 0);"),
    "x_row_of_wrong_token": ("expert_row(jb->x + s * D,", "expert_row(jb->x + (s > 0 && j == 1 ? s - 1 : s) * D,"),
    # ParallelLinear forward and backward
    "pl_gate_dropped": ("for (int64_t n = 0; n < D_out; ++n) o[n] += g * z[n];",
                        "for (int64_t n = 0; n < D_out; ++n) o[n] += z[n];"),
    "pl_grouped_out_in_route_order": ("double *o = grouped_out ? y + r * D_out : y + t * D_out;",
                                      "double *o = grouped_out ? y + f * D_out : y + t * D_out;"),
    "pl_w_row_off_by_one": ("const uint16_t *wr = we + d * D_out;\n        for (int64_t n = 0; n < D_out; ++n) z[n]",
                            "const uint16_t *wr = we + ((d + 1) % D_in) * D_out;\n        for (int64_t n = 0; n < D_out; ++n) z[n]"),
    "pl_bwd_w_not_transposed": ("s += bf16_to_double(dy[n]) * bf16_to_double(wr[n]);",
                                "s += bf16_to_double(dy[n]) * bf16_to_double(we[(n * D_in + d) % (D_in * D_out)]);"),
    "pl_bwd_dx_gate_dropped": ("for (int64_t i = 0; i < D_in; ++i) o[i] += g * c[i];",
                               "for (int64_t i = 0; i < D_in; ++i) o[i] += c[i];"),
    "pl_bwd_dx_grouped_in_route_order": ("double *o = grouped_in ? dx + r * D_in : dx + t * D_in;",
                                         "double *o = grouped_in ? dx + f * D_in : dx + t * D_in;"),
    "pl_bwd_dw_gate_dropped": ("double xa = g * bf16_to_double(in[a]);", "double xa = bf16_to_double(in[a]);"),
    "pl_bwd_dw_wrong_expert": ("double *we = dw + e * D_in * D_out;", "double *we = dw + ((e + 1) % E) * D_in * D_out;"),
    "pl_bwd_dg_gated": ("s += bf16_to_double(d[b]) * c[b];", "s += (gates ? gates[f] : 1.0) * bf16_to_double(d[b]) * c[b];"),
    # expert FFN backward
    "ffn_bwd_silu_prime_wrong": ("da[c] = dh[c] * b[c] * sg * (1.0 + a[c] * (1.0 - sg));",
                                 "da[c] = dh[c] * b[c] * sg * (1.0 + a[c] * sg);"),
    "ffn_bwd_da_db_swapped": ("db[c] = dh[c] * silu(a[c]);", "db[c] = dh[c] * b[c];"),
    "ffn_bwd_dh_gate_dropped": ("for (int64_t n = 0; n < D; ++n) s += g * go[n] * bf16_to_double(w2e[c * D + n]);",
                                "for (int64_t n = 0; n < D; ++n) s += go[n] * bf16_to_double(w2e[c * D + n]);"),
    "ffn_bwd_dx_w3_term_dropped": ("s += da[c] * bf16_to_double(w1e[d * F + c]) + db[c] * bf16_to_double(w3e[d * F + c]);",
                                   "s += da[c] * bf16_to_double(w1e[d * F + c]);"),
    "ffn_bwd_dw2_gate_dropped": ("dw2[e * F * D + c * D + n] += h[c] * g * go[n];",
                                 "dw2[e * F * D + c * D + n] += h[c] * go[n];"),
    "ffn_bwd_dw1_uses_db": ("if (dw1) dw1[e * D * F + d * F + c] += xv * da[c];",
                            "if (dw1) dw1[e * D * F + d * F + c] += xv * db[c];"),
    "ffn_bwd_dg_uses_h": ("for (int64_t n = 0; n < D; ++n) s += go[n] * y[n];",
                          "for (int64_t n = 0; n < D && n < F; ++n) s += go[n] * h[n];"),
    "ffn_bwd_w2_not_transposed": ("for (int64_t n = 0; n < D; ++n) s += g * go[n] * bf16_to_double(w2e[c * D + n]);",
                                  "for (int64_t n = 0; n < D; ++n) s += g * go[n] * bf16_to_double(w2e[(n * F + c) % (F * D)]);"),
    "pl_bwd_dg_first_term_dropped": ("for (int64_t b = 0; b < D_out; ++b) s += bf16_to_double(d[b]) * c[b];",
                                     "for (int64_t b = 1; b < D_out; ++b) s += bf16_to_double(d[b]) * c[b];"),
}


@pytest.fixture(scope="module")
def src_text():
    with open(oracle.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(src_text, name):
    old, new = MUTANTS[name]
    assert src_text.count(old) == 1, f"mutation anchor for {name} not unique"
    with tempfile.TemporaryDirectory() as td:
        src = os.path.join(td, "mutant.c")
        lib = os.path.join(td, "libmutant.so")
        with open(src, "w") as f:
            f.write(src_text.replace(old, new))
        oracle.build(src=src, out=lib)
        mut = oracle.Oracle(lib)
        failed = []
        for pin in pins.ALL_PINS:
            try:
                pin(mut)
            except (AssertionError, ValueError, IndexError):
                failed.append(pin.__name__)
        assert failed, f"mutant {name} passed every pin"
