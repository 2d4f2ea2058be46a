"""Planted mistakes in a copy of the oracle must each be caught by some pin.

Each mutant is one plausible slip (a dropped term, a wrong sign or index, a
transposed operand, an off-by-one in a mask).  The copy is compiled on the CPU
into a temporary directory; the real oracle is untouched.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = {
    "gqa_index_modulo": ("const int kh = h / G;", "const int kh = h % Hkv;"),
    "causal_top_left": ("((long long)S - n_reg - L);  /* bottom-right */", "0;"),
    "window_off_by_one": ("if (window > 0 && ip - r >= window) return 0;",
                          "if (window > 0 && ip - r > window) return 0;"),
    "registers_masked": ("if (j < n_reg) return 1;                 /* register tokens: always visible */", ""),
    "sink_dropped_from_denominator": ("if (sink) D += exp(sink[h] - M);", ""),
    "sink_sign": ("if (sink) D += exp(sink[h] - M);", "if (sink) D += exp(-sink[h] - M);"),
    "rbf_sign": ("return -gamma * acc;", "return gamma * acc;"),
    "rbf_plus": ("double d = load_elem(dtype, q, qoff + e) - load_elem(dtype, k, koff + e);",
                 "double d = load_elem(dtype, q, qoff + e) + load_elem(dtype, k, koff + e);"),
    "scale_dropped": ("return scale * acc;", "return acc;"),
    "key_row_reversed": ("z[j] = logit(dtype, q, qoff, k, (kvrow0 + j) * E, E, mode, scale, gamma) + b;",
                         "z[j] = logit(dtype, q, qoff, k, (kvrow0 + (S - 1 - j)) * E, E, mode, scale, gamma) + b;"),
    "bias_sign": ("scale, gamma) + b;", "scale, gamma) - b;"),
    "bool_mask_inverted": ("((const unsigned char*)bias)[idx] ? 0.0 : -INFINITY;",
                           "((const unsigned char*)bias)[idx] ? -INFINITY : 0.0;"),
    "key_len_ignored": ("const int padded = key_len && j >= n_reg && (j - n_reg) >= key_len[n];",
                        "const int padded = 0;"),
    "bias_head_stride_dropped": ("(long long)h * sh +", ""),
    "bwd_delta_dropped": ("dlogit_dq(dtype, q, (size_t)flat * E, k, koff, E, mode, scale, gamma, p * (dp - DEL[flat]), g);",
                          "dlogit_dq(dtype, q, (size_t)flat * E, k, koff, E, mode, scale, gamma, p * dp, g);"),
    "bwd_rbf_dk_sign": ("g[e] += w * (2.0 * gamma) * (qe - load_elem(dtype, k, koff + e));",
                        "g[e] += w * (2.0 * gamma) * (load_elem(dtype, k, koff + e) - qe);"),
    "bwd_dsink_sign": ("dsink[h] -= exp(sink[h] - LSE[flat]) * DEL[flat];", "dsink[h] += exp(sink[h] - LSE[flat]) * DEL[flat];"),
    "bwd_gqa_one_head": ("for (int h = kh * G; h < (kh + 1) * G; ++h)", "for (int h = kh * G; h < kh * G + 1; ++h)"),
    "socket_sign_flipped": ("if (x > 0.0f) code |= 1u << b;", "if (x < 0.0f) code |= 1u << b;"),
    "socket_norm_dropped": ("scores[j] = vnorm[j] * sum;", "scores[j] = sum;"),
    "socket_tau_inverted": ("a += ((c >> b) & 1 ? 1.0 : -1.0) * y[b] / tau;", "a += ((c >> b) & 1 ? 1.0 : -1.0) * y[b] * tau;"),
    "socket_bits_reversed": ("a += ((c >> b) & 1 ? 1.0 : -1.0) * y[b] / tau;",
                             "a += ((c >> (bits - 1 - b)) & 1 ? 1.0 : -1.0) * y[b] / tau;"),
    "socket_select_ties_to_higher_index": ("return (x->idx < y->idx) ? -1 : 1;", "return (x->idx > y->idx) ? -1 : 1;"),
    "socket_select_lowest_first": ("if (x->score > y->score) return -1;", "if (x->score < y->score) return -2;"),
    "socket_hash_reverse_element_order": ("for (int e = 0; e < E; ++e) x = fmaf(",
                                          "for (int e = E - 1; e >= 0; --e) x = fmaf("),
    "socket_hash_unfused": ("x = fmaf((float)load_elem(dtype, k, (size_t)j * E + e), w[e], x);",
                            "x = x + (float)load_elem(dtype, k, (size_t)j * E + e) * w[e];"),
    "bwd_dv_unweighted": ("gv[e] += p * load_elem(dtype, dout, qoff + e);", "gv[e] += load_elem(dtype, dout, qoff + e);"),
    "head_dim_truncated": ("for (int e = 0; e < E; ++e) acc += load_elem(dtype, q, qoff + e)",
                           "for (int e = 0; e < E - 1; ++e) acc += load_elem(dtype, q, qoff + e)"),
    "lse_without_max": ("lse[r] = M + log(D);", "lse[r] = log(D);"),
    "empty_row_nan": ("if (M == -INFINITY) { /* nothing visible", "if (0) { /* nothing visible"),
    "bf16_shift": ("<< 16;", "<< 15;"),
    "value_row_index": ("const size_t voff = (kvrow0 + j) * E;", "const size_t voff = (kvrow0 + (S - 1 - j)) * E;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mpath = tmp_path / "attn_oracle_mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.bind(oracle.build(force=True, src=str(mpath), out=str(tmp_path / "libmutant.so")))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
