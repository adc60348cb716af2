"""Planted-mistake check of the oracle's pins (CPU only).

Each mutant is a copy of the oracle's C source with one plausible mistake
planted textually (a dropped term, a wrong sign, index or bound, a swapped
operand, a wrong decoder constant).  It is compiled to a temporary library and
the pin suite must fail on it.  The real oracle is never modified.
"""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = {
    "scale_dropped": ("s[j - lo] = scale * dot;", "s[j - lo] = dot;"),
    "causal_excludes_self": ("*hi = causal ? (pos < Nk - 1 ? pos : Nk - 1) : Nk - 1;",
                             "*hi = causal ? (pos - 1 < Nk - 1 ? pos - 1 : Nk - 1) : Nk - 1;"),
    "causal_sees_next": ("*hi = causal ? (pos < Nk - 1 ? pos : Nk - 1) : Nk - 1;",
                         "*hi = causal ? (pos + 1 < Nk - 1 ? pos + 1 : Nk - 1) : Nk - 1;"),
    "window_one_wider": ("*lo = pos - window + 1;", "*lo = pos - window;"),
    "window_condition_off": ("if (window > 0 && pos - window + 1 > 0)", "if (window > 0 && pos - window > 0)"),
    "decode_top_left": ("int64_t pos = Nk - Nq + i;", "int64_t pos = i;"),
    "decode_offset_one_short": ("int64_t pos = Nk - Nq + i;", "int64_t pos = Nk - Nq + i - 1;"),
    "paged_slot_from_page_index": ("int64_t src = ((page * Hkv + hk) * page_size + j % page_size) * d;",
                                   "int64_t src = ((page * Hkv + hk) * page_size + j / page_size) * d;"),
    "paged_head_major_pool": ("int64_t src = ((page * Hkv + hk) * page_size + j % page_size) * d;",
                              "int64_t src = ((hk * Hkv + page) * page_size + j % page_size) * d;"),
    "paged_table_by_slot": ("int64_t page = block_table[b * max_pages + j / page_size];",
                            "int64_t page = block_table[b * max_pages + j % page_size];"),
    "kv_head_stride_uses_nq": ("int64_t kvhead = (b * Hkv + hk) * Nk * d;",
                               "int64_t kvhead = (b * Hkv + hk) * Nq * d;"),
    "gqa_modulo_map": ("int64_t hk = h / group;", "int64_t hk = h % Hkv;"),
    "k_v_swapped": ("dot += qrow[c] * load_elem(k, dtype, kvhead + j * d + c);",
                    "dot += qrow[c] * load_elem(v, dtype, kvhead + j * d + c);"),
    "key_row_dropped": ("dot += qrow[c] * load_elem(k, dtype, kvhead + j * d + c);",
                        "dot += qrow[c] * load_elem(k, dtype, kvhead + c);"),
    "exp_sign_flipped": ("double e = exp(s[j - lo] - m);", "double e = exp(m - s[j - lo]);"),
    "no_normalisation": ("o_row[c] /= l;", "o_row[c] /= 1.0;"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "lse_log2": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "value_row_wrong": ("o_row[c] += e * load_elem(v, dtype, kvhead + j * d + c);",
                        "o_row[c] += e * load_elem(v, dtype, kvhead + lo * d + c);"),
    "f16_bias_off": ("mag = ldexp((double)(frac | 0x400), expo - 25);",
                     "mag = ldexp((double)(frac | 0x400), expo - 24);"),
    "bf16_bias_off": ("mag = ldexp((double)(frac | 0x80), expo - 134);",
                      "mag = ldexp((double)(frac | 0x80), expo - 133);"),
    "f16_subnormal_off": ("mag = ldexp((double)frac, -24);", "mag = ldexp((double)frac, -25);"),
    "bwd_jacobian_term_dropped": ("double ds = p * (dp[j - lo] - dsum);", "double ds = p * dp[j - lo];"),
    "bwd_jacobian_sign_flipped": ("double ds = p * (dp[j - lo] - dsum);", "double ds = p * (dsum - dp[j - lo]);"),
    "bwd_dq_scale_dropped": ("dq_row[c] += scale * ds * load_elem(k, dtype, kvhead + j * d + c);",
                             "dq_row[c] += ds * load_elem(k, dtype, kvhead + j * d + c);"),
    "bwd_dq_uses_v": ("dq_row[c] += scale * ds * load_elem(k, dtype, kvhead + j * d + c);",
                      "dq_row[c] += scale * ds * load_elem(v, dtype, kvhead + j * d + c);"),
    "bwd_dk_uses_dout": ("dk_head[j * d + c] += scale * ds * qrow[c];", "dk_head[j * d + c] += scale * ds * dorow[c];"),
    "bwd_dv_uses_ds": ("dv_head[j * d + c] += p * dorow[c];", "dv_head[j * d + c] += ds * dorow[c];"),
    "bwd_dp_uses_k": ("g += dorow[c] * load_elem(v, dtype, kvhead + j * d + c);",
                      "g += dorow[c] * load_elem(k, dtype, kvhead + j * d + c);"),
    "bwd_unnormalised_p": ("double p = exp(s[j - lo] - m) / l;", "double p = exp(s[j - lo] - m);"),
    "bwd_gqa_first_head_only": ("for (int64_t h = hk * group; h < (hk + 1) * group; ++h)\n                    for (int64_t i = 0; i < N; ++i)\n                        bwd_row",
                                "for (int64_t h = hk * group; h < hk * group + 1; ++h)\n                    for (int64_t i = 0; i < N; ++i)\n                        bwd_row"),
    "bwd_gqa_modulo_map": ("int64_t hk = h / (Hq / Hkv);", "int64_t hk = h % Hkv;"),
    "bwd_scores_use_v": ("dot += load_elem(k, dtype, kvhead + j * d + c) * qrow[c];",
                         "dot += load_elem(v, dtype, kvhead + j * d + c) * qrow[c];"),
    "bwd_keys_scale_dropped": ("double p = exp((double)scale * dot - lse[row]);", "double p = exp(dot - lse[row]);"),
    "bwd_keys_jacobian_dropped": ("double ds = p * (g - drow[row]);", "double ds = p * g;"),
    "max_not_tracked": ("if (s[j - lo] > m)\n            m = s[j - lo];", "if (j == lo)\n            m = s[j - lo];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    so = oracle.build(force=True, src=str(mutant_src), out=str(tmp_path / "libmutant.so"))
    lib = oracle.load_library(so)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError) as e:
            # a pin that fails, or an oracle that rejects what it computes
            caught.append(f"{pin.__name__}: {str(e)[:80]}")
    assert caught, f"no pin caught mutant {name}"
