"""The oracle pins bite: plant a plausible mistake in a copy of the oracle's C
source, build the copy with gcc, and require at least one pin to fail.

Nothing here touches the GPU or the real oracle library."""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTATIONS = {
    "nibble_order_swapped": ("int nib = (i % 2 == 0) ? (b & 0x0F) : (b >> 4);",
                             "int nib = (i % 2 == 0) ? (b >> 4) : (b & 0x0F);"),
    "offset_7_not_8": ("return nib - 8;", "return nib - 7;"),
    "twos_complement_nibbles": ("return nib - 8;", "return (nib >= 8) ? nib - 16 : nib;"),
    "per_row_scale_for_fmt4": ("return (double)s[o * ng + i / gs];", "return (double)s[o * ng];"),
    "group_index_off": ("return (double)s[o * ng + i / gs];", "return (double)s[o * ng + (i + 1) / gs - ((i + 1) / gs == ng)];"),
    "fmt3_bit_order": ("int code = (b >> (2 * (i % 4))) & 0x3;", "int code = (b >> (6 - 2 * (i % 4))) & 0x3;"),
    "fmt3_offset": ("return code - 2;", "return code - 1;"),
    "fmt1_unsigned": ("return (int)(int8_t)row[i];", "return (int)row[i];"),
    "odd_tail_dropped": ("for (int64_t i = 0; i < I; i++) {\n        double w = weight_value",
                         "for (int64_t i = 0; i < (I / 2) * 2; i++) {\n        double w = weight_value"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "combine_ignores_w": ("acc += (double)w[p] * ybuf[p * nout + r];", "acc += ybuf[p * nout + r];"),
    "up_gets_silu": ("h[j] = oracle_silu(g[j]) * u[j];", "h[j] = g[j] * oracle_silu(u[j]);"),
    "router_ties_to_larger_index": ("if (!taken[e] && (best < 0 || c[e] > c[best]))",
                                    "if (!taken[e] && (best < 0 || c[e] >= c[best]))"),
    "router_weight_includes_bias": ("w[s * K + k] = pr[best];", "w[s * K + k] = c[best];"),
    "router_topp_strict": ("if (run >= topp * total) {", "if (run > topp * total) {"),
    "router_no_sigmoid": ("pr[e] = 1.0 / (1.0 + exp(-acc));", "pr[e] = acc;"),
    "router_topp_on_biased_keys": ("run += w[s * K + k];", "run += c[ids[s * K + k]];"),
    "rmsnorm_sum_not_mean": ("const double inv = 1.0 / sqrt(ss / (double)D + eps);",
                             "const double inv = 1.0 / sqrt(ss + eps);"),
    "rmsnorm_eps_outside_sqrt": ("const double inv = 1.0 / sqrt(ss / (double)D + eps);",
                                 "const double inv = 1.0 / (sqrt(ss / (double)D) + eps);"),
    "rmsnorm_weight_dropped": ("y[s * D + d] = (double)xr[d] * inv * (w ? (double)w[d] : 1.0);",
                               "y[s * D + d] = (double)xr[d] * inv;"),
    "route_unstable": ("for (int64_t p = 0; p < S * K; p++) {\n            int32_t e = ids[p];\n            if (e >= 0 && e < E)\n                perm",
                       "for (int64_t p = S * K - 1; p >= 0; p--) {\n            int32_t e = ids[p];\n            if (e >= 0 && e < E)\n                perm"),
    # MLA decode attention
    "rope_sign": ("out[2 * i] = a * c - b * s;", "out[2 * i] = a * c + b * s;"),
    "rope_frequency": ("pow(theta, -(double)(2 * i) / (double)(2 * npair))",
                       "pow(theta, -(double)(i) / (double)(2 * npair))"),
    "causal_exclusive": ("if (t <= pos_base + s) {", "if (t < pos_base + s) {"),
    "mla_scale_nope_only": ("1.0 / sqrt((double)(dn + dr))", "1.0 / sqrt((double)dn)"),
    "kvb_value_rows_first": ("double w = qt_w(kv_b, h * (dn + dv) + j, c);",
                             "double w = qt_w(kv_b, h * (dn + dv) + dv + j, c);"),
    "latent_norm_weight_dropped": ("rms_f64(ckv + s * (L + dr), L, kv_norm, eps, tmp);",
                                   "rms_f64(ckv + s * (L + dr), L, NULL, eps, tmp);"),
    "rotary_key_not_rotated": ("oracle_rope(ckv + s * (L + dr) + L, dr / 2, pos, theta, tmp);",
                               "oracle_rope(ckv + s * (L + dr) + L, dr / 2, 0, theta, tmp);"),
    "query_rotary_from_nope_part": ("oracle_rope(q + s * nq + h * (dn + dr) + dn, dr / 2,",
                                    "oracle_rope(q + s * nq + h * (dn + dr), dr / 2,"),
    "softmax_sum_misses_last_key": ("for (int64_t t = 0; t < n; t++)\n                sum += exp(z[t] - mx);",
                                    "for (int64_t t = 0; t + 1 < n; t++)\n                sum += exp(z[t] - mx);"),
    "clat_unweighted": ("double v = p[(s * H + h) * Ts + t] * (double)Lc[t * L + c];",
                        "double v = (double)Lc[t * L + c];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path):
    old, new = MUTATIONS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found in the oracle source"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    lib = oracle.build(str(path), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib_path=lib, nthreads=1)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutation {name}"
