"""The pins bite: each deliberately broken build of the oracle (a plausible
mistake planted in a copy of bra_oracle.c, compiled on the CPU) must be
rejected by at least one pin."""
import os

import pytest

import oracle
import oracle_pins
from oracle.build import SRC, build_oracle

# (name, exact text in bra_oracle.c, replacement)
MUTANTS = [
    ("ties_to_higher_id", "if (best < 0 || row[s] > row[best]) best = s;",
     "if (best < 0 || row[s] >= row[best]) best = s;"),
    ("ascending_topk", "if (best < 0 || row[s] > row[best]) best = s;",
     "if (best < 0 || row[s] < row[best]) best = s;"),
    ("raster_regions", "*y = ri * hs + slot / ws;\n    *x = rj * ws + slot % ws;",
     "int tok = r * hs * ws + slot; (void)ri; (void)rj;\n"
     "    *y = tok / c->width;\n    *x = tok % c->width;"),
    ("lepe_flipped", "w[(size_t)ch * 25 + i * 5 + j]", "w[(size_t)ch * 25 + (4 - i) * 5 + (4 - j)]"),
    ("lepe_no_bias", "double s = bias ? bias[ch] : 0.0;", "double s = 0.0; (void)bias;"),
    ("lepe_clamped_border", "if (yy < 0 || yy >= H || xx < 0 || xx >= W) continue; /* zero pad */",
     "yy = yy < 0 ? 0 : (yy >= H ? H - 1 : yy); xx = xx < 0 ? 0 : (xx >= W ? W - 1 : xx);"),
    ("lepe_of_q", "int rc = oracle_lepe(c, v, w, bias, L);", "int rc = oracle_lepe(c, q, w, bias, L);"),
    ("no_softmax_scale", "logit[m] = scale * dot;", "logit[m] = dot; (void)scale;"),
    ("mean_not_divided", "xbar[(size_t)item * hd + d] = s / (double)t;",
     "xbar[(size_t)item * hd + d] = s;"),
    ("keys_from_head0", "key_at[j * t + slot] = at(ckv, b, y, x, h * hd);",
     "key_at[j * t + slot] = at(ckv, b, y, x, 0);"),
    ("no_normalisation", "ov[d] = acc[d] / denom;", "ov[d] = acc[d]; (void)denom;"),
    ("affinity_short_dot", "for (int d = 0; d < hd; ++d) a += qr[d] * ks[d];",
     "for (int d = 0; d < hd - 1; ++d) a += qr[d] * ks[d];"),
    ("affinity_transposed", "const double* ks = kbar + ((size_t)bh * R + s) * hd;",
     "const double* ks = qbar + ((size_t)bh * R + s) * hd; (void)kbar;"),
    ("k_from_q_region_means", "oracle_region_means(c, k, kb) == 0 &&\n        oracle_route(",
     "oracle_region_means(c, q, kb) == 0 &&\n        oracle_route("),
    ("kv_pool_first_only", "s += x[at(c, b, yd * ratio + u, xq * ratio + w, ch)];",
     "s += (u | w) ? 0.0 : x[at(c, b, yd * ratio, xq * ratio, ch)] * (ratio * ratio);"),
    ("kv_pool_not_divided", "xd[at(&d, b, yd, xq, ch)] = s / (double)(ratio * ratio);",
     "xd[at(&d, b, yd, xq, ch)] = s;"),
    ("kvds_without_lepe", "for (size_t i = 0; i < n; ++i) out[i] += L[i];",
     "(void)n; (void)L;"),
    ("shared_head0_only", "for (int h = 0; h < H; ++h) {\n                    const double* qh",
     "for (int h = 0; h < 1; ++h) {\n                    const double* qh"),
    ("shared_routing_per_head0",
     "full[(((size_t)b * H + h) * R + r) * kk + j] =\n                            idx[((size_t)b * R + r) * kk + j];",
     "full[(((size_t)b * H + h) * R + r) * kk + j] =\n                            idx[((size_t)b * R + (h ? 0 : r)) * kk + j];"),
    ("linear_weight_transposed", "s += x[i * in_f + ci] * w[(size_t)o * in_f + ci];",
     "s += x[i * in_f + ci] * w[(size_t)ci * out_f + o];"),
    ("proj_no_rounding", "y[i * out_f + o] = round_to(s, round);",
     "y[i * out_f + o] = s; (void)round;"),
    ("proj_k_block_is_q", "k[i * C + ci] = P[i * 3 * C + C + ci];",
     "k[i * C + ci] = P[i * 3 * C + ci];"),
    ("bf16_ties_away", "const double r = ldexp(rint(ldexp(x, 8 - e)), e - 8);",
     "const double r = ldexp(round(ldexp(x, 8 - e)), e - 8);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    msrc = tmp_path / "bra_oracle.c"
    msrc.write_text(src.replace(old, new))
    # the header sits next to the original source
    lib = build_oracle(str(msrc), str(tmp_path / f"liboracle_{name}.so"),
                       extra_flags=["-I", os.path.dirname(SRC), "-w"])
    orc = oracle.OracleLib(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant {name}"
