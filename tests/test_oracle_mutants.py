"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle/mxref.c, applies one plausible mistake (a dropped
term, a wrong sign, a wrong index or block size, a transposed operand, a
wrong bias, a wrong rounding rule), builds the copy with gcc under a
temporary directory and runs the pins against it: at least one pin must
fail.  The oracle itself is never modified.
"""
import os
import shutil

import pytest

import oracle
import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "mxref.c")

MUTANTS = {
    "scale_block_16": ("j->te[sa[k / 32]]", "j->te[sa[k / 16]]"),
    "dropped_b_scale": ("double bv = j->tb[cb] * j->te[sb[k / 32]];", "double bv = j->tb[cb];"),
    "wrong_sign": ("s += prod;", "s -= prod;"),
    "transposed_b_row": ("*b = j->B + n * j->ldB", "*b = j->B + (n % j->M) * j->ldB"),
    "a_scale_indexed_by_n": ("*sa = j->As + m * j->KB", "*sa = j->As + (n % j->M) * j->KB"),
    "e4m3_bias_8": ("(int)e - 7 - 3", "(int)e - 8 - 3"),
    "e4m3_no_subnormal": ("v = ldexp((double)m, 1 - 7 - 3);", "v = 0.0;"),
    "e5m2_inf_as_nan": ("v = (m == 0u) ? INFINITY : NAN;", "v = NAN;"),
    "e8m0_bias_128": ("return ldexp(1.0, (int)s - 127);", "return ldexp(1.0, (int)s - 128);"),
    "e8m0_255_finite": ("    if (s == 255u)\n        return NAN;\n    return ldexp", "    return ldexp"),
    "dropped_cin": ("            s += c;\n", "\n"),
    "bf16_round_half_up": ("u += 0x7fffu + lsb;", "u += 0x8000u;"),
    "last_k_dropped": ("for (int64_t k = 0; k < j->K; ++k)", "for (int64_t k = 0; k + 1 < j->K; ++k)"),
    "mag_signed": ("mag += fabs(prod);", "mag += prod;"),
    "quant_ties_to_odd": ("(d == bd && (c & 1) == 0)", "(d == bd && (c & 1) == 1)"),
    "quant_exponent_plus_one": ("s = block_exponent(fmt, amax) + 127;", "s = block_exponent(fmt, amax) + 128;"),
    "quant_sign_dropped": ("(signbit(v) ? ncodes : 0)", "0"),
    "quant_scale_inverted": ("ldexp(x[k - k0], 127 - s)", "ldexp(x[k - k0], s - 127)"),
    "quant_e4m3_max_480": ("case MXREF_FMT_E4M3: return 448.0;", "case MXREF_FMT_E4M3: return 480.0;"),
    "packed_bit_order": ("const unsigned sh = (unsigned)(bit % 8);\n    unsigned v = row[bit / 8] >> sh;",
                         "const unsigned sh = (unsigned)(8 - bits - bit % 8) % 8u;\n    unsigned v = row[bit / 8] >> sh;"),
    "packed_a_read_as_b_width": ("const unsigned ca = code_at(a, k, j->bitsA);", "const unsigned ca = code_at(a, k, j->bitsB);"),
    "packed_straddle_dropped": ("    if (sh + (unsigned)bits > 8u)\n        v |= ", "    if (0)\n        v |= "),
    "e2m1_bias_0": ("(int)e - 1 - 1", "(int)e - 0 - 1"),
    "e2m1_no_subnormal": ("v = ldexp((double)m, 1 - 1 - 1);", "v = 0.0;"),
    "packed_row_pitch_k": ("base.ldA = row_bytes(K, base.bitsA);", "base.ldA = K;"),
    "e2m3_bias_0": ("(int)e - 1 - 3); /* (1+m/8) * 2^(e-1) */", "(int)e - 0 - 3); /* (1+m/8) * 2^(e-1) */"),
    "e3m2_mantissa_bits_3": ("unsigned s = (c >> 5) & 1u, e = (c >> 2) & 7u, m = c & 3u;",
                             "unsigned s = (c >> 5) & 1u, e = (c >> 3) & 3u, m = c & 7u;"),
    "e2m3_no_subnormal": ("v = ldexp((double)m, 1 - 1 - 3);            /* m/8 */", "v = 0.0;"),
    "quant_fp6_max_6": ("case MXREF_FMT_E2M3: return 7.5;", "case MXREF_FMT_E2M3: return 6.0;"),
    "e2m1_sign_dropped": ("    return s ? -v : v;\n}\n\n/* e8m0", "    return v;\n}\n\n/* e8m0"),
    "quant_e2m1_max_4": ("default: return 6.0; /* e2m1 */", "default: return 4.0; /* e2m1 */"),
    "quant_sign_bit_7": ("(signbit(v) ? ncodes : 0)", "(signbit(v) ? 0x80 : 0)"),
    "quant_packed_bit_order": ("    row[bit / 8] |= (uint8_t)(c << sh);", "    row[bit / 8] |= (uint8_t)(c << (8 - bits - sh) % 8u);"),
    "quant_zero_block_scale": ("int s = 0;\n            if (amax > 0.0) {", "int s = 127;\n            if (amax > 0.0) {"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found once"
    mpath = tmp_path / "mxref_mut.c"
    mpath.write_text(src.replace(old, new))
    so = str(tmp_path / "libmxref_mut.so")
    oracle.build(str(mpath), so)
    lib = oracle.load(so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"
