"""Mutation check of the oracle's pins (CPU only).

Each case below plants one plausible mistake in a copy of the oracle's C source
(a dropped term, a wrong sign, index or constant, a transposed operand, another
reading of a rounding rule), builds that copy, and runs the oracle's pin tests
against it.  The pins are only worth something if every such mistake fails at
least one of them, so each case asserts that the pin run fails.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_codec.py", "tests/test_oracle_quant.py", "tests/test_oracle_gemm.py",
             "tests/test_oracle_ue8m0.py", "tests/test_oracle_sr.py", "tests/test_oracle_swiglu.py"]

# name -> (text in oracle/fgb_oracle.c, replacement); every occurrence of the text is
# replaced (a mistake copied into both scale formats' code)
MUTANTS = {
    "ties_away_from_zero": ("return (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;", "return lo + 1.0;"),
    "ties_toward_zero": ("return (fmod(lo, 2.0) == 0.0) ? lo : lo + 1.0;", "return lo;"),
    "decode_bias_8": ("mag = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 7);",
                      "mag = (1.0 + (double)m / 8.0) * ldexp(1.0, e - 8);"),
    "decode_subnormal_scale": ("mag = (double)m * ldexp(1.0, -9);", "mag = (double)m * ldexp(1.0, -10);"),
    "negative_zero_dropped": ("uint8_t sign = signbit(f) ? 0x80 : 0x00;", "uint8_t sign = (f < 0.0f) ? 0x80 : 0x00;"),
    "overflow_to_nan": ("if (a > 448.0) return sign | 0x7E;", "if (a > 448.0) return sign | 0x7F;"),
    "subnormal_encode_scale": ("double m = rne_integer(a * 512.0);", "double m = rne_integer(a * 256.0);"),
    "binade_carry_lost": ("        m = 0.0;\n        ex += 1;", "        m = 7.0;"),
    "bf16_ulp_off_by_one": ("double ulp = ldexp(1.0, ex - 7);", "double ulp = ldexp(1.0, ex - 8);"),
    "absmax_signed": ("float av = fabsf(v[i]);", "float av = v[i];"),
    "amax_floor_ignored": ("if (amax_floor > a) a = amax_floor;", ""),
    "scale_denominator_447": ("float s = a / 448.0f;", "float s = a / 447.0f;"),
    "cast_divides_by_scale": ("float t = v[i] * inv;", "float t = v[i] / s;"),
    "zero_tile_nan_scale": ("        inv = 0.0f;\n", "        inv = 448.0f / a;\n"),
    "transpose_pad_negative_zero": ("(k < n) ? code[k] : 0x00;", "(k < n) ? code[k] : 0x80;"),
    "weight_transpose_not_transposed": ("if (qT) qT[(n0 + b) * ldqT + k0 + a] = code[a * nn + b];",
                                        "if (qT) qT[(n0 + a) * ldqT + k0 + b] = code[a * nn + b];"),
    "requant_first_block_scale": ("float sc = s[(c / ORC_TILE) * lds + r];", "float sc = s[r];"),
    "requant_scale_unapplied": ("v[r * C + c] = (float)(d * (double)sc);", "v[r * C + c] = (float)d;"),
    "gemm_partial_block_dropped": ("int64_t nblk = ceil_div(K, ORC_TILE);", "int64_t nblk = K / ORC_TILE;"),
    "gemm_b_scale_block_ignored": ("(double)sb[b * sb_sb + (j / sb_group) * sb_sj];",
                                   "(double)sb[(j / sb_group) * sb_sj];"),
    "gemm_a_scale_wrong_row": ("(double)sa[b * sa_sb + (i / sa_group) * sa_si]",
                               "(double)sa[b * sa_sb + (j / sa_group) * sa_si]"),
    "gemm_operand_transposed": ("double p = dec[A[i * lda + t]] * dec[B[j * ldb + t]];",
                                "double p = dec[A[i * lda + t]] * dec[B[t * ldb + j]];"),
    "gemm_scale_unapplied": ("r += scale * sblk;", "r += sblk;"),
    "gemm_block_sum_fp32": ("sblk += p;", "sblk = (float)(sblk + p);"),
    "gemm_aabs_signed": ("sabs += fabs(p);", "sabs += p;"),
    "ue8m0_boundary_rounds_up": ("ldexp(448.0, e) < (double)a) ++e;", "ldexp(448.0, e) <= (double)a) ++e;"),
    "ue8m0_scale_inverted": ("const double m = ldexp(1.0, -e);", "const double m = ldexp(1.0, e);"),
    "ue8m0_byte_bias_128": ("*e_out = (uint8_t)(e + 127);", "*e_out = (uint8_t)(e + 128);"),
    "ue8m0_clamp_at_minus_126": ("    int e = -127;\n", "    int e = -126;\n"),
    "e8m0_decode_bias_126": ("ldexp(1.0, (int)b - 127)", "ldexp(1.0, (int)b - 126)"),
    "requant_ue8m0_first_block_byte": ("orc_e8m0_decode(e[(c / ORC_TILE) * lde + r])", "orc_e8m0_decode(e[r])"),
    "two_stage_tile_scale_transposed": ("const double sc = (double)s[i * nb + j];",
                                        "const double sc = (double)s[j * kb + i];"),
    "two_stage_scale_unapplied": ("(float)(orc_e4m3_decode(q[(k0 + a) * ldq + n0 + b]) * sc);",
                                  "(float)(orc_e4m3_decode(q[(k0 + a) * ldq + n0 + b]));"),
    "two_stage_transpose_not_transposed": ("if (q2T) q2T[(n0 + b) * ldq2T + k0 + a] = code[a * nn + b];",
                                           "if (q2T) q2T[(n0 + a) * ldq2T + k0 + b] = code[a * nn + b];"),
    "philox_multiplier_typo": ("(uint64_t)0xD2511F53u * c0", "(uint64_t)0xD2511F57u * c0"),
    "philox_nine_rounds": ("for (int round = 0; round < 10; ++round)", "for (int round = 0; round < 9; ++round)"),
    "philox_weyl_constants_swapped": ("k0 += 0x9E3779B9u;\n        k1 += 0xBB67AE85u;",
                                      "k0 += 0xBB67AE85u;\n        k1 += 0x9E3779B9u;"),
    "sr_word_index_shifted": ("return out[c % 4];", "return out[(c + 1) % 4];"),
    "sr_counter_row_col_swapped": ("{(uint32_t)(c / 4), (uint32_t)r, salt, 0u}", "{(uint32_t)(r / 4), (uint32_t)c, salt, 0u}"),
    "sr_key_halves_swapped": ("{(uint32_t)seed, (uint32_t)(seed >> 32)}", "{(uint32_t)(seed >> 32), (uint32_t)seed}"),
    "sr_salt_ignored": ("(uint32_t)r, salt, 0u}", "(uint32_t)r, 0u, 0u}"),
    "sr_compare_le": ("int up = (double)u < frac * 4294967296.0;", "int up = (double)u <= frac * 4294967296.0;"),
    "sr_direction_inverted": ("int up = (double)u < frac * 4294967296.0;", "int up = (double)u >= frac * 4294967296.0;"),
    "sr_128x1_word_transposed": ("u[k] = orc_sr_word(seed, salt, r0 + k, c);", "u[k] = orc_sr_word(seed, salt, c, r0 + k);"),
    "sr_128x128_word_transposed": ("u[a * nn + b] = orc_sr_word(seed, salt, k0 + a, n0 + b);",
                                   "u[a * nn + b] = orc_sr_word(seed, salt, n0 + b, k0 + a);"),
    "sr_negative_zero_dropped": ("uint8_t sign = signbit(v) ? 0x80 : 0x00;", "uint8_t sign = (v < 0.0f) ? 0x80 : 0x00;"),
    "sr_saturation_to_nan": ("if (m >= 448.0) return sign | 0x7E;", "if (m >= 448.0) return sign | 0x7F;"),
    "silu_tanh_sign_flipped": ("return bf16_of_scaled(g * f * 0.5L, tanhl(0.5L * g),",
                               "return bf16_of_scaled(g * f * 0.5L, tanhl(-0.5L * g),"),
    "silu_large_gate_tie_up": ("return bf16_of_scaled(g * f, -om, -1);", "return bf16_of_scaled(g * f, -om, 1);"),
    "silu_small_gate_tie_sign": ("g > 0.0L ? 1 : (g < 0.0L ? -1 : 0));\n    long double sig",
                                 "g > 0.0L ? -1 : (g < 0.0L ? 1 : 0));\n    long double sig"),
    "dsilu_cosh_term_dropped": ("tanhl(0.5L * g) + g / (2.0L * ch * ch)", "tanhl(0.5L * g)"),
    "dsilu_uses_sigma_twice": ("return bf16_round_ld(f * (sig * (1.0L + g * om)));",
                               "return bf16_round_ld(f * (sig * (1.0L + g * sig)));"),
    "dsilu_large_gate_split_sign": ("return bf16_of_scaled(f, c, 1);", "return bf16_of_scaled(f, c, -1);"),
    "sigma_negative_branch": ("*sig = e / (1.0L + e);", "*sig = 1.0L / (1.0L + e);"),
    "bf16_ld_ties_up": ("(fmodl(lo, 2.0L) == 0.0L ? lo : lo + 1.0L)", "(lo + 1.0L)"),
    "zero_gate_tie_broken": ("if (c_sign == 0) return bf16_round_ld(hi);", "/* tie at a zero gate broken */"),
    "zero_product_sign_dropped": ("if (hi == 0.0L) return bf16_round_ld(hi);", "/* zero through hi + hi*c */"),
    "swiglu_up_read_from_gate": ("long double u = orc_bf16_to_float(gu[r * ldgu + F + c]);",
                                 "long double u = orc_bf16_to_float(gu[r * ldgu + c]);"),
    "swiglu_bwd_dequant_no_bf16": ("long double g = orc_bf16_to_float(orc_bf16_round((double)gq));",
                                   "long double g = gq;"),
    "swiglu_bwd_up_scale_block": ("s[((F + c) / ORC_TILE) * lds + r]", "s[(c / ORC_TILE) * lds + r]"),
    "swiglu_bwd_outputs_swapped": ("dgu[r * lddgu + c] = bf16_dsilu_times(g, d * u);",
                                   "dgu[r * lddgu + c] = bf16_silu_times(g, d);"),
}


def _mutant_source(src, old, new):
    assert src.count(old) >= 1, f"mutation site missing: {old!r}"
    return src.replace(old, new)


def _run_pins(name, old, new, tmpdir):
    import oracle
    with open(os.path.join(ROOT, "oracle", "fgb_oracle.c")) as f:
        src = _mutant_source(f.read(), old, new)
    c_path = os.path.join(tmpdir, f"{name}.c")
    with open(c_path, "w") as f:
        f.write(src)
    so = oracle.compile_oracle(c_path, os.path.join(tmpdir, f"lib{name}.so"))
    env = dict(os.environ, FGB_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
           "-k", "not exhaustive", *PIN_FILES]
    p = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, p.returncode, p.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(lambda kv: _run_pins(kv[0], *kv[1], str(tmp_path)), MUTANTS.items()))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    crashed = [(n, rc) for n, rc, _ in results if rc not in (0, 1)]
    for n, rc, out in results:
        print(f"{n}: pytest exit {rc}")
    assert not crashed, f"pin runs that crashed instead of failing: {crashed}"
    assert not survivors, "planted mistakes that no pin catches:\n" + "\n".join(
        f"--- {n}\n{out}" for n, out in survivors)


def test_unmutated_copy_passes_the_pins(tmp_path):
    """Control: the same build route with no mutation passes, so a failing
    mutant run fails because of its mutation."""
    name, rc, out = _run_pins("control", "#define ORC_TILE 128", "#define ORC_TILE 128", str(tmp_path))
    assert rc == 0, out
