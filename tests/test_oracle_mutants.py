"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign, index, slice or
operand, a flipped tie rule) in a copy of ``oracle/loopvq_oracle.c``, builds
that copy with gcc into a temporary directory, routes the oracle wrapper to
it, and requires at least one pin check to fail.  Everything runs on the CPU.
"""
import pathlib
import subprocess

import pytest

import oracle
import test_oracle_attention as att
import test_oracle_encode as enc

SRC = pathlib.Path(oracle.__file__).resolve().parent / "loopvq_oracle.c"

ENC_PINS = [enc.check_codeword_inputs, enc.check_exact_ties, enc.check_fp64_bruteforce,
            enc.check_row_permutation, enc.check_placement, enc.check_rounding_order]
ATT_PINS = [att.check_attend_matches_sdpa, att.check_windows_only, att.check_end_to_end,
            att.check_zero_query_mean, att.check_empty_and_single, att.check_end_to_end_page_lag,
            att.check_gqa_end_to_end, att.check_loop_groups_end_to_end]

MUTANTS = {
    "drop_last_distance_term": ("for (int i = 0; i < G; ++i) {", "for (int i = 0; i < G - 1; ++i) {"),
    "tie_keeps_last": ("dist < best_d", "dist <= best_d"),
    "sum_instead_of_difference": ("xv[i] - codeword_entry", "xv[i] + codeword_entry"),
    "abs_instead_of_square": ("float sq = e * e;", "float sq = e < 0 ? -e : e;"),
    "fused_square_add": ("float sq = e * e;\n                        dist = dist + sq;",
                         "dist = fmaf(e, e, dist);"),
    "distance_summed_descending": ("float e = xv[i] - codeword_entry(codebook, cb_bf16, H, S, cg, Tc, g, h, j, k, i);",
                                   "float e = xv[G - 1 - i] - codeword_entry(codebook, cb_bf16, H, S, cg, Tc, g, h, j, k, G - 1 - i);"),
    "subvector_channels_transposed": ("xv[t * cg + c] = bf16_bits_to_float(",
                                      "xv[c * Tc + t] = bf16_bits_to_float("),
    "codebook_code_sub_swapped": ("((((size_t)r * H + h) * LVQO_CODES + k) * S + j)",
                                  "((((size_t)r * H + h) * S + j) * LVQO_CODES + k)"),
    "codeword_slice_ignores_group": ("int r = g * Tc + i / cg, c = i % cg;",
                                     "int r = i / cg, c = i % cg;"),
    "encode_writes_group_0_rows": ("index[((((size_t)g * batch + seq) * H + h)",
                                   "index[((((size_t)0 * batch + seq) * H + h)"),
    "index_row_ignores_first_token": ("* t_max + first_token + n) * S + j]", "* t_max + n) * S + j]"),
    "dequant_reads_slice_0": ("ck, t * cg + c);", "ck, 0 * cg + c);"),
    "value_dequant_uses_key_codebook": ("codeword_entry(v_cb, cb_bf16, Hk, S, cg, Tc, g, hk, j, cv,",
                                        "codeword_entry(k_cb, cb_bf16, Hk, S, cg, Tc, g, hk, j, cv,"),
    "ring_slot_without_sink_offset": ("n_sink + (pos - n_sink) % n_recent", "n_sink + pos % n_recent"),
    "vq_count_drops_sink": (": (L - n_sink - n_recent > 0 ? L - n_sink - n_recent : 0);\n        double",
                            ": (L - n_recent > 0 ? L - n_recent : 0);\n        double"),
    "softmax_not_normalised": ("double pn = s[n] / z;", "double pn = s[n];"),
    "scale_dropped": ("s[n] = scale * acc;", "s[n] = acc;"),
    "window_value_from_key_buffer": ("vr[ch] = bf16_bits_to_float(v_win[base + ch]);",
                                     "vr[ch] = bf16_bits_to_float(k_win[base + ch]);"),
    "query_ignores_batch": ("q[((size_t)b * H + h) * d + ch]", "q[((size_t)0 * H + h) * d + ch]"),
    "window_reads_step_0": ("((((size_t)b * R + loop_step) * Hk + hk) * W + slot) * d",
                            "((((size_t)b * R + 0) * Hk + hk) * W + slot) * d"),
    "gqa_kv_head_interleaved": ("const int hk = h / (H / Hk);", "const int hk = h % Hk;"),
    "key_dot_skips_last_channel": ("for (int ch = 0; ch < d; ++ch) acc += q[ch] * K[n * d + ch];",
                                   "for (int ch = 0; ch < d - 1; ++ch) acc += q[ch] * K[n * d + ch];"),
}


def _build_mutant(tmp_path, name, old, new):
    text = SRC.read_text()
    assert text.count(old) == 1, f"{name}: pattern must occur exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(text.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(src), "-o", str(lib), "-lm"], check=True)
    return lib


def _fails(pin):
    try:
        pin()
    except (AssertionError, ValueError):
        return True
    return False


def test_unmutated_pins_pass():
    for pin in ENC_PINS + ATT_PINS:
        assert not _fails(pin), pin.__name__


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    with oracle.use_library(lib):
        caught = [p.__name__ for p in ENC_PINS + ATT_PINS if _fails(p)]
    assert caught, f"no pin caught mutant {name}"
