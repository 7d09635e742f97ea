"""Plants plausible mistakes in copies of the oracle's C source, on the CPU,
and checks that the pins (tests/pins.py) catch every one of them."""
import os

import pytest

import pins
from oracle import build as obuild
from oracle import ssu_oracle

# (name, text in oracle/ssu_oracle.c, replacement)
MUTANTS = [
    ("drop_dt_bias", "v = v + a->dt_bias[h]; /* R3 */", "v = v;"),
    ("softplus_is_exp", "if (a->dt_softplus)\n                        v = oracle_softplus(v);",
     "if (a->dt_softplus)\n                        v = expf(v);"),
    ("softplus_threshold", "if (v > 20.0f)", "if (v > 0.0f)"),
    ("decay_sign", "expf(v * a->A[h])", "expf(-v * a->A[h])"),
    ("decay_without_dt", "expf(v * a->A[h])", "expf(a->A[h])"),
    ("rank1_without_dt", "const float dtx = v * xv;\n                    float *Sd = S + d * N;\n                    for (int64_t n = 0; n < N; n++) {",
     "const float dtx = xv;\n                    float *Sd = S + d * N;\n                    for (int64_t n = 0; n < N; n++) {"),
    ("decay_after_add", "Sd[n] = Sd[n] * decay + dtx * bn;", "Sd[n] = (Sd[n] + dtx * bn) * decay;"),
    ("readout_uses_B", "const float cn = load_as_f32(a->C,", "const float cn = load_as_f32(a->B,"),
    ("drop_D", "y = y + a->D[h] * xv;", "y = y;"),
    ("gate_without_silu", "y = y * silu(load_as_f32(a->z, a->io_dtype, xi));",
     "y = y * load_as_f32(a->z, a->io_dtype, xi);"),
    ("gate_before_D",
     "if (a->D)\n                        y = y + a->D[h] * xv;\n"
     "                    if (a->z)\n"
     "                        y = y * silu(load_as_f32(a->z, a->io_dtype, xi)); /* R6 */",
     "if (a->z)\n                        y = y * silu(load_as_f32(a->z, a->io_dtype, xi));\n"
     "                    if (a->D)\n                        y = y + a->D[h] * xv;"),
    ("group_modulo", "const int64_t g = h / heads_per_group;", "const int64_t g = h % G;"),
    ("dt_per_head_index", "load_as_f32(a->dt, a->dt_dtype, r * H + h)",
     "load_as_f32(a->dt, a->dt_dtype, r * H)"),
    ("no_accepted_floor", "if (pos0 < 0)\n            pos0 = 0;", ""),
    ("accepted_not_minus_one", "pos0 = a->acc[b] - 1;", "pos0 = a->acc[b];"),
    ("pad_written", "if (wslot == a->pad)\n                    continue; /* R10 */", ""),
    ("pad_read_as_data", "S[e] = rslot == a->pad", "S[e] = rslot == -12345"),
    ("disable_ignored",
     "if (a->disable)\n                    continue;\n                int64_t wslot;",
     "int64_t wslot;"),
    ("carry_not_rounded", "/* R5: carry what the state dtype holds */\n                for (int64_t e = 0; e < tile; e++)\n                    S[e] = through_dtype(a->state_dtype, S[e]);",
     "/* R5: carry what the state dtype holds */"),
    # ReplaySSM decode
    ("replay_never_flushes", "if (h + 1 == L) {", "if (h == L) {"),
    ("replay_flush_not_rounded",
     "for (int64_t e = 0; e < tile; e++)\n                        S[e] = through_dtype(a->state_dtype, S[e]);\n                }",
     "}"),
    ("replay_gamma_without_current",
     "for (int64_t j = 0; j <= h; j++)\n                        gamma = gamma * alpha[j];",
     "for (int64_t j = 0; j < h; j++)\n                        gamma = gamma * alpha[j];"),
    ("replay_tail_includes_own_decay", "for (int64_t i = j + 1; i <= h; i++)", "for (int64_t i = j; i <= h; i++)"),
    ("replay_weight_without_dt", "y = y + dtp[j] * xs[j] * tail * w;", "y = y + xs[j] * tail * w;"),
    ("replay_readout_uses_B", "u = u + S[d * N + n] * load_as_f32(a->C,", "u = u + S[d * N + n] * load_as_f32(a->B,"),
    ("replay_append_skipped_x",
     "copy_elem(ra->bx_out, a->x, a->io_dtype, ((s * L + h) * H + hd) * P + d,",
     "copy_elem(ra->bx_out, a->x, a->io_dtype, ((s * L + h) * H + hd) * P + 0,"),
    # ReplaySSM speculative step
    ("spec_natural_fold", "const int fold = h + 2 * T > L;", "const int fold = h + T > L;"),
    ("spec_no_causal_mask", "const int64_t last = w + t; /* draft t's place in the window */",
     "const int64_t last = w + T - 1;"),
    ("spec_append_reversed", "copy_elem(ra->bx_out, a->x, a->io_dtype, ((s * L + w + t) * H + hd) * P + d,",
     "copy_elem(ra->bx_out, a->x, a->io_dtype, ((s * L + w + (T - 1 - t)) * H + hd) * P + d,"),
    ("spec_fold_not_rounded",
     "for (int64_t e = 0; e < tile; e++) /* R21: rounded after each */\n"
     "                        S[e] = through_dtype(a->state_dtype, S[e]);", ""),
    ("spec_readout_first_draft", "u = u + S[d * N + n] * DC(t, n);", "u = u + S[d * N + n] * DC(0, n);"),
    ("spec_D_of_window_start", "y = y + a->D[hd] * xs[last];", "y = y + a->D[hd] * xs[w];"),
    ("spec_draft_B_row", "wj = wj + (j < w ? BB(j, n) : DB(j - w, n)) * DC(t, n);",
     "wj = wj + (j < w ? BB(j, n) : DB(0, n)) * DC(t, n);"),
    ("spec_draft_dt_row", "const float raw = k < w ? BDT(k, d) : DDT(k - w, d);",
     "const float raw = k < w ? BDT(k, d) : DDT(0, d);"),
    # memmove-safe state copies
    ("copy_forward_bytes", "memmove(buf + dst_off[i], buf + src_off[i], (size_t)sizes[i]); /* R24 */",
     "for (int64_t k = 0; k < sizes[i]; k++) buf[dst_off[i] + k] = buf[src_off[i] + k];"),
    ("copy_backward_bytes", "memmove(buf + dst_off[i], buf + src_off[i], (size_t)sizes[i]); /* R24 */",
     "for (int64_t k = sizes[i] - 1; k >= 0; k--) buf[dst_off[i] + k] = buf[src_off[i] + k];"),
    ("conv_sd_without_bias", "memmove(dst, src + bias[r] * inner * elem_size,", "memmove(dst, src,"),
    ("conv_ds_without_bias", "memmove(dst + d * W * elem_size, src + (d * W + bias[r]) * elem_size,",
     "memmove(dst + d * W * elem_size, src + (d * W) * elem_size,"),
    ("conv_ds_as_sd", "if (layout == OR_CONV_SD) {", "if (layout != 7) {"),
    # SSD prefill
    ("ssd_never_reset", "const int opens = c == 0 || a->seq_idx[c] != a->seq_idx[c - 1]; /* R27 */",
     "const int opens = c == 0;"),
    ("ssd_reset_every_chunk", "const int opens = c == 0 || a->seq_idx[c] != a->seq_idx[c - 1]; /* R27 */",
     "const int opens = 1;"),
    ("ssd_no_floor", "if (v < a->dt_lo) /* dt_limit, after softplus */\n                    v = a->dt_lo;", ""),
    ("ssd_no_ceiling", "if (v > a->dt_hi)\n                    v = a->dt_hi;", ""),
    ("ssd_decay_without_dt", "const float decay = expf(a->A[h] * v); /* R26 */", "const float decay = expf(a->A[h]);"),
    ("ssd_init_of_chunk", "load_as_f32(a->init, a->state_dtype, (a->seq_idx[c] * H + h) * tile + e)",
     "load_as_f32(a->init, a->state_dtype, (0 * H + h) * tile + e)"),
    # MXFP8 read copy
    ("e4m3_truncates", "float q = nearbyintf((ldexpf(a, -e) - 1.0f) * 8.0f);",
     "float q = floorf((ldexpf(a, -e) - 1.0f) * 8.0f);"),
    ("e4m3_subnormal_truncates", "const float q = nearbyintf(ldexpf(a, 9));",
     "const float q = floorf(ldexpf(a, 9));"),
    ("e4m3_decode_bias", "ldexpf(1.0f + (float)m / 8.0f, e - 7)", "ldexpf(1.0f + (float)m / 8.0f, e - 8)"),
    ("mx8_scale_off_by_one", "k = (ex - 1) - 8; /* R30 */", "k = (ex - 1) - 7;"),
    ("mx8_scale_off_by_one_up", "k = (ex - 1) - 8; /* R30 */", "k = (ex - 1) - 9;"),
    ("mx4_scale_off_by_one", "k = (ex - 1) - 2; /* R34 */", "k = (ex - 1) - 1;"),
    ("mx4_scale_off_by_one_up", "k = (ex - 1) - 2; /* R34 */", "k = (ex - 1) - 3;"),
    ("e2m1_ties_away", "code = (int)nearbyintf(a * 2.0f);", "code = (int)floorf(a * 2.0f + 0.5f);"),
    ("e2m1_no_saturation", "return sign | 7; /* R34: saturate */", "return sign | 6;"),
    ("mx4_nibbles_swapped", "(oracle_e2m1_encode(ldexpf(x[2 * i + 1], -k)) << 4)); /* R33 */",
     "(oracle_e2m1_encode(ldexpf(x[2 * i + 1], -k)) >> 0)) ^ 0; /* R33 */"),
    ("e2m1_decode_bias", "ldexpf(1.0f + 0.5f * (float)m, e - 1)", "ldexpf(1.0f + 0.5f * (float)m, e)"),
    ("mx4_read_as_mx8", "                       : ra->lp_bits == 4 ? oracle_mx4_value(",
     "                       : ra->lp_bits == 5 ? oracle_mx4_value("),
    ("lp_read_at_fold", "const int from_copy = ra->lp_in && h + 1 != L && !pad;",
     "const int from_copy = ra->lp_in && !pad;"),
    ("lp_not_rewritten", "if (ra->lp_out) /* R32: the fold rewrites the read copy */", "if (0)"),
    ("default_dst_is_seq",
     "a->wtab.data ? &a->wtab : (a->rtab.data ? &a->rtab : NULL)", "a->wtab.data ? &a->wtab : NULL"),
    ("flat_write_b_plus_t", "int64_t i = tb->ndim == 1 ? bos + t :", "int64_t i = tb->ndim == 1 ? b + t :"),
    ("flat_read_b_plus_pos",
     "int64_t i = a->rtab.ndim == 1 ? bos + pos0 :", "int64_t i = a->rtab.ndim == 1 ? b + pos0 :"),
    ("no_table_reads_zero", "if (!a->rtab.data) {\n        *slot = b;",
     "if (!a->rtab.data) {\n        *slot = 0;"),
    ("f16_truncates", "if (rem > 0x1000u || (rem == 0x1000u && (q & 1u)))\n        q++;", ""),
    ("f16_ties_away", "(rem == 0x1000u && (q & 1u))", "(rem == 0x1000u)"),
    ("f16_subnormal_decode", "(127 - 15 + 1 - k)", "(127 - 15 - k)"),
    ("bf16_truncates", "round_shift(u, 16)", "(u >> 16)"),
    ("bf16_decode_shift", "(uint32_t)b << 16", "(uint32_t)b << 15"),
]


def test_mutant_list_is_distinct():
    assert len({m[0] for m in MUTANTS}) == len(MUTANTS)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, "mutation site for %s not found exactly once" % name
    path = tmp_path / ("oracle_%s.c" % name)
    path.write_text(src.replace(old, new))
    lib = obuild.build(str(path), str(tmp_path / ("liboracle_%s.so" % name)), extra=["-w"])
    orc = ssu_oracle.Oracle(lib)
    caught = None
    for pin in pins.ALL:
        try:
            pin(orc)
        except Exception as e:  # a failed assertion or an oracle refusal
            caught = (pin.__name__, type(e).__name__)
            break
    assert caught is not None, "no pin catches mutant %s" % name
    os.remove(lib)
