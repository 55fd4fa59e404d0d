"""The pins must catch plausible mistakes in the oracle.

Each mutation below plants one mistake in a temporary copy of ``oracle/oracle.c`` (a dropped
term, a wrong sign or index, a transposed operand, a skipped reset ...), builds it with gcc, and
requires that at least one pin of ``pins.py`` rejects the broken oracle.  The real oracle is never
modified.
"""
import os

import pytest

import pins
from oracle import Oracle, OracleError
from oracle.build import SRC, build

MUTATIONS = {
    "taps_reversed": ("for (int kk = 0; kk < W; ++kk) z = fmaf(wt[kk], u[kk], z);",
                      "for (int kk = 0; kk < W; ++kk) z = fmaf(wt[W - 1 - kk], u[kk], z);"),
    "history_order_reversed": ("ubits[j] = history_bits(&k, i, c, C, j);", "ubits[j] = history_bits(&k, i, c, C, H - 1 - j);"),
    "bias_dropped": ("float bias = b ? load_tap(b, b_f32, c) : 0.0f;\n          for (int64_t q = 0; q < ns; ++q) {\n            int64_t s = segs[q].s, n = segs[q].e - segs[q].s, i = segs[q].i;\n            if (pool",
                     "float bias = 0.0f; (void)b_f32;\n          for (int64_t q = 0; q < ns; ++q) {\n            int64_t s = segs[q].s, n = segs[q].e - segs[q].s, i = segs[q].i;\n            if (pool"),
    "sentinel_not_zero": ("for (int64_t t = 0; t < n; ++t) y[(s + t) * y_ld + c] = 0;", "for (int64_t t = 0; t < n; ++t) y[(s + t) * y_ld + c] = 0x3F80;"),
    "writeback_off_by_one": ("= ubits[n + j];", "= ubits[n + j - 1];"),
    "silu_sign": ("out = double_to_bf16_rne(zd * sigmoid_d(zd));", "out = double_to_bf16_rne(zd * sigmoid_d(-zd));"),
    "silu_grad_sign": ("g *= sg * (1.0 + zd * (1.0 - sg));", "g *= sg * (1.0 - zd * (1.0 - sg));"),
    "dx_index": ("int64_t tau = t + H - kk;", "int64_t tau = t + kk;"),
    "dw_offset": ("dw_acc[kk] += dz[t] * u[t + kk];", "dw_acc[kk] += dz[t] * u[t + H - kk];"),
    "dhist_tap": ("acc += (double)wf[j - tau] * dz[tau];", "acc += (double)wf[tau] * dz[tau];"),
    "has_init_ignored": ("if (slot >= 0 && k->has_init && k->has_init[i])", "if (slot >= 0)"),
    "seq_idx_no_reset": ("boundary = (seq_idx[t] != seq_idx[t - 1]);", "boundary = 0;"),
    "round_half_up": ("u += 0x7fffu + lsb;", "u += 0x8000u + 0 * lsb;"),
    "decode_shift": ("h[0] = h1;\n      h[s_pos] = h2;", "h[0] = h2;\n      h[s_pos] = h1;"),
    "db_scaled": ("db_acc += dz[t];", "db_acc += 0.5 * dz[t];"),
    "pool_strides_transposed": ("return k->pool[slot * k->s_slot + c * k->s_chan + j * k->s_pos];",
                                "return k->pool[slot * k->s_slot + c * k->s_pos + j * k->s_chan];"),
    "double_rounding_kept": ("if (r != 0.0) {", "if (0) {"),
    "spec_history_reversed": ("u[j] = h[(a - 1 + j) * s_pos];", "u[j] = h[(a + 1 - j) * s_pos];"),
    "spec_accepted_ignored": ("u[j] = h[(a - 1 + j) * s_pos];", "u[j] = h[j * s_pos];"),
    "spec_writeback_unshifted": ("for (int64_t j = 0; j < K + 2; ++j) h[j * s_pos] = u[j + 1];",
                                 "for (int64_t j = 0; j < K + 2; ++j) h[j * s_pos] = u[j];"),
    "spec_writeback_short": ("for (int64_t j = 0; j < K + 2; ++j) h[j * s_pos] = u[j + 1];",
                             "for (int64_t j = 0; j < K + 1; ++j) h[j * s_pos] = u[j + 1];"),
    "spec_token_stride": ("u[3 + t] = x[(i * K + t) * x_ld + c];", "u[3 + t] = x[(i + t) * x_ld + c];"),
    "dtail_reversed": ("acc += bf16_bits_to_float(dtail[(t + H - n) * C + c]);",
                       "acc += bf16_bits_to_float(dtail[(n - 1 - t) * C + c]);"),
    "dtail_dhist_dropped": ("if (tail && j - n >= 0) acc += bf16_bits_to_float(dtail[(j - n) * C + c]);", ""),
    "dtail_first_segment": ("const int tail = dtail && q == ns - 1;", "const int tail = dtail && q == 0;"),
    "combine_descending": ("for (int64_t sh = 1; sh < nshards; ++sh) acc = acc + parts[sh * n + e];",
                           "for (int64_t sh = nshards - 1; sh >= 1; --sh) acc = acc + parts[sh * n + e];"),
    "batch_rows_one_index": ("          v[n].i = n;\n", "          v[n].i = 0;\n"),
    "dx_mask_dropped_at_end": ("if (tau < n) acc += (double)wf[kk] * dz[tau];", "if (tau < n && tau + 1 < n) acc += (double)wf[kk] * dz[tau];"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = build(out=str(tmp_path / "libmutant.so"), src=str(mutant), extra=("-w",))
    o = Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, OracleError) as e:
            caught.append(f"{pin.__name__}: {str(e)[:80]}")
            break
    assert caught, f"no pin rejected the '{name}' mutant"
    os.remove(lib)
