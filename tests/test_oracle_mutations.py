"""Planted mistakes in the ORACLE (on the CPU): each must make at least one pin
fail.  This shows the pins would catch a plausible error in the oracle (a
swapped nibble, a wrong bias, an off-by-one, a wrong tie-break, sum instead
of max, a dropped scale, a transposed operand, a wrong rounding)."""

import numpy as np
import pytest

import oracle
from oracle import forced as FO
from oracle import formats as F
from oracle import indexer as I
from oracle import normrope as NR
from tests import test_oracle_forced as TFO
from tests import test_oracle_normrope as TNR
from tests import test_oracle_formats as TF
from tests import test_oracle_indexer as TI
from tests import test_oracle_plan as TP

PINS = [
    TF.test_e4m3_all_codes_match_torch_cast,
    TF.test_bf16_all_patterns_match_torch_cast,
    TF.test_bf16_golden_points,
    TI.test_exact_bruteforce_decode_bf16_queries,
    TF.test_e4m3_golden_points,
    TF.test_e2m1_matches_hand_typed_table,
    TF.test_encoder_matches_round_half_even_reference,
    TF.test_write_then_decode_pages,
    lambda: [TF.test_encoder_worked_examples(i) for i in range(7)],
    TI.test_hand_worked_example,
    TI.test_exact_bruteforce_decode,
    TI.test_exact_bruteforce_prefill,
    TI.test_identical_pages_tie_to_lower_id,
    TI.test_heap_selection_agrees,
    TI.test_nan_scores_rank_last,
    TI.test_nan_token_makes_page_nan_and_ranks_last,
    TI.test_nan_query_element_makes_every_page_nan,
    TI.test_rows_past_max_pages_are_refused,
    TI.test_local_page_scores_exact_bruteforce,
    TI.test_local_page_scores_causal_boundary,
    TFO.test_bruteforce_tiny_rows_local_page_competing,
    TFO.test_local_page_competes_special_cases,
    TI.test_prefill_row_equals_decode_row_at_same_position,
    TP.test_chunks_against_bruteforce_and_properties,
    TFO.test_bruteforce_tiny_rows,
    TFO.test_special_cases,
    TFO.test_output_form,
    TNR.test_rms_norm_closed_form,
    TNR.test_rms_norm_properties,
    TNR.test_rope_worked_examples,
    TNR.test_rope_group_properties,
    TNR.test_pairings_are_one_permutation_apart,
]


def _some_pin_fails():
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            return True
    return False


_orig_decode = F.decode_pages


def _decode_pages_swapped_nibbles(page_bytes):
    p = np.asarray(page_bytes, dtype=np.uint8).reshape(-1, 128, 68)
    q = p.copy()
    q[:, :, :64] = (p[:, :, :64] >> 4) | ((p[:, :, :64] & 0xF) << 4)
    return _orig_decode(q)


def _decode_pages_no_scale(page_bytes):
    p = np.asarray(page_bytes, dtype=np.uint8).reshape(-1, 128, 68).copy()
    p[:, :, 64:] = 127
    return _orig_decode(p)


def _decode_pages_reversed_scales(page_bytes):
    p = np.asarray(page_bytes, dtype=np.uint8).reshape(-1, 128, 68).copy()
    p[:, :, 64:] = p[:, :, 64:][:, :, ::-1]
    return _orig_decode(p)


def _decode_pages_transposed(page_bytes):
    v = _orig_decode(page_bytes)
    return np.swapaxes(v, 1, 2).copy()


_orig_e4m3 = F.e4m3fn_to_float


def _e4m3_bias8(codes):
    return _orig_e4m3(codes) / 2.0


_orig_bf16 = F.bf16_to_float


def _bf16_bias_126(bits):
    return _orig_bf16(bits) * 2.0


_orig_select = I.select_row


def _select_ties_high(scores, L):
    out = np.full(16, -1, dtype=np.int32)
    if L < 0:
        return out
    s = np.asarray(scores, dtype=np.float64)[:L]
    order = sorted(range(L), key=lambda j: (-s[j] if not np.isnan(s[j]) else np.inf, -j))
    n = min(15, L)
    out[:n] = order[:n]
    out[15] = L
    return out


def _select_nan_first(scores, L):
    s = np.asarray(scores, dtype=np.float64).copy()
    s[np.isnan(s)] = np.inf
    return _orig_select(s, L)


def _select_local_in_history(scores, L):
    out = _orig_select(scores, L)
    if L > 0 and L < 15:
        out[L] = L          # local page leaks into the history slots
    return out


_orig_page_scores = I.page_scores


def _page_scores_sum(q, kpages):
    q = np.asarray(q, dtype=np.float64).reshape(-1, 128)
    J = kpages.shape[0]
    if J == 0:
        return np.zeros((q.shape[0], 0))
    return (q @ kpages.reshape(J * 128, 128).T).reshape(q.shape[0], J, 128).sum(axis=2)


_orig_rows_decode = I.rows_decode


def _page_scores_nanmax(q, kpages):
    q = np.asarray(q, dtype=np.float64).reshape(-1, 128)
    J = kpages.shape[0]
    if J == 0:
        return np.zeros((q.shape[0], 0))
    dots = (q @ kpages.reshape(J * 128, 128).T).reshape(q.shape[0], J, 128)
    with np.errstate(all="ignore"):
        m = np.where(np.isnan(dots), -np.inf, dots).max(axis=2)
    return m


_orig_local_pages = I.local_pages


def _local_pages_clamped(positions, max_pages=None):
    L = _orig_local_pages(positions)
    return L if max_pages is None else np.minimum(L, max_pages)


def _local_scores_nt(delta):
    def f(q, kpage, p):
        q = np.asarray(q, dtype=np.float64).reshape(-1, 128)
        nt = int(p) % 128 + 1 + delta
        return (q @ np.asarray(kpage, dtype=np.float64)[:max(nt, 1)].T).max(axis=1)
    return f


_orig_select_forced = FO.select_forced_row


def _forced_local_ignored(scores, L, topk, init_blocks, local_blocks, max_k_tiles,
                          local_score=None):
    return _orig_select_forced(scores, L, topk, init_blocks, local_blocks, max_k_tiles,
                               local_score=-np.inf)


def _rows_decode_shifted(seq_lens, query_len):
    req, pos = _orig_rows_decode(seq_lens, query_len)
    return req, pos - 1


_orig_rows_prefill = I.rows_prefill


def _rows_prefill_off_by_one(cu, ctx):
    req, pos = _orig_rows_prefill(cu, ctx)
    return req, pos + 1


_E2M1 = F._E2M1_MAG


def _encode_ties_away(rows, chunk=8192):
    codes, sb = _orig_encode(rows, chunk)
    v = np.asarray(rows, dtype=np.float64).reshape(-1, 128)
    X = np.repeat(sb.astype(np.int64) - 127, 32, axis=1)
    x = np.abs(v) / np.exp2(X)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    up = np.isin(x, mids)
    mag = (codes & 7).astype(np.int64)
    mag = np.where(up & (mag % 2 == 0) & (np.take(_E2M1, mag) < x), mag + 1, mag)
    return (mag | (codes & 8)).astype(np.uint8), sb


_orig_encode = F.mxfp4_encode_rows


def _encode_exp_minus_one(rows, chunk=8192):
    codes, sb = _orig_encode(np.asarray(rows, dtype=np.float64) * 0.5, chunk)
    return codes, (sb.astype(np.int64) + 1).astype(np.uint8)


_orig_chunks = oracle.prefill_chunks

_orig_rms = NR.rms_norm
_orig_rope = NR.rope


def _rms_eps_outside(x, weight, eps):
    x = np.asarray(x, dtype=np.float64)
    if weight is None:
        return x.copy()
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * weight


def _rms_sum_not_mean(x, weight, eps):
    x = np.asarray(x, dtype=np.float64)
    if weight is None:
        return x.copy()
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * weight


def _rope_sin_flipped(x, positions, rotary_dim, base, style):
    return _orig_rope(x, -np.asarray(positions, dtype=np.float64), rotary_dim, base, style)


def _rope_half_frequency(x, positions, rotary_dim, base, style):
    # exponent -i/rd instead of -2i/rd: the same as doubling rotary_dim in the frequencies
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    if rotary_dim == 0:
        return out
    i = np.arange(rotary_dim // 2)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * np.power(base, -1.0 * i / rotary_dim)
    fa, fb = NR.rope_pairs(rotary_dim, style)
    a, b = x[:, fa], x[:, fb]
    out[:, fa] = a * np.cos(ang) - b * np.sin(ang)
    out[:, fb] = b * np.cos(ang) + a * np.sin(ang)
    return out


def _rope_pairs_swapped(rotary_dim, style):
    return _orig_pairs(rotary_dim, 1 - style)


_orig_pairs = NR.rope_pairs

_orig_windows = FO.forced_windows
_orig_forced = FO.select_forced_row


def _forced_select_ties_high(scores, L, topk, init_blocks, local_blocks, max_k_tiles,
                             local_score=None):
    s = np.asarray(scores, dtype=np.float64)[:max(L, 0)]
    s = np.append(s, np.nan if local_score is None else local_score)
    out = np.full(topk, -1, dtype=np.int32)
    if L < 0:
        return out
    nvp = L + 1
    if nvp <= topk:
        out[:nvp] = np.arange(nvp)
        return out
    fb, fe = _orig_windows(L, topk, init_blocks, local_blocks, max_k_tiles)
    cand = list(range(fb, nvp - fe))
    cand.sort(key=lambda j: (np.isnan(s[j]), -s[j] if not np.isnan(s[j]) else 0.0, -j))
    sel = sorted(list(range(fb)) + list(range(nvp - fe, nvp)) + cand[:topk - fb - fe])
    out[:len(sel)] = sel
    return out


def _forced_descending(scores, L, topk, init_blocks, local_blocks, max_k_tiles,
                       local_score=None):
    out = _orig_forced(scores, L, topk, init_blocks, local_blocks, max_k_tiles,
                       local_score=local_score)
    ids = out[out >= 0][::-1]
    out[:len(ids)] = ids
    return out


MUTATIONS = {
    "nibbles_swapped": [(I, "decode_pages", _decode_pages_swapped_nibbles)],
    "scale_dropped": [(I, "decode_pages", _decode_pages_no_scale)],
    "scales_reversed": [(I, "decode_pages", _decode_pages_reversed_scales)],
    "tokens_dims_transposed": [(I, "decode_pages", _decode_pages_transposed)],
    "e4m3_bias_8": [(F, "e4m3fn_to_float", _e4m3_bias8), (oracle, "e4m3fn_to_float", _e4m3_bias8),
                    (I, "e4m3fn_to_float", _e4m3_bias8)],
    "bf16_bias_126": [(F, "bf16_to_float", _bf16_bias_126), (oracle, "bf16_to_float", _bf16_bias_126),
                      (I, "bf16_to_float", _bf16_bias_126)],
    "ties_to_higher_id": [(I, "select_row", _select_ties_high), (oracle, "select_row", _select_ties_high)],
    "nan_ranks_first": [(I, "select_row", _select_nan_first), (oracle, "select_row", _select_nan_first)],
    "local_leaks": [(I, "select_row", _select_local_in_history)],
    "sum_not_max": [(I, "page_scores", _page_scores_sum)],
    "page_max_drops_nan": [(I, "page_scores", _page_scores_nanmax)],
    "rows_past_max_pages_clamped": [(I, "local_pages", _local_pages_clamped)],
    "local_score_misses_own_token": [(I, "local_page_scores", _local_scores_nt(-1))],
    "local_score_sees_next_token": [(I, "local_page_scores", _local_scores_nt(1))],
    "local_page_never_wins": [(FO, "select_forced_row", _forced_local_ignored),
                              (oracle, "select_forced_row", _forced_local_ignored)],
    "decode_positions_shifted": [(I, "rows_decode", _rows_decode_shifted),
                                 (oracle, "rows_decode", _rows_decode_shifted)],
    "prefill_positions_shifted": [(I, "rows_prefill", _rows_prefill_off_by_one),
                                  (oracle, "rows_prefill", _rows_prefill_off_by_one)],
    "encoder_ties_away": [(F, "mxfp4_encode_rows", _encode_ties_away),
                          (oracle, "mxfp4_encode_rows", _encode_ties_away)],
    "encoder_exponent_off_by_one": [(F, "mxfp4_encode_rows", _encode_exp_minus_one),
                                    (oracle, "mxfp4_encode_rows", _encode_exp_minus_one)],
    "chunks_overfill": [(oracle, "prefill_chunks",
                         lambda s, b: _orig_chunks(s, b + 1))],
    "forced_end_window_one_wider": [(FO, "forced_windows",
                                     lambda L, k, i, l, m: (lambda fb, fe: (fb, min(fe + 1, k - fb)))(
                                         *_orig_windows(L, k, i, l, m)))],
    "forced_begin_ignores_max_k_tiles": [(FO, "forced_windows",
                                          lambda L, k, i, l, m: _orig_windows(L, k, i, l, 10 ** 9))],
    "forced_ties_to_higher_id": [(FO, "select_forced_row", _forced_select_ties_high),
                                 (oracle, "select_forced_row", _forced_select_ties_high)],
    "forced_output_descending": [(FO, "select_forced_row", _forced_descending),
                                 (oracle, "select_forced_row", _forced_descending)],
    "rms_eps_outside_sqrt": [(NR, "rms_norm", _rms_eps_outside), (oracle, "rms_norm", _rms_eps_outside)],
    "rms_sum_not_mean": [(NR, "rms_norm", _rms_sum_not_mean), (oracle, "rms_norm", _rms_sum_not_mean)],
    "rope_sin_flipped": [(NR, "rope", _rope_sin_flipped), (oracle, "rope", _rope_sin_flipped)],
    "rope_half_frequency": [(NR, "rope", _rope_half_frequency),
                            (oracle, "rope", _rope_half_frequency)],
    "rope_pairings_swapped": [(NR, "rope_pairs", _rope_pairs_swapped)],
}


def test_pins_pass_on_the_unmodified_oracle():
    assert not _some_pin_fails()


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    for mod, attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, fn)
    assert _some_pin_fails(), f"no pin caught the planted mistake {name!r}"
