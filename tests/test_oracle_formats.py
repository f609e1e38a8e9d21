"""Pins of the oracle's number formats and MXFP4 encoder (CPU only)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F
from tests import pins


def test_e4m3_all_codes_match_torch_cast():
    codes = np.arange(256)
    mine = oracle.e4m3fn_to_float(codes)
    ref = pins.torch_e4m3(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.array_equal(np.signbit(mine[ok]), np.signbit(ref[ok]))


def test_e4m3_golden_points():
    for code, val in pins.golden_e4m3_points().items():
        got = float(oracle.e4m3fn_to_float(code))
        if np.isnan(val):
            assert np.isnan(got), hex(code)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), hex(code)


def test_e8m0_all_codes_match_torch_cast():
    codes = np.arange(256)
    mine = oracle.e8m0_to_float(codes)
    ref = pins.torch_e8m0(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert mine[127] == 1.0 and mine[0] == 2.0 ** -127 and mine[254] == 2.0 ** 127


def test_bf16_all_patterns_match_torch_cast():
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = F.bf16_to_float(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_bf16_golden_points():
    # hand-derived from the format: sign | 8-bit exponent (bias 127) | 7-bit mantissa
    pts = {0x3F80: 1.0, 0xC000: -2.0, 0x3FC0: 1.5, 0x0080: 2.0 ** -126,
           0x0001: 2.0 ** -133, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,
           0x7F80: np.inf, 0xFF80: -np.inf, 0x8000: -0.0, 0x4049: 3.140625}
    for b, v in pts.items():
        got = float(F.bf16_to_float(np.array([b], dtype=np.uint16))[0])
        assert got == v and np.signbit(got) == np.signbit(v), (hex(b), got, v)
    assert np.isnan(F.bf16_to_float(np.array([0x7FC0], dtype=np.uint16))[0])


def test_e2m1_matches_hand_typed_table():
    g = pins.golden_e2m1()
    got = oracle.e2m1_to_float(np.arange(16))
    for c in range(16):
        assert got[c] == g[c] and np.signbit(got[c]) == np.signbit(g[c]), c


@pytest.mark.parametrize("case", range(len(pins.golden_mxfp4_blocks())))
def test_encoder_worked_examples(case):
    vals, scale_byte, codes = pins.golden_mxfp4_blocks()[case]
    row = np.zeros(128)
    row[32:64] = vals           # put the block in the second scale block
    c, s = oracle.mxfp4_encode_rows(row[None, :])
    assert s[0, 1] == scale_byte
    assert np.array_equal(c[0, 32:64], codes)
    assert s[0, 0] == 0 and np.all(c[0, :32] == 0)


def _rne_reference(v):
    """Round |x| to the E2M1 grid by numpy's round-half-to-even at the
    grid spacing of x's binade (0.5 below 2, 1 in [2,4), 2 in [4,8)), then
    saturate at 6.  Independent of the oracle's nearest-point search."""
    a = np.abs(v)
    spacing = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    r = np.minimum(np.round(a / spacing) * spacing, 6.0)
    return np.where(np.signbit(v), -r, r)


def test_encoder_matches_round_half_even_reference():
    rng = np.random.default_rng(7)
    rows = rng.standard_normal((4000, 128)).astype(np.float32)
    # exact midpoints and saturation cases, scaled per block
    rows[:50] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, 7.9, -0.2],
                           size=(50, 128)) * 2.0 ** rng.integers(-3, 4, size=(50, 1))
    rows[50:60] *= 1e-30        # tiny blocks
    rows[60:70] *= 1e30         # huge blocks
    codes, sb = oracle.mxfp4_encode_rows(rows)
    X = sb.astype(np.int64) - 127
    x = rows.astype(np.float64).reshape(-1, 4, 32) / np.exp2(X)[:, :, None]
    want = _rne_reference(x).reshape(-1, 128)
    got = oracle.e2m1_to_float(codes)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))
    # shared exponent: amax / 2^X lies in [4, 8) for every non-zero block
    amax = np.abs(rows.astype(np.float64)).reshape(-1, 4, 32).max(axis=2)
    ratio = amax / np.exp2(X)
    assert np.all((ratio >= 4) & (ratio < 8))


def test_encoder_idempotent_and_monotone():
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((500, 128)).astype(np.float32)
    c1, s1 = oracle.mxfp4_encode_rows(rows)
    deq = oracle.e2m1_to_float(c1) * np.repeat(oracle.e8m0_to_float(s1), 32, axis=1)
    c2, s2 = oracle.mxfp4_encode_rows(deq)
    assert np.array_equal(s1, s2)
    assert np.array_equal(oracle.e2m1_to_float(c1), oracle.e2m1_to_float(c2))
    # within a block (same scale), quantisation is monotone
    blk = np.sort(rng.standard_normal((1, 32)))
    row = np.zeros((1, 128))
    row[0, :32] = blk
    c, _ = oracle.mxfp4_encode_rows(row)
    v = oracle.e2m1_to_float(c[0, :32])
    assert np.all(np.diff(v) >= 0)


def test_encoder_bf16_inputs_same_as_their_fp32_values():
    rng = np.random.default_rng(11)
    x = torch.from_numpy(rng.standard_normal((64, 128)).astype(np.float32)).to(torch.bfloat16)
    a = oracle.mxfp4_encode_rows(x.float().numpy())
    b = oracle.mxfp4_encode_rows(x.float().numpy().astype(np.float64))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_token_bytes_layout():
    codes = np.zeros((1, 128), dtype=np.uint8)
    codes[0, 0] = 0x3      # dim 0 -> low nibble of byte 0
    codes[0, 1] = 0xC      # dim 1 -> high nibble of byte 0
    codes[0, 127] = 0x7    # dim 127 -> high nibble of byte 63
    sb = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    rec = F.pack_tokens(codes, sb)
    assert rec.shape == (1, 68)
    assert rec[0, 0] == 0xC3 and rec[0, 63] == 0x70 and list(rec[0, 64:]) == [1, 2, 3, 4]


def test_write_then_decode_pages():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((300, 128)).astype(np.float32)
    pool = np.zeros((4, 8704), dtype=np.uint8)
    slots = rng.permutation(512)[:300]
    oracle.write_pages(pool, slots, k)
    vals = oracle.decode_pages(pool).reshape(512, 128)
    c, s = oracle.mxfp4_encode_rows(k)
    g = pins.golden_e2m1()
    want = np.vectorize(lambda x: g[int(x)])(c) * np.repeat(pins.torch_e8m0(s), 32, axis=1)
    assert np.array_equal(vals[slots], want)
    # error bound: half a grid step (at most 2^X) below 6 * 2^X, and under
    # 2 * 2^X for the saturated values in (6, 8) * 2^X
    err = np.abs(vals[slots] - k)
    scale = np.repeat(pins.torch_e8m0(s), 32, axis=1)
    assert np.all(err <= 2.0 * scale)
    small = np.abs(k) <= 6 * scale
    assert np.all(err[small] <= scale[small])
