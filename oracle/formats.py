"""Number formats of the index cache and index query, written out from their
definitions (test infrastructure; see the package docstring).

The pages name the formats only: the ROCm page (``indexer_mxfp4``, module
docstring) says the index-K pages hold "e2m1 / e8m0" data, 8704 bytes per
128-token page (``mxfp4_index_topk_decode`` argument comment); the NVFP4 page
(``indexer_nvfp4``, module docstring and ``reserve_workspace``) says index-Q is
E4M3 (``torch.float8_e4m3fn``).  The bit-level definitions below are those of
the OCP 8-bit floating point specification (E4M3, "fn" variant: bias 7, no
infinities, only S.1111.111 is NaN) and the OCP Microscaling (MX) v1.0
specification (E2M1 element: bias 1, no inf/NaN; E8M0 scale: 2^(b-127), 0xFF
is NaN; one scale per block of 32 elements).

Page layout (a reading: the pages print the page size and that there is a code
part and a scale part, not the byte offsets): a page is 128 tokens of 68 bytes.
Token ``t`` of a page starts at byte ``68*t``; bytes ``[0, 64)`` hold the 128
E2M1 codes of the token, two per byte, dimension ``2i`` in the low nibble of
byte ``i`` and ``2i+1`` in the high nibble; bytes ``[64, 68)`` hold the E8M0
scales of dimensions ``[0,32)``, ``[32,64)``, ``[64,96)`` and ``[96,128)``.
"""

import numpy as np

HEAD_DIM = 128
PAGE_TOKENS = 128
BLOCK = 32                      # MX block: elements sharing one E8M0 scale
CODE_BYTES = HEAD_DIM // 2      # 64 bytes of packed E2M1 codes per token
SCALE_BYTES = HEAD_DIM // BLOCK  # 4 E8M0 bytes per token
TOKEN_BYTES = CODE_BYTES + SCALE_BYTES  # 68
PAGE_BYTES = PAGE_TOKENS * TOKEN_BYTES  # 8704


def e4m3fn_to_float(codes):
    """FP8 E4M3 ("fn") byte -> float64 value.

    sign s = bit 7, exponent e = bits 6..3, mantissa m = bits 2..0.
    e == 0: (-1)^s * (m/8) * 2^(1-7)      (subnormal)
    else  : (-1)^s * (1 + m/8) * 2^(e-7)
    e == 15 and m == 7: NaN (the only non-finite code; no infinities).
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0 ** (1 - 7)
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def bf16_to_float(bits):
    """bfloat16 bit pattern (uint16) -> float64 value.

    sign s = bit 15, exponent e = bits 14..7 (bias 127), mantissa m = bits 6..0.
    e == 0  : (-1)^s * (m/128) * 2^(1-127)    (subnormal)
    e == 255: (-1)^s * inf if m == 0, else NaN
    else    : (-1)^s * (1 + m/128) * 2^(e-127)
    (The index-Q dtype the vllm "indexer_mxfp4" page accepts besides E4M3.)
    """
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    s = (b >> 15) & 1
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    sub = (m / 128.0) * 2.0 ** (1 - 127)
    nrm = (1.0 + m / 128.0) * np.exp2(e.astype(np.float64) - 127.0)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where(e == 255, np.where(m == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def e2m1_to_float(codes):
    """FP4 E2M1 nibble -> float64 value.

    sign s = bit 3, exponent e = bits 2..1, mantissa m = bit 0, bias 1.
    e == 0: (-1)^s * (m/2) * 2^(1-1)      (subnormal: 0 or 0.5)
    else  : (-1)^s * (1 + m/2) * 2^(e-1)
    Magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6.
    """
    c = np.asarray(codes).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 0x3
    m = c & 0x1
    sub = (m / 2.0) * 2.0 ** (1 - 1)
    nrm = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    mag = np.where(e == 0, sub, nrm)
    return np.where(s == 1, -mag, mag)


def e8m0_to_float(codes):
    """E8M0 scale byte -> float64: 2^(b - 127); b == 255 is NaN."""
    b = np.asarray(codes).astype(np.int64)
    v = np.exp2(b.astype(np.float64) - 127.0)
    return np.where(b == 255, np.nan, v)


# E2M1 magnitudes of codes 0..7 (the sign is bit 3).
_E2M1_MAG = e2m1_to_float(np.arange(8))


def _floor_log2(x):
    """floor(log2(x)) for finite x > 0, exactly (from the binary exponent)."""
    _, ex = np.frexp(x)          # x = f * 2^ex with f in [0.5, 1)
    return ex.astype(np.int64) - 1


def mxfp4_encode_rows(rows, chunk=8192):
    """Quantise rows of 128 values to MXFP4: returns (codes [n,128] in 0..15,
    scale bytes [n,4]).

    The OCP MX v1.0 conversion, block by block (32 elements):
      1. amax = max |v| over the block;
      2. shared exponent X = floor(log2(amax)) - emax_elem, emax_elem = 2 for
         E2M1 (its largest magnitude 6 = 1.5 * 2^2), clamped to the E8M0
         range [-127, 127]; a block of zeros takes the smallest scale
         (byte 0);
      3. each element v / 2^X is rounded to the nearest E2M1 value, ties to
         the code with an even (zero) mantissa bit; magnitudes above 6 become
         6 (the nearest grid point), and the sign bit is the sign bit of v
         (so a negative value that rounds to zero is code 8).

    Inputs must be finite.  The arithmetic is fp64, where v / 2^X is exact for
    every fp32 or bf16 input.  Rows are processed ``chunk`` at a time only to
    bound memory; each row is encoded on its own.
    """
    rows = np.asarray(rows).reshape(-1, HEAD_DIM)
    if rows.shape[0] > chunk:
        parts = [mxfp4_encode_rows(rows[i:i + chunk], chunk)
                 for i in range(0, rows.shape[0], chunk)]
        return (np.concatenate([p[0] for p in parts]),
                np.concatenate([p[1] for p in parts]))
    v = np.asarray(rows, dtype=np.float64).reshape(-1, HEAD_DIM // BLOCK, BLOCK)
    if not np.all(np.isfinite(v)):
        raise ValueError("MXFP4 encoder input must be finite")
    amax = np.abs(v).max(axis=2)                         # [n, 4]
    safe = np.where(amax > 0, amax, 1.0)
    X = np.where(amax > 0, _floor_log2(safe) - 2, -127)
    X = np.clip(X, -127, 127)
    scale_bytes = (X + 127).astype(np.uint8)             # [n, 4]
    x = np.abs(v) / np.exp2(X.astype(np.float64))[:, :, None]
    # Nearest grid magnitude by brute force over the 8 magnitudes.
    dist = np.abs(x[..., None] - _E2M1_MAG)               # [n, 4, 32, 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                                   # one or two (a tie)
    # Among tied candidates take the even mantissa (code & 1 == 0).
    even = (np.arange(8) & 1) == 0
    pick_even = cand & even
    has_even = pick_even.any(axis=-1, keepdims=True)
    choose = np.where(has_even, pick_even, cand)
    mag_code = np.argmax(choose, axis=-1)                 # first True
    sign = np.signbit(v).astype(np.int64)
    codes = (mag_code | (sign << 3)).reshape(-1, HEAD_DIM)
    return codes.astype(np.uint8), scale_bytes.reshape(-1, SCALE_BYTES)


def pack_tokens(codes, scale_bytes):
    """Codes [n,128] and scale bytes [n,4] -> token records [n,68] uint8."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes[:, 0::2]
    hi = codes[:, 1::2]
    out = np.empty((codes.shape[0], TOKEN_BYTES), dtype=np.uint8)
    out[:, :CODE_BYTES] = lo | (hi << 4)
    out[:, CODE_BYTES:] = scale_bytes
    return out


def write_pages(pages, slots, k_rows):
    """The index-K insert: quantise ``k_rows`` [n,128] (fp32 or bf16 values)
    and store token ``i`` at slot ``slots[i]`` = physical_page * 128 + offset
    of ``pages`` ([num_blocks, 8704] or [num_blocks,128,68] uint8).  Negative
    slots are skipped."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    codes, sb = mxfp4_encode_rows(np.asarray(k_rows)[keep])
    rec = pack_tokens(codes, sb)
    flat = pages.reshape(-1, PAGE_TOKENS, TOKEN_BYTES)
    s = slots[keep]
    flat[s // PAGE_TOKENS, s % PAGE_TOKENS, :] = rec
    return pages


def decode_pages(page_bytes):
    """Page bytes [J, 8704] (or [J,128,68]) -> K values [J, 128, 128] fp64."""
    p = np.asarray(page_bytes, dtype=np.uint8).reshape(-1, PAGE_TOKENS, TOKEN_BYTES)
    cb = p[:, :, :CODE_BYTES].astype(np.int64)
    codes = np.empty(p.shape[:2] + (HEAD_DIM,), dtype=np.int64)
    codes[:, :, 0::2] = cb & 0xF
    codes[:, :, 1::2] = cb >> 4
    vals = e2m1_to_float(codes)
    scales = e8m0_to_float(p[:, :, CODE_BYTES:])          # [J, 128, 4]
    return vals * np.repeat(scales, BLOCK, axis=2)
