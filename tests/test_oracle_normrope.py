"""Pins of the oracle's qk-norm and rotary embedding (``oracle.normrope``):
closed forms on hand-chosen rows, the group properties of rotations (norm
kept, position 0 the identity, angles adding, dot products depending only on
the position difference), the fixed relation between the two pairings, and
the per-pair frequencies."""

import math

import numpy as np

import oracle


def test_rms_norm_closed_form():
    x = np.zeros((1, 128))
    x[0, 0], x[0, 1] = 3.0, 4.0                           # mean square 25/128
    y = oracle.rms_norm(x, np.ones(128), 0.0)
    assert abs(y[0, 0] - 3.0 * math.sqrt(128) / 5.0) < 1e-13
    assert abs(y[0, 1] - 4.0 * math.sqrt(128) / 5.0) < 1e-13
    assert np.all(y[0, 2:] == 0.0)
    # a constant row a with eps: a / sqrt(a^2 + eps), times the weight
    x = np.full((1, 128), 0.5)
    w = np.arange(128) / 64.0
    y = oracle.rms_norm(x, w, 0.25)
    assert np.allclose(y[0], 0.5 / math.sqrt(0.25 + 0.25) * w, rtol=0, atol=1e-15)


def test_rms_norm_properties():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 128)) * rng.uniform(0.1, 10, size=(50, 1))
    y = oracle.rms_norm(x, np.ones(128), 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-12)
    assert np.allclose(oracle.rms_norm(7.5 * x, np.ones(128), 0.0), y, rtol=1e-12)
    assert np.array_equal(oracle.rms_norm(x, None, 1e-6), x)      # no weight: no norm


def test_rope_worked_examples():
    p = 3.0
    e0 = np.zeros((1, 128))
    e0[0, 0] = 1.0
    y = oracle.rope(e0, [p], 128, 10000.0, oracle.NEOX)   # pair (0, 64), frequency 1
    assert abs(y[0, 0] - math.cos(p)) < 1e-15 and abs(y[0, 64] - math.sin(p)) < 1e-15
    e1 = np.zeros((1, 128))
    e1[0, 1] = 1.0
    y = oracle.rope(e1, [p], 128, 10000.0, oracle.INTERLEAVED)   # pair (0, 1)
    assert abs(y[0, 0] + math.sin(p)) < 1e-15 and abs(y[0, 1] - math.cos(p)) < 1e-15
    # pair i turns by base^(-2i/rotary_dim) per position
    for rd, base in ((128, 10000.0), (64, 500000.0)):
        for i in (1, 5, rd // 2 - 1):
            x = np.zeros((1, 128))
            x[0, i] = 1.0
            y = oracle.rope(x, [1.0], rd, base, oracle.NEOX)
            assert abs(y[0, i] - math.cos(base ** (-2.0 * i / rd))) < 1e-15


def test_rope_group_properties():
    rng = np.random.default_rng(12)
    for style in (oracle.NEOX, oracle.INTERLEAVED):
        for rd in (128, 64, 8):
            x = rng.standard_normal((20, 128))
            pa = rng.integers(0, 300000, size=20).astype(np.float64)
            pb = rng.integers(0, 300000, size=20).astype(np.float64)
            y = oracle.rope(x, pa, rd, 10000.0, style)
            assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
            assert np.array_equal(y[:, rd:], x[:, rd:])                     # unrotated dims
            assert np.allclose(oracle.rope(x, np.zeros(20), rd, 10000.0, style), x, atol=0)
            both = oracle.rope(oracle.rope(x, pa, rd, 10000.0, style), pb, rd, 10000.0, style)
            assert np.allclose(both, oracle.rope(x, pa + pb, rd, 10000.0, style), atol=1e-8)
            k = rng.standard_normal((20, 128))
            lhs = np.sum(y * oracle.rope(k, pb, rd, 10000.0, style), axis=1)
            rhs = np.sum(oracle.rope(x, pa - pb, rd, 10000.0, style) * k, axis=1)
            assert np.allclose(lhs, rhs, atol=1e-8)


def test_pairings_are_one_permutation_apart():
    rng = np.random.default_rng(13)
    rd = 64
    x = rng.standard_normal((10, 128))
    pos = rng.integers(0, 5000, size=10)
    # dim i of the neox layout sits at 2i (i < rd/2) or 2(i - rd/2) + 1
    perm = np.arange(128)
    perm[:rd] = np.concatenate([np.arange(0, rd, 2), np.arange(1, rd, 2)])
    a = oracle.rope(x, pos, rd, 10000.0, oracle.NEOX)
    # move x into the interleaved layout, rotate, move back
    xi = np.empty_like(x)
    xi[:, perm] = x
    bi = oracle.rope(xi, pos, rd, 10000.0, oracle.INTERLEAVED)
    assert np.allclose(bi[:, perm], a, atol=1e-12)
