"""Pins of the oracle's Q/K preprocessing ([VC] §3.4 and Appendix B: rotary
embedding, key centring, QK Hadamard rotation, fused ahead of the quantisers).

Checked against things other than the oracle itself: scipy's Sylvester
Hadamard matrix, numpy complex multiplication, fp64 channel means, and the
invariance of exact fp64 softmax attention under key centring and under an
orthogonal rotation applied to both Q and K.
"""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import exact


def _bits(x):
    return oracle.f32_to_bf16_bits(np.asarray(x, np.float32))


def rope_tables(S, D, base=10000.0, offset=0):
    """1-D rotary tables: angle of pair i at position p = p * base^(-2i/D)."""
    p = np.arange(S, dtype=np.float64)[:, None] + offset
    inv = base ** (-2.0 * np.arange(D // 2) / D)
    th = p * inv[None, :]
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


@pytest.mark.parametrize("D", [64, 128])
def test_hadamard_is_sylvester_matrix(D):
    rng = np.random.default_rng(D)
    x = _bits(rng.standard_normal((50, D)) * 3)
    y, _ = oracle.prep_rows(x, oracle.PREP_HADAMARD)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    ref = xf @ scipy.linalg.hadamard(D).T.astype(np.float64)
    err = np.abs(y - ref).max(axis=1)
    assert np.all(err <= 8 * 2.0 ** -24 * np.abs(xf).sum(axis=1) * math.log2(D))
    # H H^T = D I: norms grow by sqrt(D)
    assert np.allclose((y.astype(np.float64) ** 2).sum(1), D * (xf ** 2).sum(1), rtol=1e-5)


def test_rope_is_complex_rotation():
    S, D = 40, 64
    rng = np.random.default_rng(3)
    x = _bits(rng.standard_normal((S, D)))
    c, s = rope_tables(S, D)
    y, _ = oracle.prep_rows(x, oracle.PREP_ROPE, c, s)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float64)
    z = (xf[:, 0::2] + 1j * xf[:, 1::2]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
    assert np.abs(y[:, 0::2] - z.real).max() <= 4e-6 * np.abs(xf).max()
    assert np.abs(y[:, 1::2] - z.imag).max() <= 4e-6 * np.abs(xf).max()
    # position 0 is the identity (angle 0)
    assert (y[0] == oracle.bf16_bits_to_f32(x[0])).all()


def test_centring_mean():
    S, D = 333, 64
    rng = np.random.default_rng(4)
    x = _bits(rng.standard_normal((S, D)) + rng.standard_normal(D) * 5)  # per-channel bias
    c, s = rope_tables(S, D)
    y0, _ = oracle.prep_rows(x, oracle.PREP_ROPE, c, s)
    y, mean = oracle.prep_rows(x, oracle.PREP_ROPE | oracle.PREP_CENTER, c, s)
    want = y0.astype(np.float64).mean(axis=0)
    assert np.abs(mean - want).max() <= 2.0 ** -24 + 1e-6 * np.abs(want).max()
    assert np.allclose(y, y0 - mean[None, :], atol=0, rtol=0)
    assert np.abs(y.astype(np.float64).mean(axis=0)).max() <= 1e-5 * np.abs(y0).max()


def test_prep_leaves_exact_attention_unchanged():
    # softmax(q K^T) is invariant to a vector subtracted from every key, and
    # (Hq).(Hk) = D q.k: exact attention on the prepared operands, scores
    # divided by D, equals exact attention on the rotary-embedded operands
    S, D, sm = 300, 64, 1 / 8
    rng = np.random.default_rng(5)
    q = _bits(rng.standard_normal((S, D)))
    k = _bits(rng.standard_normal((S, D)) + rng.standard_normal(D) * 4)
    v = rng.standard_normal((S, D))
    c, s = rope_tables(S, D)
    qr, _ = oracle.prep_rows(q, oracle.PREP_ROPE, c, s)
    kr, _ = oracle.prep_rows(k, oracle.PREP_ROPE, c, s)
    qp, _ = oracle.prep_rows(q, oracle.PREP_ROPE | oracle.PREP_HADAMARD, c, s)
    kp, _ = oracle.prep_rows(k, oracle.PREP_ROPE | oracle.PREP_CENTER | oracle.PREP_HADAMARD, c, s)
    ref = exact.attention_rows(qr.astype(np.float64), kr.astype(np.float64), v, sm)
    got = exact.attention_rows(qp.astype(np.float64), kp.astype(np.float64), v, sm / D)
    assert np.abs(got - ref).max() <= 1e-4 * np.abs(ref).max()


def test_pipeline_with_prep_tracks_exact_attention():
    # the quantised emulation with all three steps tracks exact attention on
    # the rotary-embedded operands to the ExpCast + FP8 level (about 0.11 on
    # these near-uniform rows, as without any preprocessing), while skipping
    # the rotary step is an order of magnitude off
    S, D, sm = 700, 64, 0.25
    rng = np.random.default_rng(6)
    q = rng.standard_normal((1, S, 1, D)).astype(np.float32)
    k = (rng.standard_normal((1, S, 1, D)) + rng.standard_normal(D) * 4).astype(np.float32)
    v = rng.standard_normal((1, S, 1, D)).astype(np.float32)
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    c, s = rope_tables(S, D)
    res = oracle.pipeline_head(qb, kb, vb, 0, 0, vsmooth=False, sm_scale=sm, prep=7, rope_cos=c, rope_sin=s)
    plain = oracle.pipeline_head(qb, kb, vb, 0, 0, vsmooth=False, sm_scale=sm)
    qr, _ = oracle.prep_rows(qb[0, :, 0], oracle.PREP_ROPE, c, s)
    kr, _ = oracle.prep_rows(kb[0, :, 0], oracle.PREP_ROPE, c, s)
    ref = exact.attention_rows(qr.astype(np.float64), kr.astype(np.float64),
                               oracle.bf16_bits_to_f32(vb[0, :, 0]).astype(np.float64), sm)
    err = np.linalg.norm(res["out_f32"] - ref) / np.linalg.norm(ref)
    assert err < 0.15, err
    assert np.linalg.norm(plain["out_f32"] - ref) / np.linalg.norm(ref) > 5 * err
