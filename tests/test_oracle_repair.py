"""Pins of the oracle's V residual repair ([OVC] "Why V residual repair"):
with one V scale per head, the top rho*S tokens by residual energy become
extra value rows (their residuals) paired with copies of their keys, visited
last, numerator only.

Checked against: numpy top-k over independently computed residual
energies; E4M3's half-step on the residual rows; the integer-score special
case, where the emulation must equal exact base-2 softmax attention over the
repaired values (a repair row counted in the denominator, or a wrong residual,
breaks it); and a lower error against exact attention on heavy-tailed V.
"""
import math

import numpy as np
import pytest

import oracle
import vcsynth
from oracle import exact


def _bits(x):
    return oracle.f32_to_bf16_bits(np.asarray(x, np.float32))


def _residuals(vb):
    """numpy residuals r = v - s dec(code) of per-head V quantisation."""
    S, D = vb.shape
    codes, sc = oracle.quantize_v(vb[None, :, None, :])
    s = np.float32(sc[0, 0, 0])
    deq = (oracle.e4m3_decode(codes[0, 0, :, :S]).T.astype(np.float32) * s).astype(np.float32)
    v = oracle.bf16_bits_to_f32(vb).astype(np.float32)
    return (v - deq).astype(np.float32), s


@pytest.mark.parametrize("R", [1, 7, 130])
def test_selection_is_top_energy(R):
    q, k, v = vcsynth.random_qkv(1, 1000, 1, 64, seed=R, v_kind="t3")
    vb = vcsynth.bf16_bits(v)[0, :, 0]
    idx, e = oracle.repair_select(vb, R)
    r, _ = _residuals(vb)
    e_np = (r.astype(np.float64) ** 2).sum(axis=1)
    assert np.allclose(e, e_np, rtol=1e-12, atol=0)
    want = np.sort(np.argsort(-e_np, kind="stable")[:R])
    assert (idx == want).all()
    assert (np.diff(idx) > 0).all()


def test_residual_rows_within_half_step():
    q, k, v = vcsynth.random_qkv(1, 900, 1, 128, seed=2, v_kind="t3")
    vb = vcsynth.bf16_bits(v)[0, :, 0]
    idx, _ = oracle.repair_select(vb, 40)
    rv = oracle.repair_rows(vb, idx)
    assert rv.shape == (128, 128) and (rv[:, 40:] == 0).all()
    r, s = _residuals(vb)
    got = oracle.e4m3_decode(rv[:, :40]).T * float(s)
    want = r[idx].astype(np.float64)
    big = np.abs(want) >= 2.0 ** -6 * float(s)
    assert np.all(np.abs(got - want)[big] <= np.abs(want)[big] * 2.0 ** -4)
    # the repaired rows are closer to V than the plain ones
    v64 = oracle.bf16_bits_to_f32(vb[idx]).astype(np.float64)
    assert np.linalg.norm(v64 - (v64 - want + got)) < 0.2 * np.linalg.norm(want)


def _integer_qk(S, D, seed):
    rng = np.random.default_rng(seed)
    q = np.zeros((S, D), np.float32)
    k = np.zeros((S, D), np.float32)
    q[:, 0] = 448.0
    k[:, 1] = 448.0
    for x in (q, k):
        for i in range(S):
            ch = rng.choice(np.arange(2, D), size=rng.integers(0, 8), replace=False)
            x[i, ch] = rng.choice([-1.0, 1.0], size=ch.size)
    return q, k


def test_integer_scores_with_repair_equal_exact_softmax():
    # c1 = 1 makes every score an integer and every code an exact power of two
    S, D, R = 400, 64, 9
    q, k = _integer_qk(S, D, seed=77)
    _, _, v = vcsynth.random_qkv(1, S, 1, D, seed=8, v_kind="t3")
    qb, kb, vb = _bits(q), _bits(k), vcsynth.bf16_bits(v)[0, :, 0]
    qc, qs = oracle.quantize_qk(qb[None, :, None, :])
    kc, ks = oracle.quantize_qk(kb[None, :, None, :])
    vc, vs = oracle.quantize_v(vb[None, :, None, :])
    idx, _ = oracle.repair_select(vb, R)
    rk, rks = oracle.quantize_f32_pow2(oracle.bf16_bits_to_f32(kb[idx]).astype(np.float32))
    assert (rks == 1).all()
    rv = oracle.repair_rows(vb, idx)
    rows = np.arange(S)
    of, _, _ = oracle.attn_emulate_rows(qc[0, 0], qs[0, 0], kc[0, 0], ks[0, 0], vc[0, 0], vs[0, 0], None, S, 1.0,
                                        rows, repair=dict(rk_codes=rk, rk_scale=rks, rv_codes_t=rv, R=R))
    s = float(vs[0, 0, 0])
    v_eff = oracle.e4m3_decode(vc[0, 0, :, :S]).T * s
    v_eff[idx] += oracle.e4m3_decode(rv[:, :R]).T * s
    qi = oracle.e4m3_decode(qc[0, 0, :S])
    ki = oracle.e4m3_decode(kc[0, 0, :S])
    ref = exact.attention_rows(qi, ki, v_eff, math.log(2.0))
    assert np.abs(of - ref).max() <= 2e-6 * np.abs(ref).max()
    # without the repair rows the same comparison is visibly off
    of0, _, _ = oracle.attn_emulate_rows(qc[0, 0], qs[0, 0], kc[0, 0], ks[0, 0], vc[0, 0], vs[0, 0], None, S, 1.0,
                                         rows)
    assert np.abs(of0 - ref).max() > 100 * np.abs(of - ref).max()


def test_repair_lowers_error_on_outlier_values():
    # the tiny workload's V has 1% outlier tokens (x20 in a few channels), so
    # the per-head V scale leaves the other tokens few bits: repairing the
    # worst 0.5% / 2% lowers the error against exact attention, on each head
    q, k, v = vcsynth.make_qkv("tiny")
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    S, D = q.shape[1], q.shape[3]
    sm = 1 / math.sqrt(D)
    for h in range(q.shape[2]):
        ref = exact.attention_rows(exact.to_f64(qb[0, :, h]), exact.to_f64(kb[0, :, h]), exact.to_f64(vb[0, :, h]),
                                   sm)
        errs = []
        for rho in (0.0, 0.005, 0.02):
            res = oracle.pipeline_head(qb, kb, vb, 0, h, vsmooth=False, sm_scale=sm, repair_rho=rho)
            errs.append(np.linalg.norm(res["out_f32"] - ref) / np.linalg.norm(ref))
        assert errs[1] < errs[0] and errs[2] < errs[1], (h, errs)
