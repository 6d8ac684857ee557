"""Pins of the oracle's 4-bit path (MXFP4: E2M1 elements, one power-of-two
scale per 32 elements), the gfx950 form of [VC]'s 4-bit V-Smooth without
ExpCast ([VC] §4.1 "Implementation" and "Scope of ExpCast-FP8").

Checked against: a generic minifloat decoder, first checked on E4M3 against
the oracle's pinned E4M3 decoder and then instantiated for E2M1 (sign, 2
exponent bits with bias 1, 1 mantissa bit, subnormals); a brute-force
nearest search with the tie rule; the minimality of the block exponent;
and, for the attention emulation, cases where every probability is exactly
representable (integer log2 scores within 3 of their block's maximum), so
the emulation must equal exact base-2 softmax attention over the dequantised
values -- with and without V-Smooth's block means, across running-max
increases.  A wrong block partition, scale, rescale or row sum breaks them.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import exact


def minifloat_decode(code, ebits, mbits, bias):
    """Generic sign/exponent/mantissa decoder with subnormals (no inf/nan)."""
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        mag = m / (1 << mbits) * 2.0 ** (1 - bias)
    else:
        mag = (1 + m / (1 << mbits)) * 2.0 ** (e - bias)
    return -mag if s else mag


def test_generic_decoder_reproduces_e4m3():
    for c in range(256):
        if (c & 0x7f) == 0x7f:
            continue  # E4M3FN NaN
        assert minifloat_decode(c, 4, 3, 7) == oracle.e4m3_decode(np.uint8(c))


def test_e2m1_decode_is_the_minifloat():
    got = [oracle.e2m1_decode(c) for c in range(16)]
    want = [minifloat_decode(c, 2, 1, 1) for c in range(16)]
    assert got == want
    assert max(got) == 6.0 and sorted(set(abs(x) for x in got)) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _nearest_even(y):
    """Brute force: nearest E2M1 magnitude, ties to the code with mantissa
    bit 0, saturation at 6."""
    mags = [(minifloat_decode(c, 2, 1, 1), c) for c in range(8)]
    a = min(abs(y), 6.0)
    best = min(mags, key=lambda vc: (abs(a - vc[0]), vc[1] & 1))
    code = best[1]
    return code | (8 if math.copysign(1.0, y) < 0 else 0)


def test_e2m1_encode_grid_midpoints_and_saturation():
    grid = np.concatenate([np.arange(-8, 8.0001, 1 / 64), [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 1e9, -1e9, -0.0]])
    grid = grid.astype(np.float32)
    got = oracle.e2m1_encode(grid)
    want = np.array([_nearest_even(float(y)) for y in grid], np.uint8)
    assert (got == want).all()


def test_mx_block_exp_is_minimal():
    rng = np.random.default_rng(0)
    vals = np.concatenate([rng.lognormal(0, 8, 2000), [6.0, 6.0 * 2 ** -10, 6.0 * 2 ** 20, 1e-38, 3.0]])
    for a in vals.astype(np.float32):
        e = oracle.mx_block_exp(float(a))
        assert float(a) <= 6.0 * 2.0 ** e
        assert e == -127 or float(a) > 6.0 * 2.0 ** (e - 1)
    assert oracle.mx_block_exp(0.0) == 0


def test_mxfp4_rows_and_cols_reconstruct_within_half_step():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((300, 64)) * np.exp(rng.standard_normal((300, 1)))).astype(np.float32)
    for codes, exps, y, axis in [(*oracle.mxfp4_rows(x), x, 1), (*oracle.mxfp4_cols(x), x.T, 0)]:
        if axis == 1:
            deq = oracle.e2m1_decode(codes[:300]) * np.exp2(np.repeat(exps[:300], 32, axis=1))
            yy = y
        else:
            deq = oracle.e2m1_decode(codes[:, :300]) * np.exp2(np.repeat(exps, 32, axis=1)[:, :300])
            yy = y
        scale = np.exp2(np.repeat(exps[:300] if axis == 1 else exps, 32, axis=1))
        if axis == 0:
            scale = scale[:, :300]
        # E2M1 spacing is 0.5 below 2, 1 below 4, 2 up to 6: half a step at most
        mag = np.abs(yy) / scale
        half = np.where(mag < 2, 0.25, np.where(mag < 4, 0.5, 1.0)) * scale
        assert np.all(np.abs(deq - yy) <= half * (1 + 1e-6))


def _codes_for(values):
    """E2M1 codes of exactly representable values (exponent 0)."""
    table = {minifloat_decode(c, 2, 1, 1): c for c in range(16) if c != 8}
    return np.array([table[float(v)] for v in np.ravel(values)], np.uint8).reshape(np.shape(values))


def _integer_case(S, D, seed, with_mu, max_at_end):
    """Scores s_k = K[k, 0] + K[k, 1] (Q = e_0 + e_1), integers within 3 of
    their 32-key block's maximum; block maxima vary, and the overall maximum
    0 sits where the traversal meets it late (the last block for the
    sequential order, block 0 -- reached last by the mid-window sweep -- for
    the other), so the running max rises."""
    rng = np.random.default_rng(seed)
    S_pad = (S + 127) // 128 * 128
    q = np.zeros((S_pad, D), np.uint8)
    q[:S, 0] = q[:S, 1] = _codes_for(1.0)  # s_k = K[k, 0] + K[k, 1]
    s = np.zeros(S, np.float64)
    hot = (S - 1) // 32 * 32 if max_at_end else 0  # the block holding the overall maximum
    for b0 in range(0, S, 32):
        b1 = min(b0 + 32, S)
        top = 0.0 if b0 == hot else rng.choice([-1.0, -2.0, -3.0, -4.0])
        s[b0:b1] = top - rng.integers(0, 4, b1 - b0)
        s[b0 + rng.integers(0, b1 - b0)] = top
    # each integer score in [-7, 0] as a sum of two E2M1 integers
    pairs = {a + b: (a, b) for a in (0, -1, -2, -3, -4, -6) for b in (0, -1, -2, -3, -4, -6)}
    k = np.zeros((S_pad, D), np.uint8)
    k[:S, 0] = _codes_for([pairs[v][0] for v in s])
    k[:S, 1] = _codes_for([pairs[v][1] for v in s])
    q_exps = np.zeros((S_pad, D // 32), np.int32)
    k_exps = np.zeros((S_pad, D // 32), np.int32)
    vals = rng.standard_normal((S, D)).astype(np.float32)
    vc, ve = oracle.mxfp4_cols(vals)
    vhat = (oracle.e2m1_decode(vc[:, :S]) * np.exp2(np.repeat(ve, 32, axis=1)[:, :S])).T
    mu = None
    if with_mu:
        mu = rng.standard_normal(((S + 127) // 128, D)).astype(np.float32)
        vhat = vhat + mu[np.arange(S) // 128].astype(np.float64)
    return q, q_exps, k, k_exps, vc, ve, mu, s, vhat


@pytest.mark.parametrize("S,D,with_mu,seq", [(700, 64, False, False), (700, 64, True, False), (384, 128, True, True),
                                             (129, 64, False, False)])
def test_attn4_equals_exact_softmax_on_representable_probabilities(S, D, with_mu, seq):
    q, qe, k, ke, vc, ve, mu, s, vhat = _integer_case(S, D, seed=S + D, with_mu=with_mu, max_at_end=seq)
    rows = np.arange(0, S, 7)
    of, _, st = oracle.attn4_emulate_rows(q, qe, k, ke, vc, ve, mu, S, rows, 2, oracle.SEQUENTIAL if seq else 0)
    w = np.exp2(s - s.max())
    want = (w[:, None] * vhat).sum(0) / w.sum()  # every query row sees the same scores
    assert np.abs(of - want[None, :]).max() <= 1e-6 * np.abs(want).max()
    assert (st[:, 0] > 0).any()  # the running max rose on some rows


def test_attn4_zero_queries_average_the_values():
    S, D = 300, 64
    rng = np.random.default_rng(5)
    q = np.zeros((384, D), np.uint8)
    qe = np.zeros((384, D // 32), np.int32)
    kx = rng.standard_normal((S, D)).astype(np.float32)
    k, ke = oracle.mxfp4_rows(kx)
    vals = rng.standard_normal((S, D)).astype(np.float32)
    vc, ve = oracle.mxfp4_cols(vals)
    vhat = (oracle.e2m1_decode(vc[:, :S]) * np.exp2(np.repeat(ve, 32, axis=1)[:, :S])).T
    of, _, _ = oracle.attn4_emulate_rows(q, qe, k, ke, vc, ve, None, S, np.array([0, 17, 299]))
    assert np.abs(of - vhat.mean(0)[None, :]).max() <= 1e-6 * np.abs(vhat).max()


def test_pipeline4_tracks_exact_attention():
    # the whole 4-bit pipeline on N(0,1) inputs composes and stays in the
    # expected range: E2M1 keeps one mantissa bit, so scores and
    # probabilities are coarse (measured: 0.27 relative L2 to exact
    # attention here, against 0.056 for the 8-bit path on the same rows)
    import vcsynth
    q, k, v = vcsynth.random_qkv(1, 512, 1, 64, seed=3)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    sm = 1 / math.sqrt(64)
    ref = exact.attention_rows(exact.to_f64(qb[0, :, 0]), exact.to_f64(kb[0, :, 0]), exact.to_f64(vb[0, :, 0]), sm)
    for vs in (False, True):
        res = oracle.pipeline4_head(qb, kb, vb, 0, 0, vsmooth=vs, nclust=8, iters=3, seed=1, sm_scale=sm)
        err = np.linalg.norm(res["out_f32"] - ref) / np.linalg.norm(ref)
        assert 0.1 < err < 0.35, (vs, err)


def _scores_of(res, row):
    """The row's log2 scores from the emulation's own codes, recomputed in
    float64 (products of E2M1 values and powers of two are exact)."""
    qd = oracle.e2m1_decode(res["q_codes"][row]) * np.exp2(np.repeat(res["q_exps"][row], 32))
    kd = oracle.e2m1_decode(res["k_codes"]) * np.exp2(np.repeat(res["k_exps"], 32, axis=1))
    return (kd @ qd).astype(np.float32)


@pytest.mark.parametrize("vs", [False, True])
def test_attn4_running_max_is_the_integer_ceiling(vs):
    # the running max is an integer: the ceiling of the row's largest score
    import vcsynth
    S, D = 700, 64
    q, k, v = vcsynth.random_qkv(1, S, 1, D, seed=11)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    rows = np.array([0, 1, 130, 311, 699])
    res = oracle.pipeline4_head(qb, kb, vb, 0, 0, vsmooth=vs, nclust=8, iters=2, seed=2, rows=rows)
    for j, r in enumerate(rows):
        s = _scores_of(res, r)[:S]
        assert res["stats"][j, 1] == math.ceil(float(s.max()))
        assert res["stats"][j, 1] == int(res["stats"][j, 1])


@pytest.mark.parametrize("vs,flags,rising", [(False, 0, False), (True, 0, False), (True, oracle.SEQUENTIAL, False),
                                             (False, oracle.SEQUENTIAL, False), (False, oracle.SEQUENTIAL, True),
                                             (True, 0, True)])
def test_attn4_deferred_rises_change_no_output(vs, flags, rising):
    # with an integer running max, a rise left unapplied (within the headroom
    # of 8) moves every P block's exponent by an integer and no code: the
    # output is the same, bit for bit, with far fewer rescales.  A max kept
    # fractional (the true max) would fail this.
    import vcsynth
    S, D = 1000, 64
    q, k, v = vcsynth.random_qkv(1, S, 1, D, seed=12)
    if rising:
        k = vcsynth.keys_rising_by_tile(k, 2)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    rows = np.arange(0, S, 3)
    kw = dict(vsmooth=vs, nclust=8, iters=2, seed=4, rows=rows, sm_scale=0.3)
    eager = oracle.pipeline4_head(qb, kb, vb, 0, 0, flags=flags, **kw)
    lazy = oracle.pipeline4_head(qb, kb, vb, 0, 0, flags=flags | oracle.DEFER4, **kw)
    assert np.array_equal(eager["out_f32"], lazy["out_f32"])
    if rising:  # rises past the headroom are applied, after the first tile too
        assert (lazy["stats"][:, 0] >= 1).mean() > 0.5
    else:
        assert eager["stats"][:, 0].sum() > 2 * lazy["stats"][:, 0].sum()
