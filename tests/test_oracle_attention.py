"""Pins of the oracle's attention: the fp64 definition and the quantised
emulation (VC-Attention paper §3.1-3.3, Appendix D; Open-VC blog
"Scheduling around ExpCast").

The strongest pin is the integer-score special case: with Q/K scales of
exactly 1, integer dot products and a softmax scale that makes the folded
factor exactly 1, every ExpCast code decodes to exactly 2^(u+8), so the whole
emulation (scale folding, running max, rescales, row sums, mean restoration,
epilogue) must equal exact base-2 softmax attention on the dequantised values.
"""
import math

import numpy as np
import pytest

import oracle
import vcsynth
from oracle import exact


def _f64(x):
    return exact.to_f64(x)


def _rand(S, D, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((S, D)) * scale


# --------------------------------------------------------------------------- #
# exact attention
# --------------------------------------------------------------------------- #

def test_exact_two_formulations_agree():
    q, k, v = _rand(300, 64, 1, 2.0), _rand(300, 64, 2, 2.0), _rand(300, 64, 3)
    a = exact.attention_rows(q, k, v, 0.125)
    b = exact.attention_rows_online(q, k, v, 0.125, block=128)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


def test_exact_matches_extended_precision_loops():
    q, k, v = _rand(40, 8, 4, 2.0), _rand(40, 8, 5, 2.0), _rand(40, 8, 6)
    a = exact.attention_rows(q, k, v, 0.5)
    c = exact.attention_rows_longdouble(q, k, v, 0.5)
    assert np.abs(a - c).max() <= 1e-12


def test_exact_permutation_invariance():
    # VC §3.2 Eq. 3: permuting K and V jointly leaves the output unchanged
    q, k, v = _rand(257, 32, 7), _rand(257, 32, 8), _rand(257, 32, 9)
    pi = np.random.default_rng(10).permutation(257)
    a = exact.attention_rows(q, k, v, 0.3)
    b = exact.attention_rows(q, k[pi], v[pi], 0.3)
    assert np.abs(a - b).max() <= 1e-12 * np.abs(a).max()


def test_exact_special_cases():
    k, v = _rand(50, 16, 11), _rand(50, 16, 12)
    # Q = 0: uniform weights, output is the mean of the value rows
    out = exact.attention_rows(np.zeros((3, 16)), k, v, 1.0)
    assert np.allclose(out, v.mean(0)[None], atol=1e-14)
    # one key 60 logits above the rest: output is that key's value row
    q = np.zeros((1, 16))
    q[0, 0] = 1.0
    kk = np.zeros((50, 16))
    kk[17, 0] = 60.0
    out = exact.attention_rows(q, kk, v, 1.0)
    assert np.allclose(out[0], v[17], atol=1e-20 + 1e-24 * np.abs(v).max() + 1e-24) or \
        np.abs(out[0] - v[17]).max() < 1e-24 + 50 * math.exp(-60) * np.abs(v).max()
    # D = 1, S = 2: logistic
    q = np.array([[1.5]])
    kk = np.array([[2.0], [-1.0]])
    vv = np.array([[3.0], [-7.0]])
    s = 1.5 * 2.0 * 0.7 - 1.5 * -1.0 * 0.7
    p0 = 1 / (1 + math.exp(-s))
    assert abs(exact.attention_rows(q, kk, vv, 0.7)[0, 0] - (3 * p0 - 7 * (1 - p0))) < 1e-14


# --------------------------------------------------------------------------- #
# traversal order (Open-VC blog, mid-window key traversal)
# --------------------------------------------------------------------------- #

def test_tile_order_mid_window():
    # query tiles 2p and 2p + 1 share one order, started `window` blocks past
    # the pair's second diagonal block
    assert list(oracle.tile_order(0, 5, 2)) == [3, 2, 1, 0, 4]
    assert list(oracle.tile_order(1, 5, 2)) == [3, 2, 1, 0, 4]
    assert list(oracle.tile_order(1, 6, 2)) == [3, 2, 1, 0, 4, 5]
    assert list(oracle.tile_order(4, 5, 2)) == [4, 3, 2, 1, 0]
    assert list(oracle.tile_order(2, 5, 0)) == [3, 2, 1, 0, 4]
    assert list(oracle.tile_order(2, 6, 1)) == [4, 3, 2, 1, 0, 5]
    assert list(oracle.tile_order(3, 5, 2, sequential=True)) == [0, 1, 2, 3, 4]
    assert list(oracle.tile_order(0, 1, 2)) == [0]
    for qt in range(30):
        o = oracle.tile_order(qt, 30, 3)
        assert sorted(o) == list(range(30))  # every block exactly once
        assert o[0] == min(2 * (qt // 2) + 1 + 3, 29)
        # down from the start to block 0, then upwards
        k = list(o).index(0)
        assert list(o[:k + 1]) == list(range(o[0], -1, -1))
        assert list(o[k + 1:]) == list(range(o[0] + 1, 30))


# --------------------------------------------------------------------------- #
# integer-score special case
# --------------------------------------------------------------------------- #

def _unit_fold_scale():
    """A float32 softmax scale s with fl32(s * fl32(log2 e)) == 1 exactly."""
    log2e = np.float32(1.4426950408889634)
    s = np.float32(1 / 1.4426950408889634)
    for _ in range(64):
        p = np.float32(s * log2e)
        if p == 1.0:
            return float(s)
        s = np.nextafter(s, np.float32(np.inf) if p < 1 else np.float32(-np.inf))
    raise AssertionError("no unit scale found")


def _integer_qk(S, D, seed):
    """bf16 Q, K with integer entries in {-1,0,1} on channels 2.., Q[:,0] = 448
    and K[:,1] = 448 so every 128-block amax is 448 (scale exactly 1), while
    Q[:,1] = K[:,0] = 0 keeps those channels out of the dot products; at most
    seven non-zero products keep every log2 score within 14 of the max."""
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


def _bits(x):
    return oracle.f32_to_bf16_bits(x.astype(np.float32))


@pytest.mark.parametrize("S,D,order", [(300, 64, "mid"), (384, 128, "mid"), (300, 64, "seq")])
def test_emulation_integer_scores_plain(S, D, order):
    q, k = _integer_qk(S, D, seed=S + D)
    v = np.random.default_rng(5).standard_normal((S, D)).astype(np.float32) * 3
    qb, kb, vb = _bits(q), _bits(k), _bits(v)
    qc, qs = oracle.quantize_qk(qb[None, :, None, :])
    kc, ks = oracle.quantize_qk(kb[None, :, None, :])
    vc, vs = oracle.quantize_v(vb[None, :, None, :])
    assert (qs == 1).all() and (ks == 1).all()
    rows = np.arange(S)
    # c1 = 1: the log2-domain score is the integer dot product itself
    of, _, st = oracle.attn_emulate_rows(qc[0, 0], qs[0, 0], kc[0, 0], ks[0, 0], vc[0, 0], vs[0, 0], None,
                                         S, 1.0, rows, window=2,
                                         flags=oracle.SEQUENTIAL if order == "seq" else 0)
    # exact attention with base-2 weights on the dequantised values
    v_deq = oracle.e4m3_decode(vc[0, 0, :, :S]).T * vs[0, 0][None, :]
    qi = oracle.e4m3_decode(qc[0, 0, :S]) * 1.0
    ki = oracle.e4m3_decode(kc[0, 0, :S]) * 1.0
    ref = exact.attention_rows(qi, ki, v_deq, math.log(2.0))
    assert np.abs(of - ref).max() <= 2e-6 * np.abs(ref).max()
    assert st[:, 0].sum() > 0  # the rescale path ran


def test_emulation_integer_scores_vsmooth():
    S, D = 500, 64
    q, k = _integer_qk(S, D, seed=99)
    qt, kt, vt = vcsynth.make_qkv("tiny")
    vb = vcsynth.bf16_bits(vt)[0, :S, 0, :D].copy()
    qb, kb = _bits(q), _bits(k)
    sm = _unit_fold_scale()
    assert oracle.q_prefactor(sm) == 8.0
    res = oracle.pipeline_head(qb[None, :, None], kb[None, :, None], vb[None, :, None], 0, 0, vsmooth=True,
                               nclust=8, iters=3, seed=1000, sm_scale=sm)
    # Q carries G = 8: amax 8 * 448 = 448 * 2^3, so the same codes under scale 8
    assert (res["q_scale"] == 8).all() and (res["k_scale"] == 1).all()
    perm = res["perm"]
    # dequantised permuted values: s_R * (R_hat + mu_scaled of the row's block)
    blk = np.arange(S) // 128
    v_eff = (oracle.e4m3_decode(res["r_codes"][:, :S]).T + res["mu_scaled"][blk].astype(np.float64)) \
        * res["r_scale"][None, :].astype(np.float64)
    qi = oracle.e4m3_decode(res["q_codes"][:S])
    ki = oracle.e4m3_decode(res["k_codes"][:S])  # permuted keys
    ref = exact.attention_rows(qi, ki, v_eff, math.log(2.0))
    assert np.abs(res["out_f32"] - ref).max() <= 2e-6 * np.abs(ref).max()
    # and the permuted-key attention equals attention on the unpermuted keys
    inv = np.argsort(perm)
    ref2 = exact.attention_rows(qi, ki[inv], v_eff[inv], math.log(2.0))
    assert np.abs(ref - ref2).max() <= 1e-12 * np.abs(ref).max()
    # dropping the mean term would be visible: the means carry real mass
    assert np.abs(res["mu_scaled"]).max() > 0.1


# --------------------------------------------------------------------------- #
# invariants on random data
# --------------------------------------------------------------------------- #

def test_emulation_convex_combination():
    # consistent denominator (Open-VC blog): each output is a weighted average
    # of the reconstructed value rows
    q, k, v = vcsynth.random_qkv(1, 700, 1, 64, seed=21, v_kind="t3")
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    res = oracle.pipeline_head(qb, kb, vb, 0, 0, vsmooth=False, sm_scale=0.3)
    v_deq = oracle.e4m3_decode(res["v_codes"][:, :700]).T * res["v_scale"][None, :]
    lo, hi = v_deq.min(0), v_deq.max(0)
    o = res["out_f32"]
    tol = 1e-6 * np.abs(v_deq).max()
    assert (o >= lo - tol).all() and (o <= hi + tol).all()


def test_emulation_within_eq15_envelope():
    # Eq. 15: per row ||o_hat - o|| <= (0.0364 + tau) diam2(V'), with o the
    # exact softmax of the dequantised scores against the dequantised values;
    # a 1e-4 slack covers the fp32 folding of the scales into the FMA
    S, D, sm = 1000, 128, 4 / math.sqrt(128)
    q, k, v = vcsynth.random_qkv(1, S, 1, D, seed=31)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    res = oracle.pipeline_head(qb, kb, vb, 0, 0, vsmooth=False, sm_scale=sm)
    blk = np.arange(S) // 128
    # Q's codes carry G = 8 fl(sm log2 e): divide it back out
    qd = oracle.e4m3_decode(res["q_codes"][:S]) * res["q_scale"][blk][:, None] / oracle.q_prefactor(sm)
    kd = oracle.e4m3_decode(res["k_codes"][:S]) * res["k_scale"][blk][:, None]
    vd = oracle.e4m3_decode(res["v_codes"][:, :S]).T * res["v_scale"][None, :]
    ref = exact.attention_rows(qd, kd, vd, sm)
    diam = exact.diam2(vd)
    u = (qd @ kd.T) * sm * exact.LOG2E
    for i in range(S):
        _, tau = exact.row_tv_check(u[i])
        assert np.linalg.norm(res["out_f32"][i] - ref[i]) <= (0.0364 + tau + 1e-4) * diam + 1e-5


def test_expcast_rows_within_prop31():
    # Prop. 3.1 / Eq. 14 on rows of real-shaped data: codes from fp64 u
    q, k, v = vcsynth.random_qkv(1, 2048, 1, 128, seed=41)
    qb, kb = vcsynth.bf16_bits(q)[0, :, 0], vcsynth.bf16_bits(k)[0, :, 0]
    for scale in (1 / math.sqrt(128), 4 / math.sqrt(128)):
        s = (_f64(qb[:64]) @ _f64(kb).T) * scale * exact.LOG2E
        for row in s:
            tv, tau = exact.row_tv_check(row)
            assert tv < 0.0364 + tau


def test_exact_exp_diagnostic_is_closer_on_average():
    # the fp32-exp-then-cast diagnostic path runs and stays close to ExpCast
    q, k, v = vcsynth.random_qkv(1, 512, 1, 64, seed=51)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    a = oracle.pipeline_head(qb, kb, vb, 0, 0, vsmooth=False, sm_scale=0.5)
    b = oracle.pipeline_head(qb, kb, vb, 0, 0, vsmooth=False, sm_scale=0.5, flags=oracle.EXACT_EXP)
    ref = exact.attention_rows(_f64(qb[0, :, 0]), _f64(kb[0, :, 0]), _f64(vb[0, :, 0]), 0.5)
    ea = np.linalg.norm(a["out_f32"] - ref) / np.linalg.norm(ref)
    eb = np.linalg.norm(b["out_f32"] - ref) / np.linalg.norm(ref)
    assert ea < 0.1 and eb < 0.1


# --------------------------------------------------------------------------- #
# per-score weights read back through a one-hot V
# --------------------------------------------------------------------------- #

def _log2_scores(res, S):
    """Log2-domain scores the emulation sees: s_Q s_K (Qhat . Khat) / 8 (Q's
    codes carry G = 8 fl(sm log2 e)), in fp64 (exact products and sums)."""
    blk = np.arange(S) // 128
    qd = oracle.e4m3_decode(res["q_codes"][:S]) * res["q_scale"][blk][:, None].astype(np.float64)
    kd = oracle.e4m3_decode(res["k_codes"][:S]) * res["k_scale"][blk][:, None].astype(np.float64)
    return (qd @ kd.T) / 8.0


@pytest.mark.parametrize("S,window,seq,exact_exp", [(300, 2, False, False), (300, 0, False, False),
                                                    (300, 2, True, False), (700, 2, False, False),
                                                    (300, 2, False, True), (700, 1, True, True)])
def test_emulation_weights_per_score(S, window, seq, exact_exp):
    # V = one-hot on key tile j (key 128 j + d carries 1 in channel d): output
    # channel d of every row is that key's final weight over the row sum,
    # w_k 448 s_V / l.  Every weight of every row is compared with the
    # definition applied score by score (tests/expcast_ref.py): the ExpCast
    # code (or, with EXACT_EXP, torch's E4M3 cast of 2^(u+8)) at the running
    # max after the key's tile, rescaled by the later increases
    import expcast_ref as ER
    D, sm = 128, 3 / math.sqrt(128)
    nblk = (S + 127) // 128
    q, k, _ = vcsynth.random_qkv(1, S, 1, D, seed=S + window)
    qb, kb = vcsynth.bf16_bits(q), vcsynth.bf16_bits(k)
    flags = (oracle.SEQUENTIAL if seq else 0) | (oracle.EXACT_EXP if exact_exp else 0)
    n_rescale = 0
    for j in range(nblk):
        v = np.zeros((1, S, 1, D), np.float32)
        nk = min(128, S - 128 * j)
        v[0, 128 * j + np.arange(nk), 0, np.arange(nk)] = 1.0
        res = oracle.pipeline_head(qb, kb, _bits(v), 0, 0, vsmooth=False, sm_scale=sm, window=window, flags=flags)
        assert (res["v_codes"][np.arange(nk), 128 * j + np.arange(nk)] == 0x7E).all()  # 448
        u = _log2_scores(res, S)
        unit = 448.0 * float(res["v_scale"][0])
        n_flip = 0
        for i in range(S):
            w, l, dw = ER.row_weights(u[i], S, ER.tile_visits(i // 128, nblk, window, seq), exact_exp=exact_exp,
                                      eps=1e-4)
            kk = 128 * j + np.arange(nk)
            want = w[kk] / l * unit
            tol = 2e-6 * want + (dw[kk] + w[kk] * dw.sum() / l) / l * unit
            got = res["out_f32"][i, :nk].astype(np.float64)
            assert np.all(np.abs(got - want) <= tol + 1e-30), (j, i)
            assert np.all(got[nk:] == 0) if nk < D else True
            n_flip += int((dw > 0).sum())
        assert n_flip <= 1e-3 * S * S, n_flip  # keys within 1e-4 of a boundary are rare: the check is tight
        n_rescale += int(res["stats"][:, 0].sum())
    assert n_rescale > 0  # rows whose max rose after their first tile
