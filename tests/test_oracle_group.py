"""Pins of the oracle's V-Smooth grouping (VC-Attention paper §3.2: online
k-means labels, pi = argsort(z), block demeaning Eq. 4, energy identity
Eq. 5, Appendix B storage of the scaled means)."""
import numpy as np

import oracle
import vcsynth
from oracle import exact


def test_splitmix64_published_vector(golden):
    g = golden("splitmix64.json")
    got = oracle.splitmix64_stream(g["seed"], len(g["outputs_hex"]))
    assert got == [int(x, 16) for x in g["outputs_hex"]]


def test_forgy_indices_distinct_and_deterministic():
    for S, k in [(1024, 8), (75600, 64), (300, 256), (5, 5)]:
        a = oracle.forgy_indices(1003, 0, 7, 40, S, k)
        b = oracle.forgy_indices(1003, 0, 7, 40, S, k)
        assert (a == b).all()
        assert len(set(a.tolist())) == k and a.min() >= 0 and a.max() < S
    # different heads draw different streams
    assert not (oracle.forgy_indices(1, 0, 0, 4, 1000, 16) == oracle.forgy_indices(1, 0, 1, 4, 1000, 16)).all()
    # k = S draws a full permutation
    assert sorted(oracle.forgy_indices(9, 0, 0, 1, 37, 37).tolist()) == list(range(37))


def _v_head(name="tiny", h=0, S=None, H=None):
    q, k, v = vcsynth.make_qkv(name, H=H)
    vb = vcsynth.bf16_bits(v)
    vh = vb[0, :, h, :]
    return np.ascontiguousarray(vh[:S] if S else vh)


def _inertia(vf, labels, cent):
    return float(((vf - cent[labels].astype(np.float64)) ** 2).sum())


def test_kmeans_labels_are_argmin_and_inertia_decreases():
    vh = _v_head()
    vf = exact.to_f64(vh)
    prev = None
    for iters in range(1, 5):
        labels, cent = oracle.kmeans_head(vh, 8, iters, 1000, 0, 0, 2)
        # re-run the last assignment against the centroids that produced it
        _, cent_prev = oracle.kmeans_head(vh, 8, iters - 1, 1000, 0, 0, 2) if iters > 1 else (None, None)
        if cent_prev is None:
            idx = oracle.forgy_indices(1000, 0, 0, 2, vh.shape[0], 8)
            cent_prev = exact.to_f64(vh[idx])
        d = ((vf[:, None, :] - cent_prev[None, :, :].astype(np.float64)) ** 2).sum(-1)
        best = d.min(1)
        mine = d[np.arange(len(labels)), labels]
        assert (mine <= best + 1e-5 * np.maximum(best, 1.0)).all()
        inert = _inertia(vf, labels, cent)
        if prev is not None:
            assert inert <= prev * (1 + 1e-9)
        prev = inert


def test_kmeans_planted_recovery():
    # well separated clusters (sigma_centre 3 >> sigma_within 0.5, D = 128)
    rng = np.random.default_rng(0)
    K, n, D = 6, 150, 128
    centres = rng.standard_normal((K, D)) * 3
    truth = np.repeat(np.arange(K), n)
    rng.shuffle(truth)
    x = centres[truth] + 0.5 * rng.standard_normal((K * n, D))
    vh = oracle.f32_to_bf16_bits(x.astype(np.float32))
    # find a seed whose initial indices hit every planted cluster
    for seed in range(100):
        idx = oracle.forgy_indices(seed, 0, 0, 1, K * n, K)
        if len(set(truth[idx].tolist())) == K:
            break
    labels, _ = oracle.kmeans_head(vh, K, 4, seed, 0, 0, 1)
    for c in range(K):  # each found cluster is pure
        assert len(set(truth[labels == c].tolist())) == 1


def test_kmeans_empty_cluster_keeps_centroid():
    # two identical tokens chosen as initial centroids: the higher index never
    # wins a tie, stays empty and keeps its centroid
    x = np.zeros((4, 64), np.float32)
    x[2:] = 5.0
    vh = oracle.f32_to_bf16_bits(x)
    init = np.stack([x[0], x[0], x[2]]).astype(np.float32)
    labels, cent = oracle.kmeans_head(vh, 3, 2, 0, 0, 0, 1, init=init)
    assert list(labels) == [0, 0, 2, 2]
    assert (cent[1] == init[1]).all()


def test_argsort_is_stable_permutation():
    rng = np.random.default_rng(1)
    labels = rng.integers(0, 13, 5000).astype(np.int32)
    perm = oracle.argsort_labels(labels, 13)
    assert sorted(perm.tolist()) == list(range(5000))
    z = labels[perm]
    assert (np.diff(z) >= 0).all()
    for c in range(13):  # token order kept inside a label
        assert (np.diff(perm[z == c]) > 0).all()
    assert (perm == np.argsort(labels, kind="stable")).all()


def test_block_means_and_residuals():
    S, D = 700, 64
    vh = _v_head(S=S)
    kh = np.ascontiguousarray(vcsynth.bf16_bits(vcsynth.make_qkv("tiny")[1])[0, :S, 0])
    labels, _ = oracle.kmeans_head(vh, 8, 3, 5, 0, 0, 1)
    perm = oracle.argsort_labels(labels, 8)
    g = oracle.smooth_apply_head(kh, vh, perm)
    vp = exact.to_f64(vh[perm])
    nblk = (S + 127) // 128
    mu_hat = exact.to_f64(g["mu_bf16"])
    for j in range(nblk):
        mu = vp[j * 128:(j + 1) * 128].mean(0)  # tail block: its valid rows
        assert (np.abs(mu_hat[j] - mu) <= 2.0 ** -8 * np.abs(mu) + 1e-30).all()
    # residual codes reconstruct V' up to E4M3 rounding (half a step, 2^-4 rel)
    blk = np.arange(S) // 128
    R = vp - mu_hat[blk]
    Rq = oracle.e4m3_decode(g["r_codes"][:, :S]).T * g["r_scale"][None, :]
    assert (np.abs(Rq - R) <= 2.0 ** -4 * np.abs(R) + g["r_scale"][None, :] * 2.0 ** -9 * 1.01).all()
    assert (g["r_codes"][:, S:] == 0).all()
    # the per-channel scale is set by the largest residual of the channel
    assert np.allclose(g["r_scale"], np.abs(R).max(0) / 448, rtol=1e-6)
    # scaled means: mu / s_R
    assert np.allclose(g["mu_scaled"], mu_hat / g["r_scale"][None, :], rtol=1e-6)
    # K' is K[pi] quantised per block
    kc, ks = oracle.quantize_qk(np.ascontiguousarray(kh[perm])[None, :, None, :])
    assert (kc[0, 0] == g["k_codes"]).all() and (ks[0, 0] == g["k_scale"]).all()


def test_block_mean_is_order_independent():
    S, D = 256, 64
    vh = _v_head(S=S)
    kh = vh.copy()
    perm = np.arange(S, dtype=np.int32)
    a = oracle.smooth_apply_head(kh, vh, perm)
    shuf = np.concatenate([np.random.default_rng(2).permutation(128), 128 + np.arange(128)[::-1]])
    b = oracle.smooth_apply_head(kh, vh, shuf.astype(np.int32))
    assert (a["mu_bf16"] == b["mu_bf16"]).all()


def test_energy_identity_eq5():
    rng = np.random.default_rng(3)
    Vj = rng.standard_normal((128, 64)) * 2 + 1.5
    mu = Vj.mean(0)
    R = Vj - mu
    for _ in range(5):
        c = rng.standard_normal(64)
        lhs = ((Vj - c) ** 2).sum()
        rhs = (R ** 2).sum() + 128 * ((c - mu) ** 2).sum()
        assert abs(lhs - rhs) <= 1e-12 * lhs
    assert abs((R ** 2).sum() - ((Vj ** 2).sum() - 128 * (mu ** 2).sum())) <= 1e-10 * (Vj ** 2).sum()


def test_sorting_raises_the_energy_share_of_the_means():
    # VC §3.2: the mean removes more block energy after sorting by cluster
    vh = _v_head("longcat", h=0, H=1)
    S = vh.shape[0]
    vf = exact.to_f64(vh)
    labels, _ = oracle.kmeans_head(vh, 64, 4, 1002, 0, 0, 1)
    perm = oracle.argsort_labels(labels, 64)

    def share(x):
        n = (x.shape[0] // 128) * 128
        b = x[:n].reshape(-1, 128, x.shape[1])
        return float((128 * (b.mean(1) ** 2).sum(-1)).sum() / (b ** 2).sum())
    seq, srt = share(vf), share(vf[perm])
    assert srt > seq + 0.1, (seq, srt)


def test_kmeans_warm_start_continues_a_cold_run():
    # warm start (VC-Attention paper §3.2, "Unbalanced clusters cost little":
    # each step starts from the previous step's centroids).  Lloyd iterations
    # compose: a cold run of a + b iterations equals a cold run of a
    # iterations followed by b iterations started from its centroids --
    # labels and centroids bit for bit.
    for name, S, k, a, b in [("tiny", None, 8, 1, 2), ("longcat", 4096, 64, 2, 2)]:
        vh = _v_head(name, S=S, H=1)
        lab_ab, cent_ab = oracle.kmeans_head(vh, k, a + b, 1000, 0, 0, 1)
        _, cent_a = oracle.kmeans_head(vh, k, a, 1000, 0, 0, 1)
        lab_w, cent_w = oracle.kmeans_head(vh, k, b, 999, 0, 0, 1, init=cent_a)  # seed unused when warm
        assert (lab_w == lab_ab).all()
        assert (cent_w == cent_ab).all()
        # and the warm start does not reuse the Forgy draw: from other centroids the result differs
        lab_o, _ = oracle.kmeans_head(vh, k, b, 1000, 0, 0, 1, init=np.roll(cent_a, 1, axis=1))
        assert not (lab_o == lab_ab).all()
