"""GPU parity at the workloads' full sizes, in the launch configuration
bench.py times (the V-Smooth path: vc_quantize(Q), vc_smooth_group(K, V,
64 clusters, 4 iterations, the workload's seed), vc_attn_fwd with the
mid-window order, W = 2; the plain path: vc_quantize(Q, K, V), vc_attn_fwd).

The whole path runs on the GPU over every head; the oracle then takes some
heads and, for each, computes the grouping bit-exactly (labels, pi) and the
quantised-pipeline emulation of sampled query rows one by one.  Bar: labels
and pi equal; attention rows within relative L2 1e-2 of the emulation per
head, and every element the bf16 rounding of a value within the bound of
tests/expcast_ref.py.  At the headline shape (H = 40, S = 75600, 591 key
tiles, the last one 80 keys) 8 heads x 256 rows are checked, the rows drawn
from every kind of query tile: both halves of a workgroup's pair, both
16-query sub-tiles of a wave, the last pair (tile 590, whose partner half is
idle) with the ragged tile's rows, plus the fp64 envelope of [VC] App. D
Eq. 15 on every checked row.
"""
import math

import numpy as np
import pytest
import torch

import expcast_ref as ER
import oracle
import vcsynth
from oracle import exact

pytestmark = pytest.mark.gpu

REL_L2_TOL = 1e-2


@pytest.fixture(scope="module")
def vc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_attention_amd as m
    m.lib()
    return m


def _rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _gpu_path(vc, name):
    w = vcsynth.WORKLOADS[name]
    print(f"case full size {name}: B={w.B} H={w.H} S={w.S} D={w.D} vsmooth={w.vsmooth}", flush=True)
    q, k, v = vcsynth.make_qkv(name, device="cuda")
    out = {}
    if w.vsmooth:
        qz = vc.vc_quantize(q, sm_scale=w.sm_scale)
        g = vc.vc_smooth_group(k, v, w.clusters, w.iters, w.seed)
        o = vc.vc_attn_fwd(qz["q8"], qz["q_scale"], g["k8"], g["k_scale"], g["r8"], g["r_scale"], g["mu_split"],
                           S=w.S, window=2)
        out["labels"], out["perm"] = g["labels"].cpu().numpy(), g["perm"].cpu().numpy()
    else:
        qz = vc.vc_quantize(q, k, v, sm_scale=w.sm_scale)
        o = vc.vc_attn_fwd(qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], qz["v8"], qz["v_scale"], None,
                           S=w.S, window=2)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all().item()
    out["qb"], out["kb"], out["vb"] = (vcsynth.bf16_bits(x) for x in (q, k, v))
    out["og"] = o.float().cpu().numpy()
    out["w"] = w
    del q, k, v, o
    torch.cuda.empty_cache()
    return out


def _check_head(run, h, rows, envelope=False):
    w = run["w"]
    res = oracle.pipeline_head(run["qb"], run["kb"], run["vb"], 0, h, vsmooth=w.vsmooth, nclust=w.clusters,
                               iters=w.iters, seed=w.seed, sm_scale=w.sm_scale, rows=rows, window=2)
    if w.vsmooth:
        assert (run["labels"][0, h] == res["labels"]).all(), ("labels", h)
        assert (run["perm"][0, h] == res["perm"]).all(), ("perm", h)
    og = run["og"][0, rows, h]
    err = _rel_l2(og, oracle.bf16_bits_to_f32(res["out_bf16"]))
    st = ER.check_rows(og, res, w.S, rows, 2, vsmooth=w.vsmooth)
    print(f"  head {h}: {rows.size} rows, rel-L2 {err:.2e}, row max {st['row_rel_l2_max']:.2e}, "
          f"bit-identical {st['bit_identical']:.4f}, boundary keys {st['n_flip']}/{st['n_scores']}", flush=True)
    assert err <= REL_L2_TOL, (h, err)
    if envelope:
        _envelope(run, h, rows, res, og)


def _envelope(run, h, rows, res, og):
    """[VC] App. D Eq. 15 plus the Q/K and V quantisation terms the
    proposition leaves out, per row, against the fp64 softmax of the inputs:
    ||o - o_exact|| <= (0.0364 + tau + TV(p_exact, p_qk) + 1e-4) diam(Vhat)
                       + max ||Vhat - V|| + 1e-2 max ||V||."""
    w = run["w"]
    S, sm = w.S, w.sm_scale
    qf = exact.to_f64(run["qb"][0, :, h])
    kf = exact.to_f64(run["kb"][0, :, h])
    vf = exact.to_f64(run["vb"][0, :, h])
    ref = exact.attention_rows(qf, kf, vf, sm, rows)
    blk = np.arange(S) // 128
    qd = oracle.e4m3_decode(res["q_codes"][:S]) * res["q_scale"][blk][:, None] / oracle.q_prefactor(sm)
    if w.vsmooth:
        kd_p = oracle.e4m3_decode(res["k_codes"][:S]) * res["k_scale"][blk][:, None]
        vd_p = (oracle.e4m3_decode(res["r_codes"][:, :S]).T + res["mu_scaled"][blk]) * res["r_scale"][None, :]
        inv = np.argsort(res["perm"])
        kd, vd = kd_p[inv], vd_p[inv]
    else:
        kd = oracle.e4m3_decode(res["k_codes"][:S]) * res["k_scale"][blk][:, None]
        vd = oracle.e4m3_decode(res["v_codes"][:, :S]).T * res["v_scale"][None, :]
    vmax = np.linalg.norm(vf, axis=1).max()
    diam_ub = 2 * np.linalg.norm(vd - vd.mean(0), axis=1).max()  # >= diam2 of the dequantised rows
    dv = np.linalg.norm(vd - vf, axis=1).max()
    s_exact = (qf[rows] @ kf.T) * sm
    s_deq = (qd[rows] @ kd.T) * sm
    worst = 0.0
    for ri in range(len(rows)):
        p_exact = np.exp(s_exact[ri] - s_exact[ri].max())
        p_exact /= p_exact.sum()
        p_qk = np.exp(s_deq[ri] - s_deq[ri].max())
        p_qk /= p_qk.sum()
        tv_qk = 0.5 * np.abs(p_exact - p_qk).sum()
        _, tau = exact.row_tv_check(s_deq[ri] * exact.LOG2E)
        bound = (0.0364 + tau + tv_qk + 1e-4) * diam_ub + dv + 1e-2 * vmax
        e = np.linalg.norm(og[ri] - ref[ri])
        assert e <= bound, (rows[ri], e, bound)
        worst = max(worst, e / bound)
    print(f"  head {h}: Eq. 15 envelope holds on {len(rows)} rows (worst error / bound {worst:.3f})", flush=True)


def _rows(S, n, seed, extra=()):
    """n query rows: fixed rows of the listed tiles (both 16-query sub-tiles
    of two waves, the tile's last row) plus random ones; always S - 1."""
    rng = np.random.default_rng(seed)
    fixed = [128 * t + off for t in extra for off in (0, 3, 17, 30, 45, 62, 64 + 16 + 9, 127)]
    fixed = [r for r in fixed if r < S] + [S - 1]
    rand = rng.choice(S, max(0, n - len(fixed)), replace=False)
    return np.unique(np.concatenate([np.array(fixed, np.int64), rand]))


@pytest.fixture(scope="module")
def wan_run(vc):
    return _gpu_path(vc, "wan")


# tiles 0 / 1: both halves of pair 0; 300 / 301: both halves of a middle
# pair; 588 / 589: the last full pair; 590: the last pair's live half A
# (half B idle), which also holds the ragged rows 75520 .. 75599
WAN_TILES = (0, 1, 300, 301, 588, 589, 590)


@pytest.mark.parametrize("heads", [(0, 1), (13, 20), (27, 33), (38, 39)])
def test_wan_full_size(wan_run, heads):
    # the headline configuration
    for h in heads:
        _check_head(wan_run, h, _rows(wan_run["w"].S, 256, 100 + h, WAN_TILES), envelope=True)


def test_minimax_full_size(vc):
    run = _gpu_path(vc, "minimax")
    for h in (0, 47):
        _check_head(run, h, _rows(run["w"].S, 64, 200 + h, (0, 1, 660, 661)))


def test_longcat_full_size(vc):
    run = _gpu_path(vc, "longcat")
    for h in (5, 31):
        _check_head(run, h, _rows(run["w"].S, 64, 300 + h, (0, 1, 254, 255)))


def test_plain_full_size(vc):
    run = _gpu_path(vc, "plain")
    for h in (0, 11, 23):
        _check_head(run, h, _rows(run["w"].S, 96, 400 + h, (0, 1, 126, 127)), envelope=True)


def test_wan_full_size_mxfp4(vc):
    # the 4-bit path at the headline shape: the same grouping, vc_quantize4,
    # vc_attn_fwd4; sampled rows of two heads against the oracle's 4-bit
    # emulation
    w = vcsynth.WORKLOADS["wan"]
    print(f"case full size wan, 4-bit: B={w.B} H={w.H} S={w.S} D={w.D}", flush=True)
    q, k, v = vcsynth.make_qkv("wan", device="cuda")
    g = vc.vc_smooth_group(k, v, w.clusters, w.iters, w.seed)
    z = vc.vc_quantize4(q, k, v, sm_scale=w.sm_scale, perm=g["perm"], mu_bf16=g["mu_bf16"])
    o = vc.vc_attn_fwd4(z["q4"], z["q4_scale"], z["k4"], z["k4_scale"], z["v4"], z["v4_scale"], g["mu_bf16"], S=w.S)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all().item()
    perm = g["perm"].cpu().numpy()
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    og = o.float().cpu().numpy()
    del q, k, v, o, z
    for h in (0, 39):
        rows = _rows(w.S, 24, 500 + h, (0, 1, 590))
        res = oracle.pipeline4_head(qb, kb, vb, 0, h, vsmooth=True, nclust=w.clusters, iters=w.iters, seed=w.seed,
                                    sm_scale=w.sm_scale, rows=rows, window=2)
        assert (perm[0, h] == res["perm"]).all(), ("perm", h)
        emu = oracle.bf16_bits_to_f32(res["out_bf16"])
        err = _rel_l2(og[0, rows, h], emu)
        row = np.linalg.norm(og[0, rows, h] - emu, axis=1) / np.linalg.norm(emu, axis=1)
        print(f"  head {h}: {rows.size} rows, rel-L2 {err:.2e}, row max {row.max():.2e}", flush=True)
        assert err <= REL_L2_TOL, (h, err)
        assert row.max() <= REL_L2_TOL, (h, row.max())
