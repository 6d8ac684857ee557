"""GPU parity at the workloads' full sizes, in the launch configuration
bench.py times (the V-Smooth path: vc_quantize(Q), vc_smooth_group(K, V,
64 clusters, 4 iterations, the workload's seed), vc_attn_fwd with the
mid-window order, W = 2; the plain path: vc_quantize(Q, K, V), vc_attn_fwd).

The whole path runs on the GPU over every head; the oracle then takes a few
heads and, for each, computes the grouping bit-exactly (labels, pi) and the
quantised-pipeline emulation of sampled query rows one by one.  Bar: labels
and pi equal; attention rows within relative L2 1e-2 of the emulation (the
tolerance of every attention parity test here).
"""
import numpy as np
import pytest
import torch

import oracle
import vcsynth

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


def _run(vc, name, heads, rows_per_head, seed_rows):
    w = vcsynth.WORKLOADS[name]
    print(f"case full size {name}: B={w.B} H={w.H} S={w.S} D={w.D} vsmooth={w.vsmooth}", flush=True)
    q, k, v = vcsynth.make_qkv(name, device="cuda")
    if w.vsmooth:
        qz = vc.vc_quantize(q, sm_scale=w.sm_scale)
        g = vc.vc_smooth_group(k, v, w.clusters, w.iters, w.seed)
        o = vc.vc_attn_fwd(qz["q8"], qz["q_scale"], g["k8"], g["k_scale"], g["r8"], g["r_scale"], g["mu_split"],
                           S=w.S, window=2)
        labels, perm = g["labels"].cpu().numpy(), g["perm"].cpu().numpy()
    else:
        qz = vc.vc_quantize(q, k, v, sm_scale=w.sm_scale)
        o = vc.vc_attn_fwd(qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], qz["v8"], qz["v_scale"], None,
                           S=w.S, window=2)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all().item()
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    og = o.float().cpu().numpy()
    del q, k, v, o
    rng = np.random.default_rng(seed_rows)
    for h in heads:
        rows = np.sort(rng.choice(w.S, rows_per_head, replace=False))
        rows[-1] = w.S - 1  # the last query row (ragged tile when S % 128 != 0)
        rows = np.unique(rows)
        res = oracle.pipeline_head(qb, kb, vb, 0, h, vsmooth=w.vsmooth, nclust=w.clusters, iters=w.iters,
                                   seed=w.seed, sm_scale=w.sm_scale, rows=rows, window=2)
        if w.vsmooth:
            assert (labels[0, h] == res["labels"]).all(), ("labels", h)
            assert (perm[0, h] == res["perm"]).all(), ("perm", h)
        emu = oracle.bf16_bits_to_f32(res["out_bf16"])
        err = _rel_l2(og[0, rows, h], emu)
        print(f"  head {h}: {rows.size} rows, rel-L2 {err:.2e}", flush=True)
        assert err <= REL_L2_TOL, (h, err)


def test_wan_full_size(vc):
    # the headline configuration
    _run(vc, "wan", heads=[0, 23, 39], rows_per_head=12, seed_rows=1)


def test_minimax_full_size(vc):
    _run(vc, "minimax", heads=[0, 47], rows_per_head=8, seed_rows=2)


def test_longcat_full_size(vc):
    _run(vc, "longcat", heads=[5, 31], rows_per_head=12, seed_rows=3)


def test_plain_full_size(vc):
    _run(vc, "plain", heads=[0, 11, 23], rows_per_head=24, seed_rows=4)


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
    rng = np.random.default_rng(5)
    for h in (0, 39):
        rows = np.unique(np.append(np.sort(rng.choice(w.S, 8, replace=False)), w.S - 1))
        res = oracle.pipeline4_head(qb, kb, vb, 0, h, vsmooth=True, nclust=w.clusters, iters=w.iters, seed=w.seed,
                                    sm_scale=w.sm_scale, rows=rows, window=2)
        assert (perm[0, h] == res["perm"]).all(), ("perm", h)
        emu = oracle.bf16_bits_to_f32(res["out_bf16"])
        err = _rel_l2(og[0, rows, h], emu)
        print(f"  head {h}: {rows.size} rows, rel-L2 {err:.2e}", flush=True)
        assert err <= REL_L2_TOL, (h, err)
