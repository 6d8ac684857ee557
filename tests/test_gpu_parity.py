"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: ExpCast codes on identical fp32 inputs, vc_quantize codes and
scales, k-means labels / centroids / permutation, block means, scaled means
(as the stored bf16 hi/lo pairs), residual codes and K' codes.  Attention
output: relative L2 <= 1e-2 against the quantised-pipeline emulation per
head, and every element the bf16 rounding of a value within the bound of
tests/expcast_ref.py (elementwise_tol: the fp32 order of the matrix cores'
sums and exp2f rescales, plus one code step only for keys whose code lies
within 1e-3 of a rounding boundary); and within the Eq. 15 envelope of the
fp64 softmax.
"""
import math

import numpy as np
import pytest
import torch

import expcast_ref as ER
import oracle
import vcsynth
from oracle import exact
from layouts import k_matches, unpack_k, unpack_v

pytestmark = pytest.mark.gpu

REL_L2_TOL = 1e-2  # the stated tolerance for the attention output vs the emulation


@pytest.fixture(scope="module")
def vc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_attention_amd as m
    m.lib()
    return m


def _np(t):
    return t.detach().cpu().numpy()


def _bf16_f32(t):
    return t.detach().float().cpu().numpy()


def _mu_split(m):
    """The stored form of the oracle's fp32 scaled means: hi = bf16(m),
    lo = bf16(m - hi), both round-half-even, packed hi | lo << 16."""
    m = np.asarray(m, np.float32)
    hi = oracle.f32_to_bf16_bits(m).astype(np.uint32)
    lo = oracle.f32_to_bf16_bits(m - oracle.bf16_bits_to_f32(hi.astype(np.uint16))).astype(np.uint32)
    return (hi | (lo << 16)).reshape(m.shape)


def _rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def test_abi_version(vc):
    assert vc.vc_abi_version() == vc.ABI_VERSION


# --------------------------------------------------------------------------- #
# ExpCast code map
# --------------------------------------------------------------------------- #

def test_expcast_exhaustive_grid(vc):
    u = (np.arange(-16 * 1024, 1) / 1024.0).astype(np.float32)  # all u in [-16, 0] step 1/1024
    a = np.array([8.0], np.float32)
    b = np.array([119.65], np.float32)
    got = _np(vc.vc_expcast_codes(torch.from_numpy(u).cuda(), torch.from_numpy(a).cuda(),
                                  torch.from_numpy(b).cuda(), u.size))
    want = oracle.expcast_codes(u, a, b, u.size)
    closed = np.array([oracle.expcast_code_u(float(x)) for x in u], np.uint8)
    assert (got == want).all()
    assert (got == closed).all()


def test_expcast_random_rows(vc):
    rng = np.random.default_rng(0)
    R, L = 257, 128
    x = (rng.standard_normal(R * L) * 30).astype(np.float32)
    a = rng.uniform(0.05, 20, R).astype(np.float32)
    b = rng.uniform(-60, 160, R).astype(np.float32)
    got = _np(vc.vc_expcast_codes(torch.from_numpy(x).cuda(), torch.from_numpy(a).cuda(),
                                  torch.from_numpy(b).cuda(), L))
    assert (got == oracle.expcast_codes(x, a, b, L)).all()


# --------------------------------------------------------------------------- #
# quantizers
# --------------------------------------------------------------------------- #

@pytest.mark.parametrize("B,S,H,D,kind", [(1, 1024, 2, 64, "tiny"), (1, 1000, 3, 128, "t3"), (2, 300, 1, 64, "n"),
                                          (1, 129, 2, 128, "n"), (1, 1, 1, 128, "n"), (1, 2048, 4, 128, "plain")])
def test_quantize_bitexact(vc, B, S, H, D, kind):
    print(f"case quantize B={B} S={S} H={H} D={D} {kind}", flush=True)
    if kind == "tiny":
        q, k, v = vcsynth.make_qkv("tiny")
    elif kind == "plain":
        q, k, v = vcsynth.make_qkv("plain", S=S, H=H)
    else:
        q, k, v = vcsynth.random_qkv(B, S, H, D, seed=S + H, v_kind="t3" if kind == "t3" else "normal")
    # Q's codes carry G = 8 fl(sm log2 e); a non-default scale on some cases
    sm = float(np.float32(0.3 if kind == "t3" else 1 / np.sqrt(D)))
    out = vc.vc_quantize(q.cuda(), k.cuda(), v.cuda(), sm_scale=sm)
    torch.cuda.synchronize()
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    codes, sc = oracle.quantize_qk(qb, oracle.q_prefactor(sm))
    assert (_np(out["q8"]) == codes).all()
    assert (_np(out["q_scale"]) == sc).all()
    codes, sc = oracle.quantize_qk(kb)
    assert k_matches(_np(out["k8"]), D, codes, S)
    assert (_np(out["k_scale"]) == sc).all()
    codes, sc = oracle.quantize_v(vb)
    assert (unpack_v(_np(out["v8"]), D) == codes).all()
    assert (_np(out["v_scale"]) == sc).all()


def test_quantize_strided_views(vc):
    # Q, K, V as views of one fused [B, S, 3, H, D] tensor
    B, S, H, D = 1, 700, 3, 128
    g = torch.Generator().manual_seed(5)
    fused = torch.randn((B, S, 3, H, D), generator=g).to(torch.bfloat16)
    fd = fused.cuda()
    q, k, v = fd[:, :, 0], fd[:, :, 1], fd[:, :, 2]
    sm = float(np.float32(1 / np.sqrt(D)))
    out = vc.vc_quantize(q, k, v, sm_scale=sm)
    torch.cuda.synchronize()
    codes, sc = oracle.quantize_qk(vcsynth.bf16_bits(fused[:, :, 0]), oracle.q_prefactor(sm))
    assert (_np(out["q8"]) == codes).all() and (_np(out["q_scale"]) == sc).all()
    codes, sc = oracle.quantize_qk(vcsynth.bf16_bits(fused[:, :, 1]))
    assert k_matches(_np(out["k8"]), D, codes, S) and (_np(out["k_scale"]) == sc).all()
    codes, sc = oracle.quantize_v(vcsynth.bf16_bits(fused[:, :, 2]))
    assert (unpack_v(_np(out["v8"]), D) == codes).all() and (_np(out["v_scale"]) == sc).all()


# --------------------------------------------------------------------------- #
# attention, plain path
# --------------------------------------------------------------------------- #

def _plain_case(vc, q, k, v, sm_scale, window=2, sequential=False, rows_per_head=None, seed=0):
    B, S, H, D = q.shape
    qz = vc.vc_quantize(q.cuda(), k.cuda(), v.cuda(), sm_scale=sm_scale)
    o = vc.vc_attn_fwd(qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], qz["v8"], qz["v_scale"], None, S=S,
                       window=window, sequential=sequential)
    torch.cuda.synchronize()
    og = _bf16_f32(o)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    rng = np.random.default_rng(seed)
    errs = []
    for b in range(B):
        for h in range(H):
            rows = np.arange(S) if rows_per_head is None else np.sort(rng.choice(S, rows_per_head, replace=False))
            res = oracle.pipeline_head(qb, kb, vb, b, h, vsmooth=False, sm_scale=sm_scale, rows=rows, window=window,
                                       flags=oracle.SEQUENTIAL if sequential else 0)
            emu = oracle.bf16_bits_to_f32(res["out_bf16"])
            errs.append(_rel_l2(og[b, rows, h], emu))
            # every element: bf16 of a value within the fp32-order / boundary-code bound
            st = ER.check_rows(og[b, rows, h], res, S, rows, window, sequential)
            print(f"  b{b} h{h}: rel-L2 {errs[-1]:.2e}, row max {st['row_rel_l2_max']:.2e}, "
                  f"bit-identical {st['bit_identical']:.4f}", flush=True)
    return max(errs), og


@pytest.mark.parametrize("B,S,H,D,sm,window,seq", [
    (1, 1024, 2, 64, 1 / 8, 2, False),
    (1, 1000, 2, 128, 1 / math.sqrt(128), 2, False),
    (1, 1000, 2, 128, 4 / math.sqrt(128), 0, False),
    (2, 300, 1, 64, 0.3, 2, True),
    (1, 129, 1, 128, 1 / math.sqrt(128), 5, False),
    (1, 64, 2, 128, 1 / math.sqrt(128), 2, False),
])
def test_attn_plain_parity(vc, B, S, H, D, sm, window, seq):
    print(f"case attn plain B={B} S={S} H={H} D={D} sm={sm:.4f} W={window} seq={seq}", flush=True)
    q, k, v = vcsynth.random_qkv(B, S, H, D, seed=7 * S + D, v_kind="t3")
    err, _ = _plain_case(vc, q, k, v, sm, window, seq)
    assert err <= REL_L2_TOL, err


def test_attn_plain_config_sampled_rows(vc):
    # the plain workload's recipe (K bias, Student-t V) at S = 16384 on 2 heads
    print("case attn plain-config S=16384 H=2 sampled", flush=True)
    q, k, v = vcsynth.make_qkv("plain", H=2)
    err, _ = _plain_case(vc, q, k, v, 1 / math.sqrt(128), rows_per_head=96, seed=3)
    assert err <= REL_L2_TOL, err


# --------------------------------------------------------------------------- #
# V-Smooth grouping
# --------------------------------------------------------------------------- #

def _group_case(vc, k, v, clusters, iters, seed):
    B, S, H, D = v.shape
    g = vc.vc_smooth_group(k.cuda(), v.cuda(), clusters, iters, seed)
    torch.cuda.synchronize()
    kb, vb = vcsynth.bf16_bits(k), vcsynth.bf16_bits(v)
    ref = oracle.smooth_group(kb, vb, clusters, iters, seed)
    for (b, h), r in ref.items():
        assert (_np(g["labels"][b, h]) == r["labels"]).all(), ("labels", b, h)
        assert (_np(g["centroids"][b, h]) == r["centroids"]).all(), ("centroids", b, h)
        assert (_np(g["perm"][b, h]) == r["perm"]).all(), ("perm", b, h)
        assert (unpack_k(_np(g["k8"][b, h]), D) == r["k_codes"]).all(), ("k8", b, h)
        assert (_np(g["k_scale"][b, h]) == r["k_scale"]).all(), ("k_scale", b, h)
        assert (_np(g["mu_bf16"][b, h]).view(np.uint16) == r["mu_bf16"]).all(), ("mu", b, h)
        assert (_np(g["mu_split"][b, h]).view(np.uint32) == _mu_split(r["mu_scaled"])).all(), ("mu_split", b, h)
        assert (_np(g["r_scale"][b, h]) == r["r_scale"]).all(), ("r_scale", b, h)
        assert (unpack_v(_np(g["r8"][b, h]), D) == r["r_codes"]).all(), ("r8", b, h)
    return g, ref


def test_smooth_group_tiny_bitexact(vc):
    print("case group tiny k=8 iters=3", flush=True)
    q, k, v = vcsynth.make_qkv("tiny")
    _group_case(vc, k, v, 8, 3, 1000)


@pytest.mark.parametrize("S,H,D,kc,iters", [(1000, 2, 128, 64, 4), (300, 1, 64, 128, 2), (5, 1, 128, 5, 3)])
def test_smooth_group_edge_bitexact(vc, S, H, D, kc, iters):
    print(f"case group S={S} H={H} D={D} k={kc} iters={iters}", flush=True)
    q, k, v = vcsynth.random_qkv(1, S, H, D, seed=S, v_kind="t3")
    _group_case(vc, k, v, kc, iters, 77)


def test_smooth_group_video_bitexact(vc):
    print("case group longcat-recipe H=1 S=32760 k=64 iters=4", flush=True)
    q, k, v = vcsynth.make_qkv("longcat", H=1)
    _group_case(vc, k, v, 64, 4, 1002)


@pytest.mark.parametrize("D,kc", [(128, 8), (64, 16), (128, 64), (64, 128)])
def test_smooth_group_ties_bitexact(vc, D, kc):
    # six distinct value rows per head, each repeated: the Forgy draw takes
    # duplicate centroids, so most tokens are equally far from two or more
    # clusters and the lowest index must win (the open-token path)
    print(f"case group ties D={D} k={kc}", flush=True)
    S, H = 1500, 2
    q, k, v = vcsynth.random_qkv(1, S, H, D, seed=31)
    g = torch.Generator().manual_seed(5)
    base = torch.randn((6, H, D), generator=g)
    pick = torch.randint(0, 6, (S,), generator=g)
    v = base[pick].unsqueeze(0).to(torch.bfloat16)
    _group_case(vc, k, v, kc, 3, 17)


@pytest.mark.parametrize("D,kc,frac", [(128, 64, 0.1), (64, 64, 0.1), (128, 64, 0.3), (64, 128, 0.3)])
def test_smooth_group_partial_ties_bitexact(vc, D, kc, frac):
    # a fraction of the tokens repeat one value row, the rest are random: the
    # Forgy draw takes about kc * frac copies of that row, so 150 to 450
    # tokens per head are open, each tied between that many candidates (7 to
    # 40), beside the random tokens settled by the matrix-core bound
    print(f"case group partial ties D={D} k={kc} frac={frac}", flush=True)
    S, H = 1500, 2
    q, k, v = vcsynth.random_qkv(1, S, H, D, seed=37, v_kind="t3")
    g = torch.Generator().manual_seed(8)
    row = torch.randn((1, 1, H, D), generator=g).to(torch.bfloat16)
    tied = (torch.rand((1, S, 1, 1), generator=g) < frac)
    v = torch.where(tied, row.expand(1, S, H, D), v)
    _group_case(vc, k, v, kc, 3, 29)


def test_smooth_group_batch2_bitexact(vc):
    # two batch entries of two heads, a ragged last tile: every (b, h) runs
    # its own k-means, sort and apply passes
    print("case group B=2 H=2 S=700 D=128 k=16", flush=True)
    q, k, v = vcsynth.random_qkv(2, 700, 2, 128, seed=53, v_kind="t3")
    _group_case(vc, k, v, 16, 3, 19)


def test_smooth_group_large_values_bitexact(vc):
    # a quarter of the tokens scaled x400 (|v| in the thousands): the slow
    # fixed-point conversion and a wide candidate margin
    print("case group large values", flush=True)
    q, k, v = vcsynth.random_qkv(1, 2000, 2, 128, seed=41, v_kind="t3")
    g = torch.Generator().manual_seed(6)
    scale = torch.where(torch.rand((1, 2000, 2, 1), generator=g) < 0.25, 400.0, 1.0)
    v = (v.float() * scale).to(torch.bfloat16)
    _group_case(vc, k, v, 64, 3, 23)


def _next_step(x, seed, sigma=0.05):
    """bf16 activations of a following denoising step: x plus small noise."""
    g = torch.Generator().manual_seed(seed)
    return (x.float() + sigma * torch.randn(x.shape, generator=g)).to(torch.bfloat16)


def _apply_matches(g, ref, b, h, D):
    assert (unpack_k(_np(g["k8"][b, h]), D) == ref["k_codes"]).all(), ("k8", b, h)
    assert (_np(g["k_scale"][b, h]) == ref["k_scale"]).all(), ("k_scale", b, h)
    assert (_np(g["mu_bf16"][b, h]).view(np.uint16) == ref["mu_bf16"]).all(), ("mu", b, h)
    assert (_np(g["mu_split"][b, h]).view(np.uint32) == _mu_split(ref["mu_scaled"])).all(), ("mu_split", b, h)
    assert (_np(g["r_scale"][b, h]) == ref["r_scale"]).all(), ("r_scale", b, h)
    assert (unpack_v(_np(g["r8"][b, h]), D) == ref["r_codes"]).all(), ("r8", b, h)


@pytest.mark.parametrize("S,H,D,kc,iters", [(1024, 2, 64, 8, 3), (1000, 2, 128, 64, 2)])
def test_smooth_group_warm_start_bitexact(vc, S, H, D, kc, iters):
    # step t groups cold; step t+1 (perturbed K, V) starts k-means from step t's centroids
    print(f"case group warm start S={S} H={H} D={D} k={kc} iters={iters}", flush=True)
    q, k, v = vcsynth.random_qkv(1, S, H, D, seed=S + 1, v_kind="t3")
    g1 = vc.vc_smooth_group(k.cuda(), v.cuda(), kc, iters, 5)
    k2, v2 = _next_step(k, 11), _next_step(v, 12)
    g2 = vc.vc_smooth_group(k2.cuda(), v2.cuda(), kc, iters, 0, warm_start=g1["centroids"])
    torch.cuda.synchronize()
    kb, vb = vcsynth.bf16_bits(k2), vcsynth.bf16_bits(v2)
    for b in range(1):
        for h in range(H):
            init = _np(g1["centroids"][b, h])
            labels, cent = oracle.kmeans_head(np.ascontiguousarray(vb[b, :, h]), kc, iters, 0, b, h, H, init=init)
            perm = oracle.argsort_labels(labels, kc)
            assert (_np(g2["labels"][b, h]) == labels).all(), ("labels", b, h)
            assert (_np(g2["centroids"][b, h]) == cent).all(), ("centroids", b, h)
            assert (_np(g2["perm"][b, h]) == perm).all(), ("perm", b, h)
            ref = oracle.smooth_apply_head(np.ascontiguousarray(kb[b, :, h]), np.ascontiguousarray(vb[b, :, h]), perm)
            _apply_matches(g2, ref, b, h, D)


def test_smooth_group_warm_start_composes_on_gpu(vc):
    # cold a + b iterations == cold a, then b iterations warm-started from it
    print("case group warm composition S=2048 H=2 D=128 k=32", flush=True)
    q, k, v = vcsynth.random_qkv(1, 2048, 2, 128, seed=9, v_kind="t3")
    kc, vcu = k.cuda(), v.cuda()
    g_ab = vc.vc_smooth_group(kc, vcu, 32, 3, 42)
    g_a = vc.vc_smooth_group(kc, vcu, 32, 1, 42)
    g_w = vc.vc_smooth_group(kc, vcu, 32, 2, 0, warm_start=g_a["centroids"])
    torch.cuda.synchronize()
    for key in ("labels", "centroids", "perm", "k8", "r8", "mu_split", "r_scale"):
        assert torch.equal(g_w[key], g_ab[key]), key


@pytest.mark.parametrize("S,H,D", [(1024, 2, 64), (1000, 2, 128), (129, 1, 128)])
def test_smooth_group_reuse_perm_bitexact(vc, S, H, D):
    # the permutation of step t applied to step t+1's K, V: no k-means, no sort
    print(f"case group reuse perm S={S} H={H} D={D}", flush=True)
    q, k, v = vcsynth.random_qkv(1, S, H, D, seed=S + 2, v_kind="t3")
    kc = min(16, S)
    g1 = vc.vc_smooth_group(k.cuda(), v.cuda(), kc, 2, 3)
    k2, v2 = _next_step(k, 21), _next_step(v, 22)
    g2 = vc.vc_smooth_group(k2.cuda(), v2.cuda(), kc, 2, 3, reuse_perm=g1["perm"])
    torch.cuda.synchronize()
    assert "labels" not in g2 and "centroids" not in g2
    kb, vb = vcsynth.bf16_bits(k2), vcsynth.bf16_bits(v2)
    for h in range(H):
        perm = _np(g1["perm"][0, h])
        ref = oracle.smooth_apply_head(np.ascontiguousarray(kb[0, :, h]), np.ascontiguousarray(vb[0, :, h]), perm)
        _apply_matches(g2, ref, 0, h, D)


def test_smooth_group_reuse_perm_clamped(vc):
    # a caller's permutation with entries outside [0, S): the apply kernels
    # clamp every gathered index into [0, S), so the result is the apply step
    # on the clamped list (wrong codes for a wrong list, never an access
    # outside K or V)
    print("case group reuse perm, out-of-range entries clamped", flush=True)
    S, H, D = 300, 2, 128
    q, k, v = vcsynth.random_qkv(1, S, H, D, seed=8, v_kind="t3")
    rng = np.random.default_rng(8)
    perm = np.stack([rng.permutation(S) for _ in range(H)])[None].astype(np.int32)
    perm[0, 0, [3, 150, 299]] = [-7, S + 5, 2 ** 31 - 1]
    perm[0, 1, [0, 128]] = [-(2 ** 31), S]
    g = vc.vc_smooth_group(k.cuda(), v.cuda(), 16, 2, 3, reuse_perm=torch.from_numpy(perm).cuda())
    torch.cuda.synchronize()
    kb, vb = vcsynth.bf16_bits(k), vcsynth.bf16_bits(v)
    for h in range(H):
        pc = np.clip(perm[0, h].astype(np.int64), 0, S - 1).astype(np.int32)
        ref = oracle.smooth_apply_head(np.ascontiguousarray(kb[0, :, h]), np.ascontiguousarray(vb[0, :, h]), pc)
        _apply_matches(g, ref, 0, h, D)


# --------------------------------------------------------------------------- #
# attention, V-Smooth path
# --------------------------------------------------------------------------- #

def _vsmooth_case(vc, q, k, v, clusters, iters, seed, sm, rows_per_head=None, window=2):
    B, S, H, D = q.shape
    qz = vc.vc_quantize(q.cuda(), sm_scale=sm)
    g = vc.vc_smooth_group(k.cuda(), v.cuda(), clusters, iters, seed)
    o = vc.vc_attn_fwd(qz["q8"], qz["q_scale"], g["k8"], g["k_scale"], g["r8"], g["r_scale"], g["mu_split"], S=S,
                       window=window)
    torch.cuda.synchronize()
    og = _bf16_f32(o)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    rng = np.random.default_rng(1)
    errs, res_all = [], {}
    for b in range(B):
        for h in range(H):
            rows = np.arange(S) if rows_per_head is None else np.sort(rng.choice(S, rows_per_head, replace=False))
            res = oracle.pipeline_head(qb, kb, vb, b, h, vsmooth=True, nclust=clusters, iters=iters, seed=seed,
                                       sm_scale=sm, rows=rows, window=window)
            emu = oracle.bf16_bits_to_f32(res["out_bf16"])
            errs.append(_rel_l2(og[b, rows, h], emu))
            st = ER.check_rows(og[b, rows, h], res, S, rows, window, vsmooth=True)
            print(f"  b{b} h{h}: rel-L2 {errs[-1]:.2e}, row max {st['row_rel_l2_max']:.2e}, "
                  f"bit-identical {st['bit_identical']:.4f}", flush=True)
            res_all[(b, h)] = res
    return max(errs), og, res_all


def test_attn_vsmooth_tiny_parity(vc):
    print("case attn vsmooth tiny", flush=True)
    q, k, v = vcsynth.make_qkv("tiny")
    err, _, _ = _vsmooth_case(vc, q, k, v, 8, 3, 1000, 1 / 8)
    assert err <= REL_L2_TOL, err


def test_attn_vsmooth_ragged_parity(vc):
    print("case attn vsmooth ragged S=1000 D=128", flush=True)
    q, k, v = vcsynth.random_qkv(1, 1000, 2, 128, seed=11, v_kind="t3")
    err, _, _ = _vsmooth_case(vc, q, k, v, 16, 3, 5, 2 / math.sqrt(128))
    assert err <= REL_L2_TOL, err


def test_attn_vsmooth_batch2_parity(vc):
    # B = 2 at D = 128: the V-Smooth kernel's (b, h) bases, an odd tile count
    # (a dead half in the last pair) and a ragged tile
    print("case attn vsmooth B=2 H=2 S=600 D=128", flush=True)
    q, k, v = vcsynth.random_qkv(2, 600, 2, 128, seed=59, v_kind="t3")
    err, _, _ = _vsmooth_case(vc, q, k, v, 16, 3, 7, 1 / math.sqrt(128))
    assert err <= REL_L2_TOL, err


def test_attn_vsmooth_video_envelope(vc):
    # longcat-recipe head, sampled rows: parity with the emulation and the
    # Eq. 15 envelope against the fp64 softmax of the original values
    print("case attn vsmooth longcat-recipe H=1 sampled + envelope", flush=True)
    q, k, v = vcsynth.make_qkv("longcat", H=1)
    S, D = q.shape[1], q.shape[3]
    sm = 1 / math.sqrt(D)
    err, og, res_all = _vsmooth_case(vc, q, k, v, 64, 4, 1002, sm, rows_per_head=48)
    assert err <= REL_L2_TOL, err
    res = res_all[(0, 0)]
    rows = res["rows"]
    qf = exact.to_f64(vcsynth.bf16_bits(q)[0, :, 0])
    kf = exact.to_f64(vcsynth.bf16_bits(k)[0, :, 0])
    vf = exact.to_f64(vcsynth.bf16_bits(v)[0, :, 0])
    ref = exact.attention_rows(qf, kf, vf, sm, rows)
    # dequantised operands: scores and values the FP8 path actually sees
    blk = np.arange(S) // 128
    # Q's codes carry G = 8 fl(sm log2 e): divide it back out
    qd = oracle.e4m3_decode(res["q_codes"][:S]) * res["q_scale"][blk][:, None] / oracle.q_prefactor(sm)
    perm = res["perm"]
    kd_p = oracle.e4m3_decode(res["k_codes"][:S]) * res["k_scale"][blk][:, None]
    vd_p = (oracle.e4m3_decode(res["r_codes"][:, :S]).T + res["mu_scaled"][blk]) * res["r_scale"][None, :]
    inv = np.argsort(perm)
    kd, vd = kd_p[inv], vd_p[inv]
    vmax = np.linalg.norm(vf, axis=1).max()
    diam_ub = 2 * np.linalg.norm(vd - vd.mean(0), axis=1).max()  # >= diam2 of the dequantised rows
    dv = np.linalg.norm(vd - vf, axis=1).max()
    for ri, i in enumerate(rows):
        s_exact = (qf[i] @ kf.T) * sm
        s_deq = (qd[i] @ kd.T) * sm
        p_exact = np.exp(s_exact - s_exact.max())
        p_exact /= p_exact.sum()
        p_qk = np.exp(s_deq - s_deq.max())
        p_qk /= p_qk.sum()
        tv_qk = 0.5 * np.abs(p_exact - p_qk).sum()
        _, tau = exact.row_tv_check(s_deq * exact.LOG2E)
        bound = (0.0364 + tau + tv_qk + 1e-4) * diam_ub + dv + 1e-2 * vmax
        assert np.linalg.norm(og[0, i, 0] - ref[ri]) <= bound, (i, bound)


# --------------------------------------------------------------------------- #
# BF16 baseline on the same skeleton (checked against exact fp64 attention)
# --------------------------------------------------------------------------- #

BF16_TOL = 1e-2  # bf16 probabilities and output rounding, 2^-9 relative each


@pytest.mark.parametrize("B,S,H,D,sm,seq,rise", [(1, 1000, 2, 128, 1 / math.sqrt(128), False, 0),
                                                 (1, 1024, 2, 64, 1 / 8, False, 0), (2, 300, 1, 64, 0.3, True, 0),
                                                 (1, 129, 1, 128, 2 / math.sqrt(128), False, 0),
                                                 (1, 64, 1, 128, 1 / math.sqrt(128), False, 0),
                                                 (1, 1000, 2, 128, 1 / math.sqrt(128), True, 3),
                                                 (1, 1000, 1, 128, 1 / math.sqrt(128), False, 3)])
def test_attn_bf16_baseline_vs_exact(vc, B, S, H, D, sm, seq, rise):
    """rise: keys of tile t scaled by 1 + rise t, so the running max rises
    past the kernel's headroom of 8 after the first step."""
    print(f"case bf16 baseline B={B} S={S} H={H} D={D} seq={seq} rise={rise}", flush=True)
    q, k, v = vcsynth.random_qkv(B, S, H, D, seed=3 * S + D, v_kind="t3")
    if rise:
        k = vcsynth.keys_rising_by_tile(k, rise)
    vt = vc.vc_pack_v_bf16(v.cuda())
    o = vc.vc_attn_fwd_bf16(q.cuda(), k.cuda(), vt, sm_scale=sm, sequential=seq)
    torch.cuda.synchronize()
    og = _bf16_f32(o)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    for b in range(B):
        for h in range(H):
            ref = exact.attention_rows(exact.to_f64(qb[b, :, h]), exact.to_f64(kb[b, :, h]),
                                       exact.to_f64(vb[b, :, h]), sm)
            assert _rel_l2(og[b, :, h], ref) <= BF16_TOL
            row = np.linalg.norm(og[b, :, h] - ref, axis=1) / np.linalg.norm(ref, axis=1)
            assert row.max() <= BF16_TOL, (b, h, row.max())  # every row, not only the pooled norm


def test_attn_bf16_baseline_plain_config(vc):
    print("case bf16 baseline plain-config S=16384 H=2 sampled", flush=True)
    q, k, v = vcsynth.make_qkv("plain", H=2)
    sm = 1 / math.sqrt(128)
    vt = vc.vc_pack_v_bf16(v.cuda())
    o = vc.vc_attn_fwd_bf16(q.cuda(), k.cuda(), vt, sm_scale=sm)
    torch.cuda.synchronize()
    og = _bf16_f32(o)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    rows = np.sort(np.random.default_rng(4).choice(q.shape[1], 128, replace=False))
    for h in range(2):
        ref = exact.attention_rows(exact.to_f64(qb[0, :, h]), exact.to_f64(kb[0, :, h]), exact.to_f64(vb[0, :, h]),
                                   sm, rows)
        assert _rel_l2(og[0, rows, h], ref) <= BF16_TOL
