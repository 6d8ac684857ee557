"""Determinism at the headline shape: the whole path run twice gives the same
bytes.

Wan2.2-720p-shaped input (B=1, H=40, S=75600, D=128), the launch
configuration bench.py times.  The second run reuses the first run's
workspace (left holding that run's final state) and writes into output
buffers filled with 0xff beforehand, so a byte the kernels do not write, or
a sum that depends on the order of its atomic additions, shows up as a
difference.  Covered: vc_quantize (Q; Q, K, V), vc_smooth_group (labels, pi,
centroids, K' codes and scales, residual codes and scales, scaled means),
vc_attn_fwd on the V-Smooth and plain paths, with repair tiles, and the
4-bit path (vc_quantize4, vc_attn_fwd4).
"""
import pytest
import torch

import vcsynth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def vc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_attention_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def wan():
    w = vcsynth.WORKLOADS["wan"]
    print(f"case determinism wan: B={w.B} H={w.H} S={w.S} D={w.D}", flush=True)
    q, k, v = vcsynth.make_qkv("wan", device="cuda")
    torch.cuda.synchronize()
    return w, q, k, v


def _poison(d):
    """A copy of the output dict with every tensor filled with 0xff bytes."""
    out = {}
    for key, t in d.items():
        if isinstance(t, torch.Tensor):
            x = torch.empty_like(t)
            x.view(torch.uint8).fill_(0xFF)
            out[key] = x
    return out


def _same(a, b, keys):
    for key in keys:
        x, y = a[key], b[key]
        assert x.shape == y.shape, key
        assert torch.equal(x.contiguous().view(torch.uint8), y.contiguous().view(torch.uint8)), key


def test_vsmooth_path_twice_same_bytes(vc, wan):
    w, q, k, v = wan
    ws = torch.empty(vc.vc_smooth_group_workspace_size(w.B, w.H, w.S, w.D, w.clusters), dtype=torch.uint8,
                     device="cuda")
    qz1 = vc.vc_quantize(q, sm_scale=w.sm_scale)
    g1 = vc.vc_smooth_group(k, v, w.clusters, w.iters, w.seed, workspace=ws)
    o1 = vc.vc_attn_fwd(qz1["q8"], qz1["q_scale"], g1["k8"], g1["k_scale"], g1["r8"], g1["r_scale"],
                        g1["mu_split"], S=w.S)
    torch.cuda.synchronize()
    qz2 = vc.vc_quantize(q, sm_scale=w.sm_scale, out=_poison(qz1))
    g2 = vc.vc_smooth_group(k, v, w.clusters, w.iters, w.seed, workspace=ws, out=_poison(g1))
    o2 = torch.empty_like(o1)
    o2.view(torch.uint8).fill_(0xFF)
    vc.vc_attn_fwd(qz2["q8"], qz2["q_scale"], g2["k8"], g2["k_scale"], g2["r8"], g2["r_scale"], g2["mu_split"],
                   S=w.S, out=o2)
    torch.cuda.synchronize()
    _same(qz1, qz2, ["q8", "q_scale"])
    _same(g1, g2, ["labels", "perm", "centroids", "k8", "k_scale", "r8", "r_scale", "mu_split", "mu_bf16"])
    _same({"o": o1}, {"o": o2}, ["o"])
    assert torch.isfinite(o1.float()).all().item()


def test_plain_and_repair_twice_same_bytes(vc, wan):
    w, q, k, v = wan
    qz1 = vc.vc_quantize(q, k, v, sm_scale=w.sm_scale)
    o1 = vc.vc_attn_fwd(qz1["q8"], qz1["q_scale"], qz1["k8"], qz1["k_scale"], qz1["v8"], qz1["v_scale"], None, S=w.S)
    R = vc.repair_count(w.S, 0.005)
    rws = torch.empty(vc.vc_repair_workspace_size(w.B, w.H, w.S, w.D), dtype=torch.uint8, device="cuda")
    rp1 = vc.vc_repair_prepare(k, v, R, workspace=rws)
    or1 = vc.vc_attn_fwd(qz1["q8"], qz1["q_scale"], qz1["k8"], qz1["k_scale"], qz1["v8"], qz1["v_scale"], None,
                         S=w.S, repair=rp1)
    torch.cuda.synchronize()
    qz2 = vc.vc_quantize(q, k, v, sm_scale=w.sm_scale, out=_poison(qz1))
    rp2 = vc.vc_repair_prepare(k, v, R, workspace=rws, out=_poison(rp1))
    o2, or2 = torch.empty_like(o1), torch.empty_like(o1)
    o2.view(torch.uint8).fill_(0xFF)
    or2.view(torch.uint8).fill_(0xFF)
    vc.vc_attn_fwd(qz2["q8"], qz2["q_scale"], qz2["k8"], qz2["k_scale"], qz2["v8"], qz2["v_scale"], None, S=w.S,
                   out=o2)
    vc.vc_attn_fwd(qz2["q8"], qz2["q_scale"], qz2["k8"], qz2["k_scale"], qz2["v8"], qz2["v_scale"], None, S=w.S,
                   out=or2, repair=rp2)
    torch.cuda.synchronize()
    _same(qz1, qz2, ["q8", "q_scale", "k8", "k_scale", "v8", "v_scale"])
    _same(rp1, rp2, [key for key, t in rp1.items() if isinstance(t, torch.Tensor)])
    _same({"o": o1, "or": or1}, {"o": o2, "or": or2}, ["o", "or"])
    assert not torch.equal(o1, or1)  # the repair tiles change the output


def test_mxfp4_path_twice_same_bytes(vc, wan):
    w, q, k, v = wan
    g = vc.vc_smooth_group(k, v, w.clusters, w.iters, w.seed)
    z1 = vc.vc_quantize4(q, k, v, sm_scale=w.sm_scale, perm=g["perm"], mu_bf16=g["mu_bf16"])
    o1 = vc.vc_attn_fwd4(z1["q4"], z1["q4_scale"], z1["k4"], z1["k4_scale"], z1["v4"], z1["v4_scale"], g["mu_bf16"],
                         S=w.S)
    torch.cuda.synchronize()
    z2 = vc.vc_quantize4(q, k, v, sm_scale=w.sm_scale, perm=g["perm"], mu_bf16=g["mu_bf16"], out=_poison(z1))
    o2 = torch.empty_like(o1)
    o2.view(torch.uint8).fill_(0xFF)
    vc.vc_attn_fwd4(z2["q4"], z2["q4_scale"], z2["k4"], z2["k4_scale"], z2["v4"], z2["v4_scale"], g["mu_bf16"],
                    S=w.S, out=o2)
    torch.cuda.synchronize()
    _same(z1, z2, [key for key, t in z1.items() if isinstance(t, torch.Tensor)])
    _same({"o": o1}, {"o": o2}, ["o"])
