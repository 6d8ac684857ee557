"""vc_smooth_group_noalloc against vc_smooth_group, through the C ABI.

The allocation-free entry point takes its workspace from the library's
static per-GPU scratch; its outputs must equal vc_smooth_group's bit for bit
(labels, permutation, centroids, K' codes and scales, residual codes and
scales, block means, scaled means).  Two calls in a row, the second on a
smaller input, show that what the first call left in the scratch does not
leak into the second.
"""
import pytest
import torch

import vcsynth

pytestmark = pytest.mark.gpu

KEYS = ("centroids", "labels", "perm", "k8", "k_scale", "r8", "r_scale", "mu_bf16", "mu_split")


@pytest.fixture(scope="module")
def vc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_attention_amd as m
    m.lib()
    return m


def _same(a, b, keys=KEYS):
    for key in keys:
        if key in a or key in b:
            assert torch.equal(a[key], b[key]), key


def test_noalloc_matches_workspace_call_twice(vc):
    cases = [(1, 2048, 4, 128, 64, 4, 11), (1, 700, 2, 128, 16, 3, 12)]  # the second smaller
    for B, S, H, D, kc, iters, seed in cases:
        print(f"case noalloc S={S} H={H} D={D} k={kc}", flush=True)
        q, k, v = vcsynth.random_qkv(B, S, H, D, seed=seed, v_kind="t3")
        kd, vd = k.cuda(), v.cuda()
        a = vc.vc_smooth_group(kd, vd, kc, iters, seed)
        b = vc.vc_smooth_group_noalloc(kd, vd, kc, iters, seed)
        torch.cuda.synchronize()
        _same(a, b)


def test_noalloc_warm_start_reuse_and_centring(vc):
    print("case noalloc warm start, permutation reuse, K centring", flush=True)
    S, H, D = 1000, 2, 64
    q, k, v = vcsynth.random_qkv(1, S, H, D, seed=5, v_kind="t3")
    kd, vd = k.cuda(), v.cuda()
    a = vc.vc_smooth_group(kd, vd, 8, 2, 3)
    b = vc.vc_smooth_group_noalloc(kd, vd, 8, 2, 3)
    torch.cuda.synchronize()
    _same(a, b)
    aw = vc.vc_smooth_group(kd, vd, 8, 2, 0, warm_start=a["centroids"])
    bw = vc.vc_smooth_group_noalloc(kd, vd, 8, 2, 0, warm_start=a["centroids"])
    torch.cuda.synchronize()
    _same(aw, bw)
    ar = vc.vc_smooth_group(kd, vd, 8, 2, 0, reuse_perm=a["perm"])
    br = vc.vc_smooth_group_noalloc(kd, vd, 8, 2, 0, reuse_perm=a["perm"])
    torch.cuda.synchronize()
    _same(ar, br, KEYS[2:])
    prep = {"flags": vc.VC_PREP_K_CENTER}
    ac = vc.vc_smooth_group(kd, vd, 8, 2, 3, prep=prep)
    bc = vc.vc_smooth_group_noalloc(kd, vd, 8, 2, 3, prep=prep)
    torch.cuda.synchronize()
    _same(ac, bc)
    assert not torch.equal(ac["k8"], a["k8"])  # the centring changed K'


def test_noalloc_refuses_oversized_shape(vc):
    # refused before anything is enqueued
    v = torch.zeros((1, 16, 1, 128), dtype=torch.bfloat16, device="cuda")
    need = vc.vc_smooth_group_noalloc_bytes(1, 200, 84672, 128, 64)
    assert need > (16 << 20)
    sh = vc.vc_shape(1, 200, 84672, 128)
    import ctypes
    ok = vc.vc_bshd(v.data_ptr(), 0, 128, 128)
    P = ctypes.c_void_p
    st = vc.lib().vc_smooth_group_noalloc(ctypes.byref(sh), ctypes.byref(ok), ctypes.byref(ok),
                                          ctypes.byref(vc.vc_group_params(64, 4, 0, 0)), None,
                                          *[P(v.data_ptr())] * 9, vc._stream())
    assert st == 7
