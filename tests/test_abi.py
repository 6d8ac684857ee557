"""CPU checks of the C ABI: the library loads, exports every entry point the
header declares, and rejects invalid arguments before touching the GPU (no
compute call is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vc_attn.h")
LIB = os.path.join(ROOT, "bit_fp8_attention_amd", "libvcattn.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int32_t|size_t|const char\*)\s+(vc_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def vc():
    if not os.path.exists(LIB):
        pytest.fail("libvcattn.so not built (run __graft_entry__.build())")
    import bit_fp8_attention_amd as m
    return m


def test_header_declares_the_calls():
    names = _declared()
    for n in ["vc_abi_version", "vc_status_str", "vc_quantize", "vc_smooth_group_workspace_size",
              "vc_smooth_group", "vc_repair_workspace_size", "vc_repair_prepare", "vc_attn_fwd",
              "vc_quantize4", "vc_attn_fwd4", "vc_pack_v_bf16", "vc_attn_fwd_bf16", "vc_expcast_codes",
              "vc_smooth_group_noalloc", "vc_smooth_group_noalloc_bytes"]:
        assert n in names


def test_library_exports_every_declared_symbol(vc):
    L = vc.lib()
    for n in _declared():
        assert hasattr(L, n), n


def test_abi_version_and_status_strings(vc):
    assert vc.vc_abi_version() == vc.ABI_VERSION == 7
    assert vc.vc_status_str(0) == "VC_OK"
    for s in range(1, 8):
        assert vc.vc_status_str(s).startswith("VC_ERR_")
    assert vc.vc_status_str(99) == "unknown vc_status"


def _shape(B=1, H=2, S=256, D=128):
    return vc_mod().vc_shape(B, H, S, D)


def vc_mod():
    import bit_fp8_attention_amd as m
    return m


FAKE = 1 << 20  # an aligned non-null address; never dereferenced (validation fails first)


def test_quantize_validation(vc):
    L, m = vc.lib(), vc
    ok = m.vc_bshd(FAKE, 256 * 2 * 128, 2 * 128, 128)
    none = m.vc_bshd(None, 0, 0, 0)
    st = ctypes.c_void_p(0)
    P = ctypes.c_void_p
    assert L.vc_quantize(None, 0.0, None, None, None, None, None, None, None, None, None, None, st) == 1
    bad_d = m.vc_shape(1, 2, 256, 96)
    assert L.vc_quantize(ctypes.byref(bad_d), 0.0, None, ctypes.byref(ok), ctypes.byref(none), ctypes.byref(none),
                         P(FAKE), P(FAKE), None, None, None, None, st) == 2
    bad_s = m.vc_shape(1, 2, 0, 128)
    assert L.vc_quantize(ctypes.byref(bad_s), 0.0, None, ctypes.byref(ok), ctypes.byref(none), ctypes.byref(none),
                         P(FAKE), P(FAKE), None, None, None, None, st) == 2
    sh = _shape()
    # q given without its outputs
    assert L.vc_quantize(ctypes.byref(sh), 0.0, None, ctypes.byref(ok), ctypes.byref(none), ctypes.byref(none),
                         None, None, None, None, None, None, st) == 1
    # misaligned input pointer and stride
    mis = m.vc_bshd(FAKE + 2, 256 * 2 * 128, 2 * 128, 128)
    assert L.vc_quantize(ctypes.byref(sh), 0.0, None, ctypes.byref(mis), ctypes.byref(none), ctypes.byref(none),
                         P(FAKE), P(FAKE), None, None, None, None, st) == 3
    mis2 = m.vc_bshd(FAKE, 256 * 2 * 128, 2 * 128 + 4, 128)
    assert L.vc_quantize(ctypes.byref(sh), 0.0, None, ctypes.byref(mis2), ctypes.byref(none), ctypes.byref(none),
                         P(FAKE), P(FAKE), None, None, None, None, st) == 3
    # misaligned output codes
    assert L.vc_quantize(ctypes.byref(sh), 0.0, None, ctypes.byref(ok), ctypes.byref(none), ctypes.byref(none),
                         P(FAKE + 8), P(FAKE), None, None, None, None, st) == 3
    # softmax scale negative, infinite or NaN
    for bad in (-1.0, float("inf"), float("nan")):
        assert L.vc_quantize(ctypes.byref(sh), bad, None, ctypes.byref(ok), ctypes.byref(none), ctypes.byref(none),
                             P(FAKE), P(FAKE), None, None, None, None, st) == 4


def test_smooth_group_validation(vc):
    L, m = vc.lib(), vc
    P = ctypes.c_void_p
    sh = _shape()
    ok = m.vc_bshd(FAKE, 256 * 2 * 128, 2 * 128, 128)
    st = ctypes.c_void_p(0)
    ws = m.vc_smooth_group_workspace_size(1, 2, 256, 128, 64)
    assert ws > 0
    assert m.vc_smooth_group_workspace_size(1, 2, 256, 96, 64) == 0

    def call(p, wsb=ws, ws_ptr=FAKE):
        return L.vc_smooth_group(ctypes.byref(sh), ctypes.byref(ok), ctypes.byref(ok), ctypes.byref(p), None,
                                 *[P(FAKE)] * 9, P(ws_ptr), wsb, st)
    assert call(m.vc_group_params(0, 4, 0, 0)) == 4       # k < 1
    assert call(m.vc_group_params(65, 4, 0, 0)) == 4      # k > 8192 / D
    assert call(m.vc_group_params(64, 0, 0, 0)) == 4      # iters < 1
    assert call(m.vc_group_params(64, 4, 0, 4)) == 4      # unknown flag
    assert call(m.vc_group_params(64, 4, 0, 3)) == 4      # warm start and permutation reuse together

    def call_ptrs(p, ptrs):
        return L.vc_smooth_group(ctypes.byref(sh), ctypes.byref(ok), ctypes.byref(ok), ctypes.byref(p), None,
                                 *[P(x) for x in ptrs], P(FAKE), ws, st)
    no_perm = [FAKE, FAKE, None] + [FAKE] * 6
    assert call_ptrs(m.vc_group_params(64, 4, 0, 2), no_perm) == 1      # reuse needs perm
    assert call_ptrs(m.vc_group_params(64, 4, 0, 1), [None] + [FAKE] * 8) == 1  # warm start needs centroids
    assert call(m.vc_group_params(64, 4, 0, 0), wsb=ws - 1) == 5
    assert call(m.vc_group_params(64, 4, 0, 0), ws_ptr=FAKE + 16) == 3
    # a token stride of 2^30 elements or more (the kernels' 32-bit row offsets)
    huge = m.vc_bshd(FAKE, 1 << 31, 1 << 30, 128)
    assert L.vc_smooth_group(ctypes.byref(sh), ctypes.byref(huge), ctypes.byref(ok),
                             ctypes.byref(m.vc_group_params(64, 4, 0, 0)), None, *[P(FAKE)] * 9, P(FAKE), ws, st) == 2
    near = m.vc_bshd(FAKE, 1 << 31, (1 << 30) - 8, 128)
    assert L.vc_smooth_group(ctypes.byref(sh), ctypes.byref(near), ctypes.byref(ok),
                             ctypes.byref(m.vc_group_params(64, 4, 0, 0)), None, *[P(FAKE)] * 9, P(FAKE), ws - 1,
                             st) == 5  # the stride passes; the workspace size is what fails
    small = m.vc_shape(1, 1, 10, 128)
    assert L.vc_smooth_group(ctypes.byref(small), ctypes.byref(ok), ctypes.byref(ok),
                             ctypes.byref(m.vc_group_params(11, 1, 0, 0)), None, *[P(FAKE)] * 9, P(FAKE), ws,
                             st) == 4


def test_smooth_group_noalloc_validation(vc):
    # the allocation-free grouping: the same argument checks, and shapes whose
    # scratch need exceeds the static array are refused with VC_ERR_SCRATCH;
    # every case here returns before any HIP call
    L, m = vc.lib(), vc
    P = ctypes.c_void_p
    st = ctypes.c_void_p(0)
    ok = m.vc_bshd(FAKE, 256 * 2 * 128, 2 * 128, 128)
    sh = _shape()

    def call(shape, p, prep=None, ptrs=None):
        ptrs = [FAKE] * 9 if ptrs is None else ptrs
        return L.vc_smooth_group_noalloc(ctypes.byref(shape), ctypes.byref(ok), ctypes.byref(ok), ctypes.byref(p),
                                         ctypes.byref(prep) if prep is not None else None, *[P(x) for x in ptrs], st)
    assert call(sh, m.vc_group_params(0, 4, 0, 0)) == 4                      # k < 1
    assert call(sh, m.vc_group_params(64, 0, 0, 0)) == 4                     # iters < 1
    assert call(sh, m.vc_group_params(64, 4, 0, 3)) == 4                     # exclusive flags
    assert call(sh, m.vc_group_params(64, 4, 0, 2), ptrs=[FAKE, FAKE, None] + [FAKE] * 6) == 1
    assert call(m.vc_shape(1, 2, 256, 96), m.vc_group_params(8, 4, 0, 0)) == 2
    # the headline shapes fit the static scratch; 200 heads of 84672 tokens do not
    need = m.vc_smooth_group_noalloc_bytes
    lim = 16 << 20
    assert 0 < need(1, 40, 75600, 128, 64) <= lim and 0 < need(1, 48, 84672, 128, 64) <= lim
    assert need(1, 48, 84672, 128, 64, m.VC_PREP_K_CENTER) == need(1, 48, 84672, 128, 64) + 48 * 128 * 8
    big = m.vc_shape(1, 200, 84672, 128)
    assert need(1, 200, 84672, 128, 64) > lim
    assert call(big, m.vc_group_params(64, 4, 0, 0)) == 7                    # VC_ERR_SCRATCH
    assert vc.vc_status_str(7).startswith("VC_ERR_SCRATCH")
    # the preparation is validated before the scratch is touched (RoPE without tables)
    pp = m.vc_prep_params(m.VC_PREP_ROPE, None, None, None, 0)
    assert call(sh, m.vc_group_params(64, 4, 0, 0), prep=pp) == 1


def test_prep_validation(vc):
    # vc_prep_params checks, before anything is enqueued
    L, m = vc.lib(), vc
    P = ctypes.c_void_p
    sh = _shape()
    ok = m.vc_bshd(FAKE, 256 * 2 * 128, 2 * 128, 128)
    none = m.vc_bshd(None, 0, 0, 0)
    st = ctypes.c_void_p(0)
    need = L.vc_prep_workspace_size(ctypes.byref(sh))
    assert need == 1 * 2 * 128 * 8
    assert L.vc_prep_workspace_size(ctypes.byref(m.vc_shape(1, 2, 256, 96))) == 0

    def q_k(pp, with_k=True):
        kk = ok if with_k else none
        return L.vc_quantize(ctypes.byref(sh), 0.0, ctypes.byref(pp), ctypes.byref(ok), ctypes.byref(kk),
                             ctypes.byref(none), P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, None, st)
    assert q_k(m.vc_prep_params(8, None, None, None, 0)) == 4                        # unknown flag
    assert q_k(m.vc_prep_params(m.VC_PREP_ROPE, None, FAKE, None, 0)) == 1           # no cos table
    assert q_k(m.vc_prep_params(m.VC_PREP_ROPE, FAKE + 4, FAKE, None, 0)) == 3       # misaligned table
    assert q_k(m.vc_prep_params(m.VC_PREP_K_CENTER, None, None, None, 0)) == 1       # no workspace
    assert q_k(m.vc_prep_params(m.VC_PREP_K_CENTER, None, None, FAKE + 4, need)) == 3
    assert q_k(m.vc_prep_params(m.VC_PREP_K_CENTER, None, None, FAKE, need - 8)) == 5
    # without K the centring workspace is not needed: validation passes up to
    # the output checks (here a missing v is fine and q/k pointers are FAKE),
    # so only check that the prep block itself is accepted by a NULL q8
    pp = m.vc_prep_params(m.VC_PREP_K_CENTER, None, None, None, 0)
    assert L.vc_quantize(ctypes.byref(sh), 0.0, ctypes.byref(pp), ctypes.byref(ok), ctypes.byref(none),
                         ctypes.byref(none), None, None, None, None, None, None, st) == 1


def test_attn_validation(vc):
    L, m = vc.lib(), vc
    P = ctypes.c_void_p
    sh = _shape()
    st = ctypes.c_void_p(0)
    o = m.vc_bshd_out(FAKE, 256 * 2 * 128, 2 * 128, 128)
    good = m.vc_attn_params(0.0, 2, 0)
    args = [P(FAKE)] * 6
    ob = ctypes.byref(o)
    assert L.vc_attn_fwd(ctypes.byref(sh), None, *args, None, None, ob, st) == 1
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(good), P(FAKE), None, *[P(FAKE)] * 4, None, None,
                         ob, st) == 1
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(m.vc_attn_params(0.0, -1, 0)), *args, None, None,
                         ob, st) == 4
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(m.vc_attn_params(-1.0, 2, 0)), *args, None, None,
                         ob, st) == 4
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(m.vc_attn_params(0.0, 2, 8)), *args, None, None,
                         ob, st) == 4
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(good), P(FAKE + 4), *[P(FAKE)] * 5, None, None,
                         ob, st) == 3
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(good), *args, None, None, None, st) == 1
    assert L.vc_attn_fwd(ctypes.byref(m.vc_shape(1, 2, 256, 32)), ctypes.byref(good), *args, None, None,
                         ob, st) == 2
    # repair rows: count in [0, S], plain path only, pointers present and aligned
    def rep(rows, k8=FAKE, ks=FAKE, v8=FAKE):
        return ctypes.byref(m.vc_repair_rows(rows, k8, ks, v8))
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(good), *args, None, rep(-1), ob, st) == 2
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(good), *args, None, rep(257), ob, st) == 2
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(good), *args, P(FAKE), rep(2), ob, st) == 4
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(good), *args, None, rep(2, k8=None), ob, st) == 1
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(good), *args, None, rep(2, v8=FAKE + 8), ob, st) == 3
    assert L.vc_attn_fwd(ctypes.byref(sh), ctypes.byref(good), *args, None, rep(2, ks=FAKE + 2), ob, st) == 3


def test_repair_validation(vc):
    L, m = vc.lib(), vc
    P = ctypes.c_void_p
    sh = _shape()
    st = ctypes.c_void_p(0)
    x = m.vc_bshd(FAKE, 256 * 2 * 128, 2 * 128, 128)
    xb = ctypes.byref(x)
    wsb = int(L.vc_repair_workspace_size(ctypes.byref(sh)))
    assert wsb == 256 + 2 * 256 * 8  # amax bits (one 256-byte line) + fp64 energies
    outs = [P(FAKE)] * 4
    assert L.vc_repair_prepare(ctypes.byref(sh), None, xb, xb, -1, *outs, P(FAKE), wsb, st) == 2
    assert L.vc_repair_prepare(ctypes.byref(sh), None, xb, xb, 257, *outs, P(FAKE), wsb, st) == 2
    assert L.vc_repair_prepare(ctypes.byref(sh), None, xb, None, 2, *outs, P(FAKE), wsb, st) == 1
    assert L.vc_repair_prepare(ctypes.byref(sh), None, xb, xb, 2, P(FAKE), None, P(FAKE), P(FAKE), P(FAKE),
                               wsb, st) == 1
    assert L.vc_repair_prepare(ctypes.byref(sh), None, xb, xb, 2, *outs, P(FAKE + 16), wsb, st) == 3
    assert L.vc_repair_prepare(ctypes.byref(sh), None, xb, xb, 2, P(FAKE + 2), *outs[1:], P(FAKE), wsb, st) == 3
    assert L.vc_repair_prepare(ctypes.byref(sh), None, xb, xb, 2, *outs, P(FAKE), wsb - 1, st) == 5
    pp = m.vc_prep_params(m.VC_PREP_K_CENTER, None, None, None, 0)  # centring without its workspace
    assert L.vc_repair_prepare(ctypes.byref(sh), ctypes.byref(pp), xb, xb, 2, *outs, P(FAKE), wsb, st) == 1
    # zero rows: validated, nothing enqueued, outputs may be NULL
    assert L.vc_repair_prepare(ctypes.byref(sh), None, xb, xb, 0, None, None, None, None, None, 0, st) == 0


def test_expcast_validation(vc):
    L = vc.lib()
    P = ctypes.c_void_p
    st = ctypes.c_void_p(0)
    assert L.vc_expcast_codes(P(FAKE), P(FAKE), P(FAKE), 10, 3, P(FAKE), st) == 2  # n % row_len
    assert L.vc_expcast_codes(P(FAKE), P(FAKE), P(FAKE), -1, 1, P(FAKE), st) == 2
    assert L.vc_expcast_codes(None, P(FAKE), P(FAKE), 4, 1, P(FAKE), st) == 1
    assert L.vc_expcast_codes(P(FAKE + 2), P(FAKE), P(FAKE), 4, 1, P(FAKE), st) == 3


def test_mxfp4_validation(vc):
    L, m = vc.lib(), vc
    P = ctypes.c_void_p
    sh = _shape()
    st = ctypes.c_void_p(0)
    x = m.vc_bshd(FAKE, 256 * 2 * 128, 2 * 128, 128)
    xb = ctypes.byref(x)
    none = m.vc_bshd(None, 0, 0, 0)
    outs = [P(FAKE)] * 6
    # K without V, perm without mu, perm without K
    assert L.vc_quantize4(ctypes.byref(sh), 0.0, xb, xb, ctypes.byref(none), None, None, *outs, st) == 1
    assert L.vc_quantize4(ctypes.byref(sh), 0.0, xb, xb, xb, P(FAKE), None, *outs, st) == 1
    assert L.vc_quantize4(ctypes.byref(sh), 0.0, xb, ctypes.byref(none), ctypes.byref(none), P(FAKE), P(FAKE),
                          *outs, st) == 1
    # bad softmax scale, misaligned outputs, a bad shape
    assert L.vc_quantize4(ctypes.byref(sh), -1.0, xb, xb, xb, None, None, *outs, st) == 4
    assert L.vc_quantize4(ctypes.byref(sh), 0.0, xb, xb, xb, None, None, P(FAKE + 8), *outs[1:], st) == 3
    assert L.vc_quantize4(ctypes.byref(sh), 0.0, xb, xb, xb, None, None, P(FAKE), P(FAKE), P(FAKE),
                          P(FAKE + 4), P(FAKE), P(FAKE), st) == 3
    assert L.vc_quantize4(ctypes.byref(m.vc_shape(1, 2, 256, 96)), 0.0, xb, xb, xb, None, None, *outs, st) == 2
    o = m.vc_bshd_out(FAKE, 256 * 2 * 128, 2 * 128, 128)
    good = m.vc_attn_params(0.0, 2, 0)
    args = [P(FAKE)] * 6
    assert L.vc_attn_fwd4(ctypes.byref(sh), None, *args, None, ctypes.byref(o), st) == 1
    assert L.vc_attn_fwd4(ctypes.byref(sh), ctypes.byref(good), P(FAKE), None, *[P(FAKE)] * 4, None,
                          ctypes.byref(o), st) == 1
    assert L.vc_attn_fwd4(ctypes.byref(sh), ctypes.byref(good), *args, P(FAKE + 8), ctypes.byref(o), st) == 3
    assert L.vc_attn_fwd4(ctypes.byref(sh), ctypes.byref(m.vc_attn_params(0.0, -1, 0)), *args, None,
                          ctypes.byref(o), st) == 4
    assert L.vc_attn_fwd4(ctypes.byref(sh), ctypes.byref(good), *args, None, None, st) == 1
