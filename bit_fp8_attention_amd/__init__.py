"""bit_fp8_attention_amd -- VC-Attention's FP8 attention hot path on MI355X.

Thin ctypes binding over ``libvcattn.so`` (the C ABI in ``include/vc_attn.h``).
Every step of the path runs in the library's HIP kernels; this module only
marshals arguments: it takes torch tensors for device memory and the current
HIP stream, allocates outputs when the caller does not pass them, and raises
on a non-OK status.  There is no CPU fallback: if the library is missing or
no GPU is present, calls fail loudly.

Entry points (same names as the C ABI): vc_abi_version, vc_status_str,
vc_quantize, vc_smooth_group_workspace_size, vc_smooth_group,
vc_smooth_group_noalloc_bytes, vc_smooth_group_noalloc,
vc_repair_workspace_size, vc_repair_prepare, vc_attn_fwd, vc_quantize4,
vc_attn_fwd4, vc_pack_v_bf16, vc_attn_fwd_bf16, vc_expcast_codes; and vsmooth_schedule, the host-side rule
for which denoising steps group, reuse or run plain, and repair_count, the
number of repair rows for a fraction rho of the tokens.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvcattn.so")
_lib = None

VC_OK = 0
VC_ATTN_SEQUENTIAL = 1
VC_GROUP_WARM_START = 1
VC_GROUP_REUSE_PERM = 2
ABI_VERSION = 7


class VcError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {vc_status_str(status)} (status {status})")
        self.status = status


class vc_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("S", ctypes.c_int32), ("D", ctypes.c_int32)]


class vc_bshd(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sB", ctypes.c_int64), ("sS", ctypes.c_int64), ("sH", ctypes.c_int64)]


class vc_bshd_out(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("sB", ctypes.c_int64), ("sS", ctypes.c_int64), ("sH", ctypes.c_int64)]


class vc_group_params(ctypes.Structure):
    _fields_ = [("clusters", ctypes.c_int32), ("iters", ctypes.c_int32), ("seed", ctypes.c_uint64),
                ("flags", ctypes.c_uint32)]


VC_PREP_ROPE = 1
VC_PREP_HADAMARD = 2
VC_PREP_K_CENTER = 4


class vc_prep_params(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("rope_cos", ctypes.c_void_p), ("rope_sin", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class vc_attn_params(ctypes.Structure):
    _fields_ = [("sm_scale", ctypes.c_float), ("window", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class vc_repair_rows(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("k8", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v8", ctypes.c_void_p)]


def lib():
    """Load libvcattn.so (built by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        L.vc_abi_version.restype = i32
        L.vc_status_str.argtypes = [i32]
        L.vc_status_str.restype = ctypes.c_char_p
        L.vc_quantize.argtypes = [P, f32] + [P] * 11
        L.vc_prep_workspace_size.argtypes = [P]
        L.vc_prep_workspace_size.restype = sz
        L.vc_quantize.restype = i32
        L.vc_smooth_group_workspace_size.argtypes = [P, i32]
        L.vc_smooth_group_workspace_size.restype = sz
        L.vc_smooth_group.argtypes = [P] * 15 + [sz, P]
        L.vc_smooth_group.restype = i32
        L.vc_smooth_group_noalloc_bytes.argtypes = [P, i32, ctypes.c_uint32]
        L.vc_smooth_group_noalloc_bytes.restype = sz
        L.vc_smooth_group_noalloc.argtypes = [P] * 15
        L.vc_smooth_group_noalloc.restype = i32
        L.vc_repair_workspace_size.argtypes = [P]
        L.vc_repair_workspace_size.restype = sz
        L.vc_repair_prepare.argtypes = [P, P, P, P, i32, P, P, P, P, P, sz, P]
        L.vc_repair_prepare.restype = i32
        L.vc_attn_fwd.argtypes = [P] * 12
        L.vc_attn_fwd.restype = i32
        L.vc_quantize4.argtypes = [P, f32] + [P] * 12
        L.vc_quantize4.restype = i32
        L.vc_attn_fwd4.argtypes = [P] * 11
        L.vc_attn_fwd4.restype = i32
        L.vc_pack_v_bf16.argtypes = [P] * 4
        L.vc_pack_v_bf16.restype = i32
        L.vc_attn_fwd_bf16.argtypes = [P] * 7
        L.vc_attn_fwd_bf16.restype = i32
        L.vc_expcast_codes.argtypes = [P, P, P, i64, i32, P, P]
        L.vc_expcast_codes.restype = i32
        _lib = L
    return _lib


def vc_abi_version() -> int:
    return int(lib().vc_abi_version())


def vc_status_str(status: int) -> str:
    return lib().vc_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != VC_OK:
        raise VcError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _shape_of(x: torch.Tensor) -> vc_shape:
    B, S, H, D = x.shape
    return vc_shape(B, H, S, D)


def _bshd(x: torch.Tensor | None) -> vc_bshd:
    if x is None:
        return vc_bshd(None, 0, 0, 0)
    assert x.dtype == torch.bfloat16 and x.dim() == 4 and x.stride(3) == 1, "bf16 [B,S,H,D], D contiguous"
    return vc_bshd(x.data_ptr(), x.stride(0), x.stride(1), x.stride(2))


def _bshd_out(x: torch.Tensor) -> vc_bshd_out:
    assert x.dtype == torch.bfloat16 and x.dim() == 4 and x.stride(3) == 1, "bf16 [B,S,H,D], D contiguous"
    return vc_bshd_out(x.data_ptr(), x.stride(0), x.stride(1), x.stride(2))


def nblk_of(S: int) -> int:
    return (S + 127) // 128


# --------------------------------------------------------------------------- #
# vc_quantize
# --------------------------------------------------------------------------- #

def _prep(prep, ref, with_k: bool):
    """A vc_prep_params for prep = None, or a dict with keys flags, and with
    VC_PREP_ROPE rope_cos / rope_sin (fp32 [S, D/2] device tensors); the
    centring workspace is allocated here when needed (or taken from
    prep["workspace"])."""
    if not prep or not prep.get("flags"):
        return None, None
    flags = int(prep["flags"])
    cs, sn = prep.get("rope_cos"), prep.get("rope_sin")
    for t in (cs, sn):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("rope tables must be contiguous fp32 [S, D/2]")
    ws = prep.get("workspace")
    if with_k and (flags & VC_PREP_K_CENTER) and ws is None:
        sh = _shape_of(ref)
        ws = torch.empty(max(int(lib().vc_prep_workspace_size(ctypes.byref(sh))), 8), dtype=torch.uint8,
                         device=ref.device)
    pp = vc_prep_params(flags, _ptr(cs), _ptr(sn), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size())
    return pp, ws


def vc_quantize(q=None, k=None, v=None, *, sm_scale: float = 0.0, prep=None, out=None):
    """FP8 operands.  q, k, v: bf16 [B,S,H,D] (any may be None); sm_scale is
    the softmax scale the attention will use (0: 1/sqrt(D)), folded into q8;
    prep: None or {"flags": VC_PREP_*, "rope_cos": ..., "rope_sin": ...}.
    Returns dict with q8, q_scale, k8, k_scale, v8, v_scale (see vc_attn.h)."""
    ref = next(x for x in (q, k, v) if x is not None)
    sh = _shape_of(ref)
    B, H, S, D = sh.B, sh.H, sh.S, sh.D
    nb = nblk_of(S)
    dev = ref.device
    o = dict(out or {})
    if q is not None:
        o.setdefault("q8", torch.empty((B, H, nb * 128, D), dtype=torch.uint8, device=dev))
        o.setdefault("q_scale", torch.empty((B, H, nb), dtype=torch.float32, device=dev))
    if k is not None:
        o.setdefault("k8", torch.empty((B, H, nb * 128, D), dtype=torch.uint8, device=dev))
        o.setdefault("k_scale", torch.empty((B, H, nb), dtype=torch.float32, device=dev))
    if v is not None:
        o.setdefault("v8", torch.empty((B, H, D, nb * 128), dtype=torch.uint8, device=dev))
        o.setdefault("v_scale", torch.empty((B, H, D), dtype=torch.float32, device=dev))
    qd, kd, vd = _bshd(q), _bshd(k), _bshd(v)
    pp, _ws = _prep(prep, ref, k is not None)
    st = lib().vc_quantize(ctypes.byref(sh), float(sm_scale), ctypes.byref(pp) if pp is not None else None,
                           ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd),
                           _ptr(o.get("q8")), _ptr(o.get("q_scale")), _ptr(o.get("k8")), _ptr(o.get("k_scale")),
                           _ptr(o.get("v8")), _ptr(o.get("v_scale")), _stream())
    _check(st, "vc_quantize")
    return o


# --------------------------------------------------------------------------- #
# vc_smooth_group
# --------------------------------------------------------------------------- #

def vc_smooth_group_workspace_size(B: int, H: int, S: int, D: int, clusters: int) -> int:
    sh = vc_shape(B, H, S, D)
    return int(lib().vc_smooth_group_workspace_size(ctypes.byref(sh), clusters))


def vc_smooth_group(k, v, clusters: int, iters: int, seed: int, *, workspace=None, out=None, warm_start=None,
                    reuse_perm=None, prep=None):
    """V-Smooth grouping.  k, v: bf16 [B,S,H,D].  Returns dict with centroids,
    labels, perm, k8, k_scale, r8, r_scale, mu_bf16, mu_split (int32 storage
    of the uint32 pairs bf16(m) | bf16(m - bf16(m)) << 16 of each scaled block
    mean m).

    warm_start: fp32 [B,H,clusters,D] centroids to start k-means from
    (VC_GROUP_WARM_START); it is copied into the returned centroids.
    reuse_perm: int32 [B,H,S] permutation of an earlier call
    (VC_GROUP_REUSE_PERM): no k-means, no sort; only the gather, block means
    and residual codes run on k, v; centroids and labels are not produced."""
    return _smooth_group(k, v, clusters, iters, seed, workspace, out, warm_start, reuse_perm, prep, noalloc=False)


def vc_smooth_group_noalloc_bytes(B: int, H: int, S: int, D: int, clusters: int, prep_flags: int = 0) -> int:
    sh = vc_shape(B, H, S, D)
    return int(lib().vc_smooth_group_noalloc_bytes(ctypes.byref(sh), clusters, prep_flags))


def vc_smooth_group_noalloc(k, v, clusters: int, iters: int, seed: int, *, out=None, warm_start=None,
                            reuse_perm=None, prep=None):
    """vc_smooth_group through the C entry point that allocates nothing: its
    workspace (and the centring sums) live in the library's static per-GPU
    scratch.  Outputs missing from `out` are allocated here, by the binding,
    as torch tensors; pass them all for a call that allocates nothing."""
    return _smooth_group(k, v, clusters, iters, seed, None, out, warm_start, reuse_perm, prep, noalloc=True)


def _smooth_group(k, v, clusters, iters, seed, workspace, out, warm_start, reuse_perm, prep, noalloc):
    if warm_start is not None and reuse_perm is not None:
        raise ValueError("warm_start and reuse_perm exclude each other")
    sh = _shape_of(v)
    B, H, S, D = sh.B, sh.H, sh.S, sh.D
    nb = nblk_of(S)
    dev = v.device
    o = dict(out or {})
    flags = 0
    if reuse_perm is None:
        o.setdefault("centroids", torch.empty((B, H, clusters, D), dtype=torch.float32, device=dev))
        o.setdefault("labels", torch.empty((B, H, S), dtype=torch.int32, device=dev))
        o.setdefault("perm", torch.empty((B, H, S), dtype=torch.int32, device=dev))
        if warm_start is not None:
            if tuple(warm_start.shape) != (B, H, clusters, D) or warm_start.dtype != torch.float32:
                raise ValueError("warm_start must be fp32 [B,H,clusters,D]")
            if warm_start.data_ptr() != o["centroids"].data_ptr():
                o["centroids"].copy_(warm_start)
            flags = VC_GROUP_WARM_START
    else:
        if tuple(reuse_perm.shape) != (B, H, S) or reuse_perm.dtype != torch.int32 or not reuse_perm.is_contiguous():
            raise ValueError("reuse_perm must be contiguous int32 [B,H,S]")
        o["perm"] = reuse_perm
        o.pop("centroids", None)
        o.pop("labels", None)
        flags = VC_GROUP_REUSE_PERM
    o.setdefault("k8", torch.empty((B, H, nb * 128, D), dtype=torch.uint8, device=dev))
    o.setdefault("k_scale", torch.empty((B, H, nb), dtype=torch.float32, device=dev))
    o.setdefault("r8", torch.empty((B, H, D, nb * 128), dtype=torch.uint8, device=dev))
    o.setdefault("r_scale", torch.empty((B, H, D), dtype=torch.float32, device=dev))
    o.setdefault("mu_bf16", torch.empty((B, H, nb, D), dtype=torch.int16, device=dev))
    o.setdefault("mu_split", torch.empty((B, H, nb, D), dtype=torch.int32, device=dev))
    p = vc_group_params(clusters, iters, seed, flags)
    kd, vd = _bshd(k), _bshd(v)
    outs = (_ptr(o.get("centroids")), _ptr(o.get("labels")), _ptr(o["perm"]), _ptr(o["k8"]), _ptr(o["k_scale"]),
            _ptr(o["r8"]), _ptr(o["r_scale"]), _ptr(o["mu_bf16"]), _ptr(o["mu_split"]))
    if noalloc:
        pp = None
        if prep and prep.get("flags"):
            pp = vc_prep_params(int(prep["flags"]), _ptr(prep.get("rope_cos")), _ptr(prep.get("rope_sin")), None, 0)
        st = lib().vc_smooth_group_noalloc(ctypes.byref(sh), ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(p),
                                           ctypes.byref(pp) if pp is not None else None, *outs, _stream())
        _check(st, "vc_smooth_group_noalloc")
        return o
    wsb = vc_smooth_group_workspace_size(B, H, S, D, clusters)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    pp, _ws = _prep(prep, k, True)
    st = lib().vc_smooth_group(ctypes.byref(sh), ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(p),
                               ctypes.byref(pp) if pp is not None else None, *outs, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream())
    _check(st, "vc_smooth_group")
    return o


def vsmooth_schedule(n_steps: int, step: int, reuse: int = 4) -> str:
    """What the V-Smooth schedule does at denoising step `step` of `n_steps`
    ([VC] §3.4 and Appendix A): grouping and demeaning run on the first
    ceil(n_steps / 4) steps; inside that window the permutation is computed
    at every `reuse`-th step ("group") and reused in between ("reuse"); the
    later steps run plain FP8 ExpCast attention ("plain")."""
    if n_steps < 1 or not 0 <= step < n_steps or reuse < 1:
        raise ValueError("need n_steps >= 1, 0 <= step < n_steps, reuse >= 1")
    window = -(-n_steps // 4)
    if step >= window:
        return "plain"
    return "group" if step % reuse == 0 else "reuse"


# --------------------------------------------------------------------------- #
# vc_attn_fwd
# --------------------------------------------------------------------------- #

def vc_attn_fwd(q8, q_scale, k8, k_scale, v8, v_scale, mu_split=None, *, S: int, out=None, window: int = 2,
                sequential: bool = False, repair=None):
    """FP8 ExpCast attention.  Codes and scales as produced by vc_quantize /
    vc_smooth_group (the softmax scale rides in q8: pass it to vc_quantize);
    S is the token count; repair: None or the dict of vc_repair_prepare
    (plain path only).  Returns bf16 [B,S,H,D]."""
    B, H, S_pad, D = q8.shape
    assert S_pad == nblk_of(S) * 128
    sh = vc_shape(B, H, S, D)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=q8.device)
    p = vc_attn_params(0.0, window, VC_ATTN_SEQUENTIAL if sequential else 0)
    od = _bshd_out(out)
    rp = None
    if repair is not None and repair["rows"] > 0:
        rp = vc_repair_rows(int(repair["rows"]), _ptr(repair["rk8"]), _ptr(repair["rk_scale"]), _ptr(repair["rv8"]))
    st = lib().vc_attn_fwd(ctypes.byref(sh), ctypes.byref(p), _ptr(q8), _ptr(q_scale), _ptr(k8), _ptr(k_scale),
                           _ptr(v8), _ptr(v_scale), _ptr(mu_split), ctypes.byref(rp) if rp is not None else None,
                           ctypes.byref(od), _stream())
    _check(st, "vc_attn_fwd")
    return out


# --------------------------------------------------------------------------- #
# vc_repair_prepare
# --------------------------------------------------------------------------- #

def repair_count(S: int, rho: float) -> int:
    """Repair rows for a fraction rho of the S tokens: ceil(rho S), at most S
    ([OVC] "Why V residual repair" uses rho = 0.5%)."""
    if rho <= 0:
        return 0
    return min(S, math.ceil(rho * S - 1e-9))


def vc_repair_workspace_size(B: int, H: int, S: int, D: int) -> int:
    sh = vc_shape(B, H, S, D)
    return int(lib().vc_repair_workspace_size(ctypes.byref(sh)))


def vc_repair_prepare(k, v, rows: int, *, prep=None, workspace=None, out=None):
    """V residual repair rows.  k, v: bf16 [B,S,H,D]; rows: R in [0, S];
    prep: K's preprocessing as given to vc_quantize.  Returns dict with rows,
    idx int32 [B,H,R], rk8 uint8 [B,H,nrb*128,D] (packed K tiles), rk_scale
    fp32 [B,H,nrb], rv8 uint8 [B,H,nrb,D,128] (packed V tiles)."""
    sh = _shape_of(v)
    B, H, S, D = sh.B, sh.H, sh.S, sh.D
    R = int(rows)
    nrb = (R + 127) // 128
    dev = v.device
    o = dict(out or {})
    o["rows"] = R
    o.setdefault("idx", torch.empty((B, H, max(R, 1)), dtype=torch.int32, device=dev))
    o.setdefault("rk8", torch.empty((B, H, max(nrb, 1) * 128, D), dtype=torch.uint8, device=dev))
    o.setdefault("rk_scale", torch.empty((B, H, max(nrb, 1)), dtype=torch.float32, device=dev))
    o.setdefault("rv8", torch.empty((B, H, max(nrb, 1), D, 128), dtype=torch.uint8, device=dev))
    wsb = vc_repair_workspace_size(B, H, S, D)
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    kd, vd = _bshd(k), _bshd(v)
    pp, _ws = _prep(prep, k, True)
    st = lib().vc_repair_prepare(ctypes.byref(sh), ctypes.byref(pp) if pp is not None else None, ctypes.byref(kd),
                                 ctypes.byref(vd), R, _ptr(o["idx"]), _ptr(o["rk8"]), _ptr(o["rk_scale"]),
                                 _ptr(o["rv8"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream())
    _check(st, "vc_repair_prepare")
    return o


# --------------------------------------------------------------------------- #
# the 4-bit path (MXFP4)
# --------------------------------------------------------------------------- #

def vc_quantize4(q=None, k=None, v=None, *, sm_scale: float = 0.0, perm=None, mu_bf16=None, out=None):
    """MXFP4 operands (see vc_attn.h).  q, k, v: bf16 [B,S,H,D] (q or k/v may
    be None); perm (int32 [B,H,S]) and mu_bf16 ([B,H,nblk,D]) from
    vc_smooth_group for V-Smooth.  Returns dict with q4, q4_scale, k4,
    k4_scale, v4, v4_scale."""
    ref = next(x for x in (q, k, v) if x is not None)
    sh = _shape_of(ref)
    B, H, S, D = sh.B, sh.H, sh.S, sh.D
    nb = nblk_of(S)
    dev = ref.device
    o = dict(out or {})
    if q is not None:
        o.setdefault("q4", torch.empty((B, H, nb * 128, D // 2), dtype=torch.uint8, device=dev))
        o.setdefault("q4_scale", torch.empty((B, H, nb * 128, D // 32), dtype=torch.uint8, device=dev))
    if k is not None:
        o.setdefault("k4", torch.empty((B, H, nb, 128, D // 2), dtype=torch.uint8, device=dev))
        o.setdefault("k4_scale", torch.empty((B, H, nb, 512), dtype=torch.uint8, device=dev))
        o.setdefault("v4", torch.empty((B, H, nb, D, 64), dtype=torch.uint8, device=dev))
        o.setdefault("v4_scale", torch.empty((B, H, nb, 512), dtype=torch.uint8, device=dev))
    qd, kd, vd = _bshd(q), _bshd(k), _bshd(v)
    st = lib().vc_quantize4(ctypes.byref(sh), float(sm_scale), ctypes.byref(qd), ctypes.byref(kd), ctypes.byref(vd),
                            _ptr(perm), _ptr(mu_bf16), _ptr(o.get("q4")), _ptr(o.get("q4_scale")),
                            _ptr(o.get("k4")), _ptr(o.get("k4_scale")), _ptr(o.get("v4")), _ptr(o.get("v4_scale")),
                            _stream())
    _check(st, "vc_quantize4")
    return o


def vc_attn_fwd4(q4, q4_scale, k4, k4_scale, v4, v4_scale, mu_bf16=None, *, S: int, out=None, window: int = 2,
                 sequential: bool = False):
    """4-bit attention on vc_quantize4's operands.  Returns bf16 [B,S,H,D]."""
    B, H, S_pad, D2 = q4.shape
    D = 2 * D2
    assert S_pad == nblk_of(S) * 128
    sh = vc_shape(B, H, S, D)
    if out is None:
        out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=q4.device)
    p = vc_attn_params(0.0, window, VC_ATTN_SEQUENTIAL if sequential else 0)
    od = _bshd_out(out)
    st = lib().vc_attn_fwd4(ctypes.byref(sh), ctypes.byref(p), _ptr(q4), _ptr(q4_scale), _ptr(k4), _ptr(k4_scale),
                            _ptr(v4), _ptr(v4_scale), _ptr(mu_bf16), ctypes.byref(od), _stream())
    _check(st, "vc_attn_fwd4")
    return out


def vc_pack_v_bf16(v, *, out=None):
    sh = _shape_of(v)
    nb = nblk_of(sh.S)
    if out is None:
        out = torch.empty((sh.B, sh.H, sh.D, nb * 128), dtype=torch.bfloat16, device=v.device)
    vd = _bshd(v)
    st = lib().vc_pack_v_bf16(ctypes.byref(sh), ctypes.byref(vd), _ptr(out), _stream())
    _check(st, "vc_pack_v_bf16")
    return out


def vc_attn_fwd_bf16(q, k, vt, *, out=None, sm_scale: float = 0.0, window: int = 2, sequential: bool = False):
    sh = _shape_of(q)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    p = vc_attn_params(sm_scale, window, VC_ATTN_SEQUENTIAL if sequential else 0)
    qd, kd, od = _bshd(q), _bshd(k), _bshd_out(out)
    st = lib().vc_attn_fwd_bf16(ctypes.byref(sh), ctypes.byref(p), ctypes.byref(qd), ctypes.byref(kd), _ptr(vt),
                                ctypes.byref(od), _stream())
    _check(st, "vc_attn_fwd_bf16")
    return out


def vc_expcast_codes(x, a, b, row_len: int, *, out=None):
    """codes[i] = min(120, RNE_clamp0(fma(a[r], x[i], b[r]))), r = i // row_len."""
    n = x.numel()
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=x.device)
    st = lib().vc_expcast_codes(_ptr(x), _ptr(a), _ptr(b), n, row_len, _ptr(out), _stream())
    _check(st, "vc_expcast_codes")
    return out


def default_sm_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)
