"""CPU oracle for the VC-Attention hot path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP library
in ``bit_fp8_attention_amd`` and never imports it.

Two parts:

* ``exact``: fp64 attention by its plain definition
  (VC-Attention paper, §3.1: S = QK^T/sqrt(d), P = softmax(S), O = PV) plus the
  closed forms of §3.3 and Appendix D used as pins.
* ``vc_oracle.c`` (wrapped here): a step-by-step emulation of the quantised
  pipeline -- E4M3 codec, per-block / per-head quantisers, the V-Smooth
  grouping (k-means, argsort, block means, residual codes) and the ExpCast
  attention recurrence, one query row at a time.

Tensors cross this wrapper as numpy arrays; bf16 values travel as their
uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libvc_oracle.so")
_lib = None

SEQUENTIAL = 1
EXACT_EXP = 2
DEFER4 = 4  # 4-bit path: rises within the headroom of 8 left unapplied

# preprocessing flags (vco_prep_rows)
PREP_ROPE = 1
PREP_HADAMARD = 2
PREP_CENTER = 4


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (IEEE fp32, no contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
               "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f32, u64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_uint64
        L.vco_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.vco_e4m3_decode.restype = ctypes.c_double
        L.vco_e4m3_encode.argtypes = [f32]
        L.vco_e4m3_encode.restype = ctypes.c_uint8
        L.vco_e4m3_encode_array.argtypes = [P, i64, P]
        L.vco_f32_to_bf16.argtypes = [f32]
        L.vco_f32_to_bf16.restype = ctypes.c_uint16
        L.vco_expcast_codes.argtypes = [P, P, P, i64, i32, P]
        L.vco_expcast_code_u.argtypes = [ctypes.c_double, ctypes.c_double]
        L.vco_expcast_code_u.restype = ctypes.c_int
        L.vco_quantize_blocks_pow2.argtypes = [P, i64, i32, i32, f32, P, P]
        L.vco_prep_rows.argtypes = [P, i64, i32, i32, i32, P, P, P, P]
        L.vco_quantize_f32_blocks_pow2.argtypes = [P, i32, i32, f32, P, P]
        L.vco_quantize_v_head.argtypes = [P, i64, i32, i32, P]
        L.vco_quantize_v_head.restype = f32
        L.vco_splitmix64_stream.argtypes = [u64, i32, P]
        L.vco_forgy_indices.argtypes = [u64, i32, i32, i32, i32, i32, P]
        L.vco_kmeans.argtypes = [P, i64, i32, i32, i32, i32, u64, i32, i32, i32, i32, P, P]
        L.vco_argsort_labels.argtypes = [P, i32, i32, P]
        L.vco_smooth_apply.argtypes = [P, i64, P, i64, i32, i32, P, P, P, P, P, P, P]
        L.vco_tile_order.argtypes = [i32, i32, i32, i32, P]
        L.vco_attn_emulate_rows.argtypes = [P, P, P, P, P, P, P, i32, i32, f32, i32, i32, P, i32, P, P, P, i32,
                                            P, P, P]
        L.vco_repair_select.argtypes = [P, i64, i32, i32, i32, P, P]
        L.vco_repair_rows.argtypes = [P, i64, i32, i32, P, i32, P]
        L.vco_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.vco_e2m1_decode.restype = ctypes.c_double
        L.vco_e2m1_encode.argtypes = [f32]
        L.vco_e2m1_encode.restype = ctypes.c_uint8
        L.vco_mx_block_exp.argtypes = [f32]
        L.vco_mx_block_exp.restype = ctypes.c_int
        L.vco_mxfp4_rows.argtypes = [P, i32, i32, f32, P, P]
        L.vco_mxfp4_cols.argtypes = [P, i32, i32, P, P]
        L.vco_attn4_emulate_rows.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, P, i32, P, P, P]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


# --------------------------------------------------------------------------- #
# scalars and small codecs
# --------------------------------------------------------------------------- #

def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    return (x.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    L = lib()
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    return np.array([L.vco_f32_to_bf16(float(v)) for v in flat], dtype=np.uint16).reshape(np.shape(x))


def e4m3_decode(codes) -> np.ndarray:
    L = lib()
    table = np.array([L.vco_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().vco_e4m3_encode_array(_p(x), x.size, _p(out))
    return out


def expcast_codes(x: np.ndarray, a: np.ndarray, b: np.ndarray, row_len: int) -> np.ndarray:
    """codes[i] = clip_[0,120](RNE(fmaf(a[row], x[i], b[row]))), row = i // row_len."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    a = np.ascontiguousarray(a, dtype=np.float32).ravel()
    b = np.ascontiguousarray(b, dtype=np.float32).ravel()
    assert x.size == a.size * row_len == b.size * row_len
    out = np.empty(x.size, dtype=np.uint8)
    lib().vco_expcast_codes(_p(x), _p(a), _p(b), x.size, row_len, _p(out))
    return out


def expcast_code_u(u: float, beta: float = -0.35) -> int:
    return int(lib().vco_expcast_code_u(float(u), float(beta)))


# --------------------------------------------------------------------------- #
# quantisers ([B,S,H,D] bf16 bits in, per-head outputs)
# --------------------------------------------------------------------------- #

def _head(x: np.ndarray, b: int, h: int) -> np.ndarray:
    return np.ascontiguousarray(x[b, :, h, :])


def q_prefactor(sm_scale: float) -> float:
    """G = 8 fl32(sm_scale * fl32(log2 e)), the factor Q carries into its codes."""
    c1 = np.float32(np.float32(sm_scale) * np.float32(1.4426950408889634))
    return float(np.float32(8.0) * c1)


def quantize_qk(x: np.ndarray, pre: float = 1.0):
    """Per-128-token-block E4M3 with power-of-two scales, after an fp32
    multiply by `pre` (G for Q, 1 for K).  x: uint16 [B,S,H,D].
    Returns codes uint8 [B,H,S_pad,D], scales fp32 [B,H,nblk]."""
    B, S, H, D = x.shape
    nblk = (S + 127) // 128
    codes = np.zeros((B, H, nblk * 128, D), np.uint8)
    scales = np.zeros((B, H, nblk), np.float32)
    L = lib()
    for b in range(B):
        for h in range(H):
            xh = _head(x, b, h)
            c = np.zeros((nblk * 128, D), np.uint8)
            s = np.zeros(nblk, np.float32)
            L.vco_quantize_blocks_pow2(_p(xh), D, S, D, float(pre), _p(c), _p(s))
            codes[b, h], scales[b, h] = c, s
    return codes, scales


def prep_rows(x_head: np.ndarray, flags: int, rope_cos=None, rope_sin=None):
    """One head's rows x_head uint16 (bf16 bits) [S,D], token position = row:
    RoPE (PREP_ROPE, tables fp32 [S, D/2]), centring (PREP_CENTER), then the
    unnormalised Hadamard rotation (PREP_HADAMARD).  Returns (y fp32 [S,D],
    channel mean fp32 [D] or None)."""
    x_head = np.ascontiguousarray(x_head, np.uint16)
    S, D = x_head.shape
    y = np.zeros((S, D), np.float32)
    mean = np.zeros(D, np.float32)
    cp = sp = None
    if flags & PREP_ROPE:
        rope_cos = np.ascontiguousarray(rope_cos, np.float32)
        rope_sin = np.ascontiguousarray(rope_sin, np.float32)
        assert rope_cos.shape == (S, D // 2) and rope_sin.shape == (S, D // 2)
        cp, sp = _p(rope_cos), _p(rope_sin)
    lib().vco_prep_rows(_p(x_head), D, S, D, int(flags), cp, sp, _p(y), _p(mean))
    return y, (mean if flags & PREP_CENTER else None)


def quantize_f32_pow2(y: np.ndarray, pre: float = 1.0):
    """Power-of-two block quantiser of one head's fp32 rows y [S,D] (after an
    fp32 multiply by pre).  Returns codes uint8 [S_pad,D], scales fp32 [nblk]."""
    y = np.ascontiguousarray(y, np.float32)
    S, D = y.shape
    nblk = (S + 127) // 128
    c = np.zeros((nblk * 128, D), np.uint8)
    sc = np.zeros(nblk, np.float32)
    lib().vco_quantize_f32_blocks_pow2(_p(y), S, D, float(pre), _p(c), _p(sc))
    return c, sc


def q_prefactor_prep(sm_scale: float, D: int, flags: int) -> float:
    """Q's pre-factor: G, divided by D (exactly) when the rotation is on."""
    G = q_prefactor(sm_scale)
    return float(np.float32(G) / np.float32(D)) if flags & PREP_HADAMARD else G


def quantize_v(x: np.ndarray):
    """Per-head E4M3, key-contiguous.  Returns codes uint8 [B,H,D,S_pad],
    scales fp32 [B,H,D] (the head's scale repeated over channels)."""
    B, S, H, D = x.shape
    S_pad = (S + 127) // 128 * 128
    codes = np.zeros((B, H, D, S_pad), np.uint8)
    scales = np.zeros((B, H, D), np.float32)
    L = lib()
    for b in range(B):
        for h in range(H):
            xh = _head(x, b, h)
            c = np.zeros((D, S_pad), np.uint8)
            s = L.vco_quantize_v_head(_p(xh), D, S, D, _p(c))
            codes[b, h], scales[b, h, :] = c, s
    return codes, scales


# --------------------------------------------------------------------------- #
# V-Smooth grouping
# --------------------------------------------------------------------------- #

def splitmix64_stream(seed: int, n: int) -> list:
    out = np.zeros(n, np.uint64)
    lib().vco_splitmix64_stream(seed, n, _p(out))
    return [int(x) for x in out]


def forgy_indices(seed: int, b: int, h: int, H: int, S: int, k: int) -> np.ndarray:
    out = np.zeros(k, np.int32)
    lib().vco_forgy_indices(seed, b, h, H, S, k, _p(out))
    return out


def kmeans_head(v_head: np.ndarray, k: int, iters: int, seed: int, b: int, h: int, H: int,
                init: np.ndarray | None = None):
    """v_head: uint16 [S,D].  Returns (labels int32 [S], centroids fp32 [k,D])."""
    v_head = np.ascontiguousarray(v_head)
    S, D = v_head.shape
    cent = np.zeros((k, D), np.float32) if init is None else np.ascontiguousarray(init, np.float32).copy()
    labels = np.zeros(S, np.int32)
    lib().vco_kmeans(_p(v_head), D, S, D, k, iters, seed, b, h, H, 0 if init is None else 1, _p(cent),
                     _p(labels))
    return labels, cent


def argsort_labels(labels: np.ndarray, k: int) -> np.ndarray:
    labels = np.ascontiguousarray(labels, np.int32)
    perm = np.zeros(labels.size, np.int32)
    lib().vco_argsort_labels(_p(labels), labels.size, k, _p(perm))
    return perm


def smooth_apply_head(k_head: np.ndarray, v_head: np.ndarray, perm: np.ndarray):
    k_head, v_head = np.ascontiguousarray(k_head), np.ascontiguousarray(v_head)
    perm = np.ascontiguousarray(perm, np.int32)
    S, D = v_head.shape
    nblk = (S + 127) // 128
    out = dict(
        mu_bf16=np.zeros((nblk, D), np.uint16),
        mu_scaled=np.zeros((nblk, D), np.float32),
        r_codes=np.zeros((D, nblk * 128), np.uint8),
        r_scale=np.zeros(D, np.float32),
        k_codes=np.zeros((nblk * 128, D), np.uint8),
        k_scale=np.zeros(nblk, np.float32),
    )
    lib().vco_smooth_apply(_p(k_head), D, _p(v_head), D, S, D, _p(perm), _p(out["mu_bf16"]),
                           _p(out["mu_scaled"]), _p(out["r_codes"]), _p(out["r_scale"]),
                           _p(out["k_codes"]), _p(out["k_scale"]))
    return out


def smooth_group(k: np.ndarray, v: np.ndarray, nclust: int, iters: int, seed: int, heads=None):
    """The whole grouping step for the listed (b, h) heads (default: all).
    k, v: uint16 [B,S,H,D].  Returns {(b,h): dict(labels, centroids, perm, ...)}."""
    B, S, H, D = v.shape
    heads = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    res = {}
    for (b, h) in heads:
        labels, cent = kmeans_head(_head(v, b, h), nclust, iters, seed, b, h, H)
        perm = argsort_labels(labels, nclust)
        d = smooth_apply_head(_head(k, b, h), _head(v, b, h), perm)
        d.update(labels=labels, centroids=cent, perm=perm)
        res[(b, h)] = d
    return res


# --------------------------------------------------------------------------- #
# attention emulation
# --------------------------------------------------------------------------- #

def tile_order(qt: int, nblk: int, window: int = 2, sequential: bool = False) -> np.ndarray:
    out = np.zeros(nblk, np.int32)
    lib().vco_tile_order(qt, nblk, window, 1 if sequential else 0, _p(out))
    return out


def repair_count(S: int, rho: float) -> int:
    """Number of repair rows for rho (the fraction of tokens): ceil(rho S)."""
    return 0 if rho <= 0 else min(S, int(np.ceil(rho * S - 1e-9)))


def repair_select(v_head: np.ndarray, R: int):
    """One head's V (uint16 bf16 bits [S,D]): residual energies (fp64 [S]) and
    the R selected token indices (int32, ascending)."""
    v_head = np.ascontiguousarray(v_head, np.uint16)
    S, D = v_head.shape
    idx = np.zeros(max(R, 1), np.int32)
    e = np.zeros(S, np.float64)
    lib().vco_repair_select(_p(v_head), D, S, D, int(R), _p(idx), _p(e))
    return idx[:R], e


def repair_rows(v_head: np.ndarray, idx: np.ndarray):
    """Residual codes of the selected tokens, key-contiguous uint8 [D, R_pad]."""
    v_head = np.ascontiguousarray(v_head, np.uint16)
    S, D = v_head.shape
    idx = np.ascontiguousarray(idx, np.int32)
    R = idx.size
    out = np.zeros((D, (R + 127) // 128 * 128), np.uint8)
    lib().vco_repair_rows(_p(v_head), D, S, D, _p(idx), R, _p(out))
    return out


def attn_emulate_rows(q_codes, q_scale, k_codes, k_scale, v_codes_t, v_scale, mu_scaled, S, c1,
                      rows, window=2, flags=0, repair=None):
    """One head.  q_codes/k_codes [S_pad,D], v_codes_t [D,S_pad], scales as
    produced by the quantisers, mu_scaled [nblk,D] or None.  c1 is the
    log2-domain score per unit of q_scale * k_scale * (Qhat . Khat): 1/8 when
    Q carries G (quantize_qk(q, q_prefactor(sm_scale))).
    repair: None or dict(rk_codes [R_pad,D], rk_scale [nrb], rv_codes_t [D,R_pad], R),
    tiles of repair rows visited after all others, numerator only.
    Returns (out_f32 [n,D], out_bf16 bits [n,D], stats [n,2])."""
    q_codes = np.ascontiguousarray(q_codes, np.uint8)
    k_codes = np.ascontiguousarray(k_codes, np.uint8)
    v_codes_t = np.ascontiguousarray(v_codes_t, np.uint8)
    q_scale = np.ascontiguousarray(q_scale, np.float32)
    k_scale = np.ascontiguousarray(k_scale, np.float32)
    v_scale = np.ascontiguousarray(v_scale, np.float32)
    D = q_codes.shape[1]
    rows = np.ascontiguousarray(rows, np.int32)
    n = rows.size
    of = np.zeros((n, D), np.float32)
    ob = np.zeros((n, D), np.uint16)
    st = np.zeros((n, 2), np.float64)
    mu_p = None
    if mu_scaled is not None:
        mu_scaled = np.ascontiguousarray(mu_scaled, np.float32)
        mu_p = _p(mu_scaled)
    rk = rks = rv = None
    R = 0
    if repair is not None and repair["R"] > 0:
        rk = np.ascontiguousarray(repair["rk_codes"], np.uint8)
        rks = np.ascontiguousarray(repair["rk_scale"], np.float32)
        rv = np.ascontiguousarray(repair["rv_codes_t"], np.uint8)
        R = int(repair["R"])
    lib().vco_attn_emulate_rows(_p(q_codes), _p(q_scale), _p(k_codes), _p(k_scale), _p(v_codes_t),
                                _p(v_scale), mu_p, S, D, float(c1), window, flags, _p(rows), n,
                                None if rk is None else _p(rk), None if rks is None else _p(rks),
                                None if rv is None else _p(rv), R, _p(of), _p(ob), _p(st))
    return of, ob, st


def pipeline_head(q, k, v, b, h, *, vsmooth, nclust=64, iters=4, seed=0, sm_scale=None, rows=None,
                  window=2, flags=0, prep=0, rope_cos=None, rope_sin=None, repair_rho=0.0):
    """Full oracle pipeline for one head from bf16 inputs [B,S,H,D]:
    quantise, (group,) emulate the listed query rows.  Returns a dict."""
    B, S, H, D = q.shape
    sm_scale = 1.0 / np.sqrt(D) if sm_scale is None else sm_scale
    rows = np.arange(S) if rows is None else np.asarray(rows)
    qh = _head(q, b, h)
    nblk = (S + 127) // 128
    if prep:
        # Q: RoPE and rotation (no centring); K: all three, before the gather
        yq, _ = prep_rows(qh, prep & ~PREP_CENTER, rope_cos, rope_sin)
        qc, qs = quantize_f32_pow2(yq, q_prefactor_prep(sm_scale, D, prep))
        yk, kmean = prep_rows(_head(k, b, h), prep, rope_cos, rope_sin)
    else:
        qc = np.zeros((nblk * 128, D), np.uint8)
        qs = np.zeros(nblk, np.float32)
        lib().vco_quantize_blocks_pow2(_p(qh), D, S, D, q_prefactor(sm_scale), _p(qc), _p(qs))
    out = dict(q_codes=qc, q_scale=qs)
    if vsmooth:
        labels, cent = kmeans_head(_head(v, b, h), nclust, iters, seed, b, h, H)
        perm = argsort_labels(labels, nclust)
        g = smooth_apply_head(_head(k, b, h), _head(v, b, h), perm)
        if prep:  # K' = prepared K gathered by pi
            g["k_codes"], g["k_scale"] = quantize_f32_pow2(yk[perm])
        out.update(g, labels=labels, centroids=cent, perm=perm)
        kc, ks, vc, vs, mu = g["k_codes"], g["k_scale"], g["r_codes"], g["r_scale"], g["mu_scaled"]
    else:
        kh = _head(k, b, h)
        if prep:
            kc, ks = quantize_f32_pow2(yk)
        else:
            kc = np.zeros((nblk * 128, D), np.uint8)
            ks = np.zeros(nblk, np.float32)
            lib().vco_quantize_blocks_pow2(_p(kh), D, S, D, 1.0, _p(kc), _p(ks))
        vc = np.zeros((D, nblk * 128), np.uint8)
        s = lib().vco_quantize_v_head(_p(_head(v, b, h)), D, S, D, _p(vc))
        vs = np.full(D, s, np.float32)
        mu = None
        out.update(k_codes=kc, k_scale=ks, v_codes=vc, v_scale=vs)
    repair = None
    R = 0 if vsmooth else repair_count(S, repair_rho)
    if R > 0:
        # [OVC] "Why V residual repair": the top R tokens by residual energy;
        # their keys (prepared alike) quantised as blocks of their own
        idx, energy = repair_select(_head(v, b, h), R)
        yk_all = yk if prep else bf16_bits_to_f32(_head(k, b, h)).astype(np.float32)
        rk, rks = quantize_f32_pow2(np.ascontiguousarray(yk_all[idx]))
        rv = repair_rows(_head(v, b, h), idx)
        repair = dict(rk_codes=rk, rk_scale=rks, rv_codes_t=rv, R=R)
        out.update(repair_idx=idx, repair_energy=energy, repair_k_codes=rk, repair_k_scale=rks,
                   repair_v_codes=rv)
    of, ob, st = attn_emulate_rows(qc, qs, kc, ks, vc, vs, mu, S, 0.125, rows, window, flags, repair)
    out.update(out_f32=of, out_bf16=ob, stats=st, rows=rows)
    return out


# --------------------------------------------------------------------------- #
# 4-bit path (MXFP4: E2M1 elements, one power-of-two scale per 32)
# --------------------------------------------------------------------------- #

def e2m1_decode(codes) -> np.ndarray:
    """Values of E2M1 codes (low 4 bits of each entry)."""
    table = np.array([lib().vco_e2m1_decode(c) for c in range(16)], np.float64)
    return table[np.asarray(codes).astype(np.int64) & 15]


def e2m1_encode(x) -> np.ndarray:
    L = lib()
    x = np.asarray(x, np.float32)
    return np.array([L.vco_e2m1_encode(float(v)) for v in x.ravel()], np.uint8).reshape(x.shape)


def mx_block_exp(amax: float) -> int:
    return int(lib().vco_mx_block_exp(float(amax)))


def q4_prefactor(sm_scale: float) -> float:
    """fl32(sm_scale * fl32(log2 e)): Q's factor on the 4-bit path, so the
    matrix cores emit scores in log2 units."""
    return float(np.float32(np.float32(sm_scale) * np.float32(1.4426950408889634)))


def mxfp4_rows(y: np.ndarray, pre: float = 1.0):
    """fp32 rows [S, D] (times pre) in blocks of 32 channels.  Returns codes
    uint8 [S_pad, D] (one code per byte; rows >= S zero) and exponents int32
    [S_pad, D/32] (rows >= S zero)."""
    y = np.ascontiguousarray(y, np.float32)
    S, D = y.shape
    S_pad = (S + 127) // 128 * 128
    codes = np.zeros((S_pad, D), np.uint8)
    exps = np.zeros((S_pad, D // 32), np.int32)
    lib().vco_mxfp4_rows(_p(y), S, D, float(pre), _p(codes), _p(exps))
    return codes, exps


def mxfp4_cols(x: np.ndarray):
    """fp32 [S, D] (rows = keys) in blocks of 32 keys per channel.  Returns
    codes uint8 [D, S_pad] and exponents int32 [D, S_pad/32]."""
    x = np.ascontiguousarray(x, np.float32)
    S, D = x.shape
    S_pad = (S + 127) // 128 * 128
    codes = np.zeros((D, S_pad), np.uint8)
    exps = np.zeros((D, S_pad // 32), np.int32)
    lib().vco_mxfp4_cols(_p(x), S, D, _p(codes), _p(exps))
    return codes, exps


def attn4_emulate_rows(q_codes, q_exps, k_codes, k_exps, v_codes_t, v_exps, mu, S, rows, window=2, flags=0):
    """One head of the 4-bit path (see vco_attn4_emulate_rows).  mu: fp32
    [nblk, D] block means or None.  Returns (out_f32, out_bf16, stats)."""
    arrs = [np.ascontiguousarray(a, t) for a, t in ((q_codes, np.uint8), (q_exps, np.int32), (k_codes, np.uint8),
                                                  (k_exps, np.int32), (v_codes_t, np.uint8), (v_exps, np.int32))]
    D = arrs[0].shape[1]
    rows = np.ascontiguousarray(rows, np.int32)
    n = rows.size
    of = np.zeros((n, D), np.float32)
    ob = np.zeros((n, D), np.uint16)
    st = np.zeros((n, 2), np.float64)
    mup = None
    if mu is not None:
        mu = np.ascontiguousarray(mu, np.float32)
        mup = _p(mu)
    lib().vco_attn4_emulate_rows(*[_p(a) for a in arrs], mup, S, D, window, flags, _p(rows), n, _p(of), _p(ob),
                                 _p(st))
    return of, ob, st


def pipeline4_head(q, k, v, b, h, *, vsmooth, nclust=64, iters=4, seed=0, sm_scale=None, rows=None, window=2,
                   flags=0):
    """The 4-bit pipeline for one head from bf16 inputs [B,S,H,D]: Q (times
    q4_prefactor) and K in MXFP4 row blocks; V, or with V-Smooth the residual
    R = fl32(V' - mu) of the grouping (same k-means, pi and block means as the
    8-bit path), in MXFP4 key blocks; then the emulation of the listed rows."""
    B, S, H, D = q.shape
    sm_scale = 1.0 / np.sqrt(D) if sm_scale is None else sm_scale
    rows = np.arange(S) if rows is None else np.asarray(rows)
    qc, qe = mxfp4_rows(bf16_bits_to_f32(_head(q, b, h)), q4_prefactor(sm_scale))
    out = dict(q_codes=qc, q_exps=qe)
    kh, vh = _head(k, b, h), _head(v, b, h)
    mu = None
    if vsmooth:
        labels, cent = kmeans_head(vh, nclust, iters, seed, b, h, H)
        perm = argsort_labels(labels, nclust)
        g = smooth_apply_head(kh, vh, perm)
        mu = bf16_bits_to_f32(g["mu_bf16"]).astype(np.float32)
        vp = bf16_bits_to_f32(vh[perm]).astype(np.float32)
        blk = np.arange(S) // 128
        r = (vp - mu[blk]).astype(np.float32)  # one fp32 subtraction per element
        kc, ke = mxfp4_rows(bf16_bits_to_f32(kh[perm]))
        vc, ve = mxfp4_cols(r)
        out.update(labels=labels, perm=perm, mu=mu, residual=r)
    else:
        kc, ke = mxfp4_rows(bf16_bits_to_f32(kh))
        vc, ve = mxfp4_cols(bf16_bits_to_f32(vh))
    out.update(k_codes=kc, k_exps=ke, v_codes=vc, v_exps=ve)
    of, ob, st = attn4_emulate_rows(qc, qe, kc, ke, vc, ve, mu, S, rows, window, flags)
    out.update(out_f32=of, out_bf16=ob, stats=st, rows=rows)
    return out
