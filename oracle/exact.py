"""fp64 parts of the oracle -- TEST INFRASTRUCTURE ONLY.

* Exact attention, VC-Attention paper §3.1: S = Q K^T * scale, P = softmax(S),
  O = P V, computed in fp64 from the bf16 inputs.  Two independent
  formulations (two-pass, and the blockwise online recurrence of Eq. 1) so
  that each can pin the other.
* Closed forms of §3.3 and Appendix D (Eqs. 9-15): Mitchell's error e(f), the
  decoded-to-exact ratio r(f), the total-variation bound, and the per-row
  check of Proposition 3.1.
"""
from __future__ import annotations

import numpy as np

from . import bf16_bits_to_f32, e4m3_decode

LOG2E = 1.4426950408889634


def to_f64(x_bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(x_bits).astype(np.float64)


# --------------------------------------------------------------------------- #
# exact attention
# --------------------------------------------------------------------------- #

def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float, rows=None):
    """Two-pass softmax attention in fp64 for one head.
    q, k, v: float64 [S, D] (already widened).  Returns [n, D]."""
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    s = (q[rows] @ k.T) * sm_scale
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    return (w @ v) / w.sum(axis=1, keepdims=True)


def attention_rows_online(q, k, v, sm_scale, rows=None, block=128):
    """The online recurrence of Eq. 1 over key blocks, fp64."""
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    n, D = len(rows), v.shape[1]
    m = np.full((n, 1), -np.inf)
    l = np.zeros((n, 1))
    A = np.zeros((n, D))
    for k0 in range(0, k.shape[0], block):
        s = (q[rows] @ k[k0:k0 + block].T) * sm_scale
        mn = np.maximum(m, s.max(axis=1, keepdims=True))
        alpha = np.exp(m - mn)
        p = np.exp(s - mn)
        A = alpha * A + p @ v[k0:k0 + block]
        l = alpha * l + p.sum(axis=1, keepdims=True)
        m = mn
    return A / l


def attention_rows_longdouble(q, k, v, sm_scale, rows=None):
    """Third formulation for tiny sizes: scalar loops in extended precision."""
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    qd, kd, vd = (np.asarray(x, np.longdouble) for x in (q, k, v))
    out = np.zeros((len(rows), v.shape[1]), np.longdouble)
    for ri, i in enumerate(rows):
        s = [sum(qd[i, d] * kd[j, d] for d in range(q.shape[1])) * np.longdouble(sm_scale)
             for j in range(k.shape[0])]
        m = max(s)
        w = [np.exp(x - m) for x in s]
        z = sum(w)
        for d in range(v.shape[1]):
            out[ri, d] = sum(w[j] * vd[j, d] for j in range(k.shape[0])) / z
    return out.astype(np.float64)


# --------------------------------------------------------------------------- #
# closed forms (§3.3, Appendix C and D)
# --------------------------------------------------------------------------- #

def mitchell_error(f):
    """Eq. 9: e(f) = 8 [f - (2^f - 1)] for f in [0, 1)."""
    f = np.asarray(f, np.float64)
    return 8.0 * (f - (np.exp2(f) - 1.0))


def ratio_r(f, beta=-0.35):
    """Eq. 10: r(f) = (1 + Round(8f + beta)/8) / 2^f, Round half-even."""
    f = np.asarray(f, np.float64)
    return (1.0 + np.round(8.0 * f + beta) / 8.0) / np.exp2(f)


def tv_bound(a: float, b: float) -> float:
    """Eq. 13: max TV over endpoint reweightings of [a, b]."""
    return (np.sqrt(b) - np.sqrt(a)) / (np.sqrt(b) + np.sqrt(a))


def tv_endpoint(q, a, b):
    """Eq. 12."""
    return q * (1 - q) * (b - a) / (a + q * (b - a))


def expcast_weights_from_u(u: np.ndarray, beta: float = -0.35) -> np.ndarray:
    """Decoded ExpCast weights of a row with log2-domain scores u <= 0,
    Eq. 7 evaluated in fp64 (round half-even), then viewed as E4M3."""
    y = 8.0 * (np.asarray(u, np.float64) + 8.0) + 56.0 + beta
    c = np.clip(np.round(y), 0, 120).astype(np.uint8)
    return e4m3_decode(c), c


def row_tv_check(u: np.ndarray, beta: float = -0.35):
    """Prop. 3.1 for one row: returns (TV, tau) with p the exact softmax of
    the scores (2^u normalised) and p_hat the normalised decoded codes;
    tau = max(p(T), p_hat(T)), T = {k : u_k < -14}."""
    u = np.asarray(u, np.float64)
    u = u - u.max()
    w = np.exp2(u)
    p = w / w.sum()
    wh, _ = expcast_weights_from_u(u, beta)
    ph = wh / wh.sum()
    T = u < -14.0
    tau = max(p[T].sum(), ph[T].sum())
    return 0.5 * np.abs(p - ph).sum(), tau


def diam2(v: np.ndarray) -> float:
    """max_{a,b} ||v_a - v_b||_2 over the rows of v (Eq. 15)."""
    v = np.asarray(v, np.float64)
    sq = (v * v).sum(axis=1)
    g = v @ v.T
    d2 = np.maximum(sq[:, None] + sq[None, :] - 2 * g, 0.0)
    return float(np.sqrt(d2.max()))
