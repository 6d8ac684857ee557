"""GPU parity of Open-VC's V residual repair ([OVC] "Why V residual repair":
the top tokens by residual energy of the per-head FP8 V get a residual value
row, paired with a copy of their key, visited after all key tiles and counted
in the numerator only) against the CPU oracle, through the C ABI.

Bit-exact: the selected indices (ties to the lower index, ascending), the
repair keys' codes and power-of-two scales (plain and with the Q/K
preprocessing), the residual value codes.  Attention with repair rows:
relative L2 <= 1e-2 against the oracle's emulation with the same rows (the
tolerance of the plain path, for the same reasons), and a lower error than
without them on values with outlier tokens.
"""
import math

import numpy as np
import pytest
import torch

import expcast_ref as ER
import oracle
import vcsynth
from oracle import exact
from layouts import unpack_k, unpack_v

pytestmark = pytest.mark.gpu

REL_L2_TOL = 1e-2


@pytest.fixture(scope="module")
def vc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_fp8_attention_amd as m
    m.lib()
    return m


def _np(t):
    return t.detach().cpu().numpy()


def _rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def rope_tables(S, D, base=10000.0):
    th = np.arange(S, dtype=np.float64)[:, None] * (base ** (-2.0 * np.arange(D // 2) / D))[None, :]
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


def _check_prepare(vc, rp, kb, vb, R, D, prep=0, cs=None, sn=None):
    """Compare one vc_repair_prepare result with the oracle, head by head."""
    B, S, H = vb.shape[0], vb.shape[1], vb.shape[2]
    nrb = (R + 127) // 128
    idx = _np(rp["idx"])
    rk8, rks, rv8 = _np(rp["rk8"]), _np(rp["rk_scale"]), _np(rp["rv8"])
    for b in range(B):
        for h in range(H):
            want, _ = oracle.repair_select(vb[b, :, h], R)
            assert (idx[b, h, :R] == want).all(), (b, h)
            if prep:
                yk, _ = oracle.prep_rows(kb[b, :, h], prep, cs, sn)
            else:
                yk = oracle.bf16_bits_to_f32(kb[b, :, h]).astype(np.float32)
            kc, ks = oracle.quantize_f32_pow2(np.ascontiguousarray(yk[want]))
            got_k = unpack_k(rk8[b, h], D)
            assert (got_k[:R] == kc[:R]).all(), (b, h)
            assert (got_k[R:nrb * 128] == got_k[R - 1]).all(), (b, h)  # padding repeats the last key
            assert (rks[b, h, :nrb] == ks).all(), (b, h)
            rv = oracle.repair_rows(vb[b, :, h], want)
            assert (unpack_v(rv8[b, h].reshape(D, nrb * 128), D) == rv).all(), (b, h)


@pytest.mark.parametrize("B,S,H,D,R,v_kind", [(1, 1000, 2, 64, 5, "t3"), (1, 300, 3, 128, 130, "normal"),
                                              (2, 257, 1, 128, 257, "normal"), (1, 129, 2, 64, 1, "t3"),
                                              (1, 5000, 2, 128, 25, "t3")])
def test_repair_prepare_bitexact(vc, B, S, H, D, R, v_kind):
    print(f"case repair prepare B={B} S={S} H={H} D={D} R={R} {v_kind}", flush=True)
    q, k, v = vcsynth.random_qkv(B, S, H, D, seed=S + R, v_kind=v_kind)
    rp = vc.vc_repair_prepare(k.cuda(), v.cuda(), R)
    torch.cuda.synchronize()
    _check_prepare(vc, rp, vcsynth.bf16_bits(k), vcsynth.bf16_bits(v), R, D)


def test_repair_ties_go_to_lower_index(vc):
    # tokens copy one of 6 rows (and some are zero), so energies tie in
    # groups; R splits a group
    print("case repair ties", flush=True)
    B, S, H, D = 1, 3000, 2, 128
    g = torch.Generator().manual_seed(3)
    base = torch.randn((6, H, D), generator=g) * torch.tensor([1, 2, 4, 8, 16, 0.0])[:, None, None]
    pick = torch.randint(0, 6, (S,), generator=g)
    v = base[pick].unsqueeze(0).to(torch.bfloat16)
    k = torch.randn((B, S, H, D), generator=g).to(torch.bfloat16)
    vb = vcsynth.bf16_bits(v)
    for R in (3, 700, 2999):
        rp = vc.vc_repair_prepare(k.cuda(), v.cuda(), R)
        torch.cuda.synchronize()
        _check_prepare(vc, rp, vcsynth.bf16_bits(k), vb, R, D)


@pytest.mark.parametrize("flags", [4, 7])
def test_repair_prepare_with_prep_bitexact(vc, flags):
    print(f"case repair prepare prep={flags}", flush=True)
    B, S, H, D = 1, 700, 2, 128
    q, k, v = vcsynth.random_qkv(B, S, H, D, seed=40 + flags, v_kind="t3")
    k = (k.float() + 2.0).to(torch.bfloat16)  # a channel mean for the centring to remove
    cs, sn = rope_tables(S, D)
    prep = {"flags": flags, "rope_cos": torch.from_numpy(cs).cuda(), "rope_sin": torch.from_numpy(sn).cuda()}
    rp = vc.vc_repair_prepare(k.cuda(), v.cuda(), 9, prep=prep)
    torch.cuda.synchronize()
    _check_prepare(vc, rp, vcsynth.bf16_bits(k), vcsynth.bf16_bits(v), 9, D, flags, cs, sn)


def _attn_repair(vc, q, k, v, sm, R, **kw):
    B, S, H, D = q.shape
    qz = vc.vc_quantize(q.cuda(), k.cuda(), v.cuda(), sm_scale=sm)
    rp = vc.vc_repair_prepare(k.cuda(), v.cuda(), R)
    o = vc.vc_attn_fwd(qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], qz["v8"], qz["v_scale"], None, S=S,
                       repair=rp, **kw)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


# S = 1000: the ragged key tile falls inside the steady loop for the first
# query pairs (followed by repair tiles) and first for the later ones;
# R = 130: two repair tiles, the second ragged; S = 100: one key tile.
@pytest.mark.parametrize("S,D,rho,seq", [(1000, 128, 0.005, False), (1000, 64, 0.13, False), (1000, 128, 0.02, True),
                                         (100, 128, 0.05, False), (1024, 128, 0.01, False)])
def test_attn_with_repair_parity(vc, S, D, rho, seq):
    print(f"case attn repair S={S} D={D} rho={rho} seq={seq}", flush=True)
    B, H = 1, 2
    q, k, v = vcsynth.random_qkv(B, S, H, D, seed=S + D, v_kind="t3")
    q = (q.float() * 1.5).to(torch.bfloat16)
    sm = float(np.float32(1 / math.sqrt(D)))
    R = oracle.repair_count(S, rho)
    assert R == vc.repair_count(S, rho) and R >= 1
    og = _attn_repair(vc, q, k, v, sm, R, sequential=seq)
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    for h in range(H):
        res = oracle.pipeline_head(qb, kb, vb, 0, h, vsmooth=False, sm_scale=sm, repair_rho=rho,
                                   flags=oracle.SEQUENTIAL if seq else 0)
        emu = oracle.bf16_bits_to_f32(res["out_bf16"])
        err = _rel_l2(og[0, :, h], emu)
        assert err <= REL_L2_TOL, (h, err)
        # every element, repair keys included (tests/expcast_ref.py)
        st = ER.check_rows(og[0, :, h], res, S, np.arange(S), 2, seq)
        print(f"  head {h}: rel-L2 {err:.2e}, row max {st['row_rel_l2_max']:.2e}, "
              f"bit-identical {st['bit_identical']:.4f}", flush=True)


def test_attn_repair_lowers_error(vc):
    # the tiny workload's V has 1% outlier tokens; repairing 2% of the tokens
    # brings the output closer to exact attention, on every head
    print("case attn repair tiny", flush=True)
    q, k, v = vcsynth.make_qkv("tiny")
    B, S, H, D = q.shape
    sm = float(np.float32(1 / math.sqrt(D)))
    o0 = _attn_repair(vc, q, k, v, sm, 0)
    o1 = _attn_repair(vc, q, k, v, sm, oracle.repair_count(S, 0.02))
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    for h in range(H):
        ref = exact.attention_rows(exact.to_f64(qb[0, :, h]), exact.to_f64(kb[0, :, h]), exact.to_f64(vb[0, :, h]),
                                   sm)
        e0, e1 = _rel_l2(o0[0, :, h], ref), _rel_l2(o1[0, :, h], ref)
        assert e1 < e0, (h, e0, e1)


def test_zero_repair_rows_change_nothing(vc):
    print("case attn repair R=0", flush=True)
    B, S, H, D = 1, 700, 2, 128
    q, k, v = vcsynth.random_qkv(B, S, H, D, seed=9)
    qz = vc.vc_quantize(q.cuda(), k.cuda(), v.cuda())
    rp = vc.vc_repair_prepare(k.cuda(), v.cuda(), 0)
    args = (qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], qz["v8"], qz["v_scale"], None)
    o1 = vc.vc_attn_fwd(*args, S=S, repair=rp)
    o0 = vc.vc_attn_fwd(*args, S=S)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1)
