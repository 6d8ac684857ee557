"""GPU parity of the fused Q/K preprocessing ([VC] §3.4 and Appendix B:
rotary embedding, key centring, QK Hadamard rotation ahead of the
quantisers) against the CPU oracle, through the C ABI.

Bit-exact: vc_quantize's Q and K codes and scales, and vc_smooth_group's K'
codes and scales, for every combination of the three steps.  Attention with
preprocessing: relative L2 <= 1e-2 against the quantised-pipeline emulation
of the same steps, and close to exact attention on the rotary-embedded
operands.
"""
import math

import numpy as np
import pytest
import torch

import expcast_ref as ER
import oracle
import vcsynth
from oracle import exact
from layouts import k_matches, unpack_k

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


def rope_tables(S, D, base=10000.0):
    """1-D rotary tables: angle of pair i at position p = p * base^(-2i/D)."""
    th = np.arange(S, dtype=np.float64)[:, None] * (base ** (-2.0 * np.arange(D // 2) / D))[None, :]
    return np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


def _prep_dict(vc, flags, cs, sn):
    return {"flags": flags, "rope_cos": torch.from_numpy(cs).cuda(), "rope_sin": torch.from_numpy(sn).cuda()}


def _qkv(B, S, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, S, H, D), generator=g)
    k = torch.randn((B, S, H, D), generator=g) + torch.randn((D,), generator=g) * 3  # channel bias
    v = torch.randn((B, S, H, D), generator=g)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


@pytest.mark.parametrize("flags", [1, 2, 4, 7])
@pytest.mark.parametrize("S,D", [(300, 128), (257, 64)])
def test_quantize_prep_bitexact(vc, flags, S, D):
    print(f"case quantize prep flags={flags} S={S} D={D}", flush=True)
    B, H = 1, 2
    q, k, v = _qkv(B, S, H, D, seed=S + flags)
    cs, sn = rope_tables(S, D)
    sm = float(np.float32(1 / math.sqrt(D)))
    out = vc.vc_quantize(q.cuda(), k.cuda(), v.cuda(), sm_scale=sm, prep=_prep_dict(vc, flags, cs, sn))
    torch.cuda.synchronize()
    qb, kb = vcsynth.bf16_bits(q), vcsynth.bf16_bits(k)
    for h in range(H):
        yq, _ = oracle.prep_rows(qb[0, :, h], flags & ~oracle.PREP_CENTER, cs, sn)
        qc, qs = oracle.quantize_f32_pow2(yq, oracle.q_prefactor_prep(sm, D, flags))
        assert (_np(out["q8"])[0, h] == qc).all(), h
        assert (_np(out["q_scale"])[0, h] == qs).all(), h
        yk, _ = oracle.prep_rows(kb[0, :, h], flags, cs, sn)
        kc, ks = oracle.quantize_f32_pow2(yk)
        assert k_matches(_np(out["k8"])[0, h], D, kc, S), h
        assert (_np(out["k_scale"])[0, h] == ks).all(), h


@pytest.mark.parametrize("flags", [4, 7])
def test_smooth_group_prep_k_bitexact(vc, flags):
    print(f"case smooth_group prep flags={flags}", flush=True)
    B, S, H, D = 1, 600, 2, 128
    q, k, v = _qkv(B, S, H, D, seed=11 + flags)
    cs, sn = rope_tables(S, D)
    g = vc.vc_smooth_group(k.cuda(), v.cuda(), 16, 3, 5, prep=_prep_dict(vc, flags, cs, sn))
    torch.cuda.synchronize()
    kb = vcsynth.bf16_bits(k)
    perm = _np(g["perm"])
    for h in range(H):
        yk, _ = oracle.prep_rows(kb[0, :, h], flags, cs, sn)
        kc, ks = oracle.quantize_f32_pow2(yk[perm[0, h]])  # keys prepared at their own positions, then gathered
        assert (unpack_k(_np(g["k8"])[0, h], D) == kc).all(), h
        assert (_np(g["k_scale"])[0, h] == ks).all(), h


@pytest.mark.parametrize("vsmooth", [False, True])
def test_attn_with_prep_parity(vc, vsmooth):
    print(f"case attn prep=7 vsmooth={vsmooth}", flush=True)
    B, S, H, D = 1, 900, 2, 128
    sm = float(np.float32(1 / math.sqrt(D)))
    q, k, v = _qkv(B, S, H, D, seed=21)
    q = (q.float() * 2).to(torch.bfloat16)  # sharper rows
    cs, sn = rope_tables(S, D)
    pd = _prep_dict(vc, 7, cs, sn)
    if vsmooth:
        qz = vc.vc_quantize(q.cuda(), sm_scale=sm, prep=pd)
        g = vc.vc_smooth_group(k.cuda(), v.cuda(), 16, 3, 7, prep=pd)
        o = vc.vc_attn_fwd(qz["q8"], qz["q_scale"], g["k8"], g["k_scale"], g["r8"], g["r_scale"], g["mu_split"], S=S)
    else:
        qz = vc.vc_quantize(q.cuda(), k.cuda(), v.cuda(), sm_scale=sm, prep=pd)
        o = vc.vc_attn_fwd(qz["q8"], qz["q_scale"], qz["k8"], qz["k_scale"], qz["v8"], qz["v_scale"], None, S=S)
    torch.cuda.synchronize()
    og = o.float().cpu().numpy()
    qb, kb, vb = (vcsynth.bf16_bits(x) for x in (q, k, v))
    for h in range(H):
        res = oracle.pipeline_head(qb, kb, vb, 0, h, vsmooth=vsmooth, nclust=16, iters=3, seed=7, sm_scale=sm,
                                   prep=7, rope_cos=cs, rope_sin=sn)
        emu = oracle.bf16_bits_to_f32(res["out_bf16"])
        err = np.linalg.norm(og[0, :, h] - emu) / np.linalg.norm(emu)
        assert err <= REL_L2_TOL, (h, err)
        # every element (tests/expcast_ref.py): the scores come from the prepared codes
        st = ER.check_rows(og[0, :, h], res, S, np.arange(S), 2, vsmooth=vsmooth)
        print(f"  head {h}: rel-L2 {err:.2e}, row max {st['row_rel_l2_max']:.2e}, "
              f"bit-identical {st['bit_identical']:.4f}", flush=True)
        # and close to exact attention on the rotary-embedded operands
        qr, _ = oracle.prep_rows(qb[0, :, h], oracle.PREP_ROPE, cs, sn)
        kr, _ = oracle.prep_rows(kb[0, :, h], oracle.PREP_ROPE, cs, sn)
        ref = exact.attention_rows(qr.astype(np.float64), kr.astype(np.float64),
                                   oracle.bf16_bits_to_f32(vb[0, :, h]).astype(np.float64), sm)
        assert np.linalg.norm(og[0, :, h] - ref) / np.linalg.norm(ref) < 0.15, h
