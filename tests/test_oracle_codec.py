"""Pins of the oracle's E4M3 codec, bf16 rounding and ExpCast code map.

Each test checks the oracle against something other than itself: the E4M3
definition the VC-Attention paper states in §3.3, values the pages print
(tests/golden), torch's own float8_e4m3fn / bfloat16 conversions (library
routines), or exhaustive enumeration.
"""
import math

import numpy as np
import torch

import oracle
from oracle import exact


def test_e4m3_decode_closed_form():
    # VC §3.3: exponent field e, mantissa field m -> 2^(e-7)(1+m/8)
    vals = oracle.e4m3_decode(np.arange(256))
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            assert math.isnan(vals[c])
            continue
        want = (m * 2.0 ** -9) if e == 0 else 2.0 ** (e - 7) * (1 + m / 8)
        assert vals[c] == (-want if s else want), c


def test_e4m3_decode_matches_torch_float8():
    ours = oracle.e4m3_decode(np.arange(256))
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_e4m3_page_values(golden):
    g = golden("pages_constants.json")
    dec = oracle.e4m3_decode
    assert dec(g["row_max_code"]["code"]) == g["row_max_code"]["decoded"]
    assert dec(g["e4m3_max_finite"]["code"]) == g["e4m3_max_finite"]["decoded"]
    # 8e + m read as an integer is 8 log2 v + 56 + eps(m), |eps| < 1 (VC §3.3)
    for c in range(8, 127):
        v = dec(c)
        eps = c - (8 * math.log2(v) + 56)
        assert -1 < eps <= 0 + 1e-12


def test_e4m3_encode_round_trip():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    got = oracle.e4m3_encode(vals)
    assert (got == codes).all()


def test_e4m3_encode_matches_torch_on_dense_sweep():
    # every code midpoint and its fp32 neighbours, plus a dense random sweep,
    # all inside the finite range where torch's cast rounds to nearest-even
    pos = oracle.e4m3_decode(np.arange(127))
    mids = (pos[:-1] + pos[1:]) / 2
    xs = [mids.astype(np.float32)]
    xs.append(np.nextafter(mids.astype(np.float32), np.float32(np.inf)))
    xs.append(np.nextafter(mids.astype(np.float32), np.float32(-np.inf)))
    rng = np.random.default_rng(7)
    xs.append((rng.standard_normal(200000) * 10.0 ** rng.uniform(-4, 2.6, 200000)).astype(np.float32))
    x = np.concatenate(xs)
    x = np.concatenate([x, -x])
    x = x[np.abs(x) <= 448]
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (ours == ref).all(), np.flatnonzero(ours != ref)[:10]


def test_e4m3_encode_saturates():
    x = np.array([448.0, 460.0, 464.0, 500.0, 1e6, -1e6], np.float32)
    got = oracle.e4m3_encode(x)
    assert list(got) == [126, 126, 126, 126, 126, 126 | 0x80]


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-30, 30, 50000)).astype(np.float32)
    # include exact ties
    ties = ((rng.integers(0, 1 << 16, 2000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ours = oracle.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (ours == ref).all()


# --------------------------------------------------------------------------- #
# ExpCast (VC §3.3 Eq. 7)
# --------------------------------------------------------------------------- #

def test_expcast_worked_example(golden):
    g = golden("expcast_worked_example.json")
    u = g["u"]
    assert abs(8 * (u + 8) + 56 - 0.35 - g["affine_value"]) < 1e-9
    c = oracle.expcast_code_u(u)
    assert c == g["code"] == 8 * g["exponent_field"] + g["mantissa_field"]
    assert oracle.e4m3_decode(c) == g["decoded"]
    assert abs(2 ** (u + 8) - g["exp_then_cast_input"]) < 0.05
    assert oracle.e4m3_decode(oracle.e4m3_encode(np.float32(2 ** (u + 8)))) == g["exp_then_cast_decoded"]
    # the fp32 fused multiply-add form gives the same byte
    fp32 = oracle.expcast_codes(np.array([u], np.float32), np.array([8.0]), np.array([119.65]), 1)
    assert fp32[0] == g["code"]


def _grid():
    return np.arange(-16 * 1024, 1) / 1024.0  # all u in [-16, 0], step 1/1024


def test_expcast_fp32_form_equals_closed_form_on_grid():
    u = _grid()
    want = np.array([oracle.expcast_code_u(x) for x in u], np.uint8)
    got = oracle.expcast_codes(u.astype(np.float32), np.array([8.0]), np.array([119.65]), u.size)
    assert (got == want).all()


def test_expcast_vs_exp_then_cast(golden):
    g = golden("pages_constants.json")
    # on a fine grid of one doubling: same byte on ~79.6%, else one code apart
    n = 1 << 16
    u = -1.0 + (np.arange(n) + 0.5) / n
    ec = np.array([oracle.expcast_code_u(x) for x in u])
    cast = oracle.e4m3_encode(np.exp2(u + 8).astype(np.float32)).astype(int)
    share = np.mean(ec == cast)
    assert abs(share - g["same_byte_share"]["value"]) < 1e-3
    assert np.abs(ec - cast).max() <= g["max_code_error"]["value"]
    # on the grid, all u >= -14 stay within one code; relative error <= 7.5%
    u = _grid()
    u = u[u >= g["normal_range_u"]["value"]]
    ec = np.array([oracle.expcast_code_u(x) for x in u])
    cast = oracle.e4m3_encode(np.exp2(u + 8).astype(np.float32)).astype(int)
    assert np.abs(ec - cast).max() <= 1
    rel = np.abs(oracle.e4m3_decode(ec) / np.exp2(u + 8) - 1)
    assert rel.max() <= g["max_relative_error"]["value"]


def test_expcast_normal_range_and_clip_margin(golden):
    g = golden("pages_constants.json")
    # entries stay normal (code >= 8) exactly down to u = -14 (Prop. 3.1)
    assert oracle.expcast_code_u(-14.0) == 8
    assert oracle.expcast_code_u(-14.0 - 2.0 / 1024) == 8
    assert oracle.expcast_code_u(-14.1) < 8
    # the upper clip fires only 0.106 log2 units (0.074 nats) above the max
    margin = (120.5 - 119.65) / 8 - 0.0  # y = 120.5 is the first value rounding past 120
    assert abs(margin * math.log(2) - g["clip_margin_nats"]["value"]) < 1e-3
    assert oracle.expcast_code_u(margin - 1e-9) == 120
    assert oracle.expcast_code_u(0.5) == 120


def test_expcast_integer_u_is_exact():
    # 8u + 119.65 rounds to 8u + 120 for integer u, whose decode is 2^(u+8)
    for u in range(-14, 1):
        assert oracle.e4m3_decode(oracle.expcast_code_u(u)) == 2.0 ** (u + 8)


def test_beta_from_mitchell_error(golden):
    g = golden("pages_constants.json")
    f = np.linspace(0, 1, 2_000_001)
    e = exact.mitchell_error(f)
    assert abs(e.min() - g["mitchell_error_range"]["lo"]) < 1e-9
    assert abs(e.max() - g["mitchell_error_range"]["hi"]) < 1e-4
    assert abs(-e.max() / 2 - g["beta_minimax"]["value"]) < 1e-4
    # the pages settle on beta = -0.35, within 0.01 of the minimax shift
    assert abs(g["beta"]["value"] - (-e.max() / 2)) < 0.01


def test_ratio_bounds_and_tv_bound(golden):
    g = golden("pages_constants.json")
    f = np.linspace(0, 1, 4_000_001)[:-1]
    r = exact.ratio_r(f)
    lo, hi = g["ratio_bounds"]["lo"], g["ratio_bounds"]["hi"]
    assert r.min() >= lo - 5e-5 and r.max() <= hi + 5e-5
    assert abs(r.min() - lo) < 1e-3 and abs(r.max() - hi) < 1e-3
    tv = exact.tv_bound(lo, hi)
    assert tv < g["tv_bound"]["value"]
    assert 2 * tv < g["l1_bound"]["value"]
    # Eq. 12 is maximised at q* = sqrt(a)/(sqrt(a)+sqrt(b)) with value Eq. 13
    q = np.linspace(0, 1, 100001)
    qs = math.sqrt(lo) / (math.sqrt(lo) + math.sqrt(hi))
    assert abs(exact.tv_endpoint(q, lo, hi).max() - tv) < 1e-8
    assert abs(exact.tv_endpoint(qs, lo, hi) - tv) < 1e-12


def test_expcast_codes_row_broadcast():
    # the per-row a, b of the code map
    x = np.linspace(-3, 3, 12).astype(np.float32)
    a = np.array([8.0, 4.0, -1.0], np.float32)
    b = np.array([119.65, 100.0, 0.0], np.float32)
    got = oracle.expcast_codes(x, a, b, 4)
    for i in range(12):
        y = np.float32(a[i // 4]) * np.float64(x[i]) + b[i // 4]
        assert got[i] == int(min(120, max(0, np.round(y))))
