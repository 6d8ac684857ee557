"""Pins of the oracle's Q/K block quantiser (power-of-two block scales).

The pages fix one scale per 128-token block for Q and K ([OVC] "Scheduling
around ExpCast") and leave its value open; the oracle reads it as the
smallest power of two 2^e (e >= -127) with amax <= 448 * 2^e, after an fp32
multiply of Q by G = 8 fl(sm_scale * log2 e).  Checked here against torch's
float8_e4m3fn conversion (a library routine), exact boundary cases of the
scale rule, and the zero-block rule.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _bits(x):
    return oracle.f32_to_bf16_bits(np.asarray(x, np.float32))


def _one_block(rows, pre=1.0):
    x = _bits(rows)
    c, s = oracle.quantize_qk(x[None, :, None, :], pre)
    return c[0, 0], s[0, 0], oracle.bf16_bits_to_f32(x).astype(np.float32)


@pytest.mark.parametrize("mag", [1e-30, 3e-5, 0.7, 1.0, 448.0, 5000.0, 3e30])
def test_scale_is_minimal_power_of_two(mag):
    rng = np.random.default_rng(int(abs(math.log(mag))) + 3)
    rows = rng.standard_normal((128, 64)).astype(np.float32) * np.float32(mag)
    _, s, x = _one_block(rows)
    amax = float(np.abs(x).max())
    e = math.frexp(float(s[0]))[1] - 1
    assert float(s[0]) == 2.0 ** e                       # a power of two
    assert amax <= 448.0 * 2.0 ** e                      # codes fit
    assert e == -127 or amax > 448.0 * 2.0 ** (e - 1)    # and no smaller one does


@pytest.mark.parametrize("k", [-20, 0, 3, 17])
def test_scale_boundaries(k):
    # amax exactly 448 * 2^k keeps e = k; one bf16 step above moves to k + 1
    rows = np.zeros((128, 64), np.float32)
    rows[5, 7] = 448.0 * 2.0 ** k
    _, s, _ = _one_block(rows)
    assert s[0] == np.float32(2.0 ** k)
    rows[5, 7] = np.float32(448.0 * 2.0 ** k) * np.float32(1 + 2 ** -7)  # next bf16 value
    _, s, _ = _one_block(rows)
    assert s[0] == np.float32(2.0 ** (k + 1))


@pytest.mark.parametrize("pre", [1.0, 8.0 * 1.4426950408889634 / math.sqrt(128), 0.3])
def test_codes_match_torch_float8(pre):
    rng = np.random.default_rng(7)
    S, D = 300, 128
    x = _bits(rng.standard_t(3, (S, D)).astype(np.float32) * 2.5)
    c, s = oracle.quantize_qk(x[None, :, None, :], pre)
    xf = oracle.bf16_bits_to_f32(x).astype(np.float32) * np.float32(pre)  # fp32 product
    for j in range((S + 127) // 128):
        blk = xf[j * 128:(j + 1) * 128]
        scaled = torch.from_numpy(blk.astype(np.float64) / float(s[0, 0, j]))  # exact: power of two
        want = scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (c[0, 0, j * 128:j * 128 + blk.shape[0]] == want).all(), j
    assert (c[0, 0, S:] == 0).all()


def test_zero_block_scale_one():
    rows = np.zeros((128, 64), np.float32)
    c, s, _ = _one_block(rows, pre=3.0)
    assert s[0] == 1.0 and (c == 0).all()


def test_q_prefactor_folds_scale_into_codes():
    # decode(code) * s ~= G x within E4M3's half-step (2^-4 relative) where
    # the scaled value is normal, for the default softmax scale
    sm = np.float32(1 / math.sqrt(128))
    G = oracle.q_prefactor(sm)
    assert G == float(np.float32(8) * np.float32(sm * np.float32(1.4426950408889634)))
    rng = np.random.default_rng(9)
    rows = rng.standard_normal((128, 128)).astype(np.float32)
    c, s, x = _one_block(rows, pre=G)
    dec = oracle.e4m3_decode(c[:128]) * float(s[0])
    ref = x.astype(np.float64) * G
    big = np.abs(ref) >= 2.0 ** -6 * float(s[0])
    assert np.all(np.abs(dec - ref)[big] <= np.abs(ref)[big] * 2.0 ** -4 + 1e-30)


# --------------------------------------------------------------------------- #
# per-head V quantiser ([VC] §3.1, X_q = s_X * Xhat; [OVC] "Scheduling around
# ExpCast": one V scale per head, V stored key-contiguous)
# --------------------------------------------------------------------------- #

def _v_head(vals):
    """quantize_v on one head: codes [D, S_pad], scale repeated over D."""
    x = _bits(vals)
    c, s = oracle.quantize_v(x[None, :, None, :])
    return c[0, 0], s[0, 0], oracle.bf16_bits_to_f32(x).astype(np.float32)


def _torch_e4m3(x64):
    return torch.from_numpy(np.asarray(x64, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("S,D,scale", [(300, 128, 2.5), (1, 64, 0.01), (129, 64, 4000.0), (1024, 128, 1e-3)])
def test_v_head_scale_and_codes_match_torch(S, D, scale):
    rng = np.random.default_rng(S + D)
    c, s, x = _v_head(rng.standard_t(3, (S, D)).astype(np.float32) * np.float32(scale))
    amax = np.float32(np.abs(x).max())             # over all S x D of the head
    assert (s == np.float32(amax / np.float32(448))).all()   # fl32(amax / 448), one value per head
    inv = np.float32(np.float32(448) / amax)       # fl32(448 / amax)
    want = _torch_e4m3(x * inv)                    # fp32 product, then torch's RNE cast
    S_pad = (S + 127) // 128 * 128
    assert c.shape == (D, S_pad)
    assert (c[:, :S] == want.T).all()              # key-contiguous: codes_t[d][token]
    assert (c[:, S:] == 0).all()                   # pad keys are code 0


def test_v_head_amax_is_over_all_channels():
    # one channel carries a x100 outlier: the head's single scale follows it,
    # so the other channels' codes are those of the outlier's scale (a
    # per-channel amax would give each channel its own scale and far larger
    # codes there)
    rng = np.random.default_rng(3)
    S, D = 500, 64
    v = rng.standard_normal((S, D)).astype(np.float32)
    v[17, 5] = 300.0
    c, s, x = _v_head(v)
    assert (s == s[0]).all() and s[0] == np.float32(np.float32(300.0) / np.float32(448))
    inv = np.float32(np.float32(448) / np.float32(300.0))
    assert (c[:, :S] == _torch_e4m3(x * inv).T).all()
    per_channel = np.stack([_torch_e4m3(x[:, d] * np.float32(448 / np.abs(x[:, d]).max())) for d in range(D)])
    assert (c[0, :S] != per_channel[0]).mean() > 0.9
    assert c[5, 17] == 0x7E  # the outlier itself maps to 448


def test_v_head_zero_scale_one():
    c, s, _ = _v_head(np.zeros((200, 64), np.float32))
    assert (s == 1.0).all() and (c == 0).all()


def test_v_head_dequantised_within_half_step():
    # s * decode(code) ~= x within E4M3's half-step where the scaled value is normal
    rng = np.random.default_rng(11)
    c, s, x = _v_head(rng.standard_normal((256, 128)).astype(np.float32) * 5)
    dec = oracle.e4m3_decode(c[:, :256]).T * float(s[0])
    ref = x.astype(np.float64)
    big = np.abs(ref) >= 2.0 ** -6 * float(s[0])
    assert np.all(np.abs(dec - ref)[big] <= np.abs(ref)[big] * 2.0 ** -4 * (1 + 1e-6))
