"""Pins for the oracle's two-tap dynamic depthwise convolution: identity and
pure-shift special cases, taps constant within a 16-channel group and equal
to the float64 matrix product W x_t (numpy), linearity in x_{t-1}."""
import numpy as np
import torch

import synth


def _x(B, L, d, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (scale * torch.randn(B, L, d, generator=g)).to(torch.bfloat16)


def test_identity_kernel(orc):
    B, L, d = 2, 5, 64
    x = _x(B, L, d, 0)
    xp = _x(B, 1, d, 1)[:, 0]
    w = torch.zeros(2 * d // 16, d, dtype=torch.bfloat16)
    base = np.stack([np.ones(d), np.zeros(d)]).astype(np.float32)
    y = orc.dynconv2(x, xp, w, base)
    np.testing.assert_array_equal(y, x.float().numpy())


def test_shift_kernel_reads_last_verified_token_first(orc):
    B, L, d = 3, 4, 32
    x = _x(B, L, d, 2)
    xp = _x(B, 1, d, 3)[:, 0]
    w = torch.zeros(2 * d // 16, d, dtype=torch.bfloat16)
    base = np.stack([np.zeros(d), np.ones(d)]).astype(np.float32)
    y = orc.dynconv2(x, xp, w, base)
    np.testing.assert_array_equal(y[:, 0], xp.float().numpy())
    np.testing.assert_array_equal(y[:, 1:], x.float().numpy()[:, :-1])
    y0 = orc.dynconv2(x, None, w, base)          # no previous token -> zeros
    np.testing.assert_array_equal(y0[:, 0], 0.0)


def test_taps_are_group_constant_and_equal_W_x(orc):
    """With no previous token and no base, y_0 = k_{0,0} . x_0 and the tap
    per channel equals (W x_0)[ch // 16]."""
    B, L, d = 2, 1, 128
    G = d // 16
    g = torch.Generator().manual_seed(4)
    x = (torch.rand(B, L, d, generator=g) + 0.5).to(torch.bfloat16)   # no zeros
    w = (0.1 * torch.randn(2 * G, d, generator=g)).to(torch.bfloat16)
    y = orc.dynconv2(x, None, w, None)
    taps = y[:, 0] / x.float().numpy()[:, 0]
    ref = x.double().numpy()[:, 0] @ w.double().numpy().T          # [B, 2G]
    for ch in range(d):
        np.testing.assert_allclose(taps[:, ch], ref[:, ch // 16], rtol=2e-6)
    # the previous-token tap uses rows G..2G-1: put x_prev = x_0 and compare
    y2 = orc.dynconv2(x, x[:, 0], w, None)
    taps2 = (y2[:, 0] - y[:, 0]) / x.float().numpy()[:, 0]
    for ch in range(d):
        np.testing.assert_allclose(taps2[:, ch], ref[:, G + ch // 16], rtol=1e-5, atol=1e-6)


def test_linear_in_previous_token(orc):
    B, L, d = 2, 3, 64
    x = _x(B, L, d, 5)
    a = _x(B, 1, d, 6)[:, 0]
    w = (0.05 * torch.randn(2 * d // 16, d, generator=torch.Generator().manual_seed(7))
         ).to(torch.bfloat16)
    base = np.stack([1 + 0.1 * np.arange(d) / d, 0.2 * np.ones(d)]).astype(np.float32)
    y0 = orc.dynconv2(x, None, w, base).astype(np.float64)
    y1 = orc.dynconv2(x, a, w, base).astype(np.float64)
    y2 = orc.dynconv2(x, (a.float() * 2).to(torch.bfloat16), w, base).astype(np.float64)
    np.testing.assert_allclose(y2[:, 0] - y0[:, 0], 2 * (y1[:, 0] - y0[:, 0]), rtol=1e-5, atol=1e-5)
    np.testing.assert_array_equal(y1[:, 1:], y0[:, 1:])   # only position 0 reads x_prev


def test_workload_site_shapes(orc):
    w = synth.scaled(synth.WORKLOADS["b32_blk16_v151936_conv"], B=2, d=64)
    x, xp, wt, bs = synth.conv_site(w, 0)
    assert x.shape == (2, 16, 64) and xp.shape == (2, 64) and wt.shape == (8, 64) and bs is None
    y = orc.dynconv2(x, xp, wt, bs)
    assert np.all(np.isfinite(y))
