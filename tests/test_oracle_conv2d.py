"""Pins for the CPU oracle of Conv2d -> AvgPool2d -> sigmoid -> sum.

Each test checks the oracle against something other than itself: PyTorch's
own CPU operators in float64 (the pages define the method as exactly that
module chain), closed forms, the box-sum identity written independently in
numpy, brute force on tiny inputs, and invariants.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import fconv_inputs as fi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_reference(x, w, b, s):
    """PyTorch CPU float64: conv2d (stride 1, no pad) -> avg_pool2d(s) -> sigmoid -> sum([1,2,3])."""
    xt = torch.from_numpy(x.astype(np.float64))
    wt = torch.from_numpy(w.astype(np.float64))
    bt = None if b is None else torch.from_numpy(b.astype(np.float64))
    conv = F.conv2d(xt, wt, bt)
    pooled = F.avg_pool2d(conv, kernel_size=s)
    return torch.sigmoid(pooled).sum(dim=(1, 2, 3)).numpy(), pooled.numpy()


SHAPES = [
    # B, Cin, H, W, Cout, K, s
    (2, 3, 16, 16, 4, 3, 4),      # the tiny workload
    (1, 1, 7, 9, 1, 3, 2),        # non-square, ragged in both directions
    (2, 2, 11, 13, 3, 5, 3),      # K=5, s=3, ragged
    (1, 4, 10, 10, 2, 1, 1),      # 1x1 conv, no pooling
    (3, 5, 9, 12, 6, 2, 4),       # even kernel, Hc=8 (exact), Wc=11 (ragged)
    (1, 2, 6, 6, 3, 3, 4),        # Hc=4 -> PH=1
    (2, 3, 21, 17, 5, 3, 2),
]


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_torch_float64(shape):
    B, Cin, H, W, Cout, K, s = shape
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=11)
    want_out, want_pooled = torch_reference(x, w, b, s)
    out, pooled = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True)
    np.testing.assert_allclose(pooled, want_pooled, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, want_out, rtol=1e-12, atol=1e-12)


def test_bias_none_is_zero_bias():
    x, w, b = fi.conv2d_inputs(2, 3, 12, 12, 4, 3, seed=3)
    a = oracle.conv2d_pool_sigmoid_sum(x, w, None, 3)
    z = oracle.conv2d_pool_sigmoid_sum(x, w, np.zeros_like(b), 3)
    want, _ = torch_reference(x, w, None, 3)
    np.testing.assert_array_equal(a, z)
    np.testing.assert_allclose(a, want, rtol=1e-12)


def test_sizes_follow_floor_pool():
    # 382 // 4 = 95 (the page's walk-through), 253 // 3 = 84 with the last conv row dropped.
    assert oracle.conv2d_sizes(384, 384, 3, 4) == (382, 382, 95, 95)
    assert oracle.conv2d_sizes(257, 257, 5, 3) == (253, 253, 84, 84)
    assert oracle.conv2d_sizes(16, 16, 3, 4) == (14, 14, 3, 3)
    assert oracle.conv2d_sizes(5, 5, 3, 4) == (3, 3, 0, 0)
    with pytest.raises(ValueError):
        oracle.conv2d_sizes(2, 5, 3, 1)


@pytest.mark.parametrize("shape", [(2, 3, 16, 16, 4, 3, 4), (1, 16, 257, 257, 128, 5, 3)])
def test_zero_weights_zero_bias_exact(shape):
    # sigmoid(0) = 1/2 for every pooled value: out = Cout*PH*PW/2 exactly.
    B, Cin, H, W, Cout, K, s = shape
    x = fi.normal((B, Cin, H, W), 5, 0)
    w = np.zeros((Cout, Cin, K, K), np.float32)
    b = np.zeros((Cout,), np.float32)
    _, _, PH, PW = oracle.conv2d_sizes(H, W, K, s)
    out = oracle.conv2d_pool_sigmoid_sum(x, w, b, s)
    assert np.all(out == Cout * PH * PW / 2.0)


def test_zero_weights_full_shape_exact():
    # The full Conv2d workload's spatial size at B=1: 64 * 95 * 95 / 2 = 288800.
    x = fi.normal((1, 8, 384, 384), 0, 0)
    out = oracle.conv2d_pool_sigmoid_sum(x, np.zeros((64, 8, 3, 3), np.float32), np.zeros(64, np.float32), 4)
    assert out[0] == 288800.0


def test_off_by_one_in_pool_is_visible():
    # Zero weights: a pool that kept the ragged row would give 85*85 per channel, not 84*84.
    x = fi.normal((1, 2, 257, 257), 1, 0)
    out = oracle.conv2d_pool_sigmoid_sum(x, np.zeros((4, 2, 5, 5), np.float32), np.zeros(4, np.float32), 3)
    assert out[0] == 4 * 84 * 84 / 2.0 and out[0] != 4 * 85 * 85 / 2.0


def test_zero_weights_bias_only():
    Cout, s = 5, 3
    b = np.array([-2.0, -0.5, 0.0, 0.25, 3.0], np.float32)
    x = fi.normal((2, 2, 14, 11), 2, 0)
    _, _, PH, PW = oracle.conv2d_sizes(14, 11, 3, s)
    out = oracle.conv2d_pool_sigmoid_sum(x, np.zeros((Cout, 2, 3, 3), np.float32), b, s)
    want = PH * PW * sum(1.0 / (1.0 + math.exp(-float(v))) for v in b)
    np.testing.assert_allclose(out, want, rtol=1e-14)


def test_constant_input_closed_form():
    # x == v everywhere: every conv output of channel co is v*sum(w[co]) + b[co].
    B, Cin, H, W, Cout, K, s = 2, 3, 13, 10, 4, 3, 2
    v = 0.375
    _, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=7)
    x = np.full((B, Cin, H, W), v, np.float32)
    _, _, PH, PW = oracle.conv2d_sizes(H, W, K, s)
    want = PH * PW * sum(
        1.0 / (1.0 + math.exp(-(v * float(w[co].astype(np.float64).sum()) + float(b[co])))) for co in range(Cout))
    out = oracle.conv2d_pool_sigmoid_sum(x, w, b, s)
    np.testing.assert_allclose(out, want, rtol=1e-13)


def test_delta_input_pooled_map():
    # x = e(ic0, y0, x0), b = 0: A[co,ph,pw] = (1/s^2) * sum over the window
    # offsets (dy,dx) of w[co, ic0, y0-ph*s-dy, x0-pw*s-dx] where that tap exists.
    B, Cin, H, W, Cout, K, s = 1, 2, 12, 11, 3, 3, 3
    _, w, _ = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=9)
    _, _, PH, PW = oracle.conv2d_sizes(H, W, K, s)
    for (ic0, y0, x0) in [(0, 0, 0), (1, 5, 4), (0, 11, 10), (1, 8, 0), (0, 7, 9)]:
        x = np.zeros((B, Cin, H, W), np.float32)
        x[0, ic0, y0, x0] = 1.0
        _, pooled = oracle.conv2d_pool_sigmoid_sum(x, w, None, s, want_pooled=True)
        want = np.zeros((Cout, PH, PW))
        for co in range(Cout):
            for ph in range(PH):
                for pw in range(PW):
                    acc = 0.0
                    for dy in range(s):
                        for dx in range(s):
                            ky, kx = y0 - ph * s - dy, x0 - pw * s - dx
                            if 0 <= ky < K and 0 <= kx < K:
                                acc += float(w[co, ic0, ky, kx])
                    want[co, ph, pw] = acc / (s * s)
        np.testing.assert_allclose(pooled[0], want, rtol=0, atol=1e-15)


def box_sum_pooled(x, w, b, s):
    """Independent formula: pooling commutes with the convolution.

    A[co,ph,pw] = b[co] + (1/s^2) * sum_{ic,ky,kx} w[co,ic,ky,kx] * S[ic, ph*s+ky, pw*s+kx]
    where S[ic,y,x] = sum_{dy,dx<s} x[ic, y+dy, x+dx]  (numpy, float64).
    """
    x = x.astype(np.float64)
    w = w.astype(np.float64)
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    Hc, Wc = H - K + 1, W - K + 1
    PH, PW = Hc // s, Wc // s
    S = np.zeros((B, Cin, H - s + 1, W - s + 1))
    for dy in range(s):
        for dx in range(s):
            S += x[:, :, dy:dy + H - s + 1, dx:dx + W - s + 1]
    A = np.zeros((B, Cout, PH, PW))
    for ky in range(K):
        for kx in range(K):
            patch = S[:, :, ky:ky + PH * s:s, kx:kx + PW * s:s]  # [B,Cin,PH,PW]
            A += np.einsum("oi,bipq->bopq", w[:, :, ky, kx], patch)
    A /= s * s
    if b is not None:
        A += b.astype(np.float64)[None, :, None, None]
    return A


@pytest.mark.parametrize("shape", [(2, 3, 16, 16, 4, 3, 4), (1, 4, 23, 19, 6, 5, 3), (2, 2, 9, 9, 3, 2, 2)])
def test_box_sum_identity(shape):
    B, Cin, H, W, Cout, K, s = shape
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=21)
    out, pooled = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True)
    A = box_sum_pooled(x, w, b, s)
    np.testing.assert_allclose(pooled, A, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, (1.0 / (1.0 + np.exp(-A))).sum(axis=(1, 2, 3)), rtol=1e-12)


def test_brute_force_pure_python():
    # Tiny case, every loop written out in Python, no array library.
    B, Cin, H, W, Cout, K, s = 1, 2, 7, 6, 2, 2, 2
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=31)
    Hc, Wc = H - K + 1, W - K + 1
    total = 0.0
    for co in range(Cout):
        conv = [[float(b[co]) + sum(float(x[0, ic, i + ky, j + kx]) * float(w[co, ic, ky, kx])
                                    for ic in range(Cin) for ky in range(K) for kx in range(K))
                 for j in range(Wc)] for i in range(Hc)]
        for ph in range(Hc // s):
            for pw in range(Wc // s):
                a = sum(conv[ph * s + dy][pw * s + dx] for dy in range(s) for dx in range(s)) / (s * s)
                total += 1.0 / (1.0 + math.exp(-a))
    out = oracle.conv2d_pool_sigmoid_sum(x, w, b, s)
    assert abs(out[0] - total) <= 1e-12 * abs(total)


def test_sigmoid_symmetry():
    # sigmoid(-a) = 1 - sigmoid(a): negating w and b gives Cout*PH*PW - out.
    x, w, b = fi.conv2d_inputs(2, 3, 17, 15, 4, 3, seed=41)
    _, _, PH, PW = oracle.conv2d_sizes(17, 15, 3, 4)
    a = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4)
    n = oracle.conv2d_pool_sigmoid_sum(x, -w, -b, 4)
    np.testing.assert_allclose(a + n, 4 * PH * PW, rtol=1e-14)


def test_saturation_no_nan():
    x = fi.normal((1, 2, 10, 10), 4, 0)
    w = np.zeros((2, 2, 3, 3), np.float32)
    for beta, want in [(40.0, 1.0), (-40.0, 1.0 / (1.0 + math.exp(40.0))), (-800.0, 0.0), (800.0, 1.0)]:
        out = oracle.conv2d_pool_sigmoid_sum(x, w, np.full(2, beta, np.float32), 2)
        assert np.isfinite(out).all()
        np.testing.assert_allclose(out, 2 * 16 * want, rtol=1e-12, atol=1e-300)


def test_batch_independence_and_channel_permutation():
    x, w, b = fi.conv2d_inputs(3, 3, 14, 14, 5, 3, seed=51)
    base = oracle.conv2d_pool_sigmoid_sum(x, w, b, 3)
    x2 = x.copy()
    x2[1] = fi.normal(x2[1].shape, 99, 0)
    alt = oracle.conv2d_pool_sigmoid_sum(x2, w, b, 3)
    assert alt[0] == base[0] and alt[2] == base[2] and alt[1] != base[1]
    perm = np.array([3, 0, 4, 1, 2])
    p = oracle.conv2d_pool_sigmoid_sum(x, w[perm], b[perm], 3)
    np.testing.assert_allclose(p, base, rtol=1e-14)


def test_batch_subset_and_part():
    x, w, b = fi.conv2d_inputs(4, 2, 12, 12, 3, 3, seed=61)
    full, part = oracle.conv2d_pool_sigmoid_sum(x, w, b, 2, want_part=True)
    sub = oracle.conv2d_pool_sigmoid_sum(x, w, b, 2, batch_idx=[3, 1])
    np.testing.assert_array_equal(sub, full[[3, 1]])
    np.testing.assert_allclose(part.sum(axis=1), full, rtol=1e-15)


def test_pooled_at_matches_full_map():
    x, w, b = fi.conv2d_inputs(2, 3, 19, 16, 4, 3, seed=71)
    _, pooled = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4, want_pooled=True)
    rng = np.random.default_rng(0)
    idx = np.stack([rng.integers(0, n, 50) for n in pooled.shape], axis=1)
    got = oracle.conv2d_pooled_at(x, w, b, 4, idx)
    np.testing.assert_allclose(got, pooled[tuple(idx.T)], rtol=1e-13, atol=1e-14)


def test_invalid_arguments_rejected():
    x, w, b = fi.conv2d_inputs(1, 2, 8, 8, 2, 3, seed=0)
    with pytest.raises(ValueError):
        oracle.conv2d_pool_sigmoid_sum(x, w, b, 0)
    with pytest.raises(ValueError):
        oracle.conv2d_pooled_at(x, w, b, 2, [[0, 0, 3, 0]])  # PH = 3, ph = 3 out of range
    with pytest.raises(ValueError):
        oracle.conv2d_pool_sigmoid_sum(x, w, b, 2, batch_idx=[1])


def test_page_figures():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        g = json.load(f)["conv2d"]
    H, K, s = g["H"], g["K"], g["pool"]
    Hc, Wc, PH, PW = oracle.conv2d_sizes(H, H, K, s)
    assert (Hc, PH) == (g["conv_out"], g["pool_out"])
    assert g["B"] * g["Cout"] * Hc * Wc == g["conv_outputs_total"]
    assert g["B"] * g["Cout"] * PH * PW == g["pooled_outputs_total"]
    assert g["macs_per_pooled_output"] == s * s * g["Cin"] * K * K
