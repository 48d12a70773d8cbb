"""Pins for the CPU oracle of depthwise Conv1d -> pointwise 1x1 Conv1d + bias.

Checked against PyTorch's CPU conv1d in float64 (the page defines the
method as exactly that pair of modules), the dense-fused 9-tap identity
written independently in numpy, a textbook GEMM special case, closed forms
for delta and constant inputs, and linearity.
"""

import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import fconv_inputs as fi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def torch_reference(x, w_dw, w_pw, b_pw, pad):
    xt = torch.from_numpy(x.astype(np.float64))
    C, K = w_dw.shape
    d = F.conv1d(xt, torch.from_numpy(w_dw.astype(np.float64)).reshape(C, 1, K), padding=pad, groups=C)
    bt = None if b_pw is None else torch.from_numpy(b_pw.astype(np.float64))
    return F.conv1d(d, torch.from_numpy(w_pw.astype(np.float64))[:, :, None], bt).numpy()


SHAPES = [
    # B, C, T, O, K, pad
    (4, 16, 256, 32, 9, 4),   # the small workload
    (2, 3, 17, 5, 9, 4),      # T not a multiple of anything
    (1, 4, 10, 2, 3, 0),      # no padding: T_out = T - K + 1
    (2, 5, 8, 7, 5, 6),       # pad larger than K//2: T_out > T
    (1, 2, 3, 3, 9, 4),       # T < K
    (3, 6, 33, 4, 1, 0),      # 1-tap depthwise
    (1, 8, 40, 16, 4, 1),     # even K, asymmetric reach
]


@pytest.mark.parametrize("shape", SHAPES)
def test_matches_torch_float64(shape):
    B, C, T, O, K, pad = shape
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=13)
    want = torch_reference(x, w_dw, w_pw, b_pw, pad)
    got = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad)
    assert got.shape == want.shape == (B, O, T + 2 * pad - K + 1)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_no_bias():
    x, w_dw, w_pw, _ = fi.dwsep_inputs(2, 4, 30, 6, 9, seed=2)
    np.testing.assert_allclose(oracle.dwsep_conv1d(x, w_dw, w_pw, None, 4),
                               torch_reference(x, w_dw, w_pw, None, 4), rtol=1e-12, atol=1e-12)


def dense_fused(x, w_dw, w_pw, b_pw, pad):
    """Independent formula: one dense conv1d with W[o,c,k] = w_pw[o,c] * w_dw[c,k] (numpy, float64)."""
    x = x.astype(np.float64)
    B, C, T = x.shape
    K = w_dw.shape[1]
    Wd = w_pw.astype(np.float64)[:, :, None] * w_dw.astype(np.float64)[None, :, :]
    Tout = T + 2 * pad - K + 1
    xp = np.zeros((B, C, T + 2 * pad))
    xp[:, :, pad:pad + T] = x
    y = np.zeros((B, w_pw.shape[0], Tout))
    for k in range(K):
        y += np.einsum("oc,bct->bot", Wd[:, :, k], xp[:, :, k:k + Tout])
    if b_pw is not None:
        y += b_pw.astype(np.float64)[None, :, None]
    return y


@pytest.mark.parametrize("shape", [(4, 16, 256, 32, 9, 4), (2, 7, 50, 9, 5, 2), (1, 3, 12, 4, 9, 8)])
def test_dense_fused_identity(shape):
    B, C, T, O, K, pad = shape
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=23)
    np.testing.assert_allclose(oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad),
                               dense_fused(x, w_dw, w_pw, b_pw, pad), rtol=1e-12, atol=1e-12)


def test_gemm_special_case():
    # K = 1, pad = 0, w_dw = 1: y[b] = w_pw @ x[b] + b_pw, a plain matrix product.
    B, C, T, O = 3, 12, 20, 7
    x, _, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, 1, seed=33)
    got = oracle.dwsep_conv1d(x, np.ones((C, 1), np.float32), w_pw, b_pw, 0)
    want = np.stack([w_pw.astype(np.float64) @ x[b].astype(np.float64) for b in range(B)])
    want += b_pw.astype(np.float64)[None, :, None]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("t0", [0, 1, 20, 62, 63])
def test_delta_input(t0):
    # x = e(c0, t0): y[o,t] - b[o] = w_pw[o,c0] * w_dw[c0, t0 - t + pad] when that tap exists, else 0.
    B, C, T, O, K, pad = 1, 5, 64, 6, 9, 4
    _, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=43)
    c0 = 3
    x = np.zeros((B, C, T), np.float32)
    x[0, c0, t0] = 1.0
    y = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad)[0] - b_pw.astype(np.float64)[:, None]
    want = np.zeros((O, T + 2 * pad - K + 1))
    for t in range(want.shape[1]):
        k = t0 - t + pad
        if 0 <= k < K:
            want[:, t] = w_pw[:, c0].astype(np.float64) * float(w_dw[c0, k])
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-15)


def test_identity_pointwise_is_fir():
    # w_pw = I: y is the per-channel cross-correlation with zero padding (numpy.correlate).
    C, T, K, pad = 4, 30, 9, 4
    x, w_dw, _, _ = fi.dwsep_inputs(1, C, T, C, K, seed=53)
    y = oracle.dwsep_conv1d(x, w_dw, np.eye(C, dtype=np.float32), None, pad)[0]
    for c in range(C):
        xp = np.concatenate([np.zeros(pad), x[0, c].astype(np.float64), np.zeros(pad)])
        np.testing.assert_allclose(y[c], np.correlate(xp, w_dw[c].astype(np.float64), mode="valid"),
                                   rtol=1e-13, atol=1e-14)


def test_linearity():
    B, C, T, O, K, pad = 2, 6, 40, 5, 9, 4
    x1, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=63)
    x2 = fi.normal((B, C, T), 64, 0)
    a, b = 0.75, -1.5
    bb = b_pw.astype(np.float64)[None, :, None]
    y1 = oracle.dwsep_conv1d(x1, w_dw, w_pw, b_pw, pad) - bb
    y2 = oracle.dwsep_conv1d(x2, w_dw, w_pw, b_pw, pad) - bb
    xs = (a * x1.astype(np.float64) + b * x2.astype(np.float64)).astype(np.float32)
    ys = oracle.dwsep_conv1d(xs, w_dw, w_pw, b_pw, pad) - bb
    # xs is rounded to float32, so compare against the same rounded input's exact linear image.
    np.testing.assert_allclose(ys, a * y1 + b * y2, rtol=1e-6, atol=1e-6)


def test_constant_input_closed_form():
    # x == v: interior t sees every tap; edge t only the taps that land in [0, T).
    B, C, T, O, K, pad = 1, 3, 24, 4, 9, 4
    _, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=73)
    v = 1.25
    x = np.full((B, C, T), v, np.float32)
    y = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad)[0]
    Tout = T + 2 * pad - K + 1
    for t in range(Tout):
        ks = [k for k in range(K) if 0 <= t + k - pad < T]
        dsum = np.array([sum(float(w_dw[c, k]) for k in ks) for c in range(C)])
        want = b_pw.astype(np.float64) + v * (w_pw.astype(np.float64) @ dsum)
        np.testing.assert_allclose(y[:, t], want, rtol=1e-13, atol=1e-14)


def test_at_matches_full():
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(3, 8, 70, 10, 9, seed=83)
    y = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, 4)
    rng = np.random.default_rng(1)
    idx = np.stack([rng.integers(0, n, 60) for n in y.shape], axis=1)
    idx[:4] = [[0, 0, 0], [2, 9, 69], [1, 3, 1], [2, 0, 68]]
    np.testing.assert_allclose(oracle.dwsep_conv1d_at(x, w_dw, w_pw, b_pw, 4, idx), y[tuple(idx.T)],
                               rtol=1e-13, atol=1e-14)
    sub = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, 4, batch_idx=[2, 0])
    np.testing.assert_array_equal(sub, y[[2, 0]])


def test_invalid_arguments_rejected():
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(1, 2, 4, 3, 9, seed=0)
    with pytest.raises(ValueError):
        oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, 0)   # T_out = 4 - 9 + 1 < 1
    with pytest.raises(ValueError):
        oracle.dwsep_conv1d(x, w_dw, w_pw[:, :1], b_pw, 4)


def test_page_figures():
    with open(os.path.join(GOLDEN, "page_figures.json")) as f:
        g = json.load(f)["dwsep"]
    assert oracle.dwsep_tout(g["T"], g["K"], g["pad"]) == g["T_out"]
    assert g["B"] * g["O"] * g["T_out"] == g["outputs_total"]
    assert g["C"] * g["K"] == g["dense_macs_per_output"]
    assert g["B"] * g["C"] * g["T_out"] * g["K"] == g["depthwise_macs"]
    assert g["B"] * g["O"] * g["T_out"] * g["C"] == g["pointwise_macs"]


def torch_reference_ex(x, w_dw, w_pw, b_pw, pad, stride, dilation):
    xt = torch.from_numpy(x.astype(np.float64))
    C, K = w_dw.shape
    d = F.conv1d(xt, torch.from_numpy(w_dw.astype(np.float64)).reshape(C, 1, K), padding=pad, groups=C,
                 stride=stride, dilation=dilation)
    bt = None if b_pw is None else torch.from_numpy(b_pw.astype(np.float64))
    return F.conv1d(d, torch.from_numpy(w_pw.astype(np.float64))[:, :, None], bt).numpy()


STRIDED = [
    # B, C, T, O, K, pad, stride, dilation
    (2, 6, 50, 8, 9, 4, 2, 1),
    (1, 5, 47, 3, 9, 4, 3, 1),
    (2, 4, 40, 6, 3, 2, 1, 2),
    (1, 3, 33, 4, 5, 0, 2, 3),
    (2, 7, 64, 9, 9, 8, 4, 2),
    (1, 2, 9, 2, 3, 0, 5, 4),    # one output step
]


@pytest.mark.parametrize("shape", STRIDED)
def test_strided_dilated_match_torch_float64(shape):
    B, C, T, O, K, pad, stride, dil = shape
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=93)
    want = torch_reference_ex(x, w_dw, w_pw, b_pw, pad, stride, dil)
    got = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad, stride=stride, dilation=dil)
    assert got.shape == want.shape
    assert oracle.dwsep_tout(T, K, pad, stride, dil) == want.shape[2]
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)
    rng = np.random.default_rng(2)
    idx = np.stack([rng.integers(0, n, 40) for n in got.shape], axis=1)
    np.testing.assert_allclose(oracle.dwsep_conv1d_at(x, w_dw, w_pw, b_pw, pad, idx, stride=stride, dilation=dil),
                               got[tuple(idx.T)], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("stride,dil", [(2, 1), (3, 2), (1, 3)])
def test_strided_delta_input(stride, dil):
    # x = e(c0, t0): y[o,t] - b[o] = w_pw[o,c0] * sum of w_dw[c0,k] over taps k with
    # t*stride + k*dil - pad == t0.
    B, C, T, O, K, pad = 1, 3, 40, 4, 5, 3
    _, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=97)
    c0 = 1
    for t0 in (0, 7, T - 1):
        x = np.zeros((B, C, T), np.float32)
        x[0, c0, t0] = 1.0
        y = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad, stride=stride, dilation=dil)[0]
        y -= b_pw.astype(np.float64)[:, None]
        want = np.zeros_like(y)
        for t in range(y.shape[1]):
            tap = sum(float(w_dw[c0, k]) for k in range(K) if t * stride + k * dil - pad == t0)
            want[:, t] = w_pw[:, c0].astype(np.float64) * tap
        np.testing.assert_allclose(y, want, rtol=0, atol=1e-15)


def test_output_length_formula():
    # [P7]: T_out = (T + 2*pad - K)/stride + 1; a dilation d makes the filter span d*(K-1)+1.
    assert oracle.dwsep_tout(4096, 9, 4, 1, 1) == 4096
    assert oracle.dwsep_tout(10, 3, 1, 2, 1) == 5
    assert oracle.dwsep_tout(10, 3, 0, 1, 2) == 6
    assert oracle.dwsep_tout(9, 3, 0, 5, 4) == 1
    assert oracle.dwsep_tout(8, 3, 0, 1, 4) == -1
