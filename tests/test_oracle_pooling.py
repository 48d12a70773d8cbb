"""Pins of the oracle's pooling generalisation (CPU): max pooling, ReLU
before the pool, ceil mode.

The operator order is the base op's with the pool generalised and an
optional ReLU after the conv (the Conv2D + ReLU + MaxPool fused operator the
[NEWS] article lists): conv + bias -> [ReLU] -> AvgPool2d or MaxPool2d
(kernel = stride = s, no padding, floor or ceil mode) -> sigmoid -> sum.
None of the checks re-types the oracle's formula: PyTorch's CPU float64
operators, PyTorch's own output-size rule, closed forms, special cases that
reduce to the floor/average path, and a pure-Python brute force.
"""

import itertools

import numpy as np
import pytest

import fconv_inputs as fi
import oracle

torch = pytest.importorskip("torch")
F = torch.nn.functional

MAX, AVG = oracle.POOL_MAX, oracle.POOL_AVG


def torch_ref(x, w, b, s, pool_mode, relu, ceil_mode):
    t = F.conv2d(torch.from_numpy(x).double(), torch.from_numpy(w).double(),
                 None if b is None else torch.from_numpy(b).double())
    if relu:
        t = F.relu(t)
    if pool_mode == MAX:
        p = F.max_pool2d(t, s, s, ceil_mode=ceil_mode)
    else:
        p = F.avg_pool2d(t, s, s, ceil_mode=ceil_mode)
    return torch.sigmoid(p).sum(dim=(1, 2, 3)).numpy(), p.numpy()


SHAPES = [
    # B, Cin, H, W, Cout, K, s: ragged maps so that ceil mode adds partial windows
    (2, 3, 16, 16, 4, 3, 4),     # 14 -> floor 3, ceil 4 (a 2-wide last window)
    (1, 2, 13, 11, 3, 3, 4),     # 11 x 9 -> ceil 3 x 3 (last windows 3 and 1 wide)
    (2, 4, 12, 20, 5, 5, 3),     # 8 x 16 -> ceil 3 x 6
    (1, 3, 10, 10, 2, 3, 2),     # 8 x 8: ceil == floor
    (1, 1, 6, 7, 2, 4, 4),       # 3 x 4: floor gives 0 rows, ceil 1
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("pool_mode,relu,ceil_mode", list(itertools.product([AVG, MAX], [False, True],
                                                                              [False, True])))
def test_matches_torch(shape, pool_mode, relu, ceil_mode):
    B, Cin, H, W, Cout, K, s = shape
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=41)
    _, _, PH, PW = oracle.conv2d_sizes(H, W, K, s, ceil_mode=ceil_mode)
    if PH == 0 or PW == 0:
        # PyTorch refuses an empty pool; the library defines the sum over it as 0
        got = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
        assert (got == 0).all()
        return
    want_out, want_map = torch_ref(x, w, b, s, pool_mode, relu, ceil_mode)
    got_out, got_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True, pool_mode=pool_mode, relu=relu,
                                                      ceil_mode=ceil_mode)
    assert got_map.shape == want_map.shape
    np.testing.assert_allclose(got_map, want_map, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got_out, want_out, rtol=1e-12, atol=1e-12)
    # the sampled form agrees with the full form everywhere
    Bq, Co, PH, PW = got_map.shape
    idx = np.array(list(itertools.product(range(Bq), range(Co), range(PH), range(PW))), dtype=np.int64)
    if idx.size:
        at = oracle.conv2d_pooled_at(x, w, b, s, idx, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
        np.testing.assert_allclose(at, got_map[tuple(idx.T)], rtol=1e-12, atol=1e-12)


def test_sizes_match_torch_output_shape():
    for n, s in itertools.product(range(1, 40), range(1, 8)):
        for ceil_mode in (False, True):
            Hc, Wc, PH, PW = oracle.conv2d_sizes(n, n + 1, 1, s, ceil_mode=ceil_mode)
            if n < s and not ceil_mode:
                assert PH == 0
                continue
            shape = F.avg_pool2d(torch.zeros(1, 1, n, n + 1), s, s, ceil_mode=ceil_mode).shape
            assert (PH, PW) == (shape[2], shape[3]), (n, s, ceil_mode)


@pytest.mark.parametrize("pool_mode", [AVG, MAX])
def test_constant_input_closed_form(pool_mode):
    # every conv output of channel co equals v*sum(w[co]) + b[co], so any pool returns it
    B, Cin, H, W, Cout, K, s = 2, 3, 15, 14, 4, 3, 4
    _, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=42)
    v = 0.75
    x = np.full((B, Cin, H, W), v, dtype=np.float32)
    for relu, ceil_mode in itertools.product([False, True], [False, True]):
        _, _, PH, PW = oracle.conv2d_sizes(H, W, K, s, ceil_mode=ceil_mode)
        a = v * w.astype(np.float64).sum(axis=(1, 2, 3)) + b.astype(np.float64)
        if relu:
            a = np.maximum(a, 0.0)
        want = PH * PW * (1.0 / (1.0 + np.exp(-a))).sum()
        got = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
        np.testing.assert_allclose(got, np.full(B, want), rtol=1e-12)


@pytest.mark.parametrize("pool_mode", [AVG, MAX])
@pytest.mark.parametrize("ceil_mode", [False, True])
def test_relu_of_negative_map_gives_half_per_output(pool_mode, ceil_mode):
    # conv outputs all below zero -> ReLU gives 0 -> sigma(0) = 1/2: out = Cout*PH*PW/2 exactly
    B, Cin, H, W, Cout, K, s = 2, 3, 14, 17, 5, 3, 4
    x, w, _ = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=43)
    b = np.full(Cout, -100.0, dtype=np.float32)
    _, _, PH, PW = oracle.conv2d_sizes(H, W, K, s, ceil_mode=ceil_mode)
    got = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, pool_mode=pool_mode, relu=True, ceil_mode=ceil_mode)
    assert (got == Cout * PH * PW / 2.0).all()


def test_ceil_equals_floor_when_windows_fit():
    x, w, b = fi.conv2d_inputs(2, 3, 18, 22, 4, 3, seed=44)  # 16 x 20 conv map, s = 4
    for pool_mode, relu in itertools.product([AVG, MAX], [False, True]):
        f = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4, pool_mode=pool_mode, relu=relu, ceil_mode=False)
        c = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4, pool_mode=pool_mode, relu=relu, ceil_mode=True)
        assert np.array_equal(f, c)


def test_max_at_least_avg():
    x, w, b = fi.conv2d_inputs(2, 4, 21, 19, 6, 3, seed=45)
    for relu, ceil_mode in itertools.product([False, True], [False, True]):
        _, mx = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4, want_pooled=True, pool_mode=MAX, relu=relu,
                                               ceil_mode=ceil_mode)
        _, av = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4, want_pooled=True, pool_mode=AVG, relu=relu,
                                               ceil_mode=ceil_mode)
        assert (mx >= av - 1e-12).all()


def brute(x, w, b, s, pool_mode, relu, ceil_mode):
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    Hc, Wc = H - K + 1, W - K + 1
    nph = -(-Hc // s) if ceil_mode else Hc // s
    npw = -(-Wc // s) if ceil_mode else Wc // s
    out = []
    for bb in range(B):
        total = 0.0
        for co in range(Cout):
            for ph in range(nph):
                for pw in range(npw):
                    vals = []
                    for y in range(ph * s, min(ph * s + s, Hc)):
                        for xx in range(pw * s, min(pw * s + s, Wc)):
                            c = float(b[co])
                            for ic in range(Cin):
                                for ky in range(K):
                                    for kx in range(K):
                                        c += float(x[bb, ic, y + ky, xx + kx]) * float(w[co, ic, ky, kx])
                            vals.append(max(c, 0.0) if relu else c)
                    a = max(vals) if pool_mode == MAX else sum(vals) / len(vals)
                    total += 1.0 / (1.0 + np.exp(-a))
        out.append(total)
    return np.array(out)


def test_brute_force_tiny():
    x, w, b = fi.conv2d_inputs(1, 2, 8, 7, 2, 2, seed=46)  # 7 x 6 conv map, s = 3: ceil adds 1-wide windows
    for pool_mode, relu, ceil_mode in itertools.product([AVG, MAX], [False, True], [False, True]):
        got = oracle.conv2d_pool_sigmoid_sum(x, w, b, 3, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
        np.testing.assert_allclose(got, brute(x, w, b, 3, pool_mode, relu, ceil_mode), rtol=1e-12)


def test_invalid_pool_arguments():
    x, w, b = fi.conv2d_inputs(1, 1, 6, 6, 1, 3, seed=47)
    with pytest.raises(ValueError):
        oracle.conv2d_pool_sigmoid_sum(x, w, b, 2, pool_mode=2)
