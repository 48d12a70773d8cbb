"""GPU parity of the generalised pool (max pooling, ReLU before the pool, ceil
mode) against the CPU oracle, through the C ABI's _ex entry points.

Bar as for the base chain: |gpu - oracle| <= 1e-4 + 1e-4*|oracle| element by
element on the pre-sigmoid pooled map and on the fused sums, oracle in
float64.  The shapes give several tiles of each matrix-core instance (K = 3 with
s = 2, 3, 4; K = 5 with s = 3), ragged tiles, partial ceil-mode windows of
every width at the bottom and right, Cin not a multiple of 4 and Cout above
64 and not a multiple of 16.
"""

import itertools
import sys

import numpy as np
import pytest

import fconv_inputs as fi
import oracle

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

RTOL = ATOL = 1e-4
CANARY = 12345.678


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import fp32_convolution_amd as fc

    return fc


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def assert_close(got, want, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    bound = ATOL + RTOL * np.abs(want)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu={got[i]!r} oracle={want[i]!r}")


AVG, MAX = oracle.POOL_AVG, oracle.POOL_MAX
COMBOS = list(itertools.product([AVG, MAX], [False, True], [False, True]))  # pool, relu, ceil


def combo_id(c):
    return f"{'max' if c[0] == MAX else 'avg'}{'-relu' if c[1] else ''}{'-ceil' if c[2] else ''}"


SHAPES = [
    # B, Cin, H, W, Cout, K, s                   conv map -> floor / ceil pooled sizes
    (2, 3, 16, 16, 4, 3, 4),        # 14x14 -> 3x3 / 4x4 (2-wide last windows)
    (2, 8, 70, 75, 64, 3, 4),       # 68x73 -> 17x18 / 17x19 (1-wide last column)
    (1, 5, 83, 150, 70, 3, 4),      # 81x148 -> 20x37 / 21x37 (1-row last), two channel ranges
    (2, 12, 40, 131, 20, 3, 4),     # 38x129 -> 9x32 / 10x33 (2-row, 1-column last), 3 quads
    (1, 8, 6, 8, 4, 3, 4),          # 4x6 -> 1x1 / 1x2
    (1, 2, 5, 9, 3, 3, 4),          # 3x7 -> 0x1 (empty) / 1x2 (3-row window)
    (1, 3, 20, 17, 5, 5, 3),        # K5/s3: 16x13 -> 5x4 / 6x5
    (1, 16, 40, 45, 70, 5, 3),      # K5/s3: 36x41 -> 12x13 / 12x14, 4 quads, two channel ranges, 2 tile columns
    (1, 4, 7, 9, 3, 5, 3),          # K5/s3: 3x5 -> 1x1 / 1x2
    (1, 2, 11, 13, 4, 3, 2),        # K3/s2: 9x11 -> 4x5 / 5x6
    (2, 6, 37, 70, 20, 3, 2),       # K3/s2: 35x68 -> 17x34 / 18x34, 3 tile columns
    (1, 5, 40, 50, 20, 3, 3),       # K3/s3: 38x48 -> 12x16 / 13x16
    # one channel quad (weights resident), two (resident) and more (streamed)
    # for every matrix-core instance
    (1, 7, 30, 40, 20, 5, 3),       # K5/s3, 2 quads: 26x36 -> 8x12 / 9x12
    (1, 10, 21, 75, 24, 3, 2),      # K3/s2, 3 quads: 19x73 -> 9x36 / 10x37, 2 tile columns
    (2, 13, 29, 44, 18, 3, 3),      # K3/s3, 4 quads: 27x42 -> 9x14 (ceil = floor)
    (1, 3, 25, 47, 8, 3, 3),        # K3/s3, 1 quad: 23x45 -> 7x15 / 8x15
    (1, 4, 12, 12, 6, 1, 5),        # K = 1, s = 5: one-thread-per-output kernel only
]

MFMA_INSTANCES = {(3, 4), (3, 2), (3, 3), (5, 3)}   # (K, s) of the per-conv-output matrix-core kernel


def has_mfma(shape):
    return (shape[5], shape[6]) in MFMA_INSTANCES


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("combo", COMBOS, ids=combo_id)
@pytest.mark.parametrize("algo", [0, 1, 2])
def test_pool_small(fc, shape, combo, algo):
    B, Cin, H, W, Cout, K, s = shape
    pool_mode, relu, ceil_mode = combo
    announce(f"pool ex {shape} {combo_id(combo)} algo={algo}")
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=51)
    xd, wd, bd = dev(x), dev(w), dev(b)
    kw = dict(algo=algo, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
    plain = pool_mode == AVG and not relu and not ceil_mode
    if algo == 1 and not has_mfma(shape) and not (plain and fc.conv2d_select_algo(Cin, Cout, K, s) != 2):
        with pytest.raises(fc.FconvError) as err:
            fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, **kw)
        assert err.value.status == fc.FCONV_EUNSUPPORTED
        return
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True, pool_mode=pool_mode,
                                                        relu=relu, ceil_mode=ceil_mode)
    got_map = fc.conv2d_pool_map(xd, wd, bd, s, **kw).cpu().numpy()
    got_out = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, **kw).cpu().numpy()
    assert_close(got_map, want_map, f"pooled map {shape} {combo_id(combo)}")
    assert_close(got_out, want_out, f"out {shape} {combo_id(combo)}")


# (K, s, largest Cin whose whole tile fits LDS, for the max / ReLU / ceil forms and for the folded
# average pool): past it the per-conv-output kernel stages CQ = 4 channel quads at a time
LDS_LIMITS = [(3, 4, 32, 40), (3, 2, 56, 56), (3, 3, 40, 40), (5, 3, 68, 68)]


@pytest.mark.parametrize("K,s,cin_max,cin_fold", LDS_LIMITS)
def test_pool_whole_and_chunked_tiles(fc, K, s, cin_max, cin_fold):
    # the matrix-core kernel at its largest whole tile (staging, plane padding and reads at the end of
    # LDS), one channel more (the first chunked case: a partial last quad), and a count that needs
    # several chunks plus a partial one; every pool form stays on the matrix cores
    H, W = 4 * s + K + 3, 17 * s + K + 1
    cins = sorted({cin_max, cin_max + 1, cin_fold, cin_fold + 1, 2 * cin_max + 19})
    for Cin in cins:
        announce(f"pool ex whole/chunked tile K={K} s={s} Cin={Cin}")
        x, w, b = fi.conv2d_inputs(1, Cin, H, W, 20, K, seed=60 + Cin)
        xd, wd, bd = dev(x), dev(w), dev(b)
        for pool_mode, relu, ceil_mode in [(MAX, True, True), (AVG, False, False), (AVG, True, False),
                                           (MAX, False, False)]:
            kw = dict(pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
            want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True, **kw)
            assert fc.conv2d_det_workspace_bytes(1, Cin, H, W, 20, K, s, 1, pool_mode, relu, ceil_mode) > 0
            got = fc.conv2d_pool_map(xd, wd, bd, s, algo=1, **kw).cpu().numpy()
            what = f"K{K} s{s} Cin {Cin} {combo_id((pool_mode, relu, ceil_mode))}"
            assert_close(got, want_map, what)
            det = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, algo=1, **kw).cpu().numpy()
            assert_close(det, want_out, f"det {what}")
            got_out = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=0, **kw).cpu().numpy()
            assert_close(got_out, want_out, f"AUTO out {what}")


CHUNKED = [
    # B, Cin, H, W, Cout, K, s: the channel-chunked per-conv-output tiling on larger maps: several tiles
    # in both directions, ragged edges, two output-channel ranges, Cin 64 and 128
    (2, 64, 38, 70, 64, 3, 4),
    (1, 128, 27, 101, 70, 3, 4),
    (1, 64, 30, 68, 40, 3, 2),
    (1, 128, 25, 64, 20, 3, 3),
    (2, 64, 31, 44, 128, 5, 3),
    (1, 130, 26, 35, 24, 5, 3),
]


@pytest.mark.parametrize("shape", CHUNKED)
@pytest.mark.parametrize("combo", COMBOS, ids=combo_id)
def test_pool_chunked_many_channels(fc, shape, combo):
    B, Cin, H, W, Cout, K, s = shape
    pool_mode, relu, ceil_mode = combo
    announce(f"pool ex chunked {shape} {combo_id(combo)}")
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=61)
    xd, wd, bd = dev(x), dev(w), dev(b)
    kw = dict(pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True, **kw)
    assert_close(fc.conv2d_pool_map(xd, wd, bd, s, algo=1, **kw).cpu().numpy(), want_map,
                 f"map {shape} {combo_id(combo)}")
    assert_close(fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=1, **kw).cpu().numpy(), want_out,
                 f"out {shape} {combo_id(combo)}")


@pytest.mark.parametrize("combo", COMBOS[1:], ids=combo_id)
def test_pool_boxsum_refused(fc, combo):
    pool_mode, relu, ceil_mode = combo
    announce(f"pool ex box-sum refused {combo_id(combo)}")
    x, w, b = fi.conv2d_inputs(1, 3, 16, 16, 4, 3, seed=52)
    with pytest.raises(fc.FconvError) as err:
        fc.conv2d_pool_sigmoid_sum(dev(x), dev(w), dev(b), 4, algo=3, pool_mode=pool_mode, relu=relu,
                                   ceil_mode=ceil_mode)
    assert err.value.status == fc.FCONV_EUNSUPPORTED


@pytest.mark.parametrize("algo", [1, 2])
def test_pool_no_bias(fc, algo):
    announce(f"pool ex no bias algo={algo}")
    x, w, _ = fi.conv2d_inputs(2, 8, 41, 70, 20, 3, seed=53)
    for pool_mode, relu, ceil_mode in COMBOS[1:]:
        want = oracle.conv2d_pool_sigmoid_sum(x, w, None, 4, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
        got = fc.conv2d_pool_sigmoid_sum(dev(x), dev(w), None, 4, algo=algo, pool_mode=pool_mode, relu=relu,
                                         ceil_mode=ceil_mode).cpu().numpy()
        assert_close(got, want, f"out, bias=None, {combo_id((pool_mode, relu, ceil_mode))}")


def test_pool_relu_of_negative_map(fc):
    # every conv output below zero: ReLU gives 0, sigma(0) = 1/2, out = Cout*PH*PW/2 exactly
    announce("pool ex relu of a negative map")
    x, w, _ = fi.conv2d_inputs(2, 8, 70, 75, 64, 3, seed=54)
    b = np.full(64, -100.0, dtype=np.float32)
    for pool_mode, ceil_mode, algo in itertools.product([AVG, MAX], [False, True], [1, 2]):
        PH, PW = fc.conv2d_out_size(70, 75, 3, 4, ceil_mode=ceil_mode)
        got = fc.conv2d_pool_sigmoid_sum(dev(x), dev(w), dev(b), 4, algo=algo, pool_mode=pool_mode, relu=True,
                                         ceil_mode=ceil_mode).cpu().numpy()
        assert (got == 64 * PH * PW / 2.0).all(), (pool_mode, ceil_mode, algo, got)


def test_pool_ceil_equals_floor_when_windows_fit(fc):
    announce("pool ex ceil == floor on a 68x72 map")
    x, w, b = fi.conv2d_inputs(2, 8, 70, 74, 64, 3, seed=55)
    xd, wd, bd = dev(x), dev(w), dev(b)
    for pool_mode, relu in itertools.product([AVG, MAX], [False, True]):
        f = fc.conv2d_pool_map(xd, wd, bd, 4, algo=1, pool_mode=pool_mode, relu=relu, ceil_mode=False)
        c = fc.conv2d_pool_map(xd, wd, bd, 4, algo=1, pool_mode=pool_mode, relu=relu, ceil_mode=True)
        if pool_mode == AVG and not relu:
            # floor mode is the base chain (its own kernel, another summation order)
            assert_close(c.cpu().numpy(), f.cpu().numpy(), "ceil vs floor, plain average")
        else:
            assert torch.equal(f, c)


@pytest.mark.parametrize("shape", [(3, 8, 70, 75, 64, 3, 4), (2, 16, 40, 45, 70, 5, 3), (2, 3, 20, 17, 5, 7, 2)])
@pytest.mark.parametrize("algo", [0, 2])
def test_pool_deterministic(fc, shape, algo):
    # partial sums + fixed-order reduction: repeated calls give identical bits, within tolerance of the oracle
    B, Cin, H, W, Cout, K, s = shape
    announce(f"pool ex deterministic {shape} algo={algo}")
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=59)
    xd, wd, bd = dev(x), dev(w), dev(b)
    for pool_mode, relu, ceil_mode in [(MAX, True, False), (MAX, False, True), (AVG, True, True)]:
        kw = dict(algo=algo, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
        want = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
        first = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, **kw).cpu().numpy()
        nbytes = fc.conv2d_det_workspace_bytes(B, Cin, H, W, Cout, K, s, algo, pool_mode, relu, ceil_mode)
        ws = torch.full((max(nbytes, 4) // 4,), float("nan"), device="cuda")
        for _ in range(3):
            again = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, workspace=ws, **kw).cpu().numpy()
            assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
        assert_close(first, want, f"deterministic out {shape} {combo_id((pool_mode, relu, ceil_mode))}")
        default = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, **kw).cpu().numpy()
        assert np.array_equal(default.view(np.uint32), first.view(np.uint32)), "default vs caller workspace"


def padded(n, pad=1024):
    whole = torch.full((n + 2 * pad,), CANARY, device="cuda")
    return whole, whole[pad:pad + n]


def canaries_intact(whole, n, pad=1024):
    h = whole.cpu().numpy()
    return bool((h[:pad] == np.float32(CANARY)).all() and (h[pad + n:] == np.float32(CANARY)).all())


@pytest.mark.parametrize("algo", [1, 2])
def test_pool_writes_only_its_outputs(fc, algo):
    B, Cin, H, W, Cout, K, s = 2, 5, 41, 70, 70, 3, 4
    announce(f"pool ex canaries algo={algo}")
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=56)
    xd, wd, bd = dev(x), dev(w), dev(b)
    for pool_mode, relu, ceil_mode in COMBOS[1:]:
        PH, PW = fc.conv2d_out_size(H, W, K, s, ceil_mode=ceil_mode)
        n = B * Cout * PH * PW
        whole, inner = padded(n)
        fc.conv2d_pool_map(xd, wd, bd, s, out=inner.view(B, Cout, PH, PW), algo=algo, pool_mode=pool_mode,
                           relu=relu, ceil_mode=ceil_mode)
        torch.cuda.synchronize()
        assert canaries_intact(whole, n)
        assert not torch.isnan(inner).any() and (inner != np.float32(CANARY)).all()
        wo, io = padded(B)
        fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, out=io, algo=algo, pool_mode=pool_mode, relu=relu,
                                   ceil_mode=ceil_mode)
        torch.cuda.synchronize()
        assert canaries_intact(wo, B)


FULL_COMBOS = [(MAX, True, False), (MAX, True, True), (AVG, True, True), (MAX, False, True)]


@pytest.fixture(scope="module")
def full_inputs():
    return fi.make("conv2d_full", seed=0)


@pytest.fixture(scope="module")
def tail_inputs():
    return fi.make("conv2d_tail", seed=0)


@pytest.mark.parametrize("combo", [(MAX, True, False), (MAX, True, True), (AVG, True, True)], ids=combo_id)
def test_pool_tail_size(fc, tail_inputs, combo):
    # x[64,16,257,257], 16 -> 128, K 5, s 3: the K5/s3 instance, two channel ranges
    pool_mode, relu, ceil_mode = combo
    announce(f"pool ex tail size {combo_id(combo)}")
    x, w, b = tail_inputs
    s = 3
    kw = dict(algo=1, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
    xd, wd, bd = dev(x), dev(w), dev(b)
    got_out = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, **kw).cpu().numpy()
    got_map = fc.conv2d_pool_map(xd, wd, bd, s, **kw).cpu().numpy()
    want_out = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, batch_idx=[63], pool_mode=pool_mode, relu=relu,
                                              ceil_mode=ceil_mode)
    assert_close(got_out[[63]], want_out, "out[63]")
    sig = (1.0 / (1.0 + np.exp(-got_map.astype(np.float64)))).sum(axis=(1, 2, 3))
    assert_close(got_out, sig, "fused sum vs sigmoid(map) sum")
    B, Cout, PH, PW = got_map.shape
    assert (PH, PW) == ((85, 85) if ceil_mode else (84, 84))
    rng = np.random.default_rng(58)
    n = 10000
    samp = np.stack([rng.integers(0, B, n), rng.integers(0, Cout, n), rng.integers(0, PH, n),
                     rng.integers(0, PW, n)], axis=1)
    edge = [0, 1, 3, 4, 9, 10, 19, 20, PH - 2, PH - 1]
    extra = [(bb, co, ph, pw) for bb in (0, B - 1) for co in (0, 63, 64, Cout - 1) for ph in edge for pw in edge]
    samp = np.concatenate([samp, np.array(extra)], axis=0)
    want = oracle.conv2d_pooled_at(x, w, b, s, samp, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
    assert_close(got_map[tuple(samp.T)], want, "sampled pooled map")


@pytest.mark.parametrize("combo", FULL_COMBOS, ids=combo_id)
def test_pool_full_size(fc, full_inputs, combo):
    # x[128,8,384,384], 8 -> 64, K 3, s 4: the matrix-core kernel in the launch the benchmark times
    pool_mode, relu, ceil_mode = combo
    announce(f"pool ex full size {combo_id(combo)}")
    x, w, b = full_inputs
    s = 4
    kw = dict(algo=0, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
    xd, wd, bd = dev(x), dev(w), dev(b)
    got_out = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, **kw).cpu().numpy()
    got_map = fc.conv2d_pool_map(xd, wd, bd, s, **kw).cpu().numpy()
    idx = [0, 127]
    want_out = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, batch_idx=idx, pool_mode=pool_mode, relu=relu,
                                              ceil_mode=ceil_mode)
    assert_close(got_out[idx], want_out, f"out[{idx}]")
    sig = (1.0 / (1.0 + np.exp(-got_map.astype(np.float64)))).sum(axis=(1, 2, 3))
    assert_close(got_out, sig, "fused sum vs sigmoid(map) sum")
    B, Cout, PH, PW = got_map.shape
    assert (PH, PW) == ((96, 96) if ceil_mode else (95, 95))
    rng = np.random.default_rng(57)
    n = 20000
    samp = np.stack([rng.integers(0, B, n), rng.integers(0, Cout, n), rng.integers(0, PH, n),
                     rng.integers(0, PW, n)], axis=1)
    edge = [0, 1, 3, 4, 15, 16, 31, 32, PH - 2, PH - 1]
    extra = [(bb, co, ph, pw) for bb in (0, B - 1) for co in (0, 15, 16, Cout - 1)
             for ph in edge for pw in edge]
    samp = np.concatenate([samp, np.array(extra)], axis=0)
    want = oracle.conv2d_pooled_at(x, w, b, s, samp, pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
    assert_close(got_map[tuple(samp.T)], want, "sampled pooled map")
