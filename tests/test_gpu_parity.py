"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (the specified fp32 tolerance): |gpu - oracle| <= 1e-4 + 1e-4*|oracle|
element by element, with the oracle in float64.  For the fused Conv2d sum the
elementwise check runs on the pre-sigmoid pooled map, which the same kernels
write; the scalar sums are checked as well.  Full-size workloads compare
sampled outputs that the oracle computes one by one, plus whole batch items.
"""

import ctypes
import sys

import numpy as np
import pytest

import fconv_inputs as fi
import oracle

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

RTOL = ATOL = 1e-4


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


# ------------------------------------------------------------------ Conv2d path

SMALL_CONV = [
    # B, Cin, H, W, Cout, K, s
    (2, 3, 16, 16, 4, 3, 4),        # the tiny workload
    (2, 8, 70, 75, 64, 3, 4),       # several tiles, ragged in both directions
    (1, 16, 60, 50, 128, 5, 3),     # K5/s3 instance: several tiles, ragged
    (2, 5, 41, 37, 20, 3, 4),       # odd Cin, Cout not a multiple of 16
    (1, 8, 40, 40, 70, 3, 4),       # Cout > 64: two channel ranges
    (1, 3, 37, 41, 7, 3, 2),        # K3/s2 instance
    (2, 4, 30, 28, 9, 3, 3),        # K3/s3 instance
    (1, 8, 37, 70, 100, 3, 2),      # K3/s2, Cout > 64: 8-wave box-sum instance, Cout not a multiple of 16
    (2, 16, 45, 50, 128, 3, 3),     # K3/s3, Cout > 64: 8-wave box-sum instance, one 128-channel range
    (1, 2, 23, 19, 5, 7, 2),        # no MFMA instance (K=7): simple path
    (1, 3, 9, 9, 4, 5, 3),          # PH = PW = 1
    # box-sum K3/s4 kernel (W % 4 == 0): one, two and streamed channel quads
    (3, 1, 20, 200, 16, 3, 4),      # Cin 1; a 1-column second tile; 3 of 4 waves' channels past Cout
    (1, 6, 38, 100, 64, 3, 4),      # Cin 6 (two quads, two zero channels); one partial tile column
    (2, 12, 45, 52, 40, 3, 4),      # Cin 12 (channel loop at run time); Cout 40; ragged rows
]


ALGOS = [0, 1, 2, 3]  # auto, direct MFMA, direct simple, box-sum


@pytest.mark.parametrize("shape", SMALL_CONV)
@pytest.mark.parametrize("algo", ALGOS)
def test_conv2d_small(fc, shape, algo):
    B, Cin, H, W, Cout, K, s = shape
    announce(f"conv2d small {shape} algo={algo}")
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=1)
    xd, wd, bd = dev(x), dev(w), dev(b)
    if algo in (1, 3) and fc.conv2d_select_algo(Cin, Cout, K, s) == 2:
        with pytest.raises(fc.FconvError) as err:
            fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=algo)
        assert err.value.status == fc.FCONV_EUNSUPPORTED
        return
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True)
    got_map = fc.conv2d_pool_map(xd, wd, bd, s, algo=algo).cpu().numpy()
    got_out = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=algo).cpu().numpy()
    assert_close(got_map, want_map, f"pooled map {shape}")
    assert_close(got_out, want_out, f"out {shape}")


BOX4_CONV = [
    # B, Cin, H, W, Cout, K=3, s=4 with W % 4 == 0: the one-column-per-lane box-sum kernel
    (2, 8, 70, 76, 64, 3, 4),       # odd number of pooled rows (17), one column tile
    (1, 12, 30, 200, 20, 3, 4),     # 3 channel quads, 49 pooled columns: a 1-column second tile
    (2, 5, 41, 100, 70, 3, 4),      # Cin not a multiple of 4, two output-channel ranges
    (1, 8, 11, 16, 4, 3, 4),        # PH = 2, PW = 3
    (1, 3, 6, 8, 4, 3, 4),          # PH = PW = 1: one window
]


@pytest.mark.parametrize("shape", BOX4_CONV)
@pytest.mark.parametrize("aligned", [True, False])
def test_conv2d_boxsum_one_column_per_lane(fc, shape, aligned):
    # aligned=False starts x 4 bytes past a 16-byte boundary (4-byte loads)
    B, Cin, H, W, Cout, K, s = shape
    announce(f"conv2d box-sum, a pooled column per lane {shape} aligned={aligned}")
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=21)
    if aligned:
        xd = dev(x)
    else:
        buf = torch.zeros(x.size + 1, device="cuda")
        buf[1:] = dev(x).reshape(-1)
        xd = buf[1:].view(*x.shape)
    wd, bd = dev(w), dev(b)
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True)
    got_map = fc.conv2d_pool_map(xd, wd, bd, s, algo=3).cpu().numpy()
    got_out = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=3).cpu().numpy()
    det = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, algo=3).cpu().numpy()
    assert_close(got_map, want_map, f"pooled map {shape}")
    assert_close(got_out, want_out, f"out {shape}")
    assert_close(det, want_out, f"deterministic out {shape}")


def largest_supported_cin(fc, K, s, H, W, algo):
    """Largest Cin (up to 256) for which the algorithm has an instance, by the host-side query."""
    best = 0
    for cin in range(1, 257):
        try:
            fc.conv2d_det_workspace_bytes(1, cin, H, W, 8, K, s, algo)
            best = cin
        except fc.FconvError as e:
            assert e.status == fc.FCONV_EUNSUPPORTED
    return best


@pytest.mark.parametrize("K,s,wx", [(3, 4, 3), (3, 4, 1), (5, 3, 3), (3, 2, 3), (3, 3, 3)])
@pytest.mark.parametrize("algo", [1, 3])
def test_conv2d_largest_lds_tile(fc, K, s, wx, algo):
    # each algorithm at the largest channel count the query probes (256), checked against the oracle.
    # Box-sum stages 8 or 16 channels at a time (32 or 16 chunks here); the direct kernels hold a whole
    # tile's channels in LDS up to Cin 32-68 and past that run the per-conv-output kernel's channel-
    # chunked tiling (16 channels per chunk).  K3/s4 with wx = 1 has W % 4 == 0, which box-sum runs on
    # its one-column-per-lane kernel.
    H, W = 5 * s + K + 2, 33 * s + K + wx
    cin = largest_supported_cin(fc, K, s, H, W, algo)
    announce(f"conv2d largest LDS tile K={K} s={s} algo={algo} Cin={cin}")
    assert cin == 256
    x, w, b = fi.conv2d_inputs(2, cin, H, W, 70, K, seed=24)
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True)
    xd, wd, bd = dev(x), dev(w), dev(b)
    assert_close(fc.conv2d_pool_map(xd, wd, bd, s, algo=algo).cpu().numpy(), want_map, f"map Cin={cin}")
    assert_close(fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=algo).cpu().numpy(), want_out, f"out Cin={cin}")


MANY_CHANNELS = [
    # B, Cin, H, W, Cout, K, s: box-sum with several LDS chunks of channels (8 per chunk for K = 3,
    # 16 for K = 5), a partial last chunk, and Cin = 64 and 128 on the matrix cores; the direct path too
    (2, 12, 30, 104, 64, 3, 4),     # one-column-per-lane kernel: chunks of 2 + 1 quads
    (1, 20, 37, 101, 70, 3, 4),     # W % 4 != 0: general kernel, chunks of 2 + 2 + 1 quads, two channel ranges
    (2, 64, 22, 200, 64, 3, 4),     # Cin 64: 8 chunks
    (1, 128, 18, 100, 64, 3, 4),    # Cin 128: 16 chunks
    (1, 128, 19, 99, 20, 3, 4),     # Cin 128, W % 4 != 0
    (2, 20, 40, 41, 128, 5, 3),     # K5/s3: chunks of 4 + 1 quads
    (1, 64, 30, 44, 128, 5, 3),     # K5/s3, Cin 64
    (1, 128, 20, 47, 40, 5, 3),     # K5/s3, Cin 128
    (1, 36, 40, 66, 30, 3, 2),      # K3/s2: 4 + 4 + 1 quads
    (1, 64, 31, 70, 64, 3, 3),      # K3/s3, Cin 64
    (1, 20, 40, 41, 200, 3, 3),     # K3/s3, 8-wave instance: chunks of 16 + 4 channels, two ranges (128 + 72)
    (1, 36, 34, 40, 130, 3, 2),     # K3/s2, 8-wave instance: chunks of 16 + 16 + 4, a 2-channel second range
]


@pytest.mark.parametrize("shape", MANY_CHANNELS)
def test_conv2d_many_channels(fc, shape):
    B, Cin, H, W, Cout, K, s = shape
    announce(f"conv2d box-sum many channels {shape}")
    assert fc.conv2d_select_algo(Cin, Cout, K, s) == fc.ALGO_BOXSUM
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=29)
    xd, wd, bd = dev(x), dev(w), dev(b)
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True)
    assert_close(fc.conv2d_pool_map(xd, wd, bd, s, algo=3).cpu().numpy(), want_map, f"map {shape}")
    assert_close(fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s).cpu().numpy(), want_out, f"out (auto) {shape}")
    assert_close(fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, algo=3).cpu().numpy(), want_out, f"det {shape}")
    # and on the direct matrix-core path (whole tiles up to Cin 32-68, channel-chunked past that)
    assert_close(fc.conv2d_pool_map(xd, wd, bd, s, algo=1).cpu().numpy(), want_map, f"direct map {shape}")


WALK_CONV = [
    # B, Cin, H, W, Cout, K, s, algo: more than 1024 units (tiles x channel ranges) per batch item, so
    # each workgroup walks several and an item gets at most 1024 partial sums
    (2, 1, 266, 6340, 4, 3, 4, 3),     # one-column-per-lane box-sum: 33 x 33 tiles of 2 x 48
    (2, 1, 266, 6339, 4, 3, 4, 3),     # general box-sum (W % 4 != 0): 17 x 99 tiles of 4 x 16
    (1, 2, 266, 6340, 4, 3, 4, 1),     # direct MFMA, folded pool: 22 x 99 tiles of 3 x 16
    (1, 2, 266, 1100, 16, 3, 4, 2),    # one thread per pooled output: 16 x 66 x 274 / 256 blocks
    (2, 2, 400, 1204, 8, 5, 3, 3),     # general box-sum K5/s3: 33 x 34 tiles of 4 x 12
    (1, 2, 400, 1204, 8, 5, 3, 1),     # direct K5/s3 (pool folded into the contraction)
    (1, 20, 266, 1026, 4, 3, 2, 3),    # general box-sum K3/s2, 3 chunks of channels
    (1, 3, 398, 1538, 4, 3, 3, 1),     # direct K3/s3
    (1, 2, 266, 3100, 72, 3, 3, 3),    # 8-wave general box-sum K3/s3 (Cout > 64): 22 x 65 tiles of 4 x 16
]


@pytest.mark.parametrize("shape", WALK_CONV)
def test_conv2d_walk(fc, shape):
    B, Cin, H, W, Cout, K, s, algo = shape
    announce(f"conv2d walk {shape}")
    assert fc.conv2d_det_workspace_bytes(B, Cin, H, W, Cout, K, s, algo) == B * 1024 * 4
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=30)
    xd, wd, bd = dev(x), dev(w), dev(b)
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True)
    assert_close(fc.conv2d_pool_map(xd, wd, bd, s, algo=algo).cpu().numpy(), want_map, f"map {shape}")
    out = torch.full((B,), 1e6, device="cuda")
    for _ in range(2):  # the second call must overwrite the first
        fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=algo, out=out)
    assert_close(out.cpu().numpy(), want_out, f"out {shape}")
    d1 = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, algo=algo).cpu().numpy()
    d2 = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, algo=algo).cpu().numpy()
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    assert_close(d1, want_out, f"det {shape}")


WALK_POOL = [
    # B, Cin, H, W, Cout, K, s, algo, pool_mode, relu, ceil: the generalised pool with more than 1024
    # units per item
    (1, 2, 266, 6340, 4, 3, 4, 1, 1, True, True),    # per-conv-output kernel, 17 x 99 tiles of 4 x 16
    (1, 2, 400, 1204, 8, 5, 3, 1, 1, False, True),   # its K5/s3 instance, 33 x 41 tiles of 4 x 10
    (1, 2, 266, 1100, 16, 3, 4, 2, 0, True, True),   # one thread per output
    (1, 33, 134, 2050, 4, 3, 4, 1, 1, True, False),  # channel-chunked per-conv-output tiling, 33 x 32 tiles of 1 x 16
    (1, 70, 154, 634, 8, 5, 3, 1, 0, True, False),   # its K5/s3 instance, 50 x 21 tiles of 1 x 10
]


@pytest.mark.parametrize("shape", WALK_POOL)
def test_conv2d_walk_pool(fc, shape):
    B, Cin, H, W, Cout, K, s, algo, pool_mode, relu, ceil_mode = shape
    announce(f"conv2d walk, generalised pool {shape}")
    kw = dict(pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
    assert fc.conv2d_det_workspace_bytes(B, Cin, H, W, Cout, K, s, algo, **kw) == B * 1024 * 4
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=31)
    xd, wd, bd = dev(x), dev(w), dev(b)
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True, **kw)
    assert_close(fc.conv2d_pool_map(xd, wd, bd, s, algo=algo, **kw).cpu().numpy(), want_map, f"map {shape}")
    assert_close(fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=algo, **kw).cpu().numpy(), want_out, f"out {shape}")
    assert_close(fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, algo=algo, **kw).cpu().numpy(), want_out,
                 f"det {shape}")


@pytest.fixture(scope="module")
def largest_item():
    # x[2,2,16384,16383]: 536,838,144 elements per batch item, just under the 2^29 the ABI accepts
    # (in-item offsets are 32-bit), 4.3 GB in all (batch offsets past 2^31 bytes)
    B, Cin, H, W, Cout, K = 2, 2, 16384, 16383, 16, 3
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=27)
    return x, w, b


@pytest.mark.parametrize("algo,pool_mode,relu,ceil_mode", [(0, 0, False, False), (1, 0, False, False),
                                                          (3, 0, False, False), (0, 1, True, True)])
def test_conv2d_largest_batch_item(fc, largest_item, algo, pool_mode, relu, ceil_mode):
    x, w, b = largest_item
    B, Cin, H, W = x.shape
    assert Cin * H * W < 2 ** 29 and B * Cin * H * W * 4 > 2 ** 31
    announce(f"conv2d largest batch item x{list(x.shape)} algo={algo} pool_mode={pool_mode} relu={relu} "
             f"ceil={ceil_mode}")
    kw = dict(pool_mode=pool_mode, relu=relu, ceil_mode=ceil_mode)
    xd, wd, bd = dev(x), dev(w), dev(b)
    got_out = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, 4, algo=algo, **kw).cpu().numpy()
    got_map = fc.conv2d_pool_map(xd, wd, bd, 4, algo=algo, **kw)
    del xd
    Bq, Cout, PH, PW = got_map.shape
    rng = np.random.default_rng(28)
    n = 3000
    samp = np.stack([rng.integers(0, Bq, n), rng.integers(0, Cout, n), rng.integers(0, PH, n),
                     rng.integers(0, PW, n)], axis=1)
    corners = [(bb, co, ph, pw) for bb in (0, Bq - 1) for co in (0, Cout - 1) for ph in (0, PH - 1)
               for pw in (0, PW - 1)]
    samp = np.concatenate([samp, np.array(corners)], axis=0)
    want = oracle.conv2d_pooled_at(x, w, b, 4, samp, **kw)
    got = got_map[tuple(torch.from_numpy(samp.T).cuda())].cpu().numpy()
    assert_close(got, want, "sampled pooled map")
    # the literal oracle keeps one full conv map (2.1 GB in double) per thread: 8 threads
    want_out = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4, batch_idx=[1], nthreads=8, **kw)
    # Both forms add at most 1024 fp32 partial sums per batch item (each workgroup walks about 260 tiles
    # here) in a fixed order: their rounding stays within 12 * 2^-24 of |out|, well inside the 1e-4 bar.
    parts = fc.conv2d_det_workspace_bytes(B, Cin, H, W, Cout, w.shape[2], 4, algo, **kw) // (4 * B)
    assert parts == 1024
    det = fc.conv2d_pool_sigmoid_sum_det(dev(x), wd, bd, 4, algo=algo, **kw).cpu().numpy()
    # the pooled-scratch call and the caller-workspace call run the same kernels: identical bits
    assert np.array_equal(got_out.view(np.uint32), det.view(np.uint32))
    for what, got in (("default", got_out), ("caller-workspace", det)):
        err = float(np.abs(got[1] - want_out[0]) / np.abs(want_out[0]))
        print(f"[gpu-case] largest item, {what} out[1]: relative error {err:.3e}", flush=True)
        assert_close(got[[1]], want_out, f"{what} out[1] (second batch item, past 2^31 bytes)")


@pytest.mark.parametrize("algo", [1, 3])
def test_conv2d_no_bias(fc, algo):
    announce(f"conv2d no bias algo={algo}")
    x, w, _ = fi.conv2d_inputs(2, 8, 40, 44, 64, 3, seed=2)
    want = oracle.conv2d_pool_sigmoid_sum(x, w, None, 4)
    got = fc.conv2d_pool_sigmoid_sum(dev(x), dev(w), None, 4, algo=algo).cpu().numpy()
    assert_close(got, want, "out, bias=None")


def test_conv2d_empty_pool_gives_zero(fc):
    announce("conv2d empty pooled map")
    x, w, b = fi.conv2d_inputs(3, 2, 5, 9, 4, 3, seed=3)   # Hc = 3 < pool 4 -> PH = 0
    out = torch.full((3,), 7.0, device="cuda")
    fc.conv2d_pool_sigmoid_sum(dev(x), dev(w), dev(b), 4, out=out)
    assert out.cpu().numpy().tolist() == [0.0, 0.0, 0.0]


def test_conv2d_repeat_calls_overwrite(fc):
    announce("conv2d repeated calls")
    x, w, b = fi.conv2d_inputs(2, 8, 40, 40, 64, 3, seed=4)
    want = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4)
    xd, wd, bd = dev(x), dev(w), dev(b)
    out = torch.full((2,), 1e6, device="cuda")
    for _ in range(3):
        fc.conv2d_pool_sigmoid_sum(xd, wd, bd, 4, out=out)
    assert_close(out.cpu().numpy(), want, "out after 3 calls")


@pytest.mark.parametrize("algo", [1, 2, 3])
def test_conv2d_deterministic(fc, algo):
    announce(f"conv2d deterministic algo={algo}")
    x, w, b = fi.conv2d_inputs(3, 8, 70, 75, 64, 3, seed=6)
    want = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4)
    xd, wd, bd = dev(x), dev(w), dev(b)
    first = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, 4, algo=algo).cpu().numpy()
    ws = torch.full((fc.conv2d_det_workspace_bytes(3, 8, 70, 75, 64, 3, 4, algo) // 4,), float("nan"),
                    device="cuda")
    for _ in range(3):
        again = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, 4, algo=algo, workspace=ws).cpu().numpy()
        assert np.array_equal(first.view(np.uint32), again.view(np.uint32))
    assert_close(first, want, f"deterministic out algo={algo}")


@pytest.mark.parametrize("algo", [0, 1, 2, 3])
def test_conv2d_default_sum_scratch(fc, algo):
    # the fused sum takes its partials' scratch from the library's pool in stream order: repeated calls give
    # identical bits (the caller-workspace call's), and calls on two streams at once each get their own
    announce(f"conv2d default-call scratch, repeats and two streams, algo={algo}")
    shapes = [(3, 8, 70, 75, 64, 3), (5, 4, 41, 90, 20, 3)]
    ins = [fi.conv2d_inputs(*sh, seed=40 + i) for i, sh in enumerate(shapes)]
    devs = [tuple(dev(a) for a in t) for t in ins]
    ref = [fc.conv2d_pool_sigmoid_sum_det(*d, 4, algo=algo).cpu().numpy() for d in devs]
    for i, (x, w, b) in enumerate(ins):
        assert_close(ref[i], oracle.conv2d_pool_sigmoid_sum(x, w, b, 4), f"shape {shapes[i]}")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full((sh[0],), float("nan"), device="cuda") for sh in shapes]
    torch.cuda.synchronize()
    for _ in range(4):
        for d, o, st in zip(devs, outs, streams):
            with torch.cuda.stream(st):
                fc.conv2d_pool_sigmoid_sum(*d, 4, out=o, algo=algo)
    torch.cuda.synchronize()
    for i in range(2):
        assert np.array_equal(outs[i].cpu().numpy().view(np.uint32), ref[i].view(np.uint32)), shapes[i]


def _hip_runtime():
    # the HIP runtime this process already runs on (torch's and the library's)
    import re

    paths = sorted(set(re.findall(r"(/\S*libamdhip64\.so\S*)", open("/proc/self/maps").read())))
    assert paths, "no HIP runtime mapped"
    hip = ctypes.CDLL(paths[0])
    hip.hipStreamCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipStreamDestroy.argtypes = [ctypes.c_void_p]
    return hip


def test_conv2d_default_sum_many_streams(fc):
    # more streams than the library keeps scratch slots for: every call on every stream, three rounds, gives
    # the caller-workspace call's bits (streams past the slots evict the least recently used one)
    announce("conv2d default-call scratch on 12 streams")
    n = 12
    shapes = [(2 + i % 3, 3 + i % 5, 40 + 3 * i, 44 + 2 * i, 8 + 4 * i, 3) for i in range(n)]
    devs = [tuple(dev(a) for a in fi.conv2d_inputs(*sh, seed=60 + i)) for i, sh in enumerate(shapes)]
    ref = [fc.conv2d_pool_sigmoid_sum_det(*d, 4).cpu().numpy() for d in devs]
    streams = [torch.cuda.Stream() for _ in range(n)]
    outs = [[torch.full((sh[0],), float("nan"), device="cuda") for sh in shapes] for _ in range(3)]
    torch.cuda.synchronize()
    for r in range(3):
        for d, o, st in zip(devs, outs[r], streams):
            with torch.cuda.stream(st):
                fc.conv2d_pool_sigmoid_sum(*d, 4, out=o)
    torch.cuda.synchronize()
    for r in range(3):
        for i in range(n):
            assert np.array_equal(outs[r][i].cpu().numpy().view(np.uint32), ref[i].view(np.uint32)), (r, shapes[i])


@pytest.mark.parametrize("nthreads", [4, 12])
def test_conv2d_default_sum_host_threads(fc, nthreads):
    # host threads, each with its own stream, issuing default calls at once through the C ABI (ctypes
    # releases the GIL during a call, so the library's slot table is entered concurrently; with 12 threads
    # there are more streams than slots, so slots pass between streams while others are in use): every
    # output matches the caller-workspace call's bits
    import threading

    announce(f"conv2d default-call scratch from {nthreads} host threads")
    base = [(3, 4, 50, 60, 24, 3), (2, 8, 70, 72, 64, 3), (4, 3, 41, 44, 16, 3), (1, 16, 60, 50, 128, 5)]
    shapes = [base[i % 4][:2] + (base[i % 4][2] + i, base[i % 4][3] + 2 * i) + base[i % 4][4:] for i in range(nthreads)]
    pools = [3 if sh[5] == 5 else 4 for sh in shapes]
    devs = [tuple(dev(a) for a in fi.conv2d_inputs(*sh, seed=80 + i)) for i, sh in enumerate(shapes)]
    ref = [fc.conv2d_pool_sigmoid_sum_det(*d, pl).cpu().numpy() for d, pl in zip(devs, pools)]
    streams = [torch.cuda.Stream() for _ in shapes]
    rounds = 25
    outs = [[torch.full((sh[0],), float("nan"), device="cuda") for _ in range(rounds)] for sh in shapes]
    torch.cuda.synchronize()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    errors = []

    def worker(i):
        sh, d, st = shapes[i], devs[i], ctypes.c_void_p(streams[i].cuda_stream)
        for r in range(rounds):
            rc = fc.lib.fconv2d_pool_sigmoid_sum(P(d[0]), sh[0], sh[1], sh[2], sh[3], P(d[1]), sh[4], sh[5],
                                                 P(d[2]), pools[i], P(outs[i][r]), st)
            if rc != 0:
                errors.append((i, r, rc))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(shapes))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i in range(len(shapes)):
        for r in range(rounds):
            assert np.array_equal(outs[i][r].cpu().numpy().view(np.uint32), ref[i].view(np.uint32)), (i, r)


def test_conv2d_default_sum_reused_stream_handle(fc):
    # a stream destroyed with calls still queued, and a new stream that gets the same handle: the new
    # stream's call must not overlap the old stream's use of that handle's scratch
    announce("conv2d default-call scratch across a destroyed and re-created stream handle")
    hip = _hip_runtime()
    sh1, sh2 = (16, 8, 256, 256, 64, 3), (6, 5, 120, 90, 24, 3)
    d1 = tuple(dev(a) for a in fi.conv2d_inputs(*sh1, seed=70))
    d2 = tuple(dev(a) for a in fi.conv2d_inputs(*sh2, seed=71))
    ref1 = fc.conv2d_pool_sigmoid_sum_det(*d1, 4).cpu().numpy()
    ref2 = fc.conv2d_pool_sigmoid_sum_det(*d2, 4).cpu().numpy()
    outs1 = [torch.full((sh1[0],), float("nan"), device="cuda") for _ in range(4)]
    out2 = torch.full((sh2[0],), float("nan"), device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    call = lambda d, sh, o, st: fc.lib.fconv2d_pool_sigmoid_sum(P(d[0]), sh[0], sh[1], sh[2], sh[3], P(d[1]), sh[4],
                                                               sh[5], P(d[2]), 4, P(o), st)
    torch.cuda.synchronize()
    handles = []
    for rep in range(3):
        a = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(a)) == 0
        for o in outs1:
            assert call(d1, sh1, o, a) == 0
        assert hip.hipStreamDestroy(a) == 0  # calls may still be queued
        b = ctypes.c_void_p()
        assert hip.hipStreamCreate(ctypes.byref(b)) == 0
        handles.append((a.value, b.value))
        assert call(d2, sh2, out2, b) == 0
        torch.cuda.synchronize()
        assert hip.hipStreamDestroy(b) == 0
        for o in outs1:
            assert np.array_equal(o.cpu().numpy().view(np.uint32), ref1.view(np.uint32)), rep
        assert np.array_equal(out2.cpu().numpy().view(np.uint32), ref2.view(np.uint32)), rep
        for o in outs1 + [out2]:
            o.fill_(float("nan"))
    print(f"[gpu-case] stream handles (destroyed, new): {handles}", flush=True)


FULL_CONV = {
    "conv2d_full": [0, 1, 63, 64, 126, 127],
    "conv2d_tail": [0, 31, 62, 63],
}


@pytest.fixture(scope="module")
def full_conv_inputs():
    return {name: fi.make(name, seed=0) for name in FULL_CONV}


@pytest.mark.parametrize("algo", [1, 3])
@pytest.mark.parametrize("name", list(FULL_CONV))
def test_conv2d_full_size(fc, full_conv_inputs, name, algo):
    cfg = fi.WORKLOADS[name]
    s = cfg["pool"]
    x, w, b = full_conv_inputs[name]
    announce(f"conv2d full size {name} algo={algo}")
    xd, wd, bd = dev(x), dev(w), dev(b)
    got_out = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=algo).cpu().numpy()
    got_map = fc.conv2d_pool_map(xd, wd, bd, s, algo=algo).cpu().numpy()
    # whole batch items through the literal oracle
    idx = FULL_CONV[name]
    want_out = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, batch_idx=idx)
    assert_close(got_out[idx], want_out, f"{name} out[{idx}]")
    # the sum over the pooled map the kernels wrote equals the fused sums
    sig = (1.0 / (1.0 + np.exp(-got_map.astype(np.float64)))).sum(axis=(1, 2, 3))
    assert_close(got_out, sig, f"{name} fused sum vs sigmoid(map) sum")
    # sampled pooled values: random, plus every corner / edge / tile seam
    B, Cout, PH, PW = got_map.shape
    rng = np.random.default_rng(5)
    n = 20000
    samp = np.stack([rng.integers(0, B, n), rng.integers(0, Cout, n), rng.integers(0, PH, n),
                     rng.integers(0, PW, n)], axis=1)
    edge = [0, 1, 3, 4, 7, 8, 11, 12, 15, 16, PH - 2, PH - 1]
    extra = [(bb, co, ph, pw) for bb in (0, B - 1) for co in (0, Cout - 1)
             for ph in edge for pw in edge if ph < PH and pw < PW]
    samp = np.concatenate([samp, np.array(extra)], axis=0)
    want = oracle.conv2d_pooled_at(x, w, b, s, samp)
    assert_close(got_map[tuple(samp.T)], want, f"{name} sampled pooled map")


@pytest.mark.parametrize("algo", [1, 3])
@pytest.mark.parametrize("name", list(FULL_CONV))
def test_conv2d_full_size_closed_forms(fc, full_conv_inputs, name, algo):
    cfg = fi.WORKLOADS[name]
    s = cfg["pool"]
    x, w, b = full_conv_inputs[name]
    announce(f"conv2d full size closed forms {name} algo={algo}")
    B, Cin, H, W = x.shape
    Cout = w.shape[0]
    PH, PW = fc.conv2d_out_size(H, W, w.shape[2], s)
    xd = dev(x)
    # zero weights and bias: sigmoid(0) = 1/2 everywhere, exactly representable sums
    z = fc.conv2d_pool_sigmoid_sum(xd, torch.zeros_like(dev(w)), torch.zeros(Cout, device="cuda"), s, algo=algo)
    assert (z.cpu().numpy() == Cout * PH * PW / 2.0).all()
    # sigma symmetry: negating w and b gives Cout*PH*PW - out
    wd, bd = dev(w), dev(b)
    pos = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=algo).cpu().numpy().astype(np.float64)
    neg = fc.conv2d_pool_sigmoid_sum(xd, -wd, -bd, s, algo=algo).cpu().numpy().astype(np.float64)
    assert_close(pos + neg, np.full(B, float(Cout * PH * PW)), f"{name} sigma symmetry")
    # the caller-workspace form repeats bit for bit and gives the default call's bits
    d1 = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, algo=algo).cpu().numpy()
    d2 = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, algo=algo).cpu().numpy()
    assert np.array_equal(d1.view(np.uint32), d2.view(np.uint32))
    assert np.array_equal(d1.view(np.uint32), pos.astype(np.float32).view(np.uint32)), f"{name} det vs default"


# ------------------------------------------------------------------ depthwise-separable path

SMALL_DW = [
    # B, C, T, O, K, pad
    (4, 16, 256, 32, 9, 4),     # the small workload
    (2, 256, 300, 512, 9, 4),   # big instance, ragged T
    (2, 64, 200, 200, 9, 4),    # mid instance, O not a multiple of 16
    (3, 10, 77, 33, 9, 4),      # C not a multiple of 4 (scalar weight loads)
    (1, 48, 70, 300, 5, 0),     # no padding, big instance with masked channels
    (2, 20, 40, 24, 3, 7),      # pad > K: Tout > T
    (1, 8, 5, 16, 9, 4),        # T < K
    (2, 100, 129, 70, 1, 0),    # 1-tap depthwise (pure GEMM), C not a multiple of 16
    (1, 300, 64, 64, 9, 4),     # C spans several chunks with a partial last chunk
]


@pytest.mark.parametrize("shape", SMALL_DW)
def test_dwsep_small(fc, shape):
    B, C, T, O, K, pad = shape
    announce(f"dwsep small {shape}")
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=7)
    want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad)
    got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), pad).cpu().numpy()
    assert_close(got, want, f"y {shape}")


TALL_DW = [
    # B, C, T, O, K, pad: O > 256 at stride 1 runs the 512 x 64 tile
    (2, 200, 130, 520, 9, 4),    # 3 full chunks + an 8-channel chunk (half a group), 2 output tiles
    (1, 68, 64, 257, 33, 16),    # runtime K, a 4-channel last chunk, one valid row in the 2nd block
    (1, 64, 100, 300, 64, 32),   # the widest window the tile takes (K = 64: 8 full blocks of 8 taps)
    (1, 64, 100, 300, 65, 32),   # one wider: the wide-window instance (three staged runs per row)
    (1, 36, 300, 300, 128, 64),  # the widest window the wide-window instance stages
    (1, 36, 300, 200, 129, 64),  # one wider: the 256-row runtime-K kernel
    (2, 35, 200, 100, 100, 50),  # wide window, 128 rows, C % 4 != 0
    (1, 36, 300, 60, 100, 50),   # wide window, 64 rows
    (1, 13, 300, 9, 128, 64),    # the widest window on a 32-row tile
    (2, 36, 130, 512, 5, 2),     # runtime K inside one block of 8 taps
    (1, 40, 96, 300, 8, 3),      # exactly one block, even K (asymmetric padding)
    (1, 24, 80, 384, 17, 8),     # a last block with one tap
    (2, 16, 50, 512, 9, 0),      # a single partial chunk, T < 64, no padding
    (1, 32, 70, 300, 1, 0),      # 1-tap depthwise
    (1, 44, 200, 1100, 3, 1),    # three output tiles, C not a multiple of 16
    # 64 < O <= 256: the same kernel with 256-row (waves of 32 x 64) and 128-row (16 x 64) tiles
    (2, 200, 130, 256, 9, 4),    # 256 rows exactly, 3 full chunks + an 8-channel chunk, a ragged time tile
    (1, 68, 100, 129, 9, 4),     # 256-row tile with one valid row in its fifth wave, a 4-channel chunk
    (1, 64, 100, 200, 64, 32),   # 256-row tile, the widest window
    (1, 36, 64, 128, 5, 2),      # 128 rows exactly, runtime K
    (2, 44, 150, 65, 9, 4),      # 128-row tile with one valid row in its fifth wave
    (1, 100, 80, 100, 17, 8),    # 128-row tile, runtime K, chunks of 64 + 36 channels
    # O <= 64: 64-row tiles (4 waves, 32-channel chunks) and 32-row tiles (2 waves, 16-channel chunks)
    (2, 36, 130, 64, 9, 4),      # 64 rows exactly, chunks of 32 + 4 channels, a ragged time tile
    (1, 40, 100, 33, 5, 2),      # 64-row tile with one valid row in its third wave, runtime K
    (2, 16, 70, 32, 9, 4),       # 32 rows exactly, one chunk
    (1, 20, 64, 1, 3, 1),        # a single output channel: 32-row tile, runtime K, chunks of 16 + 4
    (1, 64, 100, 17, 64, 32),    # the widest window on a 32-row tile
    # C not a multiple of 4: the runtime-K instances with 4-byte weight loads, at every tile height
    (2, 201, 130, 520, 9, 4),    # 512 rows, chunks of 64 x 3 + 9 (a group of 9 channels)
    (1, 67, 100, 300, 33, 16),   # 512 rows, runtime K, a 3-channel last chunk
    (1, 63, 100, 300, 64, 32),   # 512 rows, the widest window, one chunk one channel short
    (2, 45, 150, 256, 5, 2),     # 256 rows exactly
    (1, 101, 80, 129, 17, 8),    # 256 rows, one valid row in the fifth wave
    (2, 30, 70, 100, 9, 4),      # 128 rows, a 14-channel group
    (1, 1, 64, 65, 3, 1),        # one channel
    (1, 37, 100, 64, 9, 4),      # 64 rows exactly
    (2, 3, 70, 20, 5, 2),        # 32 rows, three channels
    (1, 13, 64, 1, 1, 0),        # one output channel, 1-tap depthwise
]


def test_dwsep_widest_windows(fc):
    # the runtime-K kernels up to the widest depthwise window their LDS tile stages, then refusal:
    # every supported K is checked against the oracle, and support ends at one K (no gaps)
    announce("dwsep widest windows")
    supported = []
    for K in (66, 129, 257, 400, 480, 500, 520, 600, 1000, 4000):
        B, C, T, O, pad = 1, 8, K + 40, 300, K // 2
        x, wd, wp, bp = fi.dwsep_inputs(B, C, T, O, K, seed=26)
        try:
            got = fc.dwsep_conv1d(dev(x), dev(wd), dev(wp), dev(bp), pad).cpu().numpy()
        except fc.FconvError as e:
            assert e.status == fc.FCONV_EUNSUPPORTED, K
            continue
        supported.append(K)
        assert_close(got, oracle.dwsep_conv1d(x, wd, wp, bp, pad), f"dwsep K={K}")
    assert supported and supported[0] == 66 and 400 in supported, supported
    assert supported == [k for k in (66, 129, 257, 400, 480, 500, 520, 600, 1000, 4000) if k <= supported[-1]]
    assert 4000 not in supported


@pytest.mark.parametrize("shape", TALL_DW)
def test_dwsep_tall_tile(fc, shape):
    B, C, T, O, K, pad = shape
    announce(f"dwsep tall tile {shape}")
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=13)
    want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad)
    got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), pad).cpu().numpy()
    assert_close(got, want, f"y {shape}")


@pytest.mark.parametrize("O", [300, 200, 100, 48, 20])
def test_dwsep_tall_tile_every_k(fc, O):
    # every depthwise width the tall tile takes (K = 1 .. 64; K = 9 is its compiled instance, the rest run
    # the runtime-K stage over blocks of 8 taps; K = 65 .. 128 the wide-window instances with one more
    # staged run), with odd and even padding and a partial channel chunk, against the oracle, for its
    # 512-, 256-, 128-, 64- and 32-row tiles; K = 129 goes to the older kernels and is checked the same way
    announce(f"dwsep tall tile, K = 1 .. 129, O = {O}")
    B, C, T = 1, 36, 100
    for K in range(1, 130):
        pad = K // 2 if K % 3 else (K - 1) // 2
        x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=300 + K)
        want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad)
        got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), pad).cpu().numpy()
        assert_close(got, want, f"y K={K} pad={pad}")


@pytest.mark.parametrize("dil", [3, 5, 6])
def test_dwsep_tall_tile_any_dilation_every_k(fc, dil):
    # every K the tall tile's tap-by-tap instances take at this dilation ((K - 1) * dil <= 63, and up to
    # 127 with one more staged run), and the first K past them, with odd and even padding, against the oracle
    announce(f"dwsep tall tile, dilation {dil}, every K")
    B, C, T, O = 1, 36, 100, 300
    for K in range(1, 127 // dil + 3):
        pad = (K - 1) * dil // 2 if K % 2 else (K - 2) * dil // 2
        x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=400 + K)
        want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad, dilation=dil)
        got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), pad, dilation=dil).cpu().numpy()
        assert_close(got, want, f"y K={K} pad={pad} dil={dil}")


@pytest.mark.parametrize("C", [36, 35])
def test_dwsep_tall_tile_inf_in_next_row(fc, C):
    # Padded channels of a partial group must form no product: an infinite
    # weight in row o+1 may not reach row o (with C = 35 that weight sits
    # right after row o's last channel).
    announce(f"dwsep tall tile, inf weight next to a partial group, C={C}")
    B, T, O, K, pad = 1, 64, 300, 9, 4
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=14)
    w_pw = w_pw.copy()
    w_pw[101, 0] = np.inf
    got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), pad).cpu().numpy()
    rows = [o for o in range(O) if o != 101]
    want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad)
    assert np.isfinite(got[:, rows]).all()
    assert_close(got[:, rows], want[:, rows], "finite rows")


STRIDED_DW = [
    # B, C, T, O, K, pad, stride, dilation
    (2, 64, 300, 300, 9, 4, 2, 1),     # stride 2: the tall tile's stride-2 K = 9 instance, 512 rows
    (1, 48, 257, 512, 9, 8, 1, 2),     # dilation 2: the tall tile's dilated instance, 512 rows
    (2, 20, 100, 40, 5, 3, 3, 2),      # stride 3, dilation 2, O = 40: the 64-row tile
    (1, 16, 2000, 128, 9, 4, 16, 1),   # window too wide for 64 steps: narrow instance
    (1, 32, 40, 64, 3, 0, 5, 4),       # few output steps (stride 5, dilation 4: a 64-row tile)
    # the tall tile's dilated instances: dilation 2, 4 and 8 on 512-, 256- and 128-row tiles, up to the
    # widest window it stages ((K - 1) * dilation = 63), and one past it (the 256-row kernel)
    (2, 36, 150, 300, 5, 8, 1, 4),     # dilation 4, blocks of 2 taps, a ragged time tile, a partial chunk
    (1, 64, 130, 200, 8, 28, 1, 8),    # dilation 8, one tap per block, 256 rows
    (1, 100, 120, 100, 32, 31, 1, 2),  # dilation 2, (K - 1) * dil = 62, 128 rows, chunks of 64 + 36
    (1, 40, 140, 300, 16, 30, 1, 4),   # dilation 4, (K - 1) * dil = 60
    (1, 40, 140, 300, 17, 32, 1, 4),   # (K - 1) * dil = 64: the wide-window instance
    # any other dilation: the tall tile's tap-by-tap instances
    (1, 32, 90, 300, 9, 12, 1, 3),     # dilation 3, 512 rows
    (2, 35, 150, 300, 5, 6, 1, 3),     # dilation 3, a ragged time tile, C % 4 != 0
    (1, 68, 140, 200, 10, 27, 1, 7),   # dilation 7, (K - 1) * dil = 63, 256 rows
    (1, 30, 120, 100, 4, 10, 1, 21),   # dilation 21, (K - 1) * dil = 63, 128 rows
    (1, 33, 100, 129, 7, 18, 1, 6),    # dilation 6, 256 rows with one valid row in the fifth wave
    (1, 40, 140, 300, 23, 33, 1, 3),   # (K - 1) * dil = 66: the wide-window instance, tap by tap
    (1, 36, 300, 200, 43, 63, 1, 3),   # (K - 1) * dil = 126, 256 rows
    (1, 36, 300, 100, 17, 64, 1, 8),   # (K - 1) * dil = 128: past the wide window, the 256-row kernel
    # stride 3: four staged runs per row, one workgroup per CU
    (2, 36, 400, 300, 9, 4, 3, 1),     # K = 9, 512 rows, a ragged last time tile
    (1, 35, 257, 200, 5, 2, 3, 1),     # runtime K, 256 rows, C % 4 != 0
    (1, 68, 300, 100, 64, 32, 3, 1),   # the widest window it stages, 128 rows, chunks of 64 + 4
    (1, 40, 300, 520, 65, 32, 3, 1),   # one wider: the 256-row kernel
    (1, 16, 200, 40, 9, 4, 3, 1),      # O = 40 on the 64-row tile
    # stride 2 with a dilation: the dilated stages on three staged runs
    (2, 36, 300, 300, 9, 8, 2, 2),     # dilation 2, K = 9, 512 rows, a ragged last time tile
    (1, 35, 260, 200, 16, 30, 2, 4),   # dilation 4, (K - 1) * dil = 60, 256 rows, C % 4 != 0
    (1, 64, 200, 100, 8, 28, 2, 8),    # dilation 8, one tap per block, 128 rows
    (1, 40, 300, 300, 22, 31, 2, 3),   # dilation 3, (K - 1) * dil = 63, tap by tap
    (2, 20, 180, 40, 7, 15, 2, 5),     # dilation 5, O = 40 on the 64-row tile
    (1, 24, 300, 300, 17, 32, 2, 4),   # (K - 1) * dil = 64: past the tall tile, the 256-row kernel
    # stride 5: six staged runs per row; stride 6 goes to the 256-row kernel
    (2, 36, 650, 300, 9, 4, 5, 1),     # K = 9, 512 rows, a ragged last time tile
    (1, 35, 500, 200, 64, 32, 5, 1),   # the widest window it stages, 256 rows, C % 4 != 0
    (1, 20, 400, 40, 7, 9, 5, 3),      # dilation 3 (tap by tap), 64 rows
    (1, 24, 500, 300, 65, 32, 5, 1),   # one wider: the 256-row kernel
    (1, 16, 300, 100, 9, 4, 6, 1),     # stride 6: the 256-row kernel
    # strides 3 and 4 with a dilation
    (2, 36, 500, 300, 9, 8, 3, 2),     # stride 3, dilation 2, 512 rows (256-VGPR budget)
    (1, 35, 400, 200, 10, 27, 3, 7),   # stride 3, dilation 7, (K - 1) * dil = 63, tap by tap, 256 rows
    (1, 64, 600, 300, 8, 28, 4, 8),    # stride 4, dilation 8, one tap per block, 512 rows
    (1, 30, 500, 100, 22, 31, 4, 3),   # stride 4, dilation 3, (K - 1) * dil = 63, 128 rows
    (1, 24, 500, 300, 17, 32, 3, 4),   # (K - 1) * dil = 64: past the tall tile, the 256-row kernel
    # stride 4: five staged runs per row
    (2, 36, 520, 300, 9, 4, 4, 1),     # K = 9, 512 rows, a ragged last time tile
    (1, 33, 300, 256, 7, 3, 4, 1),     # runtime K, 256 rows exactly, C % 4 != 0
    (1, 64, 400, 65, 64, 32, 4, 1),    # the widest window it stages, 128 rows with one valid row in the 5th wave
    (1, 24, 400, 300, 65, 32, 4, 1),   # one wider: the 256-row kernel
    # O <= 64 with a stride, a dilation or both: the 64- and 32-row tiles of each instance
    (1, 33, 400, 50, 9, 4, 4, 1),      # stride 4, K = 9, 64 rows
    (2, 20, 300, 17, 5, 8, 3, 3),      # stride 3, dilation 3 (tap by tap), 32 rows
    (1, 36, 200, 30, 17, 32, 1, 4),    # dilation 4, (K - 1) * dil = 64 (one more staged run), 32 rows
    (1, 24, 300, 48, 9, 16, 2, 4),     # stride 2, dilation 4, 64 rows
    (2, 36, 130, 40, 9, 8, 1, 2),      # dilation 2, O = 40
    (1, 35, 131, 64, 5, 2, 2, 1),      # stride 2, O = 64, runtime K, C % 4 != 0
    (1, 20, 100, 7, 7, 9, 1, 3),       # dilation 3, O = 7
    (2, 16, 200, 1, 9, 4, 2, 1),       # stride 2, K = 9, one output channel
    # the tall tile at stride 2 (three staged runs per row, the epilogue staged through xs and Ds)
    (1, 36, 257, 200, 5, 2, 2, 1),     # runtime K, 256 rows, an odd T (ragged last time tile)
    (2, 68, 131, 100, 9, 4, 2, 1),     # K = 9, 128 rows, chunks of 64 + 4 channels
    (1, 40, 300, 520, 64, 32, 2, 1),   # the widest window it stages, two 512-row tiles
    (1, 40, 300, 520, 65, 32, 2, 1),   # one wider: the 256-row kernel
]


@pytest.mark.parametrize("shape", STRIDED_DW)
def test_dwsep_strided_dilated(fc, shape):
    B, C, T, O, K, pad, stride, dil = shape
    announce(f"dwsep strided/dilated {shape}")
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=11)
    want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad, stride=stride, dilation=dil)
    got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), pad, stride=stride, dilation=dil).cpu().numpy()
    assert_close(got, want, f"y {shape}")


DENSE_DW = [
    # B, C, T, O, K, pad, stride, dilation
    (4, 16, 256, 32, 9, 4, 1, 1),      # the small workload
    (2, 100, 150, 70, 9, 4, 1, 1),     # C not a multiple of 16, O ragged
    (1, 64, 200, 300, 5, 2, 2, 2),     # strided and dilated
    (2, 48, 260, 520, 9, 4, 1, 1),     # whole tiles through the staged 16-byte stores; ragged last time and O tiles
]


@pytest.mark.parametrize("shape", DENSE_DW)
def test_dwsep_dense_variant(fc, shape):
    B, C, T, O, K, pad, stride, dil = shape
    announce(f"dwsep dense {shape}")
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=12)
    want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad, stride=stride, dilation=dil)
    args = (dev(x), dev(w_dw), dev(w_pw), dev(b_pw), pad)
    dense = fc.dwsep_conv1d(*args, stride=stride, dilation=dil, algo=fc.DWSEP_DENSE).cpu().numpy()
    sep = fc.dwsep_conv1d(*args, stride=stride, dilation=dil, algo=fc.DWSEP_SEPARABLE).cpu().numpy()
    assert_close(dense, want, f"dense y {shape}")
    assert_close(dense, sep, f"dense vs separable {shape}")


def test_dwsep_dense_full_size_sampled(fc):
    announce("dwsep dense full size")
    cfg = fi.WORKLOADS["dwsep_full"]
    x, w_dw, w_pw, b_pw = fi.make("dwsep_full", seed=0)
    got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), cfg["pad"], algo=fc.DWSEP_DENSE).cpu().numpy()
    rng = np.random.default_rng(8)
    samp = np.stack([rng.integers(0, n, 5000) for n in got.shape], axis=1)
    want = oracle.dwsep_conv1d_at(x, w_dw, w_pw, b_pw, cfg["pad"], samp)
    assert_close(got[tuple(samp.T)], want, "dense sampled")


def test_dwsep_stride2_full_size_sampled(fc):
    # stride 2 over x[32,256,8192] -> 512 (Tout 4096, the dwsep_full output): the tall tile's stride-2
    # instance at full size, 5000 sampled outputs with the padded edges against the oracle
    announce("dwsep stride 2 full size")
    B, C, T, O, K, pad = 32, 256, 8192, 512, 9, 4
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=41)
    got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), pad, stride=2).cpu().numpy()
    assert got.shape == (B, O, 4096)
    rng = np.random.default_rng(9)
    samp = np.stack([rng.integers(0, n, 5000) for n in got.shape], axis=1)
    samp[:100, 2] = 0
    samp[100:200, 2] = got.shape[2] - 1
    want = oracle.dwsep_conv1d_at(x, w_dw, w_pw, b_pw, pad, samp, stride=2)
    assert_close(got[tuple(samp.T)], want, "stride 2 sampled")


def test_dwsep_no_bias_and_torch_shapes(fc):
    announce("dwsep no bias, [C,1,K] and [O,C,1] weights")
    x, w_dw, w_pw, _ = fi.dwsep_inputs(2, 32, 100, 48, 9, seed=8)
    want = oracle.dwsep_conv1d(x, w_dw, w_pw, None, 4)
    got = fc.dwsep_conv1d(dev(x), dev(w_dw[:, None, :]), dev(w_pw[:, :, None]), None, 4).cpu().numpy()
    assert_close(got, want, "y no bias")


@pytest.mark.parametrize("O", [32, 48, 100, 200, 300])
def test_dwsep_unaligned_weights(fc, O):
    # w_pw starting 4 bytes past a 16-byte boundary takes the 4-byte weight loads.
    announce(f"dwsep unaligned w_pw, O={O}")
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(1, 32, 64, O, 9, seed=9)
    want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, 4)
    buf = torch.zeros(w_pw.size + 1, device="cuda")
    buf[1:] = dev(w_pw).reshape(-1)
    wp = buf[1:].view(O, 32)
    got = fc.dwsep_conv1d(dev(x), dev(w_dw), wp, dev(b_pw), 4).cpu().numpy()
    assert_close(got, want, "y unaligned")


@pytest.mark.parametrize("dense", [False, True])
@pytest.mark.parametrize("offset", [1, 2, 3])
def test_dwsep_unaligned_output(fc, offset, dense):
    # y starting 4, 8 or 12 bytes past a 16-byte boundary (Tout a multiple of 4): the tall tile (and the
    # dense-fused kernel's) stores element by element instead of in 16-byte rows; the elements around y
    # stay untouched
    announce(f"dwsep unaligned y, offset {offset} floats, dense {dense}")
    B, C, T, O, K, pad = 2, 40, 128, 300, 9, 4
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(B, C, T, O, K, seed=10 + offset)
    want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, pad)
    n = B * O * T
    buf = torch.full((n + 8,), 7.0, device="cuda")
    y = buf[offset:offset + n].view(B, O, T)
    fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), pad, out=y,
                    algo=fc.DWSEP_DENSE if dense else fc.DWSEP_SEPARABLE)
    assert_close(y.cpu().numpy(), want, f"y offset {offset}")
    rest = torch.cat([buf[:offset], buf[offset + n:]]).cpu().numpy()
    assert (rest == 7.0).all()


def test_dwsep_full_size(fc):
    name = "dwsep_full"
    cfg = fi.WORKLOADS[name]
    announce(f"dwsep full size {name}")
    x, w_dw, w_pw, b_pw = fi.make(name, seed=0)
    got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), cfg["pad"]).cpu().numpy()
    # whole batch items
    for bi in (0, 31):
        want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, cfg["pad"], batch_idx=[bi])[0]
        assert_close(got[bi], want, f"{name} y[{bi}]")
    # sampled outputs over all items, with the padded edges
    B, O, Tout = got.shape
    rng = np.random.default_rng(6)
    n = 30000
    samp = np.stack([rng.integers(0, B, n), rng.integers(0, O, n), rng.integers(0, Tout, n)], axis=1)
    edge = np.array([(bb, o, t) for bb in range(0, B, 5) for o in (0, 255, 511) for t in (0, 1, 3, 4, 63, 64,
                                                                                         Tout - 5, Tout - 1)])
    samp = np.concatenate([samp, edge])
    want = oracle.dwsep_conv1d_at(x, w_dw, w_pw, b_pw, cfg["pad"], samp)
    assert_close(got[tuple(samp.T)], want, f"{name} sampled")


def test_dwsep_full_size_linearity(fc):
    announce("dwsep full size linearity")
    cfg = fi.WORKLOADS["dwsep_full"]
    x, w_dw, w_pw, b_pw = fi.make("dwsep_full", seed=0)
    x2 = fi.normal(x.shape, 17, 0)
    wd, wp = dev(w_dw), dev(w_pw)
    y1 = fc.dwsep_conv1d(dev(x), wd, wp, None, cfg["pad"])
    y2 = fc.dwsep_conv1d(dev(x2), wd, wp, None, cfg["pad"])
    ys = fc.dwsep_conv1d(dev(x) * 0.5 - dev(x2) * 2.0, wd, wp, None, cfg["pad"])
    diff = (ys - (0.5 * y1 - 2.0 * y2)).abs().max().item()
    scale = ys.abs().max().item()
    assert diff <= 1e-4 * max(1.0, scale), (diff, scale)
