"""GPU parity on seeded random shapes: every algorithm and pool form of the
Conv2d chain and every dwsep algorithm, against the CPU oracle.

The fixed cases elsewhere pin each kernel instance at chosen edges; these
draw (B, Cin, H, W, Cout, K, s, pool form, algorithm) and (B, C, T, O, K,
pad, stride, dilation, algorithm) from seeded generators, so shapes no
one picked (odd channel counts, maps of one pooled row, tiles cut anywhere,
empty pooled maps) meet the same bar: |gpu - oracle| <= 1e-4 + 1e-4*|oracle|
on the pooled map, the fused sums and y.  A combination with no kernel must
come back as FCONV_EUNSUPPORTED, never as a wrong result.
"""

import sys

import numpy as np
import pytest

import fconv_inputs as fi
import oracle

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

RTOL = ATOL = 1e-4
AVG, MAX = oracle.POOL_AVG, oracle.POOL_MAX
# (K, s) with a matrix-core instance (direct and box-sum)
MFMA_INSTANCES = {(3, 4), (3, 2), (3, 3), (5, 3)}


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


def conv_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        K, s = [(3, 4), (3, 2), (3, 3), (5, 3), (3, 4), (5, 3), (1, 3), (2, 2), (7, 2), (3, 5)][rng.integers(10)]
        H = int(rng.integers(K, K + s * 14 + 9))
        W = int(rng.integers(K, K + s * 40 + 9))
        # two in five are the plain chain (average pool, no ReLU, floor), the only form box-sum takes
        plain = rng.random() < 0.4
        # channel counts up to past the whole-tile LDS budgets (channel-chunked tilings) and up to
        # three output-channel ranges
        cases.append(dict(B=int(rng.integers(1, 4)), Cin=int(rng.integers(1, 81)), H=H, W=W,
                          Cout=int(rng.integers(1, 261)), K=K, s=s,
                          pool_mode=AVG if plain else [AVG, MAX][rng.integers(2)],
                          relu=False if plain else bool(rng.integers(2)),
                          ceil_mode=False if plain else bool(rng.integers(2)), algo=int(rng.integers(4))))
    return cases


def dw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        K = int(rng.integers(1, 18))
        stride = [1, 1, 1, 2, 3][rng.integers(5)]
        dil = [1, 1, 2][rng.integers(3)]
        pad = int(rng.integers(0, K + 1))
        T = int(rng.integers(1, 301))
        if oracle.dwsep_tout(T, K, pad, stride, dil) < 1:
            continue
        cases.append(dict(B=int(rng.integers(1, 4)), C=int(rng.integers(1, 301)), T=T,
                          O=int(rng.integers(1, 601)), K=K, pad=pad, stride=stride, dil=dil,
                          algo=int(rng.integers(3))))
    return cases


def dw_cases_wide(n, seed):
    # strides 1 to 5 and dilations 1 to 5 in every combination, windows up to past 64 steps: the tall
    # tile's stride and dilation instances and their handover to the 256-row kernel
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        stride = int(rng.integers(1, 6))
        dil = int(rng.integers(1, 6))
        K = int(rng.integers(1, 80 // dil + 2))
        pad = int(rng.integers(0, (K - 1) * dil // 2 + 2))
        T = int(rng.integers(1, 400))
        if oracle.dwsep_tout(T, K, pad, stride, dil) < 1:
            continue
        cases.append(dict(B=int(rng.integers(1, 3)), C=int(rng.integers(1, 130)), T=T,
                          O=int(rng.integers(1, 601)), K=K, pad=pad, stride=stride, dil=dil, algo=0))
    return cases


CONV_CASES = conv_cases(160, seed=2024)
DW_CASES = dw_cases(120, seed=2025) + dw_cases_wide(80, seed=2026)


def conv_id(c):
    return "B{B}-Cin{Cin}-{H}x{W}-Cout{Cout}-K{K}s{s}-{pm}{relu}{ceil}-a{algo}".format(
        pm="max" if c["pool_mode"] == MAX else "avg", relu="-relu" if c["relu"] else "",
        ceil="-ceil" if c["ceil_mode"] else "", **{k: v for k, v in c.items() if k not in ("relu", "ceil_mode")})


@pytest.mark.parametrize("case", CONV_CASES, ids=conv_id)
def test_conv2d_random_shape(fc, case):
    c = case
    announce(f"conv2d random {conv_id(c)}")
    plain = c["pool_mode"] == AVG and not c["relu"] and not c["ceil_mode"]
    mfma = (c["K"], c["s"]) in MFMA_INSTANCES
    supported = c["algo"] in (0, 2) or (c["algo"] == 1 and mfma) or (c["algo"] == 3 and mfma and plain)
    x, w, b = fi.conv2d_inputs(c["B"], c["Cin"], c["H"], c["W"], c["Cout"], c["K"], seed=77)
    xd, wd, bd = dev(x), dev(w), dev(b)
    kw = dict(algo=c["algo"], pool_mode=c["pool_mode"], relu=c["relu"], ceil_mode=c["ceil_mode"])
    if not supported:
        with pytest.raises(fc.FconvError) as err:
            fc.conv2d_pool_sigmoid_sum(xd, wd, bd, c["s"], **kw)
        assert err.value.status == fc.FCONV_EUNSUPPORTED
        return
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, c["s"], want_pooled=True,
                                                        pool_mode=c["pool_mode"], relu=c["relu"],
                                                        ceil_mode=c["ceil_mode"])
    got_map = fc.conv2d_pool_map(xd, wd, bd, c["s"], **kw).cpu().numpy()
    got_out = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, c["s"], **kw).cpu().numpy()
    assert_close(got_map, want_map, f"pooled map {conv_id(c)}")
    assert_close(got_out, want_out, f"out {conv_id(c)}")
    if plain:
        det = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, c["s"], algo=c["algo"]).cpu().numpy()
        assert np.array_equal(det.view(np.uint32), got_out.view(np.uint32)), "default and caller-workspace sums differ"


def dw_id(c):
    return "B{B}-C{C}-T{T}-O{O}-K{K}p{pad}s{stride}d{dil}-a{algo}".format(**c)


@pytest.mark.parametrize("case", DW_CASES, ids=dw_id)
def test_dwsep_random_shape(fc, case):
    c = case
    announce(f"dwsep random {dw_id(c)}")
    x, w_dw, w_pw, b_pw = fi.dwsep_inputs(c["B"], c["C"], c["T"], c["O"], c["K"], seed=78)
    want = oracle.dwsep_conv1d(x, w_dw, w_pw, b_pw, c["pad"], stride=c["stride"], dilation=c["dil"])
    got = fc.dwsep_conv1d(dev(x), dev(w_dw), dev(w_pw), dev(b_pw), c["pad"], stride=c["stride"],
                          dilation=c["dil"], algo=c["algo"]).cpu().numpy()
    assert_close(got, want, f"y {dw_id(c)}")
