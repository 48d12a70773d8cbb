"""GPU checks beyond the seed-0 parity cases.

- Every workload with seeds 1 and 2 against the oracle (whole items for the
  small workloads; first and last items plus sampled outputs at full size).
- Full-size invariants that need no oracle: batch independence (bit for bit
  in the deterministic Conv2d form and in dwsep), and invariance under a
  permutation of the output channels.
- Canary-padded outputs: every call writes exactly its output (and its
  workspace) and nothing around it.

Tolerance as in the parity tests: |gpu - oracle| <= 1e-4 + 1e-4*|oracle|.
"""

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
    bad = err > ATOL + RTOL * np.abs(want)
    if bad.any():
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu={got[i]!r} oracle={want[i]!r}")


# ------------------------------------------------------------------ seeds 1 and 2

@pytest.mark.parametrize("seed", [1, 2])
def test_small_workloads_other_seeds(fc, seed):
    announce(f"conv2d_tiny and dwsep_small, seed {seed}")
    cfg = fi.WORKLOADS["conv2d_tiny"]
    x, w, b = fi.make("conv2d_tiny", seed=seed)
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, cfg["pool"], want_pooled=True)
    for algo in (0, 1, 2, 3):
        got = fc.conv2d_pool_sigmoid_sum(dev(x), dev(w), dev(b), cfg["pool"], algo=algo).cpu().numpy()
        got_map = fc.conv2d_pool_map(dev(x), dev(w), dev(b), cfg["pool"], algo=algo).cpu().numpy()
        assert_close(got, want_out, f"conv2d_tiny out algo={algo}")
        assert_close(got_map, want_map, f"conv2d_tiny map algo={algo}")
    cfg = fi.WORKLOADS["dwsep_small"]
    x, wd, wp, bp = fi.make("dwsep_small", seed=seed)
    want = oracle.dwsep_conv1d(x, wd, wp, bp, cfg["pad"])
    for algo in (1, 2):
        got = fc.dwsep_conv1d(dev(x), dev(wd), dev(wp), dev(bp), cfg["pad"], algo=algo).cpu().numpy()
        assert_close(got, want, f"dwsep_small algo={algo}")


@pytest.mark.parametrize("seed", [1, 2])
@pytest.mark.parametrize("name", ["conv2d_full", "conv2d_tail"])
def test_full_conv2d_other_seeds(fc, name, seed):
    announce(f"{name} seed {seed}")
    cfg = fi.WORKLOADS[name]
    s = cfg["pool"]
    x, w, b = fi.make(name, seed=seed)
    xd, wd, bd = dev(x), dev(w), dev(b)
    B = x.shape[0]
    idx = [0, B - 1]
    want_out = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, batch_idx=idx)
    for algo in (0, 1):  # AUTO (box-sum here) and direct MFMA
        got = fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, algo=algo).cpu().numpy()
        assert_close(got[idx], want_out, f"{name} out algo={algo}")
        got_map = fc.conv2d_pool_map(xd, wd, bd, s, algo=algo).cpu().numpy()
        _, Cout, PH, PW = got_map.shape
        rng = np.random.default_rng(100 + seed)
        n = 4000
        samp = np.stack([rng.integers(0, B, n), rng.integers(0, Cout, n), rng.integers(0, PH, n),
                         rng.integers(0, PW, n)], axis=1)
        want = oracle.conv2d_pooled_at(x, w, b, s, samp)
        assert_close(got_map[tuple(samp.T)], want, f"{name} sampled map algo={algo}")


@pytest.mark.parametrize("seed", [1, 2])
def test_full_dwsep_other_seeds(fc, seed):
    announce(f"dwsep_full seed {seed}")
    cfg = fi.WORKLOADS["dwsep_full"]
    x, wd, wp, bp = fi.make("dwsep_full", seed=seed)
    got = fc.dwsep_conv1d(dev(x), dev(wd), dev(wp), dev(bp), cfg["pad"]).cpu().numpy()
    want = oracle.dwsep_conv1d(x, wd, wp, bp, cfg["pad"], batch_idx=[seed])[0]
    assert_close(got[seed], want, f"dwsep_full y[{seed}]")
    B, O, Tout = got.shape
    rng = np.random.default_rng(200 + seed)
    n = 6000
    samp = np.stack([rng.integers(0, B, n), rng.integers(0, O, n), rng.integers(0, Tout, n)], axis=1)
    assert_close(got[tuple(samp.T)], oracle.dwsep_conv1d_at(x, wd, wp, bp, cfg["pad"], samp), "dwsep_full sampled")


# ------------------------------------------------------------------ full-size invariants

@pytest.mark.parametrize("algo", [1, 3])
def test_conv2d_full_batch_independence_and_channel_permutation(fc, algo):
    announce(f"conv2d_full batch independence, channel permutation, algo={algo}")
    cfg = fi.WORKLOADS["conv2d_full"]
    s = cfg["pool"]
    x, w, b = fi.make("conv2d_full", seed=0)
    xd, wd, bd = dev(x), dev(w), dev(b)
    base = fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, algo=algo).cpu().numpy()
    # changing one batch item leaves every other item's sum bit for bit unchanged
    x2 = xd.clone()
    x2[5] = -x2[5] * 0.5
    changed = fc.conv2d_pool_sigmoid_sum_det(x2, wd, bd, s, algo=algo).cpu().numpy()
    keep = [i for i in range(x.shape[0]) if i != 5]
    assert np.array_equal(base[keep].view(np.uint32), changed[keep].view(np.uint32))
    assert changed[5] != base[5]
    # permuting the output channels (rows of w and b) leaves the sums unchanged
    perm = torch.from_numpy(np.random.default_rng(9).permutation(w.shape[0])).cuda()
    permuted = fc.conv2d_pool_sigmoid_sum(xd, wd[perm].contiguous(), bd[perm].contiguous(), s, algo=algo)
    assert_close(permuted.cpu().numpy(), base, "sums after permuting output channels")


def test_dwsep_full_batch_independence_and_channel_permutation(fc):
    announce("dwsep_full batch independence, output-channel permutation")
    cfg = fi.WORKLOADS["dwsep_full"]
    x, wd, wp, bp = fi.make("dwsep_full", seed=0)
    xd, wdd, wpd, bpd = dev(x), dev(wd), dev(wp), dev(bp)
    base = fc.dwsep_conv1d(xd, wdd, wpd, bpd, cfg["pad"])
    x2 = xd.clone()
    x2[7] = torch.flip(x2[7], dims=[1])
    changed = fc.dwsep_conv1d(x2, wdd, wpd, bpd, cfg["pad"])
    keep = [i for i in range(x.shape[0]) if i != 7]
    assert torch.equal(base[keep], changed[keep])
    assert not torch.equal(base[7], changed[7])
    perm = torch.from_numpy(np.random.default_rng(10).permutation(wp.shape[0])).cuda()
    permuted = fc.dwsep_conv1d(xd, wdd, wpd[perm].contiguous(), bpd[perm].contiguous(), cfg["pad"])
    assert_close(permuted.cpu().numpy(), base[:, perm].cpu().numpy(), "y after permuting output channels")


# ------------------------------------------------------------------ canary-padded outputs

def padded(n, pad=1024):
    """A buffer of n floats inside canaries; returns (whole buffer, view of the n floats)."""
    whole = torch.full((n + 2 * pad,), CANARY, device="cuda")
    return whole, whole[pad:pad + n]


def canaries_intact(whole, n, pad=1024):
    h = whole.cpu().numpy()
    return bool((h[:pad] == np.float32(CANARY)).all() and (h[pad + n:] == np.float32(CANARY)).all())


CANARY_CONV = [
    (2, 8, 70, 76, 64, 3, 4),      # box-sum one-column-per-lane tiles, ragged
    (2, 5, 41, 37, 70, 3, 4),      # general tiles, two channel ranges
    (1, 16, 60, 50, 128, 5, 3),    # K5/s3
    (1, 2, 23, 19, 5, 7, 2),       # simple path
]


@pytest.mark.parametrize("shape", CANARY_CONV)
def test_conv2d_writes_only_its_outputs(fc, shape):
    B, Cin, H, W, Cout, K, s = shape
    announce(f"conv2d canaries {shape}")
    x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=31)
    xd, wd, bd = dev(x), dev(w), dev(b)
    want_out, want_map = oracle.conv2d_pool_sigmoid_sum(x, w, b, s, want_pooled=True)
    PH, PW = fc.conv2d_out_size(H, W, K, s)
    for algo in (0, 1, 2, 3):
        if algo in (1, 3) and fc.conv2d_select_algo(Cin, Cout, K, s) == 2:
            continue
        whole, out = padded(B)
        fc.conv2d_pool_sigmoid_sum(xd, wd, bd, s, out=out, algo=algo)
        assert canaries_intact(whole, B), f"out canaries, algo={algo}"
        assert_close(out.cpu().numpy(), want_out, f"out algo={algo}")
        n = B * Cout * PH * PW
        whole, flat = padded(n)
        fc.conv2d_pool_map(xd, wd, bd, s, out=flat.view(B, Cout, PH, PW), algo=algo)
        assert canaries_intact(whole, n), f"map canaries, algo={algo}"
        assert_close(flat.view(B, Cout, PH, PW).cpu().numpy(), want_map, f"map algo={algo}")
        nws = fc.conv2d_det_workspace_bytes(B, Cin, H, W, Cout, K, s, algo) // 4
        whole_ws, ws = padded(nws)
        whole, out = padded(B)
        fc.conv2d_pool_sigmoid_sum_det(xd, wd, bd, s, out=out, algo=algo, workspace=ws)
        assert canaries_intact(whole_ws, nws), f"workspace canaries, algo={algo}"
        assert canaries_intact(whole, B), f"det out canaries, algo={algo}"
        assert_close(out.cpu().numpy(), want_out, f"det out algo={algo}")


CANARY_DW = [
    # B, C, T, O, K, pad, stride, dilation, algo
    (2, 200, 130, 520, 9, 4, 1, 1, 0),   # tall tile, two output tiles, ragged T
    (2, 64, 200, 200, 9, 4, 1, 1, 0),    # 256-row tile, O not a multiple of 16
    (3, 10, 77, 33, 9, 4, 1, 1, 0),      # scalar weight loads
    (2, 64, 300, 300, 9, 4, 2, 1, 0),    # strided
    (1, 64, 200, 300, 5, 2, 2, 2, 2),    # dense-fused, strided and dilated
]


@pytest.mark.parametrize("shape", CANARY_DW)
def test_dwsep_writes_only_its_outputs(fc, shape):
    B, C, T, O, K, pad, stride, dil, algo = shape
    announce(f"dwsep canaries {shape}")
    x, wd, wp, bp = fi.dwsep_inputs(B, C, T, O, K, seed=32)
    Tout = fc.dwsep_out_len(T, K, pad, stride, dil)
    n = B * O * Tout
    whole, flat = padded(n)
    fc.dwsep_conv1d(dev(x), dev(wd), dev(wp), dev(bp), pad, out=flat.view(B, O, Tout), stride=stride, dilation=dil,
                    algo=algo)
    assert canaries_intact(whole, n)
    want = oracle.dwsep_conv1d(x, wd, wp, bp, pad, stride=stride, dilation=dil)
    assert_close(flat.view(B, O, Tout).cpu().numpy(), want, f"y {shape}")
