"""The allocation-free entry point, fconv2d_pool_sigmoid_sum_det_noalloc,
against the existing entry point it varies, fconv2d_pool_sigmoid_sum_det
(caller workspace), both called through the C ABI.  They run the same
kernels and the same fixed-order reduction, so the results must agree bit
for bit, and both must meet the oracle's 1e-4 bar.  Two calls in a row, the
second on a smaller input: the fixed array keeps the first call's partials,
which the second call must not pick up.
"""

import ctypes
import sys

import numpy as np
import pytest

import fconv_inputs as fi
import oracle

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


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


def ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def call_noalloc(fc, x, w, b, pool, algo, out):
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fc.lib.fconv2d_pool_sigmoid_sum_det_noalloc(ptr(x), B, Cin, H, W, ptr(w), Cout, K, ptr(b), pool, algo,
                                                       ptr(out), st)


def call_det(fc, x, w, b, pool, algo, out):
    B, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    n = ctypes.c_size_t()
    assert fc.lib.fconv2d_pool_sigmoid_sum_det_workspace(B, Cin, H, W, Cout, K, pool, algo, ctypes.byref(n)) == 0
    ws = torch.full((max(n.value, 4) // 4,), float("nan"), device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = fc.lib.fconv2d_pool_sigmoid_sum_det(ptr(x), B, Cin, H, W, ptr(w), Cout, K, ptr(b), pool, algo, ptr(ws),
                                             n.value, ptr(out), st)
    torch.cuda.synchronize()
    return rc


def check_pair(fc, name_or_shape, algo, seed):
    if isinstance(name_or_shape, str):
        x, w, b = fi.make(name_or_shape, seed=seed)
        pool = fi.WORKLOADS[name_or_shape]["pool"]
    else:
        B, Cin, H, W, Cout, K, pool = name_or_shape
        x, w, b = fi.conv2d_inputs(B, Cin, H, W, Cout, K, seed=seed)
    xd, wd, bd = dev(x), dev(w), dev(b)
    got = torch.full((x.shape[0],), float("nan"), device="cuda")
    ref = torch.full((x.shape[0],), float("nan"), device="cuda")
    assert call_noalloc(fc, xd, wd, bd, pool, algo, got) == 0
    assert call_det(fc, xd, wd, bd, pool, algo, ref) == 0
    got, ref = got.cpu().numpy(), ref.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (got, ref)
    idx = list(range(min(x.shape[0], 4)))
    want = oracle.conv2d_pool_sigmoid_sum(x, w, b, pool, batch_idx=idx)
    err = np.abs(got[idx] - want)
    assert (err <= 1e-4 + 1e-4 * np.abs(want)).all(), (got[idx], want)


@pytest.mark.parametrize("algo", [0, 1, 2])
def test_noalloc_matches_det_twice(fc, algo):
    # first the full workload (128 items x 96 or 192 partials), then a smaller input: the second call
    # must use only its own partials
    announce(f"noalloc vs det, conv2d_full then a smaller input, algo={algo}")
    if algo == 2:
        check_pair(fc, (8, 8, 100, 100, 64, 3, 4), algo, seed=40)
        check_pair(fc, (3, 3, 40, 40, 16, 3, 4), algo, seed=41)
    else:
        check_pair(fc, "conv2d_full", algo, seed=40)
        check_pair(fc, (3, 5, 70, 76, 20, 3, 4), algo, seed=41)


def test_noalloc_tail_then_tiny(fc):
    announce("noalloc vs det, conv2d_tail then conv2d_tiny")
    check_pair(fc, "conv2d_tail", 0, seed=42)
    check_pair(fc, "conv2d_tiny", 0, seed=43)


def test_noalloc_refuses_beyond_its_array(fc):
    announce("noalloc beyond the fixed array: refused, nothing enqueued")
    # one thread per pooled output, 1024 x 17 x 17 outputs per item: 1156 blocks, 1024 partials per item;
    # 300 items x 1024 > 2^18.  Real buffers of the full size, although the size check comes first.
    B, Cin, H, W, Cout, K, pool, algo = 300, 1, 19, 19, 1024, 3, 1, 2
    n = ctypes.c_size_t()
    assert fc.lib.fconv2d_pool_sigmoid_sum_det_workspace(B, Cin, H, W, Cout, K, pool, algo, ctypes.byref(n)) == 0
    assert n.value // 4 == B * 1024 > fc.NOALLOC_MAX_PARTIALS
    x = torch.zeros(B * Cin * H * W, device="cuda")
    w = torch.zeros(Cout * Cin * K * K, device="cuda")
    out = torch.full((B,), 7.0, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = fc.lib.fconv2d_pool_sigmoid_sum_det_noalloc(ptr(x), B, Cin, H, W, ptr(w), Cout, K, None, pool, algo,
                                                     ptr(out), st)
    assert rc == fc.FCONV_ESCRATCH
    torch.cuda.synchronize()
    assert (out == 7.0).all().item()
    assert b"scratch" in fc.lib.fconv_strerror(rc)
    # 256 items fit exactly
    out = torch.full((256,), 7.0, device="cuda")
    rc = fc.lib.fconv2d_pool_sigmoid_sum_det_noalloc(ptr(x), 256, Cin, H, W, ptr(w), Cout, K, None, pool, algo,
                                                     ptr(out), st)
    assert rc == 0
    torch.cuda.synchronize()
    assert (out == Cout * 17 * 17 / 2.0).all().item()   # zero input, no bias: every sigmoid is 1/2


def test_noalloc_binding_and_empty_map(fc):
    announce("noalloc through the binding; empty pooled map")
    x, w, b = fi.make("conv2d_tiny", seed=44)
    xd, wd, bd = dev(x), dev(w), dev(b)
    out = torch.empty(2, device="cuda")
    fc.conv2d_pool_sigmoid_sum_det_noalloc(xd, wd, bd, 4, out)
    want = oracle.conv2d_pool_sigmoid_sum(x, w, b, 4)
    assert (np.abs(out.cpu().numpy() - want) <= 1e-4 + 1e-4 * np.abs(want)).all()
    x0, w0, b0 = fi.conv2d_inputs(3, 2, 5, 9, 4, 3, seed=45)   # PH = 0
    out0 = torch.full((3,), 7.0, device="cuda")
    fc.conv2d_pool_sigmoid_sum_det_noalloc(dev(x0), dev(w0), dev(b0), 4, out0)
    assert out0.cpu().numpy().tolist() == [0.0, 0.0, 0.0]
