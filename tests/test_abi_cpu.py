"""Host-side tests of the C ABI (no GPU needed).

The library must load, export every function include/fconv.h declares, and
reject bad arguments with the documented status codes before any device
work.  No call here reaches a kernel launch: every argument set fails a
host check first.  The calls pass a made-up device address (FAKE); should a
host check ever regress, such a call would queue a kernel on memory that
does not exist, so every test that passes FAKE is skipped where a GPU is
visible (the GPU tests cover the same entry points with real buffers).
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fconv.h")
LIB = os.path.join(ROOT, "fp32_convolution_amd", "libfconv.so")

EINVAL, EUNSUP = -1, -2
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails a host check first


def _gpu_visible():
    import torch

    return torch.cuda.device_count() > 0  # counts devices without initialising one


# for tests that pass FAKE as a device pointer
no_gpu = pytest.mark.skipif(_gpu_visible(), reason="passes a made-up device address; host-only check")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libfconv.so is not built (python -m fp32_convolution_amd.build)")
    import fp32_convolution_amd as fc

    return fc.lib


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ["fconv2d_pool_sigmoid_sum", "dwsep_conv1d", "fconv2d_pool_map", "fconv2d_pool_debug_map",
                 "fconv_strerror",
                 "fconv_version", "fconv2d_pool_sigmoid_sum_algo", "fconv2d_pool_out_size",
                 "fconv2d_select_algo", "dwsep_conv1d_out_len", "fconv2d_pool_sigmoid_sum_ex",
                 "fconv2d_pool_map_ex", "fconv2d_pool_out_size_ex", "fconv2d_pool_sigmoid_sum_det_ex",
                 "fconv2d_pool_sigmoid_sum_det_workspace_ex"]:
        assert must in names, must


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in fconv.h but not exported"


@no_gpu
def test_ceiling_probe_library():
    # benchmark-only probes (not part of fconv.h): exported, argument checks on the host
    path = os.path.join(ROOT, "fp32_convolution_amd", "libfconv_probe.so")
    assert os.path.exists(path), "libfconv_probe.so is not built"
    probe = ctypes.CDLL(path)
    for name in ("fconv_probe_mfma_f32", "fconv_probe_fma_f32"):
        fn = getattr(probe, name)
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        assert fn(0, 10, FAKE, None) == -1
        assert fn(4, 0, FAKE, None) == -1
        assert fn(4, 10, None, None) == -1
    probe.fconv_probe_read_f32.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p,
                                           ctypes.c_void_p]
    probe.fconv_probe_write_f32.argtypes = [ctypes.c_int, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p]
    assert probe.fconv_probe_read_f32(0, 16, FAKE, FAKE, None) == -1
    assert probe.fconv_probe_read_f32(4, 0, FAKE, FAKE, None) == -1
    assert probe.fconv_probe_read_f32(4, 16, None, FAKE, None) == -1
    assert probe.fconv_probe_write_f32(0, 16, FAKE, None) == -1
    assert probe.fconv_probe_write_f32(4, 16, None, None) == -1
    ov = probe.fconv_probe_mfma_valu_f32
    ov.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert ov(0, 3, 10, 10, FAKE, None) == -1
    assert ov(4, 0, 10, 10, FAKE, None) == -1
    assert ov(4, 4, 10, 10, FAKE, None) == -1
    assert ov(4, 3, 0, 10, FAKE, None) == -1
    assert ov(4, 3, 10, 0, FAKE, None) == -1
    assert ov(4, 3, 10, 10, None, None) == -1


def test_version_and_strerror(lib):
    assert lib.fconv_version() >= 100
    for code in [0, -1, -2, -3, 7]:
        assert isinstance(lib.fconv_strerror(code), bytes) and lib.fconv_strerror(code)
    assert lib.fconv_strerror(0) == b"success"


def test_out_size(lib):
    import fp32_convolution_amd as fc

    assert fc.conv2d_out_size(384, 384, 3, 4) == (95, 95)
    assert fc.conv2d_out_size(257, 257, 5, 3) == (84, 84)
    assert fc.conv2d_out_size(16, 16, 3, 4) == (3, 3)
    assert fc.conv2d_out_size(5, 6, 3, 4) == (0, 1)
    ph, pw = ctypes.c_int64(), ctypes.c_int64()
    assert lib.fconv2d_pool_out_size(2, 5, 3, 1, ctypes.byref(ph), ctypes.byref(pw)) == EINVAL
    assert lib.fconv2d_pool_out_size(5, 5, 3, 0, ctypes.byref(ph), ctypes.byref(pw)) == EINVAL
    assert lib.fconv2d_pool_out_size(5, 5, 3, 1, None, ctypes.byref(pw)) == EINVAL


def test_dwsep_out_len(lib):
    assert lib.dwsep_conv1d_out_len(4096, 9, 4) == 4096
    assert lib.dwsep_conv1d_out_len(256, 9, 4) == 256
    assert lib.dwsep_conv1d_out_len(10, 3, 0) == 8
    assert lib.dwsep_conv1d_out_len(4, 9, 0) == -1
    assert lib.dwsep_conv1d_out_len(4, 9, -1) == -1
    assert lib.dwsep_conv1d_out_len(0, 1, 0) == -1


def test_select_algo(lib):
    assert lib.fconv2d_select_algo(8, 64, 3, 4) == 3   # box-sum instance
    assert lib.fconv2d_select_algo(16, 128, 5, 3) == 3
    assert lib.fconv2d_select_algo(3, 4, 3, 4) == 3
    assert lib.fconv2d_select_algo(3, 4, 7, 2) == 2    # no matrix-core instance for K=7 -> simple path
    # box-sum stages its channels through LDS in chunks: every channel count stays on the matrix cores
    for cin in (40, 44, 64, 128, 512, 4096):
        for K, s in ((3, 4), (5, 3), (3, 2), (3, 3)):
            assert lib.fconv2d_select_algo(cin, 64, K, s) == 3, (cin, K, s)
    assert lib.fconv2d_select_algo(0, 4, 3, 4) == EINVAL


def test_det_workspace_query(lib):
    import fp32_convolution_amd as fc

    # direct MFMA on x[128,8,384,384] (folded average pool), 3x16 pooled tiles of a 95x95 map: 32*6 per item
    assert fc.conv2d_det_workspace_bytes(128, 8, 384, 384, 64, 3, 4, algo=1) == 128 * 32 * 6 * 4
    # box-sum (K = 3, s = 4, W % 4 == 0) has 2 x 48 pooled tiles: 48 * 2 per item; with W % 4 != 0 it
    # uses the direct kernel's tiles; the simple path one workgroup per 256 pooled values of an item
    assert fc.conv2d_det_workspace_bytes(128, 8, 384, 384, 64, 3, 4, algo=3) == 128 * 48 * 2 * 4
    assert fc.conv2d_det_workspace_bytes(128, 8, 383, 383, 64, 3, 4, algo=3) == 128 * 24 * 6 * 4
    assert fc.conv2d_det_workspace_bytes(2, 3, 16, 16, 4, 3, 4, algo=2) == 2 * 1 * 4
    assert fc.conv2d_det_workspace_bytes(3, 2, 5, 9, 4, 3, 4) == 0          # empty pooled map
    # at most 1024 workgroups (partial sums) per batch item: larger maps walk several tiles each
    assert fc.conv2d_det_workspace_bytes(2, 1, 16384, 16384, 16, 3, 4, algo=3) == 2 * 1024 * 4
    assert fc.conv2d_det_workspace_bytes(2, 2, 16384, 16383, 16, 3, 4, algo=3) == 2 * 1024 * 4
    assert fc.conv2d_det_workspace_bytes(1, 2, 8192, 8192, 16, 3, 4, algo=1) == 1024 * 4
    assert fc.conv2d_det_workspace_bytes(1, 2, 4096, 4096, 16, 5, 3, algo=3) == 1024 * 4
    assert fc.conv2d_det_workspace_bytes(1, 2, 1024, 1024, 16, 3, 4, algo=2) == 1024 * 4
    # 1024 units exactly: one each (32 x 32 tiles of 2 x 48 pooled outputs)
    assert fc.conv2d_det_workspace_bytes(1, 1, 4 * 64 + 2, 4 * 32 * 48 + 4, 64, 3, 4, algo=3) == 1024 * 4
    n = ctypes.c_size_t()
    assert lib.fconv2d_pool_sigmoid_sum_det_workspace(1, 1, 8, 8, 1, 3, 2, 0, None) == EINVAL
    assert lib.fconv2d_pool_sigmoid_sum_det_workspace(1, 1, 2, 8, 1, 3, 2, 0, ctypes.byref(n)) == EINVAL
    assert lib.fconv2d_pool_sigmoid_sum_det_workspace(1, 1, 8, 8, 1, 7, 2, 1, ctypes.byref(n)) == EUNSUP


@no_gpu
def test_det_rejects_small_workspace(lib):
    # checked on the host before any launch
    args = (FAKE, 2, 3, 16, 16, FAKE, 4, 3, None, 4, 2)
    assert lib.fconv2d_pool_sigmoid_sum_det(*args, FAKE, 7, FAKE, None) == EINVAL
    assert lib.fconv2d_pool_sigmoid_sum_det(*args, None, 8, FAKE, None) == EINVAL
    assert lib.fconv2d_pool_sigmoid_sum_det(None, *args[1:], FAKE, 8, FAKE, None) == EINVAL


def conv(lib, x=FAKE, B=1, Cin=1, H=8, W=8, w=FAKE, Cout=1, K=3, b=None, pool=2, algo=0, out=FAKE):
    return lib.fconv2d_pool_sigmoid_sum_algo(x, B, Cin, H, W, w, Cout, K, b, pool, algo, out, None)


@no_gpu
@pytest.mark.parametrize("kw", [
    dict(x=None), dict(w=None), dict(out=None),
    dict(B=0), dict(Cin=0), dict(H=0), dict(W=-1), dict(Cout=0), dict(K=0), dict(pool=0),
    dict(H=2, K=3), dict(W=2, K=3),
    dict(B=2**40, Cin=2**30),       # element count overflows int64
    dict(algo=9),                   # unknown algorithm
])
def test_conv2d_einval(lib, kw):
    assert conv(lib, **kw) == EINVAL


@no_gpu
def test_conv2d_unsupported(lib):
    assert conv(lib, K=7, algo=1) == EUNSUP            # no MFMA instance for K=7
    assert conv(lib, K=7, algo=3) == EUNSUP            # nor a box-sum one
    assert conv(lib, Cin=2**16, H=2**8, W=2**8) == EUNSUP  # per-item elements beyond int32
    assert conv(lib, B=70000) == EUNSUP


@no_gpu
def test_conv2d_entry_points_share_checks(lib):
    assert lib.fconv2d_pool_sigmoid_sum(None, 1, 1, 8, 8, FAKE, 1, 3, None, 2, FAKE, None) == EINVAL
    assert lib.fconv2d_pool_map(FAKE, 1, 1, 8, 8, FAKE, 1, 3, None, 0, 0, FAKE, None) == EINVAL
    assert lib.fconv2d_pool_map(FAKE, 1, 1, 8, 8, FAKE, 1, 9, None, 2, 1, FAKE, None) == EINVAL  # H < K
    assert lib.fconv2d_pool_debug_map(FAKE, 1, 1, 8, 8, FAKE, 1, 3, None, 0, FAKE, None) == EINVAL
    assert lib.fconv2d_pool_debug_map(FAKE, 1, 1, 8, 8, FAKE, 1, 9, None, 2, FAKE, None) == EINVAL  # H < K
    assert lib.fconv2d_pool_debug_map(None, 1, 1, 8, 8, FAKE, 1, 3, None, 2, FAKE, None) == EINVAL


def conv_ex(lib, x=FAKE, B=1, Cin=1, H=8, W=8, w=FAKE, Cout=1, K=3, b=None, pool=2, pool_mode=1, flags=0, algo=0,
            out=FAKE, fn="fconv2d_pool_sigmoid_sum_ex"):
    return getattr(lib, fn)(x, B, Cin, H, W, w, Cout, K, b, pool, pool_mode, flags, algo, out, None)


@no_gpu
@pytest.mark.parametrize("fn", ["fconv2d_pool_sigmoid_sum_ex", "fconv2d_pool_map_ex"])
@pytest.mark.parametrize("kw", [
    dict(pool_mode=2), dict(pool_mode=-1),   # unknown pool
    dict(flags=4), dict(flags=-1),           # unknown flag bits
    dict(algo=4), dict(algo=-1),             # unknown algorithm
    dict(x=None), dict(out=None), dict(pool=0), dict(H=2, K=3),
    dict(pool_mode=0, flags=0, x=None),      # the plain average pool takes the base checks
])
def test_conv2d_ex_einval(lib, fn, kw):
    assert conv_ex(lib, fn=fn, **kw) == EINVAL


@no_gpu
def test_empty_map_may_be_null(lib):
    # 3 x 7 conv map, pool 4: no pooled rows in floor mode -> nothing to write, NULL accepted
    assert lib.fconv2d_pool_map(FAKE, 1, 2, 5, 9, FAKE, 3, 3, None, 4, 0, None, None) == 0
    assert conv_ex(lib, H=5, W=9, pool=4, out=None, fn="fconv2d_pool_map_ex") == 0
    # ceil mode has one pooled row there, so NULL is an error
    assert conv_ex(lib, H=5, W=9, pool=4, flags=2, out=None, fn="fconv2d_pool_map_ex") == EINVAL
    assert lib.fconv2d_pool_map(FAKE, 1, 2, 8, 9, FAKE, 3, 3, None, 4, 0, None, None) == EINVAL


@no_gpu
def test_conv2d_ex_unsupported(lib):
    assert conv_ex(lib, algo=3) == EUNSUP                          # box-sum needs a linear pool
    assert conv_ex(lib, pool_mode=0, flags=1, algo=3) == EUNSUP    # ... without ReLU
    assert conv_ex(lib, pool_mode=0, flags=2, algo=3) == EUNSUP    # ... over full windows
    assert conv_ex(lib, K=5, pool=4, algo=1, H=16, W=16) == EUNSUP  # matrix-core instances: K3 s2-4, K5 s3
    assert conv_ex(lib, K=7, pool=2, algo=1, H=16, W=16) == EUNSUP
    assert conv_ex(lib, B=70000) == EUNSUP


def test_det_ex_workspace_query(lib):
    import fp32_convolution_amd as fc

    # the per-conv-output kernel on x[128,8,384,384] (K3/s4): 24 x 6 tiles of 4 x 16 pooled outputs per item;
    # ceil mode (96 x 96) has the same tile count
    for relu, ceil_mode in [(True, False), (False, True), (True, True)]:
        assert fc.conv2d_det_workspace_bytes(128, 8, 384, 384, 64, 3, 4, algo=1, pool_mode=fc.POOL_MAX, relu=relu,
                                             ceil_mode=ceil_mode) == 128 * 24 * 6 * 4
    # K5/s3 on x[64,16,257,257]: 21 x 9 tiles of 4 x 10, two channel ranges
    assert fc.conv2d_det_workspace_bytes(64, 16, 257, 257, 128, 5, 3, algo=1, pool_mode=fc.POOL_MAX) == \
        64 * 21 * 9 * 2 * 4
    # one-thread-per-output kernel: one workgroup per 256 pooled values of an item
    assert fc.conv2d_det_workspace_bytes(2, 3, 16, 16, 4, 3, 4, algo=2, pool_mode=fc.POOL_MAX) == 2 * 1 * 4
    # past the whole-tile LDS budget (Cin 300) the channel-chunked tiling runs, 1 x 16 pooled tiles: a
    # 3 x 3 map is 3 tiles per item, for every pool form and for the direct average-pool call
    for pool_mode, relu in [(fc.POOL_MAX, False), (fc.POOL_AVG, True), (fc.POOL_AVG, False)]:
        assert fc.conv2d_det_workspace_bytes(2, 300, 16, 16, 4, 3, 4, algo=1, pool_mode=pool_mode,
                                             relu=relu) == 2 * 3 * 4
    assert lib_det_bytes(lib, 2, 300, 16, 16, 4, 3, 4, 1) == 2 * 3 * 4
    # K5/s3 at Cin 100 leaves the pool-folded kernel (largest whole tile: Cin 68) for the chunked tiling:
    # 1 x 10 pooled tiles of a 4 x 4 map, 4 x 1 tiles and two channel ranges
    assert lib_det_bytes(lib, 1, 100, 16, 16, 100, 5, 3, 1) == 1 * 4 * 2 * 4
    # floor mode, empty map -> 0; ceil mode has one pooled row there
    assert fc.conv2d_det_workspace_bytes(3, 2, 5, 9, 4, 3, 4, pool_mode=fc.POOL_MAX) == 0
    assert fc.conv2d_det_workspace_bytes(3, 2, 5, 9, 4, 3, 4, pool_mode=fc.POOL_MAX, ceil_mode=True) > 0
    # the plain average pool is the base call's workspace
    assert fc.conv2d_det_workspace_bytes(128, 8, 384, 384, 64, 3, 4, algo=3, pool_mode=fc.POOL_AVG) == \
        lib_det_bytes(lib, 128, 8, 384, 384, 64, 3, 4, 3)
    n = ctypes.c_size_t()
    q = lib.fconv2d_pool_sigmoid_sum_det_workspace_ex
    assert q(1, 1, 8, 8, 1, 3, 2, 1, 0, 0, None) == EINVAL
    assert q(1, 1, 8, 8, 1, 3, 2, 2, 0, 0, ctypes.byref(n)) == EINVAL     # unknown pool
    assert q(1, 1, 8, 8, 1, 3, 2, 1, 8, 0, ctypes.byref(n)) == EINVAL     # unknown flag
    assert q(1, 1, 8, 8, 1, 3, 2, 1, 0, 3, ctypes.byref(n)) == EUNSUP     # box-sum with a max pool
    assert q(1, 1, 8, 8, 1, 7, 2, 1, 0, 1, ctypes.byref(n)) == EUNSUP     # no matrix-core instance for K = 7


def lib_det_bytes(lib, *args):
    n = ctypes.c_size_t()
    assert lib.fconv2d_pool_sigmoid_sum_det_workspace(*args, ctypes.byref(n)) == 0
    return n.value


@no_gpu
def test_det_ex_rejects_small_workspace(lib):
    args = (FAKE, 2, 3, 16, 16, FAKE, 4, 3, None, 4, 1, 1, 2)   # max pool, ReLU, one-thread-per-output
    assert lib.fconv2d_pool_sigmoid_sum_det_ex(*args, FAKE, 7, FAKE, None) == EINVAL
    assert lib.fconv2d_pool_sigmoid_sum_det_ex(*args, None, 8, FAKE, None) == EINVAL
    assert lib.fconv2d_pool_sigmoid_sum_det_ex(None, *args[1:], FAKE, 8, FAKE, None) == EINVAL
    assert lib.fconv2d_pool_sigmoid_sum_det_ex(*args[:-3], 2, 1, 2, FAKE, 8, FAKE, None) == EINVAL  # pool mode 2


def test_out_size_ex_matches_torch_pooling():
    import torch

    import fp32_convolution_amd as fc

    F = torch.nn.functional
    for n in range(3, 30):
        for K, s in [(3, 4), (3, 2), (5, 3), (1, 7)]:
            if n < K:
                continue
            for ceil_mode in (False, True):
                ph, pw = fc.conv2d_out_size(n, n + 2, K, s, ceil_mode=ceil_mode)
                if n - K + 1 < s and not ceil_mode:
                    assert ph == 0
                    continue
                shape = F.max_pool2d(torch.zeros(1, 1, n - K + 1, n + 2 - K + 1), s, s, ceil_mode=ceil_mode).shape
                assert (ph, pw) == (shape[2], shape[3]), (n, K, s, ceil_mode)


def test_out_size_ex_checks(lib):
    ph, pw = ctypes.c_int64(), ctypes.c_int64()
    assert lib.fconv2d_pool_out_size_ex(16, 16, 3, 4, 3, ctypes.byref(ph), ctypes.byref(pw)) == 0
    assert (ph.value, pw.value) == (4, 4)
    assert lib.fconv2d_pool_out_size_ex(16, 16, 3, 4, 1, ctypes.byref(ph), ctypes.byref(pw)) == 0
    assert (ph.value, pw.value) == (3, 3)
    assert lib.fconv2d_pool_out_size_ex(16, 16, 3, 4, 4, ctypes.byref(ph), ctypes.byref(pw)) == EINVAL
    assert lib.fconv2d_pool_out_size_ex(2, 16, 3, 4, 0, ctypes.byref(ph), ctypes.byref(pw)) == EINVAL
    assert lib.fconv2d_pool_out_size_ex(16, 16, 3, 4, 0, None, ctypes.byref(pw)) == EINVAL


def dw(lib, x=FAKE, B=1, C=4, T=16, wd=FAKE, K=3, wp=FAKE, O=4, b=None, pad=1, y=FAKE):
    return lib.dwsep_conv1d(x, B, C, T, wd, K, wp, O, b, pad, y, None)


@no_gpu
@pytest.mark.parametrize("kw", [
    dict(x=None), dict(wd=None), dict(wp=None), dict(y=None),
    dict(B=0), dict(C=0), dict(T=0), dict(K=0), dict(O=0), dict(pad=-1),
    dict(T=4, K=9, pad=0),              # Tout < 1
    dict(B=2**40, C=2**30),             # overflow
])
def test_dwsep_einval(lib, kw):
    assert dw(lib, **kw) == EINVAL


@no_gpu
def test_dwsep_unsupported(lib):
    assert dw(lib, C=2**16, T=2**16) == EUNSUP
    assert dw(lib, K=4000, T=5000) == EUNSUP   # depthwise window too wide for the LDS tile
    assert dw(lib, B=70000) == EUNSUP


@no_gpu
def test_dwsep_ex_checks(lib):
    def dwx(stride=1, dil=1, K=3, T=16, pad=1, C=4):
        return lib.dwsep_conv1d_ex(FAKE, 1, C, T, FAKE, K, FAKE, 4, None, pad, stride, dil, FAKE, None)
    assert dwx(stride=0) == EINVAL
    assert dwx(dil=0) == EINVAL
    assert dwx(K=9, T=8, pad=0, dil=2) == EINVAL          # dilated filter longer than the padded input
    assert dwx(stride=2**30) == EUNSUP
    assert dwx(K=3, dil=2**29, T=2**28, pad=2**29) == EUNSUP
    assert dwx(stride=4000, T=2**20, C=16) == EUNSUP      # strided window does not fit in LDS
    assert lib.dwsep_conv1d_out_len_ex(4096, 9, 4, 1, 1) == 4096
    assert lib.dwsep_conv1d_out_len_ex(10, 3, 1, 2, 1) == 5
    assert lib.dwsep_conv1d_out_len_ex(10, 3, 0, 1, 2) == 6
    assert lib.dwsep_conv1d_out_len_ex(8, 3, 0, 1, 4) == -1
    assert lib.dwsep_conv1d_out_len_ex(8, 3, 0, 0, 1) == -1


@no_gpu
def test_dwsep_algo_checks(lib):
    args = (FAKE, 1, 4, 16, FAKE, 3, FAKE, 4, None, 1, 1, 1)
    assert lib.dwsep_conv1d_algo(*args, 3, FAKE, None) == EINVAL      # unknown algorithm
    assert lib.dwsep_conv1d_algo(*args, -1, FAKE, None) == EINVAL
    assert lib.dwsep_conv1d_algo(FAKE, 1, 4, 16, FAKE, 3, FAKE, 4, None, 1, 0, 1, 2, FAKE, None) == EINVAL
    assert lib.dwsep_conv1d_algo(FAKE, 1, 16, 2**20, FAKE, 3, FAKE, 4, None, 1, 5000, 1, 2, FAKE, None) == EUNSUP


def test_binding_rejects_cpu_tensors():
    import torch

    import fp32_convolution_amd as fc

    x = torch.zeros(1, 1, 8, 8)
    with pytest.raises(ValueError):
        fc.conv2d_pool_sigmoid_sum(x, torch.zeros(1, 1, 3, 3), None, 2)
    with pytest.raises(TypeError):
        fc.dwsep_conv1d(torch.zeros(1, 2, 8, dtype=torch.float64), torch.zeros(2, 3), torch.zeros(2, 2), None, 1)
