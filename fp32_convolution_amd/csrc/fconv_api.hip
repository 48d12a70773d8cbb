// fconv_api.hip -- the C ABI of libfconv (declared in include/fconv.h): argument
// checks, algorithm choice and kernel dispatch.  Host code only.
#include <limits.h>
#include <stdint.h>
#include <stdlib.h>
#include <stdio.h>

#include <mutex>

#include "../../include/fconv.h"
#include "fconv_internal.hpp"

// Partial sums of fconv2d_pool_sigmoid_sum_det_noalloc: a fixed device
// array, one copy per GPU the library runs on, held until the process ends.
// In host code `scratch` names a host-side stand-in; its device address comes
// from hipGetSymbolAddress (scratch_ptr below), never from the name.
static __device__ __align__(256) float scratch[FCONV_NOALLOC_MAX_PARTIALS];

namespace {

using fconv::Conv2dShape;
using fconv::DwsepShape;

constexpr int kVersion = 100;  // 0.1.0

bool mul_ok(int64_t a, int64_t b, int64_t* r) {
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *r = a * b;
    return true;
}

bool fits_i32(int64_t v) { return v >= 0 && v <= INT32_MAX; }

bool log_enabled() {
    static int on = -1;
    if (on < 0) {
        const char* e = getenv("FCONV_LOG");
        on = (e && e[0] && e[0] != '0') ? 1 : 0;
    }
    return on == 1;
}

int status_of(hipError_t e) { return e == hipSuccess ? FCONV_OK : FCONV_EHIP; }

// Validates a Conv2d call.  Returns FCONV_OK and fills `s`, or an error.
// Element counts per batch item must fit int32 (kernel offsets are 32-bit
// inside one batch item); larger shapes are FCONV_EUNSUPPORTED.
int check_conv2d(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w, int64_t Cout,
                 int64_t K, int64_t pool, const void* dst, Conv2dShape* s, bool ceil_mode = false) {
    if (!x || !w || !dst) return FCONV_EINVAL;
    if (B < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || K < 1 || pool < 1) return FCONV_EINVAL;
    if (H < K || W < K) return FCONV_EINVAL;
    int64_t t, per_item_x, nx, nw;
    if (!mul_ok(Cin, H, &t) || !mul_ok(t, W, &per_item_x) || !mul_ok(per_item_x, B, &nx)) return FCONV_EINVAL;
    if (!mul_ok(Cout, Cin, &t) || !mul_ok(t, K, &t) || !mul_ok(t, K, &nw)) return FCONV_EINVAL;
    const int64_t Hc = H - K + 1, Wc = W - K + 1;
    const int64_t PH = ceil_mode ? (Hc + pool - 1) / pool : Hc / pool;
    const int64_t PW = ceil_mode ? (Wc + pool - 1) / pool : Wc / pool;
    int64_t per_item_map, nmap;
    if (!mul_ok(Cout, PH, &t) || !mul_ok(t, PW, &per_item_map) || !mul_ok(per_item_map, B, &nmap))
        return FCONV_EINVAL;
    // Kernels address one batch item's input and the weight through buffer
    // resources (< 2^31 bytes each); other offsets are 32-bit.
    if (per_item_x >= (1 << 29) || nw >= (1 << 29) || !fits_i32(per_item_map) || B > 65535 || pool > 4096 ||
        K > 4096 || Cout > (1 << 20))
        return FCONV_EUNSUPPORTED;
    s->B = (int)B; s->Cin = (int)Cin; s->H = (int)H; s->W = (int)W; s->Cout = (int)Cout;
    s->K = (int)K; s->S = (int)pool; s->PH = (int)PH; s->PW = (int)PW;
    return FCONV_OK;
}

int auto_conv2d_algo(int Cin, int K, int S) {
    if (fconv::conv2d_boxsum_supported(Cin, K, S)) return FCONV_ALGO_BOXSUM;
    if (fconv::conv2d_mfma_supported(Cin, K, S)) return FCONV_ALGO_DIRECT_MFMA;
    return FCONV_ALGO_DIRECT_SIMPLE;
}

int pick_conv2d_algo(const Conv2dShape& s, int algo) {
    if (algo == FCONV_ALGO_AUTO) return auto_conv2d_algo(s.Cin, s.K, s.S);
    if (algo == FCONV_ALGO_DIRECT_MFMA)
        return fconv::conv2d_mfma_supported(s.Cin, s.K, s.S) ? algo : FCONV_EUNSUPPORTED;
    if (algo == FCONV_ALGO_BOXSUM)
        return fconv::conv2d_boxsum_supported(s.Cin, s.K, s.S) ? algo : FCONV_EUNSUPPORTED;
    if (algo == FCONV_ALGO_DIRECT_SIMPLE) return algo;
    return FCONV_EINVAL;
}

hipError_t launch_conv2d(int algo, const Conv2dShape& s, const float* x, const float* w, const float* bias,
                         float* dst, int mode, hipStream_t st) {
    if (algo == FCONV_ALGO_DIRECT_MFMA) return fconv::conv2d_mfma_launch(s, x, w, bias, dst, mode, st);
    if (algo == FCONV_ALGO_BOXSUM) return fconv::conv2d_boxsum_launch(s, x, w, bias, dst, mode, st);
    return fconv::conv2d_simple_launch(s, x, w, bias, dst, mode, st);
}

int64_t conv2d_parts(int algo, const Conv2dShape& s) {
    if (algo == FCONV_ALGO_DIRECT_MFMA) return fconv::conv2d_mfma_parts(s);
    if (algo == FCONV_ALGO_BOXSUM) return fconv::conv2d_boxsum_parts(s);
    return fconv::conv2d_simple_parts(s);
}

constexpr int kMaxDevices = 64;

// The memory pool of the fused-sum entry points' partial sums on the current
// device: created on first use (with that device current) and kept, with an
// unlimited release threshold, so that freed blocks stay with the pool for
// the next call instead of going back to the driver.  nullptr on failure.
hipMemPool_t partials_pool() {
    static std::mutex mu;
    static hipMemPool_t pools[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!pools[dev]) {
        hipMemPoolProps props = {};
        props.allocType = hipMemAllocationTypePinned;
        props.location.type = hipMemLocationTypeDevice;
        props.location.id = dev;
        hipMemPool_t p = nullptr;
        if (hipMemPoolCreate(&p, &props) != hipSuccess) return nullptr;
        uint64_t keep = UINT64_MAX;
        if (hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep) != hipSuccess) {
            (void)hipMemPoolDestroy(p);
            return nullptr;
        }
        pools[dev] = p;
    }
    return pools[dev];
}

// Scratch kept per (device, stream).  A stream's partial sums go to a buffer
// that only calls on that stream use, so a call makes no allocation (the
// pool's stream-ordered allocate and free cost about 8 us of host time per
// call).  Stream handles are reused (a destroyed stream's handle comes back
// for the next stream created, possibly while the old stream's work still
// runs), so each slot carries an event recorded after every use: a call
// waits on it (on the GPU) before it touches the buffer, and a buffer is
// freed only in stream order after it.  kStreamSlots streams per device hold
// a slot (the least recently used idle one passes to a new stream), each
// buffer at most kSlotMaxBytes, kept until the process ends.  A slot counts
// the calls between taking it and recording its event (other host threads
// may be inside one): a slot so in use is neither handed to another stream
// nor regrown.  Larger requests, streams being captured into a graph, and
// calls that find no idle slot allocate per call from the pool.
constexpr int kStreamSlots = 8;
constexpr size_t kSlotMaxBytes = (size_t)1 << 20;
constexpr size_t kSlotMinBytes = (size_t)64 << 10;

struct StreamSlot {
    hipStream_t stream;
    void* buf;         // from the partials pool, allocated in stream order
    size_t bytes;
    hipEvent_t done;   // recorded after the last call that used the slot
    uint64_t last;     // use counter, for eviction
    int busy;          // calls between stream_scratch and their event record
};

std::mutex g_slot_mu;
StreamSlot g_slots[kMaxDevices][kStreamSlots] = {};
uint64_t g_slot_clock = 0;

// The slot of stream `st` with a buffer of at least `bytes`, ready to use on
// st (st already waits for the slot's previous use) and counted busy until
// release_slot; nullptr when the call should allocate per call (*err says
// whether that is because of an error).
StreamSlot* stream_scratch(hipStream_t st, size_t bytes, hipMemPool_t pool, hipError_t* err) {
    *err = hipSuccess;
    if (bytes > kSlotMaxBytes) return nullptr;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_slot_mu);
    StreamSlot* e = nullptr;
    StreamSlot* lru = nullptr;  // idle slots only: empty first, else least recently used
    for (StreamSlot& t : g_slots[dev]) {
        if (t.buf && t.stream == st) e = &t;
        if (t.busy == 0 && (!lru || (!t.buf ? lru->buf != nullptr : (lru->buf && t.last < lru->last)))) lru = &t;
    }
    if (e && e->busy > 0 && e->bytes < bytes) return nullptr;  // in use by another call: not regrown
    if (!e) {
        // an empty slot, else the least recently used idle one, whose buffer
        // passes to this stream
        if (!lru) return nullptr;
        e = lru;
        if (!e->done && (*err = hipEventCreateWithFlags(&e->done, hipEventDisableTiming)) != hipSuccess) {
            e->done = nullptr;
            return nullptr;
        }
    }
    // the slot's previous use (this stream's, an earlier stream's that had
    // this handle, or an evicted stream's) before anything below touches or
    // frees its buffer
    if ((*err = hipStreamWaitEvent(st, e->done, 0)) != hipSuccess) return nullptr;
    e->stream = st;
    if (e->bytes < bytes) {
        size_t nb = e->bytes ? 2 * e->bytes : kSlotMinBytes;
        while (nb < bytes) nb *= 2;
        if (nb > kSlotMaxBytes) nb = kSlotMaxBytes;
        void* buf = nullptr;
        if ((*err = hipMallocFromPoolAsync(&buf, nb, pool, st)) != hipSuccess) return nullptr;
        if (e->buf && (*err = hipFreeAsync(e->buf, st)) != hipSuccess) {
            (void)hipFreeAsync(buf, st);
            return nullptr;
        }
        e->buf = buf;
        e->bytes = nb;
    }
    e->last = ++g_slot_clock;
    ++e->busy;
    return e;
}

// Ends a call's use of its slot (after its event is recorded).
void release_slot(StreamSlot* e) {
    std::lock_guard<std::mutex> lock(g_slot_mu);
    --e->busy;
}

// A fused sum: `launch(ws)` writes B * parts partial sums to ws (the
// stream's slot, else a block taken from the pool in stream order on `st`
// and returned after the call); reduce_partials adds each item's partials
// in a fixed order into out[b].  Calls on different streams never share
// scratch at the same time.
template <class Launch>
int sum_through_partials(int64_t parts, int B, float* out, hipStream_t st, Launch&& launch) {
    hipMemPool_t pool = partials_pool();
    if (!pool) return FCONV_EHIP;
    const size_t bytes = (size_t)parts * (size_t)B * sizeof(float);
    hipError_t e = hipSuccess;
    StreamSlot* slot = stream_scratch(st, bytes, pool, &e);
    if (e != hipSuccess) return FCONV_EHIP;
    void* ws = slot ? slot->buf : nullptr;
    if (!slot && hipMallocFromPoolAsync(&ws, bytes, pool, st) != hipSuccess) return FCONV_EHIP;
    e = launch((float*)ws);
    if (e == hipSuccess) e = fconv::reduce_partials((float*)ws, parts, B, out, st);
    // mark the slot's use (also after a failed launch: what was enqueued may still run)
    hipError_t ef;
    if (slot) {
        ef = hipEventRecord(slot->done, st);
        release_slot(slot);
    } else {
        ef = hipFreeAsync(ws, st);
    }
    return (e == hipSuccess && ef == hipSuccess) ? FCONV_OK : FCONV_EHIP;
}

// Stands in for a NULL pooled-map pointer during the argument checks.
const float kEmptyMapStorage = 0.f;
const void* const kEmptyMap = &kEmptyMapStorage;

int run_conv2d(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w, int64_t Cout,
               int64_t K, const float* bias, int64_t pool, int algo, float* dst, bool map, void* stream) {
    Conv2dShape s;
    // A map with no elements may come as a NULL pointer.
    const bool null_map = map && !dst;
    int rc = check_conv2d(x, B, Cin, H, W, w, Cout, K, pool, null_map ? kEmptyMap : dst, &s);
    if (rc != FCONV_OK) return rc;
    if (null_map && s.PH > 0 && s.PW > 0) return FCONV_EINVAL;
    const int a = pick_conv2d_algo(s, algo);
    if (a < 0) return a;
    hipStream_t st = (hipStream_t)stream;
    if (log_enabled())
        fprintf(stderr, "[fconv] conv2d%s B=%d Cin=%d H=%d W=%d Cout=%d K=%d pool=%d -> algo %d\n",
                map ? "_map" : "", s.B, s.Cin, s.H, s.W, s.Cout, s.K, s.S, a);
    if (s.PH == 0 || s.PW == 0) {
        // Empty pooled map: the sum is 0 and the map has no elements.
        return map ? FCONV_OK : status_of(fconv::fill_zero(dst, s.B, st));
    }
    if (map) return status_of(launch_conv2d(a, s, x, w, bias, dst, fconv::OUT_MAP, st));
    return sum_through_partials(conv2d_parts(a, s), s.B, dst, st, [&](float* ws) {
        return launch_conv2d(a, s, x, w, bias, ws, fconv::OUT_PARTIAL, st);
    });
}

constexpr int kPoolFlags = FCONV_RELU | FCONV_CEIL_MODE;

// The generalised pool, validated: shape, options and the resolved
// algorithm.  The plain average pool (no flags) is the base operation and
// takes its algorithms; everything else runs on the per-conv-output
// matrix-core kernel where it has an instance, else on the
// one-thread-per-output kernel.
struct ExPlan {
    Conv2dShape s;
    fconv::PoolOpts o;
    int algo;    // FCONV_ALGO_*, never AUTO
    bool plain;  // average pool, no flags
};

int plan_ex(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w, int64_t Cout, int64_t K,
            int64_t pool, int pool_mode, int flags, int algo, const void* dst, ExPlan* p) {
    if (pool_mode != FCONV_POOL_AVG && pool_mode != FCONV_POOL_MAX) return FCONV_EINVAL;
    if ((flags & ~kPoolFlags) != 0) return FCONV_EINVAL;
    if (algo != FCONV_ALGO_AUTO && algo != FCONV_ALGO_DIRECT_MFMA && algo != FCONV_ALGO_DIRECT_SIMPLE &&
        algo != FCONV_ALGO_BOXSUM)
        return FCONV_EINVAL;
    p->plain = pool_mode == FCONV_POOL_AVG && flags == 0;
    p->o = {pool_mode == FCONV_POOL_MAX, (flags & FCONV_RELU) != 0, (flags & FCONV_CEIL_MODE) != 0};
    int rc = check_conv2d(x, B, Cin, H, W, w, Cout, K, pool, dst, &p->s, p->o.ceil_mode);
    if (rc != FCONV_OK) return rc;
    if (p->plain) {
        p->algo = pick_conv2d_algo(p->s, algo);
        return p->algo < 0 ? p->algo : FCONV_OK;
    }
    const bool mfma_ok = fconv::conv2d_elem_supported(p->s.Cin, p->s.K, p->s.S);
    int a = algo;
    if (a == FCONV_ALGO_AUTO) a = mfma_ok ? FCONV_ALGO_DIRECT_MFMA : FCONV_ALGO_DIRECT_SIMPLE;
    if (a == FCONV_ALGO_BOXSUM || (a == FCONV_ALGO_DIRECT_MFMA && !mfma_ok)) return FCONV_EUNSUPPORTED;
    p->algo = a;
    return FCONV_OK;
}

hipError_t launch_ex(const ExPlan& p, const float* x, const float* w, const float* bias, float* dst, int mode,
                     hipStream_t st) {
    if (p.plain) return launch_conv2d(p.algo, p.s, x, w, bias, dst, mode, st);
    return p.algo == FCONV_ALGO_DIRECT_MFMA ? fconv::conv2d_elem_launch(p.s, x, w, bias, dst, mode, p.o, st)
                                            : fconv::conv2d_general_launch(p.s, x, w, bias, dst, mode, p.o, st);
}

// Workgroups (= partial sums) per batch item of the planned launch.
int64_t parts_ex(const ExPlan& p) {
    if (p.s.PH == 0 || p.s.PW == 0) return 0;
    if (p.plain) return conv2d_parts(p.algo, p.s);
    return p.algo == FCONV_ALGO_DIRECT_MFMA ? fconv::conv2d_elem_parts(p.s, p.o) : fconv::conv2d_general_parts(p.s);
}

int run_conv2d_ex(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w, int64_t Cout,
                  int64_t K, const float* bias, int64_t pool, int pool_mode, int flags, int algo, float* dst, bool map,
                  void* stream) {
    ExPlan p;
    const bool null_map = map && !dst;
    int rc = plan_ex(x, B, Cin, H, W, w, Cout, K, pool, pool_mode, flags, algo, null_map ? kEmptyMap : dst, &p);
    if (rc != FCONV_OK) return rc;
    if (null_map && p.s.PH > 0 && p.s.PW > 0) return FCONV_EINVAL;
    hipStream_t st = (hipStream_t)stream;
    if (log_enabled())
        fprintf(stderr, "[fconv] conv2d_ex%s B=%d Cin=%d H=%d W=%d Cout=%d K=%d pool=%d max=%d relu=%d ceil=%d -> algo %d\n",
                map ? "_map" : "", p.s.B, p.s.Cin, p.s.H, p.s.W, p.s.Cout, p.s.K, p.s.S, (int)p.o.pool_max,
                (int)p.o.relu, (int)p.o.ceil_mode, p.algo);
    if (p.s.PH == 0 || p.s.PW == 0) return map ? FCONV_OK : status_of(fconv::fill_zero(dst, p.s.B, st));
    if (map) return status_of(launch_ex(p, x, w, bias, dst, fconv::OUT_MAP, st));
    return sum_through_partials(parts_ex(p), p.s.B, dst, st,
                                [&](float* ws) { return launch_ex(p, x, w, bias, ws, fconv::OUT_PARTIAL, st); });
}

// Shape/algorithm checks shared by the deterministic entry point and its
// workspace query.  w and out may be placeholders for the query.
int det_plan(int64_t B, int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t K, int64_t pool, int algo,
             Conv2dShape* s, int* a, int64_t* parts) {
    static const float placeholder = 0.f;
    int rc = check_conv2d(&placeholder, B, Cin, H, W, &placeholder, Cout, K, pool, &placeholder, s);
    if (rc != FCONV_OK) return rc;
    *a = pick_conv2d_algo(*s, algo);
    if (*a < 0) return *a;
    *parts = (s->PH == 0 || s->PW == 0) ? 0 : conv2d_parts(*a, *s);
    return *parts < 0 ? FCONV_EUNSUPPORTED : FCONV_OK;
}

// The device address of `scratch` on the current device: looked up once per
// device (with that device current) and kept.  nullptr if the lookup failed.
float* scratch_ptr() {
    static std::mutex mu;
    static float* ptrs[kMaxDevices] = {};
    static bool looked[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!looked[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptrs[dev] = (float*)p;
        looked[dev] = true;
    }
    return ptrs[dev];
}

}  // namespace

extern "C" {

int fconv2d_pool_sigmoid_sum(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w,
                             int64_t Cout, int64_t K, const float* bias, int64_t pool, float* out, void* stream) {
    return run_conv2d(x, B, Cin, H, W, w, Cout, K, bias, pool, FCONV_ALGO_AUTO, out, false, stream);
}

int fconv2d_pool_sigmoid_sum_algo(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w,
                                  int64_t Cout, int64_t K, const float* bias, int64_t pool, int algo, float* out,
                                  void* stream) {
    return run_conv2d(x, B, Cin, H, W, w, Cout, K, bias, pool, algo, out, false, stream);
}

int fconv2d_pool_map(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w, int64_t Cout,
                     int64_t K, const float* bias, int64_t pool, int algo, float* pooled, void* stream) {
    return run_conv2d(x, B, Cin, H, W, w, Cout, K, bias, pool, algo, pooled, true, stream);
}

int fconv2d_pool_debug_map(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w,
                           int64_t Cout, int64_t K, const float* bias, int64_t pool, float* pooled, void* stream) {
    return run_conv2d(x, B, Cin, H, W, w, Cout, K, bias, pool, FCONV_ALGO_AUTO, pooled, true, stream);
}

int fconv2d_pool_sigmoid_sum_ex(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w,
                                int64_t Cout, int64_t K, const float* bias, int64_t pool, int pool_mode, int flags,
                                int algo, float* out, void* stream) {
    return run_conv2d_ex(x, B, Cin, H, W, w, Cout, K, bias, pool, pool_mode, flags, algo, out, false, stream);
}

int fconv2d_pool_map_ex(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w, int64_t Cout,
                        int64_t K, const float* bias, int64_t pool, int pool_mode, int flags, int algo, float* pooled,
                        void* stream) {
    return run_conv2d_ex(x, B, Cin, H, W, w, Cout, K, bias, pool, pool_mode, flags, algo, pooled, true, stream);
}

int fconv2d_pool_sigmoid_sum_det_workspace_ex(int64_t B, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                                               int64_t K, int64_t pool, int pool_mode, int flags, int algo,
                                               size_t* bytes) {
    if (!bytes) return FCONV_EINVAL;
    static const float placeholder = 0.f;
    ExPlan p;
    int rc = plan_ex(&placeholder, B, Cin, H, W, &placeholder, Cout, K, pool, pool_mode, flags, algo, &placeholder,
                     &p);
    if (rc != FCONV_OK) return rc;
    *bytes = (size_t)parts_ex(p) * (size_t)p.s.B * sizeof(float);
    return FCONV_OK;
}

int fconv2d_pool_sigmoid_sum_det_ex(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w,
                                    int64_t Cout, int64_t K, const float* bias, int64_t pool, int pool_mode,
                                    int flags, int algo, void* workspace, size_t workspace_bytes, float* out,
                                    void* stream) {
    ExPlan p;
    int rc = plan_ex(x, B, Cin, H, W, w, Cout, K, pool, pool_mode, flags, algo, out, &p);
    if (rc != FCONV_OK) return rc;
    const int64_t parts = parts_ex(p);
    hipStream_t st = (hipStream_t)stream;
    if (parts == 0) return status_of(fconv::fill_zero(out, p.s.B, st));
    if (!workspace || workspace_bytes < (size_t)parts * (size_t)p.s.B * sizeof(float)) return FCONV_EINVAL;
    float* ws = (float*)workspace;
    hipError_t e = launch_ex(p, x, w, bias, ws, fconv::OUT_PARTIAL, st);
    if (e != hipSuccess) return FCONV_EHIP;
    return status_of(fconv::reduce_partials(ws, parts, p.s.B, out, st));
}

int fconv2d_pool_out_size_ex(int64_t H, int64_t W, int64_t K, int64_t pool, int flags, int64_t* PH,
                             int64_t* PW) {
    if (!PH || !PW || H < 1 || W < 1 || K < 1 || pool < 1 || H < K || W < K) return FCONV_EINVAL;
    if ((flags & ~kPoolFlags) != 0) return FCONV_EINVAL;
    const int64_t Hc = H - K + 1, Wc = W - K + 1;
    const bool c = (flags & FCONV_CEIL_MODE) != 0;
    *PH = c ? (Hc + pool - 1) / pool : Hc / pool;
    *PW = c ? (Wc + pool - 1) / pool : Wc / pool;
    return FCONV_OK;
}

int fconv2d_pool_sigmoid_sum_det_workspace(int64_t B, int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t K,
                                            int64_t pool, int algo, size_t* bytes) {
    if (!bytes) return FCONV_EINVAL;
    Conv2dShape s;
    int a;
    int64_t parts;
    int rc = det_plan(B, Cin, H, W, Cout, K, pool, algo, &s, &a, &parts);
    if (rc != FCONV_OK) return rc;
    *bytes = (size_t)parts * (size_t)s.B * sizeof(float);
    return FCONV_OK;
}

int fconv2d_pool_sigmoid_sum_det(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W, const float* w,
                                 int64_t Cout, int64_t K, const float* bias, int64_t pool, int algo, void* workspace,
                                 size_t workspace_bytes, float* out, void* stream) {
    if (!x || !w || !out) return FCONV_EINVAL;
    Conv2dShape s;
    int a;
    int64_t parts;
    int rc = det_plan(B, Cin, H, W, Cout, K, pool, algo, &s, &a, &parts);
    if (rc != FCONV_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (parts == 0) return status_of(fconv::fill_zero(out, s.B, st));
    if (!workspace || workspace_bytes < (size_t)parts * (size_t)s.B * sizeof(float)) return FCONV_EINVAL;
    float* ws = (float*)workspace;
    hipError_t e = launch_conv2d(a, s, x, w, bias, ws, fconv::OUT_PARTIAL, st);
    if (e != hipSuccess) return FCONV_EHIP;
    return status_of(fconv::reduce_partials(ws, parts, s.B, out, st));
}

int fconv2d_pool_sigmoid_sum_det_noalloc(const float* x, int64_t B, int64_t Cin, int64_t H, int64_t W,
                                         const float* w, int64_t Cout, int64_t K, const float* bias, int64_t pool,
                                         int algo, float* out, void* stream) {
    if (!x || !w || !out) return FCONV_EINVAL;
    Conv2dShape s;
    int a;
    int64_t parts;
    int rc = det_plan(B, Cin, H, W, Cout, K, pool, algo, &s, &a, &parts);
    if (rc != FCONV_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    if (parts == 0) return status_of(fconv::fill_zero(out, s.B, st));
    if (parts * s.B > FCONV_NOALLOC_MAX_PARTIALS) return FCONV_ESCRATCH;
    float* ws = scratch_ptr();
    if (!ws) return FCONV_EHIP;
    // Every slot ws[0 .. B*parts) is written by the first kernel before the
    // second reads it, so nothing needs clearing between calls.
    hipError_t e = launch_conv2d(a, s, x, w, bias, ws, fconv::OUT_PARTIAL, st);
    if (e != hipSuccess) return FCONV_EHIP;
    return status_of(fconv::reduce_partials(ws, parts, s.B, out, st));
}

int fconv2d_pool_out_size(int64_t H, int64_t W, int64_t K, int64_t pool, int64_t* PH, int64_t* PW) {
    if (!PH || !PW || H < 1 || W < 1 || K < 1 || pool < 1 || H < K || W < K) return FCONV_EINVAL;
    *PH = (H - K + 1) / pool;
    *PW = (W - K + 1) / pool;
    return FCONV_OK;
}

int fconv2d_select_algo(int64_t Cin, int64_t Cout, int64_t K, int64_t pool) {
    if (Cin < 1 || Cout < 1 || K < 1 || pool < 1 || Cin > INT32_MAX || K > 4096 || pool > 4096)
        return FCONV_EINVAL;
    return auto_conv2d_algo((int)Cin, (int)K, (int)pool);
}

int64_t dwsep_conv1d_out_len_ex(int64_t T, int64_t K, int64_t pad, int64_t stride, int64_t dilation) {
    if (T < 1 || K < 1 || pad < 0 || stride < 1 || dilation < 1) return -1;
    if (pad > (INT64_MAX / 4) || K > (INT64_MAX / 4) / dilation || T > INT64_MAX / 4) return -1;
    const int64_t span = T + 2 * pad - dilation * (K - 1) - 1;
    return span < 0 ? -1 : span / stride + 1;
}

int64_t dwsep_conv1d_out_len(int64_t T, int64_t K, int64_t pad) { return dwsep_conv1d_out_len_ex(T, K, pad, 1, 1); }

int dwsep_conv1d_algo(const float* x, int64_t B, int64_t C, int64_t T, const float* w_dw, int64_t K,
                      const float* w_pw, int64_t O, const float* b_pw, int64_t pad, int64_t stride,
                      int64_t dilation, int algo, float* y, void* stream) {
    if (algo != FCONV_DWSEP_AUTO && algo != FCONV_DWSEP_SEPARABLE && algo != FCONV_DWSEP_DENSE)
        return FCONV_EINVAL;
    if (!x || !w_dw || !w_pw || !y) return FCONV_EINVAL;
    if (B < 1 || C < 1 || T < 1 || O < 1 || K < 1 || pad < 0 || stride < 1 || dilation < 1) return FCONV_EINVAL;
    const int64_t Tout = dwsep_conv1d_out_len_ex(T, K, pad, stride, dilation);
    if (Tout < 1) return FCONV_EINVAL;
    int64_t per_item_x, per_item_y, t, n;
    if (!mul_ok(C, T, &per_item_x) || !mul_ok(per_item_x, B, &n)) return FCONV_EINVAL;
    if (!mul_ok(O, Tout, &per_item_y) || !mul_ok(per_item_y, B, &n)) return FCONV_EINVAL;
    if (!mul_ok(O, C, &t) || !mul_ok(C, K, &n)) return FCONV_EINVAL;
    // The kernel reads x rows (T floats) and w_pw (O*C floats) through buffer
    // resources of < 2^31 bytes; other offsets are 32-bit per batch item.
    const int64_t lim = (int64_t)1 << 29;
    if (!fits_i32(per_item_x) || !fits_i32(per_item_y) || t >= lim || T >= lim || !fits_i32(n) || B > 65535 ||
        K > 8192 || O > (1 << 20) || pad >= lim || stride >= lim || dilation * (K - 1) >= lim)
        return FCONV_EUNSUPPORTED;
    DwsepShape s{(int)B, (int)C, (int)T, (int)K, (int)O, (int)pad, (int)Tout, (int)stride, (int)dilation};
    const bool dense = algo == FCONV_DWSEP_DENSE;
    if (dense ? !fconv::dwsep_dense_supported(s) : !fconv::dwsep_supported(s)) return FCONV_EUNSUPPORTED;
    if (log_enabled())
        fprintf(stderr, "[fconv] dwsep%s B=%d C=%d T=%d K=%d O=%d pad=%d stride=%d dil=%d Tout=%d\n",
                dense ? "_dense" : "", s.B, s.C, s.T, s.K, s.O, s.pad, s.stride, s.dil, s.Tout);
    hipStream_t st = (hipStream_t)stream;
    return status_of(dense ? fconv::dwsep_dense_launch(s, x, w_dw, w_pw, b_pw, y, st)
                           : fconv::dwsep_launch(s, x, w_dw, w_pw, b_pw, y, st));
}

int dwsep_conv1d_ex(const float* x, int64_t B, int64_t C, int64_t T, const float* w_dw, int64_t K,
                    const float* w_pw, int64_t O, const float* b_pw, int64_t pad, int64_t stride, int64_t dilation,
                    float* y, void* stream) {
    return dwsep_conv1d_algo(x, B, C, T, w_dw, K, w_pw, O, b_pw, pad, stride, dilation, FCONV_DWSEP_AUTO, y,
                             stream);
}

int dwsep_conv1d(const float* x, int64_t B, int64_t C, int64_t T, const float* w_dw, int64_t K,
                 const float* w_pw, int64_t O, const float* b_pw, int64_t pad, float* y, void* stream) {
    return dwsep_conv1d_ex(x, B, C, T, w_dw, K, w_pw, O, b_pw, pad, 1, 1, y, stream);
}

const char* fconv_strerror(int status) {
    switch (status) {
        case FCONV_OK: return "success";
        case FCONV_EINVAL: return "invalid argument";
        case FCONV_EUNSUPPORTED: return "shape not supported by the requested algorithm";
        case FCONV_EHIP: return "HIP runtime error";
        case FCONV_ESCRATCH: return "more partial sums than the fixed scratch array holds";
        default: return "unknown status";
    }
}

int fconv_version(void) { return kVersion; }

}  // extern "C"
