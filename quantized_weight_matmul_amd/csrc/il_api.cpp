// il_api.cpp -- the C ABI (include/il.h): device context, weight handles,
// argument validation, dispatch to the kernels, statistics, errors.
//
// The calls follow `trait Backend` on the oxinfer 0.0.0 src/gpu.rs page:
// upload -> il_upload (NULL for the page's None), matmul -> il_matmul (0 for
// false, "nothing was computed"), wants -> il_wants, name -> il_name,
// stats -> il_stats; `type DeviceWeight` -> il_weight.  The page's process-wide
// backend (`static ACTIVE: OnceLock`) becomes a lazily created per-device
// context.
#include "../../include/il.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cinttypes>
#include <climits>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "il_internal.h"

using il::Weight;

struct il_weight : Weight {};

namespace {

thread_local std::string g_err;

void set_err(const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
}

bool env_flag(const char *name, const char *value) {
    const char *v = getenv(name);
    if (!v) return false;
    // comma-separated list, e.g. IL_FORCE_FAIL=upload,matmul
    std::string s(v), want(value);
    size_t pos = 0;
    while (pos <= s.size()) {
        size_t end = s.find(',', pos);
        if (end == std::string::npos) end = s.size();
        if (s.compare(pos, end - pos, want) == 0) return true;
        pos = end + 1;
    }
    return false;
}

// ---------------------------------------------------------------- context
constexpr int kMaxDevices = 64;

// Scratch of the prefill path (the bf16 copy of x its GEMM units read), one
// buffer per stream.  A call holds its stream's entry locked while it
// enqueues the pre-pass that writes the buffer and the launch that reads it,
// so calls on one stream (from any thread) use it in stream order, and calls
// on different streams never share it.  A buffer grows (by at least half)
// when a call needs more; the one it replaces may still be read by work in
// flight or by a graph that captured it, so it is kept, like every buffer,
// until the process ends.
struct StreamScratch {
    hipStream_t stream = nullptr;
    void *ptr = nullptr;
    size_t bytes = 0;
    std::mutex m;
};

struct DeviceCtx {
    std::once_flag once;
    bool ok = false;
    std::string err;
    int cu_count = 0;
    hipStream_t upload_stream = nullptr;
    std::mutex scratch_m;  // guards the two vectors below
    std::vector<std::unique_ptr<StreamScratch>> scratch;
    std::vector<void *> retired;
};

DeviceCtx g_dev[kMaxDevices];

DeviceCtx *context(int *device_out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0) {
        set_err("no HIP device available (%s)", hipGetErrorString(e));
        return nullptr;
    }
    if (dev >= kMaxDevices) {
        set_err("device index %d is beyond the supported %d", dev, kMaxDevices);
        return nullptr;
    }
    DeviceCtx &c = g_dev[dev];
    std::call_once(c.once, [&] {
        hipDeviceProp_t prop;
        hipError_t pe = hipGetDeviceProperties(&prop, dev);
        if (pe != hipSuccess) {
            c.err = std::string("hipGetDeviceProperties failed: ") + hipGetErrorString(pe);
            return;
        }
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
            c.err = std::string("device is ") + prop.gcnArchName + ", this library is built for gfx950";
            return;
        }
        c.cu_count = prop.multiProcessorCount;
        pe = hipStreamCreateWithFlags(&c.upload_stream, hipStreamNonBlocking);
        if (pe != hipSuccess) {
            c.err = std::string("hipStreamCreate failed: ") + hipGetErrorString(pe);
            return;
        }
        c.ok = true;
    });
    if (!c.ok) {
        set_err("%s", c.err.c_str());
        return nullptr;
    }
    if (device_out) *device_out = dev;
    return &c;
}

// The stream's scratch entry (created on first use), returned locked.
std::unique_lock<std::mutex> stream_scratch(DeviceCtx *ctx, hipStream_t s, StreamScratch **out) {
    StreamScratch *e = nullptr;
    {
        std::lock_guard<std::mutex> g(ctx->scratch_m);
        for (auto &p : ctx->scratch)
            if (p->stream == s) e = p.get();
        if (!e) {
            ctx->scratch.push_back(std::make_unique<StreamScratch>());
            e = ctx->scratch.back().get();
            e->stream = s;
        }
    }
    *out = e;
    return std::unique_lock<std::mutex>(e->m);
}

// Makes e hold at least `need` bytes.  While the stream is being captured
// into a graph no buffer is allocated (an allocation is not a stream
// operation): *fallback is set and the caller allocates stream-ordered memory
// instead, which the graph then records as allocation nodes.
hipError_t grow_scratch(DeviceCtx *ctx, StreamScratch *e, size_t need, bool *fallback) {
    *fallback = false;
    if (e->bytes >= need) return hipSuccess;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t err = hipStreamIsCapturing(e->stream, &cs);
    if (err != hipSuccess) return err;
    if (cs != hipStreamCaptureStatusNone) {
        *fallback = true;
        return hipSuccess;
    }
    const size_t want = need > e->bytes + e->bytes / 2 ? need : e->bytes + e->bytes / 2;
    void *p = nullptr;
    err = hipMalloc(&p, want);
    if (err != hipSuccess) return err;
    if (e->ptr) {
        std::lock_guard<std::mutex> g(ctx->scratch_m);
        ctx->retired.push_back(e->ptr);
    }
    e->ptr = p;
    e->bytes = want;
    return hipSuccess;
}

// One prefill launch group (pre-pass + GEMM, or the wide-mode launches) with
// its scratch from the stream's cache.
hipError_t run_gemm(DeviceCtx *ctx, int fmt, const float *x, int t, int n_in, const il::KJob *jobs, int n_jobs,
                    hipStream_t s, bool glu, hipEvent_t after_prepass = nullptr) {
    const size_t need = il::gemm_scratch_bytes(fmt, t, n_in, jobs, n_jobs, glu);
    if (need == 0) return il::launch_gemm(fmt, x, nullptr, t, n_in, jobs, n_jobs, ctx->cu_count, s, glu);
    StreamScratch *e = nullptr;
    std::unique_lock<std::mutex> lock = stream_scratch(ctx, s, &e);
    bool fallback = false;
    hipError_t err = grow_scratch(ctx, e, need, &fallback);
    if (err != hipSuccess) return err;
    if (!fallback) return il::launch_gemm(fmt, x, e->ptr, t, n_in, jobs, n_jobs, ctx->cu_count, s, glu, after_prepass);
    void *tmp = nullptr;
    err = hipMallocAsync(&tmp, need, s);
    if (err != hipSuccess) return err;
    err = il::launch_gemm(fmt, x, tmp, t, n_in, jobs, n_jobs, ctx->cu_count, s, glu, after_prepass);
    const hipError_t fe = hipFreeAsync(tmp, s);
    return err != hipSuccess ? err : fe;
}

// ------------------------------------------------------------------ stats
struct PathStats {
    std::atomic<uint64_t> calls{0}, launches{0}, jobs{0}, bytes{0}, flops{0}, timed_ns{0};
    // prefill calls of one launch group timed with IL_TIMING=1: their count
    // and the device time of the x -> bf16 pre-pass within timed_ns
    std::atomic<uint64_t> split_calls{0}, prepass_ns{0};
};
PathStats g_stats[3];  // 0: decode GEMV, 1: prefill GEMM, 2: upload quantiser
std::atomic<uint64_t> g_uploads{0}, g_upload_bytes{0}, g_failed{0};

int64_t host_bytes(int fmt, int64_t n_out, int64_t n_in) {
    switch (fmt) {
        case il::FMT_BF16: return 2 * n_out * n_in;
        case il::FMT_Q8: return 36 * n_out * (n_in / il::kBlock);
        case il::FMT_Q4: return 18 * n_out * (n_in / il::kBlock);
        default: return -1;
    }
}

// Device allocation containing [ptr, ptr + bytes)?  Guards the kernels
// against host pointers and short buffers, which would fault the GPU.
bool device_range_ok(const void *ptr, int64_t bytes, const char *what) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, ptr) != hipSuccess ||
        (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)) {
        (void)hipGetLastError();
        set_err("%s is not a device pointer", what);
        return false;
    }
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, (hipDeviceptr_t)ptr) != hipSuccess) {
        (void)hipGetLastError();
        set_err("%s: cannot query its allocation", what);
        return false;
    }
    const char *b = static_cast<const char *>(base);
    const char *p = static_cast<const char *>(ptr);
    if (p < b || p + bytes > b + size) {
        set_err("%s: %" PRId64 " bytes from %p run past its allocation (%zu bytes at %p)", what,
                bytes, ptr, size, base);
        return false;
    }
    return true;
}

// Device (or managed) memory, and on which device; false for host memory.
bool device_pointer(const void *ptr, int *device) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged) return false;
    *device = attr.device;
    return true;
}

bool timing_on() {
    const char *v = getenv("IL_TIMING");
    return v && strcmp(v, "1") == 0;
}

bool overlaps(const void *a, int64_t na, const void *b, int64_t nb) {
    const char *pa = static_cast<const char *>(a), *pb = static_cast<const char *>(b);
    return pa < pb + nb && pb < pa + na;
}

// One weight's device planes (layouts in il_internal.h) in a single
// allocation: codes, then scales and the tiled scale copy (Q8 / Q4).
struct Planes {
    void *alloc = nullptr;
    char *codes = nullptr, *scales = nullptr, *scales_t = nullptr;
    int64_t tiled_bytes = 0;
    int64_t code_bytes = 0;
};

// A Q4 code plane has padding (zero bytes the kernels may read) unless its
// rows fill whole 16-row tiles and its blocks whole 64-byte segments.
bool q4_padded(int64_t n_out, int64_t n_in) { return n_out % 16 != 0 || (n_in / il::kBlock) % 4 != 0; }

bool alloc_planes(const char *who, int fmt, int64_t n_out, int64_t n_in, Planes *pl) {
    const int64_t nb = n_in / il::kBlock;
    int64_t code_bytes = 0, scale_size = 0;
    if (fmt == IL_BF16) code_bytes = 2 * n_out * n_in;
    if (fmt == IL_Q8) code_bytes = n_out * n_in, scale_size = 4;
    if (fmt == IL_Q4) code_bytes = il::q4_plane_bytes(n_out, nb), scale_size = 2;
    const int64_t scale_bytes = scale_size * n_out * nb;
    pl->tiled_bytes = scale_size * il::tiled_scale_count(n_out, nb);
    const int64_t code_alloc = (code_bytes + 255) / 256 * 256;
    const int64_t scale_alloc = (scale_bytes + 255) / 256 * 256;
    const int64_t total = code_alloc + scale_alloc + pl->tiled_bytes;
    hipError_t e = hipMalloc(&pl->alloc, (size_t)total);
    if (e != hipSuccess) {
        set_err("%s: hipMalloc(%" PRId64 ") failed: %s", who, total, hipGetErrorString(e));
        pl->alloc = nullptr;
        return false;
    }
    pl->codes = static_cast<char *>(pl->alloc);
    pl->code_bytes = code_bytes;
    pl->scales = scale_bytes ? pl->codes + code_alloc : nullptr;
    pl->scales_t = scale_bytes ? pl->codes + code_alloc + scale_alloc : nullptr;
    return true;
}

il_weight *make_handle(int fmt, int dev, int64_t n_out, int64_t n_in, const Planes &pl) {
    il_weight *w = new il_weight();
    w->fmt = fmt;
    w->device = dev;
    w->n_out = n_out;
    w->n_in = n_in;
    w->host_bytes = host_bytes(fmt, n_out, n_in);
    w->alloc = pl.alloc;
    w->codes = pl.codes;
    w->scales = pl.scales;
    w->scales_t = pl.scales_t;
    g_uploads++;
    g_upload_bytes += (uint64_t)w->host_bytes;
    return w;
}

bool shape_ok(const char *who, int64_t n_out, int64_t n_in) {
    if (n_out < 1 || n_out > INT_MAX) {
        set_err("%s: n_out = %" PRId64 " is outside [1, %d]", who, n_out, INT_MAX);
        return false;
    }
    if (n_in < il::kBlock || n_in % il::kBlock || n_in > INT_MAX) {
        set_err("%s: n_in = %" PRId64 " must be a positive multiple of 32", who, n_in);
        return false;
    }
    return true;
}

// Runs f with the handle's device current, restoring the caller's after.
template <class F>
auto on_device(int device, F f) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != device) (void)hipSetDevice(device);
    auto r = f();
    if (cur != device && cur >= 0) (void)hipSetDevice(cur);
    return r;
}

}  // namespace

// ===================================================================== ABI
extern "C" {

il_weight *il_upload(const void *weight, il_fmt fmt, int64_t n_out, int64_t n_in) {
    g_err.clear();
    if (!weight) {
        set_err("il_upload: weight is NULL");
        return nullptr;
    }
    if (fmt != IL_BF16 && fmt != IL_Q8 && fmt != IL_Q4) {
        set_err("il_upload: unknown format %d", fmt);
        return nullptr;
    }
    if (!shape_ok("il_upload", n_out, n_in)) return nullptr;
    if (env_flag("IL_FORCE_FAIL", "upload")) {
        set_err("il_upload: failure injected by IL_FORCE_FAIL");
        return nullptr;
    }
    int dev = -1;
    DeviceCtx *ctx = context(&dev);
    if (!ctx) return nullptr;

    const int64_t hb = host_bytes(fmt, n_out, n_in);
    Planes pl;
    if (!alloc_planes("il_upload", fmt, n_out, n_in, &pl)) return nullptr;
    char *codes = pl.codes, *scales = pl.scales, *scales_t = pl.scales_t;
    const int64_t tiled_bytes = pl.tiled_bytes;
    hipError_t e = hipSuccess;
    hipStream_t s = ctx->upload_stream;
    void *staging = nullptr;
    if (fmt == IL_BF16) {
        e = hipMemcpyAsync(codes, weight, (size_t)hb, hipMemcpyHostToDevice, s);
    } else {
        e = hipMalloc(&staging, (size_t)hb);
        if (e == hipSuccess) e = hipMemcpyAsync(staging, weight, (size_t)hb, hipMemcpyHostToDevice, s);
        // the tiled planes' padding (rows past n_out, blocks past nb) reads zero
        if (e == hipSuccess) e = hipMemsetAsync(scales_t, 0, (size_t)tiled_bytes, s);
        if (e == hipSuccess && fmt == IL_Q4 && q4_padded(n_out, n_in))
            e = hipMemsetAsync(codes, 0, (size_t)pl.code_bytes, s);
        if (e == hipSuccess && fmt == IL_Q8)
            e = il::launch_repack_q8(static_cast<const uint8_t *>(staging), reinterpret_cast<int8_t *>(codes),
                                     reinterpret_cast<float *>(scales), reinterpret_cast<float *>(scales_t), n_out,
                                     n_in, s);
        if (e == hipSuccess && fmt == IL_Q4)
            e = il::launch_repack_q4(static_cast<const uint8_t *>(staging), reinterpret_cast<uint8_t *>(codes),
                                     reinterpret_cast<uint16_t *>(scales), reinterpret_cast<uint16_t *>(scales_t),
                                     n_out, n_in, s);
    }
    hipError_t se = hipStreamSynchronize(s);
    if (e == hipSuccess) e = se;
    if (staging) (void)hipFree(staging);
    if (e != hipSuccess) {
        (void)hipFree(pl.alloc);
        set_err("il_upload: copy/repack failed: %s", hipGetErrorString(e));
        return nullptr;
    }
    return make_handle(fmt, dev, n_out, n_in, pl);
}

il_weight *il_upload_quantize(const void *weight, il_src src, il_fmt fmt, int64_t n_out, int64_t n_in) {
    g_err.clear();
    if (!weight) {
        set_err("il_upload_quantize: weight is NULL");
        return nullptr;
    }
    if (src != IL_SRC_F32 && src != IL_SRC_BF16) {
        set_err("il_upload_quantize: unknown source type %d", src);
        return nullptr;
    }
    if (fmt != IL_Q8 && fmt != IL_Q4) {
        set_err("il_upload_quantize: format %d is not a quantised format (IL_Q8 or IL_Q4)", fmt);
        return nullptr;
    }
    if (!shape_ok("il_upload_quantize", n_out, n_in)) return nullptr;
    if (env_flag("IL_FORCE_FAIL", "upload")) {
        set_err("il_upload_quantize: failure injected by IL_FORCE_FAIL");
        return nullptr;
    }
    int dev = -1;
    DeviceCtx *ctx = context(&dev);
    if (!ctx) return nullptr;
    const int64_t src_bytes = n_out * n_in * (src == IL_SRC_F32 ? 4 : 2);
    int wdev = -1;
    const bool in_hbm = device_pointer(weight, &wdev);
    if (in_hbm) {
        if (wdev != dev) {
            set_err("il_upload_quantize: weight is on device %d, the current device is %d", wdev, dev);
            return nullptr;
        }
        if (!device_range_ok(weight, src_bytes, "il_upload_quantize: weight")) return nullptr;
    }
    Planes pl;
    if (!alloc_planes("il_upload_quantize", fmt, n_out, n_in, &pl)) return nullptr;
    hipStream_t s = ctx->upload_stream;
    void *staging = nullptr;
    hipError_t e = hipSuccess;
    if (!in_hbm) {
        e = hipMalloc(&staging, (size_t)src_bytes);
        if (e == hipSuccess) e = hipMemcpyAsync(staging, weight, (size_t)src_bytes, hipMemcpyHostToDevice, s);
    }
    // the tiled planes' padding (rows past n_out, blocks past nb) reads zero
    if (e == hipSuccess) e = hipMemsetAsync(pl.scales_t, 0, (size_t)pl.tiled_bytes, s);
    if (e == hipSuccess && fmt == IL_Q4 && q4_padded(n_out, n_in))
        e = hipMemsetAsync(pl.codes, 0, (size_t)pl.code_bytes, s);
    const bool timing = timing_on();
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    if (timing) {
        (void)hipEventCreate(&ev0);
        (void)hipEventCreate(&ev1);
        (void)hipEventRecord(ev0, s);
    }
    if (e == hipSuccess)
        e = il::launch_quantize(fmt, src == IL_SRC_F32 ? il::SRC_F32 : il::SRC_BF16, in_hbm ? weight : staging,
                                reinterpret_cast<uint8_t *>(pl.codes), pl.scales, pl.scales_t, n_out, n_in, s);
    if (timing) (void)hipEventRecord(ev1, s);
    hipError_t se = hipStreamSynchronize(s);
    if (e == hipSuccess) e = se;
    if (timing) {
        float ms = 0.f;
        if (e == hipSuccess && hipEventElapsedTime(&ms, ev0, ev1) == hipSuccess)
            g_stats[2].timed_ns += (uint64_t)(ms * 1e6);
        (void)hipEventDestroy(ev0);
        (void)hipEventDestroy(ev1);
    }
    if (staging) (void)hipFree(staging);
    if (e != hipSuccess) {
        (void)hipFree(pl.alloc);
        set_err("il_upload_quantize: copy/quantise failed: %s", hipGetErrorString(e));
        return nullptr;
    }
    g_stats[2].calls++;
    g_stats[2].launches++;
    g_stats[2].jobs++;
    g_stats[2].bytes += (uint64_t)src_bytes;
    return make_handle(fmt, dev, n_out, n_in, pl);
}

int64_t il_download(const il_weight *w, void *host_out, int64_t cap) {
    g_err.clear();
    if (!w) {
        set_err("il_download: handle is NULL");
        return -1;
    }
    const int64_t hb = w->host_bytes;
    if (!host_out || cap < hb) return hb;  // size query
    return on_device(w->device, [&]() -> int64_t {
        DeviceCtx *ctx = context(nullptr);
        if (!ctx) return -1;
        hipStream_t s = ctx->upload_stream;
        void *staging = nullptr;
        hipError_t e = hipSuccess;
        if (w->fmt == IL_BF16) {
            e = hipMemcpyAsync(host_out, w->codes, (size_t)hb, hipMemcpyDeviceToHost, s);
        } else {
            e = hipMalloc(&staging, (size_t)hb);
            if (e == hipSuccess)
                e = il::launch_unrepack(w->fmt, w->codes, w->scales, static_cast<uint8_t *>(staging), w->n_out,
                                        w->n_in, s);
            if (e == hipSuccess) e = hipMemcpyAsync(host_out, staging, (size_t)hb, hipMemcpyDeviceToHost, s);
        }
        hipError_t se = hipStreamSynchronize(s);
        if (e == hipSuccess) e = se;
        if (staging) (void)hipFree(staging);
        if (e != hipSuccess) {
            set_err("il_download: %s", hipGetErrorString(e));
            return (int64_t)-1;
        }
        return hb;
    });
}

void il_free(il_weight *w) {
    if (!w) return;
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != w->device) (void)hipSetDevice(w->device);
    (void)hipFree(w->alloc);
    if (cur != w->device && cur >= 0) (void)hipSetDevice(cur);
    delete w;
}

}  // extern "C"

namespace {

// One launch group of a call: jobs of one format, at most kMaxJobs of them
// and at most `max_rows` output rows (a single job may exceed it).
struct Batch {
    int fmt;
    std::vector<il::KJob> jobs;
};

std::vector<Batch> plan_batches(const il_job *jobs, int64_t n_jobs) {
    // rows per launch: the kernels count them in 32-bit ints; IL_LAUNCH_ROWS
    // lowers the limit (tests force multi-launch splits with small weights)
    int64_t max_rows = INT_MAX;
    if (const char *v = getenv("IL_LAUNCH_ROWS")) {
        const long long r = atoll(v);
        if (r >= 1 && r < INT_MAX) max_rows = r;
    }
    std::vector<Batch> out;
    for (int fmt = 0; fmt < 3; ++fmt) {
        Batch b{fmt, {}};
        int64_t rows = 0;
        for (int64_t j = 0; j < n_jobs; ++j) {
            const il_weight *w = jobs[j].w;
            if (w->fmt != fmt) continue;
            if (!b.jobs.empty() && rows + w->n_out > max_rows) {
                out.push_back(b);
                b.jobs.clear();
                rows = 0;
            }
            b.jobs.push_back(il::KJob{w->codes, w->scales, w->scales_t, jobs[j].y, (int)w->n_out});
            rows += w->n_out;
            if ((int)b.jobs.size() == il::kMaxJobs) {
                out.push_back(b);
                b.jobs.clear();
                rows = 0;
            }
        }
        if (!b.jobs.empty()) out.push_back(b);
    }
    return out;
}

// il_matmul and il_matmul_noalloc: validation, then one launch group per
// batch.  noalloc: the prefill scratch is the device's static array, no
// event or allocation is made, and a call that would need more scratch than
// the array holds fails before anything is enqueued.
int matmul_impl(const char *who, const float *x, int64_t t, int64_t n_in, const il_job *jobs, int64_t n_jobs,
                void *hip_stream, bool noalloc) {
    g_err.clear();
    if (t < 0 || n_jobs < 0) {
        set_err("%s: negative t (%" PRId64 ") or n_jobs (%" PRId64 ")", who, t, n_jobs);
        return 0;
    }
    if (t == 0 || n_jobs == 0) return 1;  // nothing to do
    if (!jobs) {
        set_err("%s: jobs is NULL", who);
        return 0;
    }
    if (!x) {
        set_err("%s: x is NULL", who);
        return 0;
    }
    if (t > INT_MAX || n_in < il::kBlock || n_in % il::kBlock || n_in > INT_MAX) {
        set_err("%s: bad sizes t = %" PRId64 ", n_in = %" PRId64, who, t, n_in);
        return 0;
    }
    if (reinterpret_cast<uintptr_t>(x) % 16) {
        set_err("%s: x must be 16-byte aligned", who);
        return 0;
    }
    if (env_flag("IL_FORCE_FAIL", "matmul")) {
        set_err("%s: failure injected by IL_FORCE_FAIL", who);
        return 0;
    }
    int dev = -1;
    DeviceCtx *ctx = context(&dev);
    if (!ctx) return 0;

    // ---- validate everything before enqueueing anything ----
    const int64_t x_bytes = t * n_in * (int64_t)sizeof(float);
    if (!device_range_ok(x, x_bytes, "x")) return 0;
    for (int64_t j = 0; j < n_jobs; ++j) {
        const il_job &jb = jobs[j];
        const il_weight *w = jb.w;
        if (!w) {
            set_err("%s: job %" PRId64 " has no weight", who, j);
            return 0;
        }
        if (w->n_in != n_in) {
            set_err("%s: job %" PRId64 ": weight n_in %" PRId64 " != %" PRId64, who, j, w->n_in, n_in);
            return 0;
        }
        if (jb.n_out != w->n_out) {
            set_err("%s: job %" PRId64 ": n_out %" PRId64 " != weight's %" PRId64, who, j, jb.n_out, w->n_out);
            return 0;
        }
        if (w->device != dev) {
            set_err("%s: job %" PRId64 ": weight lives on device %d, current is %d", who, j, w->device, dev);
            return 0;
        }
        if (!jb.y || reinterpret_cast<uintptr_t>(jb.y) % 4) {
            set_err("%s: job %" PRId64 ": y is NULL or misaligned", who, j);
            return 0;
        }
        char what[32];
        snprintf(what, sizeof what, "job %" PRId64 " y", j);
        const int64_t y_bytes = t * jb.n_out * (int64_t)sizeof(float);
        if (!device_range_ok(jb.y, y_bytes, what)) return 0;
        if (overlaps(jb.y, y_bytes, x, x_bytes)) {
            set_err("%s: job %" PRId64 ": y overlaps x", who, j);
            return 0;
        }
        for (int64_t q = 0; q < j; ++q) {
            if (overlaps(jb.y, y_bytes, jobs[q].y, t * jobs[q].n_out * (int64_t)sizeof(float))) {
                set_err("%s: jobs %" PRId64 " and %" PRId64 " write overlapping y", who, q, j);
                return 0;
            }
        }
    }
    const bool decode = t <= il::kGemvMaxT;
    const std::vector<Batch> batches = plan_batches(jobs, n_jobs);
    void *static_xb = nullptr;
    if (noalloc && !decode) {
        size_t need = 0;
        for (const Batch &b : batches) {
            const size_t n = il::gemm_scratch_bytes(b.fmt, (int)t, (int)n_in, b.jobs.data(), (int)b.jobs.size());
            if (n > need) need = n;
        }
        if (need > il::static_scratch_bytes()) {
            set_err("%s: t * n_in = %" PRId64 " needs %zu bytes of scratch (the bf16 copy of x, and at t <= 128 "
                    "the K-split partial sums); the static buffer holds %zu (bf16 weights: t * n_in <= %zu)",
                    who, t * n_in, need, il::static_scratch_bytes(), il::static_scratch_bytes() / 2);
            return 0;
        }
        if (need > 0) {
            const hipError_t e = il::static_scratch(dev, &static_xb);
            if (e != hipSuccess) {
                set_err("%s: address of the static scratch: %s", who, hipGetErrorString(e));
                return 0;
            }
        }
    }

    // ---- one launch group per batch (a format, <= kMaxJobs jobs) ----
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    PathStats &st = g_stats[decode ? 0 : 1];
    const bool timing = !noalloc && timing_on();
    // a prefill call of one launch group also times its pre-pass apart
    const bool split = timing && !decode && batches.size() == 1 &&
                       il::gemm_scratch_bytes(batches[0].fmt, (int)t, (int)n_in, batches[0].jobs.data(),
                                              (int)batches[0].jobs.size()) > 0;
    hipEvent_t ev0 = nullptr, ev1 = nullptr, evm = nullptr;
    if (timing) {
        (void)hipEventCreate(&ev0);
        (void)hipEventCreate(&ev1);
        if (split) (void)hipEventCreate(&evm);
        (void)hipEventRecord(ev0, s);
    }
    uint64_t launches = 0, bytes = 0;
    for (const Batch &b : batches) {
        const int nb = (int)b.jobs.size();
        hipError_t e;
        if (decode)
            e = il::launch_gemv(b.fmt, x, (int)t, (int)n_in, b.jobs.data(), nb, ctx->cu_count, s);
        else if (noalloc)
            e = il::launch_gemm(b.fmt, x, static_xb, (int)t, (int)n_in, b.jobs.data(), nb, ctx->cu_count, s);
        else
            e = run_gemm(ctx, b.fmt, x, (int)t, (int)n_in, b.jobs.data(), nb, s, false, evm);
        if (e != hipSuccess) {
            set_err("%s: kernel launch failed: %s", who, hipGetErrorString(e));
            g_failed++;
            return 0;
        }
        ++launches;
    }
    for (int64_t j = 0; j < n_jobs; ++j) bytes += (uint64_t)jobs[j].w->host_bytes;
    if (timing) {
        (void)hipEventRecord(ev1, s);
        (void)hipEventSynchronize(ev1);
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, ev0, ev1) == hipSuccess) st.timed_ns += (uint64_t)(ms * 1e6);
        float pms = 0.f;
        if (split && hipEventElapsedTime(&pms, ev0, evm) == hipSuccess) {
            st.split_calls++;
            st.prepass_ns += (uint64_t)(pms * 1e6);
        }
        (void)hipEventDestroy(ev0);
        (void)hipEventDestroy(ev1);
        if (evm) (void)hipEventDestroy(evm);
    }
    uint64_t flops = 0;
    for (int64_t j = 0; j < n_jobs; ++j) flops += 2ull * (uint64_t)t * (uint64_t)jobs[j].n_out * (uint64_t)n_in;
    st.calls++;
    st.launches += launches;
    st.jobs += (uint64_t)n_jobs;
    st.bytes += bytes;
    st.flops += flops;
    return 1;
}

}  // namespace

extern "C" {

int il_matmul(const float *x, int64_t t, int64_t n_in, const il_job *jobs, int64_t n_jobs, void *hip_stream) {
    return matmul_impl("il_matmul", x, t, n_in, jobs, n_jobs, hip_stream, false);
}

int il_matmul_noalloc(const float *x, int64_t t, int64_t n_in, const il_job *jobs, int64_t n_jobs,
                      void *hip_stream) {
    return matmul_impl("il_matmul_noalloc", x, t, n_in, jobs, n_jobs, hip_stream, true);
}

int il_matmul_gelu_mul(const float *x, int64_t t, int64_t n_in, const il_weight *gate, const il_weight *up,
                       int64_t n_out, float *y, void *hip_stream) {
    g_err.clear();
    if (t < 0) {
        set_err("il_matmul_gelu_mul: negative t (%" PRId64 ")", t);
        return 0;
    }
    if (t == 0) return 1;
    if (!x || !y || !gate || !up) {
        set_err("il_matmul_gelu_mul: x, y, gate or up is NULL");
        return 0;
    }
    if (t > INT_MAX || n_in < il::kBlock || n_in % il::kBlock || n_in > INT_MAX) {
        set_err("il_matmul_gelu_mul: bad sizes t = %" PRId64 ", n_in = %" PRId64, t, n_in);
        return 0;
    }
    if (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(y) % 4) {
        set_err("il_matmul_gelu_mul: x must be 16-byte and y 4-byte aligned");
        return 0;
    }
    if (gate->fmt != up->fmt || gate->n_in != n_in || up->n_in != n_in || gate->n_out != n_out ||
        up->n_out != n_out) {
        set_err("il_matmul_gelu_mul: gate and up must share the format and the shape [n_out = %" PRId64
                ", n_in = %" PRId64 "]",
                n_out, n_in);
        return 0;
    }
    if (env_flag("IL_FORCE_FAIL", "matmul")) {
        set_err("il_matmul_gelu_mul: failure injected by IL_FORCE_FAIL");
        return 0;
    }
    int dev = -1;
    DeviceCtx *ctx = context(&dev);
    if (!ctx) return 0;
    if (gate->device != dev || up->device != dev) {
        set_err("il_matmul_gelu_mul: the weights live on another device than the current %d", dev);
        return 0;
    }
    const int64_t x_bytes = t * n_in * (int64_t)sizeof(float);
    const int64_t y_bytes = t * n_out * (int64_t)sizeof(float);
    if (!device_range_ok(x, x_bytes, "x") || !device_range_ok(y, y_bytes, "y")) return 0;
    if (overlaps(y, y_bytes, x, x_bytes)) {
        set_err("il_matmul_gelu_mul: y overlaps x");
        return 0;
    }
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const bool decode = t <= il::kGemvMaxT;
    PathStats &st = g_stats[decode ? 0 : 1];
    const bool timing = timing_on();
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    if (timing) {
        (void)hipEventCreate(&ev0);
        (void)hipEventCreate(&ev1);
        (void)hipEventRecord(ev0, s);
    }
    const il::KJob jobs[2] = {il::KJob{gate->codes, gate->scales, gate->scales_t, y, (int)n_out},
                              il::KJob{up->codes, up->scales, up->scales_t, y, (int)n_out}};
    hipError_t e = decode ? il::launch_gemv(gate->fmt, x, (int)t, (int)n_in, jobs, 2, ctx->cu_count, s, true)
                          : run_gemm(ctx, gate->fmt, x, (int)t, (int)n_in, jobs, 2, s, true);
    if (timing) {
        (void)hipEventRecord(ev1, s);
        (void)hipEventSynchronize(ev1);
        float ms = 0.f;
        if (e == hipSuccess && hipEventElapsedTime(&ms, ev0, ev1) == hipSuccess) st.timed_ns += (uint64_t)(ms * 1e6);
        (void)hipEventDestroy(ev0);
        (void)hipEventDestroy(ev1);
    }
    if (e != hipSuccess) {
        set_err("il_matmul_gelu_mul: kernel launch failed: %s", hipGetErrorString(e));
        g_failed++;
        return 0;
    }
    st.calls++;
    st.launches++;
    st.jobs += 2;
    st.bytes += (uint64_t)(gate->host_bytes + up->host_bytes);
    st.flops += 4ull * (uint64_t)t * (uint64_t)n_out * (uint64_t)n_in;
    return 1;
}

int64_t il_centroid_argmax_workspace(int64_t t, int64_t n_centroids, int64_t top_k) {
    if (t < 0 || n_centroids < 1 || top_k < 1 || t > il::kGemvMaxT || n_centroids > INT_MAX) return -1;
    if (top_k > n_centroids) top_k = n_centroids;
    return (int64_t)il::lm_head_workspace_bytes((int)t, (int)n_centroids, (int)top_k);
}

int il_centroid_argmax(const float *x, int64_t t, int64_t h, const il_weight *centroids, const il_weight *embed,
                       const uint32_t *ordering, int64_t top_k, int32_t *token, int32_t *clusters, float *score,
                       void *workspace, int64_t workspace_bytes, void *hip_stream) {
    g_err.clear();
    if (t < 0) {
        set_err("il_centroid_argmax: negative t");
        return 0;
    }
    if (t == 0) return 1;
    if (!x || !centroids || !embed || !ordering || !token) {
        set_err("il_centroid_argmax: x, centroids, embed, ordering or token is NULL");
        return 0;
    }
    if (t > il::kGemvMaxT) {
        set_err("il_centroid_argmax: t = %" PRId64 " rows; at most %d", t, il::kGemvMaxT);
        return 0;
    }
    if (centroids->fmt != IL_BF16 || embed->fmt != IL_BF16 || centroids->n_in != h || embed->n_in != h) {
        set_err("il_centroid_argmax: centroids and embed must be bf16 with n_in = h = %" PRId64, h);
        return 0;
    }
    const int64_t n_c = centroids->n_out, vocab = embed->n_out;
    if (vocab % n_c) {
        set_err("il_centroid_argmax: vocabulary %" PRId64 " is not a multiple of the %" PRId64 " centroids", vocab,
                n_c);
        return 0;
    }
    if (top_k < 1) {
        set_err("il_centroid_argmax: top_k = %" PRId64 " must be at least 1", top_k);
        return 0;
    }
    if (top_k > n_c) top_k = n_c;  // Drafter::step: k = top_k_centroids.min(num_centroids)
    if (il::lm_head_lds_bytes((int)n_c, (int)h, (int)top_k) > il::kLmHeadMaxLds) {
        set_err("il_centroid_argmax: %" PRId64 " centroids and h = %" PRId64 " exceed the LDS of one workgroup", n_c, h);
        return 0;
    }
    if (reinterpret_cast<uintptr_t>(x) % 16) {
        set_err("il_centroid_argmax: x must be 16-byte aligned");
        return 0;
    }
    if (env_flag("IL_FORCE_FAIL", "matmul")) {
        set_err("il_centroid_argmax: failure injected by IL_FORCE_FAIL");
        return 0;
    }
    int dev = -1;
    DeviceCtx *ctx = context(&dev);
    if (!ctx) return 0;
    if (centroids->device != dev || embed->device != dev) {
        set_err("il_centroid_argmax: the weights live on another device than the current %d", dev);
        return 0;
    }
    if (!device_range_ok(x, t * h * 4, "x") || !device_range_ok(ordering, vocab * 4, "ordering") ||
        !device_range_ok(token, t * 4, "token") ||
        (clusters && !device_range_ok(clusters, t * top_k * 4, "clusters")) ||
        (score && !device_range_ok(score, t * 4, "score")))
        return 0;
    if (workspace) {
        const int64_t need = (int64_t)il::lm_head_workspace_bytes((int)t, (int)n_c, (int)top_k);
        if (workspace_bytes < need) {
            set_err("il_centroid_argmax: workspace of %" PRId64 " bytes, %" PRId64 " needed", workspace_bytes, need);
            return 0;
        }
        if (!device_range_ok(workspace, need, "workspace")) return 0;
    }
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const il::KJob cj{centroids->codes, nullptr, nullptr, nullptr, (int)n_c};
    hipError_t e = il::launch_lm_head(x, (int)t, (int)h, cj, static_cast<const uint16_t *>(embed->codes),
                                      (int)vocab, ordering, (int)top_k, token, clusters, score, workspace,
                                      ctx->cu_count, s);
    if (e != hipSuccess) {
        set_err("il_centroid_argmax: launch failed: %s", hipGetErrorString(e));
        g_failed++;
        return 0;
    }
    PathStats &st = g_stats[0];
    st.calls++;
    st.launches += 3;
    st.jobs += 1;
    st.bytes += (uint64_t)(centroids->host_bytes + t * top_k * (vocab / n_c) * h * 2);
    st.flops += 2ull * (uint64_t)t * (uint64_t)h * (uint64_t)(n_c + top_k * (vocab / n_c));
    return 1;
}

int il_read_probe(const void *buf, int64_t bytes, int64_t chunk, int waves, int depth, void *sink,
                  int64_t sink_bytes, void *hip_stream) {
    g_err.clear();
    if (!buf || !sink || bytes <= 0 || chunk < 1024 || chunk % 16 || chunk >= (1ll << 31) || waves < 1 ||
        waves > 16 || (depth != 1 && depth != 2 && depth != 4 && depth != 8 && depth != 16)) {
        set_err("il_read_probe: bad arguments (chunk a multiple of 16 in [1024, 2^31), waves 1..16, depth 1, 2, 4, "
                "8 or 16)");
        return 0;
    }
    int dev = -1;
    if (!context(&dev)) return 0;
    const int64_t grid = (bytes + chunk - 1) / chunk;
    if (sink_bytes < grid * 4) {
        set_err("il_read_probe: sink of %" PRId64 " bytes, %" PRId64 " needed", sink_bytes, grid * 4);
        return 0;
    }
    if (!device_range_ok(buf, bytes, "buf") || !device_range_ok(sink, grid * 4, "sink")) return 0;
    const hipError_t e = il::launch_read_probe(buf, bytes, chunk, waves, depth, static_cast<uint32_t *>(sink),
                                               static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) {
        set_err("il_read_probe: launch failed: %s", hipGetErrorString(e));
        return 0;
    }
    return 1;
}

int il_wants(int64_t n_out, int64_t n_in, int64_t t) {
    if (n_out <= 0 || n_in <= 0 || t <= 0) return 0;
    double min_flop = 262144.0;  // 2^18
    if (const char *v = getenv("IL_WANTS_MIN_FLOP")) {
        char *end = nullptr;
        double d = strtod(v, &end);
        if (end != v && d >= 0) min_flop = d;
    }
    return 2.0 * (double)n_out * (double)n_in * (double)t >= min_flop ? 1 : 0;
}

const char *il_name(void) { return "il-hip-gfx950"; }

int64_t il_stats(char *buf, int64_t cap) {
    std::string s;
    char line[512];
    const char *names[3] = {"decode_gemv", "prefill_gemm", "upload_quantize"};
    for (int i = 0; i < 3; ++i) {
        const PathStats &p = g_stats[i];
        snprintf(line, sizeof line,
                 "%s: calls=%" PRIu64 " launches=%" PRIu64 " jobs=%" PRIu64 " weight_bytes=%" PRIu64
                 " flops=%" PRIu64 " device_ms=%.6f split_calls=%" PRIu64 " prepass_ms=%.6f\n",
                 names[i], (uint64_t)p.calls, (uint64_t)p.launches, (uint64_t)p.jobs,
                 (uint64_t)p.bytes, (uint64_t)p.flops, (double)p.timed_ns / 1e6, (uint64_t)p.split_calls,
                 (double)p.prepass_ns / 1e6);
        s += line;
    }
    snprintf(line, sizeof line, "uploads: count=%" PRIu64 " bytes=%" PRIu64 "\nfailed_calls: %" PRIu64 "\n",
             (uint64_t)g_uploads, (uint64_t)g_upload_bytes, (uint64_t)g_failed);
    s += line;
    if (buf && cap > 0) {
        size_t n = s.size() < (size_t)(cap - 1) ? s.size() : (size_t)(cap - 1);
        memcpy(buf, s.data(), n);
        buf[n] = '\0';
    }
    return (int64_t)s.size();
}

int64_t il_weight_bytes(const il_weight *w) { return w ? w->host_bytes : -1; }

const char *il_last_error(void) { return g_err.c_str(); }

}  // extern "C"
