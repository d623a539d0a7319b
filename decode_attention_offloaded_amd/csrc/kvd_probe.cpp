// Host-to-device link probe: pinned host memory copied to the device the way
// the staging ring copies it (hipMemcpyAsync from hipHostMalloc'ed memory on
// non-blocking streams at the default priority, a delivery's bytes split
// evenly between the streams), timed with HIP events.  The ring's throughput
// is reported against the plateau this measures ("F5 -- Advanced KV Cache
// Techniques", W1: a PCIe probe of the pinned host-to-device plateau).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "kvd_internal.h"

namespace {

struct ProbeResources {
    void* host = nullptr;
    void* dev = nullptr;
    std::vector<hipStream_t> streams;
    std::vector<hipEvent_t> events;
    ~ProbeResources() {
        for (hipEvent_t e : events) (void)hipEventDestroy(e);
        for (hipStream_t s : streams) (void)hipStreamDestroy(s);
        if (dev) (void)hipFree(dev);
        if (host) (void)hipHostFree(host);
    }
};

int hip_fail(const char* what, hipError_t e) {
    (void)hipGetLastError();
    return kvd::fail(KVD_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" int kvd_link_probe(size_t bytes, int32_t n_streams, int32_t reps, double* gbps) {
    kvd::clear_error();
    if (!gbps) return kvd::fail(KVD_EINVAL, "gbps is NULL");
    if (bytes < 4096 || bytes > ((size_t)8 << 30)) return kvd::fail(KVD_EINVAL, "bytes %zu out of [4096, 8 GiB]", bytes);
    if (n_streams < 1 || n_streams > 4) return kvd::fail(KVD_EINVAL, "n_streams %d out of [1, 4]", n_streams);
    if (reps < 1 || reps > 1000) return kvd::fail(KVD_EINVAL, "reps %d out of [1, 1000]", reps);
    ProbeResources r;
    hipError_t e = hipHostMalloc(&r.host, bytes, hipHostMallocDefault);
    if (e != hipSuccess) return hip_fail("hipHostMalloc", e);
    e = hipMalloc(&r.dev, bytes);
    if (e != hipSuccess) return hip_fail("hipMalloc", e);
    // touch the host pages once so the timed copies see resident memory
    for (size_t i = 0; i < bytes; i += 4096) ((volatile char*)r.host)[i] = (char)i;
    for (int i = 0; i < n_streams; ++i) {
        hipStream_t s = nullptr;
        e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
        if (e != hipSuccess) return hip_fail("hipStreamCreateWithFlags", e);
        r.streams.push_back(s);
    }
    // a start and a stop event per stream; the span of a round is from the
    // earliest start to the latest stop (events of one device share a clock)
    for (int i = 0; i < 2 * n_streams; ++i) {
        hipEvent_t ev = nullptr;
        e = hipEventCreate(&ev);
        if (e != hipSuccess) return hip_fail("hipEventCreate", e);
        r.events.push_back(ev);
    }
    // even pieces, 16-byte aligned, the last one takes the remainder
    const size_t piece = (bytes / (size_t)n_streams) & ~(size_t)15;
    std::vector<float> ms;
    for (int rep = 0; rep <= reps; ++rep) {  // rep 0 is a warm-up
        for (int i = 0; i < n_streams; ++i) {
            hipStream_t s = r.streams[i];
            const size_t off = (size_t)i * piece;
            const size_t n = (i == n_streams - 1) ? bytes - off : piece;
            if ((e = hipEventRecord(r.events[2 * i], s)) != hipSuccess) return hip_fail("hipEventRecord", e);
            e = hipMemcpyAsync((char*)r.dev + off, (const char*)r.host + off, n, hipMemcpyHostToDevice, s);
            if (e != hipSuccess) return hip_fail("hipMemcpyAsync", e);
            if ((e = hipEventRecord(r.events[2 * i + 1], s)) != hipSuccess) return hip_fail("hipEventRecord", e);
        }
        float lo = 0.f, hi = 0.f;
        for (int i = 0; i < n_streams; ++i) {
            if ((e = hipEventSynchronize(r.events[2 * i + 1])) != hipSuccess) return hip_fail("hipEventSynchronize", e);
            float a = 0.f, b = 0.f;
            if ((e = hipEventElapsedTime(&a, r.events[0], r.events[2 * i])) != hipSuccess ||
                (e = hipEventElapsedTime(&b, r.events[0], r.events[2 * i + 1])) != hipSuccess)
                return hip_fail("hipEventElapsedTime", e);
            lo = std::min(lo, a);
            hi = std::max(hi, b);
        }
        if (rep > 0) ms.push_back(hi - lo);
    }
    std::sort(ms.begin(), ms.end());
    const double med = ms[ms.size() / 2];
    *gbps = med > 0 ? (double)bytes / (med * 1e-3) / 1e9 : 0.0;
    return KVD_OK;
}
