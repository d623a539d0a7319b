// Device-memory streaming-read probe.  A grid-stride kernel reads every
// 16-byte unit of a device buffer once (non-temporal 16-byte loads, eight
// independent ones in flight per lane, consecutive lanes on consecutive
// units, one 4-wave workgroup per CU: the fastest of the shapes measured on
// MI355X, 7.0-7.3 TB/s against 6.2-6.4 with the default cache policy) and
// folds them into a per-lane XOR, stored only if it equals a fixed pattern:
// the loads cannot be dropped and, over a zeroed buffer, nothing is written.
// Timed with HIP events.  This is the read rate of this device's memory that
// the decode kernel's K/V stream is compared with, beside the vendor's peak
// (device-resident decode attention is bound by reading the KV cache: "sched:
// pipeline the delivery of a host-resident KV cache (R4)", opening paragraph,
// the attention every decode token pays for).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "kvd_internal.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;                 // 16-byte loads in flight per lane
constexpr int kBlocksPerCu = 1;
constexpr uint32_t kSinkPattern = 0x9E3779B9u;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__global__ void __launch_bounds__(kThreads)
read_stream_kernel(const u32x4* __restrict__ p, size_t n16, uint32_t* __restrict__ sink) {
    uint32_t acc = 0;
    const size_t step = (size_t)gridDim.x * kThreads * kUnroll;
    for (size_t base = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n16; base += step) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t i = base + (size_t)u * kThreads;
            v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : (u32x4){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == kSinkPattern) sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc;
}

struct ReadProbeResources {
    void* buf = nullptr;
    void* sink = nullptr;
    hipStream_t stream = nullptr;
    hipEvent_t ev[2] = {nullptr, nullptr};
    ~ReadProbeResources() {
        for (hipEvent_t e : ev)
            if (e) (void)hipEventDestroy(e);
        if (stream) {
            (void)hipStreamSynchronize(stream);
            (void)hipStreamDestroy(stream);
        }
        if (sink) (void)hipFree(sink);
        if (buf) (void)hipFree(buf);
    }
};

int hip_fail(const char* what, hipError_t e) {
    (void)hipGetLastError();
    return kvd::fail(KVD_EHIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" int kvd_hbm_read_probe(size_t bytes, int32_t reps, double* gbps) {
    kvd::clear_error();
    if (!gbps) return kvd::fail(KVD_EINVAL, "gbps is NULL");
    if (bytes < ((size_t)1 << 20) || bytes > ((size_t)64 << 30) || bytes % 16)
        return kvd::fail(KVD_EINVAL, "bytes %zu must be a multiple of 16 in [1 MiB, 64 GiB]", bytes);
    if (reps < 1 || reps > 1000) return kvd::fail(KVD_EINVAL, "reps %d out of [1, 1000]", reps);
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail("hipDeviceGetAttribute", e);
    cus = std::min(std::max(cus, 1), 4096);
    const unsigned grid = (unsigned)(cus * kBlocksPerCu);
    ReadProbeResources r;
    if ((e = hipMalloc(&r.buf, bytes)) != hipSuccess) return hip_fail("hipMalloc", e);
    if ((e = hipMalloc(&r.sink, (size_t)grid * kThreads * sizeof(uint32_t))) != hipSuccess)
        return hip_fail("hipMalloc", e);
    if ((e = hipStreamCreateWithFlags(&r.stream, hipStreamNonBlocking)) != hipSuccess)
        return hip_fail("hipStreamCreateWithFlags", e);
    for (hipEvent_t& ev : r.ev)
        if ((e = hipEventCreate(&ev)) != hipSuccess) return hip_fail("hipEventCreate", e);
    if ((e = hipMemsetAsync(r.buf, 0, bytes, r.stream)) != hipSuccess) return hip_fail("hipMemsetAsync", e);
    std::vector<float> ms;
    for (int rep = 0; rep <= reps; ++rep) {  // rep 0 is a warm-up
        if ((e = hipEventRecord(r.ev[0], r.stream)) != hipSuccess) return hip_fail("hipEventRecord", e);
        hipLaunchKernelGGL(read_stream_kernel, dim3(grid), dim3(kThreads), 0, r.stream, (const u32x4*)r.buf,
                           bytes / 16, (uint32_t*)r.sink);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail("read_stream_kernel launch", e);
        if ((e = hipEventRecord(r.ev[1], r.stream)) != hipSuccess) return hip_fail("hipEventRecord", e);
        if ((e = hipEventSynchronize(r.ev[1])) != hipSuccess) return hip_fail("hipEventSynchronize", e);
        float t = 0.f;
        if ((e = hipEventElapsedTime(&t, r.ev[0], r.ev[1])) != hipSuccess) return hip_fail("hipEventElapsedTime", e);
        if (rep > 0) ms.push_back(t);
    }
    std::sort(ms.begin(), ms.end());
    const double med = ms[ms.size() / 2];
    *gbps = med > 0 ? (double)bytes / (med * 1e-3) / 1e9 : 0.0;
    return KVD_OK;
}
