// HIP runtime transport for the staging ring, and kvd_ring_create.
// The eligibility the pages ask of a backend -- asynchronous copies, event
// record and wait, event creation ("sched: pipeline the delivery of a
// host-resident KV cache (R4)", What tensor parallelism would take) -- maps to
// hipMemcpyAsync, hipEventRecord, hipStreamWaitEvent and
// hipEventCreateWithFlags; the transfer stream is an ordinary non-blocking
// stream at the default priority, so its copies run on the DMA engines.
#include <hip/hip_runtime.h>

#include <new>

#include "kvd_ring_core.h"

namespace kvd {
// One wave that spins for about `us` microseconds (kvd_attend.hip).
hipError_t launch_spin(hipStream_t stream, uint32_t us);
}  // namespace kvd

namespace kvd {
namespace {

class HipTransport final : public Transport {
public:
    int current_device(int* dev) override { return check(hipGetDevice(dev)); }
    int alloc(size_t bytes, void** p) override {
        *p = nullptr;
        return check(hipMalloc(p, bytes));
    }
    void release(void* p) override { (void)hipFree(p); }
    int stream_create(StreamH* s) override {
        hipStream_t h = nullptr;
        const int rc = check(hipStreamCreateWithFlags(&h, hipStreamNonBlocking));
        *s = h;
        return rc;
    }
    void stream_destroy(StreamH s) override { (void)hipStreamDestroy((hipStream_t)s); }
    int event_create(EventH* e) override {
        hipEvent_t h = nullptr;
        const int rc = check(hipEventCreateWithFlags(&h, hipEventDisableTiming));
        *e = h;
        return rc;
    }
    void event_destroy(EventH e) override { (void)hipEventDestroy((hipEvent_t)e); }
    int copy_h2d(void* dst, const void* src, size_t n, StreamH s) override {
        return check(hipMemcpyAsync(dst, src, n, hipMemcpyHostToDevice, (hipStream_t)s));
    }
    int record(EventH e, StreamH s) override { return check(hipEventRecord((hipEvent_t)e, (hipStream_t)s)); }
    int wait(StreamH s, EventH e) override { return check(hipStreamWaitEvent((hipStream_t)s, (hipEvent_t)e, 0)); }
    int stream_sync(StreamH s) override { return check(hipStreamSynchronize((hipStream_t)s)); }
    int event_sync(EventH e) override { return check(hipEventSynchronize((hipEvent_t)e)); }
    int host_pinned(const void* p, size_t n, int* pinned) override {
        *pinned = 0;
        if (n == 0) n = 1;
        const void* ends[2] = {p, (const uint8_t*)p + n - 1};
        for (const void* q : ends) {
            hipPointerAttribute_t attr;
            const hipError_t e = hipPointerGetAttributes(&attr, q);
            if (e != hipSuccess) {
                (void)hipGetLastError();  // pageable memory is reported as an error; not sticky
                return 0;
            }
            if (attr.type != hipMemoryTypeHost) return 0;
        }
        *pinned = 1;
        return 0;
    }
    int delay(StreamH s, uint32_t us) override { return check(launch_spin((hipStream_t)s, us)); }
    const char* error_text() override { return last_; }

private:
    int check(hipError_t e) {
        if (e == hipSuccess) return 0;
        last_ = hipGetErrorString(e);
        (void)hipGetLastError();
        return 1;
    }
    const char* last_ = "";
};

}  // namespace
}  // namespace kvd

extern "C" kvd_ring* kvd_ring_create(int32_t depth, size_t budget_bytes) {
    kvd::clear_error();
    if (depth < 0 || depth > 64) {
        kvd::fail(KVD_EINVAL, "depth %d must be in [0, 64]", depth);
        return nullptr;
    }
    const int64_t budget = budget_bytes > (size_t)INT64_MAX ? INT64_MAX : (int64_t)budget_bytes;
    try {
        return new kvd_ring(std::unique_ptr<kvd::Transport>(new kvd::HipTransport()), depth, budget);
    } catch (const std::bad_alloc&) {
        kvd::fail(KVD_ENOMEM, "host allocation failed");
        return nullptr;
    }
}
