// Staging ring for host-resident KV: planner, budget latch, delivery cursor
// and slot state machine.  HIP-free: every device operation goes through the
// Transport interface, implemented with the HIP runtime in kvd_ring_hip.cpp
// and by a CPU simulator in the test suite.
//
// Passages followed ("sched: pipeline the delivery of a host-resident KV cache
// (R4)"): What it does 1 (stable prefix), 2 (a ring outside the allocator, a
// ready/release event pair per slot), 3 (N + 2 slots, deliveries issued after
// the consumer is enqueued, recycling ordered stream to stream); the depth
// knob (0 = ordered path exactly, only engages when deliveries exist); Device
// memory (budget checked before anything is allocated, on every plan, latched;
// transport created lazily and released with the ring).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <memory>
#include <vector>

#include "kvd_internal.h"

namespace kvd {

typedef void* StreamH;
typedef void* EventH;

// What the ring needs from a device runtime.  Every int return is 0 on
// success; error_text() describes the last failure.
class Transport {
public:
    virtual ~Transport() {}
    virtual int current_device(int* dev) = 0;
    virtual int alloc(size_t bytes, void** p) = 0;
    virtual void release(void* p) = 0;
    virtual int stream_create(StreamH* s) = 0;  // non-blocking, default priority
    virtual void stream_destroy(StreamH s) = 0;
    virtual int event_create(EventH* e) = 0;    // no timing
    virtual void event_destroy(EventH e) = 0;
    virtual int copy_h2d(void* dst, const void* src, size_t n, StreamH s) = 0;
    virtual int record(EventH e, StreamH s) = 0;
    virtual int wait(StreamH s, EventH e) = 0;  // s waits for e's latest record
    virtual int stream_sync(StreamH s) = 0;
    virtual int event_sync(EventH e) = 0;
    virtual int host_pinned(const void* p, size_t n, int* pinned) = 0;
    // Test support: hold stream s for about `us` microseconds (bounded), so
    // that the copies queued after it start late.  No-op by default.
    virtual int delay(StreamH s, uint32_t us) {
        (void)s;
        (void)us;
        return 0;
    }
    virtual const char* error_text() = 0;
};

// Ring size for depth N: N + 2 slots, each cap_rows K rows and cap_rows V rows.
// Returns false on overflow.  Depth 0 has no ring (need = 0).
bool ring_need_bytes(int32_t depth, int64_t cap_rows, int64_t row_bytes, int64_t v_row_bytes, int64_t* need);

// Bytes of one V row of a stage call (0 in the arguments means = row_bytes).
inline int64_t v_row_bytes_of(const kvd_stage_args* a) { return a->v_row_bytes ? a->v_row_bytes : a->row_bytes; }

// Transfer streams per ring: a delivery's bytes are split evenly between
// them (K on one and V on the other when the rows are equal), so two DMA
// engines copy in parallel (one engine tops out below the host link, and
// engines differ in speed).
constexpr int kXferStreams = 2;

class Ring {
public:
    Ring(std::unique_ptr<Transport> t, int32_t depth, int64_t budget);
    ~Ring();

    int stage(const kvd_stage_args* a, StreamH compute, kvd_slot_view* out);
    int release(int32_t layer, StreamH compute);
    // Test support: before every copy on a transfer stream, a delay of up to
    // max_us microseconds drawn from a generator seeded with `seed` (0 = off).
    void set_transfer_delay(uint32_t max_us, uint64_t seed) {
        delay_max_us_ = max_us;
        delay_state_ = seed | 1;
    }
    void stats(kvd_ring_stats* out) const;
    // Wait for outstanding transfers and releases, free every device resource.
    void teardown();

private:
    enum SlotState { FREE = 0, STAGED = 1, ACQUIRED = 2, RELEASED = 3 };
    struct Slot {
        void* k = nullptr;
        void* v = nullptr;
        EventH ready[kXferStreams] = {nullptr, nullptr};  // one per transfer stream
        EventH rel = nullptr;
        int state = FREE;
        int32_t layer = -1;
        int64_t prefix_rows = 0;
        int64_t row_bytes = 0;
        int64_t v_row_bytes = 0;
        const void* host_k = nullptr;
        const void* host_v = nullptr;
        uint64_t delivery = 0;  // cursor value of the current delivery
        bool released_once = false;
    };

    int validate(const kvd_stage_args* a) const;
    // Decide ordered vs ring for this call; allocates lazily.  Returns KVD_OK
    // (ring usable), KVD_DECLINED (ordered path), or an error.
    int plan(const kvd_stage_args* a);
    int engage(int64_t k_bytes, int64_t v_bytes);
    void free_resources();
    bool busy() const;  // any slot STAGED or ACQUIRED
    int find_layer(int32_t layer, int state) const;
    int deliver_prefix(const kvd_stage_args* a, int64_t rows, int* slot_out);
    int ordered_acquire(const kvd_stage_args* a, StreamH compute, kvd_slot_view* out);

    std::unique_ptr<Transport> t_;
    int32_t depth_;
    int64_t budget_;
    int32_t n_slots_;
    bool declined_ = false;
    bool engaged_ = false;
    int device_ = -1;
    int64_t slot_bytes_ = 0;    // bytes of the K buffer of a slot
    int64_t slot_v_bytes_ = 0;  // bytes of the V buffer of a slot
    int64_t need_ = 0;
    StreamH xfer_[kXferStreams] = {nullptr, nullptr};
    std::vector<Slot> slots_;
    uint64_t cursor_ = 0;        // deliveries issued so far
    kvd_ring_stats st_{};
    uint32_t delay_max_us_ = 0;
    uint64_t delay_state_ = 1;
    int transfer_delay(StreamH s);  // the test-support delay before a transfer-stream copy
};

}  // namespace kvd

// The C handle is the ring itself.
struct kvd_ring {
    kvd::Ring impl;
    kvd_ring(std::unique_ptr<kvd::Transport> t, int32_t depth, int64_t budget)
        : impl(std::move(t), depth, budget) {}
};
