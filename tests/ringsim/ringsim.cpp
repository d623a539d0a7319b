// CPU simulator of a device runtime, for testing the staging ring's ordering
// logic without a GPU (tests only; never linked into the product library).
//
// Streams are FIFO queues of operations that execute later, in an order the
// test controls (random interleavings seeded by the test).  An event wait
// captures the event's latest record at enqueue time, as hipStreamWaitEvent
// does.  Copies read host memory when they execute, as DMA does.  Fresh
// device memory is filled with 0xFF so a read of bytes never delivered shows.
// CHECK operations, enqueued by the test on the compute stream where the
// attention kernel would run, compare device bytes with a snapshot.
#include <stdint.h>
#include <string.h>

#include <deque>
#include <map>
#include <memory>
#include <random>
#include <string>
#include <vector>

#include "kvd_ring_core.h"

namespace {

struct SimEvent {
    uint64_t recorded = 0;
    uint64_t completed = 0;
};

enum OpKind { OP_COPY = 0, OP_RECORD = 1, OP_WAIT = 2, OP_CHECK = 3 };

struct Op {
    OpKind kind;
    void* dst = nullptr;
    const void* src = nullptr;
    size_t n = 0;
    SimEvent* ev = nullptr;
    uint64_t gen = 0;
    std::vector<uint8_t> expect;
    int64_t id = 0;
};

struct SimStream {
    std::deque<Op> q;
    int64_t executed[4] = {0, 0, 0, 0};
};

struct Sim {
    std::mt19937_64 rng;
    std::vector<std::unique_ptr<SimStream>> streams;
    std::vector<std::unique_ptr<SimEvent>> events;
    std::map<void*, size_t> allocs;
    int64_t dev_bytes = 0, peak = 0, n_allocs = 0, n_syncs = 0, n_streams_created = 0;
    int64_t fail_after = -1;
    int pinned = 1;
    int device = 0;
    int64_t errors = 0;
    int64_t deadlocks = 0;
    std::string log;

    explicit Sim(uint64_t seed) : rng(seed) {}

    static bool runnable(const SimStream& s) {
        if (s.q.empty()) return false;
        const Op& o = s.q.front();
        return o.kind != OP_WAIT || o.ev->completed >= o.gen;
    }

    void exec(SimStream& s) {
        Op o = std::move(s.q.front());
        s.q.pop_front();
        s.executed[o.kind]++;
        switch (o.kind) {
            case OP_COPY:
                memcpy(o.dst, o.src, o.n);
                break;
            case OP_RECORD:
                if (o.gen > o.ev->completed) o.ev->completed = o.gen;
                break;
            case OP_WAIT:
                break;
            case OP_CHECK:
                if (memcmp(o.dst, o.expect.data(), o.n) != 0) {
                    ++errors;
                    if (log.size() < 4000) log += "check " + std::to_string(o.id) + " saw wrong bytes\n";
                }
                break;
        }
    }

    // Execute one runnable operation picked at random; false if none.
    bool step() {
        std::vector<SimStream*> ready;
        for (auto& s : streams)
            if (runnable(*s)) ready.push_back(s.get());
        if (ready.empty()) return false;
        exec(*ready[rng() % ready.size()]);
        return true;
    }

    bool pending() const {
        for (auto& s : streams)
            if (!s->q.empty()) return true;
        return false;
    }

    // Run until `done` holds; a stall with work queued is a deadlock.
    template <class F>
    int run_until(F done) {
        while (!done()) {
            if (!step()) {
                ++deadlocks;
                log += "deadlock\n";
                return -1;
            }
        }
        return 0;
    }

    SimStream* new_stream() {
        streams.emplace_back(new SimStream());
        return streams.back().get();
    }
};

class SimTransport final : public kvd::Transport {
public:
    explicit SimTransport(Sim* s) : s_(s) {}
    int current_device(int* dev) override {
        *dev = s_->device;
        return 0;
    }
    int alloc(size_t bytes, void** p) override {
        *p = nullptr;
        if (s_->fail_after >= 0 && s_->n_allocs >= s_->fail_after) {
            err_ = "simulated out of device memory";
            return 1;
        }
        void* m = malloc(bytes ? bytes : 1);
        if (!m) return 1;
        memset(m, 0xFF, bytes);  // binary16 0xFFFF is NaN: undelivered bytes show
        s_->allocs[m] = bytes;
        s_->n_allocs++;
        s_->dev_bytes += (int64_t)bytes;
        if (s_->dev_bytes > s_->peak) s_->peak = s_->dev_bytes;
        *p = m;
        return 0;
    }
    void release(void* p) override {
        auto it = s_->allocs.find(p);
        if (it == s_->allocs.end()) {
            s_->errors++;
            s_->log += "free of unknown pointer\n";
            return;
        }
        s_->dev_bytes -= (int64_t)it->second;
        s_->allocs.erase(it);
        free(p);
    }
    int stream_create(kvd::StreamH* s) override {
        *s = s_->new_stream();
        s_->n_streams_created++;
        return 0;
    }
    void stream_destroy(kvd::StreamH s) override {
        SimStream* ss = (SimStream*)s;
        if (!ss->q.empty()) {
            s_->errors++;
            s_->log += "stream destroyed with queued work\n";
        }
    }
    int event_create(kvd::EventH* e) override {
        s_->events.emplace_back(new SimEvent());
        *e = s_->events.back().get();
        return 0;
    }
    void event_destroy(kvd::EventH) override {}
    int copy_h2d(void* dst, const void* src, size_t n, kvd::StreamH s) override {
        Op o;
        o.kind = OP_COPY;
        o.dst = dst;
        o.src = src;
        o.n = n;
        ((SimStream*)s)->q.push_back(std::move(o));
        return 0;
    }
    int record(kvd::EventH e, kvd::StreamH s) override {
        SimEvent* ev = (SimEvent*)e;
        Op o;
        o.kind = OP_RECORD;
        o.ev = ev;
        o.gen = ++ev->recorded;
        ((SimStream*)s)->q.push_back(std::move(o));
        return 0;
    }
    int wait(kvd::StreamH s, kvd::EventH e) override {
        SimEvent* ev = (SimEvent*)e;
        Op o;
        o.kind = OP_WAIT;
        o.ev = ev;
        o.gen = ev->recorded;  // the latest record at the time of the call
        ((SimStream*)s)->q.push_back(std::move(o));
        return 0;
    }
    int stream_sync(kvd::StreamH s) override {
        s_->n_syncs++;
        SimStream* ss = (SimStream*)s;
        return s_->run_until([ss] { return ss->q.empty(); }) == 0 ? 0 : 1;
    }
    int event_sync(kvd::EventH e) override {
        s_->n_syncs++;
        SimEvent* ev = (SimEvent*)e;
        return s_->run_until([ev] { return ev->completed >= ev->recorded; }) == 0 ? 0 : 1;
    }
    int host_pinned(const void*, size_t, int* pinned) override {
        *pinned = s_->pinned;
        return 0;
    }
    const char* error_text() override { return err_; }

private:
    Sim* s_;
    const char* err_ = "";
};

}  // namespace

extern "C" {

void* sim_new(uint64_t seed) { return new Sim(seed); }
void sim_delete(void* sim) { delete (Sim*)sim; }
void sim_configure(void* sim, int pinned, int device, int64_t fail_after) {
    Sim* s = (Sim*)sim;
    s->pinned = pinned;
    s->device = device;
    s->fail_after = fail_after;
}
void* sim_stream_new(void* sim) { return ((Sim*)sim)->new_stream(); }

kvd_ring* sim_ring_create(void* sim, int32_t depth, int64_t budget) {
    return new kvd_ring(std::unique_ptr<kvd::Transport>(new SimTransport((Sim*)sim)), depth, budget);
}

// Enqueue on `stream` a comparison of n device bytes at `dev` with a snapshot
// of `expect` taken now.
void sim_check(void* sim, void* stream, const void* dev, const void* expect, size_t n, int64_t id) {
    (void)sim;
    Op o;
    o.kind = OP_CHECK;
    o.dst = (void*)dev;
    o.n = n;
    o.expect.assign((const uint8_t*)expect, (const uint8_t*)expect + n);
    o.id = id;
    ((SimStream*)stream)->q.push_back(std::move(o));
}

int sim_run(void* sim, int max_steps) {
    Sim* s = (Sim*)sim;
    int k = 0;
    while (k < max_steps && s->step()) ++k;
    return k;
}

int sim_drain(void* sim) {
    Sim* s = (Sim*)sim;
    return s->run_until([s] { return !s->pending(); });
}

// counters: 0 errors, 1 device bytes, 2 peak device bytes, 3 live allocations,
// 4 deadlocks, 5 host syncs, 6 streams created, 7 queued ops
int64_t sim_counter(void* sim, int which) {
    Sim* s = (Sim*)sim;
    switch (which) {
        case 0: return s->errors;
        case 1: return s->dev_bytes;
        case 2: return s->peak;
        case 3: return (int64_t)s->allocs.size();
        case 4: return s->deadlocks;
        case 5: return s->n_syncs;
        case 6: return s->n_streams_created;
        case 7: {
            int64_t n = 0;
            for (auto& st : s->streams) n += (int64_t)st->q.size();
            return n;
        }
    }
    return -1;
}

// Operations of `kind` executed so far on `stream`.
int64_t sim_executed(void* stream, int kind) { return ((SimStream*)stream)->executed[kind]; }

const char* sim_log(void* sim) { return ((Sim*)sim)->log.c_str(); }

}  // extern "C"
