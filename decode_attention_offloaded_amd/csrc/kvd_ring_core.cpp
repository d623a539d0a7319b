// Staging ring core (HIP-free).  See kvd_ring_core.h for the passages followed.
#include "kvd_ring_core.h"

#include <limits.h>

#include <new>

namespace kvd {

bool ring_need_bytes(int32_t depth, int64_t cap_rows, int64_t row_bytes, int64_t v_row_bytes, int64_t* need) {
    if (depth <= 0) {
        *need = 0;
        return true;
    }
    const __int128 x = (__int128)(depth + 2) * (__int128)cap_rows * ((__int128)row_bytes + (__int128)v_row_bytes);
    if (x < 0 || x > (__int128)INT64_MAX) return false;
    *need = (int64_t)x;
    return true;
}

Ring::Ring(std::unique_ptr<Transport> t, int32_t depth, int64_t budget)
    : t_(std::move(t)), depth_(depth), budget_(budget), n_slots_(depth > 0 ? depth + 2 : 0) {
    st_.depth = depth;
    st_.n_slots = n_slots_;
    st_.budget_bytes = budget;
    st_.device = -1;
}

Ring::~Ring() { teardown(); }

int Ring::validate(const kvd_stage_args* a) const {
    if (!a) return fail(KVD_EINVAL, "args is NULL");
    if (a->flags != KVD_STAGE_PREFETCH && a->flags != KVD_STAGE_ACQUIRE)
        return fail(KVD_EINVAL, "flags %d must be KVD_STAGE_PREFETCH or KVD_STAGE_ACQUIRE", a->flags);
    if (a->layer < 0) return fail(KVD_EINVAL, "layer %d < 0", a->layer);
    if (!a->host_k || !a->host_v) return fail(KVD_EINVAL, "host_k/host_v must not be NULL");
    if (a->row_bytes <= 0 || a->row_bytes % 4 != 0 || a->row_bytes > (1 << 24))
        return fail(KVD_EINVAL, "row_bytes %lld must be a positive multiple of 4 (< 2^24)", (long long)a->row_bytes);
    if (a->v_row_bytes < 0 || a->v_row_bytes % 4 != 0 || a->v_row_bytes > (1 << 24))
        return fail(KVD_EINVAL, "v_row_bytes %lld must be 0 or a positive multiple of 4 (< 2^24)",
                    (long long)a->v_row_bytes);
    if (a->cap_rows < 1 || a->cap_rows >= ((int64_t)1 << 31))
        return fail(KVD_EINVAL, "cap_rows %lld out of range", (long long)a->cap_rows);
    if (a->n_rows < 1 || a->n_rows > a->cap_rows)
        return fail(KVD_EINVAL, "n_rows %lld must be in [1, cap_rows %lld]", (long long)a->n_rows,
                    (long long)a->cap_rows);
    if (a->stable_rows < 0 || a->stable_rows > a->n_rows)
        return fail(KVD_EINVAL, "stable_rows %lld must be in [0, n_rows %lld]", (long long)a->stable_rows,
                    (long long)a->n_rows);
    return KVD_OK;
}

bool Ring::busy() const {
    for (const Slot& s : slots_)
        if (s.state == STAGED || s.state == ACQUIRED) return true;
    return false;
}

int Ring::find_layer(int32_t layer, int state) const {
    for (size_t i = 0; i < slots_.size(); ++i)
        if (slots_[i].state == state && slots_[i].layer == layer) return (int)i;
    return -1;
}

void Ring::free_resources() {
    for (Slot& s : slots_) {
        if (s.k) t_->release(s.k);
        if (s.v) t_->release(s.v);
        for (EventH e : s.ready)
            if (e) t_->event_destroy(e);
        if (s.rel) t_->event_destroy(s.rel);
    }
    slots_.clear();
    for (StreamH& x : xfer_) {
        if (x) t_->stream_destroy(x);
        x = nullptr;
    }
}

int Ring::engage(int64_t k_bytes, int64_t v_bytes) {
    slots_.assign(n_slots_, Slot());
    bool ok = true;
    for (StreamH& x : xfer_) ok = ok && t_->stream_create(&x) == 0;
    for (int i = 0; ok && i < n_slots_; ++i) {
        Slot& s = slots_[i];
        for (EventH& e : s.ready) ok = ok && t_->event_create(&e) == 0;
        ok = ok && t_->event_create(&s.rel) == 0 && t_->alloc((size_t)k_bytes, &s.k) == 0 &&
             t_->alloc((size_t)v_bytes, &s.v) == 0;
    }
    if (!ok) {
        // a failed allocation is a decline, not an error: undo everything
        free_resources();
        return KVD_ENOMEM;
    }
    engaged_ = true;
    slot_bytes_ = k_bytes;
    slot_v_bytes_ = v_bytes;
    cursor_ = 0;
    st_.ring_bytes = (int64_t)n_slots_ * (k_bytes + v_bytes);
    return KVD_OK;
}

void Ring::teardown() {
    if (!engaged_) return;
    for (StreamH x : xfer_)
        if (x) t_->stream_sync(x);
    for (Slot& s : slots_)
        if (s.released_once && s.rel) t_->event_sync(s.rel);
    free_resources();
    engaged_ = false;
    slot_bytes_ = 0;
    slot_v_bytes_ = 0;
    cursor_ = 0;
    st_.ring_bytes = 0;
}

int Ring::plan(const kvd_stage_args* a) {
    if (depth_ == 0 || declined_) return KVD_DECLINED;
    int64_t need;
    if (!ring_need_bytes(depth_, a->cap_rows, a->row_bytes, v_row_bytes_of(a), &need)) need = INT64_MAX;
    need_ = need;
    st_.need_bytes = need;
    int dev = -1;
    if (t_->current_device(&dev) != 0) return fail(KVD_EHIP, "current device: %s", t_->error_text());
    if (engaged_ && dev != device_)
        return fail(KVD_ESTATE, "ring is bound to device %d but was called on device %d", device_, dev);
    if (need > budget_) {
        // checked before anything is allocated, on every plan; latched
        if (engaged_) {
            if (busy()) return fail(KVD_ESTATE, "ring would exceed its budget while deliveries are in flight");
            teardown();
        }
        declined_ = true;
        return KVD_DECLINED;
    }
    const int64_t slot_bytes = a->cap_rows * a->row_bytes;
    const int64_t slot_v_bytes = a->cap_rows * v_row_bytes_of(a);
    if (engaged_ && (slot_bytes > slot_bytes_ || slot_v_bytes > slot_v_bytes_)) {
        if (busy()) return fail(KVD_ESTATE, "slot capacity grew while deliveries are in flight");
        teardown();
    }
    if (!engaged_) {
        if (engage(slot_bytes, slot_v_bytes) != KVD_OK) {
            declined_ = true;
            return KVD_DECLINED;
        }
        device_ = dev;
        st_.device = dev;
        st_.slot_rows = a->cap_rows;
    }
    return KVD_OK;
}

int Ring::transfer_delay(StreamH s) {
    if (delay_max_us_ == 0) return 0;
    // xorshift64
    delay_state_ ^= delay_state_ << 13;
    delay_state_ ^= delay_state_ >> 7;
    delay_state_ ^= delay_state_ << 17;
    return t_->delay(s, (uint32_t)(delay_state_ % ((uint64_t)delay_max_us_ + 1)));
}

int Ring::deliver_prefix(const kvd_stage_args* a, int64_t rows, int* slot_out) {
    const int s = (int)(cursor_ % (uint64_t)n_slots_);
    Slot& S = slots_[s];
    if (S.state == STAGED || S.state == ACQUIRED)
        return fail(KVD_ESTATE,
                    "slot %d still holds layer %d: release it before staging layer %d (look-ahead deeper than the ring)",
                    s, S.layer, a->layer);
    // stream to stream: the copies wait for the release of the slot's previous
    // layer, recorded earlier in host order on the compute stream
    // The K and V bytes are shared evenly between the two transfer streams
    // (one DMA engine each): K on one and V on the other when the rows are
    // the same size; with narrower V rows the first stream takes the head of
    // K's bytes and the second the rest of K, then V.
    const size_t kb = (size_t)rows * (size_t)a->row_bytes;
    const size_t vb = (size_t)rows * (size_t)v_row_bytes_of(a);
    size_t split = kb;  // bytes of K on stream 0
    if (vb < kb) split = ((kb + vb) / 2) & ~(size_t)15;
    struct Piece {
        void* dst;
        const void* src;
        size_t n;
    };
    const Piece pieces[kXferStreams][2] = {
        {{S.k, a->host_k, split}, {nullptr, nullptr, 0}},
        {{(uint8_t*)S.k + split, (const uint8_t*)a->host_k + split, kb - split}, {S.v, a->host_v, vb}}};
    for (int x = 0; x < kXferStreams; ++x) {
        if (S.released_once && t_->wait(xfer_[x], S.rel) != 0)
            return fail(KVD_EHIP, "wait(release): %s", t_->error_text());
        for (const Piece& pc : pieces[x])
            if (pc.n > 0 && (transfer_delay(xfer_[x]) != 0 || t_->copy_h2d(pc.dst, pc.src, pc.n, xfer_[x]) != 0))
                return fail(KVD_EHIP, "prefix copy: %s", t_->error_text());
        if (t_->record(S.ready[x], xfer_[x]) != 0) return fail(KVD_EHIP, "record(ready): %s", t_->error_text());
    }
    S.state = STAGED;
    S.layer = a->layer;
    S.prefix_rows = rows;
    S.row_bytes = a->row_bytes;
    S.v_row_bytes = v_row_bytes_of(a);
    S.host_k = a->host_k;
    S.host_v = a->host_v;
    S.delivery = cursor_;
    ++cursor_;
    *slot_out = s;
    return KVD_OK;
}

int Ring::ordered_acquire(const kvd_stage_args* a, StreamH compute, kvd_slot_view* out) {
    if (!a->ordered_k || !a->ordered_v) return fail(KVD_EINVAL, "the ordered path needs ordered_k and ordered_v");
    const size_t kb = (size_t)a->n_rows * (size_t)a->row_bytes;
    const size_t vb = (size_t)a->n_rows * (size_t)v_row_bytes_of(a);
    if (t_->copy_h2d(a->ordered_k, a->host_k, kb, compute) != 0 ||
        t_->copy_h2d(a->ordered_v, a->host_v, vb, compute) != 0)
        return fail(KVD_EHIP, "ordered copy: %s", t_->error_text());
    st_.n_acquire_ordered++;
    st_.bytes_ordered += (int64_t)(kb + vb);
    if (out) *out = kvd_slot_view{a->ordered_k, a->ordered_v, a->n_rows, a->row_bytes, 0, -1, v_row_bytes_of(a)};
    return KVD_DECLINED;
}

int Ring::stage(const kvd_stage_args* a, StreamH compute, kvd_slot_view* out) {
    int rc = validate(a);
    if (rc != KVD_OK) return rc;
    int pinned = 0;
    const int64_t vrb = v_row_bytes_of(a);
    if (t_->host_pinned(a->host_k, (size_t)a->n_rows * (size_t)a->row_bytes, &pinned) != 0 || !pinned)
        return fail(KVD_EINVAL, "host_k is not pinned host memory");
    if (t_->host_pinned(a->host_v, (size_t)a->n_rows * (size_t)vrb, &pinned) != 0 || !pinned)
        return fail(KVD_EINVAL, "host_v is not pinned host memory");

    if (a->flags == KVD_STAGE_PREFETCH) {
        if (out) *out = kvd_slot_view{nullptr, nullptr, 0, 0, 0, -1, 0};
        rc = plan(a);
        if (rc != KVD_OK) return rc;  // KVD_DECLINED: nothing to do
        if (find_layer(a->layer, STAGED) >= 0 || find_layer(a->layer, ACQUIRED) >= 0)
            return fail(KVD_ESTATE, "layer %d is already staged", a->layer);
        int s = -1;
        rc = deliver_prefix(a, a->stable_rows, &s);
        if (rc != KVD_OK) return rc;
        st_.n_prefetch++;
        st_.bytes_early += a->stable_rows * (a->row_bytes + vrb);
        return KVD_OK;
    }

    // ACQUIRE
    rc = plan(a);
    if (rc == KVD_DECLINED) return ordered_acquire(a, compute, out);
    if (rc != KVD_OK) return rc;
    if (find_layer(a->layer, ACQUIRED) >= 0) return fail(KVD_ESTATE, "layer %d is already acquired", a->layer);
    int s = find_layer(a->layer, STAGED);
    if (s < 0) {
        // not prefetched (e.g. the first layers of a step): stage the whole layer now
        rc = deliver_prefix(a, a->n_rows, &s);
        if (rc != KVD_OK) return rc;
        st_.n_acquire_primed++;
        st_.bytes_late += a->n_rows * (a->row_bytes + vrb);
    } else {
        Slot& S = slots_[s];
        if (S.row_bytes != a->row_bytes || S.v_row_bytes != vrb || S.host_k != a->host_k || S.host_v != a->host_v)
            return fail(KVD_ESTATE, "ACQUIRE of layer %d does not match its PREFETCH (host buffers or row_bytes)",
                        a->layer);
        if (a->n_rows < S.prefix_rows)
            return fail(KVD_ESTATE, "layer %d: n_rows %lld is below the prefetched prefix %lld", a->layer,
                        (long long)a->n_rows, (long long)S.prefix_rows);
        const int64_t tail = a->n_rows - S.prefix_rows;
        if (tail > 0) {
            const size_t koff = (size_t)S.prefix_rows * (size_t)a->row_bytes;
            const size_t voff = (size_t)S.prefix_rows * (size_t)vrb;
            const size_t kn = (size_t)tail * (size_t)a->row_bytes;
            const size_t vn = (size_t)tail * (size_t)vrb;
            void* dk = (uint8_t*)S.k + koff;
            void* dv = (uint8_t*)S.v + voff;
            const void* hk = (const uint8_t*)a->host_k + koff;
            const void* hv = (const uint8_t*)a->host_v + voff;
            // The tail goes on the compute stream, never on the transfer
            // streams: a copy this small runs as a copy kernel, and between the
            // DMA copies of two prefixes it cost each transfer stream two switches
            // between the copy engine and the compute queue (90-165 us idle per
            // layer at 16384 rows).  It writes rows past the prefix, so it need
            // not wait for the prefix copy; the wait for `ready` below orders
            // the attention after both.
            if (t_->copy_h2d(dk, hk, kn, compute) != 0 || t_->copy_h2d(dv, hv, vn, compute) != 0)
                return fail(KVD_EHIP, "tail copy: %s", t_->error_text());
            st_.bytes_late += (int64_t)(kn + vn);
        }
        st_.n_acquire_pipelined++;
    }
    Slot& S = slots_[s];
    for (EventH e : S.ready)
        if (t_->wait(compute, e) != 0) return fail(KVD_EHIP, "wait(ready): %s", t_->error_text());
    S.state = ACQUIRED;
    if (out) *out = kvd_slot_view{S.k, S.v, a->n_rows, a->row_bytes, 1, s, vrb};
    return KVD_OK;
}

int Ring::release(int32_t layer, StreamH compute) {
    if (!engaged_) return KVD_OK;  // ordered path: the copy lives on the compute stream
    const int s = find_layer(layer, ACQUIRED);
    if (s < 0) return fail(KVD_ESTATE, "layer %d is not acquired", layer);
    Slot& S = slots_[s];
    if (t_->record(S.rel, compute) != 0) return fail(KVD_EHIP, "record(release): %s", t_->error_text());
    S.state = RELEASED;
    S.released_once = true;
    return KVD_OK;
}

void Ring::stats(kvd_ring_stats* out) const {
    *out = st_;
    out->engaged = engaged_ ? 1 : 0;
    out->declined = declined_ ? 1 : 0;
    out->device = engaged_ ? device_ : -1;
    out->ring_bytes = engaged_ ? (int64_t)n_slots_ * (slot_bytes_ + slot_v_bytes_) : 0;
}

}  // namespace kvd

using namespace kvd;

extern "C" int kvd_ring_stage_layer(kvd_ring* ring, const kvd_stage_args* args, void* compute_stream,
                                    kvd_slot_view* out) {
    clear_error();
    if (!ring) return fail(KVD_EINVAL, "ring is NULL");
    try {
        return ring->impl.stage(args, compute_stream, out);
    } catch (const std::bad_alloc&) {
        return fail(KVD_ENOMEM, "host allocation failed");
    }
}

extern "C" int kvd_ring_release(kvd_ring* ring, int32_t layer, void* compute_stream) {
    clear_error();
    if (!ring) return fail(KVD_EINVAL, "ring is NULL");
    return ring->impl.release(layer, compute_stream);
}

extern "C" int kvd_ring_stats_get(const kvd_ring* ring, kvd_ring_stats* out, size_t out_size) {
    clear_error();
    if (!ring || !out) return fail(KVD_EINVAL, "ring and out must not be NULL");
    if (out_size < sizeof(kvd_ring_stats))
        return fail(KVD_EINVAL, "out_size %zu < sizeof(kvd_ring_stats) %zu", out_size, sizeof(kvd_ring_stats));
    ring->impl.stats(out);
    return KVD_OK;
}

extern "C" int kvd_ring_tile_rows(int32_t depth, size_t budget_bytes, int64_t row_bytes, double max_tile_bytes,
                                  int64_t* tile_rows) {
    clear_error();
    if (!tile_rows) return fail(KVD_EINVAL, "tile_rows is NULL");
    *tile_rows = 0;
    if (depth < 1) return fail(KVD_EINVAL, "depth %d < 1: tiles are staged through a ring", depth);
    if (row_bytes <= 0 || row_bytes > (1 << 24)) return fail(KVD_EINVAL, "row_bytes %lld out of range", (long long)row_bytes);
    if (!(max_tile_bytes >= 0.0)) return fail(KVD_EINVAL, "max_tile_bytes must be >= 0");
    const int64_t budget = budget_bytes > (size_t)INT64_MAX ? INT64_MAX : (int64_t)budget_bytes;
    // largest multiple of 64 rows whose ring fits the budget (inclusive)
    int64_t rows = budget / ((int64_t)(depth + 2) * 2 * row_bytes);
    if (max_tile_bytes > 0.0) {
        const double cap = max_tile_bytes / (2.0 * (double)row_bytes);
        if (cap < (double)rows) rows = (int64_t)cap;
    }
    rows = rows / 64 * 64;
    if (rows > ((int64_t)1 << 30)) rows = (int64_t)1 << 30;
    int64_t need = 0;
    while (rows > 0 && (!ring_need_bytes(depth, rows, row_bytes, row_bytes, &need) || need > budget)) rows -= 64;
    if (rows < 64) return KVD_DECLINED;
    *tile_rows = rows;
    return KVD_OK;
}

extern "C" int kvd_ring_set_transfer_delay(kvd_ring* ring, uint32_t max_us, uint64_t seed) {
    kvd::clear_error();
    if (!ring) return kvd::fail(KVD_EINVAL, "ring is NULL");
    if (max_us > 100000) return kvd::fail(KVD_EINVAL, "max_us %u above 100000", max_us);
    ring->impl.set_transfer_delay(max_us, seed);
    return KVD_OK;
}

extern "C" void kvd_ring_destroy(kvd_ring* ring) {
    clear_error();
    delete ring;
}
