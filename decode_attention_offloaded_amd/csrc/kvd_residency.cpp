// Residency planner: which layers of a stack keep their K/V on the device and
// whether the rest go through a staging ring.  Host-only arithmetic.
//
// Passages followed: "sched: pipeline the delivery of a host-resident KV
// cache (R4)", Known limitations (at a long context the ring's bytes would
// hold about three layers' K/V; making those layers device-resident removes
// more host-to-device traffic than the ring hides); "F5 — Advanced KV Cache
// Techniques", F5-opt W4 (device-resident whenever the KV fits the VRAM
// budget, spilling only under pressure).
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "kvd_internal.h"

using namespace kvd;

namespace {

// Estimated step time of one candidate (transfer-bound model): staged bytes
// cross the link at link_gbps; compute is n_layers * compute_ms.  Ordered:
// transfer and compute in series.  Ring: they overlap, except the first staged
// layer's delivery, which only the resident prefix's compute can hide.
double est_ms(int32_t n_layers, int32_t k, int64_t layer_bytes, bool ring, double link_gbps, double compute_ms) {
    const double staged = (double)(n_layers - k) * (double)layer_bytes;
    const double t_x = staged / (link_gbps * 1e6);  // ms
    const double t_c = (double)n_layers * compute_ms;
    if (!ring || k == n_layers) return t_x + t_c;
    const double first = (double)layer_bytes / (link_gbps * 1e6);
    const double exposed = std::max(0.0, first - (double)k * compute_ms);
    return std::max(t_x, t_c) + exposed;
}

}  // namespace

extern "C" int kvd_plan_residency(int32_t n_layers, int64_t layer_bytes, size_t budget_bytes, int32_t depth,
                                  double link_gbps, double compute_ms, kvd_residency_plan* out) {
    clear_error();
    if (!out) return fail(KVD_EINVAL, "out is NULL");
    *out = kvd_residency_plan{};
    if (n_layers < 1 || n_layers > (1 << 20)) return fail(KVD_EINVAL, "n_layers %d out of range", n_layers);
    if (layer_bytes < 1 || layer_bytes > ((int64_t)1 << 50))
        return fail(KVD_EINVAL, "layer_bytes %lld out of range", (long long)layer_bytes);
    if (depth < 0) return fail(KVD_EINVAL, "depth %d < 0", depth);
    if (!(link_gbps >= 0.0) || !(compute_ms >= 0.0) || isinf(link_gbps) || isinf(compute_ms))
        return fail(KVD_EINVAL, "link_gbps and compute_ms must be finite and >= 0");
    const bool model = link_gbps > 0.0;
    const int64_t budget = budget_bytes > (size_t)INT64_MAX ? INT64_MAX : (int64_t)budget_bytes;
    // a depth-N ring of whole layers: (N + 2) slots of K + V
    const int64_t ring = depth > 0 ? (int64_t)(depth + 2) * layer_bytes : 0;

    int32_t best_k = -1;
    bool best_ring = false;
    double best_t = 0.0;
    for (int pass = 0; pass < 2; ++pass) {
        const bool with_ring = pass == 0;
        if (with_ring && depth == 0) continue;
        // most resident layers that fit beside the ring (or alone)
        int64_t room = budget - (with_ring ? ring : 0);
        if (room < 0) continue;
        int32_t k = (int32_t)std::min<int64_t>(n_layers, room / layer_bytes);
        if (with_ring && k == n_layers) continue;  // all resident: the ring is never used
        const double t = model ? est_ms(n_layers, k, layer_bytes, with_ring, link_gbps, compute_ms) : 0.0;
        bool better;
        if (best_k < 0) better = true;
        else if (model) better = t < best_t;
        else better = false;  // without a model: the ring (first pass) when it fits
        if (better) {
            best_k = k;
            best_ring = with_ring;
            best_t = t;
        }
    }
    if (best_k < 0) best_k = 0;  // nothing fits: every layer staged on the ordered path
    // every layer fits: device-resident, nothing staged
    if ((int64_t)n_layers * layer_bytes <= budget) {
        best_k = n_layers;
        best_ring = false;
        best_t = model ? est_ms(n_layers, n_layers, layer_bytes, false, link_gbps, compute_ms) : 0.0;
    }
    out->n_resident = best_k;
    out->use_ring = best_ring ? 1 : 0;
    out->resident_bytes = (int64_t)best_k * layer_bytes;
    out->ring_bytes = best_ring ? ring : 0;
    out->staged_bytes_per_step = (int64_t)(n_layers - best_k) * layer_bytes;
    out->est_ms_per_step = best_t;
    return KVD_OK;
}
