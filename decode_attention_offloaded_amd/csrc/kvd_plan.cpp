// Split plan and argument validation for kvd_attend_decode (host only).
#include "kvd_plan.h"

#include <math.h>

#include <algorithm>
#include <vector>

namespace kvd {
namespace {

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workgroups of the block-sliced kernel for splits of `rows` rows: every
// visible range cut into splits, times the KV heads.
int64_t slice_workgroups(const AttendPlan& p, int n_head_kv, int64_t rows) {
    int64_t wgs = 0;
    for (const SeqPlan& sp : p.seq) wgs += ceil_div(sp.seg[0].n_vis, rows) + ceil_div(sp.seg[1].n_vis, rows);
    return wgs * n_head_kv;
}

// 16-row sub-tiles of every (visible range, KV head), per CU: the work the
// chip shares out, in the unit a wave computes at a time.
int64_t subtiles_per_cu(const AttendPlan& p, int n_head_kv, int64_t n_cus) {
    int64_t u = 0;
    for (const SeqPlan& sp : p.seq) u += ceil_div(sp.seg[0].n_vis, 16) + ceil_div(sp.seg[1].n_vis, 16);
    return u * n_head_kv / n_cus;
}

// Waves per workgroup for a given amount of work per CU.  The decode kernel
// holds three waves per SIMD (its register count); a long context runs best
// as one workgroup of 12 waves per CU (the split's online-softmax states merge
// once per CU, and the combine has the fewest partials), a medium one as one
// of 8, and a short one (under 12 sub-tiles per CU) as 4-wave workgroups,
// whose waves each get more sub-tiles to overlap their loads with.  Measured
// on MI355X over 2048 ... 131072 rows x 8 KV heads.
int plan_waves(int64_t subtiles) {
    return subtiles >= kWaves12Subtiles ? 12 : subtiles >= kWaves8Subtiles ? 8 : 4;
}

// Share of the chip's time that splits of `rows` rows in 8- or 12-wave
// workgroups (one per CU at a time) fill with rows: visible rows x KV heads
// over CUs x split rows x rounds of workgroups.  Equal sequences fill nearly
// all of it; sequences of unequal length leave the CUs of their short last
// splits idle.
double big_plan_fill(const AttendPlan& p, int n_head_kv, int64_t rows, int64_t n_cus) {
    int64_t vis = 0;
    for (const SeqPlan& sp : p.seq) vis += (int64_t)sp.seg[0].n_vis + sp.seg[1].n_vis;
    const int64_t rounds = ceil_div(slice_workgroups(p, n_head_kv, rows), n_cus);
    return (double)(vis * n_head_kv) / ((double)n_cus * (double)rows * (double)rounds);
}

// Relative time per unit of work of a 4-wave workgroup when the busiest CU
// runs `per_cu` of them: one per CU (one wave per SIMD) hides little latency;
// up to kWavesPerSimd are resident at once, beyond that they queue in rounds.
int64_t occupancy_cost(int64_t per_cu) {
    const int64_t resident = kWavesPerSimd;
    const int64_t eff = per_cu <= resident ? per_cu : resident * ceil_div(per_cu, resident);
    const int64_t occ = per_cu == 1 ? 160 : per_cu == 2 ? 100 : 93;
    return occ * eff;
}

// Tiles (64 rows) per split.  A candidate of k tiles gives a number of
// workgroups; the busiest CU then runs ceil(workgroups / CUs) of them, each
// costing k tiles plus a fixed amount of work (start-up, merge, partial
// write).  4-wave workgroups weigh that by occupancy_cost; the 8- and 12-wave
// ones run one at a time per CU, so the cost is the number of rounds times
// (k + kBigOverheadTiles).  Candidates: every k up to 16, then steps of about
// 25%, and for r = 1 .. 4 the smallest k that gives at most r workgroups per
// CU.  The cheapest wins, the larger on a tie.
int64_t tiles_per_split(const AttendPlan& p, int n_head_kv, int64_t max_vis, int64_t n_cus, int waves) {
    const int64_t max_k = std::max<int64_t>(1, ceil_div(max_vis, kTileRows));
    auto per_cu = [&](int64_t k) { return ceil_div(slice_workgroups(p, n_head_kv, k * kTileRows), n_cus); };
    std::vector<int64_t> cand;
    for (int64_t k = 1; k <= max_k; k = k < 16 ? k + 1 : k + k / 4) cand.push_back(k);
    cand.push_back(max_k);
    for (int64_t r = 1; r <= 4; ++r) {
        // workgroups fall as k grows: bisect for the first k with per_cu(k) <= r
        int64_t lo = 1, hi = max_k;
        if (per_cu(hi) > r) continue;
        while (lo < hi) {
            const int64_t mid = lo + (hi - lo) / 2;
            if (per_cu(mid) <= r)
                hi = mid;
            else
                lo = mid + 1;
        }
        cand.push_back(lo);
    }
    std::sort(cand.begin(), cand.end());
    int64_t best_k = 1, best_cost = INT64_MAX;
    for (const int64_t k : cand) {
        const int64_t pc = per_cu(k);
        const int64_t cost =
            waves == 4 ? occupancy_cost(pc) * (k + kSliceOverheadTiles) : pc * (k + kBigOverheadTiles);
        if (cost <= best_cost) {
            best_cost = cost;
            best_k = k;
        }
    }
    return best_k;
}

}  // namespace

int plan_attend(const kvd_attn_args* a, AttendPlan* p, int n_cus) {
    if (!a || !p) return fail(KVD_EINVAL, "null argument");
    if (n_cus < 1 || n_cus > 4096) return fail(KVD_EINVAL, "compute unit count %d out of range", n_cus);
    if (a->n_seq < 1 || a->n_seq > (1 << 20)) return fail(KVD_EINVAL, "n_seq %d out of range", a->n_seq);
    if (a->n_head_kv < 1 || a->n_head_q < 1 || a->n_head_q % a->n_head_kv != 0)
        return fail(KVD_EINVAL, "n_head_q %d must be a positive multiple of n_head_kv %d", a->n_head_q,
                    a->n_head_kv);
    const int G = a->n_head_q / a->n_head_kv;
    if (G > 8) return fail(KVD_EINVAL, "GQA group %d > 8 is not supported", G);
    if (a->n_head_kv > 4096) return fail(KVD_EINVAL, "n_head_kv %d out of range", a->n_head_kv);
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(KVD_EINVAL, "head_dim %d not supported (64 or 128)", a->head_dim);
    if (a->n_seg != 1 && a->n_seg != 2) return fail(KVD_EINVAL, "n_seg %d must be 1 or 2", a->n_seg);
    if (a->window < 0) return fail(KVD_EINVAL, "window %d < 0", a->window);
    if (a->split_rows < 0 || a->split_rows % kTileRows != 0 || a->split_rows > (1 << 24))
        return fail(KVD_EINVAL, "split_rows %d must be 0 or a positive multiple of 64", a->split_rows);
    if (!isfinite(a->scale)) return fail(KVD_EINVAL, "scale is not finite");
    if (!a->q || !a->segs) return fail(KVD_EINVAL, "q and segs must not be NULL");
    if ((uintptr_t)a->q % 16) return fail(KVD_EINVAL, "q must be 16-byte aligned");

    if (a->reserved != 0) return fail(KVD_EINVAL, "reserved field must be 0");
    if (a->v_type != KVD_TYPE_Q8_0 && a->v_type != KVD_TYPE_Q4_0)
        return fail(KVD_EINVAL, "v_type %d must be KVD_TYPE_Q8_0 or KVD_TYPE_Q4_0", a->v_type);
    const int D = a->head_dim;
    const int chunk = D / 32 * 34;
    const int64_t row_bytes = (int64_t)a->n_head_kv * chunk;
    const int64_t v_row_bytes = (int64_t)a->n_head_kv * (D / 32) * (a->v_type == KVD_TYPE_Q4_0 ? 18 : 34);
    const int64_t align = (D == 128) ? 8 : 4;
    const int64_t v_align = a->v_type == KVD_TYPE_Q4_0 ? 4 : align;

    p->group = G;
    p->chunk_bytes = chunk;
    p->seq.assign(a->n_seq, SeqPlan{});

    for (int s = 0; s < a->n_seq; ++s) {
        const kvd_kv_seg* segs = a->segs + (size_t)s * a->n_seg;
        for (int j = 0; j < a->n_seg; ++j) {
            const kvd_kv_seg& g = segs[j];
            if (g.n_rows < 0 || g.n_rows >= ((int64_t)1 << 31))
                return fail(KVD_EINVAL, "seq %d seg %d: n_rows %lld out of range", s, j, (long long)g.n_rows);
            if (g.pos0 < -((int64_t)1 << 62) || g.pos0 > ((int64_t)1 << 62))
                return fail(KVD_EINVAL, "seq %d seg %d: pos0 out of range", s, j);
            if (g.n_rows == 0) continue;
            if (!g.k || !g.v) return fail(KVD_EINVAL, "seq %d seg %d: NULL k or v", s, j);
            if (g.row_stride < row_bytes || g.row_stride >= ((int64_t)1 << 25))
                return fail(KVD_EINVAL, "seq %d seg %d: row_stride %lld (row bytes %lld, limit 2^25)", s, j,
                            (long long)g.row_stride, (long long)row_bytes);
            if ((uintptr_t)g.k % align || g.row_stride % align)
                return fail(KVD_EINVAL, "seq %d seg %d: k and row_stride must be %lld-byte aligned", s, j,
                            (long long)align);
            const int64_t vs = g.v_row_stride ? g.v_row_stride : g.row_stride;
            if (a->v_type == KVD_TYPE_Q8_0 && vs != g.row_stride)
                return fail(KVD_EINVAL, "seq %d seg %d: q8_0 V rows must share the K row stride (%lld != %lld)", s, j,
                            (long long)vs, (long long)g.row_stride);
            if (g.v_row_stride < 0 || vs < v_row_bytes || vs >= ((int64_t)1 << 25))
                return fail(KVD_EINVAL, "seq %d seg %d: V row stride %lld (V row bytes %lld, limit 2^25)", s, j,
                            (long long)vs, (long long)v_row_bytes);
            if ((uintptr_t)g.v % v_align || vs % v_align)
                return fail(KVD_EINVAL, "seq %d seg %d: v and its row stride must be %lld-byte aligned", s, j,
                            (long long)v_align);
        }
        const kvd_kv_seg& last = segs[a->n_seg - 1];
        int64_t qp;
        if (a->q_pos) {
            qp = a->q_pos[s];
            if (qp < -((int64_t)1 << 62) || qp > ((int64_t)1 << 62))
                return fail(KVD_EINVAL, "seq %d: q_pos out of range", s);
        } else {
            if (last.n_rows < 1) return fail(KVD_EINVAL, "seq %d: last segment is empty and q_pos is NULL", s);
            qp = last.pos0 + last.n_rows - 1;
        }
        SeqPlan& sp = p->seq[s];
        sp.q_pos = qp;
        int64_t vis = 0;
        for (int j = 0; j < 2; ++j) {
            SegPlan& pl = sp.seg[j];
            pl = SegPlan{0, 0, 0, 0};
            if (j >= a->n_seg) continue;
            const kvd_kv_seg& g = segs[j];
            pl.n_rows = (int32_t)g.n_rows;
            // visible: pos <= q_pos and (window == 0 or q_pos - pos < window)
            int64_t lo = 0;
            if (a->window > 0) lo = std::max<int64_t>(0, qp - a->window + 1 - g.pos0);
            int64_t hi = std::min<int64_t>(g.n_rows, qp - g.pos0 + 1);
            lo = std::min<int64_t>(lo, g.n_rows);
            if (hi > lo) {
                pl.row_lo = (int32_t)lo;
                pl.n_vis = (int32_t)(hi - lo);
            }
            vis += pl.n_vis;
        }
        if (vis < 1) return fail(KVD_EINVAL, "seq %d: no row is visible to the query at position %lld", s,
                                 (long long)qp);
    }

    // rows per split: enough splits to fill the chip, at most kMaxSplits per sequence
    int64_t max_vis = 0;
    for (const SeqPlan& sp : p->seq) max_vis = std::max<int64_t>(max_vis, (int64_t)sp.seg[0].n_vis + sp.seg[1].n_vis);
    p->n_cus = n_cus;
    // A call runs as consecutive launches of up to kMaxSeqPerLaunch sequences,
    // and each launch should fill the chip: the work per CU, the wave count
    // and the split size are weighed against the CUs of all the launches
    // (64 sequences of 4096 rows x 8 KV heads: one 4096-row split per
    // sequence gave each launch 128 workgroups, half the chip, 204 us per
    // call; 2048-row splits fill it, 155 us).
    const int64_t plan_cus = (int64_t)n_cus * ceil_div(a->n_seq, kMaxSeqPerLaunch);
    p->waves = plan_waves(subtiles_per_cu(*p, a->n_head_kv, plan_cus));
    int64_t split_rows = a->split_rows;
    if (split_rows == 0) {
        int64_t k = tiles_per_split(*p, a->n_head_kv, max_vis, plan_cus, p->waves);
        // Sequences of unequal length: where 8- or 12-wave workgroups would
        // leave more than kBigPlanMinFill of the chip's time idle, 4-wave
        // workgroups in their own (smaller) splits, up to three per CU, share
        // the CUs out more evenly.  Measured on MI355X, 16 sequences of
        // lognormal lengths (1024 ... 10041 rows) in two segments: 54.2 ->
        // 49.8 us per call, with a 4096-row window 41.6 -> 34.2 us; 16 of
        // 256 ... 8192 rows: 31.5 -> 27.8 us.  Single sequences and equal
        // ones fill the chip and keep their plan (4-wave workgroups there
        // lose 2-25%).
        if (p->waves != 4 && a->n_seq > 1 &&
            big_plan_fill(*p, a->n_head_kv, k * kTileRows, plan_cus) < kBigPlanMinFill) {
            p->waves = 4;
            k = tiles_per_split(*p, a->n_head_kv, max_vis, plan_cus, p->waves);
        }
        split_rows = (int64_t)kTileRows * k;
        // segments split separately: allow one extra split per segment
        const int64_t floor_rows = ceil_div(ceil_div(max_vis, kMaxSplits - 2), kTileRows) * kTileRows;
        split_rows = std::max(split_rows, floor_rows);
        // Short contexts: one split per (sequence, segment), no combine launch.
        // With at most one workgroup per CU, a wave takes the split's
        // sub-tiles one after another, each waiting on its own loads; one
        // split beats a split plus the combine launch up to 12 sub-tiles
        // (192 rows at head_dim 128, 384 at 64), and beyond 128 rows an
        // 8-wave workgroup keeps each wave at two sub-tiles or fewer.
        // Measured on MI355X against 64-row splits.
        const int64_t one_rows = ceil_div(max_vis, kTileRows) * kTileRows;
        const bool few = slice_workgroups(*p, a->n_head_kv, one_rows) <= n_cus;
        const int64_t sub_rows = D == 128 ? 16 : 32;  // rows per sub-tile of the decode kernel
        if (few ? ceil_div(max_vis, sub_rows) <= kOneSplitSubtiles : max_vis <= kOneSplitRows) {
            split_rows = std::max<int64_t>(split_rows, one_rows);
            int64_t max_seg = 0;
            for (const SeqPlan& sp : p->seq) max_seg = std::max<int64_t>({max_seg, sp.seg[0].n_vis, sp.seg[1].n_vis});
            p->waves = few && max_seg > kOneSplitW8Rows ? 8 : plan_waves(subtiles_per_cu(*p, a->n_head_kv, n_cus));
        }
        if (split_rows > (1 << 24)) split_rows = 1 << 24;
    }
    p->split_rows = (int32_t)split_rows;

    int64_t base = 0;
    int32_t max_splits = 0;
    for (int s = 0; s < a->n_seq; ++s) {
        SeqPlan& sp = p->seq[s];
        sp.split_base = base;
        int32_t n = 0;
        for (int j = 0; j < 2; ++j) {
            sp.seg[j].n_split = (int32_t)ceil_div(sp.seg[j].n_vis, split_rows);
            n += sp.seg[j].n_split;
        }
        sp.n_split = n;
        max_splits = std::max(max_splits, n);
        base += n;
    }
    p->total_splits = base;
    p->max_splits = max_splits;
    if (max_splits > kMaxSplits)
        return fail(KVD_EINVAL, "split_rows %lld gives %d splits for one sequence (limit %d)", (long long)split_rows,
                    max_splits, kMaxSplits);
    if (base * a->n_head_kv >= ((int64_t)1 << 31) - 8) return fail(KVD_EINVAL, "too many work items");

    if (max_splits <= 1) {
        p->off_pm = p->off_pl = p->off_po = 0;
        p->ws_bytes = 0;
    } else {
        size_t off = 0;
        p->off_pm = off;
        off += round256((size_t)base * a->n_head_q * 4);
        p->off_pl = off;
        off += round256((size_t)base * a->n_head_q * 4);
        p->off_po = off;
        off += round256((size_t)base * a->n_head_q * D * 4);
        p->ws_bytes = off;
    }
    return KVD_OK;
}

}  // namespace kvd
