// Randomised argument checks of the library's host code (tests only), built
// as an executable with AddressSanitizer and UBSan by tests/ringsim_build.py:
// the split planner (kvd_plan.cpp), the tile sizer and ring core
// (kvd_ring_core.cpp, driven on the simulated runtime of ringsim.cpp) and the
// residency planner (kvd_residency.cpp).  Valid and invalid arguments alike
// must give one of the documented return codes, and every accepted plan must
// satisfy its invariants; a sanitizer report or a failed check exits non-zero.
//
//   ringsim_fuzz SEED ITERATIONS
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "kvd.h"
#include "kvd_plan.h"

extern "C" {
void* sim_new(uint64_t seed);
void sim_delete(void* sim);
void sim_configure(void* sim, int pinned, int device, int64_t fail_after);
void* sim_stream_new(void* sim);
kvd_ring* sim_ring_create(void* sim, int32_t depth, int64_t budget);
int sim_run(void* sim, int max_steps);
int sim_drain(void* sim);
int64_t sim_counter(void* sim, int which);
}

static int g_fail = 0;
static long g_plan_ok = 0, g_plan_brute = 0, g_tile_ok = 0, g_res_ok = 0, g_stage_ok = 0, g_stage_rej = 0;
#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            fprintf(stderr, "check failed: %s: ", #cond);  \
            fprintf(stderr, __VA_ARGS__);                  \
            fprintf(stderr, "\n");                         \
            if (++g_fail > 20) exit(1);                    \
        }                                                  \
    } while (0)

typedef std::mt19937_64 Rng;
static int64_t pick(Rng& r, std::initializer_list<int64_t> v) { return *(v.begin() + r() % v.size()); }
static int64_t range(Rng& r, int64_t lo, int64_t hi) { return lo + (int64_t)(r() % (uint64_t)(hi - lo + 1)); }

// ---------------------------------------------------------------- split plan
static void fuzz_plan(Rng& r) {
    // a valid call first; then, one time in four, one field made invalid
    kvd_attn_args a;
    memset(&a, 0, sizeof a);
    a.n_seq = (int32_t)range(r, 1, 20);
    a.n_head_kv = (int32_t)pick(r, {1, 2, 4, 8});
    a.n_head_q = a.n_head_kv * (int32_t)range(r, 1, 8);
    a.head_dim = (int32_t)pick(r, {64, 128});
    a.n_seg = (int32_t)pick(r, {1, 2});
    a.window = (int32_t)pick(r, {0, 0, 1, 64, 4096, range(r, 1, 5000)});
    a.split_rows = (int32_t)pick(r, {0, 0, 0, 64, 128, 64 * range(r, 1, 100)});
    a.scale = 0.088f;
    static float qbuf[8];
    a.q = (const float*)(((uintptr_t)qbuf + 15) & ~(uintptr_t)15);
    a.out = (float*)0x200000;
    a.v_type = (int32_t)pick(r, {0, 0, 1});
    const int64_t rb = (int64_t)a.n_head_kv * a.head_dim / 32 * 34;
    const int64_t vrb = (int64_t)a.n_head_kv * a.head_dim / 32 * (a.v_type ? 18 : 34);
    const int n_seq = a.n_seq;
    std::vector<kvd_kv_seg> segs((size_t)n_seq * 2);
    std::vector<int64_t> qpos((size_t)n_seq);
    for (int s = 0; s < n_seq; ++s) {
        int64_t pos = pick(r, {0, 0, range(r, 0, 100000), (int64_t)1 << 40});
        const int64_t first = pos;
        for (int j = 0; j < 2; ++j) {
            kvd_kv_seg& g = segs[(size_t)s * 2 + j];
            const bool last = j == a.n_seg - 1;
            g.n_rows = pick(r, {range(r, last ? 1 : 0, 3000), range(r, last ? 1 : 0, 300), 1, 64, 65, range(r, 1, 40000)});
            g.pos0 = pos;
            pos += g.n_rows;
            g.k = (const void*)(uintptr_t)0x10000000;
            g.v = (const void*)(uintptr_t)0x20000000;
            g.row_stride = rb + 8 * pick(r, {0, 0, 0, 1, 3});
            // q4_0 V: its own stride; q8_0 V: 0 or the K stride (anything else is refused)
            g.v_row_stride = a.v_type ? vrb + 4 * pick(r, {0, 0, 1}) : (r() % 3 == 0 ? g.row_stride : 0);
        }
        const int64_t end = segs[(size_t)s * 2 + a.n_seg - 1].pos0 + segs[(size_t)s * 2 + a.n_seg - 1].n_rows;
        qpos[s] = pick(r, {end - 1, end - 1, range(r, first, end - 1)});
    }
    if (r() % 4 == 0) {
        // one invalid field
        switch (r() % 16) {
            case 0: a.n_seq = (int32_t)pick(r, {0, -1}); break;
            case 1: a.n_head_kv = (int32_t)pick(r, {0, -3, 5000}); break;
            case 2: a.n_head_q = a.n_head_kv * 9; break;
            case 3: a.head_dim = (int32_t)pick(r, {32, 96, 256, 0}); break;
            case 4: a.n_seg = (int32_t)pick(r, {0, 3}); break;
            case 5: a.window = -1; break;
            case 6: a.split_rows = (int32_t)pick(r, {100, -64, 1 << 25}); break;
            case 7: a.scale = NAN; break;
            case 8: a.q = (r() % 2) ? nullptr : (const float*)((uintptr_t)a.q + 4); break;
            case 9: a.v_type = (int32_t)pick(r, {-1, 2}); break;
            case 10: a.reserved = 1; break;
            case 11: segs[0].n_rows = pick(r, {-1, (int64_t)1 << 31}); break;
            case 12: segs[0].row_stride = pick(r, {rb - 8, rb + 4, (int64_t)1 << 25}); break;
            case 13: segs[0].k = (r() % 2) ? nullptr : (const void*)(uintptr_t)0x10000004; break;
            case 14: segs[0].v_row_stride = a.v_type ? pick(r, {-4, vrb - 4, vrb + 2}) : segs[0].row_stride + 8; break;
            case 15: qpos[0] = pick(r, {segs[0].pos0 - 1, -((int64_t)1 << 62) - 5}); break;
        }
    }
    // the ABI takes [n_seq][n_seg]: pack
    std::vector<kvd_kv_seg> packed;
    const int n_seg = a.n_seg >= 1 && a.n_seg <= 2 ? a.n_seg : 1;
    for (int s = 0; s < n_seq; ++s)
        for (int j = 0; j < n_seg; ++j) packed.push_back(segs[(size_t)s * 2 + j]);
    a.segs = (r() % 100 == 0) ? nullptr : packed.data();
    a.q_pos = (r() % 2) ? qpos.data() : nullptr;

    kvd::AttendPlan p;
    const int n_cus = (int)pick(r, {256, 256, 80, 304, 1, 32});
    const int rc = kvd::plan_attend(&a, &p, n_cus);
    CHECK(rc == KVD_OK || rc == KVD_EINVAL, "plan rc %d", rc);
    if (rc != KVD_OK) return;
    ++g_plan_ok;
    CHECK(p.n_cus == n_cus, "n_cus %d", p.n_cus);
    CHECK(p.split_rows >= 64 && p.split_rows % 64 == 0, "split_rows %d", p.split_rows);
    if (a.split_rows > 0) CHECK(p.split_rows == a.split_rows, "split_rows %d != asked %d", p.split_rows, a.split_rows);
    int64_t base = 0, max_split = 0;
    for (int s = 0; s < a.n_seq; ++s) {
        const kvd::SeqPlan& sp = p.seq[(size_t)s];
        const kvd_kv_seg* sg = a.segs + (size_t)s * a.n_seg;
        const int64_t qp = a.q_pos ? a.q_pos[s] : sg[a.n_seg - 1].pos0 + sg[a.n_seg - 1].n_rows - 1;
        CHECK(sp.split_base == base, "split_base");
        int64_t vis = 0, n = 0;
        for (int j = 0; j < 2; ++j) {
            const kvd::SegPlan& pl = sp.seg[j];
            if (j >= a.n_seg) {
                CHECK(pl.n_vis == 0 && pl.n_split == 0, "unused segment has work");
                continue;
            }
            CHECK(pl.row_lo >= 0 && pl.n_vis >= 0 && (int64_t)pl.row_lo + pl.n_vis <= sg[j].n_rows, "visible range");
            CHECK(pl.n_split == (pl.n_vis + p.split_rows - 1) / p.split_rows, "segment splits");
            if (sg[j].n_rows <= 4000) {
                ++g_plan_brute;
                // brute force: rows visible to the query at qp (contiguous)
                int64_t lo = -1, cnt = 0;
                for (int64_t t = 0; t < sg[j].n_rows; ++t) {
                    const int64_t pos = sg[j].pos0 + t;
                    const bool v = pos <= qp && (a.window == 0 || qp - pos < a.window);
                    if (v) {
                        if (lo < 0) lo = t;
                        ++cnt;
                    }
                }
                CHECK(cnt == pl.n_vis, "n_vis %d, brute force %lld", pl.n_vis, (long long)cnt);
                if (cnt) CHECK(lo == pl.row_lo, "row_lo %d, brute force %lld", pl.row_lo, (long long)lo);
            }
            vis += pl.n_vis;
            n += pl.n_split;
        }
        CHECK(vis >= 1, "accepted a sequence with no visible row");
        CHECK(n == sp.n_split && n >= 1 && n <= 256, "sequence splits %lld", (long long)n);
        base += n;
        if (n > max_split) max_split = n;
    }
    CHECK(base == p.total_splits && max_split == p.max_splits, "totals");
    if (p.max_splits <= 1) {
        CHECK(p.ws_bytes == 0, "single splits need no workspace");
    } else {
        CHECK(p.off_pm == 0 && p.off_pl % 256 == 0 && p.off_po % 256 == 0, "offsets");
        CHECK(p.off_pl >= (size_t)p.total_splits * a.n_head_q * 4, "pm area");
        CHECK(p.off_po >= p.off_pl + (size_t)p.total_splits * a.n_head_q * 4, "pl area");
        CHECK(p.ws_bytes >= p.off_po + (size_t)p.total_splits * a.n_head_q * a.head_dim * 4, "po area");
    }
}

// ---------------------------------------------------------------- tile rows
static void fuzz_tile_rows(Rng& r) {
    const int32_t depth = (int32_t)pick(r, {1, 1, 2, 4, 0, -1, 70});
    const size_t budget = (size_t)pick(r, {128 << 20, 1 << 30, range(r, 0, 1 << 20), 0, (int64_t)1 << 40});
    const int64_t rb = pick(r, {1088, 2176, 544, range(r, 1, 1 << 20), 0, -4, ((int64_t)1 << 24) + 1});
    double cap = (double)pick(r, {0, 0, range(r, 1, 1 << 30), -1});
    if (r() % 30 == 0) cap = NAN;
    int64_t rows = -7;
    const int rc = kvd_ring_tile_rows(depth, budget, rb, cap, &rows);
    CHECK(rc == KVD_OK || rc == KVD_DECLINED || rc == KVD_EINVAL, "tile rc %d", rc);
    if (rc == KVD_OK) {
        ++g_tile_ok;
        CHECK(rows >= 64 && rows % 64 == 0, "tile rows %lld", (long long)rows);
        const __int128 need = (__int128)(depth + 2) * 2 * rows * rb;
        CHECK(need <= (__int128)budget, "tile ring over budget");
        if (cap > 0) CHECK(2.0 * (double)rows * (double)rb <= cap, "tile over its byte bound");
        const __int128 next = (__int128)(depth + 2) * 2 * (rows + 64) * rb;
        CHECK(next > (__int128)budget || (cap > 0 && 2.0 * (double)(rows + 64) * (double)rb > cap), "tile not largest");
    } else if (rc == KVD_DECLINED) {
        CHECK(rows == 0, "declined tile rows %lld", (long long)rows);
    }
}

// ---------------------------------------------------------------- residency
static void fuzz_residency(Rng& r) {
    const int32_t L = (int32_t)pick(r, {64, 1, range(r, 1, 200), 0, -1, (1 << 20) + 1});
    const int64_t lb = pick(r, {285212672, range(r, 1, 1 << 30), 0, -1, ((int64_t)1 << 50) + 1});
    const size_t budget = (size_t)pick(r, {1 << 30, (int64_t)4 << 30, range(r, 0, (int64_t)1 << 34), 0});
    const int32_t depth = (int32_t)pick(r, {0, 1, 2, -1});
    double link = (double)pick(r, {0, 57, 25}), ms = (double)pick(r, {0, 1, 0}) * 0.17;
    if (r() % 30 == 0) link = -1;
    if (r() % 30 == 0) ms = INFINITY;
    kvd_residency_plan p;
    const int rc = kvd_plan_residency(L, lb, budget, depth, link, ms, &p);
    CHECK(rc == KVD_OK || rc == KVD_EINVAL, "residency rc %d", rc);
    if (rc != KVD_OK) return;
    ++g_res_ok;
    CHECK(p.n_resident >= 0 && p.n_resident <= L, "n_resident %d", p.n_resident);
    CHECK(!p.use_ring || depth >= 1, "ring without depth");
    CHECK(p.resident_bytes == (int64_t)p.n_resident * lb, "resident bytes");
    CHECK(p.ring_bytes == (p.use_ring ? (int64_t)(depth + 2) * lb : 0), "ring bytes");
    CHECK((uint64_t)p.resident_bytes + (uint64_t)p.ring_bytes <= budget, "over budget");
    CHECK(p.staged_bytes_per_step == (int64_t)(L - p.n_resident) * lb, "staged bytes");
}

// ---------------------------------------------------------------- ring calls
static void fuzz_ring(Rng& r) {
    void* sim = sim_new(r());
    sim_configure(sim, r() % 20 ? 1 : 0, 0, r() % 10 == 0 ? (int64_t)range(r, 0, 6) : -1);
    void* compute = sim_stream_new(sim);
    const int32_t depth = (int32_t)pick(r, {0, 1, 1, 2, 3, 4});
    const int64_t rb = pick(r, {1088, 64, 128});
    const int64_t vrb = pick(r, {0, 0, rb / 2, 4});
    const int64_t cap = range(r, 1, 256);
    const int64_t budget = pick(r, {(int64_t)1 << 30, (depth + 2) * cap * (rb + (vrb ? vrb : rb)), range(r, 0, 1 << 20)});
    kvd_ring* ring = sim_ring_create(sim, depth, budget);
    const int L = 6;
    std::vector<std::vector<uint8_t>> hk(L), hv(L);
    // host and ordered buffers hold 2 * cap rows: the largest capacity a call below declares
    for (int l = 0; l < L; ++l) {
        hk[l].assign((size_t)(2 * cap * rb), (uint8_t)l);
        hv[l].assign((size_t)(2 * cap * (vrb ? vrb : rb)), (uint8_t)(100 + l));
    }
    std::vector<uint8_t> ok((size_t)(2 * cap * rb)), ov((size_t)(2 * cap * (vrb ? vrb : rb)));
    std::vector<int> acquired(L, 0);
    const int ops = (int)range(r, 1, 60);
    for (int i = 0; i < ops; ++i) {
        const int l = (int)range(r, 0, L - 1);
        const int what = (int)(r() % 4);
        if (what == 3) {
            const int rc = kvd_ring_release(ring, l, compute);
            CHECK(rc == KVD_OK || rc == KVD_ESTATE, "release rc %d", rc);
            if (rc == KVD_OK) acquired[l] = 0;
        } else {
            kvd_stage_args st;
            memset(&st, 0, sizeof st);
            st.layer = (r() % 40 == 0) ? -1 : l;
            st.flags = what == 0 ? KVD_STAGE_PREFETCH : (what == 1 ? KVD_STAGE_ACQUIRE : (int)pick(r, {1, 2, 0, 7}));
            st.host_k = (r() % 40 == 0) ? nullptr : hk[l].data();
            st.host_v = hv[l].data();
            st.row_bytes = (r() % 40 == 0) ? rb + 2 : rb;
            st.v_row_bytes = vrb;
            st.cap_rows = (r() % 40 == 0) ? cap * 2 : cap;
            st.n_rows = pick(r, {cap, range(r, 1, cap), 0, cap + 1});
            st.stable_rows = pick(r, {st.n_rows - 1, st.n_rows, range(r, 0, cap), -1});
            st.ordered_k = (r() % 30 == 0) ? nullptr : ok.data();
            st.ordered_v = ov.data();
            kvd_slot_view view;
            const int rc = kvd_ring_stage_layer(ring, &st, compute, (r() % 5 == 0) ? nullptr : &view);
            CHECK(rc == KVD_OK || rc == KVD_DECLINED || rc == KVD_EINVAL || rc == KVD_ESTATE || rc == KVD_EHIP,
                  "stage rc %d", rc);
            if (st.flags == KVD_STAGE_ACQUIRE && rc >= 0) acquired[l] = 1;
            ++(rc >= 0 ? g_stage_ok : g_stage_rej);
        }
        if (r() % 3 == 0) sim_run(sim, (int)range(r, 0, 40));
    }
    for (int l = 0; l < L; ++l)
        if (acquired[l]) kvd_ring_release(ring, l, compute);
    kvd_ring_stats stats;
    CHECK(kvd_ring_stats_get(ring, &stats, sizeof stats) == KVD_OK, "stats");
    CHECK(stats.ring_bytes <= stats.budget_bytes, "ring over budget");
    sim_drain(sim);
    kvd_ring_destroy(ring);
    CHECK(sim_counter(sim, 4) == 0, "deadlock in the simulated runtime");
    CHECK(sim_counter(sim, 3) == 0, "device memory still allocated after destroy: %lld", (long long)sim_counter(sim, 3));
    sim_delete(sim);
}

int main(int argc, char** argv) {
    const uint64_t seed = argc > 1 ? strtoull(argv[1], nullptr, 10) : 1;
    const int iters = argc > 2 ? atoi(argv[2]) : 2000;
    Rng r(seed);
    for (int i = 0; i < iters; ++i) {
        fuzz_plan(r);
        fuzz_tile_rows(r);
        fuzz_residency(r);
        if (i % 4 == 0) fuzz_ring(r);
    }
    printf("%d iterations: %ld plans accepted (%ld segments brute-forced), %ld tile sizes, %ld residency plans, "
           "%ld stage calls accepted and %ld refused; %d failed checks\n",
           iters, g_plan_ok, g_plan_brute, g_tile_ok, g_res_ok, g_stage_ok, g_stage_rej, g_fail);
    return g_fail ? 1 : 0;
}
