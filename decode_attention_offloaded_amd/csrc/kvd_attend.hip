// Split-K flash-decode attention over a q8_0 grouped-query KV cache (gfx950).
//
// What is computed (see include/kvd.h): for every sequence and query head h,
// softmax over the visible rows of scale * q.k, times V, with query head h
// reading KV head floor(h / G) ("F5 -- Advanced KV Cache Techniques", M3 What
// shipped: query heads grouped by the GQA ratio), over q8_0 rows laid out
// token-major with every KV head in a row (same page, M2 What shipped:
// [head_dim, n_head_kv, n_kv]).  The split results are merged with the
// online-softmax rule (same page, M4 step 6 and W4: partial attention results
// merged by their running maxima and sums).
//
// Shape of the work.  A split = one (sequence, KV head, row range) = one
// workgroup of D / 32 waves, wave w owning q8_0 block w (dims 32w .. 32w + 31)
// of every row.  All waves walk the same 64-row tiles: each loads a 36-byte
// window around its block (K and V, one tile ahead in registers), scores its
// block's 32 dims for all G query heads (one lane per row; the query chunks
// from LDS or, once several workgroups share a CU, from SGPRs), the D / 32
// block partials meet in LDS at one barrier per tile, every wave runs the same
// online softmax, and wave w accumulates the values of its 32 dims.  The
// arguments a split needs before its first loads are kernel arguments that the
// hardware preloads into SGPRs; the rest are read while the first tile is in
// flight.
// A split with siblings writes an unnormalised partial (m, l, o) to the
// workspace and a second, small launch merges the partials of each
// (sequence, query head) in split order, so the result depends only on the
// split plan.  (Merging inside the first launch would need device-scope
// release/acquire between workgroups, which on this chip writes back and
// invalidates the whole L2 of an XCD per workgroup.)
// No MFMA: one query row per head is not a dense contraction.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "kvd_internal.h"
#include "kvd_plan.h"

namespace kvd {
namespace {

// Constant address space: loads through it are scalar (s_load) when uniform.
typedef const float __attribute__((address_space(4)))* const_f32_ptr;

constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)

struct SegDesc {
    const uint8_t* k;
    const uint8_t* v;
    int32_t stride;   // row stride in bytes
    int32_t row_lo;   // first visible row
    int32_t n_vis;    // visible rows
    int32_t n_split;  // splits over this segment
    int32_t n_rows;   // readable rows
    int32_t vstride;  // V row stride in bytes (q4_0 V rows are shorter)
};

struct SeqDesc {
    SegDesc seg[2];
    int32_t split_base;  // first split of this sequence, relative to the launch
    int32_t n_split;     // splits of this sequence
};

struct LaunchArgs {
    SeqDesc seq[kMaxSeqPerLaunch];
    const float* q;       // this launch's first sequence
    float* out;           // this launch's first sequence
    float* pm;            // partial maxima [split][n_head_q] (absolute split index)
    float* pl;            // partial sums
    float* po;            // partial outputs [split][n_head_q][D]
    int32_t n_seq;
    int32_t n_head_kv;
    int32_t split_rows;
    int32_t n_items;
    int32_t split_off;    // absolute index of this launch's first split
    float scale_log2e;
    // Unnormalised result instead of `out` (tile-streamed attention): o
    // [seq][n_head_q][D], m and l [seq][n_head_q]; null for a normal call.
    float* part_o;
    float* part_m;
    float* part_l;
};

// Final result of one (sequence, query head) at dimension i: out = O / L, or
// the unnormalised (O, M, L) when the call asked for a partial result.
__device__ inline void write_final(const LaunchArgs& A, int D, size_t sh, int i, float O, float M, float L,
                                   bool lead) {
    if (A.part_o) {
        A.part_o[sh * D + i] = O;
        if (lead) {
            A.part_m[sh] = M;
            A.part_l[sh] = L;
        }
    } else {
        A.out[sh * D + i] = O / L;
    }
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const uint8_t* base, int32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kRsrcWord3);
}

// DPP lane moves (gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

// Lanes of rows outside ROW_MASK read 0.  With a zero `old` and bound_ctrl
// set, the compiler folds the move into the consuming add or max
// (v_add_f32_dpp), one instruction per step instead of three.
template <int CTRL, int ROW_MASK = 0xf>
__device__ inline float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, true));
}

// Reductions over the 64 lanes of a wave; the result is wave-uniform (read
// from lane 63 after the row broadcasts).
__device__ inline float wave_max(float x) {
    x = fmaxf(x, dpp<kDppQuadXor1>(x));
    x = fmaxf(x, dpp<kDppQuadXor2>(x));
    x = fmaxf(x, dpp<kDppRowHalfMirror>(x));
    x = fmaxf(x, dpp<kDppRowMirror>(x));
    x = fmaxf(x, dpp<kDppRowBcast15, 0xa>(x));
    x = fmaxf(x, dpp<kDppRowBcast31, 0xc>(x));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

__device__ inline float wave_sum(float x) {
    x += dpp<kDppQuadXor1>(x);
    x += dpp<kDppQuadXor2>(x);
    x += dpp<kDppRowHalfMirror>(x);
    x += dpp<kDppRowMirror>(x);
    x += dpp<kDppRowBcast15, 0xa>(x);
    x += dpp<kDppRowBcast31, 0xc>(x);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Order the wave's LDS writes before reads by other lanes of the same wave
// (and the reverse).  The LDS executes one wave's instructions in issue order,
// so only the compiler has to be kept from moving accesses across this point:
// wavefront-scope fences do that without a wait.  (A workgroup-scope fence
// would also wait for every outstanding global load -- the prefetched tile.)
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float half_lo(uint32_t w) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
    return (float)h;
}

__device__ inline float half_hi(uint32_t w) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
    return (float)h;
}

__device__ inline float4 ldq4(const_f32_ptr p) { return make_float4(p[0], p[1], p[2], p[3]); }

__device__ inline float sbyte(uint32_t w, int e) { return (float)(int8_t)(w >> (8 * e)); }

template <int D>
struct Geo {
    static constexpr int NB = D / 32;   // q8_0 blocks per head
    static constexpr int CB = 34 * NB;  // bytes of one head of one row
};

// Buffer descriptor for head g of the 64-row tile starting at row0 of one
// tensor (K or V).  Its range ends with head g's chunk in the last readable
// row, so loads past the segment return zeros instead of touching memory.
template <int D>
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, const SegDesc& sg, int g, int row0) {
    using G_ = Geo<D>;
    const int64_t head_off = (int64_t)row0 * sg.stride + (int64_t)g * G_::CB;
    const int64_t lim64 = (int64_t)(sg.n_rows - 1 - row0) * sg.stride + G_::CB;
    const int32_t lim = (int32_t)(lim64 > 0x7fffffff ? 0x7fffffff : lim64);
    return make_rsrc(base + head_off, lim);
}

// ---------------------------------------------------------------------------
// The decode kernel.  A workgroup has one wave per q8_0 block of the head
// (D / 32 waves) and walks the split's rows in 64-row tiles, all waves on the
// same tile:
//   * wave w loads only block w of each row (a 9-dword window around its 34
//     bytes) for K and V, one tile ahead in registers, staged through a
//     wave-private LDS tile;
//   * scores: one lane per row, the block's 32 codes against the query slice
//     (read 4 dims x G heads at a time, from LDS or SGPRs), times the block
//     scale; the D / 32 block partials meet in LDS at one workgroup barrier
//     per tile (LDS-only fences, so the prefetch stays in flight), and every
//     wave sums them in the same order, so all waves hold identical scores;
//   * online softmax, repeated identically in each wave: the running maximum
//     is only raised when a score passes it by more than kLazyMax (log2
//     units), so most tiles need no wave-wide maximum and no rescale;
//   * values: wave w accumulates the 32 dims of block w; a lane holds 4 dims
//     (G x 4 accumulators) and 8 consecutive lanes take 8 rows of a pass;
//   * at the end each wave folds its 8 row slots (three DPP steps) and writes
//     its 32 dims: the waves own disjoint dims, so no cross-wave merge.
constexpr float kLazyMax = 8.0f;

// First dword of the 9-dword window holding block b of a head chunk, and the
// byte offset of the block's scale within that window (0 or 2).
__device__ inline int win_dword(int b) { return (34 * b) >> 2; }

template <int D, int G>
struct Slice {
    static constexpr int NB = D / 32;        // waves per workgroup
    static constexpr int GP = (G + 3) / 4 * 4;
    static constexpr int T = 64;             // rows per tile
    static constexpr int W = 9;              // dwords per row window
};

__device__ inline void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Window loads: instruction i of 9 reads unit 64 i + lane of the tile's
// 64 x 9 dwords (row = unit / 9, dword = unit % 9), so the LDS copy is a
// plain lane-contiguous store and each instruction covers ~7 rows of 36
// contiguous bytes.
__device__ inline void load_win(uint32_t (&r)[9], __amdgpu_buffer_rsrc_t rs, const int32_t (&voff)[9]) {
#pragma unroll
    for (int i = 0; i < 9; ++i) r[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff[i], 0, 0);
}

__device__ inline void store_win(const uint32_t (&r)[9], uint32_t* t, int lane) {
#pragma unroll
    for (int i = 0; i < 9; ++i) t[64 * i + lane] = r[i];
}

// V windows: q8_0 V as K (9 dwords around the 34-byte block); q4_0 V: 5
// dwords around the 18-byte block, 64 rows x 5 dwords = 5 loads per lane
// (unit 64 i + lane -> row = unit / 5, dword = unit % 5).
template <int VT>
struct VWin {
    static constexpr int W = VT ? 5 : 9;        // dwords per row window
    static constexpr int BB = VT ? 18 : 34;     // bytes per block
};

template <int VW>
__device__ inline void load_vwin(uint32_t (&r)[VW], __amdgpu_buffer_rsrc_t rs, const int32_t (&voff)[VW]) {
#pragma unroll
    for (int i = 0; i < VW; ++i) r[i] = __builtin_amdgcn_raw_buffer_load_b32(rs, voff[i], 0, 0);
}

template <int VW>
__device__ inline void store_vwin(const uint32_t (&r)[VW], uint32_t* t, int lane) {
#pragma unroll
    for (int i = 0; i < VW; ++i) t[64 * i + lane] = r[i];
}

// Descriptor for head g of the V tile at row0 (V rows of their own stride and
// block size); loads past the segment return zero.
template <int D, int VT>
__device__ inline __amdgpu_buffer_rsrc_t vtile_rsrc(const SegDesc& sg, int g, int row0) {
    constexpr int CBV = (D / 32) * VWin<VT>::BB;
    const int64_t head_off = (int64_t)row0 * sg.vstride + (int64_t)g * CBV;
    const int64_t lim64 = (int64_t)(sg.n_rows - 1 - row0) * sg.vstride + CBV;
    const int32_t lim = (int32_t)(lim64 > 0x7fffffff ? 0x7fffffff : lim64);
    return make_rsrc(sg.v + head_off, lim);
}

// One split: segment `seg` (SG: its pointers, strides, first visible row and
// readable rows) of sequence s, KV head g, the sp-th split of the segment and
// the lsplit-th of the launch.  The segment's visible row count and every
// other field of A are read only after the first tile's loads are issued.
template <int D, int G, int VT, int QS, int ODD>
__device__ __forceinline__ void slice_body(const LaunchArgs& A, const SegDesc& SG, const int s, const int seg,
                                           const int g, const int sp, const int lsplit, const int n_head_kv,
                                           const int split_rows, const float* q, const int wave, const int lane,
                                           uint32_t* tk, uint32_t* tv, float* sx, float* scw, float* sq) {
    using S_ = Slice<D, G>;
    constexpr int NB = S_::NB, GP = S_::GP, T = S_::T;
    const int r_begin = SG.row_lo + sp * split_rows;
    const int n_head_q = n_head_kv * G;
    const float* __restrict__ qg = q + ((size_t)s * n_head_q + (size_t)g * G) * D + 32 * wave;

    constexpr int VW = VWin<VT>::W;
    // Unit 64 i + lane of a 9-dword window tile is row 7 i + (lane + i) / 9,
    // dword (lane + i) % 9.  With lane = 9 r0 + d0 (d0 < 9), (lane + i) / 9 is
    // r0 plus a carry (d0 + i >= 9), so each offset is one select and one
    // three-way add from a per-lane base and a wave-uniform step.
    const int r0 = (lane * 57) >> 9;  // lane / 9 for lane < 64
    const int d0 = lane - 9 * r0;
    int32_t voff[9];
    {
        const int32_t base = r0 * SG.stride + 4 * d0 + win_dword(wave) * 4;
#pragma unroll
        for (int i = 0; i < 9; ++i)
            voff[i] = base + i * (7 * SG.stride + 4) + (d0 + i >= 9 ? SG.stride - 36 : 0);
    }
    int32_t voffv[VW];
    if constexpr (VW == 9) {
        const int32_t base = r0 * SG.vstride + 4 * d0 + ((VWin<VT>::BB * wave) >> 2) * 4;
#pragma unroll
        for (int i = 0; i < 9; ++i)
            voffv[i] = base + i * (7 * SG.vstride + 4) + (d0 + i >= 9 ? SG.vstride - 36 : 0);
    } else {
        const int32_t base = ((VWin<VT>::BB * wave) >> 2) * 4;
#pragma unroll
        for (int i = 0; i < VW; ++i) {
            const int u = 64 * i + lane;
            voffv[i] = (u / VW) * SG.vstride + (u % VW) * 4 + base;
        }
    }

    // q4_0 V: o accumulates c * code over the unsigned 4-bit codes and cs the
    // weights c, so that o - 8 * cs is the sum over c * (code - 8)
    float m[G], l[G], o[G][4], cs[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
        cs[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[h][e] = 0.f;
    }
    const int slot = lane & 7;   // value phase: row slot (8 consecutive lanes = 8 rows)
    const int grp = lane >> 3;   // value phase: 4-dim group within the block

    // K of a tile is staged before its scores, V only after them, so the
    // scores of the first tile start as soon as its K has arrived; the next
    // tile's K and V are in flight in registers meanwhile.
    // The wave's query slice (G heads x 32 dims) is read by the scores as
    // wave-uniform chunks of 4 dims x G heads, from one of two places:
    //  QS = 0: LDS, filled with one vector load per lane issued first, and
    //          read back as broadcast float4s (for workgroups alone on their
    //          CU: the scalar loads below would miss a cold scalar cache
    //          there, several microseconds per call);
    //  QS = 1: SGPRs, by scalar loads one chunk ahead (once several
    //          workgroups share a CU: no LDS traffic for the query, which
    //          would otherwise be about half of the kernel's LDS reads).
    float4 qv4 = make_float4(0.f, 0.f, 0.f, 0.f);
    if (!QS && lane < G * 8) qv4 = *(const float4*)(qg + (lane >> 3) * D + 4 * (lane & 7));
    uint32_t rk[9], rv[VW];
    load_win(rk, tile_rsrc<D>(SG.k, SG, g, r_begin), voff);
    load_vwin<VW>(rv, vtile_rsrc<D, VT>(SG, g, r_begin), voffv);
    // The arguments that were not preloaded, read (and waited for) while the
    // first tile is in flight.
    const int32_t n_vis = A.seq[s].seg[seg].n_vis, seq_splits = A.seq[s].n_split, split_off = A.split_off;
    const float scale_log2e = A.scale_log2e;
    float* const out = A.out;
    float* const po = A.po;
    float* const pm = A.pm;
    float* const pl = A.pl;
    float* const part_o = A.part_o;
    float* const part_m = A.part_m;
    float* const part_l = A.part_l;
    asm volatile("" ::"s"(n_vis), "s"(seq_splits), "s"(split_off), "s"(scale_log2e));
    asm volatile("" ::"s"(out), "s"(po), "s"(pm), "s"(pl), "s"(part_o), "s"(part_m), "s"(part_l));
    const int r_end = min(r_begin + split_rows, SG.row_lo + n_vis);
    const int n_tiles = (r_end - r_begin + T - 1) / T;
    const bool single = seq_splits == 1;
    const int abs_split = split_off + lsplit;
    if (!QS && lane < G * 8) *(float4*)&sq[(lane >> 3) * 32 + 4 * (lane & 7)] = qv4;
    store_win(rk, tk, lane);

    for (int t = 0; t < n_tiles; ++t) {
        const int row0 = r_begin + t * T;
        const int nv = min(T, r_end - row0);
        const bool has_next = t + 1 < n_tiles;
        if (has_next) load_win(rk, tile_rsrc<D>(SG.k, SG, g, row0 + T), voff);
        wave_lds_sync();

        // ---- block partial scores, one lane per row
        float* sxt = sx + (t & 1) * (NB * G * 64);
        {
            const uint32_t* rp = tk + lane * 9;
            uint32_t w[9];
#pragma unroll
            for (int j = 0; j < 9; ++j) w[j] = rp[j];
            // Query chunks of 4 dims x G heads.  From LDS (QS = 0) each is read
            // just before its FMAs: the empty asm statements keep the reads
            // from being hoisted, so the query holds one chunk of VGPRs (G = 5:
            // 125 VGPRs instead of 140 when reading one chunk ahead, so four
            // workgroups fit a CU instead of three).  From SGPRs (QS = 1) the
            // scalar loads run one chunk ahead, their order pinned the same way.
            float dot[G];
#pragma unroll
            for (int h = 0; h < G; ++h) dot[h] = 0.f;
            float4 qn[G];
            if constexpr (QS) {
                const_f32_ptr qp = (const_f32_ptr)qg;
                asm volatile("" : "+s"(qp));
#pragma unroll
                for (int h = 0; h < G; ++h) qn[h] = ldq4(qp + h * D);
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
#pragma unroll
                for (int h = 0; h < G; ++h) asm volatile("" : "+v"(dot[h]));
                float4 qc[G];
                if constexpr (QS) {
#pragma unroll
                    for (int h = 0; h < G; ++h) qc[h] = qn[h];
                    if (c + 1 < 8) {
                        const_f32_ptr qp = (const_f32_ptr)qg + 4 * (c + 1);
                        asm volatile("" : "+s"(qp));
#pragma unroll
                        for (int h = 0; h < G; ++h) qn[h] = ldq4(qp + h * D);
                    }
                } else {
                    int off = 4 * c;
                    asm volatile("" : "+v"(off));
#pragma unroll
                    for (int h = 0; h < G; ++h) qc[h] = *(const float4*)&sq[h * 32 + off];
                }
                // codes 4c .. 4c+3: bytes 0..3 of dword c+1 of an odd block's
                // window; bytes 2, 3 of dword c and 0, 1 of dword c+1 of an even
                // block's (its codes start at byte 2), each converted from its byte
                const float k0 = ODD ? sbyte(w[c + 1], 0) : sbyte(w[c], 2);
                const float k1 = ODD ? sbyte(w[c + 1], 1) : sbyte(w[c], 3);
                const float k2 = ODD ? sbyte(w[c + 1], 2) : sbyte(w[c + 1], 0);
                const float k3 = ODD ? sbyte(w[c + 1], 3) : sbyte(w[c + 1], 1);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    dot[h] = fmaf(qc[h].x, k0, dot[h]);
                    dot[h] = fmaf(qc[h].y, k1, dot[h]);
                    dot[h] = fmaf(qc[h].z, k2, dot[h]);
                    dot[h] = fmaf(qc[h].w, k3, dot[h]);
                }
            }
            // block scale times the softmax scale (exp2 domain)
            const float dk = (ODD ? half_hi(w[0]) : half_lo(w[0])) * scale_log2e;
#pragma unroll
            for (int h = 0; h < G; ++h) sxt[(wave * G + h) * 64 + lane] = dot[h] * dk;
        }
        lds_barrier();
        store_vwin<VW>(rv, tv, lane);
        if (has_next) load_vwin<VW>(rv, vtile_rsrc<D, VT>(SG, g, row0 + T), voffv);
        wave_lds_sync();

        // ---- full scores (same sum order in every wave) and online softmax
        float sc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float a = sxt[h * 64 + lane];
#pragma unroll
            for (int b = 1; b < NB; ++b) a += sxt[(b * G + h) * 64 + lane];
            sc[h] = a;
        }
        if (nv < T) {
            // only a split's last tile can be partial
#pragma unroll
            for (int h = 0; h < G; ++h) sc[h] = (lane < nv) ? sc[h] : -INFINITY;
        }
        {
            // first tile: start from the score of its first row (always visible)
            // instead of a wave-wide maximum; the lazy rule below still raises
            // it if any row passes it by more than kLazyMax
            if (t == 0) {
#pragma unroll
                for (int h = 0; h < G; ++h)
                    m[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sc[h])));
            }
            bool big = false;
#pragma unroll
            for (int h = 0; h < G; ++h) big |= sc[h] > m[h] + kLazyMax;
            if (__builtin_amdgcn_ballot_w64(big)) {
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float mn = fmaxf(m[h], wave_max(sc[h]));
                    if (mn > m[h]) {
                        const float alpha = (m[h] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[h] - mn);
                        l[h] *= alpha;
                        if (VT) cs[h] *= alpha;
#pragma unroll
                        for (int e = 0; e < 4; ++e) o[h][e] *= alpha;
                        m[h] = mn;
                    }
                }
            }
        }
        {
            // rows past the visible range may hold any bits: their weight is an exact 0
            const float dv = (lane < nv) ? (ODD ? half_hi(tv[lane * VW]) : half_lo(tv[lane * VW])) : 0.f;
            float c[GP];
#pragma unroll
            for (int h = 0; h < GP; ++h) c[h] = 0.f;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float p = __builtin_amdgcn_exp2f(sc[h] - m[h]);
                l[h] += p;
                c[h] = p * dv;
                if (VT) cs[h] += c[h];
            }
#pragma unroll
            for (int h = 0; h < GP; h += 4) *(float4*)&scw[lane * GP + h] = make_float4(c[h], c[h + 1], c[h + 2], c[h + 3]);
        }
        wave_lds_sync();

        // ---- values: 4 dims per lane, 8 rows per pass
#pragma unroll 4
        for (int ps = 0; ps < 8; ++ps) {
            const int r = ps * 8 + slot;
            uint32_t x = 0;
            float vq[4];
            if constexpr (VT == 0) {
                // dims 4 grp .. 4 grp + 3, bytes picked as for the scores
                const uint32_t* rp = tv + r * 9;
                const uint32_t lo = rp[grp], hi = rp[grp + 1];
                vq[0] = ODD ? sbyte(hi, 0) : sbyte(lo, 2);
                vq[1] = ODD ? sbyte(hi, 1) : sbyte(lo, 3);
                vq[2] = ODD ? sbyte(hi, 2) : sbyte(hi, 0);
                vq[3] = ODD ? sbyte(hi, 3) : sbyte(hi, 1);
            } else {
                // dims 4 grp .. 4 grp + 3: low nibbles of code bytes 4 grp .. (grp < 4),
                // high nibbles of bytes 4 (grp - 4) .. (grp >= 4)
                const uint32_t* rp = tv + r * 5;
                const int kq = grp & 3;
                const uint32_t raw = ODD ? rp[kq + 1] : __builtin_amdgcn_alignbyte(rp[kq + 1], rp[kq], 2);
                x = (raw >> ((grp >> 2) * 4)) & 0x0F0F0F0Fu;
            }
            float c[GP];
#pragma unroll
            for (int h = 0; h < GP; h += 4) {
                const float4 cv = *(const float4*)&scw[r * GP + h];
                c[h] = cv.x;
                c[h + 1] = cv.y;
                c[h + 2] = cv.z;
                c[h + 3] = cv.w;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float vv = VT ? (float)((x >> (8 * e)) & 0xFFu) : vq[e];
#pragma unroll
                for (int h = 0; h < G; ++h) o[h][e] = fmaf(c[h], vv, o[h][e]);
            }
        }
        wave_lds_sync();
        if (has_next) store_win(rk, tk, lane);
    }

    // ---- fold the 8 row slots (same m in every slot; 8 consecutive lanes), finish l
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x = o[h][e];
            x += dpp<kDppQuadXor1>(x);
            x += dpp<kDppQuadXor2>(x);
            x += dpp<kDppRowHalfMirror>(x);
            o[h][e] = x;
        }
        l[h] = wave_sum(l[h]);
        if (VT) {
            const float c8 = 8.f * wave_sum(cs[h]);
#pragma unroll
            for (int e = 0; e < 4; ++e) o[h][e] -= c8;
        }
    }
    const int hq0 = g * G;
    const int dim0 = 32 * wave + 4 * grp;
    if (slot == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (single && part_o) {
                *(float4*)&part_o[((size_t)s * n_head_q + hq0 + h) * D + dim0] =
                    make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
            } else if (single) {
                const float inv = 1.f / l[h];
                *(float4*)&out[((size_t)s * n_head_q + hq0 + h) * D + dim0] =
                    make_float4(o[h][0] * inv, o[h][1] * inv, o[h][2] * inv, o[h][3] * inv);
            } else {
                const size_t pi = (size_t)abs_split * n_head_q + hq0 + h;
                *(float4*)&po[pi * D + dim0] = make_float4(o[h][0], o[h][1], o[h][2], o[h][3]);
            }
        }
    }
    if (wave == 0 && lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (!single) {
                const size_t pi = (size_t)abs_split * n_head_q + hq0 + h;
                pm[pi] = m[h];
                pl[pi] = l[h];
            } else if (part_o) {
                const size_t sh = (size_t)s * n_head_q + hq0 + h;
                part_m[sh] = m[h];
                part_l[sh] = l[h];
            }
        }
    }
}

// The leading arguments (14 dwords: the counts, the query and the first
// sequence's first segment) are preloaded into SGPRs when the waves start (the
// file is built with kernel-argument preloading), so the first split segment
// of a one-sequence launch issues its query and K/V loads without reading its
// arguments from memory: they sit in memory that the step's K/V stream has
// evicted from every cache since the layer's previous call.  Everything else
// comes from the LaunchArgs block, read while the first tile is in flight.
// kv_seq packs n_head_kv (low 16 bits) and the launch's sequence count.
template <int D, int G, int VT, int QS>
__global__ void __launch_bounds__(64 * (D / 32))
slice_kernel(const int32_t n_items, const int32_t kv_seq, const int32_t split_rows, const int32_t n_split0,
             const float* q, const uint8_t* k0, const uint8_t* v0, const int32_t stride0, const int32_t vstride0,
             const int32_t row_lo0, const int32_t n_rows0, const LaunchArgs A) {
    using S_ = Slice<D, G>;
    constexpr int NB = S_::NB, GP = S_::GP, T = S_::T;
    __shared__ __attribute__((aligned(16))) uint32_t s_kv[NB][2][T * 9];
    __shared__ __attribute__((aligned(16))) float s_x[2 * NB * G * 64];
    __shared__ __attribute__((aligned(16))) float s_c[NB][T * GP];
    __shared__ __attribute__((aligned(16))) float s_q[NB][QS ? 4 : G * 32];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_head_kv = kv_seq & 0xffff, n_seq = kv_seq >> 16;
    // the grid is n_items rounded up to a multiple of 8 (one run per XCD)
    const int item = (blockIdx.x & 7) * ((n_items + 7) >> 3) + (blockIdx.x >> 3);
    if (item >= n_items) return;
    const int lsplit = item / n_head_kv;
    const int g = item - lsplit * n_head_kv;
    int s = 0, sp = lsplit, seg = 0;
    SegDesc SG;
    SG.k = k0;
    SG.v = v0;
    SG.stride = stride0;
    SG.vstride = vstride0;
    SG.row_lo = row_lo0;
    SG.n_rows = n_rows0;
    if (n_seq > 1 || lsplit >= n_split0) {
        // another sequence or the second segment: its descriptor from the block
        while (s + 1 < n_seq && A.seq[s + 1].split_base <= lsplit) ++s;
        sp = lsplit - A.seq[s].split_base;
        const int n0 = A.seq[s].seg[0].n_split;
        if (sp >= n0) {
            sp -= n0;
            seg = 1;
        }
        const SegDesc& d = A.seq[s].seg[seg];
        SG.k = d.k;
        SG.v = d.v;
        SG.stride = d.stride;
        SG.vstride = d.vstride;
        SG.row_lo = d.row_lo;
        SG.n_rows = d.n_rows;
        // wait here, so that the one-sequence path meets no pending load
        asm volatile("" ::"s"(SG.k), "s"(SG.v), "s"(SG.stride), "s"(SG.vstride), "s"(SG.row_lo), "s"(SG.n_rows));
    }
    SG.n_vis = SG.n_split = 0;  // not used: slice_body reads the visible row count itself
    if (wave & 1)
        slice_body<D, G, VT, QS, 1>(A, SG, s, seg, g, sp, lsplit, n_head_kv, split_rows, q, wave, lane,
                                    s_kv[wave][0], s_kv[wave][1], s_x, s_c[wave], s_q[wave]);
    else
        slice_body<D, G, VT, QS, 0>(A, SG, s, seg, g, sp, lsplit, n_head_kv, split_rows, q, wave, lane,
                                    s_kv[wave][0], s_kv[wave][1], s_x, s_c[wave], s_q[wave]);
}

// Merge n partial results (m_k, l_k, o_k) of one (sequence, query head) in
// index order.  One wave per 32 dims; lanes take partials, 64 at a time.
// Every lane loads its partial's maximum, sum and 32 outputs together (one
// round trip), the weights follow from a wave maximum, and the 64 weighted
// rows are summed column by column through LDS in index order, so the result
// does not depend on timing.  `load(k, m, l, v)` fetches partial k (k < n);
// `after_first_load()` runs once the first 64 partials are requested.
// Returns, in lanes 0..31, dimension 32 * wave + lane of O = sum e^(m_k - M) o_k,
// with M and L = sum e^(m_k - M) l_k in every lane.
template <class Load, class Hook>
__device__ inline void merge_rows(const Load& load, const Hook& after_first_load, int n, int lane, float (*so)[33],
                                  float& O, float& M, float& L) {
    M = -INFINITY;
    L = 0.f;
    O = 0.f;
    for (int c0 = 0; c0 < n; c0 += 64) {
        const int k = c0 + lane;
        const bool ok = k < n;
        float pm, pl;
        float4 v[8];
        load(ok ? k : c0, pm, pl, v);
        if (c0 == 0) after_first_load();
        pm = ok ? pm : -INFINITY;
        pl = ok ? pl : 0.f;
        const float Mn = fmaxf(M, wave_max(pm));
        const float w = ok ? __builtin_amdgcn_exp2f(pm - Mn) : 0.f;
        const float alpha = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        L = fmaf(L, alpha, wave_sum(w * pl));
        O *= alpha;
        M = Mn;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            so[lane][4 * j] = w * v[j].x;
            so[lane][4 * j + 1] = w * v[j].y;
            so[lane][4 * j + 2] = w * v[j].z;
            so[lane][4 * j + 3] = w * v[j].w;
        }
        wave_lds_sync();
        // column sums: lanes 0..31 add rows 0..31, lanes 32..63 rows 32..63, then
        // the two halves meet (a fixed order)
        {
            const int col = lane & 31, r0 = lane & 32;
            float t = 0.f;
#pragma unroll 16
            for (int r = 0; r < 32; ++r) t += so[r0 + r][col];
            t += __shfl_xor(t, 32);
            O += t;
        }
        wave_lds_sync();
    }
}

// Merge the split partials of one (sequence, query head): one workgroup per
// (sequence, query head), one wave per 32 dims.  A separate launch, so the
// partials written by the decode kernel are visible without cache
// maintenance inside a kernel.
// Leading arguments preloaded into SGPRs as in the decode kernel: the first
// sequence's split count and the partials, so the partial loads of a
// one-sequence launch start without reading its arguments from memory.
template <int D>
__global__ void __launch_bounds__(64 * (D / 32))
combine_kernel(const int32_t n_head_q, const int32_t split_off, const int32_t n_split0, const float* ppm,
               const float* ppl, const float* ppo, const LaunchArgs A) {
    constexpr int NWV = D / 32;
    __shared__ float s_o[NWV][64][33];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hq = blockIdx.x % n_head_q;
    const int s = blockIdx.x / n_head_q;
    int32_t S = n_split0, base = 0;  // sequence 0 starts the launch's splits
    if (s > 0) {
        S = A.seq[s].n_split;
        base = A.seq[s].split_base;
    }
    if (S <= 1) return;  // written directly by the decode kernel
    const int first = split_off + base;
    auto load = [&](int k, float& pm, float& pl, float4 (&v)[8]) {
        const size_t pi = (size_t)(first + k) * n_head_q + hq;
        pm = ppm[pi];
        pl = ppl[pi];
        const float4* po = (const float4*)(ppo + pi * D + 32 * wave);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = po[j];
    };
    // the output pointers, read while the first partials are in flight
    auto read_outputs = [&]() { asm volatile("" ::"s"(A.out), "s"(A.part_o), "s"(A.part_m), "s"(A.part_l)); };
    float O, M, L;
    merge_rows(load, read_outputs, S, lane, s_o[wave], O, M, L);
    if (lane < 32) write_final(A, D, (size_t)s * n_head_q + hq, 32 * wave + lane, O, M, L, wave == 0 && lane == 0);
}

// Merge the partial results of n_part calls over disjoint row sets of the
// same sequences (tile-streamed attention): partial t holds o [S][H][D], then
// m [S][H], then l [S][H] (S sequences, H query heads), (D + 2) S H floats.
template <int D>
__global__ void __launch_bounds__(64 * (D / 32)) merge_kernel(const float* parts, int32_t n_part, int32_t n_sh,
                                                               float* out) {
    constexpr int NWV = D / 32;
    __shared__ float s_o[NWV][64][33];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const size_t sh = blockIdx.x;  // sequence * H + query head
    const size_t stride = (size_t)(D + 2) * n_sh;
    auto load = [&](int k, float& pm, float& pl, float4 (&v)[8]) {
        const float* p = parts + (size_t)k * stride;
        pm = p[(size_t)n_sh * D + sh];
        pl = p[(size_t)n_sh * (D + 1) + sh];
        const float4* po = (const float4*)(p + sh * D + 32 * wave);
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = po[j];
    };
    float O, M, L;
    merge_rows(load, [] {}, n_part, lane, s_o[wave], O, M, L);
    if (lane < 32) out[sh * D + 32 * wave + lane] = O / L;
}

typedef void (*decode_fn)(int32_t, int32_t, int32_t, int32_t, const float*, const uint8_t*, const uint8_t*, int32_t,
                          int32_t, int32_t, int32_t, const LaunchArgs);
typedef void (*combine_fn)(int32_t, int32_t, int32_t, const float*, const float*, const float*, const LaunchArgs);

combine_fn pick_combine(int D) { return D == 128 ? combine_kernel<128> : combine_kernel<64>; }

// The kernel for group G, or null for a scalar query beyond
// kScalarQueryMaxGroup (the plan never asks for one).
template <int D, int G, int VT, int QS>
decode_fn slice_ptr() {
    if constexpr (QS && G > kScalarQueryMaxGroup) return nullptr;
    else return slice_kernel<D, G, VT, QS>;
}

template <int D, int VT, int QS>
decode_fn pick_slice_g(int G) {
    switch (G) {
        case 1: return slice_ptr<D, 1, VT, QS>();
        case 2: return slice_ptr<D, 2, VT, QS>();
        case 3: return slice_ptr<D, 3, VT, QS>();
        case 4: return slice_ptr<D, 4, VT, QS>();
        case 5: return slice_ptr<D, 5, VT, QS>();
        case 6: return slice_ptr<D, 6, VT, QS>();
        case 7: return slice_ptr<D, 7, VT, QS>();
        case 8: return slice_ptr<D, 8, VT, QS>();
    }
    return nullptr;
}

template <int QS>
decode_fn pick_slice_qs(int D, int G, int VT) {
    if (VT) return D == 128 ? pick_slice_g<128, 1, QS>(G) : pick_slice_g<64, 1, QS>(G);
    return D == 128 ? pick_slice_g<128, 0, QS>(G) : pick_slice_g<64, 0, QS>(G);
}

decode_fn pick_slice(int D, int G, int VT, bool scalar_query) {
    return scalar_query ? pick_slice_qs<1>(D, G, VT) : pick_slice_qs<0>(D, G, VT);
}

}  // namespace
}  // namespace kvd

using namespace kvd;

extern "C" int kvd_attend_workspace_bytes(const kvd_attn_args* args, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(KVD_EINVAL, "bytes is NULL");
    AttendPlan p;
    const int rc = plan_attend(args, &p);
    if (rc != KVD_OK) return rc;
    *bytes = p.ws_bytes;
    return KVD_OK;
}

namespace kvd {
namespace {

// Shared by the normal and the partial-result entry points: `part` null ->
// write out; else write (o, m, l) at part (layout of merge_kernel's input).
int launch_attend(const kvd_attn_args* a, void* stream, float* part) {
    AttendPlan p;
    int rc = plan_attend(a, &p);
    if (rc != KVD_OK) return rc;
    if (!part && !a->out) return fail(KVD_EINVAL, "out must not be NULL");
    if (!part && (uintptr_t)a->out % 16) return fail(KVD_EINVAL, "out must be 16-byte aligned");
    if (part && (uintptr_t)part % 16) return fail(KVD_EINVAL, "partial must be 16-byte aligned");
    if (p.ws_bytes > 0) {
        if (!a->workspace || a->workspace_bytes < p.ws_bytes)
            return fail(KVD_EINVAL, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                        a->workspace ? a->workspace_bytes : (size_t)0);
        if ((uintptr_t)a->workspace % 256) return fail(KVD_EINVAL, "workspace must be 256-byte aligned");
    }
    const decode_fn dk = pick_slice(a->head_dim, p.group, a->v_type, p.scalar_query);
    const combine_fn ck = pick_combine(a->head_dim);
    if (!dk) return fail(KVD_EINVAL, "no kernel for head_dim %d, group %d", a->head_dim, p.group);

    uint8_t* ws = (uint8_t*)a->workspace;
    const int D = a->head_dim;
    const int n_head_q = a->n_head_q;
    const float scale_log2e = (float)((double)a->scale * 1.4426950408889634);

    for (int s0 = 0; s0 < a->n_seq; s0 += kMaxSeqPerLaunch) {
        const int ns = (a->n_seq - s0 < kMaxSeqPerLaunch) ? a->n_seq - s0 : kMaxSeqPerLaunch;
        LaunchArgs L;
        memset(&L, 0, sizeof(L));
        const int64_t base0 = p.seq[s0].split_base;
        int64_t nsplit = 0;
        for (int j = 0; j < ns; ++j) {
            const SeqPlan& sp = p.seq[s0 + j];
            const kvd_kv_seg* segs = a->segs + (size_t)(s0 + j) * a->n_seg;
            SeqDesc& d = L.seq[j];
            for (int k = 0; k < 2; ++k) {
                SegDesc& sd = d.seg[k];
                const SegPlan& pl = sp.seg[k];
                sd.n_split = pl.n_split;
                sd.row_lo = pl.row_lo;
                sd.n_vis = pl.n_vis;
                sd.n_rows = pl.n_rows;
                if (k < a->n_seg) {
                    sd.k = (const uint8_t*)segs[k].k;
                    sd.v = (const uint8_t*)segs[k].v;
                    sd.stride = (int32_t)segs[k].row_stride;
                    sd.vstride = (int32_t)(segs[k].v_row_stride ? segs[k].v_row_stride : segs[k].row_stride);
                }
            }
            d.split_base = (int32_t)(sp.split_base - base0);
            d.n_split = sp.n_split;
            nsplit += sp.n_split;
        }
        L.q = a->q + (size_t)s0 * n_head_q * D;
        const size_t n_sh = (size_t)a->n_seq * n_head_q;
        if (part) {
            L.part_o = part + (size_t)s0 * n_head_q * D;
            L.part_m = part + n_sh * D + (size_t)s0 * n_head_q;
            L.part_l = part + n_sh * (D + 1) + (size_t)s0 * n_head_q;
        } else {
            L.out = a->out + (size_t)s0 * n_head_q * D;
        }
        if (p.ws_bytes > 0) {
            L.pm = (float*)(ws + p.off_pm);
            L.pl = (float*)(ws + p.off_pl);
            L.po = (float*)(ws + p.off_po);
        }
        L.n_seq = ns;
        L.n_head_kv = a->n_head_kv;
        L.split_rows = p.split_rows;
        L.n_items = (int32_t)(nsplit * a->n_head_kv);
        L.split_off = (int32_t)base0;
        L.scale_log2e = scale_log2e;
        const unsigned grid = (unsigned)((L.n_items + 7) / 8 * 8);  // the kernel assumes this rounding
        const SegDesc& f = L.seq[0].seg[0];
        hipLaunchKernelGGL(dk, dim3(grid), dim3(64 * p.waves), 0, (hipStream_t)stream, L.n_items,
                           L.n_head_kv | (L.n_seq << 16), L.split_rows, f.n_split, L.q, f.k, f.v, f.stride, f.vstride,
                           f.row_lo, f.n_rows, L);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(KVD_EHIP, "decode kernel launch: %s", hipGetErrorString(e));
        bool multi = false;
        for (int j = 0; j < ns; ++j) multi |= L.seq[j].n_split > 1;
        if (multi) {
            hipLaunchKernelGGL(ck, dim3((unsigned)(ns * n_head_q)), dim3(2 * D), 0, (hipStream_t)stream,
                               (int32_t)n_head_q, L.split_off, L.seq[0].n_split, L.pm, L.pl, L.po, L);
            e = hipGetLastError();
            if (e != hipSuccess) return fail(KVD_EHIP, "combine kernel launch: %s", hipGetErrorString(e));
        }
    }
    return KVD_OK;
}

}  // namespace
}  // namespace kvd

extern "C" int kvd_attend_decode(const kvd_attn_args* a, void* stream) {
    clear_error();
    return launch_attend(a, stream, nullptr);
}

extern "C" int kvd_attend_decode_partial(const kvd_attn_args* a, float* partial, void* stream) {
    clear_error();
    if (!partial) return fail(KVD_EINVAL, "partial must not be NULL");
    return launch_attend(a, stream, partial);
}

extern "C" int kvd_attend_merge(const float* partials, int32_t n_part, int32_t n_seq, int32_t n_head_q,
                                int32_t head_dim, float* out, void* stream) {
    clear_error();
    if (!partials || !out) return fail(KVD_EINVAL, "partials and out must not be NULL");
    if (n_part < 1 || n_part > (1 << 20)) return fail(KVD_EINVAL, "n_part %d out of range [1, 2^20]", n_part);
    if (n_seq < 1 || n_head_q < 1 || (int64_t)n_seq * n_head_q > (1 << 24))
        return fail(KVD_EINVAL, "n_seq %d x n_head_q %d out of range", n_seq, n_head_q);
    if (head_dim != 64 && head_dim != 128) return fail(KVD_EINVAL, "head_dim %d must be 64 or 128", head_dim);
    if ((uintptr_t)partials % 16 || (uintptr_t)out % 16)
        return fail(KVD_EINVAL, "partials and out must be 16-byte aligned");
    const int32_t n_sh = n_seq * n_head_q;
    if (n_sh % 2) return fail(KVD_EINVAL, "n_seq x n_head_q must be even (partials stay 16-byte aligned)");
    if (head_dim == 128)
        hipLaunchKernelGGL(merge_kernel<128>, dim3((unsigned)n_sh), dim3(256), 0, (hipStream_t)stream, partials,
                           n_part, n_sh, out);
    else
        hipLaunchKernelGGL(merge_kernel<64>, dim3((unsigned)n_sh), dim3(128), 0, (hipStream_t)stream, partials,
                           n_part, n_sh, out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVD_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
    return KVD_OK;
}
