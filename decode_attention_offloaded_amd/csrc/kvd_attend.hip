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
// workgroup of W = 4, 8 or 12 waves (the plan picks W from the work per CU).
// Each wave walks its own 16-row sub-tiles of the split (every W-th one) over
// all head_dim dims of the head and keeps its own online-softmax state; the W
// states meet in LDS once, at the end of the split.  The two contractions of a
// sub-tile run on the matrix cores (decode_kernel has the details).  The
// arguments a split needs before its first loads are kernel arguments that
// the hardware preloads into SGPRs; the rest are read while the first sub-tile
// is in flight.
// A split with siblings writes an unnormalised partial (m, l, o) to the
// workspace and a second, small launch merges the partials of each
// (sequence, query head) in split order, so the result depends only on the
// split plan.  (Merging inside the first launch would need device-scope
// release/acquire between workgroups, which on this chip writes back and
// invalidates the whole L2 of an XCD per workgroup.)
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "kvd_internal.h"
#include "kvd_plan.h"

namespace kvd {
namespace {

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
    int32_t split_base;  // first split of this slot's sequence, relative to the launch
    int32_t n_split;     // splits of this sequence
    int32_t orig;        // the sequence's index among the launch's q / out rows
};

struct LaunchArgs {
    // First split of each slot (seq[j].split_base; INT32_MAX for unused
    // slots), together in 64 bytes so that a workgroup finds its slot with
    // one load.
    int32_t slot_split[kMaxSeqPerLaunch];
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

// The running maximum of each (wave, query head) is raised only when a score
// passes it by more than kLazyMax (log2 units), so most sub-tiles need no
// exchange of maxima and no rescale; the weights exp2(s - m) stay below 2^8.
constexpr float kLazyMax = 8.0f;

constexpr int gcd16(int x) { return (x & 15) == 0 ? 16 : (x & 7) == 0 ? 8 : (x & 3) == 0 ? 4 : (x & 1) == 0 ? 2 : 1; }

// One head of one row (CB bytes) read as whole 16-byte units: the units from
// the 16-byte boundary at or below the chunk start, enough for the largest
// offset the chunk can have within its unit.  UR units per row; in LDS a row
// is P = 4 UR dwords, the chunk `lead` bytes into it.
template <int CB>
struct RowUnits {
    static constexpr int LEAD_MAX = 16 - gcd16(CB);
    static constexpr int UR = (CB + LEAD_MAX + 15) / 16;
    static constexpr int P = 4 * UR;
};

template <int D, int VT>
struct Lay {
    static constexpr int NB = D / 32;           // q8_0 blocks per head
    static constexpr int RSETS = 4 / NB;        // row sets per sub-tile (DPP rows per block)
    static constexpr int R = 16 * RSETS;        // rows per sub-tile
    static constexpr int CB = 34 * NB;          // K bytes of one head of one row
    static constexpr int VB = VT ? 18 : 34;     // V bytes per block
    static constexpr int CBV = VB * NB;         // V bytes of one head of one row
    static constexpr int PK = RowUnits<CB>::P;  // LDS dwords per K row
    static constexpr int PV = RowUnits<CBV>::P;
    static constexpr int KUW = R * RowUnits<CB>::UR;   // 16-byte units of a K sub-tile
    static constexpr int VUW = R * RowUnits<CBV>::UR;
    static constexpr int KW = (KUW + 63) / 64;  // 16-byte loads per lane (K)
    static constexpr int VW = (VUW + 63) / 64;
    static constexpr int KN = (R * PK + 63) / 64;  // dword loads per lane (K)
    static constexpr int VN = (R * PV + 63) / 64;
    static_assert(4 * KW >= KN && 4 * VW >= VN, "the dword loads fit the registers of the 16-byte loads");
    static constexpr int KT = 4 * 64 * KW;      // LDS dwords of the K tile
    static constexpr int VT_ = 4 * 64 * VW;
};

// Per-wave LDS: the K and V sub-tile, reused at the end of the split for the
// wave's (m, l, o) before the four waves merge.
template <int D, int G, int VT, int NBUF>
struct WaveLds {
    using L_ = Lay<D, VT>;
    static constexpr int K = L_::KT;
    static constexpr int V = L_::VT_;
    static constexpr int OFF_O = (2 * G + 3) & ~3;  // o after m [G] and l [G], 16-byte aligned
    static constexpr int MERGE = OFF_O + G * D;
    static constexpr int DWORDS = (NBUF * (K + V) > MERGE ? NBUF * (K + V) : MERGE);
};

// Descriptor for head g of the sub-tile at row0 of one tensor (rows `stride`
// bytes apart, cb bytes per head).  It starts `lead` bytes before the head's
// chunk and ends with the chunk of the last readable row, so loads past the
// segment return zeros (and a sub-tile that starts past the segment reads
// nothing).
__device__ inline __amdgpu_buffer_rsrc_t sub_rsrc(const uint8_t* base, int32_t stride, int32_t n_rows, int cb, int g,
                                                  int lead, int row0) {
    const int64_t off = (int64_t)row0 * stride + (int64_t)g * cb - lead;
    const int64_t lim64 = (int64_t)(n_rows - 1 - row0) * stride + lead + cb;
    const int32_t lim = (int32_t)(lim64 > 0x7fffffff ? 0x7fffffff : lim64 < 0 ? 0 : lim64);
    return make_rsrc(base + off, lim);
}

// Offsets of the 16-byte units u = 64 m + lane of a sub-tile (row u / UR,
// unit u % UR); units past the sub-tile re-read its last unit (their LDS copy
// is never read).
template <int N, int UR, int NU>
__device__ inline void wide_offsets(int32_t (&off)[N], int lane, int32_t stride) {
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const int u = min(64 * m + lane, NU - 1);
        const int row = u / UR;
        off[m] = row * stride + 16 * (u - row * UR);
    }
}

// Offsets of the dwords u = 64 m + lane of a sub-tile (row u / P, dword u % P).
template <int N, int P, int NU>
__device__ inline void narrow_offsets(int32_t (&off)[N], int lane, int32_t stride) {
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const int u = min(64 * m + lane, NU - 1);
        const int row = u / P;
        off[m] = row * stride + 4 * (u - row * P);
    }
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// One 16-byte buffer load per lane straight into LDS: lane i's bytes land at
// t + 16 i (t wave-uniform), the layout store_wide writes from registers.
// The host pass has no LDS address space to cast to, so the body is device
// code only.
template <int AUX>
__device__ inline void load_lds16(__amdgpu_buffer_rsrc_t rs, uint32_t* t, int32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)t, 16, off, 0, 0, AUX);
#endif
}

// Wait until at most N vector-memory loads of this wave are outstanding (they
// complete in issue order); expcnt and lgkmcnt are left unconstrained.
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Cache policy of the K/V loads (the buffer instructions' aux operand): 0, or
// kLoadNonTemporal (the nt bit: the lines are marked for early eviction).
constexpr int kLoadNonTemporal = 2;

template <int N, int REG, int AUX = 0>
__device__ inline void load_wide(uint32_t (&r)[REG], __amdgpu_buffer_rsrc_t rs, const int32_t (&off)[N]) {
#pragma unroll
    for (int m = 0; m < N; ++m) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off[m], 0, AUX);
        r[4 * m] = x.x;
        r[4 * m + 1] = x.y;
        r[4 * m + 2] = x.z;
        r[4 * m + 3] = x.w;
    }
}

template <int N, int REG, int AUX = 0>
__device__ inline void load_narrow(uint32_t (&r)[REG], __amdgpu_buffer_rsrc_t rs, const int32_t (&off)[N]) {
#pragma unroll
    for (int m = 0; m < N; ++m) r[m] = __builtin_amdgcn_raw_buffer_load_b32(rs, off[m], 0, AUX);
}

template <int N, int REG>
__device__ inline void store_wide(const uint32_t (&r)[REG], uint32_t* t, int lane) {
#pragma unroll
    for (int m = 0; m < N; ++m) {
        u32x4 x;
        x.x = r[4 * m];
        x.y = r[4 * m + 1];
        x.z = r[4 * m + 2];
        x.w = r[4 * m + 3];
        *(u32x4*)&t[4 * (64 * m + lane)] = x;
    }
}

template <int N, int REG>
__device__ inline void store_narrow(const uint32_t (&r)[REG], uint32_t* t, int lane) {
#pragma unroll
    for (int m = 0; m < N; ++m) t[64 * m + lane] = r[m];
}

__device__ inline float xchg16(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}

__device__ inline float xchg32(float x, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, x)));
}

// ---------------------------------------------------------------------------
// The decode kernel.  For one KV head, the G query heads of its group against
// 16 rows are a (16 x D) by (D x G) product for the scores and a (D x 16) by
// (16 x G) product for the values, both dense; they run on MFMA with G padded
// to 16 ("F5 -- Advanced KV Cache Techniques", M3 What shipped: the query
// heads of a GQA group share every K/V row they read).  On the vector units
// alone (no packed fp32 here) the int8 conversions and fp32 multiply-adds of
// a sub-tile took longer than its transfer from HBM.
//
// Lanes: n = lane % 16, gq = lane / 16.  A 16x16 MFMA result leaves element
// (4 gq + j, n) in register j of lane (gq, n); its first operand takes row n
// from lane (gq, n) and its second operand column n, both over the k-slots of
// lane group gq (the same slots in both, so which k sits in which slot is
// this code's choice).
//   * Scores, per q8_0 block b: S_b[row][head] = sum over the block's 32 dims
//     of code[row][dim] * q'[head][dim], a 16x16x32 f16 product per query part:
//     lane (gq, n) gives the codes of row n at dims 32 b + 8 gq .. + 7
//     (binary16 holds every int8 code exactly) and q' of head n at the same
//     dims.  The query is fp32 and enters as two binary16 parts, hi = f16(q')
//     and lo = f16(q' - hi); their products with the codes are exact and add
//     up in fp32, so the score keeps about 22 significant bits of the query.
//     q' = q * scale * log2(e) * 2^(15 - E), E per head such that the largest
//     |q'| lies in [2^14, 2^15): neither part overflows or runs out of range.
//     Lane (gq, n) then holds rows 4 gq + j of head n and applies their block
//     scales: S = 2^(E - 15) sum_b dk_b S_b, in log2 units.
//   * Softmax: lane (gq, n) keeps the running maximum, the sum and the output
//     of head n.  The four lane groups of a head exchange their maxima
//     (ds_swizzle, ds_bpermute) only when a score passes the maximum by more
//     than kLazyMax.
//   * Values, per block b and half c: O[dim][head] += sum over the 16 rows of
//     code[row][dim] * (p[row][head] * dv[row][b]), a 16x16x16 bf16 product
//     whose second operand has the score layout (rows 4 gq + j of head n in
//     lane (gq, n)), so the weights never move between lanes.  They enter as
//     two bfloat16 parts (about 17 significant bits; bfloat16 has the fp32
//     exponent range, which binary16 lacks for a weight times an arbitrary
//     binary16 scale).  q8_0: MFMA row i of half c is dim 32 b + 2 i + c (a lane
//     reads one 2-byte pair per row and block); q4_0: dims 32 b + i and
//     32 b + 16 + i (the two nibbles of byte i), accumulated as the low nibble
//     and the whole byte (low + 16 high), the offset of 8 taken off through
//     the sum of the weights.
// Loads: a sub-tile of one KV head (16 or 32 rows x 34 D / 32 bytes) is read
// in 16-byte units over consecutive rows (or in dwords where a base or row
// stride is not a multiple of 16 bytes), one unit per lane per instruction,
// and copied to a wave-private LDS tile in the same order; the next sub-tile
// is in flight in registers while this one is computed.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Byte N of w as a signed integer, converted to binary16 (exact) by an SDWA
// byte select: into the low half of a new register (high half zero), or into
// the high half of d (low half kept).
template <int N>
__device__ __forceinline__ uint32_t i8_f16_lo(uint32_t w);
template <int N>
__device__ __forceinline__ void i8_f16_hi(uint32_t& d, uint32_t w);
#define KVD_I8_F16_LO(N)                                                                                    \
    template <>                                                                                              \
    __device__ __forceinline__ uint32_t i8_f16_lo<N>(uint32_t w) {                                           \
        uint32_t d;                                                                                          \
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_0 dst_unused:UNUSED_PAD src0_sel:BYTE_" #N         \
            : "=v"(d)                                                                                        \
            : "v"(w));                                                                                       \
        return d;                                                                                            \
    }
#define KVD_I8_F16_HI(N)                                                                                    \
    template <>                                                                                              \
    __device__ __forceinline__ void i8_f16_hi<N>(uint32_t & d, uint32_t w) {                                 \
        asm("v_cvt_f16_i16_sdwa %0, sext(%1) dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:BYTE_" #N    \
            : "+v"(d)                                                                                        \
            : "v"(w));                                                                                       \
    }
// (a pair starts on an even byte: low halves take bytes 0 and 2, high halves 1 and 3)
KVD_I8_F16_LO(0)
KVD_I8_F16_LO(2)
KVD_I8_F16_HI(1)
KVD_I8_F16_HI(3)
#undef KVD_I8_F16_LO
#undef KVD_I8_F16_HI

// Codes 2 P and 2 P + 1 of the 8 that start S bytes into z[0], as a binary16 pair.
template <int S, int P>
__device__ __forceinline__ uint32_t code_pair_f16(const uint32_t (&z)[3]) {
    constexpr int i0 = S + 2 * P, i1 = i0 + 1;
    uint32_t d = i8_f16_lo<i0 % 4>(z[i0 / 4]);
    i8_f16_hi<i1 % 4>(d, z[i1 / 4]);
    return d;
}

// The 8 K codes of a lane (S bytes into the LDS dword at zp) as the f16
// operand of a 16x16x32 product.
template <int S>
__device__ __forceinline__ half8_t kcodes_f16(const uint32_t* zp) {
    uint32_t z[3];
    z[0] = zp[0];
    z[1] = zp[1];
    z[2] = S ? zp[2] : 0u;
    const u32x4 h = {code_pair_f16<S, 0>(z), code_pair_f16<S, 1>(z), code_pair_f16<S, 2>(z),
                     code_pair_f16<S, 3>(z)};
    return __builtin_bit_cast(half8_t, h);
}

// Two floats as a bfloat16 pair (round to nearest even), x0 in the low half.
__device__ __forceinline__ uint32_t bf16_pair(float x0, float x1) {
    const float2_t v = {x0, x1};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// binary16 in the low (HI = 0) or high half of w, to fp32.
template <int HI>
__device__ __forceinline__ float f16_half(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(HI ? (w >> 16) : (w & 0xffffu)));
}

// The leading arguments (14 dwords: the counts, the query and the first
// sequence's first segment) are preloaded into SGPRs when the waves start (the
// file is built with kernel-argument preloading), so the first split segment
// of a one-sequence launch issues its query and K/V loads without reading its
// arguments from memory: they sit in memory that the step's K/V stream has
// evicted from every cache since the layer's previous call.  Everything else
// comes from the LaunchArgs block, read while the first sub-tile is in flight.
// kv_seq packs n_head_kv (low 16 bits) and the launch's sequence count.
// WIDE: 0 = dword loads, staged in registers; 1 = 16-byte loads, staged in
// registers; 2 = 16-byte loads straight into two LDS tiles per wave (double
// buffered), for the plans with at most 8 waves per CU.
template <int D, int G, int VT, int WIDE, int W>
__global__ void __launch_bounds__(64 * W)
decode_kernel(const int32_t n_items, const int32_t kv_seq, const int32_t split_rows, const int32_t n_split0,
                   const float* q, const uint8_t* k0, const uint8_t* v0, const int32_t stride0,
                   const int32_t vstride0, const int32_t row_lo0, const int32_t n_rows0, const LaunchArgs A) {
    using L_ = Lay<D, VT>;
    using WL = WaveLds<D, G, VT, WIDE == 2 ? 2 : 1>;
    constexpr int NB = L_::NB, R = L_::R, PK = L_::PK, PV = L_::PV, CB = L_::CB, CBV = L_::CBV, VB = L_::VB;
    constexpr int KW = L_::KW, VW = L_::VW, KN = L_::KN, VN = L_::VN;
    constexpr int RS = R / 16;  // 16-row groups of a sub-tile
    static_assert(G <= 16, "one MFMA column per query head of the group");
    __shared__ __attribute__((aligned(16))) uint32_t s_lds[W][WL::DWORDS];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n_head_kv = kv_seq & 0xffff, n_seq = kv_seq >> 16;
    // the grid is n_items rounded up to a multiple of 8 (one run per XCD)
    const int item = (blockIdx.x & 7) * ((n_items + 7) >> 3) + (blockIdx.x >> 3);
    if (item >= n_items) return;
    const int lsplit = item / n_head_kv;
    const int g = item - lsplit * n_head_kv;
    int s = 0, so = 0, sp = lsplit, seg = 0;  // slot, its sequence's q / out index, split, segment
    SegDesc SG;
    SG.k = k0;
    SG.v = v0;
    SG.stride = stride0;
    SG.vstride = vstride0;
    SG.row_lo = row_lo0;
    SG.n_rows = n_rows0;
    if (n_seq > 1 || lsplit >= n_split0) {
        // Another sequence or the second segment: the slot from one load of
        // every slot's first split, then the slot's two segment descriptors
        // read together and one picked, so that any slot waits on two round
        // trips to the argument memory before its first K/V load.  (A search
        // slot by slot waited on one per slot passed: 16 sequences of 250
        // rows 12.1 -> 9.9 us per call, 16 of 1024 rows 19.9 -> 15.9, 16 of
        // 4096 rows 38.7 -> 37.0.)
        if (n_seq > 1) {
#pragma unroll
            for (int j = 1; j < kMaxSeqPerLaunch; ++j)  // + 1 where slot_split[j] <= lsplit (both in [0, 2^31))
                s += (int)(((uint32_t)A.slot_split[j] - (uint32_t)lsplit - 1u) >> 31);
        }
        const SeqDesc& d = A.seq[s];
        const SegDesc& d0 = d.seg[0];
        const SegDesc& d1 = d.seg[1];
        const uint8_t *k0_ = d0.k, *v0_ = d0.v, *k1_ = d1.k, *v1_ = d1.v;
        const int32_t st0 = d0.stride, vs0 = d0.vstride, lo0 = d0.row_lo, nr0 = d0.n_rows, ns0 = d0.n_split;
        const int32_t st1 = d1.stride, vs1 = d1.vstride, lo1 = d1.row_lo, nr1 = d1.n_rows;
        const int32_t base = d.split_base;
        so = d.orig;
        asm volatile("" ::"s"(k0_), "s"(v0_), "s"(k1_), "s"(v1_), "s"(st0), "s"(vs0), "s"(lo0), "s"(nr0), "s"(ns0),
                     "s"(st1), "s"(vs1), "s"(lo1), "s"(nr1), "s"(base), "s"(so));
        sp = lsplit - base;
        seg = sp >= ns0 ? 1 : 0;
        sp -= seg ? ns0 : 0;
        SG.k = seg ? k1_ : k0_;
        SG.v = seg ? v1_ : v0_;
        SG.stride = seg ? st1 : st0;
        SG.vstride = seg ? vs1 : vs0;
        SG.row_lo = seg ? lo1 : lo0;
        SG.n_rows = seg ? nr1 : nr0;
        asm volatile("" ::"s"(SG.k), "s"(SG.v), "s"(SG.stride), "s"(SG.vstride), "s"(SG.row_lo), "s"(SG.n_rows), "s"(so));
    }
    const int r_begin = SG.row_lo + sp * split_rows;
    const int n_head_q = n_head_kv * G;

    const int n = lane & 15;   // MFMA row / column of the lane
    const int gq = lane >> 4;  // lane group: k-slots, and rows 4 gq .. 4 gq + 3 of a result

    // Loads.  WIDE: the launch's K/V bases and row strides are 16-byte
    // multiples, and a sub-tile is read in 16-byte units from the boundary
    // below each row's head chunk (`lead` bytes before it, a multiple of 4).
    // The buffer range check is per dword: the units of the segment's last
    // readable row that run past its chunk (always a whole number of dwords)
    // read zeros there and touch nothing beyond it.  Else the sub-tile is read
    // in dwords from the chunk start.  Both fill the same LDS layout.  (q8_0 V
    // rows have the K geometry and share the K offsets.)
    const int klead = WIDE ? (g * CB) & 15 : 0;
    const int vlead = WIDE ? (g * CBV) & 15 : 0;
    constexpr int KO = WIDE ? KW : KN, VO = WIDE ? VW : VN;
    int32_t koff[KO], voff[VO];
    if constexpr (WIDE) {
        wide_offsets<KW, RowUnits<CB>::UR, L_::KUW>(koff, lane, SG.stride);
        if constexpr (VT) wide_offsets<VW, RowUnits<CBV>::UR, L_::VUW>(voff, lane, SG.vstride);
    } else {
        narrow_offsets<KN, PK, R * PK>(koff, lane, SG.stride);
        if constexpr (VT) narrow_offsets<VN, PV, R * PV>(voff, lane, SG.vstride);
    }
    if constexpr (!VT) {
#pragma unroll
        for (int m = 0; m < KO; ++m) voff[m] = koff[m];
    }
    uint32_t rk[WIDE ? 4 * KW : KN], rv[WIDE ? 4 * VW : VN];
    // 4-wave workgroups of small calls (at most two per CU: loads straight
    // into LDS, or dword loads) stream K/V non-temporally, which leaves the
    // small data a call reuses (query, split partials) in the caches: 8.70 ->
    // 8.53 us per 4096-row call.  The other plans keep the default policy:
    // there a line that straddles two KV heads is read by two workgroups of
    // one XCD, and non-temporal loads made the second one miss (131072 rows:
    // 58.2 -> 63.2 us; 16 sequences of 1024 ... 10041 rows, three 4-wave
    // workgroups per CU with register staging: 47.6 -> 48.6 us).
    constexpr int AUX = (W == 4 && WIDE != 1) ? kLoadNonTemporal : 0;
    auto lds_k = [&](int r0, uint32_t* t) {  // WIDE == 2
        const __amdgpu_buffer_rsrc_t kr = sub_rsrc(SG.k, SG.stride, SG.n_rows, CB, g, klead, r0);
#pragma unroll
        for (int m = 0; m < KW; ++m) load_lds16<AUX>(kr, t + 256 * m, koff[m]);
    };
    auto lds_v = [&](int r0, uint32_t* t) {
        const __amdgpu_buffer_rsrc_t vr = sub_rsrc(SG.v, SG.vstride, SG.n_rows, CBV, g, vlead, r0);
#pragma unroll
        for (int m = 0; m < VW; ++m) load_lds16<AUX>(vr, t + 256 * m, voff[m]);
    };
    auto issue_k = [&](int r0) {
        const __amdgpu_buffer_rsrc_t kr = sub_rsrc(SG.k, SG.stride, SG.n_rows, CB, g, klead, r0);
        if constexpr (WIDE)
            load_wide<KW, 4 * KW, AUX>(rk, kr, koff);
        else
            load_narrow<KN, KN, AUX>(rk, kr, koff);
    };
    auto issue_v = [&](int r0) {
        const __amdgpu_buffer_rsrc_t vr = sub_rsrc(SG.v, SG.vstride, SG.n_rows, CBV, g, vlead, r0);
        if constexpr (WIDE)
            load_wide<VW, 4 * VW, AUX>(rv, vr, voff);
        else
            load_narrow<VN, VN, AUX>(rv, vr, voff);
    };
    // the query first: its two parts are computed while the first sub-tile is in flight
    float qv[NB][8];
    {
        // q of head n at dims 32 b + 8 gq .. + 7 (zero for the padding columns)
        const bool real = n < G;
        const float* qp = q + ((size_t)so * n_head_q + (size_t)g * G + (real ? n : 0)) * D + 8 * gq;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const float4 a = *(const float4*)(qp + 32 * b);
            const float4 c = *(const float4*)(qp + 32 * b + 4);
            qv[b][0] = a.x, qv[b][1] = a.y, qv[b][2] = a.z, qv[b][3] = a.w;
            qv[b][4] = c.x, qv[b][5] = c.y, qv[b][6] = c.z, qv[b][7] = c.w;
#pragma unroll
            for (int j = 0; j < 8; ++j) qv[b][j] = real ? qv[b][j] : 0.f;
        }
    }
    if constexpr (WIDE == 2) {
        lds_k(r_begin + wave * R, s_lds[wave]);
        lds_v(r_begin + wave * R, s_lds[wave] + WL::K);
    } else {
        issue_k(r_begin + wave * R);
        issue_v(r_begin + wave * R);
    }
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
    const int n_sub = (r_end - r_begin + R - 1) / R;
    const bool single = seq_splits == 1;
    const int abs_split = split_off + lsplit;

    // the query in log2 units, scaled by a power of two per head, as two binary16 parts
    half8_t qh[NB], ql[NB];
    float unscale, rescale;  // 2^(E - 15) and 2^(15 - E) for head n
    {
        float amax = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                qv[b][j] *= scale_log2e;
                amax = fmaxf(amax, fabsf(qv[b][j]));
            }
        }
        amax = fmaxf(amax, xchg16(amax));
        amax = fmaxf(amax, xchg32(amax, lane));
        int e = __builtin_amdgcn_frexp_expf(amax);  // amax = f 2^e, f in [0.5, 1); 0 for 0, inf, nan
        e = min(max(e, -100), 120);
        rescale = __builtin_ldexpf(1.f, 15 - e);
        unscale = __builtin_ldexpf(1.f, e - 15);
        // hi = q' rounded toward zero to binary16 (x - hi is then exact in
        // fp32), lo = the rest rounded the same way: |q' - hi - lo| < 2^-20 |q'|
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                const float x0 = qv[b][j] * rescale, x1 = qv[b][j + 1] * rescale;
                const auto hi = __builtin_amdgcn_cvt_pkrtz(x0, x1);
                const auto lo = __builtin_amdgcn_cvt_pkrtz(x0 - (float)hi[0], x1 - (float)hi[1]);
                qh[b][j] = hi[0];
                qh[b][j + 1] = hi[1];
                ql[b][j] = lo[0];
                ql[b][j + 1] = lo[1];
            }
        }
    }

    uint32_t* tk = s_lds[wave];  // this sub-tile's K and V tiles
    uint32_t* tv = s_lds[wave] + WL::K;
    uint32_t* nk = s_lds[wave] + (WIDE == 2 ? WL::K + WL::V : 0);  // WIDE == 2: the other pair

    float m = -INFINITY, l = 0.f, thr = -INFINITY;
    float cs[NB];  // q4_0: sum of the weights per block
    float4_t o[NB][2];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        cs[b] = 0.f;
        o[b][0] = o[b][1] = (float4_t){0.f, 0.f, 0.f, 0.f};
    }

    for (int t = wave; t < n_sub; t += W) {
        const int row0 = r_begin + t * R;
        const int nv = min(R, r_end - row0);
        {
            // Issue priority grows with the sub-tiles this wave has left.  The
            // SIMD otherwise favours its oldest waves, and the first
            // workgroups placed on a CU ran ahead and finished early, leaving
            // the last ones to run at low occupancy.
            const int rem = (n_sub - t + W - 1) / W;
            if (rem > 8)
                __builtin_amdgcn_s_setprio(3);
            else if (rem > 4)
                __builtin_amdgcn_s_setprio(2);
            else if (rem > 2)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        }
        // K is staged before the scores and V only after them, so the scores
        // start once K has landed and V arrives meanwhile; each register set
        // takes the next sub-tile's loads as soon as it is copied out.  With
        // loads straight into LDS the next sub-tile's K and V go to the other
        // pair of tiles first, and the waits count the loads still allowed in
        // flight: K(t), V(t), K(next), V(next) were issued in that order.
        const bool more = t + W < n_sub;
        if constexpr (WIDE == 2) {
            if (more) {
                lds_k(row0 + W * R, nk);
                lds_v(row0 + W * R, nk + WL::K);
                wait_vm<VW + KW + VW>();
            } else {
                wait_vm<VW>();
            }
        } else {
            if constexpr (WIDE)
                store_wide<KW>(rk, tk, lane);
            else
                store_narrow<KN>(rk, tk, lane);
            if (more) issue_k(row0 + W * R);
        }
        wave_lds_sync();

#pragma unroll
        for (int rs = 0; rs < RS; ++rs) {
            // ---- scores of rows 16 rs + 4 gq + j, head n
            float sc[4];
            {
                const uint32_t* const kc = tk + (16 * rs + n) * PK + (klead >> 2) + 2 * gq;
                const uint32_t* const ks = tk + (16 * rs + 4 * gq) * PK + (klead >> 2);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    // block b: scale at byte 34 b, codes from byte 34 b + 2
                    const uint32_t* const zp = kc + ((34 * b + 2) >> 2);
                    const half8_t a = (b & 1) ? kcodes_f16<0>(zp) : kcodes_f16<2>(zp);
                    float4_t acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, ql[b], (float4_t){0.f, 0.f, 0.f, 0.f},
                                                                          0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[b], acc, 0, 0, 0);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t w = ks[j * PK + ((34 * b) >> 2)];
                        const float dk = (b & 1) ? f16_half<1>(w) : f16_half<0>(w);
                        sc[j] = (b == 0) ? dk * acc[j] : fmaf(dk, acc[j], sc[j]);
                    }
                }
            }
            if (nv < R) {
                // only a split's last sub-tile can be partial
#pragma unroll
                for (int j = 0; j < 4; ++j) sc[j] = (16 * rs + 4 * gq + j < nv) ? sc[j] : -INFINITY;
            }
            // ---- online softmax
            {
                const float smax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
                if (__builtin_amdgcn_ballot_w64(smax > thr)) {
                    float x = fmaxf(smax, xchg16(smax));
                    x = fmaxf(x, xchg32(x, lane));
                    const float mn = fmaxf(m, x * unscale);
                    const float alpha = __builtin_amdgcn_exp2f(m - mn);
                    l *= alpha;
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        if (VT) cs[b] *= alpha;
                        o[b][0] *= alpha;
                        o[b][1] *= alpha;
                    }
                    m = mn;
                    thr = (m + kLazyMax) * rescale;
                }
            }
            float p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                p[j] = __builtin_amdgcn_exp2f(fmaf(sc[j], unscale, -m));
                l += p[j];
            }
            // ---- values
            if (rs == 0) {
                if constexpr (WIDE == 2) {
                    if (more)
                        wait_vm<KW + VW>();
                    else
                        wait_vm<0>();
                } else {
                    if constexpr (WIDE)
                        store_wide<VW>(rv, tv, lane);
                    else
                        store_narrow<VN>(rv, tv, lane);
                    if (more) issue_v(row0 + W * R);
                }
                wave_lds_sync();
            }
            const uint32_t* const vs = tv + (16 * rs + 4 * gq) * PV + (vlead >> 2);
            const uint8_t* const vc =
                (const uint8_t*)(tv + (16 * rs + 4 * gq) * PV) + vlead + 2 + (VT ? n : 2 * n);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                float x[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t w = vs[j * PV + ((VB * b) >> 2)];
                    const float dv = (b & 1) ? f16_half<1>(w) : f16_half<0>(w);
                    x[j] = p[j] * dv;
                }
                if (nv < R) {
                    // rows past the visible range may hold any bits: their weight is an exact 0
#pragma unroll
                    for (int j = 0; j < 4; ++j) x[j] = (16 * rs + 4 * gq + j < nv) ? x[j] : 0.f;
                }
                if constexpr (VT) cs[b] += (x[0] + x[1]) + (x[2] + x[3]);
                // the weights as bfloat16 hi + lo parts
                const uint32_t h01 = bf16_pair(x[0], x[1]), h23 = bf16_pair(x[2], x[3]);
                const uint32_t l01 = bf16_pair(x[0] - __builtin_bit_cast(float, h01 << 16),
                                               x[1] - __builtin_bit_cast(float, h01 & 0xffff0000u));
                const uint32_t l23 = bf16_pair(x[2] - __builtin_bit_cast(float, h23 << 16),
                                               x[3] - __builtin_bit_cast(float, h23 & 0xffff0000u));
                const short4_t wh = __builtin_bit_cast(short4_t, (uint2){h01, h23});
                const short4_t wl = __builtin_bit_cast(short4_t, (uint2){l01, l23});
                float f[2][4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (VT == 0) {
                        uint32_t y = *(const uint16_t*)(vc + j * 4 * PV + VB * b);
                        asm("" : "+v"(y));
                        f[0][j] = (float)(int8_t)y;
                        f[1][j] = (float)(int8_t)(y >> 8);
                    } else {
                        uint32_t y = vc[j * 4 * PV + VB * b];
                        asm("" : "+v"(y));
                        f[0][j] = (float)(y & 15u);
                        f[1][j] = (float)(uint8_t)y;
                    }
                }
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const short4_t a =
                        __builtin_bit_cast(short4_t, (uint2){bf16_pair(f[c][0], f[c][1]), bf16_pair(f[c][2], f[c][3])});
                    o[b][c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, wl, o[b][c], 0, 0, 0);
                    o[b][c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, wh, o[b][c], 0, 0, 0);
                }
            }
        }
        wave_lds_sync();
        if constexpr (WIDE == 2) {
            uint32_t* const x = tk;
            tk = nk;
            tv = nk + WL::K;
            nk = x;
        }
    }

    // ---- this wave's (m, l, o) to its LDS area, then the four waves merge
    // (a wave with no sub-tile still has its first loads landing in that area)
    if constexpr (WIDE == 2) wait_vm<0>();
    l += xchg16(l);
    l += xchg32(l, lane);
    if constexpr (VT) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            cs[b] += xchg16(cs[b]);
            cs[b] += xchg32(cs[b], lane);
        }
    }
    constexpr int OFF = WL::OFF_O;
    float* const mw = (float*)s_lds[wave];  // m [G], l [G], o [G][D] from OFF
    if (n < G) {
        if (gq == 0) {
            mw[n] = m;
            mw[G + n] = l;
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 4 * gq + j;  // MFMA row of the result
                if constexpr (VT == 0) {
                    mw[OFF + n * D + 32 * b + 2 * i] = o[b][0][j];
                    mw[OFF + n * D + 32 * b + 2 * i + 1] = o[b][1][j];
                } else {
                    // low nibbles and whole bytes -> dims i and i + 16, codes offset by 8
                    const float lo = o[b][0][j], hi = (o[b][1][j] - lo) * 0.0625f;
                    mw[OFF + n * D + 32 * b + i] = lo - 8.f * cs[b];
                    mw[OFF + n * D + 32 * b + 16 + i] = hi - 8.f * cs[b];
                }
            }
        }
    }
    __syncthreads();
    // the W states merged per 4 consecutive dims of a head, in wave order
    const int hq0 = g * G;
    for (int c = threadIdx.x; c < G * D / 4; c += 64 * W) {
        const int h = (4 * c) / D, d = 4 * c - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, ((const float*)s_lds[w])[h]);
        float L = 0.f;
        float4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float* mw2 = (const float*)s_lds[w];
            const float mk = mw2[h];
            const float a = (mk == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mk - M);
            const float4 x = *(const float4*)&mw2[OFF + h * D + d];
            L = fmaf(a, mw2[G + h], L);
            O.x = fmaf(a, x.x, O.x);
            O.y = fmaf(a, x.y, O.y);
            O.z = fmaf(a, x.z, O.z);
            O.w = fmaf(a, x.w, O.w);
        }
        if (single && part_o) {
            const size_t sh = (size_t)so * n_head_q + hq0 + h;
            *(float4*)&part_o[sh * D + d] = O;
            if (d == 0) {
                part_m[sh] = M;
                part_l[sh] = L;
            }
        } else if (single) {
            const float4 r = {O.x / L, O.y / L, O.z / L, O.w / L};
            *(float4*)&out[((size_t)so * n_head_q + hq0 + h) * D + d] = r;
        } else {
            const size_t pi = (size_t)abs_split * n_head_q + hq0 + h;
            *(float4*)&po[pi * D + d] = O;
            if (d == 0) {
                pm[pi] = M;
                pl[pi] = L;
            }
        }
    }
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

// Merge the split partials of one (sequence, query head, 32 dims): one
// single-wave workgroup each, so a call's merge spreads over D / 32 times
// more CUs than one workgroup per (sequence, query head) would (4096 rows:
// 9.4 -> 8.8 us per call).  A separate launch, so the partials written by the
// decode kernel are visible without cache maintenance inside a kernel.
// Leading arguments preloaded into SGPRs as in the decode kernel: the first
// slot's split count and sequence index and the partials, so the partial
// loads of a one-sequence launch start without reading its arguments from
// memory.  Slot s merges the sequence the host put there (LaunchArgs.seq[s]).
template <int D>
__global__ void __launch_bounds__(64)
combine_kernel(const int32_t n_head_q, const int32_t split_off, const int32_t n_split0, const int32_t orig0,
               const float* ppm, const float* ppl, const float* ppo, const LaunchArgs A) {
    constexpr int NWV = D / 32;
    __shared__ float s_o[64][33];
    const int lane = threadIdx.x;
    const int wave = blockIdx.x % NWV;  // the 32-dim slice of this workgroup
    const int hq = (blockIdx.x / NWV) % n_head_q;
    const int s = blockIdx.x / NWV / n_head_q;
    int32_t S = n_split0, base = 0, so = orig0;  // slot 0 starts the launch's splits
    if (s > 0) {
        S = A.seq[s].n_split;
        base = A.seq[s].split_base;
        so = A.seq[s].orig;
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
    merge_rows(load, read_outputs, S, lane, s_o, O, M, L);
    if (lane < 32) write_final(A, D, (size_t)so * n_head_q + hq, 32 * wave + lane, O, M, L, wave == 0 && lane == 0);
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

// Test support for the staging ring: one wave that holds its stream for
// about `ticks` ticks of the 100 MHz real-time counter, by polling it with
// sleeps in between; the loop also ends after 2^22 polls whatever the
// counter says.
__global__ void __launch_bounds__(64) spin_kernel(uint32_t ticks) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (uint32_t i = 0; i < (1u << 22); ++i) {
        if (__builtin_amdgcn_s_memrealtime() - t0 >= ticks) break;
        __builtin_amdgcn_s_sleep(8);
    }
}

typedef void (*decode_fn)(int32_t, int32_t, int32_t, int32_t, const float*, const uint8_t*, const uint8_t*, int32_t,
                          int32_t, int32_t, int32_t, const LaunchArgs);
typedef void (*combine_fn)(int32_t, int32_t, int32_t, int32_t, const float*, const float*, const float*, const LaunchArgs);

combine_fn pick_combine(int D) { return D == 128 ? combine_kernel<128> : combine_kernel<64>; }

template <int D, int VT, int WIDE, int W>
decode_fn pick_decode_g(int G) {
    switch (G) {
        case 1: return decode_kernel<D, 1, VT, WIDE, W>;
        case 2: return decode_kernel<D, 2, VT, WIDE, W>;
        case 3: return decode_kernel<D, 3, VT, WIDE, W>;
        case 4: return decode_kernel<D, 4, VT, WIDE, W>;
        case 5: return decode_kernel<D, 5, VT, WIDE, W>;
        case 6: return decode_kernel<D, 6, VT, WIDE, W>;
        case 7: return decode_kernel<D, 7, VT, WIDE, W>;
        case 8: return decode_kernel<D, 8, VT, WIDE, W>;
    }
    return nullptr;
}

template <int WIDE, int W>
decode_fn pick_decode_w(int D, int G, int VT) {
    if (VT) return D == 128 ? pick_decode_g<128, 1, WIDE, W>(G) : pick_decode_g<64, 1, WIDE, W>(G);
    return D == 128 ? pick_decode_g<128, 0, WIDE, W>(G) : pick_decode_g<64, 0, WIDE, W>(G);
}

// wide: the load mode (the kernel's WIDE); waves: 4, 8 or 12 per workgroup.
// Built: every mode for 4 waves, dword and LDS-direct loads for 8, dword and
// register-staged 16-byte loads for 12 (the modes the launch picks).
decode_fn pick_decode(int D, int G, int VT, int wide, int waves) {
    switch (waves) {
        case 4:
            return wide == 2 ? pick_decode_w<2, 4>(D, G, VT)
                 : wide == 1 ? pick_decode_w<1, 4>(D, G, VT)
                             : pick_decode_w<0, 4>(D, G, VT);
        case 8:
            return wide == 2 ? pick_decode_w<2, 8>(D, G, VT) : wide == 0 ? pick_decode_w<0, 8>(D, G, VT) : nullptr;
        case 12:
            return wide == 1 ? pick_decode_w<1, 12>(D, G, VT) : wide == 0 ? pick_decode_w<0, 12>(D, G, VT) : nullptr;
    }
    return nullptr;
}

}  // namespace
}  // namespace kvd

using namespace kvd;

namespace kvd {
namespace {

constexpr int kMaxDevices = 64;

// Compute units of the current device, asked once per device (the split plan
// is made for them, so it stays a function of the shapes on a given device).
// Where no device answers (a host without a GPU planning a workspace size) the
// plan is made for MI355X's count.
int device_cus() {
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kDefaultCUs;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1 || n > 4096) {
        (void)hipGetLastError();
        return kDefaultCUs;
    }
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace
}  // namespace kvd

namespace kvd {
hipError_t launch_spin(hipStream_t stream, uint32_t us) {
    hipLaunchKernelGGL(spin_kernel, dim3(1), dim3(64), 0, stream, us * 100u);
    return hipGetLastError();
}
}  // namespace kvd

namespace kvd {
namespace {

// Every K/V base and row stride of the call is a multiple of 16 bytes (the
// 16-byte load modes need it).
bool wide_segments(const kvd_attn_args* a) {
    for (size_t i = 0; i < (size_t)a->n_seq * a->n_seg; ++i) {
        const kvd_kv_seg& g = a->segs[i];
        const int64_t vs = g.v_row_stride ? g.v_row_stride : g.row_stride;
        if (g.n_rows > 0 && (((uintptr_t)g.k | (uintptr_t)g.v) % 16 || g.row_stride % 16 || vs % 16)) return false;
    }
    return true;
}

// The decode kernel's load mode (its WIDE argument) for a launch of n_items
// workgroups.  16-byte loads go straight into LDS where a CU runs at most 8
// waves (8-wave workgroups, or 4-wave ones at most two per CU): 4096 rows
// 8.45 -> 8.25 us per call, 16384 rows 14.1 -> 13.5, 32768 rows 21.3 ->
// 20.2.  With 12 waves per CU, register staging is faster (131072 rows 58.5
// against 59.9 us; the 16-sequence batch's three 4-wave workgroups per CU
// 48.7 against 50.6).
int load_mode(bool wide, int waves, int64_t n_items, int n_cus) {
    if (!wide) return 0;
    return (waves == 8 || (waves == 4 && n_items <= 2 * (int64_t)n_cus)) ? 2 : 1;
}

}  // namespace
}  // namespace kvd

extern "C" int kvd_attend_workspace_bytes(const kvd_attn_args* args, size_t* bytes) {
    clear_error();
    if (!bytes) return fail(KVD_EINVAL, "bytes is NULL");
    AttendPlan p;
    const int rc = plan_attend(args, &p, device_cus());
    if (rc != KVD_OK) return rc;
    *bytes = p.ws_bytes;
    return KVD_OK;
}

extern "C" int kvd_attend_plan(const kvd_attn_args* args, int32_t* split_rows, int32_t* waves,
                               int64_t* total_splits) {
    clear_error();
    AttendPlan p;
    const int rc = plan_attend(args, &p, device_cus());
    if (rc != KVD_OK) return rc;
    if (split_rows) *split_rows = p.split_rows;
    if (waves) *waves = p.waves;
    if (total_splits) *total_splits = p.total_splits;
    return KVD_OK;
}

extern "C" int kvd_attend_load_mode(const kvd_attn_args* args, int32_t* mode) {
    clear_error();
    if (!mode) return fail(KVD_EINVAL, "mode is NULL");
    AttendPlan p;
    const int rc = plan_attend(args, &p, device_cus());
    if (rc != KVD_OK) return rc;
    const int ns = args->n_seq < kMaxSeqPerLaunch ? args->n_seq : kMaxSeqPerLaunch;  // the first launch
    int64_t nsplit = 0;
    for (int j = 0; j < ns; ++j) nsplit += p.seq[j].n_split;
    *mode = load_mode(wide_segments(args), p.waves, nsplit * args->n_head_kv, p.n_cus);
    return KVD_OK;
}

namespace kvd {
namespace {

// Shared by the normal and the partial-result entry points: `part` null ->
// write out; else write (o, m, l) at part (layout of merge_kernel's input).
int launch_attend(const kvd_attn_args* a, void* stream, float* part) {
    AttendPlan p;
    int rc = plan_attend(a, &p, device_cus());
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
    const bool wide = wide_segments(a);
    const combine_fn ck = pick_combine(a->head_dim);

    uint8_t* ws = (uint8_t*)a->workspace;
    const int D = a->head_dim;
    const int n_head_q = a->n_head_q;
    const float scale_log2e = (float)((double)a->scale * 1.4426950408889634);

    for (int s0 = 0; s0 < a->n_seq; s0 += kMaxSeqPerLaunch) {
        const int ns = (a->n_seq - s0 < kMaxSeqPerLaunch) ? a->n_seq - s0 : kMaxSeqPerLaunch;
        LaunchArgs L;
        memset(&L, 0, sizeof(L));
        const int64_t base0 = p.seq[s0].split_base;
        // Slots in order of visible rows, longest first (ties in sequence
        // order): each XCD then starts its CUs on whole splits and ends on
        // the short last ones (16 sequences of 1024 ... 10041 rows: 55.1-57.5
        // -> 52.4-53.6 us per call).  A sequence's arithmetic does not depend
        // on its slot, so the outputs do not either.
        int order[kMaxSeqPerLaunch];
        for (int j = 0; j < ns; ++j) order[j] = j;
        auto vis = [&](int j) { return (int64_t)p.seq[s0 + j].seg[0].n_vis + p.seq[s0 + j].seg[1].n_vis; };
        std::stable_sort(order, order + ns, [&](int x, int y) { return vis(x) > vis(y); });
        int64_t nsplit = 0;
        for (int j = ns; j < kMaxSeqPerLaunch; ++j) L.slot_split[j] = INT32_MAX;  // never a slot's
        for (int j = 0; j < ns; ++j) {
            const int o = order[j];
            const SeqPlan& sp = p.seq[s0 + o];
            const kvd_kv_seg* segs = a->segs + (size_t)(s0 + o) * a->n_seg;
            SeqDesc& d = L.seq[j];
            d.orig = o;
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
            d.split_base = (int32_t)nsplit;  // slot order: the splits of slot j follow those of slot j - 1
            L.slot_split[j] = d.split_base;
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
        const int mode = load_mode(wide, p.waves, L.n_items, p.n_cus);
        const decode_fn dk = pick_decode(a->head_dim, p.group, a->v_type, mode, p.waves);
        if (!dk) return fail(KVD_EINVAL, "no kernel for head_dim %d, group %d", a->head_dim, p.group);
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
            hipLaunchKernelGGL(ck, dim3((unsigned)(ns * n_head_q * (D / 32))), dim3(64), 0, (hipStream_t)stream,
                               (int32_t)n_head_q, L.split_off, L.seq[0].n_split, L.seq[0].orig, L.pm, L.pl, L.po, L);
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

// ---------------------------------------------------------------------------
// kvd_attend_decode_noalloc: the split partials in a file-scope device array
// instead of a caller's workspace, for callers that cannot allocate.  Every
// GPU the library runs on holds its own copy of `scratch` until the process
// ends; all calls on one GPU share it (overlapping calls race).  Nothing in it
// needs clearing: each split writes its own partials before the combine
// launch of the same call reads them.
constexpr size_t kNoAllocScratchBytes = 8u << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace kvd {
namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The current device's address of `scratch`, looked up on the device's first
// call.  Host code uses only this address: the array's own name on the host
// is a stand-in, not a device address.
int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        const hipError_t e = hipGetLastError();
        return fail(KVD_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(KVD_EINVAL, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return fail(KVD_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KVD_OK;
}
}  // namespace
}  // namespace kvd

extern "C" int kvd_attend_decode_noalloc(const kvd_attn_args* a, void* stream) {
    clear_error();
    AttendPlan p;
    int rc = plan_attend(a, &p, device_cus());
    if (rc != KVD_OK) return rc;
    if (p.ws_bytes > kNoAllocScratchBytes)
        return fail(KVD_EINVAL, "the split partials of this call need %zu bytes; the built-in scratch holds %zu",
                    p.ws_bytes, kNoAllocScratchBytes);
    void* ws = nullptr;
    rc = scratch_address(&ws);
    if (rc != KVD_OK) return rc;
    kvd_attn_args b = *a;
    b.workspace = ws;
    b.workspace_bytes = kNoAllocScratchBytes;
    return launch_attend(&b, stream, nullptr);
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
