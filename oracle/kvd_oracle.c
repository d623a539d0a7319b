/*
 * kvd_oracle.c -- plain, slow, fp64 CPU reference for decode attention over a
 * q8_0-quantised grouped-query KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * loads this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or table with the HIP
 * path: it has its own binary16 decoder, its own layout arithmetic and its
 * own softmax.
 *
 * What it computes (the plain definition, no blocking, no online softmax):
 *   For every sequence s and query head h, with KV head g = floor(h / G),
 *   G = n_head_q / n_head_kv:
 *     x = d * q                        (q8_0 dequantisation, exact in fp64)
 *     s_t = scale * sum_i Q[s,h,i] * K[t,g,i]      for every visible row t
 *     m   = max_t s_t
 *     out[s,h,:] = sum_t exp(s_t - m) V[t,g,:] / sum_t exp(s_t - m)
 *
 * Sources on the pages (cited by page title and section):
 *  - "sched: pipeline the delivery of a host-resident KV cache (R4)",
 *    opening paragraph: the attention a decode token pays for over a
 *    host-resident KV window; Device memory: the ring of (N + 2) slots of one
 *    layer's K+V over the whole context, and the budget that caps it.
 *  - "F5 -- Advanced KV Cache Techniques", M2 (HeadInfer), What shipped:
 *    the KV view shape [head_dim, n_head_kv, n_kv] (innermost first), i.e.
 *    token-major rows holding every KV head; M3 (NEO), What shipped: query
 *    heads sliced at gpu_heads * gqa_ratio, i.e. query head h reads KV head
 *    floor(h / gqa_ratio); M4 (ScoutAttention), step 6 and W4 Rolling KV:
 *    the online-softmax merge of partial attention results, which is
 *    exactly softmax over the union of the rows (used by the two-segment
 *    case below, which the oracle computes directly over all rows).
 *  - "Plan: lossless long context ...", llama -- sparse attention parity
 *    boundary: model-native sliding-window attention.  The pages give no
 *    formula; the reading taken is: row at position p is visible to a query
 *    at position P iff 0 <= P - p < W (exactly W rows once the context holds
 *    W tokens), and W = 0 means full causal attention (p <= P).
 *
 * Asymmetric cache ("F5 -- Advanced KV Cache Techniques", M6 (PolyKV), S0:
 * asymmetric KV compression with q8_0 K and q4_0 V, dequantised inside
 * attention): V may instead be q4_0; K stays q8_0.
 *
 * Readings where the pages are silent (q8_0 and q4_0 are only named there):
 *  - a q8_0 block is 34 bytes: a little-endian IEEE binary16 scale d at
 *    byte 0, then 32 signed int8 codes; value = d * code; no zero point.
 *  - a q4_0 block is 18 bytes: the binary16 scale d at byte 0, then 16 bytes
 *    of 4-bit codes; value j < 16 = d * (low nibble of byte j - 8), value
 *    16 + j = d * (high nibble of byte j - 8) (the ggml q4_0 block).
 *  - a row of one token holds n_head_kv heads, each head_dim / 32 blocks,
 *    in that order; rows are row_stride bytes apart.
 *  - the query is fp32, used as is (widened to fp64 exactly).
 *  - an empty visible set is an error (returns -1).
 *
 * Parity pins live in tests/test_oracle.py (closed forms, invariants,
 * brute force, exhaustive binary16 decode against numpy).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define KVD_ORACLE_QK 32          /* codes per q8_0 block            */
#define KVD_ORACLE_BLOCK_BYTES 34 /* 2-byte scale + 32 one-byte codes */

/* IEEE 754 binary16 -> binary64, from the bit fields:
 *   exponent 0      : subnormal, value = (-1)^s * m * 2^-24
 *   exponent 1..30  : normal,    value = (-1)^s * (1024 + m) * 2^(e - 25)
 *   exponent 31     : m == 0 -> infinity, else NaN                        */
double kvd_oracle_f16_to_f64(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int e = (bits >> 10) & 0x1f;
    int m = bits & 0x3ff;
    double mag;
    if (e == 0) {
        mag = ldexp((double)m, -24);
    } else if (e == 31) {
        mag = (m == 0) ? INFINITY : NAN;
    } else {
        mag = ldexp((double)(1024 + m), e - 25);
    }
    return sign ? -mag : mag;
}

/* Value number i (0 <= i < head_dim) of KV head g in one token row. */
static double q8_0_value(const uint8_t* row, int32_t head_dim, int32_t g, int32_t i) {
    const uint8_t* head = row + (size_t)g * (size_t)(head_dim / KVD_ORACLE_QK) * KVD_ORACLE_BLOCK_BYTES;
    const uint8_t* block = head + (size_t)(i / KVD_ORACLE_QK) * KVD_ORACLE_BLOCK_BYTES;
    uint16_t d_bits = (uint16_t)(block[0] | ((uint16_t)block[1] << 8)); /* little endian */
    int8_t code = (int8_t)block[2 + (i % KVD_ORACLE_QK)];
    return kvd_oracle_f16_to_f64(d_bits) * (double)code;
}

#define KVD_ORACLE_Q4_BLOCK_BYTES 18 /* 2-byte scale + 16 bytes of nibbles */

/* Value number i of KV head g in one q4_0 token row. */
static double q4_0_value(const uint8_t* row, int32_t head_dim, int32_t g, int32_t i) {
    const uint8_t* head = row + (size_t)g * (size_t)(head_dim / KVD_ORACLE_QK) * KVD_ORACLE_Q4_BLOCK_BYTES;
    const uint8_t* block = head + (size_t)(i / KVD_ORACLE_QK) * KVD_ORACLE_Q4_BLOCK_BYTES;
    uint16_t d_bits = (uint16_t)(block[0] | ((uint16_t)block[1] << 8));
    int j = i % KVD_ORACLE_QK;
    uint8_t byte = block[2 + (j % 16)];
    int nib = (j < 16) ? (byte & 0x0f) : (byte >> 4);
    return kvd_oracle_f16_to_f64(d_bits) * (double)(nib - 8);
}

/* Dequantise a whole buffer of q4_0 blocks into fp64 (n_blocks * 32 values). */
void kvd_oracle_dequant_q4_0(const uint8_t* blocks, int64_t n_blocks, double* out) {
    for (int64_t b = 0; b < n_blocks; ++b) {
        const uint8_t* block = blocks + b * KVD_ORACLE_Q4_BLOCK_BYTES;
        uint16_t d_bits = (uint16_t)(block[0] | ((uint16_t)block[1] << 8));
        double d = kvd_oracle_f16_to_f64(d_bits);
        for (int j = 0; j < 16; ++j) {
            out[b * KVD_ORACLE_QK + j] = d * (double)((block[2 + j] & 0x0f) - 8);
            out[b * KVD_ORACLE_QK + 16 + j] = d * (double)((block[2 + j] >> 4) - 8);
        }
    }
}

/* Dequantise a whole buffer of q8_0 blocks into fp64 (n_blocks * 32 values). */
void kvd_oracle_dequant_q8_0(const uint8_t* blocks, int64_t n_blocks, double* out) {
    for (int64_t b = 0; b < n_blocks; ++b) {
        const uint8_t* block = blocks + b * KVD_ORACLE_BLOCK_BYTES;
        uint16_t d_bits = (uint16_t)(block[0] | ((uint16_t)block[1] << 8));
        double d = kvd_oracle_f16_to_f64(d_bits);
        for (int j = 0; j < KVD_ORACLE_QK; ++j) out[b * KVD_ORACLE_QK + j] = d * (double)(int8_t)block[2 + j];
    }
}

typedef struct {
    const uint8_t* k;   /* host: row 0 of this segment's K rows */
    const uint8_t* v;   /* host: row 0 of this segment's V rows */
    int64_t n_rows;     /* rows in the segment */
    int64_t pos0;       /* token position of row 0 */
    int64_t row_stride; /* bytes from one row to the next */
} kvd_oracle_seg;

/* The same with separate K and V row strides (a q4_0 V row is shorter). */
typedef struct {
    const uint8_t* k;
    const uint8_t* v;
    int64_t n_rows;
    int64_t pos0;
    int64_t k_stride;
    int64_t v_stride;
} kvd_oracle_seg_kv;

#define KVD_ORACLE_V_Q8_0 0
#define KVD_ORACLE_V_Q4_0 1

static int row_visible(int64_t pos, int64_t q_pos, int32_t window) {
    if (pos > q_pos) return 0;                     /* causal */
    if (window > 0 && q_pos - pos >= window) return 0; /* sliding window */
    return 1;
}

/* One (sequence, query head): two passes over the visible rows of every
 * segment -- first the scores and their maximum, then the weighted sum. */
static int attend_one(int32_t head_dim, int32_t g, int32_t n_seg, int32_t window, double scale,
                      const float* qh, const kvd_oracle_seg_kv* segs, int32_t v_type, int64_t q_pos,
                      double* out) {
    double m = -INFINITY;
    int64_t n_visible = 0;
    for (int32_t sg = 0; sg < n_seg; ++sg) {
        const kvd_oracle_seg_kv* S = &segs[sg];
        for (int64_t t = 0; t < S->n_rows; ++t) {
            if (!row_visible(S->pos0 + t, q_pos, window)) continue;
            const uint8_t* krow = S->k + t * S->k_stride;
            double dot = 0.0;
            for (int32_t i = 0; i < head_dim; ++i) dot += (double)qh[i] * q8_0_value(krow, head_dim, g, i);
            double s = scale * dot;
            if (s > m) m = s;
            ++n_visible;
        }
    }
    if (n_visible == 0) return -1;

    double denom = 0.0;
    double* acc = (double*)calloc((size_t)head_dim, sizeof(double));
    if (!acc) return -2;
    for (int32_t sg = 0; sg < n_seg; ++sg) {
        const kvd_oracle_seg_kv* S = &segs[sg];
        for (int64_t t = 0; t < S->n_rows; ++t) {
            if (!row_visible(S->pos0 + t, q_pos, window)) continue;
            const uint8_t* krow = S->k + t * S->k_stride;
            const uint8_t* vrow = S->v + t * S->v_stride;
            double dot = 0.0;
            for (int32_t i = 0; i < head_dim; ++i) dot += (double)qh[i] * q8_0_value(krow, head_dim, g, i);
            double w = exp(scale * dot - m);
            denom += w;
            for (int32_t i = 0; i < head_dim; ++i)
                acc[i] += w * (v_type == KVD_ORACLE_V_Q4_0 ? q4_0_value(vrow, head_dim, g, i)
                                                           : q8_0_value(vrow, head_dim, g, i));
        }
    }
    for (int32_t i = 0; i < head_dim; ++i) out[i] = acc[i] / denom;
    free(acc);
    return 0;
}

/*
 * q      : fp32 [n_seq][n_head_q][head_dim]
 * segs   : [n_seq][n_seg]
 * q_pos  : [n_seq] query positions, or NULL = position of the last row of the
 *          last segment of that sequence
 * out    : fp64 [n_seq][n_head_q][head_dim]
 * Returns 0, or -1 for bad shapes / an empty visible set, -2 on host OOM.
 */
int kvd_oracle_attend_kv_f64(int32_t n_seq, int32_t n_head_q, int32_t n_head_kv, int32_t head_dim,
                             int32_t n_seg, int32_t window, double scale, int32_t v_type, const float* q,
                             const kvd_oracle_seg_kv* segs, const int64_t* q_pos, double* out,
                             int32_t n_threads) {
    if (n_seq < 1 || n_head_kv < 1 || n_head_q < n_head_kv || n_head_q % n_head_kv != 0) return -1;
    if (head_dim < KVD_ORACLE_QK || head_dim % KVD_ORACLE_QK != 0 || n_seg < 1 || window < 0) return -1;
    if (v_type != KVD_ORACLE_V_Q8_0 && v_type != KVD_ORACLE_V_Q4_0) return -1;
    const int32_t group = n_head_q / n_head_kv;
    int rc = 0;
    const int64_t n_items = (int64_t)n_seq * n_head_q;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1) reduction(min : rc)
#endif
    for (int64_t item = 0; item < n_items; ++item) {
        int32_t s = (int32_t)(item / n_head_q);
        int32_t h = (int32_t)(item % n_head_q);
        const kvd_oracle_seg_kv* ss = segs + (size_t)s * n_seg;
        int64_t qp = q_pos ? q_pos[s] : ss[n_seg - 1].pos0 + ss[n_seg - 1].n_rows - 1;
        int r = attend_one(head_dim, h / group, n_seg, window, scale, q + item * head_dim, ss, v_type, qp,
                           out + item * head_dim);
        if (r < rc) rc = r;
    }
    (void)n_threads;
    return rc;
}

/* q8_0 K and q8_0 V with one row stride: the symmetric case above. */
int kvd_oracle_attend_f64(int32_t n_seq, int32_t n_head_q, int32_t n_head_kv, int32_t head_dim,
                          int32_t n_seg, int32_t window, double scale, const float* q,
                          const kvd_oracle_seg* segs, const int64_t* q_pos, double* out,
                          int32_t n_threads) {
    if (n_seq < 1 || n_seg < 1) return -1;
    kvd_oracle_seg_kv* kv = (kvd_oracle_seg_kv*)malloc(sizeof(kvd_oracle_seg_kv) * (size_t)n_seq * (size_t)n_seg);
    if (!kv) return -2;
    for (int64_t i = 0; i < (int64_t)n_seq * n_seg; ++i) {
        kv[i].k = segs[i].k;
        kv[i].v = segs[i].v;
        kv[i].n_rows = segs[i].n_rows;
        kv[i].pos0 = segs[i].pos0;
        kv[i].k_stride = segs[i].row_stride;
        kv[i].v_stride = segs[i].row_stride;
    }
    int rc = kvd_oracle_attend_kv_f64(n_seq, n_head_q, n_head_kv, head_dim, n_seg, window, scale,
                                      KVD_ORACLE_V_Q8_0, q, kv, q_pos, out, n_threads);
    free(kv);
    return rc;
}

/*
 * Ring sizing, from "sched: pipeline the delivery of a host-resident KV
 * cache (R4)", Device memory: a ring is N + 2 slots, each one attention
 * layer's K and V over the whole context (cap_rows rows of row_bytes each,
 * for K and again for V).  Depth 0 is the ordered path and has no ring.
 */
int64_t kvd_oracle_ring_bytes(int32_t depth, int64_t cap_rows, int64_t row_bytes) {
    if (depth <= 0) return 0;
    return (int64_t)(depth + 2) * 2 * cap_rows * row_bytes;
}

/* The same with K and V rows of different sizes (q8_0 K, q4_0 V): each slot
 * holds cap_rows K rows and cap_rows V rows. */
int64_t kvd_oracle_ring_bytes_kv(int32_t depth, int64_t cap_rows, int64_t k_row_bytes, int64_t v_row_bytes) {
    if (depth <= 0) return 0;
    return (int64_t)(depth + 2) * cap_rows * (k_row_bytes + v_row_bytes);
}

/* The budget caps the ring outright: it fits iff its size is within the
 * budget (inclusive).  Returns 1 = fits, 0 = declines. */
int kvd_oracle_ring_fits(int32_t depth, int64_t cap_rows, int64_t row_bytes, int64_t budget_bytes) {
    if (depth <= 0) return 0;
    return kvd_oracle_ring_bytes(depth, cap_rows, row_bytes) <= budget_bytes;
}
