/*
 * kvd.h -- decode attention over a q8_0 grouped-query KV cache that may live in
 * pinned host memory and reach the GPU one layer ahead (AMD Instinct MI355X,
 * gfx950).
 *
 * Passages this interface follows (cited by page title and section):
 *  [R4]  "sched: pipeline the delivery of a host-resident KV cache (R4)"
 *        -- opening paragraph (deliver one split ahead on a transfer stream of
 *        its own), What it does (1: stable prefix; 2: staging ring outside the
 *        allocator with a ready/release event pair per slot; 3: two slots of
 *        margin, deliveries issued after the consumer is enqueued, recycling
 *        ordered stream to stream), the depth knob (0 = ordered path exactly),
 *        Device memory (N + 2 slots of one layer's K+V; budget checked before
 *        anything is allocated, latched, transport created lazily), What
 *        tensor parallelism would take (an eligible backend needs async copies,
 *        event record/wait and event creation; otherwise it declines rather
 *        than racing; prefix delivery [0, prefix) and tail [prefix, nbytes)).
 *  [F5]  "F5 -- Advanced KV Cache Techniques" -- M2 What shipped (KV view
 *        [head_dim, n_head_kv, n_kv], innermost first), M3 What shipped (query
 *        heads grouped by the GQA ratio), M4 step 6 and W4 (online-softmax merge
 *        of partial attention results).
 *  [LC]  "Plan: lossless long context -- derived hot/cold sizing (#5) +
 *        host-RAM KV cold store (#3)" -- llama, sparse attention parity
 *        boundary (model-native sliding-window attention).
 *
 * Conventions
 *  - Every entry point validates all of its arguments before it enqueues
 *    anything; on a negative return nothing was enqueued.
 *  - Errors are returned as ints; kvd_last_error() gives text for the last
 *    non-OK return on the calling thread.  No C++ exception crosses this ABI.
 *  - "device pointer" = memory of the current HIP device (hipMalloc or torch);
 *    "pinned host pointer" = hipHostMalloc / torch pin_memory memory.
 *  - A stream argument is a hipStream_t passed as void* (NULL = null stream).
 *  - The library never reads environment variables.
 *
 * Data layout (reading of [F5] M2; q8_0 itself is only named on the pages):
 *  - q8_0 block: 34 bytes = little-endian binary16 scale d, then 32 int8
 *    codes; value = d * code.
 *  - A K (or V) row is one token: n_head_kv heads, each head_dim/32 blocks,
 *    heads back to back (row bytes = n_head_kv * head_dim / 32 * 34; for
 *    8 KV heads x 128 that is 1088).  Rows are row_stride bytes apart.
 *    K and V are separate buffers with the same geometry.
 *  - q and out: fp32 [n_seq][n_head_q][head_dim], contiguous.
 *  - Query head h reads KV head floor(h / (n_head_q / n_head_kv)) ([F5] M3).
 */
#ifndef KVD_H
#define KVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------ return codes */
#define KVD_OK 0
#define KVD_DECLINED 1      /* not an error: the ring is not engaged; the call
                               used (or would use) the ordered path ([R4] depth
                               knob and Device memory: declining falls back) */
#define KVD_EINVAL (-1)     /* invalid argument; nothing enqueued */
#define KVD_ENOMEM (-2)     /* host allocation failed */
#define KVD_EHIP (-3)       /* a HIP runtime call failed (text in kvd_last_error) */
#define KVD_ESTATE (-4)     /* call not valid in the object's current state
                               (wrong device, out-of-order stage/release) */

/* Text for the last non-OK return on this thread ("" if none).  The pointer
 * stays valid until the next kvd_* call on the same thread. */
const char* kvd_last_error(void);

/* Library version string, e.g. "kvd 0.1.0 gfx950". */
const char* kvd_version(void);

/* Host-link probe (measurement support): the pinned host-to-device copy rate
 * the staging ring can expect.  Copies `bytes` from hipHostMalloc'ed memory to
 * a hipMalloc'ed buffer with hipMemcpyAsync, split evenly over n_streams
 * non-blocking streams (the ring uses two, one DMA engine each), `reps` timed
 * times after one untimed; *gbps = bytes / median time, in GB/s (10^9 B/s).
 * Allocates and frees its own buffers and streams (synchronous).  ("F5 —
 * Advanced KV Cache Techniques", W1: probe the pinned host-to-device plateau.)
 * Returns KVD_OK, KVD_EINVAL (bytes outside [4096, 8 GiB], n_streams outside
 * [1, 4], reps outside [1, 1000], NULL gbps) or KVD_EHIP. */
int kvd_link_probe(size_t bytes, int32_t n_streams, int32_t reps, double* gbps);

/* Device-memory read rate: a streaming-read kernel (non-temporal 16-byte
 * loads, every byte of a `bytes`-byte device buffer read once) timed with HIP
 * events; *gbps = bytes / the median of `reps` launches, after one warm-up
 * launch, in 1e9 bytes per second.  Allocates and frees its own buffer (bytes
 * plus a small sink) on the current device and runs on a stream of its own;
 * the call returns when the timed launches are done.  Device-resident decode
 * attention is bound by reading the KV cache ([R4] opening paragraph: the
 * attention every decode token pays for), so its K/V rate is compared with
 * this besides the vendor's peak.
 * Returns KVD_OK, KVD_EINVAL (bytes not a multiple of 16 in [1 MiB, 64 GiB],
 * reps outside [1, 1000], NULL gbps; checked before any device work) or
 * KVD_EHIP. */
int kvd_hbm_read_probe(size_t bytes, int32_t reps, double* gbps);

/* ==================================================================== attention
 * kvd_attend_decode: single-token decode attention over q8_0 K/V.
 *
 * For every sequence s and query head h (KV head g = floor(h/G)):
 *   out[s,h,:] = sum_t softmax_t(scale * q[s,h,:] . K[t,g,:]) * V[t,g,:]
 * over the rows t visible to the query ([R4] opening paragraph: the attention
 * every decode token pays for).  A row at position p is visible to the query
 * at position P iff p <= P and, when window > 0, P - p < window (reading of
 * [LC]: the pages name sliding-window attention but give no formula).
 *
 * The rows of one sequence may come in one or two segments (e.g. an older
 * part staged from host memory and a newer device-resident part); softmax is
 * taken over the union of their visible rows ([F5] M4 step 6 / W4: partial
 * results merged by the online-softmax rule).
 *
 * Work is split over (sequence, KV head, row range); each split keeps an
 * online-softmax partial and the partials of one (sequence, query head) are
 * merged in a fixed order by a second launch on the same stream.  The split
 * plan depends only on the shapes and the device's compute-unit count (never
 * on pointers, timing or the ring), so two calls with equal shapes and equal
 * input bytes give bit-identical outputs.  The order in which sequences are
 * given changes no sequence's output either (the launch deals them out longest
 * first).
 */
typedef struct kvd_kv_seg {
    const void* k;       /* device: K row 0 of this segment (q8_0 rows) */
    const void* v;       /* device: V row 0 (the same rows as k: q8_0 like k, or
                            q4_0 when v_type is KVD_TYPE_Q4_0) */
    int64_t n_rows;      /* rows in the segment, 0 <= n_rows < 2^31; rows
                            [0, n_rows) must be readable */
    int64_t pos0;        /* token position of row 0 */
    int64_t row_stride;  /* bytes between rows; >= row bytes; multiple of 8
                            (head_dim 128) or 4 (head_dim 64); < 2^25 */
    int64_t v_row_stride;  /* bytes between V rows, or 0 = row_stride.  q8_0 V
                              rows have the K geometry: 0 or row_stride (else
                              KVD_EINVAL).  q4_0 V rows are shorter: >= V row
                              bytes, multiple of 4, < 2^25 */
} kvd_kv_seg;

/* Value types of the V cache (K is always q8_0).  q4_0: 18-byte blocks, a
 * little-endian binary16 scale d, then 16 bytes; value j < 16 = d * (low
 * nibble of byte j - 8), value 16 + j = d * (high nibble of byte j - 8)
 * ("F5 — Advanced KV Cache Techniques", M6 (PolyKV), S0: an asymmetric cache
 * with q8_0 K and q4_0 V, dequantised inside attention; the byte layout is
 * the reading taken of the named type). */
#define KVD_TYPE_Q8_0 0
#define KVD_TYPE_Q4_0 1

typedef struct kvd_attn_args {
    int32_t n_seq;       /* >= 1 */
    int32_t n_head_q;    /* multiple of n_head_kv; G = n_head_q/n_head_kv in 1..8 */
    int32_t n_head_kv;   /* >= 1 */
    int32_t head_dim;    /* 64 or 128 */
    int32_t n_seg;       /* segments per sequence: 1 or 2 */
    int32_t window;      /* 0 = full causal attention; W > 0 = sliding window */
    int32_t split_rows;  /* 0 = plan from shape; else rows per split, a
                            multiple of 64 (testing and tuning) */
    float scale;         /* softmax scale, usually 1/sqrt(head_dim); finite */
    const float* q;      /* device fp32 [n_seq][n_head_q][head_dim], 16-byte aligned */
    float* out;          /* device fp32 [n_seq][n_head_q][head_dim], 16-byte aligned
                            (unused, may be NULL, for kvd_attend_decode_partial) */
    const kvd_kv_seg* segs;  /* HOST array [n_seq][n_seg]; read during the call only */
    const int64_t* q_pos;    /* HOST array [n_seq] of query positions, or NULL =
                                the position of the last row of the last segment */
    void* workspace;         /* device scratch owned by the caller (256-byte aligned),
                                or NULL if kvd_attend_workspace_bytes reports 0 */
    size_t workspace_bytes;
    int32_t v_type;          /* KVD_TYPE_Q8_0 (0) or KVD_TYPE_Q4_0 */
    int32_t reserved;        /* must be 0 (KVD_EINVAL otherwise) */
} kvd_attn_args;

/* Bytes of workspace a call with these arguments needs (validates them too).
 * Returns KVD_OK and sets *bytes, or KVD_EINVAL.  The workspace holds the split
 * partials between the two launches of one call; it needs no initialisation.
 * Calls that share a workspace must not overlap in time (use one stream, or
 * order the streams). */
int kvd_attend_workspace_bytes(const kvd_attn_args* args, size_t* bytes);

/* The launch plan a call with these arguments gets on the current device,
 * without launching anything (validates the arguments too): rows per split,
 * waves per decode workgroup (4, 8 or 12, chosen from the work per compute
 * unit; calls of several sequences whose 8- or 12-wave splits would fill
 * under 85% of the chip's time take 4) and the splits of all sequences
 * together.  A call of more than 16 sequences runs as consecutive launches of
 * up to 16, all with these split rows and waves, sized for the compute units
 * of all its launches.  Any output pointer may be NULL.  Returns KVD_OK or KVD_EINVAL.  The plan depends on the shapes and the
 * device's compute-unit count only ("F5 -- Advanced KV Cache Techniques", M4:
 * split-K decode over row ranges, merged by running maxima and sums). */
int kvd_attend_plan(const kvd_attn_args* args, int32_t* split_rows, int32_t* waves, int64_t* total_splits);

/* How the decode kernel of the call's first launch loads K/V ("F5 -- Advanced
 * KV Cache Techniques", M4: the split-K decode kernel this describes): 0 =
 * dword loads (some K/V base or row stride is not a multiple of 16 bytes),
 * 1 = 16-byte loads staged in registers, 2 = 16-byte loads straight into LDS
 * (where a compute unit runs at most 8 waves: 8-wave workgroups, or 4-wave
 * ones at most two per compute unit).  Validates the arguments like
 * kvd_attend_plan and launches nothing.  Returns KVD_OK and sets *mode, or
 * KVD_EINVAL (also for a NULL mode).  For profiling: the mode is the
 * kernel's fourth template argument in a trace. */
int kvd_attend_load_mode(const kvd_attn_args* args, int32_t* mode);

/* Enqueue decode attention on `stream` (asynchronous).  Returns KVD_OK,
 * KVD_EINVAL (bad shapes, unaligned or null pointers, a sequence with no
 * visible row, workspace too small) or KVD_EHIP (launch failure). */
int kvd_attend_decode(const kvd_attn_args* args, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): as
 * kvd_attend_decode, but the split partials live in a fixed device array
 * built into the library (8 MiB per GPU, held until the process ends), so
 * the call allocates nothing; args->workspace and args->workspace_bytes are
 * ignored.  A call whose partials need more than 8 MiB (see
 * kvd_attend_workspace_bytes) returns KVD_EINVAL and enqueues nothing.
 * Every call on one GPU uses the same array: calls that may overlap in time
 * on one GPU (different streams, not ordered by events) race; order them.
 * Returns KVD_OK, KVD_EINVAL or KVD_EHIP. */
int kvd_attend_decode_noalloc(const kvd_attn_args* args, void* stream);

/* Tile-streamed attention ("F5 — Advanced KV Cache Techniques", F5-opt W4,
 * M7 Rolling KV: a slot pool, a tile loop and an inter-tile online-softmax
 * merge of the per-tile results).  A layer's rows are attended in tiles, one
 * call per tile over that tile's rows only, each leaving an unnormalised
 * result; one merge then gives the attention over the union of the tiles.
 *
 * kvd_attend_decode_partial: as kvd_attend_decode (same arguments, same
 * validation, same workspace), but instead of `out` it writes to `partial`
 * (device, 16-byte aligned, (head_dim + 2) * n_seq * n_head_q floats):
 *   o [n_seq][n_head_q][head_dim] = sum_t e^(x_t - m) V[t]
 *   m [n_seq][n_head_q]           = the reference maximum, in units of
 *                                    x_t = scale * log2(e) * q . K[t]
 *   l [n_seq][n_head_q]           = sum_t e^(x_t - m)   (e^ taken base 2)
 * over the rows visible in this call.  Every sequence needs at least one
 * visible row in every call.  `args->out` is not used. */
int kvd_attend_decode_partial(const kvd_attn_args* args, float* partial, void* stream);

/* Merge n_part partial results, laid out back to back (partial t at
 * partials + t * (head_dim + 2) * n_seq * n_head_q), into
 * out[n_seq][n_head_q][head_dim] = sum_t e^(m_t - M) o_t / sum_t e^(m_t - M) l_t
 * with M = max_t m_t, merged in t order (the result does not depend on timing).
 * Device pointers, 16-byte aligned; head_dim 64 or 128; 1 <= n_part <= 2^20;
 * n_seq * n_head_q even (so every partial starts on a 16-byte boundary).
 * Asynchronous on `stream`.  Returns KVD_OK, KVD_EINVAL or KVD_EHIP. */
int kvd_attend_merge(const float* partials, int32_t n_part, int32_t n_seq, int32_t n_head_q, int32_t head_dim,
                     float* out, void* stream);

/* ==================================================================== staging ring
 * A ring stages one attention layer's K and V from pinned host memory into
 * device slots ahead of use ([R4] What it does 2 and 3).  It has depth N
 * (look-ahead in layers) and N + 2 slots; each slot holds cap_rows rows of K
 * and of V.  Its device cost is (N + 2) * cap_rows * (row_bytes +
 * v_row_bytes), checked against budget_bytes before anything is allocated,
 * on every stage call; once over budget the ring declines for good ([R4]
 * Device memory: checked before allocating, latched).  Slots, events and the
 * ring's two transfer streams (a delivery's bytes split evenly between them,
 * one DMA engine each) are created on the first stage call that engages the
 * ring and freed by kvd_ring_destroy ([R4] Device memory: the transport is
 * lazy).  Depth 0 is the ordered path exactly: it never allocates anything.
 *
 * Per layer l of a decode step the caller does:
 *   1. write the newest row(s) of layer l into the pinned host K/V;
 *   2. kvd_ring_stage_layer(flags = ACQUIRE, layer l) -> a view of l's K/V in
 *      device memory, ordered on `compute` (the ordered path copies the whole
 *      layer there; the pipelined path copies only the tail rows there and
 *      waits for the prefix copied earlier on the transfer streams);
 *   3. enqueue attention (kvd_attend_decode) on the view, on `compute`;
 *   4. kvd_ring_release(layer l, compute): the slot is free once `compute`
 *      passes this point;
 *   5. kvd_ring_stage_layer(flags = PREFETCH, layer l + N): start copying the
 *      stable prefix of layer l + N on the transfer streams.  They wait,
 *      stream to stream, for the release of the slot it reuses ([R4] What it
 *      does 3: issued after the consumer is enqueued, never a host sync).
 * ACQUIRE of a layer that was not prefetched (e.g. the first N layers of a
 * step) stages it on the spot.  A ring serves one host thread and one device.
 */
typedef struct kvd_ring kvd_ring;

/* Create a ring.  depth >= 0 (0 = ordered path), budget in bytes (the pages'
 * default is 128 MiB per device).  The budget belongs to this ring: one ring
 * per device is the intended use, and two rings on one device each hold to
 * their own budget (the device total is their sum).  Does no device work.
 * Returns NULL iff depth < 0 or depth > 64 or host memory runs out
 * (kvd_last_error says which). */
kvd_ring* kvd_ring_create(int32_t depth, size_t budget_bytes);

#define KVD_STAGE_PREFETCH 1
#define KVD_STAGE_ACQUIRE 2

typedef struct kvd_stage_args {
    int32_t layer;        /* caller's layer id (>= 0); identifies the delivery */
    int32_t flags;        /* KVD_STAGE_PREFETCH or KVD_STAGE_ACQUIRE */
    const void* host_k;   /* PINNED host: K rows [cap_rows][row_bytes] of this layer */
    const void* host_v;   /* PINNED host: V rows, same geometry */
    int64_t row_bytes;    /* bytes of one K row (= one V row unless v_row_bytes
                             says otherwise); multiple of 4, <= 2^24 */
    int64_t n_rows;       /* rows to deliver: [0, n_rows); 1 <= n_rows <= cap_rows */
    int64_t stable_rows;  /* rows [0, stable_rows) are not written again before
                             this layer's release ([R4] What it does 1: the stable
                             prefix = the lowest row the step writes) */
    int64_t cap_rows;     /* capacity the context may grow to; sizes the slots */
    void* ordered_k;      /* device buffer >= n_rows*row_bytes, used when the ring
                             is not engaged (ACQUIRE only; may be NULL for PREFETCH) */
    void* ordered_v;      /* device buffer >= n_rows*v_row_bytes */
    int64_t v_row_bytes;  /* bytes of one V row, or 0 = row_bytes (a q4_0 V row is
                             shorter than the q8_0 K row); multiple of 4; the ring
                             is then (N + 2) * cap_rows * (row_bytes + v_row_bytes) */
} kvd_stage_args;

typedef struct kvd_slot_view {
    const void* k;        /* device: K rows [n_rows][row_bytes] */
    const void* v;        /* device: V rows */
    int64_t n_rows;
    int64_t row_stride;   /* = row_bytes */
    int32_t pipelined;    /* 1 = ring slot, 0 = ordered buffer */
    int32_t slot;         /* slot index, or -1 */
    int64_t v_row_stride; /* = v_row_bytes */
} kvd_slot_view;

/* PREFETCH: returns KVD_OK (prefix copy enqueued on the transfer streams) or
 *   KVD_DECLINED (ring not engaged: nothing done).  `out` may be NULL.
 * ACQUIRE: returns KVD_OK with a slot view (pipelined) or KVD_DECLINED with a
 *   view of ordered_k/ordered_v after enqueuing the whole-layer copy on
 *   `compute`.  Either way the view is ready for work enqueued on `compute`
 *   after this call and stays valid until kvd_ring_release(layer).
 * Errors: KVD_EINVAL (null/pageable host pointers, bad row counts, missing
 *   ordered buffers on the ordered path), KVD_ESTATE (a different device
 *   than the ring's; reusing a slot whose previous layer was never released;
 *   a layer staged twice; capacity changed while deliveries are in flight),
 *   KVD_EHIP.  A failed device allocation is not an error: the ring declines
 *   (latched) and ACQUIRE falls back to the ordered path. */
int kvd_ring_stage_layer(kvd_ring* ring, const kvd_stage_args* args, void* compute_stream,
                         kvd_slot_view* out);

/* Mark the end of `layer`'s use of its slot: records the slot's release event
 * on `compute` ([R4] What it does 2: the release half of the event pair).
 * Call it after the last work that reads the view is enqueued.  No-op
 * (KVD_OK) on the ordered path.  KVD_ESTATE if the layer is not acquired. */
int kvd_ring_release(kvd_ring* ring, int32_t layer, void* compute_stream);

typedef struct kvd_ring_stats {
    int32_t depth;
    int32_t n_slots;          /* depth + 2 when depth >= 1, else 0 */
    int32_t engaged;          /* device resources currently allocated */
    int32_t declined;         /* latched decline */
    int32_t device;           /* HIP device the ring is bound to, or -1 */
    int32_t reserved;
    int64_t budget_bytes;
    int64_t need_bytes;       /* size of the last plan: (N+2)*cap_rows*(row_bytes+v_row_bytes) */
    int64_t ring_bytes;       /* device bytes held by slots now */
    int64_t slot_rows;        /* rows per slot */
    int64_t n_prefetch;       /* prefix deliveries issued ahead */
    int64_t n_acquire_pipelined;  /* ACQUIREs served from a prefetched slot */
    int64_t n_acquire_primed;     /* ACQUIREs that staged a slot on the spot */
    int64_t n_acquire_ordered;    /* ACQUIREs on the ordered path */
    int64_t bytes_early;      /* bytes copied by PREFETCH (ahead of use) */
    int64_t bytes_late;       /* bytes copied at ACQUIRE into slots (tails, primes) */
    int64_t bytes_ordered;    /* bytes copied on the ordered path */
} kvd_ring_stats;

/* Copy the counters into *out (out_size must be >= sizeof(kvd_ring_stats)). */
int kvd_ring_stats_get(const kvd_ring* ring, kvd_ring_stats* out, size_t out_size);

/* Test support (for callers that check the ring's ordering, not for
 * production use): from now on, before every copy the ring puts on one of its
 * transfer streams, that stream is held for a random 0..max_us microseconds
 * (a one-wave spin kernel polling the real-time counter, bounded), drawn from
 * a generator seeded with `seed`.  Late deliveries must not change any
 * output: every consumer waits for its delivery's `ready` events ([R4] What
 * it does 2: a ready/release event pair per slot).  max_us = 0 turns it off.
 * Returns KVD_OK, or KVD_EINVAL (NULL ring, max_us above 100000). */
int kvd_ring_set_transfer_delay(kvd_ring* ring, uint32_t max_us, uint64_t seed);

/* Wait for the transfer streams and every slot's release, then free slots,
 * events and the transfer streams.  NULL is a no-op. */
void kvd_ring_destroy(kvd_ring* ring);

/* Tile size for tile-streamed attention through a ring of this depth and
 * budget ("F5 — Advanced KV Cache Techniques", F5-opt: tiles of a spilled
 * layer streamed through a slot pool; tile bytes bounded by
 * compute_ms * effective_bw * 0.8).  Sets *tile_rows to the largest multiple
 * of 64 rows such that the ring, (depth + 2) * 2 * tile_rows * row_bytes
 * bytes, fits budget_bytes (inclusive) and, when max_tile_bytes > 0, one
 * tile's K + V, 2 * tile_rows * row_bytes, is at most max_tile_bytes (the
 * caller passes compute_ms * effective_bw * 0.8, or 0 for no such bound).
 * Returns KVD_OK, KVD_DECLINED (*tile_rows = 0: not even 64 rows fit) or
 * KVD_EINVAL (depth < 1, row_bytes out of (0, 2^24], max_tile_bytes < 0 or
 * NaN, tile_rows NULL).  Host-only; allocates nothing. */
int kvd_ring_tile_rows(int32_t depth, size_t budget_bytes, int64_t row_bytes, double max_tile_bytes,
                       int64_t* tile_rows);

/* ==================================================================== residency
 * Which layers keep their K/V on the device ("sched: pipeline the delivery
 * of a host-resident KV cache (R4)", Known limitations: device-resident
 * layers can remove more host-to-device traffic than a ring of the same bytes
 * hides; "F5 — Advanced KV Cache Techniques", F5-opt W4: device-resident
 * whenever the KV fits the budget, spill only under pressure).
 *
 * Layers [0, n_resident) stay on the device (a resident prefix: while it is
 * computed the first staged layer's delivery is in flight); the others are
 * staged per step, through a depth-`depth` ring of whole layers when use_ring,
 * else on the ordered path.  The budget covers the resident layers plus the
 * ring ((depth + 2) * layer_bytes).
 *
 * Choice: every layer resident if all fit.  Otherwise, with link_gbps > 0 a
 * step-time estimate decides between "ring + as many resident layers as fit
 * beside it" and "no ring + as many resident layers as fit": staged bytes
 * cross the link at link_gbps; compute is n_layers * compute_ms; ordered =
 * transfer + compute; ring = max(transfer, compute) + the part of the first
 * staged layer's delivery that the resident prefix does not cover.  With
 * link_gbps == 0 the ring is kept whenever it fits.  Host-only; allocates
 * nothing. */
typedef struct kvd_residency_plan {
    int32_t n_resident;            /* layers [0, n_resident) device-resident */
    int32_t use_ring;              /* 1: stage the rest through the ring; 0: ordered */
    int64_t resident_bytes;        /* n_resident * layer_bytes */
    int64_t ring_bytes;            /* (depth + 2) * layer_bytes when use_ring, else 0 */
    int64_t staged_bytes_per_step; /* (n_layers - n_resident) * layer_bytes */
    double est_ms_per_step;        /* the estimate the choice used (0 without a model) */
} kvd_residency_plan;

/* n_layers in [1, 2^20]; layer_bytes = K + V bytes of one layer (all layers
 * alike), in [1, 2^50]; depth >= 0 (0: no ring); link_gbps and compute_ms
 * finite and >= 0.  Returns KVD_OK or KVD_EINVAL. */
int kvd_plan_residency(int32_t n_layers, int64_t layer_bytes, size_t budget_bytes, int32_t depth, double link_gbps,
                       double compute_ms, kvd_residency_plan* out);

#ifdef __cplusplus
}
#endif
#endif /* KVD_H */
