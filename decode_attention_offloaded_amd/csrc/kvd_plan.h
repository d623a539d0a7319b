// Split plan for decode attention: visible row ranges, rows per split and the
// workspace layout.  Host-only, HIP-free; depends on shapes and positions only.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "kvd_internal.h"

namespace kvd {

constexpr int kTileRows = 64;           // rows per tile of the decode kernel (split sizes are multiples)
constexpr int64_t kOneSplitRows = 256;   // contexts this short are not split when workgroups outnumber the CUs
constexpr int64_t kOneSplitSubtiles = 12;  // ... and, with at most one workgroup per CU, up to this many sub-tiles
constexpr int64_t kOneSplitW8Rows = 128;   // a sole split longer than this runs as one 8-wave workgroup
constexpr int kMaxSeqPerLaunch = 16;    // sequences described in one launch's arguments
constexpr int kDefaultCUs = 256;          // MI355X compute units, when the device cannot be asked
constexpr int64_t kSliceOverheadTiles = 3;  // fixed work of a 4-wave workgroup, in tiles
constexpr int64_t kBigOverheadTiles = 6;    // fixed work of an 8- or 12-wave workgroup, in tiles
constexpr int kWavesPerSimd = 3;            // decode-kernel waves resident per SIMD (registers)
constexpr int64_t kWaves8Subtiles = 12;     // sub-tiles per CU from which 8-wave workgroups are used
constexpr int64_t kWaves12Subtiles = 96;    // ... and 12-wave ones
constexpr double kBigPlanMinFill = 0.85;     // 8/12-wave plans filling less of the chip go to 4 waves
constexpr int kMaxSplits = 256;         // splits per (sequence, KV head) merged by one workgroup

struct SegPlan {
    int32_t row_lo;   // first visible row (segment row index)
    int32_t n_vis;    // visible rows
    int32_t n_split;  // splits over this segment
    int32_t n_rows;   // readable rows
};

struct SeqPlan {
    SegPlan seg[2];
    int32_t n_split;     // splits of the whole sequence
    int64_t split_base;  // first global split index
    int64_t q_pos;
};

struct AttendPlan {
    int32_t group;        // G = n_head_q / n_head_kv
    int32_t chunk_bytes;  // bytes of one head of one row: head_dim / 32 * 34
    int32_t split_rows;
    int32_t n_cus;        // compute units the plan was made for
    int32_t waves;        // waves per decode workgroup: 4, 8 or 12
    int32_t max_splits;   // largest per-sequence split count
    int64_t total_splits;
    std::vector<SeqPlan> seq;
    size_t off_pm, off_pl, off_po, ws_bytes;  // workspace: split maxima, sums, outputs
};

// Validate every argument that does not need the GPU and build the plan for a
// device of n_cus compute units (the plan depends on the shapes and n_cus
// only).  Returns KVD_OK or KVD_EINVAL (with kvd_last_error text).
int plan_attend(const kvd_attn_args* a, AttendPlan* p, int n_cus);

}  // namespace kvd
