// Host-side plan of the stream-K decode attention launch (shared between the two
// translation units that launch attention kernels).
#pragma once

#include <cstddef>
#include <cstdint>

#include "common.h"
#include "paged_kv.h"

namespace pkv {

// Stream-K decomposition: the (sequence, head unit, 16-token tile) tiles of the whole
// batch form one line; `waves` waves each take an equal contiguous slice of it.
// At most one wave per resident slot: compute units x 4 SIMDs x the kernel's waves per
// SIMD (on MI355X's 256 compute units: 1024 from head_dim 128; at 64, 3072 for 16-bit
// values).
inline int stream_max_waves(int compute_units, int head_dim, int elem_bytes, bool mfma) {
    return compute_units * 4 * kernel_waves_per_simd(head_dim, elem_bytes, mfma, true);
}
// The per-sequence tile prefix is built in LDS by every workgroup.
constexpr int kStreamMaxSeqs = 8192;
// Fewest tiles per wave the plan aims for (small batches get fewer waves).
constexpr int kStreamMinSlice = 16;

struct StreamPlan {
    bool mfma;             // MFMA kernel (unit = KV head) or VALU kernel (unit = query head)
    int32_t units;         // head units per sequence
    int32_t heads_per_unit;
    int32_t waves;         // W
    int64_t max_pieces;    // W + num_seqs * units: upper bound on partial results
    size_t cnt_off, m_off, l_off, acc_off, ws_bytes;
};

// Plan for a batch; `ok` false when the shape is outside what stream-K serves.
StreamPlan stream_plan(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t dtype, int32_t head_dim, int32_t max_context_len, bool* ok);

struct StreamLaunch {
    void* out;
    int32_t out_dtype;
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_tables;
    int32_t max_blocks_per_seq;
    const int32_t* context_lens;
    int32_t num_seqs;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t dtype;
    int32_t head_dim;
    int32_t block_size;
    int32_t max_context_len;
    float scale;
    // workspace, split: the per-(sequence, head unit) merge counters (zero on entry, left
    // zero) and the partial results (m, l, acc from StreamPlan::m_off on, rebased to 0)
    int32_t* counters;
    char* data;
    // Partition states (pm_tiles > 0, MFMA kernel only): instead of merging, each wave
    // stores the state of every 512-token (pm_tiles-tile) partition piece it computed
    // into rows (sequence, query head, 2 p + k) of pm_m / pm_l / pm_acc (max_parts =
    // pm_max_parts): k = 0 for the piece holding the partition's first tile, k = 1 for
    // the rest of a partition that a slice boundary cut (m = -inf when there is none);
    // the fixed-partition merge kernel then folds them.
    int32_t pm_tiles = 0;
    int32_t pm_max_parts = 0;
    float* pm_m = nullptr;
    float* pm_l = nullptr;
    float* pm_acc = nullptr;
};

// One launch: partition work and the merge of multi-piece units.
void launch_streamk_partition(const StreamLaunch& L, const StreamPlan& P, void* stream);

}  // namespace pkv
