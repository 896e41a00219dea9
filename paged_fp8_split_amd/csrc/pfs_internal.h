// pfs_internal.h -- plan layout shared by the host planner (pfs_plan.cpp) and
// the launcher (pfs_kernels.hip). Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/pfs.h"

namespace pfs {

constexpr int kPartitionTokens = 64;  // the K64 partition: unit of work and of ordering
constexpr int kMaxQHeads = 256;
constexpr int kMaxQ = 16;
// 16-row MFMA tiles per wave of the split kernel. Each wave keeps its FP32
// accumulators (16 RT rows x head_dim) and its Q^T operands in VGPRs; the cap
// keeps that, with the step's operands, within 256 VGPRs (two waves per SIMD).
constexpr int max_row_tiles(int head_dim) { return head_dim >= 256 ? 1 : (head_dim >= 128 ? 2 : 4); }
// Byte offsets of the 16-token tiles of one split sit in an LDS table.
constexpr int kTileTableEntries = 1024;
constexpr int kMaxTokensPerSplit = 16 * kTileTableEntries;
constexpr int kDefaultCUs = 256;  // MI355X compute units: the default split length fills them
// Size of the device array that holds the split partials of pfs_verify_noalloc
// (per GPU, for the life of the process).
constexpr int64_t kNoallocScratchBytes = 128ll << 20;

// A split workgroup has W = RG * TP waves: RG row groups (RT row tiles each)
// times TP token lanes; a stage holds TP 32-token steps of K and V bytes.
constexpr int split_stage_bytes(int head_dim, int token_lanes) { return token_lanes * 64 * head_dim; }
// Eight waves whenever a stage of 8 / RG steps stays within 64 KB. Batches
// with four row groups at head_dim 128 or 256 take four waves instead (one
// token lane, stages of 8 or 16 KB), so that two workgroups share a CU: one's
// pipeline fill and partial write overlap the other's stream while the
// dispatcher balances requests of unequal length. One request keeps eight
// waves: its splits all have the same length, and two per CU would double
// its partials. (Two row groups at head_dim 128 measured no gain.)
constexpr bool split_narrow(int head_dim, int row_groups, int batch) {
    return batch > 1 && head_dim >= 128 && row_groups == 4;
}
constexpr int split_waves(int head_dim, int row_groups, bool narrow = false) {
    return narrow ? 4 : (split_stage_bytes(head_dim, 8 / row_groups) <= 65536 ? 8 : 4);
}
// Four-wave workgroups with small stages run two per CU (64 KB of stages
// each); every other shape runs one per CU with up to 128 KB of stages.
constexpr int split_stages(int head_dim, int token_lanes, int waves) {
    const int s = split_stage_bytes(head_dim, token_lanes);
    const int budget = (waves == 4 && s <= 16384) ? 65536 : 131072;
    const int n = budget / s;
    return n >= 8 ? 8 : (n >= 4 ? 4 : 2);
}
constexpr int split_workgroups_per_cu(int head_dim, int token_lanes, int waves) {
    return (waves == 4 && split_stage_bytes(head_dim, token_lanes) * split_stages(head_dim, token_lanes, waves) <=
                              65536)
               ? 2
               : 1;
}

}  // namespace pfs

struct pfs_plan {
    pfs_problem p;           // copy of the problem (q_head_to_kv_head cleared)
    int32_t group;           // query heads per KV head (G)
    int32_t rows;            // rows per (request, KV head): R = G * q; row r = i * G + jj
    int32_t row_tiles;       // 16-row tiles per wave (template parameter)
    int32_t row_groups;      // waves along the rows of a workgroup (template parameter)
    int32_t token_lanes;     // waves along the tokens of a workgroup
    int32_t waves;           // waves per split workgroup: row_groups * token_lanes
    int32_t row_blocks;      // workgroups along the rows of one (request, KV head)
    int32_t capacity;        // block-table row capacity in tokens
    int32_t tokens_per_split;
    int32_t num_splits;      // splits per request (capacity / tokens_per_split, rounded up)
    int64_t ws_ml_offset;    // [num_splits][batch][num_kv_heads][rows] x (max, sum) FP32
    int64_t ws_acc_offset;   // [num_splits][batch][num_kv_heads][rows][head_dim] FP32
    int64_t ws_bytes;
    uint8_t qhead[pfs::kMaxQHeads];  // qhead[g * G + jj] = jj-th query head served by KV head g
};

// Launch helpers implemented in pfs_kernels.hip (arguments already validated).
int32_t pfs_launch_split(const pfs_plan* plan, const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                         const float* k_scale, const int32_t* block_table, const int32_t* live_len,
                         void* workspace, pfs_stream_t stream);
int32_t pfs_launch_combine(const pfs_plan* plan, const float* v_scale, const int32_t* live_len, void* out,
                           const void* workspace, pfs_stream_t stream);
// Implemented in pfs_codec.hip.
int32_t pfs_launch_append(const pfs_plan* plan, const void* k_new, const void* v_new, const float* k_scale,
                          const float* v_scale, const int32_t* block_table, const int32_t* live_len,
                          uint8_t* k_pool, uint8_t* v_pool, pfs_stream_t stream);
int32_t pfs_launch_bridge(const pfs_plan* plan, const uint8_t* pool, const float* scale, const int32_t* block_table,
                          const int32_t* live_len, void* out, pfs_stream_t stream);
