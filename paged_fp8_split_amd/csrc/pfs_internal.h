// pfs_internal.h -- plan layout shared by the host planner (pfs_plan.cpp) and
// the launcher (pfs_kernels.hip). Not part of the public ABI.
#pragma once

#include <stdint.h>

#include "../../include/pfs.h"

namespace pfs {

constexpr int kPartitionTokens = 64;  // the K64 partition: unit of work and of ordering
constexpr int kWaves = 4;             // waves per split workgroup
constexpr int kMaxQHeads = 256;
constexpr int kMaxQ = 16;
// 16-row MFMA tiles per wave of the split kernel. Each wave keeps its FP32
// accumulators (16 RT rows x head_dim) and its Q^T operands in VGPRs; the cap
// keeps that, with the step's operands, within 256 VGPRs (two waves per SIMD).
constexpr int max_row_tiles(int head_dim) { return head_dim >= 256 ? 1 : (head_dim >= 128 ? 2 : 4); }
constexpr int kDefaultTargetWorkgroups = 512;
// Pages one split workgroup can address: their byte offsets sit in LDS.
constexpr int kPageTableEntries = 1024;

// LDS of one split stage: TP 32-token steps of K and V bytes.
constexpr int split_stage_bytes(int head_dim, int token_lanes) { return token_lanes * 64 * head_dim; }
// Stages in flight: up to 64 KB of stages when two workgroups fit a CU,
// otherwise up to 128 KB for one workgroup per CU.
constexpr int split_stages(int head_dim, int token_lanes) {
    const int s = split_stage_bytes(head_dim, token_lanes);
    if (s <= 16384) {
        const int n = 65536 / s;
        return n >= 8 ? 8 : (n >= 4 ? 4 : 2);
    }
    return 131072 / s >= 4 ? 4 : 2;
}
constexpr int split_workgroups_per_cu(int head_dim, int token_lanes, int stages) {
    return split_stage_bytes(head_dim, token_lanes) * stages <= 65536 ? 2 : 1;
}

}  // namespace pfs

struct pfs_plan {
    pfs_problem p;           // copy of the problem (q_head_to_kv_head cleared)
    int32_t group;           // query heads per KV head (G)
    int32_t rows;            // rows per (request, KV head): R = G * q; row r = i * G + jj
    int32_t row_tiles;       // 16-row tiles per wave (template parameter)
    int32_t row_groups;      // waves along the rows of a workgroup (template parameter)
    int32_t token_lanes;     // waves along the tokens of a workgroup: kWaves / row_groups
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
int32_t pfs_launch_dequant(const pfs_plan* plan, const uint8_t* pool, const int32_t* block_table,
                           const int32_t* live_len, void* out, pfs_stream_t stream);
