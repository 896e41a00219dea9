// pfs_plan.cpp -- host side of libpfs: ABI version, status strings, problem
// validation, split planning and workspace sizing. No HIP call is made here,
// so every check runs (and is tested) on a machine without a GPU.
#include <limits.h>
#include <math.h>
#include <new>
#include <stdint.h>
#include <string.h>

#include "pfs_internal.h"

namespace {

bool is_multiple(int64_t v, int64_t m) { return v % m == 0; }

int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int32_t pow2_ceil(int32_t v) {
    int32_t p = 1;
    while (p < v) p *= 2;
    return p;
}

// Shape of the split workgroups: each wave folds RT 16-row tiles; RG waves
// cover the rows (row groups) and TP waves per row group take alternate
// 32-token steps (token lanes). Tiles per wave come first: every wave converts
// the E4M3 bytes it reads, so more rows per wave means fewer conversions per
// row. Rows beyond RT * RG tiles become row blocks of the grid.
void choose_split_shape(int32_t rows, int32_t head_dim, int32_t batch, pfs_plan* plan) {
    const int32_t tiles = (rows + 15) / 16 > 0 ? (rows + 15) / 16 : 1;
    const int32_t max_rt = pfs::max_row_tiles(head_dim);
    const int32_t rt = pow2_ceil(tiles) < max_rt ? pow2_ceil(tiles) : max_rt;
    const int32_t groups = pow2_ceil((tiles + rt - 1) / rt);
    const int32_t rg = groups < 4 ? groups : 4;
    plan->row_tiles = rt;
    plan->row_groups = rg;
    plan->waves = pfs::split_waves(head_dim, rg, pfs::split_narrow(head_dim, rg, batch));
    plan->token_lanes = plan->waves / rg;
    plan->row_blocks = (tiles + rt * rg - 1) / (rt * rg);
}

}  // namespace

extern "C" {

int32_t pfs_abi_version(void) { return PFS_ABI_VERSION; }

const char* pfs_status_string(int32_t status) {
    switch (status) {
        case PFS_OK: return "ok";
        case PFS_ERR_NULL: return "a required pointer is NULL";
        case PFS_ERR_SHAPE: return "inconsistent or out-of-range size or stride";
        case PFS_ERR_UNSUPPORTED: return "unsupported head_dim, q, page size, partition size, KV format or probability mode";
        case PFS_ERR_ALIGNMENT: return "a KV stride or a base pointer is not 16-byte aligned";
        case PFS_ERR_HEAD_MAP: return "head map entry out of range or KV-head groups not uniform";
        case PFS_ERR_WORKSPACE: return "workspace NULL, misaligned (256 B) or too small";
        case PFS_ERR_LAUNCH: return "HIP kernel launch failed";
        case PFS_ERR_NOMEM: return "host allocation failed";
        default: return "unknown status";
    }
}

int32_t pfs_plan_create(const pfs_problem* pr, pfs_plan** out) {
    if (!pr || !out) return PFS_ERR_NULL;
    *out = nullptr;
    const pfs_problem& p = *pr;
    if (!p.q_head_to_kv_head) return PFS_ERR_NULL;

    // sizes and ranges
    if (p.batch < 0 || p.num_q_heads < 1 || p.num_kv_heads < 1 || p.page_size < 1 ||
        p.max_pages_per_row < 1 || p.num_pool_pages < 1)
        return PFS_ERR_SHAPE;
    if (p.num_q_heads > pfs::kMaxQHeads || p.num_q_heads % p.num_kv_heads != 0) return PFS_ERR_SHAPE;
    if (p.batch > 65535) return PFS_ERR_SHAPE;  // grid z
    if (!(p.sm_scale > 0.0f) || !isfinite(p.sm_scale)) return PFS_ERR_SHAPE;
    const int64_t capacity = (int64_t)p.max_pages_per_row * p.page_size;
    if (capacity > (int64_t)INT32_MAX / 2) return PFS_ERR_SHAPE;

    // what the kernels run
    if (p.q < 1 || p.q > pfs::kMaxQ) return PFS_ERR_UNSUPPORTED;
    if (p.head_dim != 64 && p.head_dim != 128 && p.head_dim != 256) return PFS_ERR_UNSUPPORTED;
    if (p.page_size % 16 != 0) return PFS_ERR_UNSUPPORTED;
    if (p.partition_tokens != pfs::kPartitionTokens) return PFS_ERR_UNSUPPORTED;
    if (p.kv_format != PFS_KV_E4M3 && p.kv_format != PFS_KV_E5M2) return PFS_ERR_UNSUPPORTED;
    if (p.pv_mode != PFS_PV_HIGH_RESIDUAL && p.pv_mode != PFS_PV_FP16) return PFS_ERR_UNSUPPORTED;
    if (p.num_cus < 0 || p.num_cus > 65536) return PFS_ERR_SHAPE;
    if (p.tokens_per_split < 0 || !is_multiple(p.tokens_per_split, p.partition_tokens))
        return PFS_ERR_SHAPE;

    // strides: 16-byte units (the loads are 16 bytes wide), then nesting
    if (p.kv_head_stride <= 0 || p.kv_token_stride <= 0 || p.kv_page_stride <= 0) return PFS_ERR_SHAPE;
    if (!is_multiple(p.kv_head_stride, 16) || !is_multiple(p.kv_token_stride, 16) ||
        !is_multiple(p.kv_page_stride, 16))
        return PFS_ERR_ALIGNMENT;
    // The (slot, KV head) rows of a page must not overlap: either a token's
    // heads nest inside the token stride ([page][slot][head][d]) or a head's
    // tokens nest inside the head stride ([page][head][slot][d]).
    if (p.kv_head_stride < p.head_dim || p.kv_token_stride < p.head_dim) return PFS_ERR_SHAPE;
    const int64_t head_span = (int64_t)(p.num_kv_heads - 1) * p.kv_head_stride + p.head_dim;
    const int64_t token_span = (int64_t)(p.page_size - 1) * p.kv_token_stride + p.head_dim;
    const bool token_major = p.kv_token_stride >= head_span;
    const bool head_major = p.kv_head_stride >= token_span;
    if (!token_major && !head_major) return PFS_ERR_SHAPE;
    const int64_t page_span = token_major ? (int64_t)(p.page_size - 1) * p.kv_token_stride + head_span
                                          : (int64_t)(p.num_kv_heads - 1) * p.kv_head_stride + token_span;
    if (p.kv_page_stride < page_span) return PFS_ERR_SHAPE;
    if ((double)p.kv_page_stride * (double)p.num_pool_pages > 4.0e18) return PFS_ERR_SHAPE;

    // head map: in range and uniform groups
    const int32_t G = p.num_q_heads / p.num_kv_heads;
    int32_t count[pfs::kMaxQHeads] = {0};
    for (int32_t h = 0; h < p.num_q_heads; ++h) {
        const int32_t g = p.q_head_to_kv_head[h];
        if (g < 0 || g >= p.num_kv_heads) return PFS_ERR_HEAD_MAP;
        count[g]++;
    }
    for (int32_t g = 0; g < p.num_kv_heads; ++g)
        if (count[g] != G) return PFS_ERR_HEAD_MAP;

    pfs_plan* plan = new (std::nothrow) pfs_plan;
    if (!plan) return PFS_ERR_NOMEM;
    memset(plan, 0, sizeof(*plan));
    plan->p = p;
    plan->p.q_head_to_kv_head = nullptr;
    plan->group = G;
    plan->rows = G * p.q;
    plan->capacity = (int32_t)capacity;
    {
        int32_t fill[pfs::kMaxQHeads] = {0};
        for (int32_t h = 0; h < p.num_q_heads; ++h) {
            const int32_t g = p.q_head_to_kv_head[h];
            plan->qhead[g * G + fill[g]++] = (uint8_t)h;
        }
    }
    choose_split_shape(plan->rows, p.head_dim, p.batch, plan);

    // Split length: a pure function of the shape (never of device data), so a
    // plan always folds the same partitions in the same order.
    // A split's 16-token tiles must fit the kernel's LDS tile table.
    const int64_t max_tps = pfs::kMaxTokensPerSplit;
    int64_t tps = p.tokens_per_split;
    if (tps > max_tps) {
        delete plan;
        return PFS_ERR_UNSUPPORTED;
    }
    if (tps == 0) {
        const int64_t per_cu = pfs::split_workgroups_per_cu(p.head_dim, plan->token_lanes, plan->waves);
        const int64_t cus = p.num_cus > 0 ? p.num_cus : pfs::kDefaultCUs;
        const int64_t target = cus * per_cu;  // one resident round of workgroups
        const int64_t units = (int64_t)(p.batch > 0 ? p.batch : 1) * p.num_kv_heads * plan->row_blocks;
        int64_t splits = (target + units - 1) / units;
        if (splits < 1) splits = 1;
        tps = round_up((capacity + splits - 1) / splits, pfs::kPartitionTokens);
        const int64_t min_tps = 4 * (int64_t)pfs::kPartitionTokens;
        // Batches: the plan cannot see the live lengths, and with one round
        // of workgroups the longest requests' splits set the kernel time while
        // the short ones' CUs idle. Capping a split at about 1 MiB of K+V
        // bytes per KV head gives the dispatcher several rounds of small
        // units to balance (a few % slower when every request is full).
        if (p.batch > 1) {
            const int64_t cap = ((int64_t)(1 << 20) / (2 * p.head_dim)) / pfs::kPartitionTokens * pfs::kPartitionTokens;
            if (tps > cap) tps = cap;
        }
        if (tps < min_tps) tps = min_tps;
        if (tps > max_tps) tps = max_tps;
    }
    if (tps > round_up(capacity, pfs::kPartitionTokens)) tps = round_up(capacity, pfs::kPartitionTokens);
    plan->tokens_per_split = (int32_t)tps;
    plan->num_splits = (int32_t)((capacity + tps - 1) / tps);
    // the split grid (work-items in one dimension, 32-bit index math on the
    // device) must stay below 2^31
    const int64_t units = (int64_t)plan->num_splits * p.num_kv_heads * (p.batch > 0 ? p.batch : 1);
    const int64_t split_items = ((units + 7) / 8) * 8 * plan->row_blocks * 64 * plan->waves;
    if (split_items > (int64_t)INT32_MAX) {
        delete plan;
        return PFS_ERR_SHAPE;
    }

    const int64_t slots = (int64_t)plan->num_splits * (p.batch > 0 ? p.batch : 1) * p.num_kv_heads * plan->rows;
    plan->ws_ml_offset = 0;
    plan->ws_acc_offset = round_up(slots * 2 * (int64_t)sizeof(float), 256);
    plan->ws_bytes = plan->ws_acc_offset + round_up(slots * p.head_dim * (int64_t)sizeof(float), 256);
    *out = plan;
    return PFS_OK;
}

void pfs_plan_destroy(pfs_plan* plan) { delete plan; }

int64_t pfs_plan_workspace_bytes(const pfs_plan* plan) { return plan ? plan->ws_bytes : 0; }

int32_t pfs_plan_num_splits(const pfs_plan* plan) { return plan ? plan->num_splits : 0; }

int32_t pfs_plan_tokens_per_split(const pfs_plan* plan) { return plan ? plan->tokens_per_split : 0; }

namespace {

bool misaligned16(const void* p) { return ((uintptr_t)p & 15u) != 0; }
bool misaligned4(const void* p) { return ((uintptr_t)p & 3u) != 0; }

int32_t check_workspace(const pfs_plan* plan, const void* workspace, int64_t workspace_bytes) {
    if (!workspace || ((uintptr_t)workspace & 255u) || workspace_bytes < plan->ws_bytes) return PFS_ERR_WORKSPACE;
    return PFS_OK;
}

int32_t check_split_args(const pfs_plan* plan, const void* q_fp16, const uint8_t* k_pool, const uint8_t* v_pool,
                         const float* k_scale, const int32_t* block_table, const int32_t* live_len,
                         const void* workspace, int64_t workspace_bytes) {
    if (!q_fp16 || !k_pool || !v_pool || !k_scale || !block_table || !live_len) return PFS_ERR_NULL;
    if (misaligned16(q_fp16) || misaligned16(k_pool) || misaligned16(v_pool)) return PFS_ERR_ALIGNMENT;
    if (misaligned4(k_scale) || misaligned4(block_table) || misaligned4(live_len)) return PFS_ERR_ALIGNMENT;
    return check_workspace(plan, workspace, workspace_bytes);
}

int32_t check_combine_args(const pfs_plan* plan, const float* v_scale, const int32_t* live_len, const void* out_fp16,
                           const void* workspace, int64_t workspace_bytes) {
    if (!v_scale || !live_len || !out_fp16) return PFS_ERR_NULL;
    if (misaligned16(out_fp16)) return PFS_ERR_ALIGNMENT;
    if (misaligned4(v_scale) || misaligned4(live_len)) return PFS_ERR_ALIGNMENT;
    return check_workspace(plan, workspace, workspace_bytes);
}

}  // namespace

int32_t pfs_verify(const pfs_plan* plan, const void* q_fp16, const uint8_t* k_pool, const uint8_t* v_pool,
                   const float* k_scale, const float* v_scale, const int32_t* block_table,
                   const int32_t* live_len, void* out_fp16, void* workspace, int64_t workspace_bytes,
                   pfs_stream_t stream) {
    if (!plan) return PFS_ERR_NULL;
    if (plan->p.batch == 0) return PFS_OK;
    int32_t st = check_split_args(plan, q_fp16, k_pool, v_pool, k_scale, block_table, live_len, workspace,
                                  workspace_bytes);
    if (st == PFS_OK) st = check_combine_args(plan, v_scale, live_len, out_fp16, workspace, workspace_bytes);
    if (st != PFS_OK) return st;
    st = pfs_launch_split(plan, q_fp16, k_pool, v_pool, k_scale, block_table, live_len, workspace, stream);
    if (st != PFS_OK) return st;
    return pfs_launch_combine(plan, v_scale, live_len, out_fp16, workspace, stream);
}

int32_t pfs_verify_split(const pfs_plan* plan, const void* q_fp16, const uint8_t* k_pool, const uint8_t* v_pool,
                         const float* k_scale, const int32_t* block_table, const int32_t* live_len,
                         void* workspace, int64_t workspace_bytes, pfs_stream_t stream) {
    if (!plan) return PFS_ERR_NULL;
    if (plan->p.batch == 0) return PFS_OK;
    const int32_t st = check_split_args(plan, q_fp16, k_pool, v_pool, k_scale, block_table, live_len, workspace,
                                        workspace_bytes);
    if (st != PFS_OK) return st;
    return pfs_launch_split(plan, q_fp16, k_pool, v_pool, k_scale, block_table, live_len, workspace, stream);
}

int32_t pfs_verify_combine(const pfs_plan* plan, const float* v_scale, const int32_t* live_len, void* out_fp16,
                           const void* workspace, int64_t workspace_bytes, pfs_stream_t stream) {
    if (!plan) return PFS_ERR_NULL;
    if (plan->p.batch == 0) return PFS_OK;
    const int32_t st = check_combine_args(plan, v_scale, live_len, out_fp16, workspace, workspace_bytes);
    if (st != PFS_OK) return st;
    return pfs_launch_combine(plan, v_scale, live_len, out_fp16, workspace, stream);
}

int32_t pfs_dequant_paged(const pfs_plan* plan, const uint8_t* pool, const float* scale,
                          const int32_t* block_table, const int32_t* live_len, void* out_fp16,
                          pfs_stream_t stream) {
    if (!plan) return PFS_ERR_NULL;
    if (plan->p.batch == 0) return PFS_OK;
    if (!pool || !block_table || !live_len || !out_fp16) return PFS_ERR_NULL;
    if (((uintptr_t)pool | (uintptr_t)out_fp16) & 15u) return PFS_ERR_ALIGNMENT;
    if (((uintptr_t)block_table | (uintptr_t)live_len | (uintptr_t)scale) & 3u) return PFS_ERR_ALIGNMENT;
    // one work-item per 16 bytes of a request's rows: the grid's x extent
    if ((int64_t)plan->capacity * plan->p.num_kv_heads * (plan->p.head_dim / 16) > (int64_t)INT32_MAX)
        return PFS_ERR_SHAPE;
    return pfs_launch_bridge(plan, pool, scale, block_table, live_len, out_fp16, stream);
}

int32_t pfs_kv_append(const pfs_plan* plan, const void* k_new_fp16, const void* v_new_fp16, const float* k_scale,
                      const float* v_scale, const int32_t* block_table, const int32_t* live_len, uint8_t* k_pool,
                      uint8_t* v_pool, pfs_stream_t stream) {
    if (!plan) return PFS_ERR_NULL;
    if (plan->p.batch == 0) return PFS_OK;
    if (!k_new_fp16 || !v_new_fp16 || !k_scale || !v_scale || !block_table || !live_len || !k_pool || !v_pool)
        return PFS_ERR_NULL;
    if (((uintptr_t)k_new_fp16 | (uintptr_t)v_new_fp16 | (uintptr_t)k_pool | (uintptr_t)v_pool) & 15u)
        return PFS_ERR_ALIGNMENT;
    if (((uintptr_t)k_scale | (uintptr_t)v_scale | (uintptr_t)block_table | (uintptr_t)live_len) & 3u)
        return PFS_ERR_ALIGNMENT;
    // one work-item per 8 values of a draft row: the grid's x extent (the
    // plan's own split-grid bound already keeps this below 2^31)
    if ((int64_t)plan->p.batch * plan->p.q * plan->p.num_kv_heads * (plan->p.head_dim / 8) > (int64_t)INT32_MAX)
        return PFS_ERR_SHAPE;
    return pfs_launch_append(plan, k_new_fp16, v_new_fp16, k_scale, v_scale, block_table, live_len, k_pool, v_pool,
                             stream);
}

}  // extern "C"
