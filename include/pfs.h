/*
 * pfs.h -- C ABI of libpfs: E4M3 paged speculative-verify attention with FP32
 * split partials, for AMD Instinct MI355X (gfx950).
 *
 * The operation (defined by the pages "[Kernel][SM70] Add opt-in E4M3 grouped
 * attention with FP32 partials", final-status section and Scope list, and
 * "[Bugfix] Use FP32 state and E4M3 defaults for DFlash2", Purpose):
 *
 *   For request b, query head h (KV head g = head_map[h]) and draft row i in
 *   [0, q): the row attends causally to the first n_i = clamp(L_b - q + i + 1,
 *   0, L_b) tokens of the request's paged KV cache, where L_b = live_len[b]
 *   counts the q draft tokens. K and V are stored as OCP E4M3 (FN) bytes
 *   (or, on request, E5M2 bytes: PFS_KV_E5M2) with one FP32 scale per KV
 *   head:  Khat = dec(k_byte) * k_scale[g],  Vhat = dec(v_byte) * v_scale[g].
 *     s_j  = sm_scale * dot(Q[b,i,h,:], Khat_j)          for j < n_i
 *     out  = sum_j exp(s_j - max s) Vhat_j / sum_j exp(s_j - max s)
 *   rounded once to FP16 (round to nearest even). A row with n_i == 0
 *   (retired request, or L_b < q) outputs +0.0.
 *
 *   The context is cut into splits of tokens_per_split tokens, each a run of
 *   64-token partitions consumed in ascending order ("[Kernel] Finalize the
 *   audited TP2 DFlash2 31/29 ms endpoint", Purpose: K64 partition order).
 *   Every split emits an FP32 running max, an FP32 sum and an unnormalized
 *   FP32 PV accumulator into the caller's workspace; a combine pass rescales
 *   the splits, reduces them in a fixed order (stated at pfs_verify_combine),
 *   normalizes and rounds once ("[Kernel][SM70] Add opt-in E4M3 grouped
 *   attention with FP32 partials", final status, revision 3 bullet: max/sum
 *   and unnormalized PV kept in FP32 until one final combine).
 *
 * Every call returns a status code (PFS_OK == 0, errors < 0); no exception and
 * no fallback path crosses this boundary: an unsupported shape is an error.
 * The library never allocates, frees or synchronizes device memory; pfs_verify
 * only enqueues kernels on the caller's stream and is safe to capture in a HIP
 * graph.
 */
#ifndef PFS_H
#define PFS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Bumped whenever a signature, a struct layout or the numerics contract
 * changes. Callers refuse a library whose pfs_abi_version() differs from the
 * header they were built against (the pages' "stale native rejection":
 * "[Bugfix] Use FP32 state ...", Purpose, precision revision / rebuild). */
#define PFS_ABI_VERSION 5

enum {
    PFS_OK = 0,
    PFS_ERR_NULL = -1,        /* a required pointer is NULL */
    PFS_ERR_SHAPE = -2,       /* an inconsistent or out-of-range size/stride */
    PFS_ERR_UNSUPPORTED = -3, /* head_dim, q, page size or partition not supported */
    PFS_ERR_ALIGNMENT = -4,   /* a stride or a base pointer is not 16-byte aligned */
    PFS_ERR_HEAD_MAP = -5,    /* head map entry out of range or groups not uniform */
    PFS_ERR_WORKSPACE = -6,   /* workspace NULL, misaligned or smaller than required */
    PFS_ERR_LAUNCH = -7,      /* the HIP runtime reported an error at launch */
    PFS_ERR_NOMEM = -8        /* host allocation of the plan failed */
};

/* How the bytes of the KV pools encode values (pfs_problem.kv_format).
 * E4M3 is the method's format: OCP E4M3FN, bias 7, largest finite 448, no
 * infinities, S.1111.111 = NaN. E5M2 is the explicit alternative the pages
 * keep beside it ("[Bugfix] Use FP32 state and E4M3 defaults for DFlash2",
 * Purpose: E4M3 by default, E5M2 on request; "[Kernel][SM70] Add opt-in
 * E4M3 grouped attention with FP32 partials", historical scope: explicit
 * E5M2 routes kept): bias 15, largest finite 57344, S.11111.00 = infinity,
 * S.11111.xx (xx != 0) = NaN; every E5M2 value is the FP16 number whose high
 * byte it is. Only the decoder (and the quantize-on-write encoder) differs;
 * scales, layout and the rest of the arithmetic are the same. */
enum { PFS_KV_E4M3 = 0, PFS_KV_E5M2 = 1 };

/* How each probability p enters the PV product (pfs_problem.pv_mode).
 * PFS_PV_HIGH_RESIDUAL (0, the default) carries p as two FP16 operands, the
 * high part hi = RNE_fp16(p) and the residual res = RNE_fp16(p - hi), both
 * multiplied with the same FP16 V operand ("[Kernel][SM70] Add opt-in E4M3
 * grouped attention with FP32 partials", historical scope list: the PV
 * probability as high/residual FP16 operands); the row sums take hi + res
 * the same way. The kernel evaluates p as 2^(s - m_ref + 7), so the largest
 * p of a row is at least 2^7 and res stays an FP16 normal number for every
 * key within 2^-10 of it: no scaling of res (nor of V) is needed, and p
 * reaches PV with about 22 significant bits instead of 11. Any KV format.
 * PFS_PV_FP16 (1, opt-in) carries p as hi alone: about half the PV matrix
 * work, but the FP16 rounding of each probability (2^-11 relative) reaches
 * the output; with attention concentrated on a few keys whose V values
 * nearly cancel it can exceed an absolute error of 4e-3. */
enum { PFS_PV_HIGH_RESIDUAL = 0, PFS_PV_FP16 = 1 };

/* Opaque HIP stream handle (hipStream_t); NULL is the default stream. */
typedef struct ihipStream_t* pfs_stream_t;

/*
 * Static description of one problem shape. Everything a plan depends on is in
 * here; device data (pointers, live lengths, block-table contents) is not.
 *
 * KV pools: byte arrays addressed as
 *   page * kv_page_stride + slot * kv_token_stride + kv_head * kv_head_stride + d
 * for page in [0, num_pool_pages), slot in [0, page_size), d in [0, head_dim)
 * (the pages' [num_blocks, block_size, kv_heads, head_dim] uint8 layout with
 * byte strides; "... FP32 partials", AI integration review). The head_dim
 * bytes of one (page, slot, kv_head) are contiguous. The rows of a page must
 * not overlap: either the token stride holds all heads of a token
 * ([page][slot][head][d], token-major) or the head stride holds all slots of a
 * head ([page][head][slot][d], head-major). K and V pools share the same
 * strides.
 *
 * Q and out: contiguous [batch, q, num_q_heads, head_dim] FP16.
 */
typedef struct pfs_problem {
    int32_t batch;              /* requests, >= 0 (0: pfs_verify does nothing) */
    int32_t q;                  /* draft rows per request, 1..16 */
    int32_t num_q_heads;        /* multiple of num_kv_heads, <= 256 */
    int32_t num_kv_heads;       /* >= 1 */
    int32_t head_dim;           /* 64, 128 or 256 */
    int32_t page_size;          /* tokens per page, a positive multiple of 16 */
    int32_t max_pages_per_row;  /* block-table row length (capacity = this * page_size) */
    int32_t num_pool_pages;     /* physical pages in each pool */
    int32_t partition_tokens;   /* 64 (the only partition size this build runs) */
    int32_t tokens_per_split;   /* 0 = library default: a function of the shape only, the
                                   smallest multiple of 64 (at least 256, at most the
                                   capacity rounded up to 64) for which one round of
                                   split workgroups fills num_cus compute units, capped for
                                   batch > 1 at 2^20 / (2 * head_dim) tokens (about 1 MiB
                                   of K+V per request and KV head) so that requests of
                                   unequal live length can be balanced; else a multiple
                                   of partition_tokens, at most 16384 */
    int32_t kv_format;          /* PFS_KV_E4M3 (0) or PFS_KV_E5M2 (1): how the pool bytes decode */
    int32_t pv_mode;            /* PFS_PV_HIGH_RESIDUAL (0, default) or PFS_PV_FP16 (1), see above */
    int32_t num_cus;            /* compute units the default split length fills (the device's
                                   count, e.g. hipDeviceProp_t.multiProcessorCount); 0 = 256,
                                   the MI355X's. Used only when tokens_per_split == 0; a plan
                                   made for one count runs correctly on any device */
    int64_t kv_page_stride;     /* bytes, multiple of 16 */
    int64_t kv_token_stride;    /* bytes, multiple of 16 */
    int64_t kv_head_stride;     /* bytes, multiple of 16, >= head_dim */
    float sm_scale;             /* softmax scale, finite and > 0 (usually 1/sqrt(head_dim)) */
    const int32_t* q_head_to_kv_head; /* HOST array [num_q_heads]; copied at plan time */
} pfs_problem;

typedef struct pfs_plan pfs_plan;

/* The PFS_ABI_VERSION the library was built with ("[Bugfix] Use FP32 state
 * and E4M3 defaults for DFlash2", Purpose: a stale native library is
 * rejected, not silently used). */
int32_t pfs_abi_version(void);

/* Static, NUL-terminated description of a status code; never NULL, and
 * "unknown status" for a value that is not a PFS_* code. Every failure is
 * reported through these codes, none is handled by a fallback
 * ("[Kernel][SM70] Add opt-in E4M3 grouped attention with FP32 partials",
 * historical scope list: unsupported shapes and stale libraries fail closed). */
const char* pfs_status_string(int32_t status);

/*
 * Validate a problem and build a plan (host only: no HIP call, no device
 * needed). On success *out owns a plan the caller releases with
 * pfs_plan_destroy. Checks (each with its own status code): sizes and ranges,
 * head_dim / q / page size / partition support, 16-byte stride alignment
 * (the pages' counterexample, token stride 264 with a 16-byte paired loader,
 * is rejected here with PFS_ERR_ALIGNMENT), non-overlapping nesting of the
 * strides, a uniform head map (every KV head serves exactly
 * num_q_heads / num_kv_heads query heads), and a split grid below 2^31
 * work-items (PFS_ERR_SHAPE otherwise).
 * The plan is immutable and may be shared by host threads.
 */
int32_t pfs_plan_create(const pfs_problem* problem, pfs_plan** out);

/* Releases a plan made by pfs_plan_create (host memory only; NULL is a
 * no-op). The caller must not use the plan afterwards, nor destroy it while
 * another host thread is enqueuing work with it; work already enqueued does
 * not reference the plan. */
void pfs_plan_destroy(pfs_plan* plan);

/* Bytes of device workspace pfs_verify needs for this plan (> 0; 0 for a
 * NULL plan): the FP32 (max, sum) pairs followed by the FP32 unnormalized
 * accumulators of every (split, request, KV head, row), each array 256-byte
 * aligned. The workspace is owned by the caller and typed by the plan's FP32
 * partials ("[Bugfix] Use FP32 state and E4M3 defaults for DFlash2", Test
 * Plan and Results: workspaces kept separate per dtype; "[Kernel][SM70] Add
 * opt-in E4M3 grouped attention with FP32 partials", final status: the
 * workspace grows from [80,8,6] LSE values to [80,8,6,2] max/sum pairs). */
int64_t pfs_plan_workspace_bytes(const pfs_plan* plan);

/* Splits per request and tokens per split chosen by the plan. */
int32_t pfs_plan_num_splits(const pfs_plan* plan);
int32_t pfs_plan_tokens_per_split(const pfs_plan* plan);

/*
 * Enqueue one verify-attention step on `stream`: the operation stated at the
 * top of this file ("[Kernel][SM70] Add opt-in E4M3 grouped attention with
 * FP32 partials", final status and historical scope list: dense small-query
 * verify over E4M3 KV with per-query device lengths; "[Bugfix] Use FP32 state
 * and E4M3 defaults for DFlash2", Purpose: FP32 partial state, FP16
 * operands and outputs, FP8 KV storage).
 *   q_fp16       device [batch, q, num_q_heads, head_dim] FP16, 16-byte aligned
 *   k_pool/v_pool device byte pools (layout above), 16-byte aligned
 *   k_scale/v_scale device [num_kv_heads] FP32 (read on device)
 *   block_table  device [batch, max_pages_per_row] int32
 *   live_len     device [batch] int32, draft tokens included
 *   out_fp16     device [batch, q, num_q_heads, head_dim] FP16, 16-byte aligned
 *   workspace    device scratch of at least pfs_plan_workspace_bytes(plan)
 *                bytes, 256-byte aligned. Its contents need no initialization
 *                and are overwritten; one workspace serves one in-flight call
 *                at a time (stream order).
 * Device-side preconditions (not checked on the host, which must not
 * synchronize): live_len values are clamped into [0, capacity]; block-table
 * entries of logical pages below ceil(L_b / page_size) must lie in
 * [0, num_pool_pages) (only those are used to address the pools; the split
 * kernel may read other entries of the row before the live length is known,
 * and ignores them); live K/V bytes are finite codes of the
 * plan's KV format (bytes no live token owns may hold anything, NaN and
 * infinity codes included).
 * All buffers are caller-owned. Returns PFS_OK or an error status; a launch
 * error is reported as PFS_ERR_LAUNCH.
 */
int32_t pfs_verify(const pfs_plan* plan, const void* q_fp16, const uint8_t* k_pool,
                   const uint8_t* v_pool, const float* k_scale, const float* v_scale,
                   const int32_t* block_table, const int32_t* live_len, void* out_fp16,
                   void* workspace, int64_t workspace_bytes, pfs_stream_t stream);

/*
 * The two phases of pfs_verify, for callers that time or schedule them apart.
 * pfs_verify_split runs the split kernel (dequant-on-load, QK^T, online
 * softmax, PV) and leaves every split's FP32 (max, sum, unnormalized PV) in
 * the workspace; pfs_verify_combine reads those partials, rescales them,
 * sums them, normalizes and writes the FP16 output. The order of the sum is
 * fixed by the plan alone (never by timing or device data), so repeated
 * calls give bit-identical outputs:
 *   - plans with at most 32 splits: splits 0, 1, 2, ... one after another;
 *   - more splits: the S splits are cut into NB contiguous blocks of
 *     ceil(S / NB) splits (NB = 16 at head_dim 128 and 256, 32 at 64);
 *     each block is summed in ascending split order, then the NB block
 *     sums are combined in a fixed pairwise tree: (0+1), (2+3), ..., then
 *     (01+23), (45+67), ..., and so on up to one sum, the lower blocks
 *     always the left operand.
 * Before each addition the two operands are rescaled to their common
 * maximum. pfs_verify_split followed by pfs_verify_combine on the same
 * stream, plan and workspace is exactly pfs_verify. Arguments and errors as
 * for pfs_verify.
 */
int32_t pfs_verify_split(const pfs_plan* plan, const void* q_fp16, const uint8_t* k_pool,
                         const uint8_t* v_pool, const float* k_scale, const int32_t* block_table,
                         const int32_t* live_len, void* workspace, int64_t workspace_bytes,
                         pfs_stream_t stream);
int32_t pfs_verify_combine(const pfs_plan* plan, const float* v_scale, const int32_t* live_len,
                           void* out_fp16, const void* workspace, int64_t workspace_bytes,
                           pfs_stream_t stream);

/*
 * pfs_verify without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The split partials live in a device
 * array inside the library instead (one per GPU, pfs_noalloc_scratch_bytes()
 * = 128 MiB, held from the first call on that GPU until the process ends;
 * the call uses the array of the GPU that runs `stream`);
 * the kernels, the arithmetic and therefore the output bits are those of
 * pfs_verify with the same plan. The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine (its first call on a device looks
 * the array's address up once). A plan whose pfs_plan_workspace_bytes()
 * exceeds the array is refused with PFS_ERR_WORKSPACE. Calls on one GPU
 * share the array: calls that overlap in time on one GPU (different
 * streams, or host threads without stream order) race and give undefined
 * outputs; stream-ordered calls are safe. Other arguments and errors as for
 * pfs_verify.
 */
int32_t pfs_verify_noalloc(const pfs_plan* plan, const void* q_fp16, const uint8_t* k_pool,
                           const uint8_t* v_pool, const float* k_scale, const float* v_scale,
                           const int32_t* block_table, const int32_t* live_len, void* out_fp16,
                           pfs_stream_t stream);

/* Size in bytes of the per-GPU device array pfs_verify_noalloc uses. */
int64_t pfs_noalloc_scratch_bytes(void);

/*
 * Paged FP8 -> FP16 bridge: the dequant-on-load path as a call of its own,
 * turning paged E4M3 (or E5M2) bytes into a dense FP16 array
 * ("[Kernel][SM70] Add opt-in E4M3 grouped attention with FP32 partials",
 * historical scope list, the bridge between the two representations).
 * Writes out_fp16 as a dense device array [batch, capacity, num_kv_heads,
 * head_dim] (capacity = max_pages_per_row * page_size): element (b, t, g, d)
 * is dec(byte) * scale[g] rounded once to the nearest FP16 (ties to even),
 * dec being the plan's KV format decoder, for the pool byte of token t of
 * request b when t < live_len[b], and +0.0 otherwise. scale is a device
 * [num_kv_heads] FP32 array, or NULL for the unscaled decode (exact: every
 * E4M3 and E5M2 value is an FP16 number). NaN codes give NaN, E5M2
 * infinities give infinities. Same alignment and precondition rules as
 * pfs_verify; no workspace. Only the plan's batch, num_kv_heads, head_dim,
 * page size, max_pages_per_row, strides and KV format are used;
 * capacity * num_kv_heads * head_dim / 16 must stay below 2^31
 * (PFS_ERR_SHAPE otherwise).
 */
int32_t pfs_dequant_paged(const pfs_plan* plan, const uint8_t* pool, const float* scale,
                          const int32_t* block_table, const int32_t* live_len, void* out_fp16,
                          pfs_stream_t stream);

/*
 * Quantize-on-write of the draft tokens (the step before verify: the
 * draft tokens' K/V enter the paged cache; "[Kernel] Preserve DFlash2
 * sampling precision and repair QUASAR TP2", Purpose: deferred accepted-slot
 * writes; "[Bugfix] Use FP32 state and E4M3 defaults for DFlash2", Test
 * Plan: KV scaling).
 *   k_new_fp16/v_new_fp16  device [batch, q, num_kv_heads, head_dim] FP16,
 *                          16-byte aligned: the K and V of each request's q
 *                          draft tokens, row i being token live_len[b] - q + i
 *   k_scale/v_scale        device [num_kv_heads] FP32
 *   k_pool/v_pool          the plan's paged pools, written in place
 * Each value x is stored as the code of the plan's KV format nearest to
 * the FP32 quotient x / scale (IEEE single division), ties to even,
 * saturating at the largest finite value (+-448 for E4M3, +-57344 for E5M2;
 * infinities included); a NaN quotient stores 0x7F (NaN in both formats).
 * Rows that would land
 * before token 0 (live_len[b] < q) are not written; no other byte of the
 * pools changes. Lengths are clamped into [0, capacity]; block-table entries
 * of the written tokens must lie in [0, num_pool_pages) (not checked on the
 * host). Uses the plan's batch, q, num_kv_heads, head_dim, page size,
 * strides and KV format; batch * q * num_kv_heads * head_dim / 8 must stay
 * below 2^31 (PFS_ERR_SHAPE otherwise; every plan pfs_plan_create accepts
 * does). Enqueue only, no allocation; capturable.
 */
int32_t pfs_kv_append(const pfs_plan* plan, const void* k_new_fp16, const void* v_new_fp16,
                      const float* k_scale, const float* v_scale, const int32_t* block_table,
                      const int32_t* live_len, uint8_t* k_pool, uint8_t* v_pool, pfs_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PFS_H */
