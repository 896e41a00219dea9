// pfs_kernels.hip -- gfx950 (CDNA4) kernels of libpfs and their launchers.
//
//   fp8x2_to_f16x2        exact FP8 -> FP16 dequant-on-load: E4M3 through
//                         the hardware v_cvt_scalef32_pk_f16_fp8 (scale 1.0),
//                         E5M2 (the explicitly requested alternative KV
//                         format: "[Bugfix] Use FP32 state and E4M3 defaults
//                         for DFlash2", Purpose) by a byte permute, an E5M2
//                         byte being the high byte of its FP16 value
//   pfs_split_kernel      per-split QK^T (MFMA), online softmax, PV (MFMA);
//                         emits FP32 (max, sum, unnormalized PV) per split
//   pfs_combine_kernel    rescales the splits, sums them in a fixed order
//                         (ascending within contiguous split blocks, then a
//                         fixed pairwise tree over the blocks: wavefront
//                         shuffles, then LDS across waves), normalizes and
//                         rounds once to FP16
//   pfs_combine_rows_kernel  the same for plans with at most 32 splits, each
//                         thread summing its row's splits in ascending order
//                         (both read only the splits that hold visible keys;
//                         a single request issues its first reads before its
//                         live length is known)
//
// The method ("[Kernel][SM70] Add opt-in E4M3 grouped attention with FP32
// partials", final status, revision 3 bullet; "[Kernel] Finalize the audited
// TP2 DFlash2 31/29 ms endpoint", Purpose) keeps FP32 max / sum and an
// unnormalized PV accumulator per KV partition until one final combine, with
// keys consumed in 64-key partitions in a fixed order. On V100 that was a
// scalar/tensor-core kernel; here it is built around CDNA4's 64-wide
// wavefronts and v_mfma_f32_16x16x32_f16.
//
// Work decomposition of the split kernel (one workgroup per split, KV head and
// row block; W = RG * TP waves):
//  * rows: the R = G*q query rows of one KV head (row r = i*G + jj: draft row
//    i, jj-th query head of the group), padded to 16-row MFMA tiles. RG row
//    groups of RT tiles each; rows beyond RG*RT tiles become row blocks of the
//    grid. A wave's FP32 accumulators (its rows x every head_dim column) and
//    its Q^T operands stay in registers.
//  * tokens: TP token lanes; lane tl folds the 32-token steps tl, tl+TP, ... of
//    the split in ascending order. The lanes of a row group are merged in a
//    fixed tree order at the end.
//  * K/V bytes go from HBM straight into LDS stages (buffer_load_dwordx4 ...
//    lds) that all waves share: a stage holds TP steps, stages are issued
//    ahead and every stage costs one barrier. Each stage is its own LDS object
//    so that the compiler waits only for the loads into the stage it reads.
//  * the byte offset of every 16-token tile of the split is computed once from
//    the block table into an LDS table; each tile's buffer descriptor ends at
//    the live length, so bytes beyond it arrive as zeros.
//  * scores are computed transposed, S^T = K * Q^T (A = K: 16 tokens x 32 dims,
//    B = Q^T: 32 dims x 16 rows), so each lane ends up holding 4 consecutive
//    tokens of one row: exactly the token slots the PV product
//    O^T = V^T * P^T needs in its B operand. P never leaves registers.
//  * K sits in LDS where each lane reads its own MFMA A operand (16 bytes of
//    one token); V rows sit with an XOR swizzle of 16-byte chunks and are read
//    transposed with ds_read_b64_tr_b8: in each 16-lane block, lane j names 8
//    bytes of one token row and every lane receives one column of 8 tokens.
//  * with four or more stages a wave folds the QK of its next step together
//    with the PV of its current one.
//
// Numerics: FP16 MFMA operands with FP32 accumulation; the per-head K scale,
// the softmax scale and log2(e) are applied to FP32 scores (inside the exp2
// argument); probabilities are p = exp2(s - m_ref + 7) against a lazily
// raised reference maximum m_ref; the row sums come from the matrix core (a
// ones row times the same FP16 operands the PV product uses); V's scale is
// applied once in the combine. Masked scores are selected to -inf and K/V
// bytes beyond the live length are never loaded (zero), so NaN (or E5M2
// infinity) tail bytes cannot leak.
//
// Probabilities (RES, the default; "[Kernel][SM70] Add opt-in E4M3 grouped
// attention with FP32 partials", historical scope: high/residual FP16 PV
// operands): each p enters PV as hi = RNE_fp16(p) plus res = RNE_fp16(p - hi),
// both multiplied with the same FP16 V operand into the same accumulators.
// p - hi is exact in FP32. Because p carries the factor 2^7, the maximum of a
// row has p >= 2^7, and res is an FP16 normal number for every key down to
// 2^-10 of that maximum, so hi + res carries p to about 22 bits with no
// scaling of the residual or of V. (On the pages p <= 1, so their residual
// needs a 2^11 scale to stay out of FP16 subnormals, and V a matching inverse
// scale.) Keys further down lose at most 2^-25 absolute, 2^-32 of the row's
// sum. Without RES (opt-in) p enters as hi only: FP16's 2^-11 relative
// rounding of each probability then reaches the output.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "pfs_internal.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kStep = 32;  // tokens per MFMA fold step (two 16-token tiles)
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, typename F>
__device__ __forceinline__ T bit_cast_(F f) {
    static_assert(sizeof(T) == sizeof(F), "size");
    return __builtin_bit_cast(T, f);
}

// Two KV bytes (bytes 2*HI and 2*HI+1 of `word`) -> two FP16 values, exact.
// E4M3: every finite value is zero or an FP16 normal number; the hardware
// conversion decodes it. E5M2: a byte is the high byte of the FP16 number it
// encodes (same exponent width and bias), so one byte permute places both
// bytes above zero low bytes (selector 0x0C yields a zero byte).
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t word) {
    if constexpr (FMT == PFS_KV_E5M2) {
        return __builtin_amdgcn_perm(word, word, HI ? 0x030C020Cu : 0x010C000Cu);
    } else {
        const f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, HI);
        return bit_cast_<uint32_t>(h);
    }
}

// 8 KV bytes (two dwords) -> 8 FP16 values as an MFMA operand.
template <int FMT>
__device__ __forceinline__ f16x8 fp8x8_to_f16x8(uint32_t w0, uint32_t w1) {
    u32x4 r;
    r.x = fp8x2_to_f16x2<FMT, false>(w0);
    r.y = fp8x2_to_f16x2<FMT, true>(w0);
    r.z = fp8x2_to_f16x2<FMT, false>(w1);
    r.w = fp8x2_to_f16x2<FMT, true>(w1);
    return bit_cast_<f16x8>(r);
}

// Residuals of a pair of probabilities: given hi = (RNE_fp16(p0),
// RNE_fp16(p1)) packed, returns (RNE_fp16(p0 - hi.x), RNE_fp16(p1 - hi.y))
// packed. v_fma_mix{lo,hi}_f16 reads the FP16 half of hi as an FP32 operand,
// forms p * 1 - hi in one fused step (exact: p - hi is an FP32 number) and
// rounds once to FP16 into the low or high half of the result: two
// instructions where the plain sequence (convert back, subtract, convert)
// takes six. Register operands only; the low half is written first, and
// the early-clobber output keeps it apart from the inputs the second
// instruction still reads.
__device__ __forceinline__ uint32_t residual_f16x2(float p0, float p1, uint32_t hi) {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, 1.0, -%3 op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixhi_f16 %0, %2, 1.0, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
        : "=&v"(r)
        : "v"(p0), "v"(p1), "v"(hi));
    return r;
}

// Maximum of two scores that are never NaN (finite or -inf): the median of
// (a, b, +inf), one v_med3_f32, where fmaxf would first quiet both inputs
// (a v_max_f32 x, x each). pinf holds +inf in a register the compiler does
// not see through, so that it keeps the median.
__device__ __forceinline__ float max_no_nan(float a, float b, float pinf) { return __builtin_amdgcn_fmed3f(a, b, pinf); }

// Max over the four lanes l, l^16, l^32, l^48 (the lane groups holding one
// result column). v_permlane16/32_swap return both halves of a swap; the max
// of the pair is the xor-16 / xor-32 butterfly step, identical in every lane.
__device__ __forceinline__ float max_over_lane_groups(float v, float pinf) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = max_no_nan(__uint_as_float(a[0]), __uint_as_float(a[1]), pinf);
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return max_no_nan(__uint_as_float(c[0]), __uint_as_float(c[1]), pinf);
}

__device__ __forceinline__ int32_t clamp_i(int64_t v, int64_t lo, int64_t hi) {
    return (int32_t)(v < lo ? lo : (v > hi ? hi : v));
}

struct SplitArgs {
    const _Float16* qptr;
    const uint8_t* kpool;
    const uint8_t* vpool;
    const float* kscale;
    const int32_t* block_table;
    const int32_t* live_len;
    float* ws_ml;
    float* ws_acc;
    int64_t page_stride;
    int64_t token_stride;
    int64_t head_stride;
    int32_t batch;
    int32_t q;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t rows;
    int32_t page_size;
    int32_t page_shift;  // log2(page_size) when it is a power of two, else -1
    int32_t max_pages;
    int32_t capacity;
    int32_t tokens_per_split;
    int32_t num_splits;
    int32_t row_blocks;
    float sm_scale_log2e;
    uint8_t qhead[pfs::kMaxQHeads];
};

// Batches: the split grid takes the live units -- (request, KV head, split)
// with split < ceil(L_b / tokens_per_split) -- in request, KV-head, split
// order. Workgroups of empty splits would otherwise sit between live ones in
// the dispatch order, and with the round-robin over the XCDs whole XCDs
// would get only the late (mostly empty) splits of every request. Unit u of
// the grid is the u-th live unit; false past the last one (uniform over the
// workgroup). Every thread calls it. cnt: NT ints of LDS scratch, map: 3 ints
// of LDS that stay untouched afterwards.
template <int NT>
__device__ bool live_unit(const SplitArgs& a, int unit, int32_t* cnt, int32_t* map, int& split, int& g, int& b) {
    const int t = threadIdx.x;
    const int per = (a.batch + NT - 1) / NT;  // requests per thread, a contiguous run
    auto nsplit = [&](int bb) {
        const int32_t L = clamp_i(a.live_len[bb], 0, a.capacity);
        return (L + a.tokens_per_split - 1) / a.tokens_per_split;
    };
    int c = 0;
    for (int k = 0; k < per; ++k)
        if (t * per + k < a.batch) c += nsplit(t * per + k);
    cnt[t] = c * a.num_kv_heads;
    __syncthreads();
    if (t < 64) {
        constexpr int E = NT / 64;  // counts per lane
        int s = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) s += cnt[t * E + e];
        int incl = s;  // inclusive scan over the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d, 64);
            if (t >= d) incl += y;
        }
        const int total = __shfl(incl, 63, 64);
        const int excl = incl - s;
        if (t == 0 && unit >= total) map[0] = -1;
        if (unit >= excl && unit < incl) {  // exactly one lane
            int rem = unit - excl;
            int e = 0;
            while (e < E - 1 && rem >= cnt[t * E + e]) rem -= cnt[t * E + e++];
            const int bb_end = min(a.batch, (t * E + e + 1) * per);
            int bb = (t * E + e) * per, n = 0;
            for (; bb < bb_end; ++bb) {
                n = nsplit(bb);
                if (rem < n * a.num_kv_heads) break;
                rem -= n * a.num_kv_heads;
            }
            const bool found = bb < bb_end && n > 0;
            map[0] = found ? bb : -1;
            map[1] = found ? rem / n : 0;
            map[2] = found ? rem % n : 0;
        }
    }
    __syncthreads();
    b = __builtin_amdgcn_readfirstlane(map[0]);
    g = __builtin_amdgcn_readfirstlane(map[1]);
    split = __builtin_amdgcn_readfirstlane(map[2]);
    return b >= 0;
}

// Compile-time geometry of the split kernel: W = RG * TP waves (RG row groups
// of RT 16-row tiles, TP token lanes), NS LDS stages of TP 32-token steps.
template <int D, int RT, int RG, int TP, int NS>
struct SplitCfg {
    static constexpr int W = RG * TP;
    static_assert(W == 4 || W == 8, "four or eight waves per split workgroup");
    static constexpr int KSTEPS = D / 32;           // QK k-steps (32 dims each)
    static constexpr int KLOADS = D / 64;           // 1 KB loads per 16-token K tile
    static constexpr int CH = D / 16;               // 16-byte chunks per token row
    static constexpr int MD = D / 16;               // PV tiles along head_dim
    static constexpr int SWB = CH < 8 ? CH : 8;     // values of the V chunk swizzle
    static constexpr int STEP_LOADS = D / 16;       // 1 KB loads per 32-token step: K tile 0, K tile 1, V
    static constexpr int STEP_BYTES = 1024 * STEP_LOADS;
    static constexpr int V_OFF = 1024 * (D / 32);   // V rows within a step
    static constexpr int STAGE_BYTES = TP * STEP_BYTES;
    static constexpr int NW = STEP_LOADS / RG;      // loads per wave per stage
    // md tiles merged per round so that one tree level of writers fits in stage 0
    static constexpr int MERGE_DIV = RG * (TP > 1 ? TP / 2 : 1) * RT * 1024;
    static constexpr bool MERGE_IN_STAGE = STAGE_BYTES >= MERGE_DIV;  // else a buffer of its own
    static constexpr int MERGE_MD =
        MERGE_IN_STAGE ? (STAGE_BYTES / MERGE_DIV < MD ? STAGE_BYTES / MERGE_DIV : MD) : 1;
    static constexpr int MERGE_EXTRA_BYTES = (TP > 1 && !MERGE_IN_STAGE) ? MERGE_DIV : 16;
    static_assert(TP == 1 || MD % MERGE_MD == 0, "merge chunking");
    static_assert(NS == 2 || NS == 4 || NS == 8, "stages");
    static constexpr int WAVES_PER_EU = W * pfs::split_workgroups_per_cu(D, TP, W) / 4;
};

// Lazy rescaling: a row's exponentials use a reference maximum m_ref and are
// exp2(s*c - m_ref + kPBias). m_ref is raised (and the accumulators rescaled)
// only when a score exceeds it by more than kTau, so P <= 2^(kPBias + kTau) =
// 2^15 stays an FP16 number, and P only becomes FP16-subnormal for terms below
// 2^-21 of the reference maximum. The offset cancels in acc / l.
constexpr float kTau = 8.0f;
constexpr float kPBias = 7.0f;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
}

// One 16-byte-per-lane load from a buffer straight into LDS: lane l's bytes
// land at lds + 16 l (buffer_load_dwordx4 ... lds; out-of-range dwords land as
// zeros). A plain device function, so that the host pass of the kernel
// templates never sees the LDS address space.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}

// Transposed 8-byte LDS read (ds_read_b64_tr_b8) at lds + byte offset.
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* lds) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(lds));
}

template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wait until at most N of this wave's vector-memory operations are in flight
// and until its LDS reads have returned, then meet the other waves at the
// workgroup barrier. The "memory" clobber keeps the compiler from moving loads
// or LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_and_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Swizzle of the 16-byte V chunks of token t (row t of a step): chunk c sits at
// chunk position c ^ swz(t). The 8 tokens one 16-lane block reads in a
// transposed read get distinct values, so the block hits distinct banks.
__device__ __forceinline__ int v_swizzle(int t, int swb) { return ((t & 3) | ((t >> 4) << 2)) & (swb - 1); }

template <int D, int RT, int RG, int TP, int NS, int FMT, bool RES>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * RG * TP, 64 * RG * TP),
                          amdgpu_waves_per_eu(SplitCfg<D, RT, RG, TP, NS>::WAVES_PER_EU,
                                              SplitCfg<D, RT, RG, TP, NS>::WAVES_PER_EU))) void
pfs_split_kernel(const SplitArgs a) {
    using C = SplitCfg<D, RT, RG, TP, NS>;
    constexpr int W = C::W, KSTEPS = C::KSTEPS, KLOADS = C::KLOADS, CH = C::CH, MD = C::MD, NW = C::NW;
    constexpr int SWB = C::SWB;
    // One LDS object per stage: the compiler tracks the direct-to-LDS loads per
    // object, so a read of one stage waits only for the loads into that stage.
    constexpr int SB = C::STAGE_BYTES;
    __shared__ __attribute__((aligned(16))) uint8_t st0[SB];
    __shared__ __attribute__((aligned(16))) uint8_t st1[SB];
    __shared__ __attribute__((aligned(16))) uint8_t st2[NS > 2 ? SB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st3[NS > 2 ? SB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st4[NS > 4 ? SB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st5[NS > 4 ? SB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st6[NS > 4 ? SB : 16];
    __shared__ __attribute__((aligned(16))) uint8_t st7[NS > 4 ? SB : 16];
    __shared__ int64_t tile_off[pfs::kTileTableEntries];  // pool byte offset of every 16-token tile of the split
    __shared__ int32_t unit_map[3];                        // (request, KV head, split) of a batch's live unit
    __shared__ float2 lds_ml[W][RT * 16];
    __shared__ __attribute__((aligned(16))) uint8_t merge_extra[C::MERGE_EXTRA_BYTES];
    auto stage = [&](auto kc) __attribute__((always_inline)) -> uint8_t* {
        constexpr int k = decltype(kc)::value;
        if constexpr (k == 0) return st0;
        else if constexpr (k == 1) return st1;
        else if constexpr (k == 2) return st2;
        else if constexpr (k == 3) return st3;
        else if constexpr (k == 4) return st4;
        else if constexpr (k == 5) return st5;
        else if constexpr (k == 6) return st6;
        else return st7;
    };

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rg = wave % RG;  // row group: RT row tiles
    const int tl = wave / RG;  // token lane: step tl of every stage
    const int lc = lane & 15;  // column within a 16-wide MFMA tile
    const int lg = lane >> 4;  // lane group (k-group of an operand, row-quad of a result)

    // 1-D grid. Workgroups x and x + 8 run on the same XCD (dispatch is
    // round-robin over the 8 XCDs), so the row blocks of one (split, KV head,
    // request) get ids 8 apart and share that XCD's L2 for their K/V reads.
    const int x = blockIdx.x;
    const int rb = (x >> 3) % a.row_blocks;
    const int unit = ((x >> 3) / a.row_blocks) * 8 + (x & 7);  // (request, KV head, split), split fastest
    if (unit >= a.num_splits * a.num_kv_heads * a.batch) return;
    int split, g, b;
    if (a.batch == 1) {
        split = unit % a.num_splits;
        g = unit / a.num_splits;
        b = 0;
    } else if (!live_unit<64 * W>(a, unit, reinterpret_cast<int32_t*>(tile_off), unit_map, split, g, b)) {
        return;  // past the last live unit
    }

    const int r_wave = rb * (RG * RT * 16) + rg * (RT * 16);  // first row of this wave
    const int32_t tok0 = split * a.tokens_per_split;
    const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
    // the first block-table entry this thread resolves, read before the live
    // length is known (any token below the capacity has an entry) so that the
    // two reads overlap
    const int32_t t_first = tok0 + 16 * (int)threadIdx.x;
    const int32_t pg_first = t_first / a.page_size;
    // (read unconditionally, at an index clamped into the row, and selected at
    // its use: a load under a branch is waited for where the branch joins)
    const int32_t page_any = bt_row[min(pg_first, a.max_pages - 1)];
    // The live length is read with a vector load (through an opaque zero
    // index): vector loads return in order, so the kernel waits for it and the
    // block-table entry together without also waiting for the Q reads below.
    int vzero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
    // +inf for max_no_nan
    float pinf;
    asm volatile("v_mov_b32 %0, 0x7f800000" : "=v"(pinf));
    const int32_t L_raw = a.live_len[b + vzero];
    const float kscale_g = a.kscale[g];
    // ---- Q^T operands in registers: (nt, ks) holds row r_wave + 16 nt + lc,
    //      dims 64(ks/2) + 16 lg + 8(ks&1) + [0, 8). Issued before the
    //      live length is known: their cold reads overlap the live-length and
    //      block-table reads instead of following them. ----
    // Padding rows (r >= rows) read row 0 here, with no branch around the
    // loads, and are zeroed after the first K/V loads are issued.
    f16x8 qop[RT][KSTEPS];
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        const int r = r_wave + nt * 16 + lc;
        const int rr = r < a.rows ? r : 0;
        const int i = rr / a.group;
        const int h = a.qhead[g * a.group + (rr % a.group)];
        const _Float16* qrow = a.qptr + (((int64_t)b * a.q + i) * a.num_q_heads + h) * D;
#pragma unroll
        for (int j = 0; j < KSTEPS / 2; ++j) {
            qop[nt][2 * j] = bit_cast_<f16x8>(*reinterpret_cast<const u32x4*>(qrow + 64 * j + 16 * lg));
            qop[nt][2 * j + 1] = bit_cast_<f16x8>(*reinterpret_cast<const u32x4*>(qrow + 64 * j + 16 * lg + 8));
        }
    }

    const int32_t L = __builtin_amdgcn_readfirstlane(clamp_i(L_raw, 0, a.capacity));
    const int32_t page_first = (t_first < a.capacity && 16 * (int)threadIdx.x < a.tokens_per_split) ? page_any : 0;
    // A split with nothing live (tok0 >= L; only single requests shorter than
    // the capacity have them) runs on with no steps and zero-size loads and
    // returns before its partial write: the combine never reads it. (An early
    // return here would let the compiler move the Q reads behind it.)
    const bool live_split = tok0 < L;
    const int32_t tok_end = min(tok0 + a.tokens_per_split, L);
    const int32_t nsteps = (tok_end - tok0 + kStep - 1) / kStep;
    const int32_t nstages = (nsteps + TP - 1) / TP;

    // ---- tile table: pool byte offset of every 16-token tile of the split ----
    {
        const int64_t head_off = (int64_t)g * a.head_stride;
        const int32_t ntiles = min((tok_end - tok0 + 15) / 16, pfs::kTileTableEntries);
        auto put = [&](int e, int32_t page) __attribute__((always_inline)) {
            const int32_t t0 = tok0 + 16 * e;
            const int32_t slot = t0 - (t0 / a.page_size) * a.page_size;
            tile_off[e] = (int64_t)page * a.page_stride + (int64_t)slot * a.token_stride + head_off;
        };
        // the first entry of each thread, from the entry read above, outside
        // any loop (so that waiting for it does not wait for the Q reads)
        if ((int)threadIdx.x < ntiles) put(threadIdx.x, page_first);
        for (int e = threadIdx.x + 64 * W; e < ntiles; e += 64 * W) put(e, bt_row[(tok0 + 16 * e) / a.page_size]);
    }

    // causal limit of this lane's row in each row tile: keys [0, lim) are visible.
    // Padding rows (r >= rows) keep lim = L: their Q is zero, their results are
    // never written and MFMA columns do not mix, so they need no masking.
    int32_t lim[RT];
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        const int r = r_wave + nt * 16 + lc;
        lim[nt] = (r < a.rows) ? clamp_i((int64_t)L - a.q + r / a.group + 1, 0, L) : L;
    }
    const int32_t lim_lo = clamp_i((int64_t)L - a.q + 1, 0, L);  // smallest limit of any real row
    float cscale = a.sm_scale_log2e * kscale_g;  // score scale, log2 domain

    f32x4 acc[MD][RT];
    f32x4 lacc[RT];  // row sums, computed by the matrix core from the same FP16 operands
    float mref[RT], nb[RT];
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        mref[nt] = -INFINITY;
        nb[nt] = 0.0f;
        lacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int md = 0; md < MD; ++md) acc[md][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // A operand of the row-sum tile: row 0 all ones, rows 1..15 zero
    const _Float16 one_or_zero = (lc == 0) ? (_Float16)1.0f : (_Float16)0.0f;
    const f16x8 ones = f16x8{one_or_zero, one_or_zero, one_or_zero, one_or_zero,
                             one_or_zero, one_or_zero, one_or_zero, one_or_zero};

    // transposed V reads: lane j of each 16-lane block names 8 bytes of token
    // tok(lg, j >> 1) of the step, the (j & 1) half of a 16-byte chunk. With
    // the chunk swizzle below SWB, tile md sits at vaddr[md % SWB] + 16 SWB (md / SWB).
    const int tr_tok = ((lc >> 1) < 4 ? 0 : 16) + 4 * lg + ((lc >> 1) & 3);
    // Both read addresses include this token lane's step within the stage.
    int vaddr[SWB];
#pragma unroll
    for (int m = 0; m < SWB; ++m)
        vaddr[m] = tl * C::STEP_BYTES + C::V_OFF + tr_tok * D + 8 * (lc & 1) + 16 * (m ^ v_swizzle(tr_tok, SWB));
    const int kaddr = tl * C::STEP_BYTES + 16 * lane;

    // ---- direct-to-LDS loads. A stage holds TP steps; step s of a stage is
    // STEP_LOADS 1 KB loads in four groups of G = D / 64: K tile 0, K tile 1,
    // V tile 0, V tile 1 (load i = group * G + jg at byte 1024 i of the step).
    // Lane (c, g) of K load jg of a tile reads bytes [64 jg + 16 g, +16) of
    // token c: in LDS it sits exactly where that lane reads its MFMA A operand
    // for k-steps 2jg and 2jg+1. V load j = i - 2G puts stage chunk
    // p = 64 j + lane, which is token t = p / CH, chunk (p % CH) ^ swz(t), at
    // byte 16 p of the V rows. Each wave issues NW loads of step tl of every
    // stage: when RG divides G, loads [rg G/RG, (rg+1) G/RG) of every group
    // (pool and tile fixed per load); otherwise loads [rg NW, rg NW + NW).
    // Every 16-token tile has a buffer descriptor whose record count stops at
    // the live length: bytes beyond it (and whole tiles past the split) land
    // in LDS as zeros. ----
    constexpr int G = D / 64;
    constexpr bool BY_GROUP = (G % RG) == 0;
    constexpr int PG = BY_GROUP ? G / RG : 1;  // loads per group per wave
    uint32_t voff[NW];
    int ld_dst[NW];   // byte offset of each load in the step (uniform)
    int ld_group[NW]; // group of each load (compile-time when BY_GROUP)
#pragma unroll
    for (int jj = 0; jj < NW; ++jj) {
        int group, jg;
        if constexpr (BY_GROUP) {
            group = jj / PG;
            jg = rg * PG + jj % PG;
        } else {
            const int i = rg * NW + jj;
            group = i / G;
            jg = i % G;
        }
        ld_group[jj] = group;
        ld_dst[jj] = 1024 * (group * G + jg);
        if (group < 2) {
            voff[jj] = (uint32_t)lc * (uint32_t)a.token_stride + 64u * jg + 16u * lg;
        } else {
            const int p = 64 * ((group - 2) * G + jg) + lane;
            const int t = p / CH;
            const int c = (p % CH) ^ v_swizzle(t, SWB);
            voff[jj] = (uint32_t)(t & 15) * (uint32_t)a.token_stride + 16u * (uint32_t)c;
        }
    }
    // Loads of a stage are prepared one stage ahead: the tile offsets come from
    // the LDS table (a read whose latency hides behind a fold) and the record
    // counts from the live length.
    struct Pending {
        uint32_t off_lo[2], off_hi[2];  // tile byte offsets (VGPRs, uniform values)
        int32_t n[2];                   // live tokens of each tile
    };
    auto prep = [&](int32_t ss) __attribute__((always_inline)) -> Pending {
        Pending pd;
        const int32_t st = ss * TP + tl;
        const int32_t t_step = tok0 + st * kStep;
        const int32_t e = min(2 * st, pfs::kTileTableEntries - 2);
        const u32x2 o0 = *reinterpret_cast<const u32x2*>(&tile_off[e]);
        const u32x2 o1 = *reinterpret_cast<const u32x2*>(&tile_off[e + 1]);
        pd.off_lo[0] = o0.x;
        pd.off_hi[0] = o0.y;
        pd.off_lo[1] = o1.x;
        pd.off_hi[1] = o1.y;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            pd.n[mt] = (st < nsteps) ? min(max(L - (t_step + 16 * mt), 0), 16) : 0;
        return pd;
    };
    auto fire = [&](const Pending& pd, uint8_t* stg) __attribute__((always_inline)) {
        __amdgpu_buffer_rsrc_t rs[4];  // per group: K tile 0, K tile 1, V tile 0, V tile 1
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            // every value of a buffer descriptor must be wave-uniform (SGPRs)
            const int32_t n = __builtin_amdgcn_readfirstlane(pd.n[mt]);
            uint64_t off = 0;
            uint32_t rec = 0;
            if (n > 0) {
                off = ((uint64_t)__builtin_amdgcn_readfirstlane(pd.off_hi[mt]) << 32) |
                      __builtin_amdgcn_readfirstlane(pd.off_lo[mt]);
                rec = (uint32_t)n * (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a.token_stride);
            }
            rs[mt] = tile_rsrc(a.kpool + off, rec);
            rs[2 + mt] = tile_rsrc(a.vpool + off, rec);
        }
        uint8_t* dst = stg + tl * C::STEP_BYTES;
#pragma unroll
        for (int jj = 0; jj < NW; ++jj) {
            __amdgpu_buffer_rsrc_t r;
            if constexpr (BY_GROUP) {
                r = rs[jj / PG];
            } else {
                const int gi = ld_group[jj];
                r = gi == 0 ? rs[0] : (gi == 1 ? rs[1] : (gi == 2 ? rs[2] : rs[3]));
            }
            load_lds16(r, dst + ld_dst[jj], voff[jj]);
        }
    };

    // ---- the fold of one 32-token step, in pieces: QK^T (per 64-dim chunk of
    // K), the online softmax, PV (per 4 head_dim tiles). With four or more
    // stages the loop runs QK of the next step between the softmax and the PV
    // pieces of the current one, so the matrix core has work while the
    // softmax's dependent VALU chain runs. ----
    struct Scores {
        f32x4 v[2][RT];  // S^T tiles: 16 tokens (mt) x 16 rows (nt)
    };
    auto qk_zero = [&](Scores& sc) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < RT; ++nt) sc.v[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // K chunk j: bytes [64 j, 64 j + 64) of the 32 tokens (both 16-token
    // tiles), the A operands of k-steps 2j and 2j+1
    struct KChunk {
        u32x4 w[2];
    };
    auto k_read = [&](const uint8_t* sbase, int j) __attribute__((always_inline)) -> KChunk {
        KChunk kc;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            kc.w[mt] = *reinterpret_cast<const u32x4*>(sbase + kaddr + 1024 * (mt * KLOADS + j));
        return kc;
    };
    auto qk_fold = [&](const KChunk& kc, int j, Scores& sc) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            const f16x8 k_lo = fp8x8_to_f16x8<FMT>(kc.w[mt].x, kc.w[mt].y);
            const f16x8 k_hi = fp8x8_to_f16x8<FMT>(kc.w[mt].z, kc.w[mt].w);
#pragma unroll
            for (int nt = 0; nt < RT; ++nt) {
                sc.v[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_lo, qop[nt][2 * j], sc.v[mt][nt], 0, 0, 0);
                sc.v[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_hi, qop[nt][2 * j + 1], sc.v[mt][nt], 0, 0, 0);
            }
        }
    };
    auto qk_chunk = [&](const uint8_t* sbase, int j, Scores& sc) __attribute__((always_inline)) {
        qk_fold(k_read(sbase, j), j, sc);
    };
    // online softmax, log2 domain, lazy reference maximum. Scores are scaled
    // before masking, so a masked score is exactly -inf for any finite K scale.
    // The FP16 operands of one step's probabilities: hi = RNE_fp16(p) and,
    // with RES, res = RNE_fp16(p - hi), so that hi + res carries p to about
    // 22 bits.
    struct Probs {
        f16x8 hi[RT];
        f16x8 res[RT];
    };
    auto softmax = [&](int32_t t_step, const Scores& sc, bool edge, Probs& pr) __attribute__((always_inline)) {
        float xs[RT][8];
        float smax[RT];
        bool need = false;
#pragma unroll
        for (int nt = 0; nt < RT; ++nt)
#pragma unroll
            for (int e = 0; e < 8; ++e) xs[nt][e] = sc.v[e >> 2][nt][e & 3];
        if (edge) {  // uniform: only steps that cross some row's causal limit or the live length
#pragma unroll
            for (int nt = 0; nt < RT; ++nt)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    xs[nt][e] *= cscale;
                    if (t_step + (e >> 2) * 16 + 4 * lg + (e & 3) >= lim[nt]) xs[nt][e] = -INFINITY;
                }
        }
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) {
            const float m01 = max_no_nan(xs[nt][0], xs[nt][1], pinf), m23 = max_no_nan(xs[nt][2], xs[nt][3], pinf);
            const float m45 = max_no_nan(xs[nt][4], xs[nt][5], pinf), m67 = max_no_nan(xs[nt][6], xs[nt][7], pinf);
            const float mx = max_no_nan(max_no_nan(m01, m23, pinf), max_no_nan(m45, m67, pinf), pinf);
            smax[nt] = max_over_lane_groups(mx, pinf);
            if (!edge) smax[nt] *= cscale;
            need |= (smax[nt] > mref[nt] + kTau);
        }
        if (__builtin_expect(__any(need), 0)) {
#pragma unroll
            for (int nt = 0; nt < RT; ++nt) {
                const float m_new = fmaxf(mref[nt], smax[nt]);
                if (m_new != mref[nt]) {
                    const float al = (mref[nt] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mref[nt] - m_new);
                    lacc[nt] *= al;
#pragma unroll
                    for (int md = 0; md < MD; ++md) acc[md][nt] *= al;
                    mref[nt] = m_new;
                    nb[nt] = kPBias - m_new;
                }
            }
        }
        // P = exp2(x - m_ref + kPBias); masked terms are exp2(-inf) = 0 (nb is
        // finite: it only changes together with a finite m_ref)
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) {
            uint32_t hw[4], rw[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float c = edge ? 1.0f : cscale;
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[nt][e], c, nb[nt]));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(xs[nt][e + 1], c, nb[nt]));
                hw[e >> 1] = bit_cast_<uint32_t>(f16x2{(_Float16)p0, (_Float16)p1});
                if constexpr (RES) rw[e >> 1] = residual_f16x2(p0, p1, hw[e >> 1]);
            }
            pr.hi[nt] = bit_cast_<f16x8>(u32x4{hw[0], hw[1], hw[2], hw[3]});
            if constexpr (RES) pr.res[nt] = bit_cast_<f16x8>(u32x4{rw[0], rw[1], rw[2], rw[3]});
        }
    };
    // O^T += V^T * P^T for head_dim tiles [md0, md0 + 4), V^T read transposed from LDS
    struct VChunk {
        i32x2 w[4];
    };
    auto v_read = [&](const uint8_t* sbase, int md0) __attribute__((always_inline)) -> VChunk {
        VChunk vc;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int md = md0 + u;
            vc.w[u] = lds_read_tr8(sbase + vaddr[md % SWB] + 16 * SWB * (md / SWB));
        }
        return vc;
    };
    // (with RES, also O^T += V^T * RES^T, against the same V operand and into
    // the same accumulators, after the high parts of the chunk)
    auto pv_fold = [&](const VChunk& vc, int md0, const Probs& pr) __attribute__((always_inline)) {
        f16x8 vop[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            vop[u] = fp8x8_to_f16x8<FMT>((uint32_t)vc.w[u].x, (uint32_t)vc.w[u].y);
#pragma unroll
            for (int nt = 0; nt < RT; ++nt)
                acc[md0 + u][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[u], pr.hi[nt], acc[md0 + u][nt], 0, 0, 0);
        }
        if constexpr (RES) {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int nt = 0; nt < RT; ++nt)
                    acc[md0 + u][nt] =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[u], pr.res[nt], acc[md0 + u][nt], 0, 0, 0);
        }
    };
    auto pv_chunk = [&](const uint8_t* sbase, int md0, const Probs& pr) __attribute__((always_inline)) {
        pv_fold(v_read(sbase, md0), md0, pr);
    };
    // l += 1 * P^T (row sums from the same FP16 operands; with RES, + 1 * RES^T)
    auto row_sums = [&](const Probs& pr) __attribute__((always_inline)) {
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) {
            lacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pr.hi[nt], lacc[nt], 0, 0, 0);
            if constexpr (RES) lacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pr.res[nt], lacc[nt], 0, 0, 0);
        }
    };

    __syncthreads();  // tile table ready

    constexpr bool PIPE = NS >= 4;
    static_for<NS - 1>([&](auto kc) __attribute__((always_inline)) { fire(prep(decltype(kc)::value), stage(kc)); });
    Pending pend = prep(NS - 1);  // loads of the next stage to issue
    // (after the first loads are issued: these wait for Q only when there are
    // padding rows or the scale is negative)
    if (r_wave + 16 * RT > a.rows) {
#pragma unroll
        for (int nt = 0; nt < RT; ++nt)
            if (r_wave + nt * 16 + lc >= a.rows)
#pragma unroll
                for (int ks = 0; ks < KSTEPS; ++ks) qop[nt][ks] = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    if (cscale < 0.0f) {  // keep the scale non-negative: max(s) * c is then the max of the scaled scores
        cscale = -cscale;
#pragma unroll
        for (int nt = 0; nt < RT; ++nt)
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) qop[nt][ks] = -qop[nt][ks];
    }
    if constexpr (PIPE) {
        // ---- NS - 2 stages in flight ahead of the one whose QK is folded ----
        Scores sc_cur;
        Probs pop;
        wait_vm_and_barrier<(NS - 2) * NW>();  // stage 0 ready
        qk_zero(sc_cur);
#pragma unroll
        for (int j = 0; j < KLOADS; ++j) {
            qk_chunk(stage(std::integral_constant<int, 0>{}), j, sc_cur);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int32_t ss0 = 0; ss0 < nstages; ss0 += NS) {
            static_for<NS>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                const int32_t ss = ss0 + k;
                // stage ss + 1 is complete once at most (NS - 3) * NW of this
                // wave's loads are younger; past the barrier every wave is done
                // with stage ss - 1, which the issue refills
                wait_vm_and_barrier<(NS - 3) * NW>();
                fire(pend, stage(std::integral_constant<int, (k + NS - 1) % NS>{}));
                pend = prep(ss + NS);
                const int32_t st = ss * TP + tl;
                if (ss < nstages && st < nsteps) {
                    const int32_t t_step = tok0 + st * kStep;
                    const uint8_t* sb = stage(kc);
                    const uint8_t* sb_next = stage(std::integral_constant<int, (k + 1) % NS>{});
                    Scores sc_next;  // QK of this wave's next step (stage ss + 1; zeros or unused past the end)
                    // after the softmax, group c folds K chunk c of the next step
                    // and V tiles [4c, 4c + 4) of this one; the LDS reads of
                    // group c + 1 are issued before group c computes
                    KChunk k_nxt = k_read(sb_next, 0), k_cur;
                    VChunk v_nxt = v_read(sb, 0), v_cur;
                    softmax(t_step, sc_cur, t_step + kStep > lim_lo, pop);
                    qk_zero(sc_next);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int c = 0; c < KLOADS; ++c) {
                        k_cur = k_nxt;
                        v_cur = v_nxt;
                        if (c + 1 < KLOADS) {
                            k_nxt = k_read(sb_next, c + 1);
                            v_nxt = v_read(sb, 4 * (c + 1));
                        }
                        qk_fold(k_cur, c, sc_next);
                        pv_fold(v_cur, 4 * c, pop);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    row_sums(pop);
                    sc_cur = sc_next;
                }
            });
        }
    } else {
        // ---- NS - 1 stages in flight ahead of the one being folded ----
        for (int32_t ss0 = 0; ss0 < nstages; ss0 += NS) {
            static_for<NS>([&](auto kc) __attribute__((always_inline)) {
                constexpr int k = decltype(kc)::value;
                const int32_t ss = ss0 + k;
                // this wave's loads of stage ss are done once at most (NS - 2) * NW
                // younger ones are in flight; the barrier makes every wave's loads of
                // stage ss visible and retires every read of the stage refilled next
                wait_vm_and_barrier<(NS - 2) * NW>();
                fire(pend, stage(std::integral_constant<int, (k + NS - 1) % NS>{}));
                pend = prep(ss + NS);
                const int32_t st = ss * TP + tl;
                if (ss < nstages && st < nsteps) {
                    const int32_t t_step = tok0 + st * kStep;
                    const uint8_t* sb = stage(kc);
                    Scores sc;
                    Probs pop;
                    qk_zero(sc);
#pragma unroll
                    for (int j = 0; j < KLOADS; ++j) {
                        qk_chunk(sb, j, sc);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    softmax(t_step, sc, t_step + kStep > lim_lo, pop);
#pragma unroll
                    for (int c = 0; c < KLOADS; ++c) {
                        pv_chunk(sb, 4 * c, pop);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    row_sums(pop);
                }
            });
        }
    }
    wait_vm_and_barrier<0>();  // no load into LDS is still in flight

    // ---- merge the TP token lanes of each row group: ((tl0 + tl2) + (tl1 + tl3)) ... ----
    const int64_t slot_base = (((int64_t)split * a.batch + b) * a.num_kv_heads + g) * a.rows;
    float Ltot[RT];
    if constexpr (TP == 1) {
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) Ltot[nt] = lacc[nt][0];  // valid in lane group 0
    } else {
        // row sums live in result row 0 of the ones tile: lanes of lane group 0, element 0
        if (lg == 0) {
#pragma unroll
            for (int nt = 0; nt < RT; ++nt) lds_ml[wave][nt * 16 + lc] = make_float2(mref[nt], lacc[nt][0]);
        }
        __syncthreads();
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) {
            float mm = -INFINITY;
#pragma unroll
            for (int t = 0; t < TP; ++t) mm = fmaxf(mm, lds_ml[rg + RG * t][nt * 16 + lc].x);
            float f[TP], lsum[TP];
#pragma unroll
            for (int t = 0; t < TP; ++t) {
                const float2 ml = lds_ml[rg + RG * t][nt * 16 + lc];
                f[t] = (ml.x == -INFINITY) ? 0.0f : (ml.x == mm ? 1.0f : __builtin_amdgcn_exp2f(ml.x - mm));
                lsum[t] = f[t] * ml.y;
            }
#pragma unroll
            for (int h = TP / 2; h >= 1; h >>= 1)
#pragma unroll
                for (int t = 0; t < h; ++t) lsum[t] += lsum[t + h];
            Ltot[nt] = lsum[0];
            float fmine = f[0];
#pragma unroll
            for (int t = 1; t < TP; ++t)
                if (t == tl) fmine = f[t];
            mref[nt] = mm;
#pragma unroll
            for (int md = 0; md < MD; ++md) acc[md][nt] *= fmine;
        }
        u32x4* mbuf = reinterpret_cast<u32x4*>(C::MERGE_IN_STAGE ? st0 : merge_extra);
        constexpr int MM = C::MERGE_MD;
#pragma unroll
        for (int h = TP / 2; h >= 1; h >>= 1) {
#pragma unroll
            for (int m0 = 0; m0 < MD; m0 += MM) {
                if (tl >= h && tl < 2 * h) {
                    const int slot = (tl - h) * RG + rg;
#pragma unroll
                    for (int md = m0; md < m0 + MM; ++md)
#pragma unroll
                        for (int nt = 0; nt < RT; ++nt)
                            mbuf[(slot * MM * RT + (md - m0) * RT + nt) * 64 + lane] = bit_cast_<u32x4>(acc[md][nt]);
                }
                __syncthreads();
                if (tl < h) {
                    const int slot = tl * RG + rg;
#pragma unroll
                    for (int md = m0; md < m0 + MM; ++md)
#pragma unroll
                        for (int nt = 0; nt < RT; ++nt)
                            acc[md][nt] += bit_cast_<f32x4>(mbuf[(slot * MM * RT + (md - m0) * RT + nt) * 64 + lane]);
                }
                __syncthreads();
            }
        }
        if (tl != 0) return;
    }

    if (!live_split) return;
    // ---- emit the split partial: (reference max, sum) and the unnormalized PV
    // (non-temporal stores: the combine reads them once, from beyond the L2) ----
    // accumulator element i of d tile md is column 16 md + 4 lg + i of row r
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        const int r = r_wave + nt * 16 + lc;
        if (r >= a.rows) continue;
        if (lg == 0) reinterpret_cast<float2*>(a.ws_ml)[slot_base + r] = make_float2(mref[nt], Ltot[nt]);
        float* dst = a.ws_acc + (slot_base + r) * D + 4 * lg;
#pragma unroll
        for (int md = 0; md < MD; ++md) __builtin_nontemporal_store(acc[md][nt], reinterpret_cast<f32x4*>(dst + 16 * md));
    }
}

struct CombineArgs {
    const float* ws_ml;
    const float* ws_acc;
    const float* vscale;
    const int32_t* live_len;
    _Float16* out;
    int32_t batch;
    int32_t q;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t rows;
    int32_t capacity;
    int32_t tokens_per_split;
    int32_t num_splits;
    int32_t head_dim;
    uint8_t qhead[pfs::kMaxQHeads];
};

// The running state of a fold over splits: reference maximum M (log2 domain),
// weighted sum lw and weighted accumulators acc of 4 columns.
struct FoldState {
    float M, lw;
    f32x4 acc;
};

// Folds N splits (their (max, sum) pairs v and accumulators x, in ascending
// split order; invalid ones selected out beforehand as (-inf, 0) and zeros)
// into st: the maximum is raised first, the running state rescaled once, then
// the splits are added in order.
template <int N>
__device__ __forceinline__ void fold_splits(FoldState& st, const float2 (&v)[N], const f32x4 (&x)[N]) {
    float cm = st.M;
#pragma unroll
    for (int u = 0; u < N; ++u) cm = fmaxf(cm, v[u].x);
    if (cm != st.M) {  // a larger maximum: rescale the running state (empty state: factor 0)
        const float al = (st.M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(st.M - cm);
        st.lw *= al;
        st.acc *= al;
        st.M = cm;
    }
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const float f = (v[u].x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(v[u].x - st.M);
        st.lw += f * v[u].y;
        st.acc += f * x[u];
    }
}

// Loads the partials of N consecutive splits s0, s0 + 1, ... of one row
// (slot0 + s * stride), at indices clamped to split s_last so that no load
// sits under a branch; the caller selects the valid ones. Clamped loads
// repeat an address already being read and fetch nothing more from HBM.
template <int N>
__device__ __forceinline__ void load_splits(const CombineArgs& a, int64_t slot0, int64_t stride, int s0, int s_last,
                                            int col0, float2 (&v)[N], f32x4 (&x)[N]) {
    const float2* ml = reinterpret_cast<const float2*>(a.ws_ml);
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const int64_t slot = slot0 + (int64_t)min(s0 + u, s_last) * stride;
        v[u] = ml[slot];
        x[u] = *reinterpret_cast<const f32x4*>(a.ws_acc + slot * a.head_dim + col0);
    }
}

template <int N>
__device__ __forceinline__ void select_splits(int s0, int s_lim, float2 (&v)[N], f32x4 (&x)[N]) {
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const bool ok = s0 + u < s_lim;
        v[u] = ok ? v[u] : make_float2(-INFINITY, 0.0f);
        x[u] = ok ? x[u] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// Many splits: one workgroup of NW = 8 waves per (request, KV head, row,
// column slice of 4 CGW columns; CGW = 32, or 16 at head_dim 64). Lane
// (sl, cg) = (lane / CGW, lane % CGW) of wave w owns columns 4 cg .. 4 cg + 3
// of the slice and split block SL w + sl (SL = 64 / CGW), so one load
// instruction of a wave reads SL runs of 16 CGW contiguous bytes (512 B at
// head_dim 128 and 256): long runs, not the number of waves, set how fast the
// one burst of partial reads completes. The plan's splits are cut into
// SL NW contiguous blocks of C = ceil(S / (SL NW)) splits (16 blocks, 32 at
// head_dim 64); a lane folds its block in ascending order, kCombineRound
// splits at a time with their loads issued together (the first round before
// the live length has arrived: slots past the visible splits are read and
// selected out). The block states are then merged in a fixed pairwise tree:
// inside each wave by cross-lane permutes over the lane bits that select sl,
// then across the waves through LDS, (w0, w1), (w2, w3), ..., then pairs of
// pairs; the lower blocks are always the left operand. One IEEE division, one
// RNE to FP16.
constexpr int kCombineWaves = 8;  // waves per workgroup
constexpr int kCombineRound = 8;
constexpr int kCombineRowSplits = 32;  // at most this many splits: pfs_combine_rows_kernel

__host__ __device__ constexpr int combine_cgw(int d) { return d / 4 < 32 ? d / 4 : 32; }

__device__ __forceinline__ float lane_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Merges two fold states, l the lower split blocks: the larger maximum, each
// side rescaled by its own factor (0 for an empty side).
__device__ __forceinline__ FoldState merge_states(const FoldState& l, const FoldState& r) {
    FoldState o;
    o.M = fmaxf(l.M, r.M);
    const float fl = (l.M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(l.M - o.M);
    const float fr = (r.M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(r.M - o.M);
    o.lw = fl * l.lw + fr * r.lw;
    o.acc = fl * l.acc + fr * r.acc;
    return o;
}

template <int D, bool AHEAD>
__global__ __launch_bounds__(64 * kCombineWaves) void pfs_combine_kernel(const CombineArgs a) {
    constexpr int CGW = combine_cgw(D);  // 4-column groups per wave
    constexpr int SL = 64 / CGW;         // split blocks per wave
    constexpr int NW = kCombineWaves;
    constexpr int SLICES = D / (4 * CGW);
    constexpr int R = kCombineRound;
    __shared__ float part[NW - 1][CGW][6];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sl = lane / CGW;
    const int cg = lane % CGW;
    const int r = blockIdx.x / SLICES;
    const int col0 = (blockIdx.x % SLICES) * 4 * CGW + 4 * cg;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int i = r / a.group;
    const int h = a.qhead[g * a.group + (r % a.group)];
    _Float16* dst = a.out + (((int64_t)b * a.q + i) * a.num_q_heads + h) * D + col0;
    const int64_t stride = (int64_t)a.batch * a.num_kv_heads * a.rows;  // between splits
    const int64_t slot0 = ((int64_t)b * a.num_kv_heads + g) * a.rows + r;
    const int C = (a.num_splits + SL * NW - 1) / (SL * NW);
    const int s_begin = (wave * SL + sl) * C;
    const int s_end = min(s_begin + C, a.num_splits);

    // AHEAD (one request): the first round of loads goes out before the live
    // length arrives (its splits are normally all visible). A batch's lengths
    // vary, so there the loads wait for it and stop at the last visible split.
    const int32_t L_raw = a.live_len[b];
    float2 v[R];
    f32x4 x[R];
    if constexpr (AHEAD) load_splits<R>(a, slot0, stride, s_begin, a.num_splits - 1, col0, v, x);
    const int32_t L = clamp_i(L_raw, 0, a.capacity);
    const int32_t n = clamp_i((int64_t)L - a.q + i + 1, 0, L);
    const int ns = (n + a.tokens_per_split - 1) / a.tokens_per_split;  // splits holding visible keys
    const int s_lim = min(s_end, ns);
    // clamped loads repeat a visible split (or split 0); with AHEAD the loads
    // of the first round could not know the live length, nor do the others
    const int s_last = AHEAD ? a.num_splits - 1 : max(ns - 1, 0);
    if constexpr (!AHEAD) load_splits<R>(a, slot0, stride, s_begin, s_last, col0, v, x);
    FoldState st{-INFINITY, 0.0f, f32x4{0.f, 0.f, 0.f, 0.f}};
    select_splits<R>(s_begin, s_lim, v, x);
    fold_splits<R>(st, v, x);
    for (int s0 = s_begin + R; s0 < s_lim; s0 += R) {
        load_splits<R>(a, slot0, stride, s0, s_last, col0, v, x);
        select_splits<R>(s0, s_lim, v, x);
        fold_splits<R>(st, v, x);
    }
    // pairwise tree over the wave's SL blocks (the lane bits above cg)
#pragma unroll
    for (int bit = CGW; bit < 64; bit <<= 1) {
        FoldState o;
        o.M = lane_xor(st.M, bit);
        o.lw = lane_xor(st.lw, bit);
#pragma unroll
        for (int c = 0; c < 4; ++c) o.acc[c] = lane_xor(st.acc[c], bit);
        st = (lane & bit) ? merge_states(o, st) : merge_states(st, o);
    }
    // then the waves: lanes sl == 0 of waves 1.. hand their states to wave 0
    if (wave != 0 && sl == 0) {
        float* q = part[wave - 1][cg];
        q[0] = st.M;
        q[1] = st.lw;
#pragma unroll
        for (int c = 0; c < 4; ++c) q[2 + c] = st.acc[c];
    }
    __syncthreads();
    if (wave != 0 || sl != 0) return;
    FoldState w[NW];
    w[0] = st;
#pragma unroll
    for (int k = 1; k < NW; ++k) {
        const float* q = part[k - 1][cg];
        w[k].M = q[0];
        w[k].lw = q[1];
#pragma unroll
        for (int c = 0; c < 4; ++c) w[k].acc[c] = q[2 + c];
    }
#pragma unroll
    for (int span = 1; span < NW; span <<= 1)
#pragma unroll
        for (int k = 0; k + span < NW; k += 2 * span) w[k] = merge_states(w[k], w[k + span]);
    st = w[0];
    if (n == 0) {  // nothing visible: defined output +0.0
        *reinterpret_cast<uint2*>(dst) = make_uint2(0u, 0u);
        return;
    }
    const float vs = a.vscale[g];
    f16x2 o01 = f16x2{(_Float16)((st.acc[0] * vs) / st.lw), (_Float16)((st.acc[1] * vs) / st.lw)};
    f16x2 o23 = f16x2{(_Float16)((st.acc[2] * vs) / st.lw), (_Float16)((st.acc[3] * vs) / st.lw)};
    *reinterpret_cast<uint2*>(dst) = make_uint2(bit_cast_<uint32_t>(o01), bit_cast_<uint32_t>(o23));
}

// Few splits (at most kCombineRowSplits): one thread per 4 columns of one row
// folds every visible split of that row itself, in ascending order, 8 at a
// time (the first 8 loads issued before the live length has arrived), with
// no cross-lane merge; a workgroup covers 1024 / D whole rows.
template <int D, bool AHEAD>
__global__ __launch_bounds__(256) void pfs_combine_rows_kernel(const CombineArgs a) {
    constexpr int R = 8;
    constexpr int TPR = D / 4;        // threads per row
    constexpr int RPW = 256 / TPR;    // rows per workgroup
    const int t = threadIdx.x;
    const int r = blockIdx.x * RPW + t / TPR;
    if (r >= a.rows) return;
    const int col0 = 4 * (t % TPR);
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int i = r / a.group;
    const int h = a.qhead[g * a.group + (r % a.group)];
    _Float16* dst = a.out + (((int64_t)b * a.q + i) * a.num_q_heads + h) * D + col0;
    const int64_t stride = (int64_t)a.batch * a.num_kv_heads * a.rows;
    const int64_t slot0 = ((int64_t)b * a.num_kv_heads + g) * a.rows + r;

    // (the first round ahead of the live length with AHEAD, as in
    // pfs_combine_kernel)
    const int32_t L_raw = a.live_len[b];
    float2 v[R];
    f32x4 x[R];
    if constexpr (AHEAD) load_splits<R>(a, slot0, stride, 0, a.num_splits - 1, col0, v, x);
    const int32_t L = clamp_i(L_raw, 0, a.capacity);
    const int32_t n = clamp_i((int64_t)L - a.q + i + 1, 0, L);
    if (n == 0) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(0u, 0u);
        return;
    }
    const int ns = min((n + a.tokens_per_split - 1) / a.tokens_per_split, a.num_splits);
    if constexpr (!AHEAD) load_splits<R>(a, slot0, stride, 0, ns - 1, col0, v, x);
    const int s_last = AHEAD ? a.num_splits - 1 : ns - 1;
    FoldState st{-INFINITY, 0.0f, f32x4{0.f, 0.f, 0.f, 0.f}};
    select_splits<R>(0, ns, v, x);
    fold_splits<R>(st, v, x);
    for (int s0 = R; s0 < ns; s0 += R) {
        load_splits<R>(a, slot0, stride, s0, s_last, col0, v, x);
        select_splits<R>(s0, ns, v, x);
        fold_splits<R>(st, v, x);
    }
    const float vs = a.vscale[g];
    f16x2 o01 = f16x2{(_Float16)((st.acc[0] * vs) / st.lw), (_Float16)((st.acc[1] * vs) / st.lw)};
    f16x2 o23 = f16x2{(_Float16)((st.acc[2] * vs) / st.lw), (_Float16)((st.acc[3] * vs) / st.lw)};
    *reinterpret_cast<uint2*>(dst) = make_uint2(bit_cast_<uint32_t>(o01), bit_cast_<uint32_t>(o23));
}

template <int D, int RT, int RG, int FMT, bool RES, bool NARROW = false>
hipError_t launch_split(const SplitArgs& a, hipStream_t stream) {
    constexpr int W = pfs::split_waves(D, RG, NARROW);
    constexpr int TP = W / RG;
    constexpr int NS = pfs::split_stages(D, TP, W);
    const int64_t units = (int64_t)a.num_splits * a.num_kv_heads * a.batch;
    const int64_t wgs = ((units + 7) / 8) * 8 * a.row_blocks;
    hipLaunchKernelGGL((pfs_split_kernel<D, RT, RG, TP, NS, FMT, RES>), dim3((unsigned)wgs), dim3(64 * W), 0,
                       stream, a);
    return hipGetLastError();
}

// Row groups above one occur only with the most row tiles a wave can hold.
// The plan's wave count must be the one the kernel template derives.
template <int D, int RT, int FMT, bool RES>
hipError_t launch_split_rt(const SplitArgs& a, int32_t row_groups, int32_t waves, hipStream_t stream) {
    if constexpr (RT > pfs::max_row_tiles(D)) {
        return hipErrorInvalidValue;
    } else {
        if (row_groups == 1 && waves == pfs::split_waves(D, 1)) return launch_split<D, RT, 1, FMT, RES>(a, stream);
        if constexpr (RT == pfs::max_row_tiles(D)) {
            if (row_groups == 2 && waves == pfs::split_waves(D, 2)) return launch_split<D, RT, 2, FMT, RES>(a, stream);
            if (row_groups == 4 && waves == pfs::split_waves(D, 4)) return launch_split<D, RT, 4, FMT, RES>(a, stream);
            if constexpr (pfs::split_narrow(D, 4, 2)) {
                if (row_groups == 4 && waves == pfs::split_waves(D, 4, true))
                    return launch_split<D, RT, 4, FMT, RES, true>(a, stream);
            }
        }
        return hipErrorInvalidValue;
    }
}

template <int D, int FMT, bool RES>
hipError_t launch_split_d(const SplitArgs& a, int32_t row_tiles, int32_t row_groups, int32_t waves,
                          hipStream_t stream) {
    switch (row_tiles) {
        case 1: return launch_split_rt<D, 1, FMT, RES>(a, row_groups, waves, stream);
        case 2: return launch_split_rt<D, 2, FMT, RES>(a, row_groups, waves, stream);
        case 4: return launch_split_rt<D, 4, FMT, RES>(a, row_groups, waves, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int FMT, bool RES>
hipError_t launch_split_fmt(const SplitArgs& a, int32_t head_dim, int32_t row_tiles, int32_t row_groups,
                            int32_t waves, hipStream_t stream) {
    switch (head_dim) {
        case 64: return launch_split_d<64, FMT, RES>(a, row_tiles, row_groups, waves, stream);
        case 128: return launch_split_d<128, FMT, RES>(a, row_tiles, row_groups, waves, stream);
        case 256: return launch_split_d<256, FMT, RES>(a, row_tiles, row_groups, waves, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int32_t pfs_launch_split(const pfs_plan* plan, const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                         const float* k_scale, const int32_t* block_table, const int32_t* live_len,
                         void* workspace, pfs_stream_t stream) {
    const pfs_problem& p = plan->p;
    SplitArgs sa;
    sa.qptr = static_cast<const _Float16*>(q);
    sa.kpool = k_pool;
    sa.vpool = v_pool;
    sa.kscale = k_scale;
    sa.block_table = block_table;
    sa.live_len = live_len;
    sa.ws_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->ws_ml_offset);
    sa.ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan->ws_acc_offset);
    sa.page_stride = p.kv_page_stride;
    sa.token_stride = p.kv_token_stride;
    sa.head_stride = p.kv_head_stride;
    sa.batch = p.batch;
    sa.q = p.q;
    sa.num_q_heads = p.num_q_heads;
    sa.num_kv_heads = p.num_kv_heads;
    sa.group = plan->group;
    sa.rows = plan->rows;
    sa.page_size = p.page_size;
    sa.page_shift = (p.page_size & (p.page_size - 1)) == 0 ? __builtin_ctz((unsigned)p.page_size) : -1;
    sa.max_pages = p.max_pages_per_row;
    sa.capacity = plan->capacity;
    sa.tokens_per_split = plan->tokens_per_split;
    sa.num_splits = plan->num_splits;
    sa.row_blocks = plan->row_blocks;
    sa.sm_scale_log2e = p.sm_scale * kLog2e;
    for (int i = 0; i < pfs::kMaxQHeads; ++i) sa.qhead[i] = plan->qhead[i];

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.head_dim != 64 && p.head_dim != 128 && p.head_dim != 256) return PFS_ERR_UNSUPPORTED;
    hipError_t e;
    const bool res = p.pv_mode == PFS_PV_HIGH_RESIDUAL;
    const int32_t rt = plan->row_tiles, rg = plan->row_groups, w = plan->waves;
    if (p.kv_format == PFS_KV_E4M3)
        e = res ? launch_split_fmt<PFS_KV_E4M3, true>(sa, p.head_dim, rt, rg, w, s)
                : launch_split_fmt<PFS_KV_E4M3, false>(sa, p.head_dim, rt, rg, w, s);
    else if (p.kv_format == PFS_KV_E5M2)
        e = res ? launch_split_fmt<PFS_KV_E5M2, true>(sa, p.head_dim, rt, rg, w, s)
                : launch_split_fmt<PFS_KV_E5M2, false>(sa, p.head_dim, rt, rg, w, s);
    else
        return PFS_ERR_UNSUPPORTED;
    return e == hipSuccess ? PFS_OK : PFS_ERR_LAUNCH;
}

// Plans with at most kCombineRowSplits splits: one thread per 4 columns of a
// row folds every split of it (pfs_combine_rows_kernel); more splits: a
// workgroup of kCombineWaves waves per 4 combine_cgw(D) columns of a row.
// One request issues its first partial loads ahead of its live length.
template <int D>
hipError_t launch_combine(const pfs_plan& plan, const CombineArgs& ca, bool ahead, hipStream_t s) {
    const pfs_problem& p = plan.p;
    if (plan.num_splits <= kCombineRowSplits) {
        const dim3 grid((plan.rows * D / 4 + 255) / 256, p.num_kv_heads, p.batch);
        if (ahead)
            hipLaunchKernelGGL((pfs_combine_rows_kernel<D, true>), grid, dim3(256), 0, s, ca);
        else
            hipLaunchKernelGGL((pfs_combine_rows_kernel<D, false>), grid, dim3(256), 0, s, ca);
    } else {
        const dim3 grid(plan.rows * (D / (4 * combine_cgw(D))), p.num_kv_heads, p.batch);
        if (ahead)
            hipLaunchKernelGGL((pfs_combine_kernel<D, true>), grid, dim3(64 * kCombineWaves), 0, s, ca);
        else
            hipLaunchKernelGGL((pfs_combine_kernel<D, false>), grid, dim3(64 * kCombineWaves), 0, s, ca);
    }
    return hipGetLastError();
}

int32_t pfs_launch_combine(const pfs_plan* plan, const float* v_scale, const int32_t* live_len, void* out,
                           const void* workspace, pfs_stream_t stream) {
    const pfs_problem& p = plan->p;
    CombineArgs ca;
    ca.ws_ml = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + plan->ws_ml_offset);
    ca.ws_acc = reinterpret_cast<const float*>(static_cast<const char*>(workspace) + plan->ws_acc_offset);
    ca.vscale = v_scale;
    ca.live_len = live_len;
    ca.out = static_cast<_Float16*>(out);
    ca.batch = p.batch;
    ca.q = p.q;
    ca.num_q_heads = p.num_q_heads;
    ca.num_kv_heads = p.num_kv_heads;
    ca.group = plan->group;
    ca.rows = plan->rows;
    ca.capacity = plan->capacity;
    ca.tokens_per_split = plan->tokens_per_split;
    ca.num_splits = plan->num_splits;
    ca.head_dim = p.head_dim;
    for (int i = 0; i < pfs::kMaxQHeads; ++i) ca.qhead[i] = plan->qhead[i];
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const bool ahead = p.batch == 1;
    hipError_t e;
    switch (p.head_dim) {
        case 64: e = launch_combine<64>(*plan, ca, ahead, s); break;
        case 128: e = launch_combine<128>(*plan, ca, ahead, s); break;
        case 256: e = launch_combine<256>(*plan, ca, ahead, s); break;
        default: return PFS_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? PFS_OK : PFS_ERR_LAUNCH;
}
