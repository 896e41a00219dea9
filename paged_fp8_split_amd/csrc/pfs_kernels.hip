// pfs_kernels.hip -- gfx950 (CDNA4) kernels of libpfs and their launchers.
//
//   e4m3x2_to_f16x2       exact E4M3 -> FP16 dequant-on-load (hardware
//                         v_cvt_scalef32_pk_f16_fp8 with scale 1.0)
//   pfs_dequant_kernel    paged E4M3 -> dense FP16 bridge
//   pfs_split_kernel      per-split QK^T (MFMA), online softmax, PV (MFMA);
//                         emits FP32 (max, sum, unnormalized PV) per split
//   pfs_combine_kernel    rescales the splits, sums them in a fixed order
//                         (ascending runs, runs in order), normalizes and
//                         rounds once to FP16
//
// The method ("[Kernel][SM70] Add opt-in E4M3 grouped attention with FP32
// partials", final status, revision 3 bullet; "[Kernel] Finalize the audited
// TP2 DFlash2 31/29 ms endpoint", Purpose) keeps FP32 max / sum and an
// unnormalized PV accumulator per KV partition until one final combine, with
// keys consumed in 64-key partitions in a fixed order. On V100 that was a
// scalar/tensor-core kernel; here it is built around CDNA4's 64-wide
// wavefronts and v_mfma_f32_16x16x32_f16.
//
// Work decomposition of the split kernel (one workgroup = 4 waves per split,
// KV head and row block):
//  * rows: up to 64 of the R = G*q query rows of one KV head per workgroup
//    (row r = i*G + jj: draft row i, jj-th query head of the group), padded to
//    16-row MFMA tiles; more rows become row blocks of the grid. The FP32
//    accumulators of every row and every head_dim column stay in registers.
//  * tokens: wave w takes partitions w, w+4, w+8, ... of the split, in
//    ascending order; the four wave states are merged in wave order at the end.
//  * scores are computed transposed, S^T = K * Q^T (A = K: 16 tokens x 32 dims,
//    B = Q^T: 32 dims x 16 rows), so each lane ends up holding 4 consecutive
//    tokens of one row: exactly the token slots the PV product
//    O^T = V^T * P^T needs in its B operand. P never leaves registers.
//  * K goes from HBM straight into MFMA A operands: lane (c, g) of a 16-token
//    tile loads 16-byte chunks of token c, so each load instruction reads 64
//    contiguous bytes of 16 tokens; the E4M3 bytes are converted in registers.
//  * V^T needs 8 tokens of one head_dim column per lane: V rows are loaded
//    with 16-byte loads (4 whole token rows per instruction), written to the
//    wave's LDS stage with an XOR swizzle of the 16-byte chunks, and read back
//    transposed with ds_read_b64_tr_b8: in each 16-lane block, lane j names
//    8 bytes of one token row and every lane receives one column of 8 tokens.
//  * Q^T operands are staged once per workgroup in LDS in the exact per-lane
//    order the MFMA B operand needs (one ds_read_b128 per operand).
//
// Numerics: FP16 MFMA operands with FP32 accumulation; the per-head K scale,
// the softmax scale and log2(e) are applied to FP32 scores; probabilities are
// exp2(s - m_ref + 7) rounded once to FP16 against a lazily raised reference
// maximum m_ref; the row sums come from the matrix core (a ones row times the
// same FP16 P the PV product uses); V's scale is applied once in the combine.
// Masked scores are selected to -inf and K/V bytes beyond the live length are
// never loaded (zero), so NaN tail bytes cannot leak.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pfs_internal.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = pfs::kWaves;
constexpr int kPart = pfs::kPartitionTokens;
constexpr int kStep = 32;  // tokens per MFMA fold step (two 16-token tiles)
constexpr float kLog2e = 1.4426950408889634f;

template <typename T, typename F>
__device__ __forceinline__ T bit_cast_(F f) {
    static_assert(sizeof(T) == sizeof(F), "size");
    return __builtin_bit_cast(T, f);
}

// Two E4M3 bytes (bytes 2*HI and 2*HI+1 of `word`) -> two FP16 values, exact:
// every finite E4M3 value is zero or an FP16 normal number.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t word) {
    const f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, HI);
    return bit_cast_<uint32_t>(h);
}

// 8 E4M3 bytes (two dwords) -> 8 FP16 values as an MFMA operand.
__device__ __forceinline__ f16x8 e4m3x8_to_f16x8(uint32_t w0, uint32_t w1) {
    u32x4 r;
    r.x = e4m3x2_to_f16x2<false>(w0);
    r.y = e4m3x2_to_f16x2<true>(w0);
    r.z = e4m3x2_to_f16x2<false>(w1);
    r.w = e4m3x2_to_f16x2<true>(w1);
    return bit_cast_<f16x8>(r);
}

__device__ __forceinline__ float wave_max_xor_16_32(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
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
    int32_t max_pages;
    int32_t capacity;
    int32_t tokens_per_split;
    int32_t num_splits;
    int32_t row_blocks;
    float sm_scale_log2e;
    uint8_t qhead[pfs::kMaxQHeads];
};

// Compile-time geometry of the split kernel.
template <int D, int RT>
struct SplitCfg {
    static constexpr int KSTEPS = D / 32;             // QK k-steps (32 dims each)
    static constexpr int CH = D / 16;                 // 16-byte chunks per token row
    static constexpr int LOADS = CH / 2;              // 16-byte loads per lane per 32-token step (K or V)
    static constexpr int MD = D / 16;                 // PV tiles along head_dim
    static constexpr int QBYTES = RT * KSTEPS * 64 * 16;
    static constexpr int STAGE = kStep * D;           // one wave's K (or V) stage: 32 token rows
    static constexpr int MERGE_BYTES = MD * RT * 64 * 16;
    static constexpr int MAIN_BYTES = QBYTES + kWaves * 2 * STAGE;
    static constexpr int LDS_BYTES = MAIN_BYTES > MERGE_BYTES ? MAIN_BYTES : MERGE_BYTES;
};

// Lazy rescaling: a row's exponentials use a reference maximum m_ref and are
// exp2(s*c - m_ref + kPBias). m_ref is raised (and the accumulators rescaled)
// only when a score exceeds it by more than kTau, so P <= 2^(kPBias + kTau) =
// 2^15 stays an FP16 number, and P only becomes FP16-subnormal for terms below
// 2^-21 of the reference maximum. The offset cancels in acc / l.
constexpr float kTau = 8.0f;
constexpr float kPBias = 7.0f;
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past every tile: the load returns zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int D, int RT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
pfs_split_kernel(const SplitArgs a) {
    using C = SplitCfg<D, RT>;
    constexpr int KSTEPS = C::KSTEPS, CH = C::CH, LOADS = C::LOADS, MD = C::MD;
    __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
    __shared__ float2 lds_ml[kWaves][RT * 16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lc = lane & 15;  // column within a 16-wide MFMA tile
    const int lg = lane >> 4;  // lane group (k-group of an operand, row-quad of a result)

    // 1-D grid. Workgroups x and x + 8 run on the same XCD (dispatch is
    // round-robin over the 8 XCDs), so the row blocks of one (split, KV head,
    // request) get ids 8 apart and share that XCD's L2 for their K/V reads.
    const int x = blockIdx.x;
    const int rb = (x >> 3) % a.row_blocks;
    const int unit = ((x >> 3) / a.row_blocks) * 8 + (x & 7);  // (split, KV head, request), split fastest
    if (unit >= a.num_splits * a.num_kv_heads * a.batch) return;
    const int split = unit % a.num_splits;
    const int g = (unit / a.num_splits) % a.num_kv_heads;
    const int b = unit / (a.num_splits * a.num_kv_heads);

    const int32_t L = clamp_i(a.live_len[b], 0, a.capacity);
    const int32_t tok0 = split * a.tokens_per_split;
    if (tok0 >= L) return;  // nothing live in this split: the combine never reads it
    const int32_t tok1 = min(tok0 + a.tokens_per_split, L);
    const int r_begin = rb * RT * 16;

    u32x4* q_lds = reinterpret_cast<u32x4*>(smem);
    uint8_t* k_lds = smem + C::QBYTES + wave * 2 * C::STAGE;
    uint8_t* v_lds = k_lds + C::STAGE;

    // ---- stage Q^T operands in LDS: slot (nt * KSTEPS + ks) * 64 + lane holds
    //      row r_begin + 16 nt + (lane & 15), dims 64(ks/2) + 16(lane/16) + 8(ks&1) + [0, 8) ----
    for (int slot = threadIdx.x; slot < RT * KSTEPS * 64; slot += 256) {
        const int ln = slot & 63;
        const int ks = (slot >> 6) % KSTEPS;
        const int nt = (slot >> 6) / KSTEPS;
        const int r = r_begin + nt * 16 + (ln & 15);
        const int d0 = 64 * (ks >> 1) + 16 * (ln >> 4) + 8 * (ks & 1);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < a.rows) {
            const int i = r / a.group;
            const int h = a.qhead[g * a.group + (r % a.group)];
            v = *reinterpret_cast<const u32x4*>(a.qptr + (((int64_t)b * a.q + i) * a.num_q_heads + h) * D + d0);
        }
        q_lds[slot] = v;
    }

    // causal limit of this lane's row in each row tile: keys [0, lim) are visible.
    // Padding rows (r >= rows) keep lim = L: their Q is zero, their results are
    // never written and MFMA columns do not mix, so they need no masking.
    int32_t lim[RT];
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        const int r = r_begin + nt * 16 + lc;
        lim[nt] = (r < a.rows) ? clamp_i((int64_t)L - a.q + r / a.group + 1, 0, L) : L;
    }
    const int32_t lim_lo = clamp_i((int64_t)L - a.q + 1, 0, L);  // smallest limit of any real row
    const float cscale = a.sm_scale_log2e * a.kscale[g];

    f32x4 acc[MD][RT];
    f32x4 lacc[RT];  // row sums, computed by the matrix core from the same FP16 P
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

    // Load slot j of a lane: 16-byte chunk c = lane % CH of token row
    // t_j = (64 j + lane) / CH of the 32-token step (each instruction reads
    // 64 / CH whole rows). In LDS, row t keeps its chunks XOR-swizzled by t % CH.
    const int ld_c = lane % CH;
    const uint32_t ld_voff_base = 16u * (uint32_t)ld_c;
    // transposed V reads: lane j of each 16-lane block names 8 bytes of token
    // tok(lg, j >> 1) of the step, the (j & 1) half of a 16-byte chunk
    const int tr_tok = ((lc >> 1) < 4 ? 0 : 16) + 4 * lg + ((lc >> 1) & 3);
    const int tr_base = tr_tok * D + 8 * (lc & 1);
    const int tr_sw = tr_tok % CH;

    __syncthreads();

    const int64_t head_off = (int64_t)g * a.head_stride;
    const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
    const uint32_t tile_bytes = (uint32_t)(15 * a.token_stride + D);
    const int32_t p_begin = tok0 / kPart;
    const int32_t p_end = (tok1 + kPart - 1) / kPart;
    // this wave's steps: partitions p_begin + wave + 4k, two 32-token steps each
    const int32_t nparts = (p_end - p_begin - wave + kWaves - 1) / kWaves;
    int32_t nsteps = 0;
    if (nparts > 0) {
        const int32_t last_part = p_begin + wave + (nparts - 1) * kWaves;
        nsteps = 2 * nparts - ((last_part * kPart + kStep) >= L ? 1 : 0);
    }
    auto step_token = [&](int32_t st) -> int32_t {
        return (p_begin + wave + (st >> 1) * kWaves) * kPart + (st & 1) * kStep;
    };

    // ---- loads of one 32-token step into registers (tokens >= L read as zeros) ----
    u32x4 kreg[LOADS], vreg[LOADS];
    auto load_step = [&](int32_t t_step) {
        const bool live1 = t_step + 16 < L;
        const int64_t off0 = (int64_t)bt_row[t_step / a.page_size] * a.page_stride +
                             (int64_t)(t_step % a.page_size) * a.token_stride + head_off;
        const int64_t off1 = live1 ? (int64_t)bt_row[(t_step + 16) / a.page_size] * a.page_stride +
                                         (int64_t)((t_step + 16) % a.page_size) * a.token_stride + head_off
                                   : 0;
        const __amdgpu_buffer_rsrc_t k0 = tile_rsrc(a.kpool + off0, tile_bytes);
        const __amdgpu_buffer_rsrc_t k1 = tile_rsrc(a.kpool + off1, tile_bytes);
        const __amdgpu_buffer_rsrc_t v0 = tile_rsrc(a.vpool + off0, tile_bytes);
        const __amdgpu_buffer_rsrc_t v1 = tile_rsrc(a.vpool + off1, tile_bytes);
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int t = (64 * j + lane) / CH;  // token of the step; the 16-token tile is uniform in j
            const uint32_t voff = (t_step + t < L) ? (uint32_t)(t & 15) * (uint32_t)a.token_stride + ld_voff_base
                                                   : kOutOfRange;
            const bool tile1 = (64 * j) / CH >= 16;
            kreg[j] = bit_cast_<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(tile1 ? k1 : k0, voff, 0, 0));
            vreg[j] = bit_cast_<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(tile1 ? v1 : v0, voff, 0, 0));
        }
    };

    if (nsteps > 0) load_step(step_token(0));

    for (int32_t st = 0; st < nsteps; ++st) {
        const int32_t t_step = step_token(st);
        // this step's K and V -> the wave's LDS stages, then prefetch the next step
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            const int t = (64 * j + lane) / CH;
            const int off = t * D + ((ld_c ^ (t % CH)) << 4);
            *reinterpret_cast<u32x4*>(k_lds + off) = kreg[j];
            *reinterpret_cast<u32x4*>(v_lds + off) = vreg[j];
        }
        if (st + 1 < nsteps) load_step(step_token(st + 1));

        // ---- S^T = K * Q^T ----
        f32x4 s[2][RT];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < RT; ++nt) s[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
            f16x8 qop[RT];
#pragma unroll
            for (int nt = 0; nt < RT; ++nt) qop[nt] = bit_cast_<f16x8>(q_lds[(nt * KSTEPS + ks) * 64 + lane]);
            const int chunk = 4 * (ks >> 1) + lg;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int t = 16 * mt + lc;
                const u32x2 w = *reinterpret_cast<const u32x2*>(k_lds + t * D + ((chunk ^ (t % CH)) << 4) +
                                                                8 * (ks & 1));
                const f16x8 kop = e4m3x8_to_f16x8(w.x, w.y);
#pragma unroll
                for (int nt = 0; nt < RT; ++nt)
                    s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[nt], s[mt][nt], 0, 0, 0);
            }
        }

        // ---- online softmax, log2 domain, lazy reference maximum ----
        const bool edge = t_step + kStep > lim_lo;  // some (row, token) of this step is masked
        float smax[RT];
        bool need = false;
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) {
            float mx = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v = s[mt][nt][i];
                    if (edge) {
                        const int32_t t = t_step + mt * 16 + 4 * lg + i;
                        v = (t < lim[nt]) ? v : -INFINITY;
                        s[mt][nt][i] = v;
                    }
                    mx = fmaxf(mx, v);
                }
            mx = wave_max_xor_16_32(mx);
            smax[nt] = mx * cscale;  // cscale > 0; -inf stays -inf
            need |= (smax[nt] > mref[nt] + kTau);
        }
        if (__any(need)) {
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
        f16x8 pop[RT];
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) {
            _Float16 ph[8];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float v = s[mt][nt][i];
                    const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(v, cscale, nb[nt]));
                    ph[mt * 4 + i] = (_Float16)((edge && v == -INFINITY) ? 0.0f : pv);
                }
            pop[nt] = f16x8{ph[0], ph[1], ph[2], ph[3], ph[4], ph[5], ph[6], ph[7]};
        }

        // ---- O^T += V^T * P^T (V^T read transposed from LDS), l += 1 * P^T ----
#pragma unroll
        for (int md = 0; md < MD; ++md) {
            const int addr = tr_base + ((md ^ tr_sw) << 4);
            const i32x2 w = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) i32x2*)(v_lds + addr));
            const f16x8 vop = e4m3x8_to_f16x8((uint32_t)w.x, (uint32_t)w.y);
#pragma unroll
            for (int nt = 0; nt < RT; ++nt)
                acc[md][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[nt], acc[md][nt], 0, 0, 0);
        }
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) lacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pop[nt], lacc[nt], 0, 0, 0);
    }

    // ---- merge the four wave states in wave order ----
    // row sums live in result row 0 of the ones tile: lanes of lane group 0, element 0
    if (lg == 0) {
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) lds_ml[wave][nt * 16 + lc] = make_float2(mref[nt], lacc[nt][0]);
    }
    __syncthreads();  // every wave is also done with Q, K and V in LDS from here on
    float M[RT], Ltot[RT];
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        float mm = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) mm = fmaxf(mm, lds_ml[w][nt * 16 + lc].x);
        float lt = 0.0f, fmine = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float2 ml = lds_ml[w][nt * 16 + lc];
            const float f = (ml.x == -INFINITY) ? 0.0f : (ml.x == mm ? 1.0f : __builtin_amdgcn_exp2f(ml.x - mm));
            lt += f * ml.y;
            if (w == wave) fmine = f;
        }
        M[nt] = mm;
        Ltot[nt] = lt;
#pragma unroll
        for (int md = 0; md < MD; ++md) acc[md][nt] *= fmine;
    }
    u32x4* mbuf = reinterpret_cast<u32x4*>(smem);
    for (int w = 1; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int nt = 0; nt < RT; ++nt) mbuf[(md * RT + nt) * 64 + lane] = bit_cast_<u32x4>(acc[md][nt]);
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int nt = 0; nt < RT; ++nt) acc[md][nt] += bit_cast_<f32x4>(mbuf[(md * RT + nt) * 64 + lane]);
        }
        __syncthreads();
    }
    if (wave != 0) return;

    // ---- emit the split partial: (reference max, sum) and the unnormalized PV ----
    // accumulator element i of d tile md is column 16 md + 4 lg + i of row r
    const int64_t slot_base = (((int64_t)split * a.batch + b) * a.num_kv_heads + g) * a.rows;
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        const int r = r_begin + nt * 16 + lc;
        if (r >= a.rows) continue;
        if (lg == 0) reinterpret_cast<float2*>(a.ws_ml)[slot_base + r] = make_float2(M[nt], Ltot[nt]);
        float* dst = a.ws_acc + (slot_base + r) * D + 4 * lg;
#pragma unroll
        for (int md = 0; md < MD; ++md) *reinterpret_cast<f32x4*>(dst + 16 * md) = acc[md][nt];
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
    uint8_t qhead[pfs::kMaxQHeads];
};

// One workgroup of 16 waves per output row (request, KV head, row). Wave w
// sums the w-th contiguous run of the visible splits in ascending split order
// (its loads are independent, so a wave keeps its whole run in flight); the 16
// runs are then added in wave order. The global max is a plain max (exact, so
// any order). Each lane owns head_dim/64 columns.
constexpr int kCombineWaves = 16;

template <int D>
__global__ __launch_bounds__(64 * kCombineWaves) void pfs_combine_kernel(const CombineArgs a) {
    constexpr int CPL = D / 64;  // columns per lane
    __shared__ float red[kCombineWaves];
    __shared__ float part_l[kCombineWaves];
    __shared__ float part_acc[kCombineWaves][D];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int i = r / a.group;
    const int h = a.qhead[g * a.group + (r % a.group)];
    _Float16* dst = a.out + (((int64_t)b * a.q + i) * a.num_q_heads + h) * D;

    const int32_t L = clamp_i(a.live_len[b], 0, a.capacity);
    const int32_t n = clamp_i((int64_t)L - a.q + i + 1, 0, L);
    if (n == 0) {  // nothing visible: defined output +0.0
        if (wave == 0) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) dst[lane * CPL + c] = (_Float16)0.0f;
        }
        return;
    }
    const int ns = (n + a.tokens_per_split - 1) / a.tokens_per_split;  // splits holding visible keys
    const int64_t stride = (int64_t)a.batch * a.num_kv_heads * a.rows;   // between splits
    const int64_t slot0 = ((int64_t)b * a.num_kv_heads + g) * a.rows + r;
    const float2* ml = reinterpret_cast<const float2*>(a.ws_ml);

    float mx = -INFINITY;
    for (int s = threadIdx.x; s < ns; s += 64 * kCombineWaves) mx = fmaxf(mx, ml[slot0 + s * stride].x);
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < kCombineWaves; ++w) M = fmaxf(M, red[w]);

    const int per = (ns + kCombineWaves - 1) / kCombineWaves;
    const int s0 = wave * per;
    const int s1 = min(ns, s0 + per);
    float lw = 0.0f;
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
    for (int s = s0; s < s1; ++s) {
        const int64_t slot = slot0 + s * stride;
        const float2 v = ml[slot];
        const float f = (v.x == M) ? 1.0f : __builtin_amdgcn_exp2f(v.x - M);
        lw += f * v.y;
        const float* src = a.ws_acc + slot * D + lane * CPL;
        if constexpr (CPL == 4) {
            const f32x4 xx = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] += f * xx[c];
        } else if constexpr (CPL == 2) {
            const float2 xx = *reinterpret_cast<const float2*>(src);
            acc[0] += f * xx.x;
            acc[1] += f * xx.y;
        } else {
            acc[0] += f * src[0];
        }
    }
    if (lane == 0) part_l[wave] = lw;
#pragma unroll
    for (int c = 0; c < CPL; ++c) part_acc[wave][lane * CPL + c] = acc[c];
    __syncthreads();
    if (wave != 0) return;
    float lt = part_l[0];
#pragma unroll
    for (int w = 1; w < kCombineWaves; ++w) lt += part_l[w];
    const float vs = a.vscale[g];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int d = lane * CPL + c;
        float num = part_acc[0][d];
#pragma unroll
        for (int w = 1; w < kCombineWaves; ++w) num += part_acc[w][d];
        dst[d] = (_Float16)((num * vs) / lt);
    }
}

// Paged E4M3 -> dense FP16: one thread per 16 bytes of one (token, KV head).
__global__ __launch_bounds__(256) void pfs_dequant_kernel(const uint8_t* pool, const int32_t* block_table,
                                                          const int32_t* live_len, _Float16* out,
                                                          int64_t page_stride, int64_t token_stride,
                                                          int64_t head_stride, int32_t num_kv_heads,
                                                          int32_t head_dim, int32_t page_size, int32_t max_pages,
                                                          int32_t capacity) {
    const int chunks = head_dim / 16;
    const int64_t per_tok = (int64_t)num_kv_heads * chunks;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.y;
    if (idx >= (int64_t)capacity * per_tok) return;
    const int32_t t = (int32_t)(idx / per_tok);
    const int g = (int)((idx / chunks) % num_kv_heads);
    const int c = (int)(idx % chunks);
    const int32_t L = clamp_i(live_len[b], 0, capacity);
    u32x4 res[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (t < L) {
        const int64_t page = block_table[(int64_t)b * max_pages + t / page_size];
        const u32x4 w = *reinterpret_cast<const u32x4*>(pool + page * page_stride + (int64_t)(t % page_size) * token_stride +
                                                        (int64_t)g * head_stride + 16 * c);
        res[0] = bit_cast_<u32x4>(e4m3x8_to_f16x8(w.x, w.y));
        res[1] = bit_cast_<u32x4>(e4m3x8_to_f16x8(w.z, w.w));
    }
    u32x4* dst = reinterpret_cast<u32x4*>(out + (((int64_t)b * capacity + t) * num_kv_heads + g) * head_dim + 16 * c);
    dst[0] = res[0];
    dst[1] = res[1];
}

template <int D, int RT>
hipError_t launch_split(const SplitArgs& a, hipStream_t stream) {
    const int64_t units = (int64_t)a.num_splits * a.num_kv_heads * a.batch;
    const int64_t wgs = ((units + 7) / 8) * 8 * a.row_blocks;
    hipLaunchKernelGGL((pfs_split_kernel<D, RT>), dim3((unsigned)wgs), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const SplitArgs& a, int32_t row_tiles, hipStream_t stream) {
    switch (row_tiles) {
        case 1: return launch_split<D, 1>(a, stream);
        case 2: return launch_split<D, 2>(a, stream);
        case 4:
            if constexpr (pfs::max_row_tiles(D) >= 4) return launch_split<D, 4>(a, stream);
            return hipErrorInvalidValue;
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
    sa.max_pages = p.max_pages_per_row;
    sa.capacity = plan->capacity;
    sa.tokens_per_split = plan->tokens_per_split;
    sa.num_splits = plan->num_splits;
    sa.row_blocks = plan->row_blocks;
    sa.sm_scale_log2e = p.sm_scale * kLog2e;
    for (int i = 0; i < pfs::kMaxQHeads; ++i) sa.qhead[i] = plan->qhead[i];

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    switch (p.head_dim) {
        case 64: e = launch_split_d<64>(sa, plan->row_tiles, s); break;
        case 128: e = launch_split_d<128>(sa, plan->row_tiles, s); break;
        case 256: e = launch_split_d<256>(sa, plan->row_tiles, s); break;
        default: return PFS_ERR_UNSUPPORTED;
    }
    return e == hipSuccess ? PFS_OK : PFS_ERR_LAUNCH;
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
    for (int i = 0; i < pfs::kMaxQHeads; ++i) ca.qhead[i] = plan->qhead[i];
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const dim3 grid(plan->rows, p.num_kv_heads, p.batch);
    switch (p.head_dim) {
        case 64: hipLaunchKernelGGL(pfs_combine_kernel<64>, grid, dim3(64 * kCombineWaves), 0, s, ca); break;
        case 128: hipLaunchKernelGGL(pfs_combine_kernel<128>, grid, dim3(64 * kCombineWaves), 0, s, ca); break;
        case 256: hipLaunchKernelGGL(pfs_combine_kernel<256>, grid, dim3(64 * kCombineWaves), 0, s, ca); break;
        default: return PFS_ERR_UNSUPPORTED;
    }
    return hipGetLastError() == hipSuccess ? PFS_OK : PFS_ERR_LAUNCH;
}

int32_t pfs_launch_dequant(const pfs_plan* plan, const uint8_t* pool, const int32_t* block_table,
                           const int32_t* live_len, void* out, pfs_stream_t stream) {
    const pfs_problem& p = plan->p;
    const int64_t threads = (int64_t)plan->capacity * p.num_kv_heads * (p.head_dim / 16);
    const dim3 grid((unsigned)((threads + 255) / 256), p.batch);
    hipLaunchKernelGGL(pfs_dequant_kernel, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream), pool,
                       block_table, live_len, static_cast<_Float16*>(out), p.kv_page_stride, p.kv_token_stride,
                       p.kv_head_stride, p.num_kv_heads, p.head_dim, p.page_size, p.max_pages_per_row,
                       plan->capacity);
    return hipGetLastError() == hipSuccess ? PFS_OK : PFS_ERR_LAUNCH;
}
