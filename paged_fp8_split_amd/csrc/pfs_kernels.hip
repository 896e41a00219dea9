// pfs_kernels.hip -- gfx950 (CDNA4) kernels of libpfs and their launchers.
//
//   e4m3x2_to_f16x2       exact E4M3 -> FP16 dequant-on-load (hardware
//                         v_cvt_scalef32_pk_f16_fp8 with scale 1.0)
//   pfs_dequant_kernel    paged E4M3 -> dense FP16 bridge
//   pfs_split_kernel      per-split QK^T (MFMA), online softmax, PV (MFMA);
//                         emits FP32 (max, sum, unnormalized PV) per split
//   pfs_combine_kernel    rescales the splits, sums them in ascending split
//                         order, normalizes and rounds once to FP16
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
//  * rows: all R = G*q query rows of one KV head live in one workgroup (row
//    r = i*G + jj: draft row i, jj-th query head of the group), padded to 16-row
//    MFMA tiles; the FP32 accumulators of every row and every head_dim column
//    stay in registers (R*D <= 16384 -> <= 256 accumulators per lane).
//  * tokens: wave w takes partitions w, w+4, w+8, ... of the split, in
//    ascending order; the four wave states are merged in wave order at the end.
//  * scores are computed transposed, S^T = K * Q^T (A = K: 16 tokens x 32 dims,
//    B = Q^T: 32 dims x 16 rows), so each lane ends up holding 4 consecutive
//    tokens of one row: exactly the token slots the PV product
//    O^T = V^T * P^T needs in its B operand. P never leaves registers.
//  * K goes from HBM straight into MFMA A operands: lane (c, g) of a 16-token
//    tile loads 16-byte chunks of token c, so each load instruction reads 64
//    contiguous bytes of 16 tokens; the E4M3 bytes are converted in registers.
//  * V^T needs 8 tokens of one head_dim column per lane: lane (c, g) loads
//    head_dim/16 contiguous bytes (a column strip) of each of its 8 tokens,
//    then v_perm_b32 interleaves the bytes of token pairs so every
//    v_cvt_scalef32_pk_f16_fp8 yields two tokens of one column. Each load
//    instruction reads 4 whole token rows.
//  * Q^T operands are staged once per workgroup in LDS in the exact per-lane
//    order the MFMA B operand needs (one ds_read_b128 per operand).
//
// Numerics: FP16 MFMA operands with FP32 accumulation; the per-head K scale,
// the softmax scale and log2(e) are applied to FP32 scores; probabilities are
// exp2(s - m + 15) rounded once to FP16 (the 2^15 offset keeps them out of the
// FP16 subnormal range and cancels in acc / l); the running sum accumulates the
// same rounded values the PV product uses; V's scale is applied once in the
// combine. Masked scores are selected to -inf and K/V bytes beyond the live
// length are never loaded (zero), so NaN tail bytes cannot leak.
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

constexpr int kWaves = pfs::kWaves;
constexpr int kPart = pfs::kPartitionTokens;
constexpr int kStep = 32;  // tokens per MFMA fold step (two 16-token tiles)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPBias = 15.0f;  // P = exp2(s - m + 15) <= 32768

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

__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
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
    int32_t row_blocks;
    float sm_scale_log2e;
    uint8_t qhead[pfs::kMaxQHeads];
};

template <int D>
struct VChunk;  // the head_dim/16 bytes of one token a lane loads for V
template <>
struct VChunk<64> {
    static constexpr int kDwords = 1;
    typedef uint32_t type;
};
template <>
struct VChunk<128> {
    static constexpr int kDwords = 2;
    typedef u32x2 type;
};
template <>
struct VChunk<256> {
    static constexpr int kDwords = 4;
    typedef u32x4 type;
};

template <int D>
__device__ __forceinline__ uint32_t vdword(const typename VChunk<D>::type& v, int i) {
    if constexpr (D == 64) {
        return v;
    } else {
        return v[i];
    }
}

// Per-wave state of the split kernel.
template <int D, int RT>
struct WaveState {
    static constexpr int MD = D / 16;  // PV output tiles along head_dim
    f32x4 acc[MD][RT];                 // O^T tiles: [d tile][row tile]
    float m[RT];                       // running max (log2 domain) of this lane's row in each row tile
    float l[RT];                       // running sum, partial over this lane's token slots
};

template <int D, int RT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1))) void
pfs_split_kernel(const SplitArgs a) {
    constexpr int KSTEPS = D / 32;  // QK k-steps (32 dims each)
    constexpr int KLOADS = D / 64;  // 16-byte K loads per lane per 16-token tile
    constexpr int MD = D / 16;      // PV tiles along head_dim
    constexpr int VD = VChunk<D>::kDwords;
    constexpr int kQSlots = RT * KSTEPS * 64;          // 16-byte Q operand slots
    constexpr int kMergeSlots = MD * RT * 64;          // 16-byte accumulator slots of one wave
    constexpr int kLdsSlots = kQSlots > kMergeSlots ? kQSlots : kMergeSlots;
    __shared__ u32x4 lds[kLdsSlots];
    __shared__ float2 lds_ml[kWaves][RT * 16];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lc = lane & 15;   // column within a 16-wide MFMA tile
    const int lg = lane >> 4;   // lane group (k-group / row-quad)

    const int split = blockIdx.x;
    const int g = blockIdx.y / a.row_blocks;
    const int rb = blockIdx.y % a.row_blocks;
    const int b = blockIdx.z;

    const int32_t L = clamp_i(a.live_len[b], 0, a.capacity);
    const int32_t tok0 = split * a.tokens_per_split;
    if (tok0 >= L) return;  // nothing live in this split: the combine never reads it
    const int32_t tok1 = min(tok0 + a.tokens_per_split, L);
    const int r_begin = rb * RT * 16;

    // ---- stage Q^T operands in LDS (slot = (nt * KSTEPS + ks) * 64 + lane) ----
    for (int slot = threadIdx.x; slot < kQSlots; slot += 256) {
        const int ln = slot & 63;
        const int ks = (slot >> 6) % KSTEPS;
        const int nt = (slot >> 6) / KSTEPS;
        const int r = r_begin + nt * 16 + (ln & 15);
        const int d0 = 64 * (ks >> 1) + 16 * (ln >> 4) + 8 * (ks & 1);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < a.rows) {
            const int i = r / a.group;
            const int h = a.qhead[g * a.group + (r % a.group)];
            const _Float16* src = a.qptr + (((int64_t)b * a.q + i) * a.num_q_heads + h) * D + d0;
            v = *reinterpret_cast<const u32x4*>(src);
        }
        lds[slot] = v;
    }

    // causal limit of this lane's row in each row tile: keys [0, lim) are visible
    int32_t lim[RT];
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        const int r = r_begin + nt * 16 + lc;
        lim[nt] = (r < a.rows) ? clamp_i((int64_t)L - a.q + r / a.group + 1, 0, L) : 0;
    }
    const float cscale = a.sm_scale_log2e * a.kscale[g];

    WaveState<D, RT> st;
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        st.m[nt] = -INFINITY;
        st.l[nt] = 0.0f;
#pragma unroll
        for (int md = 0; md < MD; ++md) st.acc[md][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __syncthreads();

    const int64_t head_off = (int64_t)g * a.head_stride;
    const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
    const int32_t p_begin = tok0 / kPart;
    const int32_t p_end = (tok1 + kPart - 1) / kPart;

    for (int32_t part = p_begin + wave; part < p_end; part += kWaves) {
#pragma unroll 1
        for (int half = 0; half < 2; ++half) {
            const int32_t t_step = part * kPart + half * kStep;
            if (t_step >= L) break;
            // pages of the two 16-token tiles (page_size is a multiple of 16)
            const bool live1 = t_step + 16 < L;
            const int64_t pg0 = (int64_t)bt_row[t_step / a.page_size] * a.page_stride +
                                (int64_t)(t_step % a.page_size) * a.token_stride + head_off;
            const int64_t pg1 = live1 ? (int64_t)bt_row[(t_step + 16) / a.page_size] * a.page_stride +
                                            (int64_t)((t_step + 16) % a.page_size) * a.token_stride + head_off
                                      : 0;

            // ---- V loads: 8 tokens x head_dim/16 bytes (column strip lc) ----
            typename VChunk<D>::type vraw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int tt = (e < 4 ? 0 : 16) + 4 * lg + (e & 3);  // token within the step
                const bool ok = t_step + tt < L;
                const int64_t off = (e < 4 ? pg0 : pg1) + (int64_t)(tt & 15) * a.token_stride + lc * (D / 16);
                if (ok) {
                    vraw[e] = *reinterpret_cast<const typename VChunk<D>::type*>(a.vpool + off);
                } else {
                    vraw[e] = typename VChunk<D>::type{};
                }
            }

            // ---- K loads: 2 tiles x KLOADS x 16 bytes ----
            u32x4 kraw[2][KLOADS];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bool ok = t_step + mt * 16 + lc < L;
                const int64_t off = (mt == 0 ? pg0 : pg1) + (int64_t)lc * a.token_stride + 16 * lg;
#pragma unroll
                for (int j = 0; j < KLOADS; ++j) {
                    if (ok) {
                        kraw[mt][j] = *reinterpret_cast<const u32x4*>(a.kpool + off + 64 * j);
                    } else {
                        kraw[mt][j] = u32x4{0u, 0u, 0u, 0u};
                    }
                }
            }

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
                for (int nt = 0; nt < RT; ++nt) qop[nt] = bit_cast_<f16x8>(lds[(nt * KSTEPS + ks) * 64 + lane]);
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const u32x4 w = kraw[mt][ks >> 1];
                    const f16x8 kop = (ks & 1) ? e4m3x8_to_f16x8(w.z, w.w) : e4m3x8_to_f16x8(w.x, w.y);
#pragma unroll
                    for (int nt = 0; nt < RT; ++nt)
                        s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[nt], s[mt][nt], 0, 0, 0);
                }
            }

            // ---- online softmax (log2 domain) ----
            f16x8 pop[RT];
            float alpha[RT];
            bool rescale = false;
#pragma unroll
            for (int nt = 0; nt < RT; ++nt) {
                float x[8];
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int32_t t = t_step + mt * 16 + 4 * lg + i;
                        x[mt * 4 + i] = (t < lim[nt]) ? s[mt][nt][i] * cscale : -INFINITY;
                    }
                float mx = x[0];
#pragma unroll
                for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
                mx = wave_max_xor_16_32(mx);
                const float m_new = fmaxf(st.m[nt], mx);
                float al = 1.0f;
                if (m_new != -INFINITY && st.m[nt] != m_new) al = __builtin_amdgcn_exp2f(st.m[nt] - m_new);
                rescale |= (al != 1.0f);
                alpha[nt] = al;
                float lsum = 0.0f;
                _Float16 ph[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pv = (x[e] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f((x[e] - m_new) + kPBias);
                    ph[e] = (_Float16)pv;
                    lsum += (float)ph[e];
                }
                st.l[nt] = st.l[nt] * al + lsum;
                st.m[nt] = m_new;
                pop[nt] = f16x8{ph[0], ph[1], ph[2], ph[3], ph[4], ph[5], ph[6], ph[7]};
            }
            if (__any(rescale)) {
#pragma unroll
                for (int md = 0; md < MD; ++md)
#pragma unroll
                    for (int nt = 0; nt < RT; ++nt) st.acc[md][nt] *= alpha[nt];
            }

            // ---- O^T += V^T * P^T ----
#pragma unroll
            for (int q4 = 0; q4 < VD; ++q4) {
                u32x4 op[4];  // V^T operands for d tiles 4*q4 .. 4*q4+3
#pragma unroll
                for (int pr = 0; pr < 4; ++pr) {
                    const uint32_t w0 = vdword<D>(vraw[2 * pr], q4);
                    const uint32_t w1 = vdword<D>(vraw[2 * pr + 1], q4);
                    const uint32_t lo = __builtin_amdgcn_perm(w1, w0, 0x05010400u);  // b0 of w0,w1 | b1 of w0,w1
                    const uint32_t hi = __builtin_amdgcn_perm(w1, w0, 0x07030602u);  // b2 of w0,w1 | b3 of w0,w1
                    op[0][pr] = e4m3x2_to_f16x2<false>(lo);
                    op[1][pr] = e4m3x2_to_f16x2<true>(lo);
                    op[2][pr] = e4m3x2_to_f16x2<false>(hi);
                    op[3][pr] = e4m3x2_to_f16x2<true>(hi);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const f16x8 vop = bit_cast_<f16x8>(op[u]);
#pragma unroll
                    for (int nt = 0; nt < RT; ++nt)
                        st.acc[4 * q4 + u][nt] =
                            __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[nt], st.acc[4 * q4 + u][nt], 0, 0, 0);
                }
            }
        }
    }

    // ---- merge the four wave states in wave order ----
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) st.l[nt] = wave_sum_xor_16_32(st.l[nt]);
    if (lg == 0) {
#pragma unroll
        for (int nt = 0; nt < RT; ++nt) lds_ml[wave][nt * 16 + lc] = make_float2(st.m[nt], st.l[nt]);
    }
    __syncthreads();  // also: every wave is done reading Q from lds
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
        for (int md = 0; md < MD; ++md) st.acc[md][nt] *= fmine;
    }
    for (int w = 1; w < kWaves; ++w) {
        if (wave == w) {
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int nt = 0; nt < RT; ++nt) lds[(md * RT + nt) * 64 + lane] = bit_cast_<u32x4>(st.acc[md][nt]);
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int md = 0; md < MD; ++md)
#pragma unroll
                for (int nt = 0; nt < RT; ++nt)
                    st.acc[md][nt] += bit_cast_<f32x4>(lds[(md * RT + nt) * 64 + lane]);
        }
        __syncthreads();
    }
    if (wave != 0) return;

    // ---- emit the split partial: (max, sum) and the unnormalized PV ----
    const int64_t slot_base = (((int64_t)split * a.batch + b) * a.num_kv_heads + g) * a.rows;
#pragma unroll
    for (int nt = 0; nt < RT; ++nt) {
        const int r = r_begin + nt * 16 + lc;
        if (r >= a.rows) continue;
        if (lg == 0) reinterpret_cast<float2*>(a.ws_ml)[slot_base + r] = make_float2(M[nt], Ltot[nt]);
        float* dst = a.ws_acc + (slot_base + r) * D;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // accumulator element i of every d tile md is column (4*lg + i) * MD + md
            float vals[MD];
#pragma unroll
            for (int md = 0; md < MD; ++md) vals[md] = st.acc[md][nt][i];
            float* p = dst + (4 * lg + i) * MD;
#pragma unroll
            for (int k = 0; k < MD; k += 4)
                *reinterpret_cast<f32x4*>(p + k) = f32x4{vals[k], vals[k + 1], vals[k + 2], vals[k + 3]};
        }
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

// One workgroup (4 waves) per output row (request, KV head, row). Wave w sums
// a contiguous quarter of the visible splits in ascending order; the quarters
// are then added in wave order. Each lane owns head_dim/64 columns.
template <int D>
__global__ __launch_bounds__(256) void pfs_combine_kernel(const CombineArgs a) {
    constexpr int CPL = D / 64;  // columns per lane
    __shared__ float red[kWaves];
    __shared__ float part_l[kWaves];
    __shared__ float part_acc[kWaves][D];

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

    // global max over the visible splits (max is exact: any order)
    float mx = -INFINITY;
    for (int s = threadIdx.x; s < ns; s += 256) mx = fmaxf(mx, ml[slot0 + s * stride].x);
    for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    // this wave's contiguous quarter of the splits, ascending
    const int per = (ns + kWaves - 1) / kWaves;
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
            const f32x4 x = *reinterpret_cast<const f32x4*>(src);
            acc[0] += f * x[0];
            acc[1] += f * x[1];
            acc[2] += f * x[2];
            acc[3] += f * x[3];
        } else {
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] += f * src[c];
        }
    }
    if (lane == 0) part_l[wave] = lw;
#pragma unroll
    for (int c = 0; c < CPL; ++c) part_acc[wave][lane * CPL + c] = acc[c];
    __syncthreads();
    if (wave != 0) return;
    const float lt = ((part_l[0] + part_l[1]) + part_l[2]) + part_l[3];
    const float vs = a.vscale[g];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        const int d = lane * CPL + c;
        const float num = ((part_acc[0][d] + part_acc[1][d]) + part_acc[2][d]) + part_acc[3][d];
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
hipError_t launch_split(const SplitArgs& a, int32_t num_splits, hipStream_t stream) {
    const dim3 grid(num_splits, a.num_kv_heads * a.row_blocks, a.batch);
    hipLaunchKernelGGL((pfs_split_kernel<D, RT>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_split_d(const SplitArgs& a, int32_t row_tiles, int32_t num_splits, hipStream_t stream) {
    switch (row_tiles) {
        case 1: return launch_split<D, 1>(a, num_splits, stream);
        case 2: return launch_split<D, 2>(a, num_splits, stream);
        case 4: return launch_split<D, 4>(a, num_splits, stream);
        default: break;
    }
    if constexpr (D <= 128) {
        if (row_tiles == 8) return launch_split<D, 8>(a, num_splits, stream);
    }
    if constexpr (D == 64) {
        if (row_tiles == 16) return launch_split<D, 16>(a, num_splits, stream);
    }
    return hipErrorInvalidValue;
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
    sa.row_blocks = plan->row_blocks;
    sa.sm_scale_log2e = p.sm_scale * kLog2e;
    for (int i = 0; i < pfs::kMaxQHeads; ++i) sa.qhead[i] = plan->qhead[i];

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e;
    switch (p.head_dim) {
        case 64: e = launch_split_d<64>(sa, plan->row_tiles, plan->num_splits, s); break;
        case 128: e = launch_split_d<128>(sa, plan->row_tiles, plan->num_splits, s); break;
        case 256: e = launch_split_d<256>(sa, plan->row_tiles, plan->num_splits, s); break;
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
        case 64: hipLaunchKernelGGL(pfs_combine_kernel<64>, grid, dim3(256), 0, s, ca); break;
        case 128: hipLaunchKernelGGL(pfs_combine_kernel<128>, grid, dim3(256), 0, s, ca); break;
        case 256: hipLaunchKernelGGL(pfs_combine_kernel<256>, grid, dim3(256), 0, s, ca); break;
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
