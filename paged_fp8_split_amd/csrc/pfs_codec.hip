// pfs_codec.hip -- gfx950 kernels at the two ends of the paged E4M3 KV cache.
//
//   pfs_append_kernel   quantize-on-write: the FP16 K/V of every request's q
//                       draft tokens -> FP8 bytes in the paged pools (the
//                       step before verify: "[Kernel] Preserve DFlash2
//                       sampling precision and repair QUASAR TP2", Purpose,
//                       deferred accepted-slot writes; "[Bugfix] Use FP32
//                       state and E4M3 defaults for DFlash2", Test Plan, KV
//                       scaling)
//   pfs_bridge_kernel   paged FP8 -> dense FP16, optionally scaled
//                       ("[Kernel][SM70] Add opt-in E4M3 grouped attention
//                       with FP32 partials", Scope list: a call of its own
//                       that turns the paged FP8 cache into FP16)
//
// Both kernels exist for the two KV formats (template parameter FMT): OCP
// E4M3FN, the method's format, and E5M2, the explicit alternative ("[Bugfix]
// Use FP32 state and E4M3 defaults for DFlash2", Purpose).
//
// Encoding: the stored byte is the code nearest to the FP32 quotient
// x / scale (IEEE single division), ties to even, saturating at the largest
// finite value (448 for E4M3, 57344 for E5M2: the quotient is clamped first,
// so infinities saturate too); a NaN quotient stores 0x7F, a NaN code of
// both formats. The hardware conversions v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32
// round to nearest even.
//
// Bridge: dec(byte) * scale has up to 28 significant bits, so the FP32
// product can be inexact; the kernel rounds it to odd in FP32 (product plus
// its exact FMA error term) and then once to FP16, which equals one
// round-to-nearest-even of the exact product (FP32 keeps more than two bits
// beyond FP16's). Without a scale the decode is exact: E4M3 through the
// hardware conversion, E5M2 by placing each byte above a zero byte (an E5M2
// byte is the high byte of its FP16 value).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pfs_internal.h"

namespace {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int32_t clamp_len(int32_t v, int32_t hi) { return v < 0 ? 0 : (v > hi ? hi : v); }

// Code of x / s for one FP32 value pair (x0 in the low byte).
template <int FMT>
__device__ __forceinline__ uint32_t encode2(float x0, float x1, float s) {
    constexpr float kMax = FMT == PFS_KV_E5M2 ? 57344.0f : 448.0f;
    const float q0 = x0 / s, q1 = x1 / s;
    const float c0 = fminf(fmaxf(q0, -kMax), kMax);
    const float c1 = fminf(fmaxf(q1, -kMax), kMax);
    uint32_t w;
    if constexpr (FMT == PFS_KV_E5M2)
        w = (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(c0, c1, 0, false) & 0xFFFFu;
    else
        w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false) & 0xFFFFu;
    if (q0 != q0) w = (w & 0xFF00u) | 0x7Fu;
    if (q1 != q1) w = (w & 0x00FFu) | 0x7F00u;
    return w;
}

// 8 FP16 values (one 16-byte word) -> 8 code bytes (two dwords).
template <int FMT>
__device__ __forceinline__ u32x2 encode8(u32x4 h, float s) {
    u32x2 r;
    const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
    uint32_t b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f16x2 v = __builtin_bit_cast(f16x2, hw[k]);
        b[k] = encode2<FMT>((float)v.x, (float)v.y, s);
    }
    r.x = b[0] | (b[1] << 16);
    r.y = b[2] | (b[3] << 16);
    return r;
}

struct AppendArgs {
    const u32x4* k_new;  // [batch, q, Hkv, D] FP16, 16-byte words
    const u32x4* v_new;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_table;
    const int32_t* live_len;
    uint8_t* k_pool;
    uint8_t* v_pool;
    int64_t page_stride;
    int64_t token_stride;
    int64_t head_stride;
    int32_t q;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t max_pages;
    int32_t capacity;
    int64_t words;  // batch * q * Hkv * D / 8
};

// One thread per 8 elements (one FP16 word) of one (request, draft row, KV
// head): reads K and V, writes 8 bytes into each pool.
template <int FMT>
__global__ __launch_bounds__(256) void pfs_append_kernel(const AppendArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= a.words) return;
    const int wpr = a.head_dim / 8;  // words per (row, head)
    const int c = (int)(idx % wpr);
    const int g = (int)((idx / wpr) % a.num_kv_heads);
    const int64_t row = idx / ((int64_t)wpr * a.num_kv_heads);  // b * q + i
    const int i = (int)(row % a.q);
    const int b = (int)(row / a.q);
    const int32_t L = clamp_len(a.live_len[b], a.capacity);
    const int32_t t = L - a.q + i;
    if (t < 0) return;  // no slot for this draft row
    const int32_t page = a.block_table[(int64_t)b * a.max_pages + t / a.page_size];
    const int64_t off = (int64_t)page * a.page_stride + (int64_t)(t % a.page_size) * a.token_stride +
                        (int64_t)g * a.head_stride + 8 * c;
    *reinterpret_cast<u32x2*>(a.k_pool + off) = encode8<FMT>(a.k_new[idx], a.k_scale[g]);
    *reinterpret_cast<u32x2*>(a.v_pool + off) = encode8<FMT>(a.v_new[idx], a.v_scale[g]);
}

// FP16 of v * s (v an exactly decoded byte), rounded once: round the FP32
// product to odd, then to FP16.
__device__ __forceinline__ _Float16 scaled_half(float v, float s) {
    const float p = v * s;
    if (p == 0.0f || !isfinite(p)) return (_Float16)p;
    const float e = __builtin_fmaf(v, s, -p);  // v * s == p + e exactly
    uint32_t pb = __builtin_bit_cast(uint32_t, p);
    if (e != 0.0f) {
        if ((e < 0.0f) != (p < 0.0f)) pb -= 1;  // truncate toward zero
        pb |= 1u;                               // sticky bit: round to odd
    }
    return (_Float16)__builtin_bit_cast(float, pb);
}

struct BridgeArgs {
    const uint8_t* pool;
    const float* scale;  // [Hkv] or nullptr
    const int32_t* block_table;
    const int32_t* live_len;
    _Float16* out;  // [batch, capacity, Hkv, D]
    int64_t page_stride;
    int64_t token_stride;
    int64_t head_stride;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t max_pages;
    int32_t capacity;
};

// Exact FP16 of two code bytes (bytes 2*HI and 2*HI+1 of `w`).
template <int FMT, bool HI>
__device__ __forceinline__ uint32_t decode2(uint32_t w) {
    if constexpr (FMT == PFS_KV_E5M2)
        return __builtin_amdgcn_perm(w, w, HI ? 0x030C020Cu : 0x010C000Cu);
    else
        return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// One thread per 16 bytes of one (token, KV head); blockIdx.y is the request.
template <int FMT>
__global__ __launch_bounds__(256) void pfs_bridge_kernel(const BridgeArgs a) {
    const int chunks = a.head_dim / 16;
    const int64_t per_tok = (int64_t)a.num_kv_heads * chunks;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int b = blockIdx.y;
    if (idx >= (int64_t)a.capacity * per_tok) return;
    const int32_t t = (int32_t)(idx / per_tok);
    const int g = (int)((idx / chunks) % a.num_kv_heads);
    const int c = (int)(idx % chunks);
    const int32_t L = clamp_len(a.live_len[b], a.capacity);
    u32x4 res[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    if (t < L) {
        const int64_t page = a.block_table[(int64_t)b * a.max_pages + t / a.page_size];
        const u32x4 w = *reinterpret_cast<const u32x4*>(a.pool + page * a.page_stride +
                                                        (int64_t)(t % a.page_size) * a.token_stride +
                                                        (int64_t)g * a.head_stride + 16 * c);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            // exact FP16 decode of two bytes each (every E4M3 and E5M2 value is an FP16 number)
            h[2 * k] = decode2<FMT, false>(ws[k]);
            h[2 * k + 1] = decode2<FMT, true>(ws[k]);
        }
        if (a.scale) {
            const float s = a.scale[g];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const f16x2 v = __builtin_bit_cast(f16x2, h[k]);
                const f16x2 r = f16x2{scaled_half((float)v.x, s), scaled_half((float)v.y, s)};
                h[k] = __builtin_bit_cast(uint32_t, r);
            }
        }
        res[0] = u32x4{h[0], h[1], h[2], h[3]};
        res[1] = u32x4{h[4], h[5], h[6], h[7]};
    }
    u32x4* dst = reinterpret_cast<u32x4*>(a.out + (((int64_t)b * a.capacity + t) * a.num_kv_heads + g) * a.head_dim +
                                          16 * c);
    dst[0] = res[0];
    dst[1] = res[1];
}

}  // namespace

int32_t pfs_launch_append(const pfs_plan* plan, const void* k_new, const void* v_new, const float* k_scale,
                          const float* v_scale, const int32_t* block_table, const int32_t* live_len,
                          uint8_t* k_pool, uint8_t* v_pool, pfs_stream_t stream) {
    const pfs_problem& p = plan->p;
    AppendArgs a;
    a.k_new = static_cast<const u32x4*>(k_new);
    a.v_new = static_cast<const u32x4*>(v_new);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_table = block_table;
    a.live_len = live_len;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.page_stride = p.kv_page_stride;
    a.token_stride = p.kv_token_stride;
    a.head_stride = p.kv_head_stride;
    a.q = p.q;
    a.num_kv_heads = p.num_kv_heads;
    a.head_dim = p.head_dim;
    a.page_size = p.page_size;
    a.max_pages = p.max_pages_per_row;
    a.capacity = plan->capacity;
    a.words = (int64_t)p.batch * p.q * p.num_kv_heads * (p.head_dim / 8);
    const int64_t blocks = (a.words + 255) / 256;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.kv_format == PFS_KV_E5M2)
        hipLaunchKernelGGL(pfs_append_kernel<PFS_KV_E5M2>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(pfs_append_kernel<PFS_KV_E4M3>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? PFS_OK : PFS_ERR_LAUNCH;
}

int32_t pfs_launch_bridge(const pfs_plan* plan, const uint8_t* pool, const float* scale, const int32_t* block_table,
                          const int32_t* live_len, void* out, pfs_stream_t stream) {
    const pfs_problem& p = plan->p;
    BridgeArgs a;
    a.pool = pool;
    a.scale = scale;
    a.block_table = block_table;
    a.live_len = live_len;
    a.out = static_cast<_Float16*>(out);
    a.page_stride = p.kv_page_stride;
    a.token_stride = p.kv_token_stride;
    a.head_stride = p.kv_head_stride;
    a.num_kv_heads = p.num_kv_heads;
    a.head_dim = p.head_dim;
    a.page_size = p.page_size;
    a.max_pages = p.max_pages_per_row;
    a.capacity = plan->capacity;
    const int64_t threads = (int64_t)plan->capacity * p.num_kv_heads * (p.head_dim / 16);
    const dim3 grid((unsigned)((threads + 255) / 256), p.batch);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (p.kv_format == PFS_KV_E5M2)
        hipLaunchKernelGGL(pfs_bridge_kernel<PFS_KV_E5M2>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(pfs_bridge_kernel<PFS_KV_E4M3>, grid, dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? PFS_OK : PFS_ERR_LAUNCH;
}
