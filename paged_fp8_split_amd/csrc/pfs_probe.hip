// pfs_probe.hip -- libpfs_probe.so: read-bandwidth probes for the roofline
// of the verify step (bench.py --ceiling). Measurement only: nothing here is
// on the verify path, and libpfs does not use it.
//
// Both paged probes read exactly the live K and V bytes the split kernel
// reads, with its work units (one workgroup of 512 threads per (split, KV
// head), 16-byte loads, pages resolved through the block table) and no
// arithmetic, and fold what they read into a per-thread XOR written to a sink
// so that no load is dead:
//   pfs_probe_paged_regs  loads into registers, several 16-byte loads per
//                         lane in flight;
//   pfs_probe_paged_lds   loads straight into LDS (buffer_load ... lds) into a
//                         ring of four 32 KB stages with the split kernel's
//                         pipeline (two stages in flight beside the one being
//                         read, a barrier per stage).
// pfs_probe_flat_regs reads a flat buffer with the same register loads (the
// best case for the access size).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct PagedArgs {
    const uint8_t* kpool;
    const uint8_t* vpool;
    const int32_t* block_table;  // one request's row
    int64_t page_stride, token_stride, head_stride;
    int32_t page_size;
    int32_t head_dim;
    int32_t tokens_per_split;
    int32_t num_splits;
    int32_t live_len;
    uint32_t* sink;  // [grid][512]
};

constexpr int kThreads = 512;

__device__ __forceinline__ int64_t row_offset(const PagedArgs& a, int32_t t, int g) {
    const int32_t page = a.block_table[t / a.page_size];
    return (int64_t)page * a.page_stride + (int64_t)(t % a.page_size) * a.token_stride + (int64_t)g * a.head_stride;
}

// Unit (split, g): tokens [split * T, min((split + 1) * T, L)). A pass covers
// kThreads * 16 bytes of K and as many of V: (8192 / head_dim) tokens; U
// passes are loaded before any is folded.
__global__ __launch_bounds__(kThreads) void pfs_probe_paged_regs(const PagedArgs a) {
    constexpr int U = 8;
    const int split = blockIdx.x % a.num_splits;
    const int g = blockIdx.x / a.num_splits;
    const int32_t tok0 = split * a.tokens_per_split;
    const int32_t tok_end = min(tok0 + a.tokens_per_split, a.live_len);
    const int chunks = a.head_dim / 16;           // 16-byte chunks per token row
    const int tokens_per_pass = kThreads / chunks;
    const int t_lane = threadIdx.x / chunks;
    const int c_lane = threadIdx.x % chunks;
    uint32_t x = 0;
    for (int32_t t0 = tok0; t0 < tok_end; t0 += U * tokens_per_pass) {
        u32x4 kv[2 * U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t t = t0 + u * tokens_per_pass + t_lane;
            const int32_t tc = t < tok_end ? t : tok0;  // (in bounds; selected out below)
            const int64_t off = row_offset(a, tc, g) + 16 * c_lane;
            kv[2 * u] = *reinterpret_cast<const u32x4*>(a.kpool + off);
            kv[2 * u + 1] = *reinterpret_cast<const u32x4*>(a.vpool + off);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = t0 + u * tokens_per_pass + t_lane < tok_end;
            const u32x4 s = kv[2 * u] ^ kv[2 * u + 1];
            x ^= live ? (s.x ^ s.y ^ s.z ^ s.w) : 0u;
        }
    }
    a.sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = x;
}

__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voffset, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm_and_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// A stage holds two rounds of 512 threads x 16 bytes of K and as many of V
// (64 tokens' rows at head_dim 256: 32 KB, like a stage of the split kernel).
// A wave's 16-byte loads cover 64 / (head_dim / 16) consecutive tokens of one
// page (token groups are aligned and pages hold a multiple of 16 tokens), so
// each load has one buffer descriptor for the wave, at that group's first
// row, whose record count ends at the live length (rows past it land as
// zeros), and per-lane offsets. Stages 0..2 are issued first; iteration s
// waits until stage s + 1 has landed (stage s + 2 still in flight), meets the
// other waves at the barrier, issues stage s + 3 into the buffer stage s - 1
// used, and XOR-folds its own 64 bytes of stage s from LDS: two stages in
// flight beside the one being read, the split kernel's pipeline without its
// arithmetic.
__global__ __launch_bounds__(kThreads) void pfs_probe_paged_lds(const PagedArgs a) {
    constexpr int NS = 4;
    constexpr int SB = 32768;
    constexpr int LOADS = 4;  // per thread per stage: two rounds of K and V
    __shared__ __attribute__((aligned(16))) uint8_t st0[SB];
    __shared__ __attribute__((aligned(16))) uint8_t st1[SB];
    __shared__ __attribute__((aligned(16))) uint8_t st2[SB];
    __shared__ __attribute__((aligned(16))) uint8_t st3[SB];
    uint8_t* const stages[NS] = {st0, st1, st2, st3};
    const int split = blockIdx.x % a.num_splits;
    const int g = blockIdx.x / a.num_splits;
    const int32_t tok0 = split * a.tokens_per_split;
    const int32_t tok_end = min(tok0 + a.tokens_per_split, a.live_len);
    const int chunks = a.head_dim / 16;            // 16-byte chunks per token row
    const int round_tokens = kThreads / chunks;    // tokens per round of 512 loads
    const int wave_tokens = 64 / chunks;           // tokens per wave load
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t voff = (uint32_t)(lane / chunks) * (uint32_t)a.token_stride + 16u * (uint32_t)(lane % chunks);
    const int nstages = (tok_end - tok0 + 2 * round_tokens - 1) / (2 * round_tokens);
    auto issue = [&](int s, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int32_t tw = tok0 + (2 * s + rr) * round_tokens + wave * wave_tokens;  // uniform
            const int32_t n = (s < nstages) ? min(max(tok_end - tw, 0), wave_tokens) : 0;
            const int64_t off = n > 0 ? row_offset(a, tw, g) : 0;
            const uint32_t rec = (uint32_t)n * (uint32_t)a.token_stride;
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.kpool + off), (short)0, (int)rec, 0x00020000);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.vpool + off), (short)0, (int)rec, 0x00020000);
            load_lds16(rk, dst + rr * (SB / 2) + wave * 1024, voff);
            load_lds16(rv, dst + rr * (SB / 2) + SB / 4 + wave * 1024, voff);
        }
    };
    uint32_t x = 0;
    issue(0, stages[0]);
    issue(1, stages[1]);
    issue(2, stages[2]);
    for (int s0 = 0; s0 < nstages; s0 += NS) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int s = s0 + k;
            wait_vm_and_barrier<LOADS>();  // stages s and s + 1 landed (s + 2 in flight)
            issue(s + 3, stages[(k + 3) % NS]);
            if (s < nstages) {
#pragma unroll
                for (int j = 0; j < LOADS; ++j) {
                    const u32x4 w = *reinterpret_cast<const u32x4*>(stages[k] + j * (SB / 4) + 16 * threadIdx.x % (SB / 4));
                    x ^= w.x ^ w.y ^ w.z ^ w.w;
                }
            }
        }
    }
    wait_vm_and_barrier<0>();
    a.sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = x;
}

__global__ __launch_bounds__(kThreads) void pfs_probe_flat_regs(const uint8_t* buf, int64_t bytes, uint32_t* sink) {
    constexpr int U = 8;
    const int64_t stride = (int64_t)gridDim.x * kThreads * 16;
    uint32_t x = 0;
    for (int64_t base = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 16; base < bytes; base += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t o = base + u * stride;
            v[u] = *reinterpret_cast<const u32x4*>(buf + (o < bytes ? o : 0));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) x ^= (base + u * stride < bytes) ? (v[u].x ^ v[u].y ^ v[u].z ^ v[u].w) : 0u;
    }
    sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = x;
}

}  // namespace

extern "C" {

// mode 0: register loads, 1: direct-to-LDS ring. One request (the row
// block_table), num_splits x num_kv_heads workgroups of 512 threads; sink
// holds 512 uint32 per workgroup. Returns 0, or -3 for an unsupported
// head_dim (64, 128, 256) and -7 for a launch error.
int32_t pfs_probe_paged(int32_t mode, const uint8_t* k_pool, const uint8_t* v_pool, const int32_t* block_table,
                        int64_t page_stride, int64_t token_stride, int64_t head_stride, int32_t page_size,
                        int32_t head_dim, int32_t num_kv_heads, int32_t tokens_per_split, int32_t num_splits,
                        int32_t live_len, uint32_t* sink, hipStream_t stream) {
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return -3;
    PagedArgs a{k_pool, v_pool, block_table, page_stride, token_stride, head_stride, page_size, head_dim,
                tokens_per_split, num_splits, live_len, sink};
    const dim3 grid((unsigned)(num_splits * num_kv_heads));
    if (mode == 0)
        hipLaunchKernelGGL(pfs_probe_paged_regs, grid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(pfs_probe_paged_lds, grid, dim3(kThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

// Reads `bytes` (a multiple of 16) of buf with `grid` workgroups of 512
// threads; sink holds 512 uint32 per workgroup.
int32_t pfs_probe_flat(const uint8_t* buf, int64_t bytes, int32_t grid, uint32_t* sink, hipStream_t stream) {
    hipLaunchKernelGGL(pfs_probe_flat_regs, dim3((unsigned)grid), dim3(kThreads), 0, stream, buf, bytes, sink);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
