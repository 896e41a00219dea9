// Host-only fuzz of the planner (paged_fp8_split_amd/csrc/pfs_plan.cpp), built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_abi_host.py: pfs_plan_create on random problems (each field
// valid 7 times in 8, else out of range), the invariants of every plan it
// accepts, and the host-side error paths of the other calls. The kernel
// launchers are stubs that must never be reached (every call here fails its
// argument checks first). Prints the number of plans made; exit status 0 when
// every check held.
#include <stdio.h>
#include <stdlib.h>
#include <math.h>
#include <string.h>
#include "../paged_fp8_split_amd/csrc/pfs_internal.h"
static int launched = 0;
int32_t pfs_launch_split(const pfs_plan*, const void*, const uint8_t*, const uint8_t*, const float*, const int32_t*,
                         const int32_t*, void*, pfs_stream_t) { ++launched; return PFS_OK; }
int32_t pfs_launch_combine(const pfs_plan*, const float*, const int32_t*, void*, const void*, pfs_stream_t) { ++launched; return PFS_OK; }
int32_t pfs_launch_append(const pfs_plan*, const void*, const void*, const float*, const float*, const int32_t*,
                          const int32_t*, uint8_t*, uint8_t*, pfs_stream_t) { ++launched; return PFS_OK; }
int32_t pfs_launch_bridge(const pfs_plan*, const uint8_t*, const float*, const int32_t*, const int32_t*, void*,
                          pfs_stream_t) { ++launched; return PFS_OK; }
static uint64_t s = 88172645463325252ull;
static uint64_t rnd() { s ^= s << 13; s ^= s >> 7; s ^= s << 17; return s; }
static int64_t pick(const int64_t* v, int n) { return v[rnd() % n]; }
// valid values first: with probability 7/8 choose among the first nv entries
static int64_t pickv(const int64_t* v, int nv, int n) { return (rnd() % 8) ? v[rnd() % nv] : v[rnd() % n]; }
int main(int argc, char** argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 200000;
    const int64_t batches[] = {0, 1, 2, 7, 32, 65535, -1, 65536, 1 << 30};
    const int64_t qs[] = {1, 5, 8, 16, -1, 0, 17};
    const int64_t hkvs[] = {1, 2, 4, 8, 256, -3, 0, 257};
    const int64_t Gs[] = {1, 2, 6, 8, 16, 0, 64, 256};
    const int64_t Ds[] = {64, 128, 256, -64, 0, 32, 512};
    const int64_t pages[] = {16, 64, 848, 3456, -16, 0, 8, 1 << 20};
    const int64_t pprs[] = {1, 7, 4096, -1, 0, 1 << 20, 1 << 30};
    const int64_t pools[] = {1, 5000, -1, 0, 1 << 30};
    const int64_t tpss[] = {0, 64, 256, 2048, 16384, -64, 100, 16448, 1 << 30};
    const int64_t cuss[] = {0, 40, 256, 304, 65536, -1, 65537};
    const int64_t pads[] = {0, 16, 256, -16, 8, 1 << 30};
    const float sms[] = {0.0f, -1.0f, 0.0625f, INFINITY, NAN, 1e30f};
    static int32_t head_map[1024];
    int ok = 0;
    for (int it = 0; it < iters; ++it) {
        pfs_problem p;
        memset(&p, 0, sizeof(p));
        p.batch = (int32_t)pickv(batches, 6, 9); p.q = (int32_t)pickv(qs, 4, 7);
        const int64_t hkv = pickv(hkvs, 5, 8), G = pickv(Gs, 5, 8);
        p.num_kv_heads = (int32_t)hkv; p.num_q_heads = (int32_t)(hkv * G > 1024 ? 1024 : hkv * G);
        p.head_dim = (int32_t)pickv(Ds, 3, 7); p.page_size = (int32_t)pickv(pages, 4, 8);
        p.max_pages_per_row = (int32_t)pickv(pprs, 3, 7); p.num_pool_pages = (int32_t)pickv(pools, 2, 5);
        p.partition_tokens = (rnd() % 8) ? 64 : 32; p.tokens_per_split = (int32_t)pickv(tpss, 5, 9);
        p.kv_format = (rnd() % 8) ? (int32_t)(rnd() % 2) : (int32_t)(rnd() % 4) - 1; p.pv_mode = (rnd() % 8) ? (int32_t)(rnd() % 2) : (int32_t)(rnd() % 4) - 1; p.num_cus = (int32_t)pickv(cuss, 5, 7);
        const int64_t pad = pickv(pads, 3, 6);
        p.kv_token_stride = hkv * p.head_dim + pad; p.kv_head_stride = p.head_dim;
        p.kv_page_stride = (int64_t)p.page_size * p.kv_token_stride;
        if (rnd() % 4 == 0) { p.kv_head_stride = (int64_t)p.page_size * p.head_dim + pad; p.kv_token_stride = p.head_dim;
                              p.kv_page_stride = hkv * p.kv_head_stride; }
        p.sm_scale = (rnd() % 8) ? 0.0625f : sms[rnd() % 6];
        const int nq = p.num_q_heads > 0 ? p.num_q_heads : 0;
        for (int h = 0; h < nq; ++h) head_map[h] = (int32_t)((G > 0 && (rnd() % 16)) ? h / G : (int64_t)(rnd() % 600) - 100);
        p.q_head_to_kv_head = head_map;
        pfs_plan* plan = NULL;
        const int32_t st = pfs_plan_create(&p, &plan);
        if (st == PFS_OK) {
            ++ok;
            const int64_t cap = (int64_t)p.max_pages_per_row * p.page_size;
            const int32_t t = pfs_plan_tokens_per_split(plan), n = pfs_plan_num_splits(plan);
            if (t % 64 || t < 64 || t > 16384 || (int64_t)n * t < cap || (int64_t)(n - 1) * t >= cap || pfs_plan_workspace_bytes(plan) <= 0) {
                printf("invariant broken at iteration %d\n", it); return 1;
            }
            // host-side error paths of the other calls (no launch may happen)
            char buf[64];
            void* ptr = (void*)(((uintptr_t)buf + 255) & ~(uintptr_t)255);
            pfs_verify(plan, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL);
            uint8_t* b8 = (uint8_t*)ptr; pfs_verify(plan, b8 + 8, b8, b8, (const float*)ptr, (const float*)ptr, (const int32_t*)ptr, (const int32_t*)ptr, ptr, ptr, 0, NULL);
            pfs_dequant_paged(plan, NULL, NULL, NULL, NULL, NULL, NULL);
            pfs_kv_append(plan, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL);
            pfs_plan_destroy(plan);
        } else if (st > 0 || st < -8 || plan != NULL) {
            printf("bad status %d at iteration %d\n", st, it); return 1;
        }
        (void)pfs_status_string(st);
    }
    (void)pfs_status_string(12345);
    printf("plans %d of %d, launches %d\n", ok, iters, launched);
    return launched == 0 ? 0 : 1;
}
