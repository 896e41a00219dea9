/*
 * A plain C99 client of include/pfs.h, built and run by
 * tests/test_abi_host.py: it plans the 256K-context q8 verify shape (one
 * request, 16 query / 2 KV heads, head_dim 256, page 64, token-major pool),
 * prints what the plan chose, checks that a token stride the 16-byte loads
 * cannot use is refused with its own status, and releases the plan. Host only:
 * no device call is made.
 */
#include <stdint.h>
#include <stdio.h>

#include "pfs.h"

int main(void) {
    if (pfs_abi_version() != PFS_ABI_VERSION) {
        printf("abi %d against header %d\n", (int)pfs_abi_version(), PFS_ABI_VERSION);
        return 1;
    }
    int32_t head_map[16];
    for (int h = 0; h < 16; ++h) head_map[h] = h / 8;
    pfs_problem p = {0};
    p.batch = 1;
    p.q = 8;
    p.num_q_heads = 16;
    p.num_kv_heads = 2;
    p.head_dim = 256;
    p.page_size = 64;
    p.max_pages_per_row = 4096;
    p.num_pool_pages = 5120;
    p.partition_tokens = 64;
    p.tokens_per_split = 0;
    p.kv_format = PFS_KV_E4M3;
    p.pv_mode = PFS_PV_HIGH_RESIDUAL;
    p.num_cus = 0;
    p.kv_page_stride = 64 * 512;
    p.kv_token_stride = 512;
    p.kv_head_stride = 256;
    p.sm_scale = 0.0625f;
    p.q_head_to_kv_head = head_map;
    pfs_plan* plan = NULL;
    int32_t st = pfs_plan_create(&p, &plan);
    if (st != PFS_OK) {
        printf("plan: %s\n", pfs_status_string(st));
        return 1;
    }
    printf("splits %d tokens_per_split %d workspace %lld\n", (int)pfs_plan_num_splits(plan),
           (int)pfs_plan_tokens_per_split(plan), (long long)pfs_plan_workspace_bytes(plan));
    p.kv_token_stride = 264;
    pfs_plan* bad = NULL;
    st = pfs_plan_create(&p, &bad);
    printf("token stride 264: %s\n", pfs_status_string(st));
    pfs_plan_destroy(plan);
    pfs_plan_destroy(NULL);
    return (st == PFS_ERR_ALIGNMENT && bad == NULL) ? 0 : 1;
}
