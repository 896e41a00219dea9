"""pfs_verify_noalloc through the C ABI: the verify step with the split
partials in the library's per-GPU device array instead of a caller
workspace. Same plan, same kernels, so its output must equal pfs_verify's
bit for bit; checked on two calls in a row, the second with a smaller input
(fewer requests, shorter contexts), and both against the FP64 oracle."""
import numpy as np
import pytest

import paged_fp8_split_amd as pfs
from paged_fp8_split_amd import _lib
from paged_fp8_split_amd import workloads as W

from parity import device, assert_parity, log, oracle_ref, to_np

pytestmark = pytest.mark.gpu


def _both(w):
    import torch

    t = W.device_tensors(w, device())
    plan = pfs.make_plan(batch=w.batch, q=w.q, num_q_heads=w.num_q_heads, head_map=t["head_map"],
                         k_pool=t["k_pool"], max_pages_per_row=w.max_pages_per_row, sm_scale=t["sm_scale"])
    assert plan.workspace_bytes <= _lib.noalloc_scratch_bytes()
    ref_out = torch.full_like(t["q"], float("nan"))
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=t["q"].device)
    _lib.verify(plan, t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"],
                t["live_len"], ref_out, ws)
    out = torch.full_like(t["q"], float("nan"))
    _lib.verify_noalloc(plan, t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"],
                        t["live_len"], out)
    return to_np(out), to_np(ref_out)


def test_noalloc_matches_verify_on_two_calls_the_second_smaller():
    big = W.build(seed=301, batch=3, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                  lengths=[20000, 9000, 4097], outlier_frac=0.01)
    small = W.build(seed=302, batch=2, q=4, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                    lengths=[700, 33])
    for name, w in (("first, larger", big), ("second, smaller", small)):
        log(f"[noalloc] {name}: {w.name}")
        y, yref = _both(w)
        assert np.array_equal(y.view(np.uint16), yref.view(np.uint16)), name
        assert_parity(y, oracle_ref(w), f"noalloc {name}")


def test_noalloc_refuses_a_plan_beyond_its_array():
    w = W.build(seed=303, batch=1, q=1, num_q_heads=1, num_kv_heads=1, head_dim=64, page_size=16, lengths=[16])
    t = W.device_tensors(w, device())
    # 128 requests of 16 query heads at head_dim 256 over 65,536-token rows: far beyond 128 MiB of partials
    plan = _lib.Plan(batch=128, q=16, num_q_heads=16, num_kv_heads=1, head_dim=256, page_size=64,
                     max_pages_per_row=1024, num_pool_pages=4, kv_page_stride=64 * 256, kv_token_stride=256,
                     kv_head_stride=256, sm_scale=0.0625, head_map=[0] * 16)
    assert plan.workspace_bytes > _lib.noalloc_scratch_bytes()
    with pytest.raises(_lib.PfsError, match="PFS_ERR_WORKSPACE"):
        _lib.verify_noalloc(plan, t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"],
                            t["live_len"], t["q"])


def test_package_verify_noalloc_option_matches():
    """pfs.verify(..., noalloc=True) routes to pfs_verify_noalloc: same
    bytes as the workspace route; a workspace with it is an error."""
    w = W.build(seed=304, batch=2, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                lengths=[5000, 1500])
    t = W.device_tensors(w, device())
    args = (t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"], t["live_len"])
    kw = dict(head_map=t["head_map"], sm_scale=t["sm_scale"])
    a = to_np(pfs.verify(*args, **kw))
    import torch

    out = torch.full_like(t["q"], float("nan"))
    b = to_np(pfs.verify(*args, **kw, out=out, noalloc=True))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    with pytest.raises(ValueError, match="noalloc"):
        pfs.verify(*args, **kw, workspace=torch.empty(16, dtype=torch.uint8, device=t["q"].device), noalloc=True)
