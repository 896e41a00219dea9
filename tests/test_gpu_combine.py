"""The many-split combine (plans with more than 32 splits): the splits are cut
into 16 contiguous blocks (32 at head_dim 64), each folded in ascending
order, and the block states are merged in a fixed pairwise tree across the
lanes of a wave and then across the workgroup's 8 waves (include/pfs.h,
pfs_verify_combine). These cases give every head_dim a split count just above
the row kernel's 32 (so that some blocks hold no split at all), counts that
do not divide into the blocks, and a second request whose visible splits end
inside a block, so that the combine selects out splits past the live length
and merges blocks that hold nothing visible. Each output is checked against
the FP64 oracle, and a second launch must give the same bytes. A request run
alone and in a batch gives the same bytes too (both combine variants: first
reads ahead of the live length for one request, after it in a batch)."""
import numpy as np
import pytest

import paged_fp8_split_amd as pfs
from paged_fp8_split_amd import workloads as W

from parity import device, assert_parity, log, oracle_ref, run, to_np

pytestmark = pytest.mark.gpu

TPS = 64  # one split per 64-token partition: many splits from short contexts

# (head_dim, splits per request)
CASES = [(64, 33), (64, 257), (128, 33), (128, 100), (256, 47), (256, 600)]


@pytest.mark.parametrize("head_dim,splits", CASES, ids=[f"d{d}-s{s}" for d, s in CASES])
def test_many_split_combine_matches_oracle(head_dim, splits):
    cap = splits * TPS
    # request 0 fills all but the last few tokens of its last split; request 1
    # ends a third of the way in, inside a split block
    lengths = [cap - 7, cap // 3 + 5]
    w = W.build(seed=900 + head_dim + splits, batch=2, q=8, num_q_heads=8, num_kv_heads=2, head_dim=head_dim,
                page_size=64, lengths=lengths, capacity=cap, outlier_frac=0.01)
    t = W.device_tensors(w, device())
    plan = pfs.make_plan(batch=w.batch, q=w.q, num_q_heads=w.num_q_heads, head_map=t["head_map"],
                         k_pool=t["k_pool"], max_pages_per_row=w.max_pages_per_row, sm_scale=t["sm_scale"],
                         tokens_per_split=TPS)
    assert plan.num_splits == splits
    log(f"[combine] d{head_dim}: {splits} splits, lengths {lengths}")
    y1 = to_np(run(w, tokens_per_split=TPS, tensors=t)[0])
    assert_parity(y1, oracle_ref(w), f"many-split combine d{head_dim} s{splits}")
    y2 = to_np(run(w, tokens_per_split=TPS, tensors=t)[0])
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


# (head_dim, q, query heads, KV heads, tokens per split, lengths): one row
# group per row block, so a lone request and a batch share the split kernel's
# geometry; 48 and 40 splits take the many-split combine, 20 the row kernel
INVARIANCE = [(64, 8, 4, 1, 64, [3000, 1500]), (128, 4, 8, 2, 64, [2500, 900]), (256, 2, 16, 2, 256, [5000, 2100])]


@pytest.mark.parametrize("head_dim,q,hq,hkv,tps,lengths", INVARIANCE,
                         ids=[f"d{c[0]}-s{-(-max(c[5]) // c[4])}" for c in INVARIANCE])
def test_a_request_does_not_depend_on_its_batch(head_dim, q, hq, hkv, tps, lengths):
    """Request 0 alone (a one-request plan, whose combine issues its first
    reads before the live length arrives) and in a batch of two (whose combine
    waits for each length and reads only visible splits) gives the same
    bytes: the split boundaries and the order of the sum are the plan's, not
    the batch's."""
    w = W.build(seed=77 + head_dim, batch=2, q=q, num_q_heads=hq, num_kv_heads=hkv, head_dim=head_dim,
                page_size=64, lengths=lengths, outlier_frac=0.01)
    t = W.device_tensors(w, device())
    kw = dict(head_map=t["head_map"], sm_scale=t["sm_scale"], tokens_per_split=tps)
    both = to_np(pfs.verify(t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"],
                            t["live_len"], **kw))
    alone = to_np(pfs.verify(t["q"][:1], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"][:1],
                             t["live_len"][:1], **kw))
    log(f"[batch invariance] d{head_dim} q{q} {hq}/{hkv} heads, {tps}-token splits, lengths {lengths}")
    assert_parity(both, oracle_ref(w), f"batch of two d{head_dim}")
    assert np.array_equal(alone[0].view(np.uint16), both[0].view(np.uint16))
