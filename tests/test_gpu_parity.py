"""GPU parity of the HIP path against the FP64 oracle, small and medium shapes,
plus the bitwise E4M3 dequant bridge. Everything goes through the C ABI."""
import zlib

import numpy as np
import pytest

import oracle
import paged_fp8_split_amd as pfs
from paged_fp8_split_amd import workloads as W

from parity import device, assert_parity, log, oracle_ref, run, to_np

pytestmark = pytest.mark.gpu


def _all_finite_codes(n):
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    return np.resize(codes, n)


@pytest.mark.parametrize("D", [64, 128, 256])
def test_dequant_bridge_is_exact_on_every_finite_code(D):
    import torch

    w = W.build(seed=20 + D, batch=3, q=1, num_q_heads=2, num_kv_heads=2, head_dim=D, page_size=16,
                lengths=[300, 77, 0], token_pad=16, page_pad=32)
    log(f"[dequant] D={D} lengths={w.live_len.tolist()}")
    view = w.pool_view(w.k_pool)
    for b in range(w.batch):
        L = int(w.live_len[b])
        if L == 0:
            continue
        t = np.arange(L)
        n = L * w.num_kv_heads * D
        view[w.block_table[b, t // 16], t % 16] = _all_finite_codes(n + 97 * b).reshape(-1)[-n:].reshape(L, 2, D)
    t = W.device_tensors(w, device())
    got = to_np(pfs.dequant_paged(t["k_pool"], t["block_table"], t["live_len"]))
    table = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float16).numpy()
    assert np.array_equal(table[~np.isnan(table)].astype(np.float16).view(np.uint16),
                          ref[~np.isnan(table)].view(np.uint16))
    cap = w.capacity
    for b in range(w.batch):
        L = int(w.live_len[b])
        tt = np.arange(L)
        raw = view[w.block_table[b, tt // 16], tt % 16]
        exp = table[raw].astype(np.float16)
        assert np.array_equal(got[b, :L].view(np.uint16), exp.view(np.uint16)), f"request {b}"
        assert np.all(got[b, L:cap].view(np.uint16) == 0)


SMALL = [
    # (name, build kwargs, tokens_per_split)
    ("d64-q8-g4-split64", dict(batch=1, q=8, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16,
                               lengths=[1032]), 64),
    ("d64-q8-g4-default", dict(batch=1, q=8, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16,
                               lengths=[1032]), 0),
    ("d128-q1-g8-ragged", dict(batch=3, q=1, num_q_heads=16, num_kv_heads=2, head_dim=128, page_size=64,
                               lengths=[1000, 37, 513]), 256),
    ("d128-q16-g8", dict(batch=2, q=16, num_q_heads=16, num_kv_heads=2, head_dim=128, page_size=32,
                         lengths=[777, 16]), 256),
    ("d256-q8-g8", dict(batch=2, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                        lengths=[2100, 300]), 512),
    ("d256-q3-g2-short", dict(batch=4, q=3, num_q_heads=4, num_kv_heads=2, head_dim=256, page_size=16,
                              lengths=[2, 0, 3, 130]), 0),
    ("d64-q16-g16-rowblocks", dict(batch=1, q=16, num_q_heads=16, num_kv_heads=1, head_dim=64, page_size=16,
                                   lengths=[600]), 256),
    ("d256-q16-g8-rowblocks", dict(batch=1, q=16, num_q_heads=8, num_kv_heads=1, head_dim=256, page_size=64,
                                   lengths=[700]), 256),
    # batches with four row groups run four-wave workgroups, two per CU
    ("d256-q16-g8-batch-rowblocks", dict(batch=3, q=16, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                                         lengths=[2500, 0, 777]), 0),
    ("d128-q16-g8-batch-ragged", dict(batch=4, q=16, num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=64,
                                      lengths=[5000, 64, 1, 3000]), 0),
    ("d128-q5-g6-padded", dict(batch=2, q=5, num_q_heads=12, num_kv_heads=2, head_dim=128, page_size=48,
                               lengths=[400, 90], token_pad=16, page_pad=64), 0),
    ("d64-outliers-pow2", dict(batch=2, q=8, num_q_heads=8, num_kv_heads=4, head_dim=64, page_size=16,
                               lengths=[900, 333], outlier_frac=0.02, scale_mode="pow2",
                               pow2_scale_exps=[-6, -3, 1, 4]), 0),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(case):
    name, kw, tps = case
    w = W.build(seed=zlib.crc32(name.encode()) % 1000, **kw)
    log(f"[small] {name} tps={tps}")
    out, _ = run(w, tokens_per_split=tps)
    assert_parity(to_np(out), oracle_ref(w), name)


def test_rows_without_visible_keys_are_positive_zero():
    w = W.build(seed=31, batch=3, q=8, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                lengths=[0, 5, 40])
    out = to_np(run(w)[0])
    bits = out.view(np.uint16)
    assert np.all(bits[0] == 0)           # retired request
    assert np.all(bits[1, :3] == 0)       # rows that see nothing (L < q)
    assert np.all(out[1, 3:] != 0)
    assert_parity(out, oracle_ref(w), "zero rows")


def test_head_major_pool_matches_token_major_bitwise():
    """The same bytes laid out [page][head][slot][d] (strides from the tensor
    view) give the bit-identical output of the [page][slot][head][d] layout."""
    w = W.build(seed=43, batch=2, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                lengths=[3000, 700])
    y, t = run(w)
    ya = to_np(y)
    assert_parity(ya, oracle_ref(w), "token-major")
    kh = t["k_pool"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    vh = t["v_pool"].permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    log(f"[layout] head-major strides {tuple(kh.stride())}")
    yh = to_np(pfs.verify(t["q"], kh, vh, t["k_scale"], t["v_scale"], t["block_table"], t["live_len"],
                          head_map=t["head_map"], sm_scale=t["sm_scale"]))
    assert np.array_equal(ya.view(np.uint16), yh.view(np.uint16))


def test_negative_and_zero_scales():
    """k_scale and v_scale are plain FP32 factors: a negative K scale flips the
    scores, a zero K scale makes every visible key equally likely, a negative V
    scale flips the output. The oracle applies them exactly."""
    w = W.build(seed=47, batch=2, q=8, num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=32,
                lengths=[700, 260])
    # the workload's own magnitudes (absmax / 448 per head), with signs flipped and one K scale zeroed
    w.k_scale = (w.k_scale * np.array([-1.0, 0.0, 1.0, -1.0])).astype(np.float32)
    w.v_scale = (w.v_scale * np.array([1.0, -1.0, 1.0, -1.0])).astype(np.float32)
    log(f"[scales] k={w.k_scale.tolist()} v={w.v_scale.tolist()}")
    for tps in (0, 128):
        out = to_np(run(w, tokens_per_split=tps)[0])
        assert_parity(out, oracle_ref(w), f"signed scales tps={tps}")


def test_padded_strides_match_contiguous_bitwise():
    kw = dict(batch=2, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64, lengths=[1500, 400])
    a = W.build(seed=41, **kw)
    variants = [W.build(seed=41, token_pad=16, **kw), W.build(seed=41, page_pad=16 * 7, **kw),
                W.build(seed=41, token_pad=512, page_pad=256, **kw)]
    ya = to_np(run(a)[0])
    assert_parity(ya, oracle_ref(a), "contiguous")
    for v in variants:
        yv = to_np(run(v)[0])
        assert np.array_equal(ya.view(np.uint16), yv.view(np.uint16)), (v.token_stride, v.page_stride)


def test_tail_sentinels_do_not_leak():
    w = W.build(seed=42, batch=2, q=8, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=64,
                lengths=[1000, 70])
    a = to_np(run(W.set_tail_sentinel(w, W.SENTINEL_NAN))[0])
    b = to_np(run(W.set_tail_sentinel(w, W.SENTINEL_MAX))[0])
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert_parity(a, oracle_ref(w), "sentinels")


def test_power_of_two_v_scale_is_exact():
    w = W.build(seed=43, batch=1, q=8, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=64, lengths=[800])
    a = to_np(run(w)[0]).astype(np.float64)
    w2 = w.copy()
    w2.v_scale = (w.v_scale * np.float32(4.0)).astype(np.float32)
    b = to_np(run(w2)[0]).astype(np.float64)
    # exact wherever both results are FP16 normal numbers (subnormal rounding
    # is not scale invariant); elsewhere within one subnormal step
    normal = np.abs(a) >= 2.0 ** -14
    assert normal.mean() > 0.99
    assert np.array_equal(b[normal], a[normal] * 4.0)
    assert np.all(np.abs(b - a * 4.0) <= 4 * 2.0 ** -24)


def test_workspace_poison_and_reuse():
    import torch

    w = W.build(seed=44, batch=2, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                lengths=[3000, 1200])
    out, t = run(w)
    ref = to_np(out)
    plan = pfs.make_plan(batch=w.batch, q=w.q, num_q_heads=w.num_q_heads, head_map=t["head_map"],
                         k_pool=t["k_pool"], max_pages_per_row=w.max_pages_per_row, sm_scale=t["sm_scale"])
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=device())
    for fill in (0xFF, 0x7F, 0x00):  # NaN patterns and zeros
        ws.fill_(fill)
        y = to_np(run(w, tensors=t, workspace=ws)[0])
        assert np.array_equal(y.view(np.uint16), ref.view(np.uint16)), hex(fill)


def test_output_guard_bytes_untouched():
    import torch

    w = W.build(seed=45, batch=2, q=8, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                lengths=[500, 0])
    t = W.device_tensors(w, device())
    n = w.batch * w.q * w.num_q_heads * w.head_dim
    guard = 4096
    buf = torch.full((n + 2 * guard,), 12345.0, dtype=torch.float16, device=device())
    out = buf[guard:guard + n].view(w.batch, w.q, w.num_q_heads, w.head_dim)
    run(w, tensors=t, out=out)
    host = to_np(buf)
    assert np.all(host[:guard] == np.float16(12345.0)) and np.all(host[guard + n:] == np.float16(12345.0))
    assert_parity(host[guard:guard + n].reshape(out.shape), oracle_ref(w), "guarded out")


def test_two_streams_two_workspaces():
    import torch

    w = W.build(seed=46, batch=1, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64, lengths=[4000])
    t = W.device_tensors(w, device())
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        o1 = run(w, tensors=t, stream=s1)[0]
    with torch.cuda.stream(s2):
        o2 = run(w, tensors=t, stream=s2)[0]
    torch.cuda.synchronize()
    assert np.array_equal(to_np(o1).view(np.uint16), to_np(o2).view(np.uint16))


def _golden_page_sizes():
    import json
    import os

    path = os.path.join(os.path.dirname(__file__), "golden", "page_sizes.json")
    with open(path) as f:
        return json.load(f)["page_sizes"]


@pytest.mark.parametrize("page", _golden_page_sizes())
def test_page_sizes_of_the_pages(page):
    """The page sizes the pages run (none a power of two): GQA6 at head_dim
    256, q5, contexts that span several pages and end inside one."""
    w = W.build(seed=page, batch=2, q=5, num_q_heads=6, num_kv_heads=1, head_dim=256, page_size=page,
                lengths=[3 * page + 37, page - 3])
    log(f"[page] {page} lengths={w.live_len.tolist()}")
    for tps in (0, 640):
        assert_parity(to_np(run(w, tokens_per_split=tps)[0]), oracle_ref(w), f"page {page} tps={tps}")


def test_largest_split_uses_the_whole_tile_table():
    """tokens_per_split = 16384, the most a split addresses (1024 tiles of 16
    tokens): two full splits and a ragged third."""
    w = W.build(seed=71, batch=1, q=8, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=64,
                lengths=[2 * 16384 + 1000])
    log("[tps] 16384")
    assert_parity(to_np(run(w, tokens_per_split=16384)[0]), oracle_ref(w), "tps 16384")


def test_most_rows_per_kv_head():
    """q = 16 draft rows x 16 query heads per KV head = 256 rows: four row
    blocks of 64 at head_dim 256, and the most query heads (256) at head_dim 64."""
    w = W.build(seed=72, batch=1, q=16, num_q_heads=16, num_kv_heads=1, head_dim=256, page_size=64,
                lengths=[1500])
    assert_parity(to_np(run(w)[0]), oracle_ref(w), "256 rows d256")
    w2 = W.build(seed=73, batch=1, q=2, num_q_heads=256, num_kv_heads=2, head_dim=64, page_size=16,
                 lengths=[700])
    assert_parity(to_np(run(w2)[0]), oracle_ref(w2), "256 query heads d64")


def test_lengths_at_split_partition_and_tile_edges():
    """One batch whose live lengths sit on and beside every boundary the kernel
    has: 16-token tiles, 32-token steps, 64-token partitions, 256-token splits."""
    lengths = [1, 8, 9, 15, 16, 17, 31, 32, 33, 63, 64, 65, 255, 256, 257, 511, 512, 513]
    w = W.build(seed=74, batch=len(lengths), q=8, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16,
                lengths=lengths)
    r = oracle_ref(w)
    for tps in (0, 256, 64):
        assert_parity(to_np(run(w, tokens_per_split=tps)[0]), r, f"edge lengths tps={tps}")


def test_speculative_steps_in_one_graph():
    """append (quantize-on-write of the draft tokens) + verify captured as one
    HIP graph and replayed for successive steps: the live length grows by q
    and new draft K/V arrive each step; every replay equals the eager calls
    and the oracle on the host-updated pools."""
    import torch

    q = 8
    w = W.build(seed=75, batch=2, q=q, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                lengths=[4096, 4096], capacity=4096)
    w.live_len = np.array([1000, 2900], np.int32)
    dev = device()
    t = W.device_tensors(w, dev)
    rng = np.random.default_rng(76)
    kn = torch.zeros((2, q, 2, 256), dtype=torch.float16, device=dev)
    vn = torch.zeros_like(kn)
    out = torch.empty_like(t["q"])
    plan = pfs.make_plan(batch=w.batch, q=q, num_q_heads=w.num_q_heads, head_map=t["head_map"], k_pool=t["k_pool"],
                         max_pages_per_row=w.max_pages_per_row, sm_scale=t["sm_scale"])
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)

    def step():
        pfs.kv_append(kn, vn, t["k_scale"], t["v_scale"], t["block_table"], t["live_len"], t["k_pool"], t["v_pool"])
        run(w, tensors=t, out=out, workspace=ws)

    step()  # warm up the plan cache before capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    host = w.copy()
    k_dev0, v_dev0 = t["k_pool"].clone(), t["v_pool"].clone()
    for s in range(4):
        knp = rng.normal(0, 1, (2, q, 2, 256)).astype(np.float16)
        vnp = rng.normal(0, 1, (2, q, 2, 256)).astype(np.float16)
        host.live_len = (w.live_len + q * s).astype(np.int32)
        kn.copy_(torch.from_numpy(knp))
        vn.copy_(torch.from_numpy(vnp))
        t["live_len"].copy_(torch.from_numpy(host.live_len))
        k_before, v_before = t["k_pool"].clone(), t["v_pool"].clone()
        out.fill_(1)
        g.replay()
        yg = to_np(out).copy()
        kg, vg = t["k_pool"].clone(), t["v_pool"].clone()
        # the same step eagerly from the same pools
        t["k_pool"].copy_(k_before)
        t["v_pool"].copy_(v_before)
        step()
        assert np.array_equal(to_np(out).view(np.uint16), yg.view(np.uint16)), f"step {s}"
        assert torch.equal(kg, t["k_pool"]) and torch.equal(vg, t["v_pool"]), f"step {s} pools"
        host.k_pool, host.v_pool = oracle.kv_append(host, knp, vnp)
        assert_parity(yg, oracle_ref(host), f"graph step {s} lengths {host.live_len.tolist()}")
    del k_dev0, v_dev0


@pytest.mark.parametrize("case", ["one-request", "batch"])
def test_split_then_combine_is_verify(case):
    """pfs_verify_split followed by pfs_verify_combine on the same stream,
    plan and workspace gives the bytes of pfs_verify (include/pfs.h), and a
    second combine over the same partials gives them again (the combine only
    reads the workspace)."""
    import torch

    from paged_fp8_split_amd import _lib

    if case == "one-request":
        w = W.build(seed=61, batch=1, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                    lengths=[9000], outlier_frac=0.01)
    else:
        w = W.build(seed=62, batch=3, q=4, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=32,
                    lengths=[3000, 0, 1700])
    dev = device()
    t = W.device_tensors(w, dev)
    plan = pfs.make_plan(batch=w.batch, q=w.q, num_q_heads=w.num_q_heads, head_map=t["head_map"],
                         k_pool=t["k_pool"], max_pages_per_row=w.max_pages_per_row, sm_scale=t["sm_scale"])
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    log(f"[two phases] {case}: {plan.num_splits} splits x {plan.tokens_per_split} tokens")
    whole = to_np(run(w, tensors=t, workspace=ws)[0])
    out = torch.full_like(t["q"], float("nan"))
    _lib.verify_split(plan, t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["block_table"], t["live_len"], ws)
    _lib.verify_combine(plan, t["v_scale"], t["live_len"], out, ws)
    first = to_np(out).copy()
    out.fill_(0.5)
    _lib.verify_combine(plan, t["v_scale"], t["live_len"], out, ws)
    again = to_np(out)
    assert_parity(first, oracle_ref(w), f"two phases {case}")
    assert np.array_equal(first.view(np.uint16), whole.view(np.uint16))
    assert np.array_equal(again.view(np.uint16), whole.view(np.uint16))


@pytest.mark.parametrize("case", ["interleaved", "shuffled"])
def test_non_contiguous_head_maps(case):
    """A KV head's query heads need not be adjacent (any map with uniform
    groups, include/pfs.h). With the map m(h) = c(pi(h)) -- c the contiguous
    map h // G, pi a permutation of the query heads -- and the query heads
    permuted the same way, query head h gives the bytes that head pi(h) gives
    under c: each row's arithmetic does not depend on where the map puts it."""
    import dataclasses

    base = W.build(seed=83, batch=2, q=4, num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=32,
                   lengths=[900, 333], outlier_frac=0.01)
    hq, G = base.num_q_heads, base.group
    if case == "interleaved":  # query heads g, g + 4, g + 8, g + 12 share KV head g
        pi = np.array([(h % 4) * G + h // 4 for h in range(hq)])
    else:
        pi = np.random.default_rng(5).permutation(hq)
    c = np.arange(hq) // G
    w = dataclasses.replace(base, head_map=c[pi].astype(np.int32), q_fp16=np.ascontiguousarray(base.q_fp16[:, :, pi]))
    log(f"[head map] {case}: {w.head_map.tolist()}")
    y_base = to_np(run(base)[0])
    y = to_np(run(w)[0])
    assert_parity(y, oracle_ref(w), f"{case} head map")
    assert np.array_equal(y.view(np.uint16), y_base[:, :, pi].view(np.uint16))


def test_widest_group_and_widest_multi_head():
    """The extremes of the head map: all 256 query heads on one KV head at
    q = 16 (4,096 rows per KV head, 16 row blocks), and 256 KV heads with one
    query head each (one row per KV head, padded to a 16-row tile)."""
    w = W.build(seed=84, batch=1, q=16, num_q_heads=256, num_kv_heads=1, head_dim=64, page_size=16,
                lengths=[300])
    log("[heads] 256 query heads on one KV head, q16")
    assert_parity(to_np(run(w)[0]), oracle_ref(w), "group of 256")
    w2 = W.build(seed=85, batch=2, q=1, num_q_heads=256, num_kv_heads=256, head_dim=128, page_size=32,
                 lengths=[520, 77])
    log("[heads] 256 KV heads, q1")
    assert_parity(to_np(run(w2)[0]), oracle_ref(w2), "256 KV heads")


@pytest.mark.parametrize("sm_scale", [1.0e-3, 1.0, 3.0])
def test_softmax_scales(sm_scale):
    """Softmax scales far from 1/sqrt(head_dim): a tiny one (near-uniform
    attention over every visible key) and large ones (scores spread over
    hundreds of log2 units, so the lazily raised reference maximum moves
    often and most probabilities underflow), each against the oracle."""
    import dataclasses

    w = W.build(seed=86, batch=2, q=8, num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=32,
                lengths=[2500, 700], outlier_frac=0.01)
    w = dataclasses.replace(w, sm_scale=sm_scale)
    log(f"[sm_scale] {sm_scale}")
    for tps in (0, 256):
        assert_parity(to_np(run(w, tokens_per_split=tps)[0]), oracle_ref(w), f"sm_scale {sm_scale} tps={tps}")


def test_million_token_context():
    """One request of 2^20 live tokens (four times the metric's context), with
    1 % outlier tokens: the default plan (256 splits) and the largest split
    (64 splits of 16,384 tokens), each against the oracle."""
    w = W.build(seed=87, batch=1, q=2, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=64,
                lengths=[1 << 20], outlier_frac=0.01)
    ref = oracle_ref(w)
    for tps in (0, 16384):
        log(f"[1M context] tps={tps}")
        assert_parity(to_np(run(w, tokens_per_split=tps)[0]), ref, f"1M context tps={tps}")
