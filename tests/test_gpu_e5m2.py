"""GPU parity of the E5M2 KV format (the explicit alternative to E4M3): the
verify attention against the FP64 oracle on small, ragged and full-size
shapes, tail bytes holding E5M2 infinities and NaNs, and the codec kernels
(quantize-on-write, bridge) bit for bit. Everything goes through the C ABI."""
import zlib

import numpy as np
import pytest

import oracle
import paged_fp8_split_amd as pfs
from paged_fp8_split_amd import workloads as W

from parity import device, assert_parity, log, oracle_ref, run, to_np

pytestmark = pytest.mark.gpu

E5M2_INF = 0x7C

CASES = [
    # (name, build kwargs, tokens_per_split)
    ("d64-q8-g4-split64", dict(batch=1, q=8, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16,
                               lengths=[1032], scale_mode="per_tensor"), 64),
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
    ("d128-q5-g6-padded", dict(batch=2, q=5, num_q_heads=12, num_kv_heads=2, head_dim=128, page_size=48,
                               lengths=[400, 90], token_pad=16, page_pad=64), 0),
    ("d64-outliers-pow2", dict(batch=2, q=8, num_q_heads=8, num_kv_heads=4, head_dim=64, page_size=16,
                               lengths=[900, 333], outlier_frac=0.02, scale_mode="pow2",
                               pow2_scale_exps=[-14, -6, 1, 4]), 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_e5m2_parity(case):
    name, kw, tps = case
    w = W.build(seed=zlib.crc32(name.encode()) % 1000 + 5, kv_format="e5m2", **kw)
    log(f"[e5m2] {name} tps={tps}")
    out, _ = run(w, tokens_per_split=tps)
    assert_parity(to_np(out), oracle_ref(w), "e5m2 " + name)


def test_e5m2_256k_context():
    """The 256K-context q8 workload (16 query / 2 KV heads, head_dim 256, page
    64, 1 % outlier tokens) stored as E5M2, every output element."""
    w = W.config(3, kv_format="e5m2")
    log("[e5m2] 256K context")
    y = to_np(run(w)[0])
    assert_parity(y, oracle_ref(w), "e5m2 256K")


def test_e5m2_infinity_and_nan_tails_do_not_leak():
    w = W.build(seed=52, batch=2, q=8, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=64,
                lengths=[1000, 70], kv_format="e5m2")
    a = to_np(run(W.set_tail_sentinel(w, W.SENTINEL_NAN))[0])
    b = to_np(run(W.set_tail_sentinel(w, E5M2_INF))[0])
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert_parity(a, oracle_ref(w), "e5m2 sentinels")


def test_e5m2_signed_scales():
    w = W.build(seed=57, batch=2, q=8, num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=32,
                lengths=[700, 260], kv_format="e5m2")
    w.k_scale = (w.k_scale * np.array([-1.0, 0.0, 1.0, -1.0])).astype(np.float32)
    w.v_scale = (w.v_scale * np.array([1.0, -1.0, 1.0, -1.0])).astype(np.float32)
    assert_parity(to_np(run(w, tokens_per_split=128)[0]), oracle_ref(w), "e5m2 signed scales")


def test_e5m2_and_e4m3_of_the_same_bytes_differ():
    """The format reaches the kernel: the same bytes read as E4M3 and as E5M2
    give the two oracle results (bytes kept finite in both formats)."""
    w = W.build(seed=58, batch=1, q=8, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=16,
                lengths=[500])
    w.k_pool &= 0xBF
    w.v_pool &= 0xBF
    w5 = w.copy()
    w5.kv_format = "e5m2"
    assert_parity(to_np(run(w)[0]), oracle_ref(w), "bytes as e4m3")
    assert_parity(to_np(run(w5)[0]), oracle_ref(w5), "bytes as e5m2")


@pytest.mark.parametrize("scale", [None, 1.0, 0.0011, 3.0e-7, 1.0 + 2.0 ** -12])
def test_e5m2_bridge_every_code_bitwise(scale):
    w = W.build(seed=73, batch=2, q=2, num_q_heads=2, num_kv_heads=2, head_dim=128, page_size=16,
                lengths=[40, 5], kv_format="e5m2")
    view = w.pool_view(w.k_pool)
    view[w.block_table[0, 0]] = np.resize(np.arange(256, dtype=np.uint8), view[0].shape)  # every code
    sc = None if scale is None else np.array([scale, 2 * scale], dtype=np.float32)
    import torch

    t = W.device_tensors(w, device())
    s_t = None if sc is None else torch.from_numpy(sc).to(t["k_pool"].device)
    got = to_np(pfs.dequant_paged(t["k_pool"], t["block_table"], t["live_len"], scale=s_t, kv_format="e5m2"))
    want = oracle.dequant(w, scale=sc)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint16), want[~nan].view(np.uint16))


@pytest.mark.parametrize("scale", [1.0, 0.37, 2.0 ** -10, 1000.0])
def test_e5m2_append_on_every_fp16_pattern(scale):
    import torch

    w = W.build(seed=19, batch=16, q=16, num_q_heads=1, num_kv_heads=1, head_dim=256, page_size=16,
                lengths=[16] * 16, kv_format="e5m2")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(16, 16, 1, 256)
    kn = bits.view(np.float16)
    vn = np.ascontiguousarray(kn[::-1])
    w.k_scale = np.array([scale], dtype=np.float32)
    w.v_scale = np.array([scale * 3.0], dtype=np.float32)
    dev = device()
    t = W.device_tensors(w, dev)
    pfs.kv_append(torch.from_numpy(np.ascontiguousarray(kn)).to(dev), torch.from_numpy(vn).to(dev), t["k_scale"],
                  t["v_scale"], t["block_table"], t["live_len"], t["k_pool"], t["v_pool"], kv_format="e5m2")
    ek, ev = oracle.kv_append(w, kn, vn)
    assert np.array_equal(t["k_pool"].cpu().numpy().ravel(), np.asarray(ek).ravel())
    assert np.array_equal(t["v_pool"].cpu().numpy().ravel(), np.asarray(ev).ravel())


def test_e5m2_append_then_verify():
    import torch

    w = W.build(seed=79, batch=2, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                lengths=[3000, 130], kv_format="e5m2")
    rng = np.random.default_rng(80)
    kn = rng.normal(0, 1, (2, 8, 2, 256)).astype(np.float16)
    vn = rng.normal(0, 1, (2, 8, 2, 256)).astype(np.float16)
    dev = device()
    t = W.device_tensors(w, dev)
    pfs.kv_append(torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev), t["k_scale"], t["v_scale"],
                  t["block_table"], t["live_len"], t["k_pool"], t["v_pool"], kv_format="e5m2")
    w2 = w.copy()
    w2.k_pool, w2.v_pool = oracle.kv_append(w, kn, vn)
    out, _ = run(w2, tensors=t)
    assert_parity(to_np(out), oracle_ref(w2), "e5m2 append then verify")


def test_float8_pool_dtypes_select_the_format():
    """torch float8 views of the same bytes pick the format by dtype; a
    contradicting explicit format is refused."""
    import torch

    w = W.build(seed=81, batch=1, q=4, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16,
                lengths=[300], kv_format="e5m2")
    y, t = run(w)
    k8, v8 = t["k_pool"].view(torch.float8_e5m2), t["v_pool"].view(torch.float8_e5m2)
    y8 = pfs.verify(t["q"], k8, v8, t["k_scale"], t["v_scale"], t["block_table"], t["live_len"],
                    head_map=t["head_map"], sm_scale=t["sm_scale"])
    assert np.array_equal(to_np(y).view(np.uint16), to_np(y8).view(np.uint16))
    with pytest.raises(ValueError):
        pfs.verify(t["q"], k8, v8, t["k_scale"], t["v_scale"], t["block_table"], t["live_len"],
                   head_map=t["head_map"], sm_scale=t["sm_scale"], kv_format="e4m3")
