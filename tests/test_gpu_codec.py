"""GPU tests of the codec kernels at the ends of the paged E4M3 cache: the
quantize-on-write of the draft tokens (pfs_kv_append) and the scaled paged
E4M3 -> FP16 bridge (pfs_dequant_paged). Both produce bytes / FP16 bit
patterns, so they are compared with the oracle bit for bit."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import paged_fp8_split_amd as pfs
from paged_fp8_split_amd import workloads as W

from parity import device, assert_parity, log, oracle_ref, run, to_np

pytestmark = pytest.mark.gpu


def _special_fp16(n: int, rng) -> np.ndarray:
    """n FP16 values: normals of several magnitudes, zeros, infinities, NaN,
    FP16 subnormals and values that overflow 448 after scaling."""
    vals = np.concatenate([
        rng.normal(0, 1, n), rng.normal(0, 300, n), rng.normal(0, 1e-3, n),
        [0.0, -0.0, np.inf, -np.inf, np.nan, 6.0e-8, -6.0e-8, 65504.0, -65504.0],
    ]).astype(np.float16)
    return rng.permutation(vals)[:n]


@pytest.mark.parametrize("D,q,lengths", [(64, 8, [37, 5, 0, 200]), (128, 4, [64, 3, 1000]), (256, 16, [16, 513])])
def test_kv_append_matches_oracle_bitwise(D, q, lengths):
    rng = np.random.default_rng(D + q)
    w = W.build(seed=D + q, batch=len(lengths), q=q, num_q_heads=2, num_kv_heads=2, head_dim=D, page_size=16,
                lengths=lengths)
    shape = (w.batch, q, 2, D)
    kn = _special_fp16(int(np.prod(shape)), rng).reshape(shape)
    vn = _special_fp16(int(np.prod(shape)), rng).reshape(shape)
    w.k_scale = np.array([0.0123, 2.0 ** -6], dtype=np.float32)
    w.v_scale = np.array([1.7, 0.00031], dtype=np.float32)
    log(f"[append] D={D} q={q} lengths={lengths}")
    import torch

    dev = device()
    t = W.device_tensors(w, dev)
    pfs.kv_append(torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev), t["k_scale"], t["v_scale"],
                  t["block_table"], t["live_len"], t["k_pool"], t["v_pool"])
    ek, ev = oracle.kv_append(w, kn, vn)
    gk, gv = t["k_pool"].cpu().numpy().ravel(), t["v_pool"].cpu().numpy().ravel()
    assert np.array_equal(gk, np.asarray(ek).ravel())
    assert np.array_equal(gv, np.asarray(ev).ravel())


@pytest.mark.parametrize("scale", [1.0, 0.0021, 37.5, 2.0 ** -9])
def test_kv_append_on_every_fp16_pattern(scale):
    """All 65536 FP16 bit patterns through the encoder: 16 requests x 16 draft
    rows x 1 KV head x 256 values."""
    w = W.build(seed=9, batch=16, q=16, num_q_heads=1, num_kv_heads=1, head_dim=256, page_size=16,
                lengths=[16] * 16)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(16, 16, 1, 256)
    kn = bits.view(np.float16)
    vn = np.ascontiguousarray(kn[::-1])
    w.k_scale = np.array([scale], dtype=np.float32)
    w.v_scale = np.array([scale * 3.0], dtype=np.float32)
    import torch

    dev = device()
    t = W.device_tensors(w, dev)
    pfs.kv_append(torch.from_numpy(np.ascontiguousarray(kn)).to(dev), torch.from_numpy(vn).to(dev), t["k_scale"],
                  t["v_scale"], t["block_table"], t["live_len"], t["k_pool"], t["v_pool"])
    ek, ev = oracle.kv_append(w, kn, vn)
    assert np.array_equal(t["k_pool"].cpu().numpy().ravel(), np.asarray(ek).ravel())
    assert np.array_equal(t["v_pool"].cpu().numpy().ravel(), np.asarray(ev).ravel())


def test_append_then_verify_matches_oracle():
    """The draft tokens written by the GPU are the ones verify then attends to."""
    w = W.build(seed=77, batch=2, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                lengths=[3000, 130])
    rng = np.random.default_rng(78)
    kn = rng.normal(0, 1, (2, 8, 2, 256)).astype(np.float16)
    vn = rng.normal(0, 1, (2, 8, 2, 256)).astype(np.float16)
    import torch

    dev = device()
    t = W.device_tensors(w, dev)
    pfs.kv_append(torch.from_numpy(kn).to(dev), torch.from_numpy(vn).to(dev), t["k_scale"], t["v_scale"],
                  t["block_table"], t["live_len"], t["k_pool"], t["v_pool"])
    w2 = w.copy()
    w2.k_pool, w2.v_pool = oracle.kv_append(w, kn, vn)
    out, _ = run(w2, tensors=t)
    assert_parity(to_np(out), oracle_ref(w2), "append then verify")


@pytest.mark.parametrize("scale", [None, 1.0, 0.0011, 3.0e-7, 1.0 + 2.0 ** -12, 2.0 ** -9 * 3, 517.0])
def test_bridge_matches_oracle_bitwise(scale):
    w = W.build(seed=71, batch=2, q=2, num_q_heads=2, num_kv_heads=2, head_dim=128, page_size=16,
                lengths=[40, 5])
    view = w.pool_view(w.k_pool)
    view[w.block_table[0, 0]] = np.resize(np.arange(256, dtype=np.uint8), view[0].shape)  # every code
    sc = None if scale is None else np.array([scale, 2 * scale], dtype=np.float32)
    import torch

    dev = device()
    t = W.device_tensors(w, dev)
    s_t = None if sc is None else torch.from_numpy(sc).to(dev)
    got = to_np(pfs.dequant_paged(t["k_pool"], t["block_table"], t["live_len"], scale=s_t))
    want = oracle.dequant(w, scale=sc)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint16), want[~nan].view(np.uint16))
