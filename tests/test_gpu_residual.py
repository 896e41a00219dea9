"""GPU parity of the high/residual probability mode (pv_residual): every
probability enters the PV product as an FP16 high part plus an FP16 residual
scaled by 2048, against E4M3 V and V / 2048. Same bar as the default mode
against the FP64 oracle, bit-identical across launches, and its FP16 outputs
disagree with the correctly rounded oracle result less often."""
import zlib

import numpy as np
import pytest

import paged_fp8_split_amd as pfs
from paged_fp8_split_amd import workloads as W

from parity import device, judge, log, oracle_ref, to_np

pytestmark = pytest.mark.gpu


def run_mode(w, residual, tokens_per_split=0, tensors=None):
    t = tensors if tensors is not None else W.device_tensors(w, device())
    o = pfs.verify(t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"], t["live_len"],
                   head_map=t["head_map"], sm_scale=t["sm_scale"], tokens_per_split=tokens_per_split,
                   pv_residual=residual)
    return to_np(o), t


def disagreements(y16, r):
    return int((y16.view(np.uint16) != r.astype(np.float16).view(np.uint16)).sum())


CASES = [
    ("d64-q8-g4", dict(batch=1, q=8, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, lengths=[1032],
                       scale_mode="per_tensor"), 64),
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
    ("d64-outliers-pow2", dict(batch=2, q=8, num_q_heads=8, num_kv_heads=4, head_dim=64, page_size=16,
                               lengths=[900, 333], outlier_frac=0.02, scale_mode="pow2",
                               pow2_scale_exps=[-6, -3, 1, 4]), 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_residual_parity(case):
    name, kw, tps = case
    w = W.build(seed=zlib.crc32(name.encode()) % 1000 + 11, **kw)
    log(f"[residual] {name} tps={tps}")
    y, _ = run_mode(w, True, tps)
    judge(y, oracle_ref(w), "residual " + name)


def test_residual_is_deterministic_and_differs_from_the_default():
    w = W.build(seed=91, batch=2, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                lengths=[5000, 900])
    a, t = run_mode(w, True)
    b, _ = run_mode(w, True, tensors=t)
    c, _ = run_mode(w, False, tensors=t)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert not np.array_equal(a.view(np.uint16), c.view(np.uint16))  # the mode reaches the kernel


def test_residual_rejects_e5m2():
    w = W.build(seed=92, batch=1, q=2, num_q_heads=2, num_kv_heads=1, head_dim=64, page_size=16, lengths=[40],
                kv_format="e5m2")
    t = W.device_tensors(w, device())
    with pytest.raises(pfs.PfsError):
        pfs.verify(t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"], t["live_len"],
                   kv_format="e5m2", pv_residual=True)


@pytest.mark.parametrize("cfg,q", [(2, None), (3, None), (5, 8)])
def test_residual_full_size_and_disagreements(cfg, q):
    """Full-size workloads, every element: the residual mode meets the bar and
    its FP16 outputs disagree with RNE(oracle) no more often than the default."""
    w = W.config(cfg) if q is None else W.config(cfg, q=q)
    log(f"[residual] config {cfg} ({w.name})")
    r = oracle_ref(w)
    y1, t = run_mode(w, False)
    y2, _ = run_mode(w, True, tensors=t)
    judge(y2, r, f"residual {w.name}")
    d1, d2 = disagreements(y1, r), disagreements(y2, r)
    log(f"[residual] {w.name}: FP16 disagreements with RNE(oracle): default {d1}, residual {d2} of {r.size}")
    assert d2 <= d1
