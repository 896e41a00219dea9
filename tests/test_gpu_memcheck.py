"""GPU memory-safety checks in place of a device sanitizer (none is available
on this stack): every buffer the verify path touches sits inside a larger
allocation with canary bytes on both sides, at the context lengths the pages
memory-checked (1,025, 3,297 and 262,144 tokens). After the launch the
canaries must be intact, the read-only inputs bit-identical and the output
still within the parity bar. Also the 256K-context workload under graph
replay with changed live lengths."""
import numpy as np
import pytest

import paged_fp8_split_amd as pfs
from paged_fp8_split_amd import workloads as W

from parity import device, assert_parity, log, oracle_ref, run, to_np

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes of canary on each side of every buffer
CANARY = 0xA5


def _guarded(host: np.ndarray, dev):
    """Copy a host array into the middle of a canary-filled byte buffer on the
    device; returns (whole byte buffer, typed view of the payload)."""
    import torch

    raw = np.ascontiguousarray(host)
    nbytes = raw.nbytes
    buf = torch.full((nbytes + 2 * GUARD,), CANARY, dtype=torch.uint8, device=dev)
    buf[GUARD:GUARD + nbytes].copy_(torch.from_numpy(raw.view(np.uint8).reshape(-1)))
    dtype = {np.dtype(np.float16): torch.float16, np.dtype(np.float32): torch.float32,
             np.dtype(np.int32): torch.int32, np.dtype(np.uint8): torch.uint8}[raw.dtype]
    view = buf[GUARD:GUARD + nbytes].view(dtype).view(raw.shape)
    return buf, view


def _canaries_intact(buf) -> bool:
    h = buf.cpu().numpy()
    return bool(np.all(h[:GUARD] == CANARY) and np.all(h[-GUARD:] == CANARY))


@pytest.mark.parametrize("context", [1025, 3297, 262144])
def test_canaries_around_every_buffer(context):
    import torch

    w = W.build(seed=context, batch=1, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                lengths=[context], outlier_frac=0.01)
    dev = device()
    log(f"[memcheck] context {context}")
    bufs = {}
    bufs["q"], q = _guarded(w.q_fp16, dev)
    bufs["k"], kflat = _guarded(w.k_pool, dev)
    bufs["v"], vflat = _guarded(w.v_pool, dev)
    bufs["ks"], ks = _guarded(w.k_scale, dev)
    bufs["vs"], vs = _guarded(w.v_scale, dev)
    bufs["bt"], bt = _guarded(w.block_table, dev)
    bufs["ll"], ll = _guarded(w.live_len, dev)
    shape = (w.num_pool_pages, w.page_size, w.num_kv_heads, w.head_dim)
    strides = (w.page_stride, w.token_stride, w.head_stride, 1)
    kp, vp = kflat.as_strided(shape, strides), vflat.as_strided(shape, strides)
    plan = pfs.make_plan(batch=w.batch, q=w.q, num_q_heads=w.num_q_heads, head_map=list(w.head_map), k_pool=kp,
                         max_pages_per_row=w.max_pages_per_row, sm_scale=w.sm_scale)
    bufs["ws"], ws = _guarded(np.zeros(plan.workspace_bytes, np.uint8), dev)
    bufs["out"], out = _guarded(np.zeros(w.q_fp16.shape, np.float16), dev)
    before = {k: b.cpu().numpy().copy() for k, b in bufs.items() if k not in ("ws", "out")}
    pfs.verify(q, kp, vp, ks, vs, bt, ll, head_map=list(w.head_map), sm_scale=w.sm_scale, out=out, workspace=ws)
    torch.cuda.synchronize()
    for k, b in bufs.items():
        assert _canaries_intact(b), f"canary of {k} overwritten"
    for k, h in before.items():
        assert np.array_equal(bufs[k].cpu().numpy(), h), f"read-only buffer {k} changed"
    assert_parity(to_np(out), oracle_ref(w), f"guarded context {context}")


def test_256k_context_under_graph_replay_with_changed_lengths():
    import torch

    w = W.config(3)
    dev = device()
    t = W.device_tensors(w, dev)
    out = torch.empty_like(t["q"])
    plan = pfs.make_plan(batch=w.batch, q=w.q, num_q_heads=w.num_q_heads, head_map=t["head_map"],
                         k_pool=t["k_pool"], max_pages_per_row=w.max_pages_per_row, sm_scale=t["sm_scale"])
    ws = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=dev)
    run(w, tensors=t, out=out, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(w, tensors=t, out=out, workspace=ws)
    for L in (262144, 200003, 131072, 20000, 8, 0, 262144):
        wk = w.copy()
        wk.live_len = np.array([L], np.int32)
        t["live_len"].copy_(torch.from_numpy(wk.live_len))
        out.fill_(1)
        g.replay()
        yg = to_np(out).copy()
        ye = to_np(run(wk, tensors=t)[0])
        assert np.array_equal(yg.view(np.uint16), ye.view(np.uint16)), f"L={L}"
        if L == 0:
            assert np.all(yg.view(np.uint16) == 0)
        else:
            assert_parity(yg, oracle_ref(wk), f"256K graph replay L={L}")


# The outlier workload cut to a few thousand live tokens: attention
# concentrates on a few 8x-outlier keys whose V values (up to ~30) nearly
# cancel, so the relative FP16 rounding of each probability (2^-11) is
# amplified to about two FP16 ulps of an output near 3. The opt-in fp16 mode
# (one FP16 probability operand) then measures max abs 0.0041 against the
# 4e-3 bar (rel L2 2.1e-4); the default high/residual mode carries the
# probabilities to ~2^-22 and stays at the FP16 rounding of the output.
SHORT_OUTLIER_LENGTHS = (4097, 8192)


def _short_outlier_case(L, pv_mode):
    import torch

    w = W.config(3)
    w.live_len = np.array([L], np.int32)
    t = W.device_tensors(w, device())
    y = pfs.verify(t["q"], t["k_pool"], t["v_pool"], t["k_scale"], t["v_scale"], t["block_table"], t["live_len"],
                   head_map=t["head_map"], sm_scale=t["sm_scale"], pv_mode=pv_mode)
    torch.cuda.synchronize()
    return to_np(y), oracle_ref(w)


@pytest.mark.parametrize("L", SHORT_OUTLIER_LENGTHS)
def test_default_mode_on_short_outlier_contexts(L):
    y, r = _short_outlier_case(L, "high_residual")
    assert_parity(y, r, f"default (high/residual), outlier workload at L={L}")


@pytest.mark.xfail(strict=True, reason="known limit of the opt-in fp16 mode: one FP16 probability operand "
                   "reaches max abs ~0.0041 (2 ulp at |r|~3) on cancelling outlier values")
@pytest.mark.parametrize("L", SHORT_OUTLIER_LENGTHS)
def test_fp16_mode_on_short_outlier_contexts(L):
    y, r = _short_outlier_case(L, "fp16")
    rep = assert_parity(y, r, f"fp16 mode, outlier workload at L={L}")
    log(f"[known] {rep}")
