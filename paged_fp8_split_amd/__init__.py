"""paged_fp8_split_amd: E4M3 paged speculative-verify attention with FP32 split
partials on AMD Instinct MI355X (gfx950).

The hot path is the C-ABI library ``libpfs.so`` (include/pfs.h), built by
``python -m paged_fp8_split_amd.build``. This package is its thin Python
binding: it derives shapes and byte strides from torch tensors, caches plans
and passes raw device pointers and the current HIP stream. Torch provides
device memory and streams only; all arithmetic runs in the HIP kernels.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence, Tuple

__all__ = ["verify", "dequant_paged", "kv_append", "make_plan", "Plan", "PfsError", "ABI_VERSION", "KV_FORMATS",
           "PV_MODES"]

_plans: Dict[Tuple, "Plan"] = {}


def __getattr__(name):
    if name in ("Plan", "PfsError", "ABI_VERSION"):
        from . import _lib

        return getattr(_lib, name)
    raise AttributeError(name)


KV_FORMATS = {"e4m3": 0, "e5m2": 1}
# how each probability enters the PV product (include/pfs.h, PFS_PV_*)
PV_MODES = {"high_residual": 0, "fp16": 1}


def _pv_mode(pv_mode: str) -> int:
    if pv_mode not in PV_MODES:
        raise ValueError(f"pv_mode must be one of {sorted(PV_MODES)}, got {pv_mode!r}")
    return PV_MODES[pv_mode]


def _num_cus(t) -> int:
    """Compute units of the device holding tensor t (0, the library default,
    for a host tensor)."""
    import torch

    if not t.is_cuda:
        return 0
    return int(torch.cuda.get_device_properties(t.device).multi_processor_count)


def _kv_format(pool, kv_format: Optional[str]) -> int:
    """PFS_KV_* code of a pool: the explicit ``kv_format`` ("e4m3" or "e5m2"),
    else the pool's float8 dtype, else E4M3 (uint8 pools)."""
    import torch

    implied = {torch.float8_e4m3fn: "e4m3", torch.float8_e5m2: "e5m2"}.get(pool.dtype)
    if kv_format is None:
        kv_format = implied or "e4m3"
    if kv_format not in KV_FORMATS:
        raise ValueError(f"kv_format must be one of {sorted(KV_FORMATS)}, got {kv_format!r}")
    if implied is not None and implied != kv_format:
        raise ValueError(f"kv_format {kv_format!r} contradicts the pool dtype {pool.dtype}")
    return KV_FORMATS[kv_format]


def _pool_layout(pool):
    if pool.dtype.itemsize != 1 or pool.dim() != 4:
        raise ValueError("KV pools must be uint8 tensors shaped [pages, page_size, kv_heads, head_dim]")
    if pool.stride(3) != 1:
        raise ValueError("the head_dim bytes of a KV pool must be contiguous")
    pages, page, hkv, d = pool.shape
    return int(pages), int(page), int(hkv), int(d), tuple(int(s) for s in pool.stride()[:3])


# The kernels address every buffer from the plan's sizes alone, so the
# binding checks each tensor against them before a pointer crosses the ABI:
# a short block table, length vector, scale vector or output would otherwise
# be read or written past its end on the device.

def _require(ok: bool, msg: str) -> None:
    if not ok:
        raise ValueError(msg)


def _check_pools(k_pool, v_pool) -> None:
    _require(k_pool.stride() == v_pool.stride() and k_pool.shape == v_pool.shape,
             "K and V pools must share shape and strides")
    _require(v_pool.dtype == k_pool.dtype, "K and V pools must share a dtype")


def _check_request_tensors(batch: int, hkv: int, block_table, live_len, scales) -> None:
    """block_table [batch, pages per row] int32, live_len [batch] int32 and
    each named scale [hkv] float32, all contiguous."""
    import torch

    _require(block_table.dtype == torch.int32 and block_table.is_contiguous() and block_table.dim() == 2
             and int(block_table.shape[0]) == batch,
             f"block_table must be a contiguous int32 tensor [{batch}, max_pages_per_row]")
    _require(live_len.dtype == torch.int32 and live_len.is_contiguous() and live_len.numel() == batch,
             f"live_len must be a contiguous int32 tensor of {batch} lengths")
    for name, t in scales:
        _require(t.dtype == torch.float32 and t.is_contiguous() and t.numel() == hkv,
                 f"{name} must be a contiguous float32 tensor [{hkv}]")


def _check_out(out, shape) -> None:
    import torch

    _require(out.dtype == torch.float16 and out.is_contiguous() and tuple(out.shape) == tuple(shape),
             f"out must be a contiguous float16 tensor {list(shape)}")


def _check_device(tensors) -> None:
    """Every tensor on one GPU (checked last, so that a host-only caller
    sees the other errors first and no host pointer reaches the library)."""
    dev = tensors[0][1].device
    for name, t in tensors:
        _require(t.is_cuda and t.device == dev, f"{name} must be on the GPU that holds {tensors[0][0]} ({dev})")


def _check_plan(plan, *, batch, q, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_row,
                num_pool_pages, strides) -> None:
    p = plan.problem
    got = (p.batch, p.q, p.num_q_heads, p.num_kv_heads, p.head_dim, p.page_size, p.max_pages_per_row,
           p.num_pool_pages, (p.kv_page_stride, p.kv_token_stride, p.kv_head_stride))
    want = (batch, q, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_row, num_pool_pages,
            tuple(strides))
    _require(got == want, f"the plan was made for another shape: {got} against the tensors' {want}")


def make_plan(*, batch, q, num_q_heads, head_map, k_pool, max_pages_per_row, sm_scale=None,
              partition_tokens=64, tokens_per_split=0, kv_format: Optional[str] = None,
              pv_mode: str = "high_residual", num_cus: Optional[int] = None):
    """Plan (cached) for a problem whose KV pools look like ``k_pool``; the
    default split length fills the compute units of ``k_pool``'s device
    unless ``num_cus`` is given."""
    from . import _lib

    pages, page, hkv, d, (sp, st, sh) = _pool_layout(k_pool)
    fmt = _kv_format(k_pool, kv_format)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    hm = tuple(int(x) for x in head_map)
    pm = _pv_mode(pv_mode)
    cus = _num_cus(k_pool) if num_cus is None else int(num_cus)
    key = (batch, q, num_q_heads, hkv, d, page, max_pages_per_row, pages, sp, st, sh, float(sm_scale), hm,
           partition_tokens, tokens_per_split, fmt, pm, cus)
    plan = _plans.get(key)
    if plan is None:
        plan = _lib.Plan(batch=batch, q=q, num_q_heads=num_q_heads, num_kv_heads=hkv, head_dim=d, page_size=page,
                         max_pages_per_row=max_pages_per_row, num_pool_pages=pages, kv_page_stride=sp,
                         kv_token_stride=st, kv_head_stride=sh, sm_scale=sm_scale, head_map=hm,
                         partition_tokens=partition_tokens, tokens_per_split=tokens_per_split, kv_format=fmt,
                         pv_mode=pm, num_cus=cus)
        _plans[key] = plan
    return plan


def verify(q, k_pool, v_pool, k_scale, v_scale, block_table, live_len, *, head_map: Optional[Sequence[int]] = None,
           sm_scale: Optional[float] = None, partition_tokens: int = 64, tokens_per_split: int = 0, out=None,
           workspace=None, stream=None, plan=None, kv_format: Optional[str] = None,
           pv_mode: str = "high_residual", noalloc: bool = False):
    """Verify attention of q draft rows per request over a paged FP8 KV cache.

    q            [B, q, Hq, D] float16, contiguous, on the GPU
    k_pool/v_pool [pages, page_size, Hkv, D] byte tensors (uint8 or a float8
                 dtype), head_dim contiguous, identical strides (multiples of
                 16 bytes)
    kv_format    "e4m3" (default) or "e5m2"; a float8_e4m3fn / float8_e5m2
                 pool dtype implies it
    pv_mode      "high_residual" (default): each probability enters PV as an
                 FP16 high part plus an FP16 residual (about 22 bits);
                 "fp16": as one FP16 operand (about half the PV matrix work,
                 2^-11 relative rounding per probability)
    k_scale/v_scale [Hkv] float32
    block_table  [B, max_pages_per_row] int32
    live_len     [B] int32, draft tokens included
    head_map     query head -> KV head (default h // (Hq // Hkv))
    plan         a plan from ``make_plan`` for exactly these shapes and pool
                 layout (checked); its head map, scale, split length and
                 probability mode then apply
    noalloc      keep the split partials in the library's per-GPU device
                 array (pfs_verify_noalloc) instead of a workspace; with
                 ``out`` given, nothing is allocated. Calls that overlap on
                 one GPU share that array and must not run concurrently.
    Returns out [B, q, Hq, D] float16. No host synchronization.
    """
    from . import _lib
    import torch

    _require(q.dtype == torch.float16 and q.is_contiguous() and q.dim() == 4,
             "q must be a contiguous float16 tensor [B, q, Hq, D]")
    B, nq, Hq, D = (int(x) for x in q.shape)
    _check_pools(k_pool, v_pool)
    pages, page, hkv, d, strides = _pool_layout(k_pool)
    _require(d == D, f"q has head_dim {D}, the pools {d}")
    _check_request_tensors(B, hkv, block_table, live_len, (("k_scale", k_scale), ("v_scale", v_scale)))
    if out is not None:
        _check_out(out, q.shape)
    if workspace is not None:
        _require(workspace.is_contiguous(), "workspace must be contiguous")
    if head_map is None:
        head_map = [h // (Hq // hkv) for h in range(Hq)] if Hq % hkv == 0 else list(range(Hq))
    if plan is None:
        plan = make_plan(batch=B, q=nq, num_q_heads=Hq, head_map=head_map, k_pool=k_pool,
                         max_pages_per_row=int(block_table.shape[1]), sm_scale=sm_scale,
                         partition_tokens=partition_tokens, tokens_per_split=tokens_per_split,
                         kv_format=kv_format, pv_mode=pv_mode)
    else:
        _check_plan(plan, batch=B, q=nq, num_q_heads=Hq, num_kv_heads=hkv, head_dim=D, page_size=page,
                    max_pages_per_row=int(block_table.shape[1]), num_pool_pages=pages, strides=strides)
        _require(plan.kv_format == _kv_format(k_pool, kv_format), "the plan's KV format differs from the pools'")
    named = [("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("k_scale", k_scale), ("v_scale", v_scale),
             ("block_table", block_table), ("live_len", live_len)]
    named += [(n, t) for n, t in (("out", out), ("workspace", workspace)) if t is not None]
    _check_device(named)
    if out is None:
        out = torch.empty_like(q)
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc takes no workspace: the partials live in the library's device array")
        _lib.verify_noalloc(plan, q, k_pool, v_pool, k_scale, v_scale, block_table, live_len, out, stream)
        return out
    if workspace is None:
        workspace = torch.empty(plan.workspace_bytes, dtype=torch.uint8, device=q.device)
    _lib.verify(plan, q, k_pool, v_pool, k_scale, v_scale, block_table, live_len, out, workspace, stream)
    return out


def dequant_paged(pool, block_table, live_len, *, scale=None, out=None, stream=None,
                  kv_format: Optional[str] = None):
    """Paged FP8 pool -> dense float16 [B, capacity, Hkv, D]: each byte's
    value (E4M3 or E5M2, as for ``verify``) times ``scale`` (float32 [Hkv],
    optional) rounded once to FP16; tokens at or beyond a request's live
    length are +0.0."""
    from . import _lib
    import torch

    pages, page, hkv, d, _ = _pool_layout(pool)
    _require(block_table.dim() == 2, "block_table must be a 2-D int32 tensor [B, max_pages_per_row]")
    B = int(block_table.shape[0])
    _check_request_tensors(B, hkv, block_table, live_len, () if scale is None else (("scale", scale),))
    shape = (B, int(block_table.shape[1]) * page, hkv, d)
    if out is not None:
        _check_out(out, shape)
    named = [("pool", pool), ("block_table", block_table), ("live_len", live_len)]
    named += [(n, t) for n, t in (("scale", scale), ("out", out)) if t is not None]
    _check_device(named)
    plan = make_plan(batch=B, q=1, num_q_heads=hkv, head_map=list(range(hkv)), k_pool=pool,
                     max_pages_per_row=int(block_table.shape[1]), sm_scale=1.0, kv_format=kv_format)
    if out is None:
        out = torch.empty(shape, dtype=torch.float16, device=pool.device)
    _lib.dequant_paged(plan, pool, block_table, live_len, out, stream, scale=scale)
    return out


def kv_append(k_new, v_new, k_scale, v_scale, block_table, live_len, k_pool, v_pool, *, stream=None,
              kv_format: Optional[str] = None):
    """Quantize-on-write: store the FP16 K/V [B, q, Hkv, D] of every request's
    q draft tokens (row i at token live_len[b] - q + i) into the paged FP8
    pools (E4M3 or E5M2, as for ``verify``), in place: the code nearest to
    x / scale, ties to even, saturating at the largest finite value (448 or
    57344). No host synchronization."""
    from . import _lib
    import torch

    _require(k_new.dim() == 4, "k_new must be a contiguous float16 tensor [B, q, Hkv, D]")
    B, nq, hkv, d = (int(x) for x in k_new.shape)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _require(t.dtype == torch.float16 and t.is_contiguous() and tuple(t.shape) == (B, nq, hkv, d),
                 f"{name} must be a contiguous float16 tensor [B, q, Hkv, D]")
    _check_pools(k_pool, v_pool)
    pages, page, phkv, pd, _ = _pool_layout(k_pool)
    _require((phkv, pd) == (hkv, d), "k_new and the pools disagree on num_kv_heads / head_dim")
    _check_request_tensors(B, hkv, block_table, live_len, (("k_scale", k_scale), ("v_scale", v_scale)))
    _check_device([("k_new", k_new), ("v_new", v_new), ("k_scale", k_scale), ("v_scale", v_scale),
                   ("block_table", block_table), ("live_len", live_len), ("k_pool", k_pool), ("v_pool", v_pool)])
    plan = make_plan(batch=B, q=nq, num_q_heads=hkv, head_map=list(range(hkv)), k_pool=k_pool,
                     max_pages_per_row=int(block_table.shape[1]), sm_scale=1.0, kv_format=kv_format)
    _lib.kv_append(plan, k_new, v_new, k_scale, v_scale, block_table, live_len, k_pool, v_pool, stream)
