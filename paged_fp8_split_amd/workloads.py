"""Seeded synthetic inputs for the paged E4M3 verify attention.

This module only *makes inputs*: it draws random numbers, quantizes them to
E4M3 bytes with torch's ``float8_e4m3fn`` encoder (round to nearest even,
after clamping to the largest finite value 448 so that nothing saturates to
NaN), and lays the bytes out in a paged pool. It holds none of the attention
arithmetic and is shared by the tests, the benchmark and the smoke check; both
the HIP library and the CPU oracle consume exactly the bytes it produces.

The five named workloads follow the shapes, sizes and value distributions the
method is measured on (single-request q8 verify at 1K, 128K and 256K context
with 16 query / 2 KV heads at head_dim 256, a 32-request mixed batch, and a
q=1/8/16 sweep at 64K with 32 query / 4 KV heads at head_dim 128). The pages'
own inputs (real model captures) are not public; these synthetic inputs stand
in for them.

Random streams: ``numpy.random.SeedSequence(seed).spawn(6)`` gives one PCG64
stream each for Q, K, V, the page permutation, the outlier positions and the
lengths/midpoint positions, so that changing one knob leaves the other draws
unchanged.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

E4M3_MAX = 448.0
E5M2_MAX = 57344.0
SENTINEL_NAN = 0x7F  # the E4M3 NaN byte; fills every byte no live token owns
SENTINEL_MAX = 0x7E  # 448.0, the alternative tail sentinel used by tests


@dataclasses.dataclass
class Workload:
    """One verify-attention problem held in host memory (numpy arrays)."""

    name: str
    batch: int
    q: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    max_pages_per_row: int
    num_pool_pages: int
    page_stride: int  # bytes
    token_stride: int  # bytes
    head_stride: int  # bytes
    q_fp16: np.ndarray  # float16 [B, q, Hq, D]
    k_pool: np.ndarray  # uint8 flat [num_pool_pages * page_stride]
    v_pool: np.ndarray  # uint8 flat, same layout as k_pool
    k_scale: np.ndarray  # float32 [Hkv]
    v_scale: np.ndarray  # float32 [Hkv]
    block_table: np.ndarray  # int32 [B, max_pages_per_row]
    live_len: np.ndarray  # int32 [B]
    head_map: np.ndarray  # int32 [Hq]
    sm_scale: float
    partition_tokens: int = 64
    kv_format: str = "e4m3"  # how the pool bytes encode values: "e4m3" (E4M3FN) or "e5m2"
    notes: dict = dataclasses.field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def capacity(self) -> int:
        return self.max_pages_per_row * self.page_size

    def kv_bytes(self) -> int:
        """Live K+V bytes one verify step must read (both pools)."""
        L = np.clip(self.live_len.astype(np.int64), 0, self.capacity)
        return int(L.sum()) * self.num_kv_heads * self.head_dim * 2

    def pool_view(self, pool: np.ndarray) -> np.ndarray:
        """[num_pool_pages, page_size, Hkv, D] strided view of a flat pool."""
        return np.lib.stride_tricks.as_strided(
            pool,
            shape=(self.num_pool_pages, self.page_size, self.num_kv_heads, self.head_dim),
            strides=(self.page_stride, self.token_stride, self.head_stride, 1),
            writeable=True,
        )

    def copy(self) -> "Workload":
        fields = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            fields[f.name] = v.copy() if isinstance(v, (np.ndarray, dict)) else v
        return Workload(**fields)


def _e4m3_bytes(x: np.ndarray) -> np.ndarray:
    """float32 array -> E4M3FN bytes: clamp to +-448, then torch's RNE encoder."""
    import torch

    x = np.clip(np.asarray(x, dtype=np.float32), -E4M3_MAX, E4M3_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _e5m2_bytes(x: np.ndarray) -> np.ndarray:
    """float32 array -> E5M2 bytes: clamp to +-57344, then torch's RNE encoder."""
    import torch

    x = np.clip(np.asarray(x, dtype=np.float32), -E5M2_MAX, E5M2_MAX)
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy().copy()


# per format: largest finite value, encoder, and the codes of 1.0 and of the next larger value
_FORMATS = {
    "e4m3": (E4M3_MAX, _e4m3_bytes, 0x38, 0x39),
    "e5m2": (E5M2_MAX, _e5m2_bytes, 0x3C, 0x3D),
}


def build(
    *,
    batch: int,
    q: int,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    page_size: int,
    lengths: Sequence[int],
    seed: int,
    capacity: Optional[int] = None,
    scale_mode: str = "per_head",
    pow2_scale_exps: Optional[Sequence[int]] = None,
    outlier_frac: float = 0.0,
    outlier_sigma: float = 8.0,
    token_pad: int = 0,
    page_pad: int = 0,
    spare_frac: float = 0.25,
    sentinel: int = SENTINEL_NAN,
    zero_k_heads: Sequence[tuple] = (),
    midpoint: Optional[dict] = None,
    kv_format: str = "e4m3",
    name: str = "custom",
) -> Workload:
    """Build a seeded verify-attention workload.

    lengths: live length of each request (draft tokens included).
    capacity: block-table row capacity in tokens (default: max(lengths)).
    scale_mode: "per_head" (absmax/448 per KV head), "per_tensor" (absmax/448
        over all heads, repeated per head) or "pow2" (2**pow2_scale_exps[g]).
    outlier_frac: fraction of token positions (shared by K, V and all heads)
        whose pre-quantization values are drawn from N(0, outlier_sigma**2).
    token_pad / page_pad: extra bytes added to the token / page stride.
    zero_k_heads: (b, g) pairs whose live K bytes are all 0x00 (all scores 0).
    midpoint: {"b": b, "g": g, "counts": [c_0, c_1, ...]}; for that slot the V
        bytes are the code of 1.0 except counts[d % len(counts)] tokens of
        column d, which hold the next larger value (E4M3: 0x38 = 1.0 and
        0x39 = 1.125); its K bytes are 0x00.
    kv_format: "e4m3" (E4M3FN bytes, scales absmax/448) or "e5m2" (E5M2
        bytes, scales absmax/57344).
    """
    if kv_format not in _FORMATS:
        raise ValueError(f"unknown kv_format {kv_format!r}")
    fmax, encode, code_one, code_next = _FORMATS[kv_format]
    B, Hq, Hkv, D, P = batch, num_q_heads, num_kv_heads, head_dim, page_size
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    lengths = np.asarray(lengths, dtype=np.int64)
    if lengths.shape != (B,):
        raise ValueError("lengths must have one entry per request")
    ss = np.random.SeedSequence(seed)
    r_q, r_k, r_v, r_perm, r_out, r_misc = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(6)]

    cap = int(capacity) if capacity is not None else int(max(1, lengths.max(initial=0)))
    max_pages = max(1, -(-cap // P))
    pages_needed = -(-lengths // P)
    num_used = int(pages_needed.sum())
    num_pool = num_used + int(math.ceil(spare_frac * num_used)) + 1

    head_stride = D
    token_stride = Hkv * D + token_pad
    page_stride = P * token_stride + page_pad

    perm = r_perm.permutation(num_pool).astype(np.int32)
    spare_page = int(perm[num_used])  # stays sentinel-filled
    block_table = np.full((B, max_pages), spare_page, dtype=np.int32)
    k = 0
    for b in range(B):
        n = int(pages_needed[b])
        block_table[b, :n] = perm[k : k + n]
        k += n

    k_pool = np.full(num_pool * page_stride, sentinel, dtype=np.uint8)
    v_pool = np.full(num_pool * page_stride, sentinel, dtype=np.uint8)

    # token bookkeeping: every live (b, t) in request order
    n_tok = int(lengths.sum())
    tok_b = np.repeat(np.arange(B), lengths)
    tok_t = np.concatenate([np.arange(L) for L in lengths]) if n_tok else np.zeros(0, np.int64)
    tok_page = block_table[tok_b, tok_t // P] if n_tok else np.zeros(0, np.int32)
    tok_slot = tok_t % P

    outlier = np.zeros(n_tok, dtype=bool)
    if outlier_frac > 0 and n_tok:
        n_out = int(round(outlier_frac * n_tok))
        outlier[r_out.choice(n_tok, size=n_out, replace=False)] = True

    def draw(rng):
        x = rng.standard_normal((n_tok, Hkv, D), dtype=np.float32)
        if outlier.any():
            x[outlier] = rng.standard_normal((int(outlier.sum()), Hkv, D), dtype=np.float32) * np.float32(
                outlier_sigma
            )
        return x

    def scales_for(x):
        if scale_mode == "pow2":
            if pow2_scale_exps is None or len(pow2_scale_exps) != Hkv:
                raise ValueError("pow2 scale mode needs one exponent per KV head")
            return np.array([2.0 ** e for e in pow2_scale_exps], dtype=np.float32)
        if scale_mode == "per_head":
            amax = np.abs(x).max(axis=(0, 2)) if n_tok else np.ones(Hkv, np.float32)
        elif scale_mode == "per_tensor":
            amax = np.full(Hkv, np.abs(x).max() if n_tok else 1.0, dtype=np.float32)
        else:
            raise ValueError(f"unknown scale_mode {scale_mode!r}")
        amax = np.where(amax > 0, amax, 1.0).astype(np.float32)
        return (amax / np.float32(fmax)).astype(np.float32)

    def fill(pool, x, scale):
        view = np.lib.stride_tricks.as_strided(
            pool, shape=(num_pool, P, Hkv, D), strides=(page_stride, token_stride, head_stride, 1), writeable=True
        )
        if n_tok:
            view[tok_page, tok_slot] = encode(x / scale[None, :, None])

    xk = draw(r_k)
    k_scale = scales_for(xk)
    fill(k_pool, xk, k_scale)
    del xk
    xv = draw(r_v)
    v_scale = scales_for(xv)
    fill(v_pool, xv, v_scale)
    del xv

    kview = np.lib.stride_tricks.as_strided(
        k_pool, shape=(num_pool, P, Hkv, D), strides=(page_stride, token_stride, head_stride, 1), writeable=True
    )
    vview = np.lib.stride_tricks.as_strided(
        v_pool, shape=(num_pool, P, Hkv, D), strides=(page_stride, token_stride, head_stride, 1), writeable=True
    )
    for b, g in zero_k_heads:
        sel = tok_b == b
        kview[tok_page[sel], tok_slot[sel], g] = 0x00
    notes = {}
    if midpoint is not None:
        b, g, counts = int(midpoint["b"]), int(midpoint["g"]), list(midpoint["counts"])
        sel = np.nonzero(tok_b == b)[0]
        L = len(sel)
        kview[tok_page[sel], tok_slot[sel], g] = 0x00
        col = np.full((L, D), code_one, dtype=np.uint8)
        for d in range(D):
            c = counts[d % len(counts)]
            col[r_misc.choice(L, size=c, replace=False), d] = code_next
        vview[tok_page[sel], tok_slot[sel], g] = col
        notes["midpoint"] = {"b": b, "g": g, "counts": counts}

    qv = r_q.standard_normal((B, q, Hq, D), dtype=np.float32).astype(np.float16)
    return Workload(
        name=name,
        batch=B,
        q=q,
        num_q_heads=Hq,
        num_kv_heads=Hkv,
        head_dim=D,
        page_size=P,
        max_pages_per_row=max_pages,
        num_pool_pages=num_pool,
        page_stride=page_stride,
        token_stride=token_stride,
        head_stride=head_stride,
        q_fp16=qv,
        k_pool=k_pool,
        v_pool=v_pool,
        k_scale=k_scale,
        v_scale=v_scale,
        block_table=block_table,
        live_len=lengths.astype(np.int32),
        head_map=(np.arange(Hq) // (Hq // Hkv)).astype(np.int32),
        sm_scale=1.0 / math.sqrt(D),
        kv_format=kv_format,
        notes=notes,
    )


def relocate(w: Workload, seed: int) -> Workload:
    """Move every live page to a new physical page (seeded permutation of the
    whole pool) and rewrite the block table to match. The logical content of
    every request is unchanged; bytes no live token owns stay as they were on
    their physical page."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    perm = rng.permutation(w.num_pool_pages).astype(np.int32)  # old page p -> new page perm[p]
    out = w.copy()
    src_k = w.pool_view(w.k_pool)
    src_v = w.pool_view(w.v_pool)
    dst_k = out.pool_view(out.k_pool)
    dst_v = out.pool_view(out.v_pool)
    dst_k[perm] = src_k
    dst_v[perm] = src_v
    out.block_table = perm[w.block_table]
    out.name = w.name + f"+relocated{seed}"
    return out


def set_tail_sentinel(w: Workload, value: int) -> Workload:
    """Rewrite every byte no live token owns (tails of partial pages, spare
    pages, padding bytes) to ``value``; live bytes are unchanged."""
    out = w.copy()
    live = np.zeros(w.num_pool_pages * w.page_stride, dtype=bool)
    lv = np.lib.stride_tricks.as_strided(
        live,
        shape=(w.num_pool_pages, w.page_size, w.num_kv_heads, w.head_dim),
        strides=(w.page_stride, w.token_stride, w.head_stride, 1),
        writeable=True,
    )
    for b in range(w.batch):
        L = int(w.live_len[b])
        if L <= 0:
            continue
        t = np.arange(L)
        lv[w.block_table[b, t // w.page_size], t % w.page_size] = True
    out.k_pool[~live] = value
    out.v_pool[~live] = value
    return out


def _cfg4_lengths(seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 4])))
    L = rng.integers(1024, 32768, size=32, endpoint=True)
    L[rng.choice(32, size=2, replace=False)] = 0
    return L


def config(cfg: int, *, q: Optional[int] = None, seed: Optional[int] = None, **overrides) -> Workload:
    """The five named workloads (seed defaults to the config number).

    1  tiny: B1, L=1024+8, Hq4/Hkv1, D64, page 16, one per-tensor scale
    2  B1, L=131072+8, Hq16/Hkv2, D256, page 64, per-head scales
    3  B1, L=261888+256 (window at the end), Hq16/Hkv2, D256, page 64,
       per-head scales, 1% of tokens drawn at 8x magnitude
    4  B32, L_b ~ U{1024..32768} with two retired rows (L=0), Hq16/Hkv2,
       D256, page 64, capacity 32768
    5  B8, L=65536, q in {1, 8, 16}, Hq32/Hkv4, D128, page 64, power-of-two
       per-head scales 2^-6, 2^-3, 2^1, 2^4, and an FP16-midpoint slot
       (request 0, KV head 0)
    """
    seed = cfg if seed is None else seed
    if cfg == 1:
        kw = dict(batch=1, q=8, num_q_heads=4, num_kv_heads=1, head_dim=64, page_size=16, lengths=[1032],
                  scale_mode="per_tensor", name="tiny-L1032-q8-h4x1-d64-p16")
    elif cfg == 2:
        kw = dict(batch=1, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64, lengths=[131080],
                  name="L131080-q8-h16x2-d256-p64")
    elif cfg == 3:
        kw = dict(batch=1, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64, lengths=[262144],
                  outlier_frac=0.01, name="L262144-q8-h16x2-d256-p64-outliers")
    elif cfg == 4:
        kw = dict(batch=32, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                  lengths=_cfg4_lengths(seed), capacity=32768, name="B32-mixed-q8-h16x2-d256-p64")
    elif cfg == 5:
        qq = 8 if q is None else q
        exps = [round(-6 + 10 * g / 3) for g in range(4)]
        kw = dict(batch=8, q=qq, num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=64,
                  lengths=[65536] * 8, scale_mode="pow2", pow2_scale_exps=exps,
                  midpoint={"b": 0, "g": 0, "counts": [256, 768, 0, 512, 1280, 1792]},
                  name=f"B8-L65536-q{qq}-h32x4-d128-p64")
    else:
        raise ValueError(f"unknown config {cfg}")
    if q is not None and cfg != 5:
        kw["q"] = q
    kw.update(overrides)
    return build(seed=seed, **kw)


def device_tensors(w: Workload, device) -> dict:
    """Copy a workload to ``device`` as the torch tensors the binding takes.
    The pools become [pages, page_size, Hkv, D] uint8 views with the
    workload's byte strides over one flat allocation each."""
    import torch

    def pool(flat):
        t = torch.from_numpy(flat).to(device)
        return t.as_strided((w.num_pool_pages, w.page_size, w.num_kv_heads, w.head_dim),
                            (w.page_stride, w.token_stride, w.head_stride, 1))

    return {
        "q": torch.from_numpy(np.ascontiguousarray(w.q_fp16)).to(device),
        "k_pool": pool(w.k_pool),
        "v_pool": pool(w.v_pool),
        "k_scale": torch.from_numpy(w.k_scale.copy()).to(device),
        "v_scale": torch.from_numpy(w.v_scale.copy()).to(device),
        "block_table": torch.from_numpy(np.ascontiguousarray(w.block_table)).to(device),
        "live_len": torch.from_numpy(w.live_len.copy()).to(device),
        "head_map": [int(x) for x in w.head_map],
        "sm_scale": float(w.sm_scale),
        "kv_format": w.kv_format,
    }
