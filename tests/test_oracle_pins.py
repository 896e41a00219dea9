"""Pins for the FP64 oracle: checks against things other than the oracle itself.

Each test ties the oracle to a library routine it does not use (torch's FP8 and
FP16 decoders, torch's scaled-dot-product attention in float64), to a closed
form, or to an invariance the mathematics fixes. Together they are chosen so
that a plausible slip in the oracle (a wrong causal offset, a dropped scale, a
swapped K/V or head index, a wrong partition fold) fails at least one of them;
``test_pins_detect_planted_mistakes`` shows that directly.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from paged_fp8_split_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- decoders --

def test_e4m3_decode_matches_torch_on_all_bytes():
    ours = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.isnan(ours).sum() == 2  # 0x7F and 0xFF only (the FN variant)
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signs: 0x80 is -0.0, every byte b|0x80 is the negation of b
    assert math.copysign(1.0, ours[0x80]) == -1.0
    assert np.array_equal(ours[0x80:][fin[:128]], -ours[:128][fin[:128]])


def test_e4m3_range_matches_absmax_over_448_recipe():
    # the workloads quantize with scale = absmax / 448: 448 must be the largest
    # finite code and 2^-9 the smallest positive one
    t = oracle.e4m3_table()
    fin = t[~np.isnan(t)]
    assert fin.max() == 448.0 and t[0x7E] == 448.0
    assert fin[fin > 0].min() == 2.0 ** -9 and t[0x01] == 2.0 ** -9
    assert t[0x38] == 1.0 and t[0x39] == 1.125 and t[0x08] == 2.0 ** -6


def test_fp16_decode_matches_numpy_on_all_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    lib = oracle._load()
    ours = np.array([lib.oracle_fp16_value(int(b)) for b in bits])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


# ------------------------------------------------ dense reference (library) --

def _dense_kv(w, pool, scale, b, g, L):
    """Gather request b / KV head g as a dense float64 [L, D] tensor using
    torch's FP8 decoder (independent of the oracle's table)."""
    view = w.pool_view(pool)
    t = np.arange(L)
    raw = np.ascontiguousarray(view[w.block_table[b, t // w.page_size], t % w.page_size, g])
    fp8 = torch.float8_e5m2 if w.kv_format == "e5m2" else torch.float8_e4m3fn
    dec = torch.from_numpy(raw).view(fp8).to(torch.float64)
    return dec * float(scale[g])


def sdpa_reference(w):
    """torch scaled_dot_product_attention (float64, CPU) with an explicit
    bottom-right causal mask; rows with no visible key are set to 0."""
    out = np.zeros((w.batch, w.q, w.num_q_heads, w.head_dim))
    for b in range(w.batch):
        L = int(np.clip(w.live_len[b], 0, w.capacity))
        if L == 0:
            continue
        i = torch.arange(w.q)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= (L - w.q + i)
        for h in range(w.num_q_heads):
            g = int(w.head_map[h])
            K = _dense_kv(w, w.k_pool, w.k_scale, b, g, L)
            V = _dense_kv(w, w.v_pool, w.v_scale, b, g, L)
            Q = torch.from_numpy(w.q_fp16[b, :, h, :].astype(np.float64))
            o = F.scaled_dot_product_attention(Q[None, None], K[None, None], V[None, None],
                                               attn_mask=mask[None, None], scale=w.sm_scale)[0, 0]
            o = o.numpy()
            empty = ~mask.any(dim=1).numpy()
            o[empty] = 0.0
            out[b, :, h, :] = o
    return out


def _rel(a, b):
    return np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300)


SMALL = [
    dict(batch=1, q=1, num_q_heads=1, num_kv_heads=1, head_dim=16, page_size=16, lengths=[37]),
    dict(batch=2, q=3, num_q_heads=4, num_kv_heads=2, head_dim=32, page_size=16, lengths=[50, 2]),
    dict(batch=3, q=8, num_q_heads=8, num_kv_heads=2, head_dim=64, page_size=32, lengths=[300, 8, 0]),
    dict(batch=2, q=16, num_q_heads=4, num_kv_heads=1, head_dim=16, page_size=16, lengths=[129, 5]),
    dict(batch=1, q=4, num_q_heads=6, num_kv_heads=1, head_dim=32, page_size=48, lengths=[211],
         token_pad=16, page_pad=48),
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_oracle_matches_torch_sdpa(case):
    w = W.build(seed=100 + case, **SMALL[case])
    ours = oracle.verify(w)
    ref = sdpa_reference(w)
    assert np.all(np.isfinite(ours))
    assert _rel(ours, ref) < 1e-13
    assert np.abs(ours - ref).max() < 1e-12


def test_oracle_matches_torch_sdpa_with_outliers_and_pow2_scales():
    w = W.build(seed=7, batch=2, q=8, num_q_heads=8, num_kv_heads=4, head_dim=32, page_size=16,
                lengths=[260, 97], outlier_frac=0.05, scale_mode="pow2", pow2_scale_exps=[-6, -3, 1, 4])
    assert _rel(oracle.verify(w), sdpa_reference(w)) < 1e-13


# ------------------------------------------------------------ closed forms --

def test_single_visible_key_returns_that_value_row():
    # L == q: draft row 0 sees exactly key 0, so its output is V-hat of key 0
    w = W.build(seed=3, batch=1, q=4, num_q_heads=2, num_kv_heads=1, head_dim=32, page_size=16, lengths=[4])
    out = oracle.verify(w)
    v0 = _dense_kv(w, w.v_pool, w.v_scale, 0, 0, 1).numpy()[0]
    for h in range(2):
        assert np.array_equal(out[0, 0, h], v0)


def test_uniform_scores_give_the_mean_of_visible_values():
    w = W.build(seed=4, batch=1, q=8, num_q_heads=2, num_kv_heads=1, head_dim=16, page_size=16,
                lengths=[100], zero_k_heads=[(0, 0)])
    out = oracle.verify(w)
    V = _dense_kv(w, w.v_pool, w.v_scale, 0, 0, 100).numpy()
    for i in range(8):
        n = 100 - 8 + i + 1
        ref = V[:n].mean(axis=0)
        assert np.abs(out[0, i, 0] - ref).max() <= 1e-15 * np.abs(ref).max() * 4


def test_dominating_key_wins_exactly():
    # one key scores > 800 above all others: exp underflows to 0 for the rest,
    # so the output is exactly that key's V-hat
    w = W.build(seed=5, batch=1, q=1, num_q_heads=1, num_kv_heads=1, head_dim=16, page_size=16, lengths=[40],
                zero_k_heads=[(0, 0)])
    w.q_fp16[...] = np.float16(240.0)
    view = w.pool_view(w.k_pool)
    j = 17
    view[w.block_table[0, j // 16], j % 16, 0, :] = 0x7E  # 448
    w.k_scale[:] = 1.0
    out = oracle.verify(w)
    vj = _dense_kv(w, w.v_pool, w.v_scale, 0, 0, 40).numpy()[j]
    assert np.array_equal(out[0, 0, 0], vj)


@pytest.mark.parametrize("count,expect_up", [(4, False), (12, True), (20, False), (28, True)])
def test_exact_fp16_midpoints(count, expect_up):
    # K = 0 -> uniform weights; V = 1.0 except `count` of n = 1024 keys at
    # 1.125, so the mean is 1 + count * 2^-13, an exact FP16 tie when count/4
    # is odd. The oracle must land on the tie exactly; RNE picks the even side.
    n = 1024
    w = W.build(seed=6, batch=1, q=1, num_q_heads=1, num_kv_heads=1, head_dim=8, page_size=64, lengths=[n],
                midpoint={"b": 0, "g": 0, "counts": [count]}, scale_mode="pow2", pow2_scale_exps=[-6])
    out = oracle.verify(w)[0, 0, 0]
    exact = (1.0 + count * 2.0 ** -13) * 2.0 ** -6
    assert np.all(out == exact)
    r = np.float16(out[0])  # numpy's correctly rounded FP64 -> FP16
    assert abs(float(r) - exact) == 2.0 ** -17  # the tie sits half an FP16 ulp (2^-16 at 2^-6) away
    assert int(np.array(r).view(np.uint16)) & 1 == 0  # ties go to the even neighbour
    assert (float(r) > exact) == expect_up


# ------------------------------------------------------------ invariances --

@pytest.mark.parametrize("T", [0, 1, 3, 16, 64, 1000])
def test_partition_size_invariance(T):
    w = W.build(seed=8, batch=2, q=8, num_q_heads=4, num_kv_heads=2, head_dim=32, page_size=16, lengths=[301, 64])
    ref = oracle.verify(w, partition_tokens=0)
    assert _rel(oracle.verify(w, partition_tokens=T), ref) < 1e-13


def test_page_relocation_invariance_is_bitwise():
    w = W.build(seed=9, batch=3, q=8, num_q_heads=4, num_kv_heads=2, head_dim=32, page_size=16,
                lengths=[200, 33, 0])
    a = oracle.verify(w)
    b = oracle.verify(W.relocate(w, 1234))
    assert np.array_equal(a, b)


def test_tail_sentinel_invariance_is_bitwise():
    w = W.build(seed=10, batch=2, q=8, num_q_heads=4, num_kv_heads=1, head_dim=32, page_size=16, lengths=[77, 9],
                token_pad=16)
    a = oracle.verify(W.set_tail_sentinel(w, W.SENTINEL_NAN))
    b = oracle.verify(W.set_tail_sentinel(w, W.SENTINEL_MAX))
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b)


def test_power_of_two_scalings_are_exact():
    w = W.build(seed=11, batch=1, q=8, num_q_heads=4, num_kv_heads=2, head_dim=32, page_size=16, lengths=[150])
    a = oracle.verify(w)
    w2 = w.copy()
    w2.v_scale = (w.v_scale * np.float32(8.0)).astype(np.float32)
    assert np.array_equal(oracle.verify(w2), a * 8.0)
    w3 = w.copy()  # k_scale * 2 with sm_scale / 2 leaves every score unchanged
    w3.k_scale = (w.k_scale * np.float32(2.0)).astype(np.float32)
    assert np.array_equal(oracle.verify(w3, sm_scale=w.sm_scale / 2), a)


def test_causality_and_live_length():
    w = W.build(seed=12, batch=1, q=8, num_q_heads=2, num_kv_heads=1, head_dim=16, page_size=16, lengths=[90])
    a = oracle.verify(w)
    # changing the last live key only affects the last draft row
    w2 = w.copy()
    view_k, view_v = w2.pool_view(w2.k_pool), w2.pool_view(w2.v_pool)
    j = 89
    view_k[w2.block_table[0, j // 16], j % 16, 0, :] ^= 0x01
    view_v[w2.block_table[0, j // 16], j % 16, 0, :] ^= 0x01
    b = oracle.verify(w2)
    assert np.array_equal(a[0, :7], b[0, :7])
    assert not np.array_equal(a[0, 7], b[0, 7])
    # rows of a retired request (L = 0) and rows that see nothing (L < q) are +0
    w3 = w.copy()
    w3.live_len[:] = 5
    c = oracle.verify(w3)
    assert np.all(c[0, :3] == 0) and np.all(np.signbit(c[0, :3]) == False)  # noqa: E712
    assert np.all(c[0, 3:] != 0)


def test_head_map_and_batch_independence():
    w = W.build(seed=13, batch=2, q=4, num_q_heads=4, num_kv_heads=2, head_dim=16, page_size=16, lengths=[70, 40])
    a = oracle.verify(w)
    # swap the two KV heads in both pools and in the head map
    w2 = w.copy()
    for pool in (w2.k_pool, w2.v_pool):
        v = w2.pool_view(pool)
        v[:, :, [0, 1]] = v[:, :, [1, 0]]
    w2.k_scale = w.k_scale[[1, 0]].copy()
    w2.v_scale = w.v_scale[[1, 0]].copy()
    w2.head_map = 1 - w.head_map
    assert np.array_equal(oracle.verify(w2), a)
    # request 1 alone gives the same rows as in the batch
    w3 = w.copy()
    w3.batch = 1
    w3.q_fp16 = w.q_fp16[1:].copy()
    w3.block_table = w.block_table[1:].copy()
    w3.live_len = w.live_len[1:].copy()
    assert np.array_equal(oracle.verify(w3)[0], a[1])


def test_pins_detect_planted_mistakes():
    """Plant plausible mistakes (on the CPU, in the oracle's inputs so the
    oracle computes exactly what a buggy oracle would) and check the SDPA pin
    rejects every one of them at the tolerance the pins use."""
    w = W.build(seed=14, batch=2, q=8, num_q_heads=8, num_kv_heads=2, head_dim=32, page_size=16, lengths=[120, 60])
    ref = sdpa_reference(w)
    assert _rel(oracle.verify(w), ref) < 1e-13
    mutants = {}
    m = w.copy(); m.live_len = m.live_len + 1
    mutants["causal offset +1"] = oracle.verify(m)
    mutants["scale 1/D instead of 1/sqrt(D)"] = oracle.verify(w, sm_scale=1.0 / w.head_dim)
    m = w.copy(); m.k_pool, m.v_pool = w.v_pool, w.k_pool; m.k_scale, m.v_scale = w.v_scale, w.k_scale
    mutants["K and V swapped"] = oracle.verify(m)
    m = w.copy(); m.head_map = (np.arange(8) % 2).astype(np.int32)
    mutants["head map h % Hkv"] = oracle.verify(m)
    m = w.copy(); m.k_scale = np.ones_like(w.k_scale)
    mutants["k_scale dropped"] = oracle.verify(m)
    m = w.copy(); m.v_scale = np.ones_like(w.v_scale)
    mutants["v_scale dropped"] = oracle.verify(m)
    for name, out in mutants.items():
        assert not (_rel(out, ref) <= 1e-3), name  # NaN (a read past the live range) also fails the pin


# ------------------------------------------------------------- golden data --

def test_golden_workspace_growth():
    g = json.load(open(os.path.join(GOLDEN, "workspace_growth.json")))
    lse = int(np.prod(g["lse_shape"])) * 4
    ms = int(np.prod(g["max_sum_shape"])) * 4
    assert ms - lse == g["growth_bytes"] == 15 * 1024
    assert g["lse_shape"] == [g["splits"], g["q"], g["group"]]


def test_golden_page_sizes_are_multiples_of_16():
    g = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))
    assert all(p % 16 == 0 for p in g["page_sizes"])


def test_golden_stride_counterexample_arithmetic():
    g = json.load(open(os.path.join(GOLDEN, "stride_counterexample.json")))
    pages, page, heads, dim = g["shape"]
    s_page, s_tok, s_head, s_d = g["strides_bytes"]
    assert s_page == page * s_tok and s_head == dim and s_d == 1
    assert s_tok % 8 == 0 and s_tok % 16 != 0
    assert g["second_token_first_byte"] == s_tok
    assert (s_tok // 16) * 16 == g["paired_loader_would_read_from"]


def test_midpoint_construction_discriminates():
    """Negative control (CPU): the midpoint cells tell the pages' two partial
    representations apart. Normalized per-split outputs rounded to FP16 (the
    legacy representation "[Bugfix] Use FP32 state and E4M3 defaults for
    DFlash2" removes) misround at least one tie, while FP32 (max, sum,
    unnormalized PV) partials combined once round every tie like RNE(exact)."""
    n, T = 2 ** 16, 1024
    rng = np.random.default_rng(0)
    legacy_bad = 0
    for c in (256, 768, 1280, 1792):
        for trial in range(8):
            v = np.ones(n, np.float32)
            v[rng.choice(n, size=c, replace=False)] = np.float32(1.125)
            parts = v.reshape(-1, T)
            exact = (1.0 + c * 2.0 ** -19) * 2.0 ** -6
            want = np.float16(exact).view(np.uint16)
            # FP32 unnormalized partials, one final normalization
            acc = parts.sum(axis=1, dtype=np.float32)
            l = np.full(len(acc), np.float32(T))
            y32 = np.float32(acc.sum(dtype=np.float32) * np.float32(2.0 ** -6)) / np.float32(l.sum(dtype=np.float32))
            assert np.float16(y32).view(np.uint16) == want
            # normalized split outputs rounded to FP16, then averaged
            o16 = (acc / np.float32(T)).astype(np.float16).astype(np.float32)
            y16 = np.float32(o16.mean(dtype=np.float32)) * np.float32(2.0 ** -6)
            legacy_bad += int(np.float16(y16).view(np.uint16) != want)
    assert legacy_bad > 0


# ---- quantize-on-write (the E4M3 encoder and the draft-token append) ----

def _torch_e4m3_codes(v32: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8_e4m3fn conversion (round to nearest even) of
    values already clamped to +-448 (torch returns NaN above 464)."""
    t = torch.from_numpy(np.clip(v32.astype(np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_round_trips_every_finite_code():
    table = oracle.e4m3_table()
    finite = [b for b in range(256) if not math.isnan(table[b])]
    got = oracle.e4m3_encode(table[finite].astype(np.float32))
    assert np.array_equal(got, np.array(finite, dtype=np.uint8))


def test_e4m3_encode_matches_torch_and_brute_force_nearest():
    rng = np.random.default_rng(5)
    table = oracle.e4m3_table()
    codes = np.array([b for b in range(256) if not math.isnan(table[b])])
    vals = table[codes]
    mids = ((vals[:, None] + vals[None, :]) / 2).ravel()  # every midpoint between two codes (and the codes)
    x = np.concatenate([
        rng.normal(0, 1, 4000), rng.normal(0, 100, 2000), rng.uniform(-2 ** -6, 2 ** -6, 2000),
        mids[np.abs(mids) <= 448], [0.0, -0.0, 448.0, -448.0, 2 ** -10, -(2 ** -10), 3 * 2 ** -10],
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = oracle.e4m3_encode(x)
    assert np.array_equal(got, _torch_e4m3_codes(x))
    # brute force: nearest finite code by value, ties to the even code
    for v, c in zip(x[:3000], got[:3000]):
        d = np.abs(vals - float(v))
        best = codes[d == d.min()]
        best = best[best % 2 == 0] if len(best) > 1 else best
        if float(v) == 0.0:
            continue  # +-0 keep their sign (checked below)
        assert c == best[0] or (table[c] == table[best[0]]), (v, c, best)
    assert oracle.e4m3_encode(np.float32(-0.0)) == 0x80 and oracle.e4m3_encode(np.float32(0.0)) == 0x00


def test_e4m3_encode_saturates_and_maps_nan():
    big = np.array([448.0, 449.0, 463.99, 464.0, 480.0, 1.0e9, np.inf], dtype=np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    assert oracle.e4m3_encode(np.float32(np.nan)) == 0x7F


@pytest.mark.parametrize("scale", [1.0, 0.0027, 2.0 ** -6, 16.0, 3.0e-5])
def test_quantize_fp16_is_the_code_of_the_fp32_quotient(scale):
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    keep = np.isfinite(x)
    q32 = (x[keep] / np.float32(scale)).astype(np.float32)
    got = oracle.quantize_fp16(bits[keep], scale)
    big = np.abs(q32) > 448
    assert np.all(got[big & (q32 > 0)] == 0x7E) and np.all(got[big & (q32 < 0)] == 0xFE)
    assert np.array_equal(got[~big], _torch_e4m3_codes(q32[~big]))


@pytest.mark.parametrize("kv_format", ["e4m3", "e5m2"])
def test_kv_append_writes_exactly_the_draft_slots(kv_format):
    w = W.build(seed=61, batch=3, q=4, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                lengths=[37, 2, 0], kv_format=kv_format)
    rng = np.random.default_rng(62)
    kn = rng.normal(0, 3, (3, 4, 2, 64)).astype(np.float16)
    vn = rng.normal(0, 3, (3, 4, 2, 64)).astype(np.float16)
    kp, vp = oracle.kv_append(w, kn, vn)
    view_k, view_v = w.pool_view(kp), w.pool_view(vp)
    old_k = w.pool_view(np.asarray(w.k_pool))
    touched = np.zeros(view_k.shape[:2], dtype=bool)
    for b, L in enumerate(w.live_len):
        for i in range(w.q):
            t = int(L) - w.q + i
            if t < 0:
                continue
            page, slot = w.block_table[b, t // 16], t % 16
            touched[page, slot] = True
            for g in range(2):
                assert np.array_equal(view_k[page, slot, g], oracle.quantize_fp16(kn[b, i, g].view(np.uint16),
                                                                                   w.k_scale[g], kv_format))
                assert np.array_equal(view_v[page, slot, g], oracle.quantize_fp16(vn[b, i, g].view(np.uint16),
                                                                                   w.v_scale[g], kv_format))
    assert touched.sum() == 4 + 2  # request 1 (L=2 < q=4) writes only its last two rows; request 2 nothing
    assert np.array_equal(view_k[~touched], old_k[~touched])


def test_kv_append_feeds_exactly_the_causal_window_of_verify():
    """Append placement tied to verify's causal mask by behaviour alone (no
    slot formula restated): draft row i's K/V become visible to verify rows
    i and later and to no earlier row. Changing the appended V of draft row j
    changes exactly the outputs of rows i >= j; changing only a non-draft
    (history) token changes every row that sees it."""
    w = W.build(seed=63, batch=2, q=5, num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                lengths=[70, 5])
    rng = np.random.default_rng(64)
    kn = rng.normal(0, 2, (2, 5, 2, 64)).astype(np.float16)
    vn = rng.normal(0, 2, (2, 5, 2, 64)).astype(np.float16)

    def verify_after(kk, vv):
        kp, vp = oracle.kv_append(w, kk, vv)
        wk = w.copy()
        wk.k_pool, wk.v_pool = kp, vp
        return oracle.verify(wk)

    base = verify_after(kn, vn)
    assert np.all(np.isfinite(base))
    for j in range(w.q):
        v2 = vn.copy()
        v2[:, j] = (v2[:, j].astype(np.float32) + 1.0).astype(np.float16)
        out = verify_after(kn, v2)
        for b in range(w.batch):
            for i in range(w.q):
                changed = not np.array_equal(out[b, i], base[b, i])
                assert changed == (i >= j), (b, i, j)


# ---- the scaled E4M3 -> FP16 bridge ----

def test_fp16_rne_matches_numpy_double_to_half():
    rng = np.random.default_rng(7)
    halves = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    finite = halves[np.isfinite(halves)]
    nxt = np.nextafter(finite, np.inf)
    mids = (finite[:-1] + np.sort(finite)[1:]) / 2
    x = np.concatenate([finite, (finite + nxt) / 2, mids, rng.normal(0, 1e3, 5000), rng.normal(0, 1e-5, 5000),
                        [65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -25, 3 * 2.0 ** -25]])
    got = oracle.fp16_rne(x)
    with np.errstate(over="ignore"):  # values from 65520 up round to infinity, as they must
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("kv_format", ["e4m3", "e5m2"])
@pytest.mark.parametrize("scale", [None, 1.0, 0.0011, 3.0e-7, 1.0 + 2.0 ** -12, 2.0 ** -9 * 3])
def test_dequant_is_one_rounding_of_the_exact_product(scale, kv_format):
    w = W.build(seed=71, batch=2, q=2, num_q_heads=2, num_kv_heads=2, head_dim=64, page_size=16,
                lengths=[40, 5], kv_format=kv_format)
    view = w.pool_view(w.k_pool)
    codes = np.arange(256, dtype=np.uint8)
    view[w.block_table[0, 0], :, :, :] = np.resize(codes, view[0].shape)  # every code in request 0's first page
    sc = None if scale is None else np.array([scale, 2 * scale], dtype=np.float32)
    got = oracle.dequant(w, scale=sc)
    fp8 = torch.float8_e5m2 if kv_format == "e5m2" else torch.float8_e4m3fn
    table = torch.arange(256, dtype=torch.uint8).view(fp8).to(torch.float64).numpy()
    for b in range(2):
        L = int(w.live_len[b])
        t = np.arange(L)
        raw = view[w.block_table[b, t // 16], t % 16]                      # [L, Hkv, D]
        s = np.ones(2) if sc is None else sc.astype(np.float64)
        with np.errstate(over="ignore"):  # E5M2 infinities and products past 65504 become FP16 infinities
            want = (table[raw] * s[None, :, None]).astype(np.float16)      # numpy: one RNE from float64
        g = got[b, :L]
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(g), nan)
        assert np.array_equal(g[~nan].view(np.uint16), want[~nan].view(np.uint16))
        assert np.all(got[b, L:].view(np.uint16) == 0)


# ---- the E5M2 KV format (the explicit alternative to E4M3) ----

def test_e5m2_decode_matches_torch_and_the_fp16_high_byte():
    ours = oracle.e5m2_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # an E5M2 byte is the high byte of the IEEE half with the same value
    half = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(half))
    assert np.array_equal(ours[fin], half[fin])
    assert np.array_equal(oracle.kv_table("e5m2")[fin], ours[fin])


def test_e5m2_range_and_special_codes():
    t = oracle.e5m2_table()
    assert t[0x7B] == 57344.0 and t[0xFB] == -57344.0
    assert t[0x7C] == np.inf and t[0xFC] == -np.inf
    assert np.isnan(t).sum() == 6  # 0x7D..0x7F and 0xFD..0xFF
    assert t[0x01] == 2.0 ** -16 and t[0x04] == 2.0 ** -14
    assert t[0x3C] == 1.0 and t[0x3D] == 1.25


def _torch_e5m2_codes(v32: np.ndarray) -> np.ndarray:
    """torch's float32 -> float8_e5m2 conversion (round to nearest even) of
    values already clamped to +-57344."""
    t = torch.from_numpy(np.clip(v32.astype(np.float32), -57344.0, 57344.0))
    return t.to(torch.float8_e5m2).view(torch.uint8).numpy()


def test_e5m2_encode_round_trips_every_finite_code():
    table = oracle.e5m2_table()
    finite = [b for b in range(256) if np.isfinite(table[b])]
    got = oracle.e5m2_encode(table[finite].astype(np.float32))
    assert np.array_equal(got, np.array(finite, dtype=np.uint8))


def test_e5m2_encode_matches_torch_and_brute_force_nearest():
    rng = np.random.default_rng(15)
    table = oracle.e5m2_table()
    codes = np.array([b for b in range(256) if np.isfinite(table[b])])
    vals = table[codes]
    mids = ((vals[:, None] + vals[None, :]) / 2).ravel()
    x = np.concatenate([
        rng.normal(0, 1, 4000), rng.normal(0, 5000, 2000), rng.uniform(-2 ** -14, 2 ** -14, 2000),
        mids[np.abs(mids) <= 57344], [0.0, -0.0, 57344.0, -57344.0, 2 ** -17, -(2 ** -17), 3 * 2 ** -17],
    ]).astype(np.float32)
    x = x[np.abs(x) <= 57344]
    got = oracle.e5m2_encode(x)
    assert np.array_equal(got, _torch_e5m2_codes(x))
    for v, c in zip(x[:3000], got[:3000]):
        if float(v) == 0.0:
            continue
        d = np.abs(vals - float(v))
        best = codes[d == d.min()]
        best = best[best % 2 == 0] if len(best) > 1 else best
        assert c == best[0] or (table[c] == table[best[0]]), (v, c, best)
    assert oracle.e5m2_encode(np.float32(-0.0)) == 0x80 and oracle.e5m2_encode(np.float32(0.0)) == 0x00


def test_e5m2_encode_saturates_and_maps_nan():
    big = np.array([57344.0, 57345.0, 61439.0, 61440.0, 65504.0, 1.0e30, np.inf], dtype=np.float32)
    assert np.all(oracle.e5m2_encode(big) == 0x7B)
    assert np.all(oracle.e5m2_encode(-big) == 0xFB)
    assert oracle.e5m2_encode(np.float32(np.nan)) == 0x7F


@pytest.mark.parametrize("scale", [1.0, 0.37, 2.0 ** -10, 1000.0])
def test_quantize_fp16_e5m2_is_the_code_of_the_fp32_quotient(scale):
    bits = np.arange(0, 65536, 5, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16).astype(np.float32)
    keep = np.isfinite(x)
    q32 = (x[keep] / np.float32(scale)).astype(np.float32)
    got = oracle.quantize_fp16(bits[keep], scale, "e5m2")
    big = np.abs(q32) > 57344
    assert np.all(got[big & (q32 > 0)] == 0x7B) and np.all(got[big & (q32 < 0)] == 0xFB)
    assert np.array_equal(got[~big], _torch_e5m2_codes(q32[~big]))


@pytest.mark.parametrize("case", [1, 2, 4])
def test_oracle_matches_torch_sdpa_e5m2(case):
    w = W.build(seed=300 + case, kv_format="e5m2", **SMALL[case])
    ours = oracle.verify(w)
    assert np.all(np.isfinite(ours))
    assert _rel(ours, sdpa_reference(w)) < 1e-13


def test_oracle_e5m2_with_outliers_and_pow2_scales():
    w = W.build(seed=8, batch=2, q=8, num_q_heads=8, num_kv_heads=4, head_dim=32, page_size=16,
                lengths=[260, 97], outlier_frac=0.05, scale_mode="pow2", pow2_scale_exps=[-14, -6, 1, 4],
                kv_format="e5m2")
    assert _rel(oracle.verify(w), sdpa_reference(w)) < 1e-13


def test_oracle_reads_the_format_it_is_given():
    # the same bytes read as the other format give another result (the format is not ignored)
    w = W.build(seed=9, batch=1, q=2, num_q_heads=2, num_kv_heads=1, head_dim=16, page_size=16, lengths=[40])
    w.k_pool &= 0xBF  # clear bit 6: every byte is then finite in both formats
    w.v_pool &= 0xBF
    w2 = w.copy()
    w2.kv_format = "e5m2"
    assert _rel(oracle.verify(w2), oracle.verify(w)) > 1e-3
    assert _rel(oracle.verify(w2), sdpa_reference(w2)) < 1e-13
