"""Seeded random sweep of small shapes: GPU verify against the FP64 oracle.

Each case draws a batch, q, heads, head_dim, page size, KV format, strides
with padding, a block-table capacity above the longest request (so that
single requests have splits with nothing live) and live lengths that include
retired requests (0) and requests shorter than q, then checks parity and that
a repeated launch is bit-identical. Sizes stay small enough for the oracle to
finish in well under a second per case."""
import numpy as np
import pytest

from paged_fp8_split_amd import workloads as W

from parity import assert_parity, log, oracle_ref, run, to_np

pytestmark = pytest.mark.gpu

N_CASES = 40


def draw_case(k: int) -> dict:
    rng = np.random.default_rng(9000 + k)
    D = int(rng.choice([64, 128, 256]))
    hkv = int(rng.choice([1, 2, 4]))
    G = int(rng.choice([1, 2, 4, 6, 8, 16]))
    q = int(rng.choice([1, 2, 3, 5, 8, 11, 16]))
    batch = int(rng.choice([1, 1, 2, 3, 5]))
    page = int(rng.choice([16, 32, 48, 64]))
    lengths = []
    for _ in range(batch):
        u = rng.random()
        if u < 0.1:
            lengths.append(0)
        elif u < 0.2:
            lengths.append(int(rng.integers(1, q + 1)))
        else:
            lengths.append(int(rng.integers(q, 2500)))
    cap = max(max(lengths), 1) + int(rng.choice([0, 0, 1, 700, 3000]))
    tps = int(rng.choice([0, 0, 64, 128, 256, 1024]))
    fmt = "e5m2" if rng.random() < 0.2 else "e4m3"
    pad = int(rng.choice([0, 0, 16]))
    return dict(batch=batch, q=q, num_q_heads=G * hkv, num_kv_heads=hkv, head_dim=D, page_size=page,
                lengths=lengths, capacity=cap, kv_format=fmt, token_pad=pad, page_pad=2 * pad,
                outlier_frac=0.01 if rng.random() < 0.3 else 0.0, seed=700 + k), tps


@pytest.mark.parametrize("k", range(N_CASES))
def test_random_shape_parity(k):
    kw, tps = draw_case(k)
    w = W.build(**kw)
    log(f"[sweep {k}] B={kw['batch']} q={kw['q']} Hq={kw['num_q_heads']} Hkv={kw['num_kv_heads']} "
        f"D={kw['head_dim']} page={kw['page_size']} L={kw['lengths']} cap={kw['capacity']} tps={tps} {kw['kv_format']}")
    out, t = run(w, tokens_per_split=tps)
    a = to_np(out)
    b = to_np(run(w, tokens_per_split=tps, tensors=t)[0])
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "repeat launch differs"
    r = oracle_ref(w)
    assert_parity(a, r, f"sweep {k}")
    # rows that see no key are +0.0
    L = np.clip(w.live_len.astype(np.int64), 0, w.capacity)
    for bb in range(w.batch):
        for i in range(w.q):
            if L[bb] - w.q + i + 1 <= 0:
                assert np.all(a[bb, i].view(np.uint16) == 0), f"request {bb} row {i}"


MEDIUM = [
    # (batch, q, Hq, Hkv, head_dim, page, lengths, capacity): default plans, batch cap and
    # four-wave batch workgroups with several splits per request
    (4, 8, 16, 2, 256, 64, [40000, 2048, 0, 20481], 40960),
    (3, 16, 32, 4, 128, 64, [16385, 30000, 4095], 32768),
    (6, 1, 32, 4, 128, 32, [9000, 1, 12345, 0, 7, 20000], 20480),
    (2, 5, 12, 2, 256, 48, [33333, 48], 36000),
    (1, 8, 16, 2, 256, 64, [9000], 65536),   # one request far below its capacity: empty splits
    (5, 3, 8, 1, 64, 16, [25000, 100, 3, 17000, 8191], 25600),
]


@pytest.mark.parametrize("k", range(len(MEDIUM)))
def test_medium_batch_parity_default_plan(k):
    batch, q, hq, hkv, D, page, lengths, cap = MEDIUM[k]
    w = W.build(seed=800 + k, batch=batch, q=q, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=page,
                lengths=lengths, capacity=cap, outlier_frac=0.01)
    log(f"[medium {k}] B={batch} q={q} Hq={hq} Hkv={hkv} D={D} page={page} L={lengths} cap={cap}")
    out, t = run(w)
    a = to_np(out)
    b = to_np(run(w, tensors=t)[0])
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), "repeat launch differs"
    assert_parity(a, oracle_ref(w), f"medium {k}")
