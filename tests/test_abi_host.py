"""Host-only checks of the C ABI (no GPU): the library loads, exports every
symbol include/pfs.h declares, and rejects every invalid problem with its own
status code before any HIP call is made."""
import ctypes
import json
import os
import re

import pytest

from paged_fp8_split_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def header_functions():
    text = open(os.path.join(ROOT, "include", "pfs.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pfs_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = header_functions()
    assert names == sorted([
        "pfs_abi_version", "pfs_dequant_paged", "pfs_kv_append", "pfs_plan_create", "pfs_plan_destroy",
        "pfs_plan_num_splits",
        "pfs_plan_tokens_per_split", "pfs_plan_workspace_bytes", "pfs_status_string", "pfs_verify",
        "pfs_verify_combine", "pfs_verify_split", "pfs_verify_noalloc", "pfs_noalloc_scratch_bytes"])
    for n in names:
        assert hasattr(lib, n), n


def test_noalloc_scratch_size_and_refusals_without_a_gpu():
    # the stated size, and the host-side checks that run before any HIP call
    assert _lib.noalloc_scratch_bytes() == 128 << 20
    lib = _lib.load()
    assert lib.pfs_verify_noalloc(None, *([None] * 9)) == _lib.STATUS_CODE["PFS_ERR_NULL"]
    big = _lib.Plan(**dict(BASE, batch=64))  # 64 requests x 262,144 tokens: far beyond 128 MiB of partials
    assert big.workspace_bytes > _lib.noalloc_scratch_bytes()
    assert lib.pfs_verify_noalloc(big.handle, *([None] * 9)) == _lib.STATUS_CODE["PFS_ERR_WORKSPACE"]


def test_abi_version_and_status_strings():
    lib = _lib.load()
    assert lib.pfs_abi_version() == _lib.ABI_VERSION
    for code, name in _lib.STATUS.items():
        s = _lib.status_string(code)
        assert s and s != "unknown status", name
    assert _lib.status_string(12345) == "unknown status"


def test_stale_library_is_refused():
    class Stale:
        @staticmethod
        def pfs_abi_version():
            return _lib.ABI_VERSION - 1

    with pytest.raises(RuntimeError, match="does not match"):
        _lib.check_abi(Stale())


BASE = dict(batch=1, q=8, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64, max_pages_per_row=4096,
            num_pool_pages=5000, kv_page_stride=64 * 512, kv_token_stride=512, kv_head_stride=256, sm_scale=0.0625,
            head_map=[h // 8 for h in range(16)])


def test_default_split_single_request_is_one_round():
    """One request: the default split fills one round of workgroups (256 CUs,
    one per CU at head_dim 256): 4096 pages x 64 tokens over 2 KV heads ->
    128 splits of 2048 tokens."""
    p = _lib.Plan(**BASE)
    assert (p.tokens_per_split, p.num_splits) == (2048, 128)


@pytest.mark.parametrize("head_dim,cap", [(256, 2048), (128, 4096), (64, 8192)])
def test_default_split_batches_are_capped_near_one_mib(head_dim, cap):
    """Batches: the default split holds at most about 1 MiB of K+V bytes per
    KV head (cap tokens x 2 x head_dim bytes), so that splits of unequal
    requests can be balanced by the dispatcher; one round would give larger
    splits here (batch 32 x 2 KV heads at 32768 tokens: 8192)."""
    kw = dict(BASE, batch=32, head_dim=head_dim, max_pages_per_row=512, kv_page_stride=64 * 2 * head_dim,
              kv_token_stride=2 * head_dim, kv_head_stride=head_dim)
    p = _lib.Plan(**kw)
    assert p.tokens_per_split == cap
    assert p.tokens_per_split * 2 * head_dim <= 1 << 20
    assert p.num_splits == 32768 // cap


def plan_status(**over):
    kw = dict(BASE)
    kw.update(over)
    try:
        _lib.Plan(**kw)
        return 0
    except _lib.PfsError as e:
        return e.status


def test_valid_problem_plans():
    p = _lib.Plan(**BASE)
    assert p.tokens_per_split % 64 == 0
    assert p.num_splits * p.tokens_per_split >= p.capacity
    assert p.workspace_bytes > 0
    # planning is a pure function of the shape
    q = _lib.Plan(**BASE)
    assert (p.num_splits, p.tokens_per_split, p.workspace_bytes) == (q.num_splits, q.tokens_per_split,
                                                                      q.workspace_bytes)


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=96), "PFS_ERR_UNSUPPORTED"),
    (dict(head_dim=512), "PFS_ERR_UNSUPPORTED"),
    (dict(q=0), "PFS_ERR_UNSUPPORTED"),
    (dict(q=17), "PFS_ERR_UNSUPPORTED"),
    (dict(page_size=40, kv_page_stride=40 * 512), "PFS_ERR_UNSUPPORTED"),
    (dict(partition_tokens=32), "PFS_ERR_UNSUPPORTED"),
    (dict(kv_format=2), "PFS_ERR_UNSUPPORTED"),
    (dict(kv_format=-1), "PFS_ERR_UNSUPPORTED"),
    (dict(pv_mode=2), "PFS_ERR_UNSUPPORTED"),
    (dict(pv_mode=-1), "PFS_ERR_UNSUPPORTED"),
    (dict(num_cus=-1), "PFS_ERR_SHAPE"),
    (dict(tokens_per_split=100), "PFS_ERR_SHAPE"),
    (dict(tokens_per_split=16384 + 64), "PFS_ERR_UNSUPPORTED"),  # beyond the split's 1024-tile table
    # 65535 requests x 2 KV heads x 1024 splits of 64 tokens: a split grid beyond 2^31 work-items
    (dict(batch=65535, max_pages_per_row=1024, tokens_per_split=64), "PFS_ERR_SHAPE"),
    (dict(num_q_heads=15, head_map=[0] * 15), "PFS_ERR_SHAPE"),
    (dict(batch=-1), "PFS_ERR_SHAPE"),
    (dict(batch=65536), "PFS_ERR_SHAPE"),
    (dict(sm_scale=0.0), "PFS_ERR_SHAPE"),
    (dict(sm_scale=float("nan")), "PFS_ERR_SHAPE"),
    (dict(kv_head_stride=128), "PFS_ERR_SHAPE"),             # heads overlap
    (dict(kv_token_stride=496), "PFS_ERR_SHAPE"),            # tokens overlap
    (dict(kv_page_stride=63 * 512), "PFS_ERR_SHAPE"),        # pages overlap
    (dict(kv_token_stride=520, kv_page_stride=64 * 520), "PFS_ERR_ALIGNMENT"),
    (dict(kv_page_stride=64 * 512 + 8), "PFS_ERR_ALIGNMENT"),
    (dict(head_map=[0] * 16), "PFS_ERR_HEAD_MAP"),            # groups not uniform
    (dict(head_map=[h // 8 for h in range(15)] + [2]), "PFS_ERR_HEAD_MAP"),  # out of range
])
def test_invalid_problems_are_rejected(over, status):
    assert plan_status(**over) == _lib.STATUS_CODE[status]


def test_largest_split_is_accepted():
    p = _lib.Plan(**dict(BASE, tokens_per_split=16384))
    assert p.tokens_per_split == 16384 and p.num_splits == 4096 * 64 // 16384


def test_both_kv_formats_plan_identically():
    # the format changes only the decoder: same splits, same workspace
    a, b = _lib.Plan(**BASE), _lib.Plan(**dict(BASE, kv_format=1))
    assert (a.num_splits, a.tokens_per_split, a.workspace_bytes) == (b.num_splits, b.tokens_per_split,
                                                                      b.workspace_bytes)
    assert (a.kv_format, b.kv_format) == (0, 1)


def test_probability_modes_plan_alike():
    # the probability mode changes only the PV operands: same splits, same workspace,
    # in either KV format (the residual needs no scaling of V, so E5M2 takes it too)
    for fmt in (0, 1):
        a, b = _lib.Plan(**dict(BASE, kv_format=fmt)), _lib.Plan(**dict(BASE, kv_format=fmt, pv_mode=1))
        assert (a.num_splits, a.tokens_per_split, a.workspace_bytes) == (b.num_splits, b.tokens_per_split,
                                                                          b.workspace_bytes)
        assert (a.pv_mode, b.pv_mode) == (0, 1)


def test_default_split_length_fills_the_given_compute_units():
    # 0 means the MI355X's 256; a device with fewer units gets longer splits, one round each way
    base, same, half = (_lib.Plan(**dict(BASE, num_cus=c)) for c in (0, 256, 128))
    assert (base.num_splits, base.tokens_per_split) == (same.num_splits, same.tokens_per_split)
    assert half.tokens_per_split == 2 * base.tokens_per_split
    assert half.num_splits * 2 == base.num_splits
    # an explicit split length ignores it
    a, b = (_lib.Plan(**dict(BASE, tokens_per_split=1024, num_cus=c)) for c in (0, 100))
    assert (a.num_splits, a.tokens_per_split) == (b.num_splits, b.tokens_per_split)


def test_head_major_pool_layout_is_accepted():
    # [page][head][slot][d]: 2 heads x 64 slots x 256 bytes per page
    assert plan_status(kv_token_stride=256, kv_head_stride=64 * 256, kv_page_stride=2 * 64 * 256) == 0
    # the head stride must hold a head's 64 slots
    assert plan_status(kv_token_stride=256, kv_head_stride=63 * 256,
                       kv_page_stride=4 * 64 * 256) == _lib.STATUS_CODE["PFS_ERR_SHAPE"]
    # and the page stride both heads
    assert plan_status(kv_token_stride=256, kv_head_stride=64 * 256,
                       kv_page_stride=2 * 64 * 256 - 16) == _lib.STATUS_CODE["PFS_ERR_SHAPE"]


def test_pages_stride_counterexample_is_rejected():
    g = json.load(open(os.path.join(GOLDEN, "stride_counterexample.json")))
    pages, page, heads, dim = g["shape"]
    sp, st, sh, _ = g["strides_bytes"]
    s = plan_status(batch=1, q=5, num_q_heads=6, num_kv_heads=heads, head_dim=dim, page_size=page,
                    max_pages_per_row=pages, num_pool_pages=pages, kv_page_stride=sp, kv_token_stride=st,
                    kv_head_stride=sh, head_map=[0] * 6)
    assert s == _lib.STATUS_CODE["PFS_ERR_ALIGNMENT"]
    # the same cache with the token stride padded to the next 16-byte unit is accepted
    assert plan_status(batch=1, q=5, num_q_heads=6, num_kv_heads=heads, head_dim=dim, page_size=page,
                       max_pages_per_row=pages, num_pool_pages=pages, kv_page_stride=page * 272,
                       kv_token_stride=272, kv_head_stride=sh, head_map=[0] * 6) == 0


def test_pages_page_sizes_are_accepted():
    g = json.load(open(os.path.join(GOLDEN, "page_sizes.json")))
    for page in g["page_sizes"]:
        assert plan_status(page_size=page, kv_page_stride=page * 512, max_pages_per_row=2) == 0, page


def test_workspace_holds_max_sum_pairs_per_split_row():
    # the pages' workspace change: [80, 8, 6] log-sum-exp -> [80, 8, 6, 2] max/sum,
    # i.e. 15 KiB more for 80 splits x q8 x GQA6 (one KV head per rank)
    g = json.load(open(os.path.join(GOLDEN, "workspace_growth.json")))
    S, q, G = g["splits"], g["q"], g["group"]
    p = _lib.Plan(batch=1, q=q, num_q_heads=G, num_kv_heads=1, head_dim=256, page_size=64, max_pages_per_row=S,
                  num_pool_pages=S, kv_page_stride=64 * 256, kv_token_stride=256, kv_head_stride=256,
                  sm_scale=0.0625, head_map=[0] * G, tokens_per_split=64)
    assert p.num_splits == S
    ml = S * q * G * 2 * 4
    assert ml - S * q * G * 4 == g["growth_bytes"]
    acc = S * q * G * 256 * 4
    rnd = lambda x: (x + 255) // 256 * 256  # noqa: E731
    assert p.workspace_bytes == rnd(ml) + rnd(acc)


def test_verify_host_checks_need_no_device():
    p = _lib.Plan(**BASE)
    lib = _lib.load()
    ok = 1 << 20  # any 256-aligned non-null address: these calls return before touching it
    args = [ok] * 9
    # NULL pointer
    assert lib.pfs_verify(p.handle, None, *args[1:], p.workspace_bytes, None) == _lib.STATUS_CODE["PFS_ERR_NULL"]
    # misaligned Q
    bad = [ok + 8] + args[1:]
    assert lib.pfs_verify(p.handle, *bad, p.workspace_bytes, None) == _lib.STATUS_CODE["PFS_ERR_ALIGNMENT"]
    # workspace too small, NULL or misaligned
    assert lib.pfs_verify(p.handle, *args, p.workspace_bytes - 1, None) == _lib.STATUS_CODE["PFS_ERR_WORKSPACE"]
    assert lib.pfs_verify(p.handle, *args[:8], None, p.workspace_bytes, None) == \
        _lib.STATUS_CODE["PFS_ERR_WORKSPACE"]
    assert lib.pfs_verify(p.handle, *args[:8], ok + 64, p.workspace_bytes, None) == \
        _lib.STATUS_CODE["PFS_ERR_WORKSPACE"]
    # a NULL plan
    assert lib.pfs_verify(None, *args, p.workspace_bytes, None) == _lib.STATUS_CODE["PFS_ERR_NULL"]
    # the two phases check the same things
    assert lib.pfs_verify_split(p.handle, ok + 8, *([ok] * 7), p.workspace_bytes, None) == \
        _lib.STATUS_CODE["PFS_ERR_ALIGNMENT"]
    assert lib.pfs_verify_split(p.handle, *([ok] * 8), p.workspace_bytes - 1, None) == \
        _lib.STATUS_CODE["PFS_ERR_WORKSPACE"]
    assert lib.pfs_verify_combine(p.handle, ok, ok, ok + 2, ok, p.workspace_bytes, None) == \
        _lib.STATUS_CODE["PFS_ERR_ALIGNMENT"]
    assert lib.pfs_verify_combine(p.handle, None, ok, ok, ok, p.workspace_bytes, None) == \
        _lib.STATUS_CODE["PFS_ERR_NULL"]
    assert lib.pfs_plan_workspace_bytes(None) == 0
    # an empty batch is a no-op that touches nothing
    e = _lib.Plan(**dict(BASE, batch=0))
    assert lib.pfs_verify(e.handle, *([None] * 9), 0, None) == 0


def test_plan_create_null_arguments():
    lib = _lib.load()
    h = ctypes.c_void_p()
    assert lib.pfs_plan_create(None, ctypes.byref(h)) == _lib.STATUS_CODE["PFS_ERR_NULL"]
    prob = _lib.PfsProblem(1, 8, 16, 2, 256, 64, 4096, 5000, 64, 0, 0, 0, 0, 64 * 512, 512, 256, 0.0625, None)
    assert lib.pfs_plan_create(ctypes.byref(prob), ctypes.byref(h)) == _lib.STATUS_CODE["PFS_ERR_NULL"]


def test_codec_host_checks_need_no_device():
    lib = _lib.load()
    ok = 1 << 20
    p = _lib.Plan(**BASE)
    # bridge: NULL, misaligned pool or output, misaligned scale
    assert lib.pfs_dequant_paged(p.handle, None, None, ok, ok, ok, None) == _lib.STATUS_CODE["PFS_ERR_NULL"]
    assert lib.pfs_dequant_paged(p.handle, ok + 8, None, ok, ok, ok, None) == _lib.STATUS_CODE["PFS_ERR_ALIGNMENT"]
    assert lib.pfs_dequant_paged(p.handle, ok, ok + 2, ok, ok, ok, None) == _lib.STATUS_CODE["PFS_ERR_ALIGNMENT"]
    # bridge grid: capacity x KV heads x head_dim / 16 work-items must stay below 2^31
    big = _lib.Plan(**dict(BASE, max_pages_per_row=1 << 20, num_pool_pages=1 << 20))
    assert lib.pfs_dequant_paged(big.handle, ok, None, ok, ok, ok, None) == _lib.STATUS_CODE["PFS_ERR_SHAPE"]
    # append: NULL and misaligned arguments
    assert lib.pfs_kv_append(p.handle, None, *([ok] * 7), None) == _lib.STATUS_CODE["PFS_ERR_NULL"]
    assert lib.pfs_kv_append(p.handle, ok + 8, *([ok] * 7), None) == _lib.STATUS_CODE["PFS_ERR_ALIGNMENT"]
    assert lib.pfs_kv_append(p.handle, *([ok] * 2), ok + 2, *([ok] * 5), None) == \
        _lib.STATUS_CODE["PFS_ERR_ALIGNMENT"]
    # an empty batch touches nothing
    e = _lib.Plan(**dict(BASE, batch=0))
    assert lib.pfs_dequant_paged(e.handle, None, None, None, None, None, None) == 0
    assert lib.pfs_kv_append(e.handle, *([None] * 8), None) == 0


def test_build_stamp_tracks_source_content(tmp_path, monkeypatch):
    """The test session rebuilds libpfs when its sources change: the stamp is
    a digest of their content (and the headers'), not of file times."""
    from paged_fp8_split_amd import build

    src = tmp_path / "k.hip"
    src.write_text("// one\n")
    d1 = build._digest([str(src)])
    src.write_text("// two\n")
    d2 = build._digest([str(src)])
    assert d1 != d2
    src.write_text("// one\n")
    assert build._digest([str(src)]) == d1
    # a missing stamp or library counts as stale
    monkeypatch.setattr(build, "LIB", str(tmp_path / "libpfs.so"))
    assert build.stale()


def test_build_stamp_does_not_depend_on_the_tree_path(tmp_path, monkeypatch):
    """A copy of the tree elsewhere (as on another machine) keeps its build
    current: the digest hashes the include root as a placeholder."""
    import shutil

    from paged_fp8_split_amd import build

    ref = build._digest(build.SOURCES)
    pkg = tmp_path / "paged_fp8_split_amd"
    shutil.copytree(build.CSRC, pkg / "csrc")
    shutil.copytree(os.path.join(os.path.dirname(build.HERE), "include"), tmp_path / "include")
    monkeypatch.setattr(build, "HERE", str(pkg))
    monkeypatch.setattr(build, "CSRC", str(pkg / "csrc"))
    moved = [str(pkg / "csrc" / os.path.basename(s)) for s in build.SOURCES]
    assert build._digest(moved) == ref


def _host_problem():
    import torch

    B, nq, Hq, Hkv, D, page, pages, mppr = 2, 4, 4, 1, 64, 16, 8, 4
    return dict(q=torch.zeros(B, nq, Hq, D, dtype=torch.float16),
                k_pool=torch.zeros(pages, page, Hkv, D, dtype=torch.uint8),
                v_pool=torch.zeros(pages, page, Hkv, D, dtype=torch.uint8),
                k_scale=torch.ones(Hkv), v_scale=torch.ones(Hkv),
                block_table=torch.zeros(B, mppr, dtype=torch.int32), live_len=torch.zeros(B, dtype=torch.int32))


def test_package_verify_checks_every_tensor_before_the_library():
    """The kernels size every buffer from the plan, so the binding refuses a
    tensor that does not match it (a short block table, length or scale
    vector, a wrong output, a plan made for other shapes), and tensors that
    are not on the GPU, before any pointer reaches the library."""
    import torch

    import paged_fp8_split_amd as pfs

    a = _host_problem()
    q, bt, ll, ks = a["q"], a["block_table"], a["live_len"], a["k_scale"]
    bad = [
        dict(q=q.float()),
        dict(q=q[:, :, :, :32]),
        dict(q=torch.zeros(2, 4, 4, 128, dtype=torch.float16)),
        dict(v_pool=a["v_pool"][:4]),
        dict(v_pool=a["v_pool"].view(torch.float8_e5m2)),
        dict(block_table=bt[:1]),
        dict(block_table=bt.to(torch.int64)),
        dict(block_table=bt.reshape(-1)),
        dict(live_len=ll[:1]),
        dict(live_len=ll.to(torch.int64)),
        dict(k_scale=torch.ones(2)),
        dict(v_scale=ks.double()),
        dict(out=torch.zeros(1, 4, 4, 64, dtype=torch.float16)),
        dict(out=torch.zeros(2, 4, 4, 64, dtype=torch.float32)),
    ]
    for over in bad:
        with pytest.raises(ValueError) as e:
            pfs.verify(**{**a, **over})
        assert "GPU" not in str(e.value), over  # refused by its own check, not the device check
    other = pfs.make_plan(batch=1, q=4, num_q_heads=4, head_map=[0] * 4, k_pool=a["k_pool"], max_pages_per_row=4)
    with pytest.raises(ValueError, match="another shape"):
        pfs.verify(**a, plan=other)
    # every shape consistent, but host tensors: refused by the binding
    with pytest.raises(ValueError, match="GPU"):
        pfs.verify(**a)
    with pytest.raises(ValueError, match="GPU"):
        pfs.verify(**a, noalloc=True, out=torch.zeros_like(q))


def test_package_codec_calls_check_every_tensor_before_the_library():
    import torch

    import paged_fp8_split_amd as pfs

    a = _host_problem()
    kp, vp, bt, ll, ks, vs = (a[k] for k in ("k_pool", "v_pool", "block_table", "live_len", "k_scale", "v_scale"))
    for over in (dict(block_table=bt[:, :2].contiguous().to(torch.int64)), dict(live_len=ll[:1]),
                 dict(scale=torch.ones(3)), dict(out=torch.zeros(2, 32, 1, 64, dtype=torch.float16))):
        args = dict(block_table=bt, live_len=ll)
        args.update(over)
        with pytest.raises(ValueError) as e:
            pfs.dequant_paged(kp, **args)
        assert "GPU" not in str(e.value), over
    with pytest.raises(ValueError, match="GPU"):
        pfs.dequant_paged(kp, bt, ll, scale=ks, out=torch.zeros(2, 64, 1, 64, dtype=torch.float16))
    kn = torch.zeros(2, 4, 1, 64, dtype=torch.float16)
    for over in (dict(v_new=kn[:1]), dict(block_table=bt[:1]), dict(live_len=ll.to(torch.int64)),
                 dict(v_scale=torch.ones(2)), dict(v_pool=vp[:, :8]), dict(k_new=kn.reshape(2, 4, 64))):
        args = dict(k_new=kn, v_new=kn, k_scale=ks, v_scale=vs, block_table=bt, live_len=ll, k_pool=kp, v_pool=vp)
        args.update(over)
        with pytest.raises(ValueError) as e:
            pfs.kv_append(**args)
        assert "GPU" not in str(e.value), over
    with pytest.raises(ValueError, match="GPU"):
        pfs.kv_append(kn, kn, ks, vs, bt, ll, kp, vp)


def test_header_compiles_as_c99_and_a_c_client_runs(tmp_path):
    """include/pfs.h is plain C: a C99 client (tests/abi_c_client.c) compiles
    against it with every warning an error, links libpfs.so and plans a
    shape through the ABI with no Python in between."""
    import subprocess

    lib = _lib.LIB_PATH
    exe = str(tmp_path / "abi_c_client")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "abi_c_client.c"), "-o", exe, lib,
                    "-Wl,-rpath," + os.path.dirname(lib)], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "splits 128 tokens_per_split 2048 workspace 16908288" in res.stdout
    assert "token stride 264: a KV stride or a base pointer is not 16-byte aligned" in res.stdout


def test_oracle_and_product_share_no_code():
    """The oracle (oracle/) and the product (paged_fp8_split_amd/, include/)
    are independent: no product source imports, includes or loads anything
    from oracle/, the oracle imports nothing from the product, and their C
    and HIP sources include only system headers and their own files. The
    input generator (paged_fp8_split_amd/workloads.py) is the one module both
    sides may use; the oracle takes its workloads as plain objects."""
    import ast
    import glob

    def py_imports(path):
        mods = set()
        for node in ast.walk(ast.parse(open(path).read())):
            if isinstance(node, ast.Import):
                mods.update(a.name.split(".")[0] for a in node.names)
            elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
                mods.add(node.module.split(".")[0])
        return mods

    product_py = glob.glob(os.path.join(ROOT, "paged_fp8_split_amd", "*.py"))
    for f in product_py:
        assert "oracle" not in py_imports(f), f
        assert "liboracle" not in open(f).read(), f
    for f in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        assert "paged_fp8_split_amd" not in py_imports(f), f
    includes = re.compile(r'^\s*#\s*include\s*"([^"]+)"', re.M)
    for f in glob.glob(os.path.join(ROOT, "oracle", "*.c")) + glob.glob(os.path.join(ROOT, "oracle", "*.h")):
        assert includes.findall(open(f).read()) == [], f  # system headers only
    for f in glob.glob(os.path.join(ROOT, "paged_fp8_split_amd", "csrc", "*")):
        for inc in includes.findall(open(f).read()):
            assert "oracle" not in inc, (f, inc)
    for f in glob.glob(os.path.join(ROOT, "include", "*.h")):
        assert "oracle" not in open(f).read().lower(), f


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libpfs.so nothing runs: loading raises, and so does the package's
    verify (no fallback computes anything)."""
    import paged_fp8_split_amd as pfs

    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libpfs.so"))
    monkeypatch.setattr(pfs, "_plans", {})
    with pytest.raises(RuntimeError, match="is not built"):
        _lib.load()
    with pytest.raises(RuntimeError, match="is not built"):
        pfs.verify(**_host_problem())


def _plan_or_status(batch, q, hkv, G, D, page, ppr, pool, tps, fmt, mode, cus, pad, sm):
    hq = hkv * G
    token_stride = hkv * D + pad
    kw = dict(batch=batch, q=q, num_q_heads=hq, num_kv_heads=hkv, head_dim=D, page_size=page,
              max_pages_per_row=ppr, num_pool_pages=pool, kv_page_stride=page * token_stride,
              kv_token_stride=token_stride, kv_head_stride=D, sm_scale=sm,
              head_map=[h // G for h in range(hq)] if G > 0 else [], tokens_per_split=tps, kv_format=fmt,
              pv_mode=mode, num_cus=cus)
    try:
        return _lib.Plan(**kw), 0
    except _lib.PfsError as e:
        return None, e.status


def test_plan_create_on_random_problems():
    """pfs_plan_create on random problems, most of them invalid in some field:
    it always returns one of its status codes (no crash, no other value)."""
    from hypothesis import HealthCheck, given, settings
    from hypothesis import strategies as st

    codes = set(_lib.STATUS)

    @settings(max_examples=300, deadline=None, database=None, suppress_health_check=list(HealthCheck))
    @given(batch=st.integers(-2, 70000), q=st.integers(-1, 18), hkv=st.sampled_from([1, 2, 3, 4, 8, 16, 256, 257]),
           G=st.integers(0, 17), D=st.sampled_from([0, 32, 64, 96, 128, 256, 512]),
           page=st.sampled_from([0, 8, 16, 48, 64, 848, 3456]), ppr=st.integers(-1, 1 << 20),
           pool=st.integers(-1, 1 << 16), tps=st.sampled_from([0, 64, 100, 256, 2048, 16384, 16448]),
           fmt=st.integers(-1, 2), mode=st.integers(-1, 2), cus=st.integers(-1, 400),
           pad=st.sampled_from([0, 8, 16, 256]), sm=st.sampled_from([0.0, -1.0, 0.0625, float("inf"), float("nan")]))
    def check(**kw):
        plan, status = _plan_or_status(**kw)
        assert status in codes and (plan is not None) == (status == 0)

    check()


def test_plans_of_valid_problems_keep_their_invariants():
    """Problems drawn from the supported ranges: each is planned (or refused
    only because its split grid would pass 2^31 work-items), and every plan
    covers the capacity with whole 64-token partitions, keeps a split within
    the 1024-tile table, uses no empty trailing split, and sizes the
    workspace as (max, sum) pairs plus D accumulators per (split, request, KV
    head, row), each array 256-byte aligned."""
    from hypothesis import HealthCheck, given, settings
    from hypothesis import strategies as st

    accepted = []

    @settings(max_examples=300, deadline=None, database=None, suppress_health_check=list(HealthCheck))
    @given(batch=st.integers(0, 65535), q=st.integers(1, 16), hkv=st.sampled_from([1, 2, 4, 8]),
           G=st.integers(1, 16), D=st.sampled_from([64, 128, 256]), page=st.sampled_from([16, 64, 848, 3456]),
           ppr=st.integers(1, 4096), pool=st.integers(1, 65536), tps=st.sampled_from([0, 0, 0, 64, 256, 2048, 16384]),
           fmt=st.integers(0, 1), mode=st.integers(0, 1), cus=st.sampled_from([0, 40, 256, 304]),
           pad=st.sampled_from([0, 16, 256]), sm=st.just(0.0625))
    def check(batch, q, hkv, G, D, page, ppr, pool, tps, fmt, mode, cus, pad, sm):
        plan, status = _plan_or_status(batch, q, hkv, G, D, page, ppr, pool, tps, fmt, mode, cus, pad, sm)
        if plan is None:
            assert status == _lib.STATUS_CODE["PFS_ERR_SHAPE"]
            return
        accepted.append(1)
        cap = ppr * page
        assert p_ok(plan, cap)
        slots = plan.num_splits * max(batch, 1) * hkv * G * q
        rnd = lambda x: (x + 255) // 256 * 256  # noqa: E731
        assert plan.workspace_bytes == rnd(slots * 2 * 4) + rnd(slots * D * 4)

    def p_ok(plan, cap):
        t = plan.tokens_per_split
        return (t % 64 == 0 and 64 <= t <= 16384 and plan.num_splits >= 1 and plan.num_splits * t >= cap
                and (plan.num_splits - 1) * t < cap)

    check()
    assert len(accepted) >= 150, len(accepted)


def test_planner_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The host planner built with -fsanitize=address,undefined (g++, host
    code only) and driven by tests/plan_fuzz.cpp: random problems, the
    invariants of every accepted plan and the host-side error paths of the
    other calls, with no sanitizer report and no kernel launch reached."""
    import subprocess

    exe = str(tmp_path / "plan_fuzz")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "paged_fp8_split_amd", "csrc", "pfs_plan.cpp"),
                    os.path.join(ROOT, "tests", "plan_fuzz.cpp"), "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe, "30000"], capture_output=True, text=True, timeout=300, env=env)
    if "does not come first in initial library list" in res.stderr:
        pytest.skip("the environment preloads a library ahead of the AddressSanitizer runtime")
    assert res.returncode == 0, res.stdout + res.stderr
    m = re.search(r"plans (\d+) of 30000, launches 0", res.stdout)
    assert m and int(m.group(1)) > 1000, res.stdout
