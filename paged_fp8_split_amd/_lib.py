"""ctypes binding of libpfs (include/pfs.h): argument marshalling only.

Every step of the verify attention runs in the HIP kernels of libpfs.so; this
module only turns torch tensors into pointers, sizes and the current HIP
stream. If the library is missing or was built against another ABI version,
loading fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpfs.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "pfs.h")


def _header_abi_version() -> int:
    with open(HEADER) as f:
        m = re.search(r"#define\s+PFS_ABI_VERSION\s+(\d+)", f.read())
    if not m:
        raise RuntimeError("PFS_ABI_VERSION not found in include/pfs.h")
    return int(m.group(1))


ABI_VERSION = _header_abi_version()

STATUS = {
    0: "PFS_OK",
    -1: "PFS_ERR_NULL",
    -2: "PFS_ERR_SHAPE",
    -3: "PFS_ERR_UNSUPPORTED",
    -4: "PFS_ERR_ALIGNMENT",
    -5: "PFS_ERR_HEAD_MAP",
    -6: "PFS_ERR_WORKSPACE",
    -7: "PFS_ERR_LAUNCH",
    -8: "PFS_ERR_NOMEM",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}


class PfsError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{what}: {self.name}" if what else self.name)


class PfsProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_row", ctypes.c_int32),
        ("num_pool_pages", ctypes.c_int32),
        ("partition_tokens", ctypes.c_int32),
        ("tokens_per_split", ctypes.c_int32),
        ("kv_format", ctypes.c_int32),
        ("pv_mode", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("kv_page_stride", ctypes.c_int64),
        ("kv_token_stride", ctypes.c_int64),
        ("kv_head_stride", ctypes.c_int64),
        ("sm_scale", ctypes.c_float),
        ("q_head_to_kv_head", ctypes.POINTER(ctypes.c_int32)),
    ]


_lib = None


def check_abi(lib) -> None:
    got = int(lib.pfs_abi_version())
    if got != ABI_VERSION:
        raise RuntimeError(
            f"libpfs ABI version {got} does not match include/pfs.h ({ABI_VERSION}); rebuild with "
            "`python -m paged_fp8_split_amd.build`"
        )


def load():
    """Load libpfs.so (once). Raises if it is missing or stale."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -m paged_fp8_split_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c = ctypes
    P = c.c_void_p
    lib.pfs_abi_version.restype = c.c_int32
    lib.pfs_abi_version.argtypes = []
    check_abi(lib)
    lib.pfs_status_string.restype = c.c_char_p
    lib.pfs_status_string.argtypes = [c.c_int32]
    lib.pfs_plan_create.restype = c.c_int32
    lib.pfs_plan_create.argtypes = [c.POINTER(PfsProblem), c.POINTER(P)]
    lib.pfs_plan_destroy.restype = None
    lib.pfs_plan_destroy.argtypes = [P]
    lib.pfs_plan_workspace_bytes.restype = c.c_int64
    lib.pfs_plan_workspace_bytes.argtypes = [P]
    lib.pfs_plan_num_splits.restype = c.c_int32
    lib.pfs_plan_num_splits.argtypes = [P]
    lib.pfs_plan_tokens_per_split.restype = c.c_int32
    lib.pfs_plan_tokens_per_split.argtypes = [P]
    lib.pfs_verify.restype = c.c_int32
    lib.pfs_verify.argtypes = [P] * 10 + [c.c_int64, P]
    lib.pfs_verify_split.restype = c.c_int32
    lib.pfs_verify_split.argtypes = [P] * 8 + [c.c_int64, P]
    lib.pfs_verify_combine.restype = c.c_int32
    lib.pfs_verify_combine.argtypes = [P] * 5 + [c.c_int64, P]
    lib.pfs_dequant_paged.restype = c.c_int32
    lib.pfs_dequant_paged.argtypes = [P] * 7
    lib.pfs_kv_append.restype = c.c_int32
    lib.pfs_kv_append.argtypes = [P] * 10
    lib.pfs_verify_noalloc.restype = c.c_int32
    lib.pfs_verify_noalloc.argtypes = [P] * 10
    lib.pfs_noalloc_scratch_bytes.restype = c.c_int64
    lib.pfs_noalloc_scratch_bytes.argtypes = []
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pfs_status_string(int(status)).decode()


class Plan:
    """A validated problem shape (pfs_plan_create). Immutable; host only."""

    def __init__(self, *, batch, q, num_q_heads, num_kv_heads, head_dim, page_size, max_pages_per_row,
                 num_pool_pages, kv_page_stride, kv_token_stride, kv_head_stride, sm_scale, head_map,
                 partition_tokens=64, tokens_per_split=0, kv_format=0, pv_mode=0, num_cus=0):
        lib = load()
        self._lib = lib
        self._handle = None
        hm = (ctypes.c_int32 * int(num_q_heads))(*[int(x) for x in head_map])
        self.problem = PfsProblem(int(batch), int(q), int(num_q_heads), int(num_kv_heads), int(head_dim),
                                  int(page_size), int(max_pages_per_row), int(num_pool_pages),
                                  int(partition_tokens), int(tokens_per_split), int(kv_format), int(pv_mode), int(num_cus),
                                  int(kv_page_stride),
                                  int(kv_token_stride), int(kv_head_stride), float(sm_scale),
                                  ctypes.cast(hm, ctypes.POINTER(ctypes.c_int32)))
        self._head_map = hm  # the problem struct points at it
        handle = ctypes.c_void_p()
        st = lib.pfs_plan_create(ctypes.byref(self.problem), ctypes.byref(handle))
        if st != 0:
            raise PfsError(st, "pfs_plan_create")
        self._handle = handle
        self.workspace_bytes = int(lib.pfs_plan_workspace_bytes(handle))
        self.num_splits = int(lib.pfs_plan_num_splits(handle))
        self.tokens_per_split = int(lib.pfs_plan_tokens_per_split(handle))
        self.capacity = int(max_pages_per_row) * int(page_size)
        self.kv_format = int(kv_format)
        self.pv_mode = int(pv_mode)
        self.num_cus = int(num_cus)

    @property
    def handle(self):
        return self._handle

    def __del__(self):
        if getattr(self, "_handle", None) is not None:
            self._lib.pfs_plan_destroy(self._handle)
            self._handle = None


def _stream_handle(device, stream) -> Optional[int]:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def _ptr(t) -> int:
    return t.data_ptr()


def verify(plan: Plan, q, k_pool, v_pool, k_scale, v_scale, block_table, live_len, out, workspace,
           stream=None) -> None:
    """pfs_verify on torch tensors already laid out as the plan expects."""
    lib = plan._lib
    st = lib.pfs_verify(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale), _ptr(v_scale),
                        _ptr(block_table), _ptr(live_len), _ptr(out), _ptr(workspace),
                        int(workspace.numel() * workspace.element_size()), _stream_handle(q.device, stream))
    if st != 0:
        raise PfsError(st, "pfs_verify")


def verify_noalloc(plan: Plan, q, k_pool, v_pool, k_scale, v_scale, block_table, live_len, out,
                   stream=None) -> None:
    """pfs_verify_noalloc: pfs_verify with the partials in the library's
    per-GPU device array (no workspace, nothing allocated)."""
    st = plan._lib.pfs_verify_noalloc(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                      _ptr(v_scale), _ptr(block_table), _ptr(live_len), _ptr(out),
                                      _stream_handle(q.device, stream))
    if st != 0:
        raise PfsError(st, "pfs_verify_noalloc")


def noalloc_scratch_bytes() -> int:
    return int(load().pfs_noalloc_scratch_bytes())


def verify_split(plan: Plan, q, k_pool, v_pool, k_scale, block_table, live_len, workspace, stream=None) -> None:
    """pfs_verify_split: the split kernel only (partials left in workspace)."""
    st = plan._lib.pfs_verify_split(plan.handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_scale),
                                    _ptr(block_table), _ptr(live_len), _ptr(workspace),
                                    int(workspace.numel() * workspace.element_size()),
                                    _stream_handle(q.device, stream))
    if st != 0:
        raise PfsError(st, "pfs_verify_split")


def verify_combine(plan: Plan, v_scale, live_len, out, workspace, stream=None) -> None:
    """pfs_verify_combine: the combine kernel only (reads the partials)."""
    st = plan._lib.pfs_verify_combine(plan.handle, _ptr(v_scale), _ptr(live_len), _ptr(out), _ptr(workspace),
                                      int(workspace.numel() * workspace.element_size()),
                                      _stream_handle(out.device, stream))
    if st != 0:
        raise PfsError(st, "pfs_verify_combine")


def dequant_paged(plan: Plan, pool, block_table, live_len, out, stream=None, scale=None) -> None:
    """pfs_dequant_paged: paged FP8 (the plan's KV format) -> dense FP16 [B, capacity, Hkv, D],
    times ``scale`` [Hkv] (float32 tensor) rounded once, or unscaled."""
    st = plan._lib.pfs_dequant_paged(plan.handle, _ptr(pool), None if scale is None else _ptr(scale),
                                     _ptr(block_table), _ptr(live_len), _ptr(out), _stream_handle(pool.device, stream))
    if st != 0:
        raise PfsError(st, "pfs_dequant_paged")


def kv_append(plan: Plan, k_new, v_new, k_scale, v_scale, block_table, live_len, k_pool, v_pool,
              stream=None) -> None:
    """pfs_kv_append: the draft tokens' FP16 K/V [B, q, Hkv, D] -> FP8 bytes (the plan's KV format) in the pools."""
    st = plan._lib.pfs_kv_append(plan.handle, _ptr(k_new), _ptr(v_new), _ptr(k_scale), _ptr(v_scale),
                                 _ptr(block_table), _ptr(live_len), _ptr(k_pool), _ptr(v_pool),
                                 _stream_handle(k_pool.device, stream))
    if st != 0:
        raise PfsError(st, "pfs_kv_append")
