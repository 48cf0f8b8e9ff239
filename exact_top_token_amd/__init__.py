"""Python binding of libdosa_indexer.so (exact Top-K for the DSA indexer on MI355X).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch provides device memory and the stream.  The
functions mirror the C entry points of include/dosa_indexer.h:

    dosa_indexer_topk   certificate-pruned exact Top-K (seed -> plan -> bound
                        -> compaction -> survivor scoring -> select)
    dsa_indexer_topk    dense scoring of every visible key + streaming Top-K
    workspace_size, default_config, status_string

Importing the package never falls back to anything: if the shared library is
missing, :func:`lib` raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdosa_indexer.so")

DTYPES = {"f32": 0, "bf16": 1, "fp8": 2}

DOSA_NO_PRUNE = 0x1
DOSA_SORTED = 0x2
DOSA_SEPARABLE_RHO = 0x4
DOSA_NO_NEGATIVE = 0x8
DOSA_NO_PROBE = 0x10
DOSA_KEY_BLOCKS = 0x20
DOSA_TWO_ROUNDS = 0x40
DOSA_GROUP_LISTS = 0x80

STATUS = {0: "DOSA_OK", -1: "DOSA_ERR_INVALID_ARG", -2: "DOSA_ERR_UNSUPPORTED", -3: "DOSA_ERR_WORKSPACE",
          -4: "DOSA_ERR_HIP"}

EXPORTS = ("dosa_default_config", "dosa_workspace_size", "dosa_indexer_topk", "dsa_indexer_topk",
           "dosa_indexer_topk_noalloc", "dosa_status_string", "dosa_version", "dosa_profile_begin",
           "dosa_profile_end")

NOALLOC_SCRATCH_BYTES = 128 << 20   # DOSA_NOALLOC_SCRATCH_BYTES


class DosaConfig(ctypes.Structure):
    _fields_ = [
        ("num_proxies", ctypes.c_int32),
        ("seed_window", ctypes.c_int32),
        ("seed_prefix", ctypes.c_int32),
        ("buffer_cap", ctypes.c_int32),
        ("key_splits", ctypes.c_int32),
        ("neg_support_frac", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("debug_ub", ctypes.c_void_p),
        ("debug_tau", ctypes.c_void_p),
        ("debug_mask", ctypes.c_void_p),
        ("seed_idx", ctypes.c_void_p),
        ("seed_count", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class DosaStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "pairs_total", "pairs_seed", "pairs_bounded", "pairs_survived", "pairs_scored",
        "candidates_written", "reselects", "groups_skipped", "pairs_scored_list", "keys_streamed",
        "calls_unpruned", "key_blocks_skipped")]


STAT_FIELDS = [f[0] for f in DosaStats._fields_]


class DosaKernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


class DosaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def hip_runtimes_mapped() -> list:
    """Paths of the HIP runtime libraries mapped into this process (Linux)."""
    paths = set()
    try:
        with open("/proc/self/maps") as fh:
            for line in fh:
                parts = line.split()
                if len(parts) >= 6 and os.path.basename(parts[5]).startswith("libamdhip64.so"):
                    paths.add(os.path.realpath(parts[5]))
    except OSError:
        pass
    return sorted(paths)


def lib():
    """The loaded shared library (raises if it has not been built).

    PyTorch ships its own HIP runtime under the same soname as the system one
    the library is linked against.  torch is imported first, so the dynamic
    loader binds the library to the runtime torch already mapped: one HIP (and
    HSA) runtime per process, and torch's streams and device pointers are
    valid in the library's calls.  Loading fails if two runtimes are mapped.
    """
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m exact_top_token_amd.build`")
        import torch  # noqa: F401  (maps torch's HIP runtime before the library's dependency is resolved)

        L = ctypes.CDLL(LIB_PATH)
        rt = hip_runtimes_mapped()
        if len(rt) > 1:
            raise RuntimeError(f"two HIP runtimes are mapped into this process: {rt}")
        vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        L.dosa_default_config.argtypes = [i32, ctypes.POINTER(DosaConfig)]
        L.dosa_default_config.restype = ctypes.c_int
        L.dosa_workspace_size.argtypes = [i32, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                          ctypes.POINTER(DosaConfig)]
        L.dosa_workspace_size.restype = sz
        common = [vp, i32, vp, vp, vp, i32, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, vp, vp, vp, sz]
        L.dosa_indexer_topk.argtypes = common + [ctypes.POINTER(DosaConfig), vp, vp]
        L.dosa_indexer_topk.restype = ctypes.c_int
        L.dsa_indexer_topk.argtypes = common + [ctypes.POINTER(DosaConfig), vp, vp]
        L.dsa_indexer_topk.restype = ctypes.c_int
        L.dosa_indexer_topk_noalloc.argtypes = common[:-2] + [ctypes.POINTER(DosaConfig), vp, vp]
        L.dosa_indexer_topk_noalloc.restype = ctypes.c_int
        L.dosa_status_string.argtypes = [ctypes.c_int]
        L.dosa_status_string.restype = ctypes.c_char_p
        L.dosa_version.argtypes = []
        L.dosa_version.restype = ctypes.c_char_p
        L.dosa_profile_begin.argtypes = []
        L.dosa_profile_begin.restype = ctypes.c_int
        L.dosa_profile_end.argtypes = [ctypes.POINTER(DosaKernelTime), i32]
        L.dosa_profile_end.restype = ctypes.c_int
        _lib = L
    return _lib


def profile_begin() -> None:
    """Start bracketing every kernel this thread enqueues with HIP events."""
    lib().dosa_profile_begin()


def profile_end() -> dict:
    """Wait for the recorded events; {pass name: (launches, total ms)}."""
    buf = (DosaKernelTime * 32)()
    n = lib().dosa_profile_end(buf, 32)
    if n < 0:
        raise DosaError(n, status_string(n))
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(n)}


def status_string(status: int) -> str:
    return lib().dosa_status_string(int(status)).decode()


def version() -> str:
    return lib().dosa_version().decode()


def default_config(topk: int) -> DosaConfig:
    c = DosaConfig()
    lib().dosa_default_config(int(topk), ctypes.byref(c))
    return c


def _i32_array(v: Sequence[int]):
    arr = (ctypes.c_int32 * max(len(v), 1))(*[int(x) for x in v])
    return arr


def workspace_size(q_lens, kv_lens, H: int, d: int, topk: int, q_dtype: str, k_dtype: str,
                   paged: bool, dense: bool, cfg: Optional[DosaConfig] = None) -> int:
    ql, kl = _i32_array(q_lens), _i32_array(kv_lens)
    return int(lib().dosa_workspace_size(len(q_lens), ql, kl, H, d, topk, DTYPES[q_dtype], DTYPES[k_dtype],
                                         int(bool(paged)), int(bool(dense)),
                                         ctypes.byref(cfg) if cfg is not None else None))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch

        if not torch.cuda.is_available():
            return None
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


def _call(fn, tail, q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_lens, kv_lens, page_table, page_size,
          H, d, topk, out_idx, out_score, workspace):
    ql, kl = _i32_array(q_lens), _i32_array(kv_lens)
    max_pages = int(page_table.shape[1]) if page_table is not None else 0
    ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    st = fn(_ptr(q), DTYPES[q_dtype], _ptr(q_scale), _ptr(w), _ptr(k), DTYPES[k_dtype], _ptr(k_scale),
            ql, kl, len(q_lens), _ptr(page_table), int(page_size), max_pages, int(H), int(d), int(topk),
            _ptr(out_idx), _ptr(out_score), _ptr(workspace), ws_bytes, *tail)
    if st != 0:
        raise DosaError(st, status_string(st))
    return st


def dosa_indexer_topk(q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_lens, kv_lens, page_table, page_size,
                      H, d, topk, out_idx, out_score, workspace, cfg: Optional[DosaConfig] = None,
                      stats=None, stream=None):
    """Certificate-pruned exact Top-K (see include/dosa_indexer.h).  Tensors are device tensors."""
    tail = [ctypes.byref(cfg) if cfg is not None else None, _ptr(stats), _stream(stream)]
    return _call(lib().dosa_indexer_topk, tail, q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_lens, kv_lens,
                 page_table, page_size, H, d, topk, out_idx, out_score, workspace)


def dsa_indexer_topk(q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_lens, kv_lens, page_table, page_size,
                     H, d, topk, out_idx, out_score, workspace, cfg: Optional[DosaConfig] = None,
                     stats=None, stream=None):
    """Dense scoring of every visible key with streaming exact Top-K (uses cfg's
    buffer_cap, key_splits and DOSA_SORTED)."""
    tail = [ctypes.byref(cfg) if cfg is not None else None, _ptr(stats), _stream(stream)]
    return _call(lib().dsa_indexer_topk, tail, q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_lens, kv_lens,
                 page_table, page_size, H, d, topk, out_idx, out_score, workspace)


def dosa_indexer_topk_noalloc(q, q_dtype, q_scale, w, k, k_dtype, k_scale, q_lens, kv_lens, page_table,
                              page_size, H, d, topk, out_idx, out_score, cfg: Optional[DosaConfig] = None,
                              stats=None, stream=None):
    """dosa_indexer_topk in the library's own scratch memory (no workspace argument, nothing
    allocated; calls that need more than NOALLOC_SCRATCH_BYTES are rejected)."""
    ql, kl = _i32_array(q_lens), _i32_array(kv_lens)
    max_pages = int(page_table.shape[1]) if page_table is not None else 0
    st = lib().dosa_indexer_topk_noalloc(
        _ptr(q), DTYPES[q_dtype], _ptr(q_scale), _ptr(w), _ptr(k), DTYPES[k_dtype], _ptr(k_scale), ql, kl,
        len(q_lens), _ptr(page_table), int(page_size), max_pages, int(H), int(d), int(topk), _ptr(out_idx),
        _ptr(out_score), ctypes.byref(cfg) if cfg is not None else None, _ptr(stats), _stream(stream))
    if st != 0:
        raise DosaError(st, status_string(st))
    return st
