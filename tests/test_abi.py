"""The C-ABI library: it loads, exports every declared entry point, and its
argument checks reject bad calls before anything touches a GPU."""
import ctypes
import os
import re

import pytest

import exact_top_token_amd as E

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dosa_indexer.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(dosa_[a-z_]+|dsa_[a-z_]+)\s*\(",
                                 text, flags=re.M)))


def test_library_loads_and_exports_all_declared_symbols():
    L = E.lib()
    names = declared_functions()
    assert set(names) == set(E.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    assert "gfx950" in E.version()


def test_default_config_values():
    c = E.default_config(2048)
    assert (c.num_proxies, c.seed_window, c.seed_prefix, c.buffer_cap) == (3, 8192, 64, 0)
    assert E.default_config(8).seed_window == 64
    assert abs(c.neg_support_frac - 0.5) < 1e-7 and c.flags == 0


def test_struct_layout_matches_header():
    assert ctypes.sizeof(E.DosaStats) == 96
    assert ctypes.sizeof(E.DosaConfig) == 72
    assert E.DosaConfig.debug_mask.offset == 48
    assert E.DosaConfig.seed_idx.offset == 56 and E.DosaConfig.seed_count.offset == 64


def test_seed_config_checks():
    """Extra seed keys: seed_count in 0..4096 with a pointer when positive; a call with seeds
    needs a little more workspace (the groups' union lists and their regions); the dense path
    ignores them."""
    c = E.default_config(2048)
    args = ([2] * 64, [200000] * 64, 64, 128, 2048, "bf16", "fp8", True)
    base = E.workspace_size(*args, False, c)
    c.seed_idx, c.seed_count = 0x1000, 2048
    with_seeds = E.workspace_size(*args, False, c)
    assert with_seeds > base
    assert E.workspace_size(*args, True, c) == E.workspace_size(*args, True, E.default_config(2048))
    c.seed_count = 4097
    assert E.workspace_size(*args, False, c) == 0
    c.seed_count, c.seed_idx = 16, None
    assert E.workspace_size(*args, False, c) == 0
    c.seed_count = -1
    assert E.workspace_size(*args, False, c) == 0
    for cnt, ptr in ((4097, 0x1000), (8, None), (-2, 0x1000)):
        c = E.default_config(16)
        c.seed_idx, c.seed_count = ptr, cnt
        with pytest.raises(E.DosaError) as ei:
            E.dosa_indexer_topk(_Fake(), "fp8", _Fake(), _Fake(), _Fake(), "fp8", _Fake(), [4], [64], None, 0, 64,
                                128, 16, _Fake(), None, _Fake(), cfg=c, stream=0)
        assert ei.value.status == -1


def test_one_hip_runtime_when_the_library_loads_first():
    """A fresh process that loads the library before anything else maps exactly one HIP runtime
    (the one torch brings), so torch's streams and pointers are valid in library calls."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import exact_top_token_amd as E; E.lib(); import torch; "
            "rt = E.hip_runtimes_mapped(); print(len(rt)); assert len(rt) == 1, rt")
    r = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "1"


@pytest.mark.parametrize("q_len,kv_len", [(65536, 1200000), (32768, 2200000)])
def test_workspace_beyond_int32_list_offsets(q_len, kv_len):
    """Shapes whose survivor lists hold more than 2^31 entries (one list area of a tile's bounded
    keys per 32-query tile) are planned with 64-bit list offsets: the workspace covers them."""
    n = E.workspace_size([q_len], [kv_len], 64, 128, 2048, "fp8", "fp8", False, False)
    tiles = q_len // 32
    bounded = kv_len - q_len - 4 * 2048           # keys before the seed window of a tile, at least
    assert tiles * bounded > 2 ** 31
    assert n >= 4 * tiles * bounded


def test_workspace_of_long_chunks_fits_hbm():
    """The 1M-key context with 32K-query chunks: the pruned path's workspace stays a small part of
    the 288 GB of one MI355X (one list area per query tile)."""
    n = E.workspace_size([32768], [1048576], 64, 128, 2048, "fp8", "fp8", False, False)
    assert 0 < n < 20 * 2 ** 30


@pytest.mark.parametrize("H", [8, 24, 40, 48, 56, 64])
def test_head_counts_multiple_of_eight(H):
    assert E.workspace_size([5], [9], H, 128, 16, "bf16", "bf16", False, False) > 0
    assert E.workspace_size([5], [9], H, 64, 16, "f32", "f32", False, True) > 0


def test_32bit_index_limits():
    # a contiguous f32 sequence of 2^23 keys of 128 floats spans 2^32 bytes
    assert E.workspace_size([1], [1 << 23], 8, 128, 16, "f32", "f32", False, True) == 0
    assert E.workspace_size([1], [(1 << 23) - 1], 8, 128, 16, "f32", "f32", False, True) > 0
    assert E.workspace_size([1, 1], [1 << 30, 1 << 30], 8, 64, 16, "fp8", "fp8", False, True) == 0


@pytest.mark.parametrize("dense", [True, False])
def test_workspace_size(dense):
    a = E.workspace_size([4096], [131072], 64, 128, 2048, "fp8", "fp8", False, dense)
    b = E.workspace_size([4096], [8192], 64, 128, 2048, "fp8", "fp8", False, dense)
    assert a > 0 and b > 0 and a >= b
    assert E.workspace_size([5], [3], 64, 128, 2048, "fp8", "fp8", False, dense) == 0      # q_len > kv_len
    assert E.workspace_size([5], [9], 44, 128, 2048, "fp8", "fp8", False, dense) == 0      # H not a multiple of 8
    assert E.workspace_size([5], [9], 72, 128, 2048, "fp8", "fp8", False, dense) == 0      # H above 64
    assert E.workspace_size([5], [9], 64, 96, 2048, "fp8", "fp8", False, dense) == 0       # d unsupported
    assert E.workspace_size([5], [9], 64, 128, 5000, "fp8", "fp8", False, dense) == 0      # topk too large
    assert E.workspace_size([5], [9], 64, 128, 64, "fp8", "bf16", False, dense) == 0       # dtype combo


class _Fake:
    """Stands in for a device tensor: only data_ptr / numel / element_size are used."""

    def __init__(self, n=1 << 20, ptr=0x1000):
        self._n, self._p = n, ptr
        self.shape = (1, 1)

    def data_ptr(self):
        return self._p

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def _call(path, **over):
    f = _Fake()
    args = dict(q=f, q_dtype="fp8", q_scale=f, w=f, k=f, k_dtype="fp8", k_scale=f, q_lens=[4], kv_lens=[64],
                page_table=None, page_size=0, H=64, d=128, topk=16, out_idx=f, out_score=None, workspace=f)
    args.update(over)
    fn = E.dosa_indexer_topk if path == "dosa" else E.dsa_indexer_topk
    return fn(**args, stream=0)


@pytest.mark.parametrize("path", ["dosa", "dsa"])
@pytest.mark.parametrize("over,status", [
    (dict(q_lens=[5], kv_lens=[3]), -1),
    (dict(topk=0), -1),
    (dict(H=0), -1),
    (dict(H=44), -2),
    (dict(H=72), -2),
    (dict(d=96), -2),
    (dict(topk=4097), -2),
    (dict(q_dtype="fp8", k_dtype="bf16"), -2),
    (dict(q=None), -1),
    (dict(out_idx=None), -1),
    (dict(q_scale=None), -1),
    (dict(k_scale=None), -1),
    (dict(workspace=None), -3),
    (dict(workspace=_Fake(n=16)), -3),
])
def test_error_paths(path, over, status):
    with pytest.raises(E.DosaError) as ei:
        _call(path, **over)
    assert ei.value.status == status
    assert len(E.status_string(status)) > 0


def test_bad_config_rejected():
    c = E.default_config(16)
    c.num_proxies = 9
    with pytest.raises(E.DosaError) as ei:
        _call("dosa", **{}) if False else E.dosa_indexer_topk(
            _Fake(), "fp8", _Fake(), _Fake(), _Fake(), "fp8", _Fake(), [4], [64], None, 0, 64, 128, 16,
            _Fake(), None, _Fake(), cfg=c, stream=0)
    assert ei.value.status == -1
    c = E.default_config(16)
    c.buffer_cap = 20
    with pytest.raises(E.DosaError):
        E.dosa_indexer_topk(_Fake(), "fp8", _Fake(), _Fake(), _Fake(), "fp8", _Fake(), [4], [64], None, 0, 64,
                            128, 16, _Fake(), None, _Fake(), cfg=c, stream=0)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(E, "_lib", None)
    monkeypatch.setattr(E, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError):
        E.lib()
