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
    assert ctypes.sizeof(E.DosaStats) == 88
    assert ctypes.sizeof(E.DosaConfig) == 40


@pytest.mark.parametrize("dense", [True, False])
def test_workspace_size(dense):
    a = E.workspace_size([4096], [131072], 64, 128, 2048, "fp8", "fp8", False, dense)
    b = E.workspace_size([4096], [8192], 64, 128, 2048, "fp8", "fp8", False, dense)
    assert a > 0 and b > 0 and a >= b
    assert E.workspace_size([5], [3], 64, 128, 2048, "fp8", "fp8", False, dense) == 0      # q_len > kv_len
    assert E.workspace_size([5], [9], 48, 128, 2048, "fp8", "fp8", False, dense) == 0      # H unsupported
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
    (dict(H=48), -2),
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
