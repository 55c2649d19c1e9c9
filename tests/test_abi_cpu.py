"""CPU tests of the C-ABI library: it loads, exports every declared symbol, and
rejects bad arguments before touching a device (no compute call is made)."""
import ctypes
import os
import re

import pytest

import sparse_attention_indexer_fp32_amd as topk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("topk_transform.h", "indexer_topk.h")]


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:topk|indexer)_[a-z_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(topk.LIB_PATH):
        pytest.fail("libtopk_transform.so is not built (run __graft_entry__.build())")
    return topk.load()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert "topk_transform" in names and "indexer_topk" in names and len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(topk.EXPORTED)


def test_abi_version_and_status_strings(lib):
    assert topk.topk_abi_version() == 5
    for code, name in topk.STATUS.items():
        assert topk.topk_status_string(code) == name
    assert topk.topk_status_string(99) == "TOPK_UNKNOWN_STATUS"


@pytest.mark.parametrize("k,ps,batch,width,pages,expect", [
    (0, 64, 1, 16, 1, 1),          # k below range
    (2049, 64, 1, 16, 1, 1),       # k above range
    (16, 3, 1, 16, 1, 1),          # page size not a power of two
    (16, 0, 1, 16, 1, 1),
    (16, -64, 1, 16, 1, 1),
    (16, 64, -1, 16, 1, 1),        # negative batch
    (16, 64, 1, -5, 1, 1),         # negative width
    (16, 64, 1, 16, -1, 1),        # negative pages_per_row
    (16, 64, 1, 2**31, 1, 1),      # width beyond int32
    (16, 64, 0, 16, 1, 0),         # batch 0: no-op success
    (2048, 1, 0, 0, 0, 0),
    (16, 64, 3, 16, 1, 1),         # null pointers with batch > 0
])
@pytest.mark.parametrize("entry", ["topk_transform", "topk_transform_sorted"])
def test_argument_validation_without_device(lib, entry, k, ps, batch, width, pages, expect):
    st = getattr(lib, entry)(None, None, None, k, ps, None, None, None, batch, width, pages)
    assert st == expect, topk.topk_last_error()
    if expect:
        assert topk.topk_last_error()


def test_dispatch_override_validation(lib):
    assert lib.topk_set_dispatch_override(5, 0) == 1
    assert lib.topk_set_dispatch_override(4, -1) == 1
    assert lib.topk_set_dispatch_override(64, 3) == 0
    assert lib.topk_set_dispatch_override(0, 0) == 0


def test_stream_shape_validation(lib):
    """Every compiled streaming shape (0 .. STREAM_SHAPES - 1) is accepted; -1
    restores the automatic choice."""
    for shape in range(-1, topk.STREAM_SHAPES):
        assert lib.topk_set_stream_shape(shape) == 0
    assert lib.topk_set_stream_shape(topk.STREAM_SHAPES) == 1
    assert lib.topk_set_stream_shape(-2) == 1
    assert lib.topk_set_stream_shape(-1) == 0


def test_split_stream_override_validation(lib):
    for shape in range(topk.SPLIT_STREAM_SHAPES):
        assert lib.topk_set_split_stream(shape, 2) == 0
    assert lib.topk_set_split_stream(topk.SPLIT_STREAM_SHAPES, 2) == 1
    assert lib.topk_set_split_stream(0, 0) == 0     # the length-aware form
    assert lib.topk_set_split_stream(0, -1) == 1
    assert lib.topk_set_split_stream(-2, 0) == 1
    assert lib.topk_set_split_stream(-1, 0) == 0


def test_sorted_finish_override_validation(lib):
    """-1 (automatic), 0 (one workgroup per row) and 1 (rank finish) only."""
    for mode in (-1, 0, 1):
        assert lib.topk_set_sorted_finish(mode) == 0
    assert lib.topk_set_sorted_finish(2) == 1
    assert lib.topk_set_sorted_finish(-2) == 1
    assert lib.topk_set_sorted_finish(-1) == 0


def test_wait_limit_setter(lib):
    """The testing override of the split rows' wait limit takes any count; 0
    restores the default."""
    assert lib.topk_set_wait_limit(1) == 0
    assert lib.topk_set_wait_limit(0) == 0
    assert lib.topk_set_scratch_limit(1 << 20) == 0
    assert lib.topk_set_scratch_limit(0) == 0


def test_python_binding_rejects_bad_tensors():
    import torch
    s = torch.zeros((2, 8), dtype=torch.float32)
    with pytest.raises(ValueError):
        topk.topk_transform(s, torch.zeros(2, dtype=torch.int32), torch.zeros((2, 1), dtype=torch.int32), 4, 8)
    with pytest.raises(ValueError):
        topk.topk_transform(s.double(), torch.zeros(2, dtype=torch.int32), torch.zeros((2, 1), dtype=torch.int32),
                            4, 8)


def test_python_binding_rejects_strided_1d_inputs():
    """A strided 1-D view (a column of a 2-D tensor) would be read as dense
    int32 through its data pointer: the binding refuses it before any call."""
    import torch
    lens2d = torch.zeros((2, 3), dtype=torch.int32)
    with pytest.raises(ValueError, match="seq_lens"):
        topk._call(None, torch.zeros((2, 8)), lens2d[:, 0], torch.zeros((2, 1), dtype=torch.int32), 4, 8, None,
                   None, False, None)
    q = torch.zeros((2, 32, 128), dtype=torch.uint8)
    w = torch.zeros((2, 32), dtype=torch.float32)
    kv = torch.zeros((4, 128), dtype=torch.uint8)
    sc = torch.zeros((4,), dtype=torch.float32)
    ks = torch.zeros((2, 2), dtype=torch.int32)
    with pytest.raises(ValueError):
        topk._indexer_inputs(q, w, kv, sc, ks[:, 0], ks[:, 1])
    with pytest.raises(ValueError):
        topk._indexer_inputs(q, w, kv, torch.zeros((4, 2), dtype=torch.float32)[:, 0], ks[:, 0].contiguous(),
                             ks[:, 1].contiguous())



@pytest.mark.parametrize("k,num_q,num_kv,expect", [
    (0, 1, 16, 1),            # k below range
    (2049, 1, 16, 1),         # k above range
    (16, -1, 16, 1),          # negative rows
    (16, 1, -1, 1),           # negative key count
    (16, 1, 2**31, 1),        # key count beyond int32
    (16, 0, 16, 0),           # no rows: no-op success
    (16, 3, 16, 1),           # null pointers with rows
])
def test_indexer_topk_validation_without_device(lib, k, num_q, num_kv, expect):
    st = lib.indexer_topk(None, None, None, None, None, None, k, None, None, num_q, num_kv)
    assert st == expect, topk.topk_last_error()
    if expect:
        assert topk.topk_last_error()


@pytest.mark.parametrize("num_q,num_kv,stride,expect", [
    (-1, 16, 16, 1), (1, -1, 16, 1), (1, 16, -1, 1), (0, 16, 16, 0), (2, 16, 16, 1),
])
def test_indexer_logits_validation_without_device(lib, num_q, num_kv, stride, expect):
    st = lib.indexer_logits(None, None, None, None, None, None, None, None, num_q, num_kv, stride)
    assert st == expect, topk.topk_last_error()


def test_indexer_select_mode_validation(lib):
    for mode in (-1, 0, 1):
        assert lib.indexer_set_select_mode(mode) == 0
    assert lib.indexer_set_select_mode(2) == 1
    assert lib.indexer_set_select_mode(-2) == 1
    assert lib.indexer_set_select_mode(-1) == 0


def test_indexer_window_override_validation(lib):
    assert lib.indexer_set_window_override(33) == 1
    assert lib.indexer_set_window_override(96) == 1
    assert lib.indexer_set_window_override(-32) == 1
    assert lib.indexer_set_window_override(4096) == 0
    assert lib.indexer_set_window_override(0) == 0
