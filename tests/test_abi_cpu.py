"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching the GPU (CPU only: no compute calls)."""

import ctypes
import os
import re

import pytest

from tests._helpers import ensure_library

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "xqa.h")


@pytest.fixture(scope="module")
def lib():
    return ensure_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(xqa_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("xqa_create", "xqa_decode", "xqa_destroy"):
        assert must in names
    from decode_attention_paged_e5m2_amd._lib import EXPORTED
    assert sorted(EXPORTED) == names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    names = [lib.xqa_status_string(i).decode() for i in range(5)]
    assert names == ["XQA_OK", "XQA_ERR_INVALID_ARG", "XQA_ERR_UNSUPPORTED",
                     "XQA_ERR_OUT_OF_MEMORY", "XQA_ERR_HIP"]


def _cfg(**over):
    from decode_attention_paged_e5m2_amd._lib import XqaConfig
    d = dict(max_batch=16, num_q_heads=32, num_kv_heads=4, head_dim=128, page_size=16,
             max_pages_per_seq=64, max_work_items=0)
    d.update(over)
    return XqaConfig(**d)


@pytest.mark.parametrize("over,status", [
    (dict(head_dim=64), 2), (dict(page_size=32), 2), (dict(num_q_heads=30), 2),
    (dict(num_q_heads=68, num_kv_heads=4), 2), (dict(max_batch=0), 1),
    (dict(max_pages_per_seq=0), 1), (dict(max_work_items=3), 1), (dict(max_work_items=9000), 1),
    (dict(max_batch=70000), 2), (dict(max_pages_per_seq=(1 << 20) + 1), 2),
    (dict(max_query_tokens=-1), 1), (dict(max_query_tokens=3), 2),
    (dict(num_q_heads=4, num_kv_heads=4, max_query_tokens=17), 2),
    (dict(max_selected_pages=-1), 1), (dict(max_selected_pages=65), 2),
])
def test_create_rejects_bad_configs_before_hip(lib, over, status):
    h = ctypes.c_void_p()
    assert lib.xqa_create(ctypes.byref(_cfg(**over)), ctypes.byref(h)) == status
    assert h.value is None
    assert lib.xqa_last_error().decode() != ""


def test_null_arguments_are_rejected(lib):
    h = ctypes.c_void_p()
    assert lib.xqa_create(None, ctypes.byref(h)) == 1
    assert lib.xqa_create(ctypes.byref(_cfg()), None) == 1
    null = ctypes.c_void_p()
    args = [null] * 6 + [1, ctypes.c_float(0.1), null, null]
    assert lib.xqa_decode(*args) == 1
    assert lib.xqa_decode_split(*args) == 1
    assert lib.xqa_decode_multi(*args[:7], 2, *args[7:]) == 1
    assert lib.xqa_decode_fp8(null, 1, *args[1:7], 1, ctypes.c_float(0.1), ctypes.c_float(1.0),
                              ctypes.c_float(1.0), null, null) == 1
    assert lib.xqa_debug_widen_e4m3(null, null, null, 4, null) == 1
    assert lib.xqa_decode_append(null, null, null, null, null, null, null, null, 1,
                                 ctypes.c_float(0.1), null, null) == 1
    assert lib.xqa_decode_combine(null, null, 1, null, null) == 1
    assert lib.xqa_append_kv(null, null, null, null, null, 1, null, null, null) == 1
    assert lib.xqa_decode_pages(*args[:6], null, null, 1, 1, ctypes.c_float(0.1), null, null) == 1
    assert lib.xqa_get_info(null, None) == 1
    assert lib.xqa_destroy(null) == 0
    assert lib.xqa_debug_widen_e5m2(null, null, null, 4, null) == 1


def test_create_without_gpu_reports_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    assert lib.xqa_create(ctypes.byref(_cfg()), ctypes.byref(h)) == 4
    assert h.value is None


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(os.path.dirname(HEADER), "..", "decode_attention_paged_e5m2_amd")
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(root, f)).read()
                assert "oracle" not in re.sub(r"#.*|//.*", "", text).replace("oracle is", ""), f


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # Without the built library the product raises; there is no CPU path.
    from decode_attention_paged_e5m2_amd import _lib, Xqa
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libxqa.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="is missing"):
        _lib.load()
    with pytest.raises(RuntimeError, match="is missing"):
        Xqa(max_batch=1, num_q_heads=8, num_kv_heads=1, max_pages_per_seq=16)
