"""The C ABI without a GPU: the library loads, exports what the header declares,
and rejects bad configurations before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

import tree_attention_verification_verify_amd as sva
from tree_attention_verification_verify_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(spec_verify_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = sva.load_library()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", sva.LIB_PATH], capture_output=True, text=True).stdout
    for name in _declared():
        assert re.search(r"\bT %s$" % name, out, re.M), name


def test_struct_layouts_match_the_header():
    # the C structs are plain 4-byte fields / pointers: sizes follow from the field lists
    assert ctypes.sizeof(binding.Config) == 13 * 4
    assert ctypes.sizeof(binding.Inputs) == 10 * 8 + 2 * 4
    assert ctypes.sizeof(binding.Outputs) == 11 * 8
    assert ctypes.sizeof(binding.CommitArgs) == 6 * 8 + 2 * 4
    assert ctypes.sizeof(binding.PagedKV) == 3 * 8 + 3 * 4 + 4   # padded to pointer alignment


GOOD = dict(max_batch=2, max_nodes=8, num_q_heads=8, num_kv_heads=2, head_dim=128, kv_capacity=256,
            vocab=1000, dtype="bf16", mode="sampling", temperature=1.0, top_p=1.0)


@pytest.mark.parametrize("field,value,code", [
    ("max_batch", 0, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("max_nodes", 65, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("max_nodes", 0, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("num_kv_heads", 3, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("head_dim", 96, binding.SPEC_VERIFY_ERR_UNSUPPORTED),
    ("kv_capacity", 4, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("vocab", 0, binding.SPEC_VERIFY_ERR_UNSUPPORTED),
    ("temperature", 0.0, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("temperature", float("nan"), binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("top_p", 0.0, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("top_p", 1.5, binding.SPEC_VERIFY_ERR_INVALID_ARG),
])
def test_create_rejects_bad_config(field, value, code):
    cfg = dict(GOOD)
    cfg[field] = value
    with pytest.raises(sva.SpecVerifyError) as e:
        sva.spec_verify_create(sva.make_config(**cfg))
    assert e.value.code == code
    assert sva.spec_verify_last_error()


def test_create_rejects_top_p_on_huge_vocab():
    cfg = dict(GOOD, vocab=128256, top_p=0.9)
    with pytest.raises(sva.SpecVerifyError) as e:
        sva.spec_verify_create(sva.make_config(**cfg))
    assert e.value.code == binding.SPEC_VERIFY_ERR_UNSUPPORTED


def test_create_rejects_lossless_tree_in_greedy_mode_and_unknown_flags():
    with pytest.raises(sva.SpecVerifyError) as e:
        sva.spec_verify_create(sva.make_config(**dict(GOOD, mode="greedy"), lossless_tree=True))
    assert e.value.code == binding.SPEC_VERIFY_ERR_INVALID_ARG
    cfg = sva.make_config(**GOOD)
    cfg.flags = 0x80
    with pytest.raises(sva.SpecVerifyError) as e:
        sva.spec_verify_create(cfg)
    assert e.value.code == binding.SPEC_VERIFY_ERR_INVALID_ARG


def test_null_arguments():
    lib = sva.load_library()
    assert lib.spec_verify_create(None, None) == binding.SPEC_VERIFY_ERR_INVALID_ARG
    assert lib.spec_verify_run(None, None, None, None) == binding.SPEC_VERIFY_ERR_INVALID_ARG
    assert lib.spec_verify_destroy(None) == binding.SPEC_VERIFY_ERR_INVALID_ARG
    assert lib.spec_verify_commit(None, None, None) == binding.SPEC_VERIFY_ERR_INVALID_ARG
    assert lib.spec_verify_run_paged(None, None, None, None, None) == binding.SPEC_VERIFY_ERR_INVALID_ARG
    assert lib.spec_verify_commit_paged(None, None, None, None) == binding.SPEC_VERIFY_ERR_INVALID_ARG
    ms = (ctypes.c_float * 4)()
    n = ctypes.c_int32()
    assert lib.spec_verify_timing_read(None, ms, ctypes.byref(n)) == binding.SPEC_VERIFY_ERR_INVALID_ARG
