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
    assert ctypes.sizeof(binding.Outputs) == 12 * 8
    assert ctypes.sizeof(binding.CommitArgs) == 6 * 8 + 2 * 4
    assert ctypes.sizeof(binding.PagedKV) == 3 * 8 + 3 * 4 + 4   # padded to pointer alignment
    assert ctypes.sizeof(binding.TreeArgs) == 6 * 8 + 3 * 4 + 4


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
    ("vocab", 4194305, binding.SPEC_VERIFY_ERR_UNSUPPORTED),
    ("temperature", 0.0, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("temperature", float("nan"), binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("top_p", 0.0, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    ("top_p", 1.5, binding.SPEC_VERIFY_ERR_INVALID_ARG),
    # one (sequence, KV head) slice of the cache must stay below 2 GiB
    ("kv_capacity", (1 << 30) // 128, binding.SPEC_VERIFY_ERR_UNSUPPORTED),
])
def test_create_rejects_bad_config(field, value, code):
    cfg = dict(GOOD)
    cfg[field] = value
    with pytest.raises(sva.SpecVerifyError) as e:
        sva.spec_verify_create(sva.make_config(**cfg))
    assert e.value.code == code
    assert sva.spec_verify_last_error()


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
    assert lib.spec_verify_build_tree(None, None, None) == binding.SPEC_VERIFY_ERR_INVALID_ARG
    assert lib.spec_verify_tree_template(None, 1, 1, None, None) == binding.SPEC_VERIFY_ERR_INVALID_ARG
    assert lib.spec_verify_describe(None, 1, 1, None, 0) == binding.SPEC_VERIFY_ERR_INVALID_ARG
    ms = (ctypes.c_float * 4)()
    n = ctypes.c_int32()
    assert lib.spec_verify_timing_read(None, ms, ctypes.byref(n)) == binding.SPEC_VERIFY_ERR_INVALID_ARG


# ------------------------------------------------------------------ host-only tree template

@pytest.mark.parametrize("caps,nodes", [((2, 2), 7), ((10, 4, 2, 1, 1), 64), ((10, 4, 2, 1), 26), ((3, 3, 3), 40),
                                        ((5, 5), 31), ((1, 1, 1, 1), 5), ((64,), 64), ((2,) * 6, 64),
                                        ((7, 3), 1), ((4, 4, 4), 2)])
def test_tree_template_matches_the_oracle(caps, nodes):
    import oracle

    par, rank = sva.spec_verify_tree_template(caps, nodes)
    opar, orank = oracle.tree_template(caps, nodes)
    assert par == [int(x) for x in opar]
    assert rank == [int(x) for x in orank]


def test_tree_template_huge_caps_stay_cheap():
    import oracle

    # every all-zero tuple has product 1: with 63 levels the 63 kept tuples are one chain
    par, rank = sva.spec_verify_tree_template([1 << 30] * 63, 64)
    assert par == [-1] + list(range(63)) and rank == [0] * 64
    # two levels: a kept rank is at most 62, so caps of 64 keep the same tuples
    par, rank = sva.spec_verify_tree_template([1 << 30] * 2, 64)
    opar, orank = oracle.tree_template([64, 64], 64)
    assert par == [int(x) for x in opar] and rank == [int(x) for x in orank]


@pytest.mark.parametrize("caps,nodes", [((2, 2), 8), ((0, 2), 2), ((), 1), ((3,), 0), ((3,), 65)])
def test_tree_template_rejects_bad_arguments(caps, nodes):
    with pytest.raises(sva.SpecVerifyError) as e:
        sva.spec_verify_tree_template(caps, nodes)
    assert e.value.code == binding.SPEC_VERIFY_ERR_INVALID_ARG


def test_paged_kv_keeps_its_tensors_alive():
    """The PagedKV struct carries raw addresses; the tensors behind them must live
    as long as it does (pools built from temporaries were freed while in use)."""
    import gc
    import weakref

    import torch

    k = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    t = torch.zeros((1, 4), dtype=torch.int32)
    refs = [weakref.ref(x) for x in (k, v, t)]
    pk = binding.paged_kv(k, v, t)
    assert (pk.k_pool, pk.v_pool, pk.block_table) == (k.data_ptr(), v.data_ptr(), t.data_ptr())
    assert (pk.num_blocks, pk.block_size, pk.table_width) == (4, 16, 4)
    del k, v, t
    gc.collect()
    assert all(r() is not None for r in refs)
    del pk
    gc.collect()
    assert all(r() is None for r in refs)


def test_create_bounds_the_cache_slice_below_two_gib():
    # bf16, D = 128: 8388607 slots (2^31 - 256 bytes) are not refused for size;
    # 8388608 slots (2^31 bytes) are
    cfg = dict(GOOD, kv_capacity=(1 << 23))
    with pytest.raises(sva.SpecVerifyError) as e:
        sva.spec_verify_create(sva.make_config(**cfg))
    assert e.value.code == binding.SPEC_VERIFY_ERR_UNSUPPORTED and "2^31" in str(e.value)
    cfg = dict(GOOD, kv_capacity=(1 << 22), dtype="f32")        # fp32: 4 bytes per element
    with pytest.raises(sva.SpecVerifyError) as e:
        sva.spec_verify_create(sva.make_config(**cfg))
    assert e.value.code == binding.SPEC_VERIFY_ERR_UNSUPPORTED


@pytest.mark.parametrize("flags,msg", [
    (dict(skip_attention=True, skip_vocab=True), "nothing to run"),
    (dict(write_probs=True, mode="greedy"), "sampling"),
    (dict(write_probs=True, skip_vocab=True), "vocabulary pass"),
    (dict(walk_no_wait=True), "LOSSLESS"),
])
def test_create_rejects_conflicting_flags(flags, msg):
    cfg = dict(GOOD)
    cfg.update(flags)
    with pytest.raises(sva.SpecVerifyError) as e:
        sva.spec_verify_create(sva.make_config(**cfg))
    assert e.value.code == binding.SPEC_VERIFY_ERR_INVALID_ARG and msg in str(e.value)


# ------------------------------------------------------------------ binding argument checks (no GPU)

def _cpu_args(cfg, B=2, T=5, probs=False):
    import torch

    act = torch.bfloat16 if cfg.dtype == binding.SPEC_VERIFY_BF16 else torch.float32
    Hq, Hkv, D, L, V = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.kv_capacity, cfg.vocab
    i32, f32 = torch.int32, torch.float32
    ins = dict(q=torch.zeros(B, T, Hq, D, dtype=act), k_cache=torch.zeros(B, Hkv, L, D, dtype=act),
               v_cache=torch.zeros(B, Hkv, L, D, dtype=act), kv_len=torch.zeros(B, dtype=i32),
               parent=torch.zeros(B, T, dtype=i32), tokens=torch.zeros(B, T, dtype=i32),
               target_logits=torch.zeros(B, T, V, dtype=f32), draft_logits=torch.zeros(B, T, V, dtype=f32),
               u_accept=torch.zeros(B, T, dtype=f32), u_final=torch.zeros(B, dtype=f32))
    outs = sva.allocate_outputs(B, T, Hq, D, "bf16" if act == torch.bfloat16 else "f32", device="cpu",
                                vocab=V if probs else None)
    return ins, outs


def test_binding_checks_shapes_dtypes_and_layout_before_the_library():
    import torch

    cfg = sva.make_config(**GOOD)
    ins, outs = _cpu_args(cfg)
    # everything well formed: only the device is wrong (CPU tensors)
    with pytest.raises(sva.SpecVerifyError) as e:
        binding.check_run_args(cfg, ins, outs)
    assert "device tensor" in str(e.value)

    def expect(mutate, words):
        i, o = _cpu_args(cfg)
        mutate(i, o)
        with pytest.raises(sva.SpecVerifyError) as e:
            binding.check_run_args(cfg, i, o)
        assert e.value.code == binding.SPEC_VERIFY_ERR_INVALID_ARG
        for w in words:
            assert w in str(e.value), (str(e.value), w)

    # a transposed (non-contiguous) view of the right shape
    expect(lambda i, o: i.__setitem__("q", torch.zeros(2, 5, 128, 8, dtype=torch.bfloat16).transpose(2, 3)),
           ["q", "contiguous"])
    expect(lambda i, o: i.__setitem__("tokens", torch.zeros(2, 5, dtype=torch.int64)), ["tokens", "i32"])
    expect(lambda i, o: i.__setitem__("target_logits", torch.zeros(2, 5, 999)), ["target_logits", "shape"])
    expect(lambda i, o: i.__setitem__("k_cache", torch.zeros(2, 2, 256, 128, dtype=torch.float32)), ["k_cache", "bf16"])
    expect(lambda i, o: i.__setitem__("kv_len", torch.zeros(1, dtype=torch.int32)), ["kv_len", "shape"])
    expect(lambda i, o: i.__setitem__("draft_logits", None), ["draft_logits", "required"])
    expect(lambda i, o: o.__setitem__("path", torch.zeros(2, 6, dtype=torch.int32)), ["path", "shape"])
    expect(lambda i, o: o.__setitem__("node_accept", torch.zeros(2, 5, dtype=torch.int32)), ["node_accept", "u8"])
    expect(lambda i, o: o.__setitem__("attn_out", torch.zeros(2, 5, 8, 128)), ["attn_out", "bf16"])
    # more sequences of room than the batch uses is fine (first dimension only)
    i, o = _cpu_args(cfg)
    i["u_final"] = torch.zeros(4, dtype=torch.float32)
    with pytest.raises(sva.SpecVerifyError) as e:
        binding.check_run_args(cfg, i, o)
    assert "device tensor" in str(e.value)


def test_binding_checks_follow_the_skip_and_probs_flags():
    import torch

    cfg = sva.make_config(**dict(GOOD, skip_attention=True))
    ins, outs = _cpu_args(cfg)
    for k in ("q", "k_cache", "v_cache"):
        ins[k] = None
    outs["attn_out"] = None
    with pytest.raises(sva.SpecVerifyError) as e:
        binding.check_run_args(cfg, ins, outs)
    assert "device tensor" in str(e.value)          # nothing else missing
    cfg = sva.make_config(**dict(GOOD, skip_vocab=True))
    ins, _ = _cpu_args(cfg)
    for k in ("tokens", "target_logits", "draft_logits", "u_accept", "u_final"):
        ins[k] = None
    with pytest.raises(sva.SpecVerifyError) as e:
        binding.check_run_args(cfg, ins, dict(attn_out=torch.zeros(2, 5, 8, 128, dtype=torch.bfloat16)))
    assert "device tensor" in str(e.value)
    cfg = sva.make_config(**dict(GOOD, write_probs=True))
    ins, outs = _cpu_args(cfg)
    with pytest.raises(sva.SpecVerifyError) as e:
        binding.check_run_args(cfg, ins, outs)
    assert "probs" in str(e.value) and "required" in str(e.value)
    ins, outs = _cpu_args(cfg, probs=True)
    with pytest.raises(sva.SpecVerifyError) as e:
        binding.check_run_args(cfg, ins, outs)
    assert "device tensor" in str(e.value)


def test_noalloc_entry_point_refuses_before_touching_the_device():
    """Host-checkable refusals of spec_verify_run_noalloc happen before any HIP call."""
    lib = sva.load_library()
    ins, outs = binding.Inputs(), binding.Outputs()
    cfg = sva.make_config(**dict(GOOD, max_batch=2000))
    ins.batch, ins.nodes = 1025, 4
    assert lib.spec_verify_run_noalloc(ctypes.byref(cfg), ctypes.byref(ins), ctypes.byref(outs), None) == \
        binding.SPEC_VERIFY_ERR_UNSUPPORTED
    assert "1024" in sva.spec_verify_last_error()
    ins.batch = 2
    for flags in (dict(timing=True), dict(lossless_tree=True)):
        cfg = sva.make_config(**dict(GOOD, **flags))
        assert lib.spec_verify_run_noalloc(ctypes.byref(cfg), ctypes.byref(ins), ctypes.byref(outs), None) == \
            binding.SPEC_VERIFY_ERR_UNSUPPORTED
    cfg = sva.make_config(**dict(GOOD, head_dim=96))            # validated as create does
    assert lib.spec_verify_run_noalloc(ctypes.byref(cfg), ctypes.byref(ins), ctypes.byref(outs), None) == \
        binding.SPEC_VERIFY_ERR_UNSUPPORTED
    assert lib.spec_verify_run_noalloc(None, ctypes.byref(ins), ctypes.byref(outs), None) == \
        binding.SPEC_VERIFY_ERR_INVALID_ARG
    # row statistics of 1024 sequences of 64 nodes fit; the 4194304-id draw totals of 1024 do not
    cfg = sva.make_config(**dict(GOOD, max_batch=1024, max_nodes=64, vocab=4194304))
    ins.batch, ins.nodes = 1024, 64
    assert lib.spec_verify_run_noalloc(ctypes.byref(cfg), ctypes.byref(ins), ctypes.byref(outs), None) == \
        binding.SPEC_VERIFY_ERR_UNSUPPORTED
    assert "16 MiB" in sva.spec_verify_last_error()
