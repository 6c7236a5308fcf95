"""ctypes binding of libspecverify.so: argument marshalling only.

The functions mirror the C ABI in include/spec_verify.h one to one
(spec_verify_create / spec_verify_run / spec_verify_run_noalloc / spec_verify_run_paged /
spec_verify_commit / spec_verify_commit_paged / spec_verify_build_tree /
spec_verify_tree_template / spec_verify_destroy / spec_verify_last_error /
spec_verify_timing_read).  Tensors are PyTorch device
tensors; only their data pointers cross the boundary.  Every step of the
verify step runs in the library's HIP kernels: there is no fallback, and a
missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SPEC_VERIFY_OK = 0
SPEC_VERIFY_ERR_INVALID_ARG = -1
SPEC_VERIFY_ERR_UNSUPPORTED = -2
SPEC_VERIFY_ERR_HIP = -3
SPEC_VERIFY_ERR_OOM = -4
SPEC_VERIFY_F32 = 0
SPEC_VERIFY_BF16 = 1
SPEC_VERIFY_GREEDY = 0
SPEC_VERIFY_SAMPLING = 1
SPEC_VERIFY_FLAG_TIMING = 1
SPEC_VERIFY_FLAG_LOSSLESS_TREE = 2
SPEC_VERIFY_FLAG_SKIP_ATTENTION = 4
SPEC_VERIFY_FLAG_SKIP_VOCAB = 8
SPEC_VERIFY_FLAG_WRITE_PROBS = 16
SPEC_VERIFY_FLAG_WALK_NO_WAIT = 32
SPEC_VERIFY_NUM_STAGES = 3
STAGES = ("attention", "vocab", "finish")

EXPORTED = ("spec_verify_create", "spec_verify_run", "spec_verify_destroy", "spec_verify_last_error",
            "spec_verify_timing_read", "spec_verify_commit", "spec_verify_run_paged", "spec_verify_commit_paged",
            "spec_verify_build_tree", "spec_verify_tree_template", "spec_verify_run_noalloc",
            "spec_verify_describe")


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("spec_verify error %d: %s" % (code, msg))
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("max_batch", ctypes.c_int32), ("max_nodes", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("kv_capacity", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("mode", ctypes.c_int32), ("temperature", ctypes.c_float),
                ("top_p", ctypes.c_float), ("softmax_scale", ctypes.c_float), ("flags", ctypes.c_uint32)]


class Inputs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("kv_len", ctypes.c_void_p), ("parent", ctypes.c_void_p), ("tokens", ctypes.c_void_p),
                ("target_logits", ctypes.c_void_p), ("draft_logits", ctypes.c_void_p),
                ("u_accept", ctypes.c_void_p), ("u_final", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("nodes", ctypes.c_int32)]


class CommitArgs(ctypes.Structure):
    _fields_ = [("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("kv_len", ctypes.c_void_p),
                ("path", ctypes.c_void_p), ("accept_len", ctypes.c_void_p), ("final_node", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("nodes", ctypes.c_int32)]


class PagedKV(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32), ("table_width", ctypes.c_int32)]


class TreeArgs(ctypes.Structure):
    _fields_ = [("cand_logits", ctypes.c_void_p), ("root_token", ctypes.c_void_p), ("tree_parent", ctypes.c_void_p),
                ("tree_rank", ctypes.c_void_p), ("parent", ctypes.c_void_p), ("tokens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("nodes", ctypes.c_int32), ("depth", ctypes.c_int32)]


class Outputs(ctypes.Structure):
    _fields_ = [("attn_out", ctypes.c_void_p), ("accept_len", ctypes.c_void_p), ("final_node", ctypes.c_void_p),
                ("path", ctypes.c_void_p), ("out_tokens", ctypes.c_void_p), ("status", ctypes.c_void_p),
                ("node_p", ctypes.c_void_p), ("node_q", ctypes.c_void_p), ("node_accept", ctypes.c_void_p),
                ("final_from_residual", ctypes.c_void_p), ("row_token", ctypes.c_void_p),
                ("probs", ctypes.c_void_p)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libspecverify.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError("%s is missing: build it with __graft_entry__.build()" % path)
    # PyTorch brings its own HIP runtime (same soname as /opt/rocm's).  Loaded
    # first, it is the one the library binds to: one runtime per process, the
    # one that owns the tensors passed in.  (A second runtime initialised in the
    # same process finds no device.)
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    lib.spec_verify_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(ctypes.c_void_p)]
    lib.spec_verify_create.restype = ctypes.c_int
    lib.spec_verify_run.argtypes = [ctypes.c_void_p, ctypes.POINTER(Inputs), ctypes.POINTER(Outputs),
                                    ctypes.c_void_p]
    lib.spec_verify_run.restype = ctypes.c_int
    lib.spec_verify_run_noalloc.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Inputs), ctypes.POINTER(Outputs),
                                            ctypes.c_void_p]
    lib.spec_verify_run_noalloc.restype = ctypes.c_int
    lib.spec_verify_destroy.argtypes = [ctypes.c_void_p]
    lib.spec_verify_destroy.restype = ctypes.c_int
    lib.spec_verify_last_error.argtypes = []
    lib.spec_verify_last_error.restype = ctypes.c_char_p
    lib.spec_verify_timing_read.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_float),
                                            ctypes.POINTER(ctypes.c_int32)]
    lib.spec_verify_timing_read.restype = ctypes.c_int
    lib.spec_verify_commit.argtypes = [ctypes.c_void_p, ctypes.POINTER(CommitArgs), ctypes.c_void_p]
    lib.spec_verify_commit.restype = ctypes.c_int
    lib.spec_verify_run_paged.argtypes = [ctypes.c_void_p, ctypes.POINTER(Inputs), ctypes.POINTER(PagedKV),
                                          ctypes.POINTER(Outputs), ctypes.c_void_p]
    lib.spec_verify_run_paged.restype = ctypes.c_int
    lib.spec_verify_commit_paged.argtypes = [ctypes.c_void_p, ctypes.POINTER(CommitArgs), ctypes.POINTER(PagedKV),
                                             ctypes.c_void_p]
    lib.spec_verify_commit_paged.restype = ctypes.c_int
    lib.spec_verify_build_tree.argtypes = [ctypes.c_void_p, ctypes.POINTER(TreeArgs), ctypes.c_void_p]
    lib.spec_verify_build_tree.restype = ctypes.c_int
    lib.spec_verify_describe.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_char_p,
                                         ctypes.c_int32]
    lib.spec_verify_describe.restype = ctypes.c_int
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.spec_verify_tree_template.argtypes = [i32p, ctypes.c_int32, ctypes.c_int32, i32p, i32p]
    lib.spec_verify_tree_template.restype = ctypes.c_int
    _lib = lib
    return lib


def spec_verify_last_error() -> str:
    return load_library().spec_verify_last_error().decode()


def _check(rc: int) -> None:
    if rc != SPEC_VERIFY_OK:
        raise SpecVerifyError(rc, spec_verify_last_error())


def make_config(*, max_batch, max_nodes, num_q_heads, num_kv_heads, head_dim, kv_capacity, vocab,
                dtype="bf16", mode="sampling", temperature=1.0, top_p=1.0, softmax_scale=0.0,
                timing=False, lossless_tree=False, skip_attention=False, skip_vocab=False,
                write_probs=False, walk_no_wait=False) -> Config:
    flags = ((SPEC_VERIFY_FLAG_TIMING if timing else 0) | (SPEC_VERIFY_FLAG_LOSSLESS_TREE if lossless_tree else 0)
             | (SPEC_VERIFY_FLAG_SKIP_ATTENTION if skip_attention else 0)
             | (SPEC_VERIFY_FLAG_SKIP_VOCAB if skip_vocab else 0)
             | (SPEC_VERIFY_FLAG_WRITE_PROBS if write_probs else 0)
             | (SPEC_VERIFY_FLAG_WALK_NO_WAIT if walk_no_wait else 0))
    return Config(max_batch, max_nodes, num_q_heads, num_kv_heads, head_dim, kv_capacity, vocab,
                  SPEC_VERIFY_BF16 if dtype == "bf16" else SPEC_VERIFY_F32,
                  SPEC_VERIFY_SAMPLING if mode == "sampling" else SPEC_VERIFY_GREEDY,
                  temperature, top_p, softmax_scale, flags)


def spec_verify_create(cfg: Config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().spec_verify_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def spec_verify_destroy(handle: ctypes.c_void_p) -> None:
    _check(load_library().spec_verify_destroy(handle))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ------------------------------------------------------------------ argument checks
#
# The library sees raw addresses only, so a non-contiguous view, a wrong dtype
# or a wrong shape would make it read or write the wrong memory.  These checks
# run before any call into the library; they use only tensor metadata.

_DTYPES = None


def _torch_dtype(name):
    global _DTYPES
    if _DTYPES is None:
        import torch

        _DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32, "i32": torch.int32, "u8": torch.uint8}
    return _DTYPES[name]


def _check_tensor(name: str, t, dtype: str, shape, optional: bool = False, seen: Optional[list] = None) -> None:
    """shape: sizes per dimension; the first may be exceeded (room for more sequences), None = any.

    With `seen`, the tensor is appended to it and its device is left for
    _check_devices (so every shape is checked before any device)."""
    if t is None:
        if optional:
            return
        raise SpecVerifyError(SPEC_VERIFY_ERR_INVALID_ARG, "%s is required" % name)
    if not hasattr(t, "data_ptr") or not hasattr(t, "is_contiguous"):
        raise SpecVerifyError(SPEC_VERIFY_ERR_INVALID_ARG, "%s must be a torch tensor" % name)
    if t.dtype != _torch_dtype(dtype):
        raise SpecVerifyError(SPEC_VERIFY_ERR_INVALID_ARG, "%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != len(shape):
        raise SpecVerifyError(SPEC_VERIFY_ERR_INVALID_ARG,
                              "%s must have %d dimensions, got shape %s" % (name, len(shape), tuple(t.shape)))
    for k, (got, want) in enumerate(zip(t.shape, shape)):
        if want is None:
            continue
        if (got < want) if k == 0 else (got != want):
            raise SpecVerifyError(SPEC_VERIFY_ERR_INVALID_ARG,
                                  "%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if not t.is_contiguous():
        raise SpecVerifyError(SPEC_VERIFY_ERR_INVALID_ARG, "%s must be contiguous" % name)
    if seen is not None:
        seen.append((name, t))
    else:
        _check_devices([(name, t)])


def _check_devices(named) -> None:
    for name, t in named:
        if t.device.type != "cuda":
            raise SpecVerifyError(SPEC_VERIFY_ERR_INVALID_ARG,
                                  "%s must be a device tensor, got %s" % (name, t.device))


def _cfg_dims(cfg: Config):
    act = "bf16" if cfg.dtype == SPEC_VERIFY_BF16 else "f32"
    return act, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim, cfg.kv_capacity, cfg.vocab


def check_run_args(cfg: Config, inputs: Dict, outputs: Dict, paged: bool = False) -> None:
    """Every tensor of a run against the handle's config (raises SpecVerifyError).

    Dtypes, shapes and contiguity of all tensors are checked first, then that
    each one lives on the GPU."""
    seen = []
    chk = lambda name, t, dtype, shape, optional=False: _check_tensor(name, t, dtype, shape, optional, seen)
    parent = inputs.get("parent")
    chk("parent", parent, "i32", (None, None))
    B, T = parent.shape
    act, Hq, Hkv, D, Lcap, V = _cfg_dims(cfg)
    flags = cfg.flags
    attn = not flags & SPEC_VERIFY_FLAG_SKIP_ATTENTION
    vocab = not flags & SPEC_VERIFY_FLAG_SKIP_VOCAB
    sampling = cfg.mode == SPEC_VERIFY_SAMPLING
    chk("kv_len", inputs.get("kv_len"), "i32", (B,))
    if attn:
        chk("q", inputs.get("q"), act, (B, T, Hq, D))
        if not paged:
            chk("k_cache", inputs.get("k_cache"), act, (B, Hkv, Lcap, D))
            chk("v_cache", inputs.get("v_cache"), act, (B, Hkv, Lcap, D))
        chk("attn_out", outputs.get("attn_out"), act, (B, T, Hq, D))
    if vocab:
        chk("tokens", inputs.get("tokens"), "i32", (B, T))
        chk("target_logits", inputs.get("target_logits"), "f32", (B, T, V))
        chk("draft_logits", inputs.get("draft_logits"), "f32", (B, T, V), optional=not sampling)
        chk("u_accept", inputs.get("u_accept"), "f32", (B, T))
        chk("u_final", inputs.get("u_final"), "f32", (B,))
        for name in ("accept_len", "final_node", "status"):
            chk(name, outputs.get(name), "i32", (B,))
        for name in ("path", "out_tokens", "row_token"):
            chk(name, outputs.get(name), "i32", (B, T))
        for name in ("node_p", "node_q"):
            chk(name, outputs.get(name), "f32", (B, T))
        chk("node_accept", outputs.get("node_accept"), "u8", (B, T))
        chk("final_from_residual", outputs.get("final_from_residual"), "u8", (B,))
        if flags & SPEC_VERIFY_FLAG_WRITE_PROBS:
            chk("probs", outputs.get("probs"), "f32", (B, T, V))
    _check_devices(seen)


def _inputs(inputs: Dict) -> Inputs:
    B, T = inputs["parent"].shape
    return Inputs(_ptr(inputs.get("q")), _ptr(inputs.get("k_cache")), _ptr(inputs.get("v_cache")),
                  _ptr(inputs["kv_len"]), _ptr(inputs["parent"]), _ptr(inputs.get("tokens")),
                  _ptr(inputs.get("target_logits")), _ptr(inputs.get("draft_logits")), _ptr(inputs.get("u_accept")),
                  _ptr(inputs.get("u_final")), B, T)


def _outputs(outputs: Dict) -> Outputs:
    return Outputs(*[_ptr(outputs.get(f)) for f, _ in Outputs._fields_])


def paged_kv(k_pool, v_pool, block_table) -> PagedKV:
    """PagedKV from pools [num_blocks, Hkv, block_size, D] and a table [B, width] (device tensors)."""
    if k_pool is None or v_pool is None or block_table is None:
        raise SpecVerifyError(SPEC_VERIFY_ERR_INVALID_ARG, "k_pool, v_pool and block_table are required")
    # layout checks here; the device and the config are checked when a call uses it
    act = "bf16" if str(k_pool.dtype).endswith("bfloat16") else "f32"
    _check_tensor("k_pool", k_pool, act, (None, None, None, None), seen=[])
    _check_tensor("v_pool", v_pool, act, tuple(k_pool.shape), seen=[])
    _check_tensor("block_table", block_table, "i32", (None, None), seen=[])
    nb, _, bs, _ = k_pool.shape
    pk = PagedKV(_ptr(k_pool), _ptr(v_pool), _ptr(block_table), nb, bs, block_table.shape[1])
    # the struct holds raw device addresses: keep the tensors alive as long as it is
    pk._tensors = (k_pool, v_pool, block_table)
    return pk


def _check_paged(cfg: Config, paged: PagedKV) -> None:
    k_pool, v_pool, table = paged._tensors
    act, _, Hkv, D, _, _ = _cfg_dims(cfg)
    _check_tensor("k_pool", k_pool, act, (None, Hkv, None, D), seen=[])
    _check_devices([("k_pool", k_pool), ("v_pool", v_pool), ("block_table", table)])


def spec_verify_run(handle, inputs: Dict, outputs: Dict, stream=None, config: Optional[Config] = None) -> None:
    """inputs/outputs: dicts of device tensors named as the C struct fields.

    With `config` (the handle's Config) every tensor is checked against it first.
    """
    if config is not None:
        check_run_args(config, inputs, outputs)
    i, o = _inputs(inputs), _outputs(outputs)
    _check(load_library().spec_verify_run(handle, ctypes.byref(i), ctypes.byref(o),
                                          ctypes.c_void_p(_stream_handle(stream))))


def spec_verify_run_noalloc(config: Config, inputs: Dict, outputs: Dict, stream=None) -> None:
    """spec_verify_run without a handle and without any device allocation: the
    workspace is the library's static per-GPU scratch (see the C declaration)."""
    check_run_args(config, inputs, outputs)
    i, o = _inputs(inputs), _outputs(outputs)
    _check(load_library().spec_verify_run_noalloc(ctypes.byref(config), ctypes.byref(i), ctypes.byref(o),
                                                  ctypes.c_void_p(_stream_handle(stream))))


def spec_verify_run_paged(handle, inputs: Dict, paged: PagedKV, outputs: Dict, stream=None,
                          config: Optional[Config] = None) -> None:
    """spec_verify_run with the caches read through a block table (inputs' k_cache/v_cache unused)."""
    if config is not None:
        check_run_args(config, inputs, outputs, paged=True)
        _check_paged(config, paged)
    i, o = _inputs(inputs), _outputs(outputs)
    _check(load_library().spec_verify_run_paged(handle, ctypes.byref(i), ctypes.byref(paged), ctypes.byref(o),
                                                ctypes.c_void_p(_stream_handle(stream))))


def _stream_handle(stream):
    import torch

    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check_commit(cfg: Optional[Config], k_cache, v_cache, kv_len, path, accept_len, final_node, paged=False):
    _check_tensor("path", path, "i32", (None, None))
    B, T = path.shape
    _check_tensor("kv_len", kv_len, "i32", (B,))
    _check_tensor("accept_len", accept_len, "i32", (B,))
    _check_tensor("final_node", final_node, "i32", (B,))
    if cfg is not None and not paged:
        act, _, Hkv, D, Lcap, _ = _cfg_dims(cfg)
        _check_tensor("k_cache", k_cache, act, (B, Hkv, Lcap, D))
        _check_tensor("v_cache", v_cache, act, (B, Hkv, Lcap, D))


def spec_verify_commit(handle, k_cache, v_cache, kv_len, path, accept_len, final_node, stream=None,
                       config: Optional[Config] = None) -> None:
    """KV commit of the accepted paths (device tensors; kv_len is updated in place)."""
    _check_commit(config, k_cache, v_cache, kv_len, path, accept_len, final_node)
    B, T = path.shape
    a = CommitArgs(_ptr(k_cache), _ptr(v_cache), _ptr(kv_len), _ptr(path), _ptr(accept_len), _ptr(final_node),
                   B, T)
    _check(load_library().spec_verify_commit(handle, ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream))))


def spec_verify_commit_paged(handle, paged: PagedKV, kv_len, path, accept_len, final_node, stream=None,
                             config: Optional[Config] = None) -> None:
    """KV commit through a block table (the pools in `paged` and kv_len are updated in place)."""
    _check_commit(config, None, None, kv_len, path, accept_len, final_node, paged=True)
    if config is not None:
        _check_paged(config, paged)
    B, T = path.shape
    a = CommitArgs(None, None, _ptr(kv_len), _ptr(path), _ptr(accept_len), _ptr(final_node), B, T)
    _check(load_library().spec_verify_commit_paged(handle, ctypes.byref(a), ctypes.byref(paged),
                                                   ctypes.c_void_p(_stream_handle(stream))))


def spec_verify_tree_template(caps, nodes: int):
    """Host-only template of a pruned Medusa tree: (parent, rank) as lists of `nodes` ints."""
    ncaps = len(caps)
    c = (ctypes.c_int32 * max(ncaps, 1))(*[int(x) for x in caps])
    par = (ctypes.c_int32 * max(nodes, 1))()
    rk = (ctypes.c_int32 * max(nodes, 1))()
    _check(load_library().spec_verify_tree_template(c, ncaps, nodes, par, rk))
    return list(par)[:nodes], list(rk)[:nodes]


def spec_verify_build_tree(handle, cand_logits, root_token, tree_parent, tree_rank, parent, tokens,
                           stream=None, config: Optional[Config] = None) -> None:
    """Fill parent/tokens [B,T] (device) from cand_logits [B,depth,V] and root_token [B] (device)
    with the host template tree_parent/tree_rank (sequences of T ints)."""
    _check_tensor("cand_logits", cand_logits, "f32", (None, None, None if config is None else config.vocab))
    B, depth = cand_logits.shape[0], cand_logits.shape[1]
    T = len(tree_parent)
    if len(tree_rank) != T:
        raise SpecVerifyError(SPEC_VERIFY_ERR_INVALID_ARG, "tree_rank and tree_parent differ in length")
    _check_tensor("root_token", root_token, "i32", (B,))
    _check_tensor("parent", parent, "i32", (B, T))
    _check_tensor("tokens", tokens, "i32", (B, T))
    tp = (ctypes.c_int32 * T)(*[int(x) for x in tree_parent])
    tr = (ctypes.c_int32 * T)(*[int(x) for x in tree_rank])
    a = TreeArgs(_ptr(cand_logits), _ptr(root_token), ctypes.cast(tp, ctypes.c_void_p),
                 ctypes.cast(tr, ctypes.c_void_p), _ptr(parent), _ptr(tokens), B, T, depth)
    _check(load_library().spec_verify_build_tree(handle, ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream))))


def spec_verify_describe(handle, batch: int, nodes: int) -> Dict:
    """The plan (kernel names, splits) of a run on this handle, from the library itself."""
    import json

    buf = ctypes.create_string_buffer(1024)
    _check(load_library().spec_verify_describe(handle, batch, nodes, buf, len(buf)))
    return json.loads(buf.value.decode())


def spec_verify_timing_read(handle):
    """Summed per-stage kernel milliseconds over the runs since the last read, and the run count."""
    ms = (ctypes.c_float * SPEC_VERIFY_NUM_STAGES)()
    n = ctypes.c_int32()
    _check(load_library().spec_verify_timing_read(handle, ms, ctypes.byref(n)))
    return dict(zip(STAGES, list(ms))), int(n.value)


def allocate_outputs(batch: int, nodes: int, num_q_heads: int, head_dim: int, dtype: str, device="cuda",
                     vocab: Optional[int] = None):
    """Device output tensors for one run (PyTorch is only the allocator here); with `vocab`,
    also probs [B,T,V] for SPEC_VERIFY_FLAG_WRITE_PROBS."""
    import torch

    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, T = batch, nodes
    out = dict(
        attn_out=torch.empty((B, T, num_q_heads, head_dim), dtype=dt, device=device),
        accept_len=torch.empty(B, dtype=torch.int32, device=device),
        final_node=torch.empty(B, dtype=torch.int32, device=device),
        path=torch.empty((B, T), dtype=torch.int32, device=device),
        out_tokens=torch.empty((B, T), dtype=torch.int32, device=device),
        status=torch.empty(B, dtype=torch.int32, device=device),
        node_p=torch.empty((B, T), dtype=torch.float32, device=device),
        node_q=torch.empty((B, T), dtype=torch.float32, device=device),
        node_accept=torch.empty((B, T), dtype=torch.uint8, device=device),
        final_from_residual=torch.empty(B, dtype=torch.uint8, device=device),
        row_token=torch.empty((B, T), dtype=torch.int32, device=device),
    )
    if vocab is not None:
        out["probs"] = torch.empty((B, T, vocab), dtype=torch.float32, device=device)
    return out


class PreparedRun:
    """One run's arguments checked and marshalled once; each call is a single
    library call with the prebuilt structs (for loops that repeat a run on the
    same tensors: the tensors are kept alive by this object and must not be
    replaced or resized while it is used)."""

    def __init__(self, sv: "SpecVerify", inputs: Dict, outputs: Dict, stream=None, paged: Optional[PagedKV] = None):
        if paged is None:
            check_run_args(sv.cfg, inputs, outputs)
        else:
            check_run_args(sv.cfg, inputs, outputs, paged=True)
            _check_paged(sv.cfg, paged)
        lib = load_library()
        self._keep = (sv, dict(inputs), dict(outputs), paged)
        self._i, self._o = _inputs(inputs), _outputs(outputs)
        s = ctypes.c_void_p(_stream_handle(stream))
        if paged is None:
            args = (sv.handle, ctypes.byref(self._i), ctypes.byref(self._o), s)
            self._fn = lib.spec_verify_run
        else:
            args = (sv.handle, ctypes.byref(self._i), ctypes.byref(paged), ctypes.byref(self._o), s)
            self._fn = lib.spec_verify_run_paged
        self._args = args

    def __call__(self) -> None:
        rc = self._fn(*self._args)
        if rc != SPEC_VERIFY_OK:
            _check(rc)


class SpecVerify:
    """Handle owner: create on construction, destroy on close()."""

    def __init__(self, **config):
        self.config = dict(config)
        self.cfg = make_config(**config)
        self.handle = spec_verify_create(self.cfg)

    def run(self, inputs: Dict, outputs: Dict, stream=None) -> None:
        spec_verify_run(self.handle, inputs, outputs, stream, config=self.cfg)

    def run_paged(self, inputs: Dict, paged: PagedKV, outputs: Dict, stream=None) -> None:
        spec_verify_run_paged(self.handle, inputs, paged, outputs, stream, config=self.cfg)

    def prepare(self, inputs: Dict, outputs: Dict, stream=None, paged: Optional[PagedKV] = None) -> PreparedRun:
        """A callable that repeats run (or run_paged) on these tensors with no per-call marshalling."""
        return PreparedRun(self, inputs, outputs, stream, paged)

    def timing_read(self):
        return spec_verify_timing_read(self.handle)

    def describe(self, batch: int, nodes: int) -> Dict:
        return spec_verify_describe(self.handle, batch, nodes)

    def commit(self, k_cache, v_cache, kv_len, path, accept_len, final_node, stream=None) -> None:
        spec_verify_commit(self.handle, k_cache, v_cache, kv_len, path, accept_len, final_node, stream,
                           config=self.cfg)

    def commit_paged(self, paged: PagedKV, kv_len, path, accept_len, final_node, stream=None) -> None:
        spec_verify_commit_paged(self.handle, paged, kv_len, path, accept_len, final_node, stream, config=self.cfg)

    def build_tree(self, cand_logits, root_token, tree_parent, tree_rank, parent, tokens, stream=None) -> None:
        spec_verify_build_tree(self.handle, cand_logits, root_token, tree_parent, tree_rank, parent, tokens, stream,
                               config=self.cfg)

    def close(self) -> None:
        if self.handle is not None:
            spec_verify_destroy(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
