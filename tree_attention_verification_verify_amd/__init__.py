"""MI355X-native verify step of speculative / Medusa tree decoding.

libspecverify.so holds the HIP kernels (gfx950) and the C ABI declared in
include/spec_verify.h; `binding` marshals PyTorch device tensors into it.
"""
from .binding import (EXPORTED, LIB_PATH, PagedKV, SpecVerify, SpecVerifyError, allocate_outputs, load_library,
                      make_config, paged_kv, spec_verify_build_tree, spec_verify_commit, spec_verify_commit_paged,
                      spec_verify_create, spec_verify_describe, spec_verify_destroy, spec_verify_last_error, spec_verify_run,
                      spec_verify_run_noalloc, spec_verify_run_paged, spec_verify_timing_read, spec_verify_tree_template)

__all__ = ["EXPORTED", "LIB_PATH", "PagedKV", "SpecVerify", "SpecVerifyError", "allocate_outputs", "load_library",
           "make_config", "paged_kv", "spec_verify_build_tree", "spec_verify_commit", "spec_verify_commit_paged",
           "spec_verify_create", "spec_verify_describe", "spec_verify_destroy", "spec_verify_last_error", "spec_verify_run",
           "spec_verify_run_noalloc", "spec_verify_run_paged", "spec_verify_timing_read", "spec_verify_tree_template"]
