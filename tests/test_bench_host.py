"""Host-side checks of bench.py's bookkeeping (no GPU): which kernel each stage
launches for each workload, and that every named kernel is defined where the
bench looks for its source."""
import os
import re

import pytest

import bench
import synth

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "tree_attention_verification_verify_amd", "csrc")


@pytest.mark.parametrize("name,overrides,attn,vocab", [
    ("tiny-chain-f32", {}, "attn_valu_tiled_kernel", "row_stats_stream_kernel"),
    ("llama7b-medusa-greedy", {}, "attn_mfma_kernel", "row_stats_stream_kernel"),
    ("chain-batch32-topp", {}, "attn_valu_tiled_kernel", "row_stats_topp_kernel"),
    ("70b-gqa-medusa", {}, "attn_mfma_kernel", "row_stats_stream_kernel"),
    ("longctx-bigvocab", {}, "attn_mfma_kernel", "row_stats_stream_kernel"),
    ("longctx-bigvocab", {"top_p": 0.9}, "attn_mfma_kernel", "row_stats_topp_chunked_kernel"),
    ("chain-batch32-topp", {"mode": "greedy"}, "attn_valu_tiled_kernel", "row_stats_stream_kernel"),
    ("chain-batch32-topp", {"hkv": 16}, "attn_valu_kernel", "row_stats_topp_kernel"),
])
def test_stage_kernel_follows_the_dispatch_rule(name, overrides, attn, vocab):
    spec = synth.workload(name).replace(**overrides)
    assert bench.stage_kernel("attention", spec) == attn
    assert bench.stage_kernel("vocab", spec) == vocab
    assert bench.stage_kernel("finish", spec) == "finish_kernel"


@pytest.mark.parametrize("kname", sorted(bench.KERNEL_SOURCES))
def test_every_named_kernel_is_defined_in_its_source(kname):
    src = open(os.path.join(CSRC, bench.KERNEL_SOURCES[kname])).read()
    assert re.search(r"__global__.*\bvoid\s+%s\s*\(" % kname, src), kname


def test_vocab_chunk_matches_the_library_constant():
    hdr = open(os.path.join(CSRC, "kernels.h")).read()
    threads = int(re.search(r"kVocabThreads\s*=\s*(\d+)", hdr).group(1))
    per = int(re.search(r"kVocabChunk\s*=\s*kVocabThreads\s*\*\s*(\d+)", hdr).group(1))
    assert threads * per == bench.VOCAB_CHUNK
