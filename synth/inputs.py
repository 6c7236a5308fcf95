"""Seeded synthetic inputs for the verify step.

This module only draws random numbers and lays them out.  It computes no part
of the verify step (no attention, no target/draft probabilities, no
acceptance, no path selection); both the CPU oracle and the HIP path read the
arrays it returns, so neither depends on the other.

Recipe (every array has its own PCG64 stream keyed by (seed, stream id)):

  stream 0  Q             ~ N(0,1), rounded to bf16 (RNE) for bf16 cases
  stream 1  K cache       ~ N(0,1), same rounding, all Lcap slots
  stream 2  V cache       ~ N(0,1), same rounding, all Lcap slots
  stream 3  target logits ~ N(0, sigma_t^2) fp32
  stream 4  draft noise   : draft row i = target row parent[i] + N(0, sigma_d^2)
  stream 5  draft sampler : Gumbel noise for drawing x_i from the draft's
                            effective distribution (see `_draw_from_draft`)
  stream 6  u_accept      ~ U(0,1) fp32, clamped below 1
  stream 7  u_final       ~ U(0,1) fp32, clamped below 1
  stream 8  ragged prefix lengths L_b ~ U{lo..hi}
  stream 9  greedy candidate noise (children of v = r-th best of z_v + N(0,1))
  stream 10 root token (the last committed token; never verified)

Drafting is upstream of the verify step: `_draw_from_draft` stands in for a
draft model that samples its token from its own temperature/top-p
distribution, which is what the lossless rule assumes ("投机解码的五条路线",
section on exact verification).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .trees import chain_tree, medusa_tree, sibling_rank

F32_BELOW_ONE = np.float32(np.nextafter(np.float32(1.0), np.float32(0.0)))


@dataclasses.dataclass(frozen=True)
class CaseSpec:
    name: str
    batch: int
    dtype: str                  # "f32" or "bf16"
    hq: int
    hkv: int
    head_dim: int
    prefix_len: int             # L (max prefix length)
    vocab: int
    mode: str                   # "greedy" or "sampling"
    tree: Tuple                 # ("chain", gamma) or ("medusa", caps, T)
    temperature: float = 1.0
    top_p: float = 1.0
    target_sigma: float = 3.0
    draft_sigma: float = 1.0
    ragged: Optional[Tuple[int, int]] = None   # L_b ~ U{lo..hi}
    seed: Tuple[int, ...] = (0,)

    @property
    def parent(self) -> List[int]:
        if self.tree[0] == "chain":
            return chain_tree(self.tree[1])
        return medusa_tree(self.tree[1], self.tree[2])[0]

    @property
    def nodes(self) -> int:
        return len(self.parent)

    @property
    def kv_capacity(self) -> int:
        return self.prefix_len + self.nodes

    def replace(self, **kw) -> "CaseSpec":
        return dataclasses.replace(self, **kw)


MEDUSA_64 = ("medusa", (10, 4, 2, 1, 1), 64)
MEDUSA_26 = ("medusa", (10, 4, 2, 1), 26)

# The five workloads (shapes and value distributions as stated for each), by name.
WORKLOADS = {
    "tiny-chain-f32": CaseSpec("tiny-chain-f32", 1, "f32", 4, 4, 64, 128, 1000, "sampling", ("chain", 4),
                temperature=1.0, top_p=1.0, target_sigma=2.0, draft_sigma=1.0, seed=(0, 0)),
    "llama7b-medusa-greedy": CaseSpec("llama7b-medusa-greedy", 1, "bf16", 32, 32, 128, 2048, 32000, "greedy", MEDUSA_64,
                target_sigma=3.0, seed=(0, 1)),
    "chain-batch32-topp": CaseSpec("chain-batch32-topp", 32, "bf16", 32, 32, 128, 4096, 32000, "sampling", ("chain", 5),
                temperature=0.8, top_p=0.9, target_sigma=3.0, draft_sigma=1.5, ragged=(1024, 4096),
                seed=(0, 2)),
    "70b-gqa-medusa": CaseSpec("70b-gqa-medusa", 8, "bf16", 64, 8, 128, 8192, 32000, "sampling", MEDUSA_64,
                temperature=1.0, top_p=1.0, target_sigma=3.0, draft_sigma=1.0, seed=(0, 3)),
    "longctx-bigvocab": CaseSpec("longctx-bigvocab", 16, "bf16", 32, 8, 128, 32768, 128256, "sampling", MEDUSA_26,
                temperature=0.7, top_p=1.0, target_sigma=3.0, draft_sigma=1.0, seed=(0, 4)),
}


def workload(name: str, **overrides) -> CaseSpec:
    spec = WORKLOADS[name]
    return spec.replace(**overrides) if overrides else spec


def _rng(spec: CaseSpec, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(spec.seed) + [stream])))


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    b = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Widen a stored activation array (fp32 values or bf16 bits) to fp32 exactly."""
    return bf16_bits_to_f32(arr) if dtype == "bf16" else arr


def _normal_act(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return bf16_round_bits(x) if dtype == "bf16" else x


def _uniform_f32(rng: np.random.Generator, shape) -> np.ndarray:
    u = rng.random(size=shape).astype(np.float32)
    return np.minimum(u, F32_BELOW_ONE)


def _draw_from_draft(z_q: np.ndarray, temperature: float, top_p: float,
                     rng: np.random.Generator) -> int:
    """Simulated draft model: draw one token from its temperature/top-p distribution.

    Gumbel-max over the nucleus: argmax_k (z_k / T + G_k), G_k standard Gumbel.
    The nucleus is the smallest set of highest-probability tokens (ties by
    index) whose mass reaches top_p.
    """
    s = z_q.astype(np.float64) / temperature
    if top_p < 1.0:
        w = np.exp(s - s.max())
        w /= w.sum()
        order = np.lexsort((np.arange(w.size), -w))
        csum = np.cumsum(w[order])
        keep = int(np.searchsorted(csum, top_p, side="left")) + 1
        allowed = np.zeros(w.size, dtype=bool)
        allowed[order[:keep]] = True
    else:
        allowed = np.ones(s.size, dtype=bool)
    g = -np.log(-np.log(rng.random(size=s.size)))
    score = np.where(allowed, s + g, -np.inf)
    return int(np.argmax(score))


@dataclasses.dataclass
class Case:
    spec: CaseSpec
    q: np.ndarray              # [B,T,Hq,D]   fp32, or bf16 bits (uint16)
    k_cache: np.ndarray        # [B,Hkv,Lcap,D]
    v_cache: np.ndarray        # [B,Hkv,Lcap,D]
    kv_len: np.ndarray         # [B] int32
    parent: np.ndarray         # [B,T] int32
    tokens: np.ndarray         # [B,T] int32
    target_logits: np.ndarray  # [B,T,V] fp32
    draft_logits: Optional[np.ndarray]  # [B,T,V] fp32 (row 0 unused) or None in greedy mode
    u_accept: np.ndarray       # [B,T] fp32
    u_final: np.ndarray        # [B] fp32

    @property
    def batch(self) -> int:
        return self.spec.batch

    @property
    def nodes(self) -> int:
        return self.parent.shape[1]


def make_case(spec: CaseSpec, *, with_kv: bool = True) -> Case:
    B, T, V = spec.batch, spec.nodes, spec.vocab
    Lcap = spec.kv_capacity
    par = np.array(spec.parent, dtype=np.int32)
    parent = np.tile(par, (B, 1))

    q = _normal_act(_rng(spec, 0), (B, T, spec.hq, spec.head_dim), spec.dtype)
    kv_shape = (B, spec.hkv, Lcap, spec.head_dim)
    if with_kv:
        rk, rv = _rng(spec, 1), _rng(spec, 2)
        store = np.uint16 if spec.dtype == "bf16" else np.float32
        k_cache = np.empty(kv_shape, dtype=store)
        v_cache = np.empty(kv_shape, dtype=store)
        for b in range(B):  # per sequence, to bound the fp32 temporaries
            k_cache[b] = _normal_act(rk, kv_shape[1:], spec.dtype)
            v_cache[b] = _normal_act(rv, kv_shape[1:], spec.dtype)
    else:
        k_cache = v_cache = None

    if spec.ragged is not None:
        lo, hi = spec.ragged
        kv_len = _rng(spec, 8).integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    else:
        kv_len = np.full(B, spec.prefix_len, dtype=np.int32)

    target = (_rng(spec, 3).standard_normal(size=(B, T, V), dtype=np.float32)
              * np.float32(spec.target_sigma))

    tokens = np.zeros((B, T), dtype=np.int32)
    tokens[:, 0] = _rng(spec, 10).integers(0, V, size=B)
    draft = None
    if spec.mode == "sampling":
        draft = np.zeros((B, T, V), dtype=np.float32)
        rn, rs = _rng(spec, 4), _rng(spec, 5)
        for b in range(B):
            for i in range(1, T):
                noise = rn.standard_normal(size=V, dtype=np.float32) * np.float32(spec.draft_sigma)
                draft[b, i] = target[b, par[i]] + noise
                tokens[b, i] = _draw_from_draft(draft[b, i], spec.temperature, spec.top_p, rs)
    else:
        rg = _rng(spec, 9)
        rank = sibling_rank(spec.parent)
        children = {}
        for i in range(1, T):
            children.setdefault(int(par[i]), []).append(i)
        for b in range(B):
            for v in range(T):
                kids = children.get(v)
                if not kids:
                    continue
                noisy = target[b, v].astype(np.float64) + rg.standard_normal(size=V)
                order = np.argsort(-noisy, kind="stable")
                for c in kids:
                    tokens[b, c] = int(order[rank[c]])

    u_accept = _uniform_f32(_rng(spec, 6), (B, T))
    u_final = _uniform_f32(_rng(spec, 7), (B,))
    return Case(spec, q, k_cache, v_cache, kv_len, parent, tokens, target, draft, u_accept, u_final)
