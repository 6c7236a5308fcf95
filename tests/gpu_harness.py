"""Run a synthetic case through the HIP library and compare it with the CPU oracle."""
from __future__ import annotations

import sys
from typing import Dict, Optional, Sequence

import numpy as np

import oracle
import synth

ATTN_TOL = {"bf16": 2e-2, "f32": 1e-4}
PROB_RTOL = 1e-4


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (survives a crash of the process)."""
    print("[gpu] " + msg, flush=True)
    sys.stdout.flush()


def _act_tensor(arr: np.ndarray, dtype: str, torch):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))


def device_inputs(case: synth.Case, device="cuda") -> Dict:
    import torch

    d = case.spec.dtype
    out = dict(
        q=_act_tensor(case.q, d, torch).to(device),
        k_cache=_act_tensor(case.k_cache, d, torch).to(device),
        v_cache=_act_tensor(case.v_cache, d, torch).to(device),
        kv_len=torch.from_numpy(case.kv_len.astype(np.int32)).to(device),
        parent=torch.from_numpy(case.parent.astype(np.int32)).to(device),
        tokens=torch.from_numpy(case.tokens.astype(np.int32)).to(device),
        target_logits=torch.from_numpy(case.target_logits).to(device),
        draft_logits=None if case.draft_logits is None else torch.from_numpy(case.draft_logits).to(device),
        u_accept=torch.from_numpy(case.u_accept).to(device),
        u_final=torch.from_numpy(case.u_final).to(device),
    )
    return out


def handle_config(spec: synth.CaseSpec, batch: Optional[int] = None, nodes: Optional[int] = None,
                  timing: bool = False, kv_capacity: Optional[int] = None, lossless_tree: bool = False) -> Dict:
    return dict(max_batch=batch or spec.batch, max_nodes=nodes or spec.nodes, num_q_heads=spec.hq,
                num_kv_heads=spec.hkv, head_dim=spec.head_dim, kv_capacity=kv_capacity or spec.kv_capacity,
                vocab=spec.vocab, dtype=spec.dtype, mode=spec.mode, temperature=spec.temperature,
                top_p=spec.top_p, timing=timing, lossless_tree=lossless_tree)


def to_numpy(outputs: Dict) -> Dict[str, np.ndarray]:
    import torch

    res = {}
    for k, t in outputs.items():
        if t.dtype == torch.bfloat16:
            res[k] = t.float().cpu().numpy()
        else:
            res[k] = t.cpu().numpy()
    return res


def run_gpu(case: synth.Case, label: str, repeat: int = 1,
            lossless_tree: bool = False) -> Sequence[Dict[str, np.ndarray]]:
    import torch
    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs

    spec = case.spec
    note("%s: upload B=%d T=%d L<=%d V=%d %s %s" % (label, case.batch, case.nodes, int(case.kv_len.max()),
                                                    spec.vocab, spec.dtype, spec.mode))
    ins = device_inputs(case)
    results = []
    with SpecVerify(**handle_config(spec, kv_capacity=case.k_cache.shape[2], lossless_tree=lossless_tree)) as sv:
        for r in range(repeat):
            outs = allocate_outputs(case.batch, case.nodes, spec.hq, spec.head_dim, spec.dtype)
            note("%s: run %d" % (label, r))
            sv.run(ins, outs)
            torch.cuda.synchronize()
            results.append(to_numpy(outs))
    note("%s: done" % label)
    return results


def compare(case: synth.Case, got: Dict[str, np.ndarray], ref: Dict[str, np.ndarray],
            seqs: Optional[Sequence[int]] = None, attn: bool = True,
            attn_rows: Optional[Sequence] = None, rule: str = "independent") -> Dict[str, int]:
    """Element-wise parity.  `ref` holds the oracle's outputs for `seqs` (in order).

    attn_rows: optional list of (seq, node, head, oracle row) to check instead of every row.
    rule "lossless": which nodes are tested depends on earlier decisions, so a
    sequence with any near-tie has no per-node comparison either.
    Returns counts of near-ties (excluded decisions).
    """
    spec = case.spec
    seqs = list(range(case.batch)) if seqs is None else list(seqs)
    T = case.nodes
    stats = dict(seqs=len(seqs), seq_near=0, node_near=0, final_near=0)
    for n, b in enumerate(seqs):
        st = int(ref["status"][n])
        assert int(got["status"][b]) == st, ("status", b, int(got["status"][b]), st)
        if st & 3:
            assert got["accept_len"][b] == 0 and got["final_node"][b] == -1
            assert (got["path"][b] == -1).all() and (got["out_tokens"][b] == -1).all()
            continue
        node_near = ref["node_near"][n]
        stats["node_near"] += int(node_near.sum())
        stats["final_near"] += int(ref["final_near"][n])
        if rule == "lossless" and ref["seq_near"][n]:
            stats["seq_near"] += 1
            np.testing.assert_array_equal(got["row_token"][b], ref["row_token"][n], err_msg="row_token b=%d" % b)
            continue
        # per-node decisions
        for i in range(T):
            if not node_near[i]:
                assert got["node_accept"][b, i] == ref["node_accept"][n, i], ("node_accept", b, i)
        # best token of every target row (integer argmax: no band)
        np.testing.assert_array_equal(got["row_token"][b], ref["row_token"][n], err_msg="row_token b=%d" % b)
        # probabilities at the drafted tokens
        if spec.mode == "sampling":
            for name in ("node_p", "node_q"):
                g = got[name][b, 1:].astype(np.float64)
                r = ref[name][n, 1:]
                mask = ~node_near[1:]
                big = mask & (r >= 1e-30)
                rel = np.abs(g[big] - r[big]) / r[big]
                assert rel.size == 0 or rel.max() <= PROB_RTOL, (name, b, float(rel.max()))
                zero = mask & (r < 1e-30)
                assert (np.abs(g[zero]) < 1e-30).all(), (name, b, "zero mismatch")
        if ref["seq_near"][n]:
            stats["seq_near"] += 1
            continue
        for k in ("accept_len", "final_node", "final_from_residual"):
            assert int(got[k][b]) == int(ref[k][n]), (k, b, int(got[k][b]), int(ref[k][n]))
        np.testing.assert_array_equal(got["path"][b], ref["path"][n], err_msg="path b=%d" % b)
        np.testing.assert_array_equal(got["out_tokens"][b], ref["out_tokens"][n], err_msg="out_tokens b=%d" % b)
    if attn:
        tol = ATTN_TOL[spec.dtype]
        worst = 0.0
        rows = 0
        if attn_rows is None:
            for n, b in enumerate(seqs):
                if np.isnan(ref["attn_out"][n]).any():
                    continue
                err = np.abs(got["attn_out"][b].astype(np.float64) - ref["attn_out"][n]).max()
                worst = max(worst, float(err))
                rows += ref["attn_out"][n].shape[0] * ref["attn_out"][n].shape[1]
                assert err <= tol, ("attn_out", b, float(err))
        else:
            for (b, i, h, val) in attn_rows:
                err = np.abs(got["attn_out"][b, i, h].astype(np.float64) - val).max()
                worst = max(worst, float(err))
                rows += 1
                assert err <= tol, ("attn_out", b, i, h, float(err))
        stats.update(attn_rows=rows, attn_max_err=worst, attn_tol=tol)
    return stats


def sampled_attention(case: synth.Case, picks) -> list:
    """Oracle attention for some (seq, node, head) rows of a large case (one widening per sequence)."""
    rows = []
    spec = case.spec
    by_seq = {}
    for (b, i, h) in picks:
        by_seq.setdefault(b, []).append((i, h))
    for b, nh in by_seq.items():
        k = oracle.widen(case.k_cache[b], spec.dtype)
        v = oracle.widen(case.v_cache[b], spec.dtype)
        by_node = {}
        for (i, h) in nh:
            by_node.setdefault(i, []).append(h)
        for i, heads in by_node.items():
            q = oracle.widen(case.q[b, i], spec.dtype)
            out = oracle.tree_attention_node(q, k, v, int(case.kv_len[b]), case.parent[b], i, heads=heads)
            rows.extend((b, i, h, out[n]) for n, h in enumerate(heads))
    return rows


def deepest_node_rows(case: synth.Case, seqs) -> list:
    """(seq, node, head) for every head of the root and of every node at the tree's largest depth."""
    out = []
    for b in seqs:
        d = oracle.depths(case.parent[b])
        nodes = [0] + [i for i in range(len(d)) if d[i] == max(d) and i > 0]
        out.extend((b, i, h) for i in nodes for h in range(case.spec.hq))
    return out


def scale_tree_keys(case: synth.Case, factor: float = 8.0) -> None:
    """Multiply the keys of every tree slot (L_b .. L_b+T-1) by a power of two, in place.

    Exact in bf16 and fp32.  The tree keys then carry a large share of every
    node's attention weight, so a wrong tree mask changes the output by O(1)
    even over a long prefix.
    """
    T = case.nodes
    for b in range(case.batch):
        L = int(case.kv_len[b])
        sl = case.k_cache[b, :, L:L + T]
        if case.spec.dtype == "bf16":
            case.k_cache[b, :, L:L + T] = synth.bf16_round_bits(synth.bf16_bits_to_f32(sl) * np.float32(factor))
        else:
            case.k_cache[b, :, L:L + T] = sl * np.float32(factor)
