#!/usr/bin/env python3
"""Verify-step benchmark on one MI355X.

One step = one spec_verify_run over a batch of synthetic inputs already resident
in HBM: tree attention (+ split merge), vocabulary pass and selection.  The
headline workload is the 70B-shaped GQA Medusa-tree verify (batch 8, 64 query /
8 KV heads x 128, prefix 8192, 64-node tree, vocab 32000) in sampling mode; the
other four workloads (and the headline in greedy mode) are reported as
sub-records under "configs".

For every workload, before anything is timed, the GPU outputs are compared
with the CPU oracle (every decision and token, bit for bit outside the
near-tie band; attention rows of the root and the deepest nodes of a sequence
within the stated tolerance): a mismatch ends the run with exit status 3.

Timing (HIP events on the run's stream, inputs resident in HBM; every timed
part starts after at least 0.2 s of untimed steps, which bring the GPU out of
its idle clocks after the host-side parity check):
  value          B*T candidate tokens / mean time of `steps` back-to-back steps
                 (host clock around a synchronised region, as the driver's contract asks);
  warm           the same steps in 20 blocks with events only between blocks: median / min per step;
  cold           single steps, each after writing a 1 GiB buffer (flushes L2 and the
                 Infinity Cache) outside the events: median / min;
  roofline       the dominant kernel (the attention) timed alone, back to back, with a
                 handle that skips the vocabulary pass: no event between its launches.

Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
VALU_FP32_PEAK_TFLOPS = 157.3
RIDGE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)   # flop/byte
KERNEL_SOURCES = {"attn_mfma_kernel": "tree_attn.hip", "attn_valu_kernel": "tree_attn.hip",
                  "attn_valu_tiled_kernel": "tree_attn_valu.hip",
                  "row_stats_stream_kernel": "vocab_stats.hip", "row_stats_topp_kernel": "vocab_stats.hip",
                  "finish_kernel": "select_final.hip"}
HEADLINE = ("70b-gqa-medusa", None)
SUBRECORDS = [("tiny-chain-f32", None), ("llama7b-medusa-greedy", None), ("chain-batch32-topp", None),
              ("70b-gqa-medusa", "greedy"), ("longctx-bigvocab", None)]
ATTN_TOL = {"bf16": 2e-2, "f32": 1e-4}
STRICT = dict(accept_band=2e-6, cdf_band=2e-6)   # as the GPU parity tests


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE[0],
                    help="headline workload: tiny-chain-f32, llama7b-medusa-greedy, chain-batch32-topp, "
                         "70b-gqa-medusa, longctx-bigvocab")
    ap.add_argument("--mode", default=None, help="sampling or greedy (default: the workload's own)")
    ap.add_argument("--top-p", type=float, default=None, help="top-p of sampling mode (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-subrecords", action="store_true", help="time the headline workload only")
    ap.add_argument("--profile", action="store_true",
                    help="only warm-up and `steps` back-to-back steps of the headline workload, after the "
                         "parity check (for rocprofv3 traces and counters)")
    ap.add_argument("--cold-iters", type=int, default=20, help="single steps timed after a cache flush")
    ap.add_argument("--flush-bytes", type=int, default=1 << 30, help="bytes written between cold steps")
    ap.add_argument("--lossless-tree", action="store_true",
                    help="time the lossless sibling walk (SPEC_VERIFY_FLAG_LOSSLESS_TREE) as the value")
    ap.add_argument("--paged-block-size", type=int, default=16,
                    help="also time the step with the caches read through a block table of pages of this "
                         "many slots (spec_verify_run_paged); 0 = skip")
    ap.add_argument("--traffic-summary", nargs=5, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "COPY_BYTES"),
                    help="write profiles/traffic_<kernel>_<workload>.json from rocprofv3 --pmc counter CSVs "
                         "(kernel: --kernel)")
    ap.add_argument("--kernel", default="attn_mfma_kernel", help="kernel of --traffic-summary")
    ap.add_argument("--ramp-seconds", type=float, default=0.2,
                    help="untimed steps before each timed part (0 for counter collection)")
    ap.add_argument("--trace-summary", nargs=4, default=None,
                    metavar=("KERNEL_TRACE_CSV", "OUT_MD", "TITLE", "COMMAND"),
                    help="write a markdown summary of a rocprofv3 --kernel-trace csv: duration per "
                         "(kernel, grid) with the command that made it")
    ap.add_argument("--counter-summary", nargs=4, default=None,
                    metavar=("COUNTER_CSV", "OUT_MD", "TITLE", "COMMAND"),
                    help="write a markdown summary of a rocprofv3 --pmc csv (mean per (kernel, grid)), with "
                         "clock and MFMA-pipe share derived from the same dispatches")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="instead of the verify step, run a plain device copy of this many bytes "
                         "(--steps times): the reference kernel for scaling HBM counters")
    return ap.parse_args()


# ------------------------------------------------------------------ algorithmic work

def algorithmic_work(case):
    """Bytes and flops the method itself must move / do, per step.

    Attention per sequence: K and V of the L_b + T visible slots read once, Q read
    and O written once: 2*Hkv*D*e*(L_b+T) + 2*T*Hq*D*e bytes; flops 4*Hq*D per
    visible (query, key) pair, node i seeing L_b + depth(i) + 1 keys.
    Vocabulary: every target row (and every draft row in sampling mode) read once,
    4*V bytes per row.
    """
    spec = case.spec
    e = 2 if spec.dtype == "bf16" else 4
    B, T = case.parent.shape
    attn_bytes = 0
    attn_flops = 0
    for b in range(B):
        L = int(case.kv_len[b])
        attn_bytes += 2 * spec.hkv * spec.head_dim * e * (L + T) + 2 * T * spec.hq * spec.head_dim * e
        depth = [0] * T
        for i in range(1, T):
            depth[i] = depth[int(case.parent[b, i])] + 1
        visible = sum(L + d + 1 for d in depth)
        attn_flops += 4 * spec.hq * spec.head_dim * visible
    rows = T + (T - 1 if spec.mode == "sampling" else 0)
    vocab_bytes = 4 * spec.vocab * rows * B
    return dict(attention_bytes=int(attn_bytes), attention_flops=int(attn_flops), vocab_bytes=int(vocab_bytes))


def acceptance_stats(parent, node_accept, accept_len):
    """Accept-length histogram and the per-depth conditional acceptance rate.

    conditional rate at depth d: among the nodes of depth d whose parent lies on
    an accepted root path, the fraction whose own test passed (the chance a step
    goes one node deeper, given it got to the parent).  "acceptance_rate" is the
    mean accepted length over the deepest depth a tree offers.
    """
    import numpy as np

    parent = np.asarray(parent)
    node_accept = np.asarray(node_accept).astype(bool)
    accept_len = np.asarray(accept_len)
    B, T = parent.shape
    hist = {}
    for a in accept_len.tolist():
        hist[str(int(a))] = hist.get(str(int(a)), 0) + 1
    tried, passed = {}, {}
    max_depth = 0
    for b in range(B):
        acc = [True] + [False] * (T - 1)
        depth = [0] * T
        for i in range(1, T):
            p = int(parent[b, i])
            depth[i] = depth[p] + 1
            acc[i] = bool(node_accept[b, i]) and acc[p]
            if acc[p]:
                tried[depth[i]] = tried.get(depth[i], 0) + 1
                passed[depth[i]] = passed.get(depth[i], 0) + int(bool(node_accept[b, i]))
        max_depth = max(max_depth, max(depth))
    cond = {str(d): passed[d] / tried[d] for d in sorted(tried)}
    return {"accept_len_histogram": dict(sorted(hist.items(), key=lambda kv: int(kv[0]))),
            "mean_accept_len": float(accept_len.mean()),
            "accepted_tokens_per_step": int(accept_len.sum() + B),
            "acceptance_rate": float(accept_len.mean()) / max(max_depth, 1),
            "conditional_acceptance_by_depth": cond,
            "nodes_tested_by_depth": {str(d): tried[d] for d in sorted(tried)}}


def source_hash(kname):
    path = os.path.join(ROOT, "tree_attention_verification_verify_amd", "csrc", KERNEL_SOURCES[kname])
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(kname, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kname, workload))
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha256_16") != source_hash(kname):
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ helpers on the GPU

def upload(case, dev):
    import numpy as np
    import torch

    def up(a, dtype=None):
        a = np.ascontiguousarray(a)
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    spec = case.spec
    return dict(q=up(case.q, spec.dtype), k_cache=up(case.k_cache, spec.dtype), v_cache=up(case.v_cache, spec.dtype),
                kv_len=up(case.kv_len), parent=up(case.parent), tokens=up(case.tokens),
                target_logits=up(case.target_logits),
                draft_logits=None if case.draft_logits is None else up(case.draft_logits),
                u_accept=up(case.u_accept), u_final=up(case.u_final)), up


def handle_cfg(spec, case, **flags):
    B, T = case.parent.shape
    cfg = dict(max_batch=B, max_nodes=T, num_q_heads=spec.hq, num_kv_heads=spec.hkv, head_dim=spec.head_dim,
               kv_capacity=case.k_cache.shape[2], vocab=spec.vocab, dtype=spec.dtype, mode=spec.mode,
               temperature=spec.temperature, top_p=spec.top_p)
    cfg.update(flags)
    return cfg


def to_host(outs):
    import torch

    return {k: (v.float() if v.dtype == torch.bfloat16 else v).cpu().numpy() for k, v in outs.items()}


def parity_check(case, got):
    """The GPU outputs against the oracle on the same inputs (raises SystemExit(3) on a mismatch).

    Every decision and token of every sequence, outside the near-tie band;
    node_p/node_q to relative 1e-4; attention rows of the root and the deepest
    nodes of sequence 0 (all heads) within 2e-2 (bf16) / 1e-4 (fp32)."""
    import numpy as np

    import oracle

    spec = case.spec
    ref = oracle.verify(case, attention=False, **STRICT)
    bad = []
    B, T = case.parent.shape
    for b in range(B):
        if int(got["status"][b]) != int(ref["status"][b]):
            bad.append("status b=%d" % b)
            continue
        near = ref["node_near"][b]
        for i in range(T):
            if not near[i] and got["node_accept"][b, i] != ref["node_accept"][b, i]:
                bad.append("node_accept b=%d i=%d" % (b, i))
        if not (got["row_token"][b] == ref["row_token"][b]).all():
            bad.append("row_token b=%d" % b)
        if spec.mode == "sampling":
            for name in ("node_p", "node_q"):
                g, r = got[name][b, 1:].astype(np.float64), ref[name][b, 1:]
                m = ~near[1:] & (r >= 1e-30)
                if m.any() and (np.abs(g[m] - r[m]) / r[m]).max() > 1e-4:
                    bad.append("%s b=%d" % (name, b))
        if ref["seq_near"][b]:
            continue
        for k in ("accept_len", "final_node", "final_from_residual"):
            if int(got[k][b]) != int(ref[k][b]):
                bad.append("%s b=%d" % (k, b))
        for k in ("path", "out_tokens"):
            if not (got[k][b] == ref[k][b]).all():
                bad.append("%s b=%d" % (k, b))
    d = oracle.depths(case.parent[0])
    nodes = [0] + [i for i in range(T) if d[i] == max(d) and i > 0]
    err = 0.0
    q = oracle.widen(case.q[0], spec.dtype)
    k = oracle.widen(case.k_cache[0], spec.dtype)
    v = oracle.widen(case.v_cache[0], spec.dtype)
    for i in nodes:
        row = oracle.tree_attention_node(q[i], k, v, int(case.kv_len[0]), case.parent[0], i)
        err = max(err, float(np.abs(got["attn_out"][0, i].astype(np.float64) - row).max()))
    if err > ATTN_TOL[spec.dtype]:
        bad.append("attn_out max err %.3g" % err)
    if bad:
        print("bench.py: GPU outputs differ from the oracle on %s: %s" % (spec.name, ", ".join(bad[:10])),
              file=sys.stderr, flush=True)
        raise SystemExit(3)
    return {"ok": True, "sequences": B, "near_tie_sequences": int(ref["seq_near"].sum()),
            "attn_rows_checked": len(nodes) * spec.hq, "attn_max_abs_err": err, "attn_tol": ATTN_TOL[spec.dtype]}


RAMP_SECONDS = 0.2


def clock_ramp(run, seconds=None):
    """Steps for `seconds` of wall time (untimed): brings the GPU out of its idle
    clocks after host-side work (the parity check) before anything is timed."""
    import torch

    seconds = RAMP_SECONDS if seconds is None else seconds
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            run()
        torch.cuda.synchronize()
        n += 10
    return n


def time_back_to_back(run, steps, warmup, stream):
    """Mean ms per step of `steps` back-to-back runs, host clock around a synchronised region."""
    import torch

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_blocks(run, steps, stream, blocks=20):
    """Per-step ms of back-to-back runs in `blocks` blocks, events only between blocks: median and min."""
    import torch

    per = max(1, steps // blocks)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    ev[0].record(stream)
    for j in range(blocks):
        for _ in range(per):
            run()
        ev[j + 1].record(stream)
    ev[-1].synchronize()
    ms = [ev[j].elapsed_time(ev[j + 1]) / per for j in range(blocks)]
    return {"median_ms": statistics.median(ms), "min_ms": min(ms), "blocks": blocks, "steps_per_block": per}


def time_cold(run, iters, flush, stream):
    """Single steps, each after a write of the flush buffer (outside the events): median and min ms."""
    import torch

    ms = []
    pair = []
    for _ in range(iters):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
        # an empty event pair after the same flush: what the two records alone add
        flush.fill_(2)
        e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e2.record(stream)
        e3.record(stream)
        e3.synchronize()
        pair.append(e2.elapsed_time(e3))
    return {"median_ms": statistics.median(ms), "min_ms": min(ms), "iters": iters,
            "flush_bytes": flush.numel() * flush.element_size(), "empty_event_pair_ms": statistics.median(pair)}


def roofline(work, us, spec, kernel):
    """Roofline record of the attention kernel from its own time per launch (us)."""
    t = us * 1e-6
    ai = work["attention_flops"] / work["attention_bytes"]
    if ai > RIDGE and spec.dtype == "bf16":
        achieved = work["attention_flops"] / t / 1e12
        rec = dict(bound="mfma", achieved=achieved, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                   frac=achieved / MFMA_BF16_PEAK_TFLOPS)
    else:
        achieved = work["attention_bytes"] / t / 1e9
        rec = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s", frac=achieved / HBM_PEAK_GBPS)
    rec.update(kernel=kernel, us_per_launch=us, arithmetic_intensity=ai,
               method="the attention alone (handle with SPEC_VERIFY_FLAG_SKIP_VOCAB), back-to-back launches "
                      "between two events on the run's stream")
    return rec


def measure(name, mode, args, headline=False):
    """Every figure of one workload (see the module docstring).  Returns (record, state)."""
    import numpy as np
    import torch

    import synth
    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs

    overrides = {}
    if mode:
        overrides["mode"] = mode
    if headline and args.top_p is not None:
        overrides["top_p"] = args.top_p
    spec = synth.workload(name, **overrides)
    t_gen = time.perf_counter()
    case = synth.make_case(spec)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda")
    ins, up = upload(case, dev)
    B, T = case.parent.shape
    stream = torch.cuda.current_stream()
    lossless = bool(headline and args.lossless_tree and spec.mode == "sampling")
    cfg = handle_cfg(spec, case, lossless_tree=lossless)
    outs = allocate_outputs(B, T, spec.hq, spec.head_dim, spec.dtype)
    work = algorithmic_work(case)
    rec = {"workload": name, "mode": spec.mode, "batch": B, "nodes": T, "q_heads": spec.hq, "kv_heads": spec.hkv,
           "head_dim": spec.head_dim, "prefix": int(case.kv_len.max()), "vocab": spec.vocab,
           "temperature": spec.temperature, "top_p": spec.top_p, "dtype": spec.dtype,
           "tree_rule": "lossless sibling walk" if lossless else "independent per-node test"}
    with SpecVerify(**cfg) as sv:
        plan = sv.describe(B, T)
        run = sv.prepare(ins, outs, stream)      # checked and marshalled once
        for _ in range(max(args.warmup, 1)):
            run()
        torch.cuda.synchronize()
        got = to_host(outs)
        rec["parity"] = parity_check(case, got)       # before any timing; exits on a mismatch
        ramp = clock_ramp(run)
        if args.profile:
            ms = time_back_to_back(run, args.steps, 0, stream)
            return dict(rec, ms_per_step=ms, value=B * T / (ms * 1e-3), plan=plan), None
        ms = time_back_to_back(run, args.steps, args.warmup, stream)
        warm = time_blocks(run, args.steps, stream)
        flush = torch.empty(args.flush_bytes // 4, dtype=torch.int32, device=dev)
        cold = time_cold(run, args.cold_iters, flush, stream)
        del flush
    rec.update(plan=plan, value=B * T / (ms * 1e-3), unit="candidate tokens/s", ms_per_step=ms,
               warm=warm, cold=cold, clock_ramp_steps=ramp, input_generation_s=t_gen)

    # per-stage event times (events around each launch: each record adds a gap, so these
    # are upper bounds on the kernels' own times)
    with SpecVerify(timing=True, **cfg) as sv:
        trun = sv.prepare(ins, outs, stream)
        clock_ramp(trun)
        for _ in range(args.warmup):
            trun()
        torch.cuda.synchronize()
        sv.timing_read()
        for _ in range(args.steps):
            trun()
        torch.cuda.synchronize()
        stage_ms, nruns = sv.timing_read()
    stage = {k: v / max(nruns, 1) for k, v in stage_ms.items()}
    rec["stage_ms_per_launch_with_events"] = stage

    # the attention alone, back to back (kernel time per launch for the roofline)
    acfg = dict(cfg, skip_vocab=True, lossless_tree=False)
    aouts = dict(attn_out=torch.empty_like(outs["attn_out"]))
    with SpecVerify(**acfg) as sv:
        aplan = sv.describe(B, T)
        arun = sv.prepare(ins, aouts, stream)
        clock_ramp(arun)
        for _ in range(args.warmup):
            arun()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            arun()
        e1.record(stream)
        e1.synchronize()
        attn_us = e0.elapsed_time(e1) * 1e3 / args.steps
        same = bool(torch.equal(aouts["attn_out"], outs["attn_out"]))
    kernels = [aplan["attention"]] + (["finish_kernel (split merge)"] if aplan["merge"] else [])
    roof = roofline(work, attn_us, spec, aplan["attention"])
    roof["launches_timed"] = kernels
    roof["traffic"] = measured_traffic(aplan["attention"], "%s-%s" % (name, spec.mode))
    rec["roofline"] = roof
    rec["attention_alone_equals_full_run"] = same
    vocab_ms = stage["vocab"]
    step_bytes = work["attention_bytes"] + work["vocab_bytes"]
    rec["hbm"] = dict(step_GBps=step_bytes / (ms * 1e-3) / 1e9,
                      step_frac=step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                      attention_GBps=work["attention_bytes"] / (attn_us * 1e-6) / 1e9,
                      attention_TFLOPs=work["attention_flops"] / (attn_us * 1e-6) / 1e12,
                      vocab_kernel=plan["vocab"],
                      vocab_GBps_with_events=work["vocab_bytes"] / (vocab_ms * 1e-3) / 1e9,
                      vocab_frac_with_events=work["vocab_bytes"] / (vocab_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                      algorithmic_bytes_per_step=step_bytes, attention_bytes_per_step=work["attention_bytes"],
                      vocab_bytes_per_step=work["vocab_bytes"], attention_flops_per_step=work["attention_flops"])
    rec["acceptance"] = acceptance_stats(case.parent, got["node_accept"], got["accept_len"])
    return rec, dict(case=case, ins=ins, outs=outs, got=got, cfg=cfg, up=up, spec=spec, stream=stream)


# ------------------------------------------------------------------ headline extras

def time_graph(st, args):
    """The step captured once in a HIP graph and replayed; every replay checked against eager."""
    import torch

    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs

    case, ins, outs, cfg, spec = st["case"], st["ins"], st["outs"], st["cfg"], st["spec"]
    B, T = case.parent.shape
    with SpecVerify(**cfg) as sv:
        gouts = allocate_outputs(B, T, spec.hq, spec.head_dim, spec.dtype)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                sv.run(ins, gouts)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sv.run(ins, gouts)
        torch.cuda.synchronize()
        equal = True
        for _ in range(3):
            for v in gouts.values():
                v.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            equal &= all(bool(torch.equal(gouts[k], outs[k])) for k in outs)
        clock_ramp(g.replay)
        gms = time_back_to_back(g.replay, args.steps, args.warmup, st["stream"])
        del g
    return {"ms_per_step": gms, "value": B * T / (gms * 1e-3), "replays_equal_eager": bool(equal)}


def time_commit(st, args):
    """KV commit of the step's accepted paths: events around the call; kv_len restored each time."""
    import numpy as np
    import torch

    from tree_attention_verification_verify_amd import SpecVerify

    case, ins, outs, cfg, spec, stream = st["case"], st["ins"], st["outs"], st["cfg"], st["spec"], st["stream"]
    B, T = case.parent.shape
    with SpecVerify(**cfg) as sv:
        sv.run(ins, outs, stream)
        kl0 = ins["kv_len"].clone()
        kl = kl0.clone()
        total_ms, reps = 0.0, max(args.steps // 4, 10)
        for rep in range(reps + 3):
            kl.copy_(kl0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            sv.commit(ins["k_cache"], ins["v_cache"], kl, outs["path"], outs["accept_len"], outs["final_node"],
                      stream)
            e1.record(stream)
            e1.synchronize()
            if rep >= 3:
                total_ms += e0.elapsed_time(e1)
        path_np = outs["path"].cpu().numpy()
        acc_np = outs["accept_len"].cpu().numpy()
    moved = sum(int((path_np[b, 1:acc_np[b] + 1] != np.arange(1, acc_np[b] + 1)).sum()) for b in range(B))
    elem = 2 if spec.dtype == "bf16" else 4
    nbytes = moved * spec.hkv * spec.head_dim * elem * 2 * 2     # K and V, read and write
    us = total_ms * 1e3 / reps
    # the caches were modified in place: restore them
    ins["k_cache"].copy_(st["up"](case.k_cache, spec.dtype))
    ins["v_cache"].copy_(st["up"](case.v_cache, spec.dtype))
    return {"us_per_call": us, "rows_moved": moved, "bytes_moved": nbytes,
            "GBps": nbytes / (us * 1e-6) / 1e9 if us > 0 else None}


def time_other_rule(st, args):
    """The other tree rule (sampling) on the same inputs: step time and accepted tokens."""
    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs

    case, ins, cfg, spec, stream = st["case"], st["ins"], st["cfg"], st["spec"], st["stream"]
    B, T = case.parent.shape
    ocfg = dict(cfg, lossless_tree=not cfg.get("lossless_tree", False))
    oouts = allocate_outputs(B, T, spec.hq, spec.head_dim, spec.dtype)
    with SpecVerify(**ocfg) as sv:
        plan = sv.describe(B, T)
        orun = sv.prepare(ins, oouts, stream)
        clock_ramp(orun)
        ms = time_back_to_back(orun, args.steps, args.warmup, stream)
    acc = oouts["accept_len"].cpu().numpy()
    return {"rule": "lossless sibling walk" if ocfg["lossless_tree"] else "independent per-node test",
            "plan": plan, "value": B * T / (ms * 1e-3), "ms_per_step": ms,
            "accepted_tokens_per_step": int(acc.sum() + B)}


def time_paged(st, args):
    """The step with the caches read through a block table (pages scattered in a shuffled pool)."""
    import torch

    import synth
    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs, paged_kv

    case, ins, outs, cfg, spec, stream, up = (st[k] for k in ("case", "ins", "outs", "cfg", "spec", "stream", "up"))
    B, T = case.parent.shape
    _, pg = synth.page_case(case, args.paged_block_size, seed=(1,))
    pool_k, pool_v, table = up(pg.k_pool, spec.dtype), up(pg.v_pool, spec.dtype), up(pg.block_table)
    pk = paged_kv(pool_k, pool_v, table)
    pins = {k: v for k, v in ins.items() if k not in ("k_cache", "v_cache")}
    pcfg = dict(cfg, kv_capacity=pg.capacity)
    pouts = allocate_outputs(B, T, spec.hq, spec.head_dim, spec.dtype)
    with SpecVerify(**pcfg) as sv:
        prun = sv.prepare(pins, pouts, stream, paged=pk)
        clock_ramp(prun)
        ms = time_back_to_back(prun, args.steps, args.warmup, stream)
    same = all(bool(torch.equal(pouts[k], outs[k])) for k in outs)
    return {"block_size": args.paged_block_size, "pages": int(pg.num_blocks), "value": B * T / (ms * 1e-3),
            "ms_per_step": ms, "outputs_equal_dense": same}


def time_tree_build(spec, B, args, stream):
    """Candidate-tree construction (spec_verify_build_tree) for the workload's tree shape:
    per-depth top-k of B x depth logits rows (seeded N(0, 3^2)) and the template fill."""
    import ctypes

    import numpy as np
    import torch

    from tree_attention_verification_verify_amd import SpecVerify, binding, spec_verify_tree_template

    caps, T = spec.tree[1], spec.tree[2]
    parent_t, rank_t = spec_verify_tree_template(caps, T)
    depth = len(caps)
    rng = np.random.default_rng(2024)
    lg = torch.from_numpy(rng.normal(0.0, 3.0, size=(B, depth, spec.vocab)).astype(np.float32)).cuda()
    root = torch.zeros(B, dtype=torch.int32, device="cuda")
    par = torch.empty((B, T), dtype=torch.int32, device="cuda")
    tok = torch.empty((B, T), dtype=torch.int32, device="cuda")
    cfg = dict(max_batch=B, max_nodes=T, num_q_heads=spec.hq, num_kv_heads=spec.hkv, head_dim=spec.head_dim,
               kv_capacity=spec.kv_capacity, vocab=spec.vocab, dtype=spec.dtype, mode=spec.mode,
               temperature=spec.temperature, top_p=spec.top_p)
    lib = binding.load_library()
    tp = (ctypes.c_int32 * T)(*parent_t)
    tr = (ctypes.c_int32 * T)(*rank_t)
    targs = binding.TreeArgs(lg.data_ptr(), root.data_ptr(), ctypes.cast(tp, ctypes.c_void_p),
                             ctypes.cast(tr, ctypes.c_void_p), par.data_ptr(), tok.data_ptr(), B, T, depth)
    sh = ctypes.c_void_p(stream.cuda_stream)
    with SpecVerify(**cfg) as sv:
        for _ in range(10):
            sv.build_tree(lg, root, parent_t, rank_t, par, tok, stream)
        torch.cuda.synchronize()
        # prebuilt arguments: the host stays ahead of the kernels
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            lib.spec_verify_build_tree(sv.handle, ctypes.byref(targs), sh)
        e1.record(stream)
        e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    nbytes = B * depth * spec.vocab * 4
    return {"caps": list(caps), "nodes": T, "rows": B * depth, "us_per_call": us, "bytes_read": nbytes,
            "GBps": nbytes / (us * 1e-6) / 1e9}


def cpu_baseline(case, min_seconds=10.0):
    """The oracle, as it stands, on the first sequences of the same workload: one
    sequence at a time until `min_seconds` of CPU work or the whole batch."""
    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    seqs, dt = 0, 0.0
    while seqs < case.parent.shape[0] and dt < min_seconds:
        t0 = time.perf_counter()
        oracle.verify(case, attention=True, seqs=[seqs])
        dt += time.perf_counter() - t0
        seqs += 1
    T = case.parent.shape[1]
    return dict(value=seqs * T / dt, unit="candidate tokens/s", cores=int(threads), kind="oracle",
                sample="sequences 0..%d of %d (%d nodes, prefix %d, vocab %d each): attention + vocab + "
                       "acceptance + selection, %.1f s" % (seqs - 1, case.parent.shape[0], T,
                                                           int(case.kv_len[0]), case.spec.vocab, dt),
                seconds=dt, blas_threads=int(threads), host_cpu_count=os.cpu_count())


# ------------------------------------------------------------------ counters and probes

def copy_probe(nbytes, steps):
    import torch

    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_probe_bytes": nbytes, "ms_per_copy": dt * 1e3,
                      "GBps_read_plus_write": 2 * nbytes / dt / 1e9}))


def _counter_per_dispatch(csv_path, kernel_prefix, counter):
    """Mean value of `counter` over the dispatches of kernels whose name starts with kernel_prefix."""
    import csv

    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(csv_path))
            if r["Counter_Name"] == counter and
            r["Kernel_Name"].replace("void ", "").replace("sv::(anonymous namespace)::", "").startswith(kernel_prefix)]
    if not vals:
        raise SystemExit("no %s records for %s in %s" % (counter, kernel_prefix, csv_path))
    return sum(vals) / len(vals), len(vals)


def traffic_summary(paths, workload, kname):
    """Write the HBM traffic record of one kernel from rocprofv3 --pmc counter CSVs.

    paths: FETCH_SIZE csv and WRITE_SIZE csv of a bench run, then FETCH_SIZE and
    WRITE_SIZE csvs of the copy probe and the probe's byte count.  FETCH_SIZE and
    WRITE_SIZE are in KiB per dispatch; each is scaled by the ratio of the copy's
    known bytes to what the same counter reads for the copy.
    """
    fetch_csv, write_csv, cfetch_csv, cwrite_csv, copy_bytes = paths
    copy_bytes = int(copy_bytes)
    fetch_kib, nf = _counter_per_dispatch(fetch_csv, kname, "FETCH_SIZE")
    write_kib, nw = _counter_per_dispatch(write_csv, kname, "WRITE_SIZE")
    cf_kib, _ = _counter_per_dispatch(cfetch_csv, "__amd_rocclr_copyBuffer", "FETCH_SIZE")
    cw_kib, _ = _counter_per_dispatch(cwrite_csv, "__amd_rocclr_copyBuffer", "WRITE_SIZE")
    f_scale = copy_bytes / (cf_kib * 1024.0)
    w_scale = copy_bytes / (cw_kib * 1024.0)
    read_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    rec = {"kernel": kname, "workload": workload, "source": KERNEL_SOURCES[kname],
           "source_sha256_16": source_hash(kname),
           "fetch_kib_per_dispatch": fetch_kib, "write_kib_per_dispatch": write_kib,
           "dispatches": [nf, nw], "copy_probe_bytes": copy_bytes,
           "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_read_bytes_per_launch": read_b, "hbm_write_bytes_per_launch": write_b,
           "hbm_bytes_per_launch": read_b + write_b}
    out = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (kname, workload))
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def _short(name):
    name = name.replace("void ", "").replace("sv::(anonymous namespace)::", "")
    return name if len(name) <= 90 else name[:87] + "..."


def _trace_rows(path):
    """(kernel, grid threads) -> list of durations in us, from a rocprofv3 kernel-trace csv."""
    import csv

    groups = {}
    for r in csv.DictReader(open(path)):
        grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0)
        key = (_short(r["Kernel_Name"]), grid)
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return groups


def trace_summary(csv_path, out_md, title, command):
    groups = _trace_rows(csv_path)
    total = sum(sum(v) for v in groups.values())
    rows = sorted(groups.items(), key=lambda kv: -sum(kv[1]))
    lines = ["# Kernel trace: %s" % title, "",
             "Command (on the MI355X, from the repository root, with `TMPDIR=/tmp`):", "", "```", command, "```", "",
             "Per (kernel, grid size in threads), from the per-dispatch records of `run_kernel_trace.csv`",
             "(durations in microseconds; written by `python3 bench.py --trace-summary`):", "",
             "| kernel | grid | calls | median us | mean us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|---|---|"]
    for (name, grid), d in rows[:16]:
        lines.append("| `%s` | %d | %d | %.2f | %.2f | %.2f | %.2f | %.1f |" % (
            name, grid, len(d), statistics.median(d), sum(d) / len(d), min(d), max(d), 100.0 * sum(d) / total))
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("wrote", out_md)


def counter_summary(csv_path, out_md, title, command, n_xcd=8, n_simd=1024):
    """Mean counters per (kernel, grid) of a rocprofv3 --pmc csv.  Derived, from the same
    dispatches: clock = GRBM_GUI_ACTIVE / XCDs / dispatch duration (the counter sums the XCDs;
    the duration is the dispatch's own, under counter collection); MFMA pipe share =
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDs x SIMDs); VALU per MFMA."""
    import csv

    vals, durs = {}, {}
    for r in csv.DictReader(open(csv_path)):
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
        vals.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        durs.setdefault(key, {})[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    lines = ["# Counters: %s" % title, "", "Command (on the MI355X, from the repository root, with `TMPDIR=/tmp`):",
             "", "```", command, "```", "",
             "Mean per dispatch, per (kernel, grid size in threads); written by `python3 bench.py --counter-summary`.",
             "Derived from the same dispatches (durations under counter collection): MFMA rate = SQ_INSTS_MFMA x "
             "32768 / duration; for dispatches of 100 us or more, clock = GRBM_GUI_ACTIVE / %d XCDs / duration "
             "and MFMA pipe share = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d x %d SIMDs); VALU per "
             "MFMA = SQ_INSTS_VALU / SQ_INSTS_MFMA." % (n_xcd, n_xcd, n_simd), ""]
    order = sorted(vals.items(), key=lambda kv: -sum(durs[kv[0]].values()))
    for (name, grid), cs in order[:4]:
        d = list(durs[(name, grid)].values())
        lines += ["## `%s`, grid %d" % (name, grid), "", "| counter | mean per dispatch | dispatches |", "|---|---|---|"]
        mean = {c: sum(v) / len(v) for c, v in cs.items()}
        for c in sorted(cs):
            lines.append("| %s | %.6g | %d |" % (c, mean[c], len(cs[c])))
        dur = sum(d) / len(d)
        lines.append("| duration (us) | %.2f | %d |" % (dur, len(d)))
        if mean.get("SQ_INSTS_MFMA", 0) > 0:
            # every MFMA of these kernels is v_mfma_f32_32x32x16_bf16: 32768 flops per wave instruction
            lines.append("| MFMA rate (TFLOP/s, 32768 flops per instruction) | %.1f | |"
                         % (mean["SQ_INSTS_MFMA"] * 32768 / (dur * 1e-6) / 1e12))
        if "GRBM_GUI_ACTIVE" in mean and dur >= 100.0:
            # the GRBM window holds the collection's setup around the dispatch: an upper
            # bound on the clock (and a lower bound on the pipe share), close for long kernels
            cyc = mean["GRBM_GUI_ACTIVE"] / n_xcd
            lines.append("| clock (GHz, upper bound) | %.3f | |" % (cyc / (dur * 1e3)))
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                lines.append("| MFMA pipe share (lower bound) | %.3f | |"
                             % (mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * n_simd)))
        if mean.get("SQ_INSTS_MFMA", 0) > 0 and "SQ_INSTS_VALU" in mean:
            lines.append("| VALU per MFMA | %.2f | |" % (mean["SQ_INSTS_VALU"] / mean["SQ_INSTS_MFMA"]))
        if mean.get("SQ_WAVE_CYCLES", 0) > 0:
            # all three count quad-cycles of resident waves, summed over the waves
            for c, what in (("SQ_WAIT_ANY", "waiting for anything"),
                            ("SQ_WAIT_INST_ANY", "waiting for an instruction to issue"),
                            ("SQ_WAIT_INST_LDS", "waiting for an LDS instruction to issue")):
                if c in mean:
                    lines.append("| share of wave cycles %s (%s / SQ_WAVE_CYCLES) | %.3f | |"
                                 % (what, c, mean[c] / mean["SQ_WAVE_CYCLES"]))
        if "GRBM_GUI_ACTIVE" in mean and dur >= 100.0:
            cyc = mean["GRBM_GUI_ACTIVE"] / n_xcd
            if "SQ_INSTS_LDS_LOAD_BANDWIDTH" in mean:   # counts 64-byte units loaded from LDS
                lines.append("| LDS bytes loaded per CU-cycle (SQ_INSTS_LDS_LOAD_BANDWIDTH x 64 / cycles / %d CUs) "
                             "| %.1f | |" % (n_simd // 4, mean["SQ_INSTS_LDS_LOAD_BANDWIDTH"] * 64 / cyc / (n_simd // 4)))
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in mean:
                lines.append("| share of SIMD cycles with a VALU issue beside a busy MFMA pipe "
                             "(SQ_VALU_MFMA_COEXEC_CYCLES / cycles / %d SIMDs) | %.3f | |"
                             % (n_simd, mean["SQ_VALU_MFMA_COEXEC_CYCLES"] / (cyc * n_simd)))
        lines.append("")
    open(out_md, "w").write("\n".join(lines) + "\n")
    print("wrote", out_md)


def main():
    global RAMP_SECONDS
    args = parse()
    RAMP_SECONDS = args.ramp_seconds
    if args.trace_summary:
        trace_summary(*args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(*args.counter_summary)
        return
    if args.traffic_summary:
        import synth
        spec = synth.workload(args.workload, **({"mode": args.mode} if args.mode else {}))
        label = "%s-%s" % (args.workload, spec.mode)
        if args.top_p is not None:   # a top-p setting other than the workload's own
            label = "%s-topp%g-%s" % (args.workload, args.top_p, spec.mode)
        traffic_summary(args.traffic_summary, label, args.kernel)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs the verify step on one GPU only; --gpus %d is not supported "
              "(sequences would shard across GPUs with no exchange, so one GPU's throughput is the unit)"
              % args.gpus)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return

    from tree_attention_verification_verify_amd import load_library

    load_library()   # fail loudly if the HIP library is missing
    head, st = measure(args.workload, args.mode, args, headline=True)
    if args.profile:
        print(json.dumps(head))
        return
    spec, case, B, T = st["spec"], st["case"], st["case"].parent.shape[0], st["case"].parent.shape[1]
    result = {
        "metric": "verified candidate tokens/sec + achieved HBM GB/s vs peak (verify step)",
        "value": head["value"],
        "unit": "candidate tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": "%s tree verify" % args.workload, "mode": spec.mode, "batch": B, "nodes": T,
                   "q_heads": spec.hq, "kv_heads": spec.hkv, "head_dim": spec.head_dim,
                   "prefix": int(case.kv_len.max()), "vocab": spec.vocab, "temperature": spec.temperature,
                   "top_p": spec.top_p},
        "roofline": head["roofline"],
        "hbm": head["hbm"],
        "warm": head["warm"], "cold": head["cold"], "clock_ramp_steps": head["clock_ramp_steps"],
        "stage_ms_per_launch_with_events": head["stage_ms_per_launch_with_events"],
        "acceptance": head["acceptance"],
        "parity": head["parity"],
        "plan": head["plan"],
        "tree_rule": head["tree_rule"],
    }
    result["hip_graph"] = time_graph(st, args)
    result["kv_commit"] = time_commit(st, args)
    if spec.mode == "sampling":
        result["other_tree_rule"] = time_other_rule(st, args)
    if spec.tree[0] == "medusa":
        result["tree_build"] = time_tree_build(spec, B, args, st["stream"])
    if args.paged_block_size:
        result["paged_kv"] = time_paged(st, args)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case)
    result["input_generation_s"] = head["input_generation_s"]
    del st
    if not args.no_subrecords:
        import torch

        subs = []
        for name, mode in SUBRECORDS:
            if name == args.workload and (mode or None) == (args.mode or None):
                continue
            rec, sst = measure(name, mode, args)
            del sst
            torch.cuda.empty_cache()
            subs.append(rec)
        result["configs"] = subs
    print(json.dumps(result))


if __name__ == "__main__":
    main()
