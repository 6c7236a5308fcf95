#!/usr/bin/env python3
"""Verify-step benchmark on one MI355X.

One step = one spec_verify_run over a batch of synthetic inputs already resident
in HBM: tree attention + split merge + vocab pass + selection.  The default
workload is the 70B-shaped GQA Medusa-tree verify (batch 8, 64 query / 8 KV
heads x 128, prefix 8192, 64-node tree, vocab 32000) in sampling mode.

Prints one JSON line: verified candidate tokens/s (B*T per step), the roofline
of the dominant kernel (HIP events on the run's stream), HBM GB/s of the whole
step, and the CPU oracle timed on a bounded sample of the same workload.
"""
import argparse
import hashlib
import json
import os
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
                  "row_stats_topp_chunked_kernel": "vocab_stats.hip", "finish_kernel": "select_final.hip"}
VOCAB_CHUNK = 32768   # vocabulary ids one row workgroup holds on chip (kVocabChunk)


def stage_kernel(stage, spec):
    """The kernel a stage launches for this workload, by the library's own dispatch rule.

    Attention: the MFMA kernel when bf16 and the g*T query rows sharing one KV head
    number at least 16; below that the tiled VALU kernel for at most 8 rows whose K/V
    rows are 128 or 256 bytes, else the one-wave VALU kernel.  Row statistics: with
    top-p in sampling mode, the row held on chip up to VOCAB_CHUNK ids and streamed
    above; otherwise the streaming kernel.
    """
    if stage == "attention":
        rows = spec.hq // spec.hkv * spec.nodes
        if spec.dtype == "bf16" and rows >= 16:
            return "attn_mfma_kernel"
        rowb = spec.head_dim * (2 if spec.dtype == "bf16" else 4)
        return "attn_valu_tiled_kernel" if rows <= 8 and rowb in (128, 256) else "attn_valu_kernel"
    if stage == "vocab":
        if spec.mode == "sampling" and spec.top_p < 1.0:
            return "row_stats_topp_kernel" if spec.vocab <= VOCAB_CHUNK else "row_stats_topp_chunked_kernel"
        return "row_stats_stream_kernel"
    return "finish_kernel"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="70b-gqa-medusa",
                    help="one of: tiny-chain-f32, llama7b-medusa-greedy, chain-batch32-topp, "
                         "70b-gqa-medusa, longctx-bigvocab")
    ap.add_argument("--mode", default=None, help="sampling or greedy (default: the workload's own)")
    ap.add_argument("--top-p", type=float, default=None, help="top-p of sampling mode (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--lossless-tree", action="store_true",
                    help="time the lossless sibling walk (SPEC_VERIFY_FLAG_LOSSLESS_TREE) as the value")
    ap.add_argument("--paged-block-size", type=int, default=16,
                    help="also time the step with the caches read through a block table of pages of this "
                         "many slots (spec_verify_run_paged); 0 = skip")
    ap.add_argument("--traffic-summary", nargs=5, default=None,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV", "COPY_BYTES"),
                    help="write profiles/traffic_<kernel>_<workload>.json from rocprofv3 --pmc counter CSVs")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="instead of the verify step, run a plain device copy of this many bytes "
                         "(--steps times): the reference kernel for scaling HBM counters")
    return ap.parse_args()


def algorithmic_work(case):
    """Bytes and flops the method itself must move / do, per step (see the design notes)."""
    spec = case.spec
    e = 2 if spec.dtype == "bf16" else 4
    B, T = case.parent.shape
    attn_bytes = 0
    attn_flops = 0
    for b in range(B):
        L = int(case.kv_len[b])
        attn_bytes += 2 * spec.hkv * spec.head_dim * e * (L + T) + 2 * T * spec.hq * spec.head_dim * e
        depth = [0] * T          # node i sees the prefix and its depth(i) + 1 root-path nodes
        for i in range(1, T):
            depth[i] = depth[int(case.parent[b, i])] + 1
        visible = sum(L + d + 1 for d in depth)
        attn_flops += 4 * spec.hq * spec.head_dim * visible
    rows = T + (T - 1 if spec.mode == "sampling" else 0)
    vocab_bytes = 4 * spec.vocab * rows * B
    return dict(attention_bytes=int(attn_bytes), attention_flops=int(attn_flops), vocab_bytes=int(vocab_bytes))


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


def cpu_baseline(case, got, min_seconds=10.0):
    """The oracle, as it stands, on the first sequences of the same workload:
    one sequence at a time until `min_seconds` of CPU work or the whole batch.

    Also a parity spot check of those sequences against the GPU run.
    """
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    seqs, parts, dt = [], [], 0.0
    while len(seqs) < case.parent.shape[0] and dt < min_seconds:
        t0 = time.perf_counter()
        parts.append(oracle.verify(case, attention=True, seqs=[len(seqs)]))
        dt += time.perf_counter() - t0
        seqs.append(len(seqs))
    ref = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    T = case.parent.shape[1]
    ok = True
    err = 0.0
    for n, b in enumerate(seqs):
        if not ref["seq_near"][n] and int(ref["status"][n]) == 0:
            ok &= int(got["accept_len"][b]) == int(ref["accept_len"][n])
            ok &= bool((got["out_tokens"][b] == ref["out_tokens"][n]).all())
        err = max(err, float(np.abs(got["attn_out"][b].astype(np.float64) - ref["attn_out"][n]).max()))
    ok &= err <= (2e-2 if case.spec.dtype == "bf16" else 1e-4)
    return dict(value=len(seqs) * T / dt, unit="candidate tokens/s", cores=int(threads), kind="oracle",
                sample="sequences 0..%d of %d (%d nodes, prefix %d, vocab %d each): attention + vocab + "
                       "acceptance + selection, %.1f s" % (len(seqs) - 1, case.parent.shape[0], T,
                                                           int(case.kv_len[0]), case.spec.vocab, dt),
                seconds=dt), ok, err


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


def time_tree_build(spec, B, steps, stream):
    """Candidate-tree construction (spec_verify_build_tree) for the workload's tree shape:
    per-depth top-k of B x depth logits rows (seeded N(0, 3^2)) and the template fill."""
    import numpy as np
    import torch

    from tree_attention_verification_verify_amd import SpecVerify, spec_verify_tree_template

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
    import ctypes

    from tree_attention_verification_verify_amd import binding

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
        for _ in range(steps):
            lib.spec_verify_build_tree(sv.handle, ctypes.byref(targs), sh)
        e1.record(stream)
        e1.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = B * depth * spec.vocab * 4
    return {"caps": list(caps), "nodes": T, "rows": B * depth, "us_per_call": us, "bytes_read": nbytes,
            "GBps": nbytes / (us * 1e-6) / 1e9}


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


def main():
    args = parse()
    if args.traffic_summary:
        import synth
        spec = synth.workload(args.workload, **({"mode": args.mode} if args.mode else {}))
        traffic_summary(args.traffic_summary, "%s-%s" % (args.workload, spec.mode), stage_kernel("attention", spec))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs the verify step on one GPU only; --gpus %d is not supported "
              "(sequences would shard across GPUs with no exchange, so one GPU's throughput is the unit)"
              % args.gpus)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return

    import numpy as np
    import torch

    import synth
    from tree_attention_verification_verify_amd import SpecVerify, allocate_outputs, load_library

    load_library()   # fail loudly if the HIP library is missing
    overrides = {}
    if args.mode:
        overrides["mode"] = args.mode
    if args.top_p is not None:
        overrides["top_p"] = args.top_p
    spec = synth.workload(args.workload, **overrides)
    t_gen = time.perf_counter()
    case = synth.make_case(spec)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda")

    def up(a, dtype=None):
        a = np.ascontiguousarray(a)
        if dtype == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    ins = dict(q=up(case.q, spec.dtype), k_cache=up(case.k_cache, spec.dtype), v_cache=up(case.v_cache, spec.dtype),
               kv_len=up(case.kv_len), parent=up(case.parent), tokens=up(case.tokens),
               target_logits=up(case.target_logits),
               draft_logits=None if case.draft_logits is None else up(case.draft_logits),
               u_accept=up(case.u_accept), u_final=up(case.u_final))
    B, T = case.parent.shape
    outs = allocate_outputs(B, T, spec.hq, spec.head_dim, spec.dtype)
    cfg = dict(max_batch=B, max_nodes=T, num_q_heads=spec.hq, num_kv_heads=spec.hkv, head_dim=spec.head_dim,
               kv_capacity=spec.kv_capacity, vocab=spec.vocab, dtype=spec.dtype, mode=spec.mode,
               temperature=spec.temperature, top_p=spec.top_p,
               lossless_tree=bool(args.lossless_tree and spec.mode == "sampling"))
    stream = torch.cuda.current_stream()
    work = algorithmic_work(case)

    # Steps with HIP events around every kernel: per-kernel durations.  Run
    # first, so that they also bring the GPU out of its idle clocks before the
    # value is timed.
    with SpecVerify(timing=True, **cfg) as sv:
        for _ in range(args.warmup):
            sv.run(ins, outs, stream)
        torch.cuda.synchronize()
        sv.timing_read()                     # discard warm-up records
        t2 = time.perf_counter()
        for _ in range(args.steps):
            sv.run(ins, outs, stream)
        torch.cuda.synchronize()
        ms_with_events = (time.perf_counter() - t2) * 1e3 / args.steps
        stage_ms, nruns = sv.timing_read()

    # timed steps (the value): back-to-back runs, nothing else on the stream
    with SpecVerify(timing=False, **cfg) as sv:
        for _ in range(args.warmup):
            sv.run(ins, outs, stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            sv.run(ins, outs, stream)
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # the same step captured once in a HIP graph (its three launches) and
    # replayed: every replay is checked against the eager outputs above, with
    # the outputs cleared in between
    graph = None
    with SpecVerify(timing=False, **cfg) as sv:
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
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t5 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t5) * 1e3 / args.steps
        graph = {"ms_per_step": gms, "value": B * T / (gms * 1e-3), "replays_equal_eager": bool(equal)}
        del g

    per_launch = {k: v / max(nruns, 1) for k, v in stage_ms.items()}

    # KV commit of the accepted paths (spec_verify_commit) on this step's outputs: events
    # around the call alone; kv_len is restored before each call
    commit = None
    with SpecVerify(timing=False, **cfg) as sv:
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
        commit = {"us_per_call": us, "rows_moved": moved, "bytes_moved": nbytes,
                  "GBps": nbytes / (us * 1e-6) / 1e9 if us > 0 else None}
    # the caches were modified in place: restore them for any later use of `ins`
    ins["k_cache"].copy_(up(case.k_cache, spec.dtype))
    ins["v_cache"].copy_(up(case.v_cache, spec.dtype))

    # the other tree rule on the same inputs (sampling): its step time and finishing stage
    other = None
    if spec.mode == "sampling":
        ocfg = dict(cfg, lossless_tree=not cfg["lossless_tree"])
        oouts = allocate_outputs(B, T, spec.hq, spec.head_dim, spec.dtype)
        with SpecVerify(timing=True, **ocfg) as sv:
            for _ in range(args.warmup):
                sv.run(ins, oouts, stream)
            torch.cuda.synchronize()
            sv.timing_read()
            for _ in range(args.steps):
                sv.run(ins, oouts, stream)
            torch.cuda.synchronize()
            oms, on = sv.timing_read()
        with SpecVerify(timing=False, **ocfg) as sv:
            for _ in range(args.warmup):
                sv.run(ins, oouts, stream)
            torch.cuda.synchronize()
            t3 = time.perf_counter()
            for _ in range(args.steps):
                sv.run(ins, oouts, stream)
            torch.cuda.synchronize()
            oms_step = (time.perf_counter() - t3) * 1e3 / args.steps
        ores = {k: v.cpu().numpy() for k, v in oouts.items() if k in ("accept_len",)}
        other = {"rule": "lossless sibling walk" if ocfg["lossless_tree"] else "independent per-node test",
                 "value": B * T / (oms_step * 1e-3), "ms_per_step": oms_step,
                 "stage_ms_per_launch": {k: v / max(on, 1) for k, v in oms.items()},
                 "accepted_tokens_per_step": int(ores["accept_len"].sum() + B)}
    torch.cuda.synchronize()
    got = {k: v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy() for k, v in outs.items()}

    # the same step with the caches read through a block table: pages of the
    # given size scattered over a pool in random order (spec_verify_run_paged)
    paged = None
    if args.paged_block_size:
        from tree_attention_verification_verify_amd import paged_kv

        _, pg = synth.page_case(case, args.paged_block_size, seed=(1,))
        pool_k, pool_v, table = up(pg.k_pool, spec.dtype), up(pg.v_pool, spec.dtype), up(pg.block_table)
        pk = paged_kv(pool_k, pool_v, table)
        pins = {k: v for k, v in ins.items() if k not in ("k_cache", "v_cache")}
        pcfg = dict(cfg, kv_capacity=max(cfg["kv_capacity"], pg.capacity))
        pouts = allocate_outputs(B, T, spec.hq, spec.head_dim, spec.dtype)
        with SpecVerify(timing=True, **pcfg) as sv:
            for _ in range(args.warmup):
                sv.run_paged(pins, pk, pouts, stream)
            torch.cuda.synchronize()
            sv.timing_read()
            for _ in range(args.steps):
                sv.run_paged(pins, pk, pouts, stream)
            torch.cuda.synchronize()
            pms, pn = sv.timing_read()
        with SpecVerify(timing=False, **pcfg) as sv:
            for _ in range(args.warmup):
                sv.run_paged(pins, pk, pouts, stream)
            torch.cuda.synchronize()
            t4 = time.perf_counter()
            for _ in range(args.steps):
                sv.run_paged(pins, pk, pouts, stream)
            torch.cuda.synchronize()
            pms_step = (time.perf_counter() - t4) * 1e3 / args.steps
        same = all(bool(torch.equal(pouts[k], outs[k])) for k in outs)
        paged = {"block_size": args.paged_block_size, "pages": int(pg.num_blocks),
                 "value": B * T / (pms_step * 1e-3), "ms_per_step": pms_step,
                 "stage_ms_per_launch": {k: v / max(pn, 1) for k, v in pms.items()},
                 "outputs_equal_dense": same}
        del pool_k, pool_v, table

    workload = "%s-%s" % (args.workload, spec.mode)
    # dominant kernel by measured time
    dominant = max(("attention", "vocab"), key=lambda k: per_launch[k])
    if dominant == "attention":
        ai = work["attention_flops"] / work["attention_bytes"]
        t = per_launch["attention"] * 1e-3
        if ai > RIDGE and spec.dtype == "bf16":
            achieved = work["attention_flops"] / t / 1e12
            roof = dict(bound="mfma", achieved=achieved, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                        frac=achieved / MFMA_BF16_PEAK_TFLOPS)
        else:
            achieved = work["attention_bytes"] / t / 1e9
            roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=achieved / HBM_PEAK_GBPS)
    else:
        achieved = work["vocab_bytes"] / (per_launch["vocab"] * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s", frac=achieved / HBM_PEAK_GBPS)
    roof["kernel"] = stage_kernel(dominant, spec)
    roof["ms_per_launch"] = per_launch[dominant]
    roof["traffic"] = measured_traffic(roof["kernel"], workload)

    step_bytes = work["attention_bytes"] + work["vocab_bytes"]
    attn_t = per_launch["attention"] * 1e-3
    hbm = dict(step_GBps=step_bytes / (ms_per_step * 1e-3) / 1e9,
               step_frac=step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               attention_GBps=work["attention_bytes"] / attn_t / 1e9,
               attention_TFLOPs=work["attention_flops"] / attn_t / 1e12,
               vocab_GBps=work["vocab_bytes"] / (per_launch["vocab"] * 1e-3) / 1e9,
               vocab_frac=work["vocab_bytes"] / (per_launch["vocab"] * 1e-3) / 1e9 / HBM_PEAK_GBPS,
               algorithmic_bytes_per_step=step_bytes, attention_flops_per_step=work["attention_flops"])

    result = {
        "metric": "verified candidate tokens/sec + achieved HBM GB/s vs peak (verify step)",
        "value": B * T / (ms_per_step * 1e-3),
        "unit": "candidate tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": "%s tree verify" % args.workload, "mode": spec.mode, "batch": B, "nodes": T,
                   "q_heads": spec.hq, "kv_heads": spec.hkv, "head_dim": spec.head_dim,
                   "prefix": int(case.kv_len.max()), "vocab": spec.vocab, "temperature": spec.temperature,
                   "top_p": spec.top_p},
        "roofline": roof,
        "hbm": hbm,
        "stage_ms_per_launch": per_launch,
        "ms_per_step_with_event_records": ms_with_events,
        "accepted_tokens_per_step": int(got["accept_len"].sum() + B),
        "tree_rule": "lossless sibling walk" if cfg["lossless_tree"] else "independent per-node test",
    }
    if other is not None:
        result["other_tree_rule"] = other
    result["hip_graph"] = graph
    result["kv_commit"] = commit
    if spec.tree[0] == "medusa":
        result["tree_build"] = time_tree_build(spec, B, args.steps, stream)
    if paged is not None:
        result["paged_kv"] = paged
    if not args.no_cpu_baseline:
        base, ok, err = cpu_baseline(case, got)
        result["cpu_baseline"] = base
        result["parity_sample"] = {"ok": bool(ok), "attn_max_abs_err": err}
    result["input_generation_s"] = t_gen
    print(json.dumps(result))


if __name__ == "__main__":
    main()
