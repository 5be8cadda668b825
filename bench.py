"""Benchmark of the MLA + DSA decode hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload dsa_decode|paged_decode|prefill]

One step of the default workload is a full DSA decode step at T = 131072 cached tokens,
batch 1, GLM-5.2-like heads (64 heads, kv_lora 512, qk_rope 64, qk_nope 192, v_head 256,
32 indexer heads of width 128, top-2048): RoPE on the query tail, lightning-indexer scores
over every cached key, top-k selection, absorbed decode over the selected keys.  Inputs are
seeded synthetic data already resident in HBM; they rotate over several copies so that no
step finds its data in the 256 MB Infinity Cache.  Steps are replayed from HIP graphs
(one per input copy) so host launch overhead stays out of the timed region.

Output: one JSON line (metric, value, roofline of the dominant kernel, CPU-oracle baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3   # dense fp32 matrix-core rate
METRIC = "MLA+DSA decode keys·heads/sec at T=128k; achieved HBM GB/s vs peak"
IDX_KERNEL = "index_scores_mfma<0, false"   # the stand-alone indexer (no selection histogram)


def _src_hash(path):
    """SHA-256 (16 hex digits) of a source file's code: line comments and blank lines left out, so
    that a comment edit does not mark counters taken on the same code as stale."""
    code = []
    for line in open(path, encoding="utf-8"):
        line = line.split("//", 1)[0].rstrip()
        if line:
            code.append(line)
    return hashlib.sha256("\n".join(code).encode()).hexdigest()[:16]


def _traffic(counters_name: str, kernel: str):
    """HBM bytes per launch of one kernel (read + write, calibrated) from the committed counter
    summary, if the summary was taken on the current source of the kernel's file; otherwise None."""
    p = os.path.join(ROOT, "profiles", f"{counters_name}.counters.txt")
    if not os.path.exists(p):
        return None
    sec, kv = None, {}
    for line in open(p):
        line = line.strip()
        if line.startswith("[") and line.endswith("]"):
            sec = line[1:-1]
            continue
        m = re.match(r"^(\w+)\s*=\s*(\S+)", line)
        if m and sec == kernel:
            kv[m.group(1)] = m.group(2)
    src = kv.get("source")
    if not src or kv.get("source_sha256_16") != _src_hash(os.path.join(ROOT, src)):
        return None
    try:
        return float(kv["hbm_read_bytes_per_launch"]) + float(kv["hbm_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _kernel_source(kernel: str):
    """The library source file that defines a kernel (name up to its template arguments)."""
    base = kernel.split("<")[0].split("(")[0].strip()
    csrc = os.path.join(ROOT, "mla_latent_kv_dsa_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith(".hip") and re.search(r"void\s+" + re.escape(base) + r"\s*\(",
                                            open(os.path.join(csrc, f)).read()):
            return os.path.join("mla_latent_kv_dsa_amd", "csrc", f)
    return None


def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


# ----------------------------------------------------------------------------- decode
def bench_dsa_decode(args):
    import numpy as np
    import torch

    import mla_latent_kv_dsa_amd as mla
    from mla_latent_kv_dsa_amd import synth

    dev = torch.device("cuda:0")
    T, B, H, NOPE, ROPE, V, L = 131072, 1, synth.H, synth.QK_NOPE, synth.QK_ROPE, synth.V_HEAD, synth.KV_LORA
    N_IH, HD, K = synth.N_IH, synth.INDEX_HD, synth.TOPK
    sm = 1.0 / math.sqrt(NOPE + ROPE)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    d = synth.decode(3, T, B=B, dsa=True)
    copies = []
    g = torch.Generator(device=dev)
    g.manual_seed(1003)
    for c in range(args.copies):
        if c == 0:
            # the indexer pool in the 64-row tiled layout (same rows; the indexer's fast layout)
            lc, rc, ic = bf(d.lc), bf(d.rc), torch.from_numpy(synth.tile_index_keys(d.ic)).to(dev)
            qn, qr, kvb = bf(d.q_nope), bf(d.q_rope), bf(d.kv_b)
            qi, wi = torch.from_numpy(d.q_idx).to(dev), torch.from_numpy(d.w_idx).to(dev)
        else:
            rn = lambda *s, std=1.0: torch.randn(*s, generator=g, device=dev) * std
            lc, rc, ic = rn(T, L).bfloat16(), rn(T, ROPE).bfloat16(), rn(T, HD)
            qn, qr, kvb = rn(B, H, NOPE).bfloat16(), rn(B, H, ROPE).bfloat16(), rn(H * (NOPE + V), L, std=0.02).bfloat16()
            qi, wi = rn(B, N_IH, HD), rn(B, N_IH)
        seq_len = torch.full((B,), T, dtype=torch.int32, device=dev)
        kv = mla.KvCache(lc, rc, ic, seq_len=seq_len, max_seq_len=T, seq_stride=T, ic_layout=mla.MLA_IC_TILE64)
        copies.append(dict(kv=kv, qn=qn, qr=qr, kvb=kvb, qi=qi, wi=wi, seq_len=seq_len,
                           pos=torch.full((B,), T - 1, dtype=torch.int32, device=dev),
                           scores=torch.empty((B, T), dtype=torch.float32, device=dev),
                           sel=torch.empty((B, K), dtype=torch.int32, device=dev),
                           nsel=torch.empty((B,), dtype=torch.int32, device=dev),
                           out=torch.empty((B, H, V), dtype=torch.float32, device=dev)))
    step_need = mla.mla_dsa_decode_workspace_bytes(H, NOPE, ROPE, V, L, B, T, K)
    tk_need = mla.dsa_topk_workspace_bytes(B, T, K)
    sel_need = mla.dsa_index_select_workspace_bytes(B, T, K)
    dec_need = mla.mla_decode_workspace_bytes(H, NOPE, ROPE, V, L, B, K)
    for c in copies:
        c["tk_ws"] = torch.empty(max(tk_need, 1), dtype=torch.uint8, device=dev)
        c["sel_ws"] = torch.empty(max(sel_need, 1), dtype=torch.uint8, device=dev)
        c["dec_ws"] = torch.empty(max(dec_need, 1), dtype=torch.uint8, device=dev)
        c["step_ws"] = torch.empty(max(step_need, 1), dtype=torch.uint8, device=dev)

    def rope(c):
        mla.mla_rope_interleave(c["qr"], c["pos"], 0, ROPE)

    def index(c):
        mla.dsa_index_scores(c["qi"], c["wi"], c["kv"], T, scores=c["scores"])

    def topk(c):
        mla.dsa_topk_select(c["scores"], c["seq_len"], K, sel=c["sel"], nsel=c["nsel"], ws=c["tk_ws"])

    def select(c):
        mla.dsa_index_select(c["qi"], c["wi"], c["kv"], T, K, scores=c["scores"], sel=c["sel"], nsel=c["nsel"],
                             ws=c["sel_ws"])

    def absorb(c):
        mla.mla_decode_absorb(c["qn"], c["kvb"], c["dec_ws"], qk_rope=ROPE)

    def attend(c):
        mla.mla_decode_attend(c["qr"], c["kvb"], c["kv"], NOPE, sm, c["dec_ws"], sel=c["sel"], nsel=c["nsel"],
                              out=c["out"])

    def step(c):
        # the whole hot path in one call: RoPE of the query tail at T-1, indexer + top-k,
        # absorbed attention over the selected keys (the query absorption and the rotation
        # run beside the selection's final pass)
        mla.mla_dsa_decode(c["qn"], c["qr"], c["qi"], c["wi"], c["kvb"], c["kv"], T, K, sm, scores=c["scores"],
                           sel=c["sel"], nsel=c["nsel"], out=c["out"], ws=c["step_ws"])

    def separate(c):
        # the same step as four calls (RoPE in place, so only for the per-part timing)
        rope(c)
        select(c)
        absorb(c)
        attend(c)

    # eager reference of one step on copy 0 (q_rope is rotated in place, so keep a copy)
    qr0 = copies[0]["qr"].clone()
    step(copies[0])
    torch.cuda.synchronize()
    ref_sel, ref_out = copies[0]["sel"].clone(), copies[0]["out"].clone()
    copies[0]["qr"].copy_(qr0)

    graphs = []
    if not args.no_graph:
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(s):
            for c in copies:
                step(c)                       # warm the allocator-free path on this stream
        torch.cuda.current_stream(dev).wait_stream(s)
        torch.cuda.synchronize()
        copies[0]["qr"].copy_(qr0)
        for c in copies:
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(c)
            graphs.append(gr)
        # one graph with a step on every input copy, so that the per-replay launch cost is
        # shared by len(copies) steps (as it is when a decode graph holds many layers)
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for c in copies:
                step(c)
        torch.cuda.synchronize()
        copies[0]["qr"].copy_(qr0)
        graphs[0].replay()
        torch.cuda.synchronize()
        assert torch.equal(copies[0]["sel"], ref_sel), "graph replay selection differs from eager"
        assert torch.equal(copies[0]["out"], ref_out), "graph replay output differs from eager"
        g_all.replay()
        torch.cuda.synchronize()
        assert torch.equal(copies[0]["sel"], ref_sel), "graph replay selection differs from eager"
        assert torch.equal(copies[0]["out"], ref_out), "graph replay output differs from eager"

    def run_steps(n, i0=0):
        """Exactly n steps: whole replays of the all-copies graph, then single-step graphs."""
        if not graphs:
            for i in range(n):
                step(copies[(i0 + i) % len(copies)])
            return
        full, rest = divmod(n, len(copies))
        for _ in range(full):
            g_all.replay()
        for i in range(rest):
            graphs[i].replay()

    def time_steps(n, single):
        e0, e1 = _events(torch, 2)
        t = time.perf_counter()
        e0.record()
        if single:
            for i in range(n):
                graphs[i % len(graphs)].replay()
        else:
            run_steps(n)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n, time.perf_counter() - t

    run_steps(args.warmup)
    torch.cuda.synchronize()
    ms_step, t_wall = time_steps(args.steps, False)
    ms_step_single = time_steps(args.steps, True)[0] if graphs else None

    # per-kernel durations: each part alone, captured back to back over every input copy
    # (REPS passes) in one HIP graph, replayed between two events on the launch stream
    parts = {"rope": rope, "select": select, "absorb": absorb, "attend": attend, "index": index, "topk": topk,
             "separate_calls": separate, "fused_step": step}
    us = {}
    REPS = 4
    for k, f in parts.items():
        if graphs:
            gk = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gk):
                for _ in range(REPS):
                    for c in copies:
                        f(c)
            launch = gk.replay
            per = REPS * len(copies)
        else:
            def launch(f=f):
                for c in copies:
                    f(c)
            per = len(copies)
        launch()
        torch.cuda.synchronize()
        n_rep = max(3, args.steps // per)
        e0, e1 = _events(torch, 2)
        e0.record()
        for _ in range(n_rep):
            launch()
        e1.record()
        torch.cuda.synchronize()
        us[k] = e0.elapsed_time(e1) * 1e3 / (n_rep * per)

    keys_heads = T * H * B
    value = keys_heads / (ms_step * 1e-3)
    ic_bytes = T * HD * 4
    score_bytes = T * 4
    q_bytes = N_IH * HD * 4 + N_IH * 4
    idx_bytes = ic_bytes + score_bytes + q_bytes
    idx_gbs = idx_bytes / (us["index"] * 1e-6) / 1e9
    sel_kv_bytes = K * (L + ROPE) * 2
    kvb_bytes = H * (NOPE + V) * L * 2
    step_bytes = ic_bytes + sel_kv_bytes + kvb_bytes + score_bytes + B * H * (NOPE + ROPE) * 2 + B * H * V * 4
    stream_bytes = ic_bytes + sel_kv_bytes
    stream_us = ms_step * 1e3   # the fused step: indexer, selection and attention (RoPE and absorb hidden)
    traffic = _traffic("dsa_decode_T131072_B1", IDX_KERNEL)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline_decode(d, T, K, sm)
    extra = {}
    if not args.no_extra:   # the batched paged and dense decode configurations, and the prefill
        extra["batched_paged_B32"] = bench_batched_paged(args)
        extra["dense_decode_T4096"] = bench_dense_decode(args)
        extra["prefill_S4096"] = measure_prefill(args, cpu=not args.no_cpu)
        extra.update(bench_new_rows(args))

    line = {
        "metric": METRIC, "value": value, "unit": "keys·heads/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "dsa_decode_T131072_B1", "T": T, "B": B, "heads": H, "qk_nope": NOPE,
                   "qk_rope": ROPE, "v_head": V, "kv_lora": L, "index_heads": N_IH, "index_hd": HD,
                   "topk": K, "kv_dtype": "bf16", "index_dtype": "fp32", "index_layout": "tile64",
                   "input_copies": args.copies,
                   "hip_graphs": bool(graphs), "steps_per_graph_replay": len(copies) if graphs else 0},
        "roofline": {"kernel": IDX_KERNEL + " (dsa_index_scores; the step runs the same kernel with the "
                               "selection histogram added)",
                     "bound": "hbm", "achieved": idx_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": idx_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": idx_bytes, "avg_us": us["index"],
                     # the whole step against the same peak: the bytes that must stream (Ic and the
                     # selected latent rows) over the fused step's time
                     "stream_over_step": {"bytes": stream_bytes, "us": stream_us,
                                          "frac": stream_bytes / (stream_us * 1e-6) / 1e9 / HBM_PEAK_GBS}},
        "cpu_baseline": cpu,
        "breakdown_us": us,
        "stream": {"bytes": stream_bytes, "us_step": stream_us,
                   "GBs": stream_bytes / (stream_us * 1e-6) / 1e9,
                   "frac": stream_bytes / (stream_us * 1e-6) / 1e9 / HBM_PEAK_GBS},
        "whole_step": {"bytes": step_bytes, "GBs": step_bytes / (ms_step * 1e-3) / 1e9,
                       "frac": step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "wall_s_timed": t_wall,
        "ms_per_step_one_graph_per_step": ms_step_single,
        "extra_configs": extra,
    }
    print(json.dumps(line), flush=True)


def _graph_time(torch, fn, warmup, steps, per=8):
    """Mean ms per call of fn captured in a HIP graph, `per` calls back to back per replay (so the
    gap between replays is spread over them, as between the calls of a decode loop), events on
    the stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(per):
            fn()
    for _ in range(warmup):
        gr.replay()
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(steps):
        gr.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (steps * per)


def bench_batched_paged(args):
    """The batched paged decode step (32 sequences, lengths ~ U{8192..131072}, 64-token blocks
    in a seeded random physical order, every sequence past k so DSA is on everywhere): one
    mla_dsa_decode call per step.  Lengths and block table from synth.paged_batch's draws; pool
    and query values from synth.paged_values_torch (drawn on the GPU, seeded, same
    distributions).  The 3.4 GB of pools exceed the Infinity Cache, so no input rotation is
    needed."""
    import torch

    import mla_latent_kv_dsa_amd as mla
    from mla_latent_kv_dsa_amd import synth

    dev = torch.device("cuda:0")
    H, NOPE, ROPE, V, L = synth.H, synth.QK_NOPE, synth.QK_ROPE, synth.V_HEAD, synth.KV_LORA
    N_IH, HD, K = synth.N_IH, synth.INDEX_HD, synth.TOPK
    pb = synth.paged_batch(5, meta_only=True)
    B, T = pb.B, pb.max_blocks * pb.block_size
    d = synth.paged_values_torch(pb, 1005, dev)
    qn, qr, kvb, qi, wi = d["q_nope"], d["q_rope"], d["kv_b"], d["q_idx"], d["w_idx"]
    ic = synth.tile_index_keys(d.pop("ic"))
    seq_len = torch.from_numpy(pb.seq_len).to(dev)
    bt = torch.from_numpy(pb.block_table).to(dev)
    kv = mla.KvCache(d["lc"], d["rc"], ic, seq_len=seq_len, max_seq_len=T, block_table=bt, block_size=pb.block_size,
                     ic_layout=mla.MLA_IC_TILE64)
    sm = 1.0 / math.sqrt(NOPE + ROPE)
    scores = torch.empty((B, T), dtype=torch.float32, device=dev)
    sel = torch.empty((B, K), dtype=torch.int32, device=dev)
    nsel = torch.empty((B,), dtype=torch.int32, device=dev)
    out = torch.empty((B, H, V), dtype=torch.float32, device=dev)
    ws = torch.empty(mla.mla_dsa_decode_workspace_bytes(H, NOPE, ROPE, V, L, B, T, K), dtype=torch.uint8, device=dev)

    def step():
        mla.mla_dsa_decode(qn, qr, qi, wi, kvb, kv, T, K, sm, scores=scores, sel=sel, nsel=nsel, out=out, ws=ws)

    def index():
        mla.dsa_index_scores(qi, wi, kv, T, scores=scores)

    ms = _graph_time(torch, step, 3, 20, per=1)
    ms_idx = _graph_time(torch, index, 3, 20, per=1)
    sum_t = int(pb.seq_len.sum())
    keys_heads = sum_t * H
    ic_bytes = sum_t * HD * 4
    sel_kv = B * K * (L + ROPE) * 2
    kvb_bytes = H * (NOPE + V) * L * 2
    stream = ic_bytes + sel_kv
    whole = stream + kvb_bytes + sum_t * 4 + B * H * (NOPE + ROPE) * 2 + B * H * V * 4
    idx_bytes = ic_bytes + sum_t * 4 + B * N_IH * (HD + 1) * 4
    gbs = lambda nbytes, m: nbytes / (m * 1e-3) / 1e9
    return {"workload": "dsa_decode_paged_B32", "B": B, "sum_seq_len": sum_t, "block_size": pb.block_size,
            "seq_len_range": [int(pb.seq_len.min()), int(pb.seq_len.max())], "topk": K, "index_layout": "tile64",
            "ms_per_step": ms, "keys_heads_per_s": keys_heads / (ms * 1e-3),
            "stream": {"bytes": stream, "GBs": gbs(stream, ms), "frac": gbs(stream, ms) / HBM_PEAK_GBS},
            "whole_step": {"bytes": whole, "GBs": gbs(whole, ms), "frac": gbs(whole, ms) / HBM_PEAK_GBS},
            "indexer": {"ms": ms_idx, "algorithmic_bytes": idx_bytes, "GBs": gbs(idx_bytes, ms_idx),
                        "frac": gbs(idx_bytes, ms_idx) / HBM_PEAK_GBS},
            "data": "synthetic: lengths and block permutation from numpy seed 5, values torch seed 1005"}


def bench_dense_decode(args):
    """Dense absorbed decode at T = 4096 (B = 1, no selection): mla_absorbed_decode over every
    causal key, one call per step, over 16 rotated input copies (34 MB each) so that no step
    finds its inputs in the Infinity Cache."""
    import torch

    import mla_latent_kv_dsa_amd as mla
    from mla_latent_kv_dsa_amd import synth

    dev = torch.device("cuda:0")
    H, NOPE, ROPE, V, L = synth.H, synth.QK_NOPE, synth.QK_ROPE, synth.V_HEAD, synth.KV_LORA
    T, B, NC = 4096, 1, 16
    g = torch.Generator(device=dev)
    g.manual_seed(1002)
    rn = lambda *shape, std=1.0: torch.randn(*shape, generator=g, device=dev) * std
    sm = 1.0 / math.sqrt(NOPE + ROPE)
    cps = []
    for _ in range(NC):
        kv = mla.KvCache(rn(T, L).bfloat16(), rn(T, ROPE).bfloat16(),
                         seq_len=torch.full((B,), T, dtype=torch.int32, device=dev), max_seq_len=T, seq_stride=T)
        cps.append(dict(kv=kv, qn=rn(B, H, NOPE).bfloat16(), qr=rn(B, H, ROPE).bfloat16(),
                        kvb=rn(H * (NOPE + V), L, std=0.02).bfloat16(),
                        out=torch.empty((B, H, V), dtype=torch.float32, device=dev),
                        ws=torch.empty(mla.mla_decode_workspace_bytes(H, NOPE, ROPE, V, L, B, T), dtype=torch.uint8,
                                       device=dev)))

    def step_all():
        for c in cps:
            mla.mla_absorbed_decode(c["qn"], c["qr"], c["kvb"], c["kv"], sm, out=c["out"], ws=c["ws"])

    ms = _graph_time(torch, step_all, 3, 10, per=1) / NC
    kv_bytes = T * (L + ROPE) * 2
    kvb_bytes = H * (NOPE + V) * L * 2
    whole = kv_bytes + kvb_bytes + B * H * (NOPE + ROPE) * 2 + B * H * V * 4
    gbs = lambda nbytes: nbytes / (ms * 1e-3) / 1e9
    return {"workload": "dense_decode_T4096_B1", "T": T, "ms_per_step": ms, "keys_heads_per_s": T * H / (ms * 1e-3),
            "whole_step": {"bytes": whole, "GBs": gbs(whole), "frac": gbs(whole) / HBM_PEAK_GBS},
            "kv_core": {"bytes": kv_bytes, "GBs": gbs(kv_bytes), "frac": gbs(kv_bytes) / HBM_PEAK_GBS},
            "input_copies": NC, "data": "synthetic: torch seed 1002"}


def _host_cores():
    """Host cores this process may run on (the OpenMP team of the all-cores oracle run)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _oracle_timed(fn, reps, threads):
    """Median wall time of fn() over reps runs with the oracle's OpenMP team set to threads."""
    import oracle

    oracle._load()
    keep = oracle.num_threads()
    oracle.set_num_threads(threads)
    try:
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
    finally:
        oracle.set_num_threads(keep)
    return statistics.median(times)


def _time_fn(torch, fn, warmup, steps):
    """Mean ms per call of fn() from events on the current stream (eager launches)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_new_rows(args):
    """The cache-write side, the DSA-shared layer, multi-query absorbed decode (S = 4 draft queries at
    T = 131072 with their own top-2048) and DSA in prefill (S = T = 4096, top-2048 per query), each with
    its algorithmic bytes or flops against the HBM or bf16 matrix-core peak."""
    import numpy as np
    import torch

    import mla_latent_kv_dsa_amd as mla
    from mla_latent_kv_dsa_amd import synth

    dev = torch.device("cuda:0")
    H, NOPE, ROPE, V, L = synth.H, synth.QK_NOPE, synth.QK_ROPE, synth.V_HEAD, synth.KV_LORA
    N_IH, HD, K = synth.N_IH, synth.INDEX_HD, synth.TOPK
    sm = 1.0 / math.sqrt(NOPE + ROPE)
    g = torch.Generator(device=dev)
    g.manual_seed(1009)
    rn = lambda *shape, std=1.0: torch.randn(*shape, generator=g, device=dev) * std
    res = {}

    # cache write: 4096 new tokens (a prefill's append) into 64-token paged pools, tiled indexer keys
    n, bs = 4096, 64
    nb = 2 * n // bs
    pools = dict(lc=torch.zeros(nb * bs, L, dtype=torch.bfloat16, device=dev),
                 rc=torch.zeros(nb * bs, ROPE, dtype=torch.bfloat16, device=dev),
                 ic=torch.zeros(nb * bs, HD, dtype=torch.float32, device=dev))
    bt = torch.randperm(nb, generator=g, device=dev).to(torch.int32)[None]
    kv = mla.KvCache(pools["lc"], pools["rc"], pools["ic"], max_seq_len=nb * bs, block_table=bt, block_size=bs,
                     ic_layout=mla.MLA_IC_TILE64)
    comp, ik = rn(n, L + ROPE).bfloat16(), rn(n, HD).bfloat16()
    seq = torch.zeros(n, dtype=torch.int32, device=dev)
    pos = torch.arange(n, dtype=torch.int32, device=dev) + 1000
    ms = _time_fn(torch, lambda: mla.mla_cache_write(comp, seq, pos, kv, 1, ik=ik, ix_rope_off=HD - ROPE,
                                                     ix_rope_dim=ROPE), 3, 50)
    nbytes = n * ((L + ROPE) * 2 + HD * 2 + 8 + L * 2 + ROPE * 2 + HD * 4)
    res["cache_write_4096_tokens"] = {
        "ms": ms, "bytes": nbytes, "GBs": nbytes / (ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "work": "4096 tokens: read comp (576 bf16) + ik (128 bf16) + seq/pos, write Lc/Rc (bf16) + Ic (fp32, tile64)"}

    # RoPE of a prefill's queries: the qk_rope tails of 4096 tokens x 64 heads, in place
    qp = rn(n, H, NOPE + ROPE).bfloat16()
    posq = torch.arange(n, dtype=torch.int32, device=dev) + 1000
    ms = _time_fn(torch, lambda: mla.mla_rope_interleave(qp, posq, NOPE, ROPE), 3, 50)
    nbytes = 2 * n * H * ROPE * 2 + 4 * n   # the tails read and written, the positions
    res["rope_prefill_queries_4096_tokens"] = {
        "ms": ms, "bytes": nbytes, "GBs": nbytes / (ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "work": "4096 tokens x 64 heads: the 64-wide tail of each 256-wide bf16 query rotated in place"}
    del qp

    # one 131072-token sequence, its DSA selection (as the full layer of the step computes it)
    T = 131072
    lc, rc = rn(T, L).bfloat16(), rn(T, ROPE).bfloat16()
    ic = rn(T, HD)
    sl = torch.full((1,), T, dtype=torch.int32, device=dev)
    kvT = mla.KvCache(lc, rc, synth.tile_index_keys(ic), seq_len=sl, max_seq_len=T, seq_stride=T,
                      ic_layout=mla.MLA_IC_TILE64)
    qi, wi = rn(1, N_IH, HD), rn(1, N_IH)
    qn, qr, kvb = rn(1, H, NOPE).bfloat16(), rn(1, H, ROPE).bfloat16(), rn(H * (NOPE + V), L, std=0.02).bfloat16()
    _, _, sel, nsel = mla.mla_dsa_decode(qn, qr, qi, wi, kvb, kvT, T, K, sm)
    ws = torch.empty(mla.mla_decode_workspace_bytes(H, NOPE, ROPE, V, L, 1, K) + (1 << 20), dtype=torch.uint8,
                     device=dev)
    out = torch.empty(1, H, V, dtype=torch.float32, device=dev)
    ms = _graph_time(torch, lambda: mla.mla_dsa_decode_shared(qn, qr, kvb, kvT, sel, nsel, sm, out=out, ws=ws),
                     3, 50)
    sel_bytes = K * (L + ROPE) * 2
    kvb_bytes = H * (NOPE + V) * L * 2
    res["shared_layer_T131072"] = {
        "ms": ms, "keys_heads_per_s": T * H / (ms * 1e-3),
        "bytes": sel_bytes + kvb_bytes, "GBs": (sel_bytes + kvb_bytes) / (ms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "frac": (sel_bytes + kvb_bytes) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        "work": "reuses the full layer's top-2048: RoPE, absorb (W_UK), attention over 2048 rows, W_UV"}

    # multi-query absorbed decode: 4 draft queries at positions T-4 .. T-1, each with its own top-2048
    S = 4
    q4 = rn(S, H, NOPE + ROPE).bfloat16()
    qi4, wi4 = rn(S, N_IH, HD), rn(S, N_IH)
    kv4 = mla.KvCache(lc, rc, synth.tile_index_keys(ic), max_seq_len=T, seq_stride=T, ic_layout=mla.MLA_IC_TILE64)
    sc4 = torch.empty(S, T, dtype=torch.float32, device=dev)
    sel4 = torch.empty(S, K, dtype=torch.int32, device=dev)
    nsel4 = torch.empty(S, dtype=torch.int32, device=dev)
    ws_s = torch.empty(mla.lib().dsa_prefill_select_workspace_bytes(S, T - S, K), dtype=torch.uint8, device=dev)
    out4 = torch.empty(S, H, V, dtype=torch.float32, device=dev)
    d4 = mla._dims(H, NOPE, ROPE, V, L)
    import ctypes
    ws_a = torch.empty(mla.lib().mla_attention_workspace_bytes(ctypes.byref(d4), S, T - S, K, -1), dtype=torch.uint8,
                       device=dev)

    def mq_step():
        mla.dsa_prefill_select(qi4, wi4, kv4, T - S, K, scores=sc4, sel=sel4, nsel=nsel4, ws=ws_s)
        mla.mla_attention(q4, kvb, kv4, NOPE, T - S, sm, g_absorb=-1, sel=sel4, nsel=nsel4, out=out4, ws=ws_a)
    ms = _graph_time(torch, mq_step, 3, 30)
    ms_attn = _graph_time(torch, lambda: mla.mla_attention(q4, kvb, kv4, NOPE, T - S, sm, g_absorb=-1, sel=sel4,
                                                           nsel=nsel4, out=out4, ws=ws_a), 3, 30)
    kh = sum(T - S + i + 1 for i in range(S)) * H
    # Ic once (the queries share their keys) plus every query's selected rows
    stream = T * HD * 4 + S * sel_bytes
    ix_flops = 2.0 * N_IH * HD * sum(T - S + i + 1 for i in range(S))
    ms_sel = ms - ms_attn
    res["multi_query_decode_S4_T131072"] = {
        "ms": ms, "keys_heads_per_s": kh / (ms * 1e-3), "ms_attention_only": ms_attn, "ms_selection": ms_sel,
        "stream_bytes": stream, "stream_frac": stream / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"kernel": "the selection (indexer fp32 products over the 4 queries, top-k)", "bound": "mfma",
                     "achieved": ix_flops / (ms_sel * 1e-3) / 1e12, "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": ix_flops / (ms_sel * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, "algorithmic_flops": ix_flops},
        "work": "4 queries, each: indexer over its causal keys + top-2048 (dsa_prefill_select), absorbed attention "
                "over its selection (mla_attention, g_absorb auto); the indexer reads each key tile once per two "
                "queries, its fixed-order fp32 products bound it"}

    # DSA in prefill: S = T = 4096, top-2048 per query
    S = T4 = 4096
    p_lc, p_rc = rn(T4, L).bfloat16(), rn(T4, ROPE).bfloat16()
    p_ic = rn(T4, HD)
    kvp = mla.KvCache(p_lc, p_rc, synth.tile_index_keys(p_ic), max_seq_len=T4, seq_stride=T4,
                      ic_layout=mla.MLA_IC_TILE64)
    qp = rn(S, H, NOPE + ROPE).bfloat16()
    qip, wip = rn(S, N_IH, HD), rn(S, N_IH)
    scp = torch.empty(S, T4, dtype=torch.float32, device=dev)
    selp = torch.empty(S, K, dtype=torch.int32, device=dev)
    nselp = torch.empty(S, dtype=torch.int32, device=dev)
    ws_p = torch.empty(mla.lib().dsa_prefill_select_workspace_bytes(S, 0, K), dtype=torch.uint8, device=dev)
    outp = torch.empty(S, H, V, dtype=torch.float32, device=dev)
    ms_sel = _time_fn(torch, lambda: mla.dsa_prefill_select(qip, wip, kvp, 0, K, scores=scp, sel=selp, nsel=nselp,
                                                            ws=ws_p), 2, 5)
    pairs = sum(min(i + 1, K) for i in range(S))
    f_attn = 2 * H * pairs * (NOPE + ROPE + V)
    f_kvb = 2 * T4 * H * (NOPE + V) * L
    f_idx = 2 * N_IH * HD * (S * (S + 1) // 2)
    dsa = {"ms_select": ms_sel, "indexer_flops_fp32": f_idx, "selected_pairs": pairs,
           "work": "per query i: indexer over keys 0..i, top-2048, attention over its selection"}
    for gab, name in ((0, "nonabsorbed"), (1, "absorbed")):
        d_p = mla._dims(H, NOPE, ROPE, V, L)
        ws_x = torch.empty(mla.lib().mla_attention_workspace_bytes(ctypes.byref(d_p), S, 0, K, gab), dtype=torch.uint8,
                           device=dev)
        ms = _time_fn(torch, lambda: mla.mla_attention(qp, kvb, kvp, NOPE, 0, sm, g_absorb=gab, sel=selp, nsel=nselp,
                                                       out=outp, ws=ws_x), 2, 5)
        fl = f_attn + (f_kvb if gab == 0 else 0)
        dsa[name] = {"ms_attention": ms, "algorithmic_flops": fl, "TFLOPs": fl / (ms * 1e-3) / 1e12,
                     "roofline": {"bound": "mfma", "frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}}
    res["dsa_prefill_S4096"] = dsa

    # the decode step at T = 131072 with a quantized kv_b, per format; three input copies rotated
    cps = []
    for c in range(3):
        kvc = mla.KvCache(rn(T, L).bfloat16(), rn(T, ROPE).bfloat16(), synth.tile_index_keys(rn(T, HD)), seq_len=sl,
                          max_seq_len=T, seq_stride=T, ic_layout=mla.MLA_IC_TILE64)
        cps.append(dict(kv=kvc, qn=rn(1, H, NOPE).bfloat16(), qr=rn(1, H, ROPE).bfloat16(), qi=rn(1, N_IH, HD),
                        wi=rn(1, N_IH), sc=torch.empty(1, T, device=dev), sel=torch.empty(1, K, dtype=torch.int32,
                                                                                            device=dev),
                        nsel=torch.empty(1, dtype=torch.int32, device=dev), out=torch.empty(1, H, V, device=dev),
                        ws=torch.empty(mla.mla_dsa_decode_workspace_bytes(H, NOPE, ROPE, V, L, 1, T, K),
                                       dtype=torch.uint8, device=dev)))
    N = H * (NOPE + V)
    q_res = {}
    for fmt, name in ((mla.MLA_Q_FP8_E4M3, "fp8_e4m3"), (mla.MLA_Q_INT8, "int8"), (mla.MLA_Q_MXFP4, "mxfp4")):
        codes_np, scales_np = synth.quantized_kv_b(900 + fmt, fmt, N, L)
        codes, scales = torch.from_numpy(codes_np).to(dev), torch.from_numpy(scales_np).to(dev)

        def qstep():
            for c in cps:
                mla.mla_dsa_decode_q(c["qn"], c["qr"], c["qi"], c["wi"], codes, scales, fmt, c["kv"], T, K, sm,
                                     scores=c["sc"], sel=c["sel"], nsel=c["nsel"], out=c["out"], ws=c["ws"])
        ms = _graph_time(torch, qstep, 3, 20) / len(cps)
        wbytes = codes.numel() + scales.numel() * scales.element_size()
        step = T * HD * 4 + sel_bytes + wbytes
        q_res[name] = {"ms_per_step": ms, "keys_heads_per_s": T * H / (ms * 1e-3), "weight_bytes": wbytes,
                       "whole_step": {"bytes": step, "frac": step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
                       "stream": {"frac": (T * HD * 4 + sel_bytes) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}}
    res["dsa_decode_quantized_kv_b_T131072"] = q_res
    return res


def cpu_baseline_decode(d, T, K, sm):
    """The oracle (as it stands) on one full decode step of the same workload: RoPE of the query,
    indexer over all T keys, top-k, absorbed decode over the selected keys -- on all host cores and
    on one thread (median of 3 each)."""
    import numpy as np

    import oracle
    from mla_latent_kv_dsa_amd import synth

    cv = synth.bf16_bits_to_f32
    lc, rc, kvb = cv(d.lc), cv(d.rc), cv(d.kv_b)
    qn, qr0 = cv(d.q_nope[0]), cv(d.q_rope[0])

    def step():
        qr = oracle.rope_interleave(qr0[None], np.array([T - 1], np.int32), 0, d.rope)[0]
        s = oracle.index_scores(d.q_idx[0], d.w_idx[0], d.ic)
        sel, n = oracle.topk(s, T, K)
        oracle.absorbed_decode(qn, qr, kvb, lc, rc, sel[:n], d.v, sm)

    cores = _host_cores()
    t_all = _oracle_timed(step, 3, cores)
    t_one = _oracle_timed(step, 3, 1)
    return {"value": T * d.H / t_all, "unit": "keys·heads/s", "cores": cores, "kind": "oracle",
            "sample": f"one full decode step at T={T} (RoPE of the query, fixed-order fp32 indexer over all keys, "
                      f"sort-based top-{K}, fp64 absorbed decode over the selected keys), median of 3 runs",
            "seconds_per_step": t_all,
            "single_thread": {"value": T * d.H / t_one, "cores": 1, "seconds_per_step": t_one}}


# ----------------------------------------------------------------------------- prefill
PREFILL_METRIC = "MLA prefill (non-absorbed) TFLOP/s at S=T=4096"


def measure_prefill(args, cpu=True):
    """S = T = 4096 non-absorbed prefill (kv_b GEMM + causal attention, 64 heads, bf16 in, bf16
    out): TFLOP/s over the algorithmic flops (causal pairs only) against the bf16 matrix-core peak,
    and the oracle's kv_b rebuild plus 64 evenly spaced query rows as the CPU baseline."""
    import numpy as np
    import torch

    import mla_latent_kv_dsa_amd as mla
    from mla_latent_kv_dsa_amd import synth

    dev = torch.device("cuda:0")
    S = 4096
    p = synth.prefill(4, S, 0)
    sm = 1.0 / math.sqrt(p.nope + p.rope)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, lc, rc, kvb = bf(p.q), bf(p.lc), bf(p.rc), bf(p.kv_b)
    kv = mla.KvCache(lc, rc, max_seq_len=S, seq_stride=S)
    out = torch.empty((S, p.H, p.v), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(mla.mla_prefill_workspace_bytes(p.H, p.nope, p.rope, p.v, p.L, S, S), dtype=torch.uint8,
                     device=dev)
    f = lambda: mla.mla_prefill_nonabsorbed(q, kvb, kv, p.nope, 0, sm, out=out, ws=ws)
    steps = max(5, args.steps // 5)
    for _ in range(max(2, args.warmup)):
        f()
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(steps):
        f()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = S * (S + 1) // 2
    f_kvb = 2 * S * (p.H * (p.nope + p.v)) * p.L
    f_attn = 2 * p.H * pairs * (p.nope + p.rope) + 2 * p.H * pairs * p.v
    flops = f_kvb + f_attn
    tf = flops / (ms * 1e-3) / 1e12
    res = {"workload": "prefill_S4096", "S": S, "T": S, "heads": p.H, "qk_nope": p.nope, "qk_rope": p.rope,
           "v_head": p.v, "kv_lora": p.L, "out_dtype": "bf16", "steps": steps, "ms_per_step": ms,
           "TFLOPs": tf,
           "roofline": {"kernel": "pf_kvb + pf_attn (the whole mla_prefill_nonabsorbed call)", "bound": "mfma",
                        "achieved": tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": tf / BF16_PEAK_TFLOPS,
                        "traffic": _prefill_traffic(), "algorithmic_flops": flops, "flops_kv_b_gemm": f_kvb,
                        "flops_attention": f_attn},
           "data": "synthetic: numpy seed 4"}
    if cpu:
        res["cpu_baseline"] = cpu_baseline_prefill(p, sm)
    return res


def _prefill_traffic():
    """HBM bytes of one prefill call (kv_b GEMM + attention) from the committed counters."""
    t = [_traffic("prefill_S4096", k) for k in ("pf_kvb", "pf_attn")]
    return None if None in t else sum(t)


def cpu_baseline_prefill(p, sm):
    """The oracle on a bounded subset of the prefill: its kv_b rebuild of all 4096 tokens and 64
    evenly spaced query rows (0 .. S-1), all 64 heads on all host cores, and 4 of the heads on one
    thread (scaled by 16 to all heads).  Reported as query rows per second, the subset stated."""
    import numpy as np

    import oracle
    from mla_latent_kv_dsa_amd import synth

    cv = synth.bf16_bits_to_f32
    q, kvb, lc, rc = cv(p.q), cv(p.kv_b), cv(p.lc), cv(p.rc)
    rows = np.unique(np.linspace(0, p.S - 1, 64).round().astype(np.int32))
    R = p.nope + p.v
    q4, kvb4 = np.ascontiguousarray(q[:, :4]), np.ascontiguousarray(kvb[: 4 * R])
    cores = _host_cores()
    t_all = _oracle_timed(lambda: oracle.prefill_rows(q, kvb, lc, rc, 0, p.nope, p.v, sm, rows), 1, cores)
    t_one = _oracle_timed(lambda: oracle.prefill_rows(q4, kvb4, lc, rc, 0, p.nope, p.v, sm, rows), 1, 1) * 16
    return {"value": rows.size / t_all, "unit": "query rows/s (64 heads)", "cores": cores, "kind": "oracle",
            "sample": "subset: the oracle's fp64 kv_b rebuild of all 4096 tokens plus 64 evenly spaced query rows "
                      "(0 .. 4095), all heads; single thread on 4 heads scaled x16",
            "seconds": t_all, "single_thread": {"value": rows.size / t_one, "cores": 1, "seconds": t_one}}


def bench_prefill(args):
    r = measure_prefill(args, cpu=not args.no_cpu)
    line = {"metric": PREFILL_METRIC, "value": r["TFLOPs"], "unit": "TFLOP/s", "n_gpus": 1,
            "steps": r["steps"], "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {k: r[k] for k in ("workload", "S", "T", "heads", "qk_nope", "qk_rope", "v_head", "kv_lora")},
            "roofline": r["roofline"], "cpu_baseline": r.get("cpu_baseline")}
    print(json.dumps(line), flush=True)


def bench_vendor(args):
    """Context for the prefill numbers: torch's own kernels on the same shapes (bf16, 64 heads,
    S = T = 4096), timed beside mla_prefill_nonabsorbed.  torch.mm is the library GEMM
    (hipBLASLt) for the kv_b rebuild C[T][H (nope + v)] = Lc kv_b^T (kv_b^T made contiguous);
    scaled_dot_product_attention is held to its flash backend (it raises rather than falling back
    to the math path), causal, with 256-wide queries, keys and values, the widths of the
    non-absorbed attention here (192 + 64 and 256).  Same algorithmic flops as the prefill line."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    dev = torch.device("cuda:0")
    S, H, L, R = 4096, 64, 512, 192 + 256
    g = torch.Generator(device=dev)
    g.manual_seed(1011)

    def timed(f, n):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        e0, e1 = _events(torch, 2)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    lc = torch.randn(S, L, device=dev, dtype=torch.bfloat16, generator=g)
    kvbT = torch.randn(L, H * R, device=dev, dtype=torch.bfloat16, generator=g).contiguous()
    c = torch.empty(S, H * R, device=dev, dtype=torch.bfloat16)
    ms_mm = timed(lambda: torch.mm(lc, kvbT, out=c), 20)
    f_kvb = 2 * S * H * R * L
    res = {"workload": "vendor_prefill_S4096", "gemm_torch_mm": {"ms": ms_mm, "TFLOPs": f_kvb / ms_mm / 1e9}}
    del lc, kvbT, c
    q = torch.randn(1, H, S, 256, device=dev, dtype=torch.bfloat16, generator=g)
    k = torch.randn(1, H, S, 256, device=dev, dtype=torch.bfloat16, generator=g)
    v = torch.randn(1, H, S, 256, device=dev, dtype=torch.bfloat16, generator=g)
    f_attn = 2 * H * (S * (S + 1) // 2) * (256 + 256)
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            ms_fa = timed(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True), 5)
        res["attention_torch_sdpa_flash"] = {"ms": ms_fa, "TFLOPs": f_attn / ms_fa / 1e9}
    except RuntimeError as ex:   # no flash backend in this torch build
        res["attention_torch_sdpa_flash"] = {"unavailable": str(ex)[:200]}
    del q, k, v
    ours = measure_prefill(args, cpu=False)
    res["mla_prefill_nonabsorbed"] = {"ms": ours["ms_per_step"], "TFLOPs": ours["TFLOPs"]}
    print(json.dumps(res), flush=True)


# ----------------------------------------------------------------------------- counters
COPY_MIB = 256


def bench_copy(args):
    """Plain device-to-device copy of COPY_MIB MiB: the known-size kernel whose FETCH_SIZE and
    WRITE_SIZE readings calibrate the HBM byte counters."""
    import torch

    dev = torch.device("cuda:0")
    n = COPY_MIB * 2**20 // 4
    a = torch.randn(n, device=dev)
    b = torch.empty_like(a)
    res = {}
    r = torch.empty(1, device=dev)
    # the runtime's blit kernel (copy_), a one-pass elementwise kernel (mul by 1), a read-only
    # reduction (sum of the buffer into one value) and a write-only fill
    for name, f in (("copyBuffer", lambda: b.copy_(a)), ("elementwise", lambda: torch.mul(a, 1.0, out=b)),
                    ("reduce_read_only", lambda: torch.sum(a, 0, keepdim=True, out=r)),
                    ("fill_write_only", lambda: b.fill_(1.0))):
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        e0, e1 = _events(torch, 2)
        e0.record()
        for _ in range(args.steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        res[name] = {"ms": ms, "GBs": 2 * n * 4 / (ms * 1e-3) / 1e9}
    print(json.dumps({"workload": "copy", "bytes_read": n * 4, "bytes_written": n * 4, "kernels": res}), flush=True)


def _pmc_rows(csv_path):
    import csv

    return list(csv.DictReader(open(csv_path)))


def summarize_pmc(args):
    """Write profiles/<name>.counters.txt: per-dispatch means of every counter found in the
    rocprofv3 --pmc runs under --pmc-dirs (one pass per directory), for each kernel named in
    --pmc-kernels, plus the HBM bytes per launch from FETCH_SIZE / WRITE_SIZE scaled by the
    calibration runs under --calib-dir (a 256 MiB read-only reduction and a 256 MiB write-only fill
    of `bench.py --workload copy`)."""
    from collections import defaultdict

    def csvs(d):
        return [os.path.join(r, f) for r, _, fs in os.walk(d) for f in fs if f.endswith("counter_collection.csv")]

    kernels = args.pmc_kernels.split("|")
    means = {k: {} for k in kernels}
    for d in args.pmc_dirs.split(","):
        for path in csvs(d):
            acc = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
            for r in _pmc_rows(path):
                for k in kernels:
                    if k in r["Kernel_Name"]:
                        acc[k][r["Counter_Name"]][r.get("Dispatch_Id") or r.get("Correlation_Id")] += \
                            float(r["Counter_Value"])
            for k, cs in acc.items():
                for c, per in cs.items():
                    means[k][c] = (statistics.mean(per.values()), len(per))
    fetch_unit = write_unit = None
    if args.calib_dir:
        cal = defaultdict(dict)
        for path in [c for d in args.calib_dir.split(",") for c in csvs(d)]:
            for name in ("reduce_kernel", "FillFunctor", "copyBuffer"):
                m = defaultdict(lambda: defaultdict(float))
                for r in _pmc_rows(path):
                    if name in r["Kernel_Name"]:
                        m[r["Counter_Name"]][r.get("Dispatch_Id")] += float(r["Counter_Value"])
                for c, per in m.items():
                    cal[name][c] = statistics.median(per.values())
        nbytes = COPY_MIB * 2**20
        if cal["reduce_kernel"].get("FETCH_SIZE"):
            fetch_unit = nbytes / cal["reduce_kernel"]["FETCH_SIZE"]
        if cal["FillFunctor"].get("WRITE_SIZE"):
            write_unit = nbytes / cal["FillFunctor"]["WRITE_SIZE"]
    out = os.path.join(ROOT, "profiles", f"{args.counters_name}.counters.txt")
    with open(out, "w") as fo:
        fo.write(f"# rocprofv3 --pmc counters, mean per dispatch.  One pass per counter group:\n")
        for grp in args.pmc_groups.split(";"):
            fo.write(f"#   cd /tmp && rocprofv3 --pmc {grp} --output-format csv -d <dir> -- "
                     f"python3 <repo>/bench.py {args.counters_cmd}\n")
        if args.calib_dir:
            fo.write("# calibration: the same FETCH_SIZE and WRITE_SIZE passes over python3 <repo>/bench.py "
                     "--workload copy --steps 5 --warmup 1\n")
            for name, c in sorted(cal.items()):
                fo.write(f"#   {name}: " + ", ".join(f"{k} {v:.1f}" for k, v in sorted(c.items())) + "\n")
            fo.write(f"fetch_bytes_per_unit = {fetch_unit}   # {COPY_MIB} MiB read-only reduction / its FETCH_SIZE\n")
            fo.write(f"write_bytes_per_unit = {write_unit}   # {COPY_MIB} MiB write-only fill / its WRITE_SIZE\n")
        for k in kernels:
            fo.write(f"\n[{k}]\n")
            for c, (v, n) in sorted(means[k].items()):
                fo.write(f"{c} = {v:.6g}   # {n} dispatches\n")
            f = means[k].get("FETCH_SIZE")
            w = means[k].get("WRITE_SIZE")
            if f and fetch_unit:
                fo.write(f"hbm_read_bytes_per_launch = {f[0] * fetch_unit:.0f}\n")
            if w and write_unit:
                fo.write(f"hbm_write_bytes_per_launch = {w[0] * write_unit:.0f}\n")
            src = _kernel_source(k)
            if src:
                fo.write(f"source = {src}\nsource_sha256_16 = {_src_hash(os.path.join(ROOT, src))}\n")
    print(open(out).read())


def summarize_trace(args):
    """Write profiles/<name>.kernel_stats.txt from a rocprofv3 --kernel-trace --stats run."""
    import csv

    rows = list(csv.DictReader(open(args.stats_csv)))
    out = os.path.join(ROOT, "profiles", f"{args.stats_name}.kernel_stats.txt")
    with open(out, "w") as fo:
        fo.write(f"# per-kernel durations (rocprofv3 kernel trace)\n")
        fo.write(f"# command: cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d <dir> -o run -- "
                 f"python3 <repo>/bench.py {args.stats_cmd}\n")
        fo.write(f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'total%':>7}  kernel\n")
        for r in rows:
            fo.write(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}  {r['Name'][:110]}\n")
    print(open(out).read())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsa_decode",
                    choices=["dsa_decode", "dsa_decode_paged_b32", "prefill", "copy", "rows", "vendor"])
    ap.add_argument("--copies", type=int, default=6, help="input copies rotated to defeat the Infinity Cache")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the batched paged and dense decode configurations (profiling runs of the headline step)")
    ap.add_argument("--counters-name", default="dsa_decode_T131072_B1")
    ap.add_argument("--counters-cmd", default="--steps 5 --warmup 1 --no-cpu --no-extra")
    ap.add_argument("--pmc-dirs", help="summarize rocprofv3 --pmc passes (comma-separated directories) and exit")
    ap.add_argument("--pmc-kernels", default="index_scores_mfma", help="'|'-separated kernel name substrings")
    ap.add_argument("--pmc-groups", default="", help="the counter groups of the passes, ';'-separated (recorded)")
    ap.add_argument("--calib-dir", help="rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes of --workload copy "
                                        "(comma-separated directories)")
    ap.add_argument("--stats-csv", help="summarize a rocprofv3 kernel_stats.csv and exit")
    ap.add_argument("--stats-name", default="dsa_decode_T131072_B1")
    ap.add_argument("--stats-cmd", default="")
    args = ap.parse_args()
    if args.stats_csv:
        summarize_trace(args)
        return
    if args.pmc_dirs:
        summarize_pmc(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.workload == "dsa_decode":
        bench_dsa_decode(args)
    elif args.workload == "dsa_decode_paged_b32":   # the batched paged configuration on its own line
        r = bench_batched_paged(args)
        print(json.dumps({"metric": "MLA+DSA batched paged decode keys·heads/sec", "value": r["keys_heads_per_s"],
                          "unit": "keys·heads/s", "n_gpus": 1, "ms_per_step": r["ms_per_step"],
                          "higher_is_better": True, "dtype": "bf16", "data": "synthetic", "config": r}), flush=True)
    elif args.workload == "copy":
        bench_copy(args)
    elif args.workload == "vendor":   # torch's GEMM and flash attention on the prefill shapes, for context
        bench_vendor(args)
    elif args.workload == "rows":   # the cache write, shared layer, multi-query decode and DSA prefill alone
        print(json.dumps(bench_new_rows(args)), flush=True)
    else:
        bench_prefill(args)


if __name__ == "__main__":
    main()
