"""Benchmark of the KV-sparsity prefill-and-compress path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload: one Llama-3-8B-shaped layer, batch 1 - a 4000-token prompt with 32 query heads,
8 KV heads, head_dim 128, bf16 N(0,1) inputs with attention-sink keys at tokens 0 and 17
(x20 in channels 7 and 101), window alpha = 32, budget k = 400 (10x compression), 16-token
blocks, then 500 paged decode steps over the compressed cache.  Inputs are synthetic and
resident in HBM before the timed region.

One step = the whole hot path once: prefill attention with LSE, window score, top-k,
compaction into blocks, then 500 decode steps with append.  Every kernel is launched on
torch's current stream and bracketed by HIP events, so per-kernel durations come from the
GPU clock of the timed steps.  The printed JSON line carries:
  value        prefill+compress throughput: prompt tokens / GPU time of the prefill-side
               kernels (attention, score, top-k fused with compaction)
  decode       paged-decode throughput: generated tokens / GPU time of the 500 decode calls
  ms_per_step  wall time of one full step (host clock, synchronised on both sides)
  roofline     the kernel with the largest share of the step's GPU time, against MI355X's
               published peak (HBM 8 TB/s; bf16 dense MFMA 2.5 PFLOP/s); `rooflines` has all
  cpu_baseline the fp64 numpy oracle on the host cores (a bounded sample, scaled)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
REALTIME_HZ = 100e6          # the GPU's real-time counter (kvs_probe_timestamp) on MI355X
ALL_SECTIONS = ("ceiling", "lse", "scale", "long", "fp8", "prefix", "layers32", "evict", "prompt3", "prompt4",
                "prompt5", "memory")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-budget-s", type=float, default=20.0)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB mebibytes three times (reference for the "
                        "FETCH_SIZE / WRITE_SIZE counters) and exit")
    p.add_argument("--decode-mode", choices=("graph", "loop"), default="graph",
                   help="graph: the prompt-side kernels replay as one captured HIP graph and the 500 "
                        "decode steps as another (the launch mode of a serving loop); loop: one host launch "
                        "per kernel")
    p.add_argument("--sections", default="all",
                   help="comma list of the reports to add after the timed step: " + ", ".join(ALL_SECTIONS) +
                        " (default all); the timed step and its roofline always run")
    return p.parse_args()


def kernel_source_hash(name: str) -> str:
    """Hash of a kernel source and of the local headers it includes (kvs_common.h aside), so a
    counter record goes stale when any code the kernel is built from changes."""
    import re
    csrc = os.path.join(ROOT, "kv_cache_sparsification_amd", "csrc")
    text = open(os.path.join(csrc, name), "rb").read()
    h = hashlib.sha256(text)
    for inc in re.findall(rb'#include "([a-z_]+\.h)"', text):
        if inc != b"kvs_common.h" and os.path.exists(os.path.join(csrc, inc.decode())):
            h.update(open(os.path.join(csrc, inc.decode()), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str, source: str):
    """HBM bytes per launch from the committed counter summary, or None if the kernel changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_key)
    if not rec or rec.get("source_sha256_16") != kernel_source_hash(source):
        return None
    return rec.get("bytes_per_launch")


def measured_scale_traffic(key: str):
    """HBM bytes of an at-scale figure (32-layer decode step, multi-prompt prefill or compaction)
    from the committed counter summary, or None if the kernel's source changed since."""
    path = os.path.join(ROOT, "profiles", "traffic_scale.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(key)
    if not rec or rec.get("source_sha256_16") != kernel_source_hash(rec["source"]):
        return None
    return rec


def measured_mfma(kernel_key: str, source: str):
    """MFMA counters of a launch (rocprofv3: executed bf16 flops, MFMA-busy share of the SIMDs' active
    cycles) from the committed summary, or None if the kernel changed since."""
    path = os.path.join(ROOT, "profiles", "mfma.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel_key)
    if not rec or rec.get("source_sha256_16") != kernel_source_hash(source):
        return None
    return {"mfma_util": rec["mfma_util"], "executed_flops_per_launch": rec["executed_bf16_flops_per_launch"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (--gpus {args.gpus} refused)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads as wl
    import kv_cache_sparsification_amd as kvs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        nbytes = args.copy_calibration << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read": nbytes, "bytes_written": nbytes,
                          "launches": 3}), flush=True)
        return
    w = wl.WORKLOADS[2]
    n, hq, hkv, d, alpha, kb = w.fixed_len, w.hq, w.hkv, w.d, w.alpha, w.budgets[0]
    steps_dec = w.decode_steps
    k_eff = min(kb, n)

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs resident in HBM
    qb, kbits, vb, cu = wl.prefill_batch(w, 0, [n])
    q, k, v = up(qb), up(kbits), up(vb)
    cu_d = torch.from_numpy(cu).to(dev)
    dec = [wl.decode_step_inputs(w, 0, s, 1) for s in range(steps_dec)]
    dq = up(np.stack([x[0] for x in dec]))            # [steps][1][hq][d]
    dk = up(np.stack([x[1] for x in dec]))
    dv = up(np.stack([x[2] for x in dec]))
    total_tokens_cache = k_eff + steps_dec
    nblk = -(-total_tokens_cache // 16)
    alloc = kvs.BlockAllocator(nblk + 7)
    table = alloc.alloc_n(nblk)
    tbl = torch.tensor([table], dtype=torch.int32, device=dev)
    k_pool, v_pool = kvs.new_pools(nblk + 7, hkv, d, device=dev)
    ctx = torch.arange(k_eff + 1, k_eff + steps_dec + 1, dtype=torch.int32, device=dev)   # L per step
    keep_off = torch.tensor([0, k_eff], dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(hq, n, dtype=torch.float32, device=dev)
    S = torch.empty(hkv, n, dtype=torch.float32, device=dev)
    keep = torch.empty(hkv * k_eff, dtype=torch.int32, device=dev)
    od = torch.empty(steps_dec, 1, hq, d, dtype=torch.bfloat16, device=dev)
    ws_bytes = kvs.kvs_paged_decode_workspace_size(1, hq, hkv, d, total_tokens_cache)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def decode_all(mark):
        for s in range(steps_dec):
            L = k_eff + s + 1
            kvs.kvs_paged_decode(dq[s], k_pool, v_pool, tbl, ctx[s:s + 1], L, new_k=dk[s], new_v=dv[s], o=od[s],
                                 workspace=ws)
            mark("decode_end")

    def prefill_compress(mark):
        kvs.kvs_prefill_attn_lse(q, k, v, cu_d, n, o=o, lse=lse)
        mark("prefill_end")
        kvs.kvs_window_score(q, k, lse, cu_d, n, alpha, scores=S)
        mark("score_end")
        # top-k and compaction in one launch (one workgroup per (head, block), each repeating
        # the selection); kvs_topk_select and kvs_compact_paged are timed alone below as well
        kvs.kvs_topk_compact(S, k, v, cu_d, n, alpha, kb, keep_off, k_pool, v_pool, tbl, keep_idx=keep)
        mark("compact_end")

    graph = pre_graph = None
    # GPU clock stamps (100 MHz real-time counter) as the first and last launches of each
    # captured phase: [prompt begin, prompt end, decode begin, decode end], copied per timed step
    stamps = torch.zeros(4, dtype=torch.int64, device=dev)
    stamp_hist = torch.zeros(max(args.steps, 1), 4, dtype=torch.int64, device=dev)
    if args.decode_mode == "graph":
        # Both phases captured as HIP graphs, the way a serving loop launches a fixed sequence:
        # the prompt-side kernels as one graph, the 500 decode steps as another.
        # Compaction first so the captured steps see a filled cache; capture records launches.
        prefill_compress(lambda key: None)
        torch.cuda.synchronize()
        graph, pre_graph = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):             # warm the side stream outside capture
            prefill_compress(lambda key: None)
            decode_all(lambda key: None)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(pre_graph):
            kvs.kvs_probe_timestamp(stamps[0:1])
            prefill_compress(lambda key: None)
            kvs.kvs_probe_timestamp(stamps[1:2])
        with torch.cuda.graph(graph):
            kvs.kvs_probe_timestamp(stamps[2:3])
            decode_all(lambda key: None)
            kvs.kvs_probe_timestamp(stamps[3:4])
        torch.cuda.synchronize()

    def one_step(rec, i=None):
        """rec: dict of event lists, or None for warm-up; i: the timed step's index."""
        def mark(key):
            if rec is not None:
                e = ev()
                e.record(stream)
                rec.setdefault(key, []).append(e)
        mark("prefill_begin")
        if pre_graph is not None:
            pre_graph.replay()
            mark("compact_end")
        else:
            prefill_compress(mark)
        if graph is not None:
            graph.replay()
            mark("decode_end")
            if i is not None:
                stamp_hist[i].copy_(stamps)
        else:
            decode_all(mark)

    for _ in range(args.warmup):
        one_step(None)
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for i in range(args.steps):
        rec = {}
        one_step(rec, i)
        recs.append(rec)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # Per-kernel durations of the prompt-side kernels: each kernel alone, captured as a HIP graph
    # of back-to-back launches (the same inputs every launch), so no host launch gap is counted.
    launches = {
        "prefill_attn_lse": lambda: kvs.kvs_prefill_attn_lse(q, k, v, cu_d, n, o=o, lse=lse),
        "window_score": lambda: kvs.kvs_window_score(q, k, lse, cu_d, n, alpha, scores=S),
        "topk_compact": lambda: kvs.kvs_topk_compact(S, k, v, cu_d, n, alpha, kb, keep_off, k_pool, v_pool, tbl,
                                                     keep_idx=keep),
        "topk_select": lambda: kvs.kvs_topk_select(S, cu_d, n, alpha, kb, keep_off, keep_idx=keep),
        "compact_paged": lambda: kvs.kvs_compact_paged(k, v, cu_d, keep, keep_off, k_eff, k_pool, v_pool, tbl),
    }
    kernel_us = {kname: kernel_graph_us(torch, fn, 10 if kname == "prefill_attn_lse" else 50)
                 for kname, fn in launches.items()}

    # ---- per-kernel GPU durations (ms) from the timed steps' events
    def span(rec, a, b, i=0, j=0):
        return rec[a][i].elapsed_time(rec[b][j])

    dur = {kname: [us * 1e-3] for kname, us in kernel_us.items()}
    dur["paged_decode"] = []
    pre_phase, dec_phase = [], []
    for rec in recs:
        de = rec["decode_end"]
        if graph is not None:     # one event pair around the 500 captured steps
            dur["paged_decode"].append(rec["compact_end"][0].elapsed_time(de[0]) / steps_dec)
        else:
            dur["paged_decode"].append(rec["compact_end"][0].elapsed_time(de[0]))
            for s in range(1, len(de)):
                dur["paged_decode"].append(de[s - 1].elapsed_time(de[s]))
        pre_phase.append(span(rec, "prefill_begin", "compact_end"))
        dec_phase.append(rec["compact_end"][0].elapsed_time(de[-1]))
    avg_ms = {kname: float(np.mean(v)) for kname, v in dur.items()}
    # the step's kernels (the separate top-k and compaction calls are timed for reference only)
    step_kernels = ("prefill_attn_lse", "window_score", "topk_compact", "paged_decode")
    per_step_ms = {kname: avg_ms[kname] * (steps_dec if kname == "paged_decode" else 1) for kname in step_kernels}

    # ---- algorithmic work per launch
    P = sum(j + 1 for j in range(n - min(alpha, n), n))        # visited (window row, key) pairs
    mean_L = k_eff + (steps_dec + 1) / 2.0
    work = {
        "prefill_attn_lse": ("mfma", 2.0 * d * hq * n * (n + 1), "TFLOP/s", MFMA_BF16_PEAK_TFLOPS,
                             "prefill_attn.hip"),
        "window_score": ("hbm", n * hkv * d * 2 + min(alpha, n) * hq * (2 * d + 4) + 4 * hkv * n, "GB/s",
                         HBM_PEAK_GBS, "window_score.hip"),
        "topk_compact": ("hbm", 4 * hkv * n + 4 * hkv * k_eff + 8 * k_eff * hkv * d, "GB/s", HBM_PEAK_GBS,
                         "topk_select.hip"),
        "topk_select": ("hbm", 4 * hkv * n + 4 * hkv * k_eff, "GB/s", HBM_PEAK_GBS, "topk_select.hip"),
        "compact_paged": ("hbm", 8 * k_eff * hkv * d, "GB/s", HBM_PEAK_GBS, "compact_paged.hip"),
        "paged_decode": ("hbm", decode_bytes(mean_L, hq, hkv, d), "GB/s", HBM_PEAK_GBS, "paged_decode.hip"),
    }
    rooflines = {}
    for kname, (bound, amount, unit, peak, src) in work.items():
        sec = avg_ms[kname] * 1e-3
        achieved = amount / sec / (1e12 if unit == "TFLOP/s" else 1e9)
        rooflines[kname] = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                            "frac": round(achieved / peak, 4),
                            "traffic": measured_traffic(kname, src),
                            "avg_launch_us": round(avg_ms[kname] * 1e3, 2),
                            "algorithmic_per_launch": amount,
                            "timed_as": ("one decode call (decode kernel, plus the merge kernel when the "
                                         "context is split) inside the 500-step graph of the timed steps"
                                         if kname == "paged_decode" else
                                         "graph of back-to-back launches of this kernel alone"
                                         + ("; a separate call, not in the timed step (which runs topk_compact)"
                                            if kname in ("topk_select", "compact_paged") else ""))}
        if bound == "mfma":
            rooflines[kname]["counters"] = measured_mfma(kname, src)
    dominant = max(per_step_ms, key=per_step_ms.get)

    prefill_ms_events = float(np.mean(pre_phase))
    decode_ms_events = float(np.mean(dec_phase))
    if graph is not None:
        # GPU time of each captured phase from its clock stamps: the graph's start latency (the
        # gap between the previous graph's last kernel and this one's first) is not in it
        h = stamp_hist.cpu().numpy().astype(np.float64) * (1e3 / REALTIME_HZ)       # ms
        prefill_ms = float(np.mean(h[:, 1] - h[:, 0]))
        decode_ms = float(np.mean(h[:, 3] - h[:, 2]))
    else:
        prefill_ms, decode_ms = prefill_ms_events, decode_ms_events
    value = n / (prefill_ms * 1e-3)
    decode_tok_s = steps_dec / (decode_ms * 1e-3)

    line = {
        "metric": "prefill+KV-compress tok/s & paged-decode tok/s, 8B layer n=4000; % roofline",
        "value": round(value, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, sink keys x20 at tokens 0 and 17)",
        "config": {"workload": "llama3-8b-layer n=4000 prompt, 32q/8kv heads, d=128, alpha=32, k=400, "
                               "16-token blocks, then 500 paged decode steps",
                   "global_batch": 1, "seq_len": n, "parallelism": "none (1 GPU)"},
        "value_definition": ("prompt tokens / GPU time of prefill attention + window score + top-k + compaction"
                             + (", from a clock stamp launched first in the captured prompt-side graph to one "
                                "launched last (the graph's start latency is outside it: graph_start_gap_us)"
                                if graph is not None else ", between events around the eager launches")),
        "decode": {"metric": "paged-decode tok/s", "value": round(decode_tok_s, 1), "unit": "tok/s",
                   "ms_for_500_steps": round(decode_ms, 4)},
        "phase_ms": {"prefill_compress": round(prefill_ms, 4), "decode_500": round(decode_ms, 4)},
        "phase_ms_events": {"prefill_compress": round(prefill_ms_events, 4), "decode_500": round(decode_ms_events, 4),
                            "note": "events recorded on the stream around each graph replay: graph start "
                                    "latency included"},
        "graph_start_gap_us": round((prefill_ms_events - prefill_ms) * 1e3, 2) if graph is not None else None,
        "launch_mode": args.decode_mode,
        "roofline": {kk: rooflines[dominant][kk] for kk in ("bound", "achieved", "peak", "unit", "frac", "traffic")},
        "roofline_kernel": dominant,
        "rooflines": rooflines,
        "kernel_share_ms_per_step": {kk: round(vv, 4) for kk, vv in per_step_ms.items()},
    }

    sections = set(ALL_SECTIONS) if args.sections == "all" else \
        set(x.strip() for x in args.sections.split(",") if x.strip())
    unknown = sections - set(ALL_SECTIONS)
    if unknown:
        raise SystemExit(f"unknown sections: {sorted(unknown)}")
    def progress(what):
        print(f"[bench] {what}", file=sys.stderr, flush=True)

    progress(f"timed step done: {ms_per_step:.3f} ms per step")
    if "ceiling" in sections:
        progress("ceiling")
        line["hbm_ceiling"] = hbm_ceiling(kvs, torch)
    if "lse" in sections:
        progress("lse")
        line["lse_output_cost"] = lse_output_cost(kvs, torch, q, k, v, cu_d, n, o, lse)
    if "scale" in sections:
        progress("scale")
        line["decode_at_scale"] = decode_at_scale(kvs, torch, wl, 100)
    if "long" in sections:
        progress("long")
        line["decode_long_full_layer"] = decode_at_scale(kvs, torch, wl, 50, full=True)
    if "fp8" in sections:
        progress("fp8")
        line["fp8_decode_at_scale"] = decode_at_scale(kvs, torch, wl, 100, fp8=True)
        line["fp8_decode_long_full_layer"] = decode_at_scale(kvs, torch, wl, 50, fp8=True, full=True)
        line["fp8_layer"] = fp8_layer(kvs, torch, wl, w, k, v, cu_d, keep, keep_off, steps_dec)
    if "prefix" in sections:
        progress("prefix")
        line["prefix_reuse"] = prefix_reuse(kvs, torch, wl, w, q, k, v)
    if "layers32" in sections:
        progress("layers32")
        line["decode_32_layers"] = decode_32_layers(kvs, torch, wl, 10)
        line["fp8_decode_32_layers"] = decode_32_layers(kvs, torch, wl, 10, fp8=True)
    if "evict" in sections:
        # the prefill-side pass of the last step left the compressed cache in the pools
        kvs.kvs_compact_paged(k, v, cu_d, keep, keep_off, k_eff, k_pool, v_pool, tbl)
        progress("evict")
        line["decode_evict"] = decode_evict(kvs, torch, wl, w, k_pool, v_pool, tbl, S, cu_d, keep, keep_off, 200)
    for cid, key in ((3, "prompt_side_20_prompts"), (4, "prompt_side_4x30000"), (5, "prompt_side_64_prompt_mix")):
        if f"prompt{cid}" in sections:
            progress(key)
            line[key] = prompt_side(kvs, torch, wl, cid)
    if "prompt5" in sections:
        progress("admission wave")
        line["admission_wave_64_prompt_mix"] = admission_wave(kvs, torch, wl)
    if "memory" in sections:
        progress("memory")
        line["paged_memory"] = paged_memory(wl)
    if not args.no_cpu_baseline:
        progress("cpu baseline")
        line["cpu_baseline"] = cpu_baseline(w, qb, kbits, vb, dec, args.cpu_budget_s)
    print(json.dumps(line), flush=True)


def decode_at_scale(kvs, torch, wl, steps, fp8=False, full=False):
    """Paged decode where the read volume, not the latency, sets the time: the long-context
    workload's compressed layers (4 sequences, 3000 kept tokens each plus the appended ones,
    8 KV heads, d=128), or with `full` one of its full layers (all 30000 prompt tokens cached:
    491 MB of K/V per step, beyond the 256 MB MALL, so read from HBM every step), `steps`
    decode steps with append replayed as one HIP graph.  Reports the rate of the algorithmic
    bytes against the HBM peak.  fp8: the same over the 8-bit cache (codes plus one fp32 scale
    per row)."""
    import numpy as np
    w = wl.WORKLOADS[4]
    B, hq, hkv, d = w.num_seqs, w.hq, w.hkv, w.d
    layer = 0 if full else 3
    kept = w.fixed_len if full else w.budgets[layer]
    max_ctx = kept + steps
    nb_seq = -(-max_ctx // 16)
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(4242)
    if fp8:
        pools = kvs.new_pools_fp8(B * nb_seq, hkv, d, device=dev)
        for t in pools[:2]:       # finite codes of either sign (no NaN code)
            t.copy_(torch.randint(0, 0x7F, t.shape, generator=gen, device=dev, dtype=torch.uint8)
                    | (torch.randint(0, 2, t.shape, generator=gen, device=dev, dtype=torch.uint8) << 7))
        for t in pools[2:]:
            t.copy_(torch.rand(t.shape, generator=gen, device=dev) * 0.01 + 0.002)
    else:
        pools = kvs.new_pools(B * nb_seq, hkv, d, device=dev)
        for t in pools:
            t.copy_(torch.randn(t.shape, generator=gen, device=dev).to(torch.bfloat16))
    perm = np.random.default_rng(4242).permutation(B * nb_seq).astype(np.int32)
    tbl = torch.from_numpy(perm.reshape(B, nb_seq)).to(dev)
    lens = torch.tensor([[kept + s + 1] * B for s in range(steps)], dtype=torch.int32, device=dev)
    qs, nks, nvs = zip(*[wl.device_decode_step(w, layer, s, range(B), device=dev) for s in range(steps)])
    ws = torch.empty(max(kvs.kvs_paged_decode_workspace_size(B, hq, hkv, d, max_ctx), 1), dtype=torch.uint8,
                     device=dev)
    od = torch.empty(steps, B, hq, d, dtype=torch.bfloat16, device=dev)
    decode = kvs.kvs_paged_decode_fp8 if fp8 else kvs.kvs_paged_decode

    def run():
        for s in range(steps):
            decode(qs[s], *pools, tbl, lens[s], max_ctx, new_k=nks[s], new_v=nvs[s], o=od[s], workspace=ws)

    us = _graph_time_us(torch, run, steps)
    mean_L = kept + (steps + 1) / 2.0
    nbytes = B * decode_bytes(mean_L, hq, hkv, d, fp8)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"{B} sequences x {kept}-{kept + steps} cached tokens, {hq}q/{hkv}kv heads, d={d}, "
                        f"{steps} decode steps with append (HIP graph)" + (", 8-bit E4M3 cache" if fp8 else ""),
            "resident_in": ("HBM: the cache of about %d MB, read every step, is larger than the 256 MB MALL"
                            % round(nbytes / 1e6)) if nbytes > 256e6 else
                           ("Infinity Cache (MALL): the same cache of about %d MB is re-read every step, below "
                            "the 256 MB MALL, so this rate is not an HBM rate" % round(nbytes / 1e6)),
            "us_per_step": round(us, 3), "algorithmic_bytes_per_step": int(nbytes),
            "achieved_GBs": round(gbs, 1), "peak_GBs": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4),
            "tok_s": round(B / (us * 1e-6), 1)}


def decode_bytes(mean_L, hq, hkv, d, fp8=False):
    """Algorithmic HBM bytes of one sequence's decode step: the cached K and V (bf16, or codes
    plus one fp32 scale per row), the query read and output written (bf16), the new K/V read
    (bf16) and stored, and the block-table entries."""
    if fp8:
        cache = 2 * mean_L * hkv * (d + 4)
        new = 4 * hkv * d + 2 * hkv * (d + 4)
    else:
        cache = 4 * mean_L * hkv * d
        new = 8 * hkv * d
    return cache + 4 * hq * d + new + 4 * math.ceil(mean_L / 16)


def _graph_time_us(torch, run, steps, reps=3):
    """Capture `run` (steps launches) as one HIP graph and time its replays: us per step."""
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        run()                                  # warm outside capture
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * steps)


def kernel_graph_us(torch, launch, count, replays=5, warm_ms=40.0):
    """us per launch of one kernel: `count` back-to-back launches captured as one HIP graph.
    The graph is replayed for about warm_ms first (the chip's clock settles under the kernel's
    own load), then `replays` replays are timed one by one; the median replay is returned."""
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for _ in range(count):
            launch()                           # warm outside capture
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(count):
            launch()
    t0 = time.perf_counter()
    while True:
        graph.replay()
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= warm_ms:
            break
    times = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / count)
    return float(sorted(times)[len(times) // 2])


def hbm_ceiling(kvs, torch, gib=4):
    """The practical memory ceilings beside the published 8 TB/s: a hand-written streaming-read
    kernel (16 bytes per lane, four loads in flight) over a buffer far larger than the 256 MB
    Infinity Cache, best over a few grid sizes, and a plain device copy of the same size."""
    dev = torch.device("cuda:0")
    nbytes = gib << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    best = None
    per_grid = {}
    stream = torch.cuda.current_stream()
    for grid in (2048, 4096, 8192, 16384, 32768):
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
        kvs.kvs_probe_stream_read(buf, grid, sink=sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            kvs.kvs_probe_stream_read(buf, grid, sink=sink)
        e1.record(stream)
        torch.cuda.synchronize()
        gbs = 3 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
        per_grid[str(grid)] = round(gbs, 1)
        best = gbs if best is None else max(best, gbs)
    half = nbytes // 2
    src, dst = buf[:half], buf[half:]
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 3 * 2 * half / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return {"read_GBs": round(best, 1), "read_frac_of_peak": round(best / HBM_PEAK_GBS, 4),
            "read_GBs_by_grid": per_grid, "read_bytes": nbytes,
            "copy_GBs_read_plus_write": round(copy_gbs, 1), "copy_bytes_each_way": half,
            "kernel": "kvs_probe_stream_read (16-byte nontemporal loads, 4 in flight per lane, 256 threads)"}


def lse_output_cost(kvs, torch, q, k, v, cu_d, n, o, lse, rounds=3):
    """What returning the row statistics costs: the bench layer's prefill with the LSE written
    (the modified kernel) against the same kernel writing only O (the unmodified attention),
    alternated `rounds` times, each a graph of 10 back-to-back launches."""
    with_lse, without = [], []
    for _ in range(rounds):
        with_lse.append(kernel_graph_us(torch, lambda: kvs.kvs_prefill_attn_lse(q, k, v, cu_d, n, o=o, lse=lse), 10))
        without.append(kernel_graph_us(torch, lambda: kvs.kvs_prefill_attn_lse(q, k, v, cu_d, n, o=o,
                                                                                skip_lse=True), 10))
    a, b = min(with_lse), min(without)
    return {"workload": "bench layer prefill, n=4000, 32q/8kv heads, d=128",
            "us_with_lse": round(a, 2), "us_without": round(b, 2),
            "extra_us": round(a - b, 2), "extra_frac": round((a - b) / b, 4),
            "lse_bytes_written": int(lse.numel() * 4), "o_bytes_written": int(o.numel() * 2),
            "samples_us": {"with_lse": [round(x, 2) for x in with_lse], "without": [round(x, 2) for x in without]}}


def prompt_side(kvs, torch, wl, cid):
    """Prefill+compress of a multi-prompt workload, per layer class, each kernel alone as a graph
    of back-to-back launches.  Prefill attention and the window score do not depend on the
    budget, so they are timed once; top-k and compaction are timed for every distinct budget
    (keep-all compaction for the full layers).  The 32-layer figure sums the layers' kernels:
    prompt tokens / (32 prefills + a score, top-k and compaction per compressed layer + a
    keep-all compaction per full layer).  The continuous-batch mix is measured on its first
    admission wave (64 prompts, each prefilled whole: prefix reuse would only lower the work)."""
    import numpy as np
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[cid]
    if cid == 5:
        lengths = [wl.mix_sequence(w, i, i).n for i in range(w.num_seqs)]
    else:
        lengths = w.seq_lengths()
    hq, hkv, d, alpha = w.hq, w.hkv, w.d, w.alpha
    q, k, v, cu = wl.device_batch(w, 3, lengths, list(range(len(lengths))), device=dev)
    cu_d = torch.from_numpy(cu).to(dev)
    T, max_n = int(cu[-1]), max(lengths)
    o = torch.empty_like(q)
    lse = torch.empty(hq, T, dtype=torch.float32, device=dev)
    S = torch.empty(hkv, T, dtype=torch.float32, device=dev)
    big = T > 200000
    t_pre = kernel_graph_us(torch, lambda: kvs.kvs_prefill_attn_lse(q, k, v, cu_d, max_n, o=o, lse=lse),
                            2 if big else 4)
    t_score = kernel_graph_us(torch, lambda: kvs.kvs_window_score(q, k, lse, cu_d, max_n, alpha, scores=S), 10)
    flops = sum(2.0 * d * hq * n * (n + 1) for n in lengths)
    score_bytes = sum(n * hkv * d * 2 + min(alpha, n) * hq * (2 * d + 4) + 4 * hkv * n for n in lengths)
    per_budget = {}
    layer_us = []
    for kb in sorted(set(w.budgets), key=lambda x: -1 if x is None else x):
        kept = [n if kb is None or kb >= n else kb for n in lengths]
        nbs = [-(-c // 16) for c in kept]
        nb_total = sum(nbs)
        k_pool, v_pool = kvs.new_pools(nb_total, hkv, d, device=dev)
        perm = np.random.default_rng(cid).permutation(nb_total).astype(np.int32)
        tbl = np.full((len(lengths), max(nbs)), -1, np.int32)
        at = 0
        for i, nb in enumerate(nbs):
            tbl[i, :nb] = perm[at:at + nb]
            at += nb
        tbl = torch.from_numpy(tbl).to(dev)
        koff = torch.from_numpy(np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)).to(dev)
        comp_bytes = 8 * sum(kept) * hkv * d
        if kb is None:
            t_topk = 0.0
            t_comp = kernel_graph_us(torch, lambda: kvs.kvs_compact_paged(k, v, cu_d, None, None, max_n, k_pool,
                                                                          v_pool, tbl), 3 if big else 10)
            rec = {"compact_us": round(t_comp, 2)}
        else:
            keep = torch.empty(hkv * sum(kept), dtype=torch.int32, device=dev)
            t_topk = kernel_graph_us(torch, lambda: kvs.kvs_topk_select(S, cu_d, max_n, alpha, kb, koff,
                                                                         keep_idx=keep), 10)
            t_comp = kernel_graph_us(torch, lambda: kvs.kvs_compact_paged(k, v, cu_d, keep, koff, max(kept), k_pool,
                                                                          v_pool, tbl), 10)
            rec = {"topk_us": round(t_topk, 2), "compact_us": round(t_comp, 2),
                   "topk_bytes": 4 * hkv * (T + sum(kept))}
        rec.update({"kept_tokens_per_head": int(sum(kept)), "compact_bytes": int(comp_bytes),
                    "compact_GBs": round(comp_bytes / (t_comp * 1e-6) / 1e9, 1),
                    "compact_frac_of_peak": round(comp_bytes / (t_comp * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "layers": sum(1 for x in w.budgets if x == kb)})
        per_budget["full" if kb is None else f"k={kb}"] = rec
        layer = t_pre + (t_comp if kb is None else t_score + t_topk + t_comp)
        layer_us += [layer] * rec["layers"]
        del k_pool, v_pool
    total_us = sum(layer_us)
    del q, k, v, o
    torch.cuda.empty_cache()
    names = {3: "20 prompts U[1000,4000]", 4: "4 prompts x 30000", 5: "64 prompts log-uniform [512,32768] "
             "(first admission wave)"}
    budgets = "layers 0-2 full, " + ("3-31 k=%d" % w.budgets[3] if cid != 5 else "pyramid k 2048..128 on 3-31")
    if cid == 3:
        # counter figures of this workload's kernels (profiles/traffic_scale.json), while current
        per_budget["full"]["traffic"] = _traffic_rate(
            measured_scale_traffic("keep-all compaction, 20 prompts (47731 tokens)"), None,
            per_budget["full"]["compact_us"])
        per_budget["k=512"]["traffic"] = _traffic_rate(measured_scale_traffic("compaction k=512, 20 prompts"), None,
                                                        per_budget["k=512"]["compact_us"])
        prefill_traffic = _traffic_rate(measured_scale_traffic("prefill, 20 prompts (47731 tokens)"), None, t_pre)
    else:
        prefill_traffic = None
    return {"workload": f"{names[cid]}, {w.n_layers} layers ({budgets}), alpha={alpha}, {hq}q/{hkv}kv heads, d={d}",
            "prefill_traffic": prefill_traffic,
            "prompt_tokens": T,
            "prefill_us": round(t_pre, 2), "prefill_TFLOPs": round(flops / (t_pre * 1e-6) / 1e12, 1),
            "prefill_frac_of_mfma_peak": round(flops / (t_pre * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "prefill_flops": flops,
            "score_us": round(t_score, 2), "score_GBs": round(score_bytes / (t_score * 1e-6) / 1e9, 1),
            "per_budget": per_budget,
            "us_32_layers": round(total_us, 1),
            "prompt_tok_s_32_layers": round(T / (total_us * 1e-6), 1),
            "prompt_tok_s_per_layer": round(T / (total_us * 1e-6) * w.n_layers, 1)}


def _traffic_rate(rec, key, us):
    """Counter-measured HBM bytes of a launch (or step) and the rate they give at `us`."""
    if rec is None:
        return None
    nbytes = rec[key] if key else rec["read_bytes"] + rec["write_bytes"]
    return {"bytes": int(nbytes), "GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "source": "profiles/traffic_scale.json (rocprofv3 FETCH_SIZE and WRITE_SIZE, copy-calibrated)"}


def admission_wave(kvs, torch, wl):
    """The continuous-batch mix's first admission wave (64 prompts log-uniform in [512, 32768], 8
    groups of 8 sharing a 2048-token prefix) through the product's admission step in every one of
    the 32 layers: each group's prefix is written once from its first member's rows, the other
    members read it back and prefill only their own rows, then score, top-k and compaction
    into copy-on-write blocks.  Each layer's call is timed with events around it after a first
    call; the host work inside the call (tables, offsets) is counted, so this is conservative."""
    import numpy as np
    from kv_cache_sparsification_amd.cache_manager import PagedKVCache
    dev = torch.device("cuda:0")
    w = wl.WORKLOADS[5]
    seqs = [wl.mix_sequence(w, i, i) for i in range(w.num_seqs)]
    lengths = [sq.n for sq in seqs]
    cache = PagedKVCache(w.budgets, wl.mix_pool_sizes(w), prefix_len=w.prefix_len, prefix_in_compressed=True)
    plans = {sq.seq_id: cache.admit(sq.seq_id, sq.group, sq.n) for sq in seqs}
    q_all, k, v, cu = wl.device_batch(w, 3, lengths, [sq.seq_id for sq in seqs], device=dev)
    batch = [(sq.seq_id, sq.group, sq.n) for sq in seqs]
    stream = torch.cuda.current_stream()
    total_us, computed = 0.0, None
    per_class = {}
    for layer in range(w.n_layers):
        k_pool, v_pool = kvs.new_pools(cache.alloc[layer].num_blocks, w.hkv, w.d, device=dev)
        first = [kvs.prefix_rows_reused(cache, layer, plans[sq.seq_id][layer], sq.n, w.alpha) for sq in seqs]
        q = torch.cat([q_all[cu[s] + first[s]:cu[s + 1]] for s in range(len(seqs))])
        for rep in range(2):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            kvs.prefill_compress_admission(cache, layer, batch, plans, q, k, v, w.alpha, k_pool, v_pool)
            e1.record(stream)
            torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3
        total_us += us
        computed = sum(n - f for n, f in zip(lengths, first))
        cls = "full" if w.budgets[layer] is None else "compressed"
        per_class.setdefault(cls, []).append(us)
        del k_pool, v_pool
    del q_all, k, v
    torch.cuda.empty_cache()
    T = sum(lengths)
    return {"workload": "64 prompts log-uniform [512,32768], 8 groups of 8 sharing a 2048-token prefix, 32 layers "
                        "(0-2 full, pyramid k 2048..128), one admission wave with the prefix read back from the "
                        "shared blocks",
            "prompt_tokens": T, "rows_computed_per_layer": computed, "rows_reused_per_layer": T - computed,
            "us_32_layers": round(total_us, 1), "prompt_tok_s_32_layers": round(T / (total_us * 1e-6), 1),
            "us_per_layer": {c: round(float(np.mean(x)), 1) for c, x in per_class.items()}}


def paged_memory(wl, iterations=1000):
    """Slots taken from the pool that hold no token ([PAG] "How paging works": with blocks only
    the tail of each table's last block is empty).  The 32-layer, 20-prompt workload: its
    tables over the 500 decode steps, every layer.  The continuous-batch mix: the product's
    cache manager driven over the
    continuous-batch trace (shared prefixes counted once), sampled every 10 iterations; beside
    it, what reserving each slot's longest possible sequence contiguously would leave empty."""
    import numpy as np
    from kv_cache_sparsification_amd.cache_manager import PagedKVCache
    w3 = wl.WORKLOADS[3]
    lens3 = w3.seq_lengths()
    used = taken = 0
    for kb in w3.budgets:
        for n in lens3:
            c = n if kb is None or kb >= n else kb
            L = c + np.arange(w3.decode_steps + 1)
            used += int(L.sum())
            taken += int((16 * (-(-L // 16))).sum())
    w5 = wl.WORKLOADS[5]
    cache = PagedKVCache(w5.budgets, wl.mix_pool_sizes(w5), prefix_len=w5.prefix_len)
    live = []
    u5 = t5 = 0
    reserved_used = 0
    for it, (admitted, finished) in enumerate(wl.mix_trace(w5, iterations)):
        for sq in admitted:
            cache.admit(sq.seq_id, sq.group, sq.n)
            live.append(sq.seq_id)
        for sid in live:
            for l in range(w5.n_layers):
                cache.append(sid, l)
        if it % 10 == 5:
            for l in range(w5.n_layers):
                a, b = cache.slot_usage(l)
                u5 += a
                t5 += b
            reserved_used += sum(cache.length[(sid, l)] for sid in live for l in range(w5.n_layers))
        for sid in finished:
            cache.finish(sid)
            live.remove(sid)
    samples = len(range(5, iterations, 10))
    reserve = samples * w5.num_seqs * w5.n_layers * (w5.len_range[1] + w5.lifetime_range[1])
    return {"tail_slot_frac_20_prompts": round(1 - used / taken, 5),
            "note_20_prompts": "20 prompts x 32 layers, every decode step 0..500",
            "tail_slot_frac_continuous_mix": round(1 - u5 / t5, 5),
            "contiguous_reservation_waste_frac_continuous_mix": round(1 - reserved_used / reserve, 4),
            "note_continuous_mix": f"continuous-batch trace, {iterations} iterations sampled every 10, 32 layers; the "
                       "reservation figure assumes each slot holds room for 32768 + 500 tokens in every layer"}


def fp8_layer(kvs, torch, wl, w, k, v, cu_d, keep, keep_off, steps):
    """The bench layer with an 8-bit cache: the quantizing compaction of the kept rows (timed
    like the other prompt-side kernels, as a graph of back-to-back launches) and `steps` decode
    steps with append (one HIP graph)."""
    dev = torch.device("cuda:0")
    n, hq, hkv, d, kb = w.fixed_len, w.hq, w.hkv, w.d, w.budgets[0]
    k_eff = min(kb, n)
    max_ctx = k_eff + steps
    nblk = -(-max_ctx // 16)
    pools = kvs.new_pools_fp8(nblk, hkv, d, device=dev)
    tbl = torch.arange(nblk, dtype=torch.int32, device=dev).flip(0).reshape(1, nblk).contiguous()
    comp_us = kernel_graph_us(torch, lambda: kvs.kvs_compact_paged_fp8(k, v, cu_d, keep, keep_off, k_eff, *pools, tbl),
                              50)
    comp_bytes = 4 * k_eff * hkv * d + 2 * k_eff * hkv * (d + 4) + 4 * hkv * k_eff
    ctx = torch.arange(k_eff + 1, k_eff + steps + 1, dtype=torch.int32, device=dev).reshape(steps, 1)
    qs, nks, nvs = zip(*[wl.device_decode_step(w, 0, 2000 + s, [0], device=dev) for s in range(steps)])
    ws = torch.empty(max(kvs.kvs_paged_decode_workspace_size(1, hq, hkv, d, max_ctx), 1), dtype=torch.uint8,
                     device=dev)
    od = torch.empty(steps, 1, hq, d, dtype=torch.bfloat16, device=dev)

    def run():
        for s in range(steps):
            kvs.kvs_paged_decode_fp8(qs[s], *pools, tbl, ctx[s], max_ctx, new_k=nks[s], new_v=nvs[s], o=od[s],
                                     workspace=ws)

    kvs.kvs_compact_paged_fp8(k, v, cu_d, keep, keep_off, k_eff, *pools, tbl)
    us = _graph_time_us(torch, run, steps, reps=1)
    mean_L = k_eff + (steps + 1) / 2.0
    nbytes = decode_bytes(mean_L, hq, hkv, d, fp8=True)
    return {"workload": f"bench layer, 8-bit E4M3 cache: compaction of k={k_eff} kept rows per KV head, "
                        f"then {steps} decode steps with append (HIP graph)",
            "compact_us": round(comp_us, 3), "compact_algorithmic_bytes": int(comp_bytes),
            "compact_GBs": round(comp_bytes / (comp_us * 1e-6) / 1e9, 1),
            "decode_us_per_step": round(us, 3), "decode_tok_s": round(1.0 / (us * 1e-6), 1),
            "decode_algorithmic_bytes_per_step": int(nbytes),
            "decode_GBs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def decode_32_layers(kvs, torch, wl, steps, fp8=False):
    """One decode step of a whole 32-layer model's attention (the concurrency-20 workload: 20
    prompts of 1000-4000 tokens, layers 0-2 full, 3-31 at k=512), each layer with its own pools
    and tables, `steps` steps captured as one HIP graph and also launched eagerly."""
    import numpy as np
    w = wl.WORKLOADS[3]
    B, hq, hkv, d = w.num_seqs, w.hq, w.hkv, w.d
    lengths = w.seq_lengths()
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(3232)
    layers = []
    for layer in range(w.n_layers):
        k_l = w.budgets[layer]
        ctx0 = [n if k_l is None else min(k_l, n) for n in lengths]
        max_ctx = max(ctx0) + steps
        nbs = [-(-(c + steps) // 16) for c in ctx0]
        nb_total = sum(nbs)
        if fp8:
            pools = kvs.new_pools_fp8(nb_total, hkv, d, device=dev)
            for t in pools[:2]:
                t.copy_(torch.randint(0, 0x7F, t.shape, generator=gen, device=dev, dtype=torch.uint8))
            for t in pools[2:]:
                t.copy_(torch.rand(t.shape, generator=gen, device=dev) * 0.01 + 0.002)
        else:
            pools = kvs.new_pools(nb_total, hkv, d, device=dev)
            for t in pools:
                t.copy_(torch.randn(t.shape, generator=gen, device=dev).to(torch.bfloat16))
        max_blocks = max(nbs)
        tbl = np.full((B, max_blocks), -1, np.int32)
        perm = np.random.default_rng(layer).permutation(nb_total).astype(np.int32)
        used = 0
        for s_, nb in enumerate(nbs):
            tbl[s_, :nb] = perm[used:used + nb]
            used += nb
        lens = torch.tensor([[c + st + 1 for c in ctx0] for st in range(steps)], dtype=torch.int32, device=dev)
        ws = torch.empty(max(kvs.kvs_paged_decode_workspace_size(B, hq, hkv, d, max_ctx), 1), dtype=torch.uint8,
                         device=dev)
        layers.append((pools, torch.from_numpy(tbl).to(dev), lens, max_ctx, ws))
    qs = torch.randn(steps, B, hq, d, generator=gen, device=dev).to(torch.bfloat16)
    nks = torch.randn(steps, B, hkv, d, generator=gen, device=dev).to(torch.bfloat16)
    nvs = torch.randn(steps, B, hkv, d, generator=gen, device=dev).to(torch.bfloat16)
    od = torch.empty(w.n_layers, B, hq, d, dtype=torch.bfloat16, device=dev)
    decode = kvs.kvs_paged_decode_fp8 if fp8 else kvs.kvs_paged_decode

    def run():
        for st in range(steps):
            for li, (pools, tbl, lens, max_ctx, ws) in enumerate(layers):
                decode(qs[st], *pools, tbl, lens[st], max_ctx, new_k=nks[st], new_v=nvs[st], o=od[li], workspace=ws)

    graph_us = _graph_time_us(torch, run, steps)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    run()
    e1.record(stream)
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1e3 / steps
    cached = sum(sum(n if k_l is None else min(k_l, n) for n in lengths) for k_l in w.budgets)
    kv_bytes = cached * hkv * (2 * d + 8 if fp8 else 4 * d)
    return {"workload": f"{B} sequences x {min(lengths)}-{max(lengths)} prompt tokens, {w.n_layers} layers "
                        f"(3 full, 29 at k=512), {hq}q/{hkv}kv heads, d={d}: one decode step of every layer"
                        + (", 8-bit E4M3 cache" if fp8 else ""),
            "graph_us_per_step": round(graph_us, 2), "eager_us_per_step": round(eager_us, 2),
            "launches_per_step": sum(2 if kvs.kvs_paged_decode_workspace_size(B, hq, hkv, d, l[3]) else 1
                                     for l in layers),
            "cached_tokens_per_head": cached,
            "traffic": _traffic_rate(measured_scale_traffic("decode_32_layers" + ("_fp8" if fp8 else "")),
                                     "bytes_per_step", graph_us),
            # K/V bytes read per step (about 1.8 GB: more than the 256 MB Infinity Cache holds,
            # so this is an HBM rate); 8-bit rows carry one fp32 scale each for K and V
            "kv_bytes_per_step": kv_bytes,
            "achieved_GBs": round(kv_bytes / (graph_us * 1e-6) / 1e9, 1),
            "peak_GBs": HBM_PEAK_GBS,
            "frac": round(kv_bytes / (graph_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "tok_s": round(B / (graph_us * 1e-6), 1)}


def prefix_reuse(kvs, torch, wl, w, q, k, v, reps=10):
    """The bench layer when the first 2048 prompt tokens are found in the cache (block-hash
    match): their K/V come back from the blocks (gather) and only rows 2048-3999 are prefilled
    against all 4000 keys, then window score and top-k with compaction as usual, captured as one
    graph and timed with clock stamps between the launches (as the timed step's prompt phase)."""
    import numpy as np
    dev = torch.device("cuda:0")
    n, hq, hkv, d, alpha, kb = w.fixed_len, w.hq, w.hkv, w.d, w.alpha, w.budgets[0]
    P = 2048
    nblk_p = P // 16
    k_pool, v_pool = kvs.new_pools(nblk_p + 32, hkv, d, device=dev)
    tbl_p = torch.arange(nblk_p, dtype=torch.int32, device=dev).reshape(1, nblk_p)
    cu_full = torch.tensor([0, n], dtype=torch.int32, device=dev)
    kvs.kvs_compact_paged(k, v, torch.tensor([0, P], dtype=torch.int32, device=dev), None, None, P, k_pool, v_pool,
                          tbl_p)
    k_all = torch.empty_like(k)
    v_all = torch.empty_like(v)
    k_all[P:] = k[P:]
    v_all[P:] = v[P:]
    q_rows = q[P:].contiguous()
    cu_q = torch.tensor([0, n - P], dtype=torch.int32, device=dev)
    k_eff = min(kb, n)
    keep_off = torch.tensor([0, k_eff], dtype=torch.int32, device=dev)
    ctbl = torch.arange(nblk_p, nblk_p + (-(-k_eff // 16)), dtype=torch.int32, device=dev).reshape(1, -1)
    counts = torch.tensor([P], dtype=torch.int32, device=dev)
    start = torch.tensor([0], dtype=torch.int32, device=dev)
    marks = ["gather", "prefill_chunk", "window", "topk_compact"]
    o_c = torch.empty_like(q_rows)
    lse_c = torch.empty(hq, n - P, dtype=torch.float32, device=dev)
    S_c = torch.empty(hkv, n, dtype=torch.float32, device=dev)
    keep_c = torch.empty(hkv * k_eff, dtype=torch.int32, device=dev)
    stamps = torch.zeros(len(marks) + 1, dtype=torch.int64, device=dev)

    def step():
        kvs.kvs_probe_timestamp(stamps[0:1])
        kvs.kvs_gather_paged(k_pool, v_pool, tbl_p, counts, start, P, k_all, v_all)
        kvs.kvs_probe_timestamp(stamps[1:2])
        kvs.kvs_prefill_attn_lse_chunk(q_rows, k_all, v_all, cu_q, cu_full, n - P, n, o=o_c, lse=lse_c)
        kvs.kvs_probe_timestamp(stamps[2:3])
        kvs.kvs_window_score_chunk(q_rows, k_all, lse_c, cu_q, cu_full, n, alpha, scores=S_c)
        kvs.kvs_probe_timestamp(stamps[3:4])
        kvs.kvs_topk_compact(S_c, k_all, v_all, cu_full, n, alpha, kb, keep_off, k_pool, v_pool, ctbl, keep_idx=keep_c)
        kvs.kvs_probe_timestamp(stamps[4:5])

    # one captured graph, a clock stamp before each launch and after the last: each stage's span
    # is its kernel plus one in-graph launch boundary; the graph's start latency is outside
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    spans = []
    for r in range(reps + 1):
        graph.replay()
        torch.cuda.synchronize()
        if r:
            t = stamps.cpu().numpy().astype(np.float64) * (1e6 / REALTIME_HZ)      # us
            spans.append(np.diff(t))
    per = {m: float(np.mean([x[i] for x in spans])) for i, m in enumerate(marks)}
    total = sum(per.values())
    flops = 2.0 * d * hq * sum(2 * (i + 1) for i in range(P, n))
    return {"workload": f"bench layer n={n} with the first {P} tokens reused from the cache: gather, prefill of "
                        f"rows {P}-{n - 1} against {n} keys, window score, top-k with compaction (one launch)",
            "us": {m: round(v_, 2) for m, v_ in per.items()}, "total_us": round(total, 2),
            "prefill_chunk_TFLOPs": round(flops / (per["prefill_chunk"] * 1e-6) / 1e12, 1),
            "prompt_tok_s": round(n / (total * 1e-6), 1)}



def decode_evict(kvs, torch, wl, w, k_pool, v_pool, tbl, S, cu_d, keep, keep_off, steps):
    """Decode with scoring and eviction on the bench layer: the compressed cache is full
    (k_eff = k_l), so every step picks each head's lowest-score replaceable slot and runs the
    scored decode (attention, then the probabilities added to the slot scores); `steps` steps
    replayed as one HIP graph.  Two launch plans: the slot choice as its own launch before each
    step (three launches per step), and the choice for the next step made by the step's
    merge-and-score kernel (kvs_paged_decode_scored_select, two launches per step)."""
    dev = torch.device("cuda:0")
    n, hq, hkv, d, alpha, cap = w.fixed_len, w.hq, w.hkv, w.d, w.alpha, w.budgets[0]
    stride = tbl.shape[1] * 16
    sl_sc0, sl_pos0 = kvs.kvs_slot_init(S, cu_d, keep, keep_off, stride)
    n_fill = torch.tensor([cap], dtype=torch.int32, device=dev)
    pos = torch.tensor([[n + s] for s in range(steps + 1)], dtype=torch.int32, device=dev)
    qs, nks, nvs = zip(*[wl.device_decode_step(w, 0, 1000 + s, [0], device=dev) for s in range(steps)])
    ws = torch.empty(kvs.kvs_paged_decode_scored_workspace_size(1, hq, hkv, d, cap), dtype=torch.uint8, device=dev)
    od = torch.empty(steps, 1, hq, d, dtype=torch.bfloat16, device=dev)
    sl_sc, sl_pos = sl_sc0.clone(), sl_pos0.clone()
    dst = torch.empty(1, hkv, dtype=torch.int32, device=dev)
    dsts = torch.empty(steps + 1, 1, hkv, dtype=torch.int32, device=dev)

    def run3():
        for s in range(steps):
            kvs.kvs_decode_select_slot(sl_sc, sl_pos, n_fill, pos[s], cap, alpha, dst_slot=dst)
            kvs.kvs_paged_decode_scored(qs[s], k_pool, v_pool, tbl, n_fill, cap, sl_sc, new_k=nks[s], new_v=nvs[s],
                                        dst_slots=dst, o=od[s], workspace=ws)

    def run2():
        kvs.kvs_decode_select_slot(sl_sc, sl_pos, n_fill, pos[0], cap, alpha, dst_slot=dsts[0])
        for s in range(steps):
            kvs.kvs_paged_decode_scored_select(qs[s], k_pool, v_pool, tbl, n_fill, cap, sl_sc, sl_pos, cap, alpha,
                                               pos[s + 1], next_dst_slots=dsts[s + 1], new_k=nks[s], new_v=nvs[s],
                                               dst_slots=dsts[s], o=od[s], workspace=ws)

    us3 = _graph_time_us(torch, run3, steps)
    sl_sc.copy_(sl_sc0)
    sl_pos.copy_(sl_pos0)
    us2 = _graph_time_us(torch, run2, steps)
    return {"workload": f"bench layer, cache full at k={cap} (alpha={alpha}): every step evicts per KV head, "
                        f"{steps} steps (HIP graph)",
            "us_per_step": round(us2, 3), "tok_s": round(1.0 / (us2 * 1e-6), 1), "launches_per_step": 2,
            "separate_selection": {"us_per_step": round(us3, 3), "tok_s": round(1.0 / (us3 * 1e-6), 1),
                                   "launches_per_step": 3}}


def cpu_baseline(w, qb, kbits, vb, dec, budget_s):
    """The fp64 oracle, as it stands, on the host cores.

    Prefill+compress: KV-head groups (G query heads + their KV head) of the same n=4000 layer
    are run one after another until about 70% of the time budget is used (normally all 8);
    the rate is scaled from the groups done to the full layer.  Decode: oracle decode steps
    over the compressed cache (all heads), as many of the 500 as fit the rest of the budget.
    """
    from threadpoolctl import threadpool_limits
    threads = host_cores()
    with threadpool_limits(limits=threads):
        return _cpu_baseline(w, qb, kbits, vb, dec, budget_s, threads)


def host_cores() -> int:
    """Cores this process may use: its affinity mask, capped by a cgroup CPU quota if one is set."""
    cores = len(os.sched_getaffinity(0))
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if quota != "max":
            cores = min(cores, max(1, math.ceil(int(quota) / int(period))))
    except (OSError, ValueError):
        pass
    return cores


def _cpu_baseline(w, qb, kbits, vb, dec, budget_s, threads):
    import numpy as np
    import oracle
    import workloads as wl
    n, alpha, kb, G, hkv = w.fixed_len, w.alpha, w.budgets[0], w.g, w.hkv
    k_eff = min(kb, n)
    f = wl.bf16_bits_to_f64
    keeps = []
    t0 = time.perf_counter()
    for g in range(hkv):
        q = f(qb[:, g * G:(g + 1) * G])
        k = f(kbits[:, g:g + 1])
        v = f(vb[:, g:g + 1])
        O, lse, _, _ = oracle.causal_attention(q, k, v)
        S = oracle.window_score(q, k, lse, alpha)
        keep = oracle.select_keep(S[0], n, alpha, kb)
        nbk = oracle.blocks_for(k_eff)
        pk = np.zeros((nbk, 1, 16, w.d)); pv = np.zeros_like(pk)
        oracle.compact_into_pool(k, v, keep[None], list(range(nbk)), pk, pv)
        keeps.append(keep)
        if time.perf_counter() - t0 > 0.7 * budget_s:
            break
    t_pre = time.perf_counter() - t0
    groups = len(keeps)
    prefill_tok_s = n / (t_pre / groups * hkv)

    # decode over the compressed cache of every head (heads not reached above keep the
    # first group's index set: the timing does not depend on which tokens are kept)
    kf, vf = f(kbits), f(vb)
    ck = np.stack([kf[keeps[min(g, groups - 1)], g] for g in range(hkv)], axis=1)
    cv = np.stack([vf[keeps[min(g, groups - 1)], g] for g in range(hkv)], axis=1)
    t1 = time.perf_counter()
    done = 0
    for s, (dqb, dkb, dvb) in enumerate(dec):
        ck = np.concatenate([ck, f(dkb)], axis=0)
        cv = np.concatenate([cv, f(dvb)], axis=0)
        oracle.decode_attention(f(dqb)[0], ck, cv)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    t_dec = time.perf_counter() - t1
    return {"value": round(prefill_tok_s, 2), "unit": "tok/s", "cores": int(threads), "kind": "oracle",
            "sample": f"prefill+compress of {groups} of {hkv} KV-head groups of the n={n} layer "
                      f"({t_pre:.2f} s, scaled to the layer); decode: {done} of {len(dec)} steps ({t_dec:.2f} s)",
            "decode_value": round(done / t_dec, 2),
            "cores_note": "len(os.sched_getaffinity(0)), capped by the cgroup CPU quota; BLAS threads set to it",
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
