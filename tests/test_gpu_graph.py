"""A multi-layer decode step captured as one HIP graph (next row f4) gives the eager results on
every replay, with the program's own eager work and synchronisations between replays; the
eager results themselves match the fp64 oracle.  The prompt-side chain the bench captures
(prefill, window score, top-k fused with compaction) replays bit for bit as well.

Three layers of different shapes (a full layer of ragged contexts, a compressed layer, an
8-bit compressed layer) and four batched decode steps with append per replay.  Appends are
idempotent across replays (the same tokens go to the same slots), so every replay must
reproduce the eager outputs bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
import workloads as wl
from tests._parity import bf16_to_f64, i32, assert_rows_close

pytestmark = pytest.mark.gpu

kvs = pytest.importorskip("kv_cache_sparsification_amd")


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _layer(rng, lengths, hkv, d, steps, fp8):
    nbs = [-(-(n + steps) // 16) for n in lengths]
    nb = sum(nbs) + 2
    perm = rng.permutation(nb)
    tables = np.full((len(lengths), max(nbs)), -1, np.int32)
    used = 0
    for s, c in enumerate(nbs):
        tables[s, :c] = perm[used:used + c]
        used += c
    T = sum(lengths)
    kb = wl.f32_to_bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
    vb = wl.f32_to_bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    up = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
    if fp8:
        pools = kvs.new_pools_fp8(nb, hkv, d)
        kvs.kvs_compact_paged_fp8(up(kb), up(vb), i32(cu), None, None, max(lengths), *pools, i32(tables))
    else:
        pools = kvs.new_pools(nb, hkv, d)
        kvs.kvs_compact_paged(up(kb), up(vb), i32(cu), None, None, max(lengths), *pools, i32(tables))
    return dict(pools=pools, tables=tables, tbl=i32(tables), lengths=list(lengths), fp8=fp8, kb=kb, vb=vb, cu=cu,
                max_ctx=max(lengths) + steps)


def test_decode_graph_replays_match_eager_and_oracle():
    _say("three-layer decode step as a HIP graph, 4 steps, 5 replays")
    rng = np.random.default_rng(21)
    B, hq, hkv, d, steps = 6, 32, 8, 128, 4
    full_lens = [int(x) for x in rng.integers(300, 1500, B)]
    layers = [_layer(rng, full_lens, hkv, d, steps, False),
              _layer(rng, [min(256, n) for n in full_lens], hkv, d, steps, False),
              _layer(rng, [min(256, n) for n in full_lens], hkv, d, steps, True)]
    q = torch.from_numpy(rng.standard_normal((steps, B, hq, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    nk = torch.from_numpy(rng.standard_normal((steps, B, hkv, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    nv = torch.from_numpy(rng.standard_normal((steps, B, hkv, d), dtype=np.float32)).to(torch.bfloat16).cuda()
    for L in layers:
        L["lens"] = i32([[n + st + 1 for n in L["lengths"]] for st in range(steps)])
        L["ws"] = torch.empty(max(kvs.kvs_paged_decode_workspace_size(B, hq, hkv, d, L["max_ctx"]), 1),
                              dtype=torch.uint8, device="cuda")
        L["out"] = torch.empty(steps, B, hq, d, dtype=torch.bfloat16, device="cuda")

    def run():
        for st in range(steps):
            for L in layers:
                fn = kvs.kvs_paged_decode_fp8 if L["fp8"] else kvs.kvs_paged_decode
                fn(q[st], *L["pools"], L["tbl"], L["lens"][st], L["max_ctx"], new_k=nk[st], new_v=nv[st],
                   o=L["out"][st], workspace=L["ws"])

    run()                                   # eager
    torch.cuda.synchronize()
    eager = [L["out"].clone() for L in layers]

    # the eager results against the oracle (every step, every sequence): step st attends over
    # the cached rows and the new tokens of steps 0..st
    for li, L in enumerate(layers):
        for s in range(B):
            rows_k = wl.bf16_bits_to_f64(L["kb"][L["cu"][s]:L["cu"][s + 1]])
            rows_v = wl.bf16_bits_to_f64(L["vb"][L["cu"][s]:L["cu"][s + 1]])
            new_k = bf16_to_f64(nk[:, s])
            new_v = bf16_to_f64(nv[:, s])
            if L["fp8"]:
                rows_k = ofp8.dequantize_rows(*ofp8.quantize_rows(rows_k))
                rows_v = ofp8.dequantize_rows(*ofp8.quantize_rows(rows_v))
                new_k = ofp8.dequantize_rows(*ofp8.quantize_rows(new_k))
                new_v = ofp8.dequantize_rows(*ofp8.quantize_rows(new_v))
            for st in range(steps):
                kc = np.concatenate([rows_k, new_k[:st + 1]])
                vc = np.concatenate([rows_v, new_v[:st + 1]])
                o_ref, _ = oracle.decode_attention(bf16_to_f64(q[st])[s], kc, vc)
                assert_rows_close(bf16_to_f64(eager[li][st, s]), o_ref, what=f"layer {li} seq {s} step {st}")

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        run()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(5):
        for L in layers:
            L["out"].zero_()               # eager work between replays
        scratch = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for li, L in enumerate(layers):
            assert torch.equal(L["out"].view(torch.int16), eager[li].view(torch.int16)), f"replay {rep} layer {li}"
        del scratch


def test_clock_stamps_time_the_work_between_them():
    """Two clock stamps as the first and last launches of a captured graph (the bench's phase
    timer): they run in order, the counter ticks at 100 MHz (the span agrees with events around
    the replay, which add only the graph's start latency), and the span covers the work."""
    _say("clock stamps around 16 streaming reads of 256 MiB in a graph")
    buf = torch.zeros(256 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    stamps = torch.zeros(2, dtype=torch.int64, device="cuda")
    kvs.kvs_probe_stream_read(buf, 2048, sink=sink)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvs.kvs_probe_timestamp(stamps[0:1])
        for _ in range(16):
            kvs.kvs_probe_stream_read(buf, 2048, sink=sink)
        kvs.kvs_probe_timestamp(stamps[1:2])
    st = torch.cuda.current_stream()
    for rep in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        g.replay()
        e1.record(st)
        torch.cuda.synchronize()
        t0, t1 = (int(x) for x in stamps.cpu())
        span_ms = (t1 - t0) / 100e6 * 1e3
        ev_ms = e0.elapsed_time(e1)
        _say(f"replay {rep}: stamps {span_ms:.4f} ms, events {ev_ms:.4f} ms")
        assert t1 > t0 > 0
        assert 0.9 * ev_ms <= span_ms <= 1.01 * ev_ms + 0.005
    assert int(sink.abs().sum()) == 0       # the zero buffer folds to 0, never the probe's key


def test_prompt_side_graph_replays_match_eager():
    """The prompt-side chain the bench captures (prefill with LSE, window score, top-k fused with
    compaction into blocks) replayed as one graph, with eager work and synchronisations between
    replays: outputs, scores, kept indices and pools bit for bit as the eager launches left them."""
    w = wl.WORKLOADS[2]
    n, hq, hkv, d, alpha, kb = 2000, w.hq, w.hkv, w.d, w.alpha, w.budgets[0]
    _say(f"prompt-side graph: n={n} hq={hq} hkv={hkv} d={d} alpha={alpha} k={kb}")
    qb, kbits, vb, cu = wl.prefill_batch(w, 0, [n])

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, cu_d = up(qb), up(kbits), up(vb), i32(cu)
    o = torch.empty_like(q)
    lse = torch.empty(hq, n, dtype=torch.float32, device="cuda")
    S = torch.empty(hkv, n, dtype=torch.float32, device="cuda")
    keep = torch.empty(hkv * kb, dtype=torch.int32, device="cuda")
    koff = i32([0, kb])
    nblk = -(-kb // 16)
    k_pool, v_pool = kvs.new_pools(nblk + 3, hkv, d)
    tbl = i32([list(np.random.default_rng(7).permutation(nblk + 3)[:nblk])])

    def chain():
        kvs.kvs_prefill_attn_lse(q, k, v, cu_d, n, o=o, lse=lse)
        kvs.kvs_window_score(q, k, lse, cu_d, n, alpha, scores=S)
        kvs.kvs_topk_compact(S, k, v, cu_d, n, alpha, kb, koff, k_pool, v_pool, tbl, keep_idx=keep)

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in (o.view(torch.int16), lse, S, keep, k_pool.view(torch.int16),
                                    v_pool.view(torch.int16))]

    k_pool.view(torch.int16).fill_(0x7FC0)          # blocks the table does not name stay as filled
    v_pool.view(torch.int16).fill_(0x7FC0)
    chain()
    eager = snapshot()
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        chain()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain()
    for rep in range(3):
        for t in (o, lse, S):                       # eager work between replays: clobber the outputs
            t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).fill_(-1)
        keep.fill_(-1)
        k_pool.view(torch.int16).fill_(0x7FC0)
        v_pool.view(torch.int16).fill_(0x7FC0)
        torch.cuda.synchronize()
        graph.replay()
        got = snapshot()
        for name, a, b in zip(("O", "LSE", "S", "keep", "K pool", "V pool"), eager, got):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager run"
