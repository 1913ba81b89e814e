"""Seeded synthetic inputs for the KV-sparsity prefill-and-compress path.

This module is shared by the tests, the benchmark and the oracle's callers. It
holds shapes, seeds and value distributions only: none of the method's
arithmetic (no attention, scoring, selection or paging) lives here.

Value recipe (all workloads):
  * Q, K, V ~ N(0, 1) drawn in fp32 and rounded once to bf16 (round to nearest
    even).
  * Attention-sink structure: the key rows at the sink positions are scaled by
    20 in two fixed channels before rounding.  The channels are 1415 mod d and
    2533 mod d, the two feature dimensions that carry the massive activations
    of LLaMA2-7B, and the positions are the start token plus the first
    '.'-like token (index 17).  Source: Novita AI, "How KV Sparsity Achieves
    1.5x Acceleration for vLLM", Introduction, Fig. 1.  Q and V are untouched.
  * Decode queries and the appended K/V are fresh N(0, 1) per step and layer.

Seeds: workload c uses seed 1000 + c; every tensor draws from its own PCG64
stream, spawned from SeedSequence(seed, spawn_key=(layer, seq, tensor, step)).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

BLOCK_SIZE = 16

# Tensor ids used in the spawn keys.
T_Q, T_K, T_V, T_DQ, T_DK, T_DV, T_LEN, T_LIFE = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    hq: int
    hkv: int
    d: int
    alpha: int
    n_layers: int
    budgets: tuple          # per layer: None = full cache, else k_l
    decode_steps: int
    sink_positions: tuple
    num_seqs: int
    fixed_len: Optional[int] = None       # every prompt has this length
    len_range: Optional[tuple] = None     # (lo, hi) inclusive
    len_dist: str = "fixed"               # fixed | uniform | loguniform
    prefix_len: int = 0                   # shared prefix per group (mix workload)
    group_size: int = 0
    lifetime_range: Optional[tuple] = None
    iterations: int = 0

    @property
    def seed(self) -> int:
        return 1000 + self.cid

    @property
    def g(self) -> int:
        return self.hq // self.hkv

    @property
    def sink_channels(self) -> tuple:
        return (1415 % self.d, 2533 % self.d)

    def rng(self, layer: int, seq: int, tensor: int, step: int = 0) -> np.random.Generator:
        ss = np.random.SeedSequence(self.seed, spawn_key=(layer, seq, tensor, step))
        return np.random.Generator(np.random.PCG64(ss))

    def seq_lengths(self) -> list:
        if self.len_dist == "fixed":
            return [self.fixed_len] * self.num_seqs
        r = self.rng(0, 0, T_LEN)
        lo, hi = self.len_range
        if self.len_dist == "uniform":
            return [int(x) for x in r.integers(lo, hi + 1, size=self.num_seqs)]
        if self.len_dist == "loguniform":
            u = r.random(self.num_seqs)
            return [int(round(math.exp(math.log(lo) + x * (math.log(hi) - math.log(lo))))) for x in u]
        raise ValueError(self.len_dist)


def _pyramid(n_layers=32, first=3, k_first=2048, k_last=128):
    out = [None] * first
    span = n_layers - 1 - first
    for l in range(first, n_layers):
        out.append(k_first - int(round((l - first) * (k_first - k_last) / span)))
    return tuple(out)


WORKLOADS = {
    1: Workload(1, "tiny-1layer-n256", hq=4, hkv=2, d=64, alpha=16, n_layers=1, budgets=(64,),
                decode_steps=8, sink_positions=(0,), num_seqs=1, fixed_len=256),
    2: Workload(2, "llama3-8b-layer-n4000", hq=32, hkv=8, d=128, alpha=32, n_layers=1, budgets=(400,),
                decode_steps=500, sink_positions=(0, 17), num_seqs=1, fixed_len=4000),
    3: Workload(3, "32layer-conc20-n1000..4000", hq=32, hkv=8, d=128, alpha=32, n_layers=32,
                budgets=(None,) * 3 + (512,) * 29, decode_steps=500, sink_positions=(0, 17),
                num_seqs=20, len_range=(1000, 4000), len_dist="uniform"),
    4: Workload(4, "long-context-4x30000", hq=32, hkv=8, d=128, alpha=64, n_layers=32,
                budgets=(None,) * 3 + (3000,) * 29, decode_steps=500, sink_positions=(0, 17),
                num_seqs=4, fixed_len=30000),
    5: Workload(5, "continuous-mix-64-loguniform-512..32768", hq=32, hkv=8, d=128, alpha=32, n_layers=32,
                budgets=_pyramid(), decode_steps=0, sink_positions=(0, 17), num_seqs=64,
                len_range=(512, 32768), len_dist="loguniform", prefix_len=2048, group_size=8,
                lifetime_range=(100, 500), iterations=1000),
}


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).copy()
    u += ((u >> 16) & 1) + 0x7FFF
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ---------------------------------------------------------------- prefill
def _normal_rows(w: Workload, layer: int, seq: int, tensor: int, n: int, heads: int) -> np.ndarray:
    return w.rng(layer, seq, tensor).standard_normal((n, heads, w.d), dtype=np.float32)


def apply_sinks(w: Workload, k_f32: np.ndarray) -> None:
    """Scale the sink key rows by 20 in the two massive-activation channels (in place)."""
    n = k_f32.shape[0]
    for p in w.sink_positions:
        if p < n:
            for c in w.sink_channels:
                k_f32[p, :, c] *= 20.0


def prefill_seq(w: Workload, layer: int, seq: int, n: int):
    """bf16 bit patterns Q [n][Hq][d], K, V [n][Hkv][d] for one prompt."""
    q = _normal_rows(w, layer, seq, T_Q, n, w.hq)
    k = _normal_rows(w, layer, seq, T_K, n, w.hkv)
    v = _normal_rows(w, layer, seq, T_V, n, w.hkv)
    apply_sinks(w, k)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def prefill_batch(w: Workload, layer: int, lengths: Sequence[int], seq_ids: Optional[Sequence[int]] = None):
    """Ragged, token-major batch: Q [T][Hq][d], K/V [T][Hkv][d] (uint16 bf16 bits) and cu_seqlens."""
    if seq_ids is None:
        seq_ids = range(len(lengths))
    qs, ks, vs = [], [], []
    for sid, n in zip(seq_ids, lengths):
        q, k, v = prefill_seq(w, layer, sid, n)
        qs.append(q); ks.append(k); vs.append(v)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return np.concatenate(qs), np.concatenate(ks), np.concatenate(vs), cu


def decode_step_inputs(w: Workload, layer: int, step: int, batch: int, seq_ids: Optional[Sequence[int]] = None):
    """Fresh N(0,1) decode query [B][Hq][d] and the appended K/V [B][Hkv][d] (bf16 bits)."""
    if seq_ids is None:
        seq_ids = range(batch)
    q = np.stack([w.rng(layer, s, T_DQ, step).standard_normal((w.hq, w.d), dtype=np.float32) for s in seq_ids])
    k = np.stack([w.rng(layer, s, T_DK, step).standard_normal((w.hkv, w.d), dtype=np.float32) for s in seq_ids])
    v = np.stack([w.rng(layer, s, T_DV, step).standard_normal((w.hkv, w.d), dtype=np.float32) for s in seq_ids])
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def spawn_seed(w: Workload, *key) -> int:
    """A 63-bit seed for a device stream, derived from (workload seed, key)."""
    ss = np.random.SeedSequence(w.seed, spawn_key=tuple(int(x) for x in key))
    return int(ss.generate_state(1, dtype=np.uint64)[0]) & ((1 << 63) - 1)


def _device_normal_f32(shape, seed: int, device):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


# Device-drawn inputs: torch's seeded Philox streams on the GPU, one per (layer, seq, tensor,
# step).  Used where host generation of hundreds of millions of values would dominate a test
# (the 32-layer, 30k-token and mixed workloads); the oracle gets the sampled slices copied back,
# so both sides see the same bf16 values.  Same distribution and sink rule as the host path.
PREFIX_SEQ_BASE = 1 << 20    # seq id space of the shared prefixes of the mixed workload


def device_prompt(w: Workload, layer: int, seq: int, n: int, device="cuda", prefix_group=None, prefix_len=0):
    """bf16 Q [n][Hq][d], K, V [n][Hkv][d] on the device for one prompt.

    With prefix_group set, rows 0..prefix_len-1 come from the group's own streams (identical for
    every member of the group) and the rest from the prompt's streams.
    """
    import torch
    parts = []
    for tensor, heads in ((T_Q, w.hq), (T_K, w.hkv), (T_V, w.hkv)):
        if prefix_group is None or prefix_len <= 0:
            x = _device_normal_f32((n, heads, w.d), spawn_seed(w, layer, seq, tensor), device)
        else:
            pre = _device_normal_f32((prefix_len, heads, w.d),
                                     spawn_seed(w, layer, PREFIX_SEQ_BASE + prefix_group, tensor), device)
            suf = _device_normal_f32((n - prefix_len, heads, w.d), spawn_seed(w, layer, seq, tensor), device)
            x = torch.cat([pre, suf])
        if tensor == T_K:
            for p in w.sink_positions:
                if p < n:
                    for c in w.sink_channels:
                        x[p, :, c] *= 20.0
        parts.append(x.to(torch.bfloat16))
    return tuple(parts)


def device_batch(w: Workload, layer: int, lengths: Sequence[int], seq_ids: Sequence[int], device="cuda", **kw):
    """Ragged device batch (Q, K, V, cu_seqlens as int32 numpy) of the given prompts."""
    import torch
    qs, ks, vs = [], [], []
    for sid, n in zip(seq_ids, lengths):
        q, k, v = device_prompt(w, layer, sid, n, device=device, **kw)
        qs.append(q); ks.append(k); vs.append(v)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return torch.cat(qs), torch.cat(ks), torch.cat(vs), cu


def device_decode_step(w: Workload, layer: int, step: int, seq_ids: Sequence[int], device="cuda"):
    """Fresh N(0,1) decode query [B][Hq][d] and appended K/V [B][Hkv][d], bf16 on the device."""
    import torch
    out = []
    for tensor, heads in ((T_DQ, w.hq), (T_DK, w.hkv), (T_DV, w.hkv)):
        out.append(torch.stack([_device_normal_f32((heads, w.d), spawn_seed(w, layer, s, tensor, step), device)
                                for s in seq_ids]).to(torch.bfloat16))
    return tuple(out)


# ---------------------------------------------------------------- continuous-batch trace
@dataclasses.dataclass(frozen=True)
class MixSequence:
    seq_id: int        # admission index (0..63 are the initial batch)
    slot: int
    group: int         # prefix group = slot // group_size
    n: int             # prompt length
    lifetime: int      # decode tokens before it finishes


def mix_sequence(w: Workload, seq_id: int, slot: int) -> MixSequence:
    """Prompt length log-uniform in the workload's range and lifetime uniform in its range, per admission."""
    r = w.rng(0, seq_id, T_LIFE)
    lo, hi = w.len_range
    u = float(r.random())
    n = int(round(math.exp(math.log(lo) + u * (math.log(hi) - math.log(lo)))))
    llo, lhi = w.lifetime_range
    life = int(r.integers(llo, lhi + 1))
    return MixSequence(seq_id, slot, slot // w.group_size, n, life)


def mix_pool_sizes(w: Workload) -> list:
    """Blocks per layer for the continuous-batch trace: full layers hold every slot at its longest
    prompt plus decode and the group prefixes; compressed layers the budget plus decode per slot,
    the prefixes and the transient copy-on-write blocks, with room to spare."""
    full = w.num_seqs * (-(-(w.len_range[1] + w.lifetime_range[1]) // BLOCK_SIZE)) + 8 * (w.prefix_len // 16) + 64
    return [full if k is None else
            w.num_seqs * (-(-(k + w.lifetime_range[1]) // BLOCK_SIZE)) + 16 * (w.prefix_len // 16) + 64
            for k in w.budgets]


def mix_trace(w: Workload, iterations: int):
    """Per iteration: (admitted sequences, finished seq ids).

    Iteration semantics: admitted prompts are prefilled and compressed first, then every live
    sequence decodes one token, then sequences that reached their lifetime finish and free
    their slot, which the next iteration refills (slots in ascending order, admission ids
    counting up).  Depends only on the seeded lengths and lifetimes.
    """
    live = {}
    decoded = {}
    next_id = 0
    empty = list(range(w.num_seqs))
    out = []
    for _ in range(iterations):
        admitted = []
        for slot in sorted(empty):
            sq = mix_sequence(w, next_id, slot)
            next_id += 1
            live[sq.seq_id] = sq
            decoded[sq.seq_id] = 0
            admitted.append(sq)
        empty = []
        finished = []
        for sid in sorted(live):
            decoded[sid] += 1
            if decoded[sid] >= live[sid].lifetime:
                finished.append(sid)
        for sid in finished:
            empty.append(live[sid].slot)
            del live[sid]
        out.append((admitted, finished))
    return out
