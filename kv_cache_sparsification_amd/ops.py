"""Thin torch-facing binding of the libkvs device calls (argument marshalling only).

Each function has the name of the C entry point it forwards to, checks that the tensors
have the dtype, device and contiguity the C ABI expects, allocates missing outputs with
torch (device memory is the only thing torch provides here), and launches on the current
torch stream.  All arithmetic happens in the HIP kernels.
"""
from __future__ import annotations

import math
from typing import Optional

import torch

from ._lib import lib, check, BLOCK_SIZE


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, dtype, name: str):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def kvs_prefill_attn_lse(q, k, v, cu_seqlens, max_seqlen: int, scale: Optional[float] = None, o=None, lse=None,
                         rowmax=None, ell=None, stream=None, skip_lse: bool = False):
    """Causal attention + LSE.  q [T][Hq][d], k/v [T][Hkv][d] bf16; returns (o, lse [Hq][T]).
    skip_lse: the plain attention, writing only o (returns (o, None))."""
    _dev(q, torch.bfloat16, "q"); _dev(k, torch.bfloat16, "k"); _dev(v, torch.bfloat16, "v")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    T, hq, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if o is None else _dev(o, torch.bfloat16, "o")
    if skip_lse:
        lse = None
    else:
        lse = torch.empty(hq, T, device=q.device, dtype=torch.float32) if lse is None else \
            _dev(lse, torch.float32, "lse")
    for name, t in (("rowmax", rowmax), ("ell", ell)):
        if t is not None:
            _dev(t, torch.float32, name)
    check(lib.kvs_prefill_attn_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens.data_ptr(),
                                   cu_seqlens.numel() - 1, T, int(max_seqlen), hq, hkv, d, float(scale),
                                   o.data_ptr(), _ptr(lse), _ptr(rowmax), _ptr(ell), _stream(stream)))
    return o, lse


def kvs_window_score(q, k, lse, cu_seqlens, max_seqlen: int, alpha: int, scale: Optional[float] = None,
                     scores=None, stream=None):
    """Window score S [Hkv][T] from the saved LSE [Hq][T]."""
    _dev(q, torch.bfloat16, "q"); _dev(k, torch.bfloat16, "k"); _dev(lse, torch.float32, "lse")
    _dev(cu_seqlens, torch.int32, "cu_seqlens")
    T, hq, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scores = torch.empty(hkv, T, device=q.device, dtype=torch.float32) if scores is None else \
        _dev(scores, torch.float32, "scores")
    check(lib.kvs_window_score(q.data_ptr(), k.data_ptr(), lse.data_ptr(), cu_seqlens.data_ptr(),
                               cu_seqlens.numel() - 1, T, int(max_seqlen), int(alpha), hq, hkv, d, float(scale),
                               scores.data_ptr(), _stream(stream)))
    return scores


def kvs_topk_select(scores, cu_seqlens, max_seqlen: int, alpha: int, k_budget: int, keep_offsets, keep_idx=None,
                    total_keep: Optional[int] = None, stream=None):
    """Kept indices; keep_offsets [S+1] int32 (device, prefix sums of min(k, n_s)); total_keep = its last value."""
    _dev(scores, torch.float32, "scores"); _dev(cu_seqlens, torch.int32, "cu_seqlens")
    _dev(keep_offsets, torch.int32, "keep_offsets")
    hkv, T = scores.shape
    if keep_idx is None:
        if total_keep is None:
            raise ValueError("total_keep (host value of keep_offsets[-1]) is needed to size keep_idx")
        keep_idx = torch.empty(hkv * int(total_keep), device=scores.device, dtype=torch.int32)
    _dev(keep_idx, torch.int32, "keep_idx")
    check(lib.kvs_topk_select(scores.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1, T, int(max_seqlen),
                              hkv, int(alpha), int(k_budget), keep_offsets.data_ptr(), keep_idx.data_ptr(),
                              _stream(stream)))
    return keep_idx


def kvs_compact_paged(k_src, v_src, cu_seqlens, keep_idx, keep_offsets, max_keep: int, k_pool, v_pool,
                      block_tables, dst_slot_offset=None, stream=None):
    """Write kept rows (keep_idx None = every row) into the pools through the block tables."""
    _dev(k_src, torch.bfloat16, "k_src"); _dev(v_src, torch.bfloat16, "v_src")
    _dev(cu_seqlens, torch.int32, "cu_seqlens"); _dev(block_tables, torch.int32, "block_tables")
    _dev(k_pool, torch.bfloat16, "k_pool"); _dev(v_pool, torch.bfloat16, "v_pool")
    if keep_idx is not None:
        _dev(keep_idx, torch.int32, "keep_idx"); _dev(keep_offsets, torch.int32, "keep_offsets")
    if dst_slot_offset is not None:
        _dev(dst_slot_offset, torch.int32, "dst_slot_offset")
    T, hkv, d = k_src.shape
    check(lib.kvs_compact_paged(k_src.data_ptr(), v_src.data_ptr(), cu_seqlens.data_ptr(), cu_seqlens.numel() - 1,
                                hkv, d, _ptr(keep_idx), _ptr(keep_offsets), int(max_keep), k_pool.data_ptr(),
                                v_pool.data_ptr(), k_pool.shape[0], block_tables.data_ptr(), block_tables.shape[1],
                                _ptr(dst_slot_offset), _stream(stream)))


def kvs_topk_compact(scores, k_src, v_src, cu_seqlens, max_seqlen: int, alpha: int, k_budget: int, keep_offsets,
                     k_pool, v_pool, block_tables, keep_idx=None, total_keep: Optional[int] = None,
                     dst_slot_offset=None, stream=None):
    """kvs_topk_select then kvs_compact_paged of the kept rows, in one launch; returns keep_idx."""
    _dev(scores, torch.float32, "scores"); _dev(cu_seqlens, torch.int32, "cu_seqlens")
    _dev(keep_offsets, torch.int32, "keep_offsets")
    _dev(k_src, torch.bfloat16, "k_src"); _dev(v_src, torch.bfloat16, "v_src")
    _dev(k_pool, torch.bfloat16, "k_pool"); _dev(v_pool, torch.bfloat16, "v_pool")
    _dev(block_tables, torch.int32, "block_tables")
    if dst_slot_offset is not None:
        _dev(dst_slot_offset, torch.int32, "dst_slot_offset")
    hkv, T = scores.shape
    if keep_idx is None:
        if total_keep is None:
            raise ValueError("total_keep (host value of keep_offsets[-1]) is needed to size keep_idx")
        keep_idx = torch.empty(hkv * int(total_keep), device=scores.device, dtype=torch.int32)
    _dev(keep_idx, torch.int32, "keep_idx")
    d = k_src.shape[2]
    check(lib.kvs_topk_compact(scores.data_ptr(), k_src.data_ptr(), v_src.data_ptr(), cu_seqlens.data_ptr(),
                               cu_seqlens.numel() - 1, T, int(max_seqlen), hkv, d, int(alpha), int(k_budget),
                               keep_offsets.data_ptr(), keep_idx.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                               k_pool.shape[0], block_tables.data_ptr(), block_tables.shape[1],
                               _ptr(dst_slot_offset), _stream(stream)))
    return keep_idx


def kvs_paged_decode_workspace_size(batch: int, hq: int, hkv: int, d: int, max_ctx: int) -> int:
    return int(lib.kvs_paged_decode_workspace_size(batch, hq, hkv, d, max_ctx))


def kvs_paged_decode(q, k_pool, v_pool, block_tables, ctx_lens, max_ctx: int, scale: Optional[float] = None,
                     new_k=None, new_v=None, o=None, lse=None, workspace=None, stream=None):
    """One decode step: q [B][Hq][d] over the paged cache (new_k/new_v appended at slot L-1 first)."""
    _dev(q, torch.bfloat16, "q"); _dev(k_pool, torch.bfloat16, "k_pool"); _dev(v_pool, torch.bfloat16, "v_pool")
    _dev(block_tables, torch.int32, "block_tables"); _dev(ctx_lens, torch.int32, "ctx_lens")
    B, hq, d = q.shape
    hkv = k_pool.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if new_k is not None:
        _dev(new_k, torch.bfloat16, "new_k"); _dev(new_v, torch.bfloat16, "new_v")
    o = torch.empty_like(q) if o is None else _dev(o, torch.bfloat16, "o")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    need = kvs_paged_decode_workspace_size(B, hq, hkv, d, int(max_ctx))
    if need and workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib.kvs_paged_decode(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_pool.shape[0],
                               block_tables.data_ptr(), block_tables.shape[1], ctx_lens.data_ptr(), B, int(max_ctx),
                               hq, hkv, d, float(scale), _ptr(new_k), _ptr(new_v), o.data_ptr(), _ptr(lse),
                               _ptr(workspace), ws_bytes, _stream(stream)))
    return o


def kvs_paged_decode_noalloc(q, k_pool, v_pool, block_tables, ctx_lens, max_ctx: int, scale: Optional[float] = None,
                             new_k=None, new_v=None, o=None, lse=None, stream=None):
    """kvs_paged_decode with its split partials in the library's per-device scratch (no workspace)."""
    _dev(q, torch.bfloat16, "q"); _dev(k_pool, torch.bfloat16, "k_pool"); _dev(v_pool, torch.bfloat16, "v_pool")
    _dev(block_tables, torch.int32, "block_tables"); _dev(ctx_lens, torch.int32, "ctx_lens")
    B, hq, d = q.shape
    hkv = k_pool.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if new_k is not None:
        _dev(new_k, torch.bfloat16, "new_k"); _dev(new_v, torch.bfloat16, "new_v")
    o = torch.empty_like(q) if o is None else _dev(o, torch.bfloat16, "o")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    check(lib.kvs_paged_decode_noalloc(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_pool.shape[0],
                                       block_tables.data_ptr(), block_tables.shape[1], ctx_lens.data_ptr(), B,
                                       int(max_ctx), hq, hkv, d, float(scale), _ptr(new_k), _ptr(new_v), o.data_ptr(),
                                       _ptr(lse), _stream(stream)))
    return o


def kvs_slot_init(scores, cu_seqlens, keep_idx, keep_offsets, slot_stride: int, slot_scores=None, slot_pos=None,
                  stream=None):
    """Slot state after compaction: scores/positions [S][Hkv][slot_stride] (keep_idx None: keep all)."""
    _dev(scores, torch.float32, "scores"); _dev(cu_seqlens, torch.int32, "cu_seqlens")
    hkv, T = scores.shape
    S = cu_seqlens.shape[0] - 1
    if keep_idx is not None:
        _dev(keep_idx, torch.int32, "keep_idx"); _dev(keep_offsets, torch.int32, "keep_offsets")
    if slot_scores is None:
        slot_scores = torch.empty(S, hkv, slot_stride, device=scores.device, dtype=torch.float32)
    if slot_pos is None:
        slot_pos = torch.empty(S, hkv, slot_stride, device=scores.device, dtype=torch.int32)
    _dev(slot_scores, torch.float32, "slot_scores"); _dev(slot_pos, torch.int32, "slot_pos")
    check(lib.kvs_slot_init(scores.data_ptr(), _ptr(keep_idx), _ptr(keep_offsets), cu_seqlens.data_ptr(), S, T, hkv,
                            int(slot_stride), slot_scores.data_ptr(), slot_pos.data_ptr(), _stream(stream)))
    return slot_scores, slot_pos


def kvs_decode_select_slot(slot_scores, slot_pos, n_filled, new_pos, cap: int, alpha: int, dst_slot=None,
                           stream=None):
    """Slot of the new token per (sequence, KV head) [B][Hkv] int32 (updates the slot state)."""
    _dev(slot_scores, torch.float32, "slot_scores"); _dev(slot_pos, torch.int32, "slot_pos")
    _dev(n_filled, torch.int32, "n_filled"); _dev(new_pos, torch.int32, "new_pos")
    B, hkv, stride = slot_scores.shape
    if dst_slot is None:
        dst_slot = torch.empty(B, hkv, device=slot_scores.device, dtype=torch.int32)
    _dev(dst_slot, torch.int32, "dst_slot")
    check(lib.kvs_decode_select_slot(slot_scores.data_ptr(), slot_pos.data_ptr(), stride, n_filled.data_ptr(), B, hkv,
                                     int(cap), new_pos.data_ptr(), int(alpha), dst_slot.data_ptr(), _stream(stream)))
    return dst_slot


def kvs_paged_decode_scored_workspace_size(batch: int, hq: int, hkv: int, d: int, max_ctx: int) -> int:
    return int(lib.kvs_paged_decode_scored_workspace_size(batch, hq, hkv, d, max_ctx))


def kvs_paged_decode_scored(q, k_pool, v_pool, block_tables, ctx_lens, max_ctx: int, slot_scores, new_k=None,
                            new_v=None, dst_slots=None, scale: Optional[float] = None, o=None, lse=None,
                            workspace=None, stream=None):
    """Decode step writing the new token to dst_slots (per head) and adding its probabilities to slot_scores."""
    _dev(q, torch.bfloat16, "q"); _dev(k_pool, torch.bfloat16, "k_pool"); _dev(v_pool, torch.bfloat16, "v_pool")
    _dev(block_tables, torch.int32, "block_tables"); _dev(ctx_lens, torch.int32, "ctx_lens")
    _dev(slot_scores, torch.float32, "slot_scores")
    B, hq, d = q.shape
    hkv = k_pool.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if new_k is not None:
        _dev(new_k, torch.bfloat16, "new_k"); _dev(new_v, torch.bfloat16, "new_v")
    if dst_slots is not None:
        _dev(dst_slots, torch.int32, "dst_slots")
    o = torch.empty_like(q) if o is None else _dev(o, torch.bfloat16, "o")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    need = kvs_paged_decode_scored_workspace_size(B, hq, hkv, d, int(max_ctx))
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size()
    check(lib.kvs_paged_decode_scored(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_pool.shape[0],
                                      block_tables.data_ptr(), block_tables.shape[1], ctx_lens.data_ptr(), B,
                                      int(max_ctx), hq, hkv, d, float(scale), _ptr(new_k), _ptr(new_v),
                                      _ptr(dst_slots), slot_scores.data_ptr(), slot_scores.shape[2], o.data_ptr(),
                                      _ptr(lse), workspace.data_ptr(), ws_bytes, _stream(stream)))
    return o


def kvs_copy_blocks(k_pool, v_pool, src_dst_pairs, stream=None):
    """Copy whole blocks (both pools): src_dst_pairs [n][2] int32 device."""
    _dev(k_pool, torch.bfloat16, "k_pool"); _dev(v_pool, torch.bfloat16, "v_pool")
    _dev(src_dst_pairs, torch.int32, "src_dst_pairs")
    nb, hkv = k_pool.shape[0], k_pool.shape[1]
    d = k_pool.shape[3]
    check(lib.kvs_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(), nb, hkv, d, src_dst_pairs.data_ptr(),
                              src_dst_pairs.shape[0], _stream(stream)))


def new_pools(num_blocks: int, hkv: int, d: int, device="cuda"):
    """Empty K [num_blocks][hkv][16][d] and V [num_blocks][hkv][d][16] bf16 pools."""
    k_pool = torch.empty(num_blocks, hkv, BLOCK_SIZE, d, device=device, dtype=torch.bfloat16)
    v_pool = torch.empty(num_blocks, hkv, d, BLOCK_SIZE, device=device, dtype=torch.bfloat16)
    return k_pool, v_pool


# ---- 8-bit (E4M3) cache: uint8 code pools plus one fp32 scale per (block, head, slot)
def new_pools_fp8(num_blocks: int, hkv: int, d: int, device="cuda"):
    """Empty K codes [num_blocks][hkv][16][d], V codes [num_blocks][hkv][d][16] (uint8) and the
    K and V scales [num_blocks][hkv][16] (fp32)."""
    k_pool = torch.empty(num_blocks, hkv, BLOCK_SIZE, d, device=device, dtype=torch.uint8)
    v_pool = torch.empty(num_blocks, hkv, d, BLOCK_SIZE, device=device, dtype=torch.uint8)
    k_scale = torch.empty(num_blocks, hkv, BLOCK_SIZE, device=device, dtype=torch.float32)
    v_scale = torch.empty(num_blocks, hkv, BLOCK_SIZE, device=device, dtype=torch.float32)
    return k_pool, v_pool, k_scale, v_scale


def _check_fp8_pools(k_pool, v_pool, k_scale, v_scale):
    _dev(k_pool, torch.uint8, "k_pool"); _dev(v_pool, torch.uint8, "v_pool")
    _dev(k_scale, torch.float32, "k_scale"); _dev(v_scale, torch.float32, "v_scale")
    nb, hkv, bs, d = k_pool.shape
    if (tuple(v_pool.shape) != (nb, hkv, d, bs) or tuple(k_scale.shape) != (nb, hkv, bs)
            or tuple(v_scale.shape) != (nb, hkv, bs)):
        raise ValueError("8-bit pools: K [nb][hkv][16][d], V [nb][hkv][d][16], scales [nb][hkv][16]")
    return nb, hkv, d


def kvs_compact_paged_fp8(k_src, v_src, cu_seqlens, keep_idx, keep_offsets, max_keep: int, k_pool, v_pool, k_scale,
                          v_scale, block_tables, dst_slot_offset=None, stream=None):
    """kvs_compact_paged into an 8-bit cache (rows quantized with one scale each)."""
    _dev(k_src, torch.bfloat16, "k_src"); _dev(v_src, torch.bfloat16, "v_src")
    _dev(cu_seqlens, torch.int32, "cu_seqlens"); _dev(block_tables, torch.int32, "block_tables")
    nb, _, _ = _check_fp8_pools(k_pool, v_pool, k_scale, v_scale)
    if keep_idx is not None:
        _dev(keep_idx, torch.int32, "keep_idx"); _dev(keep_offsets, torch.int32, "keep_offsets")
    if dst_slot_offset is not None:
        _dev(dst_slot_offset, torch.int32, "dst_slot_offset")
    T, hkv, d = k_src.shape
    check(lib.kvs_compact_paged_fp8(k_src.data_ptr(), v_src.data_ptr(), cu_seqlens.data_ptr(),
                                    cu_seqlens.numel() - 1, hkv, d, _ptr(keep_idx), _ptr(keep_offsets),
                                    int(max_keep), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
                                    v_scale.data_ptr(), nb, block_tables.data_ptr(), block_tables.shape[1],
                                    _ptr(dst_slot_offset), _stream(stream)))


def kvs_paged_decode_fp8(q, k_pool, v_pool, k_scale, v_scale, block_tables, ctx_lens, max_ctx: int,
                         scale: Optional[float] = None, new_k=None, new_v=None, o=None, lse=None, workspace=None,
                         stream=None):
    """kvs_paged_decode over an 8-bit cache; new_k/new_v (bf16) are quantized into slot L-1."""
    _dev(q, torch.bfloat16, "q")
    nb, hkv, _ = _check_fp8_pools(k_pool, v_pool, k_scale, v_scale)
    _dev(block_tables, torch.int32, "block_tables"); _dev(ctx_lens, torch.int32, "ctx_lens")
    B, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if new_k is not None:
        _dev(new_k, torch.bfloat16, "new_k"); _dev(new_v, torch.bfloat16, "new_v")
    o = torch.empty_like(q) if o is None else _dev(o, torch.bfloat16, "o")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    need = kvs_paged_decode_workspace_size(B, hq, hkv, d, int(max_ctx))
    if need and workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    check(lib.kvs_paged_decode_fp8(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
                                   v_scale.data_ptr(), nb, block_tables.data_ptr(), block_tables.shape[1],
                                   ctx_lens.data_ptr(), B, int(max_ctx), hq, hkv, d, float(scale), _ptr(new_k),
                                   _ptr(new_v), o.data_ptr(), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))
    return o


def kvs_copy_blocks_fp8(k_pool, v_pool, k_scale, v_scale, src_dst_pairs, stream=None):
    """Copy whole blocks of an 8-bit cache (codes and scales): src_dst_pairs [n][2] int32 device."""
    nb, hkv, d = _check_fp8_pools(k_pool, v_pool, k_scale, v_scale)
    _dev(src_dst_pairs, torch.int32, "src_dst_pairs")
    check(lib.kvs_copy_blocks_fp8(k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), nb,
                                  hkv, d, src_dst_pairs.data_ptr(), src_dst_pairs.shape[0], _stream(stream)))


# ---- chunked prefill and prefix reuse
def kvs_prefill_attn_lse_chunk(q, k, v, cu_seqlens_q, cu_seqlens_k, max_q: int, max_k: int,
                               scale: Optional[float] = None, o=None, lse=None, rowmax=None, ell=None, stream=None):
    """Causal attention of chunks: q [Tq][Hq][d] holds each prompt's last m_s rows, k/v [Tk][Hkv][d]
    all n_s tokens; returns (o [Tq][Hq][d], lse [Hq][Tq])."""
    _dev(q, torch.bfloat16, "q"); _dev(k, torch.bfloat16, "k"); _dev(v, torch.bfloat16, "v")
    _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q"); _dev(cu_seqlens_k, torch.int32, "cu_seqlens_k")
    Tq, hq, d = q.shape
    hkv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q) if o is None else _dev(o, torch.bfloat16, "o")
    lse = torch.empty(hq, Tq, device=q.device, dtype=torch.float32) if lse is None else _dev(lse, torch.float32, "lse")
    for name, t in (("rowmax", rowmax), ("ell", ell)):
        if t is not None:
            _dev(t, torch.float32, name)
    check(lib.kvs_prefill_attn_lse_chunk(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                                         cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1, Tq, int(max_q),
                                         int(max_k), hq, hkv, d, float(scale), o.data_ptr(), lse.data_ptr(),
                                         _ptr(rowmax), _ptr(ell), _stream(stream)))
    return o, lse


def kvs_window_score_chunk(q, k, lse, cu_seqlens_q, cu_seqlens_k, max_k: int, alpha: int,
                           scale: Optional[float] = None, scores=None, stream=None):
    """Window score S [Hkv][Tk] when q/lse hold only each prompt's last rows (the window inside them)."""
    _dev(q, torch.bfloat16, "q"); _dev(k, torch.bfloat16, "k"); _dev(lse, torch.float32, "lse")
    _dev(cu_seqlens_q, torch.int32, "cu_seqlens_q"); _dev(cu_seqlens_k, torch.int32, "cu_seqlens_k")
    Tq, hq, d = q.shape
    Tk, hkv = k.shape[0], k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    scores = torch.empty(hkv, Tk, device=q.device, dtype=torch.float32) if scores is None else \
        _dev(scores, torch.float32, "scores")
    check(lib.kvs_window_score_chunk(q.data_ptr(), k.data_ptr(), lse.data_ptr(), cu_seqlens_q.data_ptr(),
                                     cu_seqlens_k.data_ptr(), cu_seqlens_q.numel() - 1, Tq, Tk, int(max_k),
                                     int(alpha), hq, hkv, d, float(scale), scores.data_ptr(), _stream(stream)))
    return scores


def kvs_gather_paged(k_pool, v_pool, block_tables, counts, dst_start, max_count: int, k_dst, v_dst, stream=None):
    """Read tokens 0..counts[s]-1 of each sequence back from the pools into rows dst_start[s]+t."""
    _dev(k_pool, torch.bfloat16, "k_pool"); _dev(v_pool, torch.bfloat16, "v_pool")
    _dev(block_tables, torch.int32, "block_tables"); _dev(counts, torch.int32, "counts")
    _dev(dst_start, torch.int32, "dst_start")
    _dev(k_dst, torch.bfloat16, "k_dst"); _dev(v_dst, torch.bfloat16, "v_dst")
    nb, hkv, _, d = k_pool.shape
    check(lib.kvs_gather_paged(k_pool.data_ptr(), v_pool.data_ptr(), nb, block_tables.data_ptr(),
                               block_tables.shape[1], counts.numel(), hkv, d, counts.data_ptr(), dst_start.data_ptr(),
                               int(max_count), k_dst.data_ptr(), v_dst.data_ptr(), _stream(stream)))


def kvs_paged_decode_scored_fp8(q, k_pool, v_pool, k_scale, v_scale, block_tables, ctx_lens, max_ctx: int,
                                slot_scores, new_k=None, new_v=None, dst_slots=None, scale: Optional[float] = None,
                                o=None, lse=None, workspace=None, stream=None):
    """kvs_paged_decode_scored over an 8-bit cache (the new token quantized into its slot)."""
    _dev(q, torch.bfloat16, "q")
    nb, hkv, _ = _check_fp8_pools(k_pool, v_pool, k_scale, v_scale)
    _dev(block_tables, torch.int32, "block_tables"); _dev(ctx_lens, torch.int32, "ctx_lens")
    _dev(slot_scores, torch.float32, "slot_scores")
    B, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if new_k is not None:
        _dev(new_k, torch.bfloat16, "new_k"); _dev(new_v, torch.bfloat16, "new_v")
    if dst_slots is not None:
        _dev(dst_slots, torch.int32, "dst_slots")
    o = torch.empty_like(q) if o is None else _dev(o, torch.bfloat16, "o")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    need = kvs_paged_decode_scored_workspace_size(B, hq, hkv, d, int(max_ctx))
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size()
    check(lib.kvs_paged_decode_scored_fp8(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_scale.data_ptr(),
                                          v_scale.data_ptr(), nb, block_tables.data_ptr(), block_tables.shape[1],
                                          ctx_lens.data_ptr(), B, int(max_ctx), hq, hkv, d, float(scale), _ptr(new_k),
                                          _ptr(new_v), _ptr(dst_slots), slot_scores.data_ptr(), slot_scores.shape[2],
                                          o.data_ptr(), _ptr(lse), workspace.data_ptr(), ws_bytes, _stream(stream)))
    return o


def _select_args(slot_scores, slot_pos, next_pos, next_dst_slots):
    _dev(slot_pos, torch.int32, "slot_pos"); _dev(next_pos, torch.int32, "next_pos")
    if slot_pos.shape != slot_scores.shape:
        raise ValueError("slot_pos must have slot_scores' shape [B][Hkv][stride]")
    B, hkv, _ = slot_scores.shape
    if next_dst_slots is None:
        next_dst_slots = torch.empty(B, hkv, device=slot_scores.device, dtype=torch.int32)
    return _dev(next_dst_slots, torch.int32, "next_dst_slots")


def kvs_paged_decode_scored_select(q, k_pool, v_pool, block_tables, ctx_lens, max_ctx: int, slot_scores, slot_pos,
                                   cap: int, alpha: int, next_pos, next_dst_slots=None, new_k=None, new_v=None,
                                   dst_slots=None, scale: Optional[float] = None, o=None, lse=None, workspace=None,
                                   stream=None):
    """kvs_paged_decode_scored, then the next step's slot choice in the same launches.
    Returns (o, next_dst_slots)."""
    _dev(q, torch.bfloat16, "q"); _dev(k_pool, torch.bfloat16, "k_pool"); _dev(v_pool, torch.bfloat16, "v_pool")
    _dev(block_tables, torch.int32, "block_tables"); _dev(ctx_lens, torch.int32, "ctx_lens")
    _dev(slot_scores, torch.float32, "slot_scores")
    nxt = _select_args(slot_scores, slot_pos, next_pos, next_dst_slots)
    B, hq, d = q.shape
    hkv = k_pool.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if new_k is not None:
        _dev(new_k, torch.bfloat16, "new_k"); _dev(new_v, torch.bfloat16, "new_v")
    if dst_slots is not None:
        _dev(dst_slots, torch.int32, "dst_slots")
    o = torch.empty_like(q) if o is None else _dev(o, torch.bfloat16, "o")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    need = kvs_paged_decode_scored_workspace_size(B, hq, hkv, d, int(max_ctx))
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size()
    check(lib.kvs_paged_decode_scored_select(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), k_pool.shape[0],
                                             block_tables.data_ptr(), block_tables.shape[1], ctx_lens.data_ptr(), B,
                                             int(max_ctx), hq, hkv, d, float(scale), _ptr(new_k), _ptr(new_v),
                                             _ptr(dst_slots), slot_scores.data_ptr(), slot_pos.data_ptr(),
                                             slot_scores.shape[2], int(cap), int(alpha), next_pos.data_ptr(),
                                             nxt.data_ptr(), o.data_ptr(), _ptr(lse), workspace.data_ptr(), ws_bytes,
                                             _stream(stream)))
    return o, nxt


def kvs_paged_decode_scored_select_fp8(q, k_pool, v_pool, k_scale, v_scale, block_tables, ctx_lens, max_ctx: int,
                                       slot_scores, slot_pos, cap: int, alpha: int, next_pos, next_dst_slots=None,
                                       new_k=None, new_v=None, dst_slots=None, scale: Optional[float] = None, o=None,
                                       lse=None, workspace=None, stream=None):
    """kvs_paged_decode_scored_select over an 8-bit cache.  Returns (o, next_dst_slots)."""
    _dev(q, torch.bfloat16, "q")
    nb, hkv, _ = _check_fp8_pools(k_pool, v_pool, k_scale, v_scale)
    _dev(block_tables, torch.int32, "block_tables"); _dev(ctx_lens, torch.int32, "ctx_lens")
    _dev(slot_scores, torch.float32, "slot_scores")
    nxt = _select_args(slot_scores, slot_pos, next_pos, next_dst_slots)
    B, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if new_k is not None:
        _dev(new_k, torch.bfloat16, "new_k"); _dev(new_v, torch.bfloat16, "new_v")
    if dst_slots is not None:
        _dev(dst_slots, torch.int32, "dst_slots")
    o = torch.empty_like(q) if o is None else _dev(o, torch.bfloat16, "o")
    if lse is not None:
        _dev(lse, torch.float32, "lse")
    need = kvs_paged_decode_scored_workspace_size(B, hq, hkv, d, int(max_ctx))
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    ws_bytes = workspace.numel() * workspace.element_size()
    check(lib.kvs_paged_decode_scored_select_fp8(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                                 k_scale.data_ptr(), v_scale.data_ptr(), nb, block_tables.data_ptr(),
                                                 block_tables.shape[1], ctx_lens.data_ptr(), B, int(max_ctx), hq, hkv,
                                                 d, float(scale), _ptr(new_k), _ptr(new_v), _ptr(dst_slots),
                                                 slot_scores.data_ptr(), slot_pos.data_ptr(), slot_scores.shape[2],
                                                 int(cap), int(alpha), next_pos.data_ptr(), nxt.data_ptr(),
                                                 o.data_ptr(), _ptr(lse), workspace.data_ptr(), ws_bytes,
                                                 _stream(stream)))
    return o, nxt


# ---- measurement helper
def kvs_probe_stream_read(buf, grid: int, sink=None, key: int = 0x9E3779B9, stream=None):
    """Read every byte of the contiguous device tensor buf once (the streaming-read ceiling probe)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf: contiguous device tensor expected")
    if sink is None:
        sink = torch.empty(grid, dtype=torch.int32, device=buf.device)
    check(lib.kvs_probe_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), int(grid), int(key),
                                    sink.data_ptr(), _stream(stream)))
    return sink


def kvs_probe_timestamp(out, stream=None):
    """Store the GPU's 100 MHz real-time counter into out (a device int64 tensor, element 0)
    when the launch runs."""
    if not out.is_cuda or out.dtype != torch.int64 or out.numel() < 1:
        raise ValueError("out: device int64 tensor expected")
    check(lib.kvs_probe_timestamp(out.data_ptr(), _stream(stream)))
    return out
