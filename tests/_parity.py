"""Comparison rules between the HIP path and the fp64 oracle (test infrastructure).

Tolerances (bf16 inputs, fp32 accumulation on the GPU):
  attention / decode outputs  per (row, head): max_c |o - r| <= 1e-2 * max_c |r|
  LSE                         |delta| <= 1e-3 (absolute, natural log)
  window score S              per KV head, |delta S_i| <= 1e-3 * |S_i| for every token with
                              S_i >= 1e-6 * max_i S_i; below that threshold (scores far under the
                              fp32 exponential's useful range) |delta S_i| <= 1e-3 * threshold
  kept index sets             equal, except that a GPU-only index and an oracle-only index may swap
                              when both oracle scores lie within 1e-4 (relative) of the oracle's
                              boundary score (the (k_eff - alpha)-th largest candidate score)
  block contents              bit-exact against the GPU's own kept set
"""
from __future__ import annotations

import numpy as np
import torch

from workloads import bf16_bits_to_f64

O_TOL = 1e-2
LSE_TOL = 1e-3
S_REL = 1e-3
SWAP_REL = 1e-4


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return bf16_bits_to_f64(t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def i32(x, device="cuda") -> torch.Tensor:
    return torch.as_tensor(np.asarray(x, dtype=np.int32)).to(device)


def assert_rows_close(got: np.ndarray, ref: np.ndarray, tol: float = O_TOL, what: str = "O"):
    """got/ref [..., d]: per leading index, max |got - ref| <= tol * max |ref|."""
    err = np.abs(got - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    bad = err > tol * scale
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} rows out of tolerance, e.g. {idx.tolist()} "
                             f"err={err[bad][:5]} scale={scale[bad][:5]}")


def assert_lse_close(got, ref, tol: float = LSE_TOL, what: str = "LSE"):
    d = np.abs(np.asarray(got, dtype=np.float64) - ref)
    if not (d <= tol).all():
        raise AssertionError(f"{what}: max |delta| {d.max():.3e} > {tol}")


S_FLOOR = 1e-6


def assert_scores_close(got, ref, what: str = "S") -> int:
    """got/ref [Hkv][n] (or [n]): 1e-3 relative per token above 1e-6 of the head's largest score,
    absolute 1e-3 * that threshold below it.  Returns how many tokens took the absolute branch."""
    got = np.atleast_2d(np.asarray(got, dtype=np.float64))
    ref = np.atleast_2d(np.asarray(ref, dtype=np.float64))
    thr = S_FLOOR * np.abs(ref).max(axis=-1, keepdims=True)
    small = np.abs(ref) < thr
    bound = np.where(small, S_REL * thr, S_REL * np.abs(ref))
    d = np.abs(got - ref)
    if not (d <= bound).all():
        i = np.unravel_index(np.argmax(d / np.maximum(bound, 1e-300)), d.shape)
        raise AssertionError(f"{what}: worst at {i}: got {got[i]:.6e} ref {ref[i]:.6e} "
                             f"({int(small.sum())} of {small.size} tokens under the threshold)")
    return int(small.sum())


def assert_keep_matches(keep_gpu: np.ndarray, keep_ref: np.ndarray, S_ref: np.ndarray, n: int, alpha: int,
                        k_budget: int, what: str = "keep"):
    """One KV head: kept sets equal up to legal boundary swaps (see module docstring)."""
    a, b = set(int(x) for x in keep_gpu), set(int(x) for x in keep_ref)
    assert len(keep_gpu) == len(keep_ref) == len(a), f"{what}: sizes {len(keep_gpu)} vs {len(keep_ref)}"
    assert np.all(np.diff(keep_gpu) > 0), f"{what}: GPU indices not ascending"
    if a == b:
        return
    only_gpu, only_ref = sorted(a - b), sorted(b - a)
    assert len(only_gpu) == len(only_ref)
    a_eff = min(alpha, n)
    cand = np.sort(S_ref[: n - a_eff])[::-1]
    kth = cand[k_budget - a_eff - 1]
    for i in only_gpu + only_ref:
        assert i < n - a_eff, f"{what}: window token {i} differs"
        assert abs(S_ref[i] - kth) <= SWAP_REL * abs(kth), \
            f"{what}: index {i} (S={S_ref[i]:.9e}) differs but is not at the boundary {kth:.9e}"


def gather_pools(k_pool: torch.Tensor, v_pool: torch.Tensor, table, length: int):
    """Read a sequence back from the GPU pools: logical [length][Hkv][d] bit patterns of K and V.

    K pool is [blocks][Hkv][16][d]; V pool is [blocks][Hkv][d][16] (channel-major per block).
    """
    idx = torch.as_tensor(list(table), dtype=torch.long, device=k_pool.device)
    kb = k_pool.index_select(0, idx)                         # [nb][Hkv][16][d]
    vb = v_pool.index_select(0, idx).transpose(2, 3)         # [nb][Hkv][16][d]
    nb, hkv, bs, d = kb.shape
    kk = kb.permute(0, 2, 1, 3).reshape(nb * bs, hkv, d)[:length]
    vv = vb.permute(0, 2, 1, 3).reshape(nb * bs, hkv, d)[:length]
    return bf16_bits(kk), bf16_bits(vv)
