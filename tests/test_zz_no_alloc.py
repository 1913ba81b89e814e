"""kvs_paged_decode_noalloc (the decode for callers that cannot allocate: its split partials
live in a scratch array the library holds per device) against kvs_paged_decode with a
caller-owned workspace, through the C ABI: outputs, LSE and the appended rows bit-identical,
over calls in a row that each use the scratch, each smaller than the one before (the scratch
keeps the previous call's partials), and a shape beyond the scratch rejected on the host."""
import sys

import numpy as np
import pytest
import torch

from tests._parity import i32

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


def _setup(lengths, seed, hq=32, hkv=8, d=128):
    """Pools filled with seeded N(0,1) bf16, scattered tables with room for one appended token."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(seed)
    nbs = [-(-L // 16) for L in lengths]
    nb_total = sum(nbs) + 3
    k_pool, v_pool = kvs.new_pools(nb_total, hkv, d)
    k_pool.copy_(torch.randn(k_pool.shape, generator=gen, device=dev).to(torch.bfloat16))
    v_pool.copy_(torch.randn(v_pool.shape, generator=gen, device=dev).to(torch.bfloat16))
    perm = np.random.default_rng(seed).permutation(nb_total).astype(np.int32)
    tbl = np.full((len(lengths), max(nbs)), -1, np.int32)
    at = 0
    for i, nb in enumerate(nbs):
        tbl[i, :nb] = perm[at:at + nb]
        at += nb
    B = len(lengths)
    q = torch.randn(B, hq, d, generator=gen, device=dev).to(torch.bfloat16)
    nk = torch.randn(B, hkv, d, generator=gen, device=dev).to(torch.bfloat16)
    nv = torch.randn(B, hkv, d, generator=gen, device=dev).to(torch.bfloat16)
    return k_pool, v_pool, i32(tbl), i32(lengths), q, nk, nv


def _same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int32 if a.dtype == torch.float32 else torch.int16),
                       b.contiguous().view(torch.int32 if b.dtype == torch.float32 else torch.int16))


@pytest.mark.parametrize("calls", [
    [[3100, 3000, 3050, 3099], [900], [300]],
    [[450, 700], [900], [301]],
])
def test_noalloc_decode_matches_the_workspace_decode(calls):
    for i, lengths in enumerate(calls):
        B, hq, hkv, d = len(lengths), 32, 8, 128
        max_ctx = max(lengths)
        need = kvs.kvs_paged_decode_workspace_size(B, hq, hkv, d, max_ctx)
        assert need > 0, "each call must use the split partials"
        _say(f"no-alloc decode call {i}: contexts {lengths}, {need} bytes of partials")
        k_pool, v_pool, tbl, ctx, q, nk, nv = _setup(lengths, seed=17 + 31 * i + B)
        k2, v2 = k_pool.clone(), v_pool.clone()
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        lse1 = torch.empty(B, hq, device="cuda", dtype=torch.float32)
        lse2 = torch.empty_like(lse1)
        o1 = kvs.kvs_paged_decode(q, k_pool, v_pool, tbl, ctx, max_ctx, new_k=nk, new_v=nv, lse=lse1, workspace=ws)
        o2 = kvs.kvs_paged_decode_noalloc(q, k2, v2, tbl, ctx, max_ctx, new_k=nk, new_v=nv, lse=lse2)
        torch.cuda.synchronize()
        assert _same_bits(o1, o2), f"output differs on call {i}"
        assert _same_bits(lse1, lse2), f"LSE differs on call {i}"
        assert _same_bits(k_pool, k2) and _same_bits(v_pool, v2), f"appended rows differ on call {i}"
        assert torch.isfinite(o1.float()).all() and torch.isfinite(lse1).all()


def test_noalloc_rejects_shapes_beyond_the_scratch():
    # 9 sequences of 16000 tokens: 125 pieces of 8 blocks per (sequence, head), 17.9 MiB of partials
    B, hq, hkv, d, max_ctx = 9, 32, 8, 128, 16000
    assert kvs.kvs_paged_decode_workspace_size(B, hq, hkv, d, max_ctx) > 16 << 20
    fake = 0x1000    # never dereferenced: the size check comes first
    rc = kvs.lib.kvs_paged_decode_noalloc(fake, fake, fake, 10000, fake, 1000, fake, B, max_ctx, hq, hkv, d, 0.1,
                                          None, None, fake, None, None)
    assert rc == kvs._lib.KVS_E_INVAL
    assert b"scratch" in kvs.lib.kvs_last_error()
