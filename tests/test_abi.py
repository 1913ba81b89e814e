"""CPU checks of the C ABI: every declared symbol is exported, host-side argument checks
fail before any launch, and the native allocator matches the oracle's allocator op for op."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from oracle.paged import NoBlocksError, RefcountError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvs.h")

kvs = pytest.importorskip("kv_cache_sparsification_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvs_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 18
    lib = ctypes.CDLL(kvs.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # and the binding declares a signature for each
    from kv_cache_sparsification_amd._lib import SIGNATURES
    assert sorted(SIGNATURES) == names


def test_version():
    assert b"gfx950" in kvs.lib.kvs_version()


def test_host_validation_rejects_before_launch():
    L = kvs.lib
    fake = 0x1000   # never dereferenced: the checks fail first
    rc = L.kvs_prefill_attn_lse(fake, fake, fake, fake, 1, 10, 10, 8, 3, 128, 0.1, fake, fake, None, None, None)
    assert rc == kvs._lib.KVS_E_INVAL and b"bad shape" in L.kvs_last_error()
    assert L.kvs_prefill_attn_lse(fake, fake, fake, fake, 1, 10, 10, 8, 2, 96, 0.1, fake, fake, None, None, None) == -1
    assert L.kvs_window_score(fake, fake, fake, fake, 1, 10, 10, 0, 8, 2, 128, 0.1, fake, None) == -1
    assert L.kvs_topk_select(fake, fake, 1, 10, 10, 2, 8, 4, fake, fake, None) == -1      # k < alpha
    assert b"alpha" in L.kvs_last_error()
    assert L.kvs_compact_paged(fake, fake, fake, 1, 2, 100, None, None, 8, fake, fake, 4, fake, 4, None, None) == -1
    # fused selection and compaction: k < alpha, a bad head size, a NULL pool
    tc = dict(scores=fake, k_src=fake, v_src=fake, cu=fake, num_seqs=1, total=10, max_seqlen=10, hkv=2, d=128,
              alpha=8, k=16, koff=fake, keep=fake, kp=fake, vp=fake, nb=4, tbl=fake, max_blocks=4, dst=None,
              stream=None)
    assert L.kvs_topk_compact(*dict(tc, k=4).values()) == -1 and b"alpha" in L.kvs_last_error()
    assert L.kvs_topk_compact(*dict(tc, d=96).values()) == -1 and b"bad shape" in L.kvs_last_error()
    assert L.kvs_topk_compact(*dict(tc, kp=None).values()) == -1 and b"NULL" in L.kvs_last_error()
    assert L.kvs_topk_compact(*dict(tc, num_seqs=0, total=0).values()) == 0     # nothing to do
    assert L.kvs_copy_blocks(fake, fake, 4, 2, 128, None, 3, None) == -1
    ws = L.kvs_paged_decode_workspace_size(1, 32, 8, 128, 30000)
    assert ws > 0
    assert L.kvs_paged_decode(fake, fake, fake, 64, fake, 2000, fake, 1, 30000, 32, 8, 128, 0.1, None, None, fake,
                              None, fake, ws - 1, None) == -1
    assert b"workspace" in L.kvs_last_error()
    assert L.kvs_paged_decode(fake, fake, fake, 64, fake, 10, fake, 1, 4000, 32, 8, 128, 0.1, None, None, fake,
                              None, None, 0, None) == -1                                       # 10 blocks < 4000 tokens
    # empty work is a no-op that launches nothing
    assert L.kvs_prefill_attn_lse(fake, fake, fake, fake, 0, 0, 0, 8, 2, 128, 0.1, fake, fake, None, None, None) == 0
    assert L.kvs_copy_blocks(fake, fake, 4, 2, 128, fake, 0, None) == 0
    # the read probe: sizes and alignment are checked on the host
    assert L.kvs_probe_stream_read(fake, 100, 64, 0, fake, None) == -1          # not a multiple of 16
    assert L.kvs_probe_stream_read(fake + 8, 1024, 64, 0, fake, None) == -1     # misaligned
    assert L.kvs_probe_stream_read(fake, 1024, 0, 0, fake, None) == -1          # empty grid
    assert L.kvs_probe_stream_read(None, 1024, 64, 0, fake, None) == -1
    # the scored decode that also chooses the next step's slot: its extra arguments
    args = lambda nxt, slot_pos, cap, alpha, max_ctx: (fake, fake, fake, 64, fake, 8, fake, 1, max_ctx, 32, 8, 128, 0.1,
                                                       fake, fake, fake, fake, slot_pos, 128, cap, alpha, fake, nxt,
                                                       fake, None, fake, 1 << 20, None)
    assert L.kvs_paged_decode_scored_select(*args(None, fake, 128, 32, 128)) == -1     # no next_dst_slots
    assert L.kvs_paged_decode_scored_select(*args(fake, None, 128, 32, 128)) == -1     # no slot_pos
    assert L.kvs_paged_decode_scored_select(*args(fake, fake, 128, 128, 128)) == -1    # alpha >= cap
    assert L.kvs_paged_decode_scored_select(*args(fake, fake, 100, 32, 128)) == -1     # max_ctx > cap
    assert L.kvs_paged_decode_scored_select(*args(fake, fake, 256, 32, 128)) == -1     # cap > slot_stride
    # the clock stamp: its output pointer is checked on the host
    assert L.kvs_probe_timestamp(None, None) == -1
    assert L.kvs_probe_timestamp(fake + 4, None) == -1                          # not 8-byte aligned


def test_workspace_size_policy():
    L = kvs.lib
    # a batch that fills the chip, or one round of blocks, needs no split; a single sequence does
    assert L.kvs_paged_decode_workspace_size(64, 32, 8, 128, 4000) == 0
    assert L.kvs_paged_decode_workspace_size(1, 32, 8, 128, 100) == 0
    assert L.kvs_paged_decode_workspace_size(1, 32, 8, 128, 900) > 0
    assert L.kvs_paged_decode_workspace_size(1, 32, 8, 128, 30000) > 0
    assert L.kvs_paged_decode_workspace_size(0, 32, 8, 128, 900) == 0


def test_allocator_worked_example():
    a = kvs.BlockAllocator(64, [41, 7, 19, 2, 33])
    assert a.alloc_n(3) == [41, 7, 19]
    assert a.free_list() == [2, 33]
    assert a.refcount(5) == 1 and a.refcount(2) == 0     # unlisted blocks start in use


def test_allocator_errors():
    a = kvs.BlockAllocator(2)
    b0, b1 = a.alloc(), a.alloc()
    with pytest.raises(kvs.KvsError) as e:
        a.alloc()
    assert e.value.code == -2
    a.decref(b0)
    with pytest.raises(kvs.KvsError) as e:
        a.decref(b0)
    assert e.value.code == -3
    with pytest.raises(kvs.KvsError):
        a.incref(b0)
    with pytest.raises(kvs.KvsError):
        a.refcount(7)
    with pytest.raises(kvs.KvsError):
        kvs.BlockAllocator(4, [1, 1])


@pytest.mark.parametrize("seed", range(12))
def test_allocator_matches_oracle_on_random_ops(seed):
    r = np.random.default_rng(seed)
    N = int(r.integers(4, 40))
    order = list(r.permutation(N)[: int(r.integers(1, N + 1))])
    ref = oracle.BlockAllocator(N, initial_free_order=order)
    nat = kvs.BlockAllocator(N, order)
    live = [b for b in range(N) if b not in set(order)]
    for _ in range(800):
        op = int(r.integers(0, 5))
        try:
            if op == 0:
                try:
                    b = ref.alloc()
                except NoBlocksError:
                    with pytest.raises(kvs.KvsError):
                        nat.alloc()
                    continue
                assert nat.alloc() == b
                live.append(b)
            elif live:
                b = live[int(r.integers(len(live)))]
                if op == 1:
                    ref.incref(b); nat.incref(b); live.append(b)
                elif op == 2:
                    ref.decref(b); nat.decref(b); live.remove(b)
                elif op == 3:
                    try:
                        nb, c = ref.cow(b)
                    except NoBlocksError:
                        with pytest.raises(kvs.KvsError):
                            nat.cow(b)
                        continue
                    assert nat.cow(b) == (nb, c)
                    if c:
                        live.remove(b); live.append(nb)
                else:
                    assert nat.refcount(b) == ref.ref[b]
        except RefcountError:
            raise
        assert nat.free_list() == list(ref.free)
        assert nat.num_free() == len(ref.free)
    for b in range(N):
        assert nat.refcount(b) == ref.ref[b]


def test_eviction_calls_validate_on_the_host():
    L = kvs.lib
    fake = 0x1000   # never dereferenced: the checks fail first
    # alpha must leave a replaceable slot, and cap must fit the slot rows
    assert L.kvs_decode_select_slot(fake, fake, 64, fake, 1, 2, 64, fake, 64, fake, None) == -1
    assert b"alpha" in L.kvs_last_error()
    assert L.kvs_decode_select_slot(fake, fake, 32, fake, 1, 2, 64, fake, 16, fake, None) == -1
    assert L.kvs_decode_select_slot(fake, fake, 64, fake, 0, 2, 64, fake, 16, fake, None) == 0    # empty batch
    assert L.kvs_slot_init(fake, fake, None, fake, 1, 10, 2, 64, fake, fake, None) == -1           # no offsets
    assert L.kvs_slot_init(fake, None, None, fake, 0, 0, 2, 64, fake, fake, None) == 0
    ws = L.kvs_paged_decode_scored_workspace_size(1, 32, 8, 128, 400)
    assert ws >= 32 * 400 * 4 > 0                      # the logits of one step are always kept
    args = dict(q=fake, kp=fake, vp=fake, nb=64, tbl=fake, mb=25, ctx=fake, B=1, mc=400, hq=32, hkv=8, d=128,
                sc=0.1, nk=fake, nv=fake, dst=fake, ss=fake, stride=400, o=fake, lse=None, ws=fake, wsb=ws, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return L.kvs_paged_decode_scored(*a.values())
    assert call(ss=None) == -1                          # slot scores are required
    assert call(nk=None, nv=None) == -1                 # dst_slots without a new token
    assert call(stride=399) == -1                       # slot rows shorter than the context
    assert call(wsb=ws - 1) == -1 and b"workspace" in L.kvs_last_error()


def test_fp8_calls_validate_on_the_host():
    L = kvs.lib
    fake = 0x1000   # never dereferenced: the checks fail first
    # compaction: the scale arrays are required, d is 64 or 128
    comp = dict(k=fake, v=fake, cu=fake, ns=1, hkv=2, d=128, keep=None, ko=None, mk=64, kp=fake, vp=fake, ks=fake,
                vs=fake, nb=8, tbl=fake, mb=4, off=None, st=None)

    def compact(**kw):
        return L.kvs_compact_paged_fp8(*dict(comp, **kw).values())
    assert compact(ks=None) == -1 and b"NULL" in L.kvs_last_error()
    assert compact(d=96) == -1
    assert compact(ns=0) == 0 and compact(mk=0) == 0   # nothing to write: nothing launched
    # decode: scales required, workspace as for the 16-bit decode
    ws = L.kvs_paged_decode_workspace_size(1, 32, 8, 128, 400)
    dec = dict(q=fake, kp=fake, vp=fake, ks=fake, vs=fake, nb=64, tbl=fake, mb=25, ctx=fake, B=1, mc=400, hq=32,
               hkv=8, d=128, sc=0.1, nk=fake, nv=fake, o=fake, lse=None, ws=fake, wsb=ws, st=None)

    def decode(**kw):
        return L.kvs_paged_decode_fp8(*dict(dec, **kw).values())
    assert decode(vs=None) == -1
    assert decode(nv=None) == -1                         # new_k and new_v go together
    assert decode(mb=24) == -1                           # table rows shorter than the context
    assert decode(wsb=ws - 1) == -1 and b"workspace" in L.kvs_last_error()
    assert decode(B=0) == 0
    assert L.kvs_copy_blocks_fp8(fake, fake, None, fake, 8, 2, 128, fake, 1, None) == -1
    assert L.kvs_copy_blocks_fp8(fake, fake, fake, fake, 8, 2, 128, None, 0, None) == 0


def test_chunk_and_gather_calls_validate_on_the_host():
    L = kvs.lib
    fake = 0x1000   # never dereferenced: the checks fail first
    # chunk prefill: key offsets required, max_k >= max_q
    assert L.kvs_prefill_attn_lse_chunk(fake, fake, fake, fake, None, 1, 10, 10, 20, 8, 2, 128, 0.1, fake, fake,
                                        None, None, None) == -1
    assert L.kvs_prefill_attn_lse_chunk(fake, fake, fake, fake, fake, 1, 10, 30, 20, 8, 2, 128, 0.1, fake, fake,
                                        None, None, None) == -1 and b"max_k" in L.kvs_last_error()
    assert L.kvs_prefill_attn_lse_chunk(fake, fake, fake, fake, fake, 1, 10, 10, 20, 8, 3, 128, 0.1, fake, fake,
                                        None, None, None) == -1     # hq % hkv
    assert L.kvs_prefill_attn_lse_chunk(fake, fake, fake, fake, fake, 0, 0, 0, 0, 8, 2, 128, 0.1, fake, fake,
                                        None, None, None) == 0
    # window score on chunks
    assert L.kvs_window_score_chunk(fake, fake, fake, fake, None, 1, 10, 20, 20, 4, 8, 2, 128, 0.1, fake, None) == -1
    assert L.kvs_window_score_chunk(fake, fake, fake, fake, fake, 1, 10, 20, 20, 0, 8, 2, 128, 0.1, fake, None) == -1
    # gather
    assert L.kvs_gather_paged(fake, fake, 8, fake, 4, 1, 2, 96, fake, fake, 16, fake, fake, None) == -1
    assert L.kvs_gather_paged(fake, fake, 8, fake, 4, 1, 2, 128, None, fake, 16, fake, fake, None) == -1
    assert L.kvs_gather_paged(fake, fake, 8, fake, 4, 1, 2, 128, fake, fake, 0, fake, fake, None) == 0


def test_package_refuses_to_import_without_the_library(tmp_path):
    """No CPU fallback: a copy of the package without libkvs.so fails at import, naming the build."""
    import shutil
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = os.path.join(root, "kv_cache_sparsification_amd")
    dst = tmp_path / "kv_cache_sparsification_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "__pycache__", "csrc"))
    r = subprocess.run([sys.executable, "-c", "import kv_cache_sparsification_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, PYTHONPATH=str(tmp_path)))
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "is not built" in r.stderr


def test_chunked_step_rejects_short_chunks_on_the_host():
    """A compressed layer's chunk must hold its prompt's last min(alpha, n) rows, and no chunk may
    be longer than its prompt: the pipeline raises before touching a device."""
    from kv_cache_sparsification_amd import pipeline
    pipeline.check_chunk_lengths([32, 100], [4000, 100], 32, True)
    pipeline.check_chunk_lengths([5], [5], 32, True)                  # n < alpha: the whole prompt
    pipeline.check_chunk_lengths([1], [4000], 32, False)              # a full layer needs no window
    for q, k in (([31], [4000]), ([4], [5]), ([101], [100]), ([-1], [10])):
        with pytest.raises(ValueError):
            pipeline.check_chunk_lengths(q, k, 32, True)
    with pytest.raises(ValueError):
        pipeline.prefill_compress_layer_chunked(None, None, None, None, None, [16], [4000], 32, 400, None, None,
                                                [[0]], 1)
