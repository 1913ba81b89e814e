"""GPU parity of the 8-bit (E4M3) cache (readings R22-R24) through the C ABI.

Codes and scales are integer/bit results of a float32 decision both sides take in the same
precision, so pools are compared bit-exactly with the oracle (pools are poisoned with NaN
codes and NaN scales first, so a slot written that should not be, or missed, shows).  Decode
outputs and LSE use the 16-bit decode's tolerances against the fp64 oracle attending over
code * scale.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
import workloads as wl
from tests._parity import bf16_to_f64, i32, to_dev_bf16, assert_rows_close, assert_lse_close

pytestmark = pytest.mark.gpu

kvs = pytest.importorskip("kv_cache_sparsification_amd")

NAN_CODE = 0x7F


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _gpu_pools(nb, hkv, d):
    kp, vp, ks, vs = kvs.new_pools_fp8(nb, hkv, d)
    kp.fill_(NAN_CODE); vp.fill_(NAN_CODE)
    ks.fill_(float("nan")); vs.fill_(float("nan"))
    return kp, vp, ks, vs


def _oracle_pools(nb, hkv, d):
    kp = np.full((nb, hkv, 16, d), NAN_CODE, np.uint8)
    vp = np.full((nb, hkv, 16, d), NAN_CODE, np.uint8)      # token rows; the GPU's V pool is transposed
    ks = np.full((nb, hkv, 16), np.nan, np.float32)
    vs = np.full((nb, hkv, 16), np.nan, np.float32)
    return kp, vp, ks, vs


def _assert_pools_equal(gpu, ref, what=""):
    kp, vp, ks, vs = gpu
    rk, rv, rks, rvs = ref
    np.testing.assert_array_equal(kp.cpu().numpy(), rk, err_msg=f"K codes {what}")
    np.testing.assert_array_equal(vp.permute(0, 1, 3, 2).cpu().numpy(), rv, err_msg=f"V codes {what}")
    np.testing.assert_array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32), err_msg=f"K scales {what}")
    np.testing.assert_array_equal(vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32), err_msg=f"V scales {what}")


def _bits(x_f64):
    """float64 values that bf16 holds exactly -> bf16 bit patterns."""
    b = wl.f32_to_bf16_bits(np.asarray(x_f64, np.float32))
    assert np.array_equal(wl.bf16_bits_to_f64(b), x_f64), "crafted value not exact in bf16"
    return b


def _edge_rows(rng, n, hkv, d):
    """Rows whose multiplier 448/amax is a power of two, so x * r lands exactly on chosen values:
    every tie between neighbouring codes, tiny negatives that round to -0, subnormals,
    saturation neighbours; plus a zero row, a row below 2^-112 and a row of -0."""
    pos = ofp8.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2
    pool = np.concatenate([mids, pos, [2.0 ** -11, 2.0 ** -12, 3 * 2.0 ** -11, 440.0, 444.0, 0.0]])
    x = np.empty((n, hkv, d))
    for t in range(n):
        for g in range(hkv):
            e = int(rng.integers(-12, 5))
            vals = rng.choice(pool, d) * np.where(rng.random(d) < 0.5, -1.0, 1.0)
            vals[int(rng.integers(d))] = 448.0 * (1 if rng.random() < 0.5 else -1)   # the row's amax
            x[t, g] = vals * 2.0 ** e
    x[3, 0] = 0.0
    x[4, 1] = 2.0 ** -113 * np.where(rng.random(d) < 0.5, -1.0, 1.0)
    x[5, 0] = -0.0
    return x


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_codes_on_ties_and_edges(d):
    """Keep-all compaction of crafted rows: every rounding decision bit-exact with the oracle."""
    _say(f"fp8 edge codes d={d}")
    rng = np.random.default_rng(40 + d)
    n, hkv = 48, 2
    xk, xv = _edge_rows(rng, n, hkv, d), _edge_rows(rng, n, hkv, d)
    kb, vb = _bits(xk), _bits(xv)
    # -0.0 survives as a bf16 pattern only through the bits
    kb[5, 0] = 0x8000; vb[5, 0] = 0x8000
    nb = 5
    table = [3, 0, 4]
    gpu = _gpu_pools(nb, hkv, d)
    kvs.kvs_compact_paged_fp8(to_dev_bf16(kb), to_dev_bf16(vb), i32([0, n]), None, None, n, *gpu,
                              i32([table]))
    ref = _oracle_pools(nb, hkv, d)
    ofp8.compact_into_pool_fp8(wl.bf16_bits_to_f64(kb), wl.bf16_bits_to_f64(vb), None, table, *ref)
    torch.cuda.synchronize()
    _assert_pools_equal(gpu, ref, "edge rows")
    # the crafted ties really were ties, and -0 really came out as 0x80 somewhere
    assert (ref[0] == 0x80).any()


@pytest.mark.parametrize("hkv,d", [(2, 64), (8, 128)])
def test_fp8_compaction_ragged_with_offsets(hkv, d):
    """Three prompts, per-head kept subsets, misaligned destination offsets."""
    _say(f"fp8 compaction ragged hkv={hkv} d={d}")
    rng = np.random.default_rng(7 + d)
    lengths = [37, 200, 90]
    k_effs = [20, 131, 90]
    offs = [0, 5, 16]
    T = sum(lengths)
    kx = rng.standard_normal((T, hkv, d)) * np.exp2(rng.integers(-3, 4, (T, hkv, 1)))
    vx = rng.standard_normal((T, hkv, d))
    kb, vb = wl.f32_to_bf16_bits(kx.astype(np.float32)), wl.f32_to_bf16_bits(vx.astype(np.float32))
    kf, vf = wl.bf16_bits_to_f64(kb), wl.bf16_bits_to_f64(vb)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    keep_parts, keeps = [], []
    for n, ke in zip(lengths, k_effs):
        kp_s = np.stack([np.sort(rng.choice(n, ke, replace=False)) for _ in range(hkv)])
        keeps.append(kp_s)
        keep_parts.append(kp_s.reshape(-1))
    keep_off = np.concatenate([[0], np.cumsum(k_effs)]).astype(np.int32)
    max_blocks = max(-(-(o + k) // 16) for o, k in zip(offs, k_effs))
    nb = 3 * max_blocks + 4
    perm = rng.permutation(nb)
    tables = np.full((3, max_blocks), -1, np.int32)
    used = 0
    for s in range(3):
        m = -(-(offs[s] + k_effs[s]) // 16)
        tables[s, :m] = perm[used:used + m]
        used += m
    gpu = _gpu_pools(nb, hkv, d)
    kvs.kvs_compact_paged_fp8(to_dev_bf16(kb), to_dev_bf16(vb), i32(cu), i32(np.concatenate(keep_parts)),
                              i32(keep_off), max(k_effs), *gpu, i32(tables), dst_slot_offset=i32(offs))
    ref = _oracle_pools(nb, hkv, d)
    for s in range(3):
        sl = slice(cu[s], cu[s + 1])
        ofp8.compact_into_pool_fp8(kf[sl], vf[sl], keeps[s], list(tables[s]), *ref, off=offs[s])
    torch.cuda.synchronize()
    _assert_pools_equal(gpu, ref, "ragged")


def test_fp8_copy_blocks():
    _say("fp8 copy blocks")
    rng = np.random.default_rng(3)
    nb, hkv, d = 10, 4, 128
    kp, vp, ks, vs = kvs.new_pools_fp8(nb, hkv, d)
    for t in (kp, vp):
        t.copy_(torch.from_numpy(rng.integers(0, 256, t.shape, dtype=np.uint8)))
    for t in (ks, vs):
        t.copy_(torch.from_numpy(rng.random(t.shape, dtype=np.float32)))
    before = [t.cpu().numpy().copy() for t in (kp, vp, ks, vs)]
    pairs = np.array([[1, 7], [4, 2], [9, 0]], np.int32)
    kvs.kvs_copy_blocks_fp8(kp, vp, ks, vs, i32(pairs))
    torch.cuda.synchronize()
    for t, b in zip((kp, vp, ks, vs), before):
        want = b.copy()
        for s_, d_ in pairs:
            want[d_] = b[s_]
        np.testing.assert_array_equal(t.cpu().numpy(), want)


def _decode_case(name, hq, hkv, d, k_effs, steps, seed, check_every=1, prompt_extra=64):
    """Compaction of random kept subsets into an 8-bit cache, then `steps` decode steps with
    append for every sequence; outputs, LSE and the final pools against the oracle."""
    B = len(k_effs)
    _say(f"fp8 decode {name}: B={B} hq={hq} hkv={hkv} d={d} k_eff={min(k_effs)}..{max(k_effs)} steps={steps}")
    rng = np.random.default_rng(seed)
    lengths = [k + prompt_extra for k in k_effs]
    T = sum(lengths)
    kb = wl.f32_to_bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
    vb = wl.f32_to_bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
    kf, vf = wl.bf16_bits_to_f64(kb), wl.bf16_bits_to_f64(vb)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    keeps = [np.stack([np.sort(rng.choice(n, ke, replace=False)) for _ in range(hkv)])
             for n, ke in zip(lengths, k_effs)]
    keep_off = np.concatenate([[0], np.cumsum(k_effs)]).astype(np.int32)
    max_ctx = max(k_effs) + steps
    max_blocks = -(-max_ctx // 16)
    nb = B * max_blocks + 3
    perm = rng.permutation(nb)
    tables = perm[:B * max_blocks].reshape(B, max_blocks).astype(np.int32)
    gpu = _gpu_pools(nb, hkv, d)
    tbl_d = i32(tables)
    kvs.kvs_compact_paged_fp8(to_dev_bf16(kb), to_dev_bf16(vb), i32(cu),
                              i32(np.concatenate([k.reshape(-1) for k in keeps])), i32(keep_off), max(k_effs), *gpu,
                              tbl_d)
    ref = _oracle_pools(nb, hkv, d)
    for s in range(B):
        sl = slice(cu[s], cu[s + 1])
        ofp8.compact_into_pool_fp8(kf[sl], vf[sl], keeps[s], list(tables[s]), *ref)
    torch.cuda.synchronize()
    _assert_pools_equal(gpu, ref, f"{name} after compaction")
    ws_bytes = kvs.kvs_paged_decode_workspace_size(B, hq, hkv, d, max_ctx)
    ws = torch.empty(max(ws_bytes, 1), device="cuda", dtype=torch.uint8)
    for step in range(steps):
        L = np.array(k_effs) + step + 1
        q = wl.f32_to_bf16_bits(rng.standard_normal((B, hq, d), dtype=np.float32))
        nk = wl.f32_to_bf16_bits(rng.standard_normal((B, hkv, d), dtype=np.float32) * 2)
        nv = wl.f32_to_bf16_bits(rng.standard_normal((B, hkv, d), dtype=np.float32))
        lse = torch.empty(B, hq, device="cuda", dtype=torch.float32)
        o = kvs.kvs_paged_decode_fp8(to_dev_bf16(q), *gpu, tbl_d, i32(L), max_ctx, new_k=to_dev_bf16(nk),
                                     new_v=to_dev_bf16(nv), lse=lse, workspace=ws)
        for s in range(B):
            ofp8.append_row_fp8(*ref, list(tables[s]), int(L[s]) - 1, wl.bf16_bits_to_f64(nk[s]),
                                wl.bf16_bits_to_f64(nv[s]))
        if step % check_every == 0 or step == steps - 1:
            og, lg = bf16_to_f64(o), lse.cpu().numpy()
            qf = wl.bf16_bits_to_f64(q)
            for s in range(B):
                kc = ofp8.gather_rows_fp8(ref[0], ref[2], list(tables[s]), int(L[s]))
                vc = ofp8.gather_rows_fp8(ref[1], ref[3], list(tables[s]), int(L[s]))
                o_ref, l_ref = oracle.decode_attention(qf[s], kc, vc)
                assert_rows_close(og[s], o_ref, what=f"{name} step {step} seq {s}")
                assert_lse_close(lg[s], l_ref, what=f"{name} step {step} seq {s}")
    torch.cuda.synchronize()
    _assert_pools_equal(gpu, ref, f"{name} after {steps} steps")


def test_fp8_decode_tiny():
    """d = 64, G = 2, one sequence: appends cross a block boundary."""
    _decode_case("tiny", 4, 2, 64, [60], 12, seed=1)


def test_fp8_decode_llama8b_layer():
    """The 8B layer after compression: 32 query heads over 8 KV heads, 400 kept tokens (split context)."""
    _decode_case("8B layer", 32, 8, 128, [400], 20, seed=2, check_every=4)


def test_fp8_decode_long_context_batch():
    """Four sequences of about 3000 cached tokens (the long-context budget): the read-volume launch plan."""
    _decode_case("long context", 32, 8, 128, [3000, 2950, 3001, 2990], 3, seed=3, prompt_extra=200)


def test_fp8_decode_long_contexts():
    """Two sequences of 17000-20000 cached tokens: the long-context plan (equal pieces over
    8-wavefront workgroups, the piece count chosen to fill the CUs)."""
    _decode_case("long contexts", 32, 8, 128, [20000, 17001], 2, seed=9, prompt_extra=16)


@pytest.mark.parametrize("hq,hkv,d,k_effs", [(16, 2, 64, [700, 5]), (16, 1, 64, [300, 2500]),
                                             (16, 1, 128, [1200, 7])])
def test_fp8_decode_wide_groups(hq, hkv, d, k_effs):
    """Groups of 8 and 16 query heads per KV head over the 8-bit cache: the 8- and 4-wavefront
    launch shapes at d = 64 and 128, contexts split and merged or walked by one workgroup."""
    _decode_case(f"G={hq // hkv} d={d}", hq, hkv, d, k_effs, 5, seed=hq * d + hkv, check_every=2)


def test_fp8_decode_wide_batch():
    """64 short sequences: one workgroup per (sequence, KV head), no split."""
    rng = np.random.default_rng(4)
    _decode_case("wide batch", 32, 8, 128, list(rng.integers(1, 60, 64)), 3, seed=4, prompt_extra=8)


@pytest.mark.parametrize("B,lo,hi", [(20, 400, 700), (16, 2000, 2300)])
def test_fp8_decode_wide_batch_plans(B, lo, hi):
    """Wide batches in the plans without a split (short contexts, one workgroup per sequence
    and head) and with many one-round splits (long contexts): outputs and LSE against the
    oracle attending over the quantized rows, two steps with append."""
    _say(f"fp8 decode wide batch B={B} lengths {lo}..{hi}")
    rng = np.random.default_rng(B)
    hq, hkv, d, steps = 32, 8, 128, 2
    lengths = [int(x) for x in rng.integers(lo, hi, B)]
    T = sum(lengths)
    kb = wl.f32_to_bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
    vb = wl.f32_to_bf16_bits(rng.standard_normal((T, hkv, d), dtype=np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    max_ctx = max(lengths) + steps
    nbs = [-(-(n + steps) // 16) for n in lengths]
    nb = sum(nbs)
    perm = rng.permutation(nb)
    tables = np.full((B, max(nbs)), -1, np.int32)
    used = 0
    for s, c in enumerate(nbs):
        tables[s, :c] = perm[used:used + c]
        used += c
    pools = kvs.new_pools_fp8(nb, hkv, d)
    tbl = i32(tables)
    kvs.kvs_compact_paged_fp8(to_dev_bf16(kb), to_dev_bf16(vb), i32(cu), None, None, max(lengths), *pools, tbl)
    kq = ofp8.dequantize_rows(*ofp8.quantize_rows(wl.bf16_bits_to_f64(kb)))   # the cached values
    vq = ofp8.dequantize_rows(*ofp8.quantize_rows(wl.bf16_bits_to_f64(vb)))
    ws_bytes = kvs.kvs_paged_decode_workspace_size(B, hq, hkv, d, max_ctx)
    ws = torch.empty(max(ws_bytes, 1), device="cuda", dtype=torch.uint8)
    new_k, new_v = [[] for _ in range(B)], [[] for _ in range(B)]
    for step in range(steps):
        L = np.array(lengths) + step + 1
        q = wl.f32_to_bf16_bits(rng.standard_normal((B, hq, d), dtype=np.float32))
        nk = wl.f32_to_bf16_bits(rng.standard_normal((B, hkv, d), dtype=np.float32))
        nv = wl.f32_to_bf16_bits(rng.standard_normal((B, hkv, d), dtype=np.float32))
        lse = torch.empty(B, hq, device="cuda", dtype=torch.float32)
        o = kvs.kvs_paged_decode_fp8(to_dev_bf16(q), *pools, tbl, i32(L), max_ctx, new_k=to_dev_bf16(nk),
                                     new_v=to_dev_bf16(nv), lse=lse, workspace=ws)
        og, lg = bf16_to_f64(o), lse.cpu().numpy()
        qf = wl.bf16_bits_to_f64(q)
        for s in range(B):
            new_k[s].append(ofp8.dequantize_rows(*ofp8.quantize_rows(wl.bf16_bits_to_f64(nk[s]))))
            new_v[s].append(ofp8.dequantize_rows(*ofp8.quantize_rows(wl.bf16_bits_to_f64(nv[s]))))
            kc = np.concatenate([kq[cu[s]:cu[s + 1]], np.stack(new_k[s])])
            vc = np.concatenate([vq[cu[s]:cu[s + 1]], np.stack(new_v[s])])
            o_ref, l_ref = oracle.decode_attention(qf[s], kc, vc)
            assert_rows_close(og[s], o_ref, what=f"wide batch step {step} seq {s}")
            assert_lse_close(lg[s], l_ref, what=f"wide batch step {step} seq {s}")
