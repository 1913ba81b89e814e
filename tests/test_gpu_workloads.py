"""GPU parity at the full sizes of the multi-layer workloads, through the C ABI.

  * 32 layers x 20 concurrent prompts of U[1000, 4000] tokens (layers 0-2 full, 3-31 k=512,
    alpha=32), then 500 batched decode steps at concurrency 20 on layers 0, 3 and 31;
  * 4 prompts x 30000 tokens (alpha=64, k=3000 on layers 3-31), then 500 decode steps.

Inputs are drawn on the device (seeded); the oracle gets the slices it needs copied back.
Where the fp64 oracle would take too long at full size it checks sampled outputs it can
compute one by one (seeded rows of O and LSE, every window row), and properties that hold at
any size (every prompt's scores sum to G * alpha per KV head); kept sets and block contents
are checked in full on every layer.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._parity import (bf16_to_f64, bf16_bits, i32, assert_rows_close, assert_lse_close, assert_scores_close,
                           assert_keep_matches, gather_pools)

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


def _host(t):
    return bf16_to_f64(t)


class LayerRun:
    """One layer of a batch through prefill, score, top-k and compaction, with its own pool."""

    def __init__(self, w, layer, lengths, seq_ids, decode_steps):
        self.w, self.layer, self.lengths = w, layer, list(lengths)
        self.k_budget = w.budgets[layer]
        self.q, self.k, self.v, self.cu = wl.device_batch(w, layer, lengths, seq_ids)
        self.kept = kvs.keep_counts(lengths, self.k_budget)
        need = sum(oracle.blocks_for(c + decode_steps) for c in self.kept)
        self.max_blocks = max(oracle.blocks_for(c + decode_steps) for c in self.kept)
        self.alloc = kvs.BlockAllocator(need + 8, list(np.random.default_rng(layer).permutation(need + 8)))
        self.k_pool, self.v_pool = kvs.new_pools(need + 8, w.hkv, w.d)
        self.k_pool.view(torch.int16).fill_(0x7FC0)
        self.v_pool.view(torch.int16).fill_(0x7FC0)
        self.cu_d = i32(self.cu)
        self.res = kvs.prefill_compress_layer(self.q, self.k, self.v, self.cu_d, lengths, w.alpha, self.k_budget,
                                              self.alloc, self.k_pool, self.v_pool, self.max_blocks)
        torch.cuda.synchronize()
        self.kb = bf16_bits(self.k)
        self.vb = bf16_bits(self.v)
        self.keep = None
        if self.res["keep_idx"] is not None:
            flat = self.res["keep_idx"].cpu().numpy()
            off = np.concatenate([[0], np.cumsum(self.kept)])
            self.keep = [flat[w.hkv * off[s]: w.hkv * off[s + 1]].reshape(w.hkv, self.kept[s])
                         for s in range(len(lengths))]
            self.S = self.res["scores"].cpu().numpy().astype(np.float64)

    def seq_keep(self, s):
        if self.keep is None:
            return np.tile(np.arange(self.lengths[s]), (self.w.hkv, 1))
        return self.keep[s]

    def check_blocks(self):
        for s, n in enumerate(self.lengths):
            gk, gv = gather_pools(self.k_pool, self.v_pool, self.res["tables"][s], self.kept[s])
            kp = self.seq_keep(s)
            a = self.cu[s]
            for g in range(self.w.hkv):
                np.testing.assert_array_equal(gk[:, g], self.kb[a + kp[g], g], err_msg=f"K blocks seq {s} head {g}")
                np.testing.assert_array_equal(gv[:, g], self.vb[a + kp[g], g], err_msg=f"V blocks seq {s} head {g}")

    def check_keep_same_scores(self):
        """Bit-exact against the oracle's rule applied to the GPU's own fp32 scores."""
        if self.keep is None:
            return
        w = self.w
        for s, n in enumerate(self.lengths):
            a = self.cu[s]
            for g in range(w.hkv):
                np.testing.assert_array_equal(self.keep[s][g],
                                              oracle.select_keep(self.S[g, a:a + n], n, w.alpha, self.k_budget),
                                              err_msg=f"keep seq {s} head {g}")

    def check_conservation(self):
        """Each window row's softmax sums to one: a prompt's scores add up to G * min(alpha, n) per KV head."""
        if self.keep is None:
            return
        w = self.w
        for s, n in enumerate(self.lengths):
            a = self.cu[s]
            tot = self.S[:, a:a + n].sum(axis=1)
            np.testing.assert_allclose(tot, w.g * min(w.alpha, n), rtol=1e-4, err_msg=f"conservation seq {s}")

    def check_oracle(self, s, n_rows, seed):
        """O and LSE on seeded rows plus every window row; S and keep of the whole prompt."""
        w, n = self.w, self.lengths[s]
        a0 = self.cu[s]
        win = np.arange(n - min(w.alpha, n), n)
        sample = np.random.default_rng(seed).choice(n - len(win), size=min(n_rows, n - len(win)), replace=False)
        rows = np.unique(np.concatenate([sample, win]))
        kf = _host(self.k[a0:a0 + n])
        vf = _host(self.v[a0:a0 + n])
        qrows = _host(self.q[a0 + torch.as_tensor(rows, device="cuda")])
        O_ref, lse_ref, _, _ = oracle.causal_attention(qrows, kf, vf, rows=rows, q_holds_rows=True)
        O_gpu = _host(self.res["o"][a0 + torch.as_tensor(rows, device="cuda")])
        assert_rows_close(O_gpu, O_ref, what=f"O layer {self.layer} seq {s}")
        lse_gpu = self.res["lse"][:, a0 + torch.as_tensor(rows, device="cuda")].cpu().numpy()
        assert_lse_close(lse_gpu, lse_ref, what=f"LSE layer {self.layer} seq {s}")
        if self.keep is None:
            return
        wi = np.searchsorted(rows, win)
        S_ref = oracle.window_score(qrows[wi], kf, lse_ref[:, wi], w.alpha, window_only=True)
        assert_scores_close(self.S[:, a0:a0 + n], S_ref, what=f"S layer {self.layer} seq {s}")
        for g in range(w.hkv):
            assert_keep_matches(self.keep[s][g], oracle.select_keep(S_ref[g], n, w.alpha, self.k_budget), S_ref[g],
                                n, w.alpha, self.k_budget, what=f"keep layer {self.layer} seq {s} head {g}")

    def decode(self, steps, check_steps, seq_ids, check_seqs):
        """Batched decode with append; the oracle checks the chosen (step, sequence) pairs."""
        w = self.w
        B = len(self.lengths)
        tables = [list(t) for t in self.res["tables"]]
        tbl = np.full((B, self.max_blocks), -1, np.int32)
        # oracle-side caches [L][Hkv][d], preallocated for every step
        ck, cv, clen = {}, {}, {}
        for s in check_seqs:
            kp = self.seq_keep(s)
            ck[s] = np.zeros((self.kept[s] + steps, w.hkv, w.d))
            cv[s] = np.zeros_like(ck[s])
            for g in range(w.hkv):
                idx = self.cu[s] + torch.as_tensor(kp[g], device="cuda")
                ck[s][:self.kept[s], g] = _host(self.k[idx, g])
                cv[s][:self.kept[s], g] = _host(self.v[idx, g])
            clen[s] = self.kept[s]
        max_ctx = self.kept_max_ctx(steps)
        nbytes = kvs.kvs_paged_decode_workspace_size(B, w.hq, w.hkv, w.d, max_ctx)
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        for step in range(steps):
            Ls = [c + step + 1 for c in self.kept]
            for s in range(B):
                if (Ls[s] - 1) % 16 == 0:
                    tables[s].append(self.alloc.alloc())
                tbl[s, :len(tables[s])] = tables[s]
            dq, dk, dv = wl.device_decode_step(w, self.layer, step, seq_ids)
            lse = torch.empty(B, w.hq, device="cuda", dtype=torch.float32)
            o = kvs.kvs_paged_decode(dq, self.k_pool, self.v_pool, i32(tbl), i32(Ls), max_ctx,
                                     new_k=dk, new_v=dv, lse=lse, workspace=ws)
            dkh, dvh = _host(dk), _host(dv)
            for s in check_seqs:
                ck[s][clen[s]] = dkh[s]
                cv[s][clen[s]] = dvh[s]
                clen[s] += 1
            if step in check_steps:
                og, lg = _host(o), lse.cpu().numpy()
                dqh = _host(dq)
                for s in check_seqs:
                    o_ref, l_ref = oracle.decode_attention(dqh[s], ck[s][:clen[s]], cv[s][:clen[s]])
                    assert_rows_close(og[s], o_ref, what=f"decode layer {self.layer} step {step} seq {s}")
                    assert_lse_close(lg[s], l_ref, what=f"decode lse layer {self.layer} step {step} seq {s}")

    def kept_max_ctx(self, steps):
        return max(self.kept) + steps


@pytest.mark.timeout(900)
def test_32_layers_concurrency_20():
    w = wl.WORKLOADS[3]
    lengths = w.seq_lengths()
    seq_ids = list(range(w.num_seqs))
    _say(f"32 layers x {len(lengths)} prompts, lengths {min(lengths)}..{max(lengths)}")
    dec_steps = w.decode_steps
    for layer in range(w.n_layers):
        full_check = layer in (0, 3, 31)
        _say(f"layer {layer} (full check: {full_check})")
        run = LayerRun(w, layer, lengths, seq_ids, dec_steps if full_check else 0)
        run.check_blocks()
        run.check_keep_same_scores()
        run.check_conservation()
        if full_check:
            for s in range(len(lengths)):
                run.check_oracle(s, n_rows=24, seed=100 * layer + s)
            run.decode(dec_steps, check_steps={0, 1, 15, 16, 249, 499}, seq_ids=seq_ids,
                       check_seqs=range(len(lengths)))
        del run
        torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_long_context_4x30000():
    w = wl.WORKLOADS[4]
    lengths = w.seq_lengths()
    seq_ids = list(range(w.num_seqs))
    steps = w.decode_steps
    for layer in (0, 3, 31):
        _say(f"long context layer {layer}: 4 x 30000, alpha=64, k={w.budgets[layer]}")
        run = LayerRun(w, layer, lengths, seq_ids, steps)
        run.check_blocks()
        run.check_keep_same_scores()
        run.check_conservation()
        run.check_oracle(0, n_rows=512, seed=7 + layer)
        run.decode(steps, check_steps={0, 249, 499}, seq_ids=seq_ids, check_seqs=[0, 3])
        del run
        torch.cuda.empty_cache()
