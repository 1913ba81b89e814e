// Per-layer, per-KV-head selection of the tokens to keep.
//
// [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM", Key techniques,
// 2. "Attention modification": in each layer and head the k_l highest-scoring tokens keep
// their KV entries and all others are dropped for the rest of the generation.  [KVS]
// System model: pairs with a high score and greater proximity are the ones kept.
//
// Rule (a = min(alpha, n)): k >= n keeps all n tokens; otherwise the window n-a..n-1 is
// always kept and the other k - a slots go to the highest scores among tokens i < n - a,
// equal scores going to the lower index; indices are emitted in ascending order.
//
// One workgroup per (prompt, KV head).  Scores are non-negative fp32, so their bit patterns
// order like unsigned integers: up to three radix passes (11, 11 and 10 bits) over the
// candidates find the threshold value T (the (k-a)-th largest) and how many copies of T are
// still needed; the search ends early once the threshold bin is taken whole.  Scores crowd
// into a few leading bins (most of a head's scores share their exponent), so every bin is kept
// in four copies on adjacent banks, lane l adding to copy l % 4: a quarter of the
// same-address atomics per bin, summed back when the bins are read.  The candidates are read
// from memory once, into LDS, when they fit; the passes then run on LDS.  A final pass over
// contiguous per-thread chunks keeps every score above T plus the first `ties` copies of T
// (lowest index first), placing them with two block scans, and writes the window after them.
// No sort, no device-wide traffic.
//
// The same selection also runs fused with the compaction of the kept rows ([PAG] "How paging
// works": the rows go to 16-token blocks through the block table): one workgroup per
// (prompt, KV head, destination block) repeats it and copies its block (topk_compact_kernel).
#include "compact_block.h"
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kLdsCap = 16384;   // candidates held in LDS (64 KB); longer prompts read L2 each pass
constexpr int kCopies = 4;       // copies of every histogram bin: lane l counts into copy l % 4
constexpr int kKeptCap = 2 * 2048 * kCopies;   // kept indices the fused kernel holds in the histograms' LDS
// (prompt, head, block) workgroups of a fused launch at most: one per CU (a 1024-thread workgroup
// of this kernel's registers fits a CU once), so the repeated selections run side by side
constexpr long long kFusedMaxWGs = 256;

// Inclusive scan across the 64 lanes with DPP moves (no LDS): prefix sums within rows of 16
// lanes by shifts of 1, 2, 4 and 8, then row 0's total into rows 1 and 3 (row_bcast:15) and
// rows 0-1's total into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// Block-wide inclusive scan of one int per thread; `tot` is kWaves ints of LDS, and the
// caller's next write to it must follow a barrier.
__device__ __forceinline__ int block_incl_scan(int x, int* tot) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  x = wave_incl_scan(x);
  if (lane == kWave - 1) tot[w] = x;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kWaves; ++i) x += i < w ? tot[i] : 0;
  return x;
}

// LDS of one selection: the candidates (dynamic, up to kLdsCap + 4 words), the double-buffered
// histograms, the scan totals and the chosen bin.
struct SelectLds {
  uint32_t* cand;
  int (*hist)[2048 * kCopies];
  int (*tot)[kWaves];
  int* sel;   // bin, remaining count, whole-bin flag
};

// The kept indices of one (prompt, KV head), written through `out` (global memory or LDS):
// rank t at out[t], ascending, k_eff = min(k_budget, n) of them.  `bits` are the head's scores
// of the prompt.  Every thread of the workgroup must call it; it ends without a barrier after
// its last write.
__device__ __forceinline__ void select_kept(const uint32_t* __restrict__ bits, int n, int alpha, int k_budget,
                                            int32_t* out, SelectLds L, int cand_cap) {
  const int tid = threadIdx.x;
  uint32_t* cand = L.cand;
  auto hist = L.hist;
  auto tot = L.tot;
  int& sel_bin = L.sel[0];
  int& sel_rem = L.sel[1];
  int& sel_all = L.sel[2];
  if (k_budget >= n) {
    for (int i = tid; i < n; i += kThreads) out[i] = i;
    return;
  }
  const int a = alpha < n ? alpha : n;
  const int n_cand = n - a;
  const int kk = k_budget - a;   // slots filled by score (0 when the budget is the window)
  // the window follows the kk chosen candidates (its indices are all larger); written last, so
  // that `out` may share memory with the histograms
  auto write_window = [&]() {
    for (int i = n_cand + tid; i < n; i += kThreads) out[kk + i - n_cand] = i;
  };
  if (kk == 0) {
    write_window();
    return;
  }
  const bool in_lds = n_cand <= cand_cap;   // block-uniform; cand_cap: the candidate LDS allocated
  if (in_lds) {
    // Eight loads per thread in flight before the LDS stores: one memory round trip per
    // 8 * kThreads candidates instead of one per kThreads.
    constexpr int kBatch = 8;
    for (int i0 = 0; i0 < n_cand; i0 += kThreads * kBatch) {
      uint32_t vals[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = i0 + j * kThreads + tid;
        vals[j] = i < n_cand ? bits[i] : 0u;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int i = i0 + j * kThreads + tid;
        if (i < n_cand) cand[i] = vals[j];
      }
    }
  }

  uint32_t prefix = 0, mask = 0;
  int remaining = kk;
  const int copy = tid % kCopies;
  auto clear = [&](int* h) {
    for (int b = tid; b < 2048; b += kThreads) *reinterpret_cast<u32x4*>(&h[b * kCopies]) = u32x4{0u, 0u, 0u, 0u};
  };
  auto bin_count = [&](const int* h, int b) {   // a bin's four copies, one 16-byte read
    const u32x4 c = *reinterpret_cast<const u32x4*>(&h[b * kCopies]);
    return (int)(c[0] + c[1] + c[2] + c[3]);
  };
  clear(hist[0]);
  __syncthreads();   // also publishes the candidates in LDS
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : pass == 1 ? 10 : 0;
    const int nbins = pass == 2 ? 1024 : 2048;
    int* hs = hist[pass & 1];
    // A thread's candidates tid, tid + kThreads, ... are read in batches of kBatch before their
    // atomics, so a batch costs one read round trip; LDS and global memory get loops of their
    // own (one loop over a pointer to either would compile to generic loads, each waited for).
    constexpr int kBatch = 4;
    auto count = [&](const uint32_t (&u)[kBatch], int i0) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        if (i0 + j * kThreads < n_cand && (u[j] & mask) == prefix)
          atomicAdd(&hs[((u[j] >> shift) & (nbins - 1)) * kCopies + copy], 1);
    };
    if (in_lds) {
      for (int i0 = tid; i0 < n_cand; i0 += kBatch * kThreads) {
        uint32_t u[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) u[j] = i0 + j * kThreads < n_cand ? cand[i0 + j * kThreads] : 0u;
        count(u, i0);
      }
    } else {
      for (int i0 = tid; i0 < n_cand; i0 += kBatch * kThreads) {
        uint32_t u[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) u[j] = i0 + j * kThreads < n_cand ? bits[i0 + j * kThreads] : 0u;
        count(u, i0);
      }
    }
    if (pass < 2) {   // the next pass's histogram; its last reader finished two barriers ago
      clear(hist[(pass + 1) & 1]);
    }
    __syncthreads();
    // Thread t owns bins hi = nbins-1-t*per down to hi-per+1; a scan in thread order counts the
    // candidates at or above each thread's lowest bin.  The thread where that count first
    // reaches `remaining` finds the bin holding the remaining-th largest.
    const int per = nbins / kThreads;
    const int hi = nbins - 1 - tid * per;
    int local = 0;
    for (int j = 0; j < per; ++j) local += bin_count(hs, hi - j);
    const int incl = block_incl_scan(local, tot[pass & 1]);
    if (incl >= remaining && incl - local < remaining) {
      int cum = incl - local;
      for (int j = 0; j < per; ++j) {
        const int c = bin_count(hs, hi - j);
        if (cum + c >= remaining) {
          sel_bin = hi - j;
          sel_rem = remaining - cum;
          sel_all = c == remaining - cum;   // the whole bin is taken: a later pass has nothing to split
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)sel_bin << shift;
    mask |= (uint32_t)(nbins - 1) << shift;
    remaining = sel_rem;
    // sel_* are rewritten one pass later, after that pass's two barriers
    if (sel_all) break;   // workgroup-uniform
  }
  // The candidates are compared on the bits the passes resolved (`mask`): when a pass finds
  // that every candidate of its threshold bin is taken (with scores spread over 22 bits, the
  // second pass's bin usually holds a single candidate), the remaining passes are skipped and
  // the whole bin counts as T.  The kept set is the same as with all three passes.
  const uint32_t T = prefix;
  const int ties = remaining;   // candidates equal to T (under mask) to take, lowest index first

  // Contiguous chunk per thread, in index order.  With the candidates in LDS, a chunk is a
  // multiple of four (16-byte aligned) and read once into registers with 16-byte reads: one
  // word at a time, a wavefront's lanes would hit LDS words a chunk apart, all in the same
  // few banks.
  if (in_lds) {
    const int per = ((n_cand + kThreads - 1) / kThreads + 3) & ~3;
    const int c0 = min(tid * per, n_cand), c1 = min(c0 + per, n_cand);
    // may read up to 3 words past the candidates: the allocation has 4 spare words
    auto group = [&](int i) { return *reinterpret_cast<const u32x4*>(&cand[i]); };
    int gt = 0, eq = 0;
    for (int i = c0; i < c1; i += 4) {
      const u32x4 x = group(i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = i + j < c1;
        gt += in && (x[j] & mask) > T;
        eq += in && (x[j] & mask) == T;
      }
    }
    const int eq_before = block_incl_scan(eq, tot[1]) - eq;   // tot's last reads preceded the selection barrier
    const int take_eq = min(max(ties - eq_before, 0), eq);
    const int sel = gt + take_eq;
    int pos = block_incl_scan(sel, tot[0]) - sel;
    int e = eq_before;
    for (int i = c0; i < c1; i += 4) {
      const u32x4 x = group(i);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t u = x[j] & mask;
        if (i + j < c1 && (u > T || (u == T && e++ < ties))) out[pos++] = i + j;
      }
    }
    write_window();
    return;
  }
  const int per = (n_cand + kThreads - 1) / kThreads;
  const int c0 = min(tid * per, n_cand), c1 = min(c0 + per, n_cand);
  int gt = 0, eq = 0;
  for (int i = c0; i < c1; ++i) {
    const uint32_t u = bits[i] & mask;
    gt += u > T;
    eq += u == T;
  }
  const int eq_before = block_incl_scan(eq, tot[1]) - eq;   // tot's last reads preceded the selection barrier
  const int take_eq = min(max(ties - eq_before, 0), eq);
  const int sel = gt + take_eq;
  int pos = block_incl_scan(sel, tot[0]) - sel;
  int e = eq_before;
  for (int i = c0; i < c1; ++i) {
    const uint32_t u = bits[i] & mask;
    if (u > T || (u == T && e++ < ties)) out[pos++] = i;
  }
  write_window();
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ cu_seqlens,
                                                        int total_tokens, int hkv, int alpha, int k_budget,
                                                        const int32_t* __restrict__ keep_offsets,
                                                        int32_t* __restrict__ keep_idx, int cand_cap) {
  extern __shared__ __attribute__((aligned(16))) uint32_t cand[];   // up to kLdsCap candidate bit patterns (+4 spare)
  // alternate passes: one histogram is cleared while the other is read
  __shared__ __attribute__((aligned(16))) int hist[2][2048 * kCopies];
  __shared__ int tot[2][kWaves];
  __shared__ int sel[3];

  const int g = blockIdx.x, s = blockIdx.y;
  const int base = cu_seqlens[s];
  const int n = cu_seqlens[s + 1] - base;
  if (n <= 0) return;
  const int k_eff = k_budget >= n ? n : k_budget;
  int32_t* out = keep_idx + (size_t)hkv * keep_offsets[s] + (size_t)g * k_eff;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(scores + (size_t)g * total_tokens + base);
  select_kept(bits, n, alpha, k_budget, out, SelectLds{cand, hist, tot, sel}, cand_cap);
}

// Selection fused with the compaction of the kept rows (the two calls above in one launch).
// `replicas` workgroups per (prompt, KV head) run the same selection, which gives each of them
// the whole kept list in LDS (in the histograms' space, free once the passes are done); replica
// 0 stores it as keep_idx, and replica r writes the head's blocks r, r + replicas, ... one per
// wavefront (the host launches one replica per block).  Each wavefront fetches the table entry
// of its first block before the selection, so the copy waits only for the source rows.  Needs
// k_eff <= kKeptCap.
template <int D>
__global__ __launch_bounds__(kThreads) void topk_compact_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ cu_seqlens, int total_tokens, int hkv, int alpha,
    int k_budget, const int32_t* __restrict__ keep_offsets, int32_t* __restrict__ keep_idx,
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src, uint16_t* __restrict__ k_pool,
    uint16_t* __restrict__ v_pool, int num_blocks, const int32_t* __restrict__ block_tables, int max_blocks,
    const int32_t* __restrict__ dst_slot_offset, int replicas, int cand_cap) {
  extern __shared__ __attribute__((aligned(16))) uint32_t cand[];
  __shared__ __attribute__((aligned(16))) int hist[2][2048 * kCopies];
  __shared__ int tot[2][kWaves];
  __shared__ int sel[3];

  const int r = blockIdx.x % replicas, g = blockIdx.x / replicas, s = blockIdx.y;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int base = cu_seqlens[s];
  const int n = cu_seqlens[s + 1] - base;
  const int ko = keep_offsets[s];
  const int off = dst_slot_offset ? dst_slot_offset[s] : 0;
  const int k_eff = k_budget >= n ? n : k_budget;
  if (n <= 0 || k_eff > kKeptCap) return;   // the host bounds k_eff by min(k_budget, max_seqlen)
  const int nblk = (off % kBlock + k_eff + kBlock - 1) / kBlock;   // blocks the kept rows touch
  const int step = replicas * kWaves;
  const int bi0 = r + replicas * w;
  const int tbl0 = off / kBlock + bi0;
  const int blk0 = bi0 < nblk && tbl0 < max_blocks ? block_tables[(size_t)s * max_blocks + tbl0] : -1;

  int32_t* kept = &hist[0][0];
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(scores + (size_t)g * total_tokens + base);
  select_kept(bits, n, alpha, k_budget, kept, SelectLds{cand, hist, tot, sel}, cand_cap);
  __syncthreads();

  if (r == 0) {
    int32_t* out = keep_idx + (size_t)hkv * ko + (size_t)g * k_eff;
    for (int t = tid; t < k_eff; t += kThreads) out[t] = kept[t];
  }
  for (int bi = bi0; bi < nblk; bi += step) {
    const int tbl_pos = off / kBlock + bi;
    if (tbl_pos >= max_blocks) break;
    const int blk = bi == bi0 ? blk0 : block_tables[(size_t)s * max_blocks + tbl_pos];
    if (blk < 0 || blk >= num_blocks) continue;
    const int t0 = tbl_pos * kBlock - off;           // rank written to slot 0 (may be negative)
    int srcrow[kBlock];
#pragma unroll
    for (int j = 0; j < kBlock; ++j) srcrow[j] = t0 + j >= 0 && t0 + j < k_eff ? kept[t0 + j] : -1;
    copy_kv_block<D>(k_src, v_src, base, hkv, g, srcrow, k_pool, v_pool, blk, lane);
  }
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" int kvs_topk_select(const float* scores, const int32_t* cu_seqlens, int num_seqs, int total_tokens,
                               int max_seqlen, int hkv, int alpha, int k_budget, const int32_t* keep_offsets,
                               int32_t* keep_idx, void* stream) {
  if (!scores || !cu_seqlens || !keep_offsets || !keep_idx) return fail(KVS_E_INVAL, "kvs_topk_select: NULL tensor");
  if (num_seqs < 0 || total_tokens < 0 || hkv <= 0 || max_seqlen < 0)
    return fail(KVS_E_INVAL, "kvs_topk_select: bad shape");
  if (alpha < 1 || k_budget < alpha)
    return fail(KVS_E_INVAL, "kvs_topk_select: need 1 <= alpha <= k_budget (alpha=%d k=%d)", alpha, k_budget);
  if (num_seqs == 0 || total_tokens == 0) return KVS_OK;
  const int cand_cap = min(max(max_seqlen, 1), kLdsCap);
  const size_t lds = ((size_t)cand_cap + 4) * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_kernel, dim3(hkv, num_seqs), dim3(kThreads), lds, as_stream(stream), scores, cu_seqlens,
                     total_tokens, hkv, alpha, k_budget, keep_offsets, keep_idx, cand_cap);
  return launch_status("kvs_topk_select");
}

extern "C" int kvs_topk_compact(const float* scores, const void* k_src, const void* v_src, const int32_t* cu_seqlens,
                                int num_seqs, int total_tokens, int max_seqlen, int hkv, int d, int alpha,
                                int k_budget, const int32_t* keep_offsets, int32_t* keep_idx, void* k_pool,
                                void* v_pool, int num_blocks, const int32_t* block_tables, int max_blocks,
                                const int32_t* dst_slot_offset, void* stream) {
  if (!scores || !k_src || !v_src || !cu_seqlens || !keep_offsets || !keep_idx || !k_pool || !v_pool || !block_tables)
    return fail(KVS_E_INVAL, "kvs_topk_compact: NULL tensor");
  if (num_seqs < 0 || total_tokens < 0 || hkv <= 0 || max_seqlen < 0 || (d != 64 && d != 128) || num_blocks <= 0 ||
      max_blocks <= 0)
    return fail(KVS_E_INVAL, "kvs_topk_compact: bad shape (num_seqs=%d hkv=%d d=%d)", num_seqs, hkv, d);
  if (alpha < 1 || k_budget < alpha)
    return fail(KVS_E_INVAL, "kvs_topk_compact: need 1 <= alpha <= k_budget (alpha=%d k=%d)", alpha, k_budget);
  if (num_seqs == 0 || total_tokens == 0 || max_seqlen == 0) return KVS_OK;
  const int max_keep = min(k_budget, max_seqlen);
  // One workgroup per (prompt, head, block), each repeating the selection: the copy then runs
  // on as many CUs as there are blocks, one round trip after the selection.  On the 8B layer
  // (8 heads, k = 400: 200 workgroups) 10.2 us against 11.4 for the two kernels; one workgroup
  // per 16, 8, 4 or 2 blocks took 12.5, 11.0, 10.5 and 10.2 us, the copy being bound by the
  // bytes each CU moves.  Wider launches would run the repeated selections one generation
  // after another, and candidates beyond the LDS would be re-read by every replica: there the
  // two kernels run instead.
  const int blocks = (max_keep + kBlock - 1) / kBlock + (dst_slot_offset ? 1 : 0);
  if (max_keep > kKeptCap || max_seqlen > kLdsCap || (long long)hkv * num_seqs * blocks > kFusedMaxWGs) {
    const int rc = kvs_topk_select(scores, cu_seqlens, num_seqs, total_tokens, max_seqlen, hkv, alpha, k_budget,
                                   keep_offsets, keep_idx, stream);
    if (rc != KVS_OK) return rc;
    return kvs_compact_paged(k_src, v_src, cu_seqlens, num_seqs, hkv, d, keep_idx, keep_offsets, max_keep, k_pool,
                             v_pool, num_blocks, block_tables, max_blocks, dst_slot_offset, stream);
  }
  const int replicas = blocks;
  const int cand_cap = min(max_seqlen, kLdsCap);
  const size_t lds = ((size_t)cand_cap + 4) * sizeof(uint32_t);
  const dim3 grid(hkv * replicas, num_seqs);
  auto* ks = static_cast<const uint16_t*>(k_src);
  auto* vs = static_cast<const uint16_t*>(v_src);
  auto* kp = static_cast<uint16_t*>(k_pool);
  auto* vp = static_cast<uint16_t*>(v_pool);
  if (d == 128)
    hipLaunchKernelGGL(topk_compact_kernel<128>, grid, dim3(kThreads), lds, as_stream(stream), scores, cu_seqlens,
                       total_tokens, hkv, alpha, k_budget, keep_offsets, keep_idx, ks, vs, kp, vp, num_blocks,
                       block_tables, max_blocks, dst_slot_offset, replicas, cand_cap);
  else
    hipLaunchKernelGGL(topk_compact_kernel<64>, grid, dim3(kThreads), lds, as_stream(stream), scores, cu_seqlens,
                       total_tokens, hkv, alpha, k_budget, keep_offsets, keep_idx, ks, vs, kp, vp, num_blocks,
                       block_tables, max_blocks, dst_slot_offset, replicas, cand_cap);
  return launch_status("kvs_topk_compact");
}
