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
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kLdsCap = 16384;   // candidates held in LDS (64 KB); longer prompts read L2 each pass
constexpr int kCopies = 4;       // copies of every histogram bin: lane l counts into copy l % 4

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

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ cu_seqlens,
                                                        int total_tokens, int hkv, int alpha, int k_budget,
                                                        const int32_t* __restrict__ keep_offsets,
                                                        int32_t* __restrict__ keep_idx) {
  extern __shared__ __attribute__((aligned(16))) uint32_t cand[];   // up to kLdsCap candidate bit patterns (+4 spare)
  // alternate passes: one histogram is cleared while the other is read
  __shared__ __attribute__((aligned(16))) int hist[2][2048 * kCopies];
  __shared__ int tot[2][kWaves];
  __shared__ int sel_bin, sel_rem, sel_all;

  const int g = blockIdx.x, s = blockIdx.y, tid = threadIdx.x;
  const int base = cu_seqlens[s];
  const int n = cu_seqlens[s + 1] - base;
  if (n <= 0) return;
  const int k_eff = k_budget >= n ? n : k_budget;
  int32_t* out = keep_idx + (size_t)hkv * keep_offsets[s] + (size_t)g * k_eff;
  if (k_budget >= n) {
    for (int i = tid; i < n; i += kThreads) out[i] = i;
    return;
  }
  const int a = alpha < n ? alpha : n;
  const int n_cand = n - a;
  const int kk = k_budget - a;   // slots filled by score (0 when the budget is the window)
  // the window follows the kk chosen candidates (its indices are all larger)
  for (int i = n_cand + tid; i < n; i += kThreads) out[kk + i - n_cand] = i;
  if (kk == 0) return;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(scores + (size_t)g * total_tokens + base);
  const bool in_lds = n_cand <= kLdsCap;   // block-uniform
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
  const size_t lds = ((size_t)min(max(max_seqlen, 1), kLdsCap) + 4) * sizeof(uint32_t);
  hipLaunchKernelGGL(topk_kernel, dim3(hkv, num_seqs), dim3(kThreads), lds, as_stream(stream), scores, cu_seqlens,
                     total_tokens, hkv, alpha, k_budget, keep_offsets, keep_idx);
  return launch_status("kvs_topk_select");
}
