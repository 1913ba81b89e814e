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
// order like unsigned integers: four 8-bit radix passes find the threshold value T (the
// (k-a)-th largest) and how many copies of T are still needed; a final in-order pass keeps
// every score above T plus the first `ties` indices equal to T, and writes the kept
// indices through ballot-based block prefix sums.  No sort, no device-wide traffic.
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / kWave;

// Exclusive block-wide prefix count of `flag`; returns (prefix, total).
__device__ __forceinline__ int2 block_count(bool flag, int* wave_tot) {
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  const uint64_t m = __ballot(flag);
  const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[w] = __popcll(m);
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int t = wave_tot[i];
    before += i < w ? t : 0;
    total += t;
  }
  __syncthreads();   // wave_tot is reused by the next call
  return make_int2(before + in_wave, total);
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                        const int32_t* __restrict__ cu_seqlens,
                                                        int total_tokens, int hkv, int alpha, int k_budget,
                                                        const int32_t* __restrict__ keep_offsets,
                                                        int32_t* __restrict__ keep_idx) {
  __shared__ int hist[256];
  __shared__ int wave_tot[kWaves];
  __shared__ int sel_digit, sel_remaining;

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
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(scores + (size_t)g * total_tokens + base);

  uint32_t prefix = 0, mask = 0;
  int remaining = kk;
  if (kk > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n_cand; i += kThreads) {
        const uint32_t u = bits[i];
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 0xffu], 1);
      }
      __syncthreads();
      // Thread t < 256 looks at digit b = 255 - t; an inclusive scan from the top gives the
      // number of candidates with digit >= b.  The selected digit is where that count first
      // reaches `remaining`.  Threads >= 256 take part with a zero count.
      {
        const int lane = tid % kWave, w = tid / kWave;
        const int x = tid < 256 ? hist[255 - tid] : 0;
        int incl = x;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const int y = __shfl_up(incl, o, kWave);
          if (lane >= o) incl += y;
        }
        if (lane == kWave - 1) wave_tot[w] = incl;
        __syncthreads();
        for (int q = 0; q < w; ++q) incl += wave_tot[q];
        if (tid < 256 && incl >= remaining && incl - x < remaining) {
          sel_digit = 255 - tid;
          sel_remaining = remaining - (incl - x);
        }
      }
      __syncthreads();
      prefix |= (uint32_t)sel_digit << shift;
      mask |= 0xffu << shift;
      remaining = sel_remaining;
      __syncthreads();   // sel_* and hist are rewritten next pass
    }
  }
  const uint32_t T = prefix;
  const int ties = remaining;   // copies of T still to take, lowest index first

  int carry_eq = 0, carry_out = 0;
  for (int c0 = 0; c0 < n; c0 += kThreads) {
    const int i = c0 + tid;
    const bool cand = i < n_cand;
    const uint32_t u = cand ? bits[i] : 0u;
    const bool is_eq = kk > 0 && cand && u == T;
    const int2 eq = block_count(is_eq, wave_tot);
    const bool sel = (kk > 0 && cand && (u > T || (is_eq && carry_eq + eq.x < ties))) || (i >= n_cand && i < n);
    const int2 pos = block_count(sel, wave_tot);
    if (sel) out[carry_out + pos.x] = i;
    carry_eq += eq.y;
    carry_out += pos.y;
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
  hipLaunchKernelGGL(topk_kernel, dim3(hkv, num_seqs), dim3(kThreads), 0, as_stream(stream), scores, cu_seqlens,
                     total_tokens, hkv, alpha, k_budget, keep_offsets, keep_idx);
  return launch_status("kvs_topk_select");
}
