// Decode-time scores and eviction in a compressed layer: the per-slot state after
// compaction, and the choice of the slot each KV head writes the new token to.
//
// [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM", Key techniques 1
// (step preparation): the layers after the third run a sliding-window strategy that replaces
// the KV entries with the lowest scores, under the layer's budget; Key techniques 2, last
// paragraph: PagedAttention shares FlashAttention's goal of computing the score S.
//
// Slot state of sequence b, KV head g, slot t (row stride slot_stride):
//   slot_scores  accumulated score (fp32, >= 0): the prefill S of the kept token, plus the
//                probability every decode row gave it, summed over the group's query heads
//                (the scored decode adds those);
//   slot_pos     the token's prompt-local position, -1 for an empty slot.
// While a cache has room the new token is appended; once it holds `cap` tokens each KV head
// replaces its lowest-score token among those older than the alpha most recent positions,
// ties going to the older position.  Scores are non-negative, so (score bits, position) as
// one 64-bit key orders like (score, position).
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void slot_init_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ keep_idx,
                                                             const int32_t* __restrict__ keep_offsets,
                                                             const int32_t* __restrict__ cu_seqlens, int total_tokens,
                                                             int hkv, int slot_stride, float* __restrict__ slot_scores,
                                                             int32_t* __restrict__ slot_pos) {
  const int g = blockIdx.x, s = blockIdx.y;
  const int base = cu_seqlens[s];
  const int n = cu_seqlens[s + 1] - base;
  const bool keep_all = keep_idx == nullptr;
  const int k_eff = keep_all ? n : keep_offsets[s + 1] - keep_offsets[s];
  const int32_t* keep = keep_all ? nullptr : keep_idx + (size_t)hkv * keep_offsets[s] + (size_t)g * k_eff;
  float* sc = slot_scores + ((size_t)s * hkv + g) * slot_stride;
  int32_t* ps = slot_pos + ((size_t)s * hkv + g) * slot_stride;
  for (int t = threadIdx.x; t < slot_stride; t += kThreads) {
    if (t < k_eff) {
      const int i = keep_all ? t : keep[t];
      sc[t] = scores[(size_t)g * total_tokens + base + i];
      ps[t] = i;
    } else {
      sc[t] = 0.f;
      ps[t] = -1;
    }
  }
}

__global__ __launch_bounds__(kThreads) void select_slot_kernel(float* __restrict__ slot_scores,
                                                               int32_t* __restrict__ slot_pos, int slot_stride,
                                                               const int32_t* __restrict__ n_filled, int hkv, int cap,
                                                               const int32_t* __restrict__ new_pos, int alpha,
                                                               int32_t* __restrict__ dst_slot) {
  __shared__ unsigned long long best;
  __shared__ int best_slot;
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  float* sc = slot_scores + ((size_t)b * hkv + g) * slot_stride;
  int32_t* ps = slot_pos + ((size_t)b * hkv + g) * slot_stride;
  const int n = n_filled[b];
  const int np = new_pos[b];
  int dst = n;                                    // room left: append
  if (n >= cap) {                                 // block-uniform
    if (tid == 0) {
      best = ~0ull;
      best_slot = -1;
    }
    __syncthreads();
    // Slots are read kPer per thread at a time, all loads of a round in flight together; with
    // cap <= kThreads * kPer (one round) the second pass reuses the registers.
    constexpr int kPer = 8;
    auto key_of = [&](int p, float v) {
      return (p >= 0 && p < np - alpha) ? (((unsigned long long)__float_as_uint(v) << 32) | (unsigned)p) : ~0ull;
    };
    unsigned long long keys[kPer];
    unsigned long long mine = ~0ull;
    for (int c0 = 0; c0 < cap; c0 += kThreads * kPer) {
      int p[kPer];
      float v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int t = c0 + j * kThreads + tid;
        p[j] = t < cap ? ps[t] : -1;
        v[j] = t < cap ? sc[t] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        keys[j] = key_of(p[j], v[j]);
        mine = keys[j] < mine ? keys[j] : mine;
      }
    }
    atomicMin(&best, mine);
    __syncthreads();
    if (cap <= kThreads * kPer) {                 // the registers hold the only round
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (keys[j] != ~0ull && keys[j] == best) best_slot = j * kThreads + tid;
    } else {
      for (int t = tid; t < cap; t += kThreads)   // positions are distinct: one slot matches
        if (key_of(ps[t], sc[t]) == best && best != ~0ull) best_slot = t;
    }
    __syncthreads();
    dst = best_slot;                              // -1 only if no slot may go (cap <= alpha: refused on the host)
  }
  if (tid == 0) {
    dst_slot[(size_t)b * hkv + g] = dst;
    if (dst >= 0) {
      sc[dst] = 0.f;
      ps[dst] = np;
    }
  }
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" int kvs_slot_init(const float* scores, const int32_t* keep_idx, const int32_t* keep_offsets,
                             const int32_t* cu_seqlens, int num_seqs, int total_tokens, int hkv, int slot_stride,
                             float* slot_scores, int32_t* slot_pos, void* stream) {
  if (!scores || !cu_seqlens || !slot_scores || !slot_pos) return fail(KVS_E_INVAL, "kvs_slot_init: NULL tensor");
  if (keep_idx && !keep_offsets) return fail(KVS_E_INVAL, "kvs_slot_init: keep_offsets required with keep_idx");
  if (num_seqs < 0 || total_tokens < 0 || hkv <= 0 || slot_stride <= 0)
    return fail(KVS_E_INVAL, "kvs_slot_init: bad shape");
  if (num_seqs == 0) return KVS_OK;
  hipLaunchKernelGGL(slot_init_kernel, dim3(hkv, num_seqs), dim3(kThreads), 0, as_stream(stream), scores, keep_idx,
                     keep_offsets, cu_seqlens, total_tokens, hkv, slot_stride, slot_scores, slot_pos);
  return launch_status("kvs_slot_init");
}

extern "C" int kvs_decode_select_slot(float* slot_scores, int32_t* slot_pos, int slot_stride, const int32_t* n_filled,
                                      int batch, int hkv, int cap, const int32_t* new_pos, int alpha,
                                      int32_t* dst_slot, void* stream) {
  if (!slot_scores || !slot_pos || !n_filled || !new_pos || !dst_slot)
    return fail(KVS_E_INVAL, "kvs_decode_select_slot: NULL tensor");
  if (batch < 0 || hkv <= 0 || cap <= 0 || cap > slot_stride || alpha < 0 || alpha >= cap)
    return fail(KVS_E_INVAL, "kvs_decode_select_slot: need 0 <= alpha < cap <= slot_stride (alpha=%d cap=%d stride=%d)",
                alpha, cap, slot_stride);
  if (batch == 0) return KVS_OK;
  hipLaunchKernelGGL(select_slot_kernel, dim3(hkv, batch), dim3(kThreads), 0, as_stream(stream), slot_scores,
                     slot_pos, slot_stride, n_filled, hkv, cap, new_pos, alpha, dst_slot);
  return launch_status("kvs_decode_select_slot");
}
