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
// ties going to the older position (slot_select.h).
#include "kvs_common.h"
#include "slot_select.h"

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

__global__ __launch_bounds__(kSelectThreads) void select_slot_kernel(float* __restrict__ slot_scores,
                                                                     int32_t* __restrict__ slot_pos, int slot_stride,
                                                                     const int32_t* __restrict__ n_filled, int hkv,
                                                                     int cap, const int32_t* __restrict__ new_pos,
                                                                     int alpha, int32_t* __restrict__ dst_slot) {
  const int g = blockIdx.x, b = blockIdx.y;
  select_slot_block(slot_scores + ((size_t)b * hkv + g) * slot_stride, slot_pos + ((size_t)b * hkv + g) * slot_stride,
                    n_filled[b], cap, new_pos[b], alpha, dst_slot + (size_t)b * hkv + g);
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
  hipLaunchKernelGGL(select_slot_kernel, dim3(hkv, batch), dim3(kSelectThreads), 0, as_stream(stream), slot_scores,
                     slot_pos, slot_stride, n_filled, hkv, cap, new_pos, alpha, dst_slot);
  return launch_status("kvs_decode_select_slot");
}
