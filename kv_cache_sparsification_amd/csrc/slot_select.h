// Choice of the slot a KV head's next token goes to, by one 256-thread workgroup (shared by
// kvs_decode_select_slot and the scored decode that also prepares the next step).
//
// [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM", Key techniques 1
// (step preparation): once a compressed layer's cache is at its budget, the entry with the
// lowest score is replaced.  With n live slots of capacity cap: n < cap appends at slot n;
// otherwise the slot with the lowest score among tokens older than the alpha most recent
// positions (< np - alpha), ties to the older position.  Scores are non-negative, so (score
// bits, position) as one 64-bit key orders like (score, position).  The chosen slot's score
// becomes 0 and its position np; thread 0 stores the slot (-1 if none may go) to *dst_out.
// Every thread of the workgroup must call it (it synchronises the workgroup).
#pragma once

#include "kvs_common.h"

namespace kvs {

constexpr int kSelectThreads = 256;

// (score bits, position) of a slot that may be replaced, or the largest key if it may not.
__device__ __forceinline__ unsigned long long slot_key(int p, float v, int np, int alpha) {
  return (p >= 0 && p < np - alpha) ? (((unsigned long long)__float_as_uint(v) << 32) | (unsigned)p) : ~0ull;
}

__device__ __forceinline__ void select_slot_block(float* __restrict__ sc, int32_t* __restrict__ ps, int n, int cap,
                                                  int np, int alpha, int32_t* __restrict__ dst_out) {
  __shared__ unsigned long long best;
  __shared__ int best_slot;
  const int tid = threadIdx.x;
  int dst = n;                                    // room left: append
  if (n >= cap) {                                 // block-uniform
    if (tid == 0) {
      best = ~0ull;
      best_slot = -1;
    }
    __syncthreads();
    // Slots are read kPer per thread at a time, all loads of a round in flight together; with
    // cap <= kSelectThreads * kPer (one round) the second pass reuses the registers.
    constexpr int kPer = 8;
    auto key_of = [&](int p, float v) { return slot_key(p, v, np, alpha); };
    unsigned long long keys[kPer];
    unsigned long long mine = ~0ull;
    for (int c0 = 0; c0 < cap; c0 += kSelectThreads * kPer) {
      int p[kPer];
      float v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int t = c0 + j * kSelectThreads + tid;
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
    if (cap <= kSelectThreads * kPer) {           // the registers hold the only round
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (keys[j] != ~0ull && keys[j] == best) best_slot = j * kSelectThreads + tid;
    } else {
      for (int t = tid; t < cap; t += kSelectThreads)   // positions are distinct: one slot matches
        if (key_of(ps[t], sc[t]) == best && best != ~0ull) best_slot = t;
    }
    __syncthreads();
    dst = best_slot;                              // -1 only if no slot may go (cap <= alpha: refused on the host)
  }
  if (tid == 0) {
    *dst_out = dst;
    if (dst >= 0) {
      sc[dst] = 0.f;
      ps[dst] = np;
    }
  }
}

// The same choice from values the caller already holds in registers: pos[j] and val[j] are the
// position and score of slot tid + kSelectThreads * j, for every slot below cap (the caller's K
// slots per thread cover cap).  Every thread of the workgroup must call it.
template <int K>
__device__ __forceinline__ void select_slot_regs(const int (&pos)[K], const float (&val)[K], float* __restrict__ sc,
                                                 int32_t* __restrict__ ps, int n, int cap, int np, int alpha,
                                                 int32_t* __restrict__ dst_out) {
  __shared__ unsigned long long best;
  __shared__ int best_slot;
  const int tid = threadIdx.x;
  int dst = n;                                    // room left: append
  if (n >= cap) {                                 // block-uniform
    if (tid == 0) {
      best = ~0ull;
      best_slot = -1;
    }
    __syncthreads();
    unsigned long long keys[K];
    unsigned long long mine = ~0ull;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      keys[j] = tid + kSelectThreads * j < cap ? slot_key(pos[j], val[j], np, alpha) : ~0ull;
      mine = keys[j] < mine ? keys[j] : mine;
    }
    atomicMin(&best, mine);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (keys[j] != ~0ull && keys[j] == best) best_slot = j * kSelectThreads + tid;
    __syncthreads();
    dst = best_slot;
  }
  if (tid == 0) {
    *dst_out = dst;
    if (dst >= 0) {
      sc[dst] = 0.f;
      ps[dst] = np;
    }
  }
}

}  // namespace kvs
