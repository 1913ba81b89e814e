// One wavefront's copy of up to 16 kept rows of one KV head into one 16-token cache block
// (shared by the compaction kernel and the fused selection-and-compaction kernel).
//
// [PAG] Ultralytics glossary, "PagedAttention", "How paging works": token p of a sequence
// lives in block table[p / 16], slot p % 16.  Pool layouts (bf16): K [num_blocks][hkv][16][d]
// (token rows), V [num_blocks][hkv][d][16] (each channel's 16 slots contiguous).
//
// srcrow[j] is the source row (prompt-local) of slot j, or -1 for a slot the block does not
// fill; every lane holds the same 16 values.  K moves as whole token rows with 16-byte lanes;
// for V each lane owns a pair of channels, reads them for all 16 slots (every read instruction
// covers one contiguous source row) and writes two contiguous 32-byte channel runs.  All loads
// of a side precede its stores.
#pragma once

#include "kvs_common.h"

namespace kvs {

template <int D>
__device__ __forceinline__ void copy_kv_block(const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
                                              int base, int hkv, int g, const int (&srcrow)[kBlock],
                                              uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool, int blk,
                                              int lane) {
  bool full = true;
#pragma unroll
  for (int j = 0; j < kBlock; ++j) full = full && srcrow[j] >= 0;

  // ---- K: row-major slots, 16-byte lanes
  constexpr int kLanesPerRow = D * 2 / 16;         // 16 (d=128) or 8 (d=64)
  constexpr int kRowsPerIter = kWave / kLanesPerRow;
  constexpr int kIters = kBlock / kRowsPerIter;
  uint16_t* kdst = k_pool + ((size_t)blk * hkv + g) * kBlock * D;
  {
    const int c = lane % kLanesPerRow;
    u32x4 val[kIters];
    int dst_row[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int j = it * kRowsPerIter + lane / kLanesPerRow;
      int src = srcrow[0];
#pragma unroll
      for (int jj = 1; jj < kBlock; ++jj) src = j == jj ? srcrow[jj] : src;   // select, no dynamic indexing
      dst_row[it] = src >= 0 ? j : -1;
      val[it] = u32x4{0u, 0u, 0u, 0u};
      if (src >= 0) val[it] = *reinterpret_cast<const u32x4*>(k_src + ((size_t)(base + src) * hkv + g) * D + c * 8);
    }
#pragma unroll
    for (int it = 0; it < kIters; ++it)
      if (dst_row[it] >= 0) *reinterpret_cast<u32x4*>(kdst + dst_row[it] * D + c * 8) = val[it];
  }

  // ---- V: channel-major slots; lane owns channels 2*lane and 2*lane + 1
  constexpr int kPairs = D / 2;
  if (lane >= kPairs) return;
  uint16_t* vdst = v_pool + ((size_t)blk * hkv + g) * D * kBlock;
  if (full) {
    uint32_t pair[kBlock];
#pragma unroll
    for (int j = 0; j < kBlock; ++j)
      pair[j] = *reinterpret_cast<const uint32_t*>(v_src + ((size_t)(base + srcrow[j]) * hkv + g) * D + 2 * lane);
    u32x4 lo[2], hi[2];   // channel 2*lane (low halves) and 2*lane + 1 (high halves), 16 slots each
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      // slot 2q in the low half-word, slot 2q + 1 in the high one
      lo[q / 4][q % 4] = (pair[2 * q] & 0xffffu) | (pair[2 * q + 1] << 16);
      hi[q / 4][q % 4] = (pair[2 * q] >> 16) | (pair[2 * q + 1] & 0xffff0000u);
    }
    u32x4* d0 = reinterpret_cast<u32x4*>(vdst + (size_t)(2 * lane) * kBlock);
    u32x4* d1 = reinterpret_cast<u32x4*>(vdst + (size_t)(2 * lane + 1) * kBlock);
    d0[0] = lo[0]; d0[1] = lo[1];
    d1[0] = hi[0]; d1[1] = hi[1];
  } else {
#pragma unroll
    for (int j = 0; j < kBlock; ++j) {
      const int src = srcrow[j];
      if (src < 0) continue;
      const uint32_t x = *reinterpret_cast<const uint32_t*>(v_src + ((size_t)(base + src) * hkv + g) * D + 2 * lane);
      vdst[(size_t)(2 * lane) * kBlock + j] = (uint16_t)(x & 0xffffu);
      vdst[(size_t)(2 * lane + 1) * kBlock + j] = (uint16_t)(x >> 16);
    }
  }
}

}  // namespace kvs
