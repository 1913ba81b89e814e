// Gather-compaction of kept K/V rows into 16-token blocks, the reverse gather of cached
// blocks into contiguous rows (a reused prefix), and the block copy of copy-on-write.
//
// [PAG] Ultralytics glossary, "PagedAttention", "How paging works": the cache is stored in
// fixed 16-token blocks anywhere in GPU memory and a per-request block table gives their
// order; the worked example writes token p to block table[p // 16], slot p % 16.
// [PAG] "Sharing blocks between sequences": a shared block is copied before it is written.
// [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM", Key techniques 1:
// the first three layers keep every token, the later layers only their budget.
//
// Pool layouts (bf16): K [num_blocks][hkv][16][d] (token rows), V [num_blocks][hkv][d][16]
// (each channel's 16 slots contiguous, the operand order the decode kernel's P.V product
// wants).  One wavefront fills one (destination block, head) pair (copy_kv_block: K as whole
// token rows with 16-byte lanes, V as two contiguous 32-byte channel runs per lane), so both
// sides stay coalesced with no LDS round trip.
#include "compact_block.h"
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kWavesPerWG = 4;

template <int D>
__global__ __launch_bounds__(kWavesPerWG * kWave) void compact_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
    const int32_t* __restrict__ cu_seqlens, int hkv, const int32_t* __restrict__ keep_idx,
    const int32_t* __restrict__ keep_offsets, uint16_t* __restrict__ k_pool,
    uint16_t* __restrict__ v_pool, int num_blocks, const int32_t* __restrict__ block_tables,
    int max_blocks, const int32_t* __restrict__ dst_slot_offset, int blocks_per_seq) {
  const int lane = threadIdx.x % kWave;
  const int unit = blockIdx.x * kWavesPerWG + threadIdx.x / kWave;   // (block index, head)
  const int s = blockIdx.y;
  if (unit >= blocks_per_seq * hkv) return;
  const int bi = unit / hkv;
  const int g = unit % hkv;

  // The prompt's metadata is read in one go; the block-table entry and the 16 source rows
  // then in a second; the K/V rows in a third; all loads of a round precede any store.
  const bool keep_all = keep_idx == nullptr;
  const int base = cu_seqlens[s], end = cu_seqlens[s + 1];
  const int ko0 = keep_all ? 0 : keep_offsets[s], ko1 = keep_all ? 0 : keep_offsets[s + 1];
  const int off = dst_slot_offset ? dst_slot_offset[s] : 0;
  const int n = end - base;
  const int k_eff = keep_all ? n : ko1 - ko0;
  const int tbl_pos = off / kBlock + bi;          // table entry this unit fills
  const int p0 = tbl_pos * kBlock;                 // slot position of its first slot
  if (k_eff <= 0 || p0 >= off + k_eff || tbl_pos >= max_blocks) return;
  const int32_t* keep = keep_all ? nullptr : keep_idx + (size_t)hkv * ko0 + (size_t)g * k_eff;
  const int t0 = p0 - off;                         // rank written to slot 0 (may be negative)
  // Source rows of the 16 slots (wave-uniform addresses); -1 marks a slot this block does not fill.
  int srcrow[kBlock];
#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    const int t = min(max(t0 + j, 0), k_eff - 1);
    srcrow[j] = keep_all ? t : keep[t];
  }
  const int blk = block_tables[(size_t)s * max_blocks + tbl_pos];
#pragma unroll
  for (int j = 0; j < kBlock; ++j)
    if (t0 + j < 0 || t0 + j >= k_eff) srcrow[j] = -1;
  if (blk < 0 || blk >= num_blocks) return;
  copy_kv_block<D>(k_src, v_src, base, hkv, g, srcrow, k_pool, v_pool, blk, lane);
}

// Gather: tokens 0..count-1 of a sequence read back through its block table into contiguous
// token-major rows (the inverse of a keep-all compaction).  One wavefront per (table entry,
// head): K rows move with 16-byte lanes; V comes channel-major, each lane reading the 16 slots
// of a channel pair (two 32-byte runs) and writing them back as 4-byte pieces of 16 token rows.
template <int D>
__global__ __launch_bounds__(kWavesPerWG * kWave) void gather_kernel(
    const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool, int num_blocks,
    const int32_t* __restrict__ block_tables, int max_blocks, int hkv, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ dst_start, uint16_t* __restrict__ k_dst, uint16_t* __restrict__ v_dst,
    int blocks_per_seq) {
  const int lane = threadIdx.x % kWave;
  const int unit = blockIdx.x * kWavesPerWG + threadIdx.x / kWave;
  const int s = blockIdx.y;
  if (unit >= blocks_per_seq * hkv) return;
  const int bi = unit / hkv, g = unit % hkv;
  const int cnt = counts[s];
  const int d0 = dst_start[s];
  if (bi * kBlock >= cnt || bi >= max_blocks) return;
  const int blk = block_tables[(size_t)s * max_blocks + bi];
  if (blk < 0 || blk >= num_blocks) return;
  const int valid = min(kBlock, cnt - bi * kBlock);   // slots of this block inside the count

  constexpr int kLanesPerRow = D * 2 / 16;
  constexpr int kRowsPerIter = kWave / kLanesPerRow;
  constexpr int kIters = kBlock / kRowsPerIter;
  const uint16_t* ksrc = k_pool + ((size_t)blk * hkv + g) * kBlock * D;
  {
    const int c = lane % kLanesPerRow;
    u32x4 val[kIters];
#pragma unroll
    for (int it = 0; it < kIters; ++it)
      val[it] = *reinterpret_cast<const u32x4*>(ksrc + (it * kRowsPerIter + lane / kLanesPerRow) * D + c * 8);
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int j = it * kRowsPerIter + lane / kLanesPerRow;
      if (j < valid)
        *reinterpret_cast<u32x4*>(k_dst + ((size_t)(d0 + bi * kBlock + j) * hkv + g) * D + c * 8) = val[it];
    }
  }
  constexpr int kPairs = D / 2;
  if (lane >= kPairs) return;
  const uint16_t* vsrc = v_pool + ((size_t)blk * hkv + g) * D * kBlock;
  const u32x4* c0 = reinterpret_cast<const u32x4*>(vsrc + (size_t)(2 * lane) * kBlock);
  const u32x4* c1 = reinterpret_cast<const u32x4*>(vsrc + (size_t)(2 * lane + 1) * kBlock);
  const u32x4 a0 = c0[0], a1 = c0[1], b0 = c1[0], b1 = c1[1];   // slots 0-7 and 8-15 of both channels
#pragma unroll
  for (int j = 0; j < kBlock; ++j) {
    if (j >= valid) break;
    const uint32_t wa = j < 8 ? a0[j / 2] : a1[(j - 8) / 2];
    const uint32_t wb = j < 8 ? b0[j / 2] : b1[(j - 8) / 2];
    const uint32_t lo = (j % 2 == 0) ? (wa & 0xffffu) : (wa >> 16);   // channel 2*lane, slot j
    const uint32_t hi = (j % 2 == 0) ? (wb & 0xffffu) : (wb >> 16);   // channel 2*lane + 1
    *reinterpret_cast<uint32_t*>(v_dst + ((size_t)(d0 + bi * kBlock + j) * hkv + g) * D + 2 * lane) = lo | (hi << 16);
  }
}

// One workgroup copies one (src, dst) block pair in both pools.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint16_t* __restrict__ k_pool,
                                                          uint16_t* __restrict__ v_pool, int num_blocks,
                                                          size_t block_elems,
                                                          const int32_t* __restrict__ pairs) {
  const int src = pairs[2 * blockIdx.x];
  const int dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const size_t n16 = block_elems / 8;   // 16-byte chunks per block
  const u32x4* ks = reinterpret_cast<const u32x4*>(k_pool + (size_t)src * block_elems);
  u32x4* kd = reinterpret_cast<u32x4*>(k_pool + (size_t)dst * block_elems);
  const u32x4* vs = reinterpret_cast<const u32x4*>(v_pool + (size_t)src * block_elems);
  u32x4* vd = reinterpret_cast<u32x4*>(v_pool + (size_t)dst * block_elems);
  for (size_t i = threadIdx.x; i < n16; i += blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" int kvs_compact_paged(const void* k_src, const void* v_src, const int32_t* cu_seqlens,
                                 int num_seqs, int hkv, int d, const int32_t* keep_idx,
                                 const int32_t* keep_offsets, int max_keep, void* k_pool, void* v_pool,
                                 int num_blocks, const int32_t* block_tables, int max_blocks,
                                 const int32_t* dst_slot_offset, void* stream) {
  if (!k_src || !v_src || !cu_seqlens || !k_pool || !v_pool || !block_tables)
    return fail(KVS_E_INVAL, "kvs_compact_paged: NULL tensor");
  if (keep_idx && !keep_offsets) return fail(KVS_E_INVAL, "kvs_compact_paged: keep_offsets required with keep_idx");
  if (num_seqs < 0 || hkv <= 0 || (d != 64 && d != 128) || max_keep < 0 || num_blocks <= 0 || max_blocks <= 0)
    return fail(KVS_E_INVAL, "kvs_compact_paged: bad shape (num_seqs=%d hkv=%d d=%d max_keep=%d)", num_seqs, hkv,
                d, max_keep);
  if (num_seqs == 0 || max_keep == 0) return KVS_OK;
  // A misaligned destination offset makes the kept rows straddle one extra block.
  const int blocks_per_seq = (max_keep + kBlock - 1) / kBlock + (dst_slot_offset ? 1 : 0);
  const int units = blocks_per_seq * hkv;
  dim3 grid((units + kWavesPerWG - 1) / kWavesPerWG, num_seqs);
  dim3 block(kWavesPerWG * kWave);
  auto* ks = static_cast<const uint16_t*>(k_src);
  auto* vs = static_cast<const uint16_t*>(v_src);
  auto* kp = static_cast<uint16_t*>(k_pool);
  auto* vp = static_cast<uint16_t*>(v_pool);
  if (d == 128)
    hipLaunchKernelGGL(compact_kernel<128>, grid, block, 0, as_stream(stream), ks, vs, cu_seqlens, hkv, keep_idx,
                       keep_offsets, kp, vp, num_blocks, block_tables, max_blocks, dst_slot_offset, blocks_per_seq);
  else
    hipLaunchKernelGGL(compact_kernel<64>, grid, block, 0, as_stream(stream), ks, vs, cu_seqlens, hkv, keep_idx,
                       keep_offsets, kp, vp, num_blocks, block_tables, max_blocks, dst_slot_offset, blocks_per_seq);
  return launch_status("kvs_compact_paged");
}

extern "C" int kvs_copy_blocks(void* k_pool, void* v_pool, int num_blocks, int hkv, int d,
                               const int32_t* src_dst_pairs, int n_pairs, void* stream) {
  if (!k_pool || !v_pool || (n_pairs > 0 && !src_dst_pairs))
    return fail(KVS_E_INVAL, "kvs_copy_blocks: NULL tensor");
  if (num_blocks <= 0 || hkv <= 0 || (d != 64 && d != 128) || n_pairs < 0)
    return fail(KVS_E_INVAL, "kvs_copy_blocks: bad shape");
  if (n_pairs == 0) return KVS_OK;
  const size_t block_elems = (size_t)hkv * kBlock * d;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs), dim3(256), 0, as_stream(stream),
                     static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), num_blocks, block_elems,
                     src_dst_pairs);
  return launch_status("kvs_copy_blocks");
}

extern "C" int kvs_gather_paged(const void* k_pool, const void* v_pool, int num_blocks, const int32_t* block_tables,
                                int max_blocks, int num_seqs, int hkv, int d, const int32_t* counts,
                                const int32_t* dst_start, int max_count, void* k_dst, void* v_dst, void* stream) {
  if (!k_pool || !v_pool || !block_tables || !counts || !dst_start || !k_dst || !v_dst)
    return fail(KVS_E_INVAL, "kvs_gather_paged: NULL tensor");
  if (num_seqs < 0 || hkv <= 0 || (d != 64 && d != 128) || max_count < 0 || num_blocks <= 0 || max_blocks <= 0)
    return fail(KVS_E_INVAL, "kvs_gather_paged: bad shape (num_seqs=%d hkv=%d d=%d)", num_seqs, hkv, d);
  if (num_seqs == 0 || max_count == 0) return KVS_OK;
  const int blocks_per_seq = (max_count + kBlock - 1) / kBlock;
  dim3 grid((blocks_per_seq * hkv + kWavesPerWG - 1) / kWavesPerWG, num_seqs);
  auto* kp = static_cast<const uint16_t*>(k_pool);
  auto* vp = static_cast<const uint16_t*>(v_pool);
  auto* kd = static_cast<uint16_t*>(k_dst);
  auto* vd = static_cast<uint16_t*>(v_dst);
  if (d == 128)
    hipLaunchKernelGGL(gather_kernel<128>, grid, dim3(kWavesPerWG * kWave), 0, as_stream(stream), kp, vp, num_blocks,
                       block_tables, max_blocks, hkv, counts, dst_start, kd, vd, blocks_per_seq);
  else
    hipLaunchKernelGGL(gather_kernel<64>, grid, dim3(kWavesPerWG * kWave), 0, as_stream(stream), kp, vp, num_blocks,
                       block_tables, max_blocks, hkv, counts, dst_start, kd, vd, blocks_per_seq);
  return launch_status("kvs_gather_paged");
}
