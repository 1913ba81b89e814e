// Gather-compaction of kept K/V rows into 16-token blocks of an 8-bit (E4M3) cache, and the
// block copy of copy-on-write for such a cache.
//
// [PAG] Ultralytics glossary, "PagedAttention", "How paging works" (token p goes to block
// table[p // 16], slot p % 16) and "Related techniques" (an FP8 cache stores keys and values
// at 8 bits, about half the bytes of a 16-bit one).  [KVS] Novita AI, "How KV Sparsity
// Achieves 1.5x Acceleration for vLLM", Key techniques 1: the later layers keep only their
// budget.
//
// Quantization: one fp32 scale per (token, KV head) row, scale = amax/448, codes =
// E4M3(x * (448/amax)) rounded to nearest even; a row whose amax is below 2^-112 is stored as
// scale 0 and codes 0.
//
// Pool layouts: K codes [num_blocks][hkv][16][d] bytes (token rows), V codes
// [num_blocks][hkv][d][16] bytes (each channel's 16 slots contiguous, as the decode kernel's
// P.V product wants them), scales [num_blocks][hkv][16] fp32 for K and for V.  One wavefront
// fills one (destination block, head) pair.  Both K and V are read as whole source rows with
// 16-byte lanes (a row's amax is a reduction over the lanes that hold it); K codes go straight
// out as 8-byte row pieces, V codes take a trip through the wavefront's 2 KiB of LDS to turn
// token rows into channel runs of 16 bytes.
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kWavesPerWG = 4;

// Maximum over the N lanes (N = 8 or 16) that share lane / N, with DPP lane moves inside the
// 16-lane rows instead of LDS permutes: the quad swaps (lane ^ 1, lane ^ 2) give each quad's
// maximum, the half-row mirror (lane i <- 7 - i) each 8 lanes', the row mirror (i <- 15 - i)
// each row's.  The operands are non-negative and every source lane is inside the row.
template <int kCtrl>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
  static_assert(N == 8 || N == 16, "row groups of 8 or 16 lanes");
  v = fmaxf(v, dpp_move<0xB1>(v));               // quad_perm [1, 0, 3, 2]
  v = fmaxf(v, dpp_move<0x4E>(v));               // quad_perm [2, 3, 0, 1]
  v = fmaxf(v, dpp_move<0x141>(v));              // row_half_mirror
  if constexpr (N == 16) v = fmaxf(v, dpp_move<0x140>(v));   // row_mirror
  return v;
}

template <int D>
__global__ __launch_bounds__(kWavesPerWG * kWave) void compact_fp8_kernel(
    const uint16_t* __restrict__ k_src, const uint16_t* __restrict__ v_src,
    const int32_t* __restrict__ cu_seqlens, int hkv, const int32_t* __restrict__ keep_idx,
    const int32_t* __restrict__ keep_offsets, uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
    float* __restrict__ k_scale, float* __restrict__ v_scale, int num_blocks,
    const int32_t* __restrict__ block_tables, int max_blocks, const int32_t* __restrict__ dst_slot_offset,
    int blocks_per_seq) {
  constexpr int kLanesPerRow = D * 2 / 16;         // 16-byte lanes per bf16 row: 16 (d=128) or 8 (d=64)
  constexpr int kRowsPerIter = kWave / kLanesPerRow;
  constexpr int kIters = kBlock / kRowsPerIter;
  __shared__ __align__(16) uint8_t vcodes[kWavesPerWG][kBlock * D];   // one wavefront's V codes, token rows

  const int lane = threadIdx.x % kWave;
  const int wv = threadIdx.x / kWave;
  const int unit = blockIdx.x * kWavesPerWG + wv;   // (block index, head)
  const int s = blockIdx.y;
  if (unit >= blocks_per_seq * hkv) return;
  const int bi = unit / hkv;
  const int g = unit % hkv;

  const bool keep_all = keep_idx == nullptr;
  const int base = cu_seqlens[s], end = cu_seqlens[s + 1];
  const int ko0 = keep_all ? 0 : keep_offsets[s], ko1 = keep_all ? 0 : keep_offsets[s + 1];
  const int off = dst_slot_offset ? dst_slot_offset[s] : 0;
  const int n = end - base;
  const int k_eff = keep_all ? n : ko1 - ko0;
  const int tbl_pos = off / kBlock + bi;
  const int p0 = tbl_pos * kBlock;
  if (k_eff <= 0 || p0 >= off + k_eff || tbl_pos >= max_blocks) return;
  const int32_t* keep = keep_all ? nullptr : keep_idx + (size_t)hkv * ko0 + (size_t)g * k_eff;
  const int t0 = p0 - off;                         // rank written to slot 0 (may be negative)
  const bool full = t0 >= 0 && t0 + kBlock <= k_eff;
  int srcrow[kBlock];                              // -1: slot not filled by this call
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

  const int c = lane % kLanesPerRow;               // 16-byte chunk of the row: channels 8c .. 8c+7
  u32x4 kv[kIters], vv[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int j = it * kRowsPerIter + lane / kLanesPerRow;
    int src = srcrow[0];
#pragma unroll
    for (int jj = 1; jj < kBlock; ++jj) src = j == jj ? srcrow[jj] : src;
    kv[it] = u32x4{0u, 0u, 0u, 0u};
    vv[it] = u32x4{0u, 0u, 0u, 0u};
    if (src >= 0) {
      const size_t row = ((size_t)(base + src) * hkv + g) * D + c * 8;
      kv[it] = *reinterpret_cast<const u32x4*>(k_src + row);
      vv[it] = *reinterpret_cast<const u32x4*>(v_src + row);
    }
  }

  const size_t bh = (size_t)blk * hkv + g;
  uint8_t* kdst = k_pool + bh * kBlock * D;
  float* ksc = k_scale + bh * kBlock;
  float* vsc = v_scale + bh * kBlock;
  uint8_t* lds = vcodes[wv];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int j = it * kRowsPerIter + lane / kLanesPerRow;
    const bool valid = t0 + j >= 0 && t0 + j < k_eff;
    float sk, rk, sv, rv;
    e4m3_row_params(group_max<kLanesPerRow>(absmax_bf16x8(kv[it])), sk, rk);
    e4m3_row_params(group_max<kLanesPerRow>(absmax_bf16x8(vv[it])), sv, rv);
    const u32x2 kc = e4m3x8_from_bf16(kv[it], rk);
    const u32x2 vc = e4m3x8_from_bf16(vv[it], rv);
    if (valid) {
      *reinterpret_cast<u32x2*>(kdst + j * D + c * 8) = kc;
      if (c == 0) {
        ksc[j] = sk;
        vsc[j] = sv;
      }
    }
    *reinterpret_cast<u32x2*>(lds + j * D + c * 8) = vc;
  }
  // LDS reads of a wavefront follow its LDS writes in order; the barrier keeps the compiler
  // from moving them across.
  __builtin_amdgcn_wave_barrier();

  // ---- V: lane owns channels 2*lane and 2*lane + 1; gather their 16 slots from the rows.
  constexpr int kPairs = D / 2;
  if (lane >= kPairs) return;
  uint32_t lo[4], hi[4];   // channel 2*lane (lo) and 2*lane + 1 (hi), slots 4q .. 4q+3 in word q
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = *reinterpret_cast<const uint16_t*>(lds + (4 * q + i) * D + 2 * lane);
    // x[i] = (code of channel 2*lane + 1) << 8 | (code of channel 2*lane), slot 4q + i
    const uint32_t t01 = __builtin_amdgcn_perm(x[1], x[0], 0x05010400u);   // c0 s0, c0 s1, c1 s0, c1 s1
    const uint32_t t23 = __builtin_amdgcn_perm(x[3], x[2], 0x05010400u);
    lo[q] = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    hi[q] = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
  }
  uint8_t* vdst = v_pool + bh * D * kBlock;
  if (full) {
    *reinterpret_cast<u32x4*>(vdst + (size_t)(2 * lane) * kBlock) = u32x4{lo[0], lo[1], lo[2], lo[3]};
    *reinterpret_cast<u32x4*>(vdst + (size_t)(2 * lane + 1) * kBlock) = u32x4{hi[0], hi[1], hi[2], hi[3]};
  } else {
#pragma unroll
    for (int j = 0; j < kBlock; ++j) {
      if (t0 + j < 0 || t0 + j >= k_eff) continue;
      vdst[(size_t)(2 * lane) * kBlock + j] = (uint8_t)(lo[j / 4] >> (8 * (j % 4)));
      vdst[(size_t)(2 * lane + 1) * kBlock + j] = (uint8_t)(hi[j / 4] >> (8 * (j % 4)));
    }
  }
}

// One workgroup copies one (src, dst) block pair: the code blocks and the scale rows.
__global__ __launch_bounds__(256) void copy_blocks_fp8_kernel(uint8_t* __restrict__ k_pool,
                                                              uint8_t* __restrict__ v_pool,
                                                              float* __restrict__ k_scale,
                                                              float* __restrict__ v_scale, int num_blocks,
                                                              size_t block_bytes, int scales_per_block,
                                                              const int32_t* __restrict__ pairs) {
  const int src = pairs[2 * blockIdx.x];
  const int dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  const size_t n16 = block_bytes / 16;
  const u32x4* ks = reinterpret_cast<const u32x4*>(k_pool + (size_t)src * block_bytes);
  u32x4* kd = reinterpret_cast<u32x4*>(k_pool + (size_t)dst * block_bytes);
  const u32x4* vs = reinterpret_cast<const u32x4*>(v_pool + (size_t)src * block_bytes);
  u32x4* vd = reinterpret_cast<u32x4*>(v_pool + (size_t)dst * block_bytes);
  for (size_t i = threadIdx.x; i < n16; i += blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
  for (int i = threadIdx.x; i < scales_per_block; i += blockDim.x) {
    k_scale[(size_t)dst * scales_per_block + i] = k_scale[(size_t)src * scales_per_block + i];
    v_scale[(size_t)dst * scales_per_block + i] = v_scale[(size_t)src * scales_per_block + i];
  }
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" int kvs_compact_paged_fp8(const void* k_src, const void* v_src, const int32_t* cu_seqlens, int num_seqs,
                                     int hkv, int d, const int32_t* keep_idx, const int32_t* keep_offsets,
                                     int max_keep, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                     int num_blocks, const int32_t* block_tables, int max_blocks,
                                     const int32_t* dst_slot_offset, void* stream) {
  if (!k_src || !v_src || !cu_seqlens || !k_pool || !v_pool || !k_scale || !v_scale || !block_tables)
    return fail(KVS_E_INVAL, "kvs_compact_paged_fp8: NULL tensor");
  if (keep_idx && !keep_offsets)
    return fail(KVS_E_INVAL, "kvs_compact_paged_fp8: keep_offsets required with keep_idx");
  if (num_seqs < 0 || hkv <= 0 || (d != 64 && d != 128) || max_keep < 0 || num_blocks <= 0 || max_blocks <= 0)
    return fail(KVS_E_INVAL, "kvs_compact_paged_fp8: bad shape (num_seqs=%d hkv=%d d=%d max_keep=%d)", num_seqs,
                hkv, d, max_keep);
  if (num_seqs == 0 || max_keep == 0) return KVS_OK;
  const int blocks_per_seq = (max_keep + kBlock - 1) / kBlock + (dst_slot_offset ? 1 : 0);
  const int units = blocks_per_seq * hkv;
  dim3 grid((units + kWavesPerWG - 1) / kWavesPerWG, num_seqs);
  dim3 block(kWavesPerWG * kWave);
  auto* ks = static_cast<const uint16_t*>(k_src);
  auto* vs = static_cast<const uint16_t*>(v_src);
  auto* kp = static_cast<uint8_t*>(k_pool);
  auto* vp = static_cast<uint8_t*>(v_pool);
  if (d == 128)
    hipLaunchKernelGGL(compact_fp8_kernel<128>, grid, block, 0, as_stream(stream), ks, vs, cu_seqlens, hkv, keep_idx,
                       keep_offsets, kp, vp, k_scale, v_scale, num_blocks, block_tables, max_blocks, dst_slot_offset,
                       blocks_per_seq);
  else
    hipLaunchKernelGGL(compact_fp8_kernel<64>, grid, block, 0, as_stream(stream), ks, vs, cu_seqlens, hkv, keep_idx,
                       keep_offsets, kp, vp, k_scale, v_scale, num_blocks, block_tables, max_blocks, dst_slot_offset,
                       blocks_per_seq);
  return launch_status("kvs_compact_paged_fp8");
}

extern "C" int kvs_copy_blocks_fp8(void* k_pool, void* v_pool, float* k_scale, float* v_scale, int num_blocks, int hkv,
                                   int d, const int32_t* src_dst_pairs, int n_pairs, void* stream) {
  if (!k_pool || !v_pool || !k_scale || !v_scale || (n_pairs > 0 && !src_dst_pairs))
    return fail(KVS_E_INVAL, "kvs_copy_blocks_fp8: NULL tensor");
  if (num_blocks <= 0 || hkv <= 0 || (d != 64 && d != 128) || n_pairs < 0)
    return fail(KVS_E_INVAL, "kvs_copy_blocks_fp8: bad shape");
  if (n_pairs == 0) return KVS_OK;
  const size_t block_bytes = (size_t)hkv * kBlock * d;
  hipLaunchKernelGGL(copy_blocks_fp8_kernel, dim3(n_pairs), dim3(256), 0, as_stream(stream),
                     static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), k_scale, v_scale, num_blocks,
                     block_bytes, hkv * kBlock, src_dst_pairs);
  return launch_status("kvs_copy_blocks_fp8");
}
