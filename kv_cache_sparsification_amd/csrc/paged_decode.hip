// Decode attention over the paged (compressed) cache, with the new token appended first.
//
// [PAG] Ultralytics glossary, "PagedAttention", "How paging works": the attention kernel
// follows the request's block table and gathers keys and values block by block, so the
// cache need not be contiguous.  "Related techniques", grouped-query attention: KV heads
// are shared by query heads.  [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration
// for vLLM", Key techniques 2 (last paragraph): PagedAttention does the decode-side work
// over the cache the compression left.
//
// MI355X form.  Grid (context split, KV head, sequence); a workgroup of 4 wavefronts walks
// the blocks of its split, wavefront w taking blocks w, w+4, ...  The G query heads of the
// group are the N columns of the MFMAs, so each K/V byte is read once per KV head:
//   scores^T[16 tokens][16 cols] = K_block[16][d] . Q^T       (bf16 16x16x32, keys as rows)
//   out^T[d][16 cols]          += V^T[d][16 tokens] . P^T      (bf16 16x16x16, V pool is
//                                                               channel-major, so V^T loads
//                                                               are contiguous)
// The score tile's lane layout (4 tokens of one column per lane) is exactly the B operand
// layout of the second product, so P never leaves registers.  Online softmax runs per
// column with two cross-lane maxima per block; the wavefronts of a workgroup merge through
// LDS, and when the context is split a second kernel merges the (max, sum, output) triples.
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kWaves = 4;
constexpr int kTargetWGs = 2048;

struct Split {
  int bps;      // blocks per split
  int splits;
};

inline Split choose_split(int batch, int hkv, int max_ctx) {
  const int nblk = (max_ctx + kBlock - 1) / kBlock;
  const int units = batch * hkv;
  const int want = (kTargetWGs + units - 1) / units;
  int bps = (nblk + want - 1) / want;
  if (bps < kWaves) bps = kWaves;
  Split s;
  s.bps = bps;
  s.splits = nblk > 0 ? (nblk + bps - 1) / bps : 1;
  return s;
}

template <int D>
__global__ __launch_bounds__(kWaves * kWave) void decode_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool, int num_blocks,
    const int32_t* __restrict__ tables, int max_blocks, const int32_t* __restrict__ ctx_lens, int hq, int hkv,
    float c_log2, const uint16_t* __restrict__ new_k, const uint16_t* __restrict__ new_v, uint16_t* __restrict__ o,
    float* __restrict__ lse_out, float* __restrict__ ws, int splits, int bps) {
  constexpr int KS = D / 32;     // k-steps of the score product
  constexpr int MT = D / 16;     // d tiles of the output product
  __shared__ float s_o[kWaves][D][16];
  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];

  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int col = lane % 16, grp = lane / 16;
  const int G = hq / hkv;
  const int L = ctx_lens[b];
  const int nblk = min((L + kBlock - 1) / kBlock, max_blocks);
  const int blk_begin = sp * bps;
  const int blk_end = min(blk_begin + bps, nblk);
  if (blk_begin >= blk_end) return;   // empty split: the merge skips it

  // B operand of the score product: Q^T[d][col], col = query head g*G + col (zero if col >= G).
  bf16x8 qf[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (col < G) v = *reinterpret_cast<const u32x4*>(q + ((size_t)b * hq + g * G + col) * D + st * 32 + grp * 8);
    qf[st] = __builtin_bit_cast(bf16x8, v);
  }

  const int last_blk = (L - 1) / kBlock, last_slot = (L - 1) % kBlock;
  const bool append = new_k != nullptr && new_v != nullptr;
  const int32_t* table = tables + (size_t)b * max_blocks;

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc_o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int bi = blk_begin + w; bi < blk_end; bi += kWaves) {
    const int blk = table[bi];
    if (blk < 0 || blk >= num_blocks) continue;
    const uint16_t* kb = k_pool + ((size_t)blk * hkv + g) * kBlock * D;
    const uint16_t* vb = v_pool + ((size_t)blk * hkv + g) * D * kBlock;
    const bool app_blk = append && bi == last_blk;

    // K rows (A operand): token = col, d = st*32 + grp*8 .. +8.
    bf16x8 kf[KS];
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      const uint16_t* src = (app_blk && col == last_slot) ? new_k + ((size_t)b * hkv + g) * D : kb + col * D;
      kf[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + st * 32 + grp * 8));
    }
    // V^T (A operand of the output product): d = mt*16 + col, tokens grp*4 .. +4.
    short4_t vf[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      vf[mt] = *reinterpret_cast<const short4_t*>(vb + (size_t)(mt * 16 + col) * kBlock + grp * 4);
    if (app_blk && grp == last_slot / 4) {
      const uint16_t* nv = new_v + ((size_t)b * hkv + g) * D;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) vf[mt][last_slot % 4] = (short)nv[mt * 16 + col];
    }

    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < KS; ++st) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[st], qf[st], sc, 0, 0, 0);
    // sc[i]: token grp*4 + i of this block against column col.
    float x[4];
    float bm = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = bi * kBlock + grp * 4 + i;
      x[i] = t < L ? sc[i] * c_log2 : -INFINITY;
      bm = fmaxf(bm, x[i]);
    }
    bm = fmaxf(bm, wave_xor(bm, 16));
    bm = fmaxf(bm, wave_xor(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    float p[4], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
      psum += p[i];
    }
    l_run = l_run * corr + psum;
    m_run = m_new;
    short4_t pb;
    pb[0] = (short)f32_to_bf16_bits(p[0]);
    pb[1] = (short)f32_to_bf16_bits(p[1]);
    pb[2] = (short)f32_to_bf16_bits(p[2]);
    pb[3] = (short)f32_to_bf16_bits(p[3]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc_o[mt] *= corr;
      acc_o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[mt], pb, acc_o[mt], 0, 0, 0);
    }

    if (app_blk) {   // keep the appended token in the pool for the next steps
      if (col == last_slot) {
        uint16_t* kd = k_pool + ((size_t)blk * hkv + g) * kBlock * D + last_slot * D;
        const uint16_t* nk = new_k + ((size_t)b * hkv + g) * D;
#pragma unroll
        for (int st = 0; st < KS; ++st)
          *reinterpret_cast<u32x4*>(kd + st * 32 + grp * 8) = *reinterpret_cast<const u32x4*>(nk + st * 32 + grp * 8);
      }
      if (grp == last_slot / 4) {
        uint16_t* vd = v_pool + ((size_t)blk * hkv + g) * D * kBlock;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) vd[(size_t)(mt * 16 + col) * kBlock + last_slot] = (uint16_t)vf[mt][last_slot % 4];
      }
    }
  }
  l_run += wave_xor(l_run, 16);
  l_run += wave_xor(l_run, 32);

  // acc_o[mt][i] is output channel mt*16 + grp*4 + i of column col.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[w][mt * 16 + grp * 4 + i][col] = acc_o[mt][i];
  if (grp == 0) {
    s_m[w][col] = m_run;
    s_l[w][col] = l_run;
  }
  __syncthreads();

  // Merge the 4 wavefronts: thread -> (column, channel) pairs.
  for (int e = tid; e < G * D; e += kWaves * kWave) {
    const int c = e / D, dd = e % D;
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) m = fmaxf(m, s_m[v][c]);
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float wgt = __builtin_amdgcn_exp2f(s_m[v][c] - m);   // empty wavefront: exp2(-inf) = 0
      l += s_l[v][c] * wgt;
      acc += s_o[v][dd][c] * wgt;
    }
    const int h = g * G + c;
    if (splits == 1) {
      o[((size_t)b * hq + h) * D + dd] = (uint16_t)f32_to_bf16_bits(acc / l);
      if (lse_out && dd == 0) lse_out[(size_t)b * hq + h] = (m + __log2f(l)) * kLn2;
    } else {
      float* part = ws + (((size_t)b * hq + h) * splits + sp) * (D + 2);
      part[2 + dd] = acc;
      if (dd == 0) {
        part[0] = m;
        part[1] = l;
      }
    }
  }
}

// Merge of the split partials: one workgroup per (query head, sequence), one thread per channel.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ ws, const int32_t* __restrict__ ctx_lens,
                                                        int hq, int splits, int bps, uint16_t* __restrict__ o,
                                                        float* __restrict__ lse_out) {
  const int h = blockIdx.x, b = blockIdx.y, dd = threadIdx.x;
  const int L = ctx_lens[b];
  const int nblk = (L + kBlock - 1) / kBlock;
  const int used = min((nblk + bps - 1) / bps, splits);
  const float* part = ws + ((size_t)b * hq + h) * splits * (D + 2);
  float m = -INFINITY;
  for (int sp = 0; sp < used; ++sp) m = fmaxf(m, part[sp * (D + 2)]);
  float l = 0.f, acc = 0.f;
  for (int sp = 0; sp < used; ++sp) {
    const float wgt = __builtin_amdgcn_exp2f(part[sp * (D + 2)] - m);
    l += part[sp * (D + 2) + 1] * wgt;
    acc += part[sp * (D + 2) + 2 + dd] * wgt;
  }
  o[((size_t)b * hq + h) * D + dd] = (uint16_t)f32_to_bf16_bits(acc / l);
  if (lse_out && dd == 0) lse_out[(size_t)b * hq + h] = (m + __log2f(l)) * kLn2;
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" size_t kvs_paged_decode_workspace_size(int batch, int hq, int hkv, int d, int max_ctx) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || max_ctx <= 0 || d <= 0) return 0;
  const Split s = choose_split(batch, hkv, max_ctx);
  if (s.splits <= 1) return 0;
  return (size_t)batch * hq * s.splits * (d + 2) * sizeof(float);
}

extern "C" int kvs_paged_decode(const void* q, void* k_pool, void* v_pool, int num_blocks, const int32_t* block_tables,
                                int max_blocks, const int32_t* ctx_lens, int batch, int max_ctx, int hq, int hkv, int d,
                                float scale, const void* new_k, const void* new_v, void* o, float* lse_opt,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_pool || !v_pool || !block_tables || !ctx_lens || !o)
    return fail(KVS_E_INVAL, "kvs_paged_decode: NULL tensor");
  if ((new_k == nullptr) != (new_v == nullptr)) return fail(KVS_E_INVAL, "kvs_paged_decode: new_k and new_v go together");
  if (batch < 0 || max_ctx < 1 || hq <= 0 || hkv <= 0 || hq % hkv || hq / hkv > 16 || (d != 64 && d != 128) ||
      num_blocks <= 0 || max_blocks <= 0 || !(scale > 0.f))
    return fail(KVS_E_INVAL, "kvs_paged_decode: bad shape (batch=%d hq=%d hkv=%d d=%d max_ctx=%d)", batch, hq, hkv, d,
                max_ctx);
  if ((long long)max_blocks * kBlock < max_ctx) return fail(KVS_E_INVAL, "kvs_paged_decode: max_blocks*16 < max_ctx");
  if (batch == 0) return KVS_OK;
  const Split sp = choose_split(batch, hkv, max_ctx);
  const size_t need = kvs_paged_decode_workspace_size(batch, hq, hkv, d, max_ctx);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KVS_E_INVAL, "kvs_paged_decode: workspace of %zu bytes needed, %zu given", need, workspace_bytes);
  const float c = scale * kLog2e;
  dim3 grid(sp.splits, hkv, batch);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kp = static_cast<uint16_t*>(k_pool);
  auto* vp = static_cast<uint16_t*>(v_pool);
  auto* nk = static_cast<const uint16_t*>(new_k);
  auto* nv = static_cast<const uint16_t*>(new_v);
  auto* oo = static_cast<uint16_t*>(o);
  auto* ws = static_cast<float*>(workspace);
  hipStream_t st = as_stream(stream);
  if (d == 128)
    hipLaunchKernelGGL(decode_kernel<128>, grid, dim3(kWaves * kWave), 0, st, qq, kp, vp, num_blocks, block_tables,
                       max_blocks, ctx_lens, hq, hkv, c, nk, nv, oo, lse_opt, ws, sp.splits, sp.bps);
  else
    hipLaunchKernelGGL(decode_kernel<64>, grid, dim3(kWaves * kWave), 0, st, qq, kp, vp, num_blocks, block_tables,
                       max_blocks, ctx_lens, hq, hkv, c, nk, nv, oo, lse_opt, ws, sp.splits, sp.bps);
  int rc = launch_status("kvs_paged_decode");
  if (rc != KVS_OK || sp.splits == 1) return rc;
  if (d == 128)
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3(hq, batch), dim3(128), 0, st, ws, ctx_lens, hq, sp.splits, sp.bps,
                       oo, lse_opt);
  else
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3(hq, batch), dim3(64), 0, st, ws, ctx_lens, hq, sp.splits, sp.bps,
                       oo, lse_opt);
  return launch_status("kvs_paged_decode (merge)");
}
