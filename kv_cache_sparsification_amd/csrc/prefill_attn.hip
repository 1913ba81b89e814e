// Causal prefill attention that also returns each row's log-sum-exp.
//
// [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM", Key techniques,
// 2. "Attention modification": FlashAttention2 (first Fig. 7) walks Q in chunks over the KV
// blocks, updating O, P and the row maximum as it goes and dividing O by l at the end; the
// row maximum and l are computed but not returned; the modified kernel (second Fig. 7)
// writes them out, which costs almost nothing and spares the scoring step a second pass.
// Here the pair is written as LSE = rowmax + ln(l) (plus rowmax and l on request).
//
// MI355X form (bf16 MFMA 32x32x16, fp32 accumulation, online softmax in registers):
//   * A workgroup = 4 wavefronts = 128 query rows of one query head; each wavefront owns 32
//     rows.  The product is computed transposed, S^T = K . Q^T: keys are the M dimension,
//     query rows the N dimension, so every lane holds 16 scores of a single query row per
//     32-key tile.  The row maximum is an in-lane max plus one cross-lane exchange, the row
//     scale of O is a per-lane scalar, and the exponentiated scores are already in the B
//     operand layout of O^T = V^T . P^T: P never goes through LDS.
//   * K tiles (64 keys) are staged row-major in LDS; V tiles are stored transposed (V^T,
//     channel rows of 64 keys) so the A operand of the second product is two 8-byte reads.
//     The transposing store maps lanes so a wavefront's 32-bit writes spread over all banks.
//   * Q stays in registers for the whole key loop.  Wavefronts whose rows all precede a key
//     tile skip it (causal); only the diagonal tile is masked.
//   * Workgroups are remapped so that each XCD (8 per chip, each with its own L2) works on
//     one KV head at a time, heaviest (last) query tiles first.
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kWaves = 4;
constexpr int kBQ = 128;   // query rows per workgroup
constexpr int kBK = 64;    // keys per tile
constexpr int kRowsPerWave = 32;
constexpr int kXcds = 8;

template <int D>
__global__ __launch_bounds__(kWaves * kWave, 2) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu_seqlens, int num_seqs, int total_tokens, int hq, int hkv, float c_log2,
    uint16_t* __restrict__ o, float* __restrict__ lse, float* __restrict__ rowmax, float* __restrict__ ell, int nqt,
    int total_items) {
  constexpr int KSTR = D + 8;    // bf16 per K row in LDS (16-byte pad)
  constexpr int VSTR = kBK + 4;  // bf16 per V^T row in LDS (8-byte aligned, bank-spread)
  constexpr int ST1 = D / 16;    // k-steps of S^T = K Q^T
  constexpr int MT2 = D / 32;    // channel tiles of O^T
  constexpr int KS2 = kBK / 16;  // k-steps of O^T = V^T P^T
  __shared__ __attribute__((aligned(16))) uint16_t ks[kBK * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt[D * VSTR];

  // ---- XCD-aware work mapping: item order (g, s, query tile descending, head in group).
  const int per_xcd = gridDim.x / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= total_items) return;
  const int G = hq / hkv;
  int rest = item;
  const int hl = rest % G; rest /= G;
  const int qt = nqt - 1 - rest % nqt; rest /= nqt;
  const int s = rest % num_seqs;
  const int g = rest / num_seqs;
  const int h = g * G + hl;
  const int base = cu_seqlens[s];
  const int n = cu_seqlens[s + 1] - base;
  const int r0 = qt * kBQ;
  if (r0 >= n) return;

  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int col = lane % 32, half = lane / 32;
  const int R = r0 + w * kRowsPerWave;   // first row of this wavefront
  const int row = R + col;               // this lane's query row (N index)

  // B operand of S^T: Q^T[d][row] for each 16-wide d step.
  bf16x8 qf[ST1];
#pragma unroll
  for (int st = 0; st < ST1; ++st) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row < n) x = *reinterpret_cast<const u32x4*>(q + ((size_t)(base + row) * hq + h) * D + st * 16 + half * 8);
    qf[st] = __builtin_bit_cast(bf16x8, x);
  }

  float m_run = -INFINITY;   // running max of the log2-scaled scores of `row`
  float l_lane = 0.f;        // this lane's part of the running sum (16 of every 32 keys)
  f32x16 acc_o[MT2];
#pragma unroll
  for (int mt = 0; mt < MT2; ++mt) acc_o[mt] = f32x16{};

  const int kend = min(r0 + kBQ, n);
  const int ntiles = (kend + kBK - 1) / kBK;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int kb = kt * kBK;
    __syncthreads();   // the previous tile is consumed
    // K tile -> ks (row-major), zero past the prompt.
    for (int e = tid; e < kBK * (D / 8); e += kWaves * kWave) {
      const int r = e / (D / 8), cc = e % (D / 8);
      const int key = kb + r;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < n) x = *reinterpret_cast<const u32x4*>(k + ((size_t)(base + key) * hkv + g) * D + cc * 8);
      *reinterpret_cast<u32x4*>(&ks[r * KSTR + cc * 8]) = x;
    }
    // V tile -> vt (transposed).  Item = (key pair p, 8-channel chunk cc); a wavefront covers
    // 16 pairs x 4 chunks so its 32-bit stores land on distinct banks.
    for (int e = tid; e < (kBK / 2) * (D / 8); e += kWaves * kWave) {
      const int wv = e / kWave, ln = e % kWave;
      const int p = (wv % 2) * 16 + ln % 16;
      const int cc = (wv / 2) * 4 + ln / 16;
      const int key0 = kb + 2 * p;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key0 < n) a = *reinterpret_cast<const u32x4*>(v + ((size_t)(base + key0) * hkv + g) * D + cc * 8);
      if (key0 + 1 < n) b = *reinterpret_cast<const u32x4*>(v + ((size_t)(base + key0 + 1) * hkv + g) * D + cc * 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t lo = (j % 2 == 0) ? (a[j / 2] & 0xffffu) : (a[j / 2] >> 16);
        const uint32_t hi = (j % 2 == 0) ? (b[j / 2] & 0xffffu) : (b[j / 2] >> 16);
        *reinterpret_cast<uint32_t*>(&vt[(cc * 8 + j) * VSTR + 2 * p]) = lo | (hi << 16);
      }
    }
    __syncthreads();
    if (kb > R + kRowsPerWave - 1) continue;   // every row of this wavefront precedes the tile

    // ---- S^T tile: 64 keys x 32 rows as two 32x32 products over d.
    f32x16 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      sacc[mt] = f32x16{};
#pragma unroll
      for (int st = 0; st < ST1; ++st) {
        const u32x4 ka = *reinterpret_cast<const u32x4*>(&ks[(mt * 32 + col) * KSTR + st * 16 + half * 8]);
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ka), qf[st], sacc[mt], 0, 0, 0);
      }
    }
    // sacc[mt][i] is key kb + 32*mt + 8*(i/4) + 4*half + i%4 against `row`.
    const bool diag = kb + kBK - 1 > R;
    float bm = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = sacc[mt][i] * c_log2;
        if (diag) {
          const int key = kb + mt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
          x = key <= row ? x : -INFINITY;
        }
        sacc[mt][i] = x;
        bm = fmaxf(bm, x);
      }
    bm = fmaxf(bm, wave_xor(bm, 32));
    const float m_new = fmaxf(m_run, bm);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(sacc[mt][i] - m_new);
        sacc[mt][i] = p;
        psum += p;
      }
    l_lane = l_lane * corr + psum;
    m_run = m_new;

    // P^T as B operands: k-step ks covers keys 16*ks + {4*half + 0..3, 8 + 4*half + 0..3}.
    bf16x8 pf[KS2];
#pragma unroll
    for (int ks2 = 0; ks2 < KS2; ++ks2) {
      const int mt = ks2 / 2, i0 = 8 * (ks2 % 2);
      u32x4 x;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = pack_bf16x2(sacc[mt][i0 + 2 * j], sacc[mt][i0 + 2 * j + 1]);
      pf[ks2] = __builtin_bit_cast(bf16x8, x);
    }
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt) {
      acc_o[mt] *= corr;
#pragma unroll
      for (int ks2 = 0; ks2 < KS2; ++ks2) {
        const uint16_t* vrow = &vt[(mt * 32 + col) * VSTR + ks2 * 16 + half * 4];
        const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
        const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
        const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
        acc_o[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, va), pf[ks2], acc_o[mt], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l)
  const float l = l_lane + wave_xor(l_lane, 32);
  if (row < n) {
    const float inv = 1.f / l;
    uint16_t* orow = o + ((size_t)(base + row) * hq + h) * D;
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        // acc_o[mt][4*i4 + 0..3] are channels mt*32 + 8*i4 + 4*half + 0..3
        u32x2 x;
        x[0] = pack_bf16x2(acc_o[mt][4 * i4 + 0] * inv, acc_o[mt][4 * i4 + 1] * inv);
        x[1] = pack_bf16x2(acc_o[mt][4 * i4 + 2] * inv, acc_o[mt][4 * i4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + mt * 32 + 8 * i4 + 4 * half) = x;
      }
    if (half == 0) {
      const size_t li = (size_t)h * total_tokens + base + row;
      lse[li] = (m_run + log2f(l)) * kLn2;
      if (rowmax) rowmax[li] = m_run * kLn2;
      if (ell) ell[li] = l;
    }
  }
}

}  // namespace
}  // namespace kvs

using namespace kvs;

extern "C" int kvs_prefill_attn_lse(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                    int num_seqs, int total_tokens, int max_seqlen, int hq, int hkv, int d,
                                    float scale, void* o, float* lse, float* rowmax_opt, float* ell_opt,
                                    void* stream) {
  if (!q || !k || !v || !cu_seqlens || !o || !lse) return fail(KVS_E_INVAL, "kvs_prefill_attn_lse: NULL tensor");
  if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0 || hq <= 0 || hkv <= 0 || hq % hkv || hq / hkv > 16 ||
      (d != 64 && d != 128) || !(scale > 0.f))
    return fail(KVS_E_INVAL, "kvs_prefill_attn_lse: bad shape (hq=%d hkv=%d d=%d)", hq, hkv, d);
  if (num_seqs == 0 || max_seqlen == 0 || total_tokens == 0) return KVS_OK;
  const int nqt = (max_seqlen + kBQ - 1) / kBQ;
  const long long items = (long long)hkv * num_seqs * nqt * (hq / hkv);
  if (items > (1ll << 30)) return fail(KVS_E_INVAL, "kvs_prefill_attn_lse: grid too large");
  const int grid = (int)((items + kXcds - 1) / kXcds * kXcds);
  const float c = scale * kLog2e;
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kk = static_cast<const uint16_t*>(k);
  auto* vv = static_cast<const uint16_t*>(v);
  auto* oo = static_cast<uint16_t*>(o);
  if (d == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, dim3(grid), dim3(kWaves * kWave), 0, as_stream(stream), qq, kk, vv,
                       cu_seqlens, num_seqs, total_tokens, hq, hkv, c, oo, lse, rowmax_opt, ell_opt, nqt, (int)items);
  else
    hipLaunchKernelGGL(prefill_kernel<64>, dim3(grid), dim3(kWaves * kWave), 0, as_stream(stream), qq, kk, vv,
                       cu_seqlens, num_seqs, total_tokens, hq, hkv, c, oo, lse, rowmax_opt, ell_opt, nqt, (int)items);
  return launch_status("kvs_prefill_attn_lse");
}
