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
//     channel rows of 64 keys).  The key order of the first product is permuted so that each
//     lane's share of P^T is 8 consecutive keys: the A operand of the second product is then a
//     single 16-byte LDS read.  The next tile's global loads are issued before the current tile
//     is computed.
//   * Q stays in registers for the whole key loop.  Wavefronts whose rows all precede a key
//     tile skip it (causal); only the diagonal tile is masked, and O is rescaled only when a
//     row maximum grows by more than 2^8 (wave-uniform branches).
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

// Chunk swizzle of the K tile in LDS: 16 chunk positions make one 256-byte line of the 64
// banks, so rows r of one line group (16 / KCU rows per line) rotate their chunks by
// (r / (16 / KCU)) % KCU; any 16 consecutive rows then put a given chunk on 16 distinct positions.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  constexpr int KCU = D / 8;
  return (r / (16 / KCU)) % KCU;
}

// s_waitcnt vmcnt(0) with the other counters left alone (gfx9 encoding: vmcnt 0, expcnt 7,
// lgkmcnt 15).
constexpr int kVmcntZero = 0x0F70;

// MFMA row m of the S^T product holds key kappa(m) of its 32-key tile: bits 2 and 3 of m are
// swapped.  With that order the 16 scores a lane half gets back cover 8 consecutive keys per
// 16-key step, so P^T needs no shuffling and the matching V^T operand is one 16-byte read.
__device__ __forceinline__ int kappa(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D>
__global__ __launch_bounds__(kWaves * kWave, 2) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu_seqlens, int num_seqs, int total_tokens, int hq, int hkv, float c_log2,
    uint16_t* __restrict__ o, float* __restrict__ lse, float* __restrict__ rowmax, float* __restrict__ ell, int nqt,
    int total_items) {
  constexpr int KCU = D / 8;      // 16-byte chunks per K row
  constexpr int VSTR = kBK + 8;  // bf16 per V^T row in LDS: 36 words, 16 consecutive rows on distinct banks
  constexpr int ST1 = D / 16;    // k-steps of S^T = K Q^T
  constexpr int MT2 = D / 32;    // channel tiles of O^T
  constexpr int KS2 = kBK / 16;  // k-steps of O^T = V^T P^T
  constexpr int NT = kWaves * kWave;
  // Double-buffered tiles as four distinct LDS objects: with the buffer of each access known at
  // compile time, the compiler can tell the loads into one buffer from the reads of the other
  // and does not make those reads wait for the loads.
  __shared__ __attribute__((aligned(16))) uint16_t ks0[kBK * D], ks1[kBK * D];
  __shared__ __attribute__((aligned(16))) uint16_t vt0[D * VSTR], vt1[D * VSTR];

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

  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: branches on it stay scalar
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

  // m_ref is the reference max (log2-scaled) the exponentials are taken against; it moves only
  // when some row's true maximum exceeds it by more than kLazy, so most tiles skip the rescale
  // of O (p may then reach 2^kLazy, harmless in fp32 and bf16).  m_true is the exact row max.
  constexpr float kLazy = 8.f;
  float m_ref = -INFINITY, m_true = -INFINITY;
  float l_lane = 0.f;        // this lane's part of the running sum (16 of every 32 keys)
  f32x16 acc_o[MT2];
#pragma unroll
  for (int mt = 0; mt < MT2; ++mt) acc_o[mt] = f32x16{};

  const int kend = min(r0 + kBQ, n);
  const int ntiles = (kend + kBK - 1) / kBK;

  // ---- Global -> register staging of one K/V tile, prefetched one tile ahead.
  // K item e: row r = e / (D/8), 16-byte chunk cc = e % (D/8): 16 lanes read one 256-byte row.
  // V item e: key pair p and chunk cc, 16 lanes per row as well; stored transposed.
  // The loads go through buffer resources that cover this sequence's rows of KV head g only,
  // so the ragged last tile needs no branch and the per-tile address is a scalar move of the
  // resource base.  V rows past the prompt read as zero (P is zero there, and 0 * garbage
  // could be NaN); K rows past the prompt only meet masked scores, so whatever the LDS holds
  // for them is replaced by -inf before use.
  constexpr int KCH = kBK * (D / 8) / NT;
  constexpr int VIT = (kBK / 2) * (D / 8) / NT;
  constexpr int kRowBytes = 2 * D;
  const int row_pitch = hkv * kRowBytes;                           // bytes between consecutive keys
  const int seq_bytes = (n - 1) * row_pitch + kRowBytes;           // this head's rows of the prompt
  const int tile_bytes = kBK * row_pitch;
  const char* kbase = reinterpret_cast<const char*>(k + ((size_t)base * hkv + g) * D);
  const char* vbase = reinterpret_cast<const char*>(v + ((size_t)base * hkv + g) * D);
  // K goes from memory straight into LDS: load `it` of wave w fills the 1 KB of LDS units
  // u = (it * kWaves + w) * 64 + lane (16 bytes each), unit u being chunk position
  // u % KCU of row u / KCU.  Chunk c of row r sits at position c ^ kswz(r): the 16 rows a
  // lane group reads in one product step then cover all 64 banks, with no row padding.
  int koff[KCH], voff[VIT];
#pragma unroll
  for (int it = 0; it < KCH; ++it) {
    const int u = (it * kWaves + w) * kWave + lane;
    const int r = u / KCU;
    koff[it] = r * row_pitch + ((u % KCU) ^ kswz<D>(r)) * 16;
  }
#pragma unroll
  for (int it = 0; it < VIT; ++it) {
    const int e = it * NT + tid;
    const int wv = e / kWave, ln = e % kWave;
    const int p = (wv % 2) * 16 + ln % 16;
    const int cc = (wv / 2) * 4 + ln / 16;
    voff[it] = 2 * p * row_pitch + cc * 16;
  }
  u32x4 va[VIT], vb[VIT];
  auto load_tile = [&](int kt, int buf) {   // buf: a constant at every call
    uint16_t* ks = buf ? ks1 : ks0;
    const int skip = kt * tile_bytes;   // < seq_bytes for every tile that is loaded
    const __amdgpu_buffer_rsrc_t kr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kbase) + skip, 0, seq_bytes - skip, kBufferFlags);
    const __amdgpu_buffer_rsrc_t vr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vbase) + skip, 0, seq_bytes - skip, kBufferFlags);
#pragma unroll
    for (int it = 0; it < KCH; ++it)
      buffer_load_lds16(kr, &ks[(it * kWaves + w) * kWave * 8], koff[it]);
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      va[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[it], 0, 0);
      vb[it] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[it] + row_pitch, 0, 0);
    }
  };
  // V^T goes through registers (the transpose), K is already in place once its loads land.
  auto store_tile = [&](int buf) {
    uint16_t* vt = buf ? vt1 : vt0;
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int e = it * NT + tid;
      const int wv = e / kWave, ln = e % kWave;
      const int p = (wv % 2) * 16 + ln % 16;
      const int cc = (wv / 2) * 4 + ln / 16;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // channel cc*8 + j of keys 2p (low half) and 2p + 1 (high half)
        const uint32_t word = (j % 2 == 0)
            ? __builtin_amdgcn_perm(vb[it][j / 2], va[it][j / 2], 0x05040100u)
            : __builtin_amdgcn_perm(vb[it][j / 2], va[it][j / 2], 0x07060302u);
        *reinterpret_cast<uint32_t*>(&vt[(cc * 8 + j) * VSTR + 2 * p]) = word;
      }
    }
  };

  // GEMM-1 A operand: lane col reads K row kappa(col) of each 32-key M tile, chunk 2*st + half
  // at its swizzled position (the swizzle of rows 32 apart is the same).
  const int krow = kappa(col);
  int kofs[ST1];
#pragma unroll
  for (int st = 0; st < ST1; ++st) kofs[st] = krow * D + (((2 * st + half) ^ kswz<D>(krow)) * 8);

  // One barrier per tile: tile kt+1's global loads are issued before tile kt is computed and
  // stored into the other LDS buffer right after it, while the barrier that ends iteration kt
  // makes those stores visible and guarantees nobody still reads that buffer's previous tile.
  load_tile(0, 0);
  store_tile(0);
  __builtin_amdgcn_s_waitcnt(kVmcntZero);   // this wave's K transfers into LDS have landed
  __syncthreads();
  auto tile_step = [&](const int cur, int kt) {   // cur: a constant at every call
    const int kb = kt * kBK;
    const uint16_t* ks = cur ? ks1 : ks0;
    const uint16_t* vt = cur ? vt1 : vt0;
    if (kt + 1 < ntiles) load_tile(kt + 1, cur ^ 1);   // in flight while this tile is computed
    if (kb <= R + kRowsPerWave - 1) {           // else every row of this wavefront precedes the tile
    // ---- S^T tile: 64 keys x 32 rows as two 32x32 products over d.  The 2*ST1 A fragments
    // are read from LDS in groups of four, the next group's reads in flight while the current
    // group's products run (the two 32-key halves alternate, so neighbours are independent).
    constexpr int NF1 = 2 * ST1, NG1 = NF1 / 4;
    auto kfrag = [&](int f) {
      const int mt = f % 2, st = f / 2;
      return *reinterpret_cast<const u32x4*>(&ks[mt * 32 * D + kofs[st]]);
    };
    u32x4 fr[2][4];
    f32x16 sacc[2];
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int j = 0; j < 4; ++j) fr[0][j] = kfrag(j);
#pragma unroll
    for (int grp = 0; grp < NG1; ++grp) {
      if (grp + 1 < NG1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) fr[(grp + 1) & 1][j] = kfrag(4 * (grp + 1) + j);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = 4 * grp + j;
        sacc[f % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fr[grp & 1][j]),
                                                               qf[f / 2], sacc[f % 2], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // The first group of V^T fragments is read now, to be in registers when P is.
    constexpr int NF2 = MT2 * KS2, NG2 = NF2 / 4;
    auto vfrag = [&](int f) {
      const int mt = f % MT2, ks2 = f / MT2;
      return *reinterpret_cast<const u32x4*>(&vt[(mt * 32 + col) * VSTR + ks2 * 16 + half * 8]);
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) fr[0][j] = vfrag(j);
    // sacc[mt][i] is key kb + 32*mt + 16*(i/8) + 8*half + i%8 against `row` (raw dot products).
    if (kb + kBK - 1 > R) {   // diagonal tile (wave-uniform): mask keys past the row
      const int lim = row - kb - 8 * half;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (mt * 32 + 16 * (i / 8) + (i % 8) > lim) sacc[mt][i] = -INFINITY;
    }
    float bm = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) bm = fmaxf(bm, sacc[mt][i]);
    bm = half_max(bm) * c_log2;
    m_true = fmaxf(m_true, bm);
    if (__ballot(m_true > m_ref + kLazy) != 0ull) {   // some row moved too far: rescale (rare)
      const float corr = __builtin_amdgcn_exp2f(m_ref - m_true);
      m_ref = m_true;
      l_lane *= corr;
#pragma unroll
      for (int mt = 0; mt < MT2; ++mt) acc_o[mt] *= corr;
    }
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][i], c_log2, -m_ref));
        sacc[mt][i] = p;
        psum += p;
      }
    l_lane += psum;

    // P^T as B operands: k-step ks2 holds keys 16*ks2 + 8*half + 0..7 in order.
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
    for (int grp = 0; grp < NG2; ++grp) {
      if (grp + 1 < NG2) {
#pragma unroll
        for (int j = 0; j < 4; ++j) fr[(grp + 1) & 1][j] = vfrag(4 * (grp + 1) + j);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int f = 4 * grp + j;
        acc_o[f % MT2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, fr[grp & 1][j]),
                                                                  pf[f / MT2], acc_o[f % MT2], 0, 0, 0);
      }
    }
    }
    if (kt + 1 < ntiles) store_tile(cur ^ 1);
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
  };
  for (int kt = 0; kt < ntiles; kt += 2) {
    tile_step(0, kt);
    if (kt + 1 < ntiles) tile_step(1, kt + 1);
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m_ref + log2 l)
  const float l = half_sum(l_lane);   // sum of exp2(x - m_ref)
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
      lse[li] = (m_ref + log2f(l)) * kLn2;
      if (rowmax) rowmax[li] = m_true * kLn2;
      if (ell) ell[li] = l * __builtin_amdgcn_exp2f(m_ref - m_true);   // sum of exp(s - rowmax)
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
  if ((long long)max_seqlen * hkv * d * 2 > 0x7fffffffll)   // K/V rows of one prompt are addressed with 32-bit offsets
    return fail(KVS_E_INVAL, "kvs_prefill_attn_lse: prompt of %d tokens x %d KV heads too large", max_seqlen, hkv);
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
