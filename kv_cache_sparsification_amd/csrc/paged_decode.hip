// Decode attention over the paged (compressed) cache, with the new token appended first.
//
// [PAG] Ultralytics glossary, "PagedAttention", "How paging works": the attention kernel
// follows the request's block table and gathers keys and values block by block, so the
// cache need not be contiguous.  "Related techniques", grouped-query attention: KV heads
// are shared by query heads.  [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration
// for vLLM", Key techniques 2 (last paragraph): PagedAttention does the decode-side work
// over the cache the compression left.
//
// MI355X form.  Grid (context split, KV head, sequence).  A workgroup of W wavefronts walks
// the blocks of its split, wavefront w taking blocks w, w+W, ..., NB at a time: the table
// entries of the next NB are read while the current ones are computed, so a wavefront's
// blocks cost one memory round trip per NB blocks.  The G query heads of the group are the N
// columns of the MFMAs, so each K/V byte is read once per KV head:
//   scores^T[16 tokens][16 cols] = K_block[16][d] . Q^T       (bf16 16x16x32, keys as rows)
//   out^T[d][16 cols]          += V^T[d][16 tokens] . P^T      (bf16 16x16x16, V pool is
//                                                               channel-major, so V^T loads
//                                                               are contiguous)
// The score tile's lane layout (4 tokens of one column per lane) is exactly the B operand
// layout of the second product, so P never leaves registers.  Online softmax runs per
// column with two cross-lane maxima per block; the wavefronts of a workgroup merge through
// LDS.
//
// Launch plan (see choose_plan).  When a context is split, each split stores a (max, sum,
// output) partial and a second kernel merges them.  (A merge by the last workgroup to arrive
// would save that launch, but making the partials of other XCDs visible needs an agent-scope
// release, i.e. an L2 write-back per workgroup, which costs more on this chip than the
// launch: measured about 3x slower.)
#include <mutex>

#include "kvs_common.h"
#include "slot_select.h"

namespace kvs {
namespace {

constexpr int kCUs = 256;
constexpr int kTargetWGs = 2048;
constexpr int kMaxSplitsMerge = 256;
constexpr int kBandwidthBlocks = 4096;   // (sequence, KV head, block) triples per call
constexpr int kManyBlocks = 16384;
constexpr int kLongBlocks = 1024;        // blocks per sequence from which a context counts as long
constexpr int kNoSplitBlocks = 64;       // blocks one 8-wavefront workgroup walks without a split
constexpr float kLazy = 8.f;             // log2 headroom before the reference max moves

struct Plan {
  int waves;    // wavefronts per workgroup
  int nb;       // blocks per wavefront in flight
  int bps;      // blocks per split
  int splits;
};

// One workgroup per (sequence, KV head) when the batch alone fills the chip (>= 512 pairs) or
// the context is a single round of blocks; its wavefront count follows the head size and
// group width so the LDS merge buffer (waves * G * d * 4 bytes) stays within 32 KiB and the
// blocks in flight fit the registers.  Otherwise the context is split into pieces of >= 4
// blocks so that about 2048 four-wavefront workgroups run, and a second kernel merges.
// Measured on MI355X for one 8B layer (1 sequence, 8 KV heads, 400..900 cached tokens, graph
// replay): 4 blocks per split 9.0 us per step, 8: 9.6, 16: 11.2, 32: 13.4, one workgroup per
// pair: 11.7 - a single sequence's cache is read fastest by many CUs at once.
inline Plan choose_plan(int batch, int hq, int hkv, int d, int max_ctx, bool f8) {
  const int G = hq / hkv;
  const int nblk = (max_ctx + kBlock - 1) / kBlock;
  const int units = batch * hkv;
  Plan p;
  if (d == 64) {
    p.waves = G <= 4 ? 16 : (G <= 8 ? 8 : 4);
    p.nb = 2;
  } else {
    p.waves = G <= 8 ? 8 : 4;
    p.nb = 4;
  }
  if (units >= 2 * kCUs || nblk <= p.waves) {
    p.bps = nblk > 0 ? nblk : 1;
    p.splits = 1;
    return p;
  }
  // Short contexts in a batch wide enough for 1024+ wavefronts: one 8-wavefront workgroup per
  // pair walks its blocks in a few rounds, and the merge launch is saved (20 sequences x 8 KV
  // heads x 528 tokens: 10.8 us per step, against 15.2-22 us for any split plan).  With d = 128
  // a wavefront has one block in flight per round: the 29 such layers of the 32-layer step at
  // concurrency 20 take 14.8 us less than with two (8-bit cache: 5 us less); 4, 6, 12 and 16
  // wavefronts of one block, or 8 of three, were slower still.
  if (nblk <= kNoSplitBlocks && units * 8 >= 4 * kCUs) {
    p.waves = 8;
    p.nb = d == 128 ? 1 : 2;
    p.bps = nblk;
    p.splits = 1;
    return p;
  }
  p.waves = 4;
  // Below kBandwidthBlocks a piece is one block per wavefront: with d = 128 the one-block
  // kernel's fewer registers give 7.49 against 7.56 us per step on the 8B layer, same outputs.
  if (d == 128) p.nb = 1;
  const int want = (kTargetWGs + units - 1) / units;
  int bps = (nblk + want - 1) / want;
  if (bps < p.waves) bps = p.waves;
  const int total = units * nblk;
  if (total >= kManyBlocks) {
    // Read volume far beyond one wave generation: pieces of 8 blocks over many generations of
    // workgroups.  With d = 128 a piece is two wavefronts of one block for four rounds: the
    // one-block kernel's registers (122, 160 for the 8-bit cache) let more workgroups share a
    // SIMD pair than the wider kernels (20 x 8 heads x 1100-3900 tokens, three full layers per
    // step: 143.0 us against 155.0 for four wavefronts of two blocks in one round; 8-bit cache
    // 103 us against 138 for four wavefronts of four blocks in two rounds).
    if (d == 128 && nblk >= kLongBlocks) {
      // Long contexts: 8-wavefront workgroups, each context cut into sp equal pieces, sp the
      // smallest count that minimises the generations of workgroups per piece of work,
      // ceil(units * sp / CUs) / sp (4 x 30000 tokens, 32 pairs: 8 pieces, one workgroup per
      // CU; 88 us per step against 113 for pieces of 8 blocks over 2 wavefronts, 90 for 16
      // equal pieces, 89-109 for pieces of 64-256 blocks that leave a short last piece).
      p.waves = 8;
      p.nb = 1;
      int sp = 1, gens = (units + kCUs - 1) / kCUs;
      for (int c = 2; c <= 64; ++c) {
        const int gc = (units * c + kCUs - 1) / kCUs;
        if (gc * sp < gens * c) {   // gc / c < gens / sp
          sp = c;
          gens = gc;
        }
      }
      bps = (nblk + sp - 1) / sp;
    } else if (d == 128) {
      p.waves = 2;
      p.nb = 1;
      bps = 4 * p.waves * p.nb;
    } else {
      p.nb = f8 ? 4 : 2;
      bps = f8 ? 2 * p.waves * p.nb : p.waves * p.nb;
    }
  } else if (total >= kBandwidthBlocks) {
    // Enough blocks for the read volume to set the time: pieces of 32 blocks for eight
    // wavefronts (8 KV heads x 3000+ tokens, batch 4, per step: 4 waves x 4 blocks x 1 round
    // 15.2 us, 8 x 4 x 1 14.4, 8 x 2 x 2 13.7, 8 x 2 x 3 15.1, 8 x 2 x 4 18.0; with d = 128
    // one block in flight for four rounds 13.0 against 13.3 for 8 x 2 x 2, 8-bit cache 12.0
    // against 12.3, while pieces of 16 or 24 blocks were slower).
    p.waves = 8;
    p.nb = d == 128 ? 1 : 2;
    if (bps < 32) bps = 32;
  }
  if ((nblk + bps - 1) / bps > kMaxSplitsMerge) bps = (nblk + kMaxSplitsMerge - 1) / kMaxSplitsMerge;
  p.bps = bps;
  p.splits = (nblk + bps - 1) / bps;
  return p;
}

// Extras of the scored decode (decode-time scores and eviction): the slot each KV head
// writes the new token to, the log2-scaled logits of every (query head, slot) for the score
// pass, and partials even for a single split (the merge-and-score kernel reads them).
struct DecodeExtra {
  const int32_t* dst_slots;   // [batch][hkv], or NULL: slot L-1 for every head
  float* logits;              // [batch][hq][logit_stride], or NULL
  int logit_stride;
  int force_partials;
  float* k_scale;             // 8-bit cache: per-row scales [num_blocks][hkv][16]
  float* v_scale;
};

// Max / sum over the four lanes l, l^16, l^32, l^48 (the 16-lane rows that hold one column's
// tokens), with the gfx950 row swaps instead of LDS shuffles.
__device__ __forceinline__ float max_over_rows(float v) {
  v = half_max(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Value of lane I of each group of four lanes (DPP quad permutation [I, I, I, I]).
template <int I>
__device__ __forceinline__ float quad_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), I * 0x55, 0xf, 0xf, false));
}

// Max over the 16 lanes of each row, left in the row's lane 15 (DPP row shifts; the lanes
// shifted in read 0, so the values must be >= 0).
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, true)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, true)));
  return v;
}
__device__ __forceinline__ float sum_over_rows(float v) {
  v = half_sum(v);
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 8-bit cache operands of one block, as loaded: K codes (16-byte chunks c of the lane's token
// row at bytes 64c + 16*grp, i.e. one 64-byte run per row and instruction; k-step st uses half
// st%2 of chunk st/2, and the query fragments follow the same order of d), V^T codes (4 slots
// of one channel per lane and d tile) and the scales of the lane's 4 slots.
template <int KS, int MT>
struct F8Block {
  u32x4 k[KS / 2];
  uint32_t v[MT];
  f32x4 sk, sv;
};

// d offset of the 8 values lane group grp supplies at k-step st of the 8-bit path's score product.
__device__ __forceinline__ int f8_kofs(int st, int grp) { return (st / 2) * 64 + grp * 16 + (st % 2) * 8; }

// F8: the cache holds E4M3 codes with a fp32 scale per (slot, KV head) row; codes are widened
// to bf16 (exact) for the same MFMAs, the K scale multiplies the slot's score and the V scale
// its probability (before the bf16 rounding of P), and the appended token is quantized here.
template <int D, int W, int kNB, bool F8, bool kOne = false, bool kScored = false>
__global__ __launch_bounds__(W * kWave) void decode_kernel(
    const uint16_t* __restrict__ q, void* __restrict__ k_pool_v, void* __restrict__ v_pool_v, int num_blocks,
    const int32_t* __restrict__ tables, int max_blocks, const int32_t* __restrict__ ctx_lens, int hq, int hkv,
    float c_log2, const uint16_t* __restrict__ new_k, const uint16_t* __restrict__ new_v, uint16_t* __restrict__ o,
    float* __restrict__ lse_out, float* __restrict__ ws, int splits, int bps, DecodeExtra ex) {
  constexpr int KS = D / 32;     // k-steps of the score product
  constexpr int MT = D / 16;     // d tiles of the output product
  constexpr int NT = W * kWave;
  extern __shared__ float smem[];
  uint16_t* k_pool = static_cast<uint16_t*>(k_pool_v);
  uint16_t* v_pool = static_cast<uint16_t*>(v_pool_v);
  uint8_t* k_pool8 = static_cast<uint8_t*>(k_pool_v);
  uint8_t* v_pool8 = static_cast<uint8_t*>(v_pool_v);

  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform
  const int col = lane % 16, grp = lane / 16;
  const int G = hq / hkv;
  float* s_o = smem;                   // [W][G][D]
  float* s_m = smem + W * G * D;       // [W][16]
  float* s_l = s_m + W * 16;           // [W][16]
  const int blk_begin = sp * bps;
  const int32_t* table = tables + (size_t)b * max_blocks;

  // Issued together: the first round of table entries (in bounds of the table row, read
  // before L is known), the context length and the query.
  int nxt[kNB];   // kNB: blocks per wavefront in flight
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    const int bi = blk_begin + w + W * j;
    nxt[j] = bi < max_blocks ? table[bi] : -1;
  }
  const int L = ctx_lens[b];
  const int nblk = min((L + kBlock - 1) / kBlock, max_blocks);
  const int blk_end = min(blk_begin + bps, nblk);
  if (blk_begin >= blk_end) return;   // empty split: not merged

  // B operand of the score product: Q^T[d][col], col = query head g*G + col (zero if col >= G).
  bf16x8 qf[KS];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    u32x4 x = {0u, 0u, 0u, 0u};
    const int dofs = F8 ? f8_kofs(st, grp) : st * 32 + grp * 8;
    if (col < G) x = *reinterpret_cast<const u32x4*>(q + ((size_t)b * hq + g * G + col) * D + dofs);
    qf[st] = __builtin_bit_cast(bf16x8, x);
  }

  const int dst = (kScored && ex.dst_slots) ? ex.dst_slots[b * hkv + g] : L - 1;   // slot of the new token
  const int last_blk = dst / kBlock, last_slot = dst % kBlock;
  const bool append = new_k != nullptr && new_v != nullptr && dst >= 0 && dst < L;   // else nothing is written
  const uint16_t* nk = new_k + ((size_t)b * hkv + g) * D;
  const uint16_t* nv = new_v + ((size_t)b * hkv + g) * D;

  // 8-bit cache: the wavefront whose blocks include the new token's fetches that token right
  // away (lane l: K and V values 2l, 2l+1), quantizes it while its first blocks are in flight
  // and hands each lane the codes of its operand positions; they replace the slot's loaded
  // codes when the wavefront reaches that block.
  const bool owner = F8 && append && last_blk >= blk_begin && last_blk < blk_end && (last_blk - blk_begin) % W == w;
  uint32_t nk2 = 0u, nv2 = 0u;
  if constexpr (F8) {
    if (owner && 2 * lane < D) {
      nk2 = *reinterpret_cast<const uint32_t*>(nk + 2 * lane);
      nv2 = *reinterpret_cast<const uint32_t*>(nv + 2 * lane);
    }
  }
  // 16-bit cache: the wavefront whose blocks include the new token's fetches that token's V
  // values of its channels (mt*16 + col) right away, beside its first blocks; they replace the
  // slot's loaded values when it reaches that block.
  short nvv[MT];
  if constexpr (!F8) {
    const bool v_owner = append && last_blk >= blk_begin && last_blk < blk_end && (last_blk - blk_begin) % W == w;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) nvv[mt] = v_owner ? (short)nv[mt * 16 + col] : (short)0;
  }
  u32x2 nkc[KS];                 // the new token's K codes at this lane's A positions (column last_slot)
  uint32_t nvc[MT];              // its V code of channel mt*16 + col, low byte (row last_slot / 4)
  float nks = 0.f, nvs = 0.f;    // and its scales
  bool quantized = false;

  // Online softmax per column against a lazily moved reference max m_run: a block whose
  // column max exceeds m_run by at most 2^kLazy (log2 units) is accumulated against the old
  // reference (its p stay <= 2^kLazy), so the accumulators are rescaled only when some
  // column's max jumps further; one wave vote decides.
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc_o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One round: this wavefront's kNB blocks bi0, bi0 + W, ...  With kOne (the launch's pieces
  // are a single round) it runs once, with no loop and no later round's table entries fetched:
  // 6.69 against 7.42 us per batch-1 step on the 8B layer.
  auto one_round = [&](int bi0) {
    int cur[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      cur[j] = nxt[j];
      if constexpr (!kOne) {
        const int bn = bi0 + W * kNB + W * j;          // next round's table entries
        nxt[j] = bn < blk_end ? table[bn] : -1;
      }
    }
    bf16x8 kf[kNB][KS];
    short4_t vf[kNB][MT];
    F8Block<KS, MT> f8[kNB];
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      const int bi = bi0 + W * j;
      const int blk = cur[j];
      if (bi >= blk_end || blk < 0 || blk >= num_blocks) continue;
      const size_t bh = (size_t)blk * hkv + g;
      const bool app_blk = append && bi == last_blk;
      if constexpr (F8) {
        const uint8_t* kb = k_pool8 + bh * kBlock * D;
        const uint8_t* vb = v_pool8 + bh * D * kBlock;
        // scales first (the scores wait for them, not for V): lane (col, grp) fetches the scale
        // of slot grp*4 + col%4; the quad's four lanes then share theirs
        f8[j].sk[0] = ex.k_scale[bh * kBlock + grp * 4 + (col & 3)];
        f8[j].sv[0] = ex.v_scale[bh * kBlock + grp * 4 + (col & 3)];
#pragma unroll
        for (int c = 0; c < KS / 2; ++c) f8[j].k[c] = *reinterpret_cast<const u32x4*>(kb + col * D + c * 64 + grp * 16);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          f8[j].v[mt] = *reinterpret_cast<const uint32_t*>(vb + (size_t)(mt * 16 + col) * kBlock + grp * 4);
        (void)app_blk;
      } else {
        const uint16_t* kb = k_pool + bh * kBlock * D;
        const uint16_t* vb = v_pool + bh * D * kBlock;
        // K rows (A operand): token = col, d = st*32 + grp*8 .. +8; the new token comes from new_k.
        const uint16_t* ksrc = (app_blk && col == last_slot) ? nk : kb + col * D;
#pragma unroll
        for (int st = 0; st < KS; ++st)
          kf[j][st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(ksrc + st * 32 + grp * 8));
        // V^T (A operand of the output product): d = mt*16 + col, tokens grp*4 .. +4.
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          vf[j][mt] = *reinterpret_cast<const short4_t*>(vb + (size_t)(mt * 16 + col) * kBlock + grp * 4);
        if (app_blk && grp == last_slot / 4) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) vf[j][mt][last_slot % 4] = nvv[mt];
        }
      }
    }
    if constexpr (F8) {
      if (owner && !quantized) {
        // The new token's rows: whole-wavefront amax, one scale each, two codes per lane, then
        // each lane gathers the codes of its operand positions from the lanes that made them.
        quantized = true;
        const float k0 = bf16_bits_to_f32(nk2 & 0xffffu), k1 = bf16_bits_to_f32(nk2 >> 16);
        const float v0 = bf16_bits_to_f32(nv2 & 0xffffu), v1 = bf16_bits_to_f32(nv2 >> 16);
        float ak = row_max16(max_over_rows(fmaxf(fabsf(k0), fabsf(k1))));   // lane 15 of each row: the amax
        float av = row_max16(max_over_rows(fmaxf(fabsf(v0), fabsf(v1))));
        ak = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ak), 15));
        av = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(av), 15));
        float kr, vr;
        e4m3_row_params(ak, nks, kr);
        e4m3_row_params(av, nvs, vr);
        const int kc2 = (int)(e4m3x4(k0, k1, 0.f, 0.f, kr) & 0xffffu);   // codes of K values 2l, 2l+1
        const int vc2 = (int)(e4m3x4(v0, v1, 0.f, 0.f, vr) & 0xffffu);
#pragma unroll
        for (int st = 0; st < KS; ++st) {   // K values f8_kofs(st, grp) .. +8 live in lanes f8_kofs/2 .. +4
          const int src = f8_kofs(st, grp) / 2;
          const uint32_t c0 = __builtin_amdgcn_ds_bpermute(4 * src, kc2);
          const uint32_t c1 = __builtin_amdgcn_ds_bpermute(4 * (src + 1), kc2);
          const uint32_t c2 = __builtin_amdgcn_ds_bpermute(4 * (src + 2), kc2);
          const uint32_t c3 = __builtin_amdgcn_ds_bpermute(4 * (src + 3), kc2);
          nkc[st] = u32x2{c0 | (c1 << 16), c2 | (c3 << 16)};
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {   // V channel mt*16 + col lives in lane mt*8 + col/2
          const uint32_t c = __builtin_amdgcn_ds_bpermute(4 * (mt * 8 + col / 2), vc2);
          nvc[mt] = (c >> (8 * (col & 1))) & 0xffu;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      const int bi = bi0 + W * j;
      const int blk = cur[j];
      if (bi >= blk_end || blk < 0 || blk >= num_blocks) continue;
      const size_t bh = (size_t)blk * hkv + g;
      const bool app_blk = append && bi == last_blk;
      if constexpr (F8) {
        {
          const float k0 = f8[j].sk[0], v0 = f8[j].sv[0];
          f8[j].sk = f32x4{quad_bcast<0>(k0), quad_bcast<1>(k0), quad_bcast<2>(k0), quad_bcast<3>(k0)};
          f8[j].sv = f32x4{quad_bcast<0>(v0), quad_bcast<1>(v0), quad_bcast<2>(v0), quad_bcast<3>(v0)};
        }
        if (app_blk) {   // the new token's codes and scales replace the slot's loaded ones, and are stored
          if (col == last_slot) {
            uint8_t* kd = k_pool8 + bh * kBlock * D + last_slot * D;
#pragma unroll
            for (int st = 0; st < KS; ++st) {
              f8[j].k[st / 2][2 * (st % 2)] = nkc[st][0];
              f8[j].k[st / 2][2 * (st % 2) + 1] = nkc[st][1];
              *reinterpret_cast<u32x2*>(kd + f8_kofs(st, grp)) = nkc[st];
            }
          }
          if (grp == last_slot / 4) {
            const int sh = 8 * (last_slot % 4);
            uint8_t* vd = v_pool8 + bh * D * kBlock;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
              f8[j].v[mt] = (f8[j].v[mt] & ~(0xffu << sh)) | (nvc[mt] << sh);
              vd[(size_t)(mt * 16 + col) * kBlock + last_slot] = (uint8_t)nvc[mt];
            }
            f8[j].sk[last_slot % 4] = nks;
            f8[j].sv[last_slot % 4] = nvs;
          }
          if (lane == 0) {
            ex.k_scale[bh * kBlock + last_slot] = nks;
            ex.v_scale[bh * kBlock + last_slot] = nvs;
          }
        }
#pragma unroll
        for (int st = 0; st < KS; ++st)
          kf[j][st] = e4m3x8_to_bf16(u32x2{f8[j].k[st / 2][2 * (st % 2)], f8[j].k[st / 2][2 * (st % 2) + 1]});
        // slots past the context (the last block's tail) may hold stale codes: zero them
        uint32_t vmask = 0xffffffffu;
        if (bi * kBlock + kBlock > L) {
          const int live = L - bi * kBlock - grp * 4;   // slots of the lane's 4 inside the context
          vmask = live >= 4 ? 0xffffffffu : (live <= 0 ? 0u : (0xffffffffu >> (8 * (4 - live))));
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) vf[j][mt] = e4m3x4_to_bf16x4(f8[j].v[mt] & vmask);
      } else if (bi * kBlock + kBlock > L) {
        // the last block's slots past the context were never written (they may hold NaN bit
        // patterns, and P = 0 does not cancel those in the product): zero them
        const int live = L - bi * kBlock - grp * 4;   // slots of the lane's 4 inside the context
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i >= live) vf[j][mt][i] = 0;
      }
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j][st], qf[st], sc, 0, 0, 0);
      // sc[i]: token grp*4 + i of this block against column col.
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = bi * kBlock + grp * 4 + i;
        const float si = F8 ? sc[i] * f8[j].sk[i] : sc[i];
        x[i] = t < L ? si * c_log2 : -INFINITY;
      }
      if (kScored && ex.logits) {   // scored decode only (uniform branch)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = bi * kBlock + grp * 4 + i;
          if (col < G && t < L) ex.logits[((size_t)b * hq + g * G + col) * ex.logit_stride + t] = x[i];
        }
      }
      const float bm = max_over_rows(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
      if (__builtin_amdgcn_ballot_w64(bm > m_run + kLazy) != 0) {   // rare: move the reference
        const float m_new = fmaxf(m_run, bm);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // first block: exp2(-inf) = 0
        l_run *= corr;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc_o[mt] *= corr;
        m_run = m_new;
      }
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(x[i] - m_run);
        l_run += p[i];
      }
      short4_t pb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float pi = p[i];
        if constexpr (F8) pi = x[i] == -INFINITY ? 0.f : p[i] * f8[j].sv[i];   // stale tail scales stay out
        pb[i] = (short)f32_to_bf16_bits(pi);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc_o[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[j][mt], pb, acc_o[mt], 0, 0, 0);
      if constexpr (!F8) {
        if (app_blk) {   // keep the appended token in the pool for later steps
          if (col == last_slot) {
            uint16_t* kd = k_pool + bh * kBlock * D + last_slot * D;
#pragma unroll
            for (int st = 0; st < KS; ++st)
              *reinterpret_cast<u32x4*>(kd + st * 32 + grp * 8) = *reinterpret_cast<const u32x4*>(nk + st * 32 + grp * 8);
          }
          if (grp == last_slot / 4) {
            uint16_t* vd = v_pool + bh * D * kBlock;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) vd[(size_t)(mt * 16 + col) * kBlock + last_slot] = (uint16_t)vf[j][mt][last_slot % 4];
          }
        }
      }
    }
  };
  if constexpr (kOne) {
    if (blk_begin + w < blk_end) one_round(blk_begin + w);
  } else {
    for (int bi0 = blk_begin + w; bi0 < blk_end; bi0 += W * kNB) one_round(bi0);
  }
  l_run = sum_over_rows(l_run);

  // acc_o[mt][i] is output channel mt*16 + grp*4 + i of column col; only real columns are kept.
  if (col < G) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) s_o[((size_t)w * G + col) * D + mt * 16 + grp * 4 + i] = acc_o[mt][i];
    if (grp == 0) {
      s_m[w * 16 + col] = m_run;
      s_l[w * 16 + col] = l_run;
    }
  }
  __syncthreads();

  // Merge the W wavefronts: thread -> (column, channel) pairs.
  const int used = min((nblk + bps - 1) / bps, splits);   // non-empty splits of this sequence
  for (int e = tid; e < G * D; e += NT) {
    const int c = e / D, dd = e % D;
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < W; ++v) m = fmaxf(m, s_m[v * 16 + c]);
    float l = 0.f, acc = 0.f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float wgt = __builtin_amdgcn_exp2f(s_m[v * 16 + c] - m);   // idle wavefront: exp2(-inf) = 0
      l += s_l[v * 16 + c] * wgt;
      acc += s_o[((size_t)v * G + c) * D + dd] * wgt;
    }
    const int h = g * G + c;
    if (used == 1 && !(kScored && ex.force_partials)) {
      o[((size_t)b * hq + h) * D + dd] = (uint16_t)f32_to_bf16_bits(acc / l);
      if (lse_out && dd == 0) lse_out[(size_t)b * hq + h] = (m + log2f(l)) * kLn2;
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

// Merge of the split partials.  Each thread folds its output channel over the splits 16 at a
// time, issuing all loads of a chunk (its channel plus the (max, sum) pair, shared with its
// neighbours through L1) before using any: one memory round trip per C splits (kOne: the
// caller knows there are at most C, and the fold is a single straight pass).  The loads
// cover every split the launch has (a bound known on the host), so they do not wait for the
// context length; the splits past the sequence's last non-empty one (`used`) hold stale data
// and are masked out afterwards.
// Returns the running max M (log2 units), the sum l against it and the output numerator.
template <int D, bool kOne = false, int C = 16>
__device__ __forceinline__ void merge_partials(const float* __restrict__ part, int splits, int used, int dd, float& M,
                                               float& l, float& acc) {
  M = -INFINITY;
  l = 0.f;
  acc = 0.f;
  for (int sp0 = 0; kOne ? sp0 == 0 : sp0 < splits; sp0 += C) {
    float mv[C], lv[C], ov[C];
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const float* ps = part + (size_t)(sp0 + i < splits ? sp0 + i : 0) * (D + 2);
      mv[i] = ps[0];
      lv[i] = ps[1];
      ov[i] = ps[2 + dd];
    }
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const bool in = sp0 + i < used;
      mv[i] = in ? mv[i] : -INFINITY;
      lv[i] = in ? lv[i] : 0.f;
      ov[i] = in ? ov[i] : 0.f;
    }
    float cm = M;
#pragma unroll
    for (int i = 0; i < C; ++i) cm = fmaxf(cm, mv[i]);
    const float corr = __builtin_amdgcn_exp2f(M - cm);   // first chunk: exp2(-inf) = 0
    l *= corr;
    acc *= corr;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const float wgt = __builtin_amdgcn_exp2f(mv[i] - cm);
      l += lv[i] * wgt;
      acc += ov[i] * wgt;
    }
    M = cm;
  }
}

template <int D, int C>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ ws,
                                                         const int32_t* __restrict__ ctx_lens, int hq, int hkv,
                                                         int max_blocks, int splits, int bps,
                                                         uint16_t* __restrict__ o, float* __restrict__ lse_out) {
  const int h = blockIdx.x, b = blockIdx.y, dd = threadIdx.x;
  const int L = ctx_lens[b];
  const int nblk = min((L + kBlock - 1) / kBlock, max_blocks);
  const int used = min((nblk + bps - 1) / bps, splits);
  {
    float M, l, acc;
    const float* part = ws + ((size_t)b * hq + h) * splits * (D + 2);
    if (splits <= C)   // grid-uniform: one straight pass
      merge_partials<D, true, C>(part, splits, used, dd, M, l, acc);
    else
      merge_partials<D, false, C>(part, splits, used, dd, M, l, acc);
    if (used <= 1) return;                    // written directly by the decode kernel
    o[((size_t)b * hq + h) * D + dd] = (uint16_t)f32_to_bf16_bits(acc / l);
    if (lse_out && dd == 0) lse_out[(size_t)b * hq + h] = (M + log2f(l)) * kLn2;
  }
}

// The merge of two (query head, channel) outputs at once, all loads of a chunk of C splits for
// both issued before either is folded (one memory round trip per chunk for the pair).
template <int D, int C = 16>
__device__ __forceinline__ void merge_partials_pair(const float* __restrict__ part0, const float* __restrict__ part1,
                                                    bool has1, int splits, int used, int dd0, int dd1, float (&M)[2],
                                                    float (&l)[2], float (&acc)[2]) {
  for (int k = 0; k < 2; ++k) {
    M[k] = -INFINITY;
    l[k] = 0.f;
    acc[k] = 0.f;
  }
  for (int sp0 = 0; sp0 < splits; sp0 += C) {
    float mv[2][C], lv[2][C], ov[2][C];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float* part = k == 0 ? part0 : part1;
      const int dd = k == 0 ? dd0 : dd1;
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const float* ps = part + (size_t)(sp0 + i < splits ? sp0 + i : 0) * (D + 2);
        const bool ld = k == 0 || has1;
        mv[k][i] = ld ? ps[0] : -INFINITY;
        lv[k][i] = ld ? ps[1] : 0.f;
        ov[k][i] = ld ? ps[2 + dd] : 0.f;
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const bool in = sp0 + i < used;
        mv[k][i] = in ? mv[k][i] : -INFINITY;
        lv[k][i] = in ? lv[k][i] : 0.f;
        ov[k][i] = in ? ov[k][i] : 0.f;
      }
      float cm = M[k];
#pragma unroll
      for (int i = 0; i < C; ++i) cm = fmaxf(cm, mv[k][i]);
      const float corr = __builtin_amdgcn_exp2f(M[k] - cm);   // first chunk: exp2(-inf) = 0
      l[k] *= corr;
      acc[k] *= corr;
#pragma unroll
      for (int i = 0; i < C; ++i) {
        const float wgt = __builtin_amdgcn_exp2f(mv[k][i] - cm);
        l[k] += lv[k][i] * wgt;
        acc[k] += ov[k][i] * wgt;
      }
      M[k] = cm;
    }
  }
}

// Scored decode, second kernel: one workgroup per (KV head, sequence).  Merges the partials
// of the G query heads (output, LSE), then adds every live slot's probability summed over
// those heads, exp2(logit - LSE2), to its score: the decode row's contribution to S.
// With next_dst set, the same workgroup then chooses the slot of the next step's token from the
// scores it has just updated (with the live count L as n_filled), which saves the next step a
// launch.  When a thread's slots (t = tid + 256 j, j < 2) and their G <= 8 logits fit in
// registers, they are fetched at the start, in the same round trip as the partials and the
// context length, and the choice is made from the registers; otherwise the slots are read after
// the merge.  Either way every slot is updated and chosen by the same arithmetic.
template <int D, int C>
__global__ __launch_bounds__(kSelectThreads) void decode_merge_score_kernel(
    const float* __restrict__ ws, const float* __restrict__ logits, int logit_stride,
    const int32_t* __restrict__ ctx_lens, int hq, int hkv, int max_blocks, int splits, int bps,
    uint16_t* __restrict__ o, float* __restrict__ lse_out, float* __restrict__ slot_scores, int slot_stride,
    int32_t* __restrict__ slot_pos, int cap, int alpha, const int32_t* __restrict__ next_pos,
    int32_t* __restrict__ next_dst) {
  constexpr int kRS = 2, kRG = 8;   // register path: slots per thread, query heads per group
  __shared__ float lse2[16];
  const int g = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int G = hq / hkv;
  const float* lg = logits + ((size_t)b * hq + g * G) * logit_stride;
  float* sc = slot_scores + ((size_t)b * hkv + g) * slot_stride;
  int32_t* ps = next_dst ? slot_pos + ((size_t)b * hkv + g) * slot_stride : nullptr;
  // grid-uniform, from host-known bounds (logit_stride is the launch's max_ctx >= L)
  const bool regs = G <= kRG && logit_stride <= kRS * kSelectThreads && (!next_dst || cap <= kRS * kSelectThreads);
  float lgv[kRS][kRG], scv[kRS];
  int psv[kRS];
  if (regs) {   // in bounds of the slot and logit rows whatever L is; slots >= L are ignored
#pragma unroll
    for (int j = 0; j < kRS; ++j) {
      const int t = tid + kSelectThreads * j;
#pragma unroll
      for (int c = 0; c < kRG; ++c) lgv[j][c] = (c < G && t < logit_stride) ? lg[(size_t)c * logit_stride + t] : 0.f;
      scv[j] = t < logit_stride ? sc[t] : 0.f;
      psv[j] = (ps && t < cap) ? ps[t] : -1;
    }
  }
  const int L = ctx_lens[b];
  const int nblk = min((L + kBlock - 1) / kBlock, max_blocks);
  const int used = min((nblk + bps - 1) / bps, splits);
  for (int e = tid; e < G * D; e += 2 * kSelectThreads) {
    const int e1 = e + kSelectThreads;
    const bool has1 = e1 < G * D;
    const int c0 = e / D, dd0 = e % D, c1 = has1 ? e1 / D : c0, dd1 = has1 ? e1 % D : dd0;
    const int h0 = g * G + c0, h1 = g * G + c1;
    float M[2], l[2], acc[2];
    merge_partials_pair<D, C>(ws + ((size_t)b * hq + h0) * splits * (D + 2), ws + ((size_t)b * hq + h1) * splits * (D + 2),
                           has1, splits, used, dd0, dd1, M, l, acc);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (k == 1 && !has1) break;
      const int h = k == 0 ? h0 : h1, dd = k == 0 ? dd0 : dd1, c = k == 0 ? c0 : c1;
      o[((size_t)b * hq + h) * D + dd] = (uint16_t)f32_to_bf16_bits(acc[k] / l[k]);
      if (dd == 0) {
        lse2[c] = M[k] + log2f(l[k]);
        if (lse_out) lse_out[(size_t)b * hq + h] = (M[k] + log2f(l[k])) * kLn2;
      }
    }
  }
  __syncthreads();
  if (regs) {
#pragma unroll
    for (int j = 0; j < kRS; ++j) {
      const int t = tid + kSelectThreads * j;
      if (t < L) {
        float sum = 0.f;
#pragma unroll
        for (int c = 0; c < kRG; ++c)
          if (c < G) sum += __builtin_amdgcn_exp2f(lgv[j][c] - lse2[c]);
        scv[j] += sum;
        sc[t] = scv[j];
      }
    }
    if (next_dst)   // grid-uniform; the slots below cap are below L when the cache is full
      select_slot_regs<kRS>(psv, scv, sc, ps, L, cap, next_pos[b], alpha, next_dst + (size_t)b * hkv + g);
    return;
  }
  for (int t = tid; t < L; t += kSelectThreads) {
    float sum = 0.f;
    for (int c = 0; c < G; ++c) sum += __builtin_amdgcn_exp2f(lg[(size_t)c * logit_stride + t] - lse2[c]);
    sc[t] += sum;
  }
  if (next_dst) {   // grid-uniform
    __syncthreads();   // every updated score visible to the whole workgroup
    select_slot_block(sc, ps, L, cap, next_pos[b], alpha, next_dst + (size_t)b * hkv + g);
  }
}

}  // namespace
}  // namespace kvs

using namespace kvs;

// Workspace: partials [batch][hq][splits][d + 2] fp32 = (max, sum, unnormalised output).
extern "C" size_t kvs_paged_decode_workspace_size(int batch, int hq, int hkv, int d, int max_ctx) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || max_ctx <= 0 || d <= 0) return 0;
  // the 16- and 8-bit caches may split differently: room for either
  const Plan p = choose_plan(batch, hq, hkv, d, max_ctx, false), p8 = choose_plan(batch, hq, hkv, d, max_ctx, true);
  const int splits = p.splits > p8.splits ? p.splits : p8.splits;
  if (splits <= 1) return 0;
  return (size_t)batch * hq * splits * (d + 2) * sizeof(float);
}

// Splits fetched per round trip by the merge kernels: the fewest of 4, 8, 12 or 16 that cover
// the launch's split count, so that a short split list issues no loads for splits it does not
// have (16 per round, and more than one round, past 16 splits).
static int merge_width(int splits) { return splits <= 4 ? 4 : splits <= 8 ? 8 : splits <= 12 ? 12 : 16; }

template <int D>
static void launch_merge(int cw, int batch, hipStream_t st, const float* ws, const int32_t* ctx_lens, int hq, int hkv,
                         int max_blocks, int splits, int bps, uint16_t* o, float* lse) {
  auto k = cw == 4 ? decode_merge_kernel<D, 4> : cw == 8 ? decode_merge_kernel<D, 8>
           : cw == 12 ? decode_merge_kernel<D, 12> : decode_merge_kernel<D, 16>;
  hipLaunchKernelGGL(k, dim3(hq, batch), dim3(D), 0, st, ws, ctx_lens, hq, hkv, max_blocks, splits, bps, o, lse);
}

template <int D>
static void launch_merge_score(int cw, int batch, hipStream_t st, const float* ws, const float* logits, int max_ctx,
                               const int32_t* ctx_lens, int hq, int hkv, int max_blocks, int splits, int bps,
                               uint16_t* o, float* lse, float* slot_scores, int slot_stride, int32_t* slot_pos,
                               int cap, int alpha, const int32_t* next_pos, int32_t* next_dst) {
  auto k = cw == 4 ? decode_merge_score_kernel<D, 4> : cw == 8 ? decode_merge_score_kernel<D, 8>
           : cw == 12 ? decode_merge_score_kernel<D, 12> : decode_merge_score_kernel<D, 16>;
  hipLaunchKernelGGL(k, dim3(hkv, batch), dim3(kSelectThreads), 0, st, ws, logits, max_ctx, ctx_lens, hq, hkv,
                     max_blocks, splits, bps, o, lse, slot_scores, slot_stride, slot_pos, cap, alpha, next_pos,
                     next_dst);
}

template <int D, int W, int NB, bool F8>
static void launch_one(const Plan& p, dim3 grid, size_t lds, hipStream_t st, const uint16_t* q, void* kp, void* vp,
                       int num_blocks, const int32_t* tables, int max_blocks, const int32_t* ctx, int hq, int hkv,
                       float c, const uint16_t* nk, const uint16_t* nv, uint16_t* o, float* lse, float* ws,
                       const DecodeExtra& ex) {
  // the scored decode's extras (slot choice, logits, partials for one split) as a separate build
  const bool scored = ex.dst_slots || ex.logits || ex.force_partials;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(W * kWave), lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv,
                       c, nk, nv, o, lse, ws, p.splits, p.bps, ex);
  };
  if constexpr (W == 4 && NB == 1) {   // the few-block plan: pieces of one round
    if (p.bps <= W * NB) {
      scored ? go(decode_kernel<D, W, NB, F8, true, true>) : go(decode_kernel<D, W, NB, F8, true, false>);
      return;
    }
  }
  scored ? go(decode_kernel<D, W, NB, F8, false, true>) : go(decode_kernel<D, W, NB, F8, false, false>);
}

template <int D, bool F8>
static void launch_decode(const Plan& p, dim3 grid, size_t lds, hipStream_t st, const uint16_t* q, void* kp, void* vp,
                          int num_blocks, const int32_t* tables, int max_blocks, const int32_t* ctx, int hq, int hkv,
                          float c, const uint16_t* nk, const uint16_t* nv, uint16_t* o, float* lse, float* ws,
                          const DecodeExtra& ex) {
  // (wavefronts, blocks in flight per wavefront) pairs the plans use
  if (p.waves == 8 && p.nb == 2)
    launch_one<D, 8, 2, F8>(p, grid, lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv, c, nk, nv, o,
                            lse, ws, ex);
  else if constexpr (D == 64) {
    if (p.waves == 16)
      launch_one<D, 16, 2, F8>(p, grid, lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv, c, nk, nv, o,
                               lse, ws, ex);
    else
      launch_one<D, 4, 2, F8>(p, grid, lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv, c, nk, nv, o,
                              lse, ws, ex);
  } else {
    if (p.waves == 8 && p.nb == 1)
      launch_one<D, 8, 1, F8>(p, grid, lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv, c, nk, nv, o,
                              lse, ws, ex);
    else if (p.waves == 2 && p.nb == 1)
      launch_one<D, 2, 1, F8>(p, grid, lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv, c, nk, nv, o,
                              lse, ws, ex);
    else if (p.waves == 4 && p.nb == 1)
      launch_one<D, 4, 1, F8>(p, grid, lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv, c, nk, nv, o,
                              lse, ws, ex);
    else if (p.waves == 4 && p.nb == 2)
      launch_one<D, 4, 2, F8>(p, grid, lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv, c, nk, nv, o,
                              lse, ws, ex);
    else if (p.waves == 8)
      launch_one<D, 8, 4, F8>(p, grid, lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv, c, nk, nv, o,
                              lse, ws, ex);
    else
      launch_one<D, 4, 4, F8>(p, grid, lds, st, q, kp, vp, num_blocks, tables, max_blocks, ctx, hq, hkv, c, nk, nv, o,
                              lse, ws, ex);
  }
}

// Validation, plan and launches of the plain decode (16-bit or 8-bit cache).
static int run_decode(const char* name, const void* q, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                      bool f8, int num_blocks, const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens,
                      int batch, int max_ctx, int hq, int hkv, int d, float scale, const void* new_k,
                      const void* new_v, void* o, float* lse_opt, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!q || !k_pool || !v_pool || !block_tables || !ctx_lens || !o || (f8 && (!k_scale || !v_scale)))
    return fail(KVS_E_INVAL, "%s: NULL tensor", name);
  if ((new_k == nullptr) != (new_v == nullptr)) return fail(KVS_E_INVAL, "%s: new_k and new_v go together", name);
  if (batch < 0 || max_ctx < 1 || hq <= 0 || hkv <= 0 || hq % hkv || hq / hkv > 16 || (d != 64 && d != 128) ||
      num_blocks <= 0 || max_blocks <= 0 || !(scale > 0.f))
    return fail(KVS_E_INVAL, "%s: bad shape (batch=%d hq=%d hkv=%d d=%d max_ctx=%d)", name, batch, hq, hkv, d,
                max_ctx);
  if ((long long)max_blocks * kBlock < max_ctx) return fail(KVS_E_INVAL, "%s: max_blocks*16 < max_ctx", name);
  if (batch == 0) return KVS_OK;
  Plan p = choose_plan(batch, hq, hkv, d, max_ctx, f8);
  if (f8 && p.waves == 16) p.waves = 8;   // one workgroup per pair: the 8-bit path's registers fit 8 wavefronts
  const size_t need = kvs_paged_decode_workspace_size(batch, hq, hkv, d, max_ctx);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KVS_E_INVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, workspace_bytes);
  const float c = scale * kLog2e;
  const int G = hq / hkv;
  const size_t lds = ((size_t)p.waves * G * d + 2 * (size_t)p.waves * 16) * sizeof(float);
  dim3 grid(p.splits, hkv, batch);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* nk = static_cast<const uint16_t*>(new_k);
  auto* nv = static_cast<const uint16_t*>(new_v);
  auto* oo = static_cast<uint16_t*>(o);
  float* ws = static_cast<float*>(workspace);
  hipStream_t st = as_stream(stream);
  const DecodeExtra ex{nullptr, nullptr, 0, 0, k_scale, v_scale};
  if (d == 128) {
    if (f8)
      launch_decode<128, true>(p, grid, lds, st, qq, k_pool, v_pool, num_blocks, block_tables, max_blocks, ctx_lens,
                               hq, hkv, c, nk, nv, oo, lse_opt, ws, ex);
    else
      launch_decode<128, false>(p, grid, lds, st, qq, k_pool, v_pool, num_blocks, block_tables, max_blocks, ctx_lens,
                                hq, hkv, c, nk, nv, oo, lse_opt, ws, ex);
  } else {
    if (f8)
      launch_decode<64, true>(p, grid, lds, st, qq, k_pool, v_pool, num_blocks, block_tables, max_blocks, ctx_lens,
                              hq, hkv, c, nk, nv, oo, lse_opt, ws, ex);
    else
      launch_decode<64, false>(p, grid, lds, st, qq, k_pool, v_pool, num_blocks, block_tables, max_blocks, ctx_lens,
                               hq, hkv, c, nk, nv, oo, lse_opt, ws, ex);
  }
  int rc = launch_status(name);
  if (rc != KVS_OK || p.splits == 1) return rc;
  if (d == 128)
    launch_merge<128>(merge_width(p.splits), batch, st, ws, ctx_lens, hq, hkv, max_blocks, p.splits, p.bps, oo, lse_opt);
  else
    launch_merge<64>(merge_width(p.splits), batch, st, ws, ctx_lens, hq, hkv, max_blocks, p.splits, p.bps, oo, lse_opt);
  return launch_status(name);
}

extern "C" int kvs_paged_decode(const void* q, void* k_pool, void* v_pool, int num_blocks, const int32_t* block_tables,
                                int max_blocks, const int32_t* ctx_lens, int batch, int max_ctx, int hq, int hkv, int d,
                                float scale, const void* new_k, const void* new_v, void* o, float* lse_opt,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return run_decode("kvs_paged_decode", q, k_pool, v_pool, nullptr, nullptr, false, num_blocks, block_tables,
                    max_blocks, ctx_lens, batch, max_ctx, hq, hkv, d, scale, new_k, new_v, o, lse_opt, workspace,
                    workspace_bytes, stream);
}

extern "C" int kvs_paged_decode_fp8(const void* q, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                    int num_blocks, const int32_t* block_tables, int max_blocks,
                                    const int32_t* ctx_lens, int batch, int max_ctx, int hq, int hkv, int d,
                                    float scale, const void* new_k, const void* new_v, void* o, float* lse_opt,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  return run_decode("kvs_paged_decode_fp8", q, k_pool, v_pool, k_scale, v_scale, true, num_blocks, block_tables,
                    max_blocks, ctx_lens, batch, max_ctx, hq, hkv, d, scale, new_k, new_v, o, lse_opt, workspace,
                    workspace_bytes, stream);
}

// ---- Decode for callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid allocation): the split partials go to a scratch array
// the library holds on every device it runs on, for the life of the process.
namespace {
constexpr size_t kScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, looked up once
}  // namespace

// Device address of the current device's scratch array.  In host code `scratch` only names a
// host-side stand-in: its device address comes from the runtime, once per device, with that
// device current.
static int scratch_on_current_device(const char* name, void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KVS_E_HIP, "%s: hipGetDevice: %s", name, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KVS_E_INVAL, "%s: device %d is beyond the %d tracked", name, dev,
                                                   kMaxDevices);
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice(as_stream(stream), &sdev);
    if (e != hipSuccess) return fail(KVS_E_HIP, "%s: hipStreamGetDevice: %s", name, hipGetErrorString(e));
    if (sdev != dev) return fail(KVS_E_INVAL, "%s: the stream belongs to device %d, the current device is %d", name,
                                 sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KVS_E_HIP, "%s: hipGetSymbolAddress(scratch): %s", name, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return KVS_OK;
}

extern "C" int kvs_paged_decode_noalloc(const void* q, void* k_pool, void* v_pool, int num_blocks,
                                        const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens,
                                        int batch, int max_ctx, int hq, int hkv, int d, float scale,
                                        const void* new_k, const void* new_v, void* o, float* lse_opt,
                                        void* stream) {
  const char* name = "kvs_paged_decode_noalloc";
  const size_t need = kvs_paged_decode_workspace_size(batch, hq, hkv, d, max_ctx);
  if (need > kScratchBytes)
    return fail(KVS_E_INVAL, "%s: this call needs %zu bytes of split partials, more than the %zu-byte scratch the "
                "library holds per device (use kvs_paged_decode with a workspace)", name, need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_on_current_device(name, stream, &ws);
    if (rc != KVS_OK) return rc;
  }
  return run_decode(name, q, k_pool, v_pool, nullptr, nullptr, false, num_blocks, block_tables, max_blocks, ctx_lens,
                    batch, max_ctx, hq, hkv, d, scale, new_k, new_v, o, lse_opt, ws, need > 0 ? kScratchBytes : 0,
                    stream);
}

// ---- Scored decode: partials (always, even for one split) then the logits.
static size_t scored_logits_offset(int batch, int hq, int splits, int d) {
  const size_t part = (size_t)batch * hq * splits * (d + 2) * sizeof(float);
  return (part + 255) / 256 * 256;
}

extern "C" size_t kvs_paged_decode_scored_workspace_size(int batch, int hq, int hkv, int d, int max_ctx) {
  if (batch <= 0 || hq <= 0 || hkv <= 0 || hq % hkv || max_ctx <= 0 || d <= 0) return 0;
  const Plan p = choose_plan(batch, hq, hkv, d, max_ctx, false);
  return scored_logits_offset(batch, hq, p.splits, d) + (size_t)batch * hq * max_ctx * sizeof(float);
}

static int run_scored(const char* name, const void* q, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                      bool f8, int num_blocks, const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens,
                      int batch, int max_ctx, int hq, int hkv, int d, float scale, const void* new_k,
                      const void* new_v, const int32_t* dst_slots, float* slot_scores, int slot_stride, void* o,
                      float* lse_opt, void* workspace, size_t workspace_bytes, void* stream,
                      int32_t* slot_pos = nullptr, int cap = 0, int alpha = 0, const int32_t* next_pos = nullptr,
                      int32_t* next_dst = nullptr) {
  if (!q || !k_pool || !v_pool || !block_tables || !ctx_lens || !o || !slot_scores || (f8 && (!k_scale || !v_scale)))
    return fail(KVS_E_INVAL, "%s: NULL tensor", name);
  if (next_dst && (!slot_pos || !next_pos)) return fail(KVS_E_INVAL, "%s: NULL tensor", name);
  if (next_dst && (alpha < 0 || alpha >= cap || cap > slot_stride || max_ctx > cap))
    return fail(KVS_E_INVAL, "%s: need 0 <= alpha < cap <= slot_stride and max_ctx <= cap (alpha=%d cap=%d stride=%d)",
                name, alpha, cap, slot_stride);
  if ((new_k == nullptr) != (new_v == nullptr)) return fail(KVS_E_INVAL, "%s: new_k and new_v go together", name);
  if (dst_slots && !new_k) return fail(KVS_E_INVAL, "%s: dst_slots without a new token", name);
  if (batch < 0 || max_ctx < 1 || hq <= 0 || hkv <= 0 || hq % hkv || hq / hkv > 16 || (d != 64 && d != 128) ||
      num_blocks <= 0 || max_blocks <= 0 || !(scale > 0.f) || slot_stride < max_ctx)
    return fail(KVS_E_INVAL, "%s: bad shape (batch=%d hq=%d hkv=%d d=%d max_ctx=%d stride=%d)", name, batch, hq, hkv,
                d, max_ctx, slot_stride);
  if ((long long)max_blocks * kBlock < max_ctx) return fail(KVS_E_INVAL, "%s: max_blocks*16 < max_ctx", name);
  if (batch == 0) return KVS_OK;
  Plan p = choose_plan(batch, hq, hkv, d, max_ctx, false);   // the 16-bit plan for both: it sizes the workspace
  if (f8 && p.waves == 16) p.waves = 8;
  const size_t need = kvs_paged_decode_scored_workspace_size(batch, hq, hkv, d, max_ctx);
  if (!workspace || workspace_bytes < need)
    return fail(KVS_E_INVAL, "%s: workspace of %zu bytes needed, %zu given", name, need, workspace_bytes);
  const float c = scale * kLog2e;
  const int G = hq / hkv;
  const size_t lds = ((size_t)p.waves * G * d + 2 * (size_t)p.waves * 16) * sizeof(float);
  dim3 grid(p.splits, hkv, batch);
  auto* qq = static_cast<const uint16_t*>(q);
  auto* nk = static_cast<const uint16_t*>(new_k);
  auto* nv = static_cast<const uint16_t*>(new_v);
  auto* oo = static_cast<uint16_t*>(o);
  float* ws = static_cast<float*>(workspace);
  float* logits = reinterpret_cast<float*>(static_cast<char*>(workspace) + scored_logits_offset(batch, hq, p.splits, d));
  hipStream_t st = as_stream(stream);
  const DecodeExtra ex{dst_slots, logits, max_ctx, 1, k_scale, v_scale};
  if (d == 128) {
    if (f8)
      launch_decode<128, true>(p, grid, lds, st, qq, k_pool, v_pool, num_blocks, block_tables, max_blocks, ctx_lens,
                               hq, hkv, c, nk, nv, oo, lse_opt, ws, ex);
    else
      launch_decode<128, false>(p, grid, lds, st, qq, k_pool, v_pool, num_blocks, block_tables, max_blocks, ctx_lens,
                                hq, hkv, c, nk, nv, oo, lse_opt, ws, ex);
  } else {
    if (f8)
      launch_decode<64, true>(p, grid, lds, st, qq, k_pool, v_pool, num_blocks, block_tables, max_blocks, ctx_lens,
                              hq, hkv, c, nk, nv, oo, lse_opt, ws, ex);
    else
      launch_decode<64, false>(p, grid, lds, st, qq, k_pool, v_pool, num_blocks, block_tables, max_blocks, ctx_lens,
                               hq, hkv, c, nk, nv, oo, lse_opt, ws, ex);
  }
  int rc = launch_status(name);
  if (rc != KVS_OK) return rc;
  const int cw = merge_width(p.splits);
  if (d == 128)
    launch_merge_score<128>(cw, batch, st, ws, logits, max_ctx, ctx_lens, hq, hkv, max_blocks, p.splits, p.bps, oo,
                            lse_opt, slot_scores, slot_stride, slot_pos, cap, alpha, next_pos, next_dst);
  else
    launch_merge_score<64>(cw, batch, st, ws, logits, max_ctx, ctx_lens, hq, hkv, max_blocks, p.splits, p.bps, oo,
                           lse_opt, slot_scores, slot_stride, slot_pos, cap, alpha, next_pos, next_dst);
  return launch_status(name);
}

extern "C" int kvs_paged_decode_scored(const void* q, void* k_pool, void* v_pool, int num_blocks,
                                       const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens, int batch,
                                       int max_ctx, int hq, int hkv, int d, float scale, const void* new_k,
                                       const void* new_v, const int32_t* dst_slots, float* slot_scores,
                                       int slot_stride, void* o, float* lse_opt, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return run_scored("kvs_paged_decode_scored", q, k_pool, v_pool, nullptr, nullptr, false, num_blocks, block_tables,
                    max_blocks, ctx_lens, batch, max_ctx, hq, hkv, d, scale, new_k, new_v, dst_slots, slot_scores,
                    slot_stride, o, lse_opt, workspace, workspace_bytes, stream);
}

extern "C" int kvs_paged_decode_scored_fp8(const void* q, void* k_pool, void* v_pool, float* k_scale, float* v_scale,
                                           int num_blocks, const int32_t* block_tables, int max_blocks,
                                           const int32_t* ctx_lens, int batch, int max_ctx, int hq, int hkv, int d,
                                           float scale, const void* new_k, const void* new_v,
                                           const int32_t* dst_slots, float* slot_scores, int slot_stride, void* o,
                                           float* lse_opt, void* workspace, size_t workspace_bytes, void* stream) {
  return run_scored("kvs_paged_decode_scored_fp8", q, k_pool, v_pool, k_scale, v_scale, true, num_blocks,
                    block_tables, max_blocks, ctx_lens, batch, max_ctx, hq, hkv, d, scale, new_k, new_v, dst_slots,
                    slot_scores, slot_stride, o, lse_opt, workspace, workspace_bytes, stream);
}

extern "C" int kvs_paged_decode_scored_select(const void* q, void* k_pool, void* v_pool, int num_blocks,
                                              const int32_t* block_tables, int max_blocks, const int32_t* ctx_lens,
                                              int batch, int max_ctx, int hq, int hkv, int d, float scale,
                                              const void* new_k, const void* new_v, const int32_t* dst_slots,
                                              float* slot_scores, int32_t* slot_pos, int slot_stride, int cap,
                                              int alpha, const int32_t* next_pos, int32_t* next_dst_slots, void* o,
                                              float* lse_opt, void* workspace, size_t workspace_bytes, void* stream) {
  if (!next_dst_slots) return fail(KVS_E_INVAL, "kvs_paged_decode_scored_select: NULL tensor");
  return run_scored("kvs_paged_decode_scored_select", q, k_pool, v_pool, nullptr, nullptr, false, num_blocks,
                    block_tables, max_blocks, ctx_lens, batch, max_ctx, hq, hkv, d, scale, new_k, new_v, dst_slots,
                    slot_scores, slot_stride, o, lse_opt, workspace, workspace_bytes, stream, slot_pos, cap, alpha,
                    next_pos, next_dst_slots);
}

extern "C" int kvs_paged_decode_scored_select_fp8(const void* q, void* k_pool, void* v_pool, float* k_scale,
                                                  float* v_scale, int num_blocks, const int32_t* block_tables,
                                                  int max_blocks, const int32_t* ctx_lens, int batch, int max_ctx,
                                                  int hq, int hkv, int d, float scale, const void* new_k,
                                                  const void* new_v, const int32_t* dst_slots, float* slot_scores,
                                                  int32_t* slot_pos, int slot_stride, int cap, int alpha,
                                                  const int32_t* next_pos, int32_t* next_dst_slots, void* o,
                                                  float* lse_opt, void* workspace, size_t workspace_bytes,
                                                  void* stream) {
  if (!next_dst_slots) return fail(KVS_E_INVAL, "kvs_paged_decode_scored_select_fp8: NULL tensor");
  return run_scored("kvs_paged_decode_scored_select_fp8", q, k_pool, v_pool, k_scale, v_scale, true, num_blocks,
                    block_tables, max_blocks, ctx_lens, batch, max_ctx, hq, hkv, d, scale, new_k, new_v, dst_slots,
                    slot_scores, slot_stride, o, lse_opt, workspace, workspace_bytes, stream, slot_pos, cap, alpha,
                    next_pos, next_dst_slots);
}
