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
//   * A workgroup = 8 wavefronts = 256 query rows of one query head; each wavefront owns a
//     strip of 32 rows.  The product is computed transposed, S^T = K . Q^T: keys are the M
//     dimension, query rows the N dimension, so every lane holds 16 scores of a single query
//     row per 32-key tile.  The row maximum is an in-lane max plus one lane-half swap, the row
//     scale of O is a per-lane scalar, and the exponentiated scores are already in the B
//     operand layout of O^T = V^T . P^T: P never goes through LDS.
//   * K tiles (64 keys) go from memory straight into LDS in their natural row-major layout
//     (buffer loads with an LDS destination, range-checked against the prompt), rows padded by
//     one chunk so the operand reads are free of bank conflicts.  V tiles go through registers
//     and are stored transposed (V^T, channel rows of 64 keys): 16-byte operand reads of V^T
//     run at twice the LDS rate of the transposing 8-byte read.  The key order of the first
//     product is permuted so that each lane's share of P^T is 8 consecutive keys, so the V^T
//     operand is one 16-byte read.
//   * Ping-pong: per tile a wavefront has a matrix phase (O^T product of the previous tile,
//     S^T product of this one) and a vector phase (mask, row maximum, exponentials).  The two
//     groups of four wavefronts (one of each on every SIMD) run one phase apart, separated by
//     workgroup barriers, so each SIMD's matrix core works for one group while its vector unit
//     works for the other.  Loads are issued two phases before their tile is first read.
//   * Q stays in registers for the whole key loop.  Every wavefront runs every key tile its
//     workgroup visits (the barriers of the ping-pong are shared); the causal mask applies to
//     any tile that reaches past a wavefront's first row, so the tiles that lie wholly past
//     its rows are computed and masked to P = 0.  O is rescaled only when a row maximum grows
//     by more than 2^8 (wave-uniform branch).
//   * Query tiles are aligned to the end of each prompt, so a prompt's partial tile is its
//     first (the one with the fewest key tiles) and its longest rows are all real.
//   * Workgroups are remapped so that each XCD (8 per chip, each with its own L2) works on
//     one KV head at a time, heaviest (last) query tiles first.
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kWaves = 8;
constexpr int kGroupWaves = 4;   // wavefronts per ping-pong group
constexpr int kBQ = 256;   // query rows per workgroup
constexpr int kBK = 64;    // keys per tile
constexpr int kRowsPerWave = 32;
constexpr int kXcds = 8;

// LDS layouts (one 256-byte line spans the 64 banks):
//  * K: rows padded by one 16-byte chunk (KSTR bf16).  A lane group of the first product
//    reads one chunk of 16 consecutive rows, which the pad rotates onto all 64 banks; the
//    read addresses are one register plus immediates.
//  * V^T: channel rows of kBK keys padded by one chunk (VSTR bf16, 36 words): the 16-byte
//    reads of 16 consecutive channel rows land on distinct banks.

// s_waitcnt vmcnt(0) with the other counters left alone (gfx9 encoding: vmcnt 0, expcnt 7,
// lgkmcnt 15).
constexpr int kVmcntZero = 0x0F70;

// MFMA row m of the S^T product holds key kappa(m) of its 32-key tile: bits 2 and 3 of m are
// swapped.  With that order the 16 scores a lane half gets back cover 8 consecutive keys per
// 16-key step, so P^T needs no shuffling.
__device__ __forceinline__ int kappa(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <int D>
__global__ __launch_bounds__(kWaves * kWave, 1) void prefill_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_seqlens_k, int num_seqs, int total_tokens,
    int hq, int hkv, float c_log2, uint16_t* __restrict__ o, float* __restrict__ lse, float* __restrict__ rowmax,
    float* __restrict__ ell, int nqt, int total_items) {
  constexpr int KCU = D / 8;     // 16-byte chunks per tile row
  constexpr int ST1 = D / 16;    // k-steps of S^T = K Q^T
  constexpr int MT2 = D / 32;    // channel tiles of O^T
  constexpr int KS2 = kBK / 16;  // k-steps of O^T = V^T P^T
  constexpr int NT = kWaves * kWave;
  constexpr int KSTR = D + 8;           // bf16 per K row in LDS (one pad chunk)
  constexpr int KPOS = kBK * (KCU + 1);  // 16-byte positions of a K tile, pads included
  constexpr int KLD = (KPOS + NT - 1) / NT;   // K loads per lane per tile (the last one partial)
  constexpr int VSTR = kBK + 8;          // bf16 per V^T row in LDS
  constexpr int VITEMS = (kBK / 2) * KCU;   // (key pair, 16-byte channel chunk) items of a V tile
  // Triple-buffered tiles as distinct LDS objects: with the buffer of each access known at
  // compile time, the compiler can tell the loads into one buffer from the reads of another
  // and does not make those reads wait for the loads.
  __shared__ __attribute__((aligned(16))) uint16_t ks0[kBK * KSTR], ks1[kBK * KSTR], ks2[kBK * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vs0[D * VSTR], vs1[D * VSTR], vs2[D * VSTR];
  auto kbuf = [&](int b) { return b == 0 ? ks0 : b == 1 ? ks1 : ks2; };   // b: a constant at every call
  auto vbuf = [&](int b) { return b == 0 ? vs0 : b == 1 ? vs1 : vs2; };

  // ---- XCD-aware work mapping: item order (g, s, query tile counted from the prompt's end,
  // head in group).
  const int per_xcd = gridDim.x / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= total_items) return;
  const int G = hq / hkv;
  int rest = item;
  const int hl = rest % G; rest /= G;
  const int te = rest % nqt; rest /= nqt;   // te = 0: the prompt's last kBQ rows
  const int s = rest % num_seqs;
  const int g = rest / num_seqs;
  const int h = g * G + hl;
  // Query rows [base, base + m) of Q; keys [kbase_tok, kbase_tok + n) of K/V.  A chunk's row r
  // sits at prompt position qoff + r (the chunk ends the keys), which the causal rule uses.
  const int base = cu_seqlens[s];
  const int m = cu_seqlens[s + 1] - base;
  const int kbase_tok = cu_seqlens_k ? cu_seqlens_k[s] : base;
  const int n = cu_seqlens_k ? cu_seqlens_k[s + 1] - kbase_tok : m;
  const int qoff = n - m;
  const int r0 = m - (te + 1) * kBQ;   // negative for a prompt's first, partial tile
  if (r0 + kBQ <= 0) return;

  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: branches on it stay scalar
  const int col = lane % 32, half = lane / 32;
  const int grp = w / kGroupWaves;       // ping-pong group; wavefronts w and w +- 4 share a SIMD
  const int R = r0 + (2 * (w % kGroupWaves) + grp) * kRowsPerWave;   // first row of this wavefront's strip
  const int row = R + col;               // this lane's query row (N index), chunk-local
  const int kend = min(qoff + r0 + kBQ, n);
  const int ntiles = (kend + kBK - 1) / kBK;

  // B operand of S^T: Q^T[d][row] for each 16-wide d step.
  bf16x8 qf[ST1];
#pragma unroll
  for (int st = 0; st < ST1; ++st) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (row >= 0) x = *reinterpret_cast<const u32x4*>(q + ((size_t)(base + row) * hq + h) * D + st * 16 + half * 8);
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

  // ---- Tile loads.  K: load `it` of wave w fills LDS chunk positions p = (it*kWaves + w)*64 +
  // lane of a tile (1 KB per wave per load); position p is chunk p % (KCU+1) of row
  // p / (KCU+1), the pad position taking a copy of the row's last chunk (same cache line).
  // K rows past the prompt only meet masked scores (replaced by -inf), so whatever LDS holds
  // for them does not matter.  V: thread e < VITEMS loads chunk cc of keys 2p and 2p+1 into
  // registers (rows past the prompt read as zero: P is zero there and 0 * garbage could be
  // NaN) and later stores the 8 channel pairs transposed.  Buffer resources cover this
  // sequence's rows of KV head g only, so the ragged last tile needs no branch and a tile's
  // address is a scalar move of the resource base.
  constexpr int kRowBytes = 2 * D;
  const int row_pitch = hkv * kRowBytes;                           // bytes between consecutive keys
  const int seq_bytes = (n - 1) * row_pitch + kRowBytes;           // this head's rows of the prompt
  const int tile_bytes = kBK * row_pitch;
  const char* kbase = reinterpret_cast<const char*>(k + ((size_t)kbase_tok * hkv + g) * D);
  const char* vbase = reinterpret_cast<const char*>(v + ((size_t)kbase_tok * hkv + g) * D);
  int koff[KLD];
#pragma unroll
  for (int it = 0; it < KLD; ++it) {
    const int p = (it * kWaves + w) * kWave + lane;
    const int r = p / (KCU + 1), c = p % (KCU + 1);
    koff[it] = r * row_pitch + min(c, KCU - 1) * 16;
  }
  // V item of this thread: wavefront e / 64 and lane e % 64 pick key pair p and chunk cc so
  // that 16 lanes read one 256-byte row.
  const bool v_item = tid < VITEMS;   // every thread when D = 128, half of them when D = 64
  const int vp = ((tid / kWave) % 2) * 16 + lane % 16;
  const int vcc = (tid / kWave / 2) * 4 + lane / 16;
  const int voff = 2 * vp * row_pitch + vcc * 16;
  u32x4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
  auto rsrc = [&](const char* src, int kt) {
    const int skip = kt * tile_bytes;    // < seq_bytes for every tile that is loaded
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src) + skip, 0, seq_bytes - skip, kBufferFlags);
  };
  // buf: a constant at every call
  auto load_k = [&](int kt, int buf) {
    uint16_t* dst = kbuf(buf);
    const __amdgpu_buffer_rsrc_t rs = rsrc(kbase, kt);
#pragma unroll
    for (int it = 0; it < KLD; ++it)
      if ((it * kWaves + w) * kWave < KPOS)   // wave-uniform; the last load of a tile is partial
        buffer_load_lds16(rs, &dst[(it * kWaves + w) * kWave * 8], koff[it]);
  };
  auto load_v = [&](int kt) {            // V tile kt into registers
    const __amdgpu_buffer_rsrc_t rs = rsrc(vbase, kt);
    if (v_item) {
      va = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, 0);
      vb = __builtin_amdgcn_raw_buffer_load_b128(rs, voff + row_pitch, 0, 0);
    }
  };
  auto store_v = [&](int buf) {          // the registers of load_v into V^T buffer buf
    uint16_t* vt = vbuf(buf);
    if (v_item) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // channel vcc*8 + j of keys 2vp (low half) and 2vp + 1 (high half)
        const uint32_t word = (j % 2 == 0) ? __builtin_amdgcn_perm(vb[j / 2], va[j / 2], 0x05040100u)
                                           : __builtin_amdgcn_perm(vb[j / 2], va[j / 2], 0x07060302u);
        *reinterpret_cast<uint32_t*>(&vt[(vcc * 8 + j) * VSTR + 2 * vp]) = word;
      }
    }
  };

  // ---- Operand reads.
  // S^T A operand, fragment f = 2*st + mt: lane col reads K row mt*32 + kappa(col), chunk
  // 2*st + half.
  const int kofs = kappa(col) * KSTR + half * 8;
  constexpr int NF1 = 2 * ST1, NG1 = NF1 / 4;
  auto kfrag = [&](const uint16_t* ks, int f) {
    return *reinterpret_cast<const u32x4*>(&ks[(f % 2) * 32 * KSTR + (f / 2) * 16 + kofs]);
  };
  // O^T A operand, fragment f = ks2*MT2 + mt: lane l reads V^T row 32*mt + l%32 (a channel),
  // keys 16*ks2 + 8*half + 0..7.
  const int vofs = col * VSTR + half * 8;
  constexpr int NF2 = MT2 * KS2;
  auto vfrag = [&](const uint16_t* vt, int f) {
    return *reinterpret_cast<const u32x4*>(&vt[(f % MT2) * 32 * VSTR + (f / MT2) * 16 + vofs]);
  };
  auto mfma1 = [&](f32x16 (&sacc)[2], int f, u32x4 a) {
    sacc[f % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), qf[f / 2], sacc[f % 2], 0, 0, 0);
  };
  auto mfma2 = [&](const bf16x8 (&pf)[KS2], int f, u32x4 a) {
    acc_o[f % MT2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pf[f / MT2], acc_o[f % MT2],
                                                              0, 0, 0);
  };
  // sacc[mt][i] is key kb + 32*mt + 16*(i/8) + 8*half + i%8 against `row` (raw dot products).
  // P^T as B operands: k-step ks2 holds keys 16*ks2 + 8*half + 0..7, i.e. sacc[ks2/2][8*(ks2%2) + 0..7].
  auto softmax_step = [&](f32x16 (&sacc)[2], bf16x8 (&pf)[KS2], int ks2, float& psum) {
    const int mt = ks2 / 2, i0 = 8 * (ks2 % 2);
    u32x4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][i0 + 2 * j], c_log2, -m_ref));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mt][i0 + 2 * j + 1], c_log2, -m_ref));
      psum += p0 + p1;
      x[j] = pack_bf16x2(p0, p1);
    }
    pf[ks2] = __builtin_bit_cast(bf16x8, x);
  };
  // Running maximum (log2 units) after a tile, then the lazy rescale of O and l when some row
  // moved past m_ref + kLazy (wave-uniform branch, rare after the first tiles).
  auto update_max = [&](float bm) {
    bm = half_max(bm) * c_log2;
    m_true = fmaxf(m_true, bm);
    if (__ballot(m_true > m_ref + kLazy) != 0ull) {
      const float corr = __builtin_amdgcn_exp2f(m_ref - m_true);
      m_ref = m_true;
      l_lane *= corr;
#pragma unroll
      for (int mt = 0; mt < MT2; ++mt) acc_o[mt] *= corr;
    }
  };
  auto tile_max = [&](const f32x16 (&sacc)[2]) {   // four independent chains, then combined
    float bm[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) bm[2 * mt + i / 8] = fmaxf(bm[2 * mt + i / 8], sacc[mt][i]);
    return fmaxf(fmaxf(bm[0], bm[1]), fmaxf(bm[2], bm[3]));
  };
  // Products of one tile on their own (first tile, last pipelined tile, diagonal tiles):
  // operand fragments are read from LDS in groups of four, the next group's reads in flight
  // while the current group's products run.
  auto gemm1 = [&](const uint16_t* ks, f32x16 (&sacc)[2]) {
    u32x4 fr[2][4];
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int j = 0; j < 4; ++j) fr[0][j] = kfrag(ks, j);
#pragma unroll
    for (int grp = 0; grp < NG1; ++grp) {
      if (grp + 1 < NG1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) fr[(grp + 1) & 1][j] = kfrag(ks, 4 * (grp + 1) + j);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) mfma1(sacc, 4 * grp + j, fr[grp & 1][j]);
    }
  };
  // The O^T product takes all its V^T fragments from registers: they are read during the
  // preceding vector phase, when this wavefront's LDS reads are otherwise idle, so the matrix
  // phase starts without waiting on LDS.
  u32x4 vpre[NF2];
  auto prefetch_v = [&](const uint16_t* vs) {
#pragma unroll
    for (int f = 0; f < NF2; ++f) vpre[f] = vfrag(vs, f);
  };
  auto gemm2 = [&](const bf16x8 (&pf)[KS2]) {
#pragma unroll
    for (int f = 0; f < NF2; ++f) mfma2(pf, f, vpre[f]);
  };

  // ---- Ping-pong schedule.  K tile t lives in ks{t%3}, V tile t in vs{t%3}.  Per tile t a
  // wavefront's work is a matrix phase M(t-1) (O^T += V_{t-1}^T P_{t-1}^T, then S_t = K_t Q^T)
  // and a vector phase X(t) (mask, maximum, rescale, P_t), each closed by a barrier.  Both
  // groups run the same sequence, group 1 one barrier behind (it passes one extra barrier at
  // the start, group 0 one at the end), so in every phase one group is in its matrix phase and
  // the other in its vector phase.  Iteration t issues K_{t+2} (into LDS) and V_{t+1} (into
  // registers, stored transposed at its end); their buffers were last read by M(t-2), at least
  // one barrier earlier for either group, and they are first read by M(t+1), after the
  // barrier that follows every wavefront's wait for its own loads and V^T stores.
  // Every wavefront does every tile of the workgroup: a tile past all of its rows is fully
  // masked (P = 0) by the same code that masks the diagonal, which keeps the loop free of
  // branches around the products.
  f32x16 sacc[2];
  bf16x8 pf[KS2];
  auto vector_phase = [&](int t) {                 // X(t)
    const int kb = t * kBK;
    if (kb + kBK - 1 > qoff + R) {   // wave-uniform: mask keys past the row
      const int lim = qoff + max(row, 0) - kb - 8 * half;   // rows before the prompt (never stored) act as row 0
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (mt * 32 + 16 * (i / 8) + (i % 8) > lim) sacc[mt][i] = -INFINITY;
    }
    update_max(tile_max(sacc));
    float psum[KS2];   // one chain per key step, added up at the end
#pragma unroll
    for (int ks = 0; ks < KS2; ++ks) {
      psum[ks] = 0.f;
      softmax_step(sacc, pf, ks, psum[ks]);
    }
    l_lane += (psum[0] + psum[1]) + (psum[2] + psum[3]);
  };
  auto close_phase = [&](bool wait_loads) {
    if (wait_loads) __builtin_amdgcn_s_waitcnt(kVmcntZero);
    __syncthreads();
  };
  auto iteration = [&](const int b, int t) {       // 0 < t < ntiles; b = t % 3, a constant
    if (t + 2 < ntiles) load_k(t + 2, (b + 2) % 3);
    if (t + 1 < ntiles) load_v(t + 1);
    gemm2(pf);                                     // M(t-1), V_{t-1} fragments in registers
    gemm1(kbuf(b), sacc);
    close_phase(false);
    vector_phase(t);
    prefetch_v(vbuf(b));                           // V_t for M(t)
    if (t + 1 < ntiles) store_v((b + 1) % 3);
    close_phase(true);
  };
  load_k(0, 0);
  if (1 < ntiles) load_k(1, 1);
  load_v(0);
  store_v(0);
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  if (grp == 1) __syncthreads();
  // t = 0: no O^T product yet
  if (2 < ntiles) load_k(2, 2);
  if (1 < ntiles) load_v(1);
  gemm1(ks0, sacc);
  close_phase(false);
  vector_phase(0);
  prefetch_v(vs0);
  if (1 < ntiles) store_v(1);
  close_phase(true);
  for (int t = 1; t < ntiles; t += 3) {
    iteration(1, t);
    if (t + 1 < ntiles) iteration(2, t + 1);
    if (t + 2 < ntiles) iteration(0, t + 2);
  }
  // t = ntiles: the last O^T product (all loads have landed)
  {
    gemm2(pf);
    close_phase(false);
    close_phase(false);
  }
  if (grp == 0) __syncthreads();

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m_ref + log2 l)
  const float l = half_sum(l_lane);   // sum of exp2(x - m_ref)
  // O goes out through LDS: a lane holds half the channels of one row in 4-channel pieces, so
  // stored directly every instruction would write 8 bytes into each of 32 rows; staged as
  // row-major rows (stride D + 8, 16-byte aligned), 16 lanes write one row's 2D bytes as
  // whole lines (bench layer: 134.5 us without any O store against 144 with the direct one).
  // The tile buffers are free once every wavefront has passed the last product; two
  // wavefronts' strips fit one buffer.
  constexpr int OSTR = D + 8;
  __syncthreads();
  uint16_t* stage = (w < 2 ? ks0 : w < 4 ? ks1 : w < 6 ? ks2 : vs0) + (w & 1) * (kRowsPerWave * OSTR);
  {
    const float inv = 1.f / l;   // rows before the prompt (row < 0) are staged but never stored
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        // acc_o[mt][4*i4 + 0..3] are channels mt*32 + 8*i4 + 4*half + 0..3 of row `col`
        u32x2 x;
        x[0] = pack_bf16x2(acc_o[mt][4 * i4 + 0] * inv, acc_o[mt][4 * i4 + 1] * inv);
        x[1] = pack_bf16x2(acc_o[mt][4 * i4 + 2] * inv, acc_o[mt][4 * i4 + 3] * inv);
        *reinterpret_cast<u32x2*>(&stage[col * OSTR + mt * 32 + 8 * i4 + 4 * half]) = x;
      }
  }
  __syncthreads();
  {
    constexpr int kChunks = D / 8;                  // 16-byte pieces of a row
    constexpr int kRowsPerIt = kWave / kChunks;
#pragma unroll
    for (int it = 0; it < kRowsPerWave / kRowsPerIt; ++it) {
      const int rr = it * kRowsPerIt + lane / kChunks, cc = lane % kChunks;
      const u32x4 x = *reinterpret_cast<const u32x4*>(&stage[rr * OSTR + cc * 8]);
      if (R + rr >= 0) *reinterpret_cast<u32x4*>(o + ((size_t)(base + R + rr) * hq + h) * D + cc * 8) = x;
    }
  }
  if (row >= 0) {   // rows before the prompt belong to no query (every row is < m)
    if (half == 0) {
      const size_t li = (size_t)h * total_tokens + base + row;
      if (lse) lse[li] = (m_ref + log2f(l)) * kLn2;
      if (rowmax) rowmax[li] = m_true * kLn2;
      if (ell) ell[li] = l * __builtin_amdgcn_exp2f(m_ref - m_true);   // sum of exp(s - rowmax)
    }
  }
}

}  // namespace
}  // namespace kvs

using namespace kvs;

static int run_prefill(const char* name, const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                       const int32_t* cu_seqlens_k, int num_seqs, int total_tokens, int max_seqlen, int max_seqlen_k,
                       int hq, int hkv, int d, float scale, void* o, float* lse, float* rowmax_opt, float* ell_opt,
                       void* stream) {
  if (!q || !k || !v || !cu_seqlens || !o) return fail(KVS_E_INVAL, "%s: NULL tensor", name);
  if (num_seqs < 0 || total_tokens < 0 || max_seqlen < 0 || max_seqlen_k < 0 || hq <= 0 || hkv <= 0 || hq % hkv ||
      hq / hkv > 16 || (d != 64 && d != 128) || !(scale > 0.f))
    return fail(KVS_E_INVAL, "%s: bad shape (hq=%d hkv=%d d=%d)", name, hq, hkv, d);
  if (num_seqs == 0 || max_seqlen == 0 || total_tokens == 0) return KVS_OK;
  if ((long long)max_seqlen_k * hkv * d * 2 > 0x7fffffffll)   // K/V rows of one prompt are addressed with 32-bit offsets
    return fail(KVS_E_INVAL, "%s: prompt of %d tokens x %d KV heads too large", name, max_seqlen_k, hkv);
  const int nqt = (max_seqlen + kBQ - 1) / kBQ;
  const long long items = (long long)hkv * num_seqs * nqt * (hq / hkv);
  if (items > (1ll << 30)) return fail(KVS_E_INVAL, "%s: grid too large", name);
  const int grid = (int)((items + kXcds - 1) / kXcds * kXcds);
  const float c = scale * kLog2e;
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kk = static_cast<const uint16_t*>(k);
  auto* vv = static_cast<const uint16_t*>(v);
  auto* oo = static_cast<uint16_t*>(o);
  if (d == 128)
    hipLaunchKernelGGL(prefill_kernel<128>, dim3(grid), dim3(kWaves * kWave), 0, as_stream(stream), qq, kk, vv,
                       cu_seqlens, cu_seqlens_k, num_seqs, total_tokens, hq, hkv, c, oo, lse, rowmax_opt, ell_opt, nqt,
                       (int)items);
  else
    hipLaunchKernelGGL(prefill_kernel<64>, dim3(grid), dim3(kWaves * kWave), 0, as_stream(stream), qq, kk, vv,
                       cu_seqlens, cu_seqlens_k, num_seqs, total_tokens, hq, hkv, c, oo, lse, rowmax_opt, ell_opt, nqt,
                       (int)items);
  return launch_status(name);
}

extern "C" int kvs_prefill_attn_lse(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                    int num_seqs, int total_tokens, int max_seqlen, int hq, int hkv, int d,
                                    float scale, void* o, float* lse, float* rowmax_opt, float* ell_opt,
                                    void* stream) {
  return run_prefill("kvs_prefill_attn_lse", q, k, v, cu_seqlens, nullptr, num_seqs, total_tokens, max_seqlen,
                     max_seqlen, hq, hkv, d, scale, o, lse, rowmax_opt, ell_opt, stream);
}

extern "C" int kvs_prefill_attn_lse_chunk(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                                          const int32_t* cu_seqlens_k, int num_seqs, int total_q, int max_q,
                                          int max_k, int hq, int hkv, int d, float scale, void* o, float* lse,
                                          float* rowmax_opt, float* ell_opt, void* stream) {
  if (!cu_seqlens_k) return fail(KVS_E_INVAL, "kvs_prefill_attn_lse_chunk: NULL tensor");
  if (max_k < max_q) return fail(KVS_E_INVAL, "kvs_prefill_attn_lse_chunk: max_k < max_q");
  return run_prefill("kvs_prefill_attn_lse_chunk", q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, max_q,
                     max_k, hq, hkv, d, scale, o, lse, rowmax_opt, ell_opt, stream);
}
