// Observation-window score S, rebuilt from the LSE the prefill saved.
//
// [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM", Key techniques,
// 2. "Attention modification" (the PyramidKV-style score and the modified-FlashAttention
// figure, second Fig. 7):
//   * the last alpha prompt positions form the window; the score of token i is the sum of
//     its softmax values over the window rows;
//   * softmax values come back from the saved row statistics, p = exp(qk - rowmax) / l,
//     which is exp(qk - LSE); a row-wise sum then gives S;
//   * the loop order is swapped from q.k to k.q so that the sum over window rows is a
//     register sum and no block has to talk to another;
//   * causality and the window bound mean only window rows are visited (about n * alpha
//     pairs instead of n * n).
//
// MI355X form.  A workgroup (8 wavefronts) owns 128 consecutive keys of one KV head (mapped to
// the XCD that ran that head's prefill, whose L2 holds the keys).  Wavefronts w and w + 4 own
// the same 32 keys, which are the N dimension of a bf16 32x32x16 MFMA; the G * a window rows
// of the group's query heads are the M dimension, staged through LDS in chunks of 128 rows
// (one chunk for 4 query heads x a 32-token window) together with LSE * log2(e) and each
// row's causal limit, and wavefront w takes M tiles 2(w/4) and 2(w/4) + 1 of every chunk.
// Two wavefronts per SIMD: one's exponentials run beside the other's products.  Every lane
// ends up holding 16 (row, key) products for one key per M tile, so the window sum is a
// register sum plus one cross-lane add and one add of the two wavefronts' halves through
// LDS: the pages' "row sum in registers".  The key fragment is read once per wavefront and
// kept in registers; the window rows, their LSE and their limits are fetched in one round
// trip per chunk; nothing but the window rows is ever touched.
#include "kvs_common.h"

namespace kvs {
namespace {

constexpr int kWaves = 8;
constexpr int kKeyWaves = 4;    // wavefronts across the keys; the other factor 2 splits the rows
constexpr int kKeysPerWave = 32;
constexpr int kKeysPerWG = kKeyWaves * kKeysPerWave;
constexpr int kRowChunk = 128;  // window rows staged in LDS at a time (4 M tiles, 2 per wavefront)
constexpr int kXcds = 8;

template <int D>
__global__ __launch_bounds__(kWaves * kWave) void window_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ lse,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_seqlens_k, int total_tokens, int total_k,
    int alpha, int hq, int hkv, float c_log2, float* __restrict__ S, int nkt, int num_seqs, int total_items) {
  constexpr int kStride = D + 8;                       // bf16 per LDS row (16-byte pad)
  __shared__ __attribute__((aligned(16))) uint16_t qs[kRowChunk * kStride];
  __shared__ float lse2[kRowChunk];
  __shared__ int jlim[kRowChunk];
  __shared__ float half_sums[kKeysPerWG];

  // Q rows and LSE of prompt s: [base, base + m); its keys and scores: [kbase, kbase + n).  The
  // Q rows are the prompt's last m positions (a chunk that ends the prompt, or all of it).
  // XCD-aware mapping (workgroups go to the 8 XCDs round robin): XCD x takes a contiguous run
  // of items ordered (KV head, prompt, key tile), the order the prefill gives its XCDs, so a
  // head's keys are read where the prefill just left them in L2.
  const int per_xcd = gridDim.x / kXcds;
  const int item = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
  if (item >= total_items) return;
  const int kt = item % nkt;
  const int s = (item / nkt) % num_seqs;
  const int g = item / nkt / num_seqs;
  const int base = cu_seqlens[s];
  const int m = cu_seqlens[s + 1] - base;
  const int kbase = cu_seqlens_k ? cu_seqlens_k[s] : base;
  const int n = cu_seqlens_k ? cu_seqlens_k[s + 1] - kbase : m;
  const int kb_wg = kt * kKeysPerWG;
  if (kb_wg >= n) return;   // workgroup-uniform, before any barrier
  const int G = hq / hkv;
  const int a = alpha < n ? alpha : n;
  const int rows = G * a;                               // window rows of this KV head's group

  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  const int half = lane / 32, col = lane % 32;
  const int kw = w % kKeyWaves, rh = w / kKeyWaves;     // key slice and row half of this wavefront
  const int key = kb_wg + kw * kKeysPerWave + col;      // this lane's key (N index)

  // B operand: K^T[d][key] for every 16-wide d step, kept in registers.
  bf16x8 kf[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (key < n) v = *reinterpret_cast<const u32x4*>(k + ((size_t)(kbase + key) * hkv + g) * D + st * 16 + half * 8);
    kf[st] = __builtin_bit_cast(bf16x8, v);
  }

  float acc_sum = 0.f;
  for (int r0 = 0; r0 < rows; r0 += kRowChunk) {
    // Stage kRowChunk window rows: row r = (local head r / a, window position r % a).  All of
    // a thread's loads (its Q pieces, and the LSE of row tid) are issued before any LDS
    // store, so the staging costs one memory round trip, not one per load.
    constexpr int kStage = kRowChunk * (D / 8) / (kWaves * kWave);
    u32x4 staged[kStage];
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int e = tid + i * kWaves * kWave;
      const int r = e / (D / 8), cc = e % (D / 8);
      const int rr = r0 + r;
      staged[i] = u32x4{0u, 0u, 0u, 0u};
      if (rr < rows && m - a + rr % a >= 0) {   // a window row before the chunk is not counted
        const int h = g * G + rr / a, j = m - a + rr % a;   // chunk-local row of window position n - a + rr % a
        staged[i] = *reinterpret_cast<const u32x4*>(q + ((size_t)(base + j) * hq + h) * D + cc * 8);
      }
    }
    float row_lse = 0.f;
    int row_lim = -1;                                   // padding row: masks every key
    if (tid < kRowChunk) {
      const int rr = r0 + tid;
      if (rr < rows && m - a + rr % a >= 0) {
        const int h = g * G + rr / a, j = m - a + rr % a;
        row_lse = lse[(size_t)h * total_tokens + base + j];
        row_lim = n - a + rr % a;                       // the row's prompt position: keys up to it count
      }
    }
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int e = tid + i * kWaves * kWave;
      *reinterpret_cast<u32x4*>(&qs[(e / (D / 8)) * kStride + (e % (D / 8)) * 8]) = staged[i];
    }
    if (tid < kRowChunk) {
      lse2[tid] = row_lse * kLog2e;
      jlim[tid] = row_lim;
    }
    __syncthreads();
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
      const int mt = 2 * rh + mi;
      f32x16 acc = {};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(&qs[(mt * 32 + col) * kStride + st * 16 + half * 8]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av), kf[st], acc, 0, 0, 0);
      }
      // acc[i] is window row mt*32 + 8*(i/4) + 4*half + i%4 against this lane's key.
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = mt * 32 + 8 * (i / 4) + 4 * half + (i % 4);
        const float p = __builtin_amdgcn_exp2f(acc[i] * c_log2 - lse2[r]);
        acc_sum += key <= jlim[r] ? p : 0.f;
      }
    }
    __syncthreads();   // the next chunk's staging overwrites qs, lse2 and jlim
  }
  acc_sum += wave_xor(acc_sum, 32);
  if (rh == 1 && half == 0) half_sums[kw * kKeysPerWave + col] = acc_sum;
  __syncthreads();
  if (rh == 0 && half == 0 && key < n)
    S[(size_t)g * total_k + kbase + key] = acc_sum + half_sums[kw * kKeysPerWave + col];
}

}  // namespace
}  // namespace kvs

using namespace kvs;

static int run_window(const char* name, const void* q, const void* k, const float* lse, const int32_t* cu_seqlens,
                      const int32_t* cu_seqlens_k, int num_seqs, int total_tokens, int total_k, int max_seqlen_k,
                      int alpha, int hq, int hkv, int d, float scale, float* scores, void* stream) {
  if (!q || !k || !lse || !cu_seqlens || !scores) return fail(KVS_E_INVAL, "%s: NULL tensor", name);
  if (num_seqs < 0 || total_tokens < 0 || total_k < 0 || max_seqlen_k < 0 || hq <= 0 || hkv <= 0 || hq % hkv ||
      hq / hkv > 16 || (d != 64 && d != 128) || !(scale > 0.f))
    return fail(KVS_E_INVAL, "%s: bad shape (hq=%d hkv=%d d=%d)", name, hq, hkv, d);
  if (alpha < 1) return fail(KVS_E_INVAL, "%s: alpha must be >= 1", name);
  if (num_seqs == 0 || max_seqlen_k == 0) return KVS_OK;
  const int nkt = (max_seqlen_k + kKeysPerWG - 1) / kKeysPerWG;
  const long long items = (long long)nkt * hkv * num_seqs;
  if (items > (1ll << 30)) return fail(KVS_E_INVAL, "%s: grid too large", name);
  const dim3 grid((unsigned)((items + kXcds - 1) / kXcds * kXcds));
  const float c = scale * kLog2e;
  auto* qq = static_cast<const uint16_t*>(q);
  auto* kk = static_cast<const uint16_t*>(k);
  if (d == 128)
    hipLaunchKernelGGL(window_score_kernel<128>, grid, dim3(kWaves * kWave), 0, as_stream(stream), qq, kk, lse,
                       cu_seqlens, cu_seqlens_k, total_tokens, total_k, alpha, hq, hkv, c, scores, nkt, num_seqs,
                       (int)items);
  else
    hipLaunchKernelGGL(window_score_kernel<64>, grid, dim3(kWaves * kWave), 0, as_stream(stream), qq, kk, lse,
                       cu_seqlens, cu_seqlens_k, total_tokens, total_k, alpha, hq, hkv, c, scores, nkt, num_seqs,
                       (int)items);
  return launch_status(name);
}

extern "C" int kvs_window_score(const void* q, const void* k, const float* lse, const int32_t* cu_seqlens,
                                int num_seqs, int total_tokens, int max_seqlen, int alpha, int hq, int hkv, int d,
                                float scale, float* scores, void* stream) {
  return run_window("kvs_window_score", q, k, lse, cu_seqlens, nullptr, num_seqs, total_tokens, total_tokens,
                    max_seqlen, alpha, hq, hkv, d, scale, scores, stream);
}

extern "C" int kvs_window_score_chunk(const void* q, const void* k, const float* lse, const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_k, int num_seqs, int total_q, int total_k, int max_k,
                                      int alpha, int hq, int hkv, int d, float scale, float* scores, void* stream) {
  if (!cu_seqlens_k) return fail(KVS_E_INVAL, "kvs_window_score_chunk: NULL tensor");
  return run_window("kvs_window_score_chunk", q, k, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k,
                    max_k, alpha, hq, hkv, d, scale, scores, stream);
}
