// Sparse read of the latent cache: the indexer pass and the top-k selection
// ("DeepSeek's Config Says 16 KV Heads, Its Cache Holds a Ninth of That",
// section 6, "Sparse attention": a small scorer of 64 heads x 128 dimensions
// rates every earlier token for each new token, and attention then reads only
// the 2,048 best; the full latent cache stays resident, plus one indexer key
// per token). The decode over the selected tokens is the gather mode of the
// decode kernels.
//
// Score (a reading; the pages give the scorer's size, not its formula):
//   I[b][j][t] = sum_h w[b][j][h] * max(0, q_idx[b][j][h] . k_idx[b][t])
// Selection: of the tokens query j sees (t <= L - q_len + j), the topk with
// the highest scores, equal scores going to the smaller token index, listed
// in increasing token order.
#include <map>
#include <mutex>

#include "mla_common.h"
#include "mla_append.h"
#include "mla_decode_common.h"
#include "mla_launch.h"

namespace mla {

using namespace dec;

namespace {

constexpr int kIH = 64;   // indexer heads of the MFMA kernel
constexpr int kID = 128;  // indexer key width of the MFMA kernel
constexpr int kIRow = kID * 2;                         // 256 bytes per bf16 key
constexpr int kIChunk = 32;                            // tokens per chunk: two groups of 16
constexpr int kIChunkBytes = kIChunk * kIRow;          // 8 KB
constexpr int kIRing = 4;                              // chunk slots per wave
constexpr int kIWaveChunks = 8;                        // chunks per wave
constexpr int kIdxTok = 4 * kIWaveChunks * kIChunk;    // 1,024 tokens per block
constexpr int kIChunkLoads = kIChunk * kIRow / 1024;   // 8 direct-to-LDS loads per chunk
constexpr size_t kIRingBytes = (size_t)4 * kIRing * kIChunkBytes;  // 131,072 B
constexpr int kIQBytes = kIH * kID * 2;                // 16 KB: the query's 64 x 128 bf16
constexpr size_t kILds = kIRingBytes + kIQBytes + kIH * 4;  // + the 64 head weights
static_assert(kILds <= 160 * 1024, "LDS of one CU");

constexpr int kTkThreads = 1024;
constexpr int kTkWaves = kTkThreads / 64;
constexpr int kTkCoarseBits = 12;              // coarse bins: the top 12 bits of a key
constexpr int kTkCoarse = 1 << kTkCoarseBits;
constexpr int kTkWsRow = kTkCoarse + 4;        // workspace words per query: counts, NaN flag
constexpr int kTkHistTok = 4096;               // scores per histogram block (16 per thread)
constexpr int kTkCand = 8192;                  // keys of the k-th key's coarse bin gathered in LDS
constexpr int kTkBinBits = 10;
constexpr int kTkBins = 1 << kTkBinBits;
constexpr int kTkBatch = 16;                   // score loads in flight per thread
constexpr int kTkOut = 8;                      // 64-key chunks read ahead in the output passes
constexpr int kTkRegKeys = 32;                 // register-resident keys per lane
constexpr int kTkRegSpan = 64 * kTkRegKeys;    // tokens per wave
constexpr int kTkRegTok = kTkWaves * kTkRegSpan;  // 32,768 tokens per block

// ---------------------------------------------------------------------------
// indexer key append: row n -> slot pos[n] of sequence seq_idx[n]
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void index_append_kernel(int dI, int page,
                                                          const T* __restrict__ k_new,
                                                          const int32_t* __restrict__ seq_idx,
                                                          const int32_t* __restrict__ pos,
                                                          const int32_t* __restrict__ page_table,
                                                          int batch, int max_pages,
                                                          T* __restrict__ icache,
                                                          int64_t num_pages) {
  index_append_row<T>(blockIdx.x, dI, page, k_new, seq_idx, pos, page_table, batch, max_pages,
                      icache, num_pages);
}

// ReLU that keeps a NaN (a NaN dot must not turn into a valid score)
__device__ __forceinline__ float relu_nan(float x) { return x < 0.0f ? 0.0f : x; }

// order-preserving 32-bit key of a score (-0 taken as +0); its top 12 bits
// are the top-k's coarse bin
__device__ __forceinline__ uint32_t score_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------------------
// index scores, bf16 MFMA: 64 heads x 128 dims. Block = kIdxTok tokens of one
// (sequence, query), four waves without block barriers; chunk c of wave w is
// the 32 tokens [kIdxTok * block + 32 (4 c + w), + 32), two groups of 16.
// Chunks stream through a 4-slot LDS ring per wave: a group's 16 keys are
// 4 KB of one page, copied with four 1 KB direct-to-LDS loads (page entries
// are scalar loads), chunk c + 4 going out as soon as chunk c's operands are
// in registers. Chunk k of key row r sits at 16 (k ^ (r & 15)) inside the
// row, the XOR applied on the global side, so the operand reads hit 16
// different bank groups. Per group: D[head][token] = q_idx[head][:] .
// k[token][:] on v_mfma_f32_16x16x32_bf16 (M = 16 heads, N = 16 tokens, 4
// head blocks x 4 k-steps), then lane (token n, head quarter kg) folds its 16
// heads with w * max(0, D) and the four quarters are summed with lane swaps.
// The scores are kept in registers and stored at the end (stores would share
// the load counter the ring waits on).
// kHist: the block also counts its visible scores into the top-k's coarse
// histogram as they are made (LDS atomics into the LDS that staged the
// query, once the query is in registers) and at the end adds the non-empty
// bins and the NaN flag to the query's workspace row, as topk_hist_kernel
// does; every wave then stays to the final barrier.
// ---------------------------------------------------------------------------
template <bool kHist>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void index_scores_mfma_kernel(int Q, int page, int max_seq_len, const bf16_t* __restrict__ q_idx,
                              const float* __restrict__ w_idx, const bf16_t* __restrict__ icache,
                              int64_t num_pages, const int32_t* __restrict__ page_table,
                              int max_pages, const int32_t* __restrict__ seq_lens,
                              float* __restrict__ scores, int ld, uint32_t* __restrict__ ws) {
  extern __shared__ u32x4_t lds[];
  const int b = blockIdx.y, j = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15, kg = lane >> 4;
  const int tb = blockIdx.x * kIdxTok + wave * kIChunk;  // chunk 0 of this wave
  const int L = seq_lens[b];
  const bool valid = L >= Q && L <= max_seq_len;  // else the selection reports it invalid
  // chunks of this wave that start before L (every wave stays for the barrier)
  const int nk =
      valid && L > tb ? min(kIWaveChunks, (L - tb + 4 * kIChunk - 1) / (4 * kIChunk)) : 0;
  char* const lbase = reinterpret_cast<char*>(lds);
  char* const ring = lbase + wave * kIRing * kIChunkBytes;
  char* const qs = lbase + kIRingBytes;                      // [head][dim] bf16
  const float* const wsh = reinterpret_cast<const float*>(qs + kIQBytes);
  // the query and the weights go to LDS once per block (1 KB loads i =
  // 4 w .. 4 w + 3 of wave w; the weights by wave 0), ahead of the keys
  {
    const bf16_t* qb = q_idx + ((size_t)b * Q + j) * kIH * kID;
    const uint32_t qd = __builtin_amdgcn_readfirstlane(lds_addr(qs));
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 4 * wave + ii;
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                   :
                   : "s"(qd + i * 1024), "v"((uint32_t)(i * 1024 + 16 * lane)), "s"(qb)
                   : "memory");
    }
    if (wave == 0)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2 nt"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(lds_addr(wsh))),
                     "v"((uint32_t)(4 * lane)), "s"(w_idx + ((size_t)b * Q + j) * kIH)
                   : "memory");
  }

  // load i of a group: lane l copies row 4 i + l / 16, chunk (l % 16) ^ row
  uint32_t doff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * i + (lane >> 4);
    doff[i] = (uint32_t)(r * kIRow + (((lane & 15) ^ r) << 4));
  }
  uint32_t okbits = 0u;  // bit 2 c + g: group g of chunk c has a valid page
  auto issue = [&](int c) {
    char* const slot = ring + (c % kIRing) * kIChunkBytes;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int tg = tb + 4 * kIChunk * c + 16 * g;  // wave-uniform; 16 tokens of one page
      const int pg = tg < L ? page_table[(size_t)b * max_pages + tg / page] : -1;
      const bool ok = pg >= 0 && (int64_t)pg < num_pages;
      okbits |= (ok ? 1u : 0u) << (2 * c + g);
      // (an invalid or unused group copies the pool's first rows, never read out)
      const bf16_t* src = icache + (ok ? ((size_t)pg * page + tg % page) * kID : 0);
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(slot + g * 16 * kIRow));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "s"(dst + i * 1024), "v"(doff[i]), "s"(src)
                     : "memory");
    }
  };
#pragma unroll
  for (int c = 0; c < kIRing; ++c)
    if (c < nk) issue(c);
  // own query (and weight) loads landed; then everyone's
  const int first = min(nk, kIRing);
  if (first >= 4)
    wait_vmcnt<4 * kIChunkLoads>();
  else if (first == 3)
    wait_vmcnt<3 * kIChunkLoads>();
  else if (first == 2)
    wait_vmcnt<2 * kIChunkLoads>();
  else if (first == 1)
    wait_vmcnt<kIChunkLoads>();
  else
    wait_vmcnt<0>();
  __syncthreads();
  if (!kHist && nk == 0) return;
  // queries: head 16 mt + n, dims 32 ks + 8 kg; weights of heads 16 mt + 4 kg + r
  bf16x8_t qa[4][4];
  float wv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[mt][ks] = *reinterpret_cast<const bf16x8_t*>(qs + (16 * mt + n) * kIRow + 64 * ks + 16 * kg);
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = wsh[16 * mt + 4 * kg + r];
  }
  uint32_t* const hist = reinterpret_cast<uint32_t*>(qs);  // kHist: [kTkCoarse] counts
  static_assert(kTkCoarse * 4 <= kIQBytes, "the histogram fits the query's staging");
  const int nvis = valid ? L - Q + j + 1 : 0;  // tokens the query sees
  bool nan = false;                            // a NaN among this lane's visible scores
  if constexpr (kHist) {
    __syncthreads();  // every wave has its query in registers
    for (int i = threadIdx.x; i < kTkCoarse; i += 256) hist[i] = 0u;
    __syncthreads();
  }

  float res[kIWaveChunks][2];  // lanes kg == 0: score of token 16 g + n of chunk c
#pragma unroll
  for (int c = 0; c < kIWaveChunks; ++c) {
    if (c >= nk) break;  // wave-uniform
    // chunk c landed; up to three later chunks may stay in flight
    const int later = min(nk - 1 - c, kIRing - 1);
    if (later >= 3)
      wait_vmcnt<3 * kIChunkLoads>();
    else if (later == 2)
      wait_vmcnt<2 * kIChunkLoads>();
    else if (later == 1)
      wait_vmcnt<kIChunkLoads>();
    else
      wait_vmcnt<0>();
    const char* const slot = ring + (c % kIRing) * kIChunkBytes;
    bf16x8_t kv[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kv[g][ks] = *reinterpret_cast<const bf16x8_t*>(slot + (16 * g + n) * kIRow +
                                                       (((4 * ks + kg) ^ n) << 4));
    if (c + kIRing < nk) {  // the slot is read: chunk c + 4 may land in it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(c + kIRing);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float part = 0.0f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kv[g][ks], d, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) part = fmaf(wv[mt][r], relu_nan(d[r]), part);
      }
      res[c][g] = row_sum4(part);
      if constexpr (kHist) {  // count the visible score into the coarse histogram
        const int t = tb + 4 * kIChunk * c + 16 * g + n;
        if (kg == 0 && t < nvis) {
          const float v = ((okbits >> (2 * c + g)) & 1u) ? res[c][g] : __int_as_float(0x7fc00000);
          nan |= v != v;
          atomicAdd(&hist[score_key(v) >> (32 - kTkCoarseBits)], 1u);
        }
      }
    }
  }
  wait_vmcnt<0>();
  float* out = scores + ((size_t)b * Q + j) * ld;
  if (kg == 0) {
#pragma unroll
    for (int c = 0; c < kIWaveChunks; ++c)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int t = tb + 4 * kIChunk * c + 16 * g + n;
        if (c < nk && t < L)
          out[t] = ((okbits >> (2 * c + g)) & 1u) ? res[c][g] : __int_as_float(0x7fc00000);
      }
  }
  if constexpr (kHist) {
    uint32_t* row = ws + ((size_t)b * Q + j) * kTkWsRow;
    if (__syncthreads_or(nan ? 1 : 0) && threadIdx.x == 0) row[kTkCoarse] = 1u;
    for (int i = threadIdx.x; i < kTkCoarse; i += 256)
      if (hist[i]) atomicAdd(&row[i], hist[i]);
  }
}

// index scores, any shape on the vector ALUs: one thread per token, the
// (sequence, query)'s indexer queries and weights in LDS as fp32
template <typename T>
__global__ __launch_bounds__(256) void index_scores_generic_kernel(
    int Q, int Hi, int dI, int page, int max_seq_len, const T* __restrict__ q_idx,
    const float* __restrict__ w_idx, const T* __restrict__ icache, int64_t num_pages,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int ld) {
  extern __shared__ float qs[];  // [Hi][dI], then w [Hi]
  const int b = blockIdx.y, j = blockIdx.z;
  const int L = seq_lens[b];
  if (L < Q || L > max_seq_len) return;
  const int tbase = blockIdx.x * 256;
  if (tbase >= L) return;
  float* ws = qs + Hi * dI;
  const T* qb = q_idx + ((size_t)b * Q + j) * Hi * dI;
  for (int i = threadIdx.x; i < Hi * dI; i += 256) qs[i] = Elt<T>::ld(qb + i);
  for (int i = threadIdx.x; i < Hi; i += 256) ws[i] = w_idx[((size_t)b * Q + j) * Hi + i];
  __syncthreads();
  const int t = tbase + threadIdx.x;
  if (t >= L) return;
  const int pg = page_table[(size_t)b * max_pages + t / page];
  float acc;
  if (pg < 0 || (int64_t)pg >= num_pages) {
    acc = __int_as_float(0x7fc00000);
  } else {
    const T* kp = icache + ((size_t)pg * page + t % page) * dI;
    acc = 0.0f;
    for (int h = 0; h < Hi; ++h) {
      float dot = 0.0f;
      for (int d = 0; d < dI; ++d) dot = fmaf(qs[h * dI + d], Elt<T>::ld(kp + d), dot);
      acc = fmaf(ws[h], relu_nan(dot), acc);
    }
  }
  scores[((size_t)b * Q + j) * ld + t] = acc;
}

// ---------------------------------------------------------------------------
// top-k selection in two launches.
// Scores map to order-preserving 32-bit keys (-0 taken as +0); the top 12
// bits of a key (sign, exponent, 3 mantissa bits) name one of 4,096 coarse
// bins, in key order.
//  1. topk_hist_kernel: blocks of 256 threads take 4,096 visible scores each,
//     count them per coarse bin in LDS and add the non-empty bins to the
//     query's histogram in the workspace (global atomics); a NaN sets the
//     query's flag there.
//  2. topk_select_kernel: one block of 1,024 threads (16 waves) per query
//     reads the histogram and clears it (the workspace is all zero between
//     calls), finds the coarse bin of the k-th largest key and gathers that
//     bin's keys into LDS with wave ballots; the exact k-th key T is found by
//     narrowing [lo, hi] over those keys with histograms of 1,024 bins of 2^s
//     keys (a shift, no division). When the bin holds more keys than LDS
//     takes, the narrowing reads every score instead. The output is written
//     in token order: wave w owns a contiguous span of tokens, counts its keys
//     > T and == T, and after a prefix over the 16 waves writes every key > T
//     and the first (topk - count(> T)) keys == T.
// ---------------------------------------------------------------------------
// exclusive prefix sum over the block's 1,024 threads; *total = the sum
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(inc, o, 64);
    if (lane >= o) inc += u;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    uint32_t w = lane < kTkWaves ? tmp[lane] : 0u;
#pragma unroll
    for (int o = 1; o < kTkWaves; o <<= 1) {
      const uint32_t u = __shfl_up(w, o, 64);
      if (lane >= o) w += u;
    }
    if (lane < kTkWaves) tmp[kTkWaves + lane] = w;  // inclusive over waves
  }
  __syncthreads();
  const uint32_t off = wave ? tmp[kTkWaves + wave - 1] : 0u;
  *total = tmp[2 * kTkWaves - 1];
  __syncthreads();  // tmp free for the next scan
  return off + inc - v;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// grid (ceil(max_seq_len / kTkHistTok), batch * q_len); workspace row of the
// query: kTkCoarse bin counts, then its NaN flag
__global__ __launch_bounds__(256) void topk_hist_kernel(int Q, int max_seq_len,
                                                       const float* __restrict__ scores, int ld,
                                                       const int32_t* __restrict__ seq_lens,
                                                       uint32_t* __restrict__ ws) {
  __shared__ uint32_t h[kTkCoarse];
  const int bj = blockIdx.y;
  const int b = bj / Q, j = bj % Q;
  const int L = seq_lens[b];
  if (L < Q || L > max_seq_len) return;  // the select kernel reports it
  const int n = L - Q + j + 1;
  const int t0 = blockIdx.x * kTkHistTok;
  if (t0 >= n) return;
  for (int i = threadIdx.x; i < kTkCoarse; i += 256) h[i] = 0u;
  __syncthreads();
  const float* sc = scores + (size_t)bj * ld;
  float v[kTkHistTok / 256];
#pragma unroll
  for (int u = 0; u < kTkHistTok / 256; ++u) {
    const int t = t0 + u * 256 + threadIdx.x;
    v[u] = t < n ? sc[t] : 0.0f;
  }
  bool nan = false;
#pragma unroll
  for (int u = 0; u < kTkHistTok / 256; ++u) {
    const int t = t0 + u * 256 + threadIdx.x;
    if (t < n) {
      nan |= v[u] != v[u];
      atomicAdd(&h[score_key(v[u]) >> (32 - kTkCoarseBits)], 1u);
    }
  }
  uint32_t* row = ws + (size_t)bj * kTkWsRow;
  if (__syncthreads_or(nan ? 1 : 0) && threadIdx.x == 0) row[kTkCoarse] = 1u;
  for (int i = threadIdx.x; i < kTkCoarse; i += 256)
    if (h[i]) atomicAdd(&row[i], h[i]);
}

// kReg: the query sees at most kTkRegTok tokens and every key stays in
// registers after one read of the scores: wave w holds tokens
// [kTkRegSpan w, kTkRegSpan (w + 1)), key v of lane l being token
// kTkRegSpan w + 64 v + l (each load and each ballot covers 64 consecutive
// tokens). Else every pass reads the scores again.
template <bool kReg>
__global__ __launch_bounds__(kTkThreads) void topk_select_kernel(
    int Q, int max_seq_len, int K, const float* __restrict__ scores, int ld,
    const int32_t* __restrict__ seq_lens, uint32_t* __restrict__ ws, int32_t* __restrict__ indices,
    int32_t* __restrict__ counts) {
  __shared__ uint32_t hist[kTkBins];
  __shared__ uint32_t cand[kTkCand];
  __shared__ uint32_t tmp[4 * kTkWaves];
  __shared__ uint32_t pick[4];
  const int bj = blockIdx.x;
  const int b = bj / Q, j = bj % Q;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = seq_lens[b];
  int32_t* out = indices + (size_t)bj * K;
  uint32_t* row = ws + (size_t)bj * kTkWsRow;
  // the coarse counts, four bins per thread from the top (bins 4095 - 4 tid ..)
  uint32_t c4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c4[i] = row[kTkCoarse - 1 - (4 * tid + i)];
  const bool nan = row[kTkCoarse] != 0u;
  const bool valid = !(L < Q || L > max_seq_len);
  const int n = valid ? L - Q + j + 1 : 0;  // tokens the query sees
  const float* sc = scores + (size_t)bj * ld;
  // kReg: all keys of this wave's span, one read of the scores
  uint32_t kr[kReg ? kTkRegKeys : 1];
  const int rbase = wave * kTkRegSpan + lane;
  if constexpr (kReg) {
    float v[kTkRegKeys];
#pragma unroll
    for (int u = 0; u < kTkRegKeys; ++u) {
      const int t = rbase + 64 * u;
      v[u] = t < n ? sc[t] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kTkRegKeys; ++u)
      kr[u] = rbase + 64 * u < n ? score_key(v[u]) : 0u;  // 0: below every real key
  }
  __syncthreads();  // every thread has read its counts and the flag
#pragma unroll
  for (int i = 0; i < 4; ++i) row[kTkCoarse - 1 - (4 * tid + i)] = 0u;
  if (tid == 0) row[kTkCoarse] = 0u;
  if (!valid || nan) {
    if (tid == 0) counts[bj] = -1;
    return;
  }
  if (n <= K) {
    for (int t = tid; t < n; t += kTkThreads) out[t] = t;
    if (tid == 0) counts[bj] = n;
    return;
  }
  auto key_at = [&](int t) -> uint32_t { return t < n ? score_key(sc[t]) : 0u; };

  // the coarse bin of the K-th largest key: running counts from the top
  uint32_t need = (uint32_t)K;
  {
    const uint32_t s4 = c4[0] + c4[1] + c4[2] + c4[3];
    uint32_t tot;
    uint32_t ex = block_excl_scan(s4, tmp, &tot);
    if (ex < need && ex + s4 >= need) {  // exactly one thread holds it
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (ex < need && ex + c4[i] >= need) {
          pick[0] = (uint32_t)(kTkCoarse - 1 - (4 * tid + i));
          pick[1] = ex;
          pick[2] = c4[i];
        }
        ex += c4[i];
      }
      pick[3] = 0u;
    }
    __syncthreads();
  }
  need -= pick[1];
  const int csh = 32 - kTkCoarseBits;
  uint32_t lo = pick[0] << csh;
  uint32_t hi = lo + ((1u << csh) - 1u);
  int ncand = -1;  // >= 0: the keys in [lo, hi] are cand[0 .. ncand)
  if (!kReg && pick[2] <= (uint32_t)kTkCand) {
    // gather the bin's keys (in any order): one LDS atomic per wave and batch
    auto gather = [&](const uint32_t* kk, const bool* ok) {
      uint64_t m[kTkBatch];
      uint32_t cnt = 0u;
#pragma unroll
      for (int u = 0; u < kTkBatch; ++u) {
        m[u] = __ballot(ok[u] && kk[u] >= lo && kk[u] <= hi);
        cnt += __builtin_popcountll(m[u]);
      }
      if (cnt) {
        uint32_t base = 0u;
        if (lane == 0) base = atomicAdd(&pick[3], cnt);
        base = __shfl(base, 0, 64);
#pragma unroll
        for (int u = 0; u < kTkBatch; ++u) {
          if ((m[u] >> lane) & 1ull) cand[base + lanes_below(m[u])] = kk[u];
          base += __builtin_popcountll(m[u]);
        }
      }
    };
    {
      for (int t0 = wave * 64; t0 < n; t0 += kTkBatch * kTkThreads) {
        uint32_t kk[kTkBatch];
        bool ok[kTkBatch];
#pragma unroll
        for (int u = 0; u < kTkBatch; ++u) {
          const int t = t0 + u * kTkThreads + lane;
          kk[u] = key_at(t);
          ok[u] = t < n;
        }
        gather(kk, ok);
      }
    }
    ncand = (int)pick[2];
  }
  __syncthreads();  // cand complete; pick read by all

  // narrow [lo, hi] to the single key T of the K-th largest score; `need` =
  // how many tokens with keys in [lo, hi] still belong to the selection
  while (lo < hi) {
    const uint32_t d = hi - lo;
    const int sh = max(0, (32 - __builtin_clz(d)) - kTkBinBits);
    for (int i = tid; i < kTkBins; i += kTkThreads) hist[i] = 0u;
    __syncthreads();
    if (ncand >= 0) {
      for (int i = tid; i < ncand; i += kTkThreads) {
        const uint32_t k = cand[i];
        if (k >= lo && k <= hi) atomicAdd(&hist[(k - lo) >> sh], 1u);
      }
    } else if constexpr (kReg) {  // padding keys are 0, never in range
#pragma unroll
      for (int i = 0; i < kTkRegKeys; ++i)
        if (kr[i] >= lo && kr[i] <= hi) atomicAdd(&hist[(kr[i] - lo) >> sh], 1u);
    } else {
      for (int t0 = tid; t0 < n; t0 += kTkBatch * kTkThreads) {
        uint32_t kk[kTkBatch];
#pragma unroll
        for (int u = 0; u < kTkBatch; ++u) kk[u] = key_at(t0 + u * kTkThreads);
#pragma unroll
        for (int u = 0; u < kTkBatch; ++u)
          if (t0 + u * kTkThreads < n && kk[u] >= lo && kk[u] <= hi)
            atomicAdd(&hist[(kk[u] - lo) >> sh], 1u);
      }
    }
    __syncthreads();
    const uint32_t h = hist[kTkBins - 1 - tid];  // thread i: the i-th bin from the top
    uint32_t tot;
    const uint32_t ex = block_excl_scan(h, tmp, &tot);
    if (ex < need && ex + h >= need) {  // exactly one thread
      pick[0] = (uint32_t)(kTkBins - 1 - tid);
      pick[1] = ex;
    }
    __syncthreads();
    need -= pick[1];
    const uint32_t nlo = lo + (pick[0] << sh);
    // the bin's last key, cut at hi (in 64 bits: the top bin may end past 2^32)
    hi = (uint32_t)min((uint64_t)hi, (uint64_t)nlo + ((1ull << sh) - 1ull));
    lo = nlo;
    __syncthreads();  // pick and hist are rewritten in the next pass
  }
  const uint32_t T = lo;

  if constexpr (kReg) {
    // ordered output from the registers: this wave's span in 64-token steps
    uint32_t gtw = 0u, eqw = 0u;
#pragma unroll
    for (int u = 0; u < kTkRegKeys; ++u) {
      gtw += __builtin_popcountll(__ballot(kr[u] > T));
      eqw += __builtin_popcountll(__ballot(kr[u] == T));
    }
    if (lane == 0) {
      tmp[2 * kTkWaves + wave] = gtw;
      tmp[3 * kTkWaves + wave] = eqw;
    }
    __syncthreads();
    uint32_t gb = 0u, eb = 0u;  // keys > T and == T before this wave's span
    for (int w = 0; w < wave; ++w) {
      gb += tmp[2 * kTkWaves + w];
      eb += tmp[3 * kTkWaves + w];
    }
#pragma unroll
    for (int u = 0; u < kTkRegKeys; ++u) {
      const bool gt = kr[u] > T, eq = kr[u] == T;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      const uint32_t eq_before = eb + lanes_below(me);
      if (gt || (eq && eq_before < need))
        out[gb + lanes_below(mg) + min(eq_before, need)] = rbase + 64 * u;
      gb += __builtin_popcountll(mg);
      eb += __builtin_popcountll(me);
    }
  } else {
    // ordered output: wave w owns tokens [w * span, (w + 1) * span), span a
    // multiple of 64 * kTkOut
    const int span = ((n + kTkWaves * 64 * kTkOut - 1) / (kTkWaves * 64 * kTkOut)) * 64 * kTkOut;
    const int w0 = min(n, wave * span), w1 = min(n, w0 + span);
    uint32_t gtw = 0u, eqw = 0u;
    for (int t0 = w0; t0 < w1; t0 += 64 * kTkOut) {
      uint32_t kk[kTkOut];
#pragma unroll
      for (int u = 0; u < kTkOut; ++u) kk[u] = key_at(t0 + 64 * u + lane);  // 0 past n
#pragma unroll
      for (int u = 0; u < kTkOut; ++u) {
        gtw += __builtin_popcountll(__ballot(kk[u] > T));
        eqw += __builtin_popcountll(__ballot(kk[u] == T));
      }
    }
    if (lane == 0) {
      tmp[2 * kTkWaves + wave] = gtw;
      tmp[3 * kTkWaves + wave] = eqw;
    }
    __syncthreads();
    uint32_t gb = 0u, eb = 0u;  // keys > T and == T in the waves before this one
    for (int w = 0; w < wave; ++w) {
      gb += tmp[2 * kTkWaves + w];
      eb += tmp[3 * kTkWaves + w];
    }
    for (int t0 = w0; t0 < w1; t0 += 64 * kTkOut) {
      uint32_t kk[kTkOut];
#pragma unroll
      for (int u = 0; u < kTkOut; ++u) kk[u] = key_at(t0 + 64 * u + lane);
#pragma unroll
      for (int u = 0; u < kTkOut; ++u) {
        const int t = t0 + 64 * u + lane;
        const bool gt = kk[u] > T, eq = kk[u] == T;
        const uint64_t mg = __ballot(gt), me = __ballot(eq);
        const uint32_t eq_before = eb + lanes_below(me);
        if (gt || (eq && eq_before < need))
          out[gb + lanes_below(mg) + min(eq_before, need)] = t;
        gb += __builtin_popcountll(mg);
        eb += __builtin_popcountll(me);
      }
    }
  }
  if (tid == 0) counts[bj] = K;
}

}  // namespace

int launch_index_append(const Shape& s, int dI, int n_tok, const void* k_new,
                        const int32_t* seq_idx, const int32_t* pos, const int32_t* page_table,
                        int batch, int max_pages, void* icache, int64_t num_pages, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (s.dtype == 0)
    hipLaunchKernelGGL(index_append_kernel<float>, dim3(n_tok), dim3(64), 0, st, dI, s.page,
                       (const float*)k_new, seq_idx, pos, page_table, batch, max_pages,
                       (float*)icache, num_pages);
  else
    hipLaunchKernelGGL(index_append_kernel<bf16_t>, dim3(n_tok), dim3(64), 0, st, dI, s.page,
                       (const bf16_t*)k_new, seq_idx, pos, page_table, batch, max_pages,
                       (bf16_t*)icache, num_pages);
  return (int)hipGetLastError();
}

bool index_scores_mfma_ok(const Shape& s, int Hi, int dI) {
  return s.dtype == 1 && Hi == kIH && dI == kID && s.page % 16 == 0;
}

size_t index_scores_generic_lds(int Hi, int dI) {
  return sizeof(float) * ((size_t)Hi * dI + Hi);
}

int launch_index_scores(const Shape& s, int Hi, int dI, int batch, int q_len, int max_seq_len,
                        const void* q_idx, const float* w_idx, const void* icache,
                        int64_t num_pages, const int32_t* page_table, int max_pages,
                        const int32_t* seq_lens, float* scores, int ld, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((max_seq_len + kIdxTok - 1) / kIdxTok, batch, q_len);
  if (index_scores_mfma_ok(s, Hi, dI)) {
    if (int e = set_max_lds(reinterpret_cast<const void*>(index_scores_mfma_kernel<false>),
                            (int)kILds))
      return e;
    hipLaunchKernelGGL((index_scores_mfma_kernel<false>), grid, dim3(256), kILds, st, q_len,
                       s.page, max_seq_len, (const bf16_t*)q_idx, w_idx, (const bf16_t*)icache,
                       num_pages, page_table, max_pages, seq_lens, scores, ld, nullptr);
    return (int)hipGetLastError();
  }
  const size_t lds_bytes = index_scores_generic_lds(Hi, dI);
  if (lds_bytes > 64 * 1024) {
    if (int e = set_max_lds(s.dtype == 0
                                ? reinterpret_cast<const void*>(index_scores_generic_kernel<float>)
                                : reinterpret_cast<const void*>(index_scores_generic_kernel<bf16_t>),
                            160 * 1024))
      return e;
  }
  const dim3 ggrid((max_seq_len + 255) / 256, batch, q_len);
  if (s.dtype == 0)
    hipLaunchKernelGGL(index_scores_generic_kernel<float>, ggrid, dim3(256), lds_bytes, st, q_len, Hi,
                       dI, s.page, max_seq_len, (const float*)q_idx, w_idx, (const float*)icache,
                       num_pages, page_table, max_pages, seq_lens, scores, ld);
  else
    hipLaunchKernelGGL(index_scores_generic_kernel<bf16_t>, ggrid, dim3(256), lds_bytes, st, q_len, Hi,
                       dI, s.page, max_seq_len, (const bf16_t*)q_idx, w_idx,
                       (const bf16_t*)icache, num_pages, page_table, max_pages, seq_lens, scores,
                       ld);
  return (int)hipGetLastError();
}

size_t topk_workspace_bytes(int batch, int q_len) {
  return sizeof(uint32_t) * (size_t)kTkWsRow * batch * q_len;
}

namespace {
int launch_topk_select(int batch, int q_len, int max_seq_len, int topk, const float* scores,
                       int ld, const int32_t* seq_lens, uint32_t* ws, int32_t* indices,
                       int32_t* counts, hipStream_t st);
}  // namespace

int launch_topk(int batch, int q_len, int max_seq_len, int topk, const float* scores, int ld,
                const int32_t* seq_lens, void* workspace, int32_t* indices, int32_t* counts,
                void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t* ws = reinterpret_cast<uint32_t*>(workspace);
  hipLaunchKernelGGL(topk_hist_kernel, dim3((max_seq_len + kTkHistTok - 1) / kTkHistTok,
                                            batch * q_len),
                     dim3(256), 0, st, q_len, max_seq_len, scores, ld, seq_lens, ws);
  return launch_topk_select(batch, q_len, max_seq_len, topk, scores, ld, seq_lens, ws, indices,
                            counts, st);
}

int launch_index_scores_topk(const Shape& s, int Hi, int dI, int batch, int q_len,
                             int max_seq_len, const void* q_idx, const float* w_idx,
                             const void* icache, int64_t num_pages, const int32_t* page_table,
                             int max_pages, const int32_t* seq_lens, float* scores, int ld,
                             int topk, void* workspace, int32_t* indices, int32_t* counts,
                             void* stream) {
  if (!index_scores_mfma_ok(s, Hi, dI)) {  // the separate launches
    const int e = launch_index_scores(s, Hi, dI, batch, q_len, max_seq_len, q_idx, w_idx, icache,
                                      num_pages, page_table, max_pages, seq_lens, scores, ld,
                                      stream);
    if (e != 0) return e;
    return launch_topk(batch, q_len, max_seq_len, topk, scores, ld, seq_lens, workspace, indices,
                       counts, stream);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  uint32_t* ws = reinterpret_cast<uint32_t*>(workspace);
  if (int e = set_max_lds(reinterpret_cast<const void*>(index_scores_mfma_kernel<true>),
                          (int)kILds))
    return e;
  const dim3 grid((max_seq_len + kIdxTok - 1) / kIdxTok, batch, q_len);
  hipLaunchKernelGGL((index_scores_mfma_kernel<true>), grid, dim3(256), kILds, st, q_len, s.page,
                     max_seq_len, (const bf16_t*)q_idx, w_idx, (const bf16_t*)icache, num_pages,
                     page_table, max_pages, seq_lens, scores, ld, ws);
  const int e = (int)hipGetLastError();
  if (e != 0) return e;
  return launch_topk_select(batch, q_len, max_seq_len, topk, scores, ld, seq_lens, ws, indices,
                            counts, st);
}

namespace {
int launch_topk_select(int batch, int q_len, int max_seq_len, int topk, const float* scores,
                       int ld, const int32_t* seq_lens, uint32_t* ws, int32_t* indices,
                       int32_t* counts, hipStream_t st) {
  if (max_seq_len <= kTkRegTok)
    hipLaunchKernelGGL(topk_select_kernel<true>, dim3(batch * q_len), dim3(kTkThreads), 0, st,
                       q_len, max_seq_len, topk, scores, ld, seq_lens, ws, indices, counts);
  else
    hipLaunchKernelGGL(topk_select_kernel<false>, dim3(batch * q_len), dim3(kTkThreads), 0, st,
                       q_len, max_seq_len, topk, scores, ld, seq_lens, ws, indices, counts);
  return (int)hipGetLastError();
}
}  // namespace

// ---------------------------------------------------------------------------
// The top-k workspace of callers that cannot allocate: a file-scope device
// array with the rows of up to kTopkNoallocMaxQueries queries (4,198,400
// bytes; each device holds its own copy for the life of the process). Host
// code never passes the array's name to a kernel: that name is a host-side
// stand-in. The device address comes from hipGetSymbolAddress, once per
// device with that device current, and is kept per device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint32_t scratch[(size_t)kTopkNoallocMaxQueries * kTkWsRow];

namespace {

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

struct ScratchState {
  uint32_t* ptr = nullptr;  // device address of `scratch` on this device
  bool clean = false;       // every row zero, as the selection leaves it
};
std::mutex g_scratch_mu;
std::map<int, ScratchState> g_scratch;

}  // namespace

int launch_index_scores_topk_noalloc(const Shape& s, int Hi, int dI, int batch, int q_len,
                                     int max_seq_len, const void* q_idx, const float* w_idx,
                                     const void* icache, int64_t num_pages,
                                     const int32_t* page_table, int max_pages,
                                     const int32_t* seq_lens, float* scores, int ld, int topk,
                                     int32_t* indices, int32_t* counts, void* stream) {
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return (int)he;
  uint32_t* ws = nullptr;
  bool clear = false;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchState& d = g_scratch[dev];
    if (!d.ptr) {
      void* p = nullptr;
      he = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (he != hipSuccess) return (int)he;
      d.ptr = reinterpret_cast<uint32_t*>(p);
    }
    ws = d.ptr;
    clear = !d.clean;
    d.clean = true;
  }
  auto mark_dirty = [&]() {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    g_scratch[dev].clean = false;
  };
  if (clear) {
    const size_t n = (size_t)kTopkNoallocMaxQueries * kTkWsRow;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(1024), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), ws, n);
    const int e = (int)hipGetLastError();
    if (e != 0) {
      mark_dirty();
      return e;
    }
  }
  const int e = launch_index_scores_topk(s, Hi, dI, batch, q_len, max_seq_len, q_idx, w_idx,
                                         icache, num_pages, page_table, max_pages, seq_lens,
                                         scores, ld, topk, ws, indices, counts, stream);
  if (e != 0) mark_dirty();
  return e;
}

}  // namespace mla
