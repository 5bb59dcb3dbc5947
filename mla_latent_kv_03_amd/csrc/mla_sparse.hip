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
#include "mla_common.h"
#include "mla_decode_common.h"
#include "mla_launch.h"

namespace mla {

using namespace dec;

namespace {

constexpr int kIH = 64;   // indexer heads of the MFMA kernel
constexpr int kID = 128;  // indexer key width of the MFMA kernel
constexpr int kIdxTok = 256;  // tokens per index-score block (4 waves x 64)

constexpr int kTkThreads = 1024;
constexpr int kTkBins = 1024;
constexpr int kTkLdsKeys = 36864;  // sequences up to this many visible tokens keep their keys in LDS

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
  const int n = blockIdx.x;
  const int b = seq_idx[n], p = pos[n];
  if (b < 0 || b >= batch || p < 0 || (int64_t)p >= (int64_t)max_pages * page) return;
  const int pg = page_table[(size_t)b * max_pages + p / page];
  if (pg < 0 || (int64_t)pg >= num_pages) return;
  T* dst = icache + ((size_t)pg * page + p % page) * dI;
  const T* src = k_new + (size_t)n * dI;
  for (int i = threadIdx.x; i < dI; i += 64) dst[i] = src[i];
}

// ReLU that keeps a NaN (a NaN dot must not turn into a valid score)
__device__ __forceinline__ float relu_nan(float x) { return x < 0.0f ? 0.0f : x; }

// ---------------------------------------------------------------------------
// index scores, bf16 MFMA: 64 heads x 128 dims. Block = 256 tokens of one
// (sequence, query); wave w takes tokens [64 w, 64 w + 64) in 4 groups of 16.
// Per group: D[head][token] = q_idx[head][:] . k[token][:] on
// v_mfma_f32_16x16x32_bf16 (M = 16 heads, N = 16 tokens, 4 head blocks x 4
// k-steps), then lane (token n, head quarter kg) folds its 16 heads with
// w * max(0, D) and the four quarters are summed with lane swaps.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void index_scores_mfma_kernel(
    int Q, int page, int max_seq_len, const bf16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, const bf16_t* __restrict__ icache, int64_t num_pages,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ seq_lens,
    float* __restrict__ scores, int ld) {
  const int b = blockIdx.y, j = blockIdx.z;
  const int L = seq_lens[b];
  if (L < Q || L > max_seq_len) return;  // the selection reports the sequence invalid
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const int tw = blockIdx.x * kIdxTok + wave * 64;
  if (tw >= L) return;

  // keys first (the long loads): group g, token tw + 16 g + n, dims 32 ks + 8 kg
  bf16x8_t kv[4][4];
  bool okp[4];
  const bf16x8_t zero = {};
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int t = tw + 16 * g + n;
    const bool in = t < L;
    int pg = in ? page_table[(size_t)b * max_pages + t / page] : 0;
    okp[g] = pg >= 0 && (int64_t)pg < num_pages;
    if (!okp[g]) pg = 0;
    const bf16_t* kp = icache + ((size_t)pg * page + (in ? t % page : 0)) * kID + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kv[g][ks] = in ? *reinterpret_cast<const bf16x8_t*>(kp + 32 * ks) : zero;
  }
  // queries: head 16 mt + n, dims 32 ks + 8 kg; weights of heads 16 mt + 4 kg + r
  const bf16_t* qb = q_idx + ((size_t)b * Q + j) * kIH * kID;
  const float* wb = w_idx + ((size_t)b * Q + j) * kIH;
  bf16x8_t qa[4][4];
  float wv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[mt][ks] = *reinterpret_cast<const bf16x8_t*>(qb + (16 * mt + n) * kID + 32 * ks + 8 * kg);
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = wb[16 * mt + 4 * kg + r];
  }
  float* out = scores + ((size_t)b * Q + j) * ld;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
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
    part = row_sum4(part);
    const int t = tw + 16 * g + n;
    if (kg == 0 && t < L) out[t] = okp[g] ? part : __int_as_float(0x7fc00000);
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
// top-k selection: one block of 1,024 threads per (sequence, query).
// Scores map to order-preserving 32-bit keys (-0 taken as +0). The k-th
// largest key T is found by narrowing a key range [lo, hi]: a histogram of
// 1,024 equal-width bins over the range, the bin where the count from the
// top reaches the number still needed becomes the new range (at most four
// rounds, each dividing the width by ~1,024). Then every thread takes an
// equal slice of the tokens in order (slices of odd length, so that the
// slices' LDS reads fall in distinct banks), counts keys > T and == T, and
// one block scan gives each slice its output position: all keys > T, and the
// first (topk - count(> T)) keys == T in token order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t score_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

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
    uint32_t w = lane < kTkThreads / 64 ? tmp[lane] : 0u;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const uint32_t u = __shfl_up(w, o, 64);
      if (lane >= o) w += u;
    }
    if (lane < kTkThreads / 64) tmp[16 + lane] = w;  // inclusive over waves
  }
  __syncthreads();
  const uint32_t off = wave ? tmp[16 + wave - 1] : 0u;
  *total = tmp[16 + kTkThreads / 64 - 1];
  __syncthreads();  // tmp free for the next scan
  return off + inc - v;
}

__device__ __forceinline__ uint32_t block_min_max(uint32_t v, bool want_max, uint32_t* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t u = __shfl_xor(v, o, 64);
    v = want_max ? max(v, u) : min(v, u);
  }
  if (lane == 0) tmp[wave] = v;
  __syncthreads();
  uint32_t r = tmp[0];
  for (int w = 1; w < kTkThreads / 64; ++w) r = want_max ? max(r, tmp[w]) : min(r, tmp[w]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTkThreads) void topk_kernel(int Q, int max_seq_len, int K,
                                                         int lds_keys,
                                                         const float* __restrict__ scores, int ld,
                                                         const int32_t* __restrict__ seq_lens,
                                                         int32_t* __restrict__ indices,
                                                         int32_t* __restrict__ counts) {
  extern __shared__ uint32_t skeys[];
  __shared__ uint32_t hist[kTkBins];
  __shared__ uint32_t tmp[48];
  __shared__ uint32_t pick[2];
  const int bj = blockIdx.x;
  const int b = bj / Q, j = bj % Q;
  const int tid = threadIdx.x;
  const int L = seq_lens[b];
  int32_t* out = indices + (size_t)bj * K;
  if (L < Q || L > max_seq_len) {
    if (tid == 0) counts[bj] = -1;
    return;
  }
  const int n = L - Q + j + 1;  // tokens the query sees
  const float* sc = scores + (size_t)bj * ld;
  const bool inlds = n <= lds_keys;

  // keys (kept in LDS when they fit), NaN check, key range
  uint32_t kmin = 0xffffffffu, kmax = 0u;
  bool nan = false;
  for (int t = tid; t < n; t += kTkThreads) {
    const float v = sc[t];
    nan |= v != v;
    const uint32_t k = score_key(v);
    if (inlds) skeys[t] = k;
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
  if (__syncthreads_or(nan ? 1 : 0)) {
    if (tid == 0) counts[bj] = -1;
    return;
  }
  if (n <= K) {
    for (int t = tid; t < n; t += kTkThreads) out[t] = t;
    if (tid == 0) counts[bj] = n;
    return;
  }
  kmin = block_min_max(kmin, false, tmp);
  kmax = block_min_max(kmax, true, tmp);
  auto key_at = [&](int t) { return inlds ? skeys[t] : score_key(sc[t]); };

  // narrow [lo, hi] to the single key T of the K-th largest score; `need` =
  // how many tokens with keys in [lo, hi] still belong to the selection
  uint32_t lo = kmin, hi = kmax, need = (uint32_t)K;
  while (lo < hi) {
    for (int i = tid; i < kTkBins; i += kTkThreads) hist[i] = 0u;
    __syncthreads();
    const uint64_t w = (uint64_t)(hi - lo) + 1u;
    for (int t = tid; t < n; t += kTkThreads) {
      const uint32_t k = key_at(t);
      if (k >= lo && k <= hi) atomicAdd(&hist[(uint32_t)(((uint64_t)(k - lo) * kTkBins) / w)], 1u);
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
    const uint64_t bin = pick[0];
    need -= pick[1];
    const uint64_t a = (bin * w + kTkBins - 1) / kTkBins;        // first key offset of the bin
    const uint64_t e = ((bin + 1) * w + kTkBins - 1) / kTkBins;  // one past its last
    hi = lo + (uint32_t)(e - 1);
    lo = lo + (uint32_t)a;
    __syncthreads();  // pick and hist are rewritten next round
  }
  const uint32_t T = lo;

  // ordered compaction over per-thread slices of odd length
  int seg = (n + kTkThreads - 1) / kTkThreads;
  seg |= 1;
  const int s0 = min(n, tid * seg), s1 = min(n, s0 + seg);
  uint32_t gt = 0u, eq = 0u;
  for (int t = s0; t < s1; ++t) {
    const uint32_t k = key_at(t);
    gt += k > T;
    eq += k == T;
  }
  uint32_t gtot, etot;
  const uint32_t gb = block_excl_scan(gt, tmp, &gtot);
  const uint32_t eb = block_excl_scan(eq, tmp, &etot);
  uint32_t pos = gb + min(eb, need);
  uint32_t eseen = eb;
  for (int t = s0; t < s1; ++t) {
    const uint32_t k = key_at(t);
    if (k > T) {
      out[pos++] = t;
    } else if (k == T) {
      if (eseen < need) out[pos++] = t;
      ++eseen;
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
  return s.dtype == 1 && Hi == kIH && dI == kID;
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
    hipLaunchKernelGGL(index_scores_mfma_kernel, grid, dim3(256), 0, st, q_len, s.page,
                       max_seq_len, (const bf16_t*)q_idx, w_idx, (const bf16_t*)icache, num_pages,
                       page_table, max_pages, seq_lens, scores, ld);
    return (int)hipGetLastError();
  }
  const size_t lds = index_scores_generic_lds(Hi, dI);
  if (lds > 64 * 1024) {
    static bool attr[2] = {false, false};
    if (!attr[s.dtype]) {
      hipError_t e = s.dtype == 0
                         ? hipFuncSetAttribute(
                               reinterpret_cast<const void*>(index_scores_generic_kernel<float>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024)
                         : hipFuncSetAttribute(
                               reinterpret_cast<const void*>(index_scores_generic_kernel<bf16_t>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return (int)e;
      attr[s.dtype] = true;
    }
  }
  const dim3 ggrid((max_seq_len + 255) / 256, batch, q_len);
  if (s.dtype == 0)
    hipLaunchKernelGGL(index_scores_generic_kernel<float>, ggrid, dim3(256), lds, st, q_len, Hi,
                       dI, s.page, max_seq_len, (const float*)q_idx, w_idx, (const float*)icache,
                       num_pages, page_table, max_pages, seq_lens, scores, ld);
  else
    hipLaunchKernelGGL(index_scores_generic_kernel<bf16_t>, ggrid, dim3(256), lds, st, q_len, Hi,
                       dI, s.page, max_seq_len, (const bf16_t*)q_idx, w_idx,
                       (const bf16_t*)icache, num_pages, page_table, max_pages, seq_lens, scores,
                       ld);
  return (int)hipGetLastError();
}

int launch_topk(int batch, int q_len, int max_seq_len, int topk, const float* scores, int ld,
                const int32_t* seq_lens, int32_t* indices, int32_t* counts, void* stream) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)(sizeof(uint32_t) * kTkLdsKeys));
    if (e != hipSuccess) return (int)e;
    attr = true;
  }
  const int lds_keys = max_seq_len <= kTkLdsKeys ? max_seq_len : 0;
  hipLaunchKernelGGL(topk_kernel, dim3(batch * q_len), dim3(kTkThreads),
                     sizeof(uint32_t) * (size_t)lds_keys, reinterpret_cast<hipStream_t>(stream),
                     q_len, max_seq_len, topk, lds_keys, scores, ld, seq_lens, indices, counts);
  return (int)hipGetLastError();
}

}  // namespace mla
