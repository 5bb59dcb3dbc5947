// Split-KV paged MLA decode on bf16 MFMA for the DeepSeek MLA shape
// (d_c = 512, d_r = 64: 576 bf16 = 1,152 bytes per cached row), gfx950.
//
// What it computes ("The Architecture of Memory", "Flash-Decoding and
// FlashInfer", "The Decode Phase: The Memory Bandwidth Wall"; "DeepSeek's
// Config Says 16 KV Heads", section 5): for every query row (query j, head h)
// the absorbed query q_full (576 wide) is scored against every cached row of
// its partition, the scores are softmaxed online, and the softmax weights
// multiply the 512 latent columns of the same rows. Every head reads the same
// cached rows, so one staged tile serves 16 query rows at once.
//
// Work decomposition
//   block  = (partition s of sequence b, group of 16 query rows); 4 waves.
//   wave w = independent online-softmax worker over the 16-token slices
//            w, w+4, w+8, ... of the partition, with its own LDS slice buffer
//            (no block barrier inside the token loop). The four waves merge
//            their (max, sum, output) through LDS at the end.
//   Blocks are numbered so that all row groups of one partition land on the
//   same XCD (block id % 8), where they share that XCD's L2.
//
// Per 16-token slice, per wave
//   HBM -> VGPR: 18 x 16-byte loads per lane (the slice is 18,432 contiguous
//           bytes: rows of one page are adjacent), issued one slice ahead.
//   VGPR -> LDS: rows stored with a XOR swizzle of the 16-byte chunk index,
//           chunk c of row t at t*72 + (c ^ (t & 7)), so both read patterns
//           below are free of bank conflicts.
//   S^T = C . Q^T  : 18 x v_mfma_f32_16x16x32_bf16 (M = tokens, N = rows,
//           K = 576 features); C from LDS (ds_read_b128), Q from VGPRs.
//   online softmax in the log2 domain: row max across the 4 lane groups by
//           two lane exchanges; exp2 on the vector ALU.
//   O += P . C[:, :512] : 32 x v_mfma_f32_16x16x16_bf16 (M = rows, N = 16
//           features, K = 16 tokens); P straight from the S^T accumulator
//           layout; C columns gathered with ds_read_b64 from 4 token rows
//           and transposed 4x4 in registers (v_perm).
#include <hip/hip_runtime.h>
#include <math.h>

#include "mla_common.h"
#include "mla_launch.h"

namespace mla {

int launch_decode_generic(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                          const void* q_full, const void* cache, int64_t num_pages,
                          const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                          float* o_part, float* lse_part, void* stream);

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;

constexpr int kDC = 512;
constexpr int kD = 576;
constexpr int kChunks = kD * 2 / 16;            // 72 sixteen-byte chunks per row
constexpr int kSlice = 16;                      // tokens per wave step
constexpr int kSliceChunks = kSlice * kChunks;  // 1152
constexpr int kLoads = kSliceChunks / 64;       // 18 loads per lane per slice
constexpr int kKSteps = kD / 32;                // 18 k-steps (QK)
constexpr int kFB = kDC / 64;                   // 8 feature blocks (PV)
constexpr int kWaves = 4;
constexpr int kRows = 16;                       // query rows per block
constexpr size_t kLdsLoop = (size_t)kWaves * kSliceChunks * 16;        // 73,728 B
constexpr size_t kLdsEpi = (size_t)kWaves * kRows * kDC * 4 + 1024;   // 132,096 B
constexpr size_t kLdsBytes = kLdsLoop > kLdsEpi ? kLdsLoop : kLdsEpi;

__device__ __forceinline__ int swz(int t, int c) { return t * kChunks + (c ^ (t & 7)); }

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

__device__ __forceinline__ s16x4_t as_s16x4(uint32_t lo, uint32_t hi) {
  u32x2_t v = {lo, hi};
  return __builtin_bit_cast(s16x4_t, v);
}

}  // namespace

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_mfma_kernel(int Q, int H, int S, int page, int max_seq_len, float scale_log2,
                        int units, int groups, const bf16_t* __restrict__ q_full,
                        const bf16_t* __restrict__ cache, int64_t num_pages,
                        const int32_t* __restrict__ page_table, int max_pages,
                        const int32_t* __restrict__ seq_lens, float* __restrict__ o_part,
                        float* __restrict__ lse_part) {
  extern __shared__ u32x4_t lds[];
  // block id -> (unit, row group): all groups of one unit share id % 8 (XCD)
  const int id = blockIdx.x;
  const int xcd = id & 7, kk = id >> 3;
  const int unit = (kk / groups) * 8 + xcd;
  const int grp = kk % groups;
  if (unit >= units) return;
  const int s = unit % S, b = unit / S;
  const int R = Q * H;
  const int row0 = grp * kRows;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, kg = lane >> 4;

  const int L = seq_lens[b];
  bool bad = (L < Q) || (L > max_seq_len);
  int t0 = 0, t1 = 0;
  if (!bad) split_range(L, S, page, s, &t0, &t1);
  const int nslices = (t1 - t0 + kSlice - 1) / kSlice;

  // Page-table window: lane i holds the physical page of the unit's page
  // pt_base + i, so a slice's page is a register read instead of a dependent
  // global load in front of its cache loads.
  const int upages = (t1 - t0 + page - 1) / page;
  const size_t pt_row = (size_t)b * max_pages + t0 / page;
  int pt_base = 0;
  int pt_reg = lane < upages ? page_table[pt_row + lane] : 0;

  // absorbed queries of the 16 rows as the B operand of S^T = C . Q^T
  bf16x8_t qreg[kKSteps];
  {
    const u32x4_t* qsrc =
        reinterpret_cast<const u32x4_t*>(q_full + ((size_t)b * R + row0 + n) * kD);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8_t, qsrc[ks * 4 + kg]);
  }
  // last cache position row n may see (its query's own position)
  const int p_lim = L - Q + (row0 + n) / H;

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t acc[kFB][4];
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[fb][m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4_t* buf = lds + wave * kSliceChunks;
  u32x4_t st[kLoads];

  auto issue = [&](int si) {
    const int t = t0 + si * kSlice;
    const int u = (t - t0) / page;  // unit page of this slice (wave-uniform)
    if (u - pt_base >= 64) {        // next window of 64 pages
      pt_base = u & ~63;
      pt_reg = pt_base + lane < upages ? page_table[pt_row + pt_base + lane] : 0;
    }
    int pg = __builtin_amdgcn_readlane(pt_reg, u - pt_base);
    if (pg < 0 || (int64_t)pg >= num_pages) {
      bad = true;
      pg = 0;
    }
    const u32x4_t* src =
        reinterpret_cast<const u32x4_t*>(cache + ((size_t)pg * page + (t % page)) * kD);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) st[i] = __builtin_nontemporal_load(src + i * 64 + lane);
  };

  int si = wave;
  if (si < nslices) issue(si);
  for (; si < nslices; si += kWaves) {
    const int ts = t0 + si * kSlice;
    asm volatile("" ::: "memory");  // keep last slice's LDS reads before these writes
    // staged registers -> LDS (rows past the sequence end are zeroed: they may
    // hold poison, and 0 * NaN would leak into the P . C product)
    {
      const int valid = L - ts;
      int t = 0, c = lane;
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        u32x4_t v = st[i];
        if (t >= valid) v = u32x4_t{0u, 0u, 0u, 0u};
        buf[swz(t, c)] = v;
        c += 64;
        if (c >= kChunks) {
          c -= kChunks;
          ++t;
        }
      }
    }
    if (si + kWaves < nslices) issue(si + kWaves);

    // S^T = C . Q^T over the 576 features
    f32x4_t sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, buf[swz(n, ks * 4 + kg)]);
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[ks], sacc, 0, 0, 0);
    }
    // lane holds row n, tokens ts + 4*kg + r
    float sv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = ts + 4 * kg + r;
      sv[r] = (t <= p_lim) ? sacc[r] * scale_log2 : -INFINITY;
    }
    float mloc = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sv[r] - m_use);
    l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
    if (__any(alpha != 1.0f)) {
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kg + r, 64);
#pragma unroll
      for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[fb][m][r] *= ar[r];
    }
    // P as the A operand (row n, tokens 4*kg .. 4*kg+3)
    bf16x2_t p01 = {(__bf16)p[0], (__bf16)p[1]};
    bf16x2_t p23 = {(__bf16)p[2], (__bf16)p[3]};
    const s16x4_t pa =
        as_s16x4(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
    // O += P . C[:, :512]; lane (n, kg) gathers features fb*64 + 4n .. +3 of
    // token rows 4*kg .. 4*kg+3 and transposes them into 4 B operands
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) {
      u32x2_t x[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int t = 4 * kg + j;
        const u32x2_t* src = reinterpret_cast<const u32x2_t*>(buf + swz(t, fb * 8 + (n >> 1)));
        x[j] = src[n & 1];
      }
      const s16x4_t b0 = as_s16x4(pack_lo(x[0].x, x[1].x), pack_lo(x[2].x, x[3].x));
      const s16x4_t b1 = as_s16x4(pack_hi(x[0].x, x[1].x), pack_hi(x[2].x, x[3].x));
      const s16x4_t b2 = as_s16x4(pack_lo(x[0].y, x[1].y), pack_lo(x[2].y, x[3].y));
      const s16x4_t b3 = as_s16x4(pack_hi(x[0].y, x[1].y), pack_hi(x[2].y, x[3].y));
      acc[fb][0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, b0, acc[fb][0], 0, 0, 0);
      acc[fb][1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, b1, acc[fb][1], 0, 0, 0);
      acc[fb][2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, b2, acc[fb][2], 0, 0, 0);
      acc[fb][3] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, b3, acc[fb][3], 0, 0, 0);
    }
  }

  // ---- merge the four waves ------------------------------------------------
  float l_row = l_run + __shfl_xor(l_run, 16, 64);
  l_row += __shfl_xor(l_row, 32, 64);
  __syncthreads();  // every wave is done with its slice buffer
  float* fl = reinterpret_cast<float*>(lds);
  float* sm = fl + kWaves * kRows * kDC;  // m[4][16], l[4][16], bad[4]
  if (lane < 16) {
    sm[wave * 16 + lane] = m_run;
    sm[64 + wave * 16 + lane] = l_row;
  }
  if (lane == 0) sm[128 + wave] = bad ? 1.0f : 0.0f;
  __syncthreads();
  const bool any_bad = (sm[128] + sm[129] + sm[130] + sm[131]) != 0.0f;
  float fac[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * kg + r;
    float mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mstar = fmaxf(mstar, sm[w * 16 + row]);
    const float mu = (mstar == -INFINITY) ? 0.0f : mstar;
    float lstar = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      lstar += __builtin_amdgcn_exp2f(sm[w * 16 + row] - mu) * sm[64 + w * 16 + row];
    fac[r] = lstar > 0.0f ? __builtin_amdgcn_exp2f(sm[wave * 16 + row] - mu) / lstar : 0.0f;
  }
  float* mine = fl + wave * kRows * kDC;
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4 v = make_float4(acc[fb][0][r] * fac[r], acc[fb][1][r] * fac[r],
                             acc[fb][2][r] * fac[r], acc[fb][3][r] * fac[r]);
      *reinterpret_cast<float4*>(mine + (4 * kg + r) * kDC + fb * 64 + 4 * n) = v;
    }
  __syncthreads();
  const float nanv = __int_as_float(0x7fc00000);
  const float4* f4 = reinterpret_cast<const float4*>(fl);
  for (int i = threadIdx.x; i < kRows * kDC / 4; i += 256) {
    const float4 a = f4[i], b4 = f4[i + 2048], c4 = f4[i + 4096], d4 = f4[i + 6144];
    float4 v = make_float4((a.x + b4.x) + (c4.x + d4.x), (a.y + b4.y) + (c4.y + d4.y),
                           (a.z + b4.z) + (c4.z + d4.z), (a.w + b4.w) + (c4.w + d4.w));
    if (any_bad) v = make_float4(nanv, nanv, nanv, nanv);
    const int row = i / (kDC / 4), col = i % (kDC / 4);
    float4* dst = reinterpret_cast<float4*>(o_part + (((size_t)b * R + row0 + row) * S + s) * kDC);
    dst[col] = v;
  }
  if (threadIdx.x < kRows) {
    const int row = threadIdx.x;
    float mstar = -INFINITY;
    for (int w = 0; w < kWaves; ++w) mstar = fmaxf(mstar, sm[w * 16 + row]);
    const float mu = (mstar == -INFINITY) ? 0.0f : mstar;
    float lstar = 0.0f;
    for (int w = 0; w < kWaves; ++w)
      lstar += __builtin_amdgcn_exp2f(sm[w * 16 + row] - mu) * sm[64 + w * 16 + row];
    const float lse = lstar > 0.0f ? (mstar + log2f(lstar)) * 0.69314718055994531f : -INFINITY;
    lse_part[((size_t)b * R + row0 + row) * S + s] = any_bad ? nanv : lse;
  }
}

static bool mfma_shape_ok(const Shape& s, int q_len) {
  return s.dtype == 1 && s.dc == kDC && s.dr == kD - kDC && s.page % kSlice == 0 &&
         (q_len * s.H) % kRows == 0;
}

int decode_kernel_kind(const Shape& s, int q_len) { return mfma_shape_ok(s, q_len) ? 1 : 0; }

int launch_decode(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                  const void* q_full, const void* cache, int64_t num_pages,
                  const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                  float* o_part, float* lse_part, void* stream) {
  if (!mfma_shape_ok(s, q_len))
    return launch_decode_generic(s, batch, q_len, num_splits, max_seq_len, q_full, cache,
                                 num_pages, page_table, max_pages, seq_lens, o_part, lse_part,
                                 stream);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)decode_mfma_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
    if (e != hipSuccess) return (int)e;
    attr_set = true;
  }
  const int units = batch * num_splits;
  const int groups = q_len * s.H / kRows;
  const int blocks = ((units + 7) / 8) * 8 * groups;
  const float scale_log2 = s.scale * 1.4426950408889634f;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3(blocks), dim3(256), kLdsBytes,
                     reinterpret_cast<hipStream_t>(stream), q_len, s.H, num_splits, s.page,
                     max_seq_len, scale_log2, units, groups, (const bf16_t*)q_full,
                     (const bf16_t*)cache, num_pages, page_table, max_pages, seq_lens, o_part,
                     lse_part);
  return (int)hipGetLastError();
}

}  // namespace mla
