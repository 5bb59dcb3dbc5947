// Split-KV paged MLA decode on bf16 MFMA for the DeepSeek MLA shape
// (d_c = 512, d_r = 64: 576 bf16 = 1,152 bytes per cached row), gfx950.
//
// What it computes ("The Architecture of Memory", "Flash-Decoding and
// FlashInfer", "The Decode Phase: The Memory Bandwidth Wall"; "DeepSeek's
// Config Says 16 KV Heads", section 5): every query row (query j, head h)
// scores its absorbed query q_full (576 wide) against every cached row of its
// partition, softmaxes the scores online, and weights the 512 latent columns
// of the same rows. All heads read the same cached rows, so one staged tile
// serves many query rows.
//
// Two kernels share the building blocks below:
//
//   decode_slices_kernel (16 query rows per block, e.g. V2-Lite's 16 heads)
//     The 4 waves of a block are independent online-softmax workers over the
//     16-token slices w, w+4, w+8, ... of the partition, each with its own
//     double-buffered LDS slices (no block barrier in the token loop); they
//     merge (max, sum, output) through LDS at the end.
//
//   decode_rows_kernel<RT> (64*RT query rows per block, e.g. 128 heads)
//     The 4 waves share 64-token tiles in LDS (double-buffered, one barrier
//     per tile); wave w owns 16*RT query rows and reads every tile, so each
//     cached byte leaves HBM once per block however many heads there are.
//
// Cache rows move HBM -> LDS with direct-to-LDS 16-byte loads
// (global_load_lds_dwordx4, non-temporal: the cache is streamed once), in a
// XOR-swizzled chunk order: chunk c of row t sits at t*72 + (c ^ (t & 7)), so
// both LDS read patterns are free of bank conflicts. Per 16 tokens:
//   S^T = C . Q^T  : v_mfma_f32_16x16x32_bf16 x 18 (M = tokens, N = 16 rows,
//                    K = 576); C from LDS (ds_read_b128), Q from registers.
//   softmax        : log2 domain; row max across the 4 lane groups by two lane
//                    exchanges; the running max is raised only when a score
//                    exceeds it by more than 2^8, so the accumulator rescale
//                    almost never runs (the result is exact either way: the
//                    sum uses the same reference max).
//   O += P . C     : v_mfma_f32_16x16x16_bf16 x 32 (M = rows, N = 16
//                    features, K = 16 tokens); P straight from the S^T
//                    accumulator layout; C columns gathered with ds_read_b64
//                    from 4 token rows and transposed 4x4 in registers.
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDC = 512;
constexpr int kD = 576;
constexpr int kChunks = kD * 2 / 16;            // 72 sixteen-byte chunks per row
constexpr int kSlice = 16;                      // tokens per MFMA step
constexpr int kSliceChunks = kSlice * kChunks;  // 1152 chunks = 18,432 B
constexpr int kLoads = kSliceChunks / 64;       // 18 wave-wide 16-byte loads per slice
constexpr int kKSteps = kD / 32;                // 18 k-steps (QK)
constexpr int kFB = kDC / 64;                   // 8 feature blocks (PV)
constexpr int kWaves = 4;
constexpr float kLazy = 8.0f;                   // rescale slack, log2 units
constexpr int kAux = 2;                         // non-temporal load

// slices kernel
constexpr int kRowsA = 16;
constexpr size_t kLdsA = (size_t)kWaves * 2 * kSliceChunks * 16;           // 147,456 B
constexpr size_t kEpiA = (size_t)kWaves * kRowsA * kDC * 4 + 1024;        // 132,096 B
constexpr size_t kLdsBytesA = kLdsA > kEpiA ? kLdsA : kEpiA;
// rows kernel
constexpr int kTile = 64;
constexpr int kTileChunks = kTile * kChunks;    // 4608 chunks = 73,728 B
constexpr size_t kLdsBytesB = (size_t)2 * kTileChunks * 16;                // 147,456 B

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// (a & 0xffff) | (b << 16) and (a >> 16) | (b & 0xffff0000), one v_perm_b32
// each (byte selectors index b as bytes 4..7 and a as bytes 0..3)
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ s16x4_t as_s16x4(uint32_t lo, uint32_t hi) {
  u32x2_t v = {lo, hi};
  return __builtin_bit_cast(s16x4_t, v);
}

// Direct-to-LDS copy of one block of 16 cached rows (1152 chunks of 16 B).
// Load i of a lane fills LDS chunk p = base_chunk + 64 i + lane with source
// row t = p / 72, chunk (p % 72) ^ (t & 7): the XOR swizzle is applied on the
// global side, so each load instruction still fills 1 KB of LDS contiguously.
// The per-lane source offsets are the same for every block and are computed
// once; a load is then one scalar M0 write plus one VMEM instruction.
//
// The loads are issued as inline assembly so that the compiler does not treat
// the pending LDS writes as aliasing every later LDS read (it would otherwise
// wait for all outstanding loads before the first read of the other buffer,
// serialising the pipeline); completion is awaited with s_waitcnt vmcnt.
struct RowDma {
  uint32_t off[kLoads];
  __device__ __forceinline__ void init(int base_chunk, int lane) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int p = base_chunk + i * 64 + lane;
      const int t = p / kChunks;
      off[i] = (uint32_t)((t * kChunks + ((p - t * kChunks) ^ (t & 7))) * 16);
    }
  }
  // src: wave-uniform base of the rows; lds_base: LDS byte address of chunk base_chunk
  __device__ __forceinline__ void issue(const void* src, uint32_t lds_base) const {
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                   :
                   : "s"(lds_base + i * 1024), "v"(off[i]), "s"(src)
                   : "memory");
  }
};

// Make the compiler complete the loads behind v here (it then has no loads of
// its own pending when the token loop starts, where its waits would also
// count the in-flight direct-to-LDS loads).
template <typename T>
__device__ __forceinline__ void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Zero the chunks this lane loaded whose row (within the block) is >= first_bad.
__device__ __forceinline__ void zero_rows(u32x4_t* dst, int base_chunk, int lane, int first_bad) {
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int p = base_chunk + i * 64 + lane;
    if (p / kChunks >= first_bad) dst[i * 64 + lane] = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Lane-held page-table window: lane i holds the physical page of unit page
// base + i, so a slice's page is a register read, not a dependent load.
struct PageWindow {
  const int32_t* row;  // page_table + b * max_pages + t0 / page
  int upages, base, reg;
  __device__ __forceinline__ void init(const int32_t* r, int npages, int lane) {
    row = r;
    upages = npages;
    base = 0;
    reg = lane < npages ? row[lane] : 0;
  }
  // physical page of unit page u (wave-uniform u)
  __device__ __forceinline__ int get(int u, int lane) {
    if (u - base >= 64) {
      base = u & ~63;
      reg = base + lane < upages ? row[base + lane] : 0;
      asm volatile("" ::"v"(reg));  // complete this load here, inside the rare branch
    }
    return __builtin_amdgcn_readlane(reg, u - base);
  }
};

// QK of one 16-token slice against RT 16-row tiles of queries.
// A operand: row n of the slice, chunk 4*ks + kg (swizzled): two base chunk
// indices (ks even / odd) plus 8 chunks per ks pair. LDS reads run 3 k-steps
// ahead of the MFMAs, and even / odd k-steps accumulate into separate chains.
template <int RT>
__device__ __forceinline__ void slice_qk(const u32x4_t* buf, int qk0, int qk1,
                                         const bf16x8_t (*qreg)[kKSteps], f32x4_t* sacc) {
  constexpr int kAhead = 3;
  f32x4_t s2[RT][2];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) s2[rt][0] = s2[rt][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  u32x4_t av[kKSteps];
#pragma unroll
  for (int ks = 0; ks < kAhead; ++ks) av[ks] = buf[((ks & 1) ? qk1 : qk0) + 8 * (ks >> 1)];
#pragma unroll
  for (int ks = 0; ks < kKSteps; ++ks) {
    if (ks + kAhead < kKSteps) {
      const int kn = ks + kAhead;
      av[kn] = buf[((kn & 1) ? qk1 : qk0) + 8 * (kn >> 1)];
    }
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av[ks]);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      s2[rt][ks & 1] =
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qreg[rt][ks], s2[rt][ks & 1], 0, 0, 0);
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) sacc[rt] = s2[rt][0] + s2[rt][1];
}

// PV of one 16-token slice: lane (n, kg) gathers features fb*64 + 4n .. +3 of
// token rows 4*kg .. 4*kg+3 (byte bases pv[j]) and transposes them into the 4
// B operands of features fb*64 + 4n + m, m = 0..3. The next feature block's
// LDS reads are issued before this block's MFMAs.
template <int RT>
__device__ __forceinline__ void slice_pv(const char* bufb, const int* pv, const s16x4_t* pa,
                                         f32x4_t (*acc)[kFB][4]) {
  u32x2_t x[2][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[0][j] = *reinterpret_cast<const u32x2_t*>(bufb + pv[j]);
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb) {
    const int cb = fb & 1;
    if (fb + 1 < kFB) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        x[cb ^ 1][j] = *reinterpret_cast<const u32x2_t*>(bufb + pv[j] + (fb + 1) * 128);
    }
    const u32x2_t* y = x[cb];
    const s16x4_t b0 = as_s16x4(pack_lo(y[0].x, y[1].x), pack_lo(y[2].x, y[3].x));
    const s16x4_t b1 = as_s16x4(pack_hi(y[0].x, y[1].x), pack_hi(y[2].x, y[3].x));
    const s16x4_t b2 = as_s16x4(pack_lo(y[0].y, y[1].y), pack_lo(y[2].y, y[3].y));
    const s16x4_t b3 = as_s16x4(pack_hi(y[0].y, y[1].y), pack_hi(y[2].y, y[3].y));
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      acc[rt][fb][0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa[rt], b0, acc[rt][fb][0], 0, 0, 0);
      acc[rt][fb][1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa[rt], b1, acc[rt][fb][1], 0, 0, 0);
      acc[rt][fb][2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa[rt], b2, acc[rt][fb][2], 0, 0, 0);
      acc[rt][fb][3] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa[rt], b3, acc[rt][fb][3], 0, 0, 0);
    }
  }
}

// Max / sum over the 4 lanes {l, l^16, l^32, l^48} (one query row of an MFMA
// accumulator), with the gfx950 lane-swap instructions instead of LDS
// permutes: permlane16_swap pairs lane l with l^16, permlane32_swap with l^32.
__device__ __forceinline__ float row_max4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float row_sum4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Online softmax step for one 16-row tile on one 16-token slice. sacc[r] is
// the score of row n (= lane % 16) against token 4*kg + r; tok0 is the slice's
// first token. Returns the A operand (P in bf16) and updates m, l, acc.
__device__ __forceinline__ s16x4_t slice_softmax(f32x4_t sacc, int tok0, int kg, int p_lim,
                                                 float scale_log2, float& m_run, float& l_run,
                                                 f32x4_t (*acc)[4]) {
  float sv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = tok0 + 4 * kg + r;
    sv[r] = (t <= p_lim) ? sacc[r] * scale_log2 : -INFINITY;
  }
  const float mloc = row_max4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
  // raise the reference max only when a score exceeds it by more than kLazy
  const bool raise = mloc > m_run + kLazy;
  if (__any(raise)) {
    const float m_new = raise ? mloc : m_run;
    const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
    // O is still zero for rows whose max was -inf: only finite rows rescale
    if (__any(raise && m_run != -INFINITY)) {
      const int lane = __lane_id();
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * (lane >> 4) + r, 64);
#pragma unroll
      for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[fb][m][r] *= ar[r];
    }
    m_run = m_new;
  }
  const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(sv[r] - m_use);
  l_run += (p[0] + p[1]) + (p[2] + p[3]);
  bf16x2_t p01 = {(__bf16)p[0], (__bf16)p[1]};
  bf16x2_t p23 = {(__bf16)p[2], (__bf16)p[3]};
  return as_s16x4(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
}

__device__ __forceinline__ void zero_acc(f32x4_t (*acc)[4]) {
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[fb][m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

// block id -> (unit, row group): all groups of one unit share id % 8, i.e.
// run on the same XCD and share its L2
__device__ __forceinline__ bool map_block(int units, int groups, int* unit, int* grp) {
  const int id = blockIdx.x;
  const int kk = id >> 3;
  *unit = (kk / groups) * 8 + (id & 7);
  *grp = kk % groups;
  return *unit < units;
}

}  // namespace

// ---------------------------------------------------------------------------
// 16 query rows per block, token-split waves
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_slices_kernel(int Q, int H, int S, int page, int max_seq_len, float scale_log2,
                          int units, int groups, const bf16_t* __restrict__ q_full,
                          const bf16_t* __restrict__ cache, int64_t num_pages,
                          const int32_t* __restrict__ page_table, int max_pages,
                          const int32_t* __restrict__ seq_lens, float* __restrict__ o_part,
                          float* __restrict__ lse_part) {
  extern __shared__ u32x4_t lds[];
  int unit, grp;
  if (!map_block(units, groups, &unit, &grp)) return;
  const int s = unit % S, b = unit / S;
  const int R = Q * H;
  const int row0 = grp * kRowsA;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15, kg = lane >> 4;

  const int L = seq_lens[b];
  bool bad = (L < Q) || (L > max_seq_len);
  int t0 = 0, t1 = 0;
  if (!bad) split_range(L, S, page, s, &t0, &t1);
  const int nslices = (t1 - t0 + kSlice - 1) / kSlice;

  PageWindow pw;
  pw.init(page_table + (size_t)b * max_pages + t0 / page, (t1 - t0 + page - 1) / page, lane);
  settle(pw.reg);

  u32x4_t* mybuf = lds + wave * 2 * kSliceChunks;
  RowDma dma;
  dma.init(0, lane);
  auto issue = [&](int si, u32x4_t* dst) {
    const int t = t0 + si * kSlice;
    int pg = pw.get((t - t0) / page, lane);
    if (pg < 0 || (int64_t)pg >= num_pages) {
      bad = true;
      pg = 0;
    }
    const bf16_t* src = cache + ((size_t)pg * page + (t % page)) * kD;
    dma.issue(src, __builtin_amdgcn_readfirstlane(lds_addr(dst)));
  };
  // both slice buffers start loading before the queries are fetched
  if (wave < nslices) issue(wave, mybuf);
  if (wave + kWaves < nslices) issue(wave + kWaves, mybuf + kSliceChunks);

  bf16x8_t qreg[1][kKSteps];
  {
    const u32x4_t* qsrc =
        reinterpret_cast<const u32x4_t*>(q_full + ((size_t)b * R + row0 + n) * kD);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks)
      qreg[0][ks] = __builtin_bit_cast(bf16x8_t, qsrc[ks * 4 + kg]);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) settle(qreg[0][ks]);
  }
  const int p_lim = L - Q + (row0 + n) / H;

  // LDS addressing (chunk units for QK, bytes for PV), relative to a slice buffer
  const int qk0 = n * kChunks + (kg ^ (n & 7));
  const int qk1 = n * kChunks + ((4 + kg) ^ (n & 7));
  int pv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * kg + j;
    pv[j] = 16 * (t * kChunks + ((n >> 1) ^ (t & 7))) + 8 * (n & 1);
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t acc[1][kFB][4];
  zero_acc(acc[0]);

  int k = 0;
  for (int si = wave; si < nslices; si += kWaves, ++k) {
    u32x4_t* cur = mybuf + (k & 1) * kSliceChunks;
    if (si + kWaves < nslices)
      wait_vmcnt<kLoads>();  // the next slice may stay in flight
    else
      wait_vmcnt<0>();
    const int ts = t0 + si * kSlice;
    if (ts + kSlice > L) zero_rows(cur, 0, lane, L - ts);  // may hold poison
    f32x4_t sacc[1];
    slice_qk<1>(cur, qk0, qk1, qreg, sacc);
    s16x4_t pa[1];
    pa[0] = slice_softmax(sacc[0], ts, kg, p_lim, scale_log2, m_run, l_run, acc[0]);
    slice_pv<1>(reinterpret_cast<const char*>(cur), pv, pa, acc);
    // refill the buffer just consumed (its LDS reads completed: the MFMAs used them)
    if (si + 2 * kWaves < nslices) issue(si + 2 * kWaves, cur);
  }

  // ---- merge the four waves ------------------------------------------------
  const float l_row = row_sum4(l_run);
  __syncthreads();  // every wave is done with its slice buffers
  float* fl = reinterpret_cast<float*>(lds);
  float* sm = fl + kWaves * kRowsA * kDC;  // m[4][16], l[4][16], bad[4]
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
  float* mine = fl + wave * kRowsA * kDC;
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4 v = make_float4(acc[0][fb][0][r] * fac[r], acc[0][fb][1][r] * fac[r],
                             acc[0][fb][2][r] * fac[r], acc[0][fb][3][r] * fac[r]);
      *reinterpret_cast<float4*>(mine + (4 * kg + r) * kDC + fb * 64 + 4 * n) = v;
    }
  __syncthreads();
  const float nanv = __int_as_float(0x7fc00000);
  const float4* f4 = reinterpret_cast<const float4*>(fl);
  for (int i = threadIdx.x; i < kRowsA * kDC / 4; i += 256) {
    const float4 a = f4[i], b4 = f4[i + 2048], c4 = f4[i + 4096], d4 = f4[i + 6144];
    float4 v = make_float4((a.x + b4.x) + (c4.x + d4.x), (a.y + b4.y) + (c4.y + d4.y),
                           (a.z + b4.z) + (c4.z + d4.z), (a.w + b4.w) + (c4.w + d4.w));
    if (any_bad) v = make_float4(nanv, nanv, nanv, nanv);
    const int row = i / (kDC / 4), col = i % (kDC / 4);
    float4* dst = reinterpret_cast<float4*>(o_part + (((size_t)b * R + row0 + row) * S + s) * kDC);
    dst[col] = v;
  }
  if (threadIdx.x < kRowsA) {
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

// ---------------------------------------------------------------------------
// 64 query rows per block (16 per wave) over shared 64-token tiles
//
// Per tile each wave runs three phases with no branch between the MFMAs of a
// phase, so the 4 independent QK chains and the 32 independent PV products
// overlap their LDS reads:
//   QK   S^T for the 4 16-token subtiles (4 x 18 v_mfma_f32_16x16x32_bf16)
//   max  row max over the 64 tokens (2 permlane swaps), rare rescale, P = 2^(s-m)
//   PV   two 32-token halves with v_mfma_f32_16x16x32_bf16 (K = 32 tokens):
//        the A operand takes the 8 tokens {4kg..4kg+3, 16+4kg..16+4kg+3} of
//        the half straight from two QK accumulators; the B operand gathers the
//        same 8 token rows (ds_read_b64, 4 features each) and transposes 8x4
//        in registers (v_perm_b32).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_tiles_kernel(int Q, int H, int S, int page, int max_seq_len, float scale_log2,
                         int units, int groups, const bf16_t* __restrict__ q_full,
                         const bf16_t* __restrict__ cache, int64_t num_pages,
                         const int32_t* __restrict__ page_table, int max_pages,
                         const int32_t* __restrict__ seq_lens, float* __restrict__ o_part,
                         float* __restrict__ lse_part) {
  extern __shared__ u32x4_t lds[];
  int unit, grp;
  if (!map_block(units, groups, &unit, &grp)) return;
  const int s = unit % S, b = unit / S;
  const int R = Q * H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15, kg = lane >> 4;
  const int row0 = grp * 64 + wave * 16;

  const int L = seq_lens[b];
  const bool bad_len = (L < Q) || (L > max_seq_len);
  int t0 = 0, t1 = 0;
  if (!bad_len) split_range(L, S, page, s, &t0, &t1);
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  bool bad = bad_len;

  PageWindow pw;
  pw.init(page_table + (size_t)b * max_pages + t0 / page, (t1 - t0 + page - 1) / page, lane);
  settle(pw.reg);
  RowDma dma;
  dma.init(wave * kSliceChunks, lane);
  auto issue = [&](int ti, u32x4_t* dst) {
    const int t = t0 + ti * kTile;  // a tile never crosses a page: page % 64 == 0
    int pg = pw.get((t - t0) / page, lane);
    if (pg < 0 || (int64_t)pg >= num_pages) {
      bad = true;
      pg = 0;
    }
    // this wave copies tile rows [16*wave, 16*wave + 16)
    const bf16_t* src = cache + ((size_t)pg * page + (t % page)) * kD;
    dma.issue(src, __builtin_amdgcn_readfirstlane(lds_addr(dst + wave * kSliceChunks)));
  };
  if (ntiles > 0) issue(0, lds);  // the first tile loads while the queries are fetched

  bf16x8_t qreg[kKSteps];
  const int row = row0 + n;
  {
    const u32x4_t* qsrc = reinterpret_cast<const u32x4_t*>(q_full + ((size_t)b * R + row) * kD);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8_t, qsrc[ks * 4 + kg]);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) settle(qreg[ks]);
  }
  const int p_lim = L - Q + row / H;

  // LDS addressing inside a tile: QK reads row 16u + n, chunk 4 ks + kg;
  // PV reads rows 32 v + sigma(kg, j), sigma = {4kg..4kg+3, 16+4kg..16+4kg+3}
  const int qk0 = n * kChunks + (kg ^ (n & 7));
  const int qk1 = n * kChunks + ((4 + kg) ^ (n & 7));
  int pv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = (j < 4) ? 4 * kg + j : 16 + 4 * kg + (j - 4);
    pv[j] = 16 * (t * kChunks + ((n >> 1) ^ (t & 7))) + 8 * (n & 1);
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t acc[kFB][4];
  zero_acc(acc);

  for (int ti = 0; ti < ntiles; ++ti) {
    u32x4_t* cur = lds + (ti & 1) * kTileChunks;
    wait_vmcnt<0>();
    const int ts = t0 + ti * kTile;
    if (ts + kTile > t1)  // rows past the partition end (may be poison)
      zero_rows(cur + wave * kSliceChunks, wave * kSliceChunks, lane, t1 - ts);
    __syncthreads();  // tile ti landed for every wave; tile ti-1 fully consumed
    if (ti + 1 < ntiles) issue(ti + 1, lds + ((ti + 1) & 1) * kTileChunks);

    // ---- QK: 4 independent 18-step chains
    f32x4_t s4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) s4[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // software pipeline: the 4 operands of k-step ks+1 are read while the 4
    // MFMAs of k-step ks issue (the scheduling barriers keep that order)
    u32x4_t a_cur[4], a_nxt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a_cur[u] = cur[qk0 + u * kSliceChunks];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + 1 < kKSteps) {
        const int kn = ks + 1;
        const int base = ((kn & 1) ? qk1 : qk0) + 8 * (kn >> 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) a_nxt[u] = cur[base + u * kSliceChunks];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        s4[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a_cur[u]),
                                                        qreg[ks], s4[u], 0, 0, 0);
      if (ks + 1 < kKSteps) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then 4 MFMA
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) a_cur[u] = a_nxt[u];
    }
    // ---- softmax over the tile's 64 tokens (lane: row n, tokens 16u + 4kg + r)
    float sv[16];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = ts + 16 * u + 4 * kg + r;
        sv[4 * u + r] = (t <= p_lim) ? s4[u][r] * scale_log2 : -INFINITY;
      }
    float mloc = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, sv[i]);
    mloc = row_max4(mloc);
    const bool raise = mloc > m_run + kLazy;
    if (__any(raise)) {
      const float m_new = raise ? mloc : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      if (__any(raise && m_run != -INFINITY)) {
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
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    float lsum = 0.0f;
    uint32_t pk[8];  // P as bf16 pairs: half v, tokens sigma(kg, 0..7)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int u = 2 * v + h;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = __builtin_amdgcn_exp2f(sv[4 * u + r] - m_use);
          lsum += p[r];
        }
        bf16x2_t p01 = {(__bf16)p[0], (__bf16)p[1]};
        bf16x2_t p23 = {(__bf16)p[2], (__bf16)p[3]};
        pk[4 * v + 2 * h] = __builtin_bit_cast(uint32_t, p01);
        pk[4 * v + 2 * h + 1] = __builtin_bit_cast(uint32_t, p23);
      }
    l_run += lsum;
    // ---- PV: two 32-token halves, K = 32; the 8 rows of step it+1 are read
    // while step it is transposed and multiplied
    const char* tb = reinterpret_cast<const char*>(cur);
    bf16x8_t pa[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      u32x4_t pav = {pk[4 * v], pk[4 * v + 1], pk[4 * v + 2], pk[4 * v + 3]};
      pa[v] = __builtin_bit_cast(bf16x8_t, pav);
    }
    u32x2_t xa[8], xb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xa[j] = *reinterpret_cast<const u32x2_t*>(tb + pv[j]);
#pragma unroll
    for (int it = 0; it < 2 * kFB; ++it) {
      const int v = it / kFB, fb = it % kFB;
      if (it + 1 < 2 * kFB) {
        const int vn = (it + 1) / kFB, fn = (it + 1) % kFB;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          xb[j] = *reinterpret_cast<const u32x2_t*>(tb + pv[j] + vn * (32 * kChunks * 16) + fn * 128);
      }
      u32x4_t bm[4];
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        bm[0][q2] = pack_lo(xa[2 * q2].x, xa[2 * q2 + 1].x);
        bm[1][q2] = pack_hi(xa[2 * q2].x, xa[2 * q2 + 1].x);
        bm[2][q2] = pack_lo(xa[2 * q2].y, xa[2 * q2 + 1].y);
        bm[3][q2] = pack_hi(xa[2 * q2].y, xa[2 * q2 + 1].y);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
        acc[fb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            pa[v], __builtin_bit_cast(bf16x8_t, bm[m]), acc[fb][m], 0, 0, 0);
      if (it + 1 < 2 * kFB) {
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);   // next step's LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 1);  // this step's transposes
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);   // this step's MFMAs
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) xa[j] = xb[j];
    }
  }
  wait_vmcnt<0>();

  // ---- write this wave's 16 rows ------------------------------------------
  const float nanv = __int_as_float(0x7fc00000);
  const float l_row = row_sum4(l_run);
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lr = __shfl(l_row, 4 * kg + r, 64);
    inv[r] = lr > 0.0f ? 1.0f / lr : 0.0f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int orow = row0 + 4 * kg + r;
    float* dst = o_part + (((size_t)b * R + orow) * S + s) * kDC + 4 * n;
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) {
      float4 v = make_float4(acc[fb][0][r] * inv[r], acc[fb][1][r] * inv[r],
                             acc[fb][2][r] * inv[r], acc[fb][3][r] * inv[r]);
      if (bad) v = make_float4(nanv, nanv, nanv, nanv);
      *reinterpret_cast<float4*>(dst + fb * 64) = v;
    }
  }
  if (kg == 0) {
    const float lse = l_row > 0.0f ? (m_run + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
    lse_part[((size_t)b * R + row) * S + s] = bad ? nanv : lse;
  }
}

namespace {

int pick_kernel(const Shape& s, int q_len) {
  if (!(s.dtype == 1 && s.dc == kDC && s.dr == kD - kDC)) return 0;
  const int R = q_len * s.H;
  if (s.page % 64 == 0 && R % 64 == 0) return 2;   // rows kernel, 16 rows per wave
  if (s.page % kSlice == 0 && R % kRowsA == 0) return 1;
  return 0;
}

template <typename K>
int set_lds(K kernel, size_t bytes, bool* done) {
  if (*done) return 0;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return (int)e;
  *done = true;
  return 0;
}

}  // namespace

int decode_kernel_kind(const Shape& s, int q_len) { return pick_kernel(s, q_len) ? 1 : 0; }

int launch_decode(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                  const void* q_full, const void* cache, int64_t num_pages,
                  const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                  float* o_part, float* lse_part, void* stream) {
  const int kind = pick_kernel(s, q_len);
  if (kind == 0)
    return launch_decode_generic(s, batch, q_len, num_splits, max_seq_len, q_full, cache,
                                 num_pages, page_table, max_pages, seq_lens, o_part, lse_part,
                                 stream);
  const int units = batch * num_splits;
  const int R = q_len * s.H;
  const float scale_log2 = s.scale * 1.4426950408889634f;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const bf16_t* q = (const bf16_t*)q_full;
  const bf16_t* c = (const bf16_t*)cache;
  if (kind == 1) {
    static bool attr = false;
    int rc = set_lds(decode_slices_kernel, kLdsBytesA, &attr);
    if (rc) return rc;
    const int groups = R / kRowsA;
    const int blocks = ((units + 7) / 8) * 8 * groups;
    hipLaunchKernelGGL(decode_slices_kernel, dim3(blocks), dim3(256), kLdsBytesA, st, q_len, s.H,
                       num_splits, s.page, max_seq_len, scale_log2, units, groups, q, c, num_pages,
                       page_table, max_pages, seq_lens, o_part, lse_part);
  } else {
    static bool attr = false;
    int rc = set_lds(decode_tiles_kernel, kLdsBytesB, &attr);
    if (rc) return rc;
    const int groups = R / 64;
    const int blocks = ((units + 7) / 8) * 8 * groups;
    hipLaunchKernelGGL(decode_tiles_kernel, dim3(blocks), dim3(256), kLdsBytesB, st, q_len, s.H,
                       num_splits, s.page, max_seq_len, scale_log2, units, groups, q, c, num_pages,
                       page_table, max_pages, seq_lens, o_part, lse_part);
  }
  return (int)hipGetLastError();
}

}  // namespace mla
