// bf16 MFMA kernels for the two per-query projections of the decode step:
// query absorption through W_UK (a1) and value up-projection through W_UV
// (a6) ("The Architecture of Memory", "The Weight Absorption Trick";
// "Beyond the Attention Bottleneck", "Down-Projection and Up-Projection
// Mechanics"). Both are small GEMMs per head (tokens x d_n x d_c and
// tokens x d_c x d_v) that stream the weights once; the point of these
// kernels is to spread that stream over hundreds of waves.
#include <hip/hip_runtime.h>
#include <math.h>

#include "mla_append.h"
#include "mla_append_coded.h"
#include "mla_combine.h"
#include "mla_common.h"
#include "mla_launch.h"

namespace mla {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

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
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace

// ---------------------------------------------------------------------------
// a1: q_full[n][h][0:d_c] = W_UK[h]^T q_nope[n][h]; q_full[n][h][d_c:] = RoPE.
// grid (H, d_c / 64 + 1, ceil(N / 16)). Blocks y < d_c / 64 own 64 output
// columns of 16 tokens; their 4 waves split the d_n contraction (wave w takes
// rows [w d_n / 4, (w + 1) d_n / 4)) and sum through LDS. The last block row
// (y = d_c / 64) rotates the RoPE part, in parallel with the contraction.
// v_mfma_f32_16x16x16_bf16 with M = 16 tokens, K = 16 rows of W_UK, N = 16
// columns. W_UK is row-major [d_n][d_c], so a lane loads 8 contiguous bytes
// (4 columns) from each of 4 rows and transposes the 4x4 block in registers
// into 4 B operands; MFMA m then covers columns c0 + 4*(lane%16) + m. All
// loads of a 32-row step are issued before its MFMAs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void absorb_block(int h, int by, int bz, int n_tok, int H, int dn, int dc,
                                             int dr, double log2_base,
                                             const bf16_t* __restrict__ q_nope,
                                             const bf16_t* __restrict__ q_rope,
                                             const int32_t* __restrict__ pos,
                                             const bf16_t* __restrict__ w_uk,
                                             bf16_t* __restrict__ q_full) {
  __shared__ f32x4_t red[3][4][64];
  const int n0 = bz * 16;
  const int D = dc + dr;
  if (by == dc / 64) {
    const int half = dr / 2;
    const int nt = min(16, n_tok - n0);
    for (int i = threadIdx.x; i < nt * half; i += blockDim.x) {
      const int n = n0 + i / half, p = i % half;
      const bf16_t* src = q_rope + ((size_t)n * H + h) * dr + 2 * p;
      double y0, y1;
      rope_pair(bf2f(src[0]), bf2f(src[1]), pos[n], p, dr, log2_base, &y0, &y1);
      bf16_t* dst = q_full + ((size_t)n * H + h) * D + dc + 2 * p;
      dst[0] = f2bf((float)y0);
      dst[1] = f2bf((float)y1);
    }
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nn = lane & 15, g = lane >> 4;
  const int c0 = by * 64;
  const int tok = n0 + nn;  // A-operand row of this lane
  const bool tok_ok = tok < n_tok;
  const bf16_t* qrow = q_nope + ((size_t)(tok_ok ? tok : 0) * H + h) * dn;
  const bf16_t* W = w_uk + (size_t)h * dn * dc + c0 + 4 * nn;
  const int kw = dn / 4;  // rows per wave, a multiple of 16
  const int i_end = (wave + 1) * kw;
  f32x4_t acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  auto step = [&](const u32x2_t& qa, const u32x2_t* x) {
    const s16x4_t a = __builtin_bit_cast(s16x4_t, qa);
    const s16x4_t b0 = as_s16x4(pack_lo(x[0].x, x[1].x), pack_lo(x[2].x, x[3].x));
    const s16x4_t b1 = as_s16x4(pack_hi(x[0].x, x[1].x), pack_hi(x[2].x, x[3].x));
    const s16x4_t b2 = as_s16x4(pack_lo(x[0].y, x[1].y), pack_lo(x[2].y, x[3].y));
    const s16x4_t b3 = as_s16x4(pack_hi(x[0].y, x[1].y), pack_hi(x[2].y, x[3].y));
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b0, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b1, acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b2, acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b3, acc[3], 0, 0, 0);
  };
  int i0 = wave * kw;
  for (; i0 + 32 <= i_end; i0 += 32) {
    u32x2_t qa[2], x[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      qa[u] = *reinterpret_cast<const u32x2_t*>(qrow + i0 + 16 * u + 4 * g);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        x[u][j] = *reinterpret_cast<const u32x2_t*>(W + (size_t)(i0 + 16 * u + 4 * g + j) * dc);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (!tok_ok) qa[u] = u32x2_t{0u, 0u};
      step(qa[u], x[u]);
    }
  }
  if (i0 < i_end) {  // one 16-row step left
    u32x2_t qa = *reinterpret_cast<const u32x2_t*>(qrow + i0 + 4 * g);
    u32x2_t x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[j] = *reinterpret_cast<const u32x2_t*>(W + (size_t)(i0 + 4 * g + j) * dc);
    if (!tok_ok) qa = u32x2_t{0u, 0u};
    step(qa, x);
  }
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) red[wave - 1][m][lane] = acc[m];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[m] += (red[0][m][lane] + red[1][m][lane]) + red[2][m][lane];
    // lane holds tokens n0 + 4g + r, columns c0 + 4*nn + m (m = 0..3)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = n0 + 4 * g + r;
      if (t < n_tok) {
        u32x2_t v = {pack_bf16x2(acc[0][r], acc[1][r]), pack_bf16x2(acc[2][r], acc[3][r])};
        *reinterpret_cast<u32x2_t*>(q_full + ((size_t)t * H + h) * D + c0 + 4 * nn) = v;
      }
    }
  }
}

__global__ __launch_bounds__(256) void absorb_q_mfma_kernel(
    int n_tok, int H, int dn, int dc, int dr, double log2_base, const bf16_t* __restrict__ q_nope,
    const bf16_t* __restrict__ q_rope, const int32_t* __restrict__ pos,
    const bf16_t* __restrict__ w_uk, bf16_t* __restrict__ q_full) {
  absorb_block(blockIdx.x, blockIdx.y, blockIdx.z, n_tok, H, dn, dc, dr, log2_base, q_nope, q_rope,
               pos, w_uk, q_full);
}

// a1 + a2 in one launch: blocks [0, n_abs) are the blocks of
// absorb_q_mfma_kernel in its own order (x fastest), the next n_app blocks
// append one row each, and with dI > 0 (a sparse read) the n_app after those
// append the rows' indexer keys.
__global__ __launch_bounds__(256) void absorb_append_kernel(
    int n_tok, int H, int dn, int dc, int dr, double log2_base, const bf16_t* __restrict__ q_nope,
    const bf16_t* __restrict__ q_rope, const int32_t* __restrict__ pos_q,
    const bf16_t* __restrict__ w_uk, bf16_t* __restrict__ q_full, int ny, int n_abs, int page,
    const bf16_t* __restrict__ c_kv, const bf16_t* __restrict__ k_rope,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ rope_pos, const int32_t* __restrict__ page_table, int batch,
    int max_pages, bf16_t* __restrict__ cache, int64_t num_pages, int rotate, int vec, int n_app,
    int dI, const bf16_t* __restrict__ k_idx, bf16_t* __restrict__ icache) {
  const int id = blockIdx.x;
  if (id < n_abs) {
    absorb_block(id % H, (id / H) % ny, id / (H * ny), n_tok, H, dn, dc, dr, log2_base, q_nope,
                 q_rope, pos_q, w_uk, q_full);
  } else if (id < n_abs + n_app) {
    append_row<bf16_t>(id - n_abs, dc, dr, page, c_kv, k_rope, seq_idx, pos, rope_pos, page_table,
                       batch, max_pages, cache, num_pages, rotate, log2_base, vec);
  } else {
    index_append_row<bf16_t>(id - n_abs - n_app, dI, page, k_idx, seq_idx, pos, page_table, batch,
                             max_pages, icache, num_pages);
  }
}

// a1 + the coded append (8 or 4 bits) in one launch: the absorb blocks as
// in absorb_append_kernel, then one block per appended row running the
// append kernel's body (append_coded_row) with 256 threads.
template <int kBits>
__global__ __launch_bounds__(256) void absorb_append_coded_kernel(
    int n_tok, int H, int dn, int dc, int dr, double log2_base, const bf16_t* __restrict__ q_nope,
    const bf16_t* __restrict__ q_rope, const int32_t* __restrict__ pos_q,
    const bf16_t* __restrict__ w_uk, bf16_t* __restrict__ q_full, int ny, int n_abs, int page,
    const bf16_t* __restrict__ c_kv, const bf16_t* __restrict__ k_rope,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ rope_pos, const int32_t* __restrict__ page_table, int batch,
    int max_pages, uint8_t* __restrict__ cache, int64_t num_pages, int rotate) {
  const int id = blockIdx.x;
  if (id < n_abs) {
    absorb_block(id % H, (id / H) % ny, id / (H * ny), n_tok, H, dn, dc, dr, log2_base, q_nope,
                 q_rope, pos_q, w_uk, q_full);
  } else {
    append_coded_row<bf16_t, kBits>(id - n_abs, dc, dr, page, c_kv, k_rope, seq_idx, pos,
                                    rope_pos, page_table, batch, max_pages, cache, num_pages,
                                    rotate, log2_base);
  }
}

bool absorb_mfma_ok(const Shape& s) { return s.dtype == 1 && s.dn % 64 == 0 && s.dc % 64 == 0; }

int launch_absorb_append_coded(int bits, const Shape& s, int n_tok, const void* q_nope,
                               const void* q_rope, const int32_t* pos_q, const void* w_uk,
                               void* q_full, int n_app, const void* c_kv, const void* k_rope,
                               const int32_t* seq_idx, const int32_t* pos,
                               const int32_t* rope_pos, const int32_t* page_table, int batch,
                               int max_pages, void* cache, int64_t num_pages, int rotate,
                               void* stream) {
  if (!absorb_mfma_ok(s) || n_tok == 0 || n_app == 0) {
    int rc = 0;
    if (n_tok > 0) rc = launch_absorb_q(s, n_tok, q_nope, q_rope, pos_q, w_uk, q_full, stream);
    if (rc == 0 && n_app > 0)
      rc = bits == 8 ? launch_cache_append_q8(s, n_app, c_kv, k_rope, seq_idx, pos, rope_pos,
                                              page_table, batch, max_pages, cache, num_pages,
                                              rotate, stream)
                     : launch_cache_append_q4(s, n_app, c_kv, k_rope, seq_idx, pos, rope_pos,
                                              page_table, batch, max_pages, cache, num_pages,
                                              rotate, stream);
    return rc;
  }
  const int ny = s.dc / 64 + 1;
  const int n_abs = s.H * ny * ((n_tok + 15) / 16);
  auto kern = bits == 8 ? absorb_append_coded_kernel<8> : absorb_append_coded_kernel<4>;
  hipLaunchKernelGGL(kern, dim3(n_abs + n_app), dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     n_tok, s.H, s.dn, s.dc, s.dr, s.log2_base, (const bf16_t*)q_nope,
                     (const bf16_t*)q_rope, pos_q, (const bf16_t*)w_uk, (bf16_t*)q_full, ny, n_abs,
                     s.page, (const bf16_t*)c_kv, (const bf16_t*)k_rope, seq_idx, pos, rope_pos,
                     page_table, batch, max_pages, (uint8_t*)cache, num_pages, rotate);
  return (int)hipGetLastError();
}

int launch_absorb_q_mfma(const Shape& s, int n_tok, const void* q_nope, const void* q_rope,
                         const int32_t* pos, const void* w_uk, void* q_full, void* stream) {
  dim3 grid(s.H, s.dc / 64 + 1, (n_tok + 15) / 16);
  hipLaunchKernelGGL(absorb_q_mfma_kernel, grid, dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), n_tok, s.H, s.dn, s.dc, s.dr,
                     s.log2_base, (const bf16_t*)q_nope, (const bf16_t*)q_rope, pos,
                     (const bf16_t*)w_uk, (bf16_t*)q_full);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// a6: out[n][h][v] = sum_c W_UV[h][v][c] o_lat[n][h][c].
// grid (H, d_v / 16, ceil(N / 16)); 4 waves split the d_c contraction (wave
// w takes 32-wide k-steps w, w+4, ..., loading 4 of them before their
// MFMAs), then sum through LDS.
// v_mfma_f32_16x16x32_bf16 with M = 16 tokens, N = 16 rows v of W_UV,
// K = 32 latent columns: both operands are contiguous 16-byte loads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void up_v_mfma_kernel(int n_tok, int H, int dc, int dv,
                                                        const bf16_t* __restrict__ o_lat,
                                                        const bf16_t* __restrict__ w_uv,
                                                        bf16_t* __restrict__ out) {
  __shared__ f32x4_t red[4][64];
  const int h = blockIdx.x;
  const int v0 = blockIdx.y * 16;
  const int n0 = blockIdx.z * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nn = lane & 15, g = lane >> 4;
  const int tok = n0 + nn;
  const bool tok_ok = tok < n_tok;
  const bf16_t* arow = o_lat + ((size_t)(tok_ok ? tok : 0) * H + h) * dc + 8 * g;
  const bf16_t* brow = w_uv + ((size_t)h * dv + v0 + nn) * dc + 8 * g;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // 4 k-steps per iteration (all of d_c = 512 in one): loads first, then MFMAs
  for (int k0 = wave * 32; k0 < dc; k0 += 4 * 128) {
    u32x4_t av[4], bv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * 128;
      const bool in = k < dc;
      av[u] = (in && tok_ok) ? *reinterpret_cast<const u32x4_t*>(arow + k) : u32x4_t{0u, 0u, 0u, 0u};
      bv[u] = in ? *reinterpret_cast<const u32x4_t*>(brow + k) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                    __builtin_bit_cast(bf16x8_t, bv[u]), acc, 0, 0, 0);
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t s = red[0][lane] + red[1][lane];
    s += red[2][lane] + red[3][lane];
    // lane holds tokens n0 + 4g + r, column v0 + nn
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = n0 + 4 * g + r;
      if (t < n_tok) out[((size_t)t * H + h) * dv + v0 + nn] = f2bf(s[r]);
    }
  }
}

int launch_absorb_append(const Shape& s, int n_tok, const void* q_nope, const void* q_rope,
                         const int32_t* pos_q, const void* w_uk, void* q_full, int n_app,
                         const void* c_kv, const void* k_rope, const int32_t* seq_idx,
                         const int32_t* pos, const int32_t* rope_pos, const int32_t* page_table,
                         int batch, int max_pages, void* cache, int64_t num_pages, int rotate,
                         void* stream, int dI, const void* k_idx, void* icache) {
  if (!absorb_mfma_ok(s) || n_tok == 0 || n_app == 0) {
    int rc = 0;
    if (n_tok > 0) rc = launch_absorb_q(s, n_tok, q_nope, q_rope, pos_q, w_uk, q_full, stream);
    if (rc == 0 && n_app > 0)
      rc = launch_cache_append(s, n_app, c_kv, k_rope, seq_idx, pos, rope_pos, page_table, batch,
                               max_pages, cache, num_pages, rotate, stream);
    if (rc == 0 && n_app > 0 && dI > 0)
      rc = launch_index_append(s, dI, n_app, k_idx, seq_idx, pos, page_table, batch, max_pages,
                               icache, num_pages, stream);
    return rc;
  }
  const int ny = s.dc / 64 + 1;
  const int n_abs = s.H * ny * ((n_tok + 15) / 16);
  const int n_idx = dI > 0 ? n_app : 0;
  hipLaunchKernelGGL(absorb_append_kernel, dim3(n_abs + n_app + n_idx), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), n_tok, s.H, s.dn, s.dc, s.dr,
                     s.log2_base, (const bf16_t*)q_nope, (const bf16_t*)q_rope, pos_q,
                     (const bf16_t*)w_uk, (bf16_t*)q_full, ny, n_abs, s.page, (const bf16_t*)c_kv,
                     (const bf16_t*)k_rope, seq_idx, pos, rope_pos, page_table, batch, max_pages,
                     (bf16_t*)cache, num_pages, rotate, append_vectorizable(s, c_kv, cache), n_app,
                     dI, (const bf16_t*)k_idx, (bf16_t*)icache);
  return (int)hipGetLastError();
}

bool up_v_mfma_ok(const Shape& s) { return s.dtype == 1 && s.dc % 32 == 0 && s.dv % 16 == 0; }

int launch_up_project_v_mfma(const Shape& s, int n_tok, const void* o_lat, const void* w_uv,
                             void* out, void* stream) {
  dim3 grid(s.H, s.dv / 16, (n_tok + 15) / 16);
  hipLaunchKernelGGL(up_v_mfma_kernel, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     n_tok, s.H, s.dc, s.dv, (const bf16_t*)o_lat, (const bf16_t*)w_uv,
                     (bf16_t*)out);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// a5 + a6 in one launch (bf16, d_c = 512, d_v = 128): two blocks of 6 waves
// per output row r = (token n, head h), block half j taking value columns
// [64 j, 64 j + 64): twice as many CUs share the partial and W_UV streams
// (both halves merge the whole row, which costs less than it saves).
//   waves 0, 1  merge columns [256 w, 256 w + 256) of the row exactly as the
//               combine kernel does (wave 0 also forms the weights), with the
//               row's LSEs and all of its S <= 32 partitions loaded at once;
//               the bf16 row goes to LDS, and (half 0 only) to o_lat and lse.
//   waves 2..5  load their W_UV[h] operands once the merge's loads are
//               queued (they depend on nothing), then run the MFMA sequence
//               of up_v_mfma_kernel's wave (w - 2) for this token and the
//               half's 4 v-tiles, with the token in A-operand row 0 and zeros
//               in the other rows (an MFMA output row depends only on its own
//               A row), and sum across waves in that kernel's order, so both
//               paths give the same bits.
// Blocks of one head share blockIdx % 8 (one XCD, one L2) when H % 8 == 0.
// The barriers order LDS traffic only, so they wait for LDS operations, not
// for the loads still in flight.
// ---------------------------------------------------------------------------
constexpr int kFusedDc = 512, kFusedDv = 128;
constexpr int kFusedVt = kFusedDv / 16 / 2;  // 4 v-tiles of 16 rows per block
constexpr int kFusedKs = kFusedDc / 128;     // 4 k-steps per up-projection wave
constexpr int kFusedSplits = 32;             // at most this many partitions

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__global__ __launch_bounds__(384) void combine_up_v_kernel(
    int n_tok, int H, int S, const float* __restrict__ o_part, const float* __restrict__ lse_part,
    bf16_t* __restrict__ o_lat, float* __restrict__ lse, const bf16_t* __restrict__ w_uv,
    bf16_t* __restrict__ out) {
  __shared__ float w[kFusedSplits];
  __shared__ u32x4_t orow[kFusedDc / 8];             // the bf16 o_lat row, 16-byte chunks
  __shared__ f32x4_t red[4][kFusedVt][64];
  __shared__ float cw_s[3];
  const int half = blockIdx.x & 1;
  const int id = blockIdx.x >> 1;
  int n, h;
  if (H % 8 == 0) {
    const int rest = id >> 3;
    n = rest % n_tok;
    h = (rest / n_tok) * 8 + (id & 7);
  } else {
    n = id / H;
    h = id % H;
  }
  const size_t r = (size_t)n * H + h;
  const int lane = threadIdx.x & 63;
  // wave-uniform (a scalar branch below): the two roles each pass the same
  // four block barriers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nn = lane & 15, g = lane >> 4;

  if (wave < 2) {
    const int col = wave * kCombCols + 4 * lane;
    // the row's LSEs first, then all of its partitions: these loads are
    // queued before the W_UV loads of the other waves (start barrier)
    const float lv = (wave == 0 && lane < S) ? lse_part[r * S + lane] : 0.0f;
    CombineCols<kFusedSplits, true> cc;  // every partition in flight at once
    cc.start(o_part + r * S * kFusedDc, S, kFusedDc, col);
    lds_barrier();  // start
    if (wave == 0) {
      const CombineWeights cw = combine_weights_one(lv, S, w, lane);
      if (lane == 0) {
        cw_s[0] = cw.mx;
        cw_s[1] = cw.sum;
        cw_s[2] = cw.bad ? 1.0f : 0.0f;
        if (lse && half == 0) lse[r] = cw.lse();
      }
    }
    lds_barrier();  // weights ready
    const CombineWeights cw = {cw_s[0], cw_s[1], cw_s[2] != 0.0f};
    const float4 v = cc.finish(w, cw, lane);
    if (half == 0) store4<bf16_t>(o_lat + r * kFusedDc + col, v);
    uint2 u;
    u.x = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
    u.y = (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16);
    reinterpret_cast<uint2*>(orow)[col / 4] = u;
    lds_barrier();  // row in LDS
    lds_barrier();  // partial sums in LDS
    return;
  }
  lds_barrier();  // start
  const int uw = wave - 2;  // the up-projection wave this one replays
  const int vt0 = half * kFusedVt;
  const bf16_t* brow =
      w_uv + ((size_t)h * kFusedDv + vt0 * 16 + nn) * kFusedDc + 8 * g + 32 * uw;
  u32x4_t bv[kFusedVt][kFusedKs];
#pragma unroll
  for (int vt = 0; vt < kFusedVt; ++vt)
#pragma unroll
    for (int i = 0; i < kFusedKs; ++i)
      bv[vt][i] = *reinterpret_cast<const u32x4_t*>(brow + (size_t)vt * 16 * kFusedDc + 128 * i);
  lds_barrier();  // weights ready
  lds_barrier();  // row in LDS
  f32x4_t acc[kFusedVt];
#pragma unroll
  for (int vt = 0; vt < kFusedVt; ++vt) acc[vt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < kFusedKs; ++i) {
    const int k = 32 * uw + 128 * i;
    const u32x4_t av = (nn == 0) ? orow[(k + 8 * g) / 8] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int vt = 0; vt < kFusedVt; ++vt)
      acc[vt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                        __builtin_bit_cast(bf16x8_t, bv[vt][i]),
                                                        acc[vt], 0, 0, 0);
  }
#pragma unroll
  for (int vt = 0; vt < kFusedVt; ++vt) red[uw][vt][lane] = acc[vt];
  lds_barrier();  // partial sums in LDS
  // v-tile uw of this half; output row 0 (token n) sits in lanes g == 0, r = 0
  {
    const int vt = uw;
    f32x4_t sum = red[0][vt][lane] + red[1][vt][lane];
    sum += red[2][vt][lane] + red[3][vt][lane];
    if (g == 0) out[r * kFusedDv + (vt0 + vt) * 16 + nn] = f2bf(sum[0]);
  }
}

// ---------------------------------------------------------------------------
// a5 + a6 in one launch for many rows (2,048 or more; bf16, d_c = 512,
// d_v = 128, S <= 64): one block of 8 waves per (head h, 16
// tokens), so W_UV[h] is read once per 16 tokens rather than once per row.
//   merge    wave w merges rows (token n0 + 2 w + i, head h), i = 0, 1, both
//            256-column halves, with the combine kernel's arithmetic (the
//            same weights, partitions added in the same order); the loads of
//            all four (row, half) items are issued before the first is
//            added. The bf16 rows go to o_lat, lse and an LDS tile (zero rows
//            for tokens past n_tok).
//   project  wave w computes v-tile w (rows 16 w .. 16 w + 15 of W_UV[h]) for
//            the 16 tokens: the four k-step chains of up_v_mfma_kernel's
//            waves, each in its order, summed as that kernel sums them, so
//            the output has the bits of the two separate launches.
// Blocks of one head share blockIdx % 8 (one XCD, one L2) when H % 8 == 0.
// ---------------------------------------------------------------------------
constexpr int kGrpTok = 16;
constexpr int kGrpSplits = 64;
constexpr int kGrpWaves = kFusedDv / 16;          // one v-tile per wave
constexpr int kGrpRowBytes = kFusedDc * 2 + 16;   // padded: rows start 4 banks apart
static_assert(2 * kGrpWaves == kGrpTok, "two merged rows per wave");

template <int kCH>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
void combine_up_v_group_kernel(
    int n_tok, int H, int S, const float* __restrict__ o_part, const float* __restrict__ lse_part,
    bf16_t* __restrict__ o_lat, float* __restrict__ lse, const bf16_t* __restrict__ w_uv,
    bf16_t* __restrict__ out) {
  __shared__ float w[kGrpWaves][2][kGrpSplits];
  __shared__ u32x4_t tile[kGrpTok * kGrpRowBytes / 16];
  const int ngrp = (n_tok + kGrpTok - 1) / kGrpTok;
  const int id = blockIdx.x;
  int grp, h;
  if (H % 8 == 0) {
    const int rest = id >> 3;
    grp = rest % ngrp;
    h = (rest / ngrp) * 8 + (id & 7);
  } else {
    grp = id / H;
    h = id % H;
  }
  const int n0 = grp * kGrpTok;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nn = lane & 15, g = lane >> 4;
  char* tb = reinterpret_cast<char*>(tile);

  // ---- merge: item j = (row 2 wave + (j >> 1), half j & 1)
  CombineCols<kCH> cc[4];  // kCH partitions in flight per item (2 when S <= 2)
  float lv[2];
  size_t rr[2];
  bool ok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int n = n0 + 2 * wave + i;
    ok[i] = n < n_tok;
    rr[i] = (size_t)(ok[i] ? n : 0) * H + h;  // rows past n_tok load row (0, h) and drop it
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    cc[j].start(o_part + rr[j >> 1] * S * kFusedDc, S, kFusedDc, (j & 1) * kCombCols + 4 * lane);
#pragma unroll
  for (int i = 0; i < 2; ++i) lv[i] = lane < S ? lse_part[rr[i] * S + lane] : 0.0f;
  CombineWeights cw[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) cw[i] = combine_weights_one(lv[i], S, w[wave][i], lane);
  __syncthreads();  // weights visible to every lane
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = j >> 1;
    const int col = (j & 1) * kCombCols + 4 * lane;
    const float4 v = cc[j].finish(w[wave][i], cw[i], lane);
    if (ok[i]) {
      store4<bf16_t>(o_lat + rr[i] * kFusedDc + col, v);
      if (lse && (j & 1) == 0 && lane == 0) lse[rr[i]] = cw[i].lse();
    }
    uint2 u = {0u, 0u};
    if (ok[i]) {
      u.x = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
      u.y = (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16);
    }
    *reinterpret_cast<uint2*>(tb + (2 * wave + i) * kGrpRowBytes + 2 * col) = u;
  }
  // W_UV[h] operands of v-tile `wave`: chain c, step i covers latent columns
  // 32 c + 128 i + 8 g .. + 7 of row 16 wave + nn. Loaded after the merge
  // (the other block on the CU covers their latency), which keeps the
  // register peak low enough for two blocks per CU.
  const bf16_t* brow = w_uv + ((size_t)h * kFusedDv + 16 * wave + nn) * kFusedDc + 8 * g;
  u32x4_t bv[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      bv[c][i] = *reinterpret_cast<const u32x4_t*>(brow + 32 * c + 128 * i);
  __syncthreads();  // the 16 rows are in LDS

  // ---- project: v_mfma_f32_16x16x32_bf16, M = 16 tokens, N = 16 rows of W_UV
  f32x4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4_t av =
          *reinterpret_cast<const u32x4_t*>(tb + nn * kGrpRowBytes + 2 * (32 * c + 128 * i + 8 * g));
      acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                       __builtin_bit_cast(bf16x8_t, bv[c][i]),
                                                       acc[c], 0, 0, 0);
    }
  f32x4_t sum = acc[0] + acc[1];
  sum += acc[2] + acc[3];
  // lane holds tokens n0 + 4 g + r, value column 16 wave + nn
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = n0 + 4 * g + r;
    if (t < n_tok) out[((size_t)t * H + h) * kFusedDv + 16 * wave + nn] = f2bf(sum[r]);
  }
}

// Which form merges and projects fastest (GPU time of each, measured by graph
// replay at 16 heads and 16 or 32 partitions): the per-row kernel reads
// W_UV[h] for every row (128 KB), so it wins only while the rows are few
// (128 rows: 4.9 against 5.7 us for the two launches; 256: 8.2 against 6.1);
// the per-(head, 16 tokens) kernel needs enough token groups to fill the
// chip (1,024 rows: 16.3 against 10.7 us; 2,048: 18.4 against 18.4; 4,096:
// 25.3 against 31.0); the two launches are best in between.
constexpr int kRowFormMaxRows = 160;
constexpr int kGrpFormMinRows = 2048;

int launch_combine_up_project(const Shape& s, int n_tok, int num_splits, const float* o_part,
                              const float* lse_part, void* o_lat, float* lse, const void* w_uv,
                              void* out, void* stream) {
  const bool shape_ok = s.dtype == 1 && s.dc == kFusedDc && s.dv == kFusedDv;
  const int rows = n_tok * s.H;
  if (shape_ok && rows >= kGrpFormMinRows && num_splits <= kGrpSplits) {
    const int blocks = s.H * ((n_tok + kGrpTok - 1) / kGrpTok);
    auto kern = num_splits <= 2 ? combine_up_v_group_kernel<2> : combine_up_v_group_kernel<4>;
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * kGrpWaves), 0,
                       reinterpret_cast<hipStream_t>(stream), n_tok, s.H, num_splits, o_part,
                       lse_part, (bf16_t*)o_lat, lse, (const bf16_t*)w_uv, (bf16_t*)out);
    return (int)hipGetLastError();
  }
  if (!(shape_ok && rows <= kRowFormMaxRows && num_splits <= kFusedSplits)) {
    int rc = launch_combine(s, n_tok * s.H, num_splits, o_part, lse_part, o_lat, lse, stream);
    if (rc == 0) rc = launch_up_project_v(s, n_tok, o_lat, w_uv, out, stream);
    return rc;
  }
  hipLaunchKernelGGL(combine_up_v_kernel, dim3(2 * n_tok * s.H), dim3(384), 0,
                     reinterpret_cast<hipStream_t>(stream), n_tok, s.H, num_splits, o_part,
                     lse_part, (bf16_t*)o_lat, lse, (const bf16_t*)w_uv, (bf16_t*)out);
  return (int)hipGetLastError();
}

}  // namespace mla
