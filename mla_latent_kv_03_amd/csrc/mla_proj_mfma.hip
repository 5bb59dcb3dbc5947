// bf16 MFMA kernels for the two per-query projections of the decode step:
// query absorption through W_UK (a1) and value up-projection through W_UV
// (a6) ("The Architecture of Memory", "The Weight Absorption Trick";
// "Beyond the Attention Bottleneck", "Down-Projection and Up-Projection
// Mechanics"). Both are small GEMMs per head (tokens x d_n x d_c and
// tokens x d_c x d_v) that stream the weights once; the point of these
// kernels is to spread that stream over hundreds of waves.
#include <hip/hip_runtime.h>
#include <math.h>

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
// grid (H, d_c / 256, ceil(N / 16)); 4 waves, wave w owns 64 output columns.
// v_mfma_f32_16x16x16_bf16 with M = 16 tokens, K = 16 rows of W_UK, N = 16
// columns. W_UK is row-major [d_n][d_c], so a lane loads 8 contiguous bytes
// (4 columns) from each of 4 rows and transposes the 4x4 block in registers
// into 4 B operands; MFMA m then covers columns c0 + 4*(lane%16) + m.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void absorb_q_mfma_kernel(
    int n_tok, int H, int dn, int dc, int dr, double log2_base, const bf16_t* __restrict__ q_nope,
    const bf16_t* __restrict__ q_rope, const int32_t* __restrict__ pos,
    const bf16_t* __restrict__ w_uk, bf16_t* __restrict__ q_full) {
  const int h = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nn = lane & 15, g = lane >> 4;
  const int c0 = blockIdx.y * 256 + wave * 64;
  const int n0 = blockIdx.z * 16;
  const int D = dc + dr;
  const int tok = n0 + nn;  // A-operand row of this lane
  const bool tok_ok = tok < n_tok;
  const bf16_t* qrow = q_nope + ((size_t)(tok_ok ? tok : 0) * H + h) * dn;
  const bf16_t* W = w_uk + (size_t)h * dn * dc + c0 + 4 * nn;
  f32x4_t acc[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) acc[m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  for (int i0 = 0; i0 < dn; i0 += 16) {
    u32x2_t qa = *reinterpret_cast<const u32x2_t*>(qrow + i0 + 4 * g);
    if (!tok_ok) qa = u32x2_t{0u, 0u};
    u32x2_t x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[j] = *reinterpret_cast<const u32x2_t*>(W + (size_t)(i0 + 4 * g + j) * dc);
    const s16x4_t a = __builtin_bit_cast(s16x4_t, qa);
    const s16x4_t b0 = as_s16x4(pack_lo(x[0].x, x[1].x), pack_lo(x[2].x, x[3].x));
    const s16x4_t b1 = as_s16x4(pack_hi(x[0].x, x[1].x), pack_hi(x[2].x, x[3].x));
    const s16x4_t b2 = as_s16x4(pack_lo(x[0].y, x[1].y), pack_lo(x[2].y, x[3].y));
    const s16x4_t b3 = as_s16x4(pack_hi(x[0].y, x[1].y), pack_hi(x[2].y, x[3].y));
    acc[0] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b0, acc[0], 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b1, acc[1], 0, 0, 0);
    acc[2] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b2, acc[2], 0, 0, 0);
    acc[3] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b3, acc[3], 0, 0, 0);
  }
  // lane holds tokens n0 + 4g + r, columns c0 + 4*nn + m (m = 0..3)
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = n0 + 4 * g + r;
    if (t < n_tok) {
      u32x2_t v = {pack_bf16x2(acc[0][r], acc[1][r]), pack_bf16x2(acc[2][r], acc[3][r])};
      *reinterpret_cast<u32x2_t*>(q_full + ((size_t)t * H + h) * D + c0 + 4 * nn) = v;
    }
  }
  if (blockIdx.y == 0) {
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
  }
}

bool absorb_mfma_ok(const Shape& s) { return s.dtype == 1 && s.dn % 16 == 0 && s.dc % 256 == 0; }

int launch_absorb_q_mfma(const Shape& s, int n_tok, const void* q_nope, const void* q_rope,
                         const int32_t* pos, const void* w_uk, void* q_full, void* stream) {
  dim3 grid(s.H, s.dc / 256, (n_tok + 15) / 16);
  hipLaunchKernelGGL(absorb_q_mfma_kernel, grid, dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), n_tok, s.H, s.dn, s.dc, s.dr,
                     s.log2_base, (const bf16_t*)q_nope, (const bf16_t*)q_rope, pos,
                     (const bf16_t*)w_uk, (bf16_t*)q_full);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// a6: out[n][h][v] = sum_c W_UV[h][v][c] o_lat[n][h][c].
// grid (H, d_v / 16, ceil(N / 16)); 4 waves split the d_c contraction (wave
// w takes 32-wide k-steps w, w+4, ...), then sum through LDS.
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
  for (int k = wave * 32; k < dc; k += 128) {
    u32x4_t av = *reinterpret_cast<const u32x4_t*>(arow + k);
    if (!tok_ok) av = u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(brow + k);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                  __builtin_bit_cast(bf16x8_t, bv), acc, 0, 0, 0);
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

bool up_v_mfma_ok(const Shape& s) { return s.dtype == 1 && s.dc % 32 == 0 && s.dv % 16 == 0; }

int launch_up_project_v_mfma(const Shape& s, int n_tok, const void* o_lat, const void* w_uv,
                             void* out, void* stream) {
  dim3 grid(s.H, s.dv / 16, (n_tok + 15) / 16);
  hipLaunchKernelGGL(up_v_mfma_kernel, grid, dim3(256), 0, reinterpret_cast<hipStream_t>(stream),
                     n_tok, s.H, s.dc, s.dv, (const bf16_t*)o_lat, (const bf16_t*)w_uv,
                     (bf16_t*)out);
  return (int)hipGetLastError();
}

}  // namespace mla
