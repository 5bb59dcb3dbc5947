// Quantizing append of one cached row to an 8-bit or 4-bit latent cache
// ("KV Cache Optimization: Scaling to Million-Token Contexts", technique 3
// "KV Cache Quantization"), the body shared by the append kernel and the
// launch that runs the query absorption beside it. Coding per token and
// part (latent d_c, rotated RoPE d_r): step = (max - min) / (2^bits - 1),
// code = rint((x - min) / step) in float32, 0 for a constant part; row =
// [codes][lat_min, lat_step, rope_min, rope_step f32]. The min and max are
// exact whatever the reduction order, so the bits do not depend on the
// block size (64 to 256 threads).
#pragma once

#include "mla_append.h"
#include "mla_common.h"

namespace mla {

constexpr int kQ8Meta = 16;  // bytes of per-row metadata (4 fp32)

namespace coded {

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_reduce_min(float v, float* red) {
  return -block_reduce_max(-v, red);
}

// code of x on [mn, mn + levels * step]: rint((x - mn) / step) in float32
__device__ __forceinline__ uint32_t q_code(float x, float mn, float step, float levels) {
  if (step == 0.0f) return 0u;
  const float c = rintf((x - mn) / step);
  return (uint32_t)fminf(fmaxf(c, 0.0f), levels);
}

}  // namespace coded

// Row n of the batch -> slot pos[n] of sequence seq_idx[n]; a row whose
// sequence, slot or page is invalid is dropped. The RoPE part is rotated by
// rope_pos[n] (rope_pos NULL: pos[n]) in fp64 when `rotate`. Every thread of
// the block calls this (block-uniform control flow; at most 4 waves).
template <typename T, int kBits>
__device__ __forceinline__ void append_coded_row(
    int n, int dc, int dr, int page, const T* __restrict__ c_kv, const T* __restrict__ k_rope,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ rope_pos, const int32_t* __restrict__ page_table, int batch,
    int max_pages, uint8_t* __restrict__ cache, int64_t num_pages, int rotate, double log2_base) {
  using namespace coded;
  __shared__ float red[4];
  __shared__ float kr[256];  // the (rotated) RoPE part in float32, d_r <= 256
  const int tid = threadIdx.x;
  const int b = seq_idx[n];
  const int p = pos[n];
  if (b < 0 || b >= batch || p < 0 || p >= max_pages * page) return;  // block-uniform
  const int pg = page_table[(size_t)b * max_pages + p / page];
  if (pg < 0 || (int64_t)pg >= num_pages) return;
  const int D = dc + dr;
  constexpr float kLevels = (float)((1 << kBits) - 1);  // 255 or 15
  constexpr int kPer = 32 / kBits;                       // codes per 32-bit word: 4 or 8
  uint8_t* row = cache + ((size_t)pg * page + p % page) * (size_t)(D * kBits / 8 + kQ8Meta);
  const T* src = c_kv + (size_t)n * dc;
  const T* ks = k_rope + (size_t)n * dr;
  const int rp = rope_pos ? rope_pos[n] : p;
  // RoPE part, rotated in fp64 (as the bf16 cache does) and rounded to fp32
  for (int i = tid; i < dr / 2; i += blockDim.x) {
    const float x0 = Elt<T>::ld(ks + 2 * i), x1 = Elt<T>::ld(ks + 2 * i + 1);
    if (rotate) {
      double y0, y1;
      rope_pair(x0, x1, rp, i, dr, log2_base, &y0, &y1);
      kr[2 * i] = (float)y0;
      kr[2 * i + 1] = (float)y1;
    } else {
      kr[2 * i] = x0;
      kr[2 * i + 1] = x1;
    }
  }
  // latent part: range, then codes (4 consecutive values per thread and pass)
  float lo = INFINITY, hi = -INFINITY;
  for (int i = tid; i < dc; i += blockDim.x) {
    const float v = Elt<T>::ld(src + i);
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  const float lmn = block_reduce_min(lo, red);
  const float lmx = block_reduce_max(hi, red);
  const float lstep = (lmx - lmn) / kLevels;
  for (int i = kPer * tid; i < dc; i += kPer * blockDim.x) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      w |= q_code(Elt<T>::ld(src + i + j), lmn, lstep, kLevels) << (kBits * j);
    *reinterpret_cast<uint32_t*>(row + i * kBits / 8) = w;
  }
  // RoPE part (kr is complete: the reductions above passed block barriers)
  lo = INFINITY;
  hi = -INFINITY;
  for (int i = tid; i < dr; i += blockDim.x) {
    lo = fminf(lo, kr[i]);
    hi = fmaxf(hi, kr[i]);
  }
  const float rmn = block_reduce_min(lo, red);
  const float rmx = block_reduce_max(hi, red);
  const float rstep = (rmx - rmn) / kLevels;
  for (int i = kPer * tid; i < dr; i += kPer * blockDim.x) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) w |= q_code(kr[i + j], rmn, rstep, kLevels) << (kBits * j);
    *reinterpret_cast<uint32_t*>(row + (dc + i) * kBits / 8) = w;
  }
  if (tid == 0)
    *reinterpret_cast<float4*>(row + D * kBits / 8) = make_float4(lmn, lstep, rmn, rstep);
}

}  // namespace mla
