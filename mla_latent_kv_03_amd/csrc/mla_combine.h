// Log-sum-exp merge of split-KV partials (a5; "The Architecture of Memory",
// "Flash-Decoding and FlashInfer"): for output row r with partitions
// s = 0..S-1,
//   o_lat[r] = sum_s e^(lse_s - max) o_part[r][s] / sum_s e^(lse_s - max),
//   lse[r]   = max + ln sum_s e^(lse_s - max);
// partitions of weight 0 (lse = -inf: empty or fully masked) are left out, so
// their o_part rows are never used (the decode leaves empty ones unwritten),
// and a NaN partition LSE (an invalid sequence) makes the whole row NaN. The pieces here are executed by one wave
// for 256 columns (lane l: columns 4l .. 4l+3) and shared by the combine
// kernel and the fused merge + up-projection kernel, so both produce the
// same bits.
#pragma once

#include "mla_common.h"

namespace mla {

constexpr int kMaxSplits = 4096;
constexpr int kCombCols = 256;  // latent columns per wave: 64 lanes x 4
constexpr int kCombChunk = 16;  // partitions in flight per lane

template <typename T>
__device__ __forceinline__ void store4(T* p, float4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, float4 v) {
  *reinterpret_cast<float4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float4 v) {
  uint2 u;
  u.x = (uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16);
  u.y = (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

struct CombineWeights {
  float mx, sum;
  bool bad;
  __device__ __forceinline__ float lse() const {
    return bad ? __int_as_float(0x7fc00000) : mx + logf(sum);
  }
};

// One wave: turn the S partition LSEs of a row into weights e^(lse_s - max)
// in w[0..S) (LDS). The caller makes w visible to the readers (barrier).
__device__ __forceinline__ CombineWeights combine_weights(const float* __restrict__ lp, int S,
                                                          float* w, int lane) {
  float mx = -INFINITY;
  bool nan_seen = false;
  for (int s = lane; s < S; s += 64) {
    const float v = lp[s];
    w[s] = v;
    nan_seen |= (v != v);
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  const bool bad = __any(nan_seen);
  float sum = 0.0f;
  for (int s = lane; s < S; s += 64) {
    const float e = (w[s] == -INFINITY) ? 0.0f : expf(w[s] - mx);
    w[s] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  return CombineWeights{mx, sum, bad};
}

// The same weights for S <= 64 from v = lse_part[row][lane] (any value for
// lane >= S) loaded by the caller, so that the load can be issued ahead of
// others: the operations are those of combine_weights' single iteration.
__device__ __forceinline__ CombineWeights combine_weights_one(float v, int S, float* w, int lane) {
  float mx = -INFINITY;
  bool nan_seen = false;
  if (lane < S) {
    w[lane] = v;
    nan_seen |= (v != v);
    mx = fmaxf(mx, v);
  }
  mx = wave_max(mx);
  const bool bad = __any(nan_seen);
  float sum = 0.0f;
  if (lane < S) {
    const float e = (w[lane] == -INFINITY) ? 0.0f : expf(w[lane] - mx);
    w[lane] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  return CombineWeights{mx, sum, bad};
}

// One lane's 4 columns of a row, summed over the partitions in order. The
// partials do not depend on the weights, so start() issues the first
// kCombChunk partition loads before the weights exist; finish() then adds the
// partitions, loading the next kCombChunk while it adds the current ones.
// Every load is an unconditional 16-byte load of a valid address (partition
// index clamped to S - 1, the column of an idle lane to 0); the clamped
// copies are dropped by a select, not a branch.
//
// CH partitions are in flight per lane. With kOne set the caller guarantees
// S <= CH: everything is loaded by start() and finish() issues no loads.
template <int CH = kCombChunk, bool kOne = false>
struct CombineCols {
  const float4* op;
  size_t st;
  int S;
  float4 x[CH];
  __device__ __forceinline__ void start(const float* __restrict__ o_row, int S_, int dc, int col) {
    S = S_;
    op = reinterpret_cast<const float4*>(o_row + (col < dc ? col : 0));
    st = dc / 4;  // float4 stride between partitions
#pragma unroll
    for (int u = 0; u < CH; ++u) x[u] = op[(size_t)min(u, S - 1) * st];
  }
  // Adds partitions s0 .. s0+CH-1. Whether a partition counts (inside S,
  // weight not 0) is the same for every lane of the row, so it is taken from
  // one ballot and tested as a scalar; a partition of weight 0 may be
  // unwritten and never reaches the sum.
  __device__ __forceinline__ void add(const float* w, int s0, float4& a, int lane) const {
    static_assert(CH <= 64, "one ballot per group");
    const int sl = s0 + lane % CH;
    const uint64_t use = __ballot(lane < CH && sl < S && w[min(sl, S - 1)] != 0.0f);
    float wv[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) wv[u] = w[min(s0 + u, S - 1)];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      if ((use >> u) & 1) {
        const float ws = wv[u];
        a.x = fmaf(ws, x[u].x, a.x);
        a.y = fmaf(ws, x[u].y, a.y);
        a.z = fmaf(ws, x[u].z, a.z);
        a.w = fmaf(ws, x[u].w, a.w);
      }
    }
  }
  // normalized columns (NaN for a bad row). A later group of CH partitions
  // whose weights are all 0 is neither loaded nor added.
  __device__ __forceinline__ float4 finish(const float* w, const CombineWeights& cw, int lane) {
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (kOne) {
      add(w, 0, a, lane);
    } else {
      bool use = true;  // the first group was loaded speculatively in start()
      for (int s0 = 0; s0 < S; s0 += CH) {
        const int s1 = s0 + CH;
        float4 y[CH];
        bool next = false;
        if (s1 < S) {  // wave-uniform
          const int sl = s1 + lane % CH;
          next = __any(sl < S && w[min(sl, S - 1)] != 0.0f);
          if (next) {
#pragma unroll
            for (int u = 0; u < CH; ++u) y[u] = op[(size_t)min(s1 + u, S - 1) * st];
          }
        }
        if (use) add(w, s0, a, lane);
        if (next) {
#pragma unroll
          for (int u = 0; u < CH; ++u) x[u] = y[u];
        }
        use = next;
      }
    }
    const float nanv = __int_as_float(0x7fc00000);
    const float inv = 1.0f / cw.sum;
    return cw.bad ? make_float4(nanv, nanv, nanv, nanv)
                  : make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
  }
};

}  // namespace mla
