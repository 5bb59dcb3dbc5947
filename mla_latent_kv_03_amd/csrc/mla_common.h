// Device helpers shared by the HIP kernels of libmla (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef uint16_t bf16_t;  // raw bf16 bits

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T>
struct Elt;

template <>
struct Elt<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};

template <>
struct Elt<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
};

// Rotate the pair (x0, x1) of a d_r-wide RoPE vector, pair index i, by
// pos * base^(-2i/d_r). Angle and rotation in fp64: at positions near 2^20
// an fp32 angle would be off by up to 0.06 rad.
__device__ __forceinline__ void rope_pair(double x0, double x1, int64_t pos, int i, int dr,
                                          double log2_base, double* y0, double* y1) {
  const double theta = exp2(-(2.0 * (double)i / (double)dr) * log2_base);
  const double ang = (double)pos * theta;
  double sn, cs;
  sincos(ang, &sn, &cs);
  *y0 = x0 * cs - x1 * sn;
  *y1 = x0 * sn + x1 * cs;
}

// Split plan: tokens of partition s of a length-L sequence. fixed > 0: every
// partition holds `fixed` tokens (a multiple of the page), so a long sequence
// has more non-empty partitions than a short one; fixed == 0: the S
// partitions of each sequence share it evenly, page-aligned.
__device__ __forceinline__ void split_range(int L, int S, int page, int fixed, int s, int* t0,
                                            int* t1) {
  const int64_t per = ((int64_t)L + S - 1) / S;
  const int64_t chunk = fixed > 0 ? (int64_t)fixed : (int64_t)page * ((per + page - 1) / page);
  int64_t a = (int64_t)s * chunk, e = a + chunk;
  if (a > L) a = L;
  if (e > L) e = L;
  *t0 = (int)a;
  *t1 = (int)e;
}

// Tree verification ("The Architecture of Memory", "Tree Attention
// Verification"): the last Q cached tokens of a sequence are drafted tokens
// forming a tree, parent[i] in [-1, i) being the drafted token that token i
// continues (-1: the prefix). Query j sees every prefix token and the drafted
// tokens on its own branch: bit i of its branch mask is set when i is j or an
// ancestor of j. The walk stops after Q steps (Q <= 64) whatever the entries
// hold; tree_entry_ok is the validity the kernels check first.
__host__ __device__ __forceinline__ bool tree_entry_ok(const int32_t* __restrict__ parent, int i) {
  const int p = parent[i];
  return p >= -1 && p < i;
}
__host__ __device__ __forceinline__ uint64_t tree_branch_mask(const int32_t* __restrict__ parent, int Q,
                                                              int j) {
  uint64_t m = 0;
  int i = j;
  for (int step = 0; step < Q && i >= 0 && i < Q; ++step) {
    m |= 1ull << i;
    i = parent[i];
  }
  return m;
}

// Tiles of `tile` tokens a block streams from its partition [t0, t1): up to
// the last token any of its rows sees. With a chain of drafted tokens (or a
// chunk of prefill queries) query j sees up to t_draft + j, so a block whose
// last query is jmax stops there; a tree's rows may see any drafted token.
__host__ __device__ __forceinline__ int tiles_needed(int t0, int t1, int tile, bool tree,
                                                     int t_draft, int jmax) {
  const int end = tree ? t1 : min(t1, t_draft + jmax + 1);
  return end > t0 ? (end - t0 + tile - 1) / tile : 0;
}

// Tokens ts .. ts + 63 that one query row sees, as bits (bit o = token ts + o):
// every token up to lim, and with a drafted tree the drafts on the row's branch
// (bit i of `branch` = token t_draft + i) that lie below t1. Shifts and selects
// only: a per-token short-circuit form of this test lost one of its masked
// stores in gfx950 code generation.
__host__ __device__ __forceinline__ uint64_t tile_visible(int ts, int lim, int t_draft, int t1,
                                                          uint64_t branch) {
  const int npre = lim - ts + 1;  // prefix tokens from ts on
  const uint64_t pre = npre >= 64 ? ~0ull : (npre <= 0 ? 0ull : (1ull << npre) - 1ull);
  const int rel = ts - t_draft;   // offset o holds draft o + rel
  uint64_t drafts = rel >= 0 ? (rel < 64 ? branch >> rel : 0ull)
                             : (-rel < 64 ? branch << -rel : 0ull);
  const int nin = t1 - ts;        // offsets below t1
  if (nin < 64) drafts &= nin <= 0 ? 0ull : (1ull << nin) - 1ull;
  return pre | drafts;
}

}  // namespace mla
