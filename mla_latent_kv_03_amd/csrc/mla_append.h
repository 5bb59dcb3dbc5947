// Paged cache append of one row (a2; "The Architecture of Memory",
// "PagedAttention: Virtual Memory for LLMs"): row n of c_kv / k_rope goes to
// physical row page_table[seq_idx[n]][pos[n] / page] * page + pos[n] % page,
// its RoPE part rotated by rope_pos[n] when `rotate` is set (by pos[n] when
// rope_pos is NULL; a drafted tree's token sits at a slot that need not be
// its position, "The Architecture of Memory", "Tree Attention Verification"). Rows whose sequence,
// position or page entry is out of range are skipped. The row's values do not
// depend on where it goes, so they are loaded (16 bytes per lane when `vec`:
// every source and destination row 16-byte aligned) before the page-table
// lookup resolves the destination. Executed by one whole block (any size).
#pragma once

#include "mla_common.h"

namespace mla {

template <typename T>
__device__ __forceinline__ void append_row(int n, int dc, int dr, int page, const T* __restrict__ c_kv,
                                           const T* __restrict__ k_rope,
                                           const int32_t* __restrict__ seq_idx,
                                           const int32_t* __restrict__ pos,
                                           const int32_t* __restrict__ rope_pos,
                                           const int32_t* __restrict__ page_table, int batch,
                                           int max_pages, T* __restrict__ cache, int64_t num_pages,
                                           int rotate, double log2_base, int vec) {
  constexpr int kV = 16 / sizeof(T);  // elements per 16-byte vector
  const int tid = threadIdx.x;
  const int D = dc + dr;
  const int nvec = vec ? dc / kV : 0;
  const T* src = c_kv + (size_t)n * dc;
  uint4 v0 = make_uint4(0u, 0u, 0u, 0u);
  if (tid < nvec) v0 = reinterpret_cast<const uint4*>(src)[tid];
  const T* kr = k_rope + (size_t)n * dr;
  float x0 = 0.0f, x1 = 0.0f;
  if (tid < dr / 2) {
    x0 = Elt<T>::ld(kr + 2 * tid);
    x1 = Elt<T>::ld(kr + 2 * tid + 1);
  }
  const int b = seq_idx[n];
  const int p = pos[n];
  if (b < 0 || b >= batch || p < 0 || p >= max_pages * page) return;
  const int pg = page_table[(size_t)b * max_pages + p / page];
  if (pg < 0 || (int64_t)pg >= num_pages) return;
  T* row = cache + ((size_t)pg * page + p % page) * D;
  const int rp = rope_pos ? rope_pos[n] : p;
  if (tid < nvec) reinterpret_cast<uint4*>(row)[tid] = v0;
  for (int i = tid + blockDim.x; i < nvec; i += blockDim.x)
    reinterpret_cast<uint4*>(row)[i] = reinterpret_cast<const uint4*>(src)[i];
  for (int i = nvec * kV + tid; i < dc; i += blockDim.x) row[i] = src[i];
  if (tid < dr / 2) {
    if (rotate) {
      double y0, y1;
      rope_pair(x0, x1, rp, tid, dr, log2_base, &y0, &y1);
      Elt<T>::st(row + dc + 2 * tid, (float)y0);
      Elt<T>::st(row + dc + 2 * tid + 1, (float)y1);
    } else {
      row[dc + 2 * tid] = kr[2 * tid];
      row[dc + 2 * tid + 1] = kr[2 * tid + 1];
    }
  }
  for (int i = tid + blockDim.x; i < dr / 2; i += blockDim.x) {
    if (rotate) {
      double y0, y1;
      rope_pair(Elt<T>::ld(kr + 2 * i), Elt<T>::ld(kr + 2 * i + 1), rp, i, dr, log2_base, &y0,
                &y1);
      Elt<T>::st(row + dc + 2 * i, (float)y0);
      Elt<T>::st(row + dc + 2 * i + 1, (float)y1);
    } else {
      row[dc + 2 * i] = kr[2 * i];
      row[dc + 2 * i + 1] = kr[2 * i + 1];
    }
  }
}

// Indexer key append (the sparse read's key cache, "DeepSeek's Config Says
// 16 KV Heads", section 6): row n of k_new (dI elements) to slot pos[n] of
// sequence seq_idx[n] through the latent cache's page table, copied as is;
// invalid rows are skipped. Executed by one whole block (any size).
template <typename T>
__device__ __forceinline__ void index_append_row(int n, int dI, int page,
                                                 const T* __restrict__ k_new,
                                                 const int32_t* __restrict__ seq_idx,
                                                 const int32_t* __restrict__ pos,
                                                 const int32_t* __restrict__ page_table, int batch,
                                                 int max_pages, T* __restrict__ icache,
                                                 int64_t num_pages) {
  const int b = seq_idx[n], p = pos[n];
  if (b < 0 || b >= batch || p < 0 || (int64_t)p >= (int64_t)max_pages * page) return;
  const int pg = page_table[(size_t)b * max_pages + p / page];
  if (pg < 0 || (int64_t)pg >= num_pages) return;
  T* dst = icache + ((size_t)pg * page + p % page) * dI;
  const T* src = k_new + (size_t)n * dI;
  for (int i = threadIdx.x; i < dI; i += blockDim.x) dst[i] = src[i];
}

}  // namespace mla
