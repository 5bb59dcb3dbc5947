// Internal interface between the host entry points (mla_api.cpp, plain C++)
// and the HIP launchers (*.hip). Everything here is already validated: the
// launchers trust their arguments and only map HIP errors to a return code.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mla {

struct Shape {
  int H, dc, dr, dn, dv, page, dtype;  // dtype: 0 = fp32, 1 = bf16
  float scale;
  double log2_base;                    // log2(rope_base), for fp64 RoPE angles
  int D() const { return dc + dr; }
};

// Each returns 0 on success or the hipError_t of the failed launch.
int launch_absorb_q(const Shape& s, int n_tok, const void* q_nope, const void* q_rope,
                    const int32_t* pos, const void* w_uk, void* q_full, void* stream);

int launch_cache_append(const Shape& s, int n_tok, const void* c_kv, const void* k_rope,
                        const int32_t* seq_idx, const int32_t* pos, const int32_t* page_table,
                        int batch, int max_pages, void* cache, int64_t num_pages, int rotate,
                        void* stream);

int launch_decode(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                  const void* q_full, const void* cache, int64_t num_pages,
                  const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                  float* o_part, float* lse_part, void* stream);

int launch_combine(const Shape& s, int rows, int num_splits, const float* o_part,
                   const float* lse_part, void* o_lat, float* lse, void* stream);

int launch_up_project_v(const Shape& s, int n_tok, const void* o_lat, const void* w_uv,
                        void* out, void* stream);

// Which decode kernel a shape takes (for tests and tools): 0 = generic VALU
// kernel, 1 = bf16 MFMA kernel.
int decode_kernel_kind(const Shape& s, int q_len);

}  // namespace mla
