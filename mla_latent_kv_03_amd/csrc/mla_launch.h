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
  int split_fixed = 0;                 // decode partitions of this many tokens (0: per sequence)
  int D() const { return dc + dr; }
};

// Whether the append may copy the latent part in 16-byte vectors: every
// source and destination row 16-byte aligned.
inline int append_vectorizable(const Shape& s, const void* c_kv, const void* cache) {
  const size_t es = s.dtype == 0 ? 4 : 2;
  return ((uintptr_t)c_kv % 16 == 0) && ((uintptr_t)cache % 16 == 0) && (s.dc * es) % 16 == 0 &&
         ((size_t)s.D() * es) % 16 == 0;
}

// Each returns 0 on success or the hipError_t of the failed launch.

// Raise a kernel's dynamic LDS limit to `bytes` once per kernel and device
// (the first launch on each device sets it; thread-safe). 0 or a hipError_t.
int set_max_lds(const void* kernel, int bytes);

// Drafted-token positions of one verify step: for row n = b * q_len + i,
// seq_idx[n] = b, slot[n] = L_b - q_len + i and pos[n] = L_b - q_len +
// depth_b(i) (the slot for a chain, tree_parent NULL); -1 for both when L_b
// is outside [q_len, max_seq_len] or b's tree breaks parent[i] in [-1, i).
int launch_draft_positions(int batch, int q_len, int max_seq_len, const int32_t* seq_lens,
                           const int32_t* tree_parent, int32_t* seq_idx, int32_t* slot,
                           int32_t* pos, void* stream);

// A plain streaming read of `bytes` (a multiple of 16) with 16-byte
// non-temporal loads, one checksum word per block into sink[0 .. blocks):
// the achievable HBM read rate, for context beside the decode kernels.
int launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream);
int launch_absorb_q(const Shape& s, int n_tok, const void* q_nope, const void* q_rope,
                    const int32_t* pos, const void* w_uk, void* q_full, void* stream);

// rope_pos may be NULL (rotate by pos)
int launch_cache_append(const Shape& s, int n_tok, const void* c_kv, const void* k_rope,
                        const int32_t* seq_idx, const int32_t* pos, const int32_t* rope_pos,
                        const int32_t* page_table, int batch, int max_pages, void* cache,
                        int64_t num_pages, int rotate, void* stream);

// a1 and a2 of one decode step in one launch when the absorption takes the
// bf16 MFMA kernel, else the two launches in order; results identical to
// launch_absorb_q followed by launch_cache_append. With dI > 0 the rows'
// indexer keys k_idx [n_app][dI] go to icache in the same launch (else a
// third launch, launch_index_append).
int launch_absorb_append(const Shape& s, int n_tok, const void* q_nope, const void* q_rope,
                         const int32_t* pos_q, const void* w_uk, void* q_full, int n_app,
                         const void* c_kv, const void* k_rope, const int32_t* seq_idx,
                         const int32_t* pos, const int32_t* rope_pos, const int32_t* page_table,
                         int batch, int max_pages, void* cache, int64_t num_pages, int rotate,
                         void* stream, int dI = 0, const void* k_idx = nullptr,
                         void* icache = nullptr);

// a1 and the 8-bit (bits = 8) or 4-bit (bits = 4) append in one launch when
// the absorption takes the bf16 MFMA kernel, else the two launches in order;
// results identical to launch_absorb_q followed by launch_cache_append_q8/q4.
int launch_absorb_append_coded(int bits, const Shape& s, int n_tok, const void* q_nope,
                               const void* q_rope, const int32_t* pos_q, const void* w_uk,
                               void* q_full, int n_app, const void* c_kv, const void* k_rope,
                               const int32_t* seq_idx, const int32_t* pos,
                               const int32_t* rope_pos, const int32_t* page_table, int batch,
                               int max_pages, void* cache, int64_t num_pages, int rotate,
                               void* stream);

// tree_parent: [batch][q_len] drafted-token tree (q_len <= 64), or NULL for
// the chain of drafted tokens
int launch_decode(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                  const void* q_full, const void* cache, int64_t num_pages,
                  const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                  const int32_t* tree_parent, float* o_part, float* lse_part, void* stream);

int launch_combine(const Shape& s, int rows, int num_splits, const float* o_part,
                   const float* lse_part, void* o_lat, float* lse, void* stream);

int launch_up_project_v(const Shape& s, int n_tok, const void* o_lat, const void* w_uv,
                        void* out, void* stream);

// a5 and a6 in one launch for the bf16 d_c = 512, d_v = 128 shape when the
// row count and split count are small, else the two launches in order;
// results identical to launch_combine followed by launch_up_project_v.
int launch_combine_up_project(const Shape& s, int n_tok, int num_splits, const float* o_part,
                              const float* lse_part, void* o_lat, float* lse, const void* w_uv,
                              void* out, void* stream);

// 8-bit latent cache: rows of d_c + d_r codes plus 16 bytes of (min, step)
// pairs. The decode needs the DeepSeek row (bf16, 512 + 64), page % 64 == 0
// and q_len * H % 16 == 0 (decode_q8_ok).
int launch_cache_append_q8(const Shape& s, int n_tok, const void* c_kv, const void* k_rope,
                           const int32_t* seq_idx, const int32_t* pos, const int32_t* rope_pos,
                           const int32_t* page_table, int batch, int max_pages, void* cache,
                           int64_t num_pages, int rotate, void* stream);
bool decode_q8_ok(const Shape& s, int q_len);
int launch_decode_q8(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                     const void* q_full, const void* cache, int64_t num_pages,
                     const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                     const int32_t* tree_parent, float* o_part, float* lse_part, void* stream);
// 4-bit latent cache: the same rows with two codes per byte (column 2i in the
// low nibble of byte i), (d_c + d_r) / 2 + 16 bytes; the decode has the
// 8-bit decode's limits (decode_q8_ok).
int launch_cache_append_q4(const Shape& s, int n_tok, const void* c_kv, const void* k_rope,
                           const int32_t* seq_idx, const int32_t* pos, const int32_t* rope_pos,
                           const int32_t* page_table, int batch, int max_pages, void* cache,
                           int64_t num_pages, int rotate, void* stream);
int launch_decode_q4(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                     const void* q_full, const void* cache, int64_t num_pages,
                     const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                     const int32_t* tree_parent, float* o_part, float* lse_part, void* stream);

// Chunked prefill in the unabsorbed form: one sequence, q_len query tokens
// at positions seq_len - q_len + i (their rows already in the cache), bf16
// with d_c = 512, d_r = 64, d_n = d_v = 128 (prefill_unabsorbed_ok). The
// workspace holds the expanded keys and values, the RoPE keys and the
// rotated queries (prefill_workspace_bytes).
bool prefill_unabsorbed_ok(const Shape& s);
size_t prefill_workspace_bytes(const Shape& s, int seq_len, int q_len);
int launch_prefill_unabsorbed(const Shape& s, int q_len, int seq_len, const void* q_nope,
                              const void* q_rope, const void* w_uk, const void* w_uv,
                              const void* cache, int64_t num_pages, const int32_t* page_row,
                              int max_pages, void* workspace, void* out, float* lse,
                              void* stream);

// Which decode kernel a shape takes (for tests and tools): 0 = generic VALU
// kernel, 1 = bf16 MFMA kernel with 16 query rows per block, 2 = bf16 MFMA
// kernel with 64 query rows per block.
int decode_kernel_kind(const Shape& s, int q_len);

// Sparse read. Indexer keys: rows of dI elements of type T through the same
// page table; scores: [batch][q_len][ld] f32; selection: indices
// [batch][q_len][topk] int32 and counts [batch][q_len] int32 (-1: invalid).
int launch_index_append(const Shape& s, int dI, int n_tok, const void* k_new,
                        const int32_t* seq_idx, const int32_t* pos, const int32_t* page_table,
                        int batch, int max_pages, void* icache, int64_t num_pages, void* stream);
bool index_scores_mfma_ok(const Shape& s, int Hi, int dI);
size_t index_scores_generic_lds(int Hi, int dI);
int launch_index_scores(const Shape& s, int Hi, int dI, int batch, int q_len, int max_seq_len,
                        const void* q_idx, const float* w_idx, const void* icache,
                        int64_t num_pages, const int32_t* page_table, int max_pages,
                        const int32_t* seq_lens, float* scores, int ld, void* stream);
// workspace: topk_workspace_bytes, all zero on entry and left all zero
size_t topk_workspace_bytes(int batch, int q_len);
int launch_topk(int batch, int q_len, int max_seq_len, int topk, const float* scores, int ld,
                const int32_t* seq_lens, void* workspace, int32_t* indices, int32_t* counts,
                void* stream);
int launch_index_scores_topk(const Shape& s, int Hi, int dI, int batch, int q_len,
                             int max_seq_len, const void* q_idx, const float* w_idx,
                             const void* icache, int64_t num_pages, const int32_t* page_table,
                             int max_pages, const int32_t* seq_lens, float* scores, int ld,
                             int topk, void* workspace, int32_t* indices, int32_t* counts,
                             void* stream);
// launch_index_scores_topk with the workspace in the library's own device
// array (queries batch * q_len <= kTopkNoallocMaxQueries; checked by the
// caller): allocates nothing. The array is cleared by a fill kernel on the
// first call on each device (and after a failed launch); every selection
// leaves the rows it used zero again.
constexpr int kTopkNoallocMaxQueries = 256;
int launch_index_scores_topk_noalloc(const Shape& s, int Hi, int dI, int batch, int q_len,
                                     int max_seq_len, const void* q_idx, const float* w_idx,
                                     const void* icache, int64_t num_pages,
                                     const int32_t* page_table, int max_pages,
                                     const int32_t* seq_lens, float* scores, int ld, int topk,
                                     int32_t* indices, int32_t* counts, void* stream);
// decode over the selected tokens: partition s of query (b, j) covers list
// entries [s * chunk, min(count, (s + 1) * chunk)); kind 1 = the bf16 MFMA
// kernel (16 rows per block, H % 16 == 0, chunk a multiple of 32 up to
// 1,984), 0 = generic
int decode_sparse_kind(const Shape& s, int chunk);
int launch_decode_sparse(const Shape& s, int batch, int q_len, int topk, int chunk, int num_splits,
                         int max_seq_len, const void* q_full, const void* cache, int64_t num_pages,
                         const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                         const int32_t* sel_idx, const int32_t* sel_cnt, float* o_part,
                         float* lse_part, void* stream);

}  // namespace mla
