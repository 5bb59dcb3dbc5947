// Host entry points of libmla: argument checks, sizing and the split plan.
// Plain C++ (no HIP headers): every check here runs before any launch, so the
// error paths are testable on a machine without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

// the C ABI keeps default visibility; everything else in the library is hidden
#pragma GCC visibility push(default)
#include "../../include/mla.h"
#pragma GCC visibility pop
#include "mla_launch.h"

namespace {

constexpr int kMaxSplits = 4096;
constexpr int kChunksPerCu = 6;
constexpr int kMaxTreeDrafts = 64;  // drafted tokens of a tree (one 64-bit branch mask)

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(const mla_config_t* c) { return c->dtype == MLA_F32 ? 4 : 2; }

mla_status_t check_config(const mla_config_t* c) {
  if (!c) return MLA_ERR_NULL;
  if (c->dtype != MLA_F32 && c->dtype != MLA_BF16) return MLA_ERR_DTYPE;
  const int vec = c->dtype == MLA_F32 ? 4 : 8;  // elements per 16-byte chunk
  if (c->num_heads < 1 || c->num_heads > 1024) return MLA_ERR_SHAPE;
  if (c->kv_rank < 16 || c->kv_rank > 1024 || c->kv_rank % vec) return MLA_ERR_SHAPE;
  if (c->rope_dim < 2 || c->rope_dim > 256 || c->rope_dim % 2) return MLA_ERR_SHAPE;
  if ((c->kv_rank + c->rope_dim) % vec) return MLA_ERR_SHAPE;
  if (c->nope_dim < 1 || c->nope_dim > 256) return MLA_ERR_SHAPE;
  if (c->v_dim < 1 || c->v_dim > 256) return MLA_ERR_SHAPE;
  if (!pow2(c->page_size) || c->page_size < 16 || c->page_size > 256) return MLA_ERR_SHAPE;
  if (!(c->softmax_scale > 0.0f) || !isfinite(c->softmax_scale)) return MLA_ERR_SHAPE;
  if (!(c->rope_base > 1.0f) || !isfinite(c->rope_base)) return MLA_ERR_SHAPE;
  return MLA_OK;
}

mla::Shape shape_of(const mla_config_t* c) {
  mla::Shape s;
  s.H = c->num_heads;
  s.dc = c->kv_rank;
  s.dr = c->rope_dim;
  s.dn = c->nope_dim;
  s.dv = c->v_dim;
  s.page = c->page_size;
  s.dtype = c->dtype;
  s.scale = c->softmax_scale;
  s.log2_base = log2((double)c->rope_base);
  return s;
}

mla_status_t hip_status(int rc) { return rc == 0 ? MLA_OK : MLA_ERR_HIP; }

#define MLA_REQUIRE(cond, code) \
  do {                          \
    if (!(cond)) return (code); \
  } while (0)

#define MLA_CHECK_PTR(p)                  \
  do {                                    \
    if (!(p)) return MLA_ERR_NULL;        \
    if (!aligned16(p)) return MLA_ERR_ALIGN; \
  } while (0)

mla_status_t check_absorb(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                          const void* q_rope, const int32_t* pos, const void* w_uk,
                          const void* q_full) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(n_tok >= 0, MLA_ERR_SHAPE);
  if (n_tok == 0) return MLA_OK;
  MLA_CHECK_PTR(q_nope);
  MLA_CHECK_PTR(q_rope);
  MLA_CHECK_PTR(pos);
  MLA_CHECK_PTR(w_uk);
  MLA_CHECK_PTR(q_full);
  return MLA_OK;
}

mla_status_t check_append(const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                          const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                          const int32_t* page_table, int32_t batch, int32_t max_pages,
                          const void* cache, int64_t num_pages, int32_t flags) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(n_tok >= 0 && batch >= 1 && max_pages >= 1 && num_pages >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE(flags == MLA_APPEND_RAW || flags == MLA_APPEND_ROTATE, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size <= INT32_MAX, MLA_ERR_CAPACITY);
  if (n_tok == 0) return MLA_OK;
  MLA_CHECK_PTR(c_kv);
  MLA_CHECK_PTR(k_rope);
  MLA_CHECK_PTR(seq_idx);
  MLA_CHECK_PTR(pos);
  MLA_CHECK_PTR(page_table);
  MLA_CHECK_PTR(cache);
  return MLA_OK;
}

mla_status_t decode_call(const mla_config_t* cfg, int32_t batch, int32_t q_len, int32_t fixed,
                         int32_t num_splits, int32_t max_seq_len, const void* q_full,
                         const void* cache, int64_t num_pages, const int32_t* page_table,
                         int32_t max_pages, const int32_t* seq_lens, const int32_t* tree_parent,
                         float* o_part, float* lse_part, void* stream) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(batch >= 0 && q_len >= 1 && max_pages >= 1 && num_pages >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE(num_splits >= 1 && num_splits <= kMaxSplits, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)q_len * cfg->num_heads <= 65536, MLA_ERR_SHAPE);
  MLA_REQUIRE(max_seq_len >= q_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size >= (int64_t)max_seq_len, MLA_ERR_CAPACITY);
  if (batch == 0) return MLA_OK;
  MLA_CHECK_PTR(q_full);
  MLA_CHECK_PTR(cache);
  MLA_CHECK_PTR(page_table);
  MLA_CHECK_PTR(seq_lens);
  MLA_CHECK_PTR(o_part);
  MLA_CHECK_PTR(lse_part);
  if (tree_parent) MLA_CHECK_PTR(tree_parent);
  mla::Shape sh = shape_of(cfg);
  sh.split_fixed = fixed;
  return hip_status(mla::launch_decode(sh, batch, q_len, num_splits, max_seq_len, q_full, cache,
                                       num_pages, page_table, max_pages, seq_lens, tree_parent,
                                       o_part, lse_part, stream));
}

mla_status_t check_combine(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                           int32_t num_splits, const float* o_part, const float* lse_part,
                           const void* o_lat, const float* lse) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(batch >= 0 && q_len >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE(num_splits >= 1 && num_splits <= kMaxSplits, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)batch * q_len * cfg->num_heads <= INT32_MAX, MLA_ERR_SHAPE);
  if (batch == 0) return MLA_OK;
  MLA_CHECK_PTR(o_part);
  MLA_CHECK_PTR(lse_part);
  MLA_CHECK_PTR(o_lat);
  if (lse && !aligned16(lse)) return MLA_ERR_ALIGN;
  return MLA_OK;
}

mla_status_t check_up_project(const mla_config_t* cfg, int32_t n_tok, const void* o_lat,
                              const void* w_uv, const void* out) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(n_tok >= 0, MLA_ERR_SHAPE);
  if (n_tok == 0) return MLA_OK;
  MLA_CHECK_PTR(o_lat);
  MLA_CHECK_PTR(w_uv);
  MLA_CHECK_PTR(out);
  return MLA_OK;
}

}  // namespace

extern "C" {

const char* mla_build_info(void) { return "libmla 0.1 gfx950 (HIP, MFMA bf16 decode)"; }

const char* mla_status_str(mla_status_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: size out of range or inconsistent";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: unknown element type";
    case MLA_ERR_ALIGN: return "MLA_ERR_ALIGN: device pointer not 16-byte aligned";
    case MLA_ERR_CAPACITY: return "MLA_ERR_CAPACITY: pages or lengths too small";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED: no kernel for this shape";
    case MLA_ERR_HIP: return "MLA_ERR_HIP: HIP runtime error";
  }
  return "MLA_ERR_?: unknown status";
}

mla_status_t mla_config_validate(const mla_config_t* cfg) { return check_config(cfg); }

size_t mla_cache_bytes_per_token(const mla_config_t* cfg) {
  if (check_config(cfg) != MLA_OK) return 0;
  return (size_t)(cfg->kv_rank + cfg->rope_dim) * (size_t)elem_bytes(cfg);
}

mla_status_t mla_split_chunk(const mla_config_t* cfg, int32_t seq_len, int32_t num_splits,
                             int32_t* chunk_tokens) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(chunk_tokens, MLA_ERR_NULL);
  MLA_REQUIRE(seq_len >= 0 && num_splits >= 1 && num_splits <= kMaxSplits, MLA_ERR_SHAPE);
  const int64_t per = ((int64_t)seq_len + num_splits - 1) / num_splits;
  const int64_t pg = cfg->page_size;
  *chunk_tokens = (int32_t)(pg * ((per + pg - 1) / pg));
  return MLA_OK;
}

int32_t mla_default_num_splits(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                               int32_t max_seq_len, int32_t num_cus) {
  if (check_config(cfg) != MLA_OK || batch < 1 || q_len < 1 || max_seq_len < 1) return 1;
  if (num_cus < 1) num_cus = 256;
  // Work units are (sequence, split, 128-row group); aim for about one unit
  // per compute unit with at least 16 pages (1,024 tokens) in each.
  const int64_t rows = (int64_t)q_len * cfg->num_heads;
  const int64_t groups = (rows + 127) / 128;
  const int64_t pages = ((int64_t)max_seq_len + cfg->page_size - 1) / cfg->page_size;
  int64_t want = ((int64_t)num_cus + batch * groups - 1) / (batch * groups);
  const int64_t cap = pages / 16 > 0 ? pages / 16 : 1;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  if (want > kMaxSplits) want = kMaxSplits;
  return (int32_t)want;
}

const char* mla_decode_kernel_name(const mla_config_t* cfg, int32_t q_len) {
  if (check_config(cfg) != MLA_OK || q_len < 1) return "invalid";
  switch (mla::decode_kernel_kind(shape_of(cfg), q_len)) {
    case 2:
      return "mfma_ws";
    case 1:
      return "mfma_rows16";
    default:
      return "generic";
  }
}

size_t mla_decode_partials_bytes(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                 int32_t num_splits) {
  if (check_config(cfg) != MLA_OK || batch < 0 || q_len < 0 || num_splits < 1 ||
      num_splits > kMaxSplits)
    return 0;
  return (size_t)batch * (size_t)q_len * (size_t)cfg->num_heads * (size_t)num_splits *
         (size_t)(cfg->kv_rank + 1) * sizeof(float);
}

mla_status_t mla_absorb_q(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                          const void* q_rope, const int32_t* pos, const void* w_uk,
                          void* q_full, void* stream) {
  mla_status_t st = check_absorb(cfg, n_tok, q_nope, q_rope, pos, w_uk, q_full);
  if (st != MLA_OK || n_tok == 0) return st;
  return hip_status(
      mla::launch_absorb_q(shape_of(cfg), n_tok, q_nope, q_rope, pos, w_uk, q_full, stream));
}

mla_status_t mla_cache_append(const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                              const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                              const int32_t* page_table, int32_t batch, int32_t max_pages,
                              void* cache, int64_t num_pages, int32_t flags, void* stream) {
  mla_status_t st = check_append(cfg, n_tok, c_kv, k_rope, seq_idx, pos, page_table, batch,
                                 max_pages, cache, num_pages, flags);
  if (st != MLA_OK || n_tok == 0) return st;
  return hip_status(mla::launch_cache_append(shape_of(cfg), n_tok, c_kv, k_rope, seq_idx, pos,
                                             nullptr, page_table, batch, max_pages, cache,
                                             num_pages, flags == MLA_APPEND_ROTATE, stream));
}

mla_status_t mla_cache_append_at(const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                                 const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                 const int32_t* rope_pos, const int32_t* page_table,
                                 int32_t batch, int32_t max_pages, void* cache, int64_t num_pages,
                                 int32_t flags, void* stream) {
  mla_status_t st = check_append(cfg, n_tok, c_kv, k_rope, seq_idx, pos, page_table, batch,
                                 max_pages, cache, num_pages, flags);
  if (st != MLA_OK || n_tok == 0) return st;
  if (rope_pos) MLA_CHECK_PTR(rope_pos);
  return hip_status(mla::launch_cache_append(shape_of(cfg), n_tok, c_kv, k_rope, seq_idx, pos,
                                             rope_pos, page_table, batch, max_pages, cache,
                                             num_pages, flags == MLA_APPEND_ROTATE, stream));
}

mla_status_t mla_draft_positions(int32_t batch, int32_t q_len, int32_t max_seq_len,
                                 const int32_t* seq_lens, const int32_t* tree_parent,
                                 int32_t* seq_idx, int32_t* slot, int32_t* pos, void* stream) {
  MLA_REQUIRE(batch >= 0 && q_len >= 1, MLA_ERR_SHAPE);
  if (tree_parent) MLA_REQUIRE(q_len <= kMaxTreeDrafts, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)batch * q_len <= INT32_MAX, MLA_ERR_SHAPE);
  MLA_REQUIRE(max_seq_len >= q_len, MLA_ERR_CAPACITY);
  if (batch == 0) return MLA_OK;
  MLA_CHECK_PTR(seq_lens);
  if (tree_parent) MLA_CHECK_PTR(tree_parent);
  MLA_CHECK_PTR(seq_idx);
  MLA_CHECK_PTR(slot);
  MLA_CHECK_PTR(pos);
  return hip_status(mla::launch_draft_positions(batch, q_len, max_seq_len, seq_lens, tree_parent,
                                                seq_idx, slot, pos, stream));
}

namespace {
constexpr int kPrefillUnabsorbedMinQ = 1024;  // from measured chunk times of both forms
}  // namespace

size_t mla_prefill_workspace_bytes(const mla_config_t* cfg, int32_t seq_len, int32_t q_len) {
  if (check_config(cfg) != MLA_OK || q_len < 1 || seq_len < q_len) return 0;
  return mla::prefill_workspace_bytes(shape_of(cfg), seq_len, q_len);
}

const char* mla_prefill_form(const mla_config_t* cfg, int32_t q_len, int32_t seq_len) {
  if (check_config(cfg) != MLA_OK || q_len < 1 || seq_len < q_len) return "invalid";
  return mla::prefill_unabsorbed_ok(shape_of(cfg)) && q_len >= kPrefillUnabsorbedMinQ
             ? "unabsorbed"
             : "absorbed";
}

mla_status_t mla_prefill_unabsorbed(const mla_config_t* cfg, int32_t q_len, int32_t seq_len,
                                    const void* q_nope, const void* q_rope, const void* w_uk,
                                    const void* w_uv, const void* cache, int64_t num_pages,
                                    const int32_t* page_row, int32_t max_pages,
                                    void* workspace, void* out, float* lse, void* stream) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(q_len >= 1 && max_pages >= 1 && num_pages >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE(seq_len >= q_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size >= (int64_t)seq_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE((int64_t)seq_len * cfg->num_heads <= INT32_MAX / 2, MLA_ERR_SHAPE);
  const mla::Shape sh = shape_of(cfg);
  MLA_REQUIRE(mla::prefill_unabsorbed_ok(sh), MLA_ERR_UNSUPPORTED);
  MLA_CHECK_PTR(q_nope);
  MLA_CHECK_PTR(q_rope);
  MLA_CHECK_PTR(w_uk);
  MLA_CHECK_PTR(w_uv);
  MLA_CHECK_PTR(cache);
  MLA_REQUIRE(page_row, MLA_ERR_NULL);  // a row of the page table: 4-byte aligned suffices
  MLA_REQUIRE((reinterpret_cast<uintptr_t>(page_row) & 3u) == 0, MLA_ERR_ALIGN);
  MLA_CHECK_PTR(workspace);
  MLA_CHECK_PTR(out);
  MLA_CHECK_PTR(lse);
  return hip_status(mla::launch_prefill_unabsorbed(sh, q_len, seq_len, q_nope, q_rope, w_uk, w_uv,
                                                   cache, num_pages, page_row, max_pages,
                                                   workspace, out, lse, stream));
}

mla_status_t mla_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                             void* stream) {
  MLA_REQUIRE(bytes % 16 == 0 && blocks >= 1 && blocks <= 65536, MLA_ERR_SHAPE);
  if (bytes == 0) return MLA_OK;
  MLA_CHECK_PTR(buf);
  MLA_CHECK_PTR(sink);
  return hip_status(mla::launch_stream_read(buf, bytes, sink, blocks, stream));
}

mla_status_t mla_absorb_append(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                               const void* q_rope, const int32_t* pos_q, const void* w_uk,
                               void* q_full, int32_t n_app, const void* c_kv, const void* k_rope,
                               const int32_t* seq_idx, const int32_t* pos,
                               const int32_t* page_table, int32_t batch, int32_t max_pages,
                               void* cache, int64_t num_pages, int32_t flags, void* stream) {
  mla_status_t st = check_absorb(cfg, n_tok, q_nope, q_rope, pos_q, w_uk, q_full);
  if (st != MLA_OK) return st;
  st = check_append(cfg, n_app, c_kv, k_rope, seq_idx, pos, page_table, batch, max_pages, cache,
                    num_pages, flags);
  if (st != MLA_OK || (n_tok == 0 && n_app == 0)) return st;
  return hip_status(mla::launch_absorb_append(
      shape_of(cfg), n_tok, q_nope, q_rope, pos_q, w_uk, q_full, n_app, c_kv, k_rope, seq_idx, pos,
      nullptr, page_table, batch, max_pages, cache, num_pages, flags == MLA_APPEND_ROTATE,
      stream));
}

mla_status_t mla_absorb_append_at(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                                  const void* q_rope, const int32_t* pos_q, const void* w_uk,
                                  void* q_full, int32_t n_app, const void* c_kv,
                                  const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                  const int32_t* rope_pos, const int32_t* page_table,
                                  int32_t batch, int32_t max_pages, void* cache,
                                  int64_t num_pages, int32_t flags, void* stream) {
  mla_status_t st = check_absorb(cfg, n_tok, q_nope, q_rope, pos_q, w_uk, q_full);
  if (st != MLA_OK) return st;
  st = check_append(cfg, n_app, c_kv, k_rope, seq_idx, pos, page_table, batch, max_pages, cache,
                    num_pages, flags);
  if (st != MLA_OK || (n_tok == 0 && n_app == 0)) return st;
  if (n_app > 0 && rope_pos) MLA_CHECK_PTR(rope_pos);
  return hip_status(mla::launch_absorb_append(
      shape_of(cfg), n_tok, q_nope, q_rope, pos_q, w_uk, q_full, n_app, c_kv, k_rope, seq_idx, pos,
      rope_pos, page_table, batch, max_pages, cache, num_pages, flags == MLA_APPEND_ROTATE,
      stream));
}

mla_status_t mla_decode_paged(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                              int32_t num_splits, int32_t max_seq_len, const void* q_full,
                              const void* cache, int64_t num_pages, const int32_t* page_table,
                              int32_t max_pages, const int32_t* seq_lens, float* o_part,
                              float* lse_part, void* stream) {
  return decode_call(cfg, batch, q_len, 0, num_splits, max_seq_len, q_full, cache, num_pages,
                     page_table, max_pages, seq_lens, nullptr, o_part, lse_part, stream);
}

mla_status_t mla_decode_paged_chunked(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                      int32_t chunk_tokens, int32_t num_splits,
                                      int32_t max_seq_len, const void* q_full, const void* cache,
                                      int64_t num_pages, const int32_t* page_table,
                                      int32_t max_pages, const int32_t* seq_lens, float* o_part,
                                      float* lse_part, void* stream) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(chunk_tokens >= cfg->page_size && chunk_tokens % cfg->page_size == 0,
              MLA_ERR_SHAPE);
  MLA_REQUIRE(num_splits >= 1 && num_splits <= kMaxSplits, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)chunk_tokens * num_splits >= (int64_t)max_seq_len, MLA_ERR_CAPACITY);
  return decode_call(cfg, batch, q_len, chunk_tokens, num_splits, max_seq_len, q_full, cache,
                     num_pages, page_table, max_pages, seq_lens, nullptr, o_part, lse_part,
                     stream);
}

mla_status_t mla_decode_paged_tree(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                   int32_t chunk_tokens, int32_t num_splits, int32_t max_seq_len,
                                   const void* q_full, const void* cache, int64_t num_pages,
                                   const int32_t* page_table, int32_t max_pages,
                                   const int32_t* seq_lens, const int32_t* tree_parent,
                                   float* o_part, float* lse_part, void* stream) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(q_len >= 1 && q_len <= kMaxTreeDrafts, MLA_ERR_SHAPE);
  MLA_REQUIRE(num_splits >= 1 && num_splits <= kMaxSplits, MLA_ERR_SHAPE);
  if (chunk_tokens != 0) {
    MLA_REQUIRE(chunk_tokens >= cfg->page_size && chunk_tokens % cfg->page_size == 0,
                MLA_ERR_SHAPE);
    MLA_REQUIRE((int64_t)chunk_tokens * num_splits >= (int64_t)max_seq_len, MLA_ERR_CAPACITY);
  }
  if (batch > 0) MLA_CHECK_PTR(tree_parent);
  return decode_call(cfg, batch, q_len, chunk_tokens, num_splits, max_seq_len, q_full, cache,
                     num_pages, page_table, max_pages, seq_lens, tree_parent, o_part, lse_part,
                     stream);
}

namespace {

// bits = 8 or 4: bytes of one coded row, 0 when the config cannot be coded
size_t coded_row_bytes(const mla_config_t* cfg, int bits) {
  if (check_config(cfg) != MLA_OK) return 0;
  const int D = cfg->kv_rank + cfg->rope_dim;
  if (bits == 8) return D % 16 ? 0 : (size_t)D + 16;
  if (cfg->kv_rank % 8 || cfg->rope_dim % 8 || D % 32) return 0;
  return (size_t)D / 2 + 16;
}

mla_status_t append_coded(int bits, const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                          const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                          const int32_t* rope_pos, const int32_t* page_table, int32_t batch,
                          int32_t max_pages, void* cache, int64_t num_pages, int32_t flags,
                          void* stream) {
  mla_status_t st = check_append(cfg, n_tok, c_kv, k_rope, seq_idx, pos, page_table, batch,
                                 max_pages, cache, num_pages, flags);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(coded_row_bytes(cfg, bits) != 0, MLA_ERR_UNSUPPORTED);
  if (n_tok == 0) return MLA_OK;
  if (rope_pos) MLA_CHECK_PTR(rope_pos);
  const int rot = flags == MLA_APPEND_ROTATE;
  return hip_status(
      bits == 8 ? mla::launch_cache_append_q8(shape_of(cfg), n_tok, c_kv, k_rope, seq_idx, pos,
                                              rope_pos, page_table, batch, max_pages, cache,
                                              num_pages, rot, stream)
                : mla::launch_cache_append_q4(shape_of(cfg), n_tok, c_kv, k_rope, seq_idx, pos,
                                              rope_pos, page_table, batch, max_pages, cache,
                                              num_pages, rot, stream));
}

mla_status_t decode_coded(int bits, const mla_config_t* cfg, int32_t batch, int32_t q_len,
                          int32_t chunk_tokens, int32_t num_splits, int32_t max_seq_len,
                          const void* q_full, const void* cache, int64_t num_pages,
                          const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens,
                          const int32_t* tree_parent, float* o_part, float* lse_part,
                          void* stream) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(batch >= 0 && q_len >= 1 && max_pages >= 1 && num_pages >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE(num_splits >= 1 && num_splits <= kMaxSplits, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)q_len * cfg->num_heads <= 65536, MLA_ERR_SHAPE);
  if (tree_parent) MLA_REQUIRE(q_len <= kMaxTreeDrafts, MLA_ERR_SHAPE);
  MLA_REQUIRE(max_seq_len >= q_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size >= (int64_t)max_seq_len, MLA_ERR_CAPACITY);
  if (chunk_tokens != 0) {
    MLA_REQUIRE(chunk_tokens >= cfg->page_size && chunk_tokens % cfg->page_size == 0,
                MLA_ERR_SHAPE);
    MLA_REQUIRE((int64_t)chunk_tokens * num_splits >= (int64_t)max_seq_len, MLA_ERR_CAPACITY);
  }
  mla::Shape sh = shape_of(cfg);
  MLA_REQUIRE(mla::decode_q8_ok(sh, q_len), MLA_ERR_UNSUPPORTED);
  if (batch == 0) return MLA_OK;
  MLA_CHECK_PTR(q_full);
  MLA_CHECK_PTR(cache);
  MLA_CHECK_PTR(page_table);
  MLA_CHECK_PTR(seq_lens);
  MLA_CHECK_PTR(o_part);
  MLA_CHECK_PTR(lse_part);
  if (tree_parent) MLA_CHECK_PTR(tree_parent);
  sh.split_fixed = chunk_tokens;
  return hip_status(
      bits == 8 ? mla::launch_decode_q8(sh, batch, q_len, num_splits, max_seq_len, q_full, cache,
                                        num_pages, page_table, max_pages, seq_lens, tree_parent,
                                        o_part, lse_part, stream)
                : mla::launch_decode_q4(sh, batch, q_len, num_splits, max_seq_len, q_full, cache,
                                        num_pages, page_table, max_pages, seq_lens, tree_parent,
                                        o_part, lse_part, stream));
}

}  // namespace

size_t mla_cache_q8_bytes_per_token(const mla_config_t* cfg) { return coded_row_bytes(cfg, 8); }

size_t mla_cache_q4_bytes_per_token(const mla_config_t* cfg) { return coded_row_bytes(cfg, 4); }

mla_status_t mla_cache_append_q8(const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                                 const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                 const int32_t* rope_pos, const int32_t* page_table,
                                 int32_t batch, int32_t max_pages, void* cache_q8,
                                 int64_t num_pages, int32_t flags, void* stream) {
  return append_coded(8, cfg, n_tok, c_kv, k_rope, seq_idx, pos, rope_pos, page_table, batch,
                      max_pages, cache_q8, num_pages, flags, stream);
}

mla_status_t mla_cache_append_q4(const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                                 const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                 const int32_t* rope_pos, const int32_t* page_table,
                                 int32_t batch, int32_t max_pages, void* cache_q4,
                                 int64_t num_pages, int32_t flags, void* stream) {
  return append_coded(4, cfg, n_tok, c_kv, k_rope, seq_idx, pos, rope_pos, page_table, batch,
                      max_pages, cache_q4, num_pages, flags, stream);
}

namespace {

mla_status_t absorb_append_coded(int bits, const mla_config_t* cfg, int32_t n_tok,
                                 const void* q_nope, const void* q_rope, const int32_t* pos_q,
                                 const void* w_uk, void* q_full, int32_t n_app, const void* c_kv,
                                 const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                 const int32_t* rope_pos, const int32_t* page_table,
                                 int32_t batch, int32_t max_pages, void* cache,
                                 int64_t num_pages, int32_t flags, void* stream) {
  mla_status_t st = check_absorb(cfg, n_tok, q_nope, q_rope, pos_q, w_uk, q_full);
  if (st != MLA_OK) return st;
  st = check_append(cfg, n_app, c_kv, k_rope, seq_idx, pos, page_table, batch, max_pages, cache,
                    num_pages, flags);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(coded_row_bytes(cfg, bits) != 0, MLA_ERR_UNSUPPORTED);
  if (n_tok == 0 && n_app == 0) return MLA_OK;
  if (n_app > 0 && rope_pos) MLA_CHECK_PTR(rope_pos);
  return hip_status(mla::launch_absorb_append_coded(
      bits, shape_of(cfg), n_tok, q_nope, q_rope, pos_q, w_uk, q_full, n_app, c_kv, k_rope,
      seq_idx, pos, rope_pos, page_table, batch, max_pages, cache, num_pages,
      flags == MLA_APPEND_ROTATE, stream));
}

}  // namespace

mla_status_t mla_absorb_append_q8(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                                  const void* q_rope, const int32_t* pos_q, const void* w_uk,
                                  void* q_full, int32_t n_app, const void* c_kv,
                                  const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                  const int32_t* rope_pos, const int32_t* page_table,
                                  int32_t batch, int32_t max_pages, void* cache_q8,
                                  int64_t num_pages, int32_t flags, void* stream) {
  return absorb_append_coded(8, cfg, n_tok, q_nope, q_rope, pos_q, w_uk, q_full, n_app, c_kv,
                             k_rope, seq_idx, pos, rope_pos, page_table, batch, max_pages,
                             cache_q8, num_pages, flags, stream);
}

mla_status_t mla_absorb_append_q4(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                                  const void* q_rope, const int32_t* pos_q, const void* w_uk,
                                  void* q_full, int32_t n_app, const void* c_kv,
                                  const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                  const int32_t* rope_pos, const int32_t* page_table,
                                  int32_t batch, int32_t max_pages, void* cache_q4,
                                  int64_t num_pages, int32_t flags, void* stream) {
  return absorb_append_coded(4, cfg, n_tok, q_nope, q_rope, pos_q, w_uk, q_full, n_app, c_kv,
                             k_rope, seq_idx, pos, rope_pos, page_table, batch, max_pages,
                             cache_q4, num_pages, flags, stream);
}

mla_status_t mla_decode_paged_q8(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                 int32_t chunk_tokens, int32_t num_splits, int32_t max_seq_len,
                                 const void* q_full, const void* cache_q8, int64_t num_pages,
                                 const int32_t* page_table, int32_t max_pages,
                                 const int32_t* seq_lens, const int32_t* tree_parent,
                                 float* o_part, float* lse_part, void* stream) {
  return decode_coded(8, cfg, batch, q_len, chunk_tokens, num_splits, max_seq_len, q_full,
                      cache_q8, num_pages, page_table, max_pages, seq_lens, tree_parent, o_part,
                      lse_part, stream);
}

mla_status_t mla_decode_paged_q4(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                 int32_t chunk_tokens, int32_t num_splits, int32_t max_seq_len,
                                 const void* q_full, const void* cache_q4, int64_t num_pages,
                                 const int32_t* page_table, int32_t max_pages,
                                 const int32_t* seq_lens, const int32_t* tree_parent,
                                 float* o_part, float* lse_part, void* stream) {
  return decode_coded(4, cfg, batch, q_len, chunk_tokens, num_splits, max_seq_len, q_full,
                      cache_q4, num_pages, page_table, max_pages, seq_lens, tree_parent, o_part,
                      lse_part, stream);
}

namespace {
constexpr int kMaxIndexHeads = 256;
constexpr int kMaxIndexDim = 1024;
constexpr int kMaxTopk = 65536;

mla_status_t check_index_shape(const mla_config_t* cfg, int32_t index_heads, int32_t index_dim) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(index_heads >= 1 && index_heads <= kMaxIndexHeads, MLA_ERR_SHAPE);
  MLA_REQUIRE(index_dim >= 1 && index_dim <= kMaxIndexDim, MLA_ERR_SHAPE);
  MLA_REQUIRE(index_dim % (cfg->dtype == MLA_F32 ? 4 : 8) == 0, MLA_ERR_SHAPE);
  return MLA_OK;
}

// list entries per partition of the sparse decode: ceil(topk / S) rounded up
// to a whole 32-token tile
int32_t sparse_chunk(int32_t topk, int32_t num_splits) {
  const int32_t per = (topk + num_splits - 1) / num_splits;
  return ((per + 31) / 32) * 32;
}
}  // namespace

mla_status_t mla_absorb_append_index(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                                     const void* q_rope, const int32_t* pos_q, const void* w_uk,
                                     void* q_full, int32_t n_app, const void* c_kv,
                                     const void* k_rope, const int32_t* seq_idx,
                                     const int32_t* pos, const int32_t* page_table,
                                     int32_t batch, int32_t max_pages, void* cache,
                                     int64_t num_pages, int32_t flags, int32_t index_dim,
                                     const void* k_idx, void* index_cache, void* stream) {
  mla_status_t st = check_absorb(cfg, n_tok, q_nope, q_rope, pos_q, w_uk, q_full);
  if (st != MLA_OK) return st;
  st = check_append(cfg, n_app, c_kv, k_rope, seq_idx, pos, page_table, batch, max_pages, cache,
                    num_pages, flags);
  if (st != MLA_OK) return st;
  st = check_index_shape(cfg, 1, index_dim);
  if (st != MLA_OK) return st;
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size <= INT32_MAX, MLA_ERR_CAPACITY);
  if (n_tok == 0 && n_app == 0) return MLA_OK;
  if (n_app > 0) {
    MLA_CHECK_PTR(k_idx);
    MLA_CHECK_PTR(index_cache);
  }
  return hip_status(mla::launch_absorb_append(
      shape_of(cfg), n_tok, q_nope, q_rope, pos_q, w_uk, q_full, n_app, c_kv, k_rope, seq_idx, pos,
      nullptr, page_table, batch, max_pages, cache, num_pages, flags == MLA_APPEND_ROTATE, stream,
      index_dim, k_idx, index_cache));
}

mla_status_t mla_index_append(const mla_config_t* cfg, int32_t index_dim, int32_t n_tok,
                              const void* k_idx, const int32_t* seq_idx, const int32_t* pos,
                              const int32_t* page_table, int32_t batch, int32_t max_pages,
                              void* index_cache, int64_t num_pages, void* stream) {
  mla_status_t st = check_index_shape(cfg, 1, index_dim);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(n_tok >= 0 && batch >= 1 && max_pages >= 1 && num_pages >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size <= INT32_MAX, MLA_ERR_CAPACITY);
  if (n_tok == 0) return MLA_OK;
  MLA_CHECK_PTR(k_idx);
  MLA_CHECK_PTR(seq_idx);
  MLA_CHECK_PTR(pos);
  MLA_CHECK_PTR(page_table);
  MLA_CHECK_PTR(index_cache);
  return hip_status(mla::launch_index_append(shape_of(cfg), index_dim, n_tok, k_idx, seq_idx, pos,
                                             page_table, batch, max_pages, index_cache, num_pages,
                                             stream));
}

mla_status_t mla_index_scores(const mla_config_t* cfg, int32_t index_heads, int32_t index_dim,
                              int32_t batch, int32_t q_len, int32_t max_seq_len,
                              const void* q_idx, const float* w_idx, const void* index_cache,
                              int64_t num_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens, float* scores, int32_t ld_scores,
                              void* stream) {
  mla_status_t st = check_index_shape(cfg, index_heads, index_dim);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(batch >= 0 && q_len >= 1 && max_pages >= 1 && num_pages >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE(q_len <= 65535, MLA_ERR_SHAPE);
  MLA_REQUIRE(max_seq_len >= q_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size >= (int64_t)max_seq_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE(ld_scores >= max_seq_len, MLA_ERR_SHAPE);
  mla::Shape sh = shape_of(cfg);
  if (!mla::index_scores_mfma_ok(sh, index_heads, index_dim))
    MLA_REQUIRE(mla::index_scores_generic_lds(index_heads, index_dim) <= 160 * 1024,
                MLA_ERR_UNSUPPORTED);
  if (batch == 0) return MLA_OK;
  MLA_CHECK_PTR(q_idx);
  MLA_CHECK_PTR(w_idx);
  MLA_CHECK_PTR(index_cache);
  MLA_CHECK_PTR(page_table);
  MLA_CHECK_PTR(seq_lens);
  MLA_CHECK_PTR(scores);
  return hip_status(mla::launch_index_scores(sh, index_heads, index_dim, batch, q_len, max_seq_len,
                                             q_idx, w_idx, index_cache, num_pages, page_table,
                                             max_pages, seq_lens, scores, ld_scores, stream));
}

size_t mla_topk_workspace_bytes(int32_t batch, int32_t q_len) {
  if (batch < 0 || q_len < 1 || (int64_t)batch * q_len > INT32_MAX) return 0;
  return mla::topk_workspace_bytes(batch, q_len);
}

mla_status_t mla_topk_select(int32_t batch, int32_t q_len, int32_t max_seq_len, int32_t topk,
                             const float* scores, int32_t ld_scores, const int32_t* seq_lens,
                             void* workspace, int32_t* indices, int32_t* counts, void* stream) {
  MLA_REQUIRE(batch >= 0 && q_len >= 1 && topk >= 1 && topk <= kMaxTopk, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)batch * q_len <= INT32_MAX, MLA_ERR_SHAPE);
  MLA_REQUIRE(max_seq_len >= q_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE(ld_scores >= max_seq_len, MLA_ERR_SHAPE);
  if (batch == 0) return MLA_OK;
  MLA_CHECK_PTR(scores);
  MLA_CHECK_PTR(seq_lens);
  MLA_CHECK_PTR(workspace);
  MLA_CHECK_PTR(indices);
  MLA_CHECK_PTR(counts);
  return hip_status(mla::launch_topk(batch, q_len, max_seq_len, topk, scores, ld_scores, seq_lens,
                                     workspace, indices, counts, stream));
}

mla_status_t mla_index_scores_topk(const mla_config_t* cfg, int32_t index_heads,
                                   int32_t index_dim, int32_t batch, int32_t q_len,
                                   int32_t max_seq_len, const void* q_idx, const float* w_idx,
                                   const void* index_cache, int64_t num_pages,
                                   const int32_t* page_table, int32_t max_pages,
                                   const int32_t* seq_lens, float* scores, int32_t ld_scores,
                                   int32_t topk, void* workspace, int32_t* indices,
                                   int32_t* counts, void* stream) {
  mla_status_t st = check_index_shape(cfg, index_heads, index_dim);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(batch >= 0 && q_len >= 1 && max_pages >= 1 && num_pages >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE(q_len <= 65535, MLA_ERR_SHAPE);
  MLA_REQUIRE(topk >= 1 && topk <= kMaxTopk, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)batch * q_len <= INT32_MAX, MLA_ERR_SHAPE);
  MLA_REQUIRE(max_seq_len >= q_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size >= (int64_t)max_seq_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE(ld_scores >= max_seq_len, MLA_ERR_SHAPE);
  mla::Shape sh = shape_of(cfg);
  if (!mla::index_scores_mfma_ok(sh, index_heads, index_dim))
    MLA_REQUIRE(mla::index_scores_generic_lds(index_heads, index_dim) <= 160 * 1024,
                MLA_ERR_UNSUPPORTED);
  if (batch == 0) return MLA_OK;
  MLA_CHECK_PTR(q_idx);
  MLA_CHECK_PTR(w_idx);
  MLA_CHECK_PTR(index_cache);
  MLA_CHECK_PTR(page_table);
  MLA_CHECK_PTR(seq_lens);
  MLA_CHECK_PTR(scores);
  MLA_CHECK_PTR(workspace);
  MLA_CHECK_PTR(indices);
  MLA_CHECK_PTR(counts);
  return hip_status(mla::launch_index_scores_topk(
      sh, index_heads, index_dim, batch, q_len, max_seq_len, q_idx, w_idx, index_cache, num_pages,
      page_table, max_pages, seq_lens, scores, ld_scores, topk, workspace, indices, counts,
      stream));
}

mla_status_t mla_index_scores_topk_noalloc(const mla_config_t* cfg, int32_t index_heads,
                                           int32_t index_dim, int32_t batch, int32_t q_len,
                                           int32_t max_seq_len, const void* q_idx,
                                           const float* w_idx, const void* index_cache,
                                           int64_t num_pages, const int32_t* page_table,
                                           int32_t max_pages, const int32_t* seq_lens,
                                           float* scores, int32_t ld_scores, int32_t topk,
                                           int32_t* indices, int32_t* counts, void* stream) {
  static_assert(MLA_TOPK_NOALLOC_MAX_QUERIES == mla::kTopkNoallocMaxQueries,
                "the header states the library's limit");
  mla_status_t st = check_index_shape(cfg, index_heads, index_dim);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(batch >= 0 && q_len >= 1 && max_pages >= 1 && num_pages >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE(q_len <= 65535, MLA_ERR_SHAPE);
  MLA_REQUIRE(topk >= 1 && topk <= kMaxTopk, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)batch * q_len <= MLA_TOPK_NOALLOC_MAX_QUERIES, MLA_ERR_CAPACITY);
  MLA_REQUIRE(max_seq_len >= q_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size >= (int64_t)max_seq_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE(ld_scores >= max_seq_len, MLA_ERR_SHAPE);
  mla::Shape sh = shape_of(cfg);
  if (!mla::index_scores_mfma_ok(sh, index_heads, index_dim))
    MLA_REQUIRE(mla::index_scores_generic_lds(index_heads, index_dim) <= 160 * 1024,
                MLA_ERR_UNSUPPORTED);
  if (batch == 0) return MLA_OK;
  MLA_CHECK_PTR(q_idx);
  MLA_CHECK_PTR(w_idx);
  MLA_CHECK_PTR(index_cache);
  MLA_CHECK_PTR(page_table);
  MLA_CHECK_PTR(seq_lens);
  MLA_CHECK_PTR(scores);
  MLA_CHECK_PTR(indices);
  MLA_CHECK_PTR(counts);
  return hip_status(mla::launch_index_scores_topk_noalloc(
      sh, index_heads, index_dim, batch, q_len, max_seq_len, q_idx, w_idx, index_cache,
      num_pages, page_table, max_pages, seq_lens, scores, ld_scores, topk, indices, counts,
      stream));
}

int32_t mla_sparse_chunk(int32_t topk, int32_t num_splits) {
  if (topk < 1 || topk > kMaxTopk || num_splits < 1 || num_splits > kMaxSplits) return 0;
  return sparse_chunk(topk, num_splits);
}

const char* mla_decode_sparse_kernel_name(const mla_config_t* cfg, int32_t topk,
                                          int32_t num_splits) {
  if (check_config(cfg) != MLA_OK || topk < 1 || topk > kMaxTopk || num_splits < 1 ||
      num_splits > kMaxSplits)
    return "invalid";
  return mla::decode_sparse_kind(shape_of(cfg), sparse_chunk(topk, num_splits)) == 1
             ? "mfma_rows16_gather"
             : "generic_gather";
}

mla_status_t mla_decode_sparse(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                               int32_t topk, int32_t num_splits, int32_t max_seq_len,
                               const void* q_full, const void* cache, int64_t num_pages,
                               const int32_t* page_table, int32_t max_pages,
                               const int32_t* seq_lens, const int32_t* indices,
                               const int32_t* counts, float* o_part, float* lse_part,
                               void* stream) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(batch >= 0 && q_len >= 1 && max_pages >= 1 && num_pages >= 1, MLA_ERR_SHAPE);
  MLA_REQUIRE(num_splits >= 1 && num_splits <= kMaxSplits, MLA_ERR_SHAPE);
  MLA_REQUIRE(topk >= 1 && topk <= kMaxTopk, MLA_ERR_SHAPE);
  MLA_REQUIRE((int64_t)q_len * cfg->num_heads <= 65536, MLA_ERR_SHAPE);
  MLA_REQUIRE(max_seq_len >= q_len, MLA_ERR_CAPACITY);
  MLA_REQUIRE((int64_t)max_pages * cfg->page_size >= (int64_t)max_seq_len, MLA_ERR_CAPACITY);
  if (batch == 0) return MLA_OK;
  MLA_CHECK_PTR(q_full);
  MLA_CHECK_PTR(cache);
  MLA_CHECK_PTR(page_table);
  MLA_CHECK_PTR(seq_lens);
  MLA_CHECK_PTR(indices);
  MLA_CHECK_PTR(counts);
  MLA_CHECK_PTR(o_part);
  MLA_CHECK_PTR(lse_part);
  return hip_status(mla::launch_decode_sparse(shape_of(cfg), batch, q_len, topk,
                                              sparse_chunk(topk, num_splits), num_splits,
                                              max_seq_len, q_full, cache, num_pages, page_table,
                                              max_pages, seq_lens, indices, counts, o_part,
                                              lse_part, stream));
}

mla_status_t mla_chunk_plan(const mla_config_t* cfg, int64_t total_tokens, int32_t max_seq_len,
                            int32_t num_cus, int32_t* chunk_tokens, int32_t* num_splits) {
  mla_status_t st = check_config(cfg);
  if (st != MLA_OK) return st;
  MLA_REQUIRE(chunk_tokens && num_splits, MLA_ERR_NULL);
  MLA_REQUIRE(total_tokens >= 1 && max_seq_len >= 1, MLA_ERR_SHAPE);
  if (num_cus < 1) num_cus = 256;
  // about kChunksPerCu partitions per compute unit: the block dispatcher then
  // evens out the work, and the last round is short
  const int64_t pg = cfg->page_size;
  const int64_t want = (total_tokens + (int64_t)kChunksPerCu * num_cus - 1) /
                       ((int64_t)kChunksPerCu * num_cus);
  int64_t chunk = pg * ((want + pg - 1) / pg);
  const int64_t min_chunk = pg * (((int64_t)max_seq_len + (int64_t)kMaxSplits * pg - 1) /
                                  ((int64_t)kMaxSplits * pg));
  if (chunk < min_chunk) chunk = min_chunk;
  if (chunk < pg) chunk = pg;
  if (chunk > INT32_MAX / 2) return MLA_ERR_CAPACITY;
  *chunk_tokens = (int32_t)chunk;
  *num_splits = (int32_t)(((int64_t)max_seq_len + chunk - 1) / chunk);
  return MLA_OK;
}

mla_status_t mla_splitkv_combine(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                 int32_t num_splits, const float* o_part, const float* lse_part,
                                 void* o_lat, float* lse, void* stream) {
  mla_status_t st = check_combine(cfg, batch, q_len, num_splits, o_part, lse_part, o_lat, lse);
  if (st != MLA_OK || batch == 0) return st;
  const int rows = batch * q_len * cfg->num_heads;
  return hip_status(
      mla::launch_combine(shape_of(cfg), rows, num_splits, o_part, lse_part, o_lat, lse, stream));
}

mla_status_t mla_up_project_v(const mla_config_t* cfg, int32_t n_tok, const void* o_lat,
                              const void* w_uv, void* out, void* stream) {
  mla_status_t st = check_up_project(cfg, n_tok, o_lat, w_uv, out);
  if (st != MLA_OK || n_tok == 0) return st;
  return hip_status(mla::launch_up_project_v(shape_of(cfg), n_tok, o_lat, w_uv, out, stream));
}

mla_status_t mla_combine_up_project(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                    int32_t num_splits, const float* o_part,
                                    const float* lse_part, void* o_lat, float* lse,
                                    const void* w_uv, void* out, void* stream) {
  mla_status_t st = check_combine(cfg, batch, q_len, num_splits, o_part, lse_part, o_lat, lse);
  if (st != MLA_OK || batch == 0) return st;
  const int n_tok = batch * q_len;
  st = check_up_project(cfg, n_tok, o_lat, w_uv, out);
  if (st != MLA_OK) return st;
  return hip_status(mla::launch_combine_up_project(shape_of(cfg), n_tok, num_splits, o_part,
                                                   lse_part, o_lat, lse, w_uv, out, stream));
}

}  // extern "C"
