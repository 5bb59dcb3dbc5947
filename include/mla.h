/*
 * mla.h - C ABI of the MLA latent-cache decode library (libmla.so, gfx950).
 *
 * Multi-Head Latent Attention caches one row per token and layer: a d_c-wide
 * latent c_t followed by a d_r-wide RoPE key k^R_t (rotated by the token's
 * position), D = d_c + d_r numbers ("DeepSeek's Config Says 16 KV Heads, Its
 * Cache Holds a Ninth of That", section 5 "Multi-head latent attention (MLA)";
 * "The Architecture of Memory", "Decoupled Rotary Positional Encoding (RoPE)").
 * One decode step runs five calls, in this order:
 *
 *   mla_absorb_q        query -> latent space through W_UK, RoPE on the query
 *   mla_cache_append    write the new token rows through the page table
 *   mla_decode_paged    split-KV attention of the absorbed queries over the cache
 *                       (mla_decode_paged_chunked: fixed-size partitions)
 *   mla_splitkv_combine log-sum-exp merge of the split partials
 *   mla_up_project_v    latent output -> per-head value space through W_UV
 *   mla_absorb_append, mla_combine_up_project
 *                       two pairs of the above, each in one launch
 * Verifying a tree of drafted tokens instead of a chain takes
 * mla_absorb_append_at / mla_cache_append_at (a token's cache slot and its
 * RoPE position differ) and mla_decode_paged_tree (the tree mask), with the
 * drafted rows' slots and positions from mla_draft_positions. An 8-bit
 * cache takes mla_cache_append_q8 (or mla_absorb_append_q8) and
 * mla_decode_paged_q8, a 4-bit one the _q4 calls; a sparse read (attention
 * over the top-scored tokens only) takes mla_index_append, mla_index_scores,
 * mla_topk_select and mla_decode_sparse. A chunked prefill runs the decode
 * calls with q_len = C, or mla_prefill_unabsorbed.
 *
 * Conventions shared by every call
 *   - Every pointer argument except `cfg` is a DEVICE pointer; `cfg` is a host
 *     pointer read during the call only. The caller owns all memory; the
 *     library never allocates, frees or keeps a pointer after returning.
 *   - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and returns once the work is enqueued. The
 *     library holds no per-call state; what it remembers across calls
 *     (which kernels have had their LDS limit raised on which device, and
 *     the device address of mla_index_scores_topk_noalloc's array) is set
 *     under a lock on first use, so calls may come from several threads.
 *     Calls that write the same buffers must not overlap.
 *   - Layouts are dense, row-major, in the order written in brackets; element
 *     type "T" is cfg->dtype (fp32 or bf16) for queries, weights, cache and
 *     outputs; partials are always fp32.
 *   - Device buffers must be 16-byte aligned (MLA_ERR_ALIGN otherwise).
 *   - Host-side checks run before any launch; on error nothing is enqueued
 *     and the call returns the status. MLA_ERR_HIP means a launch failed.
 *   - Device-side data that the host cannot see (page-table entries, lengths,
 *     positions) is bounds-checked in the kernels: an invalid entry is never
 *     followed out of bounds. Appends of invalid rows are dropped; a sequence
 *     whose length or pages are invalid gets NaN outputs.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype_t;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL                          */
  MLA_ERR_SHAPE = 2,       /* a size is out of range or sizes are inconsistent    */
  MLA_ERR_DTYPE = 3,       /* cfg->dtype is not an mla_dtype_t                    */
  MLA_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned             */
  MLA_ERR_CAPACITY = 5,    /* pages or lengths cannot hold what was asked         */
  MLA_ERR_UNSUPPORTED = 6, /* a valid shape this build has no kernel for          */
  MLA_ERR_HIP = 7          /* the HIP runtime reported an error                   */
} mla_status_t;

/* Shape of one MLA attention layer.
 *   num_heads  H    query heads (all share the one latent row per token)
 *   kv_rank    d_c  latent width (512 for DeepSeek-V2/V3, V2-Lite, Kimi K2)
 *   rope_dim   d_r  decoupled RoPE key width, even (64 for the same models)
 *   nope_dim   d_n  per-head content query/key width before absorption (128)
 *   v_dim      d_v  per-head value width (128)
 *   page_size       tokens per cache page; a power of two in [16, 256]
 *   dtype           mla_dtype_t of every T-typed buffer
 *   softmax_scale   multiplies q.k before the softmax (1/sqrt(d_n + d_r))
 *   rope_base       RoPE base; pair i of a d_r-wide vector at position p is
 *                   rotated by p * rope_base^(-2i/d_r) (interleaved pairs)
 * Limits of this build: 1 <= H <= 1024, 16 <= d_c <= 1024, 2 <= d_r <= 256,
 * 1 <= d_n, d_v <= 256, d_c and d_r multiples of 8 (bf16) or 4 (fp32). */
typedef struct {
  int32_t num_heads;
  int32_t kv_rank;
  int32_t rope_dim;
  int32_t nope_dim;
  int32_t v_dim;
  int32_t page_size;
  int32_t dtype;
  float softmax_scale;
  float rope_base;
} mla_config_t;

/* Append modes. */
enum { MLA_APPEND_RAW = 0, MLA_APPEND_ROTATE = 1 };

/* Library version and target, e.g. "libmla 0.1 gfx950". Static string. */
const char* mla_build_info(void);

/* Human-readable name of a status code. Static string, never NULL. */
const char* mla_status_str(mla_status_t status);

/* MLA_OK if the config is within this build's limits, else the error code. */
mla_status_t mla_config_validate(const mla_config_t* cfg);

/* Bytes of one cached row: (d_c + d_r) * sizeof(T); 0 for an invalid config.
 * 1,152 B for d_c = 512, d_r = 64 in bf16 ("DeepSeek's Config Says 16 KV
 * Heads", introduction; "The Architecture of Memory", "DeepSeek's Multi-Head
 * Latent Attention (MLA)"). */
size_t mla_cache_bytes_per_token(const mla_config_t* cfg);

/* Split-KV plan: partition s of a sequence of length L covers tokens
 * [s*chunk, min(L, (s+1)*chunk)) with chunk = page_size * ceil(ceil(L/S) /
 * page_size); partitions past the end are empty. Writes the chunk length to
 * *chunk_tokens. Host helper mirroring the kernels. */
mla_status_t mla_split_chunk(const mla_config_t* cfg, int32_t seq_len, int32_t num_splits,
                             int32_t* chunk_tokens);

/* A split count that fills the GPU for this batch (a heuristic; any value in
 * [1, 4096] is valid). num_cus = compute units of the device (256 on MI355X). */
int32_t mla_default_num_splits(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                               int32_t max_seq_len, int32_t num_cus);

/* Name of the decode kernel mla_decode_paged takes for this shape. With bf16,
 * d_c = 512 and d_r = 64: "mfma_ws" (64 query rows per block) when
 * page_size is a multiple of 8 and q_len*H a multiple of 64, else "mfma_rows16" (16 rows per
 * block) when q_len*H is a multiple of 16; otherwise "generic". Static
 * string; "invalid" for an invalid config. */
const char* mla_decode_kernel_name(const mla_config_t* cfg, int32_t q_len);

/* Bytes of o_part plus lse_part for mla_decode_paged:
 * batch*q_len*H*num_splits*(d_c + 1)*4. 0 for invalid arguments. */
size_t mla_decode_partials_bytes(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                 int32_t num_splits);

/* a1. Query absorption and query RoPE ("The Architecture of Memory", "The
 * Weight Absorption Trick" and "Decoupled Rotary Positional Encoding (RoPE)";
 * "DeepSeek's Config Says 16 KV Heads", section 5):
 *   q_full[n][h][0:d_c]   = W_UK[h]^T q_nope[n][h]          (fp32 accumulate)
 *   q_full[n][h][d_c:D]   = RoPE(q_rope[n][h], pos[n])      (angles in fp64)
 * q_nope [n_tok][H][d_n] T, q_rope [n_tok][H][d_r] T, pos [n_tok] int32,
 * w_uk [H][d_n][d_c] T, q_full [n_tok][H][D] T (out). n_tok = 0 is a no-op. */
mla_status_t mla_absorb_q(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                          const void* q_rope, const int32_t* pos, const void* w_uk,
                          void* q_full, void* stream);

/* a2. Paged cache append ("The Architecture of Memory", "PagedAttention:
 * Virtual Memory for LLMs"; "KV Cache Optimization: Scaling to Million-Token
 * Contexts", technique 7): row n goes to physical row
 *   page_table[seq_idx[n]][pos[n] / page_size] * page_size + pos[n] % page_size
 * of cache [num_pages][page_size][D] T as [c_kv[n] ; k], where k = k_rope[n]
 * rotated by pos[n] (MLA_APPEND_ROTATE) or copied unchanged (MLA_APPEND_RAW).
 * c_kv [n_tok][d_c] T, k_rope [n_tok][d_r] T, seq_idx, pos [n_tok] int32,
 * page_table [batch][max_pages] int32. Rows whose seq_idx, pos or page entry
 * is out of range are skipped. Rows that target the same slot race. */
mla_status_t mla_cache_append(const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                              const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                              const int32_t* page_table, int32_t batch, int32_t max_pages,
                              void* cache, int64_t num_pages, int32_t flags, void* stream);

/* a2 with the RoPE key rotated by rope_pos[n] instead of pos[n] (MLA_APPEND_
 * ROTATE; pos[n] still picks the slot). A drafted token of a tree sits in the
 * cache after its siblings but is positioned one past its parent ("The
 * Architecture of Memory", "Tree Attention Verification"): slot L - Q + i,
 * position L - Q + depth(i). rope_pos [n_tok] int32 (device); NULL means pos.
 * Other arguments, layouts and errors as for mla_cache_append. */
mla_status_t mla_cache_append_at(const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                                 const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                 const int32_t* rope_pos, const int32_t* page_table,
                                 int32_t batch, int32_t max_pages, void* cache, int64_t num_pages,
                                 int32_t flags, void* stream);

/* Positions of the drafted tokens of a verify step, derived on the device
 * from the lengths and the tree ("The Architecture of Memory", "Tree
 * Attention Verification": a drafted token sits in the cache after its
 * siblings but one position past its parent). For row n = b * q_len + i:
 *   seq_idx[n] = b,  slot[n] = L_b - q_len + i,  pos[n] = L_b - q_len + depth(i)
 * where depth(i) is 0 when tree_parent[b][i] = -1, else one more than the
 * parent's depth; tree_parent NULL means the chain (pos = slot). A sequence
 * whose L_b lies outside [q_len, max_seq_len] or whose tree breaks
 * tree_parent[b][i] in [-1, i) gets slot = pos = -1 for all its rows, so the
 * append calls skip them and mla_decode_paged_tree returns NaN for it.
 * seq_lens [batch], tree_parent [batch][q_len] (q_len <= 64) or NULL,
 * seq_idx, slot, pos [batch * q_len] int32 (out), all device pointers.
 * A tree step passes pos as the query positions (mla_absorb_q / the pos_q of
 * mla_absorb_append_at), slot and pos as the slot and RoPE position of each
 * drafted row (mla_cache_append_at, mla_absorb_append_at,
 * mla_cache_append_q8), and the same tree_parent to the decode: the RoPE
 * rotations then agree with the tree the decode masks by, which the decode
 * itself cannot check (it sees only rotated values). */
mla_status_t mla_draft_positions(int32_t batch, int32_t q_len, int32_t max_seq_len,
                                 const int32_t* seq_lens, const int32_t* tree_parent,
                                 int32_t* seq_idx, int32_t* slot, int32_t* pos, void* stream);

/* a1 + a2 in one launch, for callers that run both every step: the same
 * arguments, work and results (bit for bit) as
 *   mla_absorb_q(cfg, n_tok, q_nope, q_rope, pos_q, w_uk, q_full, stream);
 *   mla_cache_append(cfg, n_app, c_kv, k_rope, seq_idx, pos, page_table,
 *                    batch, max_pages, cache, num_pages, flags, stream);
 * whose outputs are disjoint. One launch when the absorption runs on bf16
 * MFMA (bf16, d_n and d_c multiples of 64), the two launches otherwise.
 * Errors as for the two calls (the absorb arguments are checked first). */
mla_status_t mla_absorb_append(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                               const void* q_rope, const int32_t* pos_q, const void* w_uk,
                               void* q_full, int32_t n_app, const void* c_kv, const void* k_rope,
                               const int32_t* seq_idx, const int32_t* pos,
                               const int32_t* page_table, int32_t batch, int32_t max_pages,
                               void* cache, int64_t num_pages, int32_t flags, void* stream);

/* mla_absorb_append with the appended RoPE keys rotated by rope_pos (NULL:
 * pos), i.e. mla_absorb_q followed by mla_cache_append_at, bit for bit. */
mla_status_t mla_absorb_append_at(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                                  const void* q_rope, const int32_t* pos_q, const void* w_uk,
                                  void* q_full, int32_t n_app, const void* c_kv,
                                  const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                  const int32_t* rope_pos, const int32_t* page_table,
                                  int32_t batch, int32_t max_pages, void* cache,
                                  int64_t num_pages, int32_t flags, void* stream);

/* a4. Split-KV paged decode ("The Architecture of Memory", "Flash-Decoding
 * and FlashInfer" and "The Decode Phase: The Memory Bandwidth Wall";
 * "Speculative Decoding: Amortizing the Memory Fetch" for q_len > 1).
 * For sequence b (length L_b = seq_lens[b], which includes the q_len newest
 * tokens), query j at position p = L_b - q_len + j, head h, partition s:
 *   score_t = softmax_scale * (q_full[b][j][h] . cache_row(b, t)),  t <= p
 *   o_part[b][j][h][s]   = sum_t e^(score_t - m) c_t / sum_t e^(score_t - m)
 *   lse_part[b][j][h][s] = m + ln sum_t e^(score_t - m)   (natural log)
 * over the tokens t of partition s (plan: mla_split_chunk). c_t = the first
 * d_c entries of the row. A partition whose tokens are all masked gives
 * o = 0, lse = -inf; an empty partition (no tokens) gives lse = -inf and
 * leaves its o_part row unwritten (mla_splitkv_combine never reads a
 * partition of weight 0).
 * q_full [batch][q_len][H][D] T, cache [num_pages][page_size][D] T,
 * page_table [batch][max_pages] int32, seq_lens [batch] int32,
 * o_part [batch][q_len][H][num_splits][d_c] f32, lse_part [batch][q_len][H][num_splits] f32.
 * Host checks: 1 <= q_len <= max_seq_len <= max_pages * page_size,
 * 1 <= num_splits <= 4096. Device: q_len <= L_b <= max_seq_len and page
 * entries in [0, num_pages), else that sequence's outputs are NaN. */
mla_status_t mla_decode_paged(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                              int32_t num_splits, int32_t max_seq_len, const void* q_full,
                              const void* cache, int64_t num_pages, const int32_t* page_table,
                              int32_t max_pages, const int32_t* seq_lens, float* o_part,
                              float* lse_part, void* stream);

/* a4 with fixed-size partitions: partition s of sequence b covers tokens
 * [s*chunk_tokens, min(L_b, (s+1)*chunk_tokens)), so a long sequence has more
 * non-empty partitions than a short one and every partition is at most
 * chunk_tokens long: with lengths that differ, the work per block stays even
 * (the per-sequence plan of mla_decode_paged gives every sequence S partitions
 * of L_b/S tokens). Partitions past a sequence's end are empty (lse_part =
 * -inf, o_part unwritten). chunk_tokens must be a positive multiple of page_size and
 * chunk_tokens*num_splits >= max_seq_len (MLA_ERR_CAPACITY otherwise). Other
 * arguments, layouts and errors as for mla_decode_paged; the outputs of
 * mla_splitkv_combine are the same for either plan up to rounding. */
mla_status_t mla_decode_paged_chunked(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                      int32_t chunk_tokens, int32_t num_splits,
                                      int32_t max_seq_len, const void* q_full, const void* cache,
                                      int64_t num_pages, const int32_t* page_table,
                                      int32_t max_pages, const int32_t* seq_lens, float* o_part,
                                      float* lse_part, void* stream);

/* a4 verifying a tree of drafted tokens ("The Architecture of Memory", "Tree
 * Attention Verification"; "Speculative Decoding: Amortizing the Memory
 * Fetch"). The last q_len cached tokens of sequence b are drafted tokens;
 * tree_parent[b][i] in [-1, i) names the drafted token that token i continues
 * (-1: it continues the prefix). Query j (its query position is
 * L_b - q_len + depth(j), as are the RoPE keys of the drafted tokens: see
 * mla_cache_append_at) sees every prefix token t < L_b - q_len with no mask
 * and the drafted tokens on its own branch: j and its ancestors. A chain
 * (tree_parent[b][i] = i - 1) gives the same bits as mla_decode_paged.
 * tree_parent [batch][q_len] int32 (device), 1 <= q_len <= 64. chunk_tokens:
 * 0 for the per-sequence plan of mla_decode_paged, else the fixed-size plan
 * of mla_decode_paged_chunked. A sequence whose tree entries break the rule
 * gets NaN outputs. Other arguments, layouts and errors as mla_decode_paged. */
mla_status_t mla_decode_paged_tree(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                   int32_t chunk_tokens, int32_t num_splits, int32_t max_seq_len,
                                   const void* q_full, const void* cache, int64_t num_pages,
                                   const int32_t* page_table, int32_t max_pages,
                                   const int32_t* seq_lens, const int32_t* tree_parent,
                                   float* o_part, float* lse_part, void* stream);

/* A fixed-size partition plan for mla_decode_paged_chunked: about six
 * partitions per compute unit over total_tokens = sum of the batch's lengths,
 * whole pages, at most 4,096 partitions per sequence. Writes chunk_tokens and
 * num_splits = ceil(max_seq_len / chunk_tokens). */
mla_status_t mla_chunk_plan(const mla_config_t* cfg, int64_t total_tokens, int32_t max_seq_len,
                            int32_t num_cus, int32_t* chunk_tokens, int32_t* num_splits);

/* 8-bit latent cache (f2; "KV Cache Optimization: Scaling to Million-Token
 * Contexts", technique 3 "KV Cache Quantization" and its comparison table):
 * a row of cache_q8 [num_pages][page_size][D + 16] bytes is the d_c + d_r
 * codes (uint8) of the row's latent part and rotated RoPE part, each coded
 * between its own minimum and maximum, followed by four fp32: latent min,
 * latent step, RoPE min, RoPE step. step = (max - min) / 255, code =
 * rint((x - min) / step) in float32 (0 when step is 0); a code stands for
 * min + code * step. 592 bytes per token for d_c = 512, d_r = 64 (1,152 in
 * bf16). mla_cache_q8_bytes_per_token: D + 16, or 0 for an invalid config or
 * when D is not a multiple of 16. */
size_t mla_cache_q8_bytes_per_token(const mla_config_t* cfg);

/* a2 into an 8-bit cache: row n is coded as above and written to the slot
 * that mla_cache_append_at picks (seq_idx[n], pos[n]); its RoPE key rotated
 * by rope_pos[n] (NULL: pos[n]) before coding (MLA_APPEND_ROTATE) or coded
 * as given (MLA_APPEND_RAW). c_kv, k_rope as for mla_cache_append (type T).
 * Errors as mla_cache_append; MLA_ERR_UNSUPPORTED when D % 16 != 0. */
mla_status_t mla_cache_append_q8(const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                                 const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                 const int32_t* rope_pos, const int32_t* page_table,
                                 int32_t batch, int32_t max_pages, void* cache_q8,
                                 int64_t num_pages, int32_t flags, void* stream);

/* a4 over an 8-bit cache: mla_decode_paged (chunk_tokens = 0) or
 * mla_decode_paged_chunked (chunk_tokens > 0), with tree_parent as in
 * mla_decode_paged_tree (NULL: the chain), reading each cached row as its
 * decoded values min + code * step. The same outputs, layouts and errors;
 * MLA_ERR_UNSUPPORTED unless bf16, d_c = 512, d_r = 64, page_size a
 * multiple of 64 and q_len * H a multiple of 16. */
mla_status_t mla_decode_paged_q8(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                 int32_t chunk_tokens, int32_t num_splits, int32_t max_seq_len,
                                 const void* q_full, const void* cache_q8, int64_t num_pages,
                                 const int32_t* page_table, int32_t max_pages,
                                 const int32_t* seq_lens, const int32_t* tree_parent,
                                 float* o_part, float* lse_part, void* stream);

/* 4-bit latent cache ("KV Cache Optimization: Scaling to Million-Token
 * Contexts", technique 3, whose listing defaults to 4 bits, and its comparison
 * table: INT4 at 4x less memory): the 8-bit cache's per-row coding with 16
 * levels, step = (max - min) / 15, code = rint((x - min) / step) in float32,
 * two codes per byte (column 2i in the low nibble of byte i, 2i + 1 in the
 * high nibble), then the same four fp32 (latent min, latent step, RoPE min,
 * RoPE step): cache_q4 [num_pages][page_size][(D / 2) + 16] bytes, 304 per
 * token for d_c = 512, d_r = 64 (1,152 in bf16, 3.79x less).
 * mla_cache_q4_bytes_per_token: D / 2 + 16, or 0 for an invalid config or
 * unless d_c and d_r are multiples of 8 and D of 32. The append and decode
 * take the arguments, checks and errors of mla_cache_append_q8 and
 * mla_decode_paged_q8 (the same kernel limits). */
size_t mla_cache_q4_bytes_per_token(const mla_config_t* cfg);
mla_status_t mla_cache_append_q4(const mla_config_t* cfg, int32_t n_tok, const void* c_kv,
                                 const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                 const int32_t* rope_pos, const int32_t* page_table,
                                 int32_t batch, int32_t max_pages, void* cache_q4,
                                 int64_t num_pages, int32_t flags, void* stream);

/* The query absorption and the coded append in one launch: the same
 * arguments, work and results (bit for bit) as
 *   mla_absorb_q(cfg, n_tok, q_nope, q_rope, pos_q, w_uk, q_full, stream);
 *   mla_cache_append_q8(cfg, n_app, c_kv, k_rope, seq_idx, pos, rope_pos,
 *                       page_table, batch, max_pages, cache_q8, num_pages,
 *                       flags, stream);      (mla_absorb_append_q4: ..._q4)
 * whose outputs are disjoint; the absorbed query of a step and its new rows
 * of an 8-bit or 4-bit cache ("KV Cache Optimization: Scaling to
 * Million-Token Contexts", technique 3). One launch when the absorption
 * runs on bf16 MFMA, the two launches otherwise. Errors as for the two
 * calls (the absorb arguments are checked first). */
mla_status_t mla_absorb_append_q8(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                                  const void* q_rope, const int32_t* pos_q, const void* w_uk,
                                  void* q_full, int32_t n_app, const void* c_kv,
                                  const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                  const int32_t* rope_pos, const int32_t* page_table,
                                  int32_t batch, int32_t max_pages, void* cache_q8,
                                  int64_t num_pages, int32_t flags, void* stream);
mla_status_t mla_absorb_append_q4(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                                  const void* q_rope, const int32_t* pos_q, const void* w_uk,
                                  void* q_full, int32_t n_app, const void* c_kv,
                                  const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                  const int32_t* rope_pos, const int32_t* page_table,
                                  int32_t batch, int32_t max_pages, void* cache_q4,
                                  int64_t num_pages, int32_t flags, void* stream);
mla_status_t mla_decode_paged_q4(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                 int32_t chunk_tokens, int32_t num_splits, int32_t max_seq_len,
                                 const void* q_full, const void* cache_q4, int64_t num_pages,
                                 const int32_t* page_table, int32_t max_pages,
                                 const int32_t* seq_lens, const int32_t* tree_parent,
                                 float* o_part, float* lse_part, void* stream);

/* Sparse read (f3; "DeepSeek's Config Says 16 KV Heads, Its Cache Holds a
 * Ninth of That", section 6 "Sparse attention"): a small scorer (the pages:
 * 64 heads of 128 dimensions) rates every cached token for each query, and
 * attention reads only the topk best (the pages: 2,048); the latent cache
 * keeps every token, next to one indexer key per token. A step runs
 *   mla_index_append   the new tokens' indexer keys into their cache
 *   mla_index_scores   I[b][j][t] for every cached token t
 *   mla_topk_select    the topk tokens each query reads
 *   mla_decode_sparse  split-KV attention over those tokens only
 * then mla_combine_up_project as for the dense decode.
 * The score is a reading (the pages give the scorer's size only):
 *   I[b][j][t] = sum_h w_idx[b][j][h] * max(0, q_idx[b][j][h] . k_idx(b, t))
 * with fp32 accumulation; a NaN dot stays NaN. */

/* Indexer keys into index_cache [num_pages][page_size][index_dim] T through
 * the page table, exactly as mla_cache_append places latent rows (pos[n]
 * picks the slot; no rotation). k_idx [n_tok][index_dim] T. index_dim a
 * multiple of 8 (bf16) or 4 (fp32), at most 1,024. Rows whose seq_idx, pos or
 * page entry is out of range are skipped. */
mla_status_t mla_index_append(const mla_config_t* cfg, int32_t index_dim, int32_t n_tok,
                              const void* k_idx, const int32_t* seq_idx, const int32_t* pos,
                              const int32_t* page_table, int32_t batch, int32_t max_pages,
                              void* index_cache, int64_t num_pages, void* stream);

/* mla_absorb_append and mla_index_append in one launch, for a sparse-read
 * step that runs all three every step: the same arguments, work and
 * results (bit for bit) as
 *   mla_absorb_append(cfg, n_tok, q_nope, q_rope, pos_q, w_uk, q_full, n_app,
 *                     c_kv, k_rope, seq_idx, pos, page_table, batch,
 *                     max_pages, cache, num_pages, flags, stream);
 *   mla_index_append(cfg, index_dim, n_app, k_idx, seq_idx, pos, page_table,
 *                    batch, max_pages, index_cache, num_pages, stream);
 * (the indexer keys k_idx [n_app][index_dim] T go to the same slots as the
 * latent rows; index_cache [num_pages][page_size][index_dim] T). One launch
 * when the absorption runs on bf16 MFMA, three launches otherwise. Errors as
 * for the calls (absorb, append, then indexer arguments). */
mla_status_t mla_absorb_append_index(const mla_config_t* cfg, int32_t n_tok, const void* q_nope,
                                     const void* q_rope, const int32_t* pos_q, const void* w_uk,
                                     void* q_full, int32_t n_app, const void* c_kv,
                                     const void* k_rope, const int32_t* seq_idx,
                                     const int32_t* pos, const int32_t* page_table,
                                     int32_t batch, int32_t max_pages, void* cache,
                                     int64_t num_pages, int32_t flags, int32_t index_dim,
                                     const void* k_idx, void* index_cache, void* stream);

/* Index scores of every cached token t < L_b for each query j:
 * scores[b][j][t] (row stride ld_scores >= max_seq_len floats) as above;
 * entries t >= L_b are not written. q_idx [batch][q_len][index_heads]
 * [index_dim] T, w_idx [batch][q_len][index_heads] f32, index_cache and
 * page_table as for mla_index_append, seq_lens [batch]. A token whose page
 * entry is invalid scores NaN; a sequence with an invalid length is not
 * written (mla_topk_select reports it). bf16 with 64 heads x 128 and a page
 * size that is a multiple of 16 runs on MFMA; other shapes need
 * index_heads * (index_dim + 1) * 4 <= 160 KiB (MLA_ERR_UNSUPPORTED
 * otherwise). index_heads in [1, 256]. */
mla_status_t mla_index_scores(const mla_config_t* cfg, int32_t index_heads, int32_t index_dim,
                              int32_t batch, int32_t q_len, int32_t max_seq_len,
                              const void* q_idx, const float* w_idx, const void* index_cache,
                              int64_t num_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens, float* scores, int32_t ld_scores,
                              void* stream);

/* The tokens each query reads: of the n = L_b - q_len + j + 1 tokens query
 * j sees, the topk with the highest scores (all n when n <= topk), equal
 * scores going to the smaller token index (-0.0 equals +0.0), written to
 * indices[b][j][0 .. count) in increasing token order, count =
 * min(topk, n) into counts[b][j]. counts[b][j] = -1 (indices unwritten)
 * when L_b is outside [q_len, max_seq_len] or a score among the n is NaN.
 * scores [batch][q_len][ld_scores] f32, indices [batch][q_len][topk] int32,
 * counts [batch][q_len] int32. 1 <= topk <= 65,536.
 * workspace: mla_topk_workspace_bytes(batch, q_len) bytes of device memory
 * that are all zero before the first call; every call leaves them all zero
 * again, so one zeroing at allocation serves every later call (calls that
 * share a workspace must not overlap). */
mla_status_t mla_topk_select(int32_t batch, int32_t q_len, int32_t max_seq_len, int32_t topk,
                             const float* scores, int32_t ld_scores, const int32_t* seq_lens,
                             void* workspace, int32_t* indices, int32_t* counts, void* stream);

/* Bytes of the workspace of mla_topk_select (per query: 4,096 histogram
 * counts and a flag); 0 for invalid arguments. */
size_t mla_topk_workspace_bytes(int32_t batch, int32_t q_len);

/* mla_index_scores followed by mla_topk_select in one call: the same scores,
 * indices and counts, the same arguments, checks and errors as those two calls
 * (workspace as for mla_topk_select). With the MFMA indexer (bf16, 64 heads
 * x 128, page size a multiple of 16) the score kernel also builds the
 * selection's histogram, one launch fewer; other shapes run the separate
 * launches. */
mla_status_t mla_index_scores_topk(const mla_config_t* cfg, int32_t index_heads,
                                   int32_t index_dim, int32_t batch, int32_t q_len,
                                   int32_t max_seq_len, const void* q_idx, const float* w_idx,
                                   const void* index_cache, int64_t num_pages,
                                   const int32_t* page_table, int32_t max_pages,
                                   const int32_t* seq_lens, float* scores, int32_t ld_scores,
                                   int32_t topk, void* workspace, int32_t* indices,
                                   int32_t* counts, void* stream);

/* mla_index_scores_topk for callers that cannot allocate device memory (code
 * under stream capture, tight serving loops, harnesses that forbid it): the
 * same arguments without `workspace`, the same scores, indices and counts
 * bit for bit. The workspace lives in a device array inside the library,
 * one per GPU, held until the process ends, sized for batch * q_len <=
 * MLA_TOPK_NOALLOC_MAX_QUERIES queries (MLA_ERR_CAPACITY beyond). The first
 * call on a device clears it with a fill kernel on `stream` (as does the
 * call after a failed launch); every selection leaves it zero. All calls on
 * one GPU share that array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller. */
enum { MLA_TOPK_NOALLOC_MAX_QUERIES = 256 };
mla_status_t mla_index_scores_topk_noalloc(const mla_config_t* cfg, int32_t index_heads,
                                           int32_t index_dim, int32_t batch, int32_t q_len,
                                           int32_t max_seq_len, const void* q_idx,
                                           const float* w_idx, const void* index_cache,
                                           int64_t num_pages, const int32_t* page_table,
                                           int32_t max_pages, const int32_t* seq_lens,
                                           float* scores, int32_t ld_scores, int32_t topk,
                                           int32_t* indices, int32_t* counts, void* stream);

/* List entries per partition of mla_decode_sparse: ceil(topk / num_splits)
 * rounded up to a multiple of 32; 0 for invalid arguments. */
int32_t mla_sparse_chunk(int32_t topk, int32_t num_splits);

/* Name of the kernel mla_decode_sparse takes: "mfma_rows16_gather" for bf16,
 * d_c = 512, d_r = 64, H a multiple of 16 and mla_sparse_chunk <= 1,984;
 * else "generic_gather"; "invalid" for invalid arguments. Static string. */
const char* mla_decode_sparse_kernel_name(const mla_config_t* cfg, int32_t topk,
                                          int32_t num_splits);

/* a4 over the selected tokens: query j of sequence b attends only over the
 * cached tokens indices[b][j][0 .. counts[b][j]) (each keeping its own
 * position; the cached RoPE keys are already rotated). Partition s covers
 * list entries [s*chunk, min(count, (s+1)*chunk)), chunk = mla_sparse_chunk;
 * the outputs, their layouts and the empty / masked conventions are those of
 * mla_decode_paged, merged the same way by mla_splitkv_combine. A query
 * whose count is outside [0, topk], or whose list holds a token it cannot
 * see (outside [0, L_b - q_len + j]) or one with an invalid page, gets NaN
 * outputs. indices, counts as written by mla_topk_select. Other arguments
 * and errors as mla_decode_paged. */
mla_status_t mla_decode_sparse(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                               int32_t topk, int32_t num_splits, int32_t max_seq_len,
                               const void* q_full, const void* cache, int64_t num_pages,
                               const int32_t* page_table, int32_t max_pages,
                               const int32_t* seq_lens, const int32_t* indices,
                               const int32_t* counts, float* o_part, float* lse_part,
                               void* stream);

/* a5. Log-sum-exp merge of the partitions ("The Architecture of Memory",
 * "Flash-Decoding and FlashInfer"), per row r = (b, j, h):
 *   LSE = ln sum_s e^(lse_s),  o_lat[r] = sum_s e^(lse_s - LSE) o_part[r][s]
 * o_part, lse_part as written by mla_decode_paged; o_lat [batch][q_len][H][d_c] T
 * (out); lse [batch][q_len][H] f32 (out, may be NULL). */
mla_status_t mla_splitkv_combine(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                 int32_t num_splits, const float* o_part, const float* lse_part,
                                 void* o_lat, float* lse, void* stream);

/* a6. Value up-projection ("Beyond the Attention Bottleneck", "Down-Projection
 * and Up-Projection Mechanics"; "DeepSeek's Config Says 16 KV Heads", section
 * 5, where the expansion is folded into the output side):
 *   out[n][h][0:d_v] = W_UV[h] o_lat[n][h]   (fp32 accumulate)
 * o_lat [n_tok][H][d_c] T, w_uv [H][d_v][d_c] T, out [n_tok][H][d_v] T. */
mla_status_t mla_up_project_v(const mla_config_t* cfg, int32_t n_tok, const void* o_lat,
                              const void* w_uv, void* out, void* stream);

/* a5 + a6 in one launch: the same arguments and results (bit for bit) as
 *   mla_splitkv_combine(cfg, batch, q_len, num_splits, o_part, lse_part,
 *                       o_lat, lse, stream);
 *   mla_up_project_v(cfg, batch * q_len, o_lat, w_uv, out, stream);
 * (o_lat is written as well). One launch for bf16 with d_c = 512, d_v = 128
 * where that is the fastest form: batch*q_len*H <= 160 with num_splits <= 32
 * (one block pair per row: small decode steps, where launch latency
 * dominates) or batch*q_len*H >= 2048 with num_splits <= 64 (one block per
 * head and 16 tokens, reading W_UV[h] once per block); the two launches
 * otherwise. */
mla_status_t mla_combine_up_project(const mla_config_t* cfg, int32_t batch, int32_t q_len,
                                    int32_t num_splits, const float* o_part,
                                    const float* lse_part, void* o_lat, float* lse,
                                    const void* w_uv, void* out, void* stream);

/* Chunked prefill in the unabsorbed form ("Beyond the Attention Bottleneck",
 * "Chunked Prefilling": the prompt enters the cache chunk by chunk, each
 * chunk's queries attending to the cache as it then stands; "Down-Projection
 * and Up-Projection Mechanics" for the per-head keys K^C = W_UK c and values
 * V = W_UV c). One sequence: its q_len newest cached tokens (already
 * appended, e.g. by mla_cache_append with MLA_APPEND_ROTATE) are the chunk,
 * query i sits at position p = seq_len - q_len + i and sees tokens t <= p.
 * Every cached latent is expanded into per-head keys and values (in the
 * workspace), then each head runs dense causal attention over 192-wide keys
 * [K^C ; RoPE key] and 128-wide values:
 *   out[i][h] = sum_t softmax_t(scale * q[i][h] . k[t][h]) V[t][h]   (d_v wide)
 *   lse[i][h] = natural log of the softmax denominator (as mla_splitkv_combine)
 * with q[i][h] = [q_nope[i][h] ; RoPE(q_rope[i][h], p)]. This is the same
 * attention as the absorbed form (the decode with q_len = C, then the merge
 * and the up-projection) without its latent output o_lat; it costs 640
 * instead of 2,176 flops per (query row, token) plus the expansion.
 * q_nope [q_len][H][d_n] bf16, q_rope [q_len][H][d_r] bf16 (unrotated), w_uk
 * [H][d_n][d_c], w_uv [H][d_v][d_c] bf16, cache as for mla_decode_paged,
 * page_row [max_pages] int32: this sequence's row of the page table (4-byte
 * alignment suffices for it),
 * workspace: mla_prefill_workspace_bytes(cfg, seq_len, q_len) bytes of device
 * memory (contents need not be initialised), out [q_len][H][d_v] bf16, lse
 * [q_len][H] f32. MLA_ERR_UNSUPPORTED unless bf16 with d_c = 512, d_r = 64,
 * d_n = d_v = 128. Tokens with an invalid page read as zero rows. */
size_t mla_prefill_workspace_bytes(const mla_config_t* cfg, int32_t seq_len, int32_t q_len);
mla_status_t mla_prefill_unabsorbed(const mla_config_t* cfg, int32_t q_len, int32_t seq_len,
                                    const void* q_nope, const void* q_rope, const void* w_uk,
                                    const void* w_uv, const void* cache, int64_t num_pages,
                                    const int32_t* page_row, int32_t max_pages,
                                    void* workspace, void* out, float* lse, void* stream);

/* Which form a prefill chunk of q_len tokens over seq_len cached tokens
 * should take: "unabsorbed" (mla_prefill_unabsorbed) when that form is
 * supported and q_len >= 1,024, where its lower flop count outweighs expanding
 * every cached token; else "absorbed" (the decode calls with q_len tokens).
 * "invalid" for invalid arguments. Static string. */
const char* mla_prefill_form(const mla_config_t* cfg, int32_t q_len, int32_t seq_len);

/* Measurement aid, not part of the decode: reads `bytes` of device memory
 * (a multiple of 16, buf 16-byte aligned) with 16-byte non-temporal loads
 * spread over `blocks` blocks of 256 threads (1 .. 65,536) and writes one
 * checksum word per block to sink [blocks] uint32, so that no load can be
 * dropped. Its rate is the HBM read rate a plain coalesced stream reaches,
 * the context for the decode kernels' fraction of the 8 TB/s peak. */
mla_status_t mla_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
