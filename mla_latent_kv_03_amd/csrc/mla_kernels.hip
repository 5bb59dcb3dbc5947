// Small kernels of the decode step (query absorption, cache append, split
// combine, value up-projection) and the generic (any-shape, fp32 or bf16)
// split-KV decode kernel. The bf16 MFMA decode kernel for the DeepSeek MLA
// shape (d_c = 512, d_r = 64) lives in mla_decode_mfma.hip.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>
#include <set>
#include <utility>

#include "mla_common.h"
#include "mla_append.h"
#include "mla_combine.h"
#include "mla_launch.h"

namespace mla {

#define HIPCHK(expr)                          \
  do {                                        \
    hipError_t e_ = (expr);                   \
    if (e_ != hipSuccess) return (int)e_;     \
  } while (0)

static inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int set_max_lds(const void* kernel, int bytes) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev})) return 0;
  HIPCHK(hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes));
  done.insert({kernel, dev});
  return 0;
}

// ---------------------------------------------------------------------------
// Drafted-token positions ("The Architecture of Memory", "Tree Attention
// Verification"): drafted token i of sequence b is cached at slot
// L_b - Q + i and positioned at L_b - Q + depth(i), its depth being 0 under
// the prefix and one more than its parent's. One 64-lane block per sequence.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void draft_positions_kernel(int Q, int max_seq_len,
                                                             const int32_t* __restrict__ seq_lens,
                                                             const int32_t* __restrict__ tree,
                                                             int32_t* __restrict__ seq_idx,
                                                             int32_t* __restrict__ slot,
                                                             int32_t* __restrict__ pos) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int L = seq_lens[b];
  const int32_t* par = tree ? tree + (size_t)b * Q : nullptr;
  bool ok = L >= Q && L <= max_seq_len;
  if (par) ok = __all(lane >= Q || tree_entry_ok(par, lane)) && ok;  // Q <= 64 with a tree
  for (int i = lane; i < Q; i += 64) {
    int d = i;
    if (par && ok) {  // a valid tree: every walk ends within i steps
      d = 0;
      for (int k = par[i]; k >= 0; k = par[k]) ++d;
    }
    const size_t n = (size_t)b * Q + i;
    seq_idx[n] = b;
    slot[n] = ok ? L - Q + i : -1;
    pos[n] = ok ? L - Q + d : -1;
  }
}

int launch_draft_positions(int batch, int q_len, int max_seq_len, const int32_t* seq_lens,
                           const int32_t* tree_parent, int32_t* seq_idx, int32_t* slot,
                           int32_t* pos, void* stream) {
  hipLaunchKernelGGL(draft_positions_kernel, dim3(batch), dim3(64), 0, as_stream(stream), q_len,
                     max_seq_len, seq_lens, tree_parent, seq_idx, slot, pos);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Streaming read for context: each block reads one contiguous chunk with
// 16-byte non-temporal loads, four per thread in flight, and XORs everything
// it read into one word (so no load can be dropped).
// ---------------------------------------------------------------------------
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_nt* __restrict__ src,
                                                          size_t n16, uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * per;
  const size_t end = beg + per < n16 ? beg + per : n16;
  u32x4_nt x = {0u, 0u, 0u, 0u};
  for (size_t i = beg + threadIdx.x; i < end; i += 4 * 256) {
    u32x4_nt v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = i + 256 * u < end ? __builtin_nontemporal_load(src + i + 256 * u) : u32x4_nt{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < 4; ++u) x ^= v[u];
  }
  uint32_t w = x.x ^ x.y ^ x.z ^ x.w;
  for (int off = 32; off > 0; off >>= 1) w ^= __shfl_xor(w, off, 64);
  __shared__ uint32_t red[4];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

int launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, as_stream(stream),
                     reinterpret_cast<const u32x4_nt*>(buf), bytes / 16, sink);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// a1: query absorption + query RoPE
// ("The Architecture of Memory", "The Weight Absorption Trick" and "Decoupled
// Rotary Positional Encoding (RoPE)")
// grid (H, ceil(n_tok / 8)), 256 threads. Each block streams W_UK[h] once and
// applies it to up to 8 tokens; thread c owns output columns c, c + 256, ...
// ---------------------------------------------------------------------------
constexpr int kAbsorbTok = 8;

template <typename T>
__global__ __launch_bounds__(256) void absorb_q_kernel(int n_tok, int H, int dn, int dc, int dr,
                                                       double log2_base, const T* __restrict__ q_nope,
                                                       const T* __restrict__ q_rope,
                                                       const int32_t* __restrict__ pos,
                                                       const T* __restrict__ w_uk,
                                                       T* __restrict__ q_full) {
  __shared__ float qs[kAbsorbTok][256];
  const int h = blockIdx.x;
  const int n0 = blockIdx.y * kAbsorbTok;
  const int nt = min(kAbsorbTok, n_tok - n0);
  const int D = dc + dr;
  for (int i = threadIdx.x; i < kAbsorbTok * dn; i += blockDim.x) {
    const int n = i / dn, k = i % dn;
    qs[n][k] = n < nt ? Elt<T>::ld(q_nope + ((size_t)(n0 + n) * H + h) * dn + k) : 0.0f;
  }
  __syncthreads();
  const T* W = w_uk + (size_t)h * dn * dc;
  for (int c = threadIdx.x; c < dc; c += blockDim.x) {
    float acc[kAbsorbTok];
#pragma unroll
    for (int n = 0; n < kAbsorbTok; ++n) acc[n] = 0.0f;
    for (int k = 0; k < dn; ++k) {
      const float w = Elt<T>::ld(W + (size_t)k * dc + c);
#pragma unroll
      for (int n = 0; n < kAbsorbTok; ++n) acc[n] = fmaf(qs[n][k], w, acc[n]);
    }
    for (int n = 0; n < nt; ++n) Elt<T>::st(q_full + ((size_t)(n0 + n) * H + h) * D + c, acc[n]);
  }
  const int half = dr / 2;
  for (int i = threadIdx.x; i < nt * half; i += blockDim.x) {
    const int n = i / half, p = i % half;
    const T* src = q_rope + ((size_t)(n0 + n) * H + h) * dr + 2 * p;
    double y0, y1;
    rope_pair(Elt<T>::ld(src), Elt<T>::ld(src + 1), pos[n0 + n], p, dr, log2_base, &y0, &y1);
    T* dst = q_full + ((size_t)(n0 + n) * H + h) * D + dc + 2 * p;
    Elt<T>::st(dst, (float)y0);
    Elt<T>::st(dst + 1, (float)y1);
  }
}

template <typename T>
static int absorb_impl(const Shape& s, int n_tok, const void* q_nope, const void* q_rope,
                       const int32_t* pos, const void* w_uk, void* q_full, void* stream) {
  dim3 grid(s.H, (n_tok + kAbsorbTok - 1) / kAbsorbTok);
  hipLaunchKernelGGL(absorb_q_kernel<T>, grid, dim3(256), 0, as_stream(stream), n_tok, s.H, s.dn,
                     s.dc, s.dr, s.log2_base, (const T*)q_nope, (const T*)q_rope, pos,
                     (const T*)w_uk, (T*)q_full);
  return (int)hipGetLastError();
}

bool absorb_mfma_ok(const Shape& s);
int launch_absorb_q_mfma(const Shape& s, int n_tok, const void* q_nope, const void* q_rope,
                         const int32_t* pos, const void* w_uk, void* q_full, void* stream);
bool up_v_mfma_ok(const Shape& s);
int launch_up_project_v_mfma(const Shape& s, int n_tok, const void* o_lat, const void* w_uv,
                             void* out, void* stream);

int launch_absorb_q(const Shape& s, int n_tok, const void* q_nope, const void* q_rope,
                    const int32_t* pos, const void* w_uk, void* q_full, void* stream) {
  if (absorb_mfma_ok(s))
    return launch_absorb_q_mfma(s, n_tok, q_nope, q_rope, pos, w_uk, q_full, stream);
  return s.dtype == 0 ? absorb_impl<float>(s, n_tok, q_nope, q_rope, pos, w_uk, q_full, stream)
                      : absorb_impl<bf16_t>(s, n_tok, q_nope, q_rope, pos, w_uk, q_full, stream);
}

// ---------------------------------------------------------------------------
// a2: paged cache append: one block per appended row (append_row, shared with
// the launch that fuses it with query absorption).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(128) void append_kernel(int dc, int dr, int page,
                                                     const T* __restrict__ c_kv,
                                                     const T* __restrict__ k_rope,
                                                     const int32_t* __restrict__ seq_idx,
                                                     const int32_t* __restrict__ pos,
                                                     const int32_t* __restrict__ rope_pos,
                                                     const int32_t* __restrict__ page_table,
                                                     int batch, int max_pages, T* __restrict__ cache,
                                                     int64_t num_pages, int rotate, double log2_base,
                                                     int vec) {
  append_row<T>(blockIdx.x, dc, dr, page, c_kv, k_rope, seq_idx, pos, rope_pos, page_table, batch,
                max_pages, cache, num_pages, rotate, log2_base, vec);
}

int launch_cache_append(const Shape& s, int n_tok, const void* c_kv, const void* k_rope,
                        const int32_t* seq_idx, const int32_t* pos, const int32_t* rope_pos,
                        const int32_t* page_table, int batch, int max_pages, void* cache,
                        int64_t num_pages, int rotate, void* stream) {
  const int vec = append_vectorizable(s, c_kv, cache);
  if (s.dtype == 0)
    hipLaunchKernelGGL(append_kernel<float>, dim3(n_tok), dim3(128), 0, as_stream(stream), s.dc,
                       s.dr, s.page, (const float*)c_kv, (const float*)k_rope, seq_idx, pos,
                       rope_pos, page_table, batch, max_pages, (float*)cache, num_pages, rotate,
                       s.log2_base, vec);
  else
    hipLaunchKernelGGL(append_kernel<bf16_t>, dim3(n_tok), dim3(128), 0, as_stream(stream), s.dc,
                       s.dr, s.page, (const bf16_t*)c_kv, (const bf16_t*)k_rope, seq_idx, pos,
                       rope_pos, page_table, batch, max_pages, (bf16_t*)cache, num_pages, rotate,
                       s.log2_base, vec);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// a4 (generic): split-KV decode for any supported shape, fp32 or bf16, on the
// vector ALUs. Block = (partition s, sequence b, group of 8 query rows).
// Tokens are staged 16 at a time in LDS (as fp32, rows padded to an odd
// stride); scores use one thread per (row, token); the online softmax keeps a
// running max m and sum l per row; thread f accumulates output columns
// f, f + 256, ... of all rows.
// kGather (sparse read, "DeepSeek's Config Says 16 KV Heads", section 6): the
// partition is a slice of its query's list of selected tokens; a block's rows
// are heads of one query, and each staged token is looked up through the list
// and the page table.
// ---------------------------------------------------------------------------
constexpr int kGenRows = 8;
constexpr int kGenTok = 16;
constexpr int kGenMaxF = 4;  // d_c <= 1024

template <typename T, bool kGather>
__global__ __launch_bounds__(256) void decode_generic_kernel(
    int Q, int H, int dc, int dr, int page, int S, int fixed, int max_seq_len, float scale,
    const T* __restrict__ q_full, const T* __restrict__ cache, int64_t num_pages,
    const int32_t* __restrict__ page_table, int max_pages, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ tree_parent, const int32_t* __restrict__ sel_idx,
    const int32_t* __restrict__ sel_cnt, int topk, float* __restrict__ o_part,
    float* __restrict__ lse_part) {
  extern __shared__ float smem[];
  const int s = blockIdx.x, b = blockIdx.y;
  const int R = Q * H;
  int r0, nr, jq = 0;  // jq: the block's query (gather)
  if constexpr (kGather) {
    const int hg = (H + kGenRows - 1) / kGenRows;
    jq = blockIdx.z / hg;
    r0 = jq * H + (blockIdx.z % hg) * kGenRows;
    nr = min(kGenRows, (jq + 1) * H - r0);
  } else {
    r0 = blockIdx.z * kGenRows;
    nr = min(kGenRows, R - r0);
  }
  const int D = dc + dr, Dp = D + 1;
  float* qs = smem;                    // [kGenRows][D]
  float* cs = qs + kGenRows * D;       // [kGenTok][Dp]
  float* ps = cs + kGenTok * Dp;       // [kGenRows][kGenTok]
  float* al = ps + kGenRows * kGenTok; // [kGenRows] rescale factors
  int64_t* rs = reinterpret_cast<int64_t*>(al + 2 * kGenRows);  // [kGenTok] gathered rows
  const int tid = threadIdx.x;

  const int L = seq_lens[b];
  bool bad = (L < Q) || (L > max_seq_len);
  const int32_t* par = (!kGather && tree_parent) ? tree_parent + (size_t)b * Q : nullptr;
  if (par) {  // every thread checks every entry: the decision is block-uniform
    for (int i = 0; i < Q; ++i) bad |= !tree_entry_ok(par, i);
  }
  int t0 = 0, t1 = 0;  // tokens (gather: list entries) of this partition
  const int32_t* lst = nullptr;
  if constexpr (kGather) {
    const int cnt = sel_cnt[(size_t)b * Q + jq];
    bad = bad || cnt < 0 || cnt > topk;
    lst = sel_idx + ((size_t)b * Q + jq) * topk;
    if (!bad) {
      t0 = min(s * fixed, cnt);
      t1 = min(t0 + fixed, cnt);
    }
  } else {
    if (!bad) split_range(L, S, page, fixed, s, &t0, &t1);
  }

  for (int i = tid; i < nr * D; i += blockDim.x)
    qs[i] = Elt<T>::ld(q_full + ((size_t)b * R + r0) * D + i);

  float acc[kGenRows][kGenMaxF];
#pragma unroll
  for (int r = 0; r < kGenRows; ++r)
#pragma unroll
    for (int k = 0; k < kGenMaxF; ++k) acc[r][k] = 0.0f;
  // per-row softmax state, replicated in the 16 threads of the row
  const int my_r = tid / kGenTok, my_k = tid % kGenTok;
  float m_run = -INFINITY, l_run = 0.0f;
  const int my_j = (r0 + my_r) / H;   // query index of this thread's row
  // tokens this row sees: t <= lim, and with a drafted tree also the drafted
  // tokens (t >= L - Q) on its branch
  const int t_draft = L - Q;  // first drafted token
  const int lim = kGather ? t1 - 1 : (par ? t_draft - 1 : t_draft + my_j);
  const uint64_t branch = (par && !bad && my_j < Q) ? tree_branch_mask(par, Q, my_j) : 0ull;

  // a chain stops after the last token the block's last query sees
  const int t_end = kGather ? t1 : t0 + kGenTok * tiles_needed(t0, t1, kGenTok, par != nullptr,
                                                                  L - Q, (r0 + nr - 1) / H);
  for (int t = t0; t < t_end && !bad; t += kGenTok) {
    const int nt = min(kGenTok, t1 - t);
    if constexpr (kGather) {
      __syncthreads();  // previous step done with cs / ps / al / rs
      if (tid < nt) {   // list entry -> cache row; -1 when not visible or its page is invalid
        const int tk = lst[t + tid];
        const int pg =
            (tk >= 0 && tk <= L - Q + jq) ? page_table[(size_t)b * max_pages + tk / page] : -1;
        rs[tid] = (pg < 0 || (int64_t)pg >= num_pages) ? -1 : (int64_t)pg * page + tk % page;
      }
      __syncthreads();
      bool badrow = false;  // every thread reads every entry: block-uniform
      for (int u = 0; u < nt; ++u) badrow |= rs[u] < 0;
      if (badrow) {
        bad = true;
        break;
      }
      for (int i = tid; i < nt * D; i += blockDim.x)
        cs[(i / D) * Dp + (i % D)] = Elt<T>::ld(cache + rs[i / D] * D + (i % D));
      __syncthreads();
    } else {
      const int pg = page_table[(size_t)b * max_pages + t / page];
      if (pg < 0 || (int64_t)pg >= num_pages) {
        bad = true;  // uniform across the block: every thread read the same entry
        break;
      }
      __syncthreads();  // previous step done with cs / ps / al
      const T* src = cache + ((size_t)pg * page + (t % page)) * D;
      for (int i = tid; i < nt * D; i += blockDim.x)
        cs[(i / D) * Dp + (i % D)] = Elt<T>::ld(src + i);
      __syncthreads();
    }
    float sc = -INFINITY;
    const bool seen = (tile_visible(t, lim, t_draft, t1, branch) >> my_k) & 1ull;
    if (my_r < nr && my_k < nt && seen) {
      const float* qr = qs + my_r * D;
      const float* cr = cs + my_k * Dp;
      float dot = 0.0f;
      for (int f = 0; f < D; ++f) dot = fmaf(qr[f], cr[f], dot);
      sc = dot * scale;
    }
    float mx = sc;
    for (int off = kGenTok / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kGenTok));
    const float m_new = fmaxf(m_run, mx);
    const float p = (sc == -INFINITY) ? 0.0f : expf(sc - m_new);
    float ps_sum = p;
    for (int off = kGenTok / 2; off > 0; off >>= 1) ps_sum += __shfl_xor(ps_sum, off, kGenTok);
    const float alpha = (m_new == -INFINITY) ? 1.0f : expf(m_run - m_new);
    l_run = l_run * alpha + ps_sum;
    m_run = m_new;
    if (my_r < kGenRows) {
      ps[my_r * kGenTok + my_k] = p;
      if (my_k == 0) al[my_r] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kGenRows; ++r) {
      if (r < nr) {
        const float a = al[r];
#pragma unroll
        for (int k = 0; k < kGenMaxF; ++k) {
          const int f = tid + 256 * k;
          if (f < dc) {
            float v = acc[r][k] * a;
            for (int u = 0; u < nt; ++u) v = fmaf(ps[r * kGenTok + u], cs[u * Dp + f], v);
            acc[r][k] = v;
          }
        }
      }
    }
  }
  // final: broadcast each row's (m, l) through LDS, then write the partials
  __syncthreads();
  if (my_k == 0 && my_r < kGenRows) {
    ps[my_r * 2] = m_run;
    ps[my_r * 2 + 1] = l_run;
  }
  __syncthreads();
  const float nanv = __int_as_float(0x7fc00000);
  for (int r = 0; r < nr; ++r) {
    const float m = ps[r * 2], l = ps[r * 2 + 1];
    const size_t row = (size_t)b * R + r0 + r;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int k = 0; k < kGenMaxF; ++k) {
      const int f = tid + 256 * k;
      // an empty partition (no tokens) leaves its o_part row unwritten
      if (f < dc && (t1 > t0 || bad)) o_part[(row * S + s) * dc + f] = bad ? nanv : acc[r][k] * inv;
    }
    if (tid == 0) lse_part[row * S + s] = bad ? nanv : (l > 0.0f ? m + logf(l) : -INFINITY);
  }
}

// dynamic LDS of the generic decode: queries, staged tokens, P, rescale
// factors (2 x kGenRows floats keep what follows 8-byte aligned) and the
// gathered row numbers
static size_t generic_lds_bytes(int D) {
  return sizeof(float) * ((size_t)kGenRows * D + (size_t)kGenTok * (D + 1) + kGenRows * kGenTok +
                          2 * kGenRows) +
         sizeof(int64_t) * kGenTok;
}

template <typename T>
static int decode_generic_impl(const Shape& s, int batch, int q_len, int num_splits,
                               int max_seq_len, const void* q_full, const void* cache,
                               int64_t num_pages, const int32_t* page_table, int max_pages,
                               const int32_t* seq_lens, const int32_t* tree_parent, float* o_part,
                               float* lse_part, void* stream) {
  const int D = s.D();
  if (int e = set_max_lds((const void*)decode_generic_kernel<T, false>, 160 * 1024)) return e;
  const int R = q_len * s.H;
  dim3 grid(num_splits, batch, (R + kGenRows - 1) / kGenRows);
  hipLaunchKernelGGL((decode_generic_kernel<T, false>), grid, dim3(256), generic_lds_bytes(D),
                     as_stream(stream), q_len, s.H, s.dc, s.dr, s.page, num_splits, s.split_fixed,
                     max_seq_len, s.scale, (const T*)q_full, (const T*)cache, num_pages,
                     page_table, max_pages, seq_lens, tree_parent, nullptr, nullptr, 0, o_part,
                     lse_part);
  return (int)hipGetLastError();
}

template <typename T>
static int decode_sparse_generic_impl(const Shape& s, int batch, int q_len, int topk, int chunk,
                                      int num_splits, int max_seq_len, const void* q_full,
                                      const void* cache, int64_t num_pages,
                                      const int32_t* page_table, int max_pages,
                                      const int32_t* seq_lens, const int32_t* sel_idx,
                                      const int32_t* sel_cnt, float* o_part, float* lse_part,
                                      void* stream) {
  if (int e = set_max_lds((const void*)decode_generic_kernel<T, true>, 160 * 1024)) return e;
  dim3 grid(num_splits, batch, q_len * ((s.H + kGenRows - 1) / kGenRows));
  hipLaunchKernelGGL((decode_generic_kernel<T, true>), grid, dim3(256), generic_lds_bytes(s.D()),
                     as_stream(stream), q_len, s.H, s.dc, s.dr, s.page, num_splits, chunk,
                     max_seq_len, s.scale, (const T*)q_full, (const T*)cache, num_pages,
                     page_table, max_pages, seq_lens, nullptr, sel_idx, sel_cnt, topk, o_part,
                     lse_part);
  return (int)hipGetLastError();
}

bool decode_sparse_rows16_ok(const Shape& s, int chunk);
int launch_decode_sparse_rows16(const Shape& s, int batch, int q_len, int topk, int chunk,
                                int num_splits, int max_seq_len, const void* q_full,
                                const void* cache, int64_t num_pages, const int32_t* page_table,
                                int max_pages, const int32_t* seq_lens, const int32_t* sel_idx,
                                const int32_t* sel_cnt, float* o_part, float* lse_part,
                                void* stream);

int decode_sparse_kind(const Shape& s, int chunk) { return decode_sparse_rows16_ok(s, chunk) ? 1 : 0; }

int launch_decode_sparse(const Shape& s, int batch, int q_len, int topk, int chunk, int num_splits,
                         int max_seq_len, const void* q_full, const void* cache, int64_t num_pages,
                         const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                         const int32_t* sel_idx, const int32_t* sel_cnt, float* o_part,
                         float* lse_part, void* stream) {
  if (decode_sparse_kind(s, chunk) == 1)
    return launch_decode_sparse_rows16(s, batch, q_len, topk, chunk, num_splits, max_seq_len,
                                       q_full, cache, num_pages, page_table, max_pages, seq_lens,
                                       sel_idx, sel_cnt, o_part, lse_part, stream);
  return s.dtype == 0
             ? decode_sparse_generic_impl<float>(s, batch, q_len, topk, chunk, num_splits,
                                                 max_seq_len, q_full, cache, num_pages, page_table,
                                                 max_pages, seq_lens, sel_idx, sel_cnt, o_part,
                                                 lse_part, stream)
             : decode_sparse_generic_impl<bf16_t>(s, batch, q_len, topk, chunk, num_splits,
                                                  max_seq_len, q_full, cache, num_pages,
                                                  page_table, max_pages, seq_lens, sel_idx,
                                                  sel_cnt, o_part, lse_part, stream);
}

bool decode_rows16_ok(const Shape& s, int q_len);
int launch_decode_rows16(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                         const void* q_full, const void* cache, int64_t num_pages,
                         const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                         const int32_t* tree_parent, float* o_part, float* lse_part,
                         void* stream);
bool decode_ws_ok(const Shape& s, int q_len);
int launch_decode_ws(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                     const void* q_full, const void* cache, int64_t num_pages,
                     const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                     const int32_t* tree_parent, float* o_part, float* lse_part, void* stream);

// bf16 MFMA kernels for the 576-wide DeepSeek row: 64 query rows per block
// (specialised QK and PV waves) when the row count and page size allow it,
// else 16; everything else takes the generic kernel
int decode_kernel_kind(const Shape& s, int q_len) {
  if (decode_ws_ok(s, q_len)) return 2;
  if (decode_rows16_ok(s, q_len)) return 1;
  return 0;
}

int launch_decode(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                  const void* q_full, const void* cache, int64_t num_pages,
                  const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                  const int32_t* tree_parent, float* o_part, float* lse_part, void* stream) {
  switch (decode_kernel_kind(s, q_len)) {
    case 2:
      return launch_decode_ws(s, batch, q_len, num_splits, max_seq_len, q_full, cache, num_pages,
                              page_table, max_pages, seq_lens, tree_parent, o_part, lse_part,
                              stream);
    case 1:
      return launch_decode_rows16(s, batch, q_len, num_splits, max_seq_len, q_full, cache,
                                  num_pages, page_table, max_pages, seq_lens, tree_parent, o_part,
                                  lse_part, stream);
    default:
      break;
  }
  return s.dtype == 0
             ? decode_generic_impl<float>(s, batch, q_len, num_splits, max_seq_len, q_full, cache,
                                          num_pages, page_table, max_pages, seq_lens, tree_parent,
                                          o_part, lse_part, stream)
             : decode_generic_impl<bf16_t>(s, batch, q_len, num_splits, max_seq_len, q_full, cache,
                                           num_pages, page_table, max_pages, seq_lens, tree_parent,
                                           o_part, lse_part, stream);
}

// ---------------------------------------------------------------------------
// a5: log-sum-exp merge of the partitions ("The Architecture of Memory",
// "Flash-Decoding and FlashInfer"). One wave per (output row, 256 latent
// columns); the arithmetic is in mla_combine.h, shared with the launch that
// fuses the merge with the value up-projection.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(64) void combine_kernel(int S, int dc, const float* __restrict__ o_part,
                                                     const float* __restrict__ lse_part,
                                                     T* __restrict__ o_lat, float* __restrict__ lse) {
  __shared__ float w[kMaxSplits];
  const int r = blockIdx.x, lane = threadIdx.x;
  const int col = blockIdx.y * kCombCols + 4 * lane;
  CombineCols<> cc;
  cc.start(o_part + (size_t)r * S * dc, S, dc, col);
  const CombineWeights cw = combine_weights(lse_part + (size_t)r * S, S, w, lane);
  __syncthreads();
  const float4 v = cc.finish(w, cw, lane);
  if (col < dc) store4<T>(o_lat + (size_t)r * dc + col, v);
  if (lse && blockIdx.y == 0 && lane == 0) lse[r] = cw.lse();
}

int launch_combine(const Shape& s, int rows, int num_splits, const float* o_part,
                   const float* lse_part, void* o_lat, float* lse, void* stream) {
  dim3 grid(rows, (s.dc + kCombCols - 1) / kCombCols);
  if (s.dtype == 0)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(64), 0, as_stream(stream), num_splits,
                       s.dc, o_part, lse_part, (float*)o_lat, lse);
  else
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(64), 0, as_stream(stream), num_splits,
                       s.dc, o_part, lse_part, (bf16_t*)o_lat, lse);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// a6: value up-projection through W_UV ("Beyond the Attention Bottleneck",
// "Down-Projection and Up-Projection Mechanics").
// grid (H, ceil(n_tok / 8)), 4 waves; wave w computes output rows v = w,
// w + 4, ... for up to 8 tokens: lanes stride the d_c axis, then a wave
// reduction.
// ---------------------------------------------------------------------------
constexpr int kUpTok = 8;

template <typename T>
__global__ __launch_bounds__(256) void up_v_kernel(int n_tok, int H, int dc, int dv,
                                                   const T* __restrict__ o_lat,
                                                   const T* __restrict__ w_uv, T* __restrict__ out) {
  __shared__ float os[kUpTok][1024];
  const int h = blockIdx.x;
  const int n0 = blockIdx.y * kUpTok;
  const int nt = min(kUpTok, n_tok - n0);
  for (int i = threadIdx.x; i < kUpTok * dc; i += blockDim.x) {
    const int n = i / dc, c = i % dc;
    os[n][c] = n < nt ? Elt<T>::ld(o_lat + ((size_t)(n0 + n) * H + h) * dc + c) : 0.0f;
  }
  __syncthreads();
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const T* W = w_uv + (size_t)h * dv * dc;
  for (int v = wave; v < dv; v += 4) {
    float acc[kUpTok];
#pragma unroll
    for (int n = 0; n < kUpTok; ++n) acc[n] = 0.0f;
    for (int c = lane; c < dc; c += 64) {
      const float w = Elt<T>::ld(W + (size_t)v * dc + c);
#pragma unroll
      for (int n = 0; n < kUpTok; ++n) acc[n] = fmaf(w, os[n][c], acc[n]);
    }
#pragma unroll
    for (int n = 0; n < kUpTok; ++n)
      for (int off = 32; off > 0; off >>= 1) acc[n] += __shfl_xor(acc[n], off, 64);
    if (lane == 0)
      for (int n = 0; n < nt; ++n) Elt<T>::st(out + ((size_t)(n0 + n) * H + h) * dv + v, acc[n]);
  }
}

int launch_up_project_v(const Shape& s, int n_tok, const void* o_lat, const void* w_uv,
                        void* out, void* stream) {
  if (up_v_mfma_ok(s)) return launch_up_project_v_mfma(s, n_tok, o_lat, w_uv, out, stream);
  dim3 grid(s.H, (n_tok + kUpTok - 1) / kUpTok);
  if (s.dtype == 0)
    hipLaunchKernelGGL(up_v_kernel<float>, grid, dim3(256), 0, as_stream(stream), n_tok, s.H, s.dc,
                       s.dv, (const float*)o_lat, (const float*)w_uv, (float*)out);
  else
    hipLaunchKernelGGL(up_v_kernel<bf16_t>, grid, dim3(256), 0, as_stream(stream), n_tok, s.H,
                       s.dc, s.dv, (const bf16_t*)o_lat, (const bf16_t*)w_uv, (bf16_t*)out);
  return (int)hipGetLastError();
}

}  // namespace mla
