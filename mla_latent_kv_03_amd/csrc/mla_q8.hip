// 8-bit latent cache (gfx950): quantizing append and split-KV decode.
//
// A cached row is coded per token in 8 bits between its own minimum and
// maximum ("KV Cache Optimization: Scaling to Million-Token Contexts",
// technique 3 "KV Cache Quantization": an INT8 cache halves the bytes),
// separately for the latent part (d_c) and the rotated RoPE part (d_r):
//   row = [codes uint8 x (d_c + d_r)][lat_min, lat_step, rope_min, rope_step f32]
// 592 bytes for the DeepSeek row (512 + 64 + 16) against 1,152 in bf16. The
// step is (max - min) / 255 and a value's code is rint((x - min) / step) in
// float32 (IEEE division, ties to even), 0 for a constant part; a code stands
// for min + code * step.
//
// The decode kernel is the 16-row split-KV kernel of the bf16 cache (one
// staged tile shared by all 16 query rows, one block barrier per tile, QK of
// tile k+1 beside P.C of tile k) on 64-token tiles: a tile is one contiguous
// 37,888-byte copy (37 direct-to-LDS loads), rows 592 bytes apart, a stride
// at which both operand read patterns below are free of LDS bank conflicts.
// A wave64 vector instruction occupies the SIMD for 4 cycles, so the codes
// are not decoded element by element: the MFMAs take them as the fp16 values
// 1024 + code (one v_perm per two), and the code -> value map is applied per
// score and per output row (see decode_q8_kernel):
//   QK  wave w scores the 16 tokens [16 w, 16 w + 16) of the tile over all
//       576 columns (18 v_mfma_f32_16x16x32_f16; A = 8 codes of one token
//       per lane, B = the query row in fp16 registers) and leaves S^T in LDS
//   max every wave reads the four subtiles' scores, takes the row max over
//       the 64 tokens and forms P (the lazy rescale of the bf16 kernel)
//   PV  wave w accumulates latent columns [128 w, 128 w + 128) of all 16
//       rows, two K = 32 blocks per tile; the B operand takes 4 codes of each
//       of its 8 tokens (ds_read_b32), interleaved and lifted by v_perm.
#include "mla_append.h"
#include "mla_decode_common.h"
#include "mla_launch.h"

namespace mla {

using namespace dec;

// ---------------------------------------------------------------------------
// Quantizing append: one block of 128 threads per row.
// ---------------------------------------------------------------------------
namespace {

constexpr int kQ8Meta = 16;  // bytes of per-row metadata (4 fp32)

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

// code of x on [mn, mn + 255 step]: rint((x - mn) / step) in float32
__device__ __forceinline__ uint32_t q8_code(float x, float mn, float step) {
  if (step == 0.0f) return 0u;
  const float c = rintf((x - mn) / step);
  return (uint32_t)fminf(fmaxf(c, 0.0f), 255.0f);
}

}  // namespace

template <typename T>
__global__ __launch_bounds__(128) void append_q8_kernel(
    int dc, int dr, int page, const T* __restrict__ c_kv, const T* __restrict__ k_rope,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ rope_pos, const int32_t* __restrict__ page_table, int batch,
    int max_pages, uint8_t* __restrict__ cache, int64_t num_pages, int rotate, double log2_base) {
  __shared__ float red[2];
  __shared__ float kr[256];  // the (rotated) RoPE part in float32, d_r <= 256
  const int n = blockIdx.x, tid = threadIdx.x;
  const int b = seq_idx[n];
  const int p = pos[n];
  if (b < 0 || b >= batch || p < 0 || p >= max_pages * page) return;  // block-uniform
  const int pg = page_table[(size_t)b * max_pages + p / page];
  if (pg < 0 || (int64_t)pg >= num_pages) return;
  const int D = dc + dr;
  uint8_t* row = cache + ((size_t)pg * page + p % page) * (size_t)(D + kQ8Meta);
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
  const float lstep = (lmx - lmn) / 255.0f;
  for (int i = 4 * tid; i < dc; i += 4 * blockDim.x) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= q8_code(Elt<T>::ld(src + i + j), lmn, lstep) << (8 * j);
    *reinterpret_cast<uint32_t*>(row + i) = w;
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
  const float rstep = (rmx - rmn) / 255.0f;
  for (int i = 4 * tid; i < dr; i += 4 * blockDim.x) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= q8_code(kr[i + j], rmn, rstep) << (8 * j);
    *reinterpret_cast<uint32_t*>(row + dc + i) = w;
  }
  if (tid == 0)
    *reinterpret_cast<float4*>(row + D) = make_float4(lmn, lstep, rmn, rstep);
}

int launch_cache_append_q8(const Shape& s, int n_tok, const void* c_kv, const void* k_rope,
                           const int32_t* seq_idx, const int32_t* pos, const int32_t* rope_pos,
                           const int32_t* page_table, int batch, int max_pages, void* cache,
                           int64_t num_pages, int rotate, void* stream) {
  if (s.dtype == 0)
    hipLaunchKernelGGL(append_q8_kernel<float>, dim3(n_tok), dim3(128), 0,
                       reinterpret_cast<hipStream_t>(stream), s.dc, s.dr, s.page,
                       (const float*)c_kv, (const float*)k_rope, seq_idx, pos, rope_pos,
                       page_table, batch, max_pages, (uint8_t*)cache, num_pages, rotate,
                       s.log2_base);
  else
    hipLaunchKernelGGL(append_q8_kernel<bf16_t>, dim3(n_tok), dim3(128), 0,
                       reinterpret_cast<hipStream_t>(stream), s.dc, s.dr, s.page,
                       (const bf16_t*)c_kv, (const bf16_t*)k_rope, seq_idx, pos, rope_pos,
                       page_table, batch, max_pages, (uint8_t*)cache, num_pages, rotate,
                       s.log2_base);
  return (int)hipGetLastError();
}

// ---------------------------------------------------------------------------
// Decode over the 8-bit cache, 16 query rows per block.
// ---------------------------------------------------------------------------
namespace {

constexpr int kQRow = kD + kQ8Meta;                 // 592 bytes per cached row
constexpr int kQT = 64;                             // tokens per tile
constexpr int kQTileBytes = kQT * kQRow;            // 37,888
constexpr int kQRing = 4;
constexpr int kQQLoads = 8 * kChunks / 64;          // 9 loads: 8 query rows of 1,152 B
constexpr size_t kQRingBytes = (size_t)kQRing * kQTileBytes;  // 151,552
constexpr size_t kQScoreBytes = (size_t)2 * kWaves * 64 * 16; // 8,192
constexpr size_t kQLds = kQRingBytes + kQScoreBytes;         // 159,744

static_assert(kQTileBytes % 1024 == 0, "a tile is whole 1 KB loads");
static_assert(kQLds + 256 <= 160 * 1024, "LDS of one CU");
static_assert(8 * kChunks * 16 <= kQTileBytes, "the query rows fit a ring slot");

// tile loads of wave w: [first, first + count), 10 + 9 + 9 + 9
__device__ __forceinline__ int q8_first_load(int w) { return w == 0 ? 0 : 1 + 9 * w; }
__device__ __forceinline__ int q8_load_count(int w) { return w == 0 ? 10 : 9; }

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
constexpr uint32_t kF16Hi = 0x64646464u;  // high byte of the fp16 value 1024 + v, v < 256

// 4 codes (one dword) -> the fp16 values 1024 + code, two per dword: one
// v_perm each places a code under the 0x64 exponent byte (bytes 0..3 of the
// selector's space are c, bytes 4..7 the constant)
__device__ __forceinline__ u32x2_t codes_f16(uint32_t c) {
  return u32x2_t{__builtin_amdgcn_perm(kF16Hi, c, 0x04010400u),
                 __builtin_amdgcn_perm(kF16Hi, c, 0x04030402u)};
}
__device__ __forceinline__ f16x8_t codes8_f16(u32x2_t c) {
  const u32x2_t lo = codes_f16(c.x), hi = codes_f16(c.y);
  return __builtin_bit_cast(f16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
}

}  // namespace

// The contractions run on fp16 MFMA over the values 1024 + code (exact in
// fp16, and one v_perm per two of them), and the affine code -> value map is
// applied per score and per output row instead of per element:
//   score: q . (min + step c) = step (q . (1024 + c)) + (min - 1024 step) sum q
//          per part (latent, RoPE), each with its own accumulator
//   P.C:   sum_t p_t (min_t + step_t c_t)
//            = sum_t P_t (1024 + c_t) + sum_t p_t min_t - 1024 sum_t P_t,
//          P_t = fp16(p_t step_t), the A operand; sum_t P_t of exactly those
//          fp16 values comes from one more MFMA against an all-ones operand
// The query rows are converted to fp16 once per block (exact for bf16 values
// within fp16 range).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_q8_kernel(int Q, int H, int S, int page, int fixed, int max_seq_len,
                      float scale_log2, int units, int groups, const bf16_t* __restrict__ q_full,
                      const uint8_t* __restrict__ cache, int64_t num_pages,
                      const int32_t* __restrict__ page_table, int max_pages,
                      const int32_t* __restrict__ seq_lens,
                      const int32_t* __restrict__ tree_parent, float* __restrict__ o_part,
                      float* __restrict__ lse_part) {
  extern __shared__ u32x4_t lds[];
  int unit, grp;
  if (!map_block(units, groups, &unit, &grp)) return;
  const int R = Q * H;
  const int row0 = grp * 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15, kg = lane >> 4;
  const int s = unit % S;
  int L;
  const int b = seq_by_rank(seq_lens, units / S, unit / S, lane, &L);
  const int32_t* par = tree_parent ? tree_parent + (size_t)b * Q : nullptr;
  const bool bad_tree = par && !__all(lane >= Q || tree_entry_ok(par, lane));
  const bool bad_len = (L < Q) || (L > max_seq_len) || bad_tree;
  int t0 = 0, t1 = 0;
  if (!bad_len) split_range(L, S, page, fixed, s, &t0, &t1);
  const int ntiles = tiles_needed(t0, t1, kQT, par != nullptr, L - Q, (row0 + 15) / H);
  bool bad = bad_len;

  char* const lbase = reinterpret_cast<char*>(lds);
  f32x4_t* sc = reinterpret_cast<f32x4_t*>(lbase + kQRingBytes);
  auto slot = [&](int k) { return lbase + (k & (kQRing - 1)) * kQTileBytes; };

  PageWindow pw;
  pw.init(page_table + (size_t)b * max_pages + t0 / page, (t1 - t0 + page - 1) / page, lane);
  settle(pw.reg);
  const int l0 = q8_first_load(wave), lc = q8_load_count(wave);
  // this wave's loads of tile k: tile bytes [1024 i, 1024 i + 1024), i in
  // [l0, l0 + lc); a tile never crosses a page (64 | page)
  auto issue = [&](int k) {
    const int t = t0 + k * kQT;
    int pg = pw.get((t - t0) / page, lane);
    if (pg < 0 || (int64_t)pg >= num_pages) {
      bad = true;
      pg = 0;
    }
    const uint8_t* src = cache + ((size_t)pg * page + (t % page)) * (size_t)kQRow;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(slot(k)));
    for (int i = l0; i < l0 + lc; ++i)  // wave-uniform bounds
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                   :
                   : "s"(dst + i * 1024), "v"((uint32_t)(i * 1024 + 16 * lane)), "s"(src)
                   : "memory");
  };
  // wait until at most `in_flight` later tiles of this wave are in flight
  auto wait_tiles = [&](int in_flight) {
    if (wave == 0) {
      if (in_flight >= 2) wait_vmcnt<20>();
      else if (in_flight == 1) wait_vmcnt<10>();
      else wait_vmcnt<0>();
    } else {
      if (in_flight >= 2) wait_vmcnt<18>();
      else if (in_flight == 1) wait_vmcnt<9>();
      else wait_vmcnt<0>();
    }
  };
  // rows past the partition end (another token's bytes, or poison): zero the
  // 16-byte chunks this wave loaded whose row is >= first_bad (a chunk never
  // straddles two rows: 16 | 592); a zero row has min = step = 0
  auto zero_tail = [&](int k, int first_bad) {
    char* base = slot(k);
    for (int i = l0; i < l0 + lc; ++i) {
      const int o = i * 1024 + 16 * lane;
      if (o / kQRow >= first_bad) *reinterpret_cast<u32x4_t*>(base + o) = u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  float off = 0.0f;  // this lane's part of sum_t p_t min_t - 1024 sum_t P_t (row n)
  f32x4_t acc[2][4], psum;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[f][m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  psum = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int t_draft = L - Q;
  const int lim = min(par ? t_draft - 1 : t_draft + (row0 + n) / H, t1 - 1);
  const uint64_t branch = (par && !bad_len) ? tree_branch_mask(par, Q, (row0 + n) / H) : 0ull;

  if (ntiles > 0) {
    // ---- prologue: queries (waves 0, 1: 8 rows each, into slot 3), tiles 0..2
    const int npre = min(ntiles, kQRing - 1);
    RowDma<kQQLoads> qdma;
    qdma.init(wave * 8 * kChunks, lane, wave * 8);
    if (wave < 2)
      qdma.issue(q_full + ((size_t)b * R + row0 + wave * 8) * kD,
                 __builtin_amdgcn_readfirstlane(lds_addr(slot(kQRing - 1) + wave * 8 * kChunks * 16)));
    issue(0);
    if (npre > 1) issue(1);
    if (npre > 2) issue(2);
    if (wave < 2) wait_vmcnt<0>();  // own query rows (and the tiles behind them)
    __syncthreads();
    // queries in fp16: row n, chunk 4 ks + kg (stored with the bf16 tile's
    // swizzle), and the row's sums over the latent and RoPE columns
    f16x8_t qh[kKSteps];
    float sq_lat = 0.0f, sq_rope = 0.0f;
    {
      const u32x4_t* qb = reinterpret_cast<const u32x4_t*>(slot(kQRing - 1));
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const int c = 4 * ks + kg;
        const bf16x8_t qv = __builtin_bit_cast(bf16x8_t, qb[n * kChunks + (c ^ (n & 7))]);
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const _Float16 h = (_Float16)(float)qv[j];
          qh[ks][j] = h;
          part += (float)h;
        }
        if (ks < kDC / 32)
          sq_lat += part;
        else
          sq_rope += part;
      }
      sq_lat = row_sum4(sq_lat) * scale_log2;    // the softmax scale folded in
      sq_rope = row_sum4(sq_rope) * scale_log2;
    }
    // own part of tile 0
    wait_tiles(npre - 1);
    if (t0 + kQT > t1) zero_tail(0, t1 - t0);
    __syncthreads();

    // QK: A operand of lane (token 16 wave + n, kg) at byte (16 wave + n) * 592 + 32 ks + 8 kg
    const int arow = (16 * wave + n) * kQRow;
    // PV: tokens sigma(kg, j) of a K-block; codes of columns 128 wave + 64 f + 4 n .. + 3
    int pvt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) pvt[j] = ((j < 4) ? 4 * kg + j : 16 + 4 * kg + (j - 4)) * kQRow;
    const f16x8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};

    // scores (log2 units) of subtile `wave` of tile k into score buffer k & 1
    auto qk = [&](int k) {
      const char* tile = slot(k);
      const char* buf = tile + arow;
      f32x4_t cl[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
      f32x4_t cr = {0.0f, 0.0f, 0.0f, 0.0f};
      u32x2_t cv[kKSteps];
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        cv[ks] = *reinterpret_cast<const u32x2_t*>(buf + 32 * ks + 8 * kg);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        const f16x8_t a = codes8_f16(cv[ks]);
        if (ks < kDC / 32)
          cl[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[ks], cl[ks & 1], 0, 0, 0);
        else
          cr = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qh[ks], cr, 0, 0, 0);
      }
      const f32x4_t al = cl[0] + cl[1];
      // lane (row n, kg) holds tokens 16 wave + 4 kg + r
      f32x4_t out;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 mt = *reinterpret_cast<const float4*>(tile + (16 * wave + 4 * kg + r) * kQRow + kD);
        const float kl = fmaf(-1024.0f, mt.y, mt.x), kr2 = fmaf(-1024.0f, mt.w, mt.z);
        out[r] = fmaf(mt.y * scale_log2, al[r],
                      fmaf(mt.w * scale_log2, cr[r], fmaf(kl, sq_lat, kr2 * sq_rope)));
      }
      sc[((k & 1) * kWaves + wave) * 64 + lane] = out;
    };
    qk(0);

    for (int k = 0; k < ntiles; ++k) {
      if (k + 1 < ntiles) {  // own part of tile k+1 (tile k+2 may stay in flight)
        wait_tiles(k + 2 < ntiles ? 1 : 0);
        const int ts1 = t0 + (k + 1) * kQT;
        if (ts1 + kQT > t1) zero_tail(k + 1, t1 - ts1);
      }
      // tile k+1 landed for every wave, the scores of tile k are complete, and
      // slot k-1 (= slot k+3) is no longer read by anyone
      __syncthreads();
      if (k + 3 < ntiles) issue(k + 3);
      if (k + 1 < ntiles) qk(k + 1);

      // ---- softmax over the tile's 64 tokens (lane: row n, tokens 16 u + 4 kg + r)
      const int ts = t0 + k * kQT;
      const f32x4_t* sk = sc + (k & 1) * kWaves * 64 + lane;
      float sv[16];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x4_t su = sk[64 * u];
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[4 * u + r] = su[r];
      }
      if (!__all(ts + kQT - 1 <= lim)) {  // some token of the tile is masked for some row
        const uint64_t vis = tile_visible(ts, lim, t_draft, t1, branch);
        const uint64_t vl = vis >> (4 * kg);
#pragma unroll
        for (int j = 0; j < 16; ++j)
          sv[j] = ((vl >> (16 * (j >> 2) + (j & 3))) & 1ull) ? sv[j] : -INFINITY;
      }
      float mloc = sv[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mloc = fmaxf(mloc, sv[j]);
      mloc = row_max4(mloc);
      const bool raise = mloc > m_run + kLazy;
      if (__any(raise)) {
        const float m_new = raise ? mloc : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        off *= alpha;
        if (__any(raise && m_run != -INFINITY)) {
          float ar[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kg + r, 64);
#pragma unroll
          for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[f][m][r] *= ar[r];
#pragma unroll
          for (int r = 0; r < 4; ++r) psum[r] *= ar[r];
        }
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      const char* tb = slot(k);
      // P for K-block blk: slots 0..3 = subtile 2 blk, 4..7 = subtile 2 blk + 1
      f16x8_t pa[2];
      float ps = 0.0f;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = __builtin_amdgcn_exp2f(sv[8 * blk + j] - m_use);
          const float2 mt = *reinterpret_cast<const float2*>(tb + blk * 32 * kQRow + pvt[j] + kD);
          ps += p;
          off = fmaf(p, mt.x, off);
          pa[blk][j] = (_Float16)(p * mt.y);
        }
      }
      l_run += ps;

      // ---- PV: this wave's 128 latent columns, two blocks of 64, two K-blocks
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const char* kb = tb + blk * 32 * kQRow;
        uint32_t cw[2][8];
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            cw[f][j] = *reinterpret_cast<const uint32_t*>(kb + pvt[j] + 128 * wave + 64 * f + 4 * n);
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          // token pairs (2 i, 2 i + 1): interleave their bytes, then lift each
          // column's byte pair to two fp16 values 1024 + code
          u32x4_t bm[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t i0 = __builtin_amdgcn_perm(cw[f][2 * i + 1], cw[f][2 * i], 0x05010400u);
            const uint32_t i1 = __builtin_amdgcn_perm(cw[f][2 * i + 1], cw[f][2 * i], 0x07030602u);
            const u32x2_t c01 = codes_f16(i0), c23 = codes_f16(i1);
            bm[0][i] = c01.x;
            bm[1][i] = c01.y;
            bm[2][i] = c23.x;
            bm[3][i] = c23.y;
          }
#pragma unroll
          for (int m = 0; m < 4; ++m)
            acc[f][m] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                pa[blk], __builtin_bit_cast(f16x8_t, bm[m]), acc[f][m], 0, 0, 0);
        }
        psum = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[blk], ones, psum, 0, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();

  // ---- write rows row0 .. row0+15, columns [128 wave, 128 wave + 128) ------
  const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;
  const float nanv = __int_as_float(0x7fc00000);
  const float l_row = row_sum4(l_run);
  const float off_row = row_sum4(off);   // sum_t p_t min_t of row n
  float inv[4], base[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lr = __shfl(l_row, 4 * kg + r, 64);
    inv[r] = lr > 0.0f ? 1.0f / lr : 0.0f;
    // row 4 kg + r: psum holds sum_t P_t of that row in every column
    base[r] = fmaf(-1024.0f, psum[r], __shfl(off_row, 4 * kg + r, 64));
  }
  // an empty partition (no tokens) leaves its o_part rows unwritten
#pragma unroll
  for (int r = 0; r < 4 && (t1 > t0 || any_bad); ++r) {
    const int orow = row0 + 4 * kg + r;
    float* dst = o_part + (((size_t)b * R + orow) * S + s) * kDC + 128 * wave + 4 * n;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      float4 v = make_float4((acc[f][0][r] + base[r]) * inv[r], (acc[f][1][r] + base[r]) * inv[r],
                             (acc[f][2][r] + base[r]) * inv[r], (acc[f][3][r] + base[r]) * inv[r]);
      if (any_bad) v = make_float4(nanv, nanv, nanv, nanv);
      *reinterpret_cast<float4*>(dst + f * 64) = v;
    }
  }
  if (wave == 0 && kg == 0) {
    const float lse = l_row > 0.0f ? (m_run + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
    lse_part[((size_t)b * R + row0 + n) * S + s] = any_bad ? nanv : lse;
  }
}

bool decode_q8_ok(const Shape& s, int q_len) {
  return s.dtype == 1 && s.dc == kDC && s.dr == kD - kDC && s.page % kQT == 0 &&
         (q_len * s.H) % 16 == 0;
}

int launch_decode_q8(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                     const void* q_full, const void* cache, int64_t num_pages,
                     const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                     const int32_t* tree_parent, float* o_part, float* lse_part, void* stream) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_q8_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kQLds);
    if (e != hipSuccess) return (int)e;
    attr = true;
  }
  const int units = batch * num_splits;
  const int groups = q_len * s.H / 16;
  const int blocks = grid_blocks(units, groups);
  hipLaunchKernelGGL(decode_q8_kernel, dim3(blocks), dim3(256), kQLds,
                     reinterpret_cast<hipStream_t>(stream), q_len, s.H, num_splits, s.page,
                     s.split_fixed, max_seq_len, s.scale * 1.4426950408889634f, units, groups,
                     (const bf16_t*)q_full, (const uint8_t*)cache, num_pages, page_table,
                     max_pages, seq_lens, tree_parent, o_part, lse_part);
  return (int)hipGetLastError();
}

}  // namespace mla
