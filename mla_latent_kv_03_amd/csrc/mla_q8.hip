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
// The decode kernel keeps 16 query rows per block and splits the partition
// into 16-token subtiles that the block's four waves stream independently:
// each wave has its own 4-slot LDS ring (a subtile is one contiguous
// 9,472-byte copy, rows 592 bytes apart, a stride at which both operand read
// patterns are free of LDS bank conflicts), its own loads and waits and its
// own online-softmax state, so the token loop has no block barrier; the four
// states are merged once at the end. A wave64 vector instruction occupies the
// SIMD for 4 cycles, so the codes are not decoded element by element: the
// MFMAs take them as the fp16 subnormals code * 2^-24 (one v_perm per two),
// and the code -> value map is applied per score and per output row (see
// decode_q8_kernel):
//   QK  16 tokens x 16 rows over all 576 columns (18 v_mfma_f32_16x16x32_f16)
//   PV  all 512 latent columns of the 16 rows over the 16 tokens
//       (32 v_mfma_f32_16x16x16_f16); the A operand is P over the 4 tokens
//       whose scores the lane holds after QK, so P never leaves registers.
#include "mla_append.h"
#include "mla_append_coded.h"
#include "mla_decode_common.h"
#include "mla_launch.h"

namespace mla {

using namespace dec;

// ---------------------------------------------------------------------------
// Quantizing append: one block of 128 threads per row (body in
// mla_append_coded.h).
// ---------------------------------------------------------------------------
template <typename T, int kBits>
__global__ __launch_bounds__(128) void append_q8_kernel(
    int dc, int dr, int page, const T* __restrict__ c_kv, const T* __restrict__ k_rope,
    const int32_t* __restrict__ seq_idx, const int32_t* __restrict__ pos,
    const int32_t* __restrict__ rope_pos, const int32_t* __restrict__ page_table, int batch,
    int max_pages, uint8_t* __restrict__ cache, int64_t num_pages, int rotate, double log2_base) {
  append_coded_row<T, kBits>(blockIdx.x, dc, dr, page, c_kv, k_rope, seq_idx, pos, rope_pos,
                             page_table, batch, max_pages, cache, num_pages, rotate, log2_base);
}

template <int kBits>
static int launch_cache_append_qn(const Shape& s, int n_tok, const void* c_kv,
                                  const void* k_rope, const int32_t* seq_idx, const int32_t* pos,
                                  const int32_t* rope_pos, const int32_t* page_table, int batch,
                                  int max_pages, void* cache, int64_t num_pages, int rotate,
                                  void* stream) {
  if (s.dtype == 0)
    hipLaunchKernelGGL((append_q8_kernel<float, kBits>), dim3(n_tok), dim3(128), 0,
                       reinterpret_cast<hipStream_t>(stream), s.dc, s.dr, s.page,
                       (const float*)c_kv, (const float*)k_rope, seq_idx, pos, rope_pos,
                       page_table, batch, max_pages, (uint8_t*)cache, num_pages, rotate,
                       s.log2_base);
  else
    hipLaunchKernelGGL((append_q8_kernel<bf16_t, kBits>), dim3(n_tok), dim3(128), 0,
                       reinterpret_cast<hipStream_t>(stream), s.dc, s.dr, s.page,
                       (const bf16_t*)c_kv, (const bf16_t*)k_rope, seq_idx, pos, rope_pos,
                       page_table, batch, max_pages, (uint8_t*)cache, num_pages, rotate,
                       s.log2_base);
  return (int)hipGetLastError();
}

int launch_cache_append_q8(const Shape& s, int n_tok, const void* c_kv, const void* k_rope,
                           const int32_t* seq_idx, const int32_t* pos, const int32_t* rope_pos,
                           const int32_t* page_table, int batch, int max_pages, void* cache,
                           int64_t num_pages, int rotate, void* stream) {
  return launch_cache_append_qn<8>(s, n_tok, c_kv, k_rope, seq_idx, pos, rope_pos, page_table,
                                   batch, max_pages, cache, num_pages, rotate, stream);
}

int launch_cache_append_q4(const Shape& s, int n_tok, const void* c_kv, const void* k_rope,
                           const int32_t* seq_idx, const int32_t* pos, const int32_t* rope_pos,
                           const int32_t* page_table, int batch, int max_pages, void* cache,
                           int64_t num_pages, int rotate, void* stream) {
  return launch_cache_append_qn<4>(s, n_tok, c_kv, k_rope, seq_idx, pos, rope_pos, page_table,
                                   batch, max_pages, cache, num_pages, rotate, stream);
}

// ---------------------------------------------------------------------------
// Decode over the 8-bit cache, 16 query rows per block, four waves that
// stream independently.
// ---------------------------------------------------------------------------
namespace {

constexpr int kQT = 16;                              // tokens per wave subtile
constexpr int kQQBytes = kKSteps * 64 * 16;          // 18,432: the query B operands in fp16
constexpr int kQQueryLoads = 16 * kD * 2 / 1024;     // 18: the 16 query rows in bf16
constexpr int kQAcc = 16 * kDC * 4;                  // 32,768: one wave's accumulators

// Row and ring geometry of a cache with kBits-bit codes (8: one code per byte;
// 4: two per byte, column 2i in the low nibble of byte i)
template <int kBits>
struct QFmt {
  static constexpr int kCode = kD * kBits / 8;       // code bytes: 576 / 288
  static constexpr int kRow = kCode + kQ8Meta;       // bytes per cached row: 592 / 304
  static constexpr int kSub = kQT * kRow;            // one subtile: 9,472 / 4,864
  static constexpr int kWide = kSub / 1024;          // loads of 16 B per lane: 9 / 4 ...
  static constexpr int kTail = (kSub - kWide * 1024) / 256;  // ... of 4 B per lane: 1 / 3
  static constexpr int kSubLoads = kWide + kTail;
  static constexpr int kRing = kBits == 8 ? 3 : 6;   // ring slots per wave
  static constexpr int kStage = (((kQQueryLoads + kWaves - 1) / kWaves) * 1024 + kSub - 1) / kSub;
  static constexpr int kWaveBytes = kRing * kSub;
  static constexpr size_t kRingLds = (size_t)kWaves * kWaveBytes + kQQBytes;
  static constexpr size_t kLds = kRingLds > (size_t)kWaves * kQAcc ? kRingLds
                                                                   : (size_t)kWaves * kQAcc;
  static_assert(kSub - kWide * 1024 == 256 * kTail, "a subtile is whole loads");
  static_assert(kRow % 16 == 0, "a 16-byte chunk never straddles two rows");
  static_assert(kStage < kRing, "the query rows are staged in the ring's last slots");
  static_assert(kLds + 4096 <= 160 * 1024, "LDS of one CU, with the static arrays");
};

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;

// A code byte under a zero high byte is the fp16 subnormal code * 2^-24,
// exact, and the MFMA takes subnormal fp16 inputs as they are. One v_perm
// lifts two codes of a dword (selector byte 0x0c yields a zero byte).
__device__ __forceinline__ f16x8_t codes8_sub(u32x2_t c) {
  return __builtin_bit_cast(f16x8_t, u32x4_t{__builtin_amdgcn_perm(0u, c.x, 0x0c010c00u),
                                              __builtin_amdgcn_perm(0u, c.x, 0x0c030c02u),
                                              __builtin_amdgcn_perm(0u, c.y, 0x0c010c00u),
                                              __builtin_amdgcn_perm(0u, c.y, 0x0c030c02u)});
}

// The same for eight 4-bit codes of a dword (codes 2i and 2i + 1 in the low
// and high nibble of byte i): the nibbles are split into two dwords of bytes,
// then one v_perm per two codes as above.
__device__ __forceinline__ f16x8_t codes4_sub(uint32_t c) {
  const uint32_t lo = c & 0x0f0f0f0fu, hi = (c >> 4) & 0x0f0f0f0fu;
  return __builtin_bit_cast(f16x8_t, u32x4_t{__builtin_amdgcn_perm(hi, lo, 0x0c040c00u),
                                              __builtin_amdgcn_perm(hi, lo, 0x0c050c01u),
                                              __builtin_amdgcn_perm(hi, lo, 0x0c060c02u),
                                              __builtin_amdgcn_perm(hi, lo, 0x0c070c03u)});
}

// The MFMA's k index 8 kg + i of step ks stands for code column
// q8_col(ks, kg) + i: in the latent part a lane's four steps 4 G .. 4 G + 3
// cover 32 contiguous codes (two 16-byte LDS reads), in the RoPE part its two
// steps cover 16. The query rows take the same columns, so the dot products
// are unchanged.
__device__ __forceinline__ int q8_col(int ks, int kg) {
  return ks < kDC / 32 ? 128 * (ks >> 2) + 32 * kg + 8 * (ks & 3)
                       : kDC + 16 * kg + 8 * (ks - kDC / 32);
}

}  // namespace

// Block: 16 query rows (row0 .. row0 + 15) of one (sequence, partition)
// unit, 4 waves. The partition is cut into 16-token subtiles; wave w takes
// subtiles w, w + 4, w + 8, ... and streams them through a 3-slot ring of its
// own (one subtile = 9,472 contiguous bytes of one page, 10 direct-to-LDS
// loads), so the token loop has no block barrier: each wave waits only for
// its own loads and keeps its own online-softmax state for all 16 rows. The
// four states are merged at the end through LDS. The query rows' fp16 MFMA
// operands (18 KB) sit in LDS beside the rings: in registers they would
// leave too few for the 128 accumulators and a subtile's operands.
//
// The contractions run on fp16 MFMA with the codes as the subnormals
// code * 2^-24, and the affine code -> value map (min + step * code, per row
// and part) is applied per score and per output row:
//   score: q . (min + step c) = step 2^24 (q . c 2^-24) + min sum q, per part
//          (latent, RoPE), QK^T = 18 v_mfma_f32_16x16x32_f16 per subtile
//          (A = 8 codes of token n per lane, B = the query rows in fp16)
//   P.C:   sum_t p_t (min_t + step_t c_t)
//            = 2^(24 - g) sum_t P_t (c_t 2^-24) + sum_t p_t min_t,
//          P_t = fp16(p_t step_t 2^g)
//          32 v_mfma_f32_16x16x16_f16 per subtile: A = P of row n over the 4
//          tokens whose scores the lane already holds, B = one column of those
//          4 tokens' codes (two v_perm), columns 64 g + 4 n + r
// The query rows are converted to fp16 once per block, each row part (latent,
// RoPE) scaled by the power of two 2^e that brings its largest magnitude into
// [2^14, 2^15): bf16 values then convert exactly unless they lie more than
// 2^28 below that largest one, where their part of a dot product is below
// what the fp32 accumulation resolves; the factor 2^-e goes into the row's
// score terms. P_t = p_t step_t 2^g carries a per-row power of two as well,
// chosen so that the largest P of the row since the last change lies in
// [2^-2, 2^12]: every P fits fp16, and one that falls into fp16's subnormal
// band is at least 2^16 below that largest term. Both factors are exact, so
// the rows' own scales (steps from 2^-100 to 2^100, queries of any finite
// bf16 magnitude) leave the rounding of the contractions unchanged.
template <int kBits>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_q8_kernel(int Q, int H, int S, int page, int fixed, int max_seq_len,
                      float scale_log2, int units, int groups, const bf16_t* __restrict__ q_full,
                      const uint8_t* __restrict__ cache, int64_t num_pages,
                      const int32_t* __restrict__ page_table, int max_pages,
                      const int32_t* __restrict__ seq_lens,
                      const int32_t* __restrict__ tree_parent, float* __restrict__ o_part,
                      float* __restrict__ lse_part) {
  using F = QFmt<kBits>;
  extern __shared__ u32x4_t lds[];
  __shared__ float st_m[kWaves][16], st_l[kWaves][16], st_o[kWaves][16];
  __shared__ int pwin[kWaves][64];     // each wave's copy of the page window
  __shared__ float sqp[kWaves][16][2];  // each wave's part of the query row sums
  __shared__ float sqa[kWaves][16][2];  // ... and of their largest magnitudes
  __shared__ int st_g[kWaves][16];      // each wave's exponent of its P factor
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
  // block-uniform: subtiles any row of the block sees; this wave's share
  const int nsub = tiles_needed(t0, t1, kQT, par != nullptr, L - Q, (row0 + 15) / H);
  const int nk = nsub > wave ? (nsub - wave + kWaves - 1) / kWaves : 0;
  bool bad = bad_len;

  char* const lbase = reinterpret_cast<char*>(lds);
  char* const wbase = lbase + wave * F::kWaveBytes;
  char* const qop = lbase + kWaves * F::kWaveBytes;  // the query B operands

  // The page-table window (lane i: unit page i of the partition) is copied
  // into LDS ahead of the query rows, so that waiting for it leaves the
  // query copy in flight.
  PageWindow pw;
  pw.row = page_table + (size_t)b * max_pages + t0 / page;
  pw.upages = (t1 - t0 + page - 1) / page;
  pw.base = 0;
  pw.reg = 0;
  // Subtiles are issued in order, k = 0, 1, 2, ...: subtile k of this wave is
  // tokens [t0 + 16 (4 k + wave), + 16), inside one page (t0 is a multiple of
  // the page size, which is a multiple of 64). The next one to issue is row
  // i_off of unit page i_up, into slot i_slot; each step moves 64 tokens on,
  // which crosses at most one page boundary.
  int i_up = 0, i_off = kQT * wave, i_slot = 0;
  const int pg_lim = (int)min(num_pages, (int64_t)0x7fffffff);
  const size_t page_bytes = (size_t)page * F::kRow;
  auto issue_next = [&]() {
    int pg = pw.get(i_up, lane);
    if (pg < 0 || pg >= pg_lim) {
      bad = true;
      pg = 0;
    }
    const uint8_t* src = cache + (size_t)pg * page_bytes + (size_t)i_off * F::kRow;
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(wbase + i_slot * F::kSub));
#pragma unroll
    for (int i = 0; i < F::kWide; ++i)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                   :
                   : "s"(dst + i * 1024), "v"((uint32_t)(i * 1024 + 16 * lane)), "s"(src)
                   : "memory");
#pragma unroll
    for (int i = 0; i < F::kTail; ++i)
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2 nt"
                   :
                   : "s"(dst + F::kWide * 1024 + i * 256),
                     "v"((uint32_t)(F::kWide * 1024 + i * 256 + 4 * lane)), "s"(src)
                   : "memory");
    i_off += kWaves * kQT;
    if (i_off >= page) {
      i_off -= page;
      ++i_up;
    }
    i_slot = i_slot == F::kRing - 1 ? 0 : i_slot + 1;
  };
  // wait until at most `in_flight` later subtiles of this wave are in flight
  auto wait_subs = [&](int in_flight) {
    static_assert(F::kRing <= 6 && 5 * F::kSubLoads <= 63, "the waits below cover the ring");
    switch (min(in_flight, F::kRing - 1)) {
      case 5: wait_vmcnt<5 * F::kSubLoads>(); break;
      case 4: wait_vmcnt<4 * F::kSubLoads>(); break;
      case 3: wait_vmcnt<3 * F::kSubLoads>(); break;
      case 2: wait_vmcnt<2 * F::kSubLoads>(); break;
      case 1: wait_vmcnt<F::kSubLoads>(); break;
      default: wait_vmcnt<0>(); break;
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  float off = 0.0f;  // this lane's part of sum_t p_t min_t (row n)
  float sq_lat = 0.0f, sq_rope = 0.0f;             // row sums of the query parts
  const float c24 = scale_log2 * 16777216.0f;
  float c24l = c24, c24r = c24;  // with the query parts' 2^-e
  int ge = 0;                    // P_t = p_t step_t 2^ge (row n)
  float pmax = 0.0f;             // largest P_t of row n since ge last changed
  f32x4_t acc[kFB][4];
#pragma unroll
  for (int g = 0; g < kFB; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[g][r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  const int t_draft = L - Q;
  const int lim = min(par ? t_draft - 1 : t_draft + (row0 + n) / H, t1 - 1);
  const uint64_t branch = (par && !bad_len) ? tree_branch_mask(par, Q, (row0 + n) / H) : 0ull;

  if (nsub > 0) {
    // ---- prologue: the page window; query load i (1 KB of the 16 bf16 rows)
    // to the last kStage slots of wave i % 4 at 1 KB * (i / 4); subtiles
    // 0 .. kRing - kStage - 1
    {
      const int* src = pw.row + min(lane, pw.upages - 1);  // pw.upages >= 1 here
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(&pwin[wave][0]));
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                   :
                   : "s"(dst), "v"(src)
                   : "memory");
      const bf16_t* qsrc = q_full + ((size_t)b * R + row0) * kD;
      const uint32_t qdst = __builtin_amdgcn_readfirstlane(
          lds_addr(wbase + (F::kRing - F::kStage) * F::kSub));
      for (int i = wave; i < kQQueryLoads; i += kWaves)  // wave-uniform bounds
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                     :
                     : "s"(qdst + (i / kWaves) * 1024), "v"((uint32_t)(i * 1024 + 16 * lane)),
                       "s"(qsrc)
                     : "memory");
      // the window has landed when at most this wave's query loads are pending
      static_assert(kQQueryLoads == 4 * kWaves + 2, "waves 0, 1 issue 5 query loads, 2, 3 four");
      if (wave < 2)
        wait_vmcnt<kQQueryLoads / kWaves + 1>();
      else
        wait_vmcnt<kQQueryLoads / kWaves>();
      pw.reg = pwin[wave][lane];
    }
    const int npre = min(nk, F::kRing - F::kStage);
    for (int k = 0; k < npre; ++k) issue_next();
    wait_subs(npre);  // own query loads (issued before the subtiles)
    __syncthreads();
    // the B operand of step ks for lane (row n, kg), columns q8_col(ks, kg) .. + 7,
    // in fp16 at qop + 1 KB * ks + 16 * lane: wave w converts the steps
    // ks = w mod 4 and its part of the row sums, which meet in LDS
    auto q_stage = [&](int ks) {
      const int gb = n * kD * 2 + 2 * q8_col(ks, kg);
      const int li = gb >> 10;
      const char* p = lbase + (li % kWaves) * F::kWaveBytes +
                      (F::kRing - F::kStage) * F::kSub + (li / kWaves) * 1024 + (gb & 1023);
      return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
    };
    {
      float al = 0.0f, ar = 0.0f;
      for (int ks = wave; ks < kKSteps; ks += kWaves) {  // wave-uniform bounds
        const bf16x8_t qv = q_stage(ks);
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf((float)qv[j]));
        if (ks < kDC / 32)
          al = fmaxf(al, a);
        else
          ar = fmaxf(ar, a);
      }
      al = row_max4(al);
      ar = row_max4(ar);
      if (kg == 0) {
        sqa[wave][n][0] = al;
        sqa[wave][n][1] = ar;
      }
    }
    __syncthreads();
    // 2^e with (largest magnitude) 2^e in [2^14, 2^15), e within [-100, 100]
    auto q_exp = [](float a) {
      if (!(a > 0.0f) || !(a < INFINITY)) return 0;
      return min(100, max(-100, 15 - __builtin_amdgcn_frexp_expf(a)));
    };
    const int el = q_exp(fmaxf(fmaxf(sqa[0][n][0], sqa[1][n][0]), fmaxf(sqa[2][n][0], sqa[3][n][0])));
    const int er = q_exp(fmaxf(fmaxf(sqa[0][n][1], sqa[1][n][1]), fmaxf(sqa[2][n][1], sqa[3][n][1])));
    {
      float sl = 0.0f, sr = 0.0f;
      for (int ks = wave; ks < kKSteps; ks += kWaves) {  // wave-uniform bounds
        const bf16x8_t qv = q_stage(ks);
        const int e = ks < kDC / 32 ? el : er;
        f16x8_t h;
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          h[j] = (_Float16)ldexpf((float)qv[j], e);
          part += (float)h[j];
        }
        *reinterpret_cast<f16x8_t*>(qop + ks * 1024 + 16 * lane) = h;
        if (ks < kDC / 32)
          sl += part;
        else
          sr += part;
      }
      sl = row_sum4(sl);
      sr = row_sum4(sr);
      if (kg == 0) {
        sqp[wave][n][0] = sl;
        sqp[wave][n][1] = sr;
      }
    }
    __syncthreads();  // the operands are written and the staging slots are free
    sq_lat = ldexpf((sqp[0][n][0] + sqp[1][n][0] + sqp[2][n][0] + sqp[3][n][0]) * scale_log2, -el);
    sq_rope = ldexpf((sqp[0][n][1] + sqp[1][n][1] + sqp[2][n][1] + sqp[3][n][1]) * scale_log2, -er);
    c24l = ldexpf(c24, -el);
    c24r = ldexpf(c24, -er);
    for (int k = npre; k < min(nk, F::kRing); ++k) issue_next();  // the staging slots

    // QK: A operand of lane (token n, kg), code columns q8_col(ks, kg) .. + 7
    // of row n; PV: B operand of lane (n, kg) from tokens 4 kg + j (8 bits:
    // columns 64 g + 4 n + r; 4 bits: columns 128 (g >> 1) + 8 n + 4 (g & 1) + r)
    const int arow = n * F::kRow;
    const int brow = 4 * kg * F::kRow + 4 * n;
    const char* const qb = qop + 16 * lane;
    int c_slot = 0;  // slot of subtile k
    for (int k = 0; k < nk; ++k) {
      wait_subs(min(nk - 1 - k, F::kRing - 1));
      const int ts = t0 + kQT * (kWaves * k + wave);
      char* tile = wbase + c_slot * F::kSub;
      c_slot = c_slot == F::kRing - 1 ? 0 : c_slot + 1;
      if (ts + kQT > t1) {  // rows past the partition end (another token, or poison) -> 0
        for (int c = (t1 - ts) * (F::kRow / 16) + lane; c < F::kSub / 16; c += 64)
          reinterpret_cast<u32x4_t*>(tile)[c] = u32x4_t{0u, 0u, 0u, 0u};
      }
      // the QK operands and the row metadata first: 8 bits, nine 16-byte
      // reads of two k-steps each; 4 bits, four 16-byte reads of four latent
      // k-steps each and one 8-byte read of the two RoPE k-steps
      constexpr int kAR = kBits == 8 ? kKSteps / 2 : 5;
      u32x4_t cv[kAR];
      if constexpr (kBits == 8) {
#pragma unroll
        for (int i = 0; i < kAR; ++i)
          cv[i] = *reinterpret_cast<const u32x4_t*>(tile + arow + q8_col(2 * i, kg));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          cv[i] = *reinterpret_cast<const u32x4_t*>(tile + arow + 64 * i + 16 * kg);
        const u32x2_t r2 = *reinterpret_cast<const u32x2_t*>(tile + arow + kDC / 2 + 8 * kg);
        cv[4] = u32x4_t{r2.x, r2.y, 0u, 0u};
      }
      float4 mt[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        mt[r] = *reinterpret_cast<const float4*>(tile + (4 * kg + r) * F::kRow + F::kCode);

      f32x4_t cl[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
      f32x4_t cr = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        f16x8_t a;
        if constexpr (kBits == 8) {
          const u32x4_t& w = cv[ks >> 1];
          a = codes8_sub((ks & 1) ? u32x2_t{w.z, w.w} : u32x2_t{w.x, w.y});
        } else {
          const u32x4_t& w = cv[ks < kDC / 32 ? ks >> 2 : 4];
          const int d = ks < kDC / 32 ? ks & 3 : ks - kDC / 32;
          a = codes4_sub(d == 0 ? w.x : d == 1 ? w.y : d == 2 ? w.z : w.w);
        }
        const f16x8_t qk = *reinterpret_cast<const f16x8_t*>(qb + ks * 1024);
        if (ks < kDC / 32)
          cl[ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qk, cl[ks & 1], 0, 0, 0);
        else
          cr = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qk, cr, 0, 0, 0);
      }
      // the PV operands: their reads overlap the score and softmax arithmetic
      // (8 bits: four codes of a token per dword, one dword per column block
      // g; 4 bits: eight codes per dword, one dword per pair of blocks)
      constexpr int kPB = kBits == 8 ? kFB : kFB / 2;
      uint32_t u[kPB][4];
#pragma unroll
      for (int g = 0; g < kPB; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          u[g][j] = *reinterpret_cast<const uint32_t*>(tile + brow + j * F::kRow + 64 * g);

      // ---- scores of row n, tokens 4 kg + r (log2 units)
      const f32x4_t al = cl[0] + cl[1];
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = fmaf(mt[r].y * c24l, al[r],
                     fmaf(mt[r].w * c24r, cr[r], fmaf(mt[r].x, sq_lat, mt[r].z * sq_rope)));
      }
      if (!__all(ts + kQT - 1 <= lim)) {  // some token of the subtile is masked for some row
        const uint32_t vl =
            (uint32_t)(tile_visible(ts, lim, t_draft, t1, branch) >> (4 * kg)) & 0xfu;
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[r] = ((vl >> r) & 1u) ? sv[r] : -INFINITY;
      }

      // ---- online softmax of this wave's rows (lazy rescale)
      const float mloc = row_max4(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
      const bool raise = mloc > m_run + kLazy;
      if (__any(raise)) {
        const float m_new = raise ? mloc : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        off *= alpha;
        pmax *= alpha;
        if (__any(raise && m_run != -INFINITY)) {
          float ar[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kg + r, 64);
#pragma unroll
          for (int g = 0; g < kFB; ++g)
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[g][c][r] *= ar[r];
        }
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(sv[r] - m_use);
        l_run += p;
        off = fmaf(p, mt[r].x, off);
        x[r] = p * ldexpf(mt[r].y, ge);
      }
      // keep the row's largest P since the last change of ge in [2^-2, 2^12]
      // (a change sets it to [1, 2) and rescales the accumulators exactly)
      const float xm = fmaxf(pmax, row_max4(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]))));
      const bool refit = xm > 4096.0f || (xm > 0.0f && xm < 0.25f);
      if (__any(refit)) {
        const int k = refit ? min(100 - ge, max(-100 - ge, 1 - __builtin_amdgcn_frexp_expf(xm)))
                            : 0;
        ge += k;
        pmax = ldexpf(xm, k);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[r] = ldexpf(x[r], k);
        int kr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) kr[r] = __shfl(k, 4 * kg + r, 64);
#pragma unroll
        for (int g = 0; g < kFB; ++g)
#pragma unroll
          for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[g][c][r] = ldexpf(acc[g][c][r], kr[r]);
      } else {
        pmax = xm;
      }
      f16x4_t pa;
#pragma unroll
      for (int r = 0; r < 4; ++r) pa[r] = (_Float16)x[r];

      // the slot is read: subtile k + kRing may land in it
      if (k + F::kRing < nk) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue_next();
      }

      // ---- PV: all 512 latent columns of the 16 rows, K = this subtile's 16 tokens
      if constexpr (kBits == 8) {
#pragma unroll
        for (int g = 0; g < kFB; ++g) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // column 64 g + 4 n + r of tokens 4 kg .. 4 kg + 3, as subnormals
            const uint32_t sel = 0x0c000c00u | ((uint32_t)(4 + r) << 16) | (uint32_t)r;
            const u32x2_t bw = {__builtin_amdgcn_perm(u[g][1], u[g][0], sel),
                                __builtin_amdgcn_perm(u[g][3], u[g][2], sel)};
            acc[g][r] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                pa, __builtin_bit_cast(f16x4_t, bw), acc[g][r], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int gp = 0; gp < kFB / 2; ++gp) {
          // the dword of token 4 kg + j holds columns 128 gp + 8 n .. + 7:
          // low nibbles (even columns) and high nibbles (odd) as bytes
          uint32_t lo[4], hi[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            lo[j] = u[gp][j] & 0x0f0f0f0fu;
            hi[j] = (u[gp][j] >> 4) & 0x0f0f0f0fu;
          }
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            // column 128 gp + 8 n + c: byte c / 2 of the low or high nibbles
            const uint32_t i = (uint32_t)(c >> 1);
            const uint32_t sel = 0x0c000c00u | ((4u + i) << 16) | i;
            const uint32_t* src = (c & 1) ? hi : lo;
            const u32x2_t bw = {__builtin_amdgcn_perm(src[1], src[0], sel),
                                __builtin_amdgcn_perm(src[3], src[2], sel)};
            acc[2 * gp + (c >> 2)][c & 3] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                pa, __builtin_bit_cast(f16x4_t, bw), acc[2 * gp + (c >> 2)][c & 3], 0, 0, 0);
          }
        }
      }
    }
  }
  wait_vmcnt<0>();

  // ---- merge the four waves' states; wave w writes columns [128 w, 128 w + 128)
  const float l_row = row_sum4(l_run);
  const float off_row = row_sum4(off);
  if (kg == 0) {
    st_m[wave][n] = m_run;
    st_l[wave][n] = l_row;
    st_o[wave][n] = off_row;
    st_g[wave][n] = ge;
  }
  const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;
  // every loop has ended: the rings and the query operands are free. Each
  // wave's raw accumulators go to kQAcc * wave, lane-major (entry (g, c) of
  // lane l at 16 (64 (4 g + c) + l)); the reader applies the streams' factors.
  {
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(lbase + wave * kQAcc) + lane;
#pragma unroll
    for (int g = 0; g < kFB; ++g)
#pragma unroll
      for (int c = 0; c < 4; ++c) dst[64 * (4 * g + c)] = acc[g][c];
  }
  __syncthreads();
  const float nanv = __int_as_float(0x7fc00000);
  // per output row 4 kg + r: each wave's factor 2^(m_w - m_all) for l and
  // sum_t p_t min_t, the same with 2^(24 - ge_w) for its accumulators, 1 / l
  float fw[kWaves][4], inv[4], base[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = 4 * kg + r;
    float mr = st_m[0][rr];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) mr = fmaxf(mr, st_m[w][rr]);
    float lr = 0.0f, orr = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = st_m[w][rr];
      const float f = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - mr);
      fw[w][r] = ldexpf(f, 24 - st_g[w][rr]);
      lr = fmaf(st_l[w][rr], f, lr);
      orr = fmaf(st_o[w][rr], f, orr);
    }
    inv[r] = lr > 0.0f ? 1.0f / lr : 0.0f;
    base[r] = orr;
  }
  // an empty partition (no tokens) leaves its o_part rows unwritten; wave w
  // writes columns [128 w, 128 w + 128)
  if (t1 > t0 || any_bad) {
#pragma unroll
    for (int gg = 0; gg < 2; ++gg) {
      const int g = 2 * wave + gg;
      f32x4_t sum[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sum[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const f32x4_t v =
              reinterpret_cast<const f32x4_t*>(lbase + w * kQAcc)[64 * (4 * g + c) + lane];
#pragma unroll
          for (int r = 0; r < 4; ++r) sum[c][r] = fmaf(fw[w][r], v[r], sum[c][r]);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int orow = row0 + 4 * kg + r;
        const int col = kBits == 8 ? 64 * g + 4 * n : 128 * (g >> 1) + 8 * n + 4 * (g & 1);
        float* dst = o_part + (((size_t)b * R + orow) * S + s) * kDC + col;
        float4 v = make_float4((sum[0][r] + base[r]) * inv[r], (sum[1][r] + base[r]) * inv[r],
                               (sum[2][r] + base[r]) * inv[r], (sum[3][r] + base[r]) * inv[r]);
        if (any_bad) v = make_float4(nanv, nanv, nanv, nanv);
        *reinterpret_cast<float4*>(dst) = v;
      }
    }
  }
  if (wave == 0 && kg == 0) {
    float m_all = st_m[0][n];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m_all = fmaxf(m_all, st_m[w][n]);
    float l_all = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = st_m[w][n];
      l_all = fmaf(st_l[w][n], mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - m_all), l_all);
    }
    const float lse = l_all > 0.0f ? (m_all + log2f(l_all)) * 0.69314718055994531f : -INFINITY;
    lse_part[((size_t)b * R + row0 + n) * S + s] = any_bad ? nanv : lse;
  }
}

bool decode_q8_ok(const Shape& s, int q_len) {
  return s.dtype == 1 && s.dc == kDC && s.dr == kD - kDC && s.page % 64 == 0 &&
         (q_len * s.H) % 16 == 0;
}

template <int kBits>
static int launch_decode_qn(const Shape& s, int batch, int q_len, int num_splits,
                            int max_seq_len, const void* q_full, const void* cache,
                            int64_t num_pages, const int32_t* page_table, int max_pages,
                            const int32_t* seq_lens, const int32_t* tree_parent, float* o_part,
                            float* lse_part, void* stream) {
  constexpr size_t kLds = QFmt<kBits>::kLds;
  if (int e = set_max_lds(reinterpret_cast<const void*>(decode_q8_kernel<kBits>), (int)kLds))
    return e;
  const int units = batch * num_splits;
  const int groups = q_len * s.H / 16;
  const int blocks = grid_blocks(units, groups);
  hipLaunchKernelGGL(decode_q8_kernel<kBits>, dim3(blocks), dim3(256), kLds,
                     reinterpret_cast<hipStream_t>(stream), q_len, s.H, num_splits, s.page,
                     s.split_fixed, max_seq_len, s.scale * 1.4426950408889634f, units, groups,
                     (const bf16_t*)q_full, (const uint8_t*)cache, num_pages, page_table,
                     max_pages, seq_lens, tree_parent, o_part, lse_part);
  return (int)hipGetLastError();
}

int launch_decode_q8(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                     const void* q_full, const void* cache, int64_t num_pages,
                     const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                     const int32_t* tree_parent, float* o_part, float* lse_part, void* stream) {
  return launch_decode_qn<8>(s, batch, q_len, num_splits, max_seq_len, q_full, cache, num_pages,
                             page_table, max_pages, seq_lens, tree_parent, o_part, lse_part,
                             stream);
}

int launch_decode_q4(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                     const void* q_full, const void* cache, int64_t num_pages,
                     const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                     const int32_t* tree_parent, float* o_part, float* lse_part, void* stream) {
  return launch_decode_qn<4>(s, batch, q_len, num_splits, max_seq_len, q_full, cache, num_pages,
                             page_table, max_pages, seq_lens, tree_parent, o_part, lse_part,
                             stream);
}

}  // namespace mla
