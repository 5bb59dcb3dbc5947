// Split-KV paged MLA decode on bf16 MFMA, 64 query rows per block with
// specialised waves (e.g. DeepSeek-V2's 128 heads), gfx950.
//
// Same computation as the other decode kernels ("The Architecture of Memory",
// "Flash-Decoding and FlashInfer"; "DeepSeek's Config Says 16 KV Heads",
// section 5). At 64+ query rows per cached row the kernel is bound by how
// its waves feed the MFMA units from LDS, and within one wave the operand
// reads and the MFMAs barely overlap. So each SIMD runs two waves with
// different jobs on the same 16 query rows, and their phases interleave:
//
//   QK wave q (0..3)    copies rows [8q, 8q + 8) of every 32-token tile into
//                       LDS (direct-to-LDS loads); scores tile k+1 for its 16
//                       rows (2 subtiles x 18 v_mfma_f32_16x16x32_bf16, query
//                       in registers), runs the online softmax (row max with
//                       two lane swaps, lazy rescale: the reference max is
//                       raised only when a score exceeds it by more than 2^8)
//                       and leaves P (bf16, already in PV A-operand order) and
//                       the rescale factors in LDS
//   PV wave 4 + q       rescales its accumulators when told to and adds P.C
//                       of tile k over all 512 latent columns (8 x 4
//                       v_mfma_f32_16x16x32_bf16, K = 32 tokens; the B
//                       operand gathers 4 columns of 8 token rows with
//                       ds_read_b64 and transposes them in registers)
//
// Waves q and 4 + q sit on the same SIMD. Tiles stream through a 4-slot LDS
// ring; one block barrier per tile covers the tile's arrival, the P hand-over
// and the reuse of the slot two tiles back.
#include "mla_decode_common.h"
#include "mla_launch.h"

namespace mla {

using namespace dec;

namespace {

constexpr int kWRows = 64;                             // query rows per block
constexpr int kWT = 32;                                // tokens per tile
constexpr int kWTChunks = kWT * kChunks;               // 2304 chunks = 36,864 B
constexpr int kWRing = 4;
constexpr int kWPartRows = kWT / 4;                    // 8 tile rows copied per QK wave
constexpr int kWPartChunks = kWPartRows * kChunks;     // 576 chunks
constexpr int kWPartLoads = kWPartChunks / 64;         // 9 loads
constexpr size_t kWRingBytes = (size_t)kWRing * kWTChunks * 16;          // 147,456 B
constexpr size_t kWPBytes = (size_t)2 * 4 * 64 * 16;                     // P hand-over: 8,192 B
constexpr size_t kWAlphaBytes = (size_t)2 * 4 * 16 * 4;                  // rescale factors: 512 B
constexpr size_t kWFlagBytes = 64;                                       // rescale flags, m/l
constexpr size_t kWLds = kWRingBytes + kWPBytes + kWAlphaBytes + 4 * 16 * 8 + kWFlagBytes;

static_assert(kWLds <= 160 * 1024, "LDS of one CU");

}  // namespace

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_ws_kernel(int Q, int H, int S, int page, int fixed, int max_seq_len,
                      float scale_log2, int units, int groups, const bf16_t* __restrict__ q_full,
                      const bf16_t* __restrict__ cache, int64_t num_pages,
                      const int32_t* __restrict__ page_table, int max_pages,
                      const int32_t* __restrict__ seq_lens, float* __restrict__ o_part,
                      float* __restrict__ lse_part) {
  extern __shared__ u32x4_t lds[];
  int unit, grp;
  if (!map_block(units, groups, &unit, &grp)) return;
  const int R = Q * H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int q4 = wave & 3;              // the 16-row group of this wave
  const bool qk_role = wave < 4;
  const int n = lane & 15, kg = lane >> 4;
  const int s = unit % S;
  int L;
  const int b = seq_by_rank(seq_lens, units / S, unit / S, lane, &L);
  const int row = grp * kWRows + q4 * 16 + n;  // this lane's query row

  char* xb = reinterpret_cast<char*>(lds) + kWRingBytes;
  u32x4_t* ex_p = reinterpret_cast<u32x4_t*>(xb);                       // [2][4][64]
  float* ex_a = reinterpret_cast<float*>(xb + kWPBytes);                // [2][4][16]
  float* ex_ml = ex_a + 2 * 4 * 16;                                     // [4][16][2]
  int* ex_f = reinterpret_cast<int*>(ex_ml + 4 * 16 * 2);               // [2][4] rescale flags
  auto slot = [&](int k) { return lds + (k & (kWRing - 1)) * kWTChunks; };

  const bool bad_len = (L < Q) || (L > max_seq_len);
  int t0 = 0, t1 = 0;
  if (!bad_len) split_range(L, S, page, fixed, s, &t0, &t1);
  const int ntiles = (t1 - t0 + kWT - 1) / kWT;
  bool bad = bad_len;
  const int p_lim = L - Q + row / H;
  const int lim = min(p_lim, t1 - 1);  // last token this row may see in this partition
  const float nanv = __int_as_float(0x7fc00000);

  if (qk_role) {
    // ======================== QK waves ========================
    PageWindow pw;
    pw.init(page_table + (size_t)b * max_pages + t0 / page, (t1 - t0 + page - 1) / page, lane);
    settle(pw.reg);
    RowDma<kWPartLoads> dma;
    dma.init(q4 * kWPartChunks, lane, q4 * kWPartRows);
    // rows [8 q4, 8 q4 + 8) of tile k (never across a page: 8 | page)
    auto issue = [&](int k) {
      const int t = t0 + k * kWT + q4 * kWPartRows;
      int pg = pw.get((t - t0) / page, lane);
      if (pg < 0 || (int64_t)pg >= num_pages) {
        bad = true;
        pg = 0;
      }
      const bf16_t* src = cache + ((size_t)pg * page + (t % page)) * kD;
      dma.issue(src, __builtin_amdgcn_readfirstlane(lds_addr(slot(k) + q4 * kWPartChunks)));
    };
    const int pre = min(ntiles, kWRing - 1);
    if (pre > 0) issue(0);
    if (pre > 1) issue(1);
    if (pre > 2) issue(2);
    bf16x8_t qreg[kKSteps];
    {
      const u32x4_t* qsrc = reinterpret_cast<const u32x4_t*>(q_full + ((size_t)b * R + row) * kD);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8_t, qsrc[ks * 4 + kg]);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) settle(qreg[ks]);  // (also lands tiles 0..2)
    }
    const int qk0 = n * kChunks + (kg ^ (n & 7));
    const int qk1 = n * kChunks + ((4 + kg) ^ (n & 7));
    float m_run = -INFINITY, l_run = 0.0f;

    // scores of tile k -> P and rescale factors into hand-over buffer k & 1
    auto qk_softmax = [&](int k) {
      const u32x4_t* buf = slot(k);
      f32x4_t c[2][2];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) c[uu][0] = c[uu][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
      u32x4_t a_cur[2], a_nxt[2];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) a_cur[uu] = buf[qk0 + uu * kSliceChunks];
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks + 1 < kKSteps) {
          const int kn = ks + 1;
          const int base = ((kn & 1) ? qk1 : qk0) + 8 * (kn >> 1);
#pragma unroll
          for (int uu = 0; uu < 2; ++uu) a_nxt[uu] = buf[base + uu * kSliceChunks];
        }
#pragma unroll
        for (int uu = 0; uu < 2; ++uu)
          c[uu][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, a_cur[uu]), qreg[ks], c[uu][ks & 1], 0, 0, 0);
        if (ks + 1 < kKSteps) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // then 2 MFMA
        }
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) a_cur[uu] = a_nxt[uu];
      }
      const int ts = t0 + k * kWT;
      float sv[8];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const f32x4_t sc = c[uu][0] + c[uu][1];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sv[4 * uu + r] = (ts + 16 * uu + 4 * kg + r <= lim) ? sc[r] * scale_log2 : -INFINITY;
      }
      float mloc = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mloc = row_max4(mloc);
      const bool raise = mloc > m_run + kLazy;
      int flag = 0;
      float alpha = 1.0f;
      if (__any(raise)) {
        const float m_new = raise ? mloc : m_run;
        alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        // the accumulators are still zero for rows whose max was -inf
        flag = __any(raise && m_run != -INFINITY) ? 1 : 0;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(sv[j] - m_use);
      l_run += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      bf16x2_t p01 = {(__bf16)p[0], (__bf16)p[1]};
      bf16x2_t p23 = {(__bf16)p[2], (__bf16)p[3]};
      bf16x2_t p45 = {(__bf16)p[4], (__bf16)p[5]};
      bf16x2_t p67 = {(__bf16)p[6], (__bf16)p[7]};
      ex_p[((k & 1) * 4 + q4) * 64 + lane] =
          u32x4_t{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23),
                  __builtin_bit_cast(uint32_t, p45), __builtin_bit_cast(uint32_t, p67)};
      if (kg == 0) ex_a[((k & 1) * 4 + q4) * 16 + n] = alpha;
      if (lane == 0) ex_f[(k & 1) * 4 + q4] = flag;
    };

    if (ntiles > 0) {
      if (pre == 3)
        wait_vmcnt<2 * kWPartLoads>();
      else if (pre == 2)
        wait_vmcnt<kWPartLoads>();
      else
        wait_vmcnt<0>();
      if (t0 + kWT > t1)
        zero_rows<kWPartLoads>(slot(0) + q4 * kWPartChunks, q4 * kWPartChunks, lane, t1 - t0);
    }
    __syncthreads();  // tile 0 landed
    if (ntiles > 0) qk_softmax(0);
    for (int k = 0; k < ntiles; ++k) {
      if (k + 1 < ntiles) {  // own part of tile k+1 (tile k+2 may stay in flight)
        if (k + 2 < ntiles)
          wait_vmcnt<kWPartLoads>();
        else
          wait_vmcnt<0>();
        const int ts1 = t0 + (k + 1) * kWT;
        if (ts1 + kWT > t1)
          zero_rows<kWPartLoads>(slot(k + 1) + q4 * kWPartChunks, q4 * kWPartChunks, lane, t1 - ts1);
      }
      // tile k+1 landed; P of tile k is handed over; slot k-1 (= k+3) is free
      __syncthreads();
      if (k + 3 < ntiles) issue(k + 3);
      if (k + 1 < ntiles) qk_softmax(k + 1);
    }
    wait_vmcnt<0>();
    const float l_row = row_sum4(l_run);
    if (kg == 0) {
      ex_ml[(q4 * 16 + n) * 2] = m_run;
      ex_ml[(q4 * 16 + n) * 2 + 1] = l_row;
    }
    const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;  // m, l handed over
    if (kg == 0) {
      const float lse = l_row > 0.0f ? (m_run + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
      lse_part[((size_t)b * R + row) * S + s] = any_bad ? nanv : lse;
    }
  } else {
    // ======================== PV waves ========================
    int pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = (j < 4) ? 4 * kg + j : 16 + 4 * kg + (j - 4);
      pv[j] = 16 * (t * kChunks + ((n >> 1) ^ (t & 7))) + 8 * (n & 1);
    }
    f32x4_t acc[kFB][4];
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[fb][m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    __syncthreads();  // tile 0 landed
    for (int k = 0; k < ntiles; ++k) {
      __syncthreads();  // P of tile k handed over
      if (ex_f[(k & 1) * 4 + q4]) {
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = ex_a[((k & 1) * 4 + q4) * 16 + 4 * kg + r];
#pragma unroll
        for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[fb][m][r] *= ar[r];
      }
      const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, ex_p[((k & 1) * 4 + q4) * 64 + lane]);
      const char* tb = reinterpret_cast<const char*>(slot(k));
      u32x2_t xa[8], xn[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xa[j] = *reinterpret_cast<const u32x2_t*>(tb + pv[j]);
#pragma unroll
      for (int fb = 0; fb < kFB; ++fb) {
        if (fb + 1 < kFB) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            xn[j] = *reinterpret_cast<const u32x2_t*>(tb + pv[j] + (fb + 1) * 128);
        }
        u32x4_t bm[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          bm[0][q2] = pack_lo(xa[2 * q2].x, xa[2 * q2 + 1].x);
          bm[1][q2] = pack_hi(xa[2 * q2].x, xa[2 * q2 + 1].x);
          bm[2][q2] = pack_lo(xa[2 * q2].y, xa[2 * q2 + 1].y);
          bm[3][q2] = pack_hi(xa[2 * q2].y, xa[2 * q2 + 1].y);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[fb][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              pa, __builtin_bit_cast(bf16x8_t, bm[m]), acc[fb][m], 0, 0, 0);
        if (fb + 1 < kFB) {
          __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);   // next block's LDS reads
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 1);  // this block's transposes
          __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);   // this block's MFMAs
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) xa[j] = xn[j];
      }
    }
    const bool any_bad = __syncthreads_or(0) != 0;  // m, l handed over
    float inv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float lr = ex_ml[(q4 * 16 + 4 * kg + r) * 2 + 1];
      inv[r] = lr > 0.0f ? 1.0f / lr : 0.0f;
    }
    // an empty partition (no tokens) leaves its o_part rows unwritten
#pragma unroll
    for (int r = 0; r < 4 && (t1 > t0 || any_bad); ++r) {
      const int orow = grp * kWRows + q4 * 16 + 4 * kg + r;
      float* dst = o_part + (((size_t)b * R + orow) * S + s) * kDC + 4 * n;
#pragma unroll
      for (int fb = 0; fb < kFB; ++fb) {
        float4 v = make_float4(acc[fb][0][r] * inv[r], acc[fb][1][r] * inv[r],
                               acc[fb][2][r] * inv[r], acc[fb][3][r] * inv[r]);
        if (any_bad) v = make_float4(nanv, nanv, nanv, nanv);
        *reinterpret_cast<float4*>(dst + fb * 64) = v;
      }
    }
  }
}

bool decode_ws_ok(const Shape& s, int q_len) {
  return s.dtype == 1 && s.dc == kDC && s.dr == kD - kDC && s.page % kWPartRows == 0 &&
         (q_len * s.H) % kWRows == 0;
}

int launch_decode_ws(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                     const void* q_full, const void* cache, int64_t num_pages,
                     const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                     float* o_part, float* lse_part, void* stream) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_ws_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWLds);
    if (e != hipSuccess) return (int)e;
    attr = true;
  }
  const int units = batch * num_splits;
  const int groups = q_len * s.H / kWRows;
  const int blocks = ((units + 7) / 8) * 8 * groups;
  hipLaunchKernelGGL(decode_ws_kernel, dim3(blocks), dim3(512), kWLds,
                     reinterpret_cast<hipStream_t>(stream), q_len, s.H, num_splits, s.page,
                     s.split_fixed, max_seq_len, s.scale * 1.4426950408889634f, units, groups,
                     (const bf16_t*)q_full, (const bf16_t*)cache, num_pages, page_table, max_pages,
                     seq_lens, o_part, lse_part);
  return (int)hipGetLastError();
}

}  // namespace mla
