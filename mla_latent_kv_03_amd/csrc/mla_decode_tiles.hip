// Split-KV paged MLA decode on bf16 MFMA, 64 query rows per block (16 per
// wave; e.g. DeepSeek-V2's 128 heads), gfx950.
//
// Same computation as the 16-row kernel ("The Architecture of Memory",
// "Flash-Decoding and FlashInfer"; "DeepSeek's Config Says 16 KV Heads",
// section 5), laid out for many heads per cached row: the 4 waves share
// 64-token tiles in LDS (double-buffered, one block barrier per tile) and each
// wave owns 16 query rows, so every cached byte leaves HBM once per block
// however many heads there are, and the MFMA work per staged byte grows with
// the row count.
#include "mla_decode_common.h"
#include "mla_launch.h"

namespace mla {

using namespace dec;

namespace {

constexpr int kTile = 64;
constexpr int kTileChunks = kTile * kChunks;    // 4608 chunks = 73,728 B
constexpr size_t kLdsBytesB = (size_t)2 * kTileChunks * 16;                // 147,456 B

__device__ __forceinline__ void zero_acc(f32x4_t (*acc)[4]) {
#pragma unroll
  for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[fb][m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

}  // namespace

// ---------------------------------------------------------------------------
// 64 query rows per block (16 per wave) over shared 64-token tiles
//
// Per tile each wave runs three phases with no branch between the MFMAs of a
// phase, so the 4 independent QK chains and the 32 independent PV products
// overlap their LDS reads:
//   QK   S^T for the 4 16-token subtiles (4 x 18 v_mfma_f32_16x16x32_bf16)
//   max  row max over the 64 tokens (2 permlane swaps), rare rescale, P = 2^(s-m)
//   PV   two 32-token halves with v_mfma_f32_16x16x32_bf16 (K = 32 tokens):
//        the A operand takes the 8 tokens {4kg..4kg+3, 16+4kg..16+4kg+3} of
//        the half straight from two QK accumulators; the B operand gathers the
//        same 8 token rows (ds_read_b64, 4 features each) and transposes 8x4
//        in registers (v_perm_b32).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_tiles_kernel(int Q, int H, int S, int page, int fixed, int max_seq_len,
                         float scale_log2, int units, int groups,
                         const bf16_t* __restrict__ q_full,
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
  const int n = lane & 15, kg = lane >> 4;
  const int row0 = grp * 64 + wave * 16;
  const int s = unit % S;
  int L;
  const int b = seq_by_rank(seq_lens, units / S, unit / S, lane, &L);
  const bool bad_len = (L < Q) || (L > max_seq_len);
  int t0 = 0, t1 = 0;
  if (!bad_len) split_range(L, S, page, fixed, s, &t0, &t1);
  const int ntiles = (t1 - t0 + kTile - 1) / kTile;
  bool bad = bad_len;

  PageWindow pw;
  pw.init(page_table + (size_t)b * max_pages + t0 / page, (t1 - t0 + page - 1) / page, lane);
  settle(pw.reg);
  RowDma<> dma;
  dma.init(wave * kSliceChunks, lane);
  auto issue = [&](int ti, u32x4_t* dst) {
    const int t = t0 + ti * kTile;  // a tile never crosses a page: page % 64 == 0
    int pg = pw.get((t - t0) / page, lane);
    if (pg < 0 || (int64_t)pg >= num_pages) {
      bad = true;
      pg = 0;
    }
    // this wave copies tile rows [16*wave, 16*wave + 16)
    const bf16_t* src = cache + ((size_t)pg * page + (t % page)) * kD;
    dma.issue(src, __builtin_amdgcn_readfirstlane(lds_addr(dst + wave * kSliceChunks)));
  };
  if (ntiles > 0) issue(0, lds);  // the first tile loads while the queries are fetched

  bf16x8_t qreg[kKSteps];
  const int row = row0 + n;
  {
    const u32x4_t* qsrc = reinterpret_cast<const u32x4_t*>(q_full + ((size_t)b * R + row) * kD);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8_t, qsrc[ks * 4 + kg]);
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) settle(qreg[ks]);
  }
  const int p_lim = L - Q + row / H;

  // LDS addressing inside a tile: QK reads row 16u + n, chunk 4 ks + kg;
  // PV reads rows 32 v + sigma(kg, j), sigma = {4kg..4kg+3, 16+4kg..16+4kg+3}
  const int qk0 = n * kChunks + (kg ^ (n & 7));
  const int qk1 = n * kChunks + ((4 + kg) ^ (n & 7));
  int pv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int t = (j < 4) ? 4 * kg + j : 16 + 4 * kg + (j - 4);
    pv[j] = 16 * (t * kChunks + ((n >> 1) ^ (t & 7))) + 8 * (n & 1);
  }

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t acc[kFB][4];
  zero_acc(acc);

  for (int ti = 0; ti < ntiles; ++ti) {
    u32x4_t* cur = lds + (ti & 1) * kTileChunks;
    wait_vmcnt<0>();
    const int ts = t0 + ti * kTile;
    if (ts + kTile > t1)  // rows past the partition end (may be poison)
      zero_rows(cur + wave * kSliceChunks, wave * kSliceChunks, lane, t1 - ts);
    __syncthreads();  // tile ti landed for every wave; tile ti-1 fully consumed
    if (ti + 1 < ntiles) issue(ti + 1, lds + ((ti + 1) & 1) * kTileChunks);

    // ---- QK: 4 independent 18-step chains
    f32x4_t s4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) s4[u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // software pipeline: the 4 operands of k-step ks+1 are read while the 4
    // MFMAs of k-step ks issue (the scheduling barriers keep that order)
    u32x4_t a_cur[4], a_nxt[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a_cur[u] = cur[qk0 + u * kSliceChunks];
#pragma unroll
    for (int ks = 0; ks < kKSteps; ++ks) {
      if (ks + 1 < kKSteps) {
        const int kn = ks + 1;
        const int base = ((kn & 1) ? qk1 : qk0) + 8 * (kn >> 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) a_nxt[u] = cur[base + u * kSliceChunks];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        s4[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a_cur[u]),
                                                        qreg[ks], s4[u], 0, 0, 0);
      if (ks + 1 < kKSteps) {
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // then 4 MFMA
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) a_cur[u] = a_nxt[u];
    }
    // ---- softmax over the tile's 64 tokens (lane: row n, tokens 16u + 4kg + r)
    float sv[16];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = ts + 16 * u + 4 * kg + r;
        sv[4 * u + r] = (t <= p_lim) ? s4[u][r] * scale_log2 : -INFINITY;
      }
    float mloc = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mloc = fmaxf(mloc, sv[i]);
    mloc = row_max4(mloc);
    const bool raise = mloc > m_run + kLazy;
    if (__any(raise)) {
      const float m_new = raise ? mloc : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
      if (__any(raise && m_run != -INFINITY)) {
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kg + r, 64);
#pragma unroll
        for (int fb = 0; fb < kFB; ++fb)
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[fb][m][r] *= ar[r];
      }
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
    float lsum = 0.0f;
    uint32_t pk[8];  // P as bf16 pairs: half v, tokens sigma(kg, 0..7)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int u = 2 * v + h;
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = __builtin_amdgcn_exp2f(sv[4 * u + r] - m_use);
          lsum += p[r];
        }
        bf16x2_t p01 = {(__bf16)p[0], (__bf16)p[1]};
        bf16x2_t p23 = {(__bf16)p[2], (__bf16)p[3]};
        pk[4 * v + 2 * h] = __builtin_bit_cast(uint32_t, p01);
        pk[4 * v + 2 * h + 1] = __builtin_bit_cast(uint32_t, p23);
      }
    l_run += lsum;
    // ---- PV: two 32-token halves, K = 32; the 8 rows of step it+1 are read
    // while step it is transposed and multiplied
    const char* tb = reinterpret_cast<const char*>(cur);
    bf16x8_t pa[2];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      u32x4_t pav = {pk[4 * v], pk[4 * v + 1], pk[4 * v + 2], pk[4 * v + 3]};
      pa[v] = __builtin_bit_cast(bf16x8_t, pav);
    }
    u32x2_t xa[8], xb[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xa[j] = *reinterpret_cast<const u32x2_t*>(tb + pv[j]);
#pragma unroll
    for (int it = 0; it < 2 * kFB; ++it) {
      const int v = it / kFB, fb = it % kFB;
      if (it + 1 < 2 * kFB) {
        const int vn = (it + 1) / kFB, fn = (it + 1) % kFB;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          xb[j] = *reinterpret_cast<const u32x2_t*>(tb + pv[j] + vn * (32 * kChunks * 16) + fn * 128);
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
            pa[v], __builtin_bit_cast(bf16x8_t, bm[m]), acc[fb][m], 0, 0, 0);
      if (it + 1 < 2 * kFB) {
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);   // next step's LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 1);  // this step's transposes
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 1);   // this step's MFMAs
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) xa[j] = xb[j];
    }
  }
  wait_vmcnt<0>();

  // ---- write this wave's 16 rows ------------------------------------------
  const float nanv = __int_as_float(0x7fc00000);
  const float l_row = row_sum4(l_run);
  float inv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float lr = __shfl(l_row, 4 * kg + r, 64);
    inv[r] = lr > 0.0f ? 1.0f / lr : 0.0f;
  }
  // an empty partition (no tokens) leaves its o_part rows unwritten
#pragma unroll
  for (int r = 0; r < 4 && (t1 > t0 || bad); ++r) {
    const int orow = row0 + 4 * kg + r;
    float* dst = o_part + (((size_t)b * R + orow) * S + s) * kDC + 4 * n;
#pragma unroll
    for (int fb = 0; fb < kFB; ++fb) {
      float4 v = make_float4(acc[fb][0][r] * inv[r], acc[fb][1][r] * inv[r],
                             acc[fb][2][r] * inv[r], acc[fb][3][r] * inv[r]);
      if (bad) v = make_float4(nanv, nanv, nanv, nanv);
      *reinterpret_cast<float4*>(dst + fb * 64) = v;
    }
  }
  if (kg == 0) {
    const float lse = l_row > 0.0f ? (m_run + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
    lse_part[((size_t)b * R + row) * S + s] = bad ? nanv : lse;
  }
}

bool decode_tiles_ok(const Shape& s, int q_len) {
  return s.dtype == 1 && s.dc == kDC && s.dr == kD - kDC && s.page % kTile == 0 &&
         (q_len * s.H) % 64 == 0;
}

int launch_decode_tiles(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                        const void* q_full, const void* cache, int64_t num_pages,
                        const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                        float* o_part, float* lse_part, void* stream) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(decode_tiles_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytesB);
    if (e != hipSuccess) return (int)e;
    attr = true;
  }
  const int units = batch * num_splits;
  const int groups = q_len * s.H / 64;
  const int blocks = ((units + 7) / 8) * 8 * groups;
  hipLaunchKernelGGL(decode_tiles_kernel, dim3(blocks), dim3(256), kLdsBytesB,
                     reinterpret_cast<hipStream_t>(stream), q_len, s.H, num_splits, s.page,
                     s.split_fixed, max_seq_len, s.scale * 1.4426950408889634f, units, groups,
                     (const bf16_t*)q_full, (const bf16_t*)cache, num_pages, page_table, max_pages,
                     seq_lens, o_part, lse_part);
  return (int)hipGetLastError();
}

}  // namespace mla
