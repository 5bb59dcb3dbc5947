// Split-KV paged MLA decode on bf16 MFMA, 64 query rows per block with
// specialised waves (e.g. DeepSeek-V2's 128 heads), gfx950.
//
// Same computation as the other decode kernels ("The Architecture of Memory",
// "Flash-Decoding and FlashInfer"; "DeepSeek's Config Says 16 KV Heads",
// section 5). At 64+ query rows per cached row the kernel is bound by how
// fast its waves feed the MFMA units from LDS, so the work is split to read
// each staged byte as few times as possible, and each SIMD runs two waves
// with different jobs whose LDS reads and MFMAs interleave:
//
//   QK wave (0..3)   rows [32 rh, 32 rh + 32), tokens [16 u, 16 u + 16) of
//                    each 32-token tile (rh = w & 1, u = w >> 1): holds its 32
//                    query rows in registers and scores its 16 tokens over all
//                    576 columns (18 k-steps x 2 row groups of
//                    v_mfma_f32_16x16x32_bf16, one LDS read per k-step serving
//                    both row groups, read 6 k-steps ahead); leaves the fp32
//                    scores in LDS. It also copies rows [8 w, 8 w + 8) of
//                    every tile into LDS (direct-to-LDS loads), one load after
//                    every second k-step of the scores two tiles earlier, so
//                    the load issue overlaps the MFMAs
//   PV wave (4..7)   rows [32 rh, 32 rh + 32), latent columns [256 fh,
//                    256 fh + 256) (rh = w & 1, fh = w >> 1): reads the scores
//                    of its rows, runs the online softmax (row max with two
//                    lane swaps; the reference max is raised only when a score
//                    exceeds it by more than 2^8, so the accumulator rescale
//                    almost never runs) and adds P.C (K = 32 tokens: P goes
//                    from the score layout straight into the A operand; the B
//                    operand, 8 tokens of one column per lane, comes from two
//                    transposing LDS reads, ds_read_b64_tr_b16, and serves
//                    both row groups)
//
// Per tile the block reads 72 KB of cache operands for the scores, 64 KB for
// P.C and 16 KB of scores from LDS (against 4 x 36 KB + 4 x 32 KB when every
// wave handles 16 rows of both contractions). The scores of tile k+1 are
// computed in the same step as the softmax and P.C of tile k; tiles stream
// through a 4-slot LDS ring and one block barrier per tile covers the tile's
// arrival, the score hand-over and the reuse of the slot two tiles back.
// With a drafted tree (tree_parent, "Tree Attention Verification") a row sees
// the prefix and the drafted tokens on its query's branch; only tiles that
// reach the drafted tokens test the branch mask.
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
constexpr int kWScoreVecs = 2 * 2 * 2 * 64;            // [rh][u][rg][lane] f32x4 of one tile
constexpr size_t kWRingBytes = (size_t)kWRing * kWTChunks * 16;          // 147,456 B
constexpr size_t kWScoreBytes = (size_t)2 * kWScoreVecs * 16;            // 16,384 B
constexpr size_t kWLds = kWRingBytes + kWScoreBytes;                     // 163,840 B

static_assert(kWLds <= 160 * 1024, "LDS of one CU");

// RowDma::issue without the non-temporal hint: the other row groups of the
// same partition (blocks on the same XCD, at about the same point of the
// partition) read the same tiles, and lines kept in L2 serve them (reads fell
// from 1.18x to 1.03x of the cache bytes at 128 heads)
template <int N>
__device__ __forceinline__ void issue_one_temporal(const RowDma<N>& d, const void* src,
                                                   uint32_t lds_base, int i) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_base + i * 1024), "v"(d.off[i]), "s"(src)
               : "memory");
}
template <int N>
__device__ __forceinline__ void issue_temporal(const RowDma<N>& d, const void* src,
                                               uint32_t lds_base) {
#pragma unroll
  for (int i = 0; i < N; ++i) issue_one_temporal(d, src, lds_base, i);
}

}  // namespace

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_ws_kernel(int Q, int H, int S, int page, int fixed, int max_seq_len,
                      float scale_log2, int units, int groups, const bf16_t* __restrict__ q_full,
                      const bf16_t* __restrict__ cache, int64_t num_pages,
                      const int32_t* __restrict__ page_table, int max_pages,
                      const int32_t* __restrict__ seq_lens,
                      const int32_t* __restrict__ tree_parent, float* __restrict__ o_part,
                      float* __restrict__ lse_part) {
  extern __shared__ u32x4_t lds[];
  int unit, grp;
  if (!map_block(units, groups, &unit, &grp)) return;
  const int R = Q * H;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int w4 = wave & 3;
  const int rh = w4 & 1;                // row half of the block (both roles)
  const bool qk_role = wave < 4;
  const int n = lane & 15, kg = lane >> 4;
  const int s = unit % S;
  int L;
  const int b = seq_by_rank(seq_lens, units / S, unit / S, lane, &L);
  const int row0 = grp * kWRows + 32 * rh;  // first of this wave's 32 query rows

  // scores of tile k: buffer k & 1, f32x4 index ((rh * 2 + u) * 2 + rg) * 64 + lane
  f32x4_t* sbuf = reinterpret_cast<f32x4_t*>(reinterpret_cast<char*>(lds) + kWRingBytes);
  auto slot = [&](int k) { return lds + (k & (kWRing - 1)) * kWTChunks; };

  const int32_t* par = tree_parent ? tree_parent + (size_t)b * Q : nullptr;
  // a malformed tree makes the sequence invalid (the same decision in every wave)
  const bool bad_tree = par && !__all(lane >= Q || tree_entry_ok(par, lane));
  const bool bad_len = (L < Q) || (L > max_seq_len) || bad_tree;
  int t0 = 0, t1 = 0;
  if (!bad_len) split_range(L, S, page, fixed, s, &t0, &t1);
  const int ntiles =
      tiles_needed(t0, t1, kWT, par != nullptr, L - Q, (grp * kWRows + kWRows - 1) / H);
  auto tstart = [&](int k) { return t0 + k * kWT; };
  // after the last tile the score buffer of step ntiles & 1 carries the QK
  // waves' out-of-range flags
  int* flags = reinterpret_cast<int*>(sbuf + (ntiles & 1) * kWScoreVecs);

  if (qk_role) {
    // ======================== QK waves ========================
    const int u = w4 >> 1;
    bool bad = bad_len;
    PageWindow pw;
    pw.init(page_table + (size_t)b * max_pages + t0 / page, (t1 - t0 + page - 1) / page, lane);
    settle(pw.reg);
    RowDma<kWPartLoads> dma;
    dma.init(w4 * kWPartChunks, lane, w4 * kWPartRows);
    // rows [8 w, 8 w + 8) of tile k (never across a page: 8 | page)
    auto issue = [&](int k) {
      const int t = tstart(k) + w4 * kWPartRows;
      int pg = pw.get((t - t0) / page, lane);
      if (pg < 0 || (int64_t)pg >= num_pages) {
        bad = true;
        pg = 0;
      }
      const bf16_t* src = cache + ((size_t)pg * page + (t % page)) * kD;
      issue_temporal(dma, src, __builtin_amdgcn_readfirstlane(lds_addr(slot(k) + w4 * kWPartChunks)));
    };
    const int pre = min(ntiles, kWRing - 1);
    if (pre > 0) issue(0);
    if (pre > 1) issue(1);
    if (pre > 2) issue(2);
    // query rows row0 + 16 rg + n, chunk 4 ks + kg (the B operand of k-step ks)
    bf16x8_t qreg[2][kKSteps];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const u32x4_t* qsrc =
          reinterpret_cast<const u32x4_t*>(q_full + ((size_t)b * R + row0 + 16 * rg + n) * kD);
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks)
        qreg[rg][ks] = __builtin_bit_cast(bf16x8_t, qsrc[ks * 4 + kg]);
    }
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) settle(qreg[rg][ks]);  // (also lands tiles 0..2)
    const int arow = (16 * u + n) * kChunks;  // A operand: token 16 u + n of the tile

    // scores of tokens [16 u, 16 u + 16) of tile k for the wave's 32 rows;
    // kiss >= 0: the copy of this wave's rows of tile kiss is issued between
    // the MFMAs (load i after k-step 2 i + 1)
    auto qk = [&](int k, int kiss) {
      const u32x4_t* buf = slot(k) + arow;
      constexpr int kAhead = 6;  // k-steps of A operand in flight
      u32x4_t a[kKSteps];
#pragma unroll
      for (int ks = 0; ks < kAhead; ++ks) a[ks] = buf[(4 * ks + kg) ^ (n & 7)];
      const bf16_t* isrc = cache;
      uint32_t ilds = 0;
      if (kiss >= 0) {
        const int t = tstart(kiss) + w4 * kWPartRows;
        int pg = pw.get((t - t0) / page, lane);
        if (pg < 0 || (int64_t)pg >= num_pages) {
          bad = true;
          pg = 0;
        }
        isrc = cache + ((size_t)pg * page + (t % page)) * kD;
        ilds = __builtin_amdgcn_readfirstlane(lds_addr(slot(kiss) + w4 * kWPartChunks));
      }
      f32x4_t c[2][2];
#pragma unroll
      for (int rg = 0; rg < 2; ++rg) c[rg][0] = c[rg][1] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < kKSteps; ++ks) {
        if (ks + kAhead < kKSteps) a[ks + kAhead] = buf[(4 * (ks + kAhead) + kg) ^ (n & 7)];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
          c[rg][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, a[ks]), qreg[rg][ks], c[rg][ks & 1], 0, 0, 0);
        if ((ks & 1) && kiss >= 0) {  // keep each load between its MFMAs
          __builtin_amdgcn_sched_barrier(0);
          issue_one_temporal(dma, isrc, ilds, ks >> 1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      f32x4_t* dst = sbuf + (k & 1) * kWScoreVecs + (rh * 2 + u) * 128 + lane;
      dst[0] = c[0][0] + c[0][1];
      dst[64] = c[1][0] + c[1][1];
    };

    if (ntiles > 0) {
      if (pre == 3)
        wait_vmcnt<2 * kWPartLoads>();
      else if (pre == 2)
        wait_vmcnt<kWPartLoads>();
      else
        wait_vmcnt<0>();
      if (tstart(0) + kWT > t1)
        zero_rows<kWPartLoads>(slot(0) + w4 * kWPartChunks, w4 * kWPartChunks, lane,
                               t1 - tstart(0));
    }
    __syncthreads();  // tile 0 landed
    if (ntiles > 0) qk(0, -1);
    for (int k = 0; k < ntiles; ++k) {
      if (k + 1 < ntiles) {  // own part of tile k+1 (tile k+2 may stay in flight)
        if (k + 2 < ntiles)
          wait_vmcnt<kWPartLoads>();
        else
          wait_vmcnt<0>();
        const int ts1 = tstart(k + 1);
        if (ts1 + kWT > t1)
          zero_rows<kWPartLoads>(slot(k + 1) + w4 * kWPartChunks, w4 * kWPartChunks, lane,
                                 t1 - ts1);
      }
      // tile k+1 landed; the scores of tile k are handed over; slot k-1
      // (= k+3) and score buffer k+1 are no longer read
      __syncthreads();
      if (k + 1 < ntiles) qk(k + 1, k + 3 < ntiles ? k + 3 : -1);
    }
    wait_vmcnt<0>();
    if (lane == 0) flags[w4] = bad ? 1 : 0;
    __syncthreads();  // flags handed over
    return;
  }

  // ======================== PV waves ========================
  const int fh = w4 >> 1;
  // B operand of P.C for columns c0 .. c0 + 15 (lane n: column c0 + n; tokens
  // sigma(kg, j), the order of P in the A operand): in each 16-lane group a
  // transposing read hands lane 4a + b element b of the 8 bytes that lanes
  // a, a + 4, a + 8, a + 12 address, so lane s = a + 4 i of group kg reads
  // token 16 h + 4 kg + i, columns c0 + 4 a .. + 3. pvt[h][m]: byte offset for
  // half h and c0 = 256 fh + 16 m (+ 64 fb: + 128 bytes, within the swizzle)
  int pvt[2][4];
  {
    const int a = n & 3, i = n >> 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = 16 * h + 4 * kg + i;
#pragma unroll
      for (int m = 0; m < 4; ++m)
        pvt[h][m] = 16 * (t * kChunks + 32 * fh + ((2 * m + (a >> 1)) ^ (t & 7))) + 8 * (a & 1);
    }
  }
  auto bop = [&](uint32_t tbase, int fb, int m) {
    const s16x4_t lo = ds_read_tr16(tbase + pvt[0][m] + fb * 128);
    const s16x4_t hi = ds_read_tr16(tbase + pvt[1][m] + fb * 128);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  f32x4_t acc[2][kFB / 2][4];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int fb = 0; fb < kFB / 2; ++fb)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[rg][fb][m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
  // tokens each row of this lane sees in this partition: t <= lim, and with a
  // drafted tree also the drafted tokens (t >= t_draft) on its query's branch
  const int t_draft = L - Q;
  int lim[2];
  uint64_t branch[2];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int j = (row0 + 16 * rg + n) / H;
    lim[rg] = min(par ? t_draft - 1 : t_draft + j, t1 - 1);
    branch[rg] = (par && !bad_len) ? tree_branch_mask(par, Q, j) : 0ull;
  }

  __syncthreads();  // tile 0 landed
  for (int k = 0; k < ntiles; ++k) {
    __syncthreads();  // scores of tile k handed over
    const uint32_t tbase = lds_addr(slot(k));
    bf16x8_t bcur[4], bnxt[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) bcur[m] = bop(tbase, 0, m);

    // ---- online softmax of both row groups (lane: row n, tokens sigma(kg, j))
    const int ts = tstart(k);
    const f32x4_t* sk = sbuf + (k & 1) * kWScoreVecs + rh * 256 + lane;
    bf16x8_t pa[2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const f32x4_t s0 = sk[rg * 64];        // tokens 4 kg + r
      const f32x4_t s1 = sk[128 + rg * 64];  // tokens 16 + 4 kg + r
      float sv[8];
      // lane's tokens: ts + 4 kg + r (subtile 0) and ts + 16 + 4 kg + r (subtile 1)
      uint64_t vl = ~0ull;
      if (!__all(ts + kWT - 1 <= lim[rg]))
        vl = tile_visible(ts, lim[rg], t_draft, t1, branch[rg]) >> (4 * kg);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = ((vl >> r) & 1ull) ? s0[r] * scale_log2 : -INFINITY;
        sv[4 + r] = ((vl >> (16 + r)) & 1ull) ? s1[r] * scale_log2 : -INFINITY;
      }
      float mloc = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mloc = row_max4(mloc);
      const bool raise = mloc > m_run[rg] + kLazy;
      if (__any(raise)) {
        const float m_new = raise ? mloc : m_run[rg];
        const float alpha =
            (m_run[rg] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[rg] - m_new);
        l_run[rg] *= alpha;
        // the accumulators are still zero for rows whose max was -inf
        if (__any(raise && m_run[rg] != -INFINITY)) {
          float ar[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * kg + r, 64);
#pragma unroll
          for (int fb = 0; fb < kFB / 2; ++fb)
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[rg][fb][m][r] *= ar[r];
        }
        m_run[rg] = m_new;
      }
      const float m_use = (m_run[rg] == -INFINITY) ? 0.0f : m_run[rg];
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(sv[j] - m_use);
      l_run[rg] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      bf16x2_t p01 = {(__bf16)p[0], (__bf16)p[1]};
      bf16x2_t p23 = {(__bf16)p[2], (__bf16)p[3]};
      bf16x2_t p45 = {(__bf16)p[4], (__bf16)p[5]};
      bf16x2_t p67 = {(__bf16)p[6], (__bf16)p[7]};
      const u32x4_t pav = {__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23),
                           __builtin_bit_cast(uint32_t, p45), __builtin_bit_cast(uint32_t, p67)};
      pa[rg] = __builtin_bit_cast(bf16x8_t, pav);
    }

    // ---- P.C over this wave's 256 latent columns, 4 blocks of 64
#pragma unroll
    for (int fb = 0; fb < kFB / 2; ++fb) {
      if (fb + 1 < kFB / 2) {
#pragma unroll
        for (int m = 0; m < 4; ++m) bnxt[m] = bop(tbase, fb + 1, m);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
          acc[rg][fb][m] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[rg], bcur[m], acc[rg][fb][m], 0, 0, 0);
#pragma unroll
      for (int m = 0; m < 4; ++m) bcur[m] = bnxt[m];
    }
  }
  __syncthreads();  // flags handed over
  const bool any_bad = (flags[0] | flags[1] | flags[2] | flags[3]) != 0;
  const float nanv = __int_as_float(0x7fc00000);
  float l_row[2];  // row sums over the 4 lanes of each row (whole wave active)
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) l_row[rg] = row_sum4(l_run[rg]);
  // an empty partition (no tokens) leaves its o_part rows unwritten
  if (t1 > t0 || any_bad) {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      float inv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float lr = __shfl(l_row[rg], 4 * kg + r, 64);
        inv[r] = lr > 0.0f ? 1.0f / lr : 0.0f;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // row 4 kg + r, column 256 fh + 64 fb + 16 m + n
        const int orow = row0 + 16 * rg + 4 * kg + r;
        float* dst = o_part + (((size_t)b * R + orow) * S + s) * kDC + 256 * fh + n;
#pragma unroll
        for (int fb = 0; fb < kFB / 2; ++fb)
#pragma unroll
          for (int m = 0; m < 4; ++m)
            dst[64 * fb + 16 * m] = any_bad ? nanv : acc[rg][fb][m][r] * inv[r];
      }
    }
  }
  if (fh == 0 && kg == 0) {
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const float lse =
          l_row[rg] > 0.0f ? (m_run[rg] + log2f(l_row[rg])) * 0.69314718055994531f : -INFINITY;
      lse_part[((size_t)b * R + row0 + 16 * rg + n) * S + s] = any_bad ? nanv : lse;
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
                     const int32_t* tree_parent, float* o_part, float* lse_part, void* stream) {
  if (int e = set_max_lds(reinterpret_cast<const void*>(decode_ws_kernel), (int)kWLds)) return e;
  const int units = batch * num_splits;
  const int groups = q_len * s.H / kWRows;
  const int blocks = grid_blocks(units, groups);
  hipLaunchKernelGGL(decode_ws_kernel, dim3(blocks), dim3(512), kWLds,
                     reinterpret_cast<hipStream_t>(stream), q_len, s.H, num_splits, s.page,
                     s.split_fixed, max_seq_len, s.scale * 1.4426950408889634f, units, groups,
                     (const bf16_t*)q_full, (const bf16_t*)cache, num_pages, page_table, max_pages,
                     seq_lens, tree_parent, o_part, lse_part);
  return (int)hipGetLastError();
}

}  // namespace mla
