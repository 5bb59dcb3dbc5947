// Split-KV paged MLA decode on bf16 MFMA, 16 query rows per block (e.g.
// DeepSeek-V2-Lite's 16 heads at one query token), gfx950.
//
// What it computes ("The Architecture of Memory", "Flash-Decoding and
// FlashInfer", "The Decode Phase: The Memory Bandwidth Wall"; "DeepSeek's
// Config Says 16 KV Heads", section 5): every query row (query j, head h)
// scores its absorbed query q_full (576 wide) against every cached row of its
// partition, softmaxes the scores online, and weights the 512 latent columns
// of the same rows. All heads read the same cached rows, so one staged tile
// serves all 16 query rows.
//
// The partition streams through a ring of four 32-token tiles in LDS, one
// block barrier per tile. The 8 waves divide each tile's work instead of
// taking separate tiles, so they stay in step and nothing is merged at the
// end; waves 0-3 score, waves 4-7 run the softmax and P.V, and wave w shares a
// SIMD with wave w + 4, so one's MFMAs run under the other's vector work:
//   QK   wave w < 4 copies rows [8 w, 8 w + 8) of every tile into the ring and
//        scores 16-token subtile (w & 1) of the tile over half (w >> 1) of the
//        576 columns (9 v_mfma_f32_16x16x32_bf16, M = tokens, N = 16 rows),
//        leaving the partial S^T in LDS;
//   max  every softmax wave adds the two halves of both subtiles (the same
//        values in every wave), takes the row max over the 32 tokens with two
//        lane swaps and forms P = 2^(s - m); the running max is raised only
//        when a score exceeds it by more than 2^8, so the accumulator rescale
//        almost never runs (the result is exact either way: the sum uses the
//        same max);
//   PV   wave 4 + c accumulates latent columns [128 c, 128 c + 128) of all 16
//        rows (8 v_mfma_f32_16x16x32_bf16, K = 32 tokens): the A operand is P
//        straight from the score layout, the B operand gathers 4 columns of 8
//        token rows (ds_read_b64) and transposes them in registers.
// The scores of tile k+1 are computed in the same step as P.V of tile k, so
// one barrier per tile covers both the tile's arrival and the score exchange.
// The block's queries arrive by the same direct-to-LDS path (through the ring
// slot that tile 3 later takes), so the waits for the first tiles never
// include ordinary loads.
// With a drafted tree (tree_parent, "Tree Attention Verification") a row
// sees the prefix and the drafted tokens on its query's branch; only tiles
// that reach the drafted tokens test the branch mask.
// Sparse read (kGather; "DeepSeek's Config Says 16 KV Heads", section 6):
// the partition is a slice of the query's list of selected tokens instead of
// a token range. The block resolves its slice to physical cache rows once
// (index list, then page table, into LDS); each tile load then gathers its 8
// rows per scoring wave with per-lane 64-bit addresses. The 16 rows of a block are
// heads of one query (H % 16 == 0), so they share one list.
#include "mla_decode_common.h"
#include "mla_launch.h"

namespace mla {

using namespace dec;

namespace {

constexpr int kRows = 16;
constexpr int kT = 32;                              // tokens per tile
constexpr int kTChunks = kT * kChunks;              // 2304 chunks = 36,864 B
constexpr int kRing = 4;                            // tiles in the LDS ring
constexpr int kPartRows = kT / kWaves;              // 8 rows of each tile per scoring wave
constexpr int kPartChunks = kPartRows * kChunks;    // 576 chunks
constexpr int kPartLoads = kPartChunks / 64;        // 9 loads per scoring wave per tile
constexpr int kHalfSteps = kKSteps / 2;             // 9 QK k-steps per scoring wave
constexpr size_t kRingBytes = (size_t)kRing * kTChunks * 16;   // 147,456 B
constexpr size_t kScoreBytes = (size_t)2 * kWaves * 64 * 16;   // 8,192 B
constexpr size_t kLdsBytes = kRingBytes + kScoreBytes;         // 155,648 B
constexpr int kGatherMaxChunk = 1984;                          // list entries per partition
constexpr size_t kGatherLdsBytes = kLdsBytes + 4 * kGatherMaxChunk;  // + resolved rows
constexpr size_t kStaticLds = 256;  // the block reductions' own LDS

static_assert(kPartChunks % 64 == 0, "a wave's share of a tile is whole loads");
static_assert(kGatherLdsBytes + kStaticLds <= 160 * 1024, "LDS of one CU");
static_assert(kGatherMaxChunk % kT == 0, "whole tiles");

}  // namespace

template <bool kGather>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_rows16_kernel(int Q, int H, int S, int page, int fixed, int max_seq_len,
                          float scale_log2, int units, int groups,
                          const bf16_t* __restrict__ q_full,
                          const bf16_t* __restrict__ cache, int64_t num_pages,
                          const int32_t* __restrict__ page_table, int max_pages,
                          const int32_t* __restrict__ seq_lens,
                          const int32_t* __restrict__ tree_parent,
                          const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ sel_cnt,
                          int topk, float* __restrict__ o_part, float* __restrict__ lse_part) {
  extern __shared__ u32x4_t lds[];
  int unit, grp;
  if (!map_block(units, groups, &unit, &grp)) return;
  const int R = Q * H;
  const int row0 = grp * kRows;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15, kg = lane >> 4;
  // waves 0-3 score (and copy the tiles), waves 4-7 run the softmax and P.V;
  // wave w and w + 4 share a SIMD
  const bool qk_wave = wave < kWaves;
  const int role = wave & (kWaves - 1);  // QK: the wave's task; PV: its column block
  const int sub = role & 1, khalf = role >> 1;  // QK share: subtile, half of the columns
  const int s = unit % S;
  int L, b;
  if constexpr (kGather) {
    b = unit / S;
    L = seq_lens[b];
  } else {
    b = seq_by_rank(seq_lens, units / S, unit / S, lane, &L);
  }
  const int jq = row0 / H;  // the query of every row of the block (gather: H % 16 == 0)
  const int32_t* par = (!kGather && tree_parent) ? tree_parent + (size_t)b * Q : nullptr;
  // a malformed tree makes the sequence invalid (the same decision in every wave)
  const bool bad_tree = par && !__all(lane >= Q || tree_entry_ok(par, lane));
  bool bad_len = (L < Q) || (L > max_seq_len) || bad_tree;
  int cnt = 0;  // gather: length of the query's list
  if constexpr (kGather) {
    cnt = sel_cnt[(size_t)b * Q + jq];
    bad_len = bad_len || cnt < 0 || cnt > topk;
  }
  int t0 = 0, t1 = 0;  // tokens (gather: list entries) of this partition
  if (!bad_len) {
    if constexpr (kGather) {
      t0 = min(s * fixed, cnt);
      t1 = min(t0 + fixed, cnt);
    } else {
      split_range(L, S, page, fixed, s, &t0, &t1);
    }
  }
  // (gather: every listed token is visible, the list slice is the range)
  const int ntiles =
      kGather ? (t1 - t0 + kT - 1) / kT
              : tiles_needed(t0, t1, kT, par != nullptr, L - Q, (row0 + kRows - 1) / H);
  bool bad = bad_len;

  f32x4_t* sc = reinterpret_cast<f32x4_t*>(reinterpret_cast<char*>(lds) + kRingBytes);
  int* const rows = reinterpret_cast<int*>(reinterpret_cast<char*>(lds) + kLdsBytes);
  auto slot = [&](int k) { return lds + (k & (kRing - 1)) * kTChunks; };

  RowDma<kPartLoads> dma;
  dma.init(role * kPartChunks, lane, role * kPartRows);
  PageWindow pw;
  if constexpr (!kGather) {
    // the page window (lane i: unit page i of the partition) is copied into
    // the score buffer, unused until the first scores, ahead of the query
    // rows, so that waiting for it leaves the query copy in flight
    pw.row = page_table + (size_t)b * max_pages + t0 / page;
    pw.upages = (t1 - t0 + page - 1) / page;
    pw.base = 0;
    pw.reg = 0;
    if (qk_wave && ntiles > 0) {  // then pw.upages >= 1
      const int* win = reinterpret_cast<const int*>(sc) + 64 * wave;
      const int* src = pw.row + min(lane, pw.upages - 1);
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                   :
                   : "s"(__builtin_amdgcn_readfirstlane(lds_addr(win))), "v"(src)
                   : "memory");
      if (wave < 2) {
        dma.issue(q_full + ((size_t)b * R + row0 + wave * kPartRows) * kD,
                  __builtin_amdgcn_readfirstlane(lds_addr(slot(kRing - 1) + wave * kPartChunks)));
        wait_vmcnt<kPartLoads>();
      } else {
        wait_vmcnt<0>();
      }
      pw.reg = win[lane];
    }
  } else {
    // the queries go out first (their latency overlaps the lookups below)
    if (wave < 2 && ntiles > 0)
      dma.issue(q_full + ((size_t)b * R + row0 + wave * kPartRows) * kD,
                __builtin_amdgcn_readfirstlane(lds_addr(slot(kRing - 1) + wave * kPartChunks)));
    // the partition's list entries -> cache rows (0 past the end or for an
    // entry that is not visible to the query or whose page is invalid)
    const int32_t* lst = sel_idx + ((size_t)b * Q + jq) * topk;
    const int vis = L - Q + jq;  // the query's own position
    const int nfill = ntiles * kT;
    for (int i = threadIdx.x; i < nfill; i += blockDim.x) {
      int row = 0;
      if (i < t1 - t0) {
        const int t = lst[t0 + i];
        const int pg = (t >= 0 && t <= vis) ? page_table[(size_t)b * max_pages + t / page] : -1;
        if (pg < 0 || (int64_t)pg >= num_pages)
          bad = true;
        else
          row = pg * page + t % page;
      }
      rows[i] = row;
    }
    __syncthreads();
  }
  // this (QK) wave's rows [8 role, 8 role + 8) of tile k (never across a page: 8 | page)
  auto issue = [&](int k) {
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(slot(k) + role * kPartChunks));
    if constexpr (kGather) {
      // load i covers part chunks [64 i, 64 i + 64): rows ra and ra + 1, lane
      // l of load i reading row ra + (l >= split); dma.off[i] holds
      // (that row) * row bytes + the swizzled chunk offset
      const int lt = k * kT + role * kPartRows;
      const int4 r03 = *reinterpret_cast<const int4*>(rows + lt);
      const int4 r47 = *reinterpret_cast<const int4*>(rows + lt + 4);
      const int rr[kPartRows] = {r03.x, r03.y, r03.z, r03.w, r47.x, r47.y, r47.z, r47.w};
      const char* cb = reinterpret_cast<const char*>(cache);
#pragma unroll
      for (int i = 0; i < kPartLoads; ++i) {
        const int ra = (64 * i) / kChunks;
        const int split = kChunks * (ra + 1) - 64 * i;
        const bool second = lane >= split;
        const int rsel = second ? rr[ra + 1 < kPartRows ? ra + 1 : ra] : rr[ra];
        const int rrel = second ? ra + 1 : ra;
        const char* src = cb + ((int64_t)rsel - rrel) * (int64_t)(kD * 2) + dma.off[i];
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt"
                     :
                     : "s"(dst + i * 1024), "v"(src)
                     : "memory");
      }
    } else {
      const int t = t0 + k * kT + role * kPartRows;
      int pg = pw.get((t - t0) / page, lane);
      if (pg < 0 || (int64_t)pg >= num_pages) {
        bad = true;
        pg = 0;
      }
      const bf16_t* src = cache + ((size_t)pg * page + (t % page)) * kD;
      dma.issue(src, dst);
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  f32x4_t acc[2][4];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int m = 0; m < 4; ++m) acc[f][m] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // tokens row n sees in this partition: t <= lim, and with a drafted tree
  // also the drafted tokens (t >= t_draft) on its query's branch
  const int t_draft = L - Q;
  const int lim = kGather ? t1 - 1 : min(par ? t_draft - 1 : t_draft + (row0 + n) / H, t1 - 1);
  const uint64_t branch = (par && !bad_len) ? tree_branch_mask(par, Q, (row0 + n) / H) : 0ull;

  if (ntiles > 0) {
    // ---- prologue: queries (waves 0, 1: 8 rows each, into slot 3, issued
    // above), tiles 0..2
    const int pre = min(ntiles, kRing - 1);  // (the queries are already on their way)
    if (qk_wave) {
      issue(0);
      if (pre > 1) issue(1);
      if (pre > 2) issue(2);
    }
    if (wave < 2) {  // own query rows landed (the tiles behind them may still fly)
      if (pre == 3)
        wait_vmcnt<3 * kPartLoads>();
      else if (pre == 2)
        wait_vmcnt<2 * kPartLoads>();
      else
        wait_vmcnt<kPartLoads>();
    }
    __syncthreads();
    // queries: row n, k-steps [9 khalf, 9 khalf + 9), chunk 4 ks + kg
    bf16x8_t qreg[kHalfSteps];
    if (qk_wave) {
      const u32x4_t* qb = slot(kRing - 1);
#pragma unroll
      for (int j = 0; j < kHalfSteps; ++j) {
        const int c = 4 * (kHalfSteps * khalf + j) + kg;
        qreg[j] = __builtin_bit_cast(bf16x8_t, qb[n * kChunks + (c ^ (n & 7))]);
      }
#pragma unroll
      for (int j = 0; j < kHalfSteps; ++j) settle(qreg[j]);
    }
    // own part of tile 0
    if (qk_wave) {
      if (pre == 3)
        wait_vmcnt<2 * kPartLoads>();
      else if (pre == 2)
        wait_vmcnt<kPartLoads>();
      else
        wait_vmcnt<0>();
      if (t0 + kT > t1)  // rows past the partition end (may be poison)
        zero_rows<kPartLoads>(slot(0) + role * kPartChunks, role * kPartChunks, lane, t1 - t0);
    }
    __syncthreads();

    // LDS addressing inside a tile. QK: row 16 sub + n, chunk 4 ks + kg.
    // PV: rows sigma(kg, j) = {4kg..4kg+3, 16+4kg..16+4kg+3}, columns
    // 128 wave + 64 f + 4n .. +3 (byte offsets).
    const int qrow = (16 * sub + n) * kChunks;
    int pv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = (j < 4) ? 4 * kg + j : 16 + 4 * kg + (j - 4);
      pv[j] = 16 * (t * kChunks + ((2 * role * 8 + (n >> 1)) ^ (t & 7))) + 8 * (n & 1);
    }

    // scores of this wave's share of tile k into score buffer k & 1
    auto qk = [&](int k) {
      const u32x4_t* buf = slot(k);
      f32x4_t c2[2] = {f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}};
      u32x4_t av[kHalfSteps];
#pragma unroll
      for (int j = 0; j < kHalfSteps; ++j) {
        const int c = 4 * (kHalfSteps * khalf + j) + kg;
        av[j] = buf[qrow + (c ^ (n & 7))];
      }
#pragma unroll
      for (int j = 0; j < kHalfSteps; ++j)
        c2[j & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[j]),
                                                            qreg[j], c2[j & 1], 0, 0, 0);
      sc[((k & 1) * kWaves + role) * 64 + lane] = c2[0] + c2[1];
    };
    if (qk_wave) qk(0);

    for (int k = 0; k < ntiles; ++k) {
      if (qk_wave && k + 1 < ntiles) {  // own part of tile k+1 (tile k+2 may stay in flight)
        if (k + 2 < ntiles)
          wait_vmcnt<kPartLoads>();
        else
          wait_vmcnt<0>();
        const int ts1 = t0 + (k + 1) * kT;
        if (ts1 + kT > t1)
          zero_rows<kPartLoads>(slot(k + 1) + role * kPartChunks, role * kPartChunks, lane, t1 - ts1);
      }
      // tile k+1 landed for every wave, the scores of tile k are complete, and
      // slot k-1 (= slot k+3) is no longer read by anyone
      __syncthreads();
      if (qk_wave) {
        if (k + 3 < ntiles) issue(k + 3);
        if (k + 1 < ntiles) qk(k + 1);
        continue;
      }

      // ---- softmax over the tile's 32 tokens (lane: row n, tokens sigma(kg, j))
      const int ts = t0 + k * kT;
      const f32x4_t* sk = sc + (k & 1) * kWaves * 64 + lane;
      const f32x4_t s0 = sk[0] + sk[128];   // subtile 0: column halves 0 + 1
      const f32x4_t s1 = sk[64] + sk[192];  // subtile 1
      float sv[8];
      // lane's tokens: ts + 4 kg + r (subtile 0) and ts + 16 + 4 kg + r (subtile 1)
      uint64_t vl = ~0ull;
      if (!__all(ts + kT - 1 <= lim)) vl = tile_visible(ts, lim, t_draft, t1, branch) >> (4 * kg);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = ((vl >> r) & 1ull) ? s0[r] * scale_log2 : -INFINITY;
        sv[4 + r] = ((vl >> (16 + r)) & 1ull) ? s1[r] * scale_log2 : -INFINITY;
      }
      float mloc = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
      mloc = row_max4(mloc);
      const bool raise = mloc > m_run + kLazy;
      if (__any(raise)) {
        const float m_new = raise ? mloc : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        // O is still zero for rows whose max was -inf: only finite rows rescale
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
        }
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
      const u32x4_t pav = {__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23),
                           __builtin_bit_cast(uint32_t, p45), __builtin_bit_cast(uint32_t, p67)};
      const bf16x8_t pa = __builtin_bit_cast(bf16x8_t, pav);

      // ---- PV: this wave's 128 latent columns, two blocks of 64
      const char* tb = reinterpret_cast<const char*>(slot(k));
      u32x2_t x[2][8];
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[f][j] = *reinterpret_cast<const u32x2_t*>(tb + pv[j] + f * 128);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        u32x4_t bm[4];
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) {
          bm[0][q2] = pack_lo(x[f][2 * q2].x, x[f][2 * q2 + 1].x);
          bm[1][q2] = pack_hi(x[f][2 * q2].x, x[f][2 * q2 + 1].x);
          bm[2][q2] = pack_lo(x[f][2 * q2].y, x[f][2 * q2 + 1].y);
          bm[3][q2] = pack_hi(x[f][2 * q2].y, x[f][2 * q2 + 1].y);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m)
          acc[f][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa, __builtin_bit_cast(bf16x8_t, bm[m]),
                                                              acc[f][m], 0, 0, 0);
      }
    }
  }
  wait_vmcnt<0>();

  // ---- the softmax waves write rows row0 .. row0+15, columns [128 role, 128 role + 128)
  const bool any_bad = __syncthreads_or(bad ? 1 : 0) != 0;
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
  for (int r = 0; r < 4 && !qk_wave && (t1 > t0 || any_bad); ++r) {
    const int orow = row0 + 4 * kg + r;
    float* dst = o_part + (((size_t)b * R + orow) * S + s) * kDC + 128 * role + 4 * n;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      float4 v = make_float4(acc[f][0][r] * inv[r], acc[f][1][r] * inv[r], acc[f][2][r] * inv[r],
                             acc[f][3][r] * inv[r]);
      if (any_bad) v = make_float4(nanv, nanv, nanv, nanv);
      *reinterpret_cast<float4*>(dst + f * 64) = v;
    }
  }
  if (wave == kWaves && kg == 0) {
    const float lse = l_row > 0.0f ? (m_run + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
    lse_part[((size_t)b * R + row0 + n) * S + s] = any_bad ? nanv : lse;
  }
}

bool decode_rows16_ok(const Shape& s, int q_len) {
  return s.dtype == 1 && s.dc == kDC && s.dr == kD - kDC && s.page % kPartRows == 0 &&
         (q_len * s.H) % kRows == 0;
}

bool decode_sparse_rows16_ok(const Shape& s, int chunk) {
  return s.dtype == 1 && s.dc == kDC && s.dr == kD - kDC && s.H % kRows == 0 && chunk > 0 &&
         chunk <= kGatherMaxChunk && chunk % kT == 0;
}

int launch_decode_rows16(const Shape& s, int batch, int q_len, int num_splits, int max_seq_len,
                         const void* q_full, const void* cache, int64_t num_pages,
                         const int32_t* page_table, int max_pages, const int32_t* seq_lens,
                         const int32_t* tree_parent, float* o_part, float* lse_part,
                         void* stream) {
  if (int e = set_max_lds(reinterpret_cast<const void*>(decode_rows16_kernel<false>),
                          (int)kLdsBytes))
    return e;
  const int units = batch * num_splits;
  const int groups = q_len * s.H / kRows;
  const int blocks = grid_blocks(units, groups);
  hipLaunchKernelGGL(decode_rows16_kernel<false>, dim3(blocks), dim3(2 * kWaves * 64), kLdsBytes,
                     reinterpret_cast<hipStream_t>(stream), q_len, s.H, num_splits, s.page,
                     s.split_fixed, max_seq_len, s.scale * 1.4426950408889634f, units, groups,
                     (const bf16_t*)q_full, (const bf16_t*)cache, num_pages, page_table, max_pages,
                     seq_lens, tree_parent, nullptr, nullptr, 0, o_part, lse_part);
  return (int)hipGetLastError();
}

int launch_decode_sparse_rows16(const Shape& s, int batch, int q_len, int topk, int chunk,
                                int num_splits, int max_seq_len, const void* q_full,
                                const void* cache, int64_t num_pages, const int32_t* page_table,
                                int max_pages, const int32_t* seq_lens, const int32_t* sel_idx,
                                const int32_t* sel_cnt, float* o_part, float* lse_part,
                                void* stream) {
  if (int e = set_max_lds(reinterpret_cast<const void*>(decode_rows16_kernel<true>),
                          (int)kGatherLdsBytes))
    return e;
  const int units = batch * num_splits;
  const int groups = q_len * s.H / kRows;
  const int blocks = grid_blocks(units, groups);
  hipLaunchKernelGGL(decode_rows16_kernel<true>, dim3(blocks), dim3(2 * kWaves * 64), kGatherLdsBytes,
                     reinterpret_cast<hipStream_t>(stream), q_len, s.H, num_splits, s.page, chunk,
                     max_seq_len, s.scale * 1.4426950408889634f, units, groups,
                     (const bf16_t*)q_full, (const bf16_t*)cache, num_pages, page_table, max_pages,
                     seq_lens, nullptr, sel_idx, sel_cnt, topk, o_part, lse_part);
  return (int)hipGetLastError();
}

}  // namespace mla
