// Chunked prefill in the unabsorbed form (gfx950).
//
// A prefill chunk of C query tokens over a cache of L tokens ("Beyond the
// Attention Bottleneck", "Chunked Prefilling": the prompt enters the cache
// chunk by chunk; the chunk's tokens are in the cache before its queries
// attend, query i at position P + i = L - C + i seeing t <= P + i) can run in
// either form of MLA attention. The absorbed form is the decode with q_len = C
// (every score over 576 columns and P.C over 512). The unabsorbed form
// expands each cached latent into per-head keys and values first
// ("Beyond the Attention Bottleneck", "Down-Projection and Up-Projection
// Mechanics": K^C = W_UK c, V = W_UV c; the decoupled RoPE key is shared by
// the heads, "The RoPE Compatibility Problem"), then runs dense causal
// attention per head over 192-wide keys and 128-wide values:
//   2 (192 + 128) = 640 flops per (query row, token) instead of 2,176, plus
//   the expansion, 2 x 512 x 256 flops per (token, head).
// Three launches:
//   prefill_expand_kernel  K^C [H][Lp][128] and V [H][Lp][128] of every cached
//                          token (bf16 MFMA GEMM: the 128-token tile of latents
//                          staged once in LDS, the head's weight rows streamed
//                          from L2 eight k-steps ahead), and the rotated RoPE
//                          keys R [Lp][64]
//   prefill_query_kernel   Q [H][Cp][192] = [q_nope ; RoPE(q_rope, P + i)]
//   prefill_attn_kernel    128 query rows of one head per block (4 waves of
//                          32 rows, two blocks per CU): 64-token tiles of
//                          K^C | R | V through two LDS stages; S^T = K Q^T
//                          (48 v_mfma_f32_16x16x32_bf16 per wave and tile),
//                          online softmax, O^T += V^T P^T (32 more), so each
//                          lane holds four consecutive output values of its row
#include "mla_decode_common.h"
#include "mla_launch.h"

namespace mla {

using namespace dec;

namespace {

constexpr int kPDN = 128;                 // d_n: content key width
constexpr int kPDV = 128;                 // d_v: value width
constexpr int kPDR = 64;                  // d_r: RoPE key width
constexpr int kPQK = kPDN + kPDR;         // 192: the score width per head
constexpr int kPTile = 128;               // tokens per expansion block, query rows per attention block

// ---- expansion: the latent tile, 128 rows of 64 16-byte chunks (128 KB),
// chunk j of row t at t * 64 + (j ^ (t & 15))
constexpr size_t kELds = (size_t)kPTile * kDC * 2;

// ---- attention: one stage = the K^C tile (64 rows x 16 chunks), the R tile
// (64 x 8) and the V tile (64 x 16); chunk j of row t at t * w + (j ^ (t & m))
constexpr int kAT = 64;                                   // key tokens per tile
constexpr int kAKBytes = kAT * kPDN * 2;                  // 16,384
constexpr int kARBytes = kAT * kPDR * 2;                  //  8,192
constexpr int kAVBytes = kAT * kPDV * 2;                  // 16,384
constexpr int kAStage = kAKBytes + kARBytes + kAVBytes;   // 40,960
constexpr int kALoads = kAStage / 1024 / kWaves;          // 10 loads of 1 KB per wave and tile
constexpr size_t kALds = 2 * (size_t)kAStage;             // 81,920: two blocks per CU

static_assert(kAStage % (1024 * kWaves) == 0, "a stage is whole loads for every wave");

}  // namespace

// ---------------------------------------------------------------------------
// Expansion. Block = tokens [128 tt, 128 tt + 128), all heads: the latent
// tile is staged in LDS once and every head's weights stream past it. 8
// waves, two per SIMD. Per head h, D^T = W C^T with M = the head's 256 output
// columns (128 of W_UK[h], 128 of W_UV[h]), N = 128 tokens, K = 512: wave w
// owns columns [32 w, 32 w + 32) (2 M-tiles) x all 8 N-tiles, 16 k-steps of
// v_mfma_f32_16x16x32_bf16. A = weight rows from global memory (L2), 16
// bytes per lane and M-tile, kept eight k-steps ahead in a register ring
// that runs on across the heads; B = latent rows from LDS. Lane (n, kg) ends
// with columns 4 kg .. +3 of token n of each tile: one 8-byte store each.
// Tokens past L (and tokens with an invalid page) are zero rows, so their
// outputs are zero.
// ---------------------------------------------------------------------------
constexpr int kEWaves = 8;
constexpr int kEAhead = 8;  // k-steps of weight operands in flight

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_expand_kernel(int H, int L, int Lp, int page, const bf16_t* __restrict__ cache,
                           int64_t num_pages, const int32_t* __restrict__ page_row,
                           int max_pages, const bf16_t* __restrict__ w_uk,
                           const bf16_t* __restrict__ w_uv, bf16_t* __restrict__ k_exp,
                           bf16_t* __restrict__ v_exp, bf16_t* __restrict__ r_exp) {
  extern __shared__ u32x4_t lds[];
  const int tt = blockIdx.x;
  const int t0 = tt * kPTile;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kg = lane >> 4;
  constexpr int kRowsPerWave = kPTile / kEWaves;  // 16
  constexpr int kKS = kDC / 32;                   // 16 k-steps per head

  // ---- the weight operands start first (they come from L2): M-tile mt of
  // step g = 16 h + ks is weight row 32 w' + 16 mt + n of head h, k = 32 ks + 8 kg
  const bf16_t* wsrc = (wave < 4 ? w_uk : w_uv) + (size_t)32 * (wave & 3) * kDC;
  auto aload = [&](int g, u32x4_t* a) {
    const bf16_t* w = wsrc + (size_t)(g / kKS) * kPDN * kDC + 32 * (g % kKS) + 8 * kg;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
      a[mt] = *reinterpret_cast<const u32x4_t*>(w + (size_t)(16 * mt + n) * kDC);
  };
  u32x4_t aring[kEAhead][2];
#pragma unroll
  for (int i = 0; i < kEAhead; ++i) aload(i, aring[i]);

  // ---- the latent tile: wave w loads rows 16 w .. 16 w + 15, one row (1 KB)
  // per load instruction, lane l reading the row's chunk l ^ (row & 15);
  // lane i < 16 looks up the page of row 16 w + i first, so the loads go out
  // back to back
  const int pg_lim = (int)min(num_pages, (int64_t)0x7fffffff);
  const int tok_l = t0 + kRowsPerWave * wave + lane;
  int pg_l = -1;
  if (lane < kRowsPerWave && tok_l < L && tok_l / page < max_pages) pg_l = page_row[tok_l / page];
  const bool ok_l = lane < kRowsPerWave && tok_l < L && pg_l >= 0 && pg_l < pg_lim;
  // rows of this wave with no valid latent (bit i: row 16 w + i)
  const uint32_t zero_mask = ~(uint32_t)__ballot(ok_l) & 0xffffu;
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int t = kRowsPerWave * wave + i;
    const int tok = t0 + t;
    if ((zero_mask >> i) & 1u) continue;
    const int pg = __builtin_amdgcn_readlane(pg_l, i);
    const bf16_t* src =
        cache + ((size_t)pg * page + tok % page) * kD + 8 * (lane ^ (t & 15));
    const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(lds + t * 64));
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(dst), "v"(src)
                 : "memory");
  }
  // rotated RoPE keys of the tile
  {
    for (int i = threadIdx.x; i < kPTile * 8; i += 64 * kEWaves) {  // 8 chunks of 16 B per token
      const int t = i >> 3, c = i & 7;
      const int tok = t0 + t;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (tok < L && tok / page < max_pages) {
        const int pg = page_row[tok / page];
        if (pg >= 0 && pg < pg_lim)
          v = *reinterpret_cast<const u32x4_t*>(cache + ((size_t)pg * page + tok % page) * kD +
                                                 kDC + 8 * c);
      }
      *reinterpret_cast<u32x4_t*>(r_exp + (size_t)tok * kPDR + 8 * c) = v;
    }
  }
  wait_vmcnt<0>();
  for (int i = 0; i < kRowsPerWave; ++i)
    if ((zero_mask >> i) & 1u) lds[(kRowsPerWave * wave + i) * 64 + lane] = u32x4_t{0u, 0u, 0u, 0u};
  __syncthreads();

  // ---- per head: D^T = W C^T
  static_assert(kKS % kEAhead == 0, "whole rounds of the weight ring per head");
  const int nsteps = H * kKS;
#pragma nounroll
  for (int h = 0; h < H; ++h) {
    f32x4_t acc[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma nounroll
    for (int k0 = 0; k0 < kKS; k0 += kEAhead) {
#pragma unroll
      for (int u = 0; u < kEAhead; ++u) {
        const int ks = k0 + u;
        const int g = kKS * h + ks;
        const u32x4_t a[2] = {aring[u][0], aring[u][1]};
        if (g + kEAhead < nsteps) aload(g + kEAhead, aring[u]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const int t = 16 * nt + n;  // chunk 4 ks + kg of row t, swizzled by t & 15 = n
          const u32x4_t bv = lds[t * 64 + ((4 * ks + kg) ^ n)];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, a[mt]), __builtin_bit_cast(bf16x8_t, bv),
                acc[mt][nt], 0, 0, 0);
        }
      }
    }
    // lane: columns 16 mt + 4 kg + r (of the wave's 32) of token 16 nt + n
    bf16_t* dst = (wave < 4 ? k_exp : v_exp) + (size_t)h * Lp * kPDN + 32 * (wave & 3) + 4 * kg;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int tok = t0 + 16 * nt + n;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const f32x4_t v = acc[mt][nt];
        const uint32_t lo = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
        const uint32_t hi = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
        *reinterpret_cast<u32x2_t*>(dst + (size_t)tok * kPDN + 16 * mt) = u32x2_t{lo, hi};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Queries: Q[h][i] = [q_nope[i][h] ; RoPE(q_rope[i][h], P + i)] for i < C
// (angles and rotation in fp64), zero rows for C <= i < Cp. Block = one query
// row, all heads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void prefill_query_kernel(int H, int C, int Cp, int P,
                                                            double log2_base,
                                                            const bf16_t* __restrict__ q_nope,
                                                            const bf16_t* __restrict__ q_rope,
                                                            bf16_t* __restrict__ q_exp) {
  const int i = blockIdx.x;
  for (int e = threadIdx.x; e < H * (kPDN / 8 + kPDR / 2); e += 256) {
    const int h = e / (kPDN / 8 + kPDR / 2), j = e % (kPDN / 8 + kPDR / 2);
    bf16_t* row = q_exp + ((size_t)h * Cp + i) * kPQK;
    if (j < kPDN / 8) {  // 16 bytes of the content query
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (i < C) v = *reinterpret_cast<const u32x4_t*>(q_nope + ((size_t)i * H + h) * kPDN + 8 * j);
      *reinterpret_cast<u32x4_t*>(row + 8 * j) = v;
    } else {             // one rotated pair of the RoPE query
      const int p = j - kPDN / 8;
      float y0 = 0.0f, y1 = 0.0f;
      if (i < C) {
        const bf16_t* src = q_rope + ((size_t)i * H + h) * kPDR + 2 * p;
        double d0, d1;
        rope_pair(bf2f(src[0]), bf2f(src[1]), (int64_t)P + i, p, kPDR, log2_base, &d0, &d1);
        y0 = (float)d0;
        y1 = (float)d1;
      }
      row[kPDN + 2 * p] = f2bf(y0);
      row[kPDN + 2 * p + 1] = f2bf(y1);
    }
  }
}

// ---------------------------------------------------------------------------
// Attention. Block = head h, query rows [128 qt, 128 qt + 128) (block id
// qt + nq h), wave w rows r0 = 128 qt + 32 w .. + 31 in two row groups of 16.
// Tiles of 64 key tokens, [0, min(L, P + 128 qt + 128)), two LDS stages: the
// loads of tile k + 1 are issued right after the barrier that opens tile k.
//   S^T[token][row] = K Q^T: A = the tile's key rows (token 16 g + n; the
//   first 4 k-steps from K^C, the last 2 from R), B = the wave's query rows
//   from registers; 4 token groups x 2 row groups x 6 k-steps.
//   O^T[dim][row] += V^T P^T: A = 8 tokens of one value column per lane (two
//   transposing reads, ds_read_b64_tr_b16), B = P straight from the score
//   layout (tokens 32 kk + 4 kg + r and 32 kk + 16 + 4 kg + r of row n), so a
//   lane's accumulators all belong to its own row.
// The online softmax raises a row's reference only when a score exceeds it
// by more than 2^8 (log2 units), as in the decode kernels.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_attn_kernel(int H, int C, int L, int Lp, int Cp, int nq, float scale_log2,
                         const bf16_t* __restrict__ q_exp, const bf16_t* __restrict__ k_exp,
                         const bf16_t* __restrict__ v_exp, const bf16_t* __restrict__ r_exp,
                         bf16_t* __restrict__ out, float* __restrict__ lse) {
  extern __shared__ u32x4_t lds[];
  const int qt = blockIdx.x % nq, h = blockIdx.x / nq;
  const int P = L - C;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, kg = lane >> 4;
  const int r0 = kPTile * qt + 32 * wave;
  const int tend = min(L, P + kPTile * qt + kPTile);  // tokens any row of the block sees
  const int ntiles = tend > 0 ? (tend + kAT - 1) / kAT : 0;

  // ---- the tile loads: wave w issues loads 10 w .. 10 w + 9 of a stage's 40;
  // load i of a stage fills its LDS bytes [1 KB i, 1 KB (i + 1)): K^C rows
  // (loads 0..15, 4 rows each), R rows (16..23, 8 rows each), V rows (24..39)
  const bf16_t* kh = k_exp + (size_t)h * Lp * kPDN;
  const bf16_t* vh = v_exp + (size_t)h * Lp * kPDV;
  uint32_t voff[kALoads];   // byte offset of this lane's 16 bytes from the tile's first row
  int vsrc[kALoads];        // 0: K^C, 1: R, 2: V
#pragma unroll
  for (int u = 0; u < kALoads; ++u) {
    const int i = kALoads * wave + u;
    if (i < 16) {          // K^C: row 4 i + l / 16, chunk (l % 16) ^ (row & 15)
      const int t = 4 * i + (lane >> 4), j = lane & 15;
      voff[u] = (uint32_t)(t * kPDN * 2 + 16 * (j ^ (t & 15)));
      vsrc[u] = 0;
    } else if (i < 24) {   // R: row 8 (i - 16) + l / 8, chunk (l % 8) ^ (row & 7)
      const int t = 8 * (i - 16) + (lane >> 3), j = lane & 7;
      voff[u] = (uint32_t)(t * kPDR * 2 + 16 * (j ^ (t & 7)));
      vsrc[u] = 1;
    } else {               // V: row 4 (i - 24) + l / 16, chunk (l % 16) ^ (row & 15)
      const int t = 4 * (i - 24) + (lane >> 4), j = lane & 15;
      voff[u] = (uint32_t)(t * kPDV * 2 + 16 * (j ^ (t & 15)));
      vsrc[u] = 2;
    }
  }
  auto issue = [&](int k) {
    const int tok0 = kAT * k;
    char* stage = reinterpret_cast<char*>(lds) + (k & 1) * kAStage;
#pragma unroll
    for (int u = 0; u < kALoads; ++u) {
      const int i = kALoads * wave + u;  // wave-uniform
      const bf16_t* base = vsrc[u] == 0 ? kh + (size_t)tok0 * kPDN
                           : vsrc[u] == 1 ? r_exp + (size_t)tok0 * kPDR
                                          : vh + (size_t)tok0 * kPDV;
      const uint32_t dst = __builtin_amdgcn_readfirstlane(lds_addr(stage + 1024 * i));
      asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :
                   : "s"(dst), "v"(voff[u]), "s"(base)
                   : "memory");
    }
  };

  // ---- the wave's query rows (B operand of S^T): row r0 + 16 rg + n, k = 32 ks + 8 kg
  bf16x8_t qreg[2][6];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const bf16_t* qrow = q_exp + ((size_t)h * Cp + r0 + 16 * rg + n) * kPQK + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < 6; ++ks)
      qreg[rg][ks] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(qrow + 32 * ks));
  }
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int ks = 0; ks < 6; ++ks) settle(qreg[rg][ks]);
  if (ntiles > 0) issue(0);

  // value operand offsets (bytes within the V tile) for column block dt,
  // token half hh of k-step kk: lane s = a + 4 i of group kg reads token
  // 32 kk + 16 hh + 4 kg + i, columns 16 dt + 4 a .. + 3
  int vto[2];
  {
    const int a = n & 3, i = n >> 2;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) vto[hh] = 16 * hh + 4 * kg + i;
    (void)a;
  }
  auto vaddr = [&](uint32_t vbase, int kk, int hh, int dt) {
    const int a = n & 3;
    const int t = 32 * kk + vto[hh];
    return vbase + 16 * (t * 16 + ((2 * dt + (a >> 1)) ^ (t & 15))) + 8 * (a & 1);
  };

  f32x4_t acc[2][8];
#pragma unroll
  for (int rg = 0; rg < 2; ++rg)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[rg][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};

  for (int k = 0; k < ntiles; ++k) {
    wait_vmcnt<0>();
    __syncthreads();  // tile k landed everywhere; stage (k + 1) & 1 is free
    if (k + 1 < ntiles) issue(k + 1);
    const char* stage = reinterpret_cast<const char*>(lds) + (k & 1) * kAStage;
    const u32x4_t* kt = reinterpret_cast<const u32x4_t*>(stage);
    const u32x4_t* rt = reinterpret_cast<const u32x4_t*>(stage + kAKBytes);
    const uint32_t vbase = lds_addr(stage + kAKBytes + kARBytes);

    // ---- S^T: token group g (tokens 16 g + 4 kg + r of row n)
    f32x4_t s[2][4];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg)
#pragma unroll
      for (int g = 0; g < 4; ++g) s[rg][g] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int t = 16 * g + n;
      u32x4_t av[6];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) av[ks] = kt[t * 16 + ((4 * ks + kg) ^ (t & 15))];
#pragma unroll
      for (int ks = 4; ks < 6; ++ks) av[ks] = rt[t * 8 + ((4 * (ks - 4) + kg) ^ (t & 7))];
#pragma unroll
      for (int ks = 0; ks < 6; ++ks)
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
          s[rg][g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[ks]),
                                                             qreg[rg][ks], s[rg][g], 0, 0, 0);
    }

    // ---- online softmax; P as the B operand of k-step kk: 8 bf16
    const int tok0 = kAT * k;
    bf16x8_t pb[2][2];
#pragma unroll
    for (int rg = 0; rg < 2; ++rg) {
      const int row = r0 + 16 * rg + n;
      const int lim = min(P + row, L - 1);  // the last token this row sees
      float sv[16];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[4 * g + r] = s[rg][g][r] * scale_log2;
      if (!__all(tok0 + kAT - 1 <= lim)) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            sv[4 * g + r] = (tok0 + 16 * g + 4 * kg + r <= lim) ? sv[4 * g + r] : -INFINITY;
      }
      float mloc = sv[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mloc = fmaxf(mloc, sv[j]);
      mloc = row_max4(mloc);
      const bool raise = mloc > m_run[rg] + kLazy;
      if (__any(raise)) {
        const float m_new = raise ? mloc : m_run[rg];
        const float alpha =
            (m_run[rg] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[rg] - m_new);
        l_run[rg] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[rg][dt][r] *= alpha;
        m_run[rg] = m_new;
      }
      const float m_use = (m_run[rg] == -INFINITY) ? 0.0f : m_run[rg];
      float p[16];
      float ls = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        p[j] = __builtin_amdgcn_exp2f(sv[j] - m_use);
        ls += p[j];
      }
      l_run[rg] += ls;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = (__bf16)p[4 * (2 * kk) + r];
          v[4 + r] = (__bf16)p[4 * (2 * kk + 1) + r];
        }
        pb[rg][kk] = v;
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const s16x4_t lo = ds_read_tr16(vaddr(vbase, kk, 0, dt));
        const s16x4_t hi = ds_read_tr16(vaddr(vbase, kk, 1, dt));
        const bf16x8_t va =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rg = 0; rg < 2; ++rg)
          acc[rg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[rg][kk], acc[rg][dt], 0,
                                                                0, 0);
      }
    }
  }

  // ---- output: lane (n, kg) holds dims 16 dt + 4 kg .. + 3 of row r0 + 16 rg + n
#pragma unroll
  for (int rg = 0; rg < 2; ++rg) {
    const int row = r0 + 16 * rg + n;
    const float l_row = row_sum4(l_run[rg]);
    if (row < C) {
      const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
      bf16_t* dst = out + ((size_t)row * H + h) * kPDV + 4 * kg;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const f32x4_t v = acc[rg][dt];
        const uint32_t lo = (uint32_t)f2bf(v[0] * inv) | ((uint32_t)f2bf(v[1] * inv) << 16);
        const uint32_t hi = (uint32_t)f2bf(v[2] * inv) | ((uint32_t)f2bf(v[3] * inv) << 16);
        *reinterpret_cast<u32x2_t*>(dst + 16 * dt) = u32x2_t{lo, hi};
      }
      if (kg == 0)
        lse[(size_t)row * H + h] =
            l_row > 0.0f ? (m_run[rg] + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

bool prefill_unabsorbed_ok(const Shape& s) {
  return s.dtype == 1 && s.dc == kDC && s.dr == kPDR && s.dn == kPDN && s.dv == kPDV;
}

size_t prefill_workspace_bytes(const Shape& s, int seq_len, int q_len) {
  const size_t Lp = (size_t)(seq_len + kPTile - 1) / kPTile * kPTile;
  const size_t Cp = (size_t)(q_len + kPTile - 1) / kPTile * kPTile;
  return 2 * ((size_t)s.H * Lp * (kPDN + kPDV) + Lp * kPDR + (size_t)s.H * Cp * kPQK);
}

int launch_prefill_unabsorbed(const Shape& s, int q_len, int seq_len, const void* q_nope,
                              const void* q_rope, const void* w_uk, const void* w_uv,
                              const void* cache, int64_t num_pages, const int32_t* page_row,
                              int max_pages, void* workspace, void* out, float* lse,
                              void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int H = s.H, L = seq_len, C = q_len;
  const int Lp = (L + kPTile - 1) / kPTile * kPTile;
  const int Cp = (C + kPTile - 1) / kPTile * kPTile;
  bf16_t* k_exp = reinterpret_cast<bf16_t*>(workspace);
  bf16_t* v_exp = k_exp + (size_t)H * Lp * kPDN;
  bf16_t* r_exp = v_exp + (size_t)H * Lp * kPDV;
  bf16_t* q_exp = r_exp + (size_t)Lp * kPDR;
  if (int e = set_max_lds(reinterpret_cast<const void*>(prefill_expand_kernel), (int)kELds))
    return e;
  hipLaunchKernelGGL(prefill_expand_kernel, dim3(Lp / kPTile), dim3(64 * kEWaves), kELds,
                     st, H, L,
                     Lp, s.page, (const bf16_t*)cache, num_pages, page_row, max_pages,
                     (const bf16_t*)w_uk, (const bf16_t*)w_uv, k_exp, v_exp, r_exp);
  if (int e = (int)hipGetLastError()) return e;
  hipLaunchKernelGGL(prefill_query_kernel, dim3(Cp), dim3(256), 0, st, H, C, Cp, L - C,
                     s.log2_base, (const bf16_t*)q_nope, (const bf16_t*)q_rope, q_exp);
  if (int e = (int)hipGetLastError()) return e;
  if (int e = set_max_lds(reinterpret_cast<const void*>(prefill_attn_kernel), (int)kALds))
    return e;
  const int nq = Cp / kPTile;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(nq * H), dim3(256), kALds, st, H, C, L, Lp, Cp, nq,
                     s.scale * 1.4426950408889634f, q_exp, k_exp, v_exp, r_exp, (bf16_t*)out,
                     lse);
  return (int)hipGetLastError();
}

}  // namespace mla
