// Device building blocks shared by the two bf16 MFMA decode kernels
// (decode_rows16_kernel, decode_ws_kernel) for the DeepSeek MLA row shape:
// d_c = 512 latent + d_r = 64 RoPE columns, 576 bf16 = 1,152 bytes per cached
// row ("The Architecture of Memory", "Flash-Decoding and FlashInfer";
// "DeepSeek's Config Says 16 KV Heads", section 5).
//
// Cache rows move HBM -> LDS with direct-to-LDS 16-byte loads
// (global_load_lds_dwordx4, non-temporal: the cache is streamed once), in a
// XOR-swizzled chunk order: chunk c of row t sits at t*72 + (c ^ (t & 7)), so
// the LDS reads of both contractions are free of bank conflicts.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

#include "mla_common.h"

namespace mla {
namespace dec {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2_t;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDC = 512;
constexpr int kD = 576;
constexpr int kChunks = kD * 2 / 16;            // 72 sixteen-byte chunks per row
constexpr int kSlice = 16;                      // tokens per MFMA step
constexpr int kSliceChunks = kSlice * kChunks;  // 1152 chunks = 18,432 B
constexpr int kLoads = kSliceChunks / 64;       // 18 wave-wide 16-byte loads per slice
constexpr int kKSteps = kD / 32;                // 18 k-steps (QK)
constexpr int kFB = kDC / 64;                   // 8 feature blocks (PV)
constexpr int kWaves = 4;
constexpr float kLazy = 8.0f;                   // rescale slack, log2 units

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// (a & 0xffff) | (b << 16) and (a >> 16) | (b & 0xffff0000), one v_perm_b32
// each (byte selectors index b as bytes 4..7 and a as bytes 0..3)
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}
__device__ __forceinline__ s16x4_t as_s16x4(uint32_t lo, uint32_t hi) {
  u32x2_t v = {lo, hi};
  return __builtin_bit_cast(s16x4_t, v);
}

// Direct-to-LDS copy of N x 64 sixteen-byte chunks of consecutive cached
// rows (N = 18: one block of 16 rows). Load i of a lane fills LDS chunk
// p = part_chunk + 64 i + lane with source row t = p / 72 (row t of the
// buffer), chunk (p % 72) ^ (t & 7): the XOR swizzle is applied on the global
// side, so each load instruction still fills 1 KB of LDS contiguously. Source
// offsets are relative to row src_row0 of the buffer (the row the source
// pointer passed to issue() addresses). They are the same for every block and
// computed once; a load is then one scalar M0 write plus one VMEM instruction.
//
// The loads are issued as inline assembly so that the compiler does not treat
// the pending LDS writes as aliasing every later LDS read (it would otherwise
// wait for all outstanding loads before the first read of the other buffer,
// serialising the pipeline); completion is awaited with s_waitcnt vmcnt.
template <int N = kLoads>
struct RowDma {
  uint32_t off[N];
  __device__ __forceinline__ void init(int part_chunk, int lane, int src_row0 = 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int p = part_chunk + i * 64 + lane;
      const int t = p / kChunks;
      off[i] = (uint32_t)(((t - src_row0) * kChunks + ((p - t * kChunks) ^ (t & 7))) * 16);
    }
  }
  // src: wave-uniform address of buffer row src_row0; lds_base: LDS byte
  // address of chunk part_chunk
  __device__ __forceinline__ void issue(const void* src, uint32_t lds_base) const {
#pragma unroll
    for (int i = 0; i < N; ++i) issue_one(src, lds_base, i);
  }
  // load i alone (i a compile-time constant after unrolling)
  __device__ __forceinline__ void issue_one(const void* src, uint32_t lds_base, int i) const {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(lds_base + i * 1024), "v"(off[i]), "s"(src)
                 : "memory");
  }
};

// ds_read_b64_tr_b16 (gfx950): in each group of 16 lanes, lane 4 a + b
// receives 16-bit element b of the 8 bytes addressed by lanes a, a + 4,
// a + 8 and a + 12 of its group, in that order (layout checked on the device)
__device__ __forceinline__ s16x4_t ds_read_tr16(uint32_t lds_byte_addr) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)lds_byte_addr);
}

// Make the compiler complete the loads behind v here (it then has no loads of
// its own pending when the token loop starts, where its waits would also
// count the in-flight direct-to-LDS loads).
template <typename T>
__device__ __forceinline__ void settle(const T& v) {
  asm volatile("" ::"v"(v));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Zero the chunks this lane loaded (N loads from base_chunk) whose buffer
// row is >= first_bad.
template <int N = kLoads>
__device__ __forceinline__ void zero_rows(u32x4_t* dst, int base_chunk, int lane, int first_bad) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int p = base_chunk + i * 64 + lane;
    if (p / kChunks >= first_bad) dst[i * 64 + lane] = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// Lane-held page-table window: lane i holds the physical page of unit page
// base + i, so a slice's page is a register read, not a dependent load.
struct PageWindow {
  const int32_t* row;  // page_table + b * max_pages + t0 / page
  int upages, base, reg;
  __device__ __forceinline__ void init(const int32_t* r, int npages, int lane) {
    row = r;
    upages = npages;
    base = 0;
    reg = lane < npages ? row[lane] : 0;
  }
  // physical page of unit page u (wave-uniform u; u may also move back)
  __device__ __forceinline__ int get(int u, int lane) {
    if ((unsigned)(u - base) >= 64u) {
      base = u & ~63;
      reg = base + lane < upages ? row[base + lane] : 0;
      asm volatile("" ::"v"(reg));  // complete this load here, inside the rare branch
    }
    return __builtin_amdgcn_readlane(reg, u - base);
  }
};

// Max / sum over the 4 lanes {l, l^16, l^32, l^48} (one query row of an MFMA
// accumulator), with the gfx950 lane-swap instructions instead of LDS
// permutes: permlane16_swap pairs lane l with l^16, permlane32_swap with l^32.
__device__ __forceinline__ float row_max4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}
__device__ __forceinline__ float row_sum4(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Blocks start in id order, and the partitions of a sequence in the
// per-sequence plan all hold about L_b / S tokens, so a batch of uneven
// lengths finishes soonest when its longest sequences start first (the short
// ones then fill the tail). For batch <= 64 each block ranks the lengths
// (longest first, ties by index) with one lane per sequence and takes the
// sequence of rank `rank`; larger batches keep their order. Writes that
// sequence's length to *len. A partition's result does not depend on which
// block computes it, so the order changes no output.
__device__ __forceinline__ int seq_by_rank(const int32_t* __restrict__ seq_lens, int batch,
                                           int rank, int lane, int* len) {
  if (batch > 64) {
    *len = seq_lens[rank];
    return rank;
  }
  const int li = lane < batch ? seq_lens[lane] : 0;
  int r = 0;
  for (int j = 0; j < batch; ++j) {
    const int lj = __builtin_amdgcn_readlane(li, j);
    r += (lj > li) || (lj == li && j < lane);
  }
  const uint64_t hit = __ballot(lane < batch && r == rank);
  const int b = hit ? __builtin_ctzll(hit) : rank;
  *len = __builtin_amdgcn_readlane(li, b);
  return b;
}

// block id -> (unit, row group). With 8 units or more, all groups of one unit
// share id % 8, i.e. run on the same XCD and share its L2. With fewer (one
// long prefill chunk is one unit with many row groups) that would leave XCDs
// idle, so the work items (unit, group) are split into 8 contiguous ranges,
// one per XCD: block 8 r + x takes item x * per + r.
__host__ __device__ __forceinline__ int grid_blocks(int units, int groups) {
  return units >= 8 ? ((units + 7) / 8) * 8 * groups : 8 * ((units * groups + 7) / 8);
}
__device__ __forceinline__ bool map_block(int units, int groups, int* unit, int* grp) {
  const int id = blockIdx.x;
  if (units < 8) {
    const int per = (units * groups + 7) / 8;
    const int f = (id & 7) * per + (id >> 3);
    *unit = f % units;
    *grp = f / units;
    return f < units * groups;
  }
  const int kk = id >> 3;
  *unit = (kk / groups) * 8 + (id & 7);
  *grp = kk % groups;
  return *unit < units;
}

}  // namespace dec
}  // namespace mla
