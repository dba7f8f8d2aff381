// Device helpers shared by the attention kernels (forward and backward):
// vector types, the LDS tile swizzle, global -> LDS tile copies, lane-pair
// reductions and scheduling hints.  gfx950 only.
#ifndef SQA_DEVICE_COMMON_H
#define SQA_DEVICE_COMMON_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sqa {
namespace dev {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
#define SQA_LDS __attribute__((address_space(3)))


// 16-byte chunk swizzle inside a tile row.  XOR-linear in the low row bits;
// chosen so that (a) 32 consecutive rows read at one chunk (K operand) and
// (b) 4 rows x 2 adjacent chunks per 16 lanes (transposed V reads) hit
// distinct banks.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) {
    const int r = row & 15;
    return r ^ ((r & 3) << 2);
  } else if constexpr (D == 64) {
    const int r0 = row & 1, r1 = (row >> 1) & 1, r2 = (row >> 2) & 1, r3 = (row >> 3) & 1;
    return r1 | ((r0 ^ r2) << 1) | ((r0 ^ r1 ^ r3) << 2);
  } else {
    return row & 3;
  }
}

// element offset of (row, col) inside a swizzled [keys][D] tile
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
}

__device__ __forceinline__ float wave_pair_max(float x) {
  // x from lane l and lane l^32 (the other half of the wave)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Global -> LDS copy of 16 bytes per lane: lane i reads sbase + voff and
// writes LDS at lds + 16*i.  Issued from inline asm so that the compiler's
// wait-count bookkeeping does not treat every later LDS read as dependent on
// it (the caller waits for these copies explicitly with vmcnt before the
// barrier that publishes the tile).  No output registers.  The LDS address
// goes in through an M0 operand constraint, so the compiler itself writes M0
// and knows its value at every copy (a plain clobber of M0, a reserved
// register, would not make it preserve its own uses).
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds) : "memory");
}

// Wait until this wave's outstanding global -> LDS copies have landed.
__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const SQA_LDS void* p) { return (uint32_t)(uintptr_t)p; }

// Scheduling pattern for an MFMA chain fed from LDS: READS loads per MFMA,
// issued AHEAD MFMAs before their use.
template <int N, int READS, int AHEAD>
__device__ __forceinline__ void lds_mfma_pipeline_hint() {
  __builtin_amdgcn_sched_group_barrier(0x100, READS * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
  }
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
}

// Stage one [KEYS][D] tile of K or V into LDS with global->LDS copies of 16
// bytes per lane.  Copy u (u = j*WAVES + wave) fills LDS chunks u*64 ...
// u*64+63, so lane i of copy u fetches the global chunk the swizzle places at
// LDS chunk u*64+i.  `lane_off[j]` is that chunk's element offset from the
// tile's first row; it does not depend on the tile.  In the tail tile, rows at
// or past S are clamped to S-1 (in bounds; their scores are masked and their
// probabilities are exactly 0).
template <int D, int WAVES, int KEYS>
struct TileCopy {
  static constexpr int CH = D / 8;
  static constexpr int COPIES = KEYS * CH / 64;
  static constexpr int PER_WAVE = COPIES / WAVES;
  static_assert(COPIES % WAVES == 0, "tile copies must split evenly over the waves");
  int lane_off[PER_WAVE];
  int row[PER_WAVE];
  int chunk[PER_WAVE];

  __device__ __forceinline__ void init(int64_t row_stride, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int pc = (j * WAVES + wave) * 64 + lane;
      row[j] = pc / CH;
      chunk[j] = (pc % CH) ^ swz<D>(row[j]);
      lane_off[j] = row[j] * (int)row_stride + chunk[j] * 8;
    }
  }

  __device__ __forceinline__ void issue(const uint16_t* tile_base, int64_t row_stride, int rows_left,
                                        SQA_LDS uint16_t* tile, int wave) const {
    if (rows_left >= KEYS) {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j)
        dma16(tile_base, (uint32_t)lane_off[j] * 2u, lds_addr(tile + (j * WAVES + wave) * 512));
    } else {
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) {
        const int r = min(row[j], rows_left - 1);
        dma16(tile_base, (uint32_t)(r * (int)row_stride + chunk[j] * 8) * 2u, lds_addr(tile + (j * WAVES + wave) * 512));
      }
    }
  }
};

// fp32 kernels: tiles of 32 rows of D floats (256 threads) staged through
// registers into LDS rows padded
// by one float (an MFMA operand that reads a column -- 32 rows at one
// dim -- hits 32 distinct banks).  Thread tid moves 16-byte chunks
// j * 256 + tid; rows at or past S are clamped to S - 1 (in bounds; their
// contributions are masked).
template <int D>
struct F32Tile {
  static constexpr int LD = D + 1;
  static constexpr int F4 = 32 * D / 4 / 256;
  static_assert(F4 >= 1 && (32 * D / 4) % 256 == 0, "tile copies must split evenly");
  f32x4 r[F4];
  __device__ __forceinline__ void load(const float* base, int64_t stride, int row0, int S, int tid) {
#pragma unroll
    for (int j = 0; j < F4; ++j) {
      const int idx = j * 256 + tid;
      r[j] = *(const f32x4*)(base + (int64_t)min(row0 + idx / (D / 4), S - 1) * stride + 4 * (idx % (D / 4)));
    }
  }
  __device__ __forceinline__ void store(float* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < F4; ++j) {
      const int idx = j * 256 + tid;
      const int o = (idx / (D / 4)) * LD + 4 * (idx % (D / 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) lds[o + e] = r[j][e];
    }
  }
};

}  // namespace dev
}  // namespace sqa

#endif
