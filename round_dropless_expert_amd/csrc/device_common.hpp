// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename Elem>
__device__ __forceinline__ Elem from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
// float -> bf16 rounds to nearest even (gfx950 has a hardware conversion).
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) {
  return static_cast<bf16>(v);
}

// Inclusive prefix sum across the 64 lanes of a wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const int t = __shfl_xor(v, off, kWave);
    v = v > t ? v : t;
  }
  return v;
}

// Largest e in [0, n) with pre[e] <= i, for a non-decreasing pre[0] = 0.
__device__ __forceinline__ int segment_of(const int* pre, int n, int i) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Rows of expert e in round r under per-expert capacity ce.
__device__ __forceinline__ int rows_in_round(int n_e, int r, int ce) {
  const int64_t m = (int64_t)n_e - (int64_t)r * ce;
  return m <= 0 ? 0 : (m >= ce ? ce : (int)m);
}

}  // namespace moe

namespace moe {

// Tiled matrix layout used for the round buffers and for packed weights.
// A matrix of R rows (R a multiple of 64 after padding) and Kb bytes per
// row (a multiple of 64) is stored as 4 KiB blocks of 64 rows x 64 bytes,
// block (row / 64, byte / 64) at index (row / 64) * (Kb / 64) + byte / 64.
// Inside a block, row r holds its four 16-byte chunks in the order
// c ^ ((r >> 2) & 3) -- the bank swizzle the GEMM's LDS stages use -- so a
// block can be copied into LDS verbatim, and one K stage of a 64-row band
// is one contiguous 4 KiB read.
constexpr int kTileRows = 64;
constexpr int kTileRowBytes = 64;
constexpr int kTileBytes = kTileRows * kTileRowBytes;

__host__ __device__ __forceinline__ int64_t tiled_offset(int64_t row,
                                                         int64_t byte,
                                                         int64_t row_bytes) {
  const int64_t blk = (row >> 6) * (row_bytes >> 6) + (byte >> 6);
  const int r = (int)(row & 63);
  const int b = (int)(byte & 63);
  return blk * kTileBytes + r * kTileRowBytes + (((b >> 4) ^ ((r >> 2) & 3)) << 4) +
         (b & 15);
}

}  // namespace moe
