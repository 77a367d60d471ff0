// Backward helpers of the layer that are not GEMMs: the router-weight
// gradient from the unweighted expert outputs z, the one-time packing of the
// weights the dgrad GEMMs read (transposed, tiled), and a fill.
//
// Router (readings: the selection passes no gradient; the k weights are the
// softmax of the k chosen logits): with dw_j = <z[pos[t*k + j]], dy[t]>,
// dlogit[t][idx[t][j]] = w_j (dw_j - sum_j' w_j' dw_j'), every other logit
// of the token 0.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kMaxK = kBackwardMaxK;

// One wavefront per token: each lane takes 8-element (16-byte) pieces of
// the row, k partial dot products, then a butterfly sum over the lanes.
__global__ __launch_bounds__(256) void router_backward_kernel(
    const bf16* __restrict__ z, const bf16* __restrict__ dy,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ idx,
    const float* __restrict__ weight, int64_t T, int k, int E, int d,
    float* __restrict__ dlogits) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  const int nv = d / 8;
  for (int64_t t = wave; t < T; t += nwaves) {
    float part[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) part[j] = 0.f;
    const bf16x8* dyr = reinterpret_cast<const bf16x8*>(dy + t * (int64_t)d);
    for (int v = lane; v < nv; v += kWave) {
      const bf16x8 g = dyr[v];
#pragma unroll
      for (int j = 0; j < kMaxK; ++j) {
        if (j < k) {
          const int64_t row = pos[t * k + j];
          const bf16x8 o = reinterpret_cast<const bf16x8*>(z + row * (int64_t)d)[v];
#pragma unroll
          for (int q = 0; q < 8; ++q) part[j] = fmaf(to_f32(o[q]), to_f32(g[q]), part[j]);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) part[j] += __shfl_xor(part[j], off, kWave);
    float mean = 0.f;
    for (int j = 0; j < k; ++j) mean += weight[t * k + j] * part[j];
    if (lane < E) {
      float val = 0.f;
#pragma unroll
      for (int j = 0; j < kMaxK; ++j)
        if (j < k && idx[t * k + j] == lane) val = weight[t * k + j] * (part[j] - mean);
      dlogits[t * E + lane] = val;
    }
  }
}

// out (tiled, [E][rows][cols]) with out_e[i][j] = src_e[j][i], where src_e
// is src0[e] for j < split and src1[e] (row j - split) otherwise; both
// sources row-major with `rows` elements per row. A workgroup turns a
// 64 (j) x 64 (i) tile around in LDS: it reads the 64 source rows as 128-byte
// pieces (16 bytes a lane), and writes the tile's output, two 4 KiB blocks
// of the tiled layout (rows i, 32 j per block), as whole 1 KiB pieces per
// wavefront. rows and cols are multiples of 64 and split a multiple of 64,
// so a tile lies in one source.
__global__ __launch_bounds__(256) void pack_transposed_kernel(
    const bf16* __restrict__ src0, const bf16* __restrict__ src1, int split,
    int64_t E, int rows, int cols, char* __restrict__ out) {
  constexpr int kLdsPitch = 64 * 2 + 4;  // bytes per j row of the tile
  __shared__ __attribute__((aligned(16))) char tile[64 * kLdsPitch];
  const int tid = threadIdx.x;
  const int ti = rows / 64, tj = cols / 64;
  const int64_t t = blockIdx.x;
  const int64_t e = t / ((int64_t)ti * tj);
  const int rem = (int)(t % ((int64_t)ti * tj));
  const int i0 = (rem / tj) * 64, j0 = (rem % tj) * 64;
  const bf16* src = j0 < split ? src0 + (e * split + j0) * (int64_t)rows
                               : src1 + (e * (cols - split) + (j0 - split)) * (int64_t)rows;
  // 64 rows x 128 bytes: thread -> row tid / 8 (+ 32), 16-byte piece tid % 8
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = tid / 8 + 32 * u, q = tid % 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + (int64_t)r * rows + i0 + 8 * q);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&v);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<uint32_t*>(&tile[r * kLdsPitch + q * 16 + 4 * k]) = w[k];
  }
  __syncthreads();
  // output: 512 16-byte chunks; chunk q = tid + 256 u -> block q / 256 (32 j
  // each), row i = (q % 256) / 4, physical chunk position q % 4 (logical
  // chunk position ^ ((i / 4) % 4), the tiled layout's swizzle)
  const int64_t row_bytes = (int64_t)cols * 2;
  char* base = out + e * (int64_t)rows * row_bytes +
               ((int64_t)(i0 / 64) * (row_bytes / 64) + j0 / 32) * 4096;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = tid + 256 * u;
    const int blk = q / 256, i = (q % 256) / 4, pos = q % 4;
    const int c = pos ^ ((i >> 2) & 3);
    const int jb = blk * 32 + c * 8;
    bf16x8 v;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = *reinterpret_cast<const bf16*>(&tile[(jb + k) * kLdsPitch + i * 2]);
    *reinterpret_cast<bf16x8*>(base + blk * 4096 + i * 64 + pos * 16) = v;
  }
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, int64_t n,
                                                   float value) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = value;
}

int64_t blocks_for(int64_t items, int per_block, int num_cus, int per_cu) {
  int64_t b = (items + per_block - 1) / per_block;
  const int64_t cap = (int64_t)num_cus * per_cu;
  if (b > cap) b = cap;
  return b < 1 ? 1 : b;
}

}  // namespace

hipError_t launch_router_backward(const Shape& s, const void* z, const void* dy,
                                  const PlanBuffers& b, float* dlogits, int num_cus,
                                  hipStream_t st) {
  hipLaunchKernelGGL(router_backward_kernel,
                     dim3((unsigned)blocks_for(s.T, 4, num_cus, 8)), dim3(256), 0, st,
                     static_cast<const bf16*>(z), static_cast<const bf16*>(dy), b.pos,
                     b.idx, b.weight, s.T, s.k, s.E, s.d, dlogits);
  return hipGetLastError();
}

hipError_t launch_pack_backward(const Shape& s, const void* w_gate, const void* w_up,
                                const void* w_down, void* out_down_t, void* out_gu_t,
                                int num_cus, hipStream_t st) {
  (void)num_cus;
  // Wd [E][d][f] -> [E][f][d]: out rows f, cols d
  const int64_t n1 = (int64_t)s.E * (s.f / 64) * (s.d / 64);
  hipLaunchKernelGGL(pack_transposed_kernel, dim3((unsigned)n1), dim3(256), 0, st,
                     static_cast<const bf16*>(w_down), static_cast<const bf16*>(w_down),
                     s.d, (int64_t)s.E, s.f, s.d, static_cast<char*>(out_down_t));
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // [Wg; Wu] [E][2f][d] -> [E][d][2f]: out rows d, cols 2f
  const int64_t n2 = (int64_t)s.E * (s.d / 64) * (2 * s.f / 64);
  hipLaunchKernelGGL(pack_transposed_kernel, dim3((unsigned)n2), dim3(256), 0, st,
                     static_cast<const bf16*>(w_gate), static_cast<const bf16*>(w_up),
                     s.f, (int64_t)s.E, s.d, 2 * s.f, static_cast<char*>(out_gu_t));
  return hipGetLastError();
}

hipError_t launch_fill(float* p, int64_t n, float value, int num_cus, hipStream_t st) {
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks_for(n, 256, num_cus, 8)),
                     dim3(256), 0, st, p, n, value);
  return hipGetLastError();
}

}  // namespace moe
