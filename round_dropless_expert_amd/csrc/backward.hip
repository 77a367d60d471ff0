// Backward helpers of the layer that are not GEMMs: the router-weight
// gradient from the unweighted expert outputs z, and a fill.
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

hipError_t launch_fill(float* p, int64_t n, float value, int num_cus, hipStream_t st) {
  hipLaunchKernelGGL(fill_kernel, dim3((unsigned)blocks_for(n, 256, num_cus, 8)),
                     dim3(256), 0, st, p, n, value);
  return hipGetLastError();
}

}  // namespace moe
