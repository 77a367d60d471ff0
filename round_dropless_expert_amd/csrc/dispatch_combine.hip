// Dispatch (gather into the fixed round buffer) and weighted combine of the
// multi-round dropless MoE layer (gfx950). Both are HBM-bound row copies:
// one wavefront moves one row with 16-byte loads and stores.
//
// Sources: "Frontier Pre-training at Microsoft AI (MAI-Base-2)", section
// "Key claims" (dispatch -> compute -> collect rounds with a fixed
// per-expert token capacity); "Microsoft AI's MAI-Base-2 trained on 16K GPUs
// with Muon", section "Expert groups keep memory fixed when tokens pile up".
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

// Copy of one row into a tiled matrix by one wavefront: 16-byte chunk q of
// the source row goes to tiled_offset(row, 16 q) of the destination; four
// loads in flight per lane before the stores.
__device__ __forceinline__ void wave_copy_row_tiled(const u32x4* __restrict__ src,
                                                    char* __restrict__ dst_mat,
                                                    int64_t row, int64_t row_bytes,
                                                    int lane) {
  const int n16 = (int)(row_bytes / 16);
  const int64_t band = (row >> 6) * (row_bytes >> 6) * kTileBytes;
  const int r = (int)(row & 63);
  const int sw = (r >> 2) & 3;
  auto dst = [&](int q) -> u32x4* {
    return reinterpret_cast<u32x4*>(dst_mat + band + (int64_t)(q >> 2) * kTileBytes +
                                    r * kTileRowBytes + (((q & 3) ^ sw) << 4));
  };
  int v = lane;
  for (; v + 3 * kWave < n16; v += 4 * kWave) {
    const u32x4 a0 = src[v], a1 = src[v + kWave], a2 = src[v + 2 * kWave],
                a3 = src[v + 3 * kWave];
    *dst(v) = a0;
    *dst(v + kWave) = a1;
    *dst(v + 2 * kWave) = a2;
    *dst(v + 3 * kWave) = a3;
  }
  for (; v < n16; v += kWave) *dst(v) = src[v];
}

// Round r: the round's rows are numbered expert by expert; row i belongs to
// expert e with pre[e] <= i < pre[e+1] (pre = prefix of m(r, e)) and is slot
// c = i - pre[e]. Its source token is perm[offsets[e] + r*C' + c] / k and its
// destination is row c of expert e's tiled round-buffer matrix.
__global__ __launch_bounds__(256) void dispatch_kernel(
    const char* __restrict__ x, int64_t row_bytes, int E, int k, int ce,
    int ce_pad, int r,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ perm, char* __restrict__ xr) {
  __shared__ int pre[kWave + 1];
  if (threadIdx.x < kWave) {
    const int e = threadIdx.x;
    const int m = e < E ? rows_in_round(counts[e], r, ce) : 0;
    const int incl = wave_inclusive_scan(m);
    pre[e + 1] = incl;
    if (e == 0) pre[0] = 0;
  }
  __syncthreads();
  const int rows = pre[E];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  for (int64_t i = wave; i < rows; i += nwaves) {
    const int e = segment_of(pre, E + 1, (int)i);
    const int c = (int)i - pre[e];
    const int a = perm[offsets[e] + (int64_t)r * ce + c];
    const int64_t t = a / k;
    wave_copy_row_tiled(reinterpret_cast<const u32x4*>(x + t * row_bytes),
                        xr + (int64_t)e * ce_pad * row_bytes, c, row_bytes, lane);
  }
}

hipError_t launch_dispatch(const Shape& s, int r, const void* x,
                           const PlanBuffers& b, void* xr, int num_cus,
                           hipStream_t st) {
  const int64_t row_bytes = (int64_t)s.d * (s.bf16 ? 2 : 4);
  // at most min(T*k, E*C') rows in a round; 4 rows per workgroup per pass
  int64_t max_rows = s.T * s.k;
  if ((int64_t)s.E * s.ce < max_rows) max_rows = (int64_t)s.E * s.ce;
  int64_t blocks = (max_rows + 3) / 4;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(dispatch_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const char*>(x), row_bytes, s.E, s.k, s.ce,
                     s.ce_pad(), r,
                     b.counts, b.offsets, b.perm, static_cast<char*>(xr));
  return hipGetLastError();
}

// Row-major [E][rows][cols] -> tiled per expert (moe_pack_weights): one
// thread per 16-byte chunk, reads coalesced.
__global__ __launch_bounds__(256) void pack_tiled_kernel(
    const char* __restrict__ src, char* __restrict__ dst, int64_t chunks,
    int rows, int64_t row_bytes) {
  const int64_t cpr = row_bytes / 16;
  const int64_t per_mat = (int64_t)rows * cpr;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < chunks;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = g / per_mat;
    const int64_t w = g - e * per_mat;
    const int64_t row = w / cpr;
    const int64_t q = w - row * cpr;
    const int64_t base = e * per_mat * 16;
    *reinterpret_cast<u32x4*>(dst + base + tiled_offset(row, q * 16, row_bytes)) =
        *reinterpret_cast<const u32x4*>(src + g * 16);
  }
}

hipError_t launch_pack_weights(const Shape& s, const void* src, void* dst,
                               int rows, int cols, int num_cus, hipStream_t st) {
  const int64_t row_bytes = (int64_t)cols * (s.bf16 ? 2 : 4);
  const int64_t chunks = (int64_t)s.E * rows * (row_bytes / 16);
  int64_t blocks = (chunks + 255) / 256;
  const int64_t cap = (int64_t)num_cus * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(pack_tiled_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const char*>(src), static_cast<char*>(dst), chunks,
                     rows, row_bytes);
  return hipGetLastError();
}

// y[t] = sum_{j<k} weight[t][j] * z[pos[t*k + j]], fp32 fused multiply-adds
// over ascending j starting from zero, rounded once to the element type. z
// holds the expert outputs in expert-sorted order (row i = assignment
// perm[i]), so pos[a] is assignment a's row: the collect is this gather.
// One wavefront per token streams its k rows (16-byte vectors) and writes d.
template <typename Elem>
__global__ __launch_bounds__(256) void combine_kernel(
    const Elem* __restrict__ z, const float* __restrict__ weight,
    const int32_t* __restrict__ pos, int64_t T, int k, int d, Elem* __restrict__ y) {
  constexpr int kVec = 16 / sizeof(Elem);  // elements per 16-byte vector
  typedef Elem vec_t __attribute__((ext_vector_type(kVec)));
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  const int nv = d / kVec;
  for (int64_t t = wave; t < T; t += nwaves) {
    const float wl = lane < k ? weight[t * k + lane] : 0.f;
    const int rl = lane < k ? pos[t * k + lane] : 0;
    vec_t* yt = reinterpret_cast<vec_t*>(y + t * (int64_t)d);
    for (int v = lane; v < nv; v += kWave) {
      float acc[kVec];
#pragma unroll
      for (int q = 0; q < kVec; ++q) acc[q] = 0.f;
      for (int j = 0; j < k; ++j) {
        const float wj = __shfl(wl, j, kWave);
        const int64_t row = __shfl(rl, j, kWave);
        const vec_t zv = reinterpret_cast<const vec_t*>(z + row * d)[v];
#pragma unroll
        for (int q = 0; q < kVec; ++q) acc[q] = fmaf(wj, to_f32(zv[q]), acc[q]);
      }
      vec_t out;
#pragma unroll
      for (int q = 0; q < kVec; ++q) out[q] = from_f32<Elem>(acc[q]);
      yt[v] = out;
    }
  }
}

hipError_t launch_combine(const Shape& s, const void* z, const float* weight,
                          const int32_t* pos, void* y, int num_cus, hipStream_t st) {
  int64_t blocks = (s.T + 3) / 4;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (s.bf16)
    hipLaunchKernelGGL(combine_kernel<bf16>, dim3((unsigned)blocks), dim3(256),
                       0, st, static_cast<const bf16*>(z), weight, pos, s.T, s.k,
                       s.d, static_cast<bf16*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)blocks), dim3(256),
                       0, st, static_cast<const float*>(z), weight, pos, s.T, s.k,
                       s.d, static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace moe
