// Matrix-core throughput calibration for the benchmark (not part of the
// layer's C ABI; built into its own library, libmoe_calibrate.so).
//
// The bf16 roofline uses MI355X's published dense peak (2.5 PFLOP/s at
// 2.4 GHz). Under sustained matrix load the chip lowers its clock to stay
// within its power budget, and how far depends on the data the MFMAs
// switch. This kernel measures the rate the matrix cores actually sustain:
// every wavefront runs back-to-back independent v_mfma_f32_32x32x16_bf16
// (16 accumulators, the same count per wavefront as the layer's GEMM
// tiles), with operands taken from a caller-supplied bf16 buffer (random
// values give the layer's switching activity), one 4-wavefront workgroup
// per CU at a time, no memory traffic inside the loop.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kOperandVecs = 1024;  // 8192 bf16 values

__global__ __launch_bounds__(256, 1) void mfma_ceiling_kernel(const bf16x8* __restrict__ src,
                                                              int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int w = (threadIdx.x >> 6) + 4 * (blockIdx.x & 7);
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = src[((w * 8 + i) * 64 + lane) % kOperandVecs];
    b[i] = src[((w * 8 + 4 + i) * 64 + lane) % kOperandVecs];
  }
  f32x16 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j % 4], b[j / 4], acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// operands: at least 8192 bf16 values on the device; out: grid * 256
// floats on the device. One launch of `grid` workgroups of 256 threads,
// each wavefront running iters * 16 MFMAs (grid * 4 * iters * 16 * 32768
// FLOP in all). Asynchronous on stream; returns the launch's hipError_t.
extern "C" int moe_calibrate_mfma_bf16(const void* operands, float* out, int grid, int iters,
                                       void* stream) {
  if (!operands || !out || grid < 1 || iters < 1) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3((unsigned)grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const bf16x8*>(operands),
                     iters, out);
  return (int)hipGetLastError();
}
