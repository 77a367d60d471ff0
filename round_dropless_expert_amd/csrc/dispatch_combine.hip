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

// Rounds [r0, r0 + nr), token-major: one wavefront per token reads the
// token's row of x once and writes it to every slot the token holds in those
// rounds. The token's k assignments a = t*k + j carry their expert idx[a],
// round r = round_of[a] and slot row_of[a] = g*G*C' + ubase(r,e) + c (g =
// e / G, c the assignment's index among e's entries of round r); assignment
// j goes to row c of the matrix of (r, e), which starts at buffer row
// brow(r,e), a multiple of 64, so the whole buffer is one tiled matrix:
// each lane moves 16-byte chunks q = lane + 64 i of the row, and chunk q of
// buffer row p lands in 4 KiB block q / 4 of p's 64-row band, at row p % 64
// and chunk position (q % 4) ^ ((p / 4) % 4).
template <int kChunks>  // 16-byte chunks per lane held in registers
__global__ __launch_bounds__(256) void dispatch_kernel(
    const char* __restrict__ x, int64_t T, int row_bytes, int E, int k, int ce,
    int G, int r0, int nr, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ round_of, const int32_t* __restrict__ row_of,
    const int32_t* __restrict__ ubase, const int32_t* __restrict__ brow,
    char* __restrict__ xr) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  const int n16 = row_bytes / 16;
  const int64_t band_bytes = (int64_t)row_bytes * kTileRows;
  for (int64_t t = wave; t < T; t += nwaves) {
    int64_t prow = 0;  // buffer row of this lane's assignment
    bool mine = false;
    if (lane < k) {
      const int64_t a = t * k + lane;
      const int r = round_of[a];
      mine = r >= r0 && r - r0 < nr;
      if (mine) {
        const int e = idx[a];
        const int64_t at = (int64_t)r * E + e;
        const int c = row_of[a] - (e / G) * G * ce - ubase[at];
        prow = (int64_t)brow[at] + c;
      }
    }
    uint64_t todo = __builtin_amdgcn_ballot_w64(mine);
    if (todo == 0) continue;
    const u32x4* src = reinterpret_cast<const u32x4*>(x + t * (int64_t)row_bytes);
    for (int base = 0; base < n16; base += kChunks * kWave) {
      u32x4 v[kChunks];
#pragma unroll
      for (int i = 0; i < kChunks; ++i) {
        const int q = base + lane + i * kWave;
        if (q < n16) v[i] = src[q];
      }
      for (uint64_t m = todo; m; m &= m - 1) {
        const int j = __builtin_ctzll(m);
        const int64_t pj = __shfl(prow, j, kWave);
        char* dst = xr + (pj >> 6) * band_bytes + (pj & 63) * kTileRowBytes;
        const int sw = (int)((pj >> 2) & 3);
#pragma unroll
        for (int i = 0; i < kChunks; ++i) {
          const int q = base + lane + i * kWave;
          if (q < n16)
            *reinterpret_cast<u32x4*>(dst + (int64_t)(q >> 2) * kTileBytes +
                                      (((q & 3) ^ sw) << 4)) = v[i];
        }
      }
    }
  }
}

hipError_t launch_dispatch(const Shape& s, int r0, int nr, const void* x,
                           const PlanBuffers& b, void* xr, int num_cus,
                           hipStream_t st) {
  const int row_bytes = s.d * (s.bf16 ? 2 : 4);
  int64_t blocks = (s.T + 3) / 4;  // 4 tokens per workgroup per pass
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  const int64_t tbl = s.max_rounds() * s.E;
  hipLaunchKernelGGL(dispatch_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, st,
                     static_cast<const char*>(x), s.T, row_bytes, s.E, s.k, s.ce,
                     s.G, r0, nr, b.idx, b.round_of, b.row_of,
                     b.rounds + kUbase * tbl, b.rounds + kBrow * tbl,
                     static_cast<char*>(xr));
  return hipGetLastError();
}

// Row-major [E][rows][cols] -> tiled per expert (moe_pack_weights). rows
// and the row bytes are multiples of 64, and the experts' matrices follow
// each other, so the input is E * rows / 64 whole bands of 64 rows, each
// the same bytes of the output. Workgroup b packs band b: for each 4 KiB
// output block of the band (64 rows x 64 bytes), thread t writes its bytes
// [16 t, 16 t + 16): physical row t / 4, chunk t % 4, which holds logical
// chunk (t % 4) ^ ((t / 16) % 4) of that row. Four blocks per step, so
// each thread has four loads in flight; stores are whole 1 KiB pieces per
// wavefront.
__global__ __launch_bounds__(256) void pack_tiled_kernel(
    const char* __restrict__ src, char* __restrict__ dst, int64_t row_bytes) {
  const int t = threadIdx.x;
  const int r = t >> 2;
  const int lc = (t & 3) ^ ((r >> 2) & 3);
  const int64_t band = (int64_t)blockIdx.x * kTileRows * row_bytes;
  const char* s = src + band + r * row_bytes + lc * 16;
  char* d = dst + band + t * 16;
  const int nblk = (int)(row_bytes / kTileRowBytes);
  int b = 0;
  for (; b + 4 <= nblk; b += 4) {
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = *reinterpret_cast<const u32x4*>(s + (int64_t)(b + i) * kTileRowBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(d + (int64_t)(b + i) * kTileBytes) = v[i];
  }
  for (; b < nblk; ++b)
    *reinterpret_cast<u32x4*>(d + (int64_t)b * kTileBytes) =
        *reinterpret_cast<const u32x4*>(s + (int64_t)b * kTileRowBytes);
}

hipError_t launch_pack_weights(const Shape& s, const void* src, void* dst,
                               int rows, int cols, int num_cus, hipStream_t st) {
  (void)num_cus;
  const int64_t row_bytes = (int64_t)cols * (s.bf16 ? 2 : 4);
  const int64_t bands = (int64_t)s.E * rows / kTileRows;  // rows % 64 == 0
  hipLaunchKernelGGL(pack_tiled_kernel, dim3((unsigned)bands), dim3(256), 0, st,
                     static_cast<const char*>(src), static_cast<char*>(dst), row_bytes);
  return hipGetLastError();
}

// y[t] = sum_{j<k} weight[t][j] * z[pos[t*k + j]], fp32 fused multiply-adds
// over ascending j starting from zero, rounded once to the element type. z
// holds the expert outputs in expert-sorted order (row i = assignment
// perm[i]), so pos[a] is assignment a's row: the collect is this gather.
// One wavefront per token; each lane takes kVecs 16-byte vectors of the
// row and loads them from up to kMaxK rows before it adds (up to
// kMaxK * kVecs loads in flight; with k <= 4 a lane covers a 2048-element
// bf16 row in one pass). z is read exactly once, so its loads are
// non-temporal (a tenth faster on the balanced layer, same result). For
// bf16 with k up to 8, four vectors per lane (32 loads in flight, two
// wavefronts per SIMD) read faster than two (four wavefronts per SIMD):
// on the hot-expert layer's 2.4 GB, 430 against 440 us.
template <typename Elem, int kVecs, int kMaxK>
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
    for (int base = 0; base < nv; base += kVecs * kWave) {
      float acc[kVecs][kVec];
#pragma unroll
      for (int i = 0; i < kVecs; ++i)
#pragma unroll
        for (int q = 0; q < kVec; ++q) acc[i][q] = 0.f;
      for (int j0 = 0; j0 < k; j0 += kMaxK) {
        vec_t zv[kMaxK][kVecs];
#pragma unroll
        for (int jj = 0; jj < kMaxK; ++jj) {
          if (j0 + jj < k) {
            const int64_t row = __shfl(rl, j0 + jj, kWave);
            const vec_t* zr = reinterpret_cast<const vec_t*>(z + row * d);
#pragma unroll
            for (int i = 0; i < kVecs; ++i) {
              const int v = base + lane + i * kWave;
              if (v < nv) zv[jj][i] = __builtin_nontemporal_load(zr + v);
            }
          }
        }
#pragma unroll
        for (int jj = 0; jj < kMaxK; ++jj) {
          if (j0 + jj < k) {
            const float wj = __shfl(wl, j0 + jj, kWave);
#pragma unroll
            for (int i = 0; i < kVecs; ++i)
#pragma unroll
              for (int q = 0; q < kVec; ++q)
                acc[i][q] = fmaf(wj, to_f32(zv[jj][i][q]), acc[i][q]);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < kVecs; ++i) {
        const int v = base + lane + i * kWave;
        if (v < nv) {
          vec_t out;
#pragma unroll
          for (int q = 0; q < kVec; ++q) out[q] = from_f32<Elem>(acc[i][q]);
          yt[v] = out;
        }
      }
    }
  }
}

hipError_t launch_combine(const Shape& s, const void* z, const float* weight,
                          const int32_t* pos, void* y, int num_cus, hipStream_t st) {
  int64_t blocks = (s.T + 3) / 4;
  const int64_t cap = (int64_t)num_cus * 8;
  if (blocks > cap) blocks = cap;
  if (s.bf16 && s.k <= 4)
    hipLaunchKernelGGL((combine_kernel<bf16, 4, 4>), dim3((unsigned)blocks), dim3(256),
                       0, st, static_cast<const bf16*>(z), weight, pos, s.T, s.k,
                       s.d, static_cast<bf16*>(y));
  else if (s.bf16)
    hipLaunchKernelGGL((combine_kernel<bf16, 4, 8>), dim3((unsigned)blocks), dim3(256),
                       0, st, static_cast<const bf16*>(z), weight, pos, s.T, s.k,
                       s.d, static_cast<bf16*>(y));
  else
    hipLaunchKernelGGL((combine_kernel<float, 2, 8>), dim3((unsigned)blocks), dim3(256),
                       0, st, static_cast<const float*>(z), weight, pos, s.T, s.k,
                       s.d, static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace moe
