// Weight gradients of the expert FFN for one round of the backward (the
// backward of "Frontier Pre-training at Microsoft AI (MAI-Base-2)",
// section "Key claims": grouped expert compute per round; here its
// gradient with respect to the expert weights).
//
// For every expert e with rows in round r, out_e[a][b] (+)= sum over the
// expert's rows c of the round of U[c][a] * V[c][b], where U (A features)
// and V (B features) are token-major round buffers in the tiled layout,
// expert e's matrix starting at buffer row (e / G) * Q + pbase(r, e). Rows
// a < A0 go to out0[e][a][b], the others to out1[e][a - A0][b] (dW_gate and
// dW_up from one dgu buffer). out is fp32, row-major; round 0 stores, later
// rounds add (the contraction over an expert's rows is then split at the
// round boundaries).
//
// The contraction runs over tokens, which are rows of both operands, while
// the matrix cores want each lane to hold consecutive K (token) values of
// one feature: every 32-token stage is therefore written to LDS turned
// around ([feature][token]), from registers, and read back as 16-byte MFMA
// fragments. A workgroup computes a 128 (b) x 128 (a) tile with 2 x 2
// wavefronts of 64 x 64 (2 x 2 blocks of v_mfma_f32_32x32x16_bf16; the
// output block is [b][a], so a lane holds four consecutive b of one a: one
// 16-byte fp32 store). Stages are double-buffered: the next stage's global
// loads are in flight while the current one is multiplied.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kTile = 128;        // a and b extent of a tile
constexpr int kStageTok = 32;     // tokens per stage
constexpr int kPitch = 80;        // bytes per LDS row: 32 tokens + 16 pad
constexpr int kOpBytes = kTile * kPitch;  // one operand of one stage

struct WgradParams {
  const bf16* U;   // round buffer, A features per row (tiled)
  const bf16* V;   // round buffer, B features per row (tiled)
  float* out0;     // [E][A0][B]
  float* out1;     // [E][A - A0][B] (NULL when A0 == A)
  const int32_t* rounds;
  const int32_t* n_rounds;
  int E, r, A, A0, B, G, max_rounds, pool_rows;
  int all_experts;  // tiles of every expert (round 0: experts without rows get zeros)
  int accumulate;   // add to out (else store)
};

__global__ __launch_bounds__(256) void wgrad_kernel(WgradParams p) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][kOpBytes];  // [buf][U|V]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wa = wave & 1, wb = wave >> 1;  // this wavefront's 64 x 64 quarter
  const int l32 = lane & 31, half = lane >> 5;
  if (p.r >= *p.n_rounds) return;

  // tile -> expert: expert-major, tiles_a x tiles_b per expert
  const int ta = (p.A + kTile - 1) / kTile, tb = (p.B + kTile - 1) / kTile;
  const int per = ta * tb;
  const int64_t tbl = (int64_t)p.max_rounds * p.E;
  const int slot = (int)blockIdx.x / per;
  const int local = (int)blockIdx.x % per;
  int e;
  if (p.all_experts) {
    e = slot;
  } else {  // the slot-th expert with rows in this round
    const bool act = lane < p.E && p.rounds[kAlloc * tbl + (int64_t)p.r * p.E + lane] > 0;
    const uint64_t mask = __builtin_amdgcn_ballot_w64(act);
    const uint64_t below = lane == 0 ? 0ull : (mask & (~0ull >> (64 - lane)));
    const bool hit = act && __builtin_popcountll(below) == slot;
    const uint64_t h = __builtin_amdgcn_ballot_w64(hit);
    if (h == 0) return;
    e = __builtin_ctzll(h);
  }
  if (e >= p.E) return;
  const int64_t at = (int64_t)p.r * p.E + e;
  const int m = p.rounds[kAlloc * tbl + at];
  const int64_t row0 = (int64_t)(e / p.G) * p.pool_rows + p.rounds[kPbase * tbl + at];
  const int a0 = (local / tb) * kTile, b0 = (local % tb) * kTile;

  // loads of a stage: thread -> token c = tid % 32, 16-byte chunks
  // j = tid / 32 and j + 8 of the tile's 128 features (8 per chunk)
  const int lc = tid & 31, lj = tid >> 5;
  const int64_t ubytes = (int64_t)p.A * 2, vbytes = (int64_t)p.B * 2;
  auto load = [&](int k0, u32x4 (&ur)[2], u32x4 (&vr)[2]) {
    const int c = k0 + lc;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int fa = a0 + (lj + 8 * i) * 8, fb = b0 + (lj + 8 * i) * 8;
      ur[i] = u32x4{0, 0, 0, 0};
      vr[i] = u32x4{0, 0, 0, 0};
      if (c < m && fa < p.A)
        ur[i] = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(p.U) +
            tiled_offset(row0 + c, (int64_t)fa * 2, ubytes));
      if (c < m && fb < p.B)
        vr[i] = *reinterpret_cast<const u32x4*>(
            reinterpret_cast<const char*>(p.V) +
            tiled_offset(row0 + c, (int64_t)fb * 2, vbytes));
    }
  };
  // turned around: feature row (8 chunk + v), token column c
  auto store_lds = [&](int buf, const u32x4 (&ur)[2], const u32x4 (&vr)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int f0 = (lj + 8 * i) * 8;
      const bf16x8 uv = __builtin_bit_cast(bf16x8, ur[i]);
      const bf16x8 vv = __builtin_bit_cast(bf16x8, vr[i]);
#pragma unroll
      for (int v = 0; v < 8; ++v) {
        *reinterpret_cast<bf16*>(&lds[buf][0][(f0 + v) * kPitch + lc * 2]) = uv[v];
        *reinterpret_cast<bf16*>(&lds[buf][1][(f0 + v) * kPitch + lc * 2]) = vv[v];
      }
    }
  };

  f32x16 acc[2][2];  // [b block][a block]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int stages = (m + kStageTok - 1) / kStageTok;
  u32x4 ur[2], vr[2];
  if (stages > 0) load(0, ur, vr);
  for (int s = 0; s < stages; ++s) {
    const int buf = s & 1;
    store_lds(buf, ur, vr);
    __syncthreads();
    if (s + 1 < stages) load((s + 1) * kStageTok, ur, vr);
#pragma unroll
    for (int ks = 0; ks < kStageTok / 16; ++ks) {
      const int tok = ks * 16 + half * 8;
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int brow = wb * 64 + i * 32 + l32;
        const int arow = wa * 64 + i * 32 + l32;
        fb[i] = *reinterpret_cast<const bf16x8*>(&lds[buf][1][brow * kPitch + tok * 2]);
        fa[i] = *reinterpret_cast<const bf16x8*>(&lds[buf][0][arow * kPitch + tok * 2]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[i], fa[j], acc[i][j],
                                                              0, 0, 0);
    }
  }

  // lane: a = column l32 of the block, b = rows 8 g4 + 4 half + q
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int a = a0 + wa * 64 + j * 32 + l32;
      if (a >= p.A) continue;
      float* row = a < p.A0 ? p.out0 + ((int64_t)e * p.A0 + a) * p.B
                            : p.out1 + ((int64_t)e * (p.A - p.A0) + (a - p.A0)) * p.B;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int b = b0 + wb * 64 + i * 32 + 8 * g4 + 4 * half;
        if (b >= p.B) continue;
        float4 v = make_float4(acc[i][j][4 * g4], acc[i][j][4 * g4 + 1],
                               acc[i][j][4 * g4 + 2], acc[i][j][4 * g4 + 3]);
        float4* dst = reinterpret_cast<float4*>(row + b);
        if (p.accumulate) {
          const float4 o = *dst;
          v.x += o.x;
          v.y += o.y;
          v.z += o.z;
          v.w += o.w;
        }
        *dst = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_wgrad(const Shape& s, int r, const void* U, const void* V,
                        int A, int A0, int B, float* out0, float* out1,
                        const PlanBuffers& b, const int32_t* rows_host,
                        hipStream_t st) {
  int active = 0;
  for (int e = 0; e < s.E; ++e) active += rows_host[e] > 0;
  const bool all = r == 0;
  const int n = all ? s.E : active;
  if (n == 0) return hipSuccess;
  const int per = ((A + kTile - 1) / kTile) * ((B + kTile - 1) / kTile);
  WgradParams p{static_cast<const bf16*>(U), static_cast<const bf16*>(V), out0, out1,
                b.rounds, b.n_rounds, s.E, r, A, A0, B, s.G, (int)s.max_rounds(),
                (int)s.pool_rows(), all ? 1 : 0, r == 0 ? 0 : 1};
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)(n * per)), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace moe
