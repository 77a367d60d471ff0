// Grouped expert GEMMs of one round of the multi-round dropless MoE layer
// (gfx950 matrix cores).
//
// Sources: "Frontier Pre-training at Microsoft AI (MAI-Base-2)", section
// "Key claims": experts of a group run dispatch -> compute -> collect rounds
// with a fixed per-expert token capacity, and per-expert overhead is cut by
// running one grouped GEMM for the whole expert group. The expert FFN is
// SwiGLU without biases: h = silu(x.Wg^T) * (x.Wu^T), o = h.Wd^T.
//
// One persistent launch covers every active expert of the round. Tiles are
// numbered expert by expert (token tile fastest, then feature tile); the
// launch's workgroups walk them in an order that gives each XCD a contiguous
// run, so the workgroups sharing an expert's weights and rows share an L2.
//
// Matrix-core mapping (swapped operands): the MFMA "A" operand is a 32-row
// block of weight rows (output features), the "B" operand a 32-row block of
// token rows; both are K-contiguous in memory (x.W^T with W stored
// [out][in]). Each lane then holds, for one token, four runs of four
// consecutive output features, which become 8-byte (bf16) or 16-byte (fp32)
// stores in the epilogue.
//
// Tiles: 256 threads = 2 x 2 wavefronts; wavefront (wm, wn) owns WJ 32-token
// blocks and WI 32-weight-row blocks. K advances 128 bytes per stage
// (64 bf16 or 32 fp32), double-buffered in LDS with one barrier per stage.
// LDS rows are 128 bytes; the 16-byte chunk c of row q is stored at chunk
// c ^ (q & 7), so the eight rows read together by a fragment load fall in
// distinct banks.
//
// Determinism: every output element is one fixed sequence of MFMA steps
// over K in ascending order, whatever the round, the slot or the tile it
// falls in, so the result of a token does not depend on the capacity.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

template <typename Elem>
struct MmaOp;

// v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) and k-run
// [8*(l/32), 8*(l/32)+8) of its operand.
template <>
struct MmaOp<bf16> {
  static constexpr int kSteps = 4;  // instructions per 128-byte k stage
  typedef bf16x8 frag_t;
  __device__ static __forceinline__ frag_t load(const char* row, int step,
                                                int half, int swz) {
    const int chunk = (2 * step + half) ^ swz;
    return *reinterpret_cast<const frag_t*>(row + chunk * 16);
  }
  __device__ static __forceinline__ void mma(f32x16& acc, frag_t a, frag_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
};

// v_mfma_f32_32x32x2f32: lane l supplies row (l % 32) and k = l / 32.
template <>
struct MmaOp<float> {
  static constexpr int kSteps = 16;
  typedef float frag_t;
  __device__ static __forceinline__ frag_t load(const char* row, int step,
                                                int half, int swz) {
    const int byte = (2 * step + half) * 4;
    const int chunk = (byte >> 4) ^ swz;
    return *reinterpret_cast<const float*>(row + chunk * 16 + (byte & 15));
  }
  __device__ static __forceinline__ void mma(f32x16& acc, frag_t a, frag_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
  }
};

template <typename Elem>
struct GemmParams {
  const Elem* act;   // round rows [E*ce][K]: xr (gate/up) or h (down)
  const Elem* w0;    // [E][*][K]: gate (gate/up) or down weights
  const Elem* w1;    // [E][N][K]: up weights (gate/up only)
  Elem* out;         // h [E*ce][N] (gate/up) or z [T*k][N] (down)
  const int32_t* counts;
  const int32_t* offsets;
  const int32_t* perm;
  int E, ce, r, K, N;  // N = output features: f (gate/up) or d (down)
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

template <typename Elem, int WI, int WJ, bool kGateUp>
__global__ __launch_bounds__(256, 1) void grouped_ffn_gemm_kernel(
    GemmParams<Elem> p) {
  typedef MmaOp<Elem> Op;
  constexpr int kVec = 16 / sizeof(Elem);        // elements per 16 B chunk
  constexpr int kStageK = 128 / sizeof(Elem);    // k elements per stage
  constexpr int BN = 64 * WI;                    // weight rows per tile
  constexpr int BM = 64 * WJ;                    // token rows per tile
  constexpr int NF = kGateUp ? BN / 2 : BN;      // output features per tile
  constexpr int kWPasses = BN / 32;              // 32 rows per load pass
  constexpr int kTPasses = BM / 32;
  constexpr int kStageBytes = (BN + BM) * 128;

  __shared__ __attribute__((aligned(16))) char smem[2 * kStageBytes];
  __shared__ int tile_pre[kWave + 1];
  __shared__ int rows_m[kWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave_id = tid / kWave;
  const int wn = wave_id & 1;   // weight-row half of the tile
  const int wm = wave_id >> 1;  // token half of the tile
  const int half = lane / 32;
  const int l32 = lane & 31;
  const int swz = lane & 7;

  const int nt = (p.N + NF - 1) / NF;
  if (tid < kWave) {
    const int e = tid;
    const int m = e < p.E ? rows_in_round(p.counts[e], p.r, p.ce) : 0;
    rows_m[e] = m;
    const int tiles = ((m + BM - 1) / BM) * nt;
    const int incl = wave_inclusive_scan(tiles);
    tile_pre[e + 1] = incl;
    if (e == 0) tile_pre[0] = 0;
  }
  __syncthreads();
  const int total = tile_pre[p.E];

  // XCD-contiguous walk: workgroup b runs on XCD b % 8.
  const int G = gridDim.x;
  const int slot = (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8);

  // load-pass geometry: thread covers chunk ch of rows r0 + 32*i
  const int r0 = tid >> 3;
  const int ch = tid & 7;

  for (int tile = slot; tile < total; tile += G) {
    const int e = segment_of(tile_pre, p.E + 1, tile);
    const int m = rows_m[e];
    const int mt = (m + BM - 1) / BM;
    const int local = tile - tile_pre[e];
    const int n0 = (local / mt) * NF;
    const int m0 = (local % mt) * BM;

    const Elem* wbase0 = p.w0 + (int64_t)e * p.N * p.K;
    const Elem* wbase1 = kGateUp ? p.w1 + (int64_t)e * p.N * p.K : nullptr;
    const Elem* abase = p.act + (int64_t)e * p.ce * p.K;

    // per-pass source rows as 32-bit element offsets inside the expert's
    // matrices (the layer's limits keep N*K and C'*K below 2^31). For gate/up
    // the first half of each wavefront's weight rows are gate rows and the
    // second half up rows of the same features; which one a pass loads is
    // fixed by the pass index alone.
    int32_t off[kWPasses + kTPasses];
#pragma unroll
    for (int i = 0; i < kWPasses; ++i) {
      int feat;
      if (kGateUp)
        feat = n0 + (i / WI) * (BN / 4) + 32 * ((i % WI) % (WI / 2)) + r0;
      else
        feat = n0 + 32 * i + r0;
      feat = feat < p.N ? feat : p.N - 1;
      off[i] = feat * p.K + ch * kVec;
    }
#pragma unroll
    for (int j = 0; j < kTPasses; ++j) {
      int c = m0 + r0 + 32 * j;
      c = c < m ? c : m - 1;
      off[kWPasses + j] = c * p.K + ch * kVec;
    }
    const int lds_w = (r0 * 128) + ((ch ^ (r0 & 7)) * 16);

    f32x16 acc[WI][WJ];
#pragma unroll
    for (int ib = 0; ib < WI; ++ib)
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[ib][jb][v] = 0.f;

    auto src = [&](int i) -> const Elem* {
      if (i >= kWPasses) return abase + off[i];
      if (kGateUp && (i % WI) >= WI / 2) return wbase1 + off[i];
      return wbase0 + off[i];
    };
    u32x4 stage[kWPasses + kTPasses];
    const int KT = p.K / kStageK;

    // prologue: stage 0
#pragma unroll
    for (int i = 0; i < kWPasses + kTPasses; ++i)
      stage[i] = *reinterpret_cast<const u32x4*>(src(i));
#pragma unroll
    for (int i = 0; i < kWPasses + kTPasses; ++i)
      *reinterpret_cast<u32x4*>(smem + lds_w + i * 32 * 128) = stage[i];
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const char* buf = smem + (kt & 1) * kStageBytes;
      const bool more = kt + 1 < KT;
      if (more) {
        const int koff = (kt + 1) * kStageK;
#pragma unroll
        for (int i = 0; i < kWPasses + kTPasses; ++i)
          stage[i] = *reinterpret_cast<const u32x4*>(src(i) + koff);
      }
      const char* wrow = buf + (wn * (BN / 2) + l32) * 128;
      const char* trow = buf + BN * 128 + (wm * (BM / 2) + l32) * 128;
#pragma unroll
      for (int s = 0; s < Op::kSteps; ++s) {
        typename Op::frag_t a[WI], b[WJ];
#pragma unroll
        for (int ib = 0; ib < WI; ++ib) a[ib] = Op::load(wrow + ib * 32 * 128, s, half, swz);
#pragma unroll
        for (int jb = 0; jb < WJ; ++jb) b[jb] = Op::load(trow + jb * 32 * 128, s, half, swz);
#pragma unroll
        for (int ib = 0; ib < WI; ++ib)
#pragma unroll
          for (int jb = 0; jb < WJ; ++jb) Op::mma(acc[ib][jb], a[ib], b[jb]);
      }
      if (more) {
        char* nbuf = smem + ((kt + 1) & 1) * kStageBytes;
#pragma unroll
        for (int i = 0; i < kWPasses + kTPasses; ++i)
          *reinterpret_cast<u32x4*>(nbuf + lds_w + i * 32 * 128) = stage[i];
      }
      __syncthreads();
    }

    // epilogue
    typedef Elem vec4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int jb = 0; jb < WJ; ++jb) {
      const int c = m0 + wm * (BM / 2) + jb * 32 + l32;
      if (c >= m) continue;
      Elem* orow;
      if (kGateUp) {
        orow = p.out + ((int64_t)e * p.ce + c) * p.N;
      } else {
        const int a = p.perm[p.offsets[e] + (int64_t)p.r * p.ce + c];
        orow = p.out + (int64_t)a * p.N;
      }
      if (kGateUp) {
#pragma unroll
        for (int ib = 0; ib < WI / 2; ++ib) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int feat = n0 + wn * (BN / 4) + ib * 32 + 8 * g4 + 4 * half;
            if (feat >= p.N) continue;
            vec4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              o[q] = from_f32<Elem>(silu_mul(acc[ib][jb][4 * g4 + q],
                                             acc[ib + WI / 2][jb][4 * g4 + q]));
            *reinterpret_cast<vec4_t*>(orow + feat) = o;
          }
        }
      } else {
#pragma unroll
        for (int ib = 0; ib < WI; ++ib) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int feat = n0 + wn * (BN / 2) + ib * 32 + 8 * g4 + 4 * half;
            if (feat >= p.N) continue;
            vec4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = from_f32<Elem>(acc[ib][jb][4 * g4 + q]);
            *reinterpret_cast<vec4_t*>(orow + feat) = o;
          }
        }
      }
    }
  }
}

// Tile shapes: bf16 uses 256 x 256 tiles (4 x 4 MFMA blocks per wavefront);
// fp32 uses 128 x 128.
template <typename Elem>
struct TileCfg;
template <>
struct TileCfg<bf16> {
  static constexpr int WI = 4, WJ = 4;
};
template <>
struct TileCfg<float> {
  static constexpr int WI = 2, WJ = 2;
};

template <typename Elem, bool kGateUp>
static hipError_t launch_gemm(const GemmParams<Elem>& p, int num_cus,
                              hipStream_t st) {
  constexpr int WI = TileCfg<Elem>::WI, WJ = TileCfg<Elem>::WJ;
  int G = num_cus;  // one 256-thread workgroup per CU (LDS-limited)
  G = (G + 7) / 8 * 8;
  hipLaunchKernelGGL((grouped_ffn_gemm_kernel<Elem, WI, WJ, kGateUp>), dim3(G),
                     dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_gate_up(const Shape& s, int r, const void* xr,
                          const void* wg, const void* wu, const int32_t* counts,
                          void* h, int num_cus, hipStream_t st) {
  if (s.bf16) {
    GemmParams<bf16> p{static_cast<const bf16*>(xr), static_cast<const bf16*>(wg),
                       static_cast<const bf16*>(wu), static_cast<bf16*>(h),
                       counts, nullptr, nullptr, s.E, s.ce, r, s.d, s.f};
    return launch_gemm<bf16, true>(p, num_cus, st);
  }
  GemmParams<float> p{static_cast<const float*>(xr), static_cast<const float*>(wg),
                      static_cast<const float*>(wu), static_cast<float*>(h),
                      counts, nullptr, nullptr, s.E, s.ce, r, s.d, s.f};
  return launch_gemm<float, true>(p, num_cus, st);
}

hipError_t launch_down(const Shape& s, int r, const void* h, const void* wd,
                       const PlanBuffers& b, void* z, int num_cus,
                       hipStream_t st) {
  if (s.bf16) {
    GemmParams<bf16> p{static_cast<const bf16*>(h), static_cast<const bf16*>(wd),
                       nullptr, static_cast<bf16*>(z), b.counts, b.offsets,
                       b.perm, s.E, s.ce, r, s.f, s.d};
    return launch_gemm<bf16, false>(p, num_cus, st);
  }
  GemmParams<float> p{static_cast<const float*>(h), static_cast<const float*>(wd),
                      nullptr, static_cast<float*>(z), b.counts, b.offsets,
                      b.perm, s.E, s.ce, r, s.f, s.d};
  return launch_gemm<float, false>(p, num_cus, st);
}

}  // namespace moe
