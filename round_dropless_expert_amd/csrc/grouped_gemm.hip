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
// blocks and WI 32-weight-row blocks. K advances 64 bytes per stage (32 bf16
// or 16 fp32); SPB stages form a slot of a four-slot LDS ring filled by
// LDS-direct buffer loads, with up to three slots in flight and one barrier
// per slot. Fragment reads run one MFMA step ahead of the MFMAs that use
// them. Two tile shapes: 256 weight rows x 256 tokens, and 128 x 64 (three
// stages per slot) for rounds with too few rows to give every CU a large
// tile, which mostly stream weights and need many workgroups.
//
// Determinism: every output element is one fixed sequence of MFMA steps
// over K in ascending order, whatever the round, the slot or the tile it
// falls in, so the result of a token does not depend on the capacity.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

template <typename Elem>
struct MmaOp;

// LDS stage layout: every tile row (weight rows first, then token rows)
// holds 64 bytes of K per stage, as four 16-byte chunks; logical chunk c of
// row q sits at physical chunk c ^ ((q >> 2) & 3). The 16 rows that one
// ds_read_b128 touches per LDS cycle then cover all 64 banks once.
constexpr int kRowBytes = 64;

__device__ __forceinline__ int lds_swizzle(int row, int chunk) {
  return (chunk ^ ((row >> 2) & 3)) * 16;
}

// v_mfma_f32_32x32x16_bf16: lane l supplies row (l % 32) and k-run
// [8*(l/32), 8*(l/32)+8) of its operand; one stage holds 2 such steps.
template <>
struct MmaOp<bf16> {
  static constexpr int kSteps = 2;
  typedef bf16x8 frag_t;
  __device__ static __forceinline__ frag_t load(const char* stage, int row,
                                                int step, int half) {
    return *reinterpret_cast<const frag_t*>(stage + row * kRowBytes +
                                            lds_swizzle(row, 2 * step + half));
  }
  __device__ static __forceinline__ void mma(f32x16& acc, frag_t a, frag_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
};

// v_mfma_f32_32x32x2f32: lane l supplies row (l % 32) and k = l / 32; one
// stage (16 floats) holds 8 steps.
template <>
struct MmaOp<float> {
  static constexpr int kSteps = 8;
  typedef float frag_t;
  __device__ static __forceinline__ frag_t load(const char* stage, int row,
                                                int step, int half) {
    const int byte = (2 * step + half) * 4;
    return *reinterpret_cast<const float*>(stage + row * kRowBytes +
                                           lds_swizzle(row, byte >> 4) + (byte & 15));
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
  int ce_pad;          // round-buffer rows per expert (multiple of 64)
  int tiled_w;         // weights in the tiled layout (else row-major)
};

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// Buffer resource word 3 for gfx9-family raw (untyped) buffer access.
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((address_space(3))) char lds_char;
// Wait until at most N of this wavefront's vector-memory operations are
// outstanding (the LDS-direct loads of later stages), then join the
// workgroup barrier. A bare s_barrier: __syncthreads() would also drain
// every in-flight stage.
template <int N>
__device__ __forceinline__ void wait_vmem_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename Elem, int WI, int WJ>
struct Frags {
  typename MmaOp<Elem>::frag_t a[WI], b[WJ];
};

template <typename Elem, int WI, int WJ>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[WI][WJ],
                                         const Frags<Elem, WI, WJ>& f) {
#pragma unroll
  for (int ib = 0; ib < WI; ++ib)
#pragma unroll
    for (int jb = 0; jb < WJ; ++jb) MmaOp<Elem>::mma(acc[ib][jb], f.a[ib], f.b[jb]);
}

// Scheduling pins for one MFMA step: one LDS fragment read after each of
// the first MFMAs, then (when a stage is being fetched) one LDS-direct
// buffer load after each of the following MFMAs, then the remaining MFMAs.
template <int kMfma, int kReads, int kLoads>
__device__ __forceinline__ void pin_step() {
  constexpr int nl = kReads < kMfma ? kReads : kMfma;
#pragma unroll
  for (int g = 0; g < nl; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
  if constexpr (kReads > nl) __builtin_amdgcn_sched_group_barrier(0x100, kReads - nl, 0);
  constexpr int room = kMfma - nl;
  constexpr int nv = kLoads < room ? kLoads : room;
#pragma unroll
  for (int g = 0; g < nv; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // VMEM read
  }
  if constexpr (kLoads > nv) __builtin_amdgcn_sched_group_barrier(0x020, kLoads - nv, 0);
  if constexpr (room - nv > 0) __builtin_amdgcn_sched_group_barrier(0x008, room - nv, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// K pipeline: a ring of kSlots LDS slots, each holding SPB consecutive
// 64-byte K stages (a "super-stage"). Each super-stage has one barrier,
// placed before its last MFMA step; the barrier waits for super-stage
// ks + 1 (ks + 2 and ks + 3 stay in flight), after which the next
// super-stage's first fragments load while the last step's MFMAs run. The
// first MFMA step of super-stage ks issues the fetch of ks + kSlots - 1 into
// the slot freed at the previous barrier, one load between MFMAs.
constexpr int kSlots = 4;  // the stage loop below names four slots

// Tile configurations (WI / WJ: 32-row MFMA blocks per wavefront along
// weight rows / tokens; the 2 x 2 wavefronts cover 64*WI weight rows and
// 64*WJ tokens; SPB: 64-byte K stages per slot and barrier).
struct TileBig {    // rounds with more than 64 rows in some expert
  static constexpr int WI = 4, WJ = 4, SPB = 1;
};
struct TileSmall {  // rounds too small to give every CU a large tile: such
                    // a round mostly streams expert weights; spread them
                    // over more workgroups and keep more bytes in flight
  static constexpr int WI = 2, WJ = 1, SPB = 3;
};

template <typename Elem, int WI, int WJ, int SPB, bool kGateUp>
__global__ __launch_bounds__(256, 1) void grouped_ffn_gemm_kernel(
    GemmParams<Elem> p) {
  typedef Frags<Elem, WI, WJ> frags_t;
  constexpr int kEs = sizeof(Elem);
  constexpr int kStageK = kRowBytes / kEs;       // k elements per stage
  constexpr int BN = 64 * WI;                    // weight rows per tile
  constexpr int BM = 64 * WJ;                    // token rows per tile
  constexpr int NF = kGateUp ? BN / 2 : BN;      // output features per tile
  constexpr int kWPasses = BN / 64;              // 64 rows per load pass
  constexpr int kTPasses = BM / 64;
  constexpr int kPasses = kWPasses + kTPasses;
  constexpr int kStageBytes = (BN + BM) * kRowBytes;
  constexpr int kSlotBytes = SPB * kStageBytes;
  constexpr int kLoads = SPB * kPasses;          // loads per slot and thread
  constexpr int kSteps = MmaOp<Elem>::kSteps;
  constexpr int kMfmaPerStep = WI * WJ;
  constexpr int kReadsPerStep = WI + WJ;
  static_assert(kSteps % 2 == 0, "fragment sets alternate by step");
  static_assert(WI % 2 == 0, "gate/up pairs and the 2 x 2 wavefront grid");
  static_assert(kLoads * (kSlots - 2) <= 63, "vmcnt budget");

  // the ring: kSlots slots as separate LDS objects, so the compiler can
  // tell a fragment read of one slot from a pending LDS-direct fill of
  // another and needs no conservative wait between them
  __shared__ __attribute__((aligned(1024))) char slot0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char slot1[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char slot2[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char slot3[kSlotBytes];
  __shared__ int tile_pre[kWave + 1];
  __shared__ int rows_m[kWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave_id = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wn = wave_id & 1;   // weight-row half of the tile
  const int wm = wave_id >> 1;  // token half of the tile
  const int half = lane / 32;
  const int l32 = lane & 31;

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
  const int total = __builtin_amdgcn_readfirstlane(tile_pre[p.E]);

  // XCD-contiguous walk: workgroup b runs on XCD b % 8.
  const int G = gridDim.x;
  const int slot = (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8);

  // Row order inside a stage: weight rows, then token rows. For gate/up the
  // weight rows are all gate rows (features n0 .. n0+NF-1), then all up
  // rows of the same features, so every 64-row load pass reads one matrix.
  // Load passes: pass i fills stage rows 64*i .. 64*i+63; lane tid writes
  // bytes [16*tid, 16*tid+16) of the pass: row r0 = tid / 4, physical
  // chunk tid % 4, i.e. logical chunk (tid % 4) ^ ((r0 >> 2) & 3).
  const int r0 = tid >> 2;
  const int chunk = (tid & 3) ^ ((r0 >> 2) & 3);
  // fragment rows of this lane: weight block ib, token block 0
  auto wrow_of = [&](int ib) {
    if (kGateUp)
      return (ib < WI / 2 ? 0 : BN / 2) + wn * (BN / 4) + (ib % (WI / 2)) * 32 + l32;
    return wn * (BN / 2) + ib * 32 + l32;
  };
  const int trow = BN + wm * (BM / 2) + l32;

  for (int tile = slot; tile < total; tile += G) {
    const int e = __builtin_amdgcn_readfirstlane(segment_of(tile_pre, p.E + 1, tile));
    const int m = __builtin_amdgcn_readfirstlane(rows_m[e]);
    const int mt = (m + BM - 1) / BM;
    const int local = tile - __builtin_amdgcn_readfirstlane(tile_pre[e]);
    const int n0 = (local / mt) * NF;
    const int m0 = (local % mt) * BM;

    const uint32_t wbytes = (uint32_t)p.N * p.K * kEs;
    const uint32_t kbytes = (uint32_t)p.K * kEs;    // bytes of one row
    const uint32_t band_bytes = kbytes * kTileRows;  // one 64-row band, tiled
    const __amdgpu_buffer_rsrc_t rw0 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w0 + (int64_t)e * p.N * p.K), 0, (int)wbytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw1 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kGateUp ? p.w1 + (int64_t)e * p.N * p.K : p.w0), 0, (int)wbytes,
        kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.act + (int64_t)e * p.ce_pad * p.K), 0,
        (int)((uint32_t)p.ce_pad * kbytes), kRsrcWord3);

    // Byte offsets (k = 0) of what this lane fetches in each pass. A pass
    // covers one 64-row band: tiled operands give one contiguous 4 KiB
    // block per stage (the lane's 16 bytes at 16 * tid); row-major weights
    // give this lane's row r0 of the band, logical chunk `chunk`.
    uint32_t voff[kPasses];
#pragma unroll
    for (int i = 0; i < kWPasses; ++i) {
      int feat0 = n0 + 64 * i;
      if (kGateUp && 64 * i >= BN / 2) feat0 -= BN / 2;  // an up-row pass
      if (p.tiled_w) {
        const int band = feat0 < p.N ? feat0 / 64 : p.N / 64 - 1;
        voff[i] = (uint32_t)band * band_bytes + tid * 16;
      } else {
        int feat = feat0 + r0;
        feat = feat < p.N ? feat : p.N - 1;
        voff[i] = (uint32_t)feat * kbytes + chunk * 16;
      }
    }
#pragma unroll
    for (int j = 0; j < kTPasses; ++j)  // bands past ce_pad read as zeros
      voff[kWPasses + j] = (uint32_t)(m0 / 64 + j) * band_bytes + tid * 16;
    const uint32_t wstride = p.tiled_w ? (uint32_t)kTileBytes : (uint32_t)kRowBytes;

    f32x16 acc[WI][WJ];
#pragma unroll
    for (int ib = 0; ib < WI; ++ib)
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[ib][jb][v] = 0.f;

    const int KT = p.K / kStageK;

    // Fetch super-stage ks (stages ks*SPB .. ks*SPB+SPB-1) into `slot` with
    // LDS-direct buffer loads (lane i of a wavefront writes bytes
    // [16 i, 16 i + 16) of its 1 KiB share of each 4 KiB pass). A stage at
    // or past the end of K is fetched with an offset beyond the buffer: the
    // hardware returns zeros without touching memory, so such a stage adds
    // exact zeros to the accumulators. K is walked in groups of kSlots
    // super-stages, the last group padded this way.
    auto fetch = [&](char* slot_mem, int ks) {
#pragma unroll
      for (int sub = 0; sub < SPB; ++sub) {
        const int g = ks * SPB + sub;
        lds_char* dst = (lds_char*)slot_mem + sub * kStageBytes + wave_id * 1024;
        const bool live = g < KT;
        const uint32_t soff_w = live ? (uint32_t)g * wstride : 0x80000000u;
#pragma unroll
        for (int i = 0; i < kPasses; ++i) {
          const __amdgpu_buffer_rsrc_t rs =
              i >= kWPasses ? ra : ((kGateUp && 64 * i >= BN / 2) ? rw1 : rw0);
          // token bands at or past the expert's m rows feed only outputs
          // that are never stored: fetch them as zeros too
          const bool band_live = i < kWPasses || m0 + 64 * (i - kWPasses) < m;
          const uint32_t soff = i < kWPasses
                                    ? soff_w
                                    : (live && band_live ? (uint32_t)g * kTileBytes
                                                         : 0x80000000u);
          // (scalar copy: clang's host pass drops the launch stub when an
          // array element is passed to this builtin directly)
          const uint32_t vo = voff[i];
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              rs, (void __attribute__((address_space(3)))*)(dst + i * 4096), 16, vo,
              soff, 0, 0);
        }
      }
    };

    frags_t f0, f1;
    // fragments of step s of the stage at `stage`
    auto frags = [&](frags_t& f, const char* stage, int s) {
#pragma unroll
      for (int ib = 0; ib < WI; ++ib)
        f.a[ib] = MmaOp<Elem>::load(stage, wrow_of(ib), s, half);
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb)
        f.b[jb] = MmaOp<Elem>::load(stage, trow + 32 * jb, s, half);
    };

#define MOE_SUPER(CUR, NXT, FSLOT, KS_)                                          \
    _Pragma("unroll") for (int sub = 0; sub < SPB; ++sub) {                     \
      const char* cs = CUR + sub * kStageBytes;                                 \
      const char* ns = sub + 1 < SPB ? CUR + (sub + 1) * kStageBytes : NXT;     \
      _Pragma("unroll") for (int s = 0; s < kSteps; s += 2) {                   \
        frags(f1, cs, s + 1);                                                   \
        if (sub == 0 && s == 0) fetch(FSLOT, (KS_) + kSlots - 1);               \
        mma_step<Elem, WI, WJ>(acc, f0);                                        \
        if (sub == 0 && s == 0)                                                 \
          pin_step<kMfmaPerStep, kReadsPerStep, kLoads>();                      \
        else                                                                    \
          pin_step<kMfmaPerStep, kReadsPerStep, 0>();                           \
        if (s + 2 < kSteps) {                                                   \
          frags(f0, cs, s + 2);                                                 \
        } else {                                                                \
          if (sub + 1 == SPB) wait_vmem_barrier<(kSlots - 2) * kLoads>();       \
          frags(f0, ns, 0);                                                     \
        }                                                                       \
        mma_step<Elem, WI, WJ>(acc, f1);                                        \
        pin_step<kMfmaPerStep, kReadsPerStep, 0>();                             \
      }                                                                         \
    }

    // prologue: super-stages 0 .. kSlots-2 in flight; wait for the first
    fetch(slot0, 0);
    fetch(slot1, 1);
    fetch(slot2, 2);
    wait_vmem_barrier<(kSlots - 2) * kLoads>();
    frags(f0, slot0, 0);
    const int KS = (KT + SPB - 1) / SPB;
    const int KS4 = (KS + kSlots - 1) / kSlots * kSlots;
    for (int ks = 0; ks < KS4; ks += kSlots) {
      MOE_SUPER(slot0, slot1, slot3, ks)
      MOE_SUPER(slot1, slot2, slot0, ks + 1)
      MOE_SUPER(slot2, slot3, slot1, ks + 2)
      MOE_SUPER(slot3, slot0, slot2, ks + 3)
    }
#undef MOE_SUPER

    // epilogue: lane holds, for token j = l32 of each 32-token block, four
    // runs of four consecutive output features
    typedef Elem vec4_t __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int jb = 0; jb < WJ; ++jb) {
      const int c = m0 + wm * (BM / 2) + jb * 32 + l32;
      if (c >= m) continue;
      if (kGateUp) {
        // h: row c of expert e's tiled matrix
        char* hmat = reinterpret_cast<char*>(p.out + (int64_t)e * p.ce_pad * p.N);
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
            *reinterpret_cast<vec4_t*>(
                hmat + tiled_offset(c, (int64_t)feat * kEs, (int64_t)p.N * kEs)) = o;
          }
        }
      } else {
        // z: the assignment's token slot
        const int a = p.perm[p.offsets[e] + (int64_t)p.r * p.ce + c];
        Elem* orow = p.out + (int64_t)a * p.N;
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
    // the next tile's prologue refills the ring: every wavefront must be
    // done with its last fragment reads
    __syncthreads();
  }
}

// Tiles one round needs under configuration Cfg (host side, from counts).
template <typename Cfg>
static int64_t round_tiles(const Shape& s, const int32_t* counts_host, int r,
                           int N, bool gate_up) {
  const int BM = 64 * Cfg::WJ;
  const int NF = gate_up ? 32 * Cfg::WI : 64 * Cfg::WI;
  const int64_t nt = (N + NF - 1) / NF;
  int64_t tiles = 0;
  for (int e = 0; e < s.E; ++e) {
    int64_t m = (int64_t)counts_host[e] - (int64_t)r * s.ce;
    m = m < 0 ? 0 : (m > s.ce ? s.ce : m);
    tiles += (m + BM - 1) / BM * nt;
  }
  return tiles;
}

// Workgroups for a round: one per CU, or fewer when the round has fewer
// tiles; a multiple of 8 (the XCD-contiguous walk assumes it).
static int grid_for(int64_t tiles, int num_cus) {
  int64_t g = tiles < num_cus ? tiles : num_cus;
  g = (g + 7) / 8 * 8;
  return (int)(g < 8 ? 8 : g);
}

template <typename Elem, typename Cfg, bool kGateUp>
static hipError_t launch_gemm_cfg(const GemmParams<Elem>& p, int grid,
                                  hipStream_t st) {
  hipLaunchKernelGGL(
      (grouped_ffn_gemm_kernel<Elem, Cfg::WI, Cfg::WJ, Cfg::SPB, kGateUp>),
      dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

// counts_host (nullable): per-expert counts on the host. With them the
// round's tile shape and grid are chosen from its largest expert; without
// them the large tile and one workgroup per CU are used. Both shapes run the
// same MFMA sequence over K for every output, so results are identical.
template <typename Elem, bool kGateUp>
static hipError_t launch_gemm(const Shape& s, const GemmParams<Elem>& p,
                              const int32_t* counts_host, int num_cus,
                              hipStream_t st) {
  const int N = kGateUp ? s.f : s.d;
  if (counts_host) {
    int64_t mmax = 0;
    for (int e = 0; e < s.E; ++e) {
      int64_t m = (int64_t)counts_host[e] - (int64_t)p.r * s.ce;
      m = m < 0 ? 0 : (m > s.ce ? s.ce : m);
      mmax = m > mmax ? m : mmax;
    }
    if (mmax == 0) return hipSuccess;  // nothing in this round
    // the large tile when it gives every CU at least one tile, else the
    // small one (rounds of a few rows per expert stream weights)
    const int64_t tb = round_tiles<TileBig>(s, counts_host, p.r, N, kGateUp);
    if (tb >= num_cus)
      return launch_gemm_cfg<Elem, TileBig, kGateUp>(p, grid_for(tb, num_cus), st);
    const int64_t t = round_tiles<TileSmall>(s, counts_host, p.r, N, kGateUp);
    return launch_gemm_cfg<Elem, TileSmall, kGateUp>(p, grid_for(t, num_cus), st);
  }
  return launch_gemm_cfg<Elem, TileBig, kGateUp>(p, grid_for(num_cus, num_cus), st);
}

hipError_t launch_gate_up(const Shape& s, int r, const void* xr,
                          const void* wg, const void* wu, const int32_t* counts,
                          const int32_t* counts_host, void* h, int num_cus,
                          hipStream_t st) {
  if (s.bf16) {
    GemmParams<bf16> p{static_cast<const bf16*>(xr), static_cast<const bf16*>(wg),
                       static_cast<const bf16*>(wu), static_cast<bf16*>(h),
                       counts, nullptr, nullptr, s.E, s.ce, r, s.d, s.f,
                       s.ce_pad(), s.tiled_w};
    return launch_gemm<bf16, true>(s, p, counts_host, num_cus, st);
  }
  GemmParams<float> p{static_cast<const float*>(xr), static_cast<const float*>(wg),
                      static_cast<const float*>(wu), static_cast<float*>(h),
                      counts, nullptr, nullptr, s.E, s.ce, r, s.d, s.f,
                      s.ce_pad(), s.tiled_w};
  return launch_gemm<float, true>(s, p, counts_host, num_cus, st);
}

hipError_t launch_down(const Shape& s, int r, const void* h, const void* wd,
                       const PlanBuffers& b, const int32_t* counts_host, void* z,
                       int num_cus, hipStream_t st) {
  if (s.bf16) {
    GemmParams<bf16> p{static_cast<const bf16*>(h), static_cast<const bf16*>(wd),
                       nullptr, static_cast<bf16*>(z), b.counts, b.offsets,
                       b.perm, s.E, s.ce, r, s.f, s.d, s.ce_pad(), s.tiled_w};
    return launch_gemm<bf16, false>(s, p, counts_host, num_cus, st);
  }
  GemmParams<float> p{static_cast<const float*>(h), static_cast<const float*>(wd),
                      nullptr, static_cast<float*>(z), b.counts, b.offsets,
                      b.perm, s.E, s.ce, r, s.f, s.d, s.ce_pad(), s.tiled_w};
  return launch_gemm<float, false>(s, p, counts_host, num_cus, st);
}

}  // namespace moe
