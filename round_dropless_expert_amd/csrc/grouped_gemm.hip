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
// them. Three tile shapes, chosen per round: 256 weight rows x 256 tokens,
// 256 x 128, and 128 x 64 (two stages per slot) for rounds of a few rows
// per expert, which mostly stream weights and need many workgroups.
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

// What a launch computes (the operand passes and the epilogue):
//   kModeGateUp    forward: h = silu(xr Wg^T) * (xr Wu^T) into h; with
//                  kGather the token rows are read from x through the plan
//                  instead of from a dispatched round buffer xr (below)
//   kModeDown      forward: o = h Wd^T into z rows
//   kModeRecompute backward: g = xr Wg^T and u = xr Wu^T into gu
//                  ([rows][2f]: g, then u) and w * silu(g) u into hw
//   kModeDgate     backward: dh = dyr Wd, then dg = w dh u silu'(g) and
//                  du = w dh silu(g) into dgu ([rows][2f]), with g, u read
//                  from gu
//   kModeDx        backward: dx rows = dgu [Wg; Wu] into dz rows (as z)
// The last two contract over the weights' rows (Wd [d][f] over d, Wg and
// Wu [f][d] over f): they read the forward's weight matrices transposed
// (below), so the backward needs no second copy of the weights.
enum GemmMode {
  kModeGateUp = 0,
  kModeDown = 1,
  kModeRecompute = 2,
  kModeDgate = 3,
  kModeDx = 4
};

template <typename Elem>
struct GemmParams {
  const Elem* act;   // round buffer [rows][K]: xr (gate/up) or h (down)
  const Elem* x;     // gathering gate/up: the layer's input x [T][K]
  int x_bytes;       // its bytes (at most 2^30)
  int topk;          // k: assignment a is token a / k's
  const Elem* w0;    // [E][N][K]: gate (gate/up) or down weights; dgate:
                     // down weights [E][K][N]; dx: gate weights [E][K/2][N]
  const Elem* w1;    // [E][N][K]: up weights (gate/up); dx: up [E][K/2][N]
  Elem* out;         // h [rows][N] (gate/up) or z [T*k][N] (down)
  Elem* out2;        // hw [rows][N] (recompute only)
  const Elem* aux;   // gu [rows][2N] (dgate only)
  const float* weight;     // routing weights [T*k] (recompute, dgate)
  const int32_t* perm;     // the plan's permutation (recompute, dgate)
  const int32_t* rounds;   // the plan's round tables (RoundTable)
  const int32_t* n_rounds; // R: rounds >= R have no pairs (their tables are unset)
  int E, r0, nr, K, N; // rounds [r0, r0 + nr) of one batch; N = output
                       // features: f (gate/up) or d (down)
  int max_rounds;      // rows of each round table
  int tiled_w;         // weights in the tiled layout (else row-major)
};

// silu(g) * u = g * u / (1 + e^-g), with the hardware base-2 exponential
// (e^-g = 2^(-g log2 e)) and reciprocal (each about 1 ulp): a handful of
// instructions per element instead of a full-precision exp and divide,
// since the epilogue runs while the matrix cores idle. Large -g gives
// 2^+inf = inf and a zero reciprocal (silu -> -0), large g gives 1.
__device__ __forceinline__ float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  return g * u * __builtin_amdgcn_rcpf(1.0f + e);
}

// An accumulator element, read from its AGPR at this point of the program
// (asm, so that the epilogue moves a few values at a time into VGPRs rather
// than the compiler copying every accumulator out at once).
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// Buffer resource word 3 for gfx9-family raw (untyped) buffer access.
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((address_space(3))) char lds_char;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Buffer-to-LDS loads (LDS-direct): lane i reads `bytes` at voff + soff
// of the buffer and writes them to LDS at m0 + bytes * i. Written as asm:
// the compiler then neither tracks them (every wait on them is the kernel's
// own, explicit and exact, vmcnt count) nor moves them, so they stay
// exactly where the stage loop interleaves them with the MFMAs. They have
// no register results. M0 is declared clobbered (the compiler restores it
// where it needs it); one wait state separates the M0 write from the load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                           uint32_t soff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
      : "m0");
}
#pragma clang diagnostic pop

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

// One MFMA step (WI x WJ MFMAs) with kOps other instructions spread over
// it in a fixed order: op(x) for x = 0 .. kOps-1 (fragment reads of the
// next step first, then LDS-direct loads), issued after MFMA i for
// x in [i*kOps/M, (i+1)*kOps/M). Each group is fenced, so the compiler keeps
// the order; it still inserts the LDS-read waits before the MFMAs of the
// next step that consume them.
template <typename Elem, int WI, int WJ, int kOps, typename Op>
__device__ __forceinline__ void mma_step(f32x16 (&acc)[WI][WJ],
                                         const Frags<Elem, WI, WJ>& f, Op op) {
  constexpr int M = WI * WJ;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    MmaOp<Elem>::mma(acc[i / WJ][i % WJ], f.a[i / WJ], f.b[i % WJ]);
#pragma unroll
    for (int x = i * kOps / M; x < (i + 1) * kOps / M; ++x) op(x);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// K pipeline: a ring of kSlots LDS slots, each holding SPB consecutive
// 64-byte K stages (a "super-stage"). Each super-stage has one barrier,
// placed before its last MFMA step; the barrier waits for super-stage
// ks + 1 (ks + 2 and ks + 3 stay in flight), after which the next
// super-stage's first fragments load while the last step's MFMAs run. The
// first MFMA step of super-stage ks issues the fetch of ks + 3 into the slot
// freed at the previous barrier, one load between MFMAs. The ring runs on
// across tiles: the last three fetches of a tile bring the first three
// super-stages of the workgroup's next tile, so a tile's SwiGLU / store
// epilogue overlaps those loads and the next tile starts with data in LDS.
constexpr int kSlots = 4;  // the stage loop below names four slots

// Tile configurations (WI / WJ: 32-row MFMA blocks per wavefront along
// weight rows / tokens; the 2 x 2 wavefronts cover 64*WI weight rows and
// 64*WJ tokens; SPB: 64-byte K stages per slot and barrier).
// The host picks, per round, the shape with the least estimated time
// (waves of tiles over the CUs x tile area / relative MFMA efficiency).
struct TileBig {     // 256 weight rows x 256 tokens: 128 FLOP per byte
  static constexpr int WI = 4, WJ = 4, SPB = 1;
  static constexpr float kEff = 1.0f;
};
struct TileMedium {  // 256 x 128: rounds of one or a few experts with
                     // thousands of rows, which 256 x 256 tiles leave
                     // mostly idle
  static constexpr int WI = 4, WJ = 2, SPB = 1;
  static constexpr float kEff = 0.85f;
};
struct TileSmall {   // 128 x 64, two K stages per slot: rounds of a few
                     // rows per expert, which mostly stream weights and
                     // need many workgroups
  static constexpr int WI = 2, WJ = 1, SPB = 2;
  static constexpr float kEff = 0.45f;
};

// Cache-policy operand of a buffer store: non-temporal (streaming).
constexpr int kNonTemporal = 2;

// Offset that puts a buffer load out of range: the load returns zeros and
// touches no memory (every real offset is below 2^31, so a real base plus
// this offset is still out of range).
constexpr uint32_t kOutOfRange = 0x80000000u;

// Where one tile's operands live: buffer descriptors over the expert's
// weights and round rows, and the uniform byte offset (k = 0) of each 64-row
// load pass. Everything is wavefront-uniform (scalar registers).
template <int kWPasses, int kTPasses>
struct TileSrc {
  __amdgpu_buffer_rsrc_t rw0, rw1, ra;
  uint32_t wbase[kWPasses];  // weight pass offsets
  uint32_t tbase[kTPasses];  // token pass offsets (past the rows: out of range)
  uint32_t vt[kTPasses];     // gathering: this lane's token row offset in x
                             // for each token pass (per lane, not uniform)
};

// Offset of a gathered token row past the pair's m rows: beyond any x (at
// most 2^30 bytes), and still below 2^32 with a stage offset added, even the
// out-of-range one of a stage past the end of K.
constexpr uint32_t kDeadRow = 0x40000000u;

template <typename Elem, int WI, int WJ, int SPB, int kMode, bool kGather>
__global__ __launch_bounds__(256, 1) void grouped_ffn_gemm_kernel(
    GemmParams<Elem> p) {
  static_assert(!kGather || kMode == kModeGateUp, "gathering: forward gate/up only");
  // two weight matrices per tile (gate rows, then up rows of the same
  // features)
  constexpr bool kGateUp = kMode == kModeGateUp || kMode == kModeRecompute;
  // weights read transposed: K runs along the matrices' rows
  constexpr bool kTransW = kMode == kModeDgate || kMode == kModeDx;
  typedef Frags<Elem, WI, WJ> frags_t;
  constexpr int kEs = sizeof(Elem);
  static_assert(!kTransW || kEs == 2, "transposed weights: bf16 only");
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
  constexpr int kReadsPerStep = WI + WJ;
  // The fetch of a super-stage is spread over all its MFMA steps (at most
  // kLoadsPerStep loads after the fragment reads of each step), so that the
  // address unit is never handed more loads than it retires while the
  // MFMAs run: a burst of LDS-direct loads stalls the issuing wavefront,
  // and with it the matrix core.
  constexpr int kStepsPerSuper = SPB * kSteps;
  constexpr int kLoadsPerStep = (kLoads + kStepsPerSuper - 1) / kStepsPerSuper;
  constexpr int kLoadsLast =  // loads in the last step (after the barrier)
      kLoads - (kStepsPerSuper - 1) * kLoadsPerStep > 0
          ? kLoads - (kStepsPerSuper - 1) * kLoadsPerStep : 0;
  // A barrier waits for the fetch of super-stage ks + 1; behind it in issue
  // order: the fetch of ks + 2 and the part of ks + 3 issued before it
  constexpr int kWait = kLoads + (kLoads - kLoadsLast);
  typedef TileSrc<kWPasses, kTPasses> src_t;
  static_assert(kSteps % 2 == 0, "fragment sets alternate by step");
  static_assert(WI % 2 == 0, "gate/up pairs and the 2 x 2 wavefront grid");
  static_assert(kWait <= 63, "vmcnt budget");

  // the ring: kSlots slots as separate LDS objects, so the compiler can
  // tell a fragment read of one slot from a pending LDS-direct fill of
  // another and needs no conservative wait between them
  __shared__ __attribute__((aligned(1024))) char slot0[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char slot1[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char slot2[kSlotBytes];
  __shared__ __attribute__((aligned(1024))) char slot3[kSlotBytes];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave_id = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wn = wave_id & 1;   // weight-row half of the tile
  const int wm = wave_id >> 1;  // token half of the tile
  const int half = lane / 32;
  const int l32 = lane & 31;

  // Every wavefront keeps the launch's tile table in registers: lane v holds
  // pair v of the launch (a round's expert with rows; the pairs of rounds
  // [r0, r0 + nr) are [rbeg[r0], rend[r0 + nr - 1]) of the plan's pair
  // tables): its expert, its rows m_v, the inclusive prefix of the tile
  // counts, the first buffer row of its matrix and, past gate/up, its first
  // row of z (offsets[e] + the index of its first entry of the round). A
  // launch reaching past R has no pairs.
  const int nt = (p.N + NF - 1) / NF;
  const int64_t tbl = (int64_t)p.max_rounds * p.E;
  const int32_t* rb = p.rounds + kTables * tbl;
  const int g0 = rb[p.r0];
  const int g1 = rb[p.max_rounds + p.r0 + p.nr - 1];
  const int nv = p.r0 + p.nr <= *p.n_rounds ? g1 - g0 : 0;
  const bool lv = lane < nv;
  const int64_t gi = (int64_t)g0 + lane;
  const int lane_e = lv ? p.rounds[kPairE * tbl + gi] : 0;
  const int lane_m = lv ? p.rounds[kPairM * tbl + gi] : 0;
  const int lane_incl = wave_inclusive_scan(((lane_m + BM - 1) / BM) * nt);
  const int total = __builtin_amdgcn_readlane(lane_incl, kWave - 1);
  const int lane_row = lv ? p.rounds[kPairRow * tbl + gi] : 0;
  const int lane_off =
      (kMode != kModeGateUp || kGather) && lv ? p.rounds[kPairZ * tbl + gi] : 0;

  // XCD-contiguous walk: workgroup b runs on XCD b % 8.
  const int G = gridDim.x;
  int tile = (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8);
  if (tile >= total) return;

  const uint32_t kbytes = (uint32_t)p.K * kEs;    // bytes of one row
  const uint32_t band_bytes = kbytes * kTileRows;  // one 64-row band, tiled
  // one expert's weight matrix (dx: each of its two), elements and bytes
  const int64_t wmat = (int64_t)p.N * (kMode == kModeDx ? p.K / 2 : p.K);
  const uint32_t wbytes = (uint32_t)(wmat * kEs);
  const uint32_t wstride = p.tiled_w ? (uint32_t)kTileBytes : (uint32_t)kRowBytes;
  // transposed weights: one matrix row holds N features; a tiled 64-row
  // band of the matrix is N / 32 blocks of 4 KiB
  const uint32_t nbytes = (uint32_t)p.N * kEs;
  const uint32_t band_bytes_t = nbytes * kTileRows;

  // Row order inside a stage: weight rows, then token rows. For gate/up the
  // weight rows are all gate rows (features n0 .. n0+NF-1), then all up
  // rows of the same features, so every 64-row load pass reads one matrix.
  // Load passes: pass i fills stage rows 64*i .. 64*i+63; lane tid writes
  // bytes [16*tid, 16*tid+16) of the pass: row r0 = tid / 4, physical
  // chunk tid % 4, i.e. logical chunk (tid % 4) ^ ((r0 >> 2) & 3). The
  // lane's part of the source offset is the same for every pass: a tiled
  // band is one contiguous 4 KiB block per stage; a row-major band gives
  // row r0 of the band, logical chunk `chunk`.
  //
  // Transposed weights: a stage is 32 K rows of the matrix, and pass i holds
  // the tile's output features 64 i .. 64 i + 63 as two 2 KiB half blocks,
  // one per 32 features: 32 rows (K) of 64 bytes (32 features), with the
  // tiled layout's chunk swizzle by row. From a tiled matrix each half block
  // is the upper or lower half of one 4 KiB block (rows k0 % 64 ..), copied
  // as it lies: lane tid moves bytes [16 (tid % 128), + 16) of half block
  // tid / 128. From a row-major matrix the lane gathers the 16 bytes that
  // belong at that place: row rt = (tid % 128) / 4, logical chunk
  // (tid % 4) ^ ((rt >> 2) & 3).
  const int r0 = tid >> 2;
  const int chunk = (tid & 3) ^ ((r0 >> 2) & 3);
  uint32_t vo_w;
  if constexpr (kTransW) {
    const int hb = tid >> 7, rt = (tid & 127) >> 2;
    const int lc = (tid & 3) ^ ((rt >> 2) & 3);
    vo_w = p.tiled_w ? (uint32_t)hb * kTileBytes + (uint32_t)(tid & 127) * 16
                     : (uint32_t)rt * nbytes + (uint32_t)(32 * hb + 8 * lc) * kEs;
  } else {
    vo_w = p.tiled_w ? (uint32_t)tid * 16 : (uint32_t)r0 * kbytes + chunk * 16;
  }
  const uint32_t vo_t = (uint32_t)tid * 16;

  // Tile t: pair (te, below), feature block and token block, and its operand
  // sources.
  // Weight rows at or past N and token bands past the expert's m rows fall
  // outside the descriptors' ranges, so they read as zeros; they only feed
  // outputs that are never stored. Offsets stay below 2^32: the matrices'
  // bytes are below 2^31 and a tile reaches at most three bands past them.
  int e = 0, m = 0, n0 = 0, m0 = 0;
  auto locate = [&](int t, int& te, int& tm, int& tn0, int& tm0) {
    // pair of the tile: the number of pairs whose tiles all come first
    te = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane_incl <= t));
    tm = __builtin_amdgcn_readlane(lane_m, te);
    const int mt = (tm + BM - 1) / BM;
    const int local = t - (te > 0 ? __builtin_amdgcn_readlane(lane_incl, te - 1) : 0);
    tn0 = (local / mt) * NF;
    tm0 = (local % mt) * BM;
  };
  auto sources = [&](int te, int tm, int tn0, int tm0, bool exists) {
    src_t S;
    const uint32_t wb = exists ? wbytes : 0u;  // no next tile: all out of range
    const int64_t ex = __builtin_amdgcn_readlane(lane_e, te);  // the pair's expert
    S.rw0 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(p.w0 + ex * wmat), 0, (int)wb, kRsrcWord3);
    S.rw1 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(kGateUp || kMode == kModeDx ? p.w1 + ex * wmat : p.w0), 0, (int)wb,
        kRsrcWord3);
    // pair te's matrix: its m rows padded to 64, from its first row
    // (gathering: all of x; each lane's row offsets select the rows)
    if constexpr (kGather)
      S.ra = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, p.x_bytes, kRsrcWord3);
    else
      S.ra = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.act + (int64_t)__builtin_amdgcn_readlane(lane_row, te) * p.K), 0,
          exists ? (int)((uint32_t)((tm + 63) & ~63) * kbytes) : 0, kRsrcWord3);
#pragma unroll
    for (int i = 0; i < kWPasses; ++i) {
      int feat0 = tn0 + 64 * i;
      if (kGateUp && 64 * i >= BN / 2) feat0 -= BN / 2;  // an up-row pass
      if constexpr (kTransW)  // the pass's first column (features past N: zeros)
        S.wbase[i] = feat0 >= p.N ? kOutOfRange
                     : p.tiled_w ? (uint32_t)(feat0 / 32) * kTileBytes
                                 : (uint32_t)feat0 * kEs;
      else
        S.wbase[i] = p.tiled_w ? (uint32_t)(feat0 / 64) * band_bytes
                               : (uint32_t)feat0 * kbytes;
    }
#pragma unroll
    for (int j = 0; j < kTPasses; ++j)
      S.tbase[j] = kGather ? 0u : (uint32_t)(tm0 / 64 + j) * band_bytes;
    return S;
  };
  // Gathering: token pass j of a tile holds the pair's rows tm0 + 64 j ..
  // + 63, and this lane fetches row tm0 + 64 j + r0 of them, logical chunk
  // `chunk` of each stage (as a row-major weight band), from x. Row c of
  // pair te is the assignment perm[z0 + c] (z0: the pair's first entry in
  // expert order), i.e. token perm[z0 + c] / k. perm_rows loads those
  // assignments (-1: past the pair's rows, or no tile); token_offs turns
  // them into the lane's byte offsets in x. The loads are the compiler's
  // own, issued a whole tile before token_offs uses them: the compiler,
  // which does not see the LDS-direct loads, waits there for the whole
  // vector-memory counter, at the top of a tile, where the ring's first
  // barrier waits for nearly all of it anyway (a build of the kernel that
  // reads xr with that full wait added ran at the same speed).
  auto perm_rows = [&](int te, int tm, int tm0, bool exists, int32_t (&pa)[kTPasses]) {
    const int64_t z0 = exists ? __builtin_amdgcn_readlane(lane_off, te) : 0;
#pragma unroll
    for (int j = 0; j < kTPasses; ++j) {
      const int row = tm0 + 64 * j + r0;
      pa[j] = exists && row < tm ? p.perm[z0 + row] : -1;
    }
  };
  auto token_offs = [&](const int32_t (&pa)[kTPasses], src_t& S) {
#pragma unroll
    for (int j = 0; j < kTPasses; ++j)
      S.vt[j] = pa[j] < 0 ? kDeadRow
                          : (uint32_t)(pa[j] / p.topk) * kbytes + (uint32_t)chunk * 16;
  };
  // Recompute and dgate: the epilogue scales row c of token block jb (c =
  // m0 + wm BM/2 + 32 jb + l32) by its assignment's routing weight,
  // weight[perm[z0 + c]]. Both loads are issued ahead (the assignments two
  // tiles, the weights one tile before the epilogue that uses them), so
  // that the compiler's waits for them fall at the top of a tile, like the
  // gathered rows' above, instead of two dependent loads with a wait each
  // in every epilogue block.
  constexpr bool kRowWeight = kMode == kModeRecompute || kMode == kModeDgate;
  auto epi_perm = [&](int te, int tm, int tm0, bool exists, int32_t (&pw)[WJ]) {
    const int64_t z0 = exists ? __builtin_amdgcn_readlane(lane_off, te) : 0;
#pragma unroll
    for (int jb = 0; jb < WJ; ++jb) {
      const int c = tm0 + wm * (BM / 2) + jb * 32 + l32;
      pw[jb] = exists && c < tm ? p.perm[z0 + c] : -1;
    }
  };
  auto epi_weight = [&](const int32_t (&pw)[WJ], float (&w)[WJ]) {
#pragma unroll
    for (int jb = 0; jb < WJ; ++jb) w[jb] = pw[jb] < 0 ? 0.f : p.weight[pw[jb]];
  };

  const int KT = p.K / kStageK;            // 64-byte K stages
  const int KS = (KT + SPB - 1) / SPB;     // super-stages of one tile
  const int KS4 = (KS + kSlots - 1) / kSlots * kSlots;

  // Load x of a super-stage's fetch into `slot_mem`: stage sub = x /
  // kPasses of the super-stage, pass i = x % kPasses (64 rows: weight rows,
  // then token rows); lane i of a wavefront writes bytes [16 i, 16 i + 16)
  // of its 1 KiB share of the pass's 4 KiB. The stage offsets along K are
  // computed once per super-stage (stage_off); a stage at or past the end of
  // K gets an out-of-range offset, reads as zeros and adds exact zeros. The
  // per-load scalar work is then one add: with one wavefront per SIMD every
  // instruction takes an issue slot the MFMA stream could use.
  const uint32_t lds_wave = (uint32_t)wave_id * 1024;
  // Transposed weights: stage g is rows 32 g' .. 32 g' + 31 of the matrix
  // (g' = g, or for dx g - KT / 2 of the up matrix once g reaches the
  // second half of K): half of a tiled band, or 32 row-major rows.
  struct StageOff {
    uint32_t w[SPB], t[SPB];
    bool up[SPB];  // dx: the stage's rows are up-matrix rows
  };
  auto stage_off = [&](int ks) {
    StageOff o;
#pragma unroll
    for (int sub = 0; sub < SPB; ++sub) {
      const int g = ks * SPB + sub;
      const bool in = g < KT;
      if constexpr (kTransW) {
        o.up[sub] = kMode == kModeDx && g >= KT / 2;
        const int gh = o.up[sub] ? g - KT / 2 : g;
        o.w[sub] = !in ? kOutOfRange
                   : p.tiled_w ? (uint32_t)(gh >> 1) * band_bytes_t +
                                     (uint32_t)(gh & 1) * (kTileBytes / 2)
                               : (uint32_t)gh * 32u * nbytes;
      } else {
        o.up[sub] = false;
        o.w[sub] = in ? (uint32_t)g * wstride : kOutOfRange;
      }
      o.t[sub] = in ? (uint32_t)g * (uint32_t)(kGather ? kRowBytes : kTileBytes)
                    : kOutOfRange;
    }
    return o;
  };
  auto fetch_one = [&](char* slot_mem, const StageOff& o, const src_t& S, int x) {
    const int sub = x / kPasses, i = x % kPasses;
    const bool w = i < kWPasses;
    const bool use_w1 = kTransW ? o.up[sub] : (kGateUp && 64 * i >= BN / 2);
    const __amdgpu_buffer_rsrc_t rs = !w ? S.ra : (use_w1 ? S.rw1 : S.rw0);
    const uint32_t soff = w ? S.wbase[i] + o.w[sub] : S.tbase[i - kWPasses] + o.t[sub];
    const uint32_t lds = (uint32_t)(uintptr_t)(lds_char*)slot_mem +
                         sub * kStageBytes + i * 4096 + lds_wave;
    lds_load16(rs, w ? vo_w : kGather ? S.vt[i - kWPasses] : vo_t, soff, lds);
  };
  // fragment rows of this lane: weight block ib, token block 0
  auto wrow_of = [&](int ib) {
    if (kGateUp)
      return (ib < WI / 2 ? 0 : BN / 2) + wn * (BN / 4) + (ib % (WI / 2)) * 32 + l32;
    return wn * (BN / 2) + ib * 32 + l32;
  };
  const int trow = BN + wm * (BM / 2) + l32;
  // Transposed weight fragments come from gfx950's transposing LDS read
  // (ds_read_b64_tr_b16): in each group of 16 lanes, lane i receives 16-bit
  // element i % 4 of the 8 bytes addressed by lanes 4 j + i / 4, j = 0..3.
  // Lanes 4 j + q of group g address K row 8 (g / 2) + j (+ 4 for the second
  // read) of the step and features 16 (g % 2) + 4 q .. + 3 of the half
  // block, so lane l receives feature l % 32 at K rows 8 (l / 32) .. + 7 of
  // the step: the MFMA operand of that feature. The swizzle repeats every 16
  // rows, so the per-lane offsets do not depend on the step.
  const int tgrp = lane >> 4, tgq = lane & 3;
  const int t_row = 8 * (tgrp >> 1) + ((lane >> 2) & 3);
  const int t_chunk = 2 * (tgrp & 1) + (tgq >> 1);
  const int t_lo = t_row * 64 + ((t_chunk ^ ((t_row >> 2) & 3)) << 4) + (tgq & 1) * 8;
  const int t_hi =
      (t_row + 4) * 64 + ((t_chunk ^ (((t_row + 4) >> 2) & 3)) << 4) + (tgq & 1) * 8;
  auto wfrag_t = [&](const char* stage, int hb, int s) {
    const char* blk = stage + hb * (kTileBytes / 2) + s * 16 * kRowBytes;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(lds_char*)(blk + t_lo));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(lds_char*)(blk + t_hi));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  frags_t f0, f1;
  // fragment r of step s of the stage at `stage`: weight blocks, then token
  // blocks
  auto read_one = [&](frags_t& f, const char* stage, int s, int r) {
    if (r < WI) {
      if constexpr (kTransW)  // half block of the wavefront's features
        f.a[r] = wfrag_t(stage, wn * (BN / 64) + r, s);
      else
        f.a[r] = MmaOp<Elem>::load(stage, wrow_of(r), s, half);
    } else {
      f.b[r - WI] = MmaOp<Elem>::load(stage, trow + 32 * (r - WI), s, half);
    }
  };

  // prologue of the workgroup's first tile: super-stages 0 .. 2 in flight;
  // wait for the first
  locate(tile, e, m, n0, m0);
  src_t cur = sources(e, m, n0, m0, true);
  // gathering: pa holds the assignments of the tile after the one being
  // computed, loaded one tile ahead of their use
  int32_t pa[kTPasses];
  if constexpr (kGather) {
    perm_rows(e, m, m0, true, pa);
    token_offs(pa, cur);
    const int t1 = tile + (int)gridDim.x;
    int e1 = 0, m1 = 0, n01 = 0, m01 = 0;
    if (t1 < total) locate(t1, e1, m1, n01, m01);
    perm_rows(e1, m1, m01, t1 < total, pa);
  }
  // row weights: w_pend holds the tile's (the top of the loop moves them to
  // w_cur), pw the next tile's assignments
  int32_t pw[WJ];
  float w_pend[WJ], w_cur[WJ];
  if constexpr (kRowWeight) {
    int32_t p0[WJ];
    epi_perm(e, m, m0, true, p0);
    epi_weight(p0, w_pend);
    const int t1 = tile + (int)gridDim.x;
    int e1 = 0, m1 = 0, n01 = 0, m01 = 0;
    if (t1 < total) locate(t1, e1, m1, n01, m01);
    epi_perm(e1, m1, m01, t1 < total, pw);
  }
  {
    const StageOff o0 = stage_off(0), o1 = stage_off(1), o2 = stage_off(2);
#pragma unroll
    for (int x = 0; x < kLoads; ++x) fetch_one(slot0, o0, cur, x);
#pragma unroll
    for (int x = 0; x < kLoads; ++x) fetch_one(slot1, o1, cur, x);
#pragma unroll
    for (int x = 0; x < kLoads; ++x) fetch_one(slot2, o2, cur, x);
  }
  wait_vmem_barrier<kWait>();
#pragma unroll
  for (int r = 0; r < kReadsPerStep; ++r) read_one(f0, slot0, 0, r);

  typedef Elem vec4_t __attribute__((ext_vector_type(4)));
  f32x16 acc[WI][WJ];
  while (true) {
    // the next tile of this workgroup, whose first super-stages the ring
    // fetches at the end of this one
    const int tile_n = tile + G;
    const bool has_next = tile_n < total;
    int e_n = 0, m_n = 0, n0_n = 0, m0_n = 0;
    if (has_next) locate(tile_n, e_n, m_n, n0_n, m0_n);
    src_t nxt = sources(e_n, m_n, n0_n, m0_n, has_next);
    if constexpr (kGather) {
      token_offs(pa, nxt);
      const int tile_nn = tile_n + G;
      int e2 = 0, m2 = 0, n02 = 0, m02 = 0;
      if (tile_nn < total) locate(tile_nn, e2, m2, n02, m02);
      perm_rows(e2, m2, m02, tile_nn < total, pa);
    }
    if constexpr (kRowWeight) {
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb) {
        w_cur[jb] = w_pend[jb];
        // in a register here, so the wait for its load is at this point
        asm volatile("" : "+v"(w_cur[jb]));
      }
      epi_weight(pw, w_pend);
      const int tile_nn = tile_n + G;
      int e2 = 0, m2 = 0, n02 = 0, m02 = 0;
      if (tile_nn < total) locate(tile_nn, e2, m2, n02, m02);
      epi_perm(e2, m2, m02, tile_nn < total, pw);
    }

#pragma unroll
    for (int ib = 0; ib < WI; ++ib)
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[ib][jb][v] = 0.f;

    // Super-stage ks in slot CUR (NXT holds ks + 1). Its MFMA steps also
    // fetch ring position ks + 3 into FSLOT (this tile's super-stage ks + 3
    // or, past the tile's end KS4, the next tile's), kLoadsPerStep loads a
    // step; the last step follows the barrier, which waits for ks + 1.
#define MOE_SUPER(CUR, NXT, FSLOT, KS_)                                          \
    {                                                                           \
      const StageOff SO = stage_off((KS_) + kSlots - 1 - fofs);                 \
      _Pragma("unroll") for (int sub = 0; sub < SPB; ++sub) {                   \
        const char* cs = CUR + sub * kStageBytes;                               \
        const char* ns = sub + 1 < SPB ? CUR + (sub + 1) * kStageBytes : NXT;   \
        _Pragma("unroll") for (int s = 0; s < kSteps; s += 2) {                 \
          const int ja = sub * kSteps + s; /* step index in the super-stage */  \
          const bool last = s + 2 >= kSteps && sub + 1 == SPB;                  \
          mma_step<Elem, WI, WJ, kReadsPerStep + kLoadsPerStep>(acc, f0, [&](int x) { \
            if (x < kReadsPerStep) {                                            \
              read_one(f1, cs, s + 1, x);                                       \
            } else {                                                            \
              const int li = ja * kLoadsPerStep + x - kReadsPerStep;            \
              if (li < kLoads) fetch_one(FSLOT, SO, F, li);                    \
            }                                                                   \
          });                                                                   \
          if (last) wait_vmem_barrier<kWait>();                                 \
          const char* rs_ = s + 2 < kSteps ? cs : ns;                           \
          const int rstep = s + 2 < kSteps ? s + 2 : 0;                         \
          mma_step<Elem, WI, WJ, kReadsPerStep + kLoadsPerStep>(acc, f1, [&](int x) { \
            if (x < kReadsPerStep) {                                            \
              read_one(f0, rs_, rstep, x);                                      \
            } else {                                                            \
              const int li = (ja + 1) * kLoadsPerStep + x - kReadsPerStep;      \
              if (li < kLoads) fetch_one(FSLOT, SO, F, li);                    \
            }                                                                   \
          });                                                                   \
        }                                                                       \
      }                                                                         \
    }

    // fetch source: this tile's until the ring reaches position KS4, then
    // the next tile's (from the second super-stage of the last pass on)
    src_t F = cur;
    int fofs = 0;
    for (int ks = 0; ks < KS4; ks += kSlots) {
      MOE_SUPER(slot0, slot1, slot3, ks)
      if (ks + kSlots == KS4) {
        F = nxt;
        fofs = KS4;
      }
      MOE_SUPER(slot1, slot2, slot0, ks + 1)
      MOE_SUPER(slot2, slot3, slot1, ks + 2)
      MOE_SUPER(slot3, slot0, slot2, ks + 3)
    }
#undef MOE_SUPER

    // Epilogue: lane holds, for token c (row l32 of each 32-token block),
    // four runs of four consecutive output features. Straight-line code:
    // outputs outside the tile's m rows or N features get an out-of-range
    // offset and the buffer unit drops the store, so there is no divergent
    // branch and every group of four is finished before the next starts.
    // (the accumulators are read by asm below: give the last MFMAs the wait
    // states a VALU read of their results needs, which the compiler cannot
    // see through the asm)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    typedef uint32_t st_t __attribute__((ext_vector_type(kEs == 2 ? 2 : 4)));
    auto store4 = [&](__amdgpu_buffer_rsrc_t rs, uint32_t off, vec4_t o) {
      if constexpr (kEs == 2)
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(st_t, o), rs, off, 0, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(st_t, o), rs, off, 0, 0);
    };
    if constexpr (kMode == kModeRecompute) {
      // gu (g in columns [0, N), u in [N, 2N)) and hw = w * silu(g) u: rows
      // c of expert e's tiled matrices of the round; w is the routing
      // weight of the row's assignment (w_cur, loaded ahead)
      const int rowb = __builtin_amdgcn_readlane(lane_row, e);
      const uint32_t mrows = (uint32_t)((m + 63) & ~63);
      const __amdgpu_buffer_rsrc_t rgu = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.out + (int64_t)rowb * 2 * p.N), 0,
          (int)(mrows * 2 * p.N * kEs), kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rhw = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.out2 + (int64_t)rowb * p.N), 0, (int)(mrows * p.N * kEs),
          kRsrcWord3);
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb) {
        const int c = m0 + wm * (BM / 2) + jb * 32 + l32;
        const float wc = w_cur[jb];
#pragma unroll
        for (int ib = 0; ib < WI / 2; ++ib) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int feat = n0 + wn * (BN / 4) + ib * 32 + 8 * g4 + 4 * half;
            vec4_t og, ou, oh;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float g = acc_read(acc[ib][jb][4 * g4 + q]);
              const float u = acc_read(acc[ib + WI / 2][jb][4 * g4 + q]);
              og[q] = from_f32<Elem>(g);
              ou[q] = from_f32<Elem>(u);
              oh[q] = from_f32<Elem>(wc * silu_mul(g, u));
            }
            const bool ok = c < m && feat < p.N;
            const int64_t rb2 = (int64_t)2 * p.N * kEs;
            store4(rgu, ok ? (uint32_t)tiled_offset(c, (int64_t)feat * kEs, rb2)
                           : kOutOfRange, og);
            store4(rgu, ok ? (uint32_t)tiled_offset(c, (int64_t)(p.N + feat) * kEs, rb2)
                           : kOutOfRange, ou);
            store4(rhw, ok ? (uint32_t)tiled_offset(c, (int64_t)feat * kEs,
                                                    (int64_t)p.N * kEs)
                           : kOutOfRange, oh);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else if constexpr (kMode == kModeDgate) {
      // dh = w * (dyr Wd) for row c and features feat..feat+3; with g, u of
      // the same row and features (from gu): du = dh silu(g), dg = dh u
      // silu'(g) = dh u s (1 + g (1 - s)), s = sigmoid(g); into dgu (dg in
      // columns [0, N), du in [N, 2N)), rows c of expert e's tiled matrix
      const int rowb = __builtin_amdgcn_readlane(lane_row, e);
      const uint32_t range =
          (uint32_t)((m + 63) & ~63) * 2 * (uint32_t)p.N * kEs;
      const __amdgpu_buffer_rsrc_t rin = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.aux + (int64_t)rowb * 2 * p.N), 0, (int)range, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rout = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.out + (int64_t)rowb * 2 * p.N), 0, (int)range, kRsrcWord3);
      const int64_t rb2 = (int64_t)2 * p.N * kEs;
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb) {
        const int c = m0 + wm * (BM / 2) + jb * 32 + l32;
        const float wc = w_cur[jb];  // routing weight (loaded ahead)
        // this token's g and u for every output of the block, loaded first
        u32x2 gv[WI][4], uv[WI][4];
#pragma unroll
        for (int ib = 0; ib < WI; ++ib) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int feat = n0 + wn * (BN / 2) + ib * 32 + 8 * g4 + 4 * half;
            const bool ok = c < m && feat < p.N;
            gv[ib][g4] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                rin, ok ? (uint32_t)tiled_offset(c, (int64_t)feat * kEs, rb2) : kOutOfRange,
                0, 0));
            uv[ib][g4] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                rin, ok ? (uint32_t)tiled_offset(c, (int64_t)(p.N + feat) * kEs, rb2)
                        : kOutOfRange,
                0, 0));
          }
        }
#pragma unroll
        for (int ib = 0; ib < WI; ++ib) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int feat = n0 + wn * (BN / 2) + ib * 32 + 8 * g4 + 4 * half;
            const vec4_t gq = __builtin_bit_cast(vec4_t, gv[ib][g4]);
            const vec4_t uq = __builtin_bit_cast(vec4_t, uv[ib][g4]);
            vec4_t odg, odu;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float dh = wc * acc_read(acc[ib][jb][4 * g4 + q]);
              const float g = to_f32(gq[q]), u = to_f32(uq[q]);
              const float sg = __builtin_amdgcn_rcpf(
                  1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
              odu[q] = from_f32<Elem>(dh * (g * sg));
              odg[q] = from_f32<Elem>(dh * u * sg * (1.0f + g * (1.0f - sg)));
            }
            const bool ok = c < m && feat < p.N;
            store4(rout, ok ? (uint32_t)tiled_offset(c, (int64_t)feat * kEs, rb2)
                            : kOutOfRange, odg);
            store4(rout, ok ? (uint32_t)tiled_offset(c, (int64_t)(p.N + feat) * kEs, rb2)
                            : kOutOfRange, odu);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else if constexpr (kMode == kModeGateUp && kEs == 2) {
      // h: expert e's tiled matrix of the round. A 32-token x 32-feature
      // block of the accumulators is one contiguous 2 KiB half of a 4 KiB
      // tiled block (rows c0 % 64 .. + 31 of the band, 64 bytes each), but
      // the lane layout spreads it over 32 rows, 8 bytes a store. Each
      // wavefront writes the block into 2 KiB of its 4 KiB share of slot3
      // (free as in the z epilogue below) in the tiled order, swizzle
      // included, and copies it out as two whole 1 KiB stores. Rows past m
      // (up to the 64-row padding the descriptor covers) receive values
      // computed from the padding rows of the operand; no kernel reads them
      // for a stored output.
      const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.out + (int64_t)__builtin_amdgcn_readlane(lane_row, e) * p.N), 0,
          (int)((uint32_t)((m + 63) & ~63) * p.N * kEs), kRsrcWord3);
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      char* const stg0 = slot3 + wave_id * 4096;
      const int put_off = l32 * 64 + half * 8;  // this lane's row of the block
      const int put_swz = (l32 >> 2) & 3;
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb) {
        const int c0 = m0 + wm * (BM / 2) + jb * 32;
#pragma unroll
        for (int ib = 0; ib < WI / 2; ++ib) {
          const int f0 = n0 + wn * (BN / 4) + ib * 32;
          char* stg = stg0 + ((jb * (WI / 2) + ib) & 1) * 2048;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            vec4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              o[q] = from_f32<Elem>(silu_mul(acc_read(acc[ib][jb][4 * g4 + q]),
                                             acc_read(acc[ib + WI / 2][jb][4 * g4 + q])));
            *reinterpret_cast<u32x2*>(stg + put_off + ((g4 ^ put_swz) << 4)) =
                __builtin_bit_cast(u32x2, o);
          }
          const uint32_t off =
              f0 < p.N ? (uint32_t)tiled_offset(c0, (int64_t)f0 * kEs, (int64_t)p.N * kEs)
                       : kOutOfRange;
#pragma unroll
          for (int hk = 0; hk < 2; ++hk)
            __builtin_amdgcn_raw_buffer_store_b128(
                *reinterpret_cast<const u32x4*>(stg + hk * 1024 + lane * 16), rh,
                off + (uint32_t)(hk * 1024 + lane * 16), 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // every wavefront's staging reads are done before the next tile's ring
      // writes slot3
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else if constexpr (kMode == kModeGateUp) {
      // h (fp32): row c, four features per 16-byte store
      const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.out + (int64_t)__builtin_amdgcn_readlane(lane_row, e) * p.N), 0,
          (int)((uint32_t)((m + 63) & ~63) * p.N * kEs), kRsrcWord3);
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb) {
        const int c = m0 + wm * (BM / 2) + jb * 32 + l32;
#pragma unroll
        for (int ib = 0; ib < WI / 2; ++ib) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int feat = n0 + wn * (BN / 4) + ib * 32 + 8 * g4 + 4 * half;
            vec4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
              o[q] = from_f32<Elem>(silu_mul(acc_read(acc[ib][jb][4 * g4 + q]),
                                             acc_read(acc[ib + WI / 2][jb][4 * g4 + q])));
            const uint32_t off =
                c < m && feat < p.N
                    ? (uint32_t)tiled_offset(c, (int64_t)feat * kEs, (int64_t)p.N * kEs)
                    : kOutOfRange;
            store4(rh, off, o);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    } else if constexpr (kEs == 2) {
      // z: rows i0 + c (c < m) of the expert-sorted order, i0 = offsets[e]
      // + the index of e's first entry of the round: the slot of assignment
      // perm[i0 + c]. z rows are long (N features), so the lane layout of
      // the accumulators (one token per lane, 8 bytes of it per store) would
      // touch 32 rows per store; instead each wavefront turns a block of 32
      // tokens x 64 features around in LDS and stores whole 128-byte row
      // pieces, 8 rows per store. The staging area is slot3, which the last
      // super-stage has consumed (every wavefront passed the barrier after
      // its last read of it) and which the next tile's ring first fills in
      // its super-stage 0, after the barrier below.
      const int64_t i0 = (int64_t)__builtin_amdgcn_readlane(lane_off, e);
      const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.out + i0 * p.N), 0, (int)((uint32_t)m * p.N * kEs), kRsrcWord3);
      // 32 rows of 128 bytes per wavefront; 16-byte chunk q of row r sits at
      // chunk q ^ (r % 8), so that neither the writes (32 rows, one chunk
      // each) nor the reads (8 rows, all chunks) pile onto a few banks
      char* stg = slot3 + wave_id * 4096;
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const int rrow = lane >> 3, rchunk = lane & 7;  // read-back position
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb) {
        const int cb = m0 + wm * (BM / 2) + jb * 32;  // first token of the block
#pragma unroll
        for (int ip = 0; ip < WI / 2; ++ip) {
          // lane (l32, half) holds token l32's features 32 u + 8 g4 + 4 half
          // + q of the 64, q < 4
#pragma unroll
          for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              vec4_t o;
#pragma unroll
              for (int q = 0; q < 4; ++q)
                o[q] = from_f32<Elem>(acc_read(acc[2 * ip + u][jb][4 * g4 + q]));
              const int chunk = (u * 4 + g4) ^ (l32 & 7);
              *reinterpret_cast<u32x2*>(stg + l32 * 128 + chunk * 16 + half * 8) =
                  __builtin_bit_cast(u32x2, o);
            }
          }
          const int feat = n0 + wn * (BN / 2) + ip * 64 + rchunk * 8;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = i * 8 + rrow;
            const u32x4 v = *reinterpret_cast<const u32x4*>(
                stg + r * 128 + ((rchunk ^ (r & 7)) * 16));
            // rows c >= m fall past the descriptor's range
            const uint32_t off =
                feat < p.N ? ((uint32_t)(cb + r) * p.N + feat) * kEs : kOutOfRange;
            // non-temporal: z is next read by the combine, after every
            // round, so its lines should not displace the operands that
            // the following tiles fetch through L2
            __builtin_amdgcn_raw_buffer_store_b128(v, rz, off, 0, kNonTemporal);
          }
        }
      }
      // every wavefront's staging reads are done before the next tile's ring
      // writes slot3
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      // z (fp32): as above, straight from the accumulator layout
      const int64_t i0 = (int64_t)__builtin_amdgcn_readlane(lane_off, e);
      const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(p.out + i0 * p.N), 0, (int)((uint32_t)m * p.N * kEs), kRsrcWord3);
#pragma unroll
      for (int jb = 0; jb < WJ; ++jb) {
        const int c = m0 + wm * (BM / 2) + jb * 32 + l32;
#pragma unroll
        for (int ib = 0; ib < WI; ++ib) {
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int feat = n0 + wn * (BN / 2) + ib * 32 + 8 * g4 + 4 * half;
            vec4_t o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = from_f32<Elem>(acc_read(acc[ib][jb][4 * g4 + q]));
            // rows c >= m fall past the descriptor's range
            const uint32_t off = feat < p.N ? ((uint32_t)c * p.N + feat) * kEs : kOutOfRange;
            store4(rz, off, o);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    if (!has_next) break;
    // the next tile's first fragments (its super-stage 0 is in slot0, ring
    // position KS4): read here rather than in the last MFMA step, so that
    // they do not occupy registers during the epilogue
#pragma unroll
    for (int r = 0; r < kReadsPerStep; ++r) read_one(f0, slot0, 0, r);
    tile = tile_n;
    e = e_n;
    m = m_n;
    n0 = n0_n;
    m0 = m0_n;
    cur = nxt;
  }
  // the fetches that ran past the last tile read nothing, but they still
  // write LDS: let them land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Tiles one round needs under configuration Cfg (host side, from the rows
// of every expert in the round).
template <typename Cfg>
static int64_t round_tiles(const int32_t* rows, int nv, int N, bool gate_up) {
  const int BM = 64 * Cfg::WJ;
  const int NF = gate_up ? 32 * Cfg::WI : 64 * Cfg::WI;
  const int64_t nt = (N + NF - 1) / NF;
  int64_t tiles = 0;
  for (int v = 0; v < nv; ++v) tiles += ((int64_t)rows[v] + BM - 1) / BM * nt;
  return tiles;
}

// Estimated time of a round in a tile shape: waves of tiles over the CUs
// times the tile's area over its relative MFMA efficiency.
template <typename Cfg>
static float est_cost(int64_t tiles, int num_cus) {
  const int64_t waves = (tiles + num_cus - 1) / num_cus;
  return (float)waves * (64.0f * Cfg::WI) * (64.0f * Cfg::WJ) / Cfg::kEff;
}

// Workgroups for a round: one per CU, or fewer when the round has fewer
// tiles; a multiple of 8 (the XCD-contiguous walk assumes it).
static int grid_for(int64_t tiles, int num_cus) {
  int64_t g = tiles < num_cus ? tiles : num_cus;
  g = (g + 7) / 8 * 8;
  return (int)(g < 8 ? 8 : g);
}

template <typename Elem, typename Cfg, int kMode, bool kGather>
static hipError_t launch_gemm_cfg(const GemmParams<Elem>& p, int grid,
                                  hipStream_t st) {
  hipLaunchKernelGGL(
      (grouped_ffn_gemm_kernel<Elem, Cfg::WI, Cfg::WJ, Cfg::SPB, kMode, kGather>),
      dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

// rows_host (nullable): rows of the launch's nv pairs, on the host. With
// them the launch's tile shape and grid are chosen from its tile counts;
// without them the large tile and one workgroup per CU are used. Every shape
// runs the same MFMA sequence over K for every output, so results are
// identical. p.N is the number of output features.
template <typename Elem, int kMode, bool kGather = false>
static hipError_t launch_gemm(const Shape& s, const GemmParams<Elem>& p,
                              const int32_t* rows_host, int nv, int num_cus,
                              hipStream_t st) {
  constexpr bool kDual = kMode == kModeGateUp || kMode == kModeRecompute;
  const int N = p.N;
  (void)s;
  if (rows_host) {
    int64_t mmax = 0;
    for (int v = 0; v < nv; ++v) mmax = rows_host[v] > mmax ? rows_host[v] : mmax;
    if (mmax == 0) return hipSuccess;  // nothing in this launch
    const int64_t tb = round_tiles<TileBig>(rows_host, nv, N, kDual);
    const int64_t tm = round_tiles<TileMedium>(rows_host, nv, N, kDual);
    const int64_t ts = round_tiles<TileSmall>(rows_host, nv, N, kDual);
    const float cb = est_cost<TileBig>(tb, num_cus);
    const float cm = est_cost<TileMedium>(tm, num_cus);
    const float cs = est_cost<TileSmall>(ts, num_cus);
    if (cb <= cm && cb <= cs)
      return launch_gemm_cfg<Elem, TileBig, kMode, kGather>(p, grid_for(tb, num_cus), st);
    if (cm <= cs)
      return launch_gemm_cfg<Elem, TileMedium, kMode, kGather>(p, grid_for(tm, num_cus),
                                                               st);
    return launch_gemm_cfg<Elem, TileSmall, kMode, kGather>(p, grid_for(ts, num_cus), st);
  }
  return launch_gemm_cfg<Elem, TileBig, kMode, kGather>(p, grid_for(num_cus, num_cus), st);
}

// Parameters of a launch over round r: activations act [rows][K], weights
// w0 (and w1) [E][N][K], output out; K and N as given.
template <typename Elem>
static GemmParams<Elem> params(const Shape& s, int r0, int nr, const void* act,
                               const void* w0, const void* w1, void* out,
                               const PlanBuffers& b, int K, int N, bool tiled_w) {
  GemmParams<Elem> p{};
  p.act = static_cast<const Elem*>(act);
  p.w0 = static_cast<const Elem*>(w0);
  p.w1 = static_cast<const Elem*>(w1);
  p.out = static_cast<Elem*>(out);
  p.weight = b.weight;
  p.perm = b.perm;
  p.rounds = b.rounds;
  p.n_rounds = b.n_rounds;
  p.E = s.E;
  p.r0 = r0;
  p.nr = nr;
  p.K = K;
  p.N = N;
  p.max_rounds = (int)s.max_rounds();
  p.tiled_w = tiled_w ? 1 : 0;
  return p;
}

bool gather_fits(const Shape& s) {
  return s.T * s.d * (s.bf16 ? 2 : 4) <= ((int64_t)1 << 30);
}

template <typename Elem>
static hipError_t gate_up(const Shape& s, int r0, int nr, const void* xr,
                          const void* x, const void* wg, const void* wu,
                          const PlanBuffers& b, const int32_t* rows_host, int nv,
                          void* h, int num_cus, hipStream_t st) {
  GemmParams<Elem> p = params<Elem>(s, r0, nr, xr, wg, wu, h, b, s.d, s.f, s.tiled_w);
  if (!x) return launch_gemm<Elem, kModeGateUp>(s, p, rows_host, nv, num_cus, st);
  if (!gather_fits(s)) return hipErrorInvalidValue;
  p.x = static_cast<const Elem*>(x);
  p.x_bytes = (int)(s.T * s.d * (int64_t)sizeof(Elem));
  p.topk = s.k;
  return launch_gemm<Elem, kModeGateUp, true>(s, p, rows_host, nv, num_cus, st);
}

hipError_t launch_gate_up(const Shape& s, int r0, int nr, const void* xr,
                          const void* wg, const void* wu, const PlanBuffers& b,
                          const int32_t* rows_host, int nv, void* h, int num_cus,
                          hipStream_t st, const void* x) {
  if (s.bf16) return gate_up<bf16>(s, r0, nr, xr, x, wg, wu, b, rows_host, nv, h, num_cus, st);
  return gate_up<float>(s, r0, nr, xr, x, wg, wu, b, rows_host, nv, h, num_cus, st);
}

hipError_t launch_down(const Shape& s, int r0, int nr, const void* h, const void* wd,
                       const PlanBuffers& b, const int32_t* rows_host, int nv,
                       void* z, int num_cus, hipStream_t st) {
  if (s.bf16)
    return launch_gemm<bf16, kModeDown>(
        s, params<bf16>(s, r0, nr, h, wd, nullptr, z, b, s.f, s.d, s.tiled_w),
        rows_host, nv, num_cus, st);
  return launch_gemm<float, kModeDown>(
      s, params<float>(s, r0, nr, h, wd, nullptr, z, b, s.f, s.d, s.tiled_w),
      rows_host, nv, num_cus, st);
}

hipError_t launch_recompute(const Shape& s, int r, const void* xr, const void* wg,
                            const void* wu, const PlanBuffers& b,
                            const int32_t* rows_host, int nv, void* gu, void* hw,
                            int num_cus, hipStream_t st) {
  GemmParams<bf16> p = params<bf16>(s, r, 1, xr, wg, wu, gu, b, s.d, s.f, s.tiled_w);
  p.out2 = static_cast<bf16*>(hw);
  return launch_gemm<bf16, kModeRecompute>(s, p, rows_host, nv, num_cus, st);
}

hipError_t launch_dgate(const Shape& s, int r, const void* dyr, const void* wd,
                        const PlanBuffers& b, const int32_t* rows_host, int nv,
                        const void* gu, void* dgu, int num_cus, hipStream_t st) {
  GemmParams<bf16> p =
      params<bf16>(s, r, 1, dyr, wd, nullptr, dgu, b, s.d, s.f, s.tiled_w);
  p.aux = static_cast<const bf16*>(gu);
  return launch_gemm<bf16, kModeDgate>(s, p, rows_host, nv, num_cus, st);
}

hipError_t launch_dx(const Shape& s, int r, const void* dgu, const void* wg,
                     const void* wu, const PlanBuffers& b, const int32_t* rows_host,
                     int nv, void* dz, int num_cus, hipStream_t st) {
  return launch_gemm<bf16, kModeDx>(
      s, params<bf16>(s, r, 1, dgu, wg, wu, dz, b, 2 * s.f, s.d, s.tiled_w),
      rows_host, nv, num_cus, st);
}

}  // namespace moe
