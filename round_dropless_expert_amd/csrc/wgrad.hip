// Weight gradients of the expert FFN for one round of the backward (the
// backward of "Frontier Pre-training at Microsoft AI (MAI-Base-2)",
// section "Key claims": grouped expert compute per round; here its
// gradient with respect to the expert weights).
//
// For every expert e with rows in round r (or in rounds r and r + 1, whose
// buffers are the two sets of the backward's round buffers), out_e[a][b]
// (+)= sum over the expert's rows c of those rounds of U[c][a] * V[c][b],
// where U (A features) and V (B features) are token-major round buffers in
// the tiled layout, expert e's matrix of round r starting at buffer row
// (e / G) * Q + pbase(r, e). Rows a < A0 go to out0[e][a][b], the others to
// out1[e][a - A0][b] (dW_gate and dW_up from one dgu buffer). out is fp32,
// row-major; the launch that covers round 0 stores, later ones add (the
// contraction over an expert's rows is then split at every second round
// boundary).
//
// The contraction runs over tokens, which are rows of both operands, while
// the matrix cores want each lane to hold consecutive K (token) values of
// one feature. Stages of 32 tokens are copied into LDS as they lie in the
// tiled round buffers (halves of 4 KiB blocks: 32 tokens x 32 features,
// 64-byte rows with the block's XOR swizzle) by LDS-direct loads, and the
// fragments are read back with gfx950's transposing LDS read
// (ds_read_b64_tr_b16): in each group of 16 lanes, lane i receives 16-bit
// element i % 4 of the 8 bytes addressed by lanes 4 j + i / 4, j = 0..3
// (checked on the device). Lanes 4 j + p of a group address tokens t0 + j,
// features c0 + 4 p .. + 3, so lane i gets feature c0 + i at tokens t0 ..
// t0 + 3: two such reads make one 8-token fragment, and the four rows a
// group touches cover different banks. A workgroup computes a 256 (a) x
// 256 (b) tile with 2 x 2 wavefronts of 128 x 128 (4 x 4 blocks of
// v_mfma_f32_32x32x16_bf16, 256 accumulators). The MFMA's row operand is
// the a fragment and its column operand the b fragment, so the 32 lanes of
// a half wavefront hold 32 consecutive b of one a: each fp32 store writes
// two whole 128-byte row pieces (row-major out), rather than 32-byte
// pieces of 32 rows. Four LDS slots form a ring with three stages in
// flight; the kernel waits on its own loads with exact vmcnt counts, as the
// grouped GEMM does. The fragments of one K step are read while the
// previous step's MFMAs run (two register sets), interleaved with the
// MFMAs at fixed points. The launch is persistent (below).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kTile = 256;        // a and b extent of a tile
constexpr int kStageTok = 32;     // tokens per stage
constexpr int kHalfBlock = 2048;  // 32 tokens x 64 bytes
constexpr int kOpBytes = 8 * kHalfBlock;   // 256 features of one operand
constexpr int kSlotBytes = 2 * kOpBytes;   // U then V
constexpr int kSlots = 4;
constexpr int kLoads = kSlotBytes / (256 * 16);  // 16-byte loads per thread per stage
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int kRsrcWord3 = 0x00020000;

typedef __attribute__((address_space(3))) char lds_char;

// Buffer-to-LDS loads (LDS-direct) of two 1 KiB pieces: lane i reads 16
// bytes at v0 + soff of the buffer into LDS at m0 + 16 i, and 16 bytes at
// v1 + soff + 1024 into LDS at m0 + 1024 + 16 i (the immediate offset
// advances both addresses). Asm, so that the compiler neither moves nor
// waits on them: every wait on these loads is the kernel's own, exact vmcnt
// count. M0 is declared clobbered (the compiler restores it where it needs
// it); one wait state separates its write from the loads.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load_pair(__amdgpu_buffer_rsrc_t rsrc, uint32_t v0,
                                              uint32_t v1, uint32_t soff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %3, %4 offen lds\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen offset:1024 lds"
      :
      : "s"(lds), "v"(v0), "v"(v1), "s"(rsrc), "s"(soff)
      : "m0");
}
#pragma clang diagnostic pop

// At most N of this wavefront's vector-memory operations outstanding, its
// LDS reads done, then the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_vmem_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// An accumulator element, read from its AGPR at this point of the program
// (asm: the epilogue then moves four values at a time into VGPRs instead of
// the compiler copying all 256 accumulators out at once).
__device__ __forceinline__ float acc_get(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct WgradParams {
  const bf16* U;   // round r's buffer, A features per row (tiled)
  const bf16* V;   // round r's buffer, B features per row (tiled)
  const bf16* U1;  // round r + 1's buffers (second set; used when nr == 2)
  const bf16* V1;
  float* out0;     // [E][A0][B]
  float* out1;     // [E][A - A0][B] (NULL when A0 == A)
  const int32_t* rounds;
  const int32_t* n_rounds;
  int E, r, A, A0, B, max_rounds;
  int nr;           // rounds contracted by this launch: r, or r and r + 1
  int tiles;        // tiles of the launch
  int all_experts;  // tiles of every expert (round 0: experts without rows get zeros)
  int accumulate;   // add to out (else store)
};

// Persistent: each workgroup walks a list of tiles. XCD x (workgroups b
// with b % 8 == x) takes the tiles [x n8, (x + 1) n8), n8 = ceil(tiles / 8),
// and its Q workgroups take every Q-th of them, so that at any time an
// XCD's workgroups work on consecutive tiles of one expert, which share its
// operand panels in that XCD's L2. The LDS ring runs on across the tiles of
// a workgroup: the fetches three stages ahead of the MFMAs reach into the
// next tile, whose first stages then land while the current tile's
// epilogue stores its results.
__global__ __launch_bounds__(256, 1) void wgrad_kernel(WgradParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[kSlots][kSlotBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wa = wave & 1, wb = wave >> 1;  // this wavefront's 128 x 128 quarter
  const int l32 = lane & 31, half = lane >> 5;
  const int R = *p.n_rounds;
  if (p.r >= R) return;
  const bool two = p.nr == 2 && p.r + 1 < R;

  const int Q = (int)gridDim.x / 8;
  const int xcd = (int)(blockIdx.x % 8), q = (int)(blockIdx.x / 8);
  const int n8 = (p.tiles + 7) / 8;
  const int t_first = xcd * n8 + q;
  const int t_end = (xcd + 1) * n8 < p.tiles ? (xcd + 1) * n8 : p.tiles;
  if (t_first >= t_end) return;

  // The launch's expert table, in every wavefront's registers: lane e < E
  // holds expert e's rows in round r (segment 0) and r + 1 (segment 1, the
  // second buffer set) and the first buffer row of each of its matrices;
  // lrank: the number of experts with rows below lane e.
  const int64_t tbl = (int64_t)p.max_rounds * p.E;
  const bool le = lane < p.E;
  const int64_t at = (int64_t)p.r * p.E + lane;
  const int lm0 = le ? p.rounds[kAlloc * tbl + at] : 0;
  const int lm1 = le && two ? p.rounds[kAlloc * tbl + at + p.E] : 0;
  const int lrow0 = le ? p.rounds[kBrow * tbl + at] : 0;
  const int lrow1 = le && two ? p.rounds[kBrow * tbl + at + p.E] : 0;
  const bool lact = lm0 > 0 || lm1 > 0;
  const int lrank =
      __builtin_popcountll(__builtin_amdgcn_ballot_w64(lact) & ((1ull << lane) - 1));

  // tile t -> expert (expert-major: ta x tb tiles each; without all_experts,
  // the (t / per)-th expert with rows) and its a, b origin
  const int ta = (p.A + kTile - 1) / kTile, tb = (p.B + kTile - 1) / kTile;
  const int per = ta * tb;
  struct Tile {
    int e, a0, b0, m0, m1, stages;
    int64_t row0, row1;
  };
  auto tile_at = [&](int t) {
    Tile T;
    const int slot = t / per, local = t % per;
    T.e = p.all_experts ? slot
                        : (int)__builtin_ctzll(
                              __builtin_amdgcn_ballot_w64(lact && lrank == slot));
    T.m0 = __builtin_amdgcn_readlane(lm0, T.e);
    T.m1 = __builtin_amdgcn_readlane(lm1, T.e);
    T.row0 = __builtin_amdgcn_readlane(lrow0, T.e);
    T.row1 = __builtin_amdgcn_readlane(lrow1, T.e);
    T.a0 = (local / tb) * kTile;
    T.b0 = (local % tb) * kTile;
    T.stages = (T.m0 + kStageTok - 1) / kStageTok + (T.m1 + kStageTok - 1) / kStageTok;
    return T;
  };

  // Loads of a stage: wavefronts 0-1 fetch U, 2-3 fetch V. A wavefront
  // moves four 32-feature half blocks h = 0..3 (features fbase + 32 h of
  // the operand, LDS half block 4 (wave % 2) + h), each as two 1 KiB parts:
  // lane i moves 16 bytes, of token k0 + 16 part + i / 4 of the stage's
  // segment (zeros past its m, and past A or B). One M0 value serves both
  // parts of a half block, whose LDS and buffer addresses both advance by
  // the load's 1 KiB immediate offset. A tile's stages are segment 0's,
  // then segment 1's.
  const int op = wave >> 1;
  const uint32_t rb = op == 0 ? (uint32_t)p.A * 2 : (uint32_t)p.B * 2;  // row bytes
  const int flim = op == 0 ? p.A : p.B;
  const bf16* src0 = op == 0 ? p.U : p.V;
  const bf16* src1 = two ? (op == 0 ? p.U1 : p.V1) : src0;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)&lds[0][0];
  const uint32_t dst0 = lds0 + (uint32_t)(op * kOpBytes + 4 * (wave & 1) * kHalfBlock);
  // what this wavefront fetches of a tile: its operand's two segments and,
  // per half block, this lane's offset inside a stage's 64-row band (out of
  // range for feature blocks at or past A or B: the range check then
  // zero-fills whatever the stage's offset is)
  struct FetchTile {
    __amdgpu_buffer_rsrc_t rs0, rs1;
    int S0, stages, m0, m1;
    uint32_t vh[4];
  };
  auto fetch_tile = [&](const Tile& T) {
    FetchTile F;
    const int64_t row = (int64_t)(rb / 2);  // elements per buffer row
    F.rs0 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src0 + T.row0 * row), 0, (int)((uint32_t)((T.m0 + 63) & ~63) * rb), kRsrcWord3);
    F.rs1 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(src1 + T.row1 * row), 0, (int)((uint32_t)((T.m1 + 63) & ~63) * rb), kRsrcWord3);
    F.S0 = (T.m0 + kStageTok - 1) / kStageTok;
    F.stages = T.stages;
    F.m0 = T.m0;
    F.m1 = T.m1;
    const int fbase = (op == 0 ? T.a0 : T.b0) + 128 * (wave & 1);
#pragma unroll
    for (int h = 0; h < 4; ++h)
      F.vh[h] = fbase + 32 * h < flim
                    ? (uint32_t)((fbase >> 5) + h) * 4096u + (uint32_t)lane * 16u
                    : kOutOfRange;
    return F;
  };
  // Per stage: the segment's descriptor, the stage's band offset and, per
  // half block and part, this lane's offset (out of range for tokens past
  // the segment's m, and for every stage past the workgroup's last tile).
  struct StageLd {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t koff;
    uint32_t vo[4][2];
  };
  auto stage_ld = [&](const FetchTile& F, int s, bool valid) {
    StageLd L;
    const bool seg1 = s >= F.S0;
    const int k0 = (seg1 ? s - F.S0 : s) * kStageTok;
    const int m = valid ? (seg1 ? F.m1 : F.m0) : 0;
    L.rs = seg1 ? F.rs1 : F.rs0;
    L.koff = (uint32_t)(k0 >> 6) * (rb >> 6) * 4096u + (uint32_t)((k0 >> 5) & 1) * kHalfBlock;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const bool in = k0 + part * 16 + (lane >> 2) < m;
#pragma unroll
      for (int h = 0; h < 4; ++h) L.vo[h][part] = in ? F.vh[h] : kOutOfRange;
    }
    return L;
  };
  // half block h of a stage into ring slot `slot`
  auto fetch = [&](const StageLd& L, int slot, int h) {
    lds_load_pair(L.rs, L.vo[h][0], L.vo[h][1], L.koff,
                  dst0 + (uint32_t)(slot * kSlotBytes + h * kHalfBlock));
  };
  // The fetch cursor: tile ft of the workgroup's list, its stage fs. Each
  // call hands out the next stage of the workgroup's sequence (tiles without
  // rows have no stages and are passed over); past the last tile, stages
  // that load nothing, so that every stage issues the same loads.
  int ft = t_first, fs = 0;
  FetchTile F = fetch_tile(tile_at(ft));
  auto next_stage = [&]() {
    while (ft < t_end && fs >= F.stages) {
      ft += Q;
      fs = 0;
      if (ft < t_end) F = fetch_tile(tile_at(ft));
    }
    const StageLd L = stage_ld(F, fs, ft < t_end);
    ++fs;
    return L;
  };

  // this lane's part of a transposed read: group g = lane / 16, position
  // 4 j + q in it -> token 8 (g / 2) + j (+ 4 for the second read) and
  // features 16 (g % 2) + 4 q of a 32-feature block: 16-byte chunk
  // 2 (g % 2) + q / 2, 8-byte half q % 2, swizzled by the row (the swizzle
  // repeats every 16 rows, so it does not depend on the K step)
  const int grp = lane >> 4, gj = (lane >> 2) & 3, gq = lane & 3;
  const int tr_row = 8 * (grp >> 1) + gj;
  const int tr_chunk = 2 * (grp & 1) + (gq >> 1);
  const int tr_half = (gq & 1) * 8;
  const int tr_lo = tr_row * 64 + ((tr_chunk ^ ((tr_row >> 2) & 3)) << 4) + tr_half;
  const int tr_hi = (tr_row + 4) * 64 + ((tr_chunk ^ (((tr_row + 4) >> 2) & 3)) << 4) + tr_half;
  const lds_char* ldsb = (const lds_char*)&lds[0][0];
  const lds_char* base_a = ldsb + wa * 4 * kHalfBlock;
  const lds_char* base_b = ldsb + kOpBytes + wb * 4 * kHalfBlock;
  // fragment of operand o (0: a, 1: b), this wavefront's 32-feature block
  // blk (0..3), K step ks of the stage in ring slot `slot`
  auto frag = [&](int o, int slot, int blk, int ks) {
    const lds_char* b = (o == 0 ? base_a : base_b) + slot * kSlotBytes + blk * kHalfBlock +
                        ks * 1024;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + tr_lo));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + tr_hi));
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 acc[4][4];  // [b block][a block]: rows a, columns b
  auto zero_acc = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  };

  // the fragments of one K step (16 tokens): b blocks, then a blocks
  bf16x8 fb0[4], fa0[4], fb1[4], fa1[4];
  // fragment x of a K step, in the order the MFMAs first use them: b
  // block 0, a blocks 0 .. 3, b blocks 1 .. 3
  auto read_one = [&](bf16x8 (&fb)[4], bf16x8 (&fa)[4], int slot, int ks, int x) {
    if (x == 0)
      fb[0] = frag(1, slot, 0, ks);
    else if (x <= 4)
      fa[x - 1] = frag(0, slot, x - 1, ks);
    else
      fb[x - 4] = frag(1, slot, x - 4, ks);
  };
  // One K step's 16 MFMAs with kOps other operations spread over them in a
  // fixed order (op(x) after MFMA i for x in [i kOps / 16, (i + 1) kOps /
  // 16)), each group fenced so that the compiler keeps the order.
  constexpr int kOps = 10;  // 8 fragment reads, 2 half-block fetches
  auto mma_step = [&](const bf16x8 (&fb)[4], const bf16x8 (&fa)[4], auto op) {
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int i = n / 4, j = n % 4;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[j], fb[i], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int x = n * kOps / 16; x < (n + 1) * kOps / 16; ++x) op(x);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Epilogue of tile T. lane: b = column l32 of the block, a = rows
  // 8 (v / 4) + 4 half + v % 4 for its values v: every store writes two
  // 128-byte row pieces. (The accumulators are read by asm: give the last
  // MFMAs the wait states a VALU read of their results needs, which the
  // compiler cannot see.)
  const uint32_t rowb = (uint32_t)p.B * 4u;
  auto epilogue = [&](const Tile& T) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ab = T.a0 + wa * 128 + j * 32;
      if (ab >= p.A) continue;
      float* base = ab < p.A0 ? p.out0 + ((int64_t)T.e * p.A0 + ab) * p.B
                              : p.out1 + ((int64_t)T.e * (p.A - p.A0) + (ab - p.A0)) * p.B;
      const __amdgpu_buffer_rsrc_t ro =
          __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)(32u * rowb), kRsrcWord3);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int bb = T.b0 + wb * 128 + i * 32;
        if (bb >= p.B) continue;
        const uint32_t vo = (uint32_t)(4 * half) * rowb + (uint32_t)(bb + l32) * 4u;
        auto so = [&](int v) { return (int)((uint32_t)(8 * (v / 4) + v % 4) * rowb); };
        if (p.accumulate) {  // later launches: add to the stored sums
          float o[16];
#pragma unroll
          for (int v = 0; v < 16; ++v)
            o[v] = __builtin_bit_cast(float,
                                      __builtin_amdgcn_raw_buffer_load_b32(ro, (int)vo, so(v), 0));
#pragma unroll
          for (int v = 0; v < 16; ++v)
            __builtin_amdgcn_raw_buffer_store_b32(
                __builtin_bit_cast(uint32_t, acc_get(acc[i][j][v]) + o[v]), ro, (int)vo, so(v), 0);
        } else {
#pragma unroll
          for (int v = 0; v < 16; ++v)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc_get(acc[i][j][v])),
                                                  ro, (int)vo, so(v), 0);
        }
      }
    }
  };

  // prologue: the first three stages of the sequence in flight, wait for
  // the first, read its first step
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const StageLd L = next_stage();
#pragma unroll
    for (int h = 0; h < 4; ++h) fetch(L, st, h);
  }
  wait_vmem_barrier<2 * kLoads>();
#pragma unroll
  for (int x = 0; x < 8; ++x) read_one(fb0, fa0, 0, 0, x);

  // Tiles of the workgroup in order; g counts its stages (ring slot g % 4).
  // A tile without rows (an expert without rows in a launch over every
  // expert) has no stages and is stored as zeros.
  //
  // Stage g: the first K step's MFMAs run while the second step's fragments
  // are read and half blocks 0-1 of stage g + 3 are fetched into the slot
  // of g - 1 (every wavefront's reads of it finished before the previous
  // barrier); then the barrier waits for stage g + 1 (g + 2 and the first
  // half of g + 3 stay in flight), and the second step's MFMAs run while
  // stage g + 1's first fragments are read and half blocks 2-3 of g + 3
  // are fetched. (After an epilogue the barrier's count also waits for
  // most of its stores, which were issued after the loads of g + 1.)
  int g = 0;
  for (int ct = t_first; ct < t_end; ct += Q) {
    const Tile CT = tile_at(ct);
    zero_acc();
    for (int cs = 0; cs < CT.stages; ++cs, ++g) {
      const int u = g & 3;
      const StageLd L = next_stage();
      mma_step(fb0, fa0, [&](int x) {
        if (x < 8)
          read_one(fb1, fa1, u, 1, x);
        else
          fetch(L, (u + 3) & 3, x - 8);
      });
      wait_vmem_barrier<kLoads + kLoads / 2>();
      mma_step(fb1, fa1, [&](int x) {
        if (x < 8)
          read_one(fb0, fa0, (u + 1) & 3, 0, x);
        else
          fetch(L, (u + 3) & 3, x - 6);
      });
    }
    epilogue(CT);
  }
  // the loads that ran past the last stage read nothing but still write
  // LDS: let them land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

hipError_t launch_wgrad(const Shape& s, int r, int nr, const void* U, const void* V,
                        const void* U1, const void* V1, int A, int A0, int B,
                        float* out0, float* out1, const PlanBuffers& b,
                        const int32_t* rows0, const int32_t* rows1, int num_cus,
                        hipStream_t st) {
  int active = 0;
  for (int e = 0; e < s.E; ++e) active += rows0[e] > 0 || (nr == 2 && rows1[e] > 0);
  const bool all = r == 0;
  const int n = all ? s.E : active;
  if (n == 0) return hipSuccess;
  const int per = ((A + kTile - 1) / kTile) * ((B + kTile - 1) / kTile);
  const int tiles = n * per;
  // one workgroup per CU (or per tile), a multiple of 8 for the XCD walk
  int grid = tiles < num_cus ? tiles : num_cus;
  grid = (grid + 7) / 8 * 8;
  WgradParams p{static_cast<const bf16*>(U), static_cast<const bf16*>(V),
                static_cast<const bf16*>(U1), static_cast<const bf16*>(V1), out0, out1,
                b.rounds, b.n_rounds, s.E, r, A, A0, B, (int)s.max_rounds(),
                nr, tiles, all ? 1 : 0, r == 0 ? 0 : 1};
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace moe
