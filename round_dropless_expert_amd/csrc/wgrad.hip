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
// MFMAs at fixed points, and the stage loop is unrolled over the four ring
// slots, so that every LDS address is a per-lane base plus an immediate
// offset (one wavefront per SIMD: each address instruction would take an
// issue slot from the matrix core).
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
  int tiles;        // tiles of the launch (the grid is this rounded up to 8)
  int all_experts;  // tiles of every expert (round 0: experts without rows get zeros)
  int accumulate;   // add to out (else store)
};

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

  // tile -> expert: expert-major, tiles_a x tiles_b per expert
  const int ta = (p.A + kTile - 1) / kTile, tb = (p.B + kTile - 1) / kTile;
  const int per = ta * tb;
  const int64_t tbl = (int64_t)p.max_rounds * p.E;
  // XCD-contiguous walk: workgroup b runs on XCD b % 8, so XCD x takes
  // tiles [x n / 8, (x + 1) n / 8): an expert's tiles, which share its
  // operand panels, stay on one XCD's L2
  const int per_xcd = (int)gridDim.x / 8;
  const int tile = (int)(blockIdx.x % 8) * per_xcd + (int)(blockIdx.x / 8);
  if (tile >= p.tiles) return;
  const int slot = tile / per;
  const int local = tile % per;
  int e;
  if (p.all_experts) {
    e = slot;
  } else {  // the slot-th expert with rows in these rounds
    const bool act =
        lane < p.E && (p.rounds[kAlloc * tbl + (int64_t)p.r * p.E + lane] > 0 ||
                       (two && p.rounds[kAlloc * tbl + (int64_t)(p.r + 1) * p.E + lane] > 0));
    const uint64_t mask = __builtin_amdgcn_ballot_w64(act);
    const uint64_t below = lane == 0 ? 0ull : (mask & (~0ull >> (64 - lane)));
    const bool hit = act && __builtin_popcountll(below) == slot;
    const uint64_t h = __builtin_amdgcn_ballot_w64(hit);
    if (h == 0) return;
    e = __builtin_ctzll(h);
  }
  if (e >= p.E) return;
  // the expert's rows in round r (segment 0) and, with two rounds, in round
  // r + 1 (segment 1, the second buffer set): m rows padded to 64 each
  const int64_t at0 = (int64_t)p.r * p.E + e, at1 = at0 + p.E;
  const int m0 = __builtin_amdgcn_readfirstlane(p.rounds[kAlloc * tbl + at0]);
  const int m1 = two ? __builtin_amdgcn_readfirstlane(p.rounds[kAlloc * tbl + at1]) : 0;
  const int64_t row00 = p.rounds[kBrow * tbl + at0];
  const int64_t row01 = two ? p.rounds[kBrow * tbl + at1] : 0;
  const int a0 = (local / tb) * kTile, b0 = (local % tb) * kTile;

  const uint32_t ubytes = (uint32_t)p.A * 2, vbytes = (uint32_t)p.B * 2;
  const uint32_t mpad0 = (uint32_t)((m0 + 63) & ~63), mpad1 = (uint32_t)((m1 + 63) & ~63);
  const __amdgpu_buffer_rsrc_t ru0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.U + row00 * p.A), 0, (int)(mpad0 * ubytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.V + row00 * p.B), 0, (int)(mpad0 * vbytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ru1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(two ? p.U1 + row01 * p.A : p.U), 0, (int)(mpad1 * ubytes), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv1 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(two ? p.V1 + row01 * p.B : p.V), 0, (int)(mpad1 * vbytes), kRsrcWord3);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)&lds[0][0];

  // Loads of a stage: wavefronts 0-1 fetch U, 2-3 fetch V. A wavefront
  // moves four 32-feature half blocks h = 0..3 (features fbase + 32 h of
  // the operand, LDS half block 4 (wave % 2) + h), each as two 1 KiB parts:
  // lane i moves 16 bytes, of token k0 + 16 part + i / 4 of the stage's
  // segment (zeros past its m, and past A or B). One M0 value serves both
  // parts of a half block, whose LDS and buffer addresses both advance by
  // the load's 1 KiB immediate offset. Stages 0 .. S0-1 are segment 0's,
  // then segment 1's.
  const int op = wave >> 1;
  const __amdgpu_buffer_rsrc_t rsrc0 = op == 0 ? ru0 : rv0;
  const __amdgpu_buffer_rsrc_t rsrc1 = op == 0 ? ru1 : rv1;
  const int S0 = (m0 + kStageTok - 1) / kStageTok;
  const uint32_t rb = op == 0 ? ubytes : vbytes;
  const int fbase = (op == 0 ? a0 : b0) + 128 * (wave & 1);
  const int flim = op == 0 ? p.A : p.B;
  const uint32_t dst0 = lds0 + (uint32_t)(op * kOpBytes + 4 * (wave & 1) * kHalfBlock);
  // per tile: this lane's offset of half block h inside a stage's 64-row
  // band (out of range for feature blocks at or past A or B; the range
  // check then zero-fills whatever the stage's offset is)
  uint32_t vh[4];
#pragma unroll
  for (int h = 0; h < 4; ++h)
    vh[h] = fbase + 32 * h < flim ? (uint32_t)((fbase >> 5) + h) * 4096u + (uint32_t)lane * 16u
                                  : kOutOfRange;
  // Per stage: the segment's descriptor, the stage's band offset and, per
  // half block and part, this lane's offset (out of range for tokens past
  // the segment's m).
  struct StageLd {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t koff;
    uint32_t vo[4][2];
  };
  auto stage_ld = [&](int s) {
    StageLd L;
    const bool seg1 = s >= S0;
    const int k0 = (seg1 ? s - S0 : s) * kStageTok;
    const int m = seg1 ? m1 : m0;
    L.rs = seg1 ? rsrc1 : rsrc0;
    L.koff = (uint32_t)(k0 >> 6) * (rb >> 6) * 4096u + (uint32_t)((k0 >> 5) & 1) * kHalfBlock;
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const bool in = k0 + part * 16 + (lane >> 2) < m;
#pragma unroll
      for (int h = 0; h < 4; ++h) L.vo[h][part] = in ? vh[h] : kOutOfRange;
    }
    return L;
  };
  // half block h of a stage into ring slot `slot`
  auto fetch = [&](const StageLd& L, int slot, int h) {
    lds_load_pair(L.rs, L.vo[h][0], L.vo[h][1], L.koff,
                  dst0 + (uint32_t)(slot * kSlotBytes + h * kHalfBlock));
  };

  // this lane's part of a transposed read: group g = lane / 16, position
  // 4 j + q in it -> token 8 (g / 2) + j (+ 4 for the second read) and
  // features 16 (g % 2) + 4 q of a 32-feature block: 16-byte chunk
  // 2 (g % 2) + q / 2, 8-byte half q % 2, swizzled by the row (the swizzle
  // repeats every 16 rows, so it does not depend on the K step). The
  // fragment reads of a slot, block and K step then differ only by
  // immediate offsets from eight per-lane bases: operand a or b, first or
  // second read, slots 0-1 or 2-3 (the offset field holds 16 bits).
  const int grp = lane >> 4, gj = (lane >> 2) & 3, gq = lane & 3;
  const int tr_row = 8 * (grp >> 1) + gj;
  const int tr_chunk = 2 * (grp & 1) + (gq >> 1);
  const int tr_half = (gq & 1) * 8;
  const int tr_lo = tr_row * 64 + ((tr_chunk ^ ((tr_row >> 2) & 3)) << 4) + tr_half;
  const int tr_hi = (tr_row + 4) * 64 + ((tr_chunk ^ (((tr_row + 4) >> 2) & 3)) << 4) + tr_half;
  const lds_char* ldsb = (const lds_char*)&lds[0][0];
  const lds_char* base_a = ldsb + wa * 4 * kHalfBlock;
  const lds_char* base_b = ldsb + kOpBytes + wb * 4 * kHalfBlock;
  const lds_char* rd[2][2][2];  // [a, b][first, second read][slots 0-1, 2-3]
#pragma unroll
  for (int sp = 0; sp < 2; ++sp) {
    rd[0][0][sp] = base_a + tr_lo + sp * 2 * kSlotBytes;
    rd[0][1][sp] = base_a + tr_hi + sp * 2 * kSlotBytes;
    rd[1][0][sp] = base_b + tr_lo + sp * 2 * kSlotBytes;
    rd[1][1][sp] = base_b + tr_hi + sp * 2 * kSlotBytes;
  }
  // fragment of operand o (0: a, 1: b), this wavefront's 32-feature block
  // blk (0..3), K step ks of the stage in ring slot `slot`
  auto frag = [&](int o, int slot, int blk, int ks) {
    const int off = (slot & 1) * kSlotBytes + blk * kHalfBlock + ks * 1024;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(rd[o][0][slot >> 1] + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(rd[o][1][slot >> 1] + off));
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 acc[4][4];  // [b block][a block]: rows a, columns b
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int stages = S0 + (m1 + kStageTok - 1) / kStageTok;
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
  // prologue: stages 0, 1, 2 in flight, wait for stage 0, read its first
  // step
#pragma unroll
  for (int st = 0; st < 3; ++st) {
    const StageLd L = stage_ld(st);
#pragma unroll
    for (int h = 0; h < 4; ++h) fetch(L, st, h);
  }
  wait_vmem_barrier<2 * kLoads>();
#pragma unroll
  for (int x = 0; x < 8; ++x) read_one(fb0, fa0, 0, 0, x);
  // Stage s (in slot u = s % 4): the first K step's MFMAs run while the
  // second step's fragments are read and half blocks 0-1 of stage s + 3 are
  // fetched into the slot of s - 1 (every wavefront's reads of it finished
  // before the previous barrier); then the barrier waits for stage s + 1
  // (s + 2 and the first half of s + 3 stay in flight), and the second
  // step's MFMAs run while stage s + 1's first fragments are read and half
  // blocks 2-3 of s + 3 are fetched. The loop is unrolled over the four
  // slots so that every LDS address is an immediate offset.
  auto stage = [&](int s, int u) {
    const StageLd L = stage_ld(s + 3);
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
  };
  for (int s = 0; s < stages; s += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s + u < stages) stage(s + u, u);
  }
  // the loads that ran past the last stage read nothing but still write
  // LDS: let them land before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // lane: b = column l32 of the block, a = rows 8 (v / 4) + 4 half + v % 4
  // for its values v: every store writes two 128-byte row pieces. (The
  // accumulators are read by asm: give the last MFMAs the wait states a
  // VALU read of their results needs, which the compiler cannot see.)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  const uint32_t rowb = (uint32_t)p.B * 4u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ab = a0 + wa * 128 + j * 32;
    if (ab >= p.A) continue;
    float* base = ab < p.A0 ? p.out0 + ((int64_t)e * p.A0 + ab) * p.B
                            : p.out1 + ((int64_t)e * (p.A - p.A0) + (ab - p.A0)) * p.B;
    const __amdgpu_buffer_rsrc_t ro =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)(32u * rowb), kRsrcWord3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int bb = b0 + wb * 128 + i * 32;
      if (bb >= p.B) continue;
      const uint32_t vo = (uint32_t)(4 * half) * rowb + (uint32_t)(bb + l32) * 4u;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t so = (uint32_t)(8 * (v / 4) + v % 4) * rowb;
        float x = acc_get(acc[i][j][v]);
        if (p.accumulate)
          x += __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ro, (int)vo, (int)so, 0));
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x), ro, (int)vo, (int)so, 0);
      }
    }
  }
}

}  // namespace

hipError_t launch_wgrad(const Shape& s, int r, int nr, const void* U, const void* V,
                        const void* U1, const void* V1, int A, int A0, int B,
                        float* out0, float* out1, const PlanBuffers& b,
                        const int32_t* rows0, const int32_t* rows1, hipStream_t st) {
  int active = 0;
  for (int e = 0; e < s.E; ++e) active += rows0[e] > 0 || (nr == 2 && rows1[e] > 0);
  const bool all = r == 0;
  const int n = all ? s.E : active;
  if (n == 0) return hipSuccess;
  const int per = ((A + kTile - 1) / kTile) * ((B + kTile - 1) / kTile);
  const int tiles = n * per;
  WgradParams p{static_cast<const bf16*>(U), static_cast<const bf16*>(V),
                static_cast<const bf16*>(U1), static_cast<const bf16*>(V1), out0, out1,
                b.rounds, b.n_rounds, s.E, r, A, A0, B, (int)s.max_rounds(),
                nr, tiles, all ? 1 : 0, r == 0 ? 0 : 1};
  hipLaunchKernelGGL(wgrad_kernel, dim3((unsigned)((tiles + 7) / 8 * 8)), dim3(256), 0,
                     st, p);
  return hipGetLastError();
}

}  // namespace moe
