// Host-side launchers of the MoE layer kernels (internal interface between
// the C ABI and the kernel translation units). All launchers enqueue on the
// given stream and return the HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct Shape {
  int64_t T;
  int E, k, d, f;
  int ce;        // min(C, T)
  bool bf16;     // element type of x, weights, y and the round buffers
  bool tiled_w;  // weights in the tiled layout of moe_pack_weights
  int G;         // experts per capacity group
  int ce_pad() const { return (ce + 63) / 64 * 64; }
  // round-buffer rows per group: each expert's rows of a round start at a
  // multiple of 64, so a group of G > 1 needs up to 64 more per expert
  int64_t pool_rows() const {
    return G == 1 ? (int64_t)ce_pad() : (int64_t)G * (ce_pad() + 64);
  }
  int64_t buf_rows() const { return (int64_t)(E / G) * pool_rows(); }
  int64_t max_rounds() const { return (T + ce - 1) / ce; }
};

// Plan-internal granularity: the router counts an expert histogram for
// every 8 consecutive tokens (one workgroup each); a reduction sums them per
// chunk of 256 tokens, and the ranking kernel takes one chunk per workgroup.
constexpr int kHistTokens = 8;
constexpr int kRankTokens = 256;

inline int64_t hist_rows(const Shape& s) {
  return (s.T + kHistTokens - 1) / kHistTokens;
}
inline int64_t rank_blocks(const Shape& s) {
  return (s.T + kRankTokens - 1) / kRankTokens;
}
// plan scratch: hist [hist_rows][E], then chunk sums [rank_blocks][E]
inline int64_t plan_scratch_ints(const Shape& s) {
  return (hist_rows(s) + rank_blocks(s)) * s.E;
}

// Largest k the backward supports (the router gradient keeps a token's k
// dot products in registers).
constexpr int kBackwardMaxK = 8;

struct PlanBuffers {
  int32_t* idx;
  float* weight;
  int32_t* counts;
  int32_t* offsets;
  int32_t* n_rounds;
  int32_t* perm;
  int32_t* pos;
  int32_t* round_of;
  int32_t* row_of;
  int32_t* scratch;  // hist [hist_rows][E], chunk sums [rank_blocks][E]
  // [4][max_rounds][E]: rows m(r,e), first list index cum(r,e), rows of the
  // lower experts of the group ubase(r,e), the same padded to 64 pbase(r,e)
  int32_t* rounds;
};

// Tables of PlanBuffers::rounds.
enum RoundTable { kAlloc = 0, kCum = 1, kUbase = 2, kPbase = 3 };

hipError_t launch_route(const Shape& s, const float* logits, PlanBuffers b,
                        hipStream_t st);
hipError_t launch_plan(const Shape& s, PlanBuffers b, hipStream_t st);
hipError_t launch_dispatch(const Shape& s, int r, const void* x,
                           const PlanBuffers& b, void* xr, int num_cus,
                           hipStream_t st);
// rows_host: the round's rows m(r,e) of every expert on the host, or NULL.
// With them the round gets the tile shape and grid that fit it (results are
// identical either way); without them the large tile and one workgroup per
// CU are used.
hipError_t launch_gate_up(const Shape& s, int r, const void* xr,
                          const void* wg, const void* wu, const PlanBuffers& b,
                          const int32_t* rows_host, void* h, int num_cus,
                          hipStream_t st);
hipError_t launch_down(const Shape& s, int r, const void* h, const void* wd,
                       const PlanBuffers& b, const int32_t* rows_host, void* z,
                       int num_cus, hipStream_t st);

// Backward GEMMs of round r (bf16; weights of the dgrad launches packed by
// launch_pack_backward): the recompute of g and u into gu [rows][2f] and of
// w * h into hw [rows][f]; dh = dyr Wd turned into dg and du (with gu) in
// dgu [rows][2f]; and dx rows = dgu [Wg | Wu] into dz [T*k][d] at the
// assignments' expert-sorted rows, like z.
hipError_t launch_recompute(const Shape& s, int r, const void* xr, const void* wg,
                            const void* wu, const PlanBuffers& b,
                            const int32_t* rows_host, void* gu, void* hw,
                            int num_cus, hipStream_t st);
hipError_t launch_dgate(const Shape& s, int r, const void* dyr, const void* wd_t,
                        const PlanBuffers& b, const int32_t* rows_host,
                        const void* gu, void* dgu, int num_cus, hipStream_t st);
hipError_t launch_dx(const Shape& s, int r, const void* dgu, const void* wgu_t,
                     const PlanBuffers& b, const int32_t* rows_host, void* dz,
                     int num_cus, hipStream_t st);

// Weight gradients of rounds r .. r + nr - 1 (nr = 1 or 2; round r's
// buffers U, V, round r + 1's U1, V1): out_e[a][b] (+)= sum over expert e's
// rows c of those rounds of U[c][a] V[c][b] (U: A features per row, V: B,
// tiled round buffers), rows a < A0 into out0 [E][A0][B], the rest into
// out1 [E][A-A0][B]; fp32. The launch with r = 0 stores (every expert,
// zeros where it has no rows), later launches add. rows0, rows1: the
// rounds' rows per expert on the host.
hipError_t launch_wgrad(const Shape& s, int r, int nr, const void* U, const void* V,
                        const void* U1, const void* V1, int A, int A0, int B,
                        float* out0, float* out1, const PlanBuffers& b,
                        const int32_t* rows0, const int32_t* rows1, hipStream_t st);

// Router-weight gradient dlogits [T][E] (fp32) from z and dy (bf16).
hipError_t launch_router_backward(const Shape& s, const void* z, const void* dy,
                                  const PlanBuffers& b, float* dlogits, int num_cus,
                                  hipStream_t st);
// The dgrad GEMMs' weights from row-major Wg, Wu [E][f][d] and Wd [E][d][f]
// (bf16): Wd transposed to [E][f][d] and [Wg; Wu] transposed to
// [E][d][2f], both tiled.
hipError_t launch_pack_backward(const Shape& s, const void* w_gate, const void* w_up,
                                const void* w_down, void* out_down_t, void* out_gu_t,
                                int num_cus, hipStream_t st);
hipError_t launch_fill(float* p, int64_t n, float value, int num_cus, hipStream_t st);

// Host copy of the plan's fill rule: from the entries each expert has left
// (rem[E], updated), the rows m(r,e) of every expert in the next round.
void host_next_round(const Shape& s, int64_t* rem, int32_t* rows_out);
hipError_t launch_pack_weights(const Shape& s, const void* src, void* dst,
                               int rows, int cols, int num_cus, hipStream_t st);
hipError_t launch_combine(const Shape& s, const void* z, const float* weight,
                          const int32_t* pos, void* y, int num_cus, hipStream_t st);

}  // namespace moe
