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
  int ce_pad() const { return (ce + 63) / 64 * 64; }  // round-buffer rows per expert
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
};

hipError_t launch_route(const Shape& s, const float* logits, PlanBuffers b,
                        hipStream_t st);
hipError_t launch_plan(const Shape& s, PlanBuffers b, hipStream_t st);
hipError_t launch_dispatch(const Shape& s, int r, const void* x,
                           const PlanBuffers& b, void* xr, int num_cus,
                           hipStream_t st);
// counts_host: the plan's per-expert counts read back to the host, or NULL.
// With them each round gets the tile shape and grid that fit its largest
// expert (results are identical either way); without them the large tile
// and one workgroup per CU are used.
hipError_t launch_gate_up(const Shape& s, int r, const void* xr,
                          const void* wg, const void* wu, const int32_t* counts,
                          const int32_t* counts_host, void* h, int num_cus,
                          hipStream_t st);
hipError_t launch_down(const Shape& s, int r, const void* h, const void* wd,
                       const PlanBuffers& b, const int32_t* counts_host, void* z,
                       int num_cus, hipStream_t st);
hipError_t launch_pack_weights(const Shape& s, const void* src, void* dst,
                               int rows, int cols, int num_cus, hipStream_t st);
hipError_t launch_combine(const Shape& s, const void* z, const float* weight,
                          const int32_t* pos, void* y, int num_cus, hipStream_t st);

}  // namespace moe
