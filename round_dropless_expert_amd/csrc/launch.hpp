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
  // consecutive rounds share launches while their (round, expert) pairs fit
  // the round buffer's E expert regions (G = 1 with one set of round
  // buffers); otherwise every round is launched on its own
  bool pack;
  int ce_pad() const { return (ce + 63) / 64 * 64; }
  // round-buffer rows per group: each expert's rows of a round start at a
  // multiple of 64, so a group of G > 1 needs up to 64 more per expert
  int64_t pool_rows() const {
    return G == 1 ? (int64_t)ce_pad() : (int64_t)G * (ce_pad() + 64);
  }
  int64_t buf_rows() const { return (int64_t)(E / G) * pool_rows(); }
  int64_t max_rounds() const { return (T + ce - 1) / ce; }
};

// Plan-internal granularity: the ranking kernel takes one chunk of 256
// tokens per workgroup and needs each chunk's expert counts. The wavefront
// router (k > 8) counts an expert histogram for every 8 consecutive tokens
// (one workgroup each) and a reduction sums them per chunk.
constexpr int kHistTokens = 8;
constexpr int kRankTokens = 256;

inline int64_t hist_rows(const Shape& s) {
  return (s.T + kHistTokens - 1) / kHistTokens;
}
inline int64_t rank_blocks(const Shape& s) {
  return (s.T + kRankTokens - 1) / kRankTokens;
}
// The router for k <= 8 (one token per lane, one ranking chunk per
// workgroup) writes the chunk sums itself; for larger k the wavefront
// router writes the 8-token histogram and a reduction sums it per chunk.
inline bool route_sums_chunks(const Shape& s) { return s.k <= 8; }
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
  // the round tables, see RoundTable
  int32_t* rounds;
};

// Tables of PlanBuffers::rounds: kTables tables of [max_rounds][E] int32,
// then rbeg and rend, [max_rounds] each.
//
// Launch batches: the forward runs consecutive rounds in one dispatch and
// one launch of each grouped GEMM while their (round, expert) pairs with
// rows fit the E expert regions of the round buffer (Shape::pack; the
// results are identical, each output keeps its fixed K order). Batch b's
// pairs are numbered v = 0, 1, ... round by round, experts ascending inside
// a round; pair v's matrix starts at buffer row v * P. Without packing every
// round is a batch of its own and expert e's matrix of round r starts at
// its group's block plus pbase(r,e). The pair tables are indexed by the
// global pair index b * E + v; rbeg[r] and rend[r] are the global indices
// of round r's first pair and one past its last, so a launch over rounds
// [r0, r1] of one batch covers the pairs [rbeg[r0], rend[r1]).
enum RoundTable {
  kAlloc = 0,    // [r][e] rows m(r,e)
  kCum = 1,      // [r][e] index in e's list of its first entry of round r
  kUbase = 2,    // [r][e] rows of the lower experts of e's group in round r
  kPbase = 3,    // [r][e] the same with each expert's rows rounded up to 64
  kBrow = 4,     // [r][e] first buffer row (inside a set) of e's matrix of round r
  kPairE = 5,    // [b*E + v] expert of pair v of batch b
  kPairM = 6,    // its rows
  kPairRow = 7,  // its first buffer row
  kPairZ = 8,    // its first row of z: offsets[e] + cum(r,e)
  kTables = 9
};
inline int64_t round_table_ints(const Shape& s) {
  return (int64_t)kTables * s.max_rounds() * s.E + 2 * s.max_rounds();
}

hipError_t launch_route(const Shape& s, const float* logits, PlanBuffers b,
                        hipStream_t st);
hipError_t launch_plan(const Shape& s, PlanBuffers b, hipStream_t st);
// Dispatch of the rounds [r0, r0 + nr): every assignment of those rounds
// to its slot of the round buffer.
hipError_t launch_dispatch(const Shape& s, int r0, int nr, const void* x,
                           const PlanBuffers& b, void* xr, int num_cus,
                           hipStream_t st);
// Grouped GEMMs over the rounds [r0, r0 + nr), which lie in one launch
// batch (nothing runs unless r0 + nr <= R). rows_host: the rows of the
// launch's pairs on the host (nv of them, in pair order), or NULL. With
// them the launch gets the tile shape and grid that fit it (results are
// identical either way); without them the large tile and one workgroup per
// CU are used. x: NULL, or the layer's input, from which the launch then
// gathers each pair's token rows through the plan (the dispatch fused into
// the GEMM's operand fetch; xr is not read); only where gather_fits(s).
hipError_t launch_gate_up(const Shape& s, int r0, int nr, const void* xr,
                          const void* wg, const void* wu, const PlanBuffers& b,
                          const int32_t* rows_host, int nv, void* h, int num_cus,
                          hipStream_t st, const void* x = nullptr);
// x small enough for the gathering gate/up (at most 2^30 bytes)
bool gather_fits(const Shape& s);
hipError_t launch_down(const Shape& s, int r0, int nr, const void* h, const void* wd,
                       const PlanBuffers& b, const int32_t* rows_host, int nv,
                       void* z, int num_cus, hipStream_t st);

// Backward GEMMs of round r (bf16; the forward's weights, in the shape's
// weight layout): the recompute of g and u into gu [rows][2f] and of w * h
// into hw [rows][f]; dh = dyr Wd turned into dg and du (with gu) in dgu
// [rows][2f]; and dx rows = dgu [Wg; Wu] into dz [T*k][d] at the
// assignments' expert-sorted rows, like z. The last two read Wd, Wg and Wu
// transposed.
hipError_t launch_recompute(const Shape& s, int r, const void* xr, const void* wg,
                            const void* wu, const PlanBuffers& b,
                            const int32_t* rows_host, int nv, void* gu, void* hw,
                            int num_cus, hipStream_t st);
hipError_t launch_dgate(const Shape& s, int r, const void* dyr, const void* wd,
                        const PlanBuffers& b, const int32_t* rows_host, int nv,
                        const void* gu, void* dgu, int num_cus, hipStream_t st);
hipError_t launch_dx(const Shape& s, int r, const void* dgu, const void* wg,
                     const void* wu, const PlanBuffers& b, const int32_t* rows_host,
                     int nv, void* dz, int num_cus, hipStream_t st);

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
                        const int32_t* rows0, const int32_t* rows1, int num_cus,
                        hipStream_t st);

// Router-weight gradient dlogits [T][E] (fp32) from z and dy (bf16).
hipError_t launch_router_backward(const Shape& s, const void* z, const void* dy,
                                  const PlanBuffers& b, float* dlogits, int num_cus,
                                  hipStream_t st);
hipError_t launch_fill(float* p, int64_t n, float value, int num_cus, hipStream_t st);

// Host copy of the plan's fill rule: from the entries each expert has left
// (rem[E], updated), the rows m(r,e) of every expert in the next round.
void host_next_round(const Shape& s, int64_t* rem, int32_t* rows_out);

// One launch batch (see RoundTable): rounds [r0, r0 + nr) and the rows of
// its nv pairs in pair order.
struct LaunchBatch {
  int r0, nr, nv;
  int32_t rows[64];
};

// Host copy of the plan's launch batches, walked in order from the counts
// (no heap memory: the forward that allocates nothing uses it too).
class BatchWalker {
 public:
  BatchWalker(const Shape& s, const int32_t* counts);
  // the next batch; false after the last
  bool next(LaunchBatch* out);

 private:
  Shape s_;
  int64_t rem_[64];
  int64_t left_;
  int r_;
  int32_t pending_[64];  // rows of round r_, computed but not yet placed
  bool have_pending_;
};

// The rows of the experts with rows (the pairs of one round), in expert
// order; returns how many.
int round_pairs(int E, const int32_t* rows, int32_t* out);
hipError_t launch_pack_weights(const Shape& s, const void* src, void* dst,
                               int rows, int cols, int num_cus, hipStream_t st);
hipError_t launch_combine(const Shape& s, const void* z, const float* weight,
                          const int32_t* pos, void* y, int num_cus, hipStream_t st);

}  // namespace moe
