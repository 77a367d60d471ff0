// Router and round plan of the multi-round dropless MoE layer (gfx950).
//
// Router ("Microsoft AI's MAI-Base-2 trained on 16K GPUs with Muon", section
// "Expert groups keep memory fixed when tokens pile up": routing assigns every
// token to a small number of experts): top-k over the raw fp32 logits, ties to the lower
// expert index, ordered by descending logit; weights are the softmax of the
// k chosen logits (equal to the full softmax renormalised over them).
//
// Plan ("Frontier Pre-training at Microsoft AI (MAI-Base-2)", section "Key
// claims": fixed per-expert token capacity, overflow takes an extra round):
// a stable counting sort of the assignment ids by expert, and the split of
// each expert's list into rounds of at most C'. Every position comes from a
// histogram and prefix scans; no atomic decides an order.
#include "device_common.hpp"
#include "launch.hpp"

namespace moe {

// ---------------------------------------------------------------- router
// One wavefront serves 64/EP rows; lane e of a row segment holds logit e.
// The k picks are k butterfly arg-max reductions over the segment, keyed by
// (logit descending, expert ascending), a strict total order since experts
// are distinct, so every lane of the segment agrees on the winner.
template <int EP>
__global__ __launch_bounds__(256) void topk_softmax_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k,
    int32_t* __restrict__ idx, float* __restrict__ weight) {
  constexpr int kRowsPerWave = kWave / EP;
  const int lane = threadIdx.x & (kWave - 1);
  const int seg = lane / EP;
  const int e = lane % EP;
  const int64_t wave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * blockDim.x / kWave;
  for (int64_t row0 = wave * kRowsPerWave; row0 < T;
       row0 += nwaves * kRowsPerWave) {
    const int64_t row = row0 + seg;
    const bool live = row < T && e < E;
    float v = live ? logits[row * E + e] : -INFINITY;
    int key = live ? e : kWave + e;  // padding lanes lose every tie
    int sel_e = 0;
    float sel_v = 0.f, top = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = v;
      int be = key;
#pragma unroll
      for (int off = EP / 2; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, EP);
        const int oe = __shfl_xor(be, off, EP);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
      if (j == 0) top = bv;
      if (e == j) {
        sel_e = be;
        sel_v = bv;
      }
      if (key == be) {  // the winner leaves the race
        v = -INFINITY;
        key = 2 * kWave + e;
      }
    }
    // lanes j < k hold the j-th pick; softmax over the picks
    const float ex = (e < k) ? expf(sel_v - top) : 0.f;
    float sum = ex;
#pragma unroll
    for (int off = EP / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, EP);
    if (row < T && e < k) {
      idx[row * k + e] = sel_e;
      weight[row * k + e] = ex / sum;
    }
  }
}

template <int EP>
static hipError_t route_ep(const Shape& s, const float* logits, PlanBuffers b,
                           hipStream_t st) {
  constexpr int rows_per_block = 4 * (kWave / EP);
  int64_t blocks = (s.T + rows_per_block - 1) / rows_per_block;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(topk_softmax_kernel<EP>, dim3((unsigned)blocks), dim3(256),
                     0, st, logits, s.T, s.E, s.k, b.idx, b.weight);
  return hipGetLastError();
}

hipError_t launch_route(const Shape& s, const float* logits, PlanBuffers b,
                        hipStream_t st) {
  if (s.E <= 1) return route_ep<1>(s, logits, b, st);
  if (s.E <= 2) return route_ep<2>(s, logits, b, st);
  if (s.E <= 4) return route_ep<4>(s, logits, b, st);
  if (s.E <= 8) return route_ep<8>(s, logits, b, st);
  if (s.E <= 16) return route_ep<16>(s, logits, b, st);
  if (s.E <= 32) return route_ep<32>(s, logits, b, st);
  return route_ep<64>(s, logits, b, st);
}

// ------------------------------------------------------------------ plan
// Phase 1: per-chunk histogram of experts (LDS counters; a count does not
// depend on the order the increments land in).
__global__ __launch_bounds__(256) void plan_hist_kernel(
    const int32_t* __restrict__ idx, int64_t TK, int E,
    int32_t* __restrict__ hist) {
  __shared__ int h[kWave];
  if (threadIdx.x < kWave) h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kPlanChunk;
  const int64_t end = base + kPlanChunk < TK ? base + kPlanChunk : TK;
  for (int64_t a = base + threadIdx.x; a < end; a += blockDim.x)
    atomicAdd(&h[idx[a]], 1);
  __syncthreads();
  if (threadIdx.x < E) hist[(int64_t)blockIdx.x * E + threadIdx.x] = h[threadIdx.x];
}

// Phase 2 (one wavefront): counts, exclusive offsets, R, and for every
// chunk b the first position of expert e's entries from that chunk:
// offsets[e] + sum_{b' < b} hist[b'][e] (written over hist).
__global__ __launch_bounds__(64) void plan_scan_kernel(
    int32_t* __restrict__ hist, int64_t nblocks, int E, int ce,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ n_rounds) {
  const int e = threadIdx.x;
  int n = 0;
  if (e < E)
    for (int64_t b = 0; b < nblocks; ++b) n += hist[b * E + e];
  const int incl = wave_inclusive_scan(n);
  const int excl = incl - n;
  if (e < E) {
    counts[e] = n;
    offsets[e] = excl;
  }
  if (e == E - 1) offsets[E] = incl;
  const int r = (e < E) ? (int)(((int64_t)n + ce - 1) / ce) : 0;
  const int rmax = wave_max(r);
  if (e == 0) *n_rounds = rmax;
  if (e < E) {
    int run = excl;
    for (int64_t b = 0; b < nblocks; ++b) {
      const int c = hist[b * E + e];
      hist[b * E + e] = run;
      run += c;
    }
  }
}

// Phase 3: stable ranking inside each chunk. The chunk is walked in order,
// 256 assignments per step; inside a wavefront the lanes holding the same
// expert are found with six ballots (one per bit of the expert index), the
// rank is the number of such lanes below, and per-wave totals are combined
// in wave order through LDS. Then the position, its inverse and the round
// split are written.
__global__ __launch_bounds__(256) void plan_rank_kernel(
    const int32_t* __restrict__ idx, int64_t TK, int E, int ce,
    const int32_t* __restrict__ chunk_base, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ pos,
    int32_t* __restrict__ round_of, int32_t* __restrict__ row_of) {
  __shared__ int running[kWave];
  __shared__ int cnt[4][kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  if (tid < kWave)
    running[tid] = (tid < E) ? chunk_base[(int64_t)blockIdx.x * E + tid] : 0;
  const int64_t start = (int64_t)blockIdx.x * kPlanChunk;
  const int64_t end = start + kPlanChunk < TK ? start + kPlanChunk : TK;
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  __syncthreads();
  for (int64_t s = start; s < end; s += blockDim.x) {
    const int64_t a = s + tid;
    const bool live = a < end;
    const int e = live ? idx[a] : 0;
    cnt[wv][lane] = 0;
    uint64_t same = __ballot(live);
#pragma unroll
    for (int bit = 0; bit < 6; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t b = __ballot(live && set);
      same &= set ? b : ~b;
    }
    if (!live) same = 0;
    const int rank = __popcll(same & below);
    if (live && rank == 0) cnt[wv][e] = __popcll(same);
    __syncthreads();
    int p = 0;
    if (live) {
      int pre = running[e];
      for (int w2 = 0; w2 < wv; ++w2) pre += cnt[w2][e];
      p = pre + rank;
    }
    __syncthreads();
    if (tid < kWave) running[tid] += cnt[0][tid] + cnt[1][tid] + cnt[2][tid] + cnt[3][tid];
    __syncthreads();
    if (live) {
      perm[p] = (int32_t)a;
      pos[a] = p;
      const int i = p - offsets[e];
      round_of[a] = i / ce;
      row_of[a] = e * ce + i % ce;
    }
  }
}

hipError_t launch_plan(const Shape& s, PlanBuffers b, hipStream_t st) {
  const int64_t TK = s.T * s.k;
  const int64_t nb = plan_blocks(s);
  hipLaunchKernelGGL(plan_hist_kernel, dim3((unsigned)nb), dim3(256), 0, st,
                     b.idx, TK, s.E, b.scratch);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(64), 0, st, b.scratch, nb,
                     s.E, s.ce, b.counts, b.offsets, b.n_rounds);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(plan_rank_kernel, dim3((unsigned)nb), dim3(256), 0, st,
                     b.idx, TK, s.E, s.ce, b.scratch, b.offsets, b.perm, b.pos,
                     b.round_of, b.row_of);
  return hipGetLastError();
}

}  // namespace moe
