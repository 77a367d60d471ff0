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
// Wavefront router (k > 8; topk_lane_kernel below serves k <= 8).
// Workgroup b routes the tokens [kHistTokens*b, kHistTokens*(b+1)): one
// wavefront serves 64/EP rows at a time, lane e of a row segment holding
// logit e. The k picks are k butterfly arg-max reductions over the segment,
// keyed by (logit descending, expert ascending), a strict total order since
// experts are distinct, so every lane of the segment agrees on the winner.
// Their expert histogram (plan phase 1) is counted on the way in LDS: a
// count does not depend on the order the increments land in.
template <int EP>
__global__ __launch_bounds__(256) void topk_softmax_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k,
    int32_t* __restrict__ idx, float* __restrict__ weight,
    int32_t* __restrict__ hist) {
  constexpr int kRowsPerWave = kWave / EP;
  constexpr int kRowsPerPass = 4 * kRowsPerWave;
  __shared__ int h[kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int seg = lane / EP;
  const int e = lane % EP;
  if (threadIdx.x < kWave) h[threadIdx.x] = 0;
  __syncthreads();
  const int64_t first = (int64_t)blockIdx.x * kHistTokens;
  const int64_t last = first + kHistTokens < T ? first + kHistTokens : T;
  for (int64_t row0 = first + wv * kRowsPerWave; row0 < last; row0 += kRowsPerPass) {
    const int64_t row = row0 + seg;
    const bool live = row < last && e < E;
    float v = live ? logits[row * E + e] : -INFINITY;
    // A NaN compares false both ways and would break the total order: every
    // NaN lane would keep its own value, consider itself the winner, and a
    // later pick could fall on a retired or padding key (>= 64), i.e. an
    // expert index out of range. As -inf it still ranks below every number
    // and, with key e < 64, above padding (64 + e) and retired lanes
    // (128 + e); k <= E leaves enough live lanes, so the k picks are always
    // k distinct experts in [0, E).
    if (!(v == v)) v = -INFINITY;
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
    if (row < last && e < k) {
      idx[row * k + e] = sel_e;
      weight[row * k + e] = ex / sum;
      atomicAdd(&h[sel_e], 1);
    }
  }
  __syncthreads();
  if (threadIdx.x < E) hist[(int64_t)blockIdx.x * E + threadIdx.x] = h[threadIdx.x];
}

// Router for k <= 8: lanes 4 t .. 4 t + 3 of workgroup b route token
// kRankTokens * b + t. Lane q of the four holds experts q M .. q M + M - 1
// (M = EP / 4) and keeps its K best (value, expert) pairs (K: k rounded up
// to a power of two) in registers, sorted by the same strict total order
// (logit descending, expert ascending): each insertion carries the losing
// pair down the list, and placeholders (-inf, 64 + i) lose to every real
// expert, -inf included. Two exchange rounds with the lanes at xor distance
// 1 and 2 then merge the four lists: the pairwise better of a[i] and the
// partner's b[K-1-i] are the K best of both lists in bitonic order, which
// K/2 log2 K compare-exchanges sort (both lanes of a pair end with the same
// list). The workgroup's 256 tokens are exactly one ranking chunk, so it
// writes that chunk's expert counts (plan phase 1 summed per chunk)
// directly. kVec: the logits rows are 16-byte aligned and each lane's M
// logits are read four at a time.
struct Pick {
  float v;
  int e;
};

__device__ __forceinline__ bool pick_better(float v1, int e1, float v2, int e2) {
  // bitwise, not short-circuit: no branch per comparison
  return (v1 > v2) | ((v1 == v2) & (e1 < e2));
}

template <int EP, int K, bool kVec>
__global__ __launch_bounds__(1024) void topk_lane_kernel(
    const float* __restrict__ logits, int64_t T, int E, int k,
    int32_t* __restrict__ idx, float* __restrict__ weight,
    int32_t* __restrict__ sums) {
  constexpr int L = 4, M = EP / L;
  static_assert(K <= 8 && EP <= kWave && EP >= L, "lane router: k <= 8, E <= 64");
  static_assert(!kVec || M % 4 == 0, "four logits per load");
  __shared__ int h[kWave];
  if (threadIdx.x < kWave) h[threadIdx.x] = 0;
  __syncthreads();
  const int q = threadIdx.x & (L - 1);
  const int64_t row = (int64_t)blockIdx.x * kRankTokens + threadIdx.x / L;
  const bool live = row < T;
  const int e0 = q * M;
  const float* lr = logits + (live ? row : 0) * E + e0;
  float lv[M];
  if constexpr (kVec) {
#pragma unroll
    for (int c = 0; c < M / 4; ++c) {
      const float4 f = live && e0 + 4 * c < E ? reinterpret_cast<const float4*>(lr)[c]
                                              : make_float4(0.f, 0.f, 0.f, 0.f);
      lv[4 * c] = f.x;
      lv[4 * c + 1] = f.y;
      lv[4 * c + 2] = f.z;
      lv[4 * c + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < M; ++m) lv[m] = live && e0 + m < E ? lr[m] : 0.f;
  }
  Pick t[K];
#pragma unroll
  for (int i = 0; i < K; ++i) t[i] = {-INFINITY, kWave + i};
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (e0 + m < E) {
      // NaN as -inf, as in the wavefront router: it ranks below every
      // number and above no real expert's place
      Pick c = {lv[m] == lv[m] ? lv[m] : -INFINITY, e0 + m};
#pragma unroll
      for (int i = 0; i < K; ++i) {
        const bool win = pick_better(c.v, c.e, t[i].v, t[i].e);
        const Pick d = win ? t[i] : c;
        t[i] = win ? c : t[i];
        c = d;
      }
    }
  }
  // merge with the lanes at xor distance 1, then 2 (all lanes take part)
#pragma unroll
  for (int x = 1; x < L; x <<= 1) {
    Pick b[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      b[i].v = __shfl_xor(t[i].v, x);
      b[i].e = __shfl_xor(t[i].e, x);
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const Pick o = b[K - 1 - i];
      t[i] = pick_better(t[i].v, t[i].e, o.v, o.e) ? t[i] : o;
    }
#pragma unroll
    for (int st = K / 2; st > 0; st >>= 1)
#pragma unroll
      for (int i = 0; i < K; ++i)
        if ((i & st) == 0) {
          const Pick a = t[i], c = t[i + st];
          const bool keep = pick_better(a.v, a.e, c.v, c.e);
          t[i] = keep ? a : c;
          t[i + st] = keep ? c : a;
        }
  }
  if (live && q == 0) {
    // softmax over the k picks
    float ex[K], sum = 0.f;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      ex[j] = j < k ? expf(t[j].v - t[0].v) : 0.f;
      sum += ex[j];
    }
#pragma unroll
    for (int j = 0; j < K; ++j)
      if (j < k) {
        idx[row * k + j] = t[j].e;
        weight[row * k + j] = ex[j] / sum;
        atomicAdd(&h[t[j].e], 1);
      }
  }
  __syncthreads();
  if (threadIdx.x < E) sums[(int64_t)blockIdx.x * E + threadIdx.x] = h[threadIdx.x];
}

template <int EP>
static hipError_t route_ep(const Shape& s, const float* logits, PlanBuffers b,
                           hipStream_t st) {
  hipLaunchKernelGGL(topk_softmax_kernel<EP>, dim3((unsigned)hist_rows(s)),
                     dim3(256), 0, st, logits, s.T, s.E, s.k, b.idx, b.weight,
                     b.scratch);
  return hipGetLastError();
}

template <int EP, int K>
static hipError_t route_lane(const Shape& s, const float* logits, PlanBuffers b,
                             hipStream_t st) {
  static_assert(kRankTokens * 4 == 1024, "one ranking chunk per workgroup, 4 lanes a token");
  int32_t* sums = b.scratch + hist_rows(s) * s.E;
  constexpr bool kCanVec = EP >= 16;  // four logits or more per lane
  const bool vec = kCanVec && s.E % 4 == 0 && ((uintptr_t)logits & 15) == 0;
  if (vec)
    hipLaunchKernelGGL((topk_lane_kernel<EP, K, kCanVec>), dim3((unsigned)rank_blocks(s)),
                       dim3(1024), 0, st, logits, s.T, s.E, s.k, b.idx, b.weight, sums);
  else
    hipLaunchKernelGGL((topk_lane_kernel<EP, K, false>), dim3((unsigned)rank_blocks(s)),
                       dim3(1024), 0, st, logits, s.T, s.E, s.k, b.idx, b.weight, sums);
  return hipGetLastError();
}

template <int EP>
static hipError_t route_lane_k(const Shape& s, const float* logits, PlanBuffers b,
                               hipStream_t st) {
  if (s.k <= 1) return route_lane<EP, 1>(s, logits, b, st);
  if (s.k <= 2) return route_lane<EP, 2>(s, logits, b, st);
  if (s.k <= 4) return route_lane<EP, 4>(s, logits, b, st);
  return route_lane<EP, 8>(s, logits, b, st);
}

hipError_t launch_route(const Shape& s, const float* logits, PlanBuffers b,
                        hipStream_t st) {
  if (route_sums_chunks(s)) {
    if (s.E <= 4) return route_lane_k<4>(s, logits, b, st);
    if (s.E <= 8) return route_lane_k<8>(s, logits, b, st);
    if (s.E <= 16) return route_lane_k<16>(s, logits, b, st);
    if (s.E <= 32) return route_lane_k<32>(s, logits, b, st);
    return route_lane_k<64>(s, logits, b, st);
  }
  if (s.E <= 1) return route_ep<1>(s, logits, b, st);
  if (s.E <= 2) return route_ep<2>(s, logits, b, st);
  if (s.E <= 4) return route_ep<4>(s, logits, b, st);
  if (s.E <= 8) return route_ep<8>(s, logits, b, st);
  if (s.E <= 16) return route_ep<16>(s, logits, b, st);
  if (s.E <= 32) return route_ep<32>(s, logits, b, st);
  return route_ep<64>(s, logits, b, st);
}

// ------------------------------------------------------------------ plan
// Phase 1 is the router's histogram hist[q][e] of the tokens [8 q, 8 q + 8);
// this kernel sums it per chunk of 256 tokens: sums[b][e] = sum of rows
// 32 b .. 32 b + 31 (wavefront w adds rows w, w + 4, ...; the order of the
// terms of a sum does not matter).
__global__ __launch_bounds__(256) void plan_chunk_sum_kernel(
    const int32_t* __restrict__ hist, int64_t nrows, int E,
    int32_t* __restrict__ sums) {
  constexpr int kRows = kRankTokens / kHistTokens;
  __shared__ int part[4][kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int64_t q0 = (int64_t)blockIdx.x * kRows;
  int n = 0;
  if (lane < E)
#pragma unroll
    for (int i = wv; i < kRows; i += 4)
      if (q0 + i < nrows) n += hist[(q0 + i) * E + lane];
  part[wv][lane] = n;
  __syncthreads();
  if (threadIdx.x < E)
    sums[(int64_t)blockIdx.x * E + threadIdx.x] =
        part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] +
        part[3][threadIdx.x];
}

// Launch batches (see RoundTable), one wavefront, lane = expert e. The
// cursor is wavefront-uniform: the current batch and the pairs it holds.
struct BatchCursor {
  int b = 0, used = 0;
};

// Places round r: lane e (on: e < E) has m rows in it, the first of which is
// entry `cum` of its list; off_e = offsets[e]; nobrow is where e's matrix
// of the round starts without packing. Round r joins the current batch if
// packing is on and its pairs still fit the E regions, else it opens the
// next batch. Writes kBrow, the pair tables and rbeg/rend of round r.
__device__ __forceinline__ void place_round(int r, int lane, bool on, int m, int cum,
                                            int off_e, int nobrow, int E, int P,
                                            bool pack, int64_t max_rounds,
                                            int32_t* __restrict__ rounds,
                                            BatchCursor& cur) {
  const int64_t tbl = max_rounds * E;
  const bool act = on && m > 0;
  const uint64_t bal = __ballot(act);
  const int a = __popcll(bal);
  if (r > 0 && (!pack || cur.used + a > E)) {
    ++cur.b;
    cur.used = 0;
  }
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  const int v = cur.used + __popcll(bal & below);
  const int brow = pack ? v * P : nobrow;
  if (on) rounds[kBrow * tbl + (int64_t)r * E + lane] = act ? brow : nobrow;
  if (act) {
    const int64_t g = (int64_t)cur.b * E + v;
    rounds[kPairE * tbl + g] = lane;
    rounds[kPairM * tbl + g] = m;
    rounds[kPairRow * tbl + g] = brow;
    rounds[kPairZ * tbl + g] = off_e + cum;
  }
  if (lane == 0) {
    int32_t* rb = rounds + kTables * tbl;
    rb[r] = cur.b * E + cur.used;
    rb[max_rounds + r] = cur.b * E + cur.used + a;
  }
  cur.used += a;
}

// Phase 2 (one workgroup): counts n_e = sum_b sums[b][e], exclusive offsets
// over e, the rounds and their tables, and, when there are more than
// kSelfScanMaxChunks chunks, every chunk's first position of expert e's
// entries, offsets[e] + sum_{b' < b} sums[b'][e], written in place of the
// sums (with fewer chunks each ranking workgroup sums its prefix itself).
//
// Rounds (wavefront 0, lane e = expert): with rem_e entries left, expert e
// first takes min(rem_e, C') rows; the slots its group of G experts leaves
// unused (G*C' minus the group's sum) then go to the group's experts with
// entries left over, in ascending expert order. Group sums and prefixes are
// segments of a wavefront-wide inclusive scan. Per round r the tables get
// m(r,e), the index of e's first entry of the round, and the rows of the
// lower experts of e's group in the round (plain and each rounded up to 64,
// which is where e's rows start in the group's block of the round buffer).
// R is the number of rounds until nothing is left.
__global__ __launch_bounds__(1024) void plan_scan_kernel(
    int32_t* __restrict__ sums, int64_t nchunks, int E, int ce, int G,
    bool write_starts, int64_t max_rounds, bool pack, int pool_rows,
    int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ n_rounds,
    int32_t* __restrict__ rounds) {
  constexpr int kWaves = 16;
  __shared__ int part[kWaves][kWave];
  __shared__ int base[kWave];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const bool on = lane < E;
  // column sums: wavefront w takes chunks w, w + 16, ...
  int n = 0;
  if (on)
    for (int64_t b = wv; b < nchunks; b += kWaves) n += sums[b * E + lane];
  part[wv][lane] = n;
  __syncthreads();
  if (wv == 0) {
    int tot = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tot += part[w][lane];
    if (!on) tot = 0;
    const int incl = wave_inclusive_scan(tot);
    const int excl = incl - tot;
    if (on) {
      counts[lane] = tot;
      offsets[lane] = excl;
    }
    if (lane == E - 1) offsets[E] = incl;
    base[lane] = excl;

    // the rounds
    const int g0 = lane - lane % G;  // first lane of this lane's group
    auto in_group_excl = [&](int v) {  // exclusive prefix inside the group
      const int inc = wave_inclusive_scan(v);
      const int before = __shfl(inc, g0 > 0 ? g0 - 1 : 0, kWave);
      return inc - v - (g0 > 0 ? before : 0);
    };
    auto group_sum = [&](int v) {
      const int inc = wave_inclusive_scan(v);
      const int last = __shfl(inc, g0 + G - 1, kWave);
      const int before = __shfl(inc, g0 > 0 ? g0 - 1 : 0, kWave);
      return last - (g0 > 0 ? before : 0);
    };
    const int64_t tbl = max_rounds * E;
    const int P = (ce + 63) & ~63;
    BatchCursor cur;
    int rem = tot;
    int r = 0;
    while (__ballot(rem > 0) != 0ull) {
      const int own = rem < ce ? rem : ce;
      const int spare = G * ce - group_sum(own);
      const int over = rem - own;
      int extra = spare - in_group_excl(over);
      extra = extra < 0 ? 0 : (extra > over ? over : extra);
      const int m = own + extra;
      const int ub = in_group_excl(m);
      const int pb = in_group_excl((m + 63) & ~63);
      if (on && r < max_rounds) {
        const int64_t at = (int64_t)r * E + lane;
        rounds[kAlloc * tbl + at] = m;
        rounds[kCum * tbl + at] = tot - rem;
        rounds[kUbase * tbl + at] = ub;
        rounds[kPbase * tbl + at] = pb;
      }
      if (r < max_rounds)
        place_round(r, lane, on, m, tot - rem, excl, (lane / G) * pool_rows + pb, E, P,
                    pack, max_rounds, rounds, cur);
      rem -= m;
      ++r;
    }
    if (lane == 0) *n_rounds = r;
  }
  __syncthreads();
  if (!write_starts) return;
  // chunk starts, 16 consecutive chunks at a time: wavefront w takes chunk
  // 16 t + w, and the starts follow from an exclusive scan over the group
  for (int64_t b0 = 0; b0 < nchunks; b0 += kWaves) {
    const int64_t b = b0 + wv;
    const int c = on && b < nchunks ? sums[b * E + lane] : 0;
    part[wv][lane] = c;
    __syncthreads();
    int pre = base[lane];
    for (int w = 0; w < wv; ++w) pre += part[w][lane];
    if (on && b < nchunks) sums[b * E + lane] = pre;
    __syncthreads();
    if (wv == 0) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) add += part[w][lane];
      base[lane] += add;
    }
    __syncthreads();
  }
}

// Where a ranking workgroup's starts come from.
enum RankMode {
  kStartsGiven = 0,  // phase 2 left each chunk's starts in place of its sums
  kSelfPrefix = 1,   // offsets from phase 2; the prefix over chunks summed here
  kSelfAll = 2,      // G = 1, no phase 2: totals, offsets and the prefix
                     // summed here; workgroup 0 also writes counts, offsets,
                     // R and the round tables (closed form for G = 1)
};

// Phase 3: stable ranking inside each chunk. The chunk is walked in order,
// 256 assignments per step; inside a wavefront the lanes holding the same
// expert are found with six ballots (one per bit of the expert index), the
// rank is the number of such lanes below, and per-wave totals are combined
// in wave order through LDS. Then the position, its inverse and the round
// and row are written. Workgroup b ranks the assignments of tokens
// [256 b, 256 b + 256); its starts are offsets[e] plus the chunk sums of
// the chunks before it (see RankMode).
// An entry's round is i / C' and its row e*C' + i % C' for G = 1; with
// groups, the last round whose first index is <= i (binary search in the
// tables), and its row g*G*C' + (rows of the group's lower experts) +
// (i - first index).
template <int kMode>
__global__ __launch_bounds__(256) void plan_rank_kernel(
    const int32_t* __restrict__ idx, int64_t TK, int E, int k, int ce, int G,
    int64_t nchunks, const int32_t* __restrict__ sums,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ n_rounds, int32_t* __restrict__ rounds,
    int64_t max_rounds, bool pack, int32_t* __restrict__ perm,
    int32_t* __restrict__ pos, int32_t* __restrict__ round_of,
    int32_t* __restrict__ row_of) {
  __shared__ int running[kWave];
  __shared__ int offs[kWave];
  __shared__ int cnt[4][kWave];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int64_t blk = blockIdx.x;
  const int64_t tbl = max_rounds * E;
  if (kMode == kSelfAll) {
    // column totals and the prefix over the chunks before this one:
    // wavefront w takes chunks w, w + 4, ... (a sum does not depend on the
    // order of its terms)
    int tot = 0, pre = 0;
    if (lane < E) {
      int64_t q = wv;
      for (; q + 12 < nchunks; q += 16) {  // four loads in flight
        const int v0 = sums[q * E + lane], v1 = sums[(q + 4) * E + lane];
        const int v2 = sums[(q + 8) * E + lane], v3 = sums[(q + 12) * E + lane];
        tot += v0 + v1 + v2 + v3;
        pre += (q < blk ? v0 : 0) + (q + 4 < blk ? v1 : 0) +
               (q + 8 < blk ? v2 : 0) + (q + 12 < blk ? v3 : 0);
      }
      for (; q < nchunks; q += 4) {
        const int v = sums[q * E + lane];
        tot += v;
        if (q < blk) pre += v;
      }
    }
    cnt[wv][lane] = tot;
    __syncthreads();
    __shared__ int tots[kWave];
    __shared__ int rmax_sh;
    if (wv == 0) {
      int n = cnt[0][lane] + cnt[1][lane] + cnt[2][lane] + cnt[3][lane];
      if (lane >= E) n = 0;
      const int incl = wave_inclusive_scan(n);
      offs[lane] = incl - n;
      tots[lane] = n;
      const int rmax = wave_max(lane < E ? (int)(((int64_t)n + ce - 1) / ce) : 0);
      if (lane == 0) rmax_sh = rmax;
      if (blk == 0) {
        if (lane < E) {
          counts[lane] = n;
          offsets[lane] = incl - n;
        }
        if (lane == E - 1) offsets[E] = incl;
        if (lane == 0) *n_rounds = rmax;
      }
    }
    __syncthreads();
    if (blk == 0) {
      // round r: expert e has min(C', n_e - r C') rows (none past its last
      // round), its first entry is the round's r C'-th, and with one expert
      // per group there are no lower experts in its group
      const int64_t cells = (int64_t)rmax_sh * E;
      for (int64_t c = tid; c < cells; c += blockDim.x) {
        const int e = (int)(c % E);
        const int64_t first = (c / E) * ce;
        const int64_t n = tots[e];
        const int64_t left = n - first;
        rounds[kAlloc * tbl + c] = (int)(left <= 0 ? 0 : (left < ce ? left : ce));
        rounds[kCum * tbl + c] = (int)(first < n ? first : n);
        rounds[kUbase * tbl + c] = 0;
        rounds[kPbase * tbl + c] = 0;
      }
      // the launch batches, round by round on wavefront 0
      if (wv == 0) {
        const int P = (ce + 63) & ~63;
        const bool on = lane < E;
        const int64_t n = on ? tots[lane] : 0;
        BatchCursor cur;
        for (int r = 0; r < rmax_sh; ++r) {
          const int64_t first = (int64_t)r * ce;
          const int64_t left = n - first;
          const int m = (int)(left <= 0 ? 0 : (left < ce ? left : ce));
          place_round(r, lane, on, m, (int)(first < n ? first : n), on ? offs[lane] : 0,
                      lane * P, E, P, pack, max_rounds, rounds, cur);
        }
      }
    }
    cnt[wv][lane] = pre;
    __syncthreads();
    if (tid < kWave)
      running[tid] = offs[tid] + cnt[0][tid] + cnt[1][tid] + cnt[2][tid] + cnt[3][tid];
  } else if (kMode == kSelfPrefix) {
    // the prefix over the chunks before this one, as above
    int pre = 0;
    if (lane < E) {
      int64_t q = wv;
      for (; q + 12 < blk; q += 16)  // four loads in flight
        pre += sums[q * E + lane] + sums[(q + 4) * E + lane] +
               sums[(q + 8) * E + lane] + sums[(q + 12) * E + lane];
      for (; q < blk; q += 4) pre += sums[q * E + lane];
    }
    cnt[wv][lane] = pre;
    __syncthreads();
    if (tid < kWave) {
      offs[tid] = tid < E ? offsets[tid] : 0;
      running[tid] = offs[tid] + cnt[0][tid] + cnt[1][tid] + cnt[2][tid] + cnt[3][tid];
    }
  } else {
    if (tid < kWave) {
      running[tid] = tid < E ? sums[blk * E + tid] : 0;
      offs[tid] = tid < E ? offsets[tid] : 0;
    }
  }
  // rounds (only needed for G > 1, when phase 2 has written them)
  const int R = G == 1 ? 0 : *n_rounds;
  const int64_t start = blk * kRankTokens * k;
  const int64_t end = start + (int64_t)kRankTokens * k < TK
                          ? start + (int64_t)kRankTokens * k : TK;
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
      const int i = p - offs[e];
      if (G == 1) {
        round_of[a] = i / ce;
        row_of[a] = e * ce + i % ce;
      } else {
        int lo = 0, hi = R - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (rounds[kCum * tbl + (int64_t)mid * E + e] <= i) lo = mid; else hi = mid - 1;
        }
        const int64_t at = (int64_t)lo * E + e;
        round_of[a] = lo;
        row_of[a] = (e - e % G) * ce + rounds[kUbase * tbl + at] +
                    (i - rounds[kCum * tbl + at]);
      }
    }
  }
}

// Chunks up to which every ranking workgroup sums its prefix itself
// (up to chunks * E reads per workgroup, from L2).
constexpr int64_t kSelfScanMaxChunks = 1024;

hipError_t launch_plan(const Shape& s, PlanBuffers b, hipStream_t st) {
  const int64_t TK = s.T * s.k;
  const int64_t nrows = hist_rows(s);
  const int64_t nb = rank_blocks(s);
  int32_t* sums = b.scratch + nrows * s.E;
  hipError_t err = hipSuccess;
  if (!route_sums_chunks(s)) {  // else the router wrote the chunk sums
    hipLaunchKernelGGL(plan_chunk_sum_kernel, dim3((unsigned)nb), dim3(256), 0, st,
                       b.scratch, nrows, s.E, sums);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const bool self = nb <= kSelfScanMaxChunks;
  const int64_t mr = s.max_rounds();
  if (self && s.G == 1) {  // one pass: no phase 2
    hipLaunchKernelGGL(plan_rank_kernel<kSelfAll>, dim3((unsigned)nb), dim3(256), 0,
                       st, b.idx, TK, s.E, s.k, s.ce, s.G, nb, sums, b.counts,
                       b.offsets, b.n_rounds, b.rounds, mr, s.pack, b.perm, b.pos,
                       b.round_of, b.row_of);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(plan_scan_kernel, dim3(1), dim3(1024), 0, st, sums, nb, s.E,
                     s.ce, s.G, !self, mr, s.pack, (int)s.pool_rows(), b.counts,
                     b.offsets, b.n_rounds, b.rounds);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (self)
    hipLaunchKernelGGL(plan_rank_kernel<kSelfPrefix>, dim3((unsigned)nb), dim3(256),
                       0, st, b.idx, TK, s.E, s.k, s.ce, s.G, nb, sums, b.counts,
                       b.offsets, b.n_rounds, b.rounds, mr, s.pack, b.perm, b.pos,
                       b.round_of, b.row_of);
  else
    hipLaunchKernelGGL(plan_rank_kernel<kStartsGiven>, dim3((unsigned)nb), dim3(256),
                       0, st, b.idx, TK, s.E, s.k, s.ce, s.G, nb, sums, b.counts,
                       b.offsets, b.n_rounds, b.rounds, mr, s.pack, b.perm, b.pos,
                       b.round_of, b.row_of);
  return hipGetLastError();
}

// The same fill rule on the host, for launch shapes: from the entries each
// expert has left (rem, updated), the rows of every expert in the next
// round.
void host_next_round(const Shape& s, int64_t* rem, int32_t* rows_out) {
  for (int g0 = 0; g0 < s.E; g0 += s.G) {
    int64_t spare = (int64_t)s.G * s.ce;
    for (int e = g0; e < g0 + s.G; ++e) {
      rows_out[e] = (int32_t)(rem[e] < s.ce ? rem[e] : s.ce);
      spare -= rows_out[e];
    }
    for (int e = g0; e < g0 + s.G; ++e) {
      const int64_t over = rem[e] - rows_out[e];
      const int64_t more = over < spare ? over : spare;
      rows_out[e] += (int32_t)more;
      spare -= more;
    }
    for (int e = g0; e < g0 + s.G; ++e) rem[e] -= rows_out[e];
  }
}

// The batches of place_round on the host: rounds in order, each joining
// the current batch while its pairs fit the E regions (packing), else
// opening the next.
BatchWalker::BatchWalker(const Shape& s, const int32_t* counts)
    : s_(s), left_(0), r_(0), have_pending_(false) {
  for (int e = 0; e < s.E; ++e) {
    rem_[e] = counts[e];
    left_ += counts[e];
  }
}

bool BatchWalker::next(LaunchBatch* out) {
  out->r0 = r_;
  out->nr = 0;
  out->nv = 0;
  while (true) {
    if (!have_pending_) {
      if (left_ <= 0) break;
      host_next_round(s_, rem_, pending_);
      for (int e = 0; e < s_.E; ++e) left_ -= pending_[e];
      have_pending_ = true;
    }
    int a = 0;
    for (int e = 0; e < s_.E; ++e) a += pending_[e] > 0;
    if (out->nr > 0 && (!s_.pack || out->nv + a > s_.E)) break;
    out->nv += round_pairs(s_.E, pending_, out->rows + out->nv);
    ++out->nr;
    ++r_;
    have_pending_ = false;
  }
  return out->nr > 0;
}

int round_pairs(int E, const int32_t* rows, int32_t* out) {
  int n = 0;
  for (int e = 0; e < E; ++e)
    if (rows[e] > 0) out[n++] = rows[e];
  return n;
}

}  // namespace moe
