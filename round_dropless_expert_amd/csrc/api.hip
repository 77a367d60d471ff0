// C ABI of the multi-round dropless MoE layer: argument validation, the
// workspace layouts (pure functions of the config), the round loops of the
// forward and the backward, and the capacity helpers.
//
// The round loop follows "Frontier Pre-training at Microsoft AI
// (MAI-Base-2)", section "Key claims" (one or more rounds of dispatch,
// expert compute and collect with a fixed per-expert capacity; memory
// static whatever the token imbalance) and "Microsoft AI's MAI-Base-2
// trained on 16K GPUs with Muon", section "Expert groups keep memory fixed
// when tokens pile up" (overflow waits for an extra round). The plan stays
// on the device; the host reads back only the E counts and R, once, to
// size each round's launches.
#include <atomic>
#include <cstdio>
#include <mutex>
#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "../../include/moe_rounds.h"
#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

moe_status_t fail(moe_status_t s, const char* msg, const char* name = nullptr) {
  if (name)
    std::snprintf(g_err, sizeof g_err, "%s: %s", name, msg);
  else
    std::snprintf(g_err, sizeof g_err, "%s", msg);
  return s;
}

moe_status_t hip_fail(hipError_t e, const char* where) {
  std::snprintf(g_err, sizeof g_err, "%s: %s (%d)", where, hipGetErrorString(e),
                (int)e);
  return MOE_ERR_HIP;
}

size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

constexpr int kMaxExperts = 64;

int64_t eff_capacity(const moe_config_t* c) { return c->C < c->T ? c->C : c->T; }

int group_of(const moe_config_t* c) { return c->group == 0 ? 1 : c->group; }

// Sets of round buffers (xr, h): round r uses set r % sets.
int sets_of(const moe_config_t* c) {
  return c->round_buffers == 0 ? 1 : c->round_buffers;
}

moe::Shape shape_of(const moe_config_t* c) {
  return moe::Shape{c->T,       c->E, c->k, c->d_model, c->d_ff, (int)eff_capacity(c),
                    c->dtype == MOE_BF16, c->weight_layout == MOE_WEIGHTS_TILED,
                    group_of(c), group_of(c) == 1 && sets_of(c) == 1};
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

moe_status_t check_cfg(const moe_config_t* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->T < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 1");
  if (c->E < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "E must be >= 1");
  if (c->k < 1 || c->k > c->E)
    return fail(MOE_ERR_INVALID_ARGUMENT, "k must satisfy 1 <= k <= E");
  if (c->C < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "C must be >= 1");
  if (c->d_model < 1 || c->d_ff < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "d_model and d_ff must be >= 1");
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown dtype");
  if (c->weight_layout != MOE_WEIGHTS_ROW_MAJOR && c->weight_layout != MOE_WEIGHTS_TILED)
    return fail(MOE_ERR_INVALID_ARGUMENT, "unknown weight layout");
  if (c->group < 0 || (c->group > 0 && c->E % c->group != 0))
    return fail(MOE_ERR_INVALID_ARGUMENT, "group must divide E (0 means 1)");
  if (c->round_buffers < 0 || c->round_buffers > 2)
    return fail(MOE_ERR_INVALID_ARGUMENT, "round_buffers must be 0, 1 or 2");
  if (c->E > kMaxExperts) return fail(MOE_ERR_UNSUPPORTED, "E > 64 is not supported");
  if (c->d_model % 64 || c->d_ff % 64)
    return fail(MOE_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of 64");
  const int64_t TK = c->T * (int64_t)c->k;
  if (c->T >= (int64_t(1) << 31) || TK >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T*k must be < 2^31");
  // per-expert and per-group matrices are addressed with 32-bit byte offsets
  const int64_t ce_pad = (eff_capacity(c) + 63) / 64 * 64;
  const int64_t dm = c->d_model > c->d_ff ? c->d_model : c->d_ff;
  const int64_t es = c->dtype == MOE_BF16 ? 2 : 4;
  const int64_t G = group_of(c);
  if ((int64_t)c->E * (G == 1 ? ce_pad : ce_pad + 64) >= (int64_t(1) << 31) ||
      G * (ce_pad + 64) * dm * es >= (int64_t(1) << 31) ||
      (int64_t)c->d_model * c->d_ff * es >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED,
                "round-buffer rows, their bytes per group and d*f*elem must be < 2^31");
  return MOE_OK;
}

void layout_of(const moe_config_t* c, moe_workspace_layout_t* L) {
  const size_t TK = (size_t)c->T * c->k;
  const size_t E = (size_t)c->E;
  const size_t ce = (size_t)eff_capacity(c);
  const size_t es = c->dtype == MOE_BF16 ? 2 : 4;
  const moe::Shape s = shape_of(c);
  (void)ce;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  L->idx = take(TK * 4);
  L->weight = take(TK * 4);
  // R sits right after the E counts, so one read returns both
  L->counts = take((E + 1) * 4);
  L->n_rounds = L->counts + E * 4;
  L->offsets = take((E + 1) * 4);
  L->perm = take(TK * 4);
  L->pos = take(TK * 4);
  L->round_of = take(TK * 4);
  L->row_of = take(TK * 4);
  L->rounds = take((size_t)moe::round_table_ints(s) * 4);
  L->scratch = take((size_t)moe::plan_scratch_ints(s) * 4);
  const size_t sets = (size_t)sets_of(c);
  L->h = take(sets * (size_t)s.buf_rows() * (size_t)c->d_ff * es);
  L->z = take(TK * (size_t)c->d_model * es);
  // last, so that callers that never dispatch into it (the forward when
  // its gate/up launches gather from x, and the backward) can leave it out
  L->xr = take(sets * (size_t)s.buf_rows() * (size_t)c->d_model * es);
  L->total = off;
}

// Bytes moe_forward and moe_backward need: everything before xr when the
// forward's gate/up launches gather their rows from x, else all of it.
size_t forward_bytes(const moe_config_t* c, const moe_workspace_layout_t& L) {
  return moe::gather_fits(shape_of(c)) ? L.xr : L.total;
}

struct Bound {
  moe::Shape s;
  moe_workspace_layout_t L;
  char* ws;
  moe::PlanBuffers pb;
  int sets;  // round-buffer sets
  // round r's set of the round buffers
  char* xr(int r) const {
    return ws + L.xr + (size_t)(r % sets) * (size_t)s.buf_rows() * s.d * (s.bf16 ? 2 : 4);
  }
  char* h(int r) const {
    return ws + L.h + (size_t)(r % sets) * (size_t)s.buf_rows() * s.f * (s.bf16 ? 2 : 4);
  }
};

// forward: the call is moe_forward, moe_forward_static or moe_backward,
// which need only forward_bytes of the workspace.
moe_status_t bind(const moe_config_t* c, void* ws, size_t ws_bytes, Bound* b,
                  bool forward = false) {
  moe_status_t st = check_cfg(c);
  if (st != MOE_OK) return st;
  if (!ws) return fail(MOE_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (!aligned16(ws))
    return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  layout_of(c, &b->L);
  if (ws_bytes < (forward ? forward_bytes(c, b->L) : b->L.total))
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "workspace too small");
  b->s = shape_of(c);
  b->sets = sets_of(c);
  b->ws = static_cast<char*>(ws);
  char* w = b->ws;
  const moe_workspace_layout_t& L = b->L;
  b->pb = moe::PlanBuffers{
      reinterpret_cast<int32_t*>(w + L.idx),      reinterpret_cast<float*>(w + L.weight),
      reinterpret_cast<int32_t*>(w + L.counts),   reinterpret_cast<int32_t*>(w + L.offsets),
      reinterpret_cast<int32_t*>(w + L.n_rounds), reinterpret_cast<int32_t*>(w + L.perm),
      reinterpret_cast<int32_t*>(w + L.pos),      reinterpret_cast<int32_t*>(w + L.round_of),
      reinterpret_cast<int32_t*>(w + L.row_of),   reinterpret_cast<int32_t*>(w + L.scratch),
      reinterpret_cast<int32_t*>(w + L.rounds)};
  return MOE_OK;
}

moe_status_t check_ptr(const void* p, const char* name) {
  if (!p) return fail(MOE_ERR_INVALID_ARGUMENT, "is NULL", name);
  if (!aligned16(p))
    return fail(MOE_ERR_INVALID_ARGUMENT, "must be 16-byte aligned", name);
  return MOE_OK;
}

moe_status_t check_round(const Bound& b, int32_t round, int32_t n_rounds = 1) {
  const int64_t max_rounds = (b.s.T + b.s.ce - 1) / b.s.ce;
  if (round < 0 || round >= max_rounds)
    return fail(MOE_ERR_INVALID_ARGUMENT, "round out of range [0, ceil(T/C'))");
  if (n_rounds < 1 || (int64_t)round + n_rounds > max_rounds)
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "n_rounds must be >= 1 with round + n_rounds <= ceil(T/C')");
  return MOE_OK;
}

// Compute units of the current device, cached per device id.
std::atomic<int> g_cus[64];

moe_status_t num_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev >= 0 && dev < 64) {
    const int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v > 0) {
      *out = v;
      return MOE_OK;
    }
  }
  int n = 0;
  e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  if (n < 1) n = 1;
  if (dev >= 0 && dev < 64) g_cus[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return MOE_OK;
}

// The forward's and backward's read of the plan: a small pinned host buffer
// that receives the counts and R, a side stream (default priority) that
// copies them, and events: "planned" on the caller's stream behind the
// plan, "done" on the side stream behind the copy, "joined" behind the side
// stream's rounds. moe_forward queues round 0's dispatch on the caller's
// stream while the side stream copies, so neither the copy nor the host's
// wake-up delays the GPU. The sets live in a pool per device: a call takes
// one for its duration and returns it, so there are never more sets than
// calls that were in flight at once on that device, whatever the number of
// calling threads; they are kept until the process ends. A returned set may
// still have the previous call's side-stream rounds queued; the next call's
// work on it queues behind them.
struct PlanReadback {
  int32_t* host = nullptr;  // kMaxExperts + 1 int32, hipHostMalloc
  hipStream_t side = nullptr;
  hipEvent_t planned = nullptr;
  hipEvent_t done = nullptr;
  hipEvent_t joined = nullptr;  // the side stream's rounds are done
};

struct ReadbackPool {
  std::mutex mu;
  std::vector<PlanReadback*> idle;
};
ReadbackPool g_readback_pool[64];

moe_status_t make_readback(PlanReadback* r) {
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, (kMaxExperts + 1) * sizeof(int32_t), hipHostMallocDefault);
  if (e != hipSuccess) return hip_fail(e, "hipHostMalloc of the plan readback");
  r->host = static_cast<int32_t*>(h);
  e = hipStreamCreateWithFlags(&r->side, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags");
  hipEvent_t* evs[3] = {&r->planned, &r->done, &r->joined};
  for (hipEvent_t* ev : evs) {
    e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
  }
  return MOE_OK;
}

// A readback set of the current device for the duration of one call.
class ReadbackLease {
 public:
  ~ReadbackLease() {
    if (set_) {
      ReadbackPool& pool = g_readback_pool[dev_];
      std::lock_guard<std::mutex> lock(pool.mu);
      pool.idle.push_back(set_);
    }
  }
  moe_status_t acquire(PlanReadback** out) {
    hipError_t e = hipGetDevice(&dev_);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev_ < 0 || dev_ >= 64) return fail(MOE_ERR_UNSUPPORTED, "device id >= 64");
    ReadbackPool& pool = g_readback_pool[dev_];
    {
      std::lock_guard<std::mutex> lock(pool.mu);
      if (!pool.idle.empty()) {
        set_ = pool.idle.back();
        pool.idle.pop_back();
      }
    }
    if (!set_) {
      PlanReadback* r = new PlanReadback();
      moe_status_t st = make_readback(r);
      if (st != MOE_OK) {  // release what was made; the error text stays
        if (r->host) (void)hipHostFree(r->host);
        if (r->side) (void)hipStreamDestroy(r->side);
        if (r->planned) (void)hipEventDestroy(r->planned);
        if (r->done) (void)hipEventDestroy(r->done);
        if (r->joined) (void)hipEventDestroy(r->joined);
        delete r;
        return st;
      }
      set_ = r;
    }
    *out = set_;
    return MOE_OK;
  }

 private:
  int dev_ = 0;
  PlanReadback* set_ = nullptr;
};

#define MOE_HIP(call, where)                         \
  do {                                               \
    hipError_t _e = (call);                          \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

moe_status_t run_plan(const Bound& b, const float* logits, hipStream_t st) {
  MOE_HIP(moe::launch_route(b.s, logits, b.pb, st), "route launch");
  MOE_HIP(moe::launch_plan(b.s, b.pb, st), "plan launch");
  return MOE_OK;
}

// The E counts and R (adjacent in the workspace) to the host; waits.
moe_status_t read_plan(const Bound& b, int32_t* out, hipStream_t st) {
  MOE_HIP(hipMemcpyAsync(out, b.pb.counts, (b.s.E + 1) * sizeof(int32_t),
                         hipMemcpyDeviceToHost, st),
          "read of counts and R");
  MOE_HIP(hipStreamSynchronize(st), "stream sync");
  return MOE_OK;
}

// The grouped GEMMs of the rounds [r0, r0 + nr) (one launch batch; its
// buffer set is round r0's), with the rows of its nv pairs on the host.
moe_status_t run_ffn(const Bound& b, int r0, int nr, const void* wg, const void* wu,
                     const void* wd, const int32_t* pair_rows, int nv, int cus,
                     hipStream_t st, const void* x = nullptr) {
  MOE_HIP(moe::launch_gate_up(b.s, r0, nr, b.xr(r0), wg, wu, b.pb, pair_rows, nv,
                              b.h(r0), cus, st, x),
          "gate/up launch");
  MOE_HIP(moe::launch_down(b.s, r0, nr, b.h(r0), wd, b.pb, pair_rows, nv,
                           b.ws + b.L.z, cus, st),
          "down launch");
  return MOE_OK;
}

// The rows of the pairs of rounds [r0, r0 + nr) (experts with rows, round
// by round, in expert order) from host counts, in *pairs; NULL if counts is
// NULL. The rounds must lie in one launch batch of the forward (else
// MOE_ERR_INVALID_ARGUMENT): their pairs are then at most E.
moe_status_t pairs_from_counts(const moe::Shape& s, const int32_t* counts, int r0, int nr,
                               int32_t* pair_rows, const int32_t** pairs, int* nv) {
  *nv = 0;
  *pairs = nullptr;
  if (!counts) return MOE_OK;
  for (int e = 0; e < s.E; ++e)
    if (counts[e] < 0 || counts[e] > s.T)
      return fail(MOE_ERR_INVALID_ARGUMENT, "counts_host: a count is outside [0, T]");
  moe::BatchWalker walk(s, counts);
  moe::LaunchBatch lb;
  while (walk.next(&lb)) {
    if (r0 >= lb.r0 + lb.nr) continue;  // a later batch holds r0
    if (r0 + nr > lb.r0 + lb.nr)
      return fail(MOE_ERR_INVALID_ARGUMENT,
                  "rounds [round, round + n_rounds) are not in one launch batch");
    int64_t rem[kMaxExperts];
    int32_t rows[kMaxExperts];
    for (int e = 0; e < s.E; ++e) rem[e] = counts[e];
    for (int r = 0; r < r0 + nr; ++r) {
      moe::host_next_round(s, rem, rows);
      if (r >= r0) *nv += moe::round_pairs(s.E, rows, pair_rows + *nv);
    }
    break;
  }
  // (rounds past the counts' last round have no pairs)
  *pairs = pair_rows;
  return MOE_OK;
}

// Observed counts must be a plan's: every n_e in [0, T] and their sum T*k.
moe_status_t check_counts(const moe_config_t* c, const int32_t* counts,
                          int64_t n_steps) {
  if (!counts) return fail(MOE_ERR_INVALID_ARGUMENT, "counts is NULL");
  if (n_steps < 1) return fail(MOE_ERR_INVALID_ARGUMENT, "n_steps must be >= 1");
  for (int64_t s = 0; s < n_steps; ++s) {
    int64_t sum = 0;
    for (int e = 0; e < c->E; ++e) {
      const int64_t n = counts[s * c->E + e];
      if (n < 0 || n > c->T)
        return fail(MOE_ERR_INVALID_ARGUMENT, "a count is outside [0, T]");
      sum += n;
    }
    if (sum != c->T * (int64_t)c->k)
      return fail(MOE_ERR_INVALID_ARGUMENT, "counts of a step do not sum to T*k");
  }
  return MOE_OK;
}

// Rounds of the plan at capacity C for one step's counts: every round gives
// a group of G experts min(left, G*C') rows (C' = min(C, T)), so R is the
// largest ceil(N_g / (G*C')) over the groups' totals N_g.
int64_t rounds_at(const moe_config_t* c, const int32_t* n, int64_t C) {
  const int64_t ce = C < c->T ? C : c->T;
  const int64_t G = group_of(c);
  int64_t R = 0;
  for (int g0 = 0; g0 < c->E; g0 += (int)G) {
    int64_t N = 0;
    for (int e = g0; e < g0 + G; ++e) N += n[e];
    const int64_t r = (N + G * ce - 1) / (G * ce);
    R = r > R ? r : R;
  }
  return R;
}


void bwd_layout_of(const moe_config_t* c, moe_backward_layout_t* L) {
  const moe::Shape s = shape_of(c);
  const size_t rows = (size_t)s.buf_rows(), d = (size_t)s.d, f = (size_t)s.f;
  const size_t TK = (size_t)s.T * (size_t)s.k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  };
  // two sets of xr, dyr, hw and dgu (rounds r and r + 1 of a pair), one gu
  L->xr = take(2 * rows * d * 2);
  L->dyr = take(2 * rows * d * 2);
  L->gu = take(rows * 2 * f * 2);
  L->hw = take(2 * rows * f * 2);
  L->dgu = take(2 * rows * 2 * f * 2);
  L->dz = take(TK * d * 2);
  L->ones = take(TK * 4);
  L->total = off;
}

moe_status_t check_bwd_cfg(const moe_config_t* c) {
  moe_status_t st = check_cfg(c);
  if (st != MOE_OK) return st;
  if (c->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "the backward supports bf16 only");
  // the router gradient keeps the k dot products of a token in registers
  if (c->k > moe::kBackwardMaxK)
    return fail(MOE_ERR_UNSUPPORTED, "the backward supports k <= 8");
  const int64_t ce_pad = (eff_capacity(c) + 63) / 64 * 64;
  if ((int64_t)group_of(c) * (ce_pad + 64) * 2 * c->d_ff * 2 >= (int64_t(1) << 31) ||
      (int64_t)c->d_model * 2 * c->d_ff * 2 >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "G*(C'+64)*2*d_ff*2 and d*2*d_ff*2 must be < 2^31");
  return MOE_OK;
}


// Workspace of moe_forward_static: one static device array, which every GPU
// the library runs on holds, at its own address, until the process ends.
// Host code never uses the array's name for its memory (on the host the name
// is only a stand-in): it uses the device address hipGetSymbolAddress returns
// for the current device, fetched once per device.
static __device__ __align__(256) char scratch[MOE_STATIC_WORKSPACE_BYTES];

std::mutex g_scratch_mu;
char* g_scratch_ptr[64];

moe_status_t static_workspace(char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(MOE_ERR_UNSUPPORTED, "device id >= 64");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static workspace");
    if (!ptr) return fail(MOE_ERR_HIP, "hipGetSymbolAddress returned NULL");
    g_scratch_ptr[dev] = static_cast<char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// The grouped GEMM launches of a stage call over rounds [round, round +
// n_rounds): the pairs' rows from the counts (if given) size the launch.
enum StageGemm { kStageBoth = 0, kStageGateUp = 1, kStageDown = 2 };

moe_status_t stage_gemm(const moe_config_t* cfg, int32_t round, int32_t n_rounds,
                        const void* w_gate, const void* w_up, const void* w_down,
                        const int32_t* counts_host, void* ws, size_t ws_bytes,
                        void* stream, StageGemm which, const void* x = nullptr) {
  Bound b;
  moe_status_t st = bind(cfg, ws, ws_bytes, &b);
  if (st != MOE_OK) return st;
  if (which != kStageDown) {
    if ((st = check_ptr(w_gate, "w_gate")) != MOE_OK) return st;
    if ((st = check_ptr(w_up, "w_up")) != MOE_OK) return st;
  }
  if (which != kStageGateUp && (st = check_ptr(w_down, "w_down")) != MOE_OK) return st;
  if ((st = check_round(b, round, n_rounds)) != MOE_OK) return st;
  int32_t rows[kMaxExperts];
  const int32_t* pr = nullptr;
  int nv = 0;
  if ((st = pairs_from_counts(b.s, counts_host, round, n_rounds, rows, &pr, &nv)) != MOE_OK)
    return st;
  int cus = 0;
  if ((st = num_cus(&cus)) != MOE_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (which != kStageDown)
    MOE_HIP(moe::launch_gate_up(b.s, round, n_rounds, b.xr(round), w_gate, w_up, b.pb, pr,
                                nv, b.h(round), cus, hs, x),
            "gate/up launch");
  if (which != kStageGateUp)
    MOE_HIP(moe::launch_down(b.s, round, n_rounds, b.h(round), w_down, b.pb, pr, nv,
                             b.ws + b.L.z, cus, hs),
            "down launch");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

int32_t moe_hip_runtime_version(void) {
  int v = 0;
  if (hipRuntimeGetVersion(&v) != hipSuccess) return -1;
  return v;
}

moe_status_t moe_check_config(const moe_config_t* cfg) { return check_cfg(cfg); }

moe_status_t moe_workspace_size(const moe_config_t* cfg, size_t* bytes) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  moe_workspace_layout_t L;
  layout_of(cfg, &L);
  *bytes = L.total;
  return MOE_OK;
}

moe_status_t moe_forward_workspace_size(const moe_config_t* cfg, size_t* bytes) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  moe_workspace_layout_t L;
  layout_of(cfg, &L);
  *bytes = forward_bytes(cfg, L);
  return MOE_OK;
}

moe_status_t moe_capacity_curve(const moe_config_t* cfg, const int32_t* counts,
                                int64_t n_steps, const int64_t* capacities,
                                int32_t n_capacities, int32_t* rounds,
                                size_t* ws_bytes) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_counts(cfg, counts, n_steps)) != MOE_OK) return st;
  if (!capacities || !rounds || !ws_bytes || n_capacities < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "capacity list or outputs missing");
  for (int32_t i = 0; i < n_capacities; ++i) {
    moe_config_t c = *cfg;
    c.C = capacities[i];
    if ((st = check_cfg(&c)) != MOE_OK) return st;
  }
  for (int32_t i = 0; i < n_capacities; ++i) {
    moe_config_t c = *cfg;
    c.C = capacities[i];
    moe_workspace_layout_t L;
    layout_of(&c, &L);
    ws_bytes[i] = L.total;
    for (int64_t s = 0; s < n_steps; ++s)
      rounds[i * n_steps + s] = (int32_t)rounds_at(&c, counts + s * cfg->E, c.C);
  }
  return MOE_OK;
}

moe_status_t moe_capacity_for_rounds(const moe_config_t* cfg, const int32_t* counts,
                                     int64_t n_steps, int32_t target_rounds,
                                     double quantile, int64_t* capacity) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_counts(cfg, counts, n_steps)) != MOE_OK) return st;
  if (target_rounds < 1 || !capacity || !(quantile > 0.0 && quantile <= 1.0))
    return fail(MOE_ERR_INVALID_ARGUMENT,
                "target_rounds >= 1, quantile in (0, 1] and capacity required");
  // per step: the smallest C with R <= target is ceil(max_g N_g / (G*target))
  // (R falls as C grows, and C = T always gives one round)
  const int64_t G = group_of(cfg);
  std::vector<int64_t> need((size_t)n_steps);
  for (int64_t s = 0; s < n_steps; ++s) {
    const int32_t* n = counts + s * cfg->E;
    int64_t top = 0;
    for (int g0 = 0; g0 < cfg->E; g0 += (int)G) {
      int64_t N = 0;
      for (int e = g0; e < g0 + G; ++e) N += n[e];
      top = N > top ? N : top;
    }
    int64_t C = (top + G * target_rounds - 1) / (G * target_rounds);
    C = C < 1 ? 1 : (C > cfg->T ? cfg->T : C);
    need[(size_t)s] = C;
  }
  std::sort(need.begin(), need.end());
  // the ceil(quantile * n_steps)-th smallest: at least that share of the
  // observed steps fits in target_rounds rounds
  int64_t rank = (int64_t)std::ceil(quantile * (double)n_steps);
  rank = rank < 1 ? 1 : (rank > n_steps ? n_steps : rank);
  *capacity = need[(size_t)(rank - 1)];
  return MOE_OK;
}

moe_status_t moe_workspace_layout(const moe_config_t* cfg,
                                  moe_workspace_layout_t* out) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!out) return fail(MOE_ERR_INVALID_ARGUMENT, "out is NULL");
  layout_of(cfg, out);
  return MOE_OK;
}

moe_status_t moe_plan(const moe_config_t* cfg, const float* logits, void* ws,
                      size_t ws_bytes, int32_t* plan_host, void* stream) {
  Bound b;
  moe_status_t st = bind(cfg, ws, ws_bytes, &b);
  if (st != MOE_OK) return st;
  if ((st = check_ptr(logits, "logits")) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = run_plan(b, logits, s)) != MOE_OK) return st;
  if (plan_host) return read_plan(b, plan_host, s);
  return MOE_OK;
}

moe_status_t moe_launch_batches(const moe_config_t* cfg, const int32_t* counts_host,
                                int32_t max_batches, int32_t* first_round,
                                int32_t* n_rounds, int32_t* n_batches) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_counts(cfg, counts_host, 1)) != MOE_OK) return st;
  if (!first_round || !n_rounds || !n_batches || max_batches < 1)
    return fail(MOE_ERR_INVALID_ARGUMENT, "outputs missing or max_batches < 1");
  const moe::Shape s = shape_of(cfg);
  moe::BatchWalker walk(s, counts_host);
  moe::LaunchBatch lb;
  int32_t n = 0;
  while (walk.next(&lb)) {
    if (n == max_batches)
      return fail(MOE_ERR_INVALID_ARGUMENT, "more batches than max_batches");
    first_round[n] = lb.r0;
    n_rounds[n] = lb.nr;
    ++n;
  }
  *n_batches = n;
  return MOE_OK;
}

moe_status_t moe_dispatch(const moe_config_t* cfg, int32_t round, int32_t n_rounds,
                          const void* x, void* ws, size_t ws_bytes, void* stream) {
  Bound b;
  moe_status_t st = bind(cfg, ws, ws_bytes, &b);
  if (st != MOE_OK) return st;
  if ((st = check_ptr(x, "x")) != MOE_OK) return st;
  if ((st = check_round(b, round, n_rounds)) != MOE_OK) return st;
  int cus = 0;
  if ((st = num_cus(&cus)) != MOE_OK) return st;
  MOE_HIP(moe::launch_dispatch(b.s, round, n_rounds, x, b.pb, b.xr(round), cus,
                               static_cast<hipStream_t>(stream)),
          "dispatch launch");
  return MOE_OK;
}

moe_status_t moe_expert_ffn(const moe_config_t* cfg, int32_t round, int32_t n_rounds,
                            const void* w_gate, const void* w_up,
                            const void* w_down, const int32_t* counts_host,
                            void* ws, size_t ws_bytes, void* stream) {
  return stage_gemm(cfg, round, n_rounds, w_gate, w_up, w_down, counts_host, ws,
                    ws_bytes, stream, kStageBoth);
}

moe_status_t moe_expert_gate_up(const moe_config_t* cfg, int32_t round, int32_t n_rounds,
                                const void* w_gate, const void* w_up,
                                const int32_t* counts_host, void* ws,
                                size_t ws_bytes, void* stream) {
  return stage_gemm(cfg, round, n_rounds, w_gate, w_up, nullptr, counts_host, ws,
                    ws_bytes, stream, kStageGateUp);
}

moe_status_t moe_expert_down(const moe_config_t* cfg, int32_t round, int32_t n_rounds,
                             const void* w_down, const int32_t* counts_host,
                             void* ws, size_t ws_bytes, void* stream) {
  return stage_gemm(cfg, round, n_rounds, nullptr, nullptr, w_down, counts_host, ws,
                    ws_bytes, stream, kStageDown);
}

moe_status_t moe_dispatch_gate_up(const moe_config_t* cfg, int32_t round,
                                  int32_t n_rounds, const void* x, const void* w_gate,
                                  const void* w_up, const int32_t* counts_host,
                                  void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_ptr(x, "x")) != MOE_OK) return st;
  if (!moe::gather_fits(shape_of(cfg)))
    return fail(MOE_ERR_UNSUPPORTED,
                "x holds more than 2^30 bytes: dispatch with moe_dispatch and run "
                "moe_expert_gate_up");
  return stage_gemm(cfg, round, n_rounds, w_gate, w_up, nullptr, counts_host, ws,
                    ws_bytes, stream, kStageGateUp, x);
}

moe_status_t moe_pack_weights(const moe_config_t* cfg, const void* w_gate,
                              const void* w_up, const void* w_down,
                              void* out_gate, void* out_up, void* out_down,
                              void* stream) {
  if (!cfg) return fail(MOE_ERR_INVALID_ARGUMENT, "config is NULL");
  moe_config_t c = *cfg;
  c.weight_layout = MOE_WEIGHTS_ROW_MAJOR;
  moe_status_t st = check_cfg(&c);
  if (st != MOE_OK) return st;
  const void* in[3] = {w_gate, w_up, w_down};
  void* out[3] = {out_gate, out_up, out_down};
  const char* names[6] = {"w_gate", "w_up", "w_down", "out_gate", "out_up", "out_down"};
  for (int i = 0; i < 3; ++i) {
    if ((st = check_ptr(in[i], names[i])) != MOE_OK) return st;
    if ((st = check_ptr(out[i], names[3 + i])) != MOE_OK) return st;
  }
  int cus = 0;
  if ((st = num_cus(&cus)) != MOE_OK) return st;
  const moe::Shape s = shape_of(&c);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  MOE_HIP(moe::launch_pack_weights(s, w_gate, out_gate, c.d_ff, c.d_model, cus, hs),
          "pack launch");
  MOE_HIP(moe::launch_pack_weights(s, w_up, out_up, c.d_ff, c.d_model, cus, hs),
          "pack launch");
  MOE_HIP(moe::launch_pack_weights(s, w_down, out_down, c.d_model, c.d_ff, cus, hs),
          "pack launch");
  return MOE_OK;
}

moe_status_t moe_backward_workspace_size(const moe_config_t* cfg, size_t* bytes) {
  moe_status_t st = check_bwd_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARGUMENT, "bytes is NULL");
  moe_backward_layout_t L;
  bwd_layout_of(cfg, &L);
  *bytes = L.total;
  return MOE_OK;
}

moe_status_t moe_backward_layout(const moe_config_t* cfg, moe_backward_layout_t* out) {
  moe_status_t st = check_bwd_cfg(cfg);
  if (st != MOE_OK) return st;
  if (!out) return fail(MOE_ERR_INVALID_ARGUMENT, "out is NULL");
  bwd_layout_of(cfg, out);
  return MOE_OK;
}

moe_status_t moe_backward(const moe_config_t* cfg, const void* x, const void* w_gate,
                          const void* w_up, const void* w_down, const void* dy, void* dx,
                          float* dlogits, float* dw_gate, float* dw_up, float* dw_down,
                          const void* ws, size_t ws_bytes, void* bws, size_t bws_bytes,
                          void* stream) {
  moe_status_t st = check_bwd_cfg(cfg);
  if (st != MOE_OK) return st;
  Bound b;
  if ((st = bind(cfg, const_cast<void*>(ws), ws_bytes, &b, true)) != MOE_OK) return st;
  const void* ptrs[] = {x, w_gate, w_up, w_down, dy, dx, dlogits,
                        dw_gate, dw_up, dw_down, bws};
  const char* names[] = {"x", "w_gate", "w_up", "w_down", "dy", "dx",
                         "dlogits", "dw_gate", "dw_up", "dw_down", "bws"};
  for (int i = 0; i < 11; ++i)
    if ((st = check_ptr(ptrs[i], names[i])) != MOE_OK) return st;
  moe_backward_layout_t L;
  bwd_layout_of(cfg, &L);
  if (bws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "backward workspace too small");
  char* w = static_cast<char*>(bws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cus = 0;
  if ((st = num_cus(&cus)) != MOE_OK) return st;
  // the forward's counts and R, read once (as in moe_forward)
  ReadbackLease lease;
  PlanReadback* rb = nullptr;
  if ((st = lease.acquire(&rb)) != MOE_OK) return st;
  MOE_HIP(hipEventRecord(rb->planned, s), "hipEventRecord");
  MOE_HIP(hipStreamWaitEvent(rb->side, rb->planned, 0), "hipStreamWaitEvent");
  MOE_HIP(hipMemcpyAsync(rb->host, b.pb.counts, (b.s.E + 1) * sizeof(int32_t),
                         hipMemcpyDeviceToHost, rb->side),
          "read of counts and R");
  MOE_HIP(hipEventRecord(rb->done, rb->side), "hipEventRecord");
  // independent of the rounds: the router gradient and the combine weights
  MOE_HIP(moe::launch_router_backward(b.s, b.ws + b.L.z, dy, b.pb, dlogits, cus, s),
          "router backward launch");
  float* ones = reinterpret_cast<float*>(w + L.ones);
  MOE_HIP(moe::launch_fill(ones, b.s.T * (int64_t)b.s.k, 1.0f, cus, s), "fill launch");
  const int d = b.s.d, f = b.s.f;
  const size_t set = (size_t)b.s.buf_rows() * 2;  // bytes per feature of a set
  char* xr[2] = {w + L.xr, w + L.xr + set * d};
  char* dyr[2] = {w + L.dyr, w + L.dyr + set * d};
  char* hw[2] = {w + L.hw, w + L.hw + set * f};
  char* dgu[2] = {w + L.dgu, w + L.dgu + set * 2 * f};
  char *gu = w + L.gu, *dz = w + L.dz;
  // Round 0's gathers and its recompute and dgrad GEMMs need nothing from
  // the host (as in moe_forward, where a full round 0 fills the chip with
  // 256 x 256 tiles): queued before the wait for the counts.
  const bool early = (int64_t)b.s.E * ((b.s.ce + 255) / 256) * ((b.s.f + 127) / 128) >= cus;
  auto round_work = [&](int rr, int q, const int32_t* prow, int nv) -> moe_status_t {
    MOE_HIP(moe::launch_dispatch(b.s, rr, 1, x, b.pb, xr[q], cus, s), "dispatch launch");
    MOE_HIP(moe::launch_dispatch(b.s, rr, 1, dy, b.pb, dyr[q], cus, s), "dispatch launch");
    MOE_HIP(moe::launch_recompute(b.s, rr, xr[q], w_gate, w_up, b.pb, prow, nv, gu, hw[q],
                                  cus, s),
            "recompute launch");
    MOE_HIP(moe::launch_dgate(b.s, rr, dyr[q], w_down, b.pb, prow, nv, gu, dgu[q], cus, s),
            "dgate launch");
    MOE_HIP(moe::launch_dx(b.s, rr, dgu[q], w_gate, w_up, b.pb, prow, nv, dz, cus, s),
            "dx launch");
    return MOE_OK;
  };
  if (early && (st = round_work(0, 0, nullptr, 0)) != MOE_OK) return st;
  MOE_HIP(hipEventSynchronize(rb->done), "wait for the plan");
  int32_t counts_r[kMaxExperts + 1];
  std::memcpy(counts_r, rb->host, (b.s.E + 1) * sizeof(int32_t));
  const int32_t R = counts_r[b.s.E];
  const int64_t max_rounds = (b.s.T + b.s.ce - 1) / b.s.ce;
  if (R < 1 || R > max_rounds)
    return fail(MOE_ERR_HIP, "device plan reported an impossible round count");
  int64_t rem[kMaxExperts];
  for (int e = 0; e < b.s.E; ++e) rem[e] = counts_r[e];
  int32_t rows[2][kMaxExperts];
  int32_t prow[kMaxExperts];
  // rounds in pairs: each round's gathers, recompute and dgrad GEMMs into
  // its set, then one weight-gradient contraction over both rounds
  for (int r = 0; r < R; r += 2) {
    const int nr = R - r >= 2 ? 2 : 1;
    for (int q = 0; q < nr; ++q) {
      const int rr = r + q;
      moe::host_next_round(b.s, rem, rows[q]);
      if (early && rr == 0) continue;  // queued before the wait
      const int nv = moe::round_pairs(b.s.E, rows[q], prow);
      if ((st = round_work(rr, q, prow, nv)) != MOE_OK) return st;
    }
    MOE_HIP(moe::launch_wgrad(b.s, r, nr, dyr[0], hw[0], dyr[1], hw[1], d, d, f, dw_down,
                              nullptr, b.pb, rows[0], rows[1], cus, s),
            "wgrad launch");
    MOE_HIP(moe::launch_wgrad(b.s, r, nr, dgu[0], xr[0], dgu[1], xr[1], 2 * f, f, d,
                              dw_gate, dw_up, b.pb, rows[0], rows[1], cus, s),
            "wgrad launch");
  }
  MOE_HIP(moe::launch_combine(b.s, dz, ones, b.pb.pos, dx, cus, s), "combine launch");
  return MOE_OK;
}

moe_status_t moe_combine(const moe_config_t* cfg, const void* ws,
                         size_t ws_bytes, void* y, void* stream) {
  Bound b;
  moe_status_t st = bind(cfg, const_cast<void*>(ws), ws_bytes, &b);
  if (st != MOE_OK) return st;
  if ((st = check_ptr(y, "y")) != MOE_OK) return st;
  int cus = 0;
  if ((st = num_cus(&cus)) != MOE_OK) return st;
  MOE_HIP(moe::launch_combine(b.s, b.ws + b.L.z, b.pb.weight, b.pb.pos, y, cus,
                              static_cast<hipStream_t>(stream)),
          "combine launch");
  return MOE_OK;
}

moe_status_t moe_forward(const moe_config_t* cfg, const float* logits,
                         const void* x, const void* w_gate, const void* w_up,
                         const void* w_down, void* y, void* ws, size_t ws_bytes,
                         void* stream) {
  Bound b;
  moe_status_t st = bind(cfg, ws, ws_bytes, &b, true);
  if (st != MOE_OK) return st;
  if ((st = check_ptr(logits, "logits")) != MOE_OK) return st;
  if ((st = check_ptr(x, "x")) != MOE_OK) return st;
  if ((st = check_ptr(w_gate, "w_gate")) != MOE_OK) return st;
  if ((st = check_ptr(w_up, "w_up")) != MOE_OK) return st;
  if ((st = check_ptr(w_down, "w_down")) != MOE_OK) return st;
  if ((st = check_ptr(y, "y")) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cus = 0;
  if ((st = num_cus(&cus)) != MOE_OK) return st;
  if ((st = run_plan(b, logits, s)) != MOE_OK) return st;
  // One read of the E per-expert counts followed by R into pinned memory,
  // on the side stream behind the plan. Round 0 always exists, and neither
  // its dispatch nor its grouped GEMMs need anything from the host (they
  // read their pairs from the plan's tables; without host counts the GEMMs
  // take the 256 x 256 tile and one workgroup per CU, the shape a full
  // round gets, and every shape gives the same results), so they are queued
  // on the caller's stream first: the GPU gathers and computes round 0
  // while the counts travel and the host waits for them.
  ReadbackLease lease;
  PlanReadback* rb = nullptr;
  if ((st = lease.acquire(&rb)) != MOE_OK) return st;
  MOE_HIP(hipEventRecord(rb->planned, s), "hipEventRecord");
  // The gate/up GEMM gathers each slot's token row from x through the plan
  // (where x has at most 2^30 bytes), so no round is dispatched into xr;
  // otherwise each launch batch's dispatch comes first.
  const void* gx = moe::gather_fits(b.s) ? x : nullptr;
  if (!gx)
    MOE_HIP(moe::launch_dispatch(b.s, 0, 1, x, b.pb, b.xr(0), cus, s), "dispatch launch");
  // (only where a full round 0 fills the chip with 256 x 256 tiles; a small
  // layer's round 0 keeps the shape its counts choose)
  const bool early = (int64_t)b.s.E * ((b.s.ce + 255) / 256) * ((b.s.f + 127) / 128) >= cus;
  if (early &&
      (st = run_ffn(b, 0, 1, w_gate, w_up, w_down, nullptr, 0, cus, s, gx)) != MOE_OK)
    return st;
  MOE_HIP(hipStreamWaitEvent(rb->side, rb->planned, 0), "hipStreamWaitEvent");
  MOE_HIP(hipMemcpyAsync(rb->host, b.pb.counts, (b.s.E + 1) * sizeof(int32_t),
                         hipMemcpyDeviceToHost, rb->side),
          "read of counts and R");
  MOE_HIP(hipEventRecord(rb->done, rb->side), "hipEventRecord");
  // With two sets of round buffers the odd rounds run on the side stream
  // (set 1) and the even rounds on the caller's (set 0): consecutive rounds
  // use different buffers, so the dispatch of round r + 1 and the expert
  // compute of round r overlap, and each stream keeps its own rounds in
  // order. Round 1's dispatch is queued before the wait as well; with R = 1
  // it finds no assignment of round 1 and moves nothing.
  const int64_t max_rounds = (b.s.T + b.s.ce - 1) / b.s.ce;
  const bool two = b.sets == 2 && max_rounds >= 2;
  if (two && !gx)
    MOE_HIP(moe::launch_dispatch(b.s, 1, 1, x, b.pb, b.xr(1), cus, rb->side),
            "dispatch launch");
  MOE_HIP(hipEventSynchronize(rb->done), "wait for the plan");
  int32_t counts_r[kMaxExperts + 1];
  std::memcpy(counts_r, rb->host, (b.s.E + 1) * sizeof(int32_t));
  const int32_t R = counts_r[b.s.E];
  if (R < 1 || R > max_rounds)
    return fail(MOE_ERR_HIP, "device plan reported an impossible round count");
  // The launch batches (one round each with two sets): the rest of each
  // batch's dispatch (rounds not queued before the wait), then one launch
  // of each grouped GEMM over the batch's pairs not yet computed. If round
  // 0's GEMMs ran above and the first batch holds later rounds as well,
  // those are one launch over rounds 1 .. of that batch (its pairs after
  // round 0's).
  const int queued = two ? 2 : 1;
  int round0_pairs = 0;
  {
    int64_t rem[kMaxExperts];
    int32_t rows0[kMaxExperts];
    for (int e = 0; e < b.s.E; ++e) rem[e] = counts_r[e];
    moe::host_next_round(b.s, rem, rows0);
    for (int e = 0; e < b.s.E; ++e) round0_pairs += rows0[e] > 0;
  }
  moe::BatchWalker walk(b.s, counts_r);
  moe::LaunchBatch lb;
  while (walk.next(&lb)) {
    hipStream_t sr = two && (lb.r0 & 1) ? rb->side : s;
    const int d0 = lb.r0 < queued ? queued : lb.r0;
    if (!gx && lb.r0 + lb.nr > d0)
      MOE_HIP(moe::launch_dispatch(b.s, d0, lb.r0 + lb.nr - d0, x, b.pb, b.xr(lb.r0),
                                   cus, sr),
              "dispatch launch");
    const int skip = early && lb.r0 == 0 ? 1 : 0;  // round 0 is computed
    if (lb.nr > skip &&
        (st = run_ffn(b, lb.r0 + skip, lb.nr - skip, w_gate, w_up, w_down,
                      lb.rows + (skip ? round0_pairs : 0), lb.nv - (skip ? round0_pairs : 0),
                      cus, sr, gx)) != MOE_OK)
      return st;
  }
  if (two) {  // the combine reads z rows of every round
    MOE_HIP(hipEventRecord(rb->joined, rb->side), "hipEventRecord");
    MOE_HIP(hipStreamWaitEvent(s, rb->joined, 0), "hipStreamWaitEvent");
  }
  MOE_HIP(moe::launch_combine(b.s, b.ws + b.L.z, b.pb.weight, b.pb.pos, y, cus, s),
          "combine launch");
  return MOE_OK;
}

moe_status_t moe_forward_static(const moe_config_t* cfg, const float* logits,
                                const void* x, const void* w_gate, const void* w_up,
                                const void* w_down, void* y, void* stream) {
  moe_status_t st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  moe_workspace_layout_t L;
  layout_of(cfg, &L);
  const size_t need = forward_bytes(cfg, L);
  if (need > (size_t)MOE_STATIC_WORKSPACE_BYTES) {
    std::snprintf(g_err, sizeof g_err,
                  "the config needs a workspace of %zu bytes; the static workspace "
                  "holds %zu",
                  need, (size_t)MOE_STATIC_WORKSPACE_BYTES);
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  }
  const void* ptrs[] = {logits, x, w_gate, w_up, w_down, y};
  const char* names[] = {"logits", "x", "w_gate", "w_up", "w_down", "y"};
  for (int i = 0; i < 6; ++i)
    if ((st = check_ptr(ptrs[i], names[i])) != MOE_OK) return st;
  char* ws = nullptr;
  if ((st = static_workspace(&ws)) != MOE_OK) return st;
  Bound b;
  if ((st = bind(cfg, ws, (size_t)MOE_STATIC_WORKSPACE_BYTES, &b, true)) != MOE_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int cus = 0;
  if ((st = num_cus(&cus)) != MOE_OK) return st;
  // Nothing in the workspace has to start at zero: the plan writes every
  // entry it later reads, and the rows of a round buffer past an expert's
  // rows only feed outputs that are never stored.
  if ((st = run_plan(b, logits, s)) != MOE_OK) return st;
  // gate/up gathers from x as in moe_forward, else round 0 is dispatched
  const void* gx = moe::gather_fits(b.s) ? x : nullptr;
  if (!gx)
    MOE_HIP(moe::launch_dispatch(b.s, 0, 1, x, b.pb, b.xr(0), cus, s), "dispatch launch");
  // counts and R into host memory of this frame, then one wait
  int32_t counts_r[kMaxExperts + 1];
  MOE_HIP(hipMemcpyAsync(counts_r, b.pb.counts, (b.s.E + 1) * sizeof(int32_t),
                         hipMemcpyDeviceToHost, s),
          "read of counts and R");
  MOE_HIP(hipStreamSynchronize(s), "stream sync");
  const int32_t R = counts_r[b.s.E];
  const int64_t max_rounds = (b.s.T + b.s.ce - 1) / b.s.ce;
  if (R < 1 || R > max_rounds)
    return fail(MOE_ERR_HIP, "device plan reported an impossible round count");
  // every launch batch on the caller's stream, in order (as moe_forward;
  // with two sets one round per batch, round r in set r % S)
  moe::BatchWalker walk(b.s, counts_r);
  moe::LaunchBatch lb;
  while (walk.next(&lb)) {
    const int d0 = lb.r0 < 1 ? 1 : lb.r0;
    if (!gx && lb.r0 + lb.nr > d0)
      MOE_HIP(moe::launch_dispatch(b.s, d0, lb.r0 + lb.nr - d0, x, b.pb, b.xr(lb.r0),
                                   cus, s),
              "dispatch launch");
    if ((st = run_ffn(b, lb.r0, lb.nr, w_gate, w_up, w_down, lb.rows, lb.nv, cus, s,
                      gx)) != MOE_OK)
      return st;
  }
  MOE_HIP(moe::launch_combine(b.s, b.ws + b.L.z, b.pb.weight, b.pb.pos, y, cus, s),
          "combine launch");
  return MOE_OK;
}

}  // extern "C"
