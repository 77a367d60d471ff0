/*
 * moe_rounds.h -- C ABI of the multi-round dropless mixture-of-experts layer
 * (forward, backward and capacity helpers) on one AMD Instinct MI355X
 * (gfx950).
 *
 * The method (sources: "Frontier Pre-training at Microsoft AI (MAI-Base-2)",
 * section "Key claims", item on multi-round dropless MoE; "Microsoft AI's
 * MAI-Base-2 trained on 16K GPUs with Muon", section "Expert groups keep
 * memory fixed when tokens pile up"; "MAI-Base-2: Microsoft details its new
 * training infrastructure", section "Optimizations to prevent memory loss"):
 * routing assigns every token to a small number of experts; the experts then
 * work in one or more rounds of dispatch, compute and collect, and a round
 * holds at most C tokens per expert. Assignments beyond an expert's capacity
 * are deferred to a later round, so none is lost, and the device memory the
 * layer needs depends only on the shapes and C, never on how skewed the
 * routing is.
 *
 * Capacity groups (same sources: an overloaded expert first uses capacity
 * that other experts of its group leave unused, and only what still does
 * not fit waits for another round): experts e with the same e / G form a
 * group that owns G*C' slots per round. In every round each expert first
 * takes up to C' of its remaining assignments; the group's unused slots
 * then go to its overloaded experts in ascending expert order. G = 1 is a
 * strict per-expert capacity.
 *
 * Notation: T tokens, E experts, top-k routing, d = d_model, f = d_ff,
 * assignment id a = t*k + j (j-th choice of token t), n_e = assignments of
 * expert e, C' = min(C, T) (a capacity above T acts as T), G experts per
 * capacity group, m(r,e) = rows of expert e in round r (for G = 1,
 * clamp(n_e - r*C', 0, C')), R rounds (for G = 1, max_e ceil(n_e / C');
 * in general max over groups of ceil(sum of the group's n_e / (G*C'))).
 *
 * Layouts (row-major, contiguous, no padding):
 *   logits  float32 [T][E]            (always fp32)
 *   x, y    elem    [T][d]
 *   w_gate  elem    [E][f][d]         (out-features x in-features)
 *   w_up    elem    [E][f][d]
 *   w_down  elem    [E][d][f]
 * where elem is float32 (MOE_F32) or bfloat16 (MOE_BF16). With bf16 the
 * products run on the matrix cores with fp32 accumulation; the SwiGLU
 * activation is rounded to bf16 once (to nearest even), each expert output
 * row once, and y once after an fp32 weighted sum.
 *
 * Ownership: the caller allocates every buffer, including the workspace of
 * moe_workspace_size() bytes (moe_forward_workspace_size() bytes suffice for
 * moe_forward and moe_backward). The library allocates no device memory; its
 * only state is, per device, a pool of the small pinned host buffer, side
 * stream and events with which moe_forward and moe_backward read the
 * plan's counts (see moe_forward), and the static workspace of
 * moe_forward_static. All work is enqueued on the caller's
 * HIP stream (`stream` is a hipStream_t; NULL means the null stream). Calls
 * on one workspace must not overlap in time. Device pointers must be
 * 16-byte aligned and point to memory of the current device: the library
 * sees plain addresses and cannot tell a host pointer from a device one (a
 * host address reaching a kernel faults the GPU; the Python binding checks
 * that its tensor arguments live on the device).
 *
 * Errors: every call returns a moe_status_t and validates its arguments
 * before touching the GPU, so an argument error enqueues nothing. A failed
 * HIP call returns MOE_ERR_HIP and moe_last_error() gives its text (thread
 * local). Device data are not validated. A NaN logit ranks as -inf; a row
 * with NaN or infinite logits still gets k distinct experts in [0, E) (so
 * the plan and every buffer access stay in range), but which ones, and its
 * routing weights (NaN where the top logit is infinite), are unspecified.
 *
 * Limits of this version: 1 <= E <= 64, 1 <= k <= E, T >= 1, T*k < 2^31,
 * C >= 1, G divides E, d and f positive multiples of 64, and the
 * round-buffer rows (E*P for G = 1, E*(P+64) otherwise, P = C' rounded up
 * to 64), G*(P+64)*max(d, f) elements' bytes and d*f elements' bytes each
 * below 2^31 (MOE_ERR_UNSUPPORTED otherwise).
 */
#ifndef MOE_ROUNDS_H
#define MOE_ROUNDS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Layout of w_gate, w_up and w_down as the calls below read them:
 *   MOE_WEIGHTS_ROW_MAJOR  [E][out][in] row-major, as documented above;
 *   MOE_WEIGHTS_TILED      the tiled layout written by moe_pack_weights:
 *                          each expert's [out][in] matrix stored as 4 KiB
 *                          blocks of 64 rows x 64 bytes (see "Tiled layout").
 * The arithmetic and the results are identical; the tiled layout lets every
 * 64-row band of a K stage be fetched as one contiguous 4 KiB read. */
typedef enum { MOE_WEIGHTS_ROW_MAJOR = 0, MOE_WEIGHTS_TILED = 1 } moe_weight_layout_t;

typedef struct {
  int64_t T;             /* tokens */
  int32_t E;             /* experts */
  int32_t k;             /* experts per token */
  int32_t d_model;       /* d */
  int32_t d_ff;          /* f */
  int64_t C;             /* per-expert capacity of one round */
  int32_t dtype;         /* moe_dtype_t of x, weights and y */
  int32_t weight_layout; /* moe_weight_layout_t of the expert weights */
  int32_t group;         /* G: experts per capacity group (0 means 1) */
  int32_t round_buffers; /* S: sets of round buffers, 1 or 2 (0 means 1);
                            round r uses set r % S. With 2, moe_forward
                            overlaps consecutive rounds (see there) */
} moe_config_t;

/* Tiled layout. A matrix with R rows (R padded up to a multiple of 64) and
 * Kb = K * sizeof(elem) bytes per row (a multiple of 64) is a sequence of
 * 4096-byte blocks. Block b = (row / 64) * (Kb / 64) + byte / 64 holds rows
 * row - row % 64 .. +63 and bytes byte - byte % 64 .. +63 of each; inside it,
 * row r = row % 64 occupies bytes [64 r, 64 r + 64), and the 16-byte chunk
 * c = (byte % 64) / 16 of that row sits at position c ^ ((r / 4) % 4):
 *   offset(row, byte) = 4096 * b + 64 * r + 16 * (c ^ ((r >> 2) & 3))
 *                       + byte % 16.
 * Weights: expert e's matrix starts at element e * out * in of its array. */

/* Byte offsets of the internal buffers inside the workspace. Every offset is
 * a multiple of 256 except n_rounds, which directly follows the E counts
 * (counts + 4 E) so that one read returns both. Contents (all produced by the calls below):
 *   idx      int32 [T][k]    expert of assignment a (top-k, ties to the lower
 *                            index, ordered by descending logit)
 *   weight   float [T][k]    routing weight: softmax of the k chosen logits
 *   counts   int32 [E]       n_e
 *   offsets  int32 [E+1]     exclusive prefix sum of counts
 *   n_rounds int32 [1]       R
 *   perm     int32 [T*k]     assignment ids sorted by (expert, a) -- stable
 *   pos      int32 [T*k]     inverse of perm
 *   round_of int32 [T*k]     round of assignment a (for G = 1: i / C')
 *   row_of   int32 [T*k]     slot of a in its round: g*G*C' + (rows of the
 *                            lower experts of its group in that round) +
 *                            c (for G = 1: e*C' + i % C'), i = pos[a] -
 *                            offsets[e] its index in expert e's list, c
 *                            its index among e's entries of the round
 *   rounds   int32 [9][M][E] + [2][M], M = ceil(T/C'): per round r and
 *                            expert e, m(r,e); the index in e's list of
 *                            its first entry of round r; the rows of the
 *                            lower experts of e's group in round r; the
 *                            same with each expert's rows rounded up to
 *                            64; brow(r,e), the buffer row where e's
 *                            matrix of round r starts (see "Launch
 *                            batches"). Then the pair tables, indexed by
 *                            b*E + v: expert, rows, buffer row and first
 *                            row of z of pair v of launch batch b. Then
 *                            rbeg[M], rend[M]: the pair indices of round
 *                            r's first pair and one past its last.
 *                            Entries of rounds r >= R are unused.
 *   scratch  int32 [...]     plan-internal partial counts
 *   h        elem [S][E/G][Q][f] SwiGLU activations of the round (set r % S
 *                            for round r): Q = P
 *                            (G = 1) or G*(P+64) rows per group, P = C'
 *                            rounded up to a multiple of 64. In round r
 *                            expert e's rows start at row brow(r,e) of the
 *                            set, as an m(r,e) x f matrix in the tiled
 *                            layout (its slot c is row c; rows up to the
 *                            next multiple of 64 hold stale data)
 *   z        elem [T*k][d]   unweighted expert output of every assignment,
 *                            in expert-sorted order: row i holds the output
 *                            of assignment perm[i] (so assignment a's row
 *                            is pos[a])
 *   xr       elem [S][E/G][Q][d] round buffers of gathered token rows, same
 *                            layout as h with d columns (written by
 *                            moe_dispatch); laid out last
 * The offsets follow this order. The layout, and so the size, is a pure
 * function of the config.
 */
/* Launch batches. The forward does not need one dispatch and one launch of
 * each grouped GEMM per round: with G = 1 and one set of round buffers, a
 * round's experts with rows (its "pairs") fill only some of the E expert
 * regions of the round buffer, so consecutive rounds run together while
 * their pairs fit in the E regions (a per-execution schedule of the same
 * plan: rounds, slots and results are unchanged, memory stays the same
 * buffer). Rounds are taken in order; a round joins the current batch if
 * its pairs still fit, else it opens the next one. Pair v of a batch
 * (numbered round by round, experts ascending inside a round) uses region
 * v: its matrix starts at buffer row brow(r,e) = v * P. With G > 1 or two
 * sets of round buffers every round is a batch of its own and brow(r,e) is
 * the expert's place in its group's block, (e / G) * Q + (padded rows of
 * the group's lower experts). moe_launch_batches lists the batches from a
 * step's counts. */

typedef struct {
  size_t idx, weight, counts, offsets, n_rounds, perm, pos, round_of, row_of,
      rounds, scratch, xr, h, z;
  size_t total;
} moe_workspace_layout_t;

/* Human-readable name of a status code (static storage). */
const char *moe_status_string(moe_status_t status);

/* Text of the last MOE_ERR_HIP / validation failure on this thread. */
const char *moe_last_error(void);

/* HIP runtime version the library runs against (hipRuntimeGetVersion), or a
 * negative value if the query fails. Makes no other HIP call. */
int32_t moe_hip_runtime_version(void);

/* Validate a config (no pointers). Pure host function. */
moe_status_t moe_check_config(const moe_config_t *cfg);

/* Workspace bytes for a config: a pure host function, no HIP call. The size
 * depends on (T, E, k, d, f, C, dtype, G, S) only, never on routing -- the fixed
 * memory of the method ("Expert groups keep memory fixed when tokens pile
 * up"). */
moe_status_t moe_workspace_size(const moe_config_t *cfg, size_t *bytes);

/* Workspace bytes that moe_forward and moe_backward need (also a pure host
 * function of the config): the workspace up to the round buffer xr, which
 * is laid out last, when the forward's gate/up launches read their token
 * rows from x (x of at most 2^30 bytes, see moe_dispatch_gate_up), else
 * moe_workspace_size's. These two calls accept a workspace of this size
 * (its offsets are moe_workspace_layout's); every other call that takes a
 * workspace needs moe_workspace_size bytes. */
moe_status_t moe_forward_workspace_size(const moe_config_t *cfg, size_t *bytes);

/* Offsets of every internal buffer (pure host function). */
moe_status_t moe_workspace_layout(const moe_config_t *cfg,
                                  moe_workspace_layout_t *out);

/* Capacity tuning ("Microsoft AI's MAI-Base-2 trained on 16K GPUs with
 * Muon", section "Expert groups keep memory fixed when tokens pile up": a
 * larger capacity needs more memory and fewer rounds; "Frontier
 * Pre-training at Microsoft AI (MAI-Base-2)", section "Key claims": the
 * capacity is tunable). Pure host functions, no HIP call.
 *
 * counts: host, n_steps x E int32, row s the per-expert counts n_e of one
 * observed step (the first E values moe_plan stores in plan_host); every
 * n_e must lie in [0, T] and each row must sum to T*k, else
 * MOE_ERR_INVALID_ARGUMENT. The rounds a plan needs at capacity C follow
 * from the counts alone: a round gives each group of G experts min(left,
 * G*C') rows (C' = min(C, T)), so R = max over groups of ceil(N_g /
 * (G*C')) with N_g the group's total (for G = 1, max_e ceil(n_e / C')),
 * the same R moe_plan reports for that step.
 *
 * moe_capacity_curve: for each of the n_capacities values C_i (each must
 * give a valid config with the other fields of cfg), writes
 * rounds[i * n_steps + s] = R of step s at C_i and ws_bytes[i] = the
 * workspace size of cfg with C = C_i: the memory-against-rounds curve.
 *
 * moe_capacity_for_rounds: the smallest C such that at least a share
 * `quantile` (in (0, 1]) of the observed steps needs at most target_rounds
 * rounds (>= 1): per step the least such C is ceil(max_g N_g / (G *
 * target_rounds)), at most T; *capacity gets the ceil(quantile *
 * n_steps)-th smallest of these. quantile = 1 covers every observed step;
 * target_rounds = 1 gives the steady-state single round. */
moe_status_t moe_capacity_curve(const moe_config_t *cfg, const int32_t *counts,
                                int64_t n_steps, const int64_t *capacities,
                                int32_t n_capacities, int32_t *rounds,
                                size_t *ws_bytes);
moe_status_t moe_capacity_for_rounds(const moe_config_t *cfg,
                                     const int32_t *counts, int64_t n_steps,
                                     int32_t target_rounds, double quantile,
                                     int64_t *capacity);

/* Route and plan. Routing: every token is sent to a few experts ("Microsoft
 * AI's MAI-Base-2 trained on 16K GPUs with Muon", section "Expert groups
 * keep memory fixed when tokens pile up"), here its top-k by logit with the
 * softmax of the k chosen logits as weights. Plan: each expert's
 * assignments, in stable token order, are split into rounds of fixed
 * capacity, C' per expert, shared inside its group of G; what does not fit
 * waits for a later round and nothing is dropped ("Frontier Pre-training at
 * Microsoft AI (MAI-Base-2)", section "Key claims", item on multi-round
 * dropless MoE; same section of the page above). The plan stays on the
 * device: the later calls read it there. Reads logits [T][E]; writes idx, weight, counts, offsets,
 * perm, pos, round_of, row_of, rounds and n_rounds in the workspace. If plan_host is not NULL
 * (host memory, E + 1 int32) the call waits for the stream and stores the
 * E counts n_e followed by R there; otherwise it is asynchronous. */
moe_status_t moe_plan(const moe_config_t *cfg, const float *logits, void *ws,
                      size_t ws_bytes, int32_t *plan_host, void *stream);

/* The launch batches of a step (see "Launch batches") from its counts
 * (host, E int32 as moe_plan stores them; each in [0, T] and summing to
 * T*k): batch i covers rounds [first_round[i], first_round[i] +
 * n_rounds[i]). Writes at most max_batches entries and their number to
 * *n_batches (MOE_ERR_INVALID_ARGUMENT if there are more). Pure host
 * function, no HIP call. */
moe_status_t moe_launch_batches(const moe_config_t *cfg, const int32_t *counts_host,
                                int32_t max_batches, int32_t *first_round,
                                int32_t *n_rounds, int32_t *n_batches);

/* Dispatch of rounds r = round .. round + n_rounds - 1, the first of a
 * round's dispatch, compute and collect steps ("Frontier Pre-training at
 * Microsoft AI (MAI-Base-2)", section "Key claims", item on multi-round
 * dropless MoE: each round moves at most the fixed capacity of tokens to
 * every expert): for every expert e and slot c < m(r,e), copies
 * x[perm[offsets[e] + s + c] / k] (s = the index of e's first entry of
 * round r) into row c of the matrix of (r, e), at buffer row brow(r,e) of
 * set round % S (tiled layout). Other rows are left untouched. The rounds
 * must lie in one launch batch (n_rounds = 1 always does); rounds >= R move
 * nothing. 0 <= round, 1 <= n_rounds, round + n_rounds <= ceil(T / C').
 * Asynchronous. */
moe_status_t moe_dispatch(const moe_config_t *cfg, int32_t round,
                          int32_t n_rounds, const void *x, void *ws,
                          size_t ws_bytes, void *stream);

/* Expert compute and collect of rounds r = round .. round + n_rounds - 1
 * (one launch batch): for every pair (r, e) with m(r,e) > 0, h =
 * silu(xr_re . w_gate[e]^T) * (xr_re . w_up[e]^T) on the first m(r,e) rows
 * of the matrix of (r, e), then o = h . w_down[e]^T, and row c of o is
 * stored at z[offsets[e] + s + c], the row of assignment perm[offsets[e] +
 * s + c] (s as for moe_dispatch; the combine collects these rows back to
 * token order). Each product is one grouped GEMM launch over all the
 * pairs (one GEMM per expert group rather than per expert: "Frontier
 * Pre-training at Microsoft AI (MAI-Base-2)", section "Key claims",
 * summarizing the post's "Reducing per-expert overhead").
 * counts_host: NULL, or a host copy of the E counts n_e (the first E values
 * moe_plan stores in plan_host). With it the launch shape fits the pairs'
 * rows: the output tile (256 x 256, 256 x 128 or 128 x 64) with the least
 * estimated time, and no more workgroups than tiles (what moe_forward
 * does), and rounds that are not in one launch batch are refused
 * (MOE_ERR_INVALID_ARGUMENT); without it the 256 x 256 tile and one
 * workgroup per CU are used, and such rounds compute nothing. The results
 * are bit-identical either way. Rounds >= R compute nothing. 0 <= round,
 * 1 <= n_rounds, round + n_rounds <= ceil(T / C'). Asynchronous. */
moe_status_t moe_expert_ffn(const moe_config_t *cfg, int32_t round,
                            int32_t n_rounds, const void *w_gate,
                            const void *w_up, const void *w_down,
                            const int32_t *counts_host, void *ws,
                            size_t ws_bytes, void *stream);

/* The two halves of moe_expert_ffn, for callers that time or schedule them
 * separately: gate/up writes h for round r (first m(r,e) rows of each
 * expert's region), down reads h and writes the round's rows of z. Same
 * arguments, layouts and asynchrony as moe_expert_ffn. */
moe_status_t moe_expert_gate_up(const moe_config_t *cfg, int32_t round,
                                int32_t n_rounds, const void *w_gate,
                                const void *w_up, const int32_t *counts_host,
                                void *ws, size_t ws_bytes, void *stream);
moe_status_t moe_expert_down(const moe_config_t *cfg, int32_t round,
                             int32_t n_rounds, const void *w_down,
                             const int32_t *counts_host, void *ws,
                             size_t ws_bytes, void *stream);

/* Dispatch and gate/up of rounds round .. round + n_rounds - 1 in one
 * grouped GEMM launch: h exactly as moe_dispatch followed by
 * moe_expert_gate_up computes it (bit for bit), but each slot's token row is
 * read from x (row-major [T][d]) through the plan's permutation while the
 * GEMM fetches its operands, so the round buffer xr is neither written nor
 * read. This is the dispatch step of the rounds ("Frontier Pre-training at
 * Microsoft AI (MAI-Base-2)", section "Key claims": dispatch, compute,
 * collect) on one GPU, where the dispatch moves rows within one device
 * memory and a separate copy into xr would only add a write and a read of
 * every assignment's row; moe_forward takes this path. x must hold at most
 * 2^30 bytes (T * d * sizeof(elem)), else MOE_ERR_UNSUPPORTED (use
 * moe_dispatch and moe_expert_gate_up). Other arguments, checks and
 * asynchrony as moe_expert_gate_up. */
moe_status_t moe_dispatch_gate_up(const moe_config_t *cfg, int32_t round,
                                  int32_t n_rounds, const void *x,
                                  const void *w_gate, const void *w_up,
                                  const int32_t *counts_host, void *ws,
                                  size_t ws_bytes, void *stream);

/* Repack expert weights from the row-major layout into the tiled layout
 * (MOE_WEIGHTS_TILED): gate and up are [E][f][d], down is [E][d][f]; each
 * output array has the size of its input. cfg->weight_layout is ignored.
 * Meant to run once, when the weights are loaded. Asynchronous. */
moe_status_t moe_pack_weights(const moe_config_t *cfg, const void *w_gate,
                              const void *w_up, const void *w_down,
                              void *out_gate, void *out_up, void *out_down,
                              void *stream);

/* Collect and weighted combine after the last round, the collect step of
 * the rounds ("Frontier Pre-training at Microsoft AI (MAI-Base-2)", section
 * "Key claims", item on multi-round dropless MoE); the k outputs of a token
 * are weighted by its routing weights (the pages leave the combine open;
 * this is the plain reading): y[t] =
 * sum_{j<k} weight[t][j] * z[pos[t*k + j]] (gathering every assignment's
 * expert output back to its token), summed in fp32 over ascending j and
 * rounded once to elem. Reads only the workspace. Asynchronous. */
moe_status_t moe_combine(const moe_config_t *cfg, const void *ws,
                         size_t ws_bytes, void *y, void *stream);

/* The whole layer: plan, one wait to learn the counts and R, then the R
 * rounds of dispatch and expert compute, one launch of each grouped GEMM
 * per launch batch (see "Launch batches"; launch shapes fitted to each
 * batch as with counts_host above), then the collect and weighted combine.
 * y is written in full. The dispatch is the gate/up launch's own fetch of
 * the token rows from x (as moe_dispatch_gate_up) when x holds at most 2^30
 * bytes, else one moe_dispatch launch per batch before its GEMMs; the
 * results are the same bits either way. ws_bytes: at least
 * moe_forward_workspace_size (with the gathering launches the round buffer
 * xr is neither read nor written).
 * Returns after enqueueing the combine (the plan's wait is the only host
 * synchronisation; round 0's dispatch, and its GEMMs where a full round 0
 * fills the GPU, are queued before it). For that read
 * the call takes from a pool of the current device a set of a pinned host
 * buffer of 65 int32, a side stream of default priority that does the copy
 * and three events, and returns it when it returns: sets are created when
 * no idle one is left, so a device never holds more than the most calls in
 * flight on it at once (from any number of threads), and are kept until the
 * process ends. With S = 2 the rounds overlap as the method
 * overlaps dispatch with compute ("Frontier Pre-training at Microsoft AI
 * (MAI-Base-2)", section "Key claims"): odd rounds run on the side stream with buffer set 1, even rounds
 * on the caller's stream with set 0 (round 1's dispatch, where it is a
 * launch of its own, is also queued before the wait), and the caller's stream waits for the side stream
 * before the combine, so the caller still sees one stream's order. The
 * result does not depend on C, G or S. */
moe_status_t moe_forward(const moe_config_t *cfg, const float *logits,
                         const void *x, const void *w_gate, const void *w_up,
                         const void *w_down, void *y, void *ws,
                         size_t ws_bytes, void *stream);

/* Bytes of the static workspace moe_forward_static uses: a device array
 * inside the library, one per GPU the library runs on, held until the
 * process ends. */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

/* moe_forward for callers that cannot allocate memory: serving loops and
 * harnesses that must not call hipMalloc or create streams and events. The
 * same layer, kernels and launch shapes as moe_forward, with bit-identical
 * y, but the workspace is the library's static device array of
 * MOE_STATIC_WORKSPACE_BYTES on the current device instead of a caller
 * buffer, and the call creates and allocates nothing (no device or pinned
 * memory, no stream, no event). The caller passes the inputs and y as for
 * moe_forward. The plan's counts and R are read into the call's own host
 * frame with one wait on `stream`; every launch batch then runs on
 * `stream` in order (with round_buffers = 2 the two buffer sets alternate,
 * without overlap). A config whose moe_forward_workspace_size exceeds
 * MOE_STATIC_WORKSPACE_BYTES returns MOE_ERR_WORKSPACE_TOO_SMALL before any
 * HIP call. All calls on one GPU share its array and it keeps the last
 * call's contents: calls that overlap in time on one GPU (on different
 * streams or from different threads) race and give wrong results; calls
 * queued on one stream do not overlap. */
moe_status_t moe_forward_static(const moe_config_t *cfg, const float *logits,
                                const void *x, const void *w_gate,
                                const void *w_up, const void *w_down, void *y,
                                void *stream);

/* ------------------------------------------------------------------------
 * Backward (bf16 only). The gradient of a loss through y = layer(x, logits,
 * W), given dy = dL/dy [T][d], with respect to x, the router logits and the
 * expert weights, computed on the forward's round schedule ("Frontier
 * Pre-training at Microsoft AI (MAI-Base-2)", section "Key claims": rounds
 * of dispatch, expert compute and collect with fixed per-round memory; the
 * backward keeps that memory fixed by recomputing each round's expert
 * activations from x instead of storing them). Readings: the top-k
 * selection passes no gradient; the k routing weights are the softmax of
 * the k chosen logits, so only those logits get a gradient:
 * dlogits[t][idx[t][j]] = w_j (dw_j - sum_j' w_j' dw_j') with dw_j =
 * <z[pos[t*k + j]], dy[t]> (z, the forward's unweighted expert outputs);
 * every other logit 0. Per round r, for expert e's rows c (assignment a,
 * token t, weight w):
 *   xr, dyr   gathered rows of x and dy (as moe_dispatch)
 *   g, u      xr Wg^T, xr Wu^T (recomputed; stored bf16 in gu)
 *   hw        w * silu(g) u (bf16)
 *   dh        w * (dyr Wd);  du = dh silu(g);  dg = dh u silu'(g)
 *   dz[pos[a]] = dg Wg + du Wu  (the assignment's input gradient)
 *   dW_down[e] += dyr^T hw;  dW_gate[e] += dg^T xr;  dW_up[e] += du^T xr
 * and finally dx[t] = sum_j dz[pos[t*k + j]] (fp32, j ascending, rounded
 * once). GEMMs take bf16 operands with fp32 accumulation; the weight
 * gradients are fp32 and sum an expert's rows a pair of rounds at a time. */

/* Byte offsets of the backward workspace's buffers (a pure function of the
 * config; 256-byte aligned): round buffers xr, dyr [2][E/G][Q][d], gu
 * [E/G][Q][2f], dgu [2][E/G][Q][2f], hw [2][E/G][Q][f] (tiled, as the
 * forward's xr; rounds are taken in pairs, the second round of a pair in
 * set 1, and the weight gradients contract both in one pass), dz [T*k][d]
 * (expert-sorted order, as z) and ones [T*k] float. */
typedef struct {
  size_t xr, dyr, gu, hw, dgu, dz, ones;
  size_t total;
} moe_backward_layout_t;

/* Bytes of the backward workspace (pure host function). MOE_ERR_UNSUPPORTED
 * for fp32 configs, for k > 8, and unless G*(P+64)*2f and d*2f bf16
 * elements stay below 2^31 bytes (P = C' rounded up to 64). */
moe_status_t moe_backward_workspace_size(const moe_config_t *cfg, size_t *bytes);
moe_status_t moe_backward_layout(const moe_config_t *cfg,
                                 moe_backward_layout_t *out);

/* The backward of the layer. ws: the forward's workspace after moe_forward
 * with the same cfg, logits and x (its plan and z are read, nothing in it
 * is written). x, w_gate, w_up and w_down as given to moe_forward (in
 * cfg->weight_layout; the input-gradient GEMMs read the same matrices
 * transposed, so no second copy of the weights exists). dy [T][d] bf16.
 * Outputs (written in full): dx
 * [T][d] bf16, dlogits [T][E] float, dw_gate, dw_up [E][f][d] and dw_down
 * [E][d][f] float. ws_bytes: at least moe_forward_workspace_size (the
 * forward's xr is not used). bws: moe_backward_workspace_size bytes. Waits once for
 * the forward's counts and R (as moe_forward), then asynchronous on stream.
 * dx and dlogits do not depend on C or G; the weight gradients' summation
 * order follows the rounds. */
moe_status_t moe_backward(const moe_config_t *cfg, const void *x,
                          const void *w_gate, const void *w_up,
                          const void *w_down, const void *dy, void *dx,
                          float *dlogits,
                          float *dw_gate, float *dw_up, float *dw_down,
                          const void *ws, size_t ws_bytes, void *bws,
                          size_t bws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUNDS_H */
