/*
 * moe.h — C interface of a single-GPU Mixture-of-Experts layer forward for
 * AMD Instinct MI355X (gfx950): route -> permute -> grouped SwiGLU experts
 * -> weighted combine, for one GPU's local experts.
 *
 * Sources (web pages, cited by title and section):
 *   [MC] "MoE我们喜欢你（三）：Megatron Core MoE 源码路径解析" — §2 layer main
 *        path, §3 gating, §4 top-k routing, §5 score functions, §7 expert
 *        bias, §8 token dropping, §9 dispatcher, §10 grouped experts,
 *        §11 shared expert.
 *   [DS] "MoE Internals: DeepSpeed-Megatron Expert Parallel Implementation"
 *        — §3 capacity knobs, §8 the forward steps.
 *   [MG] "Scalable Training of Mixture-of-Experts Models with Megatron Core"
 *        (daily-arxiv summary) — grouped GEMM and sync-free dropless
 *        execution under "计算效率优化".
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates or frees device memory and keeps no state
 *     between calls beyond the thread-local error message (and, for
 *     moe_route_permute_noalloc only, a static scratch array on each GPU
 *     and its device address).
 *   - Tensors are dense, row-major (last index fastest), with no padding.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it and return; they never synchronise and never read
 *     device data on the host (tokens_per_expert stays on the device).
 *   - Host-side argument checks run before any launch.  On failure the call
 *     returns a non-zero moe_status, launches nothing, and moe_last_error()
 *     describes the problem.  A failed launch returns MOE_ERR_HIP.
 *   - Device-resident index inputs (routing_map, tokens_per_expert,
 *     row_id_map) are never trusted for addressing: kernels clamp to the
 *     caller-stated sizes, so malformed values give wrong numbers, not
 *     out-of-bounds accesses.  NaN/Inf inputs are outside the contract.
 *   - Element dtypes: moe_dtype selects fp32 or bf16 for activations,
 *     expert weights and outputs.  The router always computes in fp32.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = 1,          /* invalid argument (null pointer, bad size, K > E, ...) */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not implemented (e.g. a size constraint below) */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than *_workspace_size() */
  MOE_ERR_HIP = 4           /* a HIP launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1, MOE_SCORE_SQRTSOFTPLUS = 2 } moe_score;

/* Which tokens an expert keeps when more than its capacity are routed to it
 * ([MC] §8): the earliest tokens ("position"), or the tokens with the
 * largest routing probs ("probs"; equal probs: the earlier token). */
typedef enum { MOE_DROP_POSITION = 0, MOE_DROP_PROBS = 1 } moe_drop_policy;

/* Version of this interface (2: drop policy, padding to capacity,
 * sqrtsoftplus scores, router side outputs, gathering FC1, MXFP8 GEMMs;
 * 3: moe_route_permute, moe_grouped_fc2_combine,
 * moe_grouped_fc2_combine_mxfp8; 4: moe_grouped_fc1_swiglu_gather_shared,
 * moe_grouped_fc2_shared; 5: moe_route_permute_noalloc; 6: the queue
 * argument of the bf16 GEMM entry points; 7: moe_clock_probe; 8: the
 * queue argument of the MXFP8 GEMM entry points,
 * moe_grouped_fc1_swiglu_mxfp8_shared, moe_grouped_fc2_mxfp8_shared). */
int moe_abi_version(void);

/* Message for the last non-OK status returned on the calling thread. */
const char* moe_last_error(void);

/* Measurement utility, not a stage of the layer: the shader clock the GPU
 * runs at while other work is in flight.  Launches one wave on `stream`
 * that waits spin_us microseconds of the GPU's constant 100 MHz counter and
 * then writes two values to `out` (device memory, 2 x uint64, caller-owned):
 * out[0] = shader-clock cycles elapsed (s_memtime), out[1] = 100 MHz ticks
 * elapsed (s_memrealtime); the clock in MHz is 100 * out[0] / out[1].  The
 * wave sleeps between reads and holds no LDS, so it shares a CU with other
 * kernels' workgroups.  Errors: MOE_ERR_ARG (out null, spin_us outside
 * (0, 1e6]); MOE_ERR_HIP. */
moe_status moe_clock_probe(uint64_t* out, int64_t spin_us, void* stream);

/* ------------------------------------------------------------------------
 * Router: gating linear + score function + top-k + capacity drop.
 * [MC] §3 (logits = x W^T (+ b) in fp32), §4 (routing returns probs and a
 * [T,E] routing map), §5 (score functions, selection-only expert bias), §8
 * (capacity, the "position" and "probs" drop policies, padding to
 * capacity); [DS] §3 (capacity factor, minimum capacity).
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t T;                /* tokens (sequence x batch, flattened) */
  int64_t h;                /* hidden size; must be a multiple of 8 */
  int64_t E;                /* experts, 1..1024 */
  int64_t K;                /* experts per token, 1..E and <= 64 */
  int32_t x_dtype;          /* moe_dtype of x */
  int32_t score;            /* moe_score */
  int32_t pre_softmax;      /* softmax only: 1 = softmax over all E, then top-K
                               (probs are those softmax values); 0 = top-K of
                               the logits, then softmax over the K chosen */
  float capacity_factor;    /* <= 0: dropless.  > 0: capacity per expert =
                               max(ceil(T*K*capacity_factor/E), min_capacity)
                               (ratio computed in double) */
  int64_t min_capacity;     /* lower bound of the capacity; 0 = none */
  int32_t drop_policy;      /* moe_drop_policy (with a capacity) */
  int32_t pad_to_capacity;  /* with a capacity: 1 = every expert receives
                               exactly min(capacity, T) tokens: the capacity
                               mask itself becomes the routing map, so an
                               expert with fewer routed tokens is padded with
                               the earliest tokens not routed to it (prob 0);
                               a capacity >= T routes every token to every
                               expert.  0 = map AND mask */
} moe_route_desc;

/* Bytes of device workspace moe_route needs (0 is a valid answer only for
 * T == 0). */
size_t moe_route_workspace_size(const moe_route_desc* desc);

/* Per-expert capacity for desc, or -1 when routing is dropless or when the
 * capacity is at least T (then nothing can be dropped). */
int64_t moe_route_capacity(const moe_route_desc* desc);

/* Upper bound on the number of routed rows N = sum(tokens_per_expert):
 * T*K when dropless, else min(T*K, E*capacity); E*min(capacity, T) when
 * padding to capacity.  Size permute/expert buffers with it. */
int64_t moe_max_rows(const moe_route_desc* desc);

/*
 * moe_route — router forward.
 *   x            [T,h]  x_dtype         hidden states (ignored if logits_in)
 *   w_router     [E,h]  fp32            gating weight (ignored if logits_in)
 *   b_router     [E]    fp32 or NULL    gating bias; part of the logits, so it
 *                                       affects both the choice and the probs
 *   expert_bias  [E]    fp32 or NULL    sigmoid / sqrtsoftplus only: added to the
 *                                       scores for the top-K choice, never to
 *                                       the probs ([MC] §5, §7)
 *   logits_in    [T,E]  fp32 or NULL    route from these logits instead of
 *                                       computing x w^T (+b)
 *   logits_out   [T,E]  fp32 or NULL    receives the logits
 *   scores_out   [T,E]  fp32 or NULL    receives the score function over all E
 *                                       (softmax over E, sigmoid or sqrtsoftplus)
 *   probs        [T,E]  fp32            out: combine weights, 0 off the map
 *   routing_map  [T,E]  uint8           out: 1 where token t is routed to e
 *   tokens_per_expert [E] int32         out: routing_map summed over tokens
 *   workspace    moe_route_workspace_size(desc) bytes of device memory
 * Top-K order: larger key first, lower expert index on ties.  Keys: the fp32
 * logits for softmax (softmax is increasing); score(logit) (+ expert_bias)
 * for sigmoid and sqrtsoftplus = sqrt(log(1 + e^x)), both evaluated by
 * fixed sequences of IEEE fp32 operations so that their bits are
 * reproducible.  Sigmoid / sqrtsoftplus probs are the chosen scores over
 * (their sum + 1e-20).  With a capacity, the drop policy and padding act on
 * these probs and map after the choice; dropped entries get map 0, prob 0.
 */
moe_status moe_route(const moe_route_desc* desc, const void* x, const float* w_router,
                     const float* b_router, const float* expert_bias, const float* logits_in,
                     float* logits_out, float* scores_out, float* probs, uint8_t* routing_map,
                     int32_t* tokens_per_expert, void* workspace, size_t workspace_bytes,
                     void* stream);

/* ------------------------------------------------------------------------
 * Router side outputs.  [MC] §6: the switch load-balancing loss has the form
 * E * sum_i f_i * P_i; §7: loss-free balance keeps an fp32 expert bias and
 * a running per-expert token count, and moves the bias one step of the
 * update rate by the sign of (mean count - count).
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace moe_router_aux_loss needs. */
size_t moe_aux_loss_workspace_size(int64_t T, int64_t E);

/*
 * moe_router_aux_loss — forward value of the load-balancing loss (no
 * coefficient): loss = E * sum_e f_e * P_e with f_e = tokens_per_expert[e]
 * / (T*K) and P_e = mean over tokens of the router's probability mass on e:
 * the softmax scores as given, or for sigmoid / sqrtsoftplus the scores
 * normalised per token to sum 1 (over their sum + 1e-20).  fp32, summed in a
 * fixed order (reproducible).
 *   scores            [T,E] fp32   the scores_out of moe_route
 *   tokens_per_expert [E]   int32  the moe_route output (after dropping)
 *   loss              [1]   fp32   out
 */
moe_status moe_router_aux_loss(int64_t T, int64_t E, int64_t K, int32_t score,
                               const float* scores, const int32_t* tokens_per_expert,
                               float* loss, void* workspace, size_t workspace_bytes,
                               void* stream);

/* local_tokens_per_expert[e] += tokens_per_expert[e]   (int64 running count) */
moe_status moe_accumulate_tokens_per_expert(int64_t E, const int32_t* tokens_per_expert,
                                            int64_t* local_tokens_per_expert, void* stream);

/*
 * moe_update_expert_bias — one controller step on one GPU (no all-reduce):
 *   expert_bias[e] += sign(mean - local[e]) * update_rate   (one fp32 add)
 * where the sign is decided exactly as sign(sum(local) - E * local[e]).  With
 * reset != 0 the running counts are then set to 0.
 *   local_tokens_per_expert [E] int64 (in, and out when reset)
 *   expert_bias             [E] fp32  (in/out)
 */
moe_status moe_update_expert_bias(int64_t E, int64_t* local_tokens_per_expert, float* expert_bias,
                                  float update_rate, int32_t reset, void* stream);

/* ------------------------------------------------------------------------
 * Dispatch preprocess: permute token rows into expert-major order.
 * [MC] §2 and §9 (rows go from token-major to expert-major order before the
 * experts); [DS] §8 step 4.
 * ------------------------------------------------------------------------ */

/* Bytes of device workspace moe_permute needs. */
size_t moe_permute_workspace_size(int64_t T, int64_t E);

/*
 * moe_permute — rows sorted by (expert ascending, token ascending).
 *   x              [T,h]        dtype   h must be a multiple of 8
 *   routing_map    [T,E]        uint8   nonzero = routed (any number per row:
 *                                       padding to capacity adds entries)
 *   probs          [T,E]        fp32    at most K nonzero per row
 *   permuted_x     [max_rows,h] dtype   out: permuted_x[i] = x[sorted_token[i]];
 *                                       may be NULL (then x may be NULL too): no
 *                                       rows are copied, for the gathering FC1
 *   permuted_probs [max_rows]   fp32    out: probs[sorted_token[i], expert of row i]
 *   sorted_token   [max_rows]   int32   out: source token of row i
 *   row_id_map     [T,K]        int32   out: row of token t's k-th map entry with
 *                                       a nonzero prob (ascending expert order),
 *                                       -1 if unused.  Entries with prob 0 get
 *                                       rows but no slot: they add nothing to
 *                                       the combine.
 *   expert_offsets [E+1]        int32   out: first row of each expert; [E] = N
 * Rows at index >= N are left untouched.  Rows beyond max_rows and nonzero
 * probs beyond K in a row are not written (outside the contract).
 */
moe_status moe_permute(int64_t T, int64_t h, int64_t E, int64_t K, int32_t dtype, const void* x,
                       const uint8_t* routing_map, const float* probs, int64_t max_rows,
                       void* permuted_x, float* permuted_probs, int32_t* sorted_token,
                       int32_t* row_id_map, int32_t* expert_offsets, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Bytes of device workspace moe_route_permute needs (0 when T == 0 or the
 * descriptor is invalid). */
size_t moe_route_permute_workspace_size(const moe_route_desc* d);

/*
 * moe_route_permute — moe_route, then moe_permute of its routing_map and
 * probs (with h = d->h, E = d->E, K = d->K, dtype = d->x_dtype), in one
 * call: the router and the dispatch preprocess of [MC] §2 back to back.
 * Every output is bitwise what the two calls write.  The permute's row of
 * an entry needs, per token block and expert, the count of that expert's
 * kept entries in earlier blocks; the router's counting pass already has
 * them (under the position policy, or when nothing is dropped, an expert
 * keeps its earliest entries, so the kept count before a block is
 * min(routed count before it, capacity)), so the permute's own counting
 * passes are skipped there (two kernels fewer).  The probs policy and
 * padding to capacity count the final map again.
 *   route arguments    as moe_route
 *   permute arguments  as moe_permute (x may be NULL when logits_in is given
 *                      and permuted_x is NULL)
 *   workspace          moe_route_permute_workspace_size(d) bytes
 * Errors: those of moe_route and moe_permute.
 */
moe_status moe_route_permute(const moe_route_desc* d, const void* x, const float* w_router,
                             const float* b_router, const float* expert_bias,
                             const float* logits_in, float* logits_out, float* scores_out,
                             float* probs, uint8_t* routing_map, int32_t* tokens_per_expert,
                             int64_t max_rows, void* permuted_x, float* permuted_probs,
                             int32_t* sorted_token, int32_t* row_id_map, int32_t* expert_offsets,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_permute_noalloc — moe_route_permute for callers that cannot
 * allocate device memory (code under graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same outputs, bit for bit, with the
 * workspace taken from a static scratch array that the library holds on
 * each GPU it runs on (MOE_NOALLOC_SCRATCH_BYTES per GPU, kept until the
 * process ends; its device address is looked up once per device).  No
 * allocation of any kind happens in the call.
 *   arguments  as moe_route_permute, without workspace and workspace_bytes
 * Errors: those of moe_route_permute; MOE_ERR_UNSUPPORTED (before anything
 * is launched) when moe_route_permute_workspace_size(d) exceeds
 * MOE_NOALLOC_SCRATCH_BYTES; MOE_ERR_HIP if the scratch address cannot be
 * found.  Every call on one GPU uses the same scratch: calls that overlap
 * in time on one GPU (different streams, or threads) race and must be
 * serialised by the caller.  Nothing in the scratch needs clearing between
 * calls (each call writes every word it reads).
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
moe_status moe_route_permute_noalloc(const moe_route_desc* d, const void* x,
                                     const float* w_router, const float* b_router,
                                     const float* expert_bias, const float* logits_in,
                                     float* logits_out, float* scores_out, float* probs,
                                     uint8_t* routing_map, int32_t* tokens_per_expert,
                                     int64_t max_rows, void* permuted_x, float* permuted_probs,
                                     int32_t* sorted_token, int32_t* row_id_map,
                                     int32_t* expert_offsets, void* stream);

/* ------------------------------------------------------------------------
 * Experts: SwiGLU MLP of every local expert as one grouped GEMM per layer.
 * [MC] §10 (all local experts' MLPs run as a grouped GEMM instead of a loop
 * of small GEMMs); [MG] 计算效率优化 (grouped GEMM; dropless routing without a
 * host-device synchronisation).  The expert MLP is SwiGLU without biases:
 *   act = silu(x W_gate[e]^T) * (x W_up[e]^T),   y = act W_down[e]^T,
 * silu(g) = g * sigmoid(g).  Rows [off_e, off_e + n_e) belong to expert e,
 * where n_e = tokens_per_expert[e] (read on the device only) and off_e is
 * its prefix sum.  Accumulation is fp32; act and y are stored in `dtype`
 * (bf16 rounded to nearest-even).  Sizes for MOE_BF16: h and f multiples
 * of 64.  Rows at index >= sum(n_e) of act/expert_out are left untouched;
 * counts are clamped so that no row index reaches max_rows.
 *
 * queue (every GEMM entry point below that takes one): NULL, or a device
 * buffer of MOE_GEMM_QUEUE_BYTES that is all zero before the first call
 * that uses it.  With a queue, a bf16 or MXFP8 launch of 2 to 256 experts
 * whose average row count (max_rows / E) is >= 192 runs one workgroup per CU,
 * and each takes the next tile of its XCD's share from a counter in the
 * queue (tile groups of 32 dealt to the XCDs in turn), instead of one
 * workgroup per tile handed out by the hardware; other launches ignore the
 * queue.  The last workgroup leaves the counters at zero, so
 * one queue serves any number of calls in stream order.  Calls that can
 * run at the same time (different streams) need different queues.  The
 * results do not depend on it (each tile is computed by one workgroup, in
 * the same way).  NULL: one workgroup per tile.
 * ------------------------------------------------------------------------ */
#define MOE_GEMM_QUEUE_BYTES ((size_t)2048)

/*
 * moe_grouped_fc2_combine — moe_grouped_fc2 with moe_combine as its
 * epilogue, for top-1 routing (K = 1) without a shared expert: [MC] §2's
 * combine weights each token's single expert output by its prob, so row r
 * of the grouped GEMM goes straight to out[sorted_token[r]] as
 * p[r] * y[r], and the tokens whose entry was dropped (row_id_map[t]
 * outside [0, max_rows)) get zero rows.  The rounding is the two calls'
 * (y to bf16, then p*y in fp32, then to bf16): out is bitwise what
 * moe_grouped_fc2 followed by moe_combine (K = 1, no shared_out) writes,
 * without the expert_out round trip through HBM.  bf16 only.
 *   act, tokens_per_expert, w_down  as moe_grouped_fc2
 *   permuted_probs [max_rows] fp32, sorted_token [max_rows] int32 (values
 *                  clamped to [0, T)), row_id_map [T] int32  as moe_permute
 *                  writes them with K = 1
 *   out            [T,h]  bf16  out
 * Errors: those of moe_grouped_fc2; MOE_ERR_UNSUPPORTED for fp32.
 */
moe_status moe_grouped_fc2_combine(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                   int32_t dtype, int64_t T, const void* act,
                                   const int32_t* tokens_per_expert, const void* w_down,
                                   const float* permuted_probs, const int32_t* sorted_token,
                                   const int32_t* row_id_map, void* out, void* stream);

/*
 *   permuted_x        [max_rows,h]  dtype
 *   tokens_per_expert [E]           int32 (device)
 *   w_gate, w_up      [E,f,h]       dtype
 *   w_down            [E,h,f]       dtype
 *   act               [max_rows,f]  dtype   out (intermediate activation)
 *   expert_out        [max_rows,h]  dtype   out (unweighted expert outputs)
 */
moe_status moe_grouped_mlp(int64_t E, int64_t h, int64_t f, int64_t max_rows, int32_t dtype,
                           const void* permuted_x, const int32_t* tokens_per_expert,
                           const void* w_gate, const void* w_up, const void* w_down, void* act,
                           void* expert_out, void* queue, void* stream);

/* The first half of moe_grouped_mlp: act = silu(x W_gate^T) * (x W_up^T). */
moe_status moe_grouped_fc1_swiglu(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                  int32_t dtype, const void* permuted_x,
                                  const int32_t* tokens_per_expert, const void* w_gate,
                                  const void* w_up, void* act, void* queue, void* stream);

/*
 * moe_grouped_fc1_swiglu_gather — the first half of moe_grouped_mlp reading
 * its rows straight from the token-major input: row i of the grouped GEMM is
 * x[sorted_token[i]] (moe_permute's sorted_token; values are clamped to
 * [0, T)), so permuted_x need not be materialised.  [MG] 计算效率优化 lists
 * memory-efficient permutation among the MoE optimisations; the result is
 * identical to moe_grouped_fc1_swiglu on moe_permute's permuted_x.
 *   x            [T,h]         dtype
 *   sorted_token [max_rows]    int32
 *   (other arguments as moe_grouped_fc1_swiglu)
 */
moe_status moe_grouped_fc1_swiglu_gather(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                         int32_t dtype, int64_t T, const void* x,
                                         const int32_t* sorted_token,
                                         const int32_t* tokens_per_expert, const void* w_gate,
                                         const void* w_up, void* act, void* queue, void* stream);

/*
 * moe_grouped_fc1_swiglu_gather_shared — moe_grouped_fc1_swiglu_gather and
 * the shared expert's FC1 in ONE launch.  [MC] §2 and §11: the shared
 * expert runs on every token beside the routed experts and its output is
 * added after the combine; here its tiles ride in the routed launch (the
 * last workgroups of a one-tile-per-workgroup launch, the first tiles a
 * tile-queue launch hands out) instead of competing with the router on a
 * second stream.
 *   routed arguments  as moe_grouped_fc1_swiglu_gather (max_rows may be 0)
 *   fs                shared expert ffn size (a multiple of 64)
 *   shared_gate, shared_up [fs,h] bf16
 *   shared_act        [T,fs]  bf16  out: silu(x Wsg^T) * (x Wsu^T) for every token
 * Results are bitwise those of the separate calls (moe_grouped_fc1_swiglu
 * with E = 1 and T rows for the shared part).  bf16 only
 * (MOE_ERR_UNSUPPORTED for fp32).
 */
moe_status moe_grouped_fc1_swiglu_gather_shared(int64_t E, int64_t h, int64_t f,
                                                int64_t max_rows, int32_t dtype, int64_t T,
                                                const void* x, const int32_t* sorted_token,
                                                const int32_t* tokens_per_expert,
                                                const void* w_gate, const void* w_up, void* act,
                                                int64_t fs, const void* shared_gate,
                                                const void* shared_up, void* shared_act,
                                                void* queue, void* stream);

/*
 * moe_grouped_fc2_shared — moe_grouped_fc2 and the shared expert's FC2 in
 * ONE launch (as moe_grouped_fc1_swiglu_gather_shared is to FC1).
 *   routed arguments  as moe_grouped_fc2 (max_rows may be 0)
 *   T, fs             tokens and shared ffn size
 *   shared_act        [T,fs] bf16
 *   shared_down       [h,fs] bf16
 *   shared_out        [T,h]  bf16  out: shared_act Wsd^T (pass it to moe_combine)
 * Bitwise the separate calls.  bf16 only.
 */
moe_status moe_grouped_fc2_shared(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                  int32_t dtype, const void* act,
                                  const int32_t* tokens_per_expert, const void* w_down,
                                  void* expert_out, int64_t T, int64_t fs,
                                  const void* shared_act, const void* shared_down,
                                  void* shared_out, void* queue, void* stream);

/* The second half of moe_grouped_mlp: expert_out = act W_down^T. */
moe_status moe_grouped_fc2(int64_t E, int64_t h, int64_t f, int64_t max_rows, int32_t dtype,
                           const void* act, const int32_t* tokens_per_expert,
                           const void* w_down, void* expert_out, void* queue, void* stream);

/* ------------------------------------------------------------------------
 * MXFP8 expert GEMMs.  [MG] FP8/FP4 低精度训练 and 计算效率优化 name FP8 GEMMs for
 * the MoE experts without a scaling recipe; the format here is the OCP
 * Microscaling MXFP8-E4M3 block format, which gfx950's scaled MFMA executes:
 * 32 consecutive values along the reduction dimension share an E8M0 scale
 * byte X = 2^(floor(log2 amax) - 8) (code = exponent + 127; an all-zero
 * block has code 0); each value is stored as the E4M3 code of V / X
 * (nearest, ties to even, saturated to +-448).  Codes are [rows, cols]
 * uint8.  Scales are uint8 in one of two layouts: row-major [rows, cols/32],
 * or k-tiled with R rows per group, [rows/R, cols/128, R, 4] (the 4 scales
 * of one 128-wide k stage of R consecutive rows are contiguous), which the
 * GEMMs read for the weights (R = rows per expert) and for act.
 * ------------------------------------------------------------------------ */

/* moe_mxfp8_quantize — quantise src [rows, cols] (dtype bf16 or fp32) along
 * cols (a multiple of 32) into codes [rows, cols] and scales: row-major when
 * tile_rows = 0, else k-tiled with R = tile_rows (cols % 128 == 0, rows %
 * tile_rows == 0).  Use it on x per forward (row-major), and once on the
 * weights (k-tiled: [E*f, h] with tile_rows = f for W_gate and W_up,
 * [E*h, f] with tile_rows = h for W_down). */
moe_status moe_mxfp8_quantize(int64_t rows, int64_t cols, int64_t tile_rows, int32_t dtype,
                              const void* src, uint8_t* codes, uint8_t* scales, void* stream);

/*
 * moe_grouped_fc1_swiglu_mxfp8 — act = silu(x Wg^T) * (x Wu^T) on MXFP8
 * operands, fp32 accumulation in the MFMA, act quantised to MXFP8 along f.
 *   x_codes, x_scales   [T,h], row-major [T,h/32]   token-major MXFP8 x
 *   sorted_token        [max_rows] int32 or NULL: GEMM row i reads x row
 *                       sorted_token[i] (clamped to [0, T)); NULL: rows are
 *                       already expert-major ([max_rows, h])
 *   wg_*, wu_*          codes [E,f,h], scales k-tiled with R = f
 *   act_codes           [max_rows,f]                          out
 *   act_scales          k-tiled [f/128, max_rows, 4] (R = max_rows)   out
 *   queue               NULL, or a tile queue as for the bf16 GEMMs
 *                       (MOE_GEMM_QUEUE_BYTES, zero on entry, zero again
 *                       when the launch ends); used from 192 rows per
 *                       expert on average, same results either way
 * h and f multiples of 128.  Rows >= sum(tokens_per_expert) untouched.
 */
moe_status moe_grouped_fc1_swiglu_mxfp8(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                        int64_t T, const uint8_t* x_codes, const uint8_t* x_scales,
                                        const int32_t* sorted_token,
                                        const int32_t* tokens_per_expert, const uint8_t* wg_codes,
                                        const uint8_t* wg_scales, const uint8_t* wu_codes,
                                        const uint8_t* wu_scales, uint8_t* act_codes,
                                        uint8_t* act_scales, void* queue, void* stream);

/* moe_grouped_fc1_swiglu_mxfp8_shared — moe_grouped_fc1_swiglu_mxfp8 (with
 * the gather) plus the shared expert's FC1 + SwiGLU in the same launch
 * ([MC] §11: one expert that every token passes through), its tiles after
 * the routed experts'.  The shared expert reads x_codes/x_scales as they
 * are (all T rows, not gathered); sg_*, su_* are its weights (codes [fs,h],
 * scales k-tiled with R = fs); shared_act_codes [T,fs] and
 * shared_act_scales k-tiled [fs/128, T, 4] are written bitwise as
 * moe_grouped_fc1_swiglu_mxfp8 with E = 1, counts {T}, max_rows = T and no
 * gather writes them.  fs a multiple of 128.  Errors: those of
 * moe_grouped_fc1_swiglu_mxfp8; MOE_ERR_ARG when sorted_token is NULL or a
 * shared tensor is NULL (act may be NULL only when max_rows = 0).  T = 0
 * is a no-op. */
moe_status moe_grouped_fc1_swiglu_mxfp8_shared(
    int64_t E, int64_t h, int64_t f, int64_t max_rows, int64_t T, const uint8_t* x_codes,
    const uint8_t* x_scales, const int32_t* sorted_token, const int32_t* tokens_per_expert,
    const uint8_t* wg_codes, const uint8_t* wg_scales, const uint8_t* wu_codes,
    const uint8_t* wu_scales, uint8_t* act_codes, uint8_t* act_scales, int64_t fs,
    const uint8_t* sg_codes, const uint8_t* sg_scales, const uint8_t* su_codes,
    const uint8_t* su_scales, uint8_t* shared_act_codes, uint8_t* shared_act_scales, void* queue,
    void* stream);

/* moe_grouped_fc2_mxfp8 — expert_out [max_rows,h] (bf16) = act Wd^T on MXFP8
 * act (as moe_grouped_fc1_swiglu_mxfp8 writes it) and Wd (codes [E,h,f],
 * scales k-tiled with R = h).  queue: as for moe_grouped_fc1_swiglu_mxfp8. */
moe_status moe_grouped_fc2_mxfp8(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                 const uint8_t* act_codes, const uint8_t* act_scales,
                                 const int32_t* tokens_per_expert, const uint8_t* wd_codes,
                                 const uint8_t* wd_scales, void* expert_out, void* queue,
                                 void* stream);

/* moe_grouped_fc2_mxfp8_shared — moe_grouped_fc2_mxfp8 plus the shared
 * expert's FC2 in the same launch, its tiles after the routed experts':
 * shared_out [T,h] (bf16) = shared_act sd^T, bitwise what
 * moe_grouped_fc2_mxfp8 with E = 1, counts {T} and max_rows = T writes
 * (shared_act as moe_grouped_fc1_swiglu_mxfp8_shared writes it; sd codes
 * [h,fs], scales k-tiled with R = h).  Errors: those of
 * moe_grouped_fc2_mxfp8; MOE_ERR_ARG for T out of range or a NULL shared
 * tensor.  T = 0 is a no-op. */
moe_status moe_grouped_fc2_mxfp8_shared(
    int64_t E, int64_t h, int64_t f, int64_t max_rows, const uint8_t* act_codes,
    const uint8_t* act_scales, const int32_t* tokens_per_expert, const uint8_t* wd_codes,
    const uint8_t* wd_scales, void* expert_out, int64_t T, int64_t fs,
    const uint8_t* shared_act_codes, const uint8_t* shared_act_scales, const uint8_t* sd_codes,
    const uint8_t* sd_scales, void* shared_out, void* queue, void* stream);

/* moe_grouped_fc2_combine_mxfp8 — moe_grouped_fc2_mxfp8 with the top-1
 * combine as its epilogue, as moe_grouped_fc2_combine is to
 * moe_grouped_fc2 ([MC] §2: each token's one expert output weighted by its
 * prob; dropped tokens get zero rows).  out [T,h] bf16 is bitwise what
 * moe_grouped_fc2_mxfp8 followed by moe_combine (K = 1, no shared_out)
 * writes.  permuted_probs, sorted_token, row_id_map as moe_permute writes
 * them with K = 1.  Errors: those of moe_grouped_fc2_mxfp8; MOE_ERR_ARG for
 * T out of range or a NULL tensor (act, probs and sorted_token may be NULL
 * only when max_rows = 0).  T = 0 is a no-op. */
moe_status moe_grouped_fc2_combine_mxfp8(int64_t E, int64_t h, int64_t f, int64_t max_rows,
                                         int64_t T, const uint8_t* act_codes,
                                         const uint8_t* act_scales,
                                         const int32_t* tokens_per_expert,
                                         const uint8_t* wd_codes, const uint8_t* wd_scales,
                                         const float* permuted_probs,
                                         const int32_t* sorted_token, const int32_t* row_id_map,
                                         void* out, void* stream);

/* ------------------------------------------------------------------------
 * Combine: unpermute and weight.  [MC] §2 (combine takes the expert outputs
 * and the router probs; the shared expert's output is added afterwards),
 * §11; [DS] §8 step 8.
 *   out[t] = sum_{k: row_id_map[t,k] >= 0} permuted_probs[r] * expert_out[r]
 *            (+ shared_out[t]),   r = row_id_map[t,k],
 * summed in fp32 in ascending k (= ascending expert) order and rounded once
 * to `dtype`: the result is bitwise reproducible.
 *   expert_out     [max_rows,h] dtype
 *   permuted_probs [max_rows]   fp32
 *   row_id_map     [T,K]        int32   entries outside [0, max_rows) are skipped
 *   shared_out     [T,h]        dtype or NULL
 *   out            [T,h]        dtype   out
 * h must be a multiple of 8.
 * ------------------------------------------------------------------------ */
moe_status moe_combine(int64_t T, int64_t h, int64_t K, int32_t dtype, const void* expert_out,
                       const float* permuted_probs, const int32_t* row_id_map, int64_t max_rows,
                       const void* shared_out, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
