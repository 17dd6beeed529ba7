/*
 * moe_nvfp4.h -- C ABI of the routed NVFP4 mixture-of-experts FFN and the MXFP8
 * block-scaled projection, for AMD Instinct MI355X (gfx950).
 *
 * The layer (as described on the pages "NVIDIA FP4-Local checkpoints on DGX Spark
 * (TP=1, TP=2): format, model and speed plan in rounds #565", §4 Round 1, and
 * "bloomery 0.3.9" release notes, New / From our contributors):
 *   1. moe_route_topk        route a whole batch of tokens in one run: top-k experts
 *                            per token, renormalized softmax weights, and per-expert
 *                            row lists so every selected expert is read once (#740, #808);
 *   2. moe_expert_ffn_nvfp4  per routed row: gate and up products, SwiGLU, down product,
 *                            over NVFP4 weights held as stored -- U8 bytes of two E2M1
 *                            codes, one F8_E4M3 scale per 16-element block, one fp32
 *                            scale per expert tensor (#489, #517, #545, #766);
 *   1+2. moe_route_expert_ffn_nvfp4  both in one launch for a few tokens;
 *   1+2+3. moe_layer_nvfp4   the whole layer in one launch for a few tokens (optionally with
 *                            a gated shared expert and the residual);
 *   3. moe_combine           the router-weighted sum of each token's expert rows (#701);
 *                            moe_combine_shared adds a gated shared expert's rows (#686),
 *                            moe_combine_residual also the block's residual stream;
 *   0. moe_router_logits     the router projection that produces the logits step 1 takes:
 *                            activations times the router matrix kept in its stored BF16
 *                            words, summed in fp32 (#732, #763);
 *   4. mxfp8_gemm            y = x . W^T for MXFP8 weights: E4M3 elements in blocks of 32
 *                            along K with one E8M0 scale a block, as a gemv (M = 1) and a
 *                            wide GEMM (#521); mxfp8_quantize + mxfp8_gemm_mx, the same
 *                            product with MXFP8 activations (W8A8, #769).
 *
 * Conventions for every entry point
 *   - Every data pointer is a DEVICE pointer, allocated and owned by the caller; the
 *     library never allocates, frees or retains memory. Its only global state is a
 *     per-process call counter (moe_expert_ffn_nvfp4 tags its workspace words with it),
 *     the wait limit and the per-device flag of moe_async_status, and device properties
 *     cached per device (behind a lock: every entry point may be called from several
 *     host threads).
 *   - `stream` is a hipStream_t (NULL = the default stream). A call only enqueues work
 *     on it; results are valid once the stream reaches the call.
 *   - Calls may be captured in a HIP graph. A few-token FFN or layer call (T <= 16) tags the
 *     words it hands between workgroups with a per-call value; a kernel argument would be
 *     frozen in the graph, so under capture such a call also captures a one-thread kernel
 *     that advances a word kept at the end of its workspace, and every replay reads its own
 *     tag from there (the workspace queries include that word). Replays see the inputs as
 *     they are when they run.
 *   - Arguments are checked on the host before any HIP call; a call that returns a
 *     non-zero status has enqueued nothing, except MOE_E_LAUNCH (a launch failed; the
 *     HIP error text is available from moe_last_error()).
 *   - Every pointer must be 16-byte aligned (a misaligned view is refused at the call,
 *     after the pages' practice [#565 page, §10, #520]), except where an entry point says
 *     otherwise (moe_layer_nvfp4's shared_gate_logit).
 *   - Unsafe contract (documented, not checked on the device): router logits are finite;
 *     no E4M3 NaN codes (0x7F, 0xFF) in block scales or MXFP8 weights, no E8M0 0xFF;
 *     tensor scales are finite; outputs do not alias inputs; calls that share a
 *     workspace are ordered on one stream.
 *   - Element layouts (row-major):
 *       bf16 tensors are uint16_t bit patterns;
 *       NVFP4 codes: byte j of a row holds element 2j in its low nibble and element 2j+1
 *       in its high nibble; E2M1 = sign | 2 exponent bits (bias 1) | 1 mantissa bit;
 *       E4M3 = the "fn" variant (bias 7, no inf, S.1111.111 = NaN);
 *       E8M0 = 2^(c - 127).
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes; moe_status_string() names them. */
enum {
  MOE_OK = 0,
  MOE_E_NULL = 1,      /* a required pointer is NULL                                  */
  MOE_E_SHAPE = 2,     /* a size is out of range (see each entry point)               */
  MOE_E_ALIGN = 3,     /* a pointer is not 16-byte aligned                             */
  MOE_E_WORKSPACE = 4, /* workspace NULL or smaller than the size query returns        */
  MOE_E_LAUNCH = 5,    /* a HIP launch failed; see moe_last_error()                    */
  MOE_E_POLICY = 6,    /* an unknown routing policy                                   */
  MOE_E_WAIT_EXPIRED = 7 /* moe_async_status: a few-token launch gave up a wait          */
};

/* Routing normalization policies (moe_route_topk_policy). The pages make the router's
 * normalization policy a named value ("bloomery 0.3.9" release notes, From our
 * contributors, #772) without listing the values; these are the ones offered. */
enum {
  MOE_ROUTE_SOFTMAX_RENORM = 0, /* softmax over the selected k logits (= softmax, top k, renormalize) */
  MOE_ROUTE_SOFTMAX = 1,        /* the selected entries of the softmax over all E logits           */
  MOE_ROUTE_SIGMOID_RENORM = 2, /* sigmoid of each selected logit, divided by their sum            */
  MOE_ROUTE_SIGMOID = 3         /* sigmoid of each selected logit                                  */
};

/* One routed NVFP4 expert stack, stacked over the E experts, bytes as stored. The
 * struct itself lives in host memory; its members are device pointers. */
typedef struct moe_nvfp4_experts {
  const uint8_t* gate_q;  /* [E][f][d/2]   E2M1 pairs                                    */
  const uint8_t* gate_s;  /* [E][f][d/16]  E4M3 block scales (block = 16 along K = d)    */
  const float* gate_ts;   /* [E]           fp32 tensor scale of each expert's gate       */
  const uint8_t* up_q;    /* [E][f][d/2]                                                 */
  const uint8_t* up_s;    /* [E][f][d/16]                                                */
  const float* up_ts;     /* [E]                                                         */
  const uint8_t* down_q;  /* [E][d][f/2]                                                 */
  const uint8_t* down_s;  /* [E][d][f/16]  (block = 16 along K = f)                      */
  const float* down_ts;   /* [E]                                                         */
} moe_nvfp4_experts;

/* ---------------------------------------------------------------------------------
 * moe_route_topk -- top-k routing of a whole batch, and the per-expert row lists.
 *
 * Per token t (logits[t][0..E-1], fp32): the k experts with the largest logits, ordered
 * by (logit descending, expert index ascending; -0.0 equals +0.0) -> topk_ids[t][0..k-1];
 * topk_w[t][j] = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), a softmax over the experts
 * renormalized to the selected k (the router normalization policy is named on
 * "bloomery 0.3.9" release notes, Fixed (#772); this is the renormalized-softmax one).
 *
 * Row lists (assignment a = t*k + j, T*k assignments):
 *   expert_offsets[E+1]: exclusive prefix sum of the per-expert counts, [E] = T*k;
 *   sorted_rows[T*k]:   for e = 0..E-1, every a with topk_ids.flat[a] == e in increasing a
 *                       (a stable counting sort: bit-for-bit deterministic);
 *   row_of[T*k]:        the inverse, row_of[sorted_rows[p]] = p.
 *
 * Sizes: 1 <= T, 1 <= E <= 1024, 1 <= k <= min(E, 32), T*k < 2^31.
 * Workspace: at least moe_route_topk_workspace(T, E, k) bytes of device memory
 * (0 is valid when the query returns 0; pass NULL then).
 */
size_t moe_route_topk_workspace(int T, int E, int k);
int moe_route_topk(const float* logits, int T, int E, int k,
                   int32_t* topk_ids, float* topk_w,
                   int32_t* expert_offsets, int32_t* sorted_rows, int32_t* row_of,
                   void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_route_topk_policy -- moe_route_topk under a named normalization policy (the
 * MOE_ROUTE_* values above; MOE_ROUTE_SOFTMAX_RENORM with bias NULL is moe_route_topk)
 * and an optional correction bias.
 *
 * bias: NULL, or fp32 [E] (16-byte aligned). With a bias the choice is made on the
 * fp32 sums logits[t][e] + bias[e] (ordered as above); the weights always use the
 * unbiased logits of the chosen experts:
 *   MOE_ROUTE_SOFTMAX_RENORM  w_j = exp(l_j) / sum over the k chosen of exp(l);
 *   MOE_ROUTE_SOFTMAX         w_j = exp(l_j) / sum over all E experts of exp(l);
 *   MOE_ROUTE_SIGMOID_RENORM  w_j = s_j / sum over the k chosen of s, s = 1 / (1 + exp(-l));
 *   MOE_ROUTE_SIGMOID         w_j = 1 / (1 + exp(-l_j)).
 * Row lists, sizes and workspace as for moe_route_topk. An unknown policy returns
 * MOE_E_POLICY. Unsafe contract: logits[t][e] + bias[e] is finite.
 */
int moe_route_topk_policy(const float* logits, int T, int E, int k, int policy, const float* bias,
                          int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                          int32_t* sorted_rows, int32_t* row_of, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_expert_ffn_nvfp4 -- the expert FFN of every routed row, in row-list order.
 *
 * For row-list position p of expert e (expert_offsets[e] <= p < expert_offsets[e+1]) and
 * token t = sorted_rows[p] / k, with W[n][i] = E2M1(code) * E4M3(scale[n][i/16]) (exact):
 *   G = gate_ts[e] * (x[t] . W_gate[e]^T)      fp32 accumulation     [f]
 *   U = up_ts[e]   * (x[t] . W_up[e]^T)                                [f]
 *   H = bf16_rne(silu(G) * U)                  silu(g) = g / (1 + exp(-g))
 *   y_rows[p] = down_ts[e] * (H . W_down[e]^T) fp32, not rounded       [d]
 * x is bf16 [T][d]; y_rows is fp32 [T*k][d]. expert_offsets / sorted_rows are the
 * device outputs of moe_route_topk for the same T, E, k.
 * Sizes: 1 <= T, d and f multiples of 32 (>= 32), 1 <= E <= 1024, 1 <= k <= min(E, 32).
 * Workspace: at least moe_expert_ffn_nvfp4_workspace(T, d, f, E, k) bytes (holds H and, for
 * batches, two work counters that each call clears itself; no initial contents needed). Calls that share a workspace must be ordered on one stream;
 * calls with different workspaces may run concurrently on different streams.
 * Few tokens (T <= 16, d <= 4096, f <= 1024 and T * (max(d, f) + 8) * 2 <= 64 KiB) run as
 * one launch in which the down-product workgroups wait for the gate/up workgroups of the
 * same expert. The launch has as many workgroups as the GPU holds at once, but the
 * waits do not depend on them all being resident (work on other streams or processes
 * can keep some from starting): a down-product workgroup that still misses some of its
 * expert's H slices after a number of polls computes those gate/up items itself, with
 * the same code, so the results are the same bits either way. As a last guard a wait
 * gives up after a bound (moe_set_wait_limits): the affected y_rows are then NaN and
 * moe_async_status reports MOE_E_WAIT_EXPIRED; that cannot happen with the defaults.
 */
size_t moe_expert_ffn_nvfp4_workspace(int T, int d, int f, int E, int k);
int moe_expert_ffn_nvfp4(const uint16_t* x, int T, int d, int f, int E, int k,
                         const moe_nvfp4_experts* w,
                         const int32_t* expert_offsets, const int32_t* sorted_rows,
                         float* y_rows, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_expert_ffn_nvfp4_scratch -- moe_expert_ffn_nvfp4 that allocates nothing and takes no
 * workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid it). H lives in a static device
 * array of MOE_SCRATCH_BYTES that the library holds on every device it runs on for the
 * life of the process. Arguments, results and refusals as moe_expert_ffn_nvfp4; a shape
 * whose moe_expert_ffn_nvfp4_workspace exceeds MOE_SCRATCH_BYTES is refused with
 * MOE_E_WORKSPACE (moe_last_error says how many bytes it needs). Every call on a device
 * shares that device's array: calls that overlap on one device (different streams or
 * host threads) race and must not be made; calls ordered on one stream are fine (the
 * array keeps the last call's contents, which no call needs cleared). The first call on
 * a device looks up the array's address (no allocation).
 */
#define MOE_SCRATCH_BYTES ((size_t)32 << 20)
int moe_expert_ffn_nvfp4_scratch(const uint16_t* x, int T, int d, int f, int E, int k,
                                 const moe_nvfp4_experts* w,
                                 const int32_t* expert_offsets, const int32_t* sorted_rows,
                                 float* y_rows, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_route_expert_ffn_nvfp4 -- moe_route_topk (default policy, no bias) and
 * moe_expert_ffn_nvfp4 in one launch, for few tokens: the launch routes its tokens itself
 * (a whole batch routed in one run, "NVIDIA FP4-Local checkpoints on DGX Spark" page,
 * §4 Round 1, #740) instead of waiting for a routing launch, and writes the same routing
 * outputs (topk_ids, topk_w, expert_offsets, sorted_rows, row_of: bit-identical to
 * moe_route_topk's) and y_rows (as moe_expert_ffn_nvfp4's few-token path).
 * Sizes: those of the few-token path of moe_expert_ffn_nvfp4 (T <= 16, d <= 4096,
 * f <= 1024, T * (max(d, f) + 8) * 2 <= 64 KiB), E <= 256, k <= 16; otherwise
 * MOE_E_SHAPE (call the two entry points instead). Workspace: moe_expert_ffn_nvfp4_workspace.
 */
int moe_route_expert_ffn_nvfp4(const float* logits, const uint16_t* x, int T, int d, int f, int E, int k,
                               const moe_nvfp4_experts* w, int32_t* topk_ids, float* topk_w,
                               int32_t* expert_offsets, int32_t* sorted_rows, int32_t* row_of,
                               float* y_rows, void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_layer_nvfp4 -- the whole routed layer for few tokens in one launch: routing (default
 * policy, no bias), the routed experts' FFN, an optional shared expert, and the combine
 *   out[t] = bf16_rne( sum_j topk_w[t][j] * y[row_of[t*k+j]]  (+ g_t * S[t])  (+ residual[t]) ),
 * g_t = 1 / (1 + exp(-shared_gate_logit[t * gate_ld])) (1 without a gate logit), summed in
 * fp32 in that order and rounded once: the same bits as moe_route_topk, moe_expert_ffn_nvfp4
 * (for the shared expert: one expert, offsets {0, T}, row p = token p) and
 * moe_combine_residual / moe_combine_shared / moe_combine called one after the other. The
 * pages route a whole batch in one run (#740), fold the expert sum into the combine (#701)
 * and the shared expert's add into its producer ("NVIDIA FP4-Local checkpoints on DGX
 * Spark" page, §4 Round 1 and §4 remaining items); here all of it is one launch, and the
 * block whose down product completes a token's 128-column tile (an arrival counter per
 * token and tile, in the workspace) sums that tile: no block waits for work that has not
 * started, so the launch does not depend on all of its blocks being resident.
 * logits fp32, row t at logits + t * logits_ld (logits_ld >= E, 0 means E; columns past E are
 * not read, so a router that also projects the shared gate may leave its logit in column E);
 * x bf16 [T][d]; w the routed experts; shared NULL or one expert of the same d and f;
 * shared_gate_logit NULL or fp32, token t's at shared_gate_logit[t * gate_ld] (4-byte
 * aligned; given only with a shared expert); residual NULL or bf16 [T][d]; out bf16 [T][d].
 * topk_ids, topk_w, expert_offsets, sorted_rows, row_of: each NULL or written as by
 * moe_route_topk. Sizes: those of moe_route_expert_ffn_nvfp4 (T <= 16, d <= 4096, f <= 1024,
 * T * (max(d, f) + 8) * 2 <= 64 KiB, E <= 256, k <= 16); otherwise MOE_E_SHAPE (the
 * workspace query returns 0). Workspace: at least moe_layer_nvfp4_workspace(T, d, f, E, k,
 * shared != NULL) bytes, zero-filled before its first use (it starts with the arrival
 * counters, which every call leaves at zero; the rest needs no contents); calls that share
 * it must be ordered on one stream. A workspace that was not zero-filled is reported by
 * moe_async_status (MOE_E_WAIT_EXPIRED), with some out elements NaN or not written. Waits:
 * as moe_expert_ffn_nvfp4's few-token path (moe_async_status reports a wait that gave up;
 * its out elements are then NaN).
 */
size_t moe_layer_nvfp4_workspace(int T, int d, int f, int E, int k, int with_shared);
int moe_layer_nvfp4(const float* logits, int logits_ld, const uint16_t* x, int T, int d, int f, int E, int k,
                    const moe_nvfp4_experts* w, const moe_nvfp4_experts* shared, const float* shared_gate_logit,
                    int gate_ld, const uint16_t* residual, int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                    int32_t* sorted_rows, int32_t* row_of, uint16_t* out, void* workspace, size_t workspace_bytes,
                    void* stream);

/* ---------------------------------------------------------------------------------
 * moe_combine -- out[t][c] = bf16_rne( sum_{j=0..k-1} topk_w[t][j] * y_rows[row_of[t*k+j]][c] ),
 * summed in fp32 in j order (so the result is deterministic), rounded once.
 * Sizes: 1 <= T, 1 <= k <= 32, d a multiple of 32 (>= 32).
 */
int moe_combine(const float* y_rows, const int32_t* row_of, const float* topk_w,
                int T, int k, int d, uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_combine_shared -- moe_combine with a shared expert's rows added (the pages run a
 * shared expert beside the routed ones, "NVIDIA FP4-Local checkpoints on DGX Spark"
 * page, §4 Round 1, #686, and fold its add into the producing kernel, §4 remaining items):
 *   out[t][c] = bf16_rne( sum_j topk_w[t][j] * y_rows[row_of[t*k+j]][c] + g_t * shared_rows[t][c] ),
 *   g_t = 1 / (1 + exp(-shared_gate_logit[t])), or 1 when shared_gate_logit is NULL;
 * the routed sum in j order, the shared term added last, one rounding.
 * shared_rows fp32 [T][d]: the shared expert's output rows, e.g. moe_expert_ffn_nvfp4 with
 * one expert (E = 1, k = 1, expert_offsets = {0, T}, sorted_rows[p] = p); shared_gate_logit
 * fp32 [T] (NULL allowed), e.g. moe_router_logits with the gate vector as a one-row router.
 * Sizes and alignment as for moe_combine; shared_rows is required (MOE_E_NULL).
 */
int moe_combine_shared(const float* y_rows, const int32_t* row_of, const float* topk_w,
                       int T, int k, int d, const float* shared_rows,
                       const float* shared_gate_logit, uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_combine_residual -- the block's output with its residual stream: the pages fold the
 * adds that follow a producer into it ("NVIDIA FP4-Local checkpoints on DGX Spark" page,
 * §4 remaining items; §4 Round 1, #701):
 *   out[t][c] = bf16_rne( sum_j topk_w[t][j] * y_rows[row_of[t*k+j]][c]
 *                         + g_t * shared_rows[t][c] + residual[t][c] ),
 * the routed sum in j order, then the shared term (omitted when shared_rows is NULL; g_t as
 * for moe_combine_shared), then the residual, in fp32, rounded once. residual bf16 [T][d]
 * (the block's input activations). shared_gate_logit without shared_rows: MOE_E_NULL.
 * Sizes and alignment as for moe_combine.
 */
int moe_combine_residual(const float* y_rows, const int32_t* row_of, const float* topk_w,
                         int T, int k, int d, const float* shared_rows,
                         const float* shared_gate_logit, const uint16_t* residual,
                         uint16_t* out, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_router_logits -- logits[t][e] = sum_i x[t][i] * w_r[e][i], fp32 accumulation
 * ("NVIDIA FP4-Local checkpoints on DGX Spark" page, §4 Round 1: the router read as the
 * checkpoint's BF16 words, #732; the routers' prompt logits on a float32 tile, #763).
 * x bf16 [T][d] (the layer's activations), w_r bf16 [E][d] (the router matrix, one row
 * an expert), logits fp32 [T][E] -- the input of moe_route_topk.
 * Sizes: T, E >= 1, E <= 2^20, d a multiple of 32 (>= 32), T * d * 2 < 2^31 and
 * E * d * 2 < 2^31. The sum over i is taken in a fixed order (deterministic); it differs
 * from the exact sum by at most (d + 8) * 2^-24 * sum_i |x[t][i] * w_r[e][i]|.
 */
int moe_router_logits(const uint16_t* x, const uint16_t* w_r, int T, int d, int E,
                      float* logits, void* stream);

/* ---------------------------------------------------------------------------------
 * mxfp8_gemm -- y[m][n] = bf16_rne( sum_i x[m][i] * W[n][i] ), fp32 accumulation,
 * W[n][i] = E4M3(w[n][i]) * 2^(s[n][i/32] - 127) (exact in bf16 for the scales in use).
 * x bf16 [M][K], w E4M3 [N][K], s E8M0 [N][K/32], y bf16 [M][N].
 * Sizes: M, N >= 1, K a multiple of 32 (>= 32), M * K * 2 < 2^31 and N * K < 2^31.
 * M > 16 runs as a tiled GEMM (128 x 192 output tiles). M <= 16 runs the kernel
 * mxfp8_autotune picked for (this device, M, N, K), or without a pick the vector-ALU
 * gemv for M <= 4 and the MFMA gemv up to 16.
 */
int mxfp8_gemm(const uint16_t* x, int M, int N, int K,
               const uint8_t* w, const uint8_t* s, uint16_t* y, void* stream);

/* ---------------------------------------------------------------------------------
 * moe_async_status -- waits for `stream`, then reports whether any few-token launch on
 * the current device gave up a wait since the last report (MOE_E_WAIT_EXPIRED; its
 * affected y_rows are then NaN) or not (MOE_OK), and clears the flag. The flag is one
 * per device and process. A HIP error while waiting returns MOE_E_LAUNCH. The pages
 * refuse bad results by name rather than pass them on silently [#565 page, §9 Rules and
 * related work, Accuracy]; this is the report for the one condition that only the
 * device sees.
 */
int moe_async_status(void* stream);

/* moe_set_wait_limits -- the polls of the few-token launch's waits, for the calls
 * enqueued after it, process-wide: `steal_after` polls of a missing H slice before a
 * down-product workgroup computes the missing gate/up items itself (default 256), and
 * `give_up` polls of its full H read before it writes NaN rows and raises the flag of
 * moe_async_status (default 1048576); each poll is followed by a short sleep. Stealing
 * happens only when steal_after < give_up. Test hooks: (0, default) makes every
 * down-product workgroup that finds H missing compute it itself (the results stay the
 * same bits); (0, 0) gives up at once, forcing the guard's exit path without any fault.
 * moe_get_wait_limits reads the current values (either pointer may be NULL). */
void moe_set_wait_limits(uint32_t steal_after, uint32_t give_up);
void moe_get_wait_limits(uint32_t* steal_after, uint32_t* give_up);

/* ---------------------------------------------------------------------------------
 * moe_read_ceiling -- a measurement helper, not a step of the layer: reads the given byte
 * ranges once with plain coalesced 16-byte loads (the expert kernels' non-temporal hint)
 * and nothing else, so that a benchmark can report the expert kernels against the rate
 * this part reads the same bytes at (the pages measure against a baseline, "NVIDIA
 * FP4-Local checkpoints on DGX Spark" page, §3 How results are measured).
 * ranges: device memory, n pairs (device address, byte count), each a multiple of 16 and
 * 16-byte aligned, total_bytes their sum; 1 <= n <= 1024. sink: device uint32 [sink_words]
 * (one word a workgroup; at most sink_words workgroups). Contents of sink: unspecified.
 */
int moe_read_ceiling(const uint64_t* ranges, int n, uint64_t total_bytes, uint32_t* sink, int sink_words,
                     void* stream);

/* ---------------------------------------------------------------------------------
 * mxfp8_autotune -- picks the fastest few-row MXFP8 kernel for this card: for every
 * M = 1 .. M_max (<= 16) it times the vector-ALU gemv (M <= 8), the MFMA gemv and the
 * tiled GEMM on the caller's operands (one warm-up and `reps` launches each on `stream`,
 * HIP events; the call waits for them) and records the fastest for (current device, M,
 * N, K); later mxfp8_gemm calls of that shape use it (the multi-column gemv picked per
 * card, "bloomery 0.3.13" release notes, Also: an autotuned MXFP8 gemv at 4-8 columns).
 * x bf16 [M_max][K], w [N][K], s [N][K/32], y bf16 [M_max][N] (overwritten). Optional
 * outputs: picks int [M_max] (kernel ids: 0 vector-ALU gemv, 1 MFMA gemv, 2 tiled GEMM),
 * us float [M_max][3] (microseconds a launch; entries of kernels not timed untouched).
 * Every kernel gives results within the band of the same definition; the pick changes
 * only the speed. Thread-safe; the records last for the process.
 */
int mxfp8_autotune(const uint16_t* x, int M_max, int N, int K, const uint8_t* w, const uint8_t* s,
                   uint16_t* y, int reps, int* picks, float* us, void* stream);

/* mxfp8_force_kernel -- a test hook: every later mxfp8_gemm call with M <= 16 runs the
 * given kernel id (0, 1, 2 as above; 0 only for M <= 8, otherwise the MFMA gemv), or
 * follows the records again with -1. Process-wide. Other values: MOE_E_SHAPE. */
int mxfp8_force_kernel(int kernel);

/* ---------------------------------------------------------------------------------
 * moe_ffn_autotune -- picks the faster few-token path of moe_expert_ffn_nvfp4 for this card
 * and shape (the multi-column NVFP4 decode picked per card, "NVIDIA FP4-Local checkpoints
 * on DGX Spark" page, §4 remaining items, and "bloomery 0.3.13" release notes, Also): for
 * T <= 16 (every expert then has at most 16 rows) it times, on the caller's operands and
 * routing, the one-launch decode kernel (path 0; only within its size limits, see
 * moe_expert_ffn_nvfp4) and the two weight-streaming kernels (path 1), one warm-up and
 * `reps` calls each on `stream` (HIP events; the call waits for them), and records the
 * faster for (current device, T, d, f, E, k): later moe_expert_ffn_nvfp4 calls of that
 * shape take it (without a record: path 0 where it applies, else path 1). Arguments as
 * moe_expert_ffn_nvfp4 (y_rows and the workspace are overwritten), plus reps >= 1 and the
 * optional outputs pick (the path recorded) and us float [2] (microseconds a call; the
 * entry of a path not timed is untouched). Both paths give results within the band of the
 * same definition (their fp32 sums run in different orders); the pick changes only the
 * speed. Thread-safe; the records last for the process. T > 16: MOE_E_SHAPE.
 */
int moe_ffn_autotune(const uint16_t* x, int T, int d, int f, int E, int k, const moe_nvfp4_experts* w,
                     const int32_t* expert_offsets, const int32_t* sorted_rows, float* y_rows, void* workspace,
                     size_t workspace_bytes, int reps, int* pick, float* us, void* stream);

/* moe_ffn_force_path -- a test hook: every later few-token moe_expert_ffn_nvfp4 call takes
 * path 0 (the decode kernel, where its size limits allow it; otherwise path 1) or path 1
 * (the streaming kernels), or follows the records again with -1. Process-wide. Other
 * values: MOE_E_SHAPE. */
int moe_ffn_force_path(int path);

/* ---------------------------------------------------------------------------------
 * mxfp8_quantize -- bf16 activations to MXFP8 (the W8A8 variant of the MXFP8 projection,
 * "NVIDIA FP4-Local checkpoints on DGX Spark" page, §4 Round 1, #769), by the OCP MX v1.0
 * conversion: per block of 32 along K, the E8M0 scale code is
 * clamp(floor(log2 max|v|) - 8 + 127, 0, 254) (0 for an all-zero block) and each element
 * is v / scale rounded to the nearest E4M3 value, ties to even, saturated to +-448 (the
 * sign of zero kept).
 * x bf16 [M][K] -> xq E4M3 [M][K], xs E8M0 [M][K/32]. Sizes: M >= 1, K a multiple of 32,
 * M * K * 2 < 2^31. Unsafe contract: x finite.
 */
int mxfp8_quantize(const uint16_t* x, int M, int K, uint8_t* xq, uint8_t* xs, void* stream);

/* ---------------------------------------------------------------------------------
 * mxfp8_gemm_mx -- y[m][n] = bf16_rne( sum_i X[m][i] * W[n][i] ) with MXFP8 activations
 * X = E4M3(xq) * 2^(xs - 127) (mxfp8_quantize) and MXFP8 weights as for mxfp8_gemm, both
 * scales applied by gfx950's block-scaled matrix instruction, fp32 accumulation.
 * xq [M][K], xs [M][K/32], w [N][K], s [N][K/32], y bf16 [M][N]. Sizes: M, N >= 1, K a
 * multiple of 512, at most 4096; M * K and N * K < 2^31. The results differ from
 * mxfp8_gemm's by the activation quantization (beyond the bf16 band); against the W8A8
 * definition they are within it.
 */
int mxfp8_gemm_mx(const uint8_t* xq, const uint8_t* xs, int M, int N, int K,
                  const uint8_t* w, const uint8_t* s, uint16_t* y, void* stream);

/* Name of a status code ("MOE_OK", "MOE_E_SHAPE", ...); never NULL. */
const char* moe_status_string(int status);
/* Text of the last HIP error seen by a call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_NVFP4_H */
