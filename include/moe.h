/*
 * moe.h -- C ABI of the MI355X (gfx950) routed-expert MoE layer library
 * (libmoe.so).
 *
 * The layer: a sigmoid top-k router with a per-expert selection bias, per-
 * expert token bucketing, a SwiGLU expert FFN over packed int4 / int8 / int2
 * weights with fp32 per-row scales and int8 activations (exact int32 integer
 * dot products, dequantisation on use), and a weighted combine with an
 * always-on shared expert.
 *
 * Pages the operations come from:
 *  [P-feat]  agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on consumer
 *            hardware", section "Key features": int8, packed int4 and packed
 *            int2 kernels with per-row scales and dequantisation on use; int8
 *            matmuls computed as integer dot products.
 *  [P-mem]   same page, section "Memory split": shared experts stay resident;
 *            a routed int4 expert is about 19 MB (three 6144 x 2048 matrices).
 *  [P-load]  same page, section "Loading mechanism": a per-layer LRU keeps
 *            experts resident; the next block is read while the current one
 *            is computed.
 *  [P-route] tech.takumi3488.com, "Trying colibri", self-test section: a
 *            DeepSeek-V3-family router; section on the real 744B model:
 *            hidden 6144, 256 experts per layer, top-8.
 *  [P-moe]   remio.ai, "Colibri shows how to run GLM-5.2 on a low-spec PC",
 *            section "How Colibri runs GLM-5.2": the router picks a few
 *            feed-forward experts per token.
 *  [P-dedup] same page, section "The RAM wall became a storage problem": an
 *            expert requested by several batch positions is read once; an
 *            expert's matrices are stored together and fetched in one go.
 *  [P-topp]  agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on consumer
 *            hardware", measured-benchmark table and community remarks: the
 *            --topp 0.7 setting loads fewer experts per token (1.6x end to
 *            end on a RAM-bound machine).
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors)
 *    unless the parameter name ends in _host. Arrays are row-major and
 *    contiguous; device pointers must be 16-byte aligned.
 *  - H (hidden) and I (expert intermediate) must be positive multiples of 64
 *    and at most 8192. T (tokens) may be 0 (the call does nothing).
 *  - Every call enqueues work on the context's stream and returns without
 *    synchronising (unless stated); kernel faults surface at the caller's next
 *    synchronisation. Invalid arguments are rejected before anything is
 *    enqueued.
 *  - Ownership: the caller owns every tensor it passes; the library never
 *    frees caller memory. The library owns only the context's scratch memory
 *    and pools. Scratch grows on demand with hipMalloc when a call needs more
 *    than the context holds; a buffer it outgrows is kept, not freed, until
 *    moe_ctx_destroy, so work already enqueued and HIP graphs captured from
 *    earlier calls keep valid addresses (an eager call at a larger size
 *    between two replays of a graph is safe). A call made during graph
 *    capture that needs to grow the scratch fails (hipMalloc cannot be
 *    captured): run one call at the largest size before capturing.
 *  - A context is bound to one device and one stream and is not thread-safe;
 *    calls on one context must not overlap.
 *  - Errors: every call returns a moe_status; on failure moe_last_error()
 *    returns a thread-local description. No C++ exception crosses the ABI.
 *
 * Packed weight layout (bit-exact contract, [P-feat]): per-row symmetric
 * absmax quantisation, qmax = 2^(bits-1)-1, scale s = max|w| / qmax (fp32),
 * codes q = clamp(rint(w/s), -qmax, qmax) (round half to even); int8 codes
 * are two's-complement bytes; int4 codes are nibbles q+8 with element 2i in
 * the low nibble of byte i; int2 codes are 2-bit fields q+2 with element 4i+j
 * in bits 2j..2j+1 of byte i. Rows are contiguous with no padding.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,       /* bad argument (shape, pointer, alignment, value) */
  MOE_ENOMEM = -2,       /* device or host allocation failed */
  MOE_EHIP = -3,         /* a HIP runtime call failed (text in moe_last_error) */
  MOE_EUNSUPPORTED = -4, /* valid but outside what the kernels handle */
  MOE_EPOOL = -5,        /* expert pool cannot satisfy the request */
  MOE_ETIMEOUT = -6      /* a bounded device-side wait gave up (see moe_ctx_check) */
} moe_status;

typedef struct moe_ctx moe_ctx;

/* One expert's weights: device pointers, layout as above.
 * gate, up: [I][H*bits/8]; down: [H][I*bits/8]; s_gate, s_up: [I]; s_down: [H]. */
typedef struct {
  const uint8_t *gate, *up, *down;
  const float *s_gate, *s_up, *s_down;
} moe_expert_w;

/* Router configuration ([P-route], [P-moe]).
 * n_experts: E routed experts (1..1024); top_k: k (1..min(E, 16));
 * routed_scale: factor applied to the normalised weights (1.0 for plain
 * normalisation); logits_in: 0 = the router computes logits from hidden
 * states, 1 = the caller passes logits [T][E]; top_p ([P-topp]): 0 (or less)
 * keeps all k experts; otherwise, in rank order, the normalised weights
 * sig_j / sum_k sig accumulate (fp32, in that order) and only the shortest
 * prefix whose cumulative weight reaches top_p is kept (all k if none does),
 * its weights renormalised over the kept experts; the other slots get id -1
 * and weight 0. */
typedef struct {
  int n_experts;
  int top_k;
  float routed_scale;
  int logits_in;
  float top_p;
} moe_router_cfg;

/* ---------------------------------------------------------------------- */
/* Context                                                                */
/* ---------------------------------------------------------------------- */

/* Create a context on `device`. hip_stream: a hipStream_t to borrow (the
 * caller keeps it alive), or NULL for the null stream. */
moe_status moe_ctx_create(int device, void *hip_stream, moe_ctx **out);
/* Free the context's scratch memory. Waits for the stream first. */
void moe_ctx_destroy(moe_ctx *ctx);
/* Re-bind the context to another stream of the same device. */
moe_status moe_ctx_set_stream(moe_ctx *ctx, void *hip_stream);
/* Thread-local text of the last failure ("" if none). */
const char *moe_last_error(void);
int moe_abi_version(void);
/* Which kernels compute the expert FFN of moe_expert_ffn_q* and of the
 * multi-token path of moe_layer_forward. MOE_FFN_AUTO (the default), from
 * the measured crossover at the GLM shape: up to 3 tokens the single-token
 * kernels of the whole-layer decode path (without its router and combine)
 * run once per token, where the shape fits them; from 4 tokens on the int8
 * matrix-core kernels, whose tiles read each expert once for all its
 * tokens; the vector dot-product kernels where neither takes the shape.
 * MOE_FFN_DOT4: always the vector kernels. MOE_FFN_MFMA: always the
 * matrix-core kernels. All take every shape they are chosen for and compute
 * the same exact integer sums and the same fp32 epilogue, so their results
 * are bit-identical. Any other value: MOE_EINVAL.
 * Host-only setting; enqueues nothing. */
enum { MOE_FFN_AUTO = 0, MOE_FFN_DOT4 = 1, MOE_FFN_MFMA = 2 };
moe_status moe_ctx_set_ffn_kernels(moe_ctx *ctx, int which);
/* Synchronise the stream and report device-side errors recorded by earlier
 * calls (a bounded wait that gave up -> MOE_ETIMEOUT). Clears the record. */
moe_status moe_ctx_check(moe_ctx *ctx);

/* One expert as a single contiguous block ([P-dedup]: an expert's matrices
 * are stored together and fetched in one read): gate | up | down | s_gate |
 * s_up | s_down, each part starting on a 256-byte boundary. Writes the six
 * byte offsets to offsets_host[6] (nullable) and returns the block size in
 * bytes, or 0 for invalid arguments (bits not in {8,4,2}, H or I not a
 * positive multiple of 64). Host-only; enqueues nothing. At bits 4, H 6144,
 * I 2048 the block is 18,915,328 bytes (the pages' "about 19 MB"). */
size_t moe_expert_block_layout(int bits, int H, int I, size_t *offsets_host);

/* ---------------------------------------------------------------------- */
/* Quantisation ([P-feat])                                                */
/* ---------------------------------------------------------------------- */

/* Quantise and pack rows of w (fp32 [rows][cols]) at bits in {8,4,2}:
 * packed uint8 [rows][cols*bits/8], scales fp32 [rows]. cols must be a
 * positive multiple of 64. Bit-exact contract as in the header comment. */
moe_status moe_quantize_rows(moe_ctx *ctx, int bits, const float *w, int64_t rows, int cols, uint8_t *packed,
                             float *scales);

/* Per-token int8 quantisation of hidden states: x fp32 [T][H] ->
 * xq int8 [T][H], sx fp32 [T]; sx = max|x| / 127, xq = clamp(rint(x/sx)).
 * A zero row gives sx = 0 and xq = 0. */
moe_status moe_quantize_act_i8(moe_ctx *ctx, const float *x, int T, int H, int8_t *xq, float *sx);

/* ---------------------------------------------------------------------- */
/* Router ([P-route], [P-moe])                                            */
/* ---------------------------------------------------------------------- */

/* logits z = x w_router^T (x fp32 [T][H], w_router fp32 [E][H]; fp32
 * arithmetic) or z = x when cfg->logits_in (x is fp32 [T][E], w_router
 * ignored, H ignored). sig = 1/(1+exp(-z)); key = sig + bias[e] (bias fp32
 * [E] or NULL); topk_idx int32 [T][k] = experts with the k largest keys in
 * descending key order (equal keys: lower id first); topk_w fp32 [T][k] =
 * routed_scale * sig / sum of the selected sig (the bias selects, it does not
 * weight). With cfg->top_p > 0 the selection is truncated as described at
 * moe_router_cfg: dropped slots hold id -1 and weight 0. */
moe_status moe_router_topk(moe_ctx *ctx, const moe_router_cfg *cfg, const float *x, const float *w_router,
                           const float *bias, int T, int H, int32_t *topk_idx, float *topk_w);

/* Per-expert bucketing ([P-dedup]): counts int32 [E]; offsets int32 [E+1]
 * (exclusive prefix sums); perm int32 [T*k] = entries t*k+j grouped by
 * expert, ascending (t, j) inside a group; only the first offsets[E] entries
 * are written. An id of -1 (a slot dropped by top-p) gets no entry and is no
 * error. Any other index outside [0, E), and an id repeated within one
 * token's k slots (the later slot), gets no entry and is reported by
 * moe_ctx_check as MOE_EINVAL. */
moe_status moe_bucket_tokens(moe_ctx *ctx, const int32_t *topk_idx, int T, int k, int E, int32_t *counts,
                             int32_t *offsets, int32_t *perm);

/* ---------------------------------------------------------------------- */
/* Expert FFN ([P-feat], [P-mem], [P-dedup])                              */
/* ---------------------------------------------------------------------- */

/* For every token t and slot j < k: y_slots[t][j] = FFN_{e}(token t) with
 * e = topk_idx[t][j]; if shared != NULL also y_slots[t][k] = FFN_shared(t).
 * FFN(t): accg[i] = sum_h qg[i,h] xq[t,h] and accu likewise (exact int32);
 * g = (float)accg * s_gate[i] * sx[t]; u likewise; a = silu(g) * u (fp32,
 * silu(g) = g / (1 + exp(-g)) with exp by Cody-Waite reduction and a degree-7
 * Taylor polynomial in fused multiply-adds); sa = max|a| / 127; aq =
 * clamp(rint(a / sa)); accd[r] = sum_i qd[r,i] aq[i]; y[r] = (float)accd *
 * s_down[r] * sa. Each expert's weights are streamed once per call for all
 * the tokens routed to it.
 *
 * experts: DEVICE array [E] of moe_expert_w (the structs' members are device
 * pointers). shared: HOST pointer to one moe_expert_w, or NULL.
 * expert_bits: DEVICE uint8 [E] or NULL. When given, only experts whose
 * entry equals this entry point's width are computed (slots of the others
 * are left untouched), so a mixed-precision layer is one call per width (or
 * one moe_expert_ffn_mixed call).
 * xq int8 [T][H], sx fp32 [T]: from moe_quantize_act_i8. topk_idx int32
 * [T][k]; an id of -1 (a slot dropped by top-p) names no expert: its slot is
 * not computed and not written; any other id outside [0, E), or an id
 * repeated within one token's k slots, is an error reported by
 * moe_ctx_check (that slot, the later one of a repeated pair, is not
 * written). y_slots fp32 [T][k+1][H] (slot k is the shared
 * expert's; it is written only when shared != NULL). */
moe_status moe_expert_ffn_q4(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                             const uint8_t *expert_bits, const int8_t *xq, const float *sx, const int32_t *topk_idx,
                             int T, int H, int I, int E, int k, float *y_slots);
moe_status moe_expert_ffn_q8(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                             const uint8_t *expert_bits, const int8_t *xq, const float *sx, const int32_t *topk_idx,
                             int T, int H, int I, int E, int k, float *y_slots);
moe_status moe_expert_ffn_q2(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                             const uint8_t *expert_bits, const int8_t *xq, const float *sx, const int32_t *topk_idx,
                             int T, int H, int I, int E, int k, float *y_slots);
/* A mixed-precision layer's expert FFN in one call ([P-feat]: int8, int4 and
 * int2 experts side by side): every slot computed at its expert's width
 * expert_bits[e] (DEVICE uint8 [E], required), bit-identical to the calls
 * of moe_expert_ffn_q8/q4/q2 with that filter. widths_mask: bit b set (b in
 * {8, 4, 2}) when the layer has experts of width b. The shared expert
 * (nullable) is computed at shared_bits, which then counts as set in the
 * mask too. A slot whose expert's width is not in the mask (0: not
 * resident) is not computed and not written. out (DEVICE fp32 [T][H],
 * nullable; needs topk_w, DEVICE fp32 [T][k]): also the combine of the
 * y_slots this call leaves, exactly as moe_combine computes it (with the
 * shared slot when shared != NULL). Everything runs on the context stream.
 * One token whose experts (the shared one included) are int4 and int2 runs
 * one chain of single-token kernels in which every slot has its own width;
 * other one-token mixes run each width's single-token kernels in turn, the
 * shared expert's width last, whose down kernel then also does the combine;
 * more tokens run each width's call in turn, then the combine. Other
 * arguments, errors and y_slots as for moe_expert_ffn_q4. */
moe_status moe_expert_ffn_mixed(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                                int shared_bits, const uint8_t *expert_bits, int widths_mask, const int8_t *xq,
                                const float *sx, const int32_t *topk_idx, const float *topk_w, int T, int H, int I,
                                int E, int k, float *y_slots, float *out);
/* The same call on fp32 hidden states x (DEVICE fp32 [T][H], 16-byte
 * aligned) instead of their codes: the activation rule of
 * moe_quantize_act_i8 ([P-feat]: int8 activations) is applied inside -- for
 * one token on the single-token kernels, by every gate/up workgroup on its
 * own copy of the row, so the call launches no quantisation kernel; for more
 * tokens by the quantisation kernel into the context's io scratch. y_slots
 * and out are bit-identical to moe_quantize_act_i8 followed by
 * moe_expert_ffn_mixed. The codes are not returned. Other arguments and
 * errors as for moe_expert_ffn_mixed. */
moe_status moe_expert_ffn_mixed_x(moe_ctx *ctx, const moe_expert_w *experts, const moe_expert_w *shared,
                                  int shared_bits, const uint8_t *expert_bits, int widths_mask, const float *x,
                                  const int32_t *topk_idx, const float *topk_w, int T, int H, int I, int E, int k,
                                  float *y_slots, float *out);

/* ---------------------------------------------------------------------- */
/* Combine ([P-moe], [P-mem])                                             */
/* ---------------------------------------------------------------------- */

/* out fp32 [T][H] = (has_shared ? y_slots[t][k] : 0) + sum_{j<k}
 * topk_w[t][j] * y_slots[t][j], accumulated in fp32 in that order; slots of
 * zero weight are skipped (their y is not read, so slots dropped by top-p may
 * hold anything). y_slots fp32 [T][k+1][H]. */
moe_status moe_combine(moe_ctx *ctx, const float *y_slots, const float *topk_w, int T, int k, int H, int has_shared,
                       float *out);

/* ---------------------------------------------------------------------- */
/* Whole layer in one call                                                */
/* ---------------------------------------------------------------------- */

/* The layer's hot path for T tokens in one call, all steps on the context
 * stream: activation quantisation, router (on x with w_router, or on the
 * given logits when cfg->logits_in), expert FFN of every routed expert and of
 * the shared expert at `bits` (8, 4 or 2; every expert at that width), and
 * the combine. Results equal moe_quantize_act_i8 -> moe_router_topk ->
 * moe_expert_ffn_q* -> moe_combine on the same inputs (the same arithmetic
 * in the same order; a single token runs three fused kernels: router logits
 * with the activation quantisation, top-k with gate/up, and the
 * requantisation of the intermediate with down and the combine).
 *
 * x fp32 [T][H] hidden states; logits fp32 [T][E] (only with
 * cfg->logits_in, else NULL); w_router fp32 [E][H] (ignored with logits);
 * bias fp32 [E] or NULL; experts DEVICE array [E]; shared HOST pointer or
 * NULL. out fp32 [T][H] (required). Optional outputs (NULL = not returned):
 * topk_idx int32 [T][k], topk_w fp32 [T][k], xq int8 [T][H], sx fp32 [T],
 * y_slots fp32 [T][k+1][H]. */
moe_status moe_layer_forward(moe_ctx *ctx, int bits, const moe_router_cfg *cfg, const float *x, const float *logits,
                             const float *w_router, const float *bias, const moe_expert_w *experts,
                             const moe_expert_w *shared, int T, int H, int I, float *out, int32_t *topk_idx,
                             float *topk_w, int8_t *xq, float *sx, float *y_slots);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer call as moe_layer_forward -- same arguments, kernels, arithmetic and
 * results -- whose scratch is the library's static device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU (resident from the library's first
 * context on that GPU until the process ends) instead of the context's
 * growable scratch. The call allocates nothing: no hipMalloc, no hipFree, no
 * stream or event creation. The caller still provides every input and the
 * outputs it names. Scratch needed: one token at most a few hundred KB; more
 * tokens at the GLM shape (H 6144, I 2048, E 256, k 8) about 330 KB per
 * token, so up to about 140 tokens fit. A call needing more than the array
 * holds is MOE_EINVAL before anything is enqueued, as is a call with
 * per-kernel timing on (moe_ctx_enable_timing records events). Every call of
 * this entry point on one GPU shares that GPU's array, which keeps the last
 * call's contents (no part of it needs clearing: each call writes every word
 * it reads): calls that overlap on one GPU -- from two contexts, or on two
 * streams without ordering between them -- race. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)48 << 20)
moe_status moe_layer_forward_noalloc(moe_ctx *ctx, int bits, const moe_router_cfg *cfg, const float *x,
                                     const float *logits, const float *w_router, const float *bias,
                                     const moe_expert_w *experts, const moe_expert_w *shared, int T, int H, int I,
                                     float *out, int32_t *topk_idx, float *topk_w, int8_t *xq, float *sx,
                                     float *y_slots);

/* ---------------------------------------------------------------------- */
/* Expert pool ([P-load], [P-mem], [P-dedup])                             */
/* ---------------------------------------------------------------------- */

/* An HBM cache of expert blocks (the moe_expert_block_layout layout) for a
 * stack of layers, refilled from caller-owned host memory: [P-load] keeps
 * experts resident under an LRU and reads the next block while the current
 * one computes; [P-dedup] reads an expert needed by several tokens once.
 * Blocks of different widths share one slab (first fit with coalescing). One
 * least-recently-used order spans every layer's resident experts; a pinned
 * expert, once resident, is never evicted. Refills run on the pool's own copy
 * stream; the context stream waits for them. A context re-bound to another
 * stream (moe_ctx_set_stream) gets those waits and the layer's table again on
 * the new stream; kernels still pending on the previous stream that read the
 * slab must be ordered before the next prepare call by the caller (evictions
 * are ordered against the context's current stream). Not thread-safe;
 * destroy a pool before its context. */
typedef struct moe_pool moe_pool;

/* Create a pool of capacity_bytes of HBM (allocated now on ctx's device) for
 * n_layers x n_experts experts of hidden H and intermediate I (multiples of
 * 64). ctx == NULL creates a bookkeeping-only pool: no memory and no copies,
 * the same residency decisions and statistics (capacity planning, tests on a
 * host without a GPU). MOE_ENOMEM if the slab cannot be allocated. With a
 * context the pool also allocates the layers' own device tables
 * (moe_pool_layer_table): n_layers x (n_experts x 49 bytes, rounded up to
 * 256), and eight pinned host staging buffers of n_experts x 49 bytes. */
moe_status moe_pool_create(moe_ctx *ctx, size_t capacity_bytes, int n_layers, int n_experts, int H, int I,
                           moe_pool **out);
/* Wait for the pool's copies and for the context stream (whose kernels may
 * read the slab), then free everything the pool owns. The pool's context
 * must still exist: destroy pools before their context. */
void moe_pool_destroy(moe_pool *pool);
/* Register expert (layer, expert) at `bits` in {8,4,2}: block_host holds its
 * block (bytes must equal moe_expert_block_layout(bits, H, I)); the caller
 * owns it and keeps it alive and unchanged until moe_pool_destroy. It should
 * be pinned memory (hipHostMalloc, torch pin_memory) for the refill to be an
 * asynchronous DMA. block_host may be NULL for a bookkeeping-only pool.
 * pin != 0: never evicted once resident. Registering twice is MOE_EINVAL. */
moe_status moe_pool_register(moe_pool *pool, int layer, int expert, int bits, const void *block_host,
                             size_t bytes, int pin);
/* Make the distinct experts of topk_idx_host (HOST int32 [T][k]) of `layer`
 * resident. Hits move to the most-recently-used end; each miss takes slab
 * space, evicting from the least-recently-used end experts this call does
 * not need, and is copied from its host block on the copy stream, after the
 * context stream has passed every earlier call that could read the evicted
 * bytes. The context stream then waits for this call's copies and receives,
 * in order, the layer's table: table_dev DEVICE moe_expert_w [E] (resident
 * experts point into the slab, the others are zero) and bits_dev DEVICE
 * uint8 [E] (the experts' widths, 0 when absent; nullable) -- ready for
 * moe_expert_ffn_q* with expert_bits = bits_dev (when bits_dev starts right
 * after the E table entries, one copy carries both). table_dev may be the
 * layer's own table of the pool (moe_pool_layer_table; bits_dev then NULL or
 * that table's widths): the pool copies into it only when the layer's table
 * bytes changed since its last copy there (an expert of the layer loaded,
 * evicted or re-loaded), so at a high hit rate most calls copy nothing. A
 * pointer into another layer's own table is MOE_EINVAL. n_miss_host
 * (nullable): this
 * call's misses; an id of -1 (a slot dropped by top-p) is skipped.
 * MOE_EINVAL for another id outside [0, E) or an unregistered
 * expert; MOE_EPOOL when the slab cannot hold this call's experts beside the
 * pinned ones, even after evicting every other unpinned expert (placement is
 * first-fit without moving resident blocks, so the free space left between
 * this call's resident experts can refuse a call whose total would fit; the
 * pool stays consistent). A bookkeeping-only pool takes
 * table_dev = bits_dev = NULL. */
moe_status moe_pool_prepare(moe_pool *pool, int layer, const int32_t *topk_idx_host, int T, int k,
                            moe_expert_w *table_dev, uint8_t *bits_dev, int *n_miss_host);
/* The pool's own device table of `layer` (a pool with a context): DEVICE
 * moe_expert_w [E] at *table_dev, its widths uint8 [E] right after it at
 * *bits_dev (nullable). Allocated with the pool, freed by moe_pool_destroy;
 * written only by moe_pool_prepare of that layer (callers only read it).
 * Host-only. */
moe_status moe_pool_layer_table(moe_pool *pool, int layer, moe_expert_w **table_dev, uint8_t **bits_dev);
/* The widths the latest moe_pool_prepare call's experts are resident at:
 * bit b set (b in {8, 4, 2}) when one of them is at width b (0 after a
 * call with no expert). A mixed layer's caller can pass it as widths_mask
 * to moe_expert_ffn_mixed, so that a width none of the token's experts has
 * costs no launches. Host-only. */
moe_status moe_pool_call_widths(const moe_pool *pool, int *mask_host);
/* Table copies of moe_pool_prepare: made, and skipped because the layer's
 * own table already held the bytes. Host-only. */
moe_status moe_pool_table_stats(const moe_pool *pool, uint64_t *copies, uint64_t *skipped);
/* Read-ahead ([P-load]; remio.ai, "Colibri shows how to run GLM-5.2 on a
 * low-spec PC", section "The RAM wall became a storage problem": the engine
 * predicts the next layer's routing and fetches those experts early). Starts
 * the refill of the experts ids_host[0..n) (HOST int32; -1 entries skipped)
 * of `layer` that are not resident, on the copy stream, so that a later
 * moe_pool_prepare of that layer finds them (it then waits for their copies
 * as for its own). Best effort: it never evicts an expert that the latest
 * moe_pool_prepare made resident (its kernels may not be enqueued yet) and
 * stops at the first expert it cannot place. n_issued_host (nullable): the
 * refills started. The prefetched experts count as recently used. MOE_EINVAL
 * for an id that is not a registered expert of the layer. */
moe_status moe_pool_prefetch(moe_pool *pool, int layer, const int32_t *ids_host, int n, int *n_issued_host);
/* Usage-learned pinning ([P-load]: the engine records the experts' routing in
 * a usage file and pins the hottest at start-up). moe_pool_usage writes, for
 * every (layer, expert) in layer-major order (HOST uint64 [n_layers][E]), the
 * number of moe_pool_prepare calls that requested it. moe_pool_pin_hot pins
 * registered experts in descending order of counts_host (same layout; NULL =
 * this pool's own counts; ties: lower layer, then lower id; zero counts never)
 * while their blocks fit in budget_bytes (at most the capacity), making each
 * resident now when room can be found without evicting the latest call's
 * experts (else on its first use); pinned experts are never evicted. Leave
 * room for a call's unpinned experts, or moe_pool_prepare may fail with
 * MOE_EPOOL. n_pinned_host (nullable): the experts pinned by this call. */
moe_status moe_pool_usage(const moe_pool *pool, uint64_t *counts_host);
moe_status moe_pool_pin_hot(moe_pool *pool, const uint64_t *counts_host, size_t budget_bytes, int *n_pinned_host);
/* Prefetch outcome: refills started by moe_pool_prefetch, and how many of
 * those experts a later moe_pool_prepare requested while still resident. */
moe_status moe_pool_prefetch_stats(const moe_pool *pool, uint64_t *issued, uint64_t *used);
/* Precision tiers ([P-feat]: int8, int4 and int2 kernels with per-row
 * scales). moe_pool_register_alt gives a registered expert a second, narrower
 * block (bits 4 under an int8 block, or 2 under an int4 one; same ownership
 * rules as moe_pool_register; bytes must equal moe_expert_block_layout(bits,
 * H, I); one per expert; MOE_EINVAL otherwise). With demotion on
 * (moe_pool_set_demotion(pool, 1); off at creation), a refill of an unpinned
 * expert with a narrower block loads that block instead when no free extent
 * of the slab holds the full-width one (the pool is under pressure),
 * evicting for the narrower size only. The expert keeps the width it was
 * loaded at until evicted; the width reaches the FFN calls through bits_dev,
 * so a layer's experts of each width go to that width's entry point. A
 * pinned expert always loads at full width: moe_pool_pin_hot re-loads a
 * demoted one now (or, if the latest call uses it, at its next request).
 * moe_pool_tier_stats: loads at the narrower width, requests served by a
 * narrower copy (hits and misses), and host-to-device bytes saved against
 * full-width loads. */
moe_status moe_pool_register_alt(moe_pool *pool, int layer, int expert, int bits, const void *block_host,
                                 size_t bytes);
moe_status moe_pool_set_demotion(moe_pool *pool, int enable);
moe_status moe_pool_tier_stats(const moe_pool *pool, uint64_t *demoted_loads, uint64_t *demoted_uses,
                               uint64_t *bytes_saved);
/* Width of the resident copy of (layer, expert): 8, 4 or 2; 0 if not
 * resident; -1 for invalid arguments. */
int moe_pool_resident_bits(const moe_pool *pool, int layer, int expert);
/* Cumulative expert hits, misses and bytes copied host-to-device. */
moe_status moe_pool_stats(const moe_pool *pool, uint64_t *hits, uint64_t *misses, uint64_t *bytes_h2d);
/* 1 if (layer, expert) is resident, 0 if not, -1 for invalid arguments. */
int moe_pool_resident(const moe_pool *pool, int layer, int expert);

/* ---------------------------------------------------------------------- */
/* Measurement                                                            */
/* ---------------------------------------------------------------------- */

/* Kernel stages the library times when timing is on. */
enum {
  MOE_STAGE_ROUTER = 0,   /* activation quantisation + router (+ top-k) */
  MOE_STAGE_BUCKET = 1,   /* per-expert bucketing */
  MOE_STAGE_GATEUP = 2,   /* gate/up GEMV with the SwiGLU epilogue */
  MOE_STAGE_REQUANT = 3,  /* int8 requantisation of the intermediate (several tokens) */
  MOE_STAGE_DOWN = 4,     /* down GEMV (one token: with the requantisation and the combine) */
  MOE_STAGE_COMBINE = 5,  /* weighted combine */
  MOE_N_STAGES = 6
};

/* Switch per-kernel timing on or off. When on, every kernel launched by
 * moe_layer_forward and moe_expert_ffn_* is bracketed by two hipEvents
 * recorded on the context stream (must not be on during graph capture).
 * Switching changes nothing else. */
moe_status moe_ctx_enable_timing(moe_ctx *ctx, int enable);
/* Wait for the recorded events and return, per stage, the summed kernel
 * time in milliseconds (ms_host[MOE_N_STAGES]) and the number of launches
 * (n_host[MOE_N_STAGES]); then forget the records. Either pointer may be NULL. */
moe_status moe_ctx_read_timing(moe_ctx *ctx, double *ms_host, int *n_host);

/* Streaming-read probe: the measured HBM read ceiling for a launch of a
 * given size, with which the weight-streaming kernels are compared beside
 * the data-sheet peak. Launches `reps` times a plain read kernel
 * (ctx->n_cu * wg_per_cu workgroups of 256 threads, 16-byte loads four deep,
 * grid-stride) on the context stream; launch r reads bytes_per_launch bytes
 * of buf (DEVICE, 16-byte aligned) at window r mod (buf_bytes /
 * bytes_per_launch), so a buffer larger than the last-level cache keeps every
 * launch cold. Synchronises the context stream. xor_host (nullable): the XOR
 * of every 32-bit word of the last launch's window; us_host (nullable): the
 * average launch duration in microseconds (hipEvents around each launch).
 * MOE_EINVAL for a misaligned buffer, bytes_per_launch not a positive
 * multiple of 16 or above buf_bytes, wg_per_cu outside [1, 64] or reps
 * outside [1, 100000]. */
moe_status moe_probe_stream_read(moe_ctx *ctx, const void *buf, size_t buf_bytes, size_t bytes_per_launch,
                                 int wg_per_cu, int reps, uint32_t *xor_host, double *us_host);

/* ---------------------------------------------------------------------- */
/* Test visibility                                                        */
/* ---------------------------------------------------------------------- */

/* Optional capture of the FFN's intermediates (all DEVICE pointers, each
 * may be NULL). Pair index p = t*(k+1) + slot. accg, accu int32 [T*(k+1)][I];
 * a fp32 [T*(k+1)][I]; aq int8 [T*(k+1)][I]; sa fp32 [T*(k+1)]; accd int32
 * [T*(k+1)][H]. Passing NULL for dbg switches capture off. The pointers must
 * stay valid until capture is switched off. */
typedef struct {
  int32_t *accg, *accu;
  float *a;
  int8_t *aq;
  float *sa;
  int32_t *accd;
} moe_debug_bufs;
moe_status moe_ctx_set_debug(moe_ctx *ctx, const moe_debug_bufs *dbg);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
