/*
 * moe_oracle.h -- plain, slow, scalar CPU oracle of the routed-expert MoE
 * layer. TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg may call it; the GPU library never does and
 * shares no code, header, table or constant with it.
 *
 * Pages followed (each function cites its passage):
 *  - agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on consumer
 *    hardware", section "Key features" (int8 / packed int4 / packed int2
 *    kernels with per-row scales and dequantisation on use; int8 matmuls via
 *    an integer dot product).
 *  - tech.takumi3488.com, "Trying colibri ...", section "Verifying the
 *    architecture with the self-test" (a DeepSeek-V3-family router) and
 *    section "Downloading and running the real 744B model" (hidden 6144,
 *    256 experts per layer, top-8).
 *  - remio.ai, "Colibri shows how to run GLM-5.2 on a low-spec PC ...",
 *    section "How Colibri runs GLM-5.2" (the router picks a few feed-forward
 *    modules per token) and section "The RAM wall became a storage problem"
 *    (a request for the same expert from several batch positions is served
 *    by one read).
 * The pages never write the layer's arithmetic out; the readings taken where
 * they are silent are listed in the design notes and repeated at each
 * function below.
 *
 * Conventions: row-major contiguous arrays; all pointers are host pointers.
 * Functions return 0 on success and a negative value on invalid arguments.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One expert: packed weight rows and fp32 per-row scales.
 * gate, up: [I][H*bits/8]; down: [H][I*bits/8]; s_gate, s_up: [I]; s_down: [H]. */
typedef struct {
  const uint8_t *gate, *up, *down;
  const float *s_gate, *s_up, *s_down;
} orc_expert;

/* --- O1: per-row symmetric quantisation and packing ----------------------
 * qmax = 2^(bits-1) - 1. Per row r: a = max_c |w[r,c]|; s = a / qmax (fp32);
 * q = clamp(rint(w / s), -qmax, qmax) with round-half-to-even; a == 0 gives
 * s = 0 and q = 0. Codes: bits 8 -> two's-complement byte; bits 4 -> nibble
 * u = q + 8, element 2i in the low nibble of byte i; bits 2 -> u = q + 2,
 * element 4i+j in bits [2j, 2j+1] of byte i. */
int orc_quantize_rows(int bits, const float *w, int64_t rows, int cols, uint8_t *packed, float *scales);
/* Inverse of the packing: codes q[r][c] as signed bytes. */
int orc_unpack_rows(int bits, const uint8_t *packed, int64_t rows, int cols, int8_t *q);

/* --- O2: per-token int8 activation quantisation (qmax 127) --------------- */
int orc_quantize_act(const float *x, int T, int H, int8_t *xq, float *sx);

/* --- exp and SiLU in float32 ---------------------------------------------
 * exp by Cody-Waite argument reduction (x = n ln2 + r, |r| <= ln2/2) and the
 * degree-7 Taylor polynomial of e^r, evaluated with fused multiply-adds;
 * silu(g) = g / (1 + exp(-g)). Every operation is a correctly rounded fp32
 * operation, so any implementation of the same steps gives the same bits. */
float orc_exp_f32(float x);
float orc_silu_f32(float g);

/* --- O3: sigmoid router with selection bias and top-k --------------------
 * logits_in = 0: z[t,e] = sum_h x[t,h] * wr[e,h] (fp64 accumulation);
 * logits_in = 1: z = x, given as [T][E].
 * sig = 1 / (1 + exp(-z)); key = sig + bias[e] (bias may be NULL = 0);
 * idx[t] = the k experts with the largest keys, in descending key order,
 * equal keys ordered by lower expert id; w[t,j] = scale * sig_j / sum sig.
 * keys_out [T][E] and sig_out [T][E] (fp64, nullable) expose the keys. */
int orc_router(int logits_in, const float *x, const float *wr, const float *bias, int T, int H, int E, int k,
               double routed_scale, int32_t *idx, float *w, double *keys_out, double *sig_out);

/* --- O4: per-expert bucketing (stable counting sort) --------------------
 * counts[e] = #{(t,j): idx[t,j] = e}; offsets[0..E] exclusive prefix sums;
 * perm[offsets[e] .. offsets[e+1]) = the entries t*k+j routed to e in
 * ascending (t, j) order. */
int orc_bucket(const int32_t *idx, int T, int k, int E, int32_t *counts, int32_t *offsets, int32_t *perm);

/* --- O5: one expert's SwiGLU FFN on one token ------------------------------
 * accg[i] = sum_h qg[i,h] xq[h]; accu likewise (exact integers);
 * g = (float)accg * sg[i] * sx; u = (float)accu * su[i] * sx;
 * a = silu(g) * u (fp32); sa = max|a| / 127; aq = clamp(rint(a / sa), +-127);
 * accd[r] = sum_i qd[r,i] aq[i]; y[r] = (float)accd * sd[r] * sa.
 * Any intermediate pointer may be NULL except y. */
int orc_expert_token(int bits, const orc_expert *ex, const int8_t *xq_t, float sx_t, int H, int I, int32_t *accg,
                     int32_t *accu, float *a, int8_t *aq, float *sa, int32_t *accd, float *y);

/* --- O7: weighted combine ---------------------------------------------------
 * y_slots [T][S][H] with S = k + has_shared (slot k = shared expert);
 * out[t] = y_shared[t] + sum_{j<k} w[t,j] * y_j[t], summed in fp64 in that
 * order, rounded to fp32. */
int orc_combine(const float *y_slots, const float *w, int T, int k, int H, int has_shared, float *out);

/* --- full layer: O2 -> O3 -> O5/O6 -> O7 ------------------------------------
 * experts [E] host structs, bits [E] per-expert precision (8, 4 or 2);
 * shared may be NULL. x: [T][H] hidden states (always needed for the FFN);
 * logits: [T][E] when logits_in, else NULL (router runs on x with wr).
 * Outputs: xq [T][H], sx [T], idx [T][k], w [T][k], y_slots [T][S][H],
 * out [T][H] (any output except out may be NULL). */
/* Top-p truncation of a top-k selection: the shortest rank-order prefix whose
 * cumulative normalised weight reaches top_p is kept and renormalised;
 * dropped slots get id -1 and weight 0; top_p <= 0 changes nothing. */
int orc_topp(int T, int E, int k, const double *sig, double routed_scale, double top_p, int32_t *idx, float *w,
             double *cum_out);
int orc_layer(const float *x, const float *logits, const float *wr, const float *bias, double routed_scale,
              const orc_expert *experts, const uint8_t *bits, const orc_expert *shared, int shared_bits, int T, int H,
              int I, int E, int k, double top_p, int8_t *xq, float *sx, int32_t *idx, float *w, float *y_slots,
              float *out);

/* Unquantised reference SwiGLU in fp64 (for the quantisation-error sanity
 * figure only): y = Wd (silu(Wg x) * (Wu x)). wg, wu [I][H]; wd [H][I]. */
int orc_swiglu_f64(const float *wg, const float *wu, const float *wd, const float *x, int H, int I, double *y);

/* Threads the layer spreads its (token, slot) pairs over (OpenMP builds):
 * n > 0 sets them; returns the number now in use (1 without OpenMP). */
int orc_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
