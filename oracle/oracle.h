/*
 * oracle.h -- plain fp64 CPU oracle for Flint's decode-attention hot path.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's
 * cpu_baseline leg may load this library.  It shares no code, header, table
 * or constant with the HIP library; neither includes the other.
 *
 * Every function computes the plain definition in double precision from the
 * same bf16-rounded inputs the GPU sees.  Sources (page titles and sections):
 *   [vLLM-day0]  "Day-0 Support for Flint on vLLM" (newruntime.com),
 *                section "What happened": 49 layers, 35 sliding-window layers
 *                over 513 tokens, 14 full-context layers, 28 KiB of KV per
 *                token, fused normalisation / rotary / cache operations.
 *   [arch]       "Day-0 Support for Flint on vLLM" (hnkhoi.com), section
 *                "Model architecture": RoPE on the sliding layers, no
 *                positional encoding on the full layers, learned attention
 *                sinks, GQA with 32 query and 4 KV heads, per-head Q/K RMSNorm.
 *   [models-json] "Recursive Flint" model JSON (studiotvai.com), fields
 *                "architecture" (GQA 4 KV x 128) and "kvCacheGiBPerRequest".
 * Where the pages leave a step open the reading taken is stated next to it.
 *
 * Cache layout (the oracle's own statement of the library's format): one K
 * and one V array per layer, one contiguous tile of bs * d elements per
 * (page, KV head), elements placed as orc_k_offset / orc_v_offset below
 * state; logical token p of request b lives in physical page
 * block_tables[b][p/16], row p%16.
 *
 * moe.c adds the MoE sublayer (O9, O10) with its own sources and readings.
 */
#ifndef FLINT_ORACLE_H
#define FLINT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int hq;         /* query heads (32)                                   */
  int hkv;        /* KV heads (4); q head h reads KV head h/(hq/hkv)     */
  int d;          /* head dim (128)                                     */
  int bs;         /* tokens per page (16)                               */
  int window;     /* 0: keys 0..t;  W>0: keys max(0,t-W+1)..t           */
  int use_rope;   /* 1 on sliding layers, 0 on full layers              */
  double theta;   /* RoPE base (10000)                                  */
  double eps;     /* RMSNorm epsilon (1e-6)                              */
  double scale;   /* softmax scale (1/sqrt(d))                           */
  int kv_fp8;     /* 0: bf16 cache elements; 1: fp8 E4M3 (x / scale)     */
  double k_scale; /* fp8 cache: K element = code value * k_scale         */
  double v_scale; /* fp8 cache: V element = code value * v_scale         */
} orc_layer;

/* O1: fp32 -> bf16 by round-to-nearest-even, chosen between the two
 * neighbouring bf16 values by comparing exact distances (NaN stays NaN). */
uint16_t orc_bf16_rne(float x);
double orc_bf16_value(uint16_t b);
/* O1 applied to n reals (rounds each fp64 value once, no fp32 step). */
void orc_bf16_rne_array(const double* x, uint16_t* y, int64_t n);

/* fp8 E4M3 (the "fp8" column of the models JSON "kvCacheGiBPerRequest";
 * reading: the OCP E4M3 format -- 1 sign, 4 exponent bits of bias 7, 3
 * mantissa bits, subnormals, no infinities, S.1111.111 is NaN, largest
 * finite value 448).  Round to nearest, ties to the even code, |x| > 448
 * saturates to +-448, NaN stays NaN. */
uint8_t orc_fp8_rne(double x);
double orc_fp8_value(uint8_t c);

/* Cache layout (the library's convention): element offset of K / V element
 * (page, KV head g, row, dim) in its cache array.  Each (page, g) owns one
 * contiguous tile of bs * d elements.  bf16 (d a multiple of 8): K at
 * (dim >> 5) * bs * 32 + ((dim >> 3) & 3) * bs * 8 + row * 8 + (dim & 7), V
 * dim-major (dim * bs + row).  fp8 E4M3 (d = 128, bs = 16 only; the other
 * functions return -2, or a NaN lse, for an fp8 layer of another shape), in
 * the 2048-byte tile:
 *   K: ((dim >> 4) & 1) * 1024 + (dim >> 5) * 256 + row * 16 + (dim & 15)
 *   V: (dim >> 6) * 1024 + ((row >> 2) * 16 + (dim & 15)) * 16
 *      + ((dim >> 4) & 3) * 4 + (row & 3) */
int64_t orc_k_offset(const orc_layer* L, int64_t page, int g, int row, int dim);
int64_t orc_v_offset(const orc_layer* L, int64_t page, int g, int row, int dim);

/* O2: per-head RMSNorm: y = x / sqrt(mean(x^2) + eps) * w, n values. */
void orc_rmsnorm(const float* x, const float* w, int n, double eps, double* y);

/* O3: rotate-half RoPE in place on one head of d values at position pos:
 * pairs (i, i+d/2) turn by pos * theta^(-2i/d). */
void orc_rope(double* x, int d, double pos, double theta);

/* O8: physical slot (page*bs + row) of logical token pos of request b. */
int64_t orc_slot(const int32_t* block_tables, int bt_stride, int bs, int b, int pos);

/* O4: per token t: q_out[t] = rope?(rmsnorm(q_in[t], qw)) for every q head;
 * K row at slot_mapping[t] = bf16(rope?(rmsnorm(k_in[t], kw))), V row = bf16(v_in[t])
 * (fp8 cache: fp8(K / k_scale) and fp8(v_in[t] / v_scale), each rounded once).
 * Caches are uint16 bf16 codes or (kv_fp8) uint8 fp8 codes in the same layout.
 * slot < 0 skips the cache write for that token.  q_out may be NULL.
 * Returns 0, or -1 on a slot outside [0, num_blocks*bs). */
int orc_append(const orc_layer* L, int T, const float* q_in, const float* k_in,
               const float* v_in, const float* qw, const float* kw,
               const int32_t* positions, const int32_t* slot_mapping,
               double* q_out, void* k_cache, void* v_cache, int num_blocks);

/* O5: one query of request b (absolute position t = seq_lens[b]-1) for every
 * q head, keys lo..t read through the page table; the sink of head h is an
 * extra logit in the softmax denominator that carries no value.
 * q: [B][hq][d] doubles; out: [B][hq][d].  Work is spread over nthreads
 * (<=0: all cores).  Returns 0, or -1 on a page id outside [0, num_blocks). */
int orc_attn_decode(const orc_layer* L, int B, const double* q,
                    const void* k_cache, const void* v_cache, int num_blocks,
                    const int32_t* block_tables, int bt_stride, const int32_t* seq_lens,
                    const float* sinks, double* out, int nthreads);

/* O6: partial over keys [j0, j1) of request b for q head h: normalised
 * o_tilde[d] and lse = m + ln(sum exp(s_j - m)); an empty range gives
 * lse = -inf and o_tilde = 0. */
void orc_attn_partial(const orc_layer* L, const double* q_h, int h,
                      const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int bt_stride, int b,
                      int j0, int j1, double* o_tilde, double* lse);

/* O6: fold S partials and the sink logit of one head into its output. */
void orc_merge(int S, int d, const double* o_tildes, const double* lses,
               double sink, double* out);

/* O7: causal prefill.  Request b owns query rows cu_q_lens[b] ..
 * cu_q_lens[b+1]-1; row i of it sits at position seq_lens[b] - q_len_b + i.
 * q: [total_q][hq][d]; out: [total_q][hq][d].  If rows != NULL only those
 * global rows are computed (others untouched).  Returns 0 or -1. */
int orc_attn_prefill(const orc_layer* L, int B, const double* q, const int32_t* cu_q_lens,
                     const void* k_cache, const void* v_cache, int num_blocks,
                     const int32_t* block_tables, int bt_stride, const int32_t* seq_lens,
                     const float* sinks, double* out, const int32_t* rows, int nrows,
                     int nthreads);

/* Bytes of KV per token kept by `full_layers` full-context layers. */
int64_t orc_full_kv_bytes_per_token(int full_layers, int hkv, int d, int elem_bytes);

/* KV bytes one request holds at context ctx: full layers keep every token,
 * sliding layers keep min(ctx, window) tokens. */
int64_t orc_kv_bytes_per_request(int64_t ctx, int full_layers, int sliding_layers,
                                 int window, int hkv, int d, int elem_bytes);

/* Number of threads the parallel oracle calls use for nthreads <= 0. */
int orc_default_threads(void);

/* O9/O10 (moe.c): Flint's MoE sublayer at decode.  Shapes: hidden 2048, 256
 * routed experts, top 6, one shared expert; `inter` is the expert FFN width
 * (a reading: 512).  Weights are bf16 bit patterns:
 *   w_router [experts][hidden], w_gate_up [experts + shared][2][inter][hidden]
 *   (gate rows then up rows), w_down [experts + shared][hidden][inter]. */
typedef struct {
  int hidden;
  int experts;   /* routed experts                   */
  int top_k;     /* experts selected per token       */
  int inter;     /* FFN width of every expert         */
  int shared;    /* always-active experts (weight 1)  */
} orc_moe;

/* O9: logits z_e = <x, w_router[e]> (fp64); the top_k experts by z rounded
 * to fp32, ties to the lower index; weights sigmoid(z) normalised over the
 * selected experts.  Returns 0, or -1 if top_k is outside [1, experts]. */
int orc_moe_route(const orc_moe* M, const float* x, const uint16_t* w_router, int32_t* ids,
                  double* weights);

/* O10: y[t] = sum_k weights[t][k] E_{ids[t][k]}(x[t]) + sum_s E_{experts+s}(x[t]),
 * E(x) = W_down (silu(W_gate x) * (W_up x)), fp64 throughout.  ids, weights
 * are outputs ([T][top_k]); y [T][hidden].  Returns 0 or -1. */
int orc_moe_forward(const orc_moe* M, int T, const float* x, const uint16_t* w_router,
                    const uint16_t* w_gate_up, const uint16_t* w_down, int32_t* ids,
                    double* weights, double* y, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
