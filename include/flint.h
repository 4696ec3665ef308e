/*
 * flint.h -- C ABI of the MI355X (gfx950) decode-attention library for the
 * Flint 40B-A2.5B MoE.
 *
 * What is computed (sources by page title and section):
 *   "Day-0 Support for Flint on vLLM" (newruntime.com), "What happened":
 *       49 layers; 35 attend over a 513-token sliding window, 14 attend to the
 *       full context and alone keep KV for the whole sequence (28 KiB per
 *       token); fused normalisation, rotary-position and cache operations and
 *       a low-latency small-batch decode path.
 *   "Day-0 Support for Flint on vLLM" (hnkhoi.com), "Model architecture":
 *       the sliding layers use RoPE, the full layers use no positional
 *       encoding; learned attention sinks; GQA with 32 query and 4 KV heads;
 *       per-head Q/K RMSNorm.
 *   "Recursive Flint" model JSON (studiotvai.com), "architecture": 4 KV
 *       heads of dim 128; "maxContext": 262,144 tokens.
 * Readings taken where the pages are silent: the sink of query head h is one
 * scalar logit that joins the softmax denominator, is not multiplied by the
 * softmax scale and carries no value; the window holds keys t-512..t of a
 * query at position t; RoPE is rotate-half over all 128 dims with absolute
 * 0-based positions; q head h reads KV head h / (num_q_heads/num_kv_heads).
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless stated otherwise, owned by the
 *     caller.  The library never allocates or frees memory and keeps no state
 *     between calls; scratch space comes from the caller's workspace (the
 *     prefill's work-item counter in it is zero before and after a call).
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     All work is enqueued on it; no call synchronises or reads device memory
 *     back, so every call can be captured into a HIP graph.
 *   - bf16 values are passed as their uint16 bit patterns; cache pointers are
 *     untyped (void*), their element type set by the layer's kv_dtype.
 *   - Arguments the host can see are checked before anything is launched and
 *     a status is returned; flint_last_error() then describes the problem.
 *     Device-resident indices (positions, slots, page ids, seq_lens) are
 *     bounds-checked inside the kernels: nothing outside the caller's buffers
 *     is ever read or written, and the affected outputs are set to NaN.
 *   - Supported shape: head_dim 128, block_size 16, num_q_heads =
 *     8 * num_kv_heads with 1 <= num_kv_heads <= 8, window 0 or >= 1.
 *
 * Paged KV cache layout (one K array and one V array per layer)
 *   A page holds 16 consecutive tokens of one request.  Logical token p of
 *   request b lives in physical page block_tables[b * bt_stride + p / 16],
 *   row p % 16.  Per page and KV head the data is one contiguous 4 KiB tile
 *   at element (page * num_kv_heads + g) * 2048:
 *     K: element (row, dim) at (dim >> 5) * 512 + ((dim >> 3) & 3) * 128
 *        + row * 8 + (dim & 7) in the tile (blocks of 32 dims, each of four
 *        groups of 8 dims holding those dims of all 16 rows in turn)
 *     V: element (row, dim) at dim * 16 + row (dim-major: the 16 tokens of
 *        one dim are 32 contiguous bytes)
 *   This is the order the matrix cores take their operands in: each 64-lane
 *   K load reads one 32-dim block of all 16 rows (1 KiB contiguous), and V
 *   is dim-major because the P.V contraction runs over tokens, so both
 *   operands load straight from HBM with full coalescing.
 *   A conventional row-major paged cache ([page][head][16][128] K and V rows)
 *   is NOT accepted by any call: the cache must be written by
 *   flint_qk_norm_rope_append or flint_attn_decode_step, which place every
 *   element in the tile order above.
 *
 * KV element formats (flint_attn_layer.kv_dtype)
 *   FLINT_KV_BF16: 2-byte bf16 elements (uint16 bit patterns), 4 KiB tiles.
 *   FLINT_KV_FP8_E4M3: 1-byte elements, still one contiguous tile per
 *   (page, KV head), now 2 KiB, halving the bytes decode streams ("Recursive
 *   Flint" model JSON, "kvCacheGiBPerRequest" lists an fp8 column beside
 *   bf16).  Inside a tile the order is the one the matrix-core operands are
 *   loaded in, so that every 64-lane load reads 1 KiB of contiguous bytes:
 *     K[row][dim] at ((dim >> 4) & 1) * 1024 + (dim >> 5) * 256 + row * 16
 *                    + (dim & 15)
 *     V[row][dim] at (dim >> 6) * 1024 + ((row >> 2) * 16 + (dim & 15)) * 16
 *                    + ((dim >> 4) & 3) * 4 + (row & 3)
 *   (row = token within the page, tile at ((page * num_kv_heads + g) * 2048)).  Reading of the
 *   format: OCP E4M3 -- sign, 4 exponent bits of bias 7, 3 mantissa bits,
 *   subnormals, no infinities, S.1111.111 is NaN, largest finite 448.  The
 *   cache holds K / k_scale and V / v_scale (one pair of scales per layer):
 *   an element reads back as code value * scale.  Writes round to nearest,
 *   ties to the even code, once from the exact (fp64) quotient; magnitudes
 *   at or above 448 saturate to +-448 and NaN stays NaN.
 */
#ifndef FLINT_H
#define FLINT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FLINT_ABI_VERSION 4

typedef enum {
  FLINT_OK = 0,
  FLINT_ERR_INVALID_ARGUMENT = 1,   /* a host-visible argument is wrong       */
  FLINT_ERR_UNSUPPORTED = 2,        /* a shape this library does not support  */
  FLINT_ERR_WORKSPACE_TOO_SMALL = 3,/* workspace_bytes below the size query   */
  FLINT_ERR_HIP = 4                 /* the HIP runtime refused a launch       */
} flint_status;

/* One attention layer.  The pages fix num_q_heads 32, num_kv_heads 4,
 * head_dim 128; window 513 with use_rope 1 for the 35 sliding layers and
 * window 0 with use_rope 0 for the 14 full layers. */
typedef struct {
  int32_t num_q_heads;   /* 8 * num_kv_heads                                */
  int32_t num_kv_heads;  /* 1..8 (Flint: 4)                                  */
  int32_t head_dim;      /* 128                                              */
  int32_t block_size;    /* tokens per page: 16                              */
  int32_t window;        /* 0: keys 0..t;  W >= 1: keys max(0, t-W+1)..t     */
  int32_t use_rope;      /* 1: rotate q and k (sliding layers); 0: NoPE      */
  float rope_theta;      /* RoPE base (10000)                                */
  float rms_eps;         /* RMSNorm epsilon (1e-6)                           */
  float softmax_scale;   /* multiplies q.k (1/sqrt(128))                     */
  int32_t kv_dtype;      /* FLINT_KV_BF16 or FLINT_KV_FP8_E4M3               */
  float k_scale;         /* fp8 cache: K = code value * k_scale (finite > 0) */
  float v_scale;         /* fp8 cache: V = code value * v_scale (finite > 0) */
} flint_attn_layer;     /* the scales are ignored for a bf16 cache         */

enum { FLINT_KV_BF16 = 0, FLINT_KV_FP8_E4M3 = 1 };

/*
 * Fused per-head Q/K RMSNorm, optional RoPE and paged KV append for
 * num_tokens tokens ("What happened": fused normalisation, rotary-position
 * and cache operations; "Model architecture": per-head Q/K RMSNorm, RoPE on
 * the sliding layers only).
 *   q_in  [T][num_q_heads][128] fp32, k_in, v_in [T][num_kv_heads][128] fp32
 *   q_norm_w, k_norm_w [128] fp32 (one weight vector shared by all heads)
 *   positions [T] int32: absolute 0-based position of each token (RoPE angle)
 *   slot_mapping [T] int32: page * 16 + row to write; < 0 skips the token
 *   q_out_f32 [T][num_q_heads][128] (decode) or q_out_bf16 (prefill): exactly
 *     one is non-NULL; q_out_f32 may alias q_in.
 *   k_cache, v_cache: [num_blocks] pages in the layout above.
 * Per token and head: y = x / sqrt(mean(x^2) + eps) * w, then RoPE(y,
 * position) when use_rope, computed in fp64; q_out is y rounded once to fp32
 * (or bf16), K is y rounded once to bf16 (round-to-nearest-even) and V is v
 * rounded to bf16; K and V are written at the slot.  V is not normalised.
 * An fp8 cache receives fp8(y / k_scale) and fp8(v / v_scale) instead.
 * A slot >= num_blocks*16 or a negative position is not written and the
 * token's q_out row is set to NaN.
 */
flint_status flint_qk_norm_rope_append(const flint_attn_layer* L, int32_t num_tokens,
                                       const float* q_in, const float* k_in, const float* v_in,
                                       const float* q_norm_w, const float* k_norm_w,
                                       const int32_t* positions, const int32_t* slot_mapping,
                                       float* q_out_f32, uint16_t* q_out_bf16,
                                       void* k_cache, void* v_cache, int32_t num_blocks,
                                       void* stream);

/*
 * Decode attention: one new query per request over its paged KV (bf16 or
 * fp8; for fp8, K_j and V_j below are the scaled code values).  Sources:
 * "Day-0 Support for Flint on vLLM" (hnkhoi.com), "Model architecture": GQA
 * of 32 query over 4 KV heads, learned attention sinks, RoPE sliding layers
 * and NoPE full layers; (newruntime.com), "What happened": a 513-token window
 * on 35 layers, the full context on 14, and the batch-1 decode at a
 * 100,000-token context this call serves.
 * Request b's query sits at position t = seq_lens[b] - 1 (seq_lens counts the
 * new token, which must already be appended) and attends to keys lo..t,
 * lo = 0 (window 0) or max(0, t - window + 1).  For query head h of KV group
 * g = h / 8:
 *   s_j   = softmax_scale * <q[b][h], K_j>
 *   out   = sum_j e^{s_j} V_j / (e^{sinks[h]} + sum_j e^{s_j})
 *   q      [B][num_q_heads][128] fp32 (normalised, rotated by the append)
 *   block_tables [B][bt_stride] int32 page ids; seq_lens [B] int32 on device
 *   max_seq_len  host-side upper bound of seq_lens (<= bt_stride * 16)
 *   sinks  [num_q_heads] fp32 logits (-inf allowed: plain softmax)
 *   out    [B][num_q_heads][128] fp32; must not alias q
 * Work is split over key ranges (split-K) and merged with log-sum-exp
 * weights; the sink joins in the merge.  A request whose seq_len is outside
 * [1, max_seq_len] or whose pages include an id outside [0, num_blocks) gets
 * NaN outputs.  workspace: >= flint_attn_decode_workspace_size(...) bytes
 * (0 when one split covers the range), 256-byte aligned, owned by the caller;
 * its contents need not be initialised.  Calls that share a workspace must
 * not run concurrently.
 */
size_t flint_attn_decode_workspace_size(const flint_attn_layer* L, int32_t num_seqs,
                                        int32_t max_seq_len);
flint_status flint_attn_decode(const flint_attn_layer* L, int32_t num_seqs, const float* q,
                               const void* k_cache, const void* v_cache,
                               int32_t num_blocks, const int32_t* block_tables,
                               int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                               const float* sinks, float* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Same as flint_attn_decode with the split size fixed by the caller:
 * pages_per_split > 0 pages of 16 keys per split (0 = the library's choice).
 * The workspace query must be made with the same pages_per_split. */
size_t flint_attn_decode_workspace_size_ex(const flint_attn_layer* L, int32_t num_seqs,
                                           int32_t max_seq_len, int32_t pages_per_split);
flint_status flint_attn_decode_ex(const flint_attn_layer* L, int32_t num_seqs, const float* q,
                                  const void* k_cache, const void* v_cache,
                                  int32_t num_blocks, const int32_t* block_tables,
                                  int32_t bt_stride, const int32_t* seq_lens,
                                  int32_t max_seq_len, const float* sinks, float* out,
                                  void* workspace, size_t workspace_bytes,
                                  int32_t pages_per_split, void* stream);

/*
 * One decode step of one layer in a single launch: the fused per-head
 * RMSNorm / RoPE / append of each request's new token followed by decode
 * attention ("What happened": fused normalisation, rotary-position and cache
 * operations).  Same results, bit for bit, as
 *   flint_qk_norm_rope_append(L, B, q_in, k_in, v_in, q_norm_w, k_norm_w,
 *                             positions = seq_lens - 1, slot_mapping, q_out, ...)
 * followed by flint_attn_decode on that q_out, without the intermediate q
 * round trip or a second launch.
 *   q_in [B][num_q_heads][128], k_in, v_in [B][num_kv_heads][128] fp32 raw
 *   slot_mapping [B]: must equal the slot the page table gives position
 *     seq_lens[b]-1 (page * 16 + row); otherwise nothing is written and that
 *     request's output is NaN
 *   q_out: optional [B][num_q_heads][128] fp32 normalised (rotated) q, or NULL;
 *     unlike the stand-alone append it must not overlap q_in (every split
 *     workgroup reads the raw q_in while one of them writes q_out), else
 *     FLINT_ERR_INVALID_ARGUMENT
 *   pages_per_split: as for flint_attn_decode_ex (0 = the library's choice);
 *     size the workspace with flint_attn_decode_workspace_size_ex.
 */
flint_status flint_attn_decode_step(const flint_attn_layer* L, int32_t num_seqs,
                                    const float* q_in, const float* k_in, const float* v_in,
                                    const float* q_norm_w, const float* k_norm_w,
                                    const int32_t* slot_mapping, float* q_out,
                                    void* k_cache, void* v_cache, int32_t num_blocks,
                                    const int32_t* block_tables, int32_t bt_stride,
                                    const int32_t* seq_lens, int32_t max_seq_len,
                                    const float* sinks, float* out, void* workspace,
                                    size_t workspace_bytes, int32_t pages_per_split,
                                    void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * flint_attn_decode_step without the workspace arguments, same results bit for
 * bit.  The split partials live in a static device array of
 * FLINT_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the call allocates nothing.  A batch whose plan
 * needs more partials than that (flint_attn_decode_workspace_size_ex above
 * the limit; e.g. more than ~16 requests at a 100,000-token context) returns
 * FLINT_ERR_WORKSPACE_TOO_SMALL before any launch.  All calls on one GPU share
 * the array: calls that may overlap on one GPU (several streams, several host
 * threads) race on it and must be serialised by the caller.  Its contents
 * need no initialisation: every call writes each partial before reading it.
 */
#define FLINT_NOALLOC_SCRATCH_BYTES (16u << 20)
flint_status flint_attn_decode_step_noalloc(const flint_attn_layer* L, int32_t num_seqs,
                                            const float* q_in, const float* k_in,
                                            const float* v_in, const float* q_norm_w,
                                            const float* k_norm_w, const int32_t* slot_mapping,
                                            float* q_out, void* k_cache, void* v_cache,
                                            int32_t num_blocks, const int32_t* block_tables,
                                            int32_t bt_stride, const int32_t* seq_lens,
                                            int32_t max_seq_len, const float* sinks, float* out,
                                            int32_t pages_per_split, void* stream);

/* The split plan flint_attn_decode_ex would use (host only, no HIP call):
 * writes the pages per split and the number of splits per request. */
flint_status flint_attn_decode_plan(const flint_attn_layer* L, int32_t num_seqs,
                                    int32_t max_seq_len, int32_t pages_per_split,
                                    int32_t* out_pages_per_split, int32_t* out_num_splits);

/*
 * The two halves of flint_attn_decode on their own: the split partials (no
 * sink), then their log-sum-exp merge with the sink.  They serve a caller
 * that holds the keys of one request on several devices (each computes the
 * partials of its range; the merge folds them), and they let each half be
 * checked and timed alone.  flint_attn_decode_ex with the same
 * pages_per_split (when the plan has more than one split) produces the same
 * output, bit for bit, as this pair.
 *
 * flint_attn_decode_partials: request b's key range lo..t (t = seq_lens[b]-1,
 * lo as for decode) is cut by logical page: split s holds the keys of pages
 * lo/16 + s*P .. lo/16 + (s+1)*P - 1 that lie in lo..t, where P and the split
 * count S are what flint_attn_decode_plan returns for this pages_per_split
 * (>= 1; num_splits must equal S).  For query head h, with
 * s_j = softmax_scale * q.k_j over the split's keys:
 *   part_lse[(b*S + s)*Hq + h]           = log2( sum_j e^{s_j} )   (base 2)
 *   part_o[((b*S + s)*Hq + h)*128 + d]   = sum_j e^{s_j} V_j[d] / sum_j e^{s_j}
 * An empty split has part_lse = -inf (part_o left as it was); a request with
 * a bad seq_len or page id has NaN part_lse in every split.
 *   part_o [B][S][num_q_heads][128] fp32, part_lse [B][S][num_q_heads] fp32
 */
flint_status flint_attn_decode_partials(const flint_attn_layer* L, int32_t num_seqs,
                                        const float* q, const void* k_cache,
                                        const void* v_cache, int32_t num_blocks,
                                        const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* seq_lens, int32_t max_seq_len,
                                        int32_t pages_per_split, int32_t num_splits,
                                        float* part_o, float* part_lse, void* stream);

/*
 * flint_attn_merge: out[b][h] from the S partials of (b, h) and the sink
 * ("Model architecture": learned attention sinks), M = max(sink_h, lse_s):
 *   out = sum_s 2^{lse_s - M} o_s / (2^{sink_h*log2(e) - M} + sum_s 2^{lse_s - M})
 * with lse_s in the base-2 form above and M in the same units.  Splits with
 * lse = -inf are skipped (their part_o is not read as a number); a NaN lse
 * makes that output NaN.  out [B][num_q_heads][128] fp32.
 */
flint_status flint_attn_merge(const flint_attn_layer* L, int32_t num_seqs, int32_t num_splits,
                              const float* part_o, const float* part_lse, const float* sinks,
                              float* out, void* stream);

/*
 * Causal (optionally windowed) prefill attention over the paged cache, on
 * the matrix cores ("Day-0 Support for Flint on vLLM", newruntime.com, "What
 * happened": the 8,192-token prefill of the optimised path; hnkhoi.com,
 * "Model architecture": the same sink, window and GQA rules as decode).
 * Request b owns query rows cu_q_lens[b] ..
 * cu_q_lens[b+1]-1 (cu_q_lens [B+1] int32 on device, cu_q_lens[0] = 0); row
 * i of it sits at position seq_lens[b] - q_len_b + i and attends to keys
 * lo..that position, whose K/V must already be appended.
 *   q   [total_q][num_q_heads][128] bf16 (normalised, rotated)
 *   total_q    rows of q and of out (host side; 0 is a no-op)
 *   max_q_len  host-side bound of every q_len; max_seq_len as for decode
 *   out [total_q][num_q_heads][128] fp32
 * Same per-row result as decode; the sink joins every row's denominator.
 * Rows of a request with q_len > seq_len or seq_len > max_seq_len, or whose
 * pages include an id outside [0, num_blocks), are set to NaN.  A request
 * whose rows cu_q_lens[b] .. cu_q_lens[b+1]-1 do not lie inside
 * [0, total_q) is skipped: none of q or out is touched for it.
 * An fp8 cache is widened as its pages are staged: K to bf16, V to fp16
 * (both exactly).  The value product P.V takes P in fp16 (relative rounding
 * at most 2^-11, so an output moves by at most 2^-11 of the largest |V| it
 * averages) against V in fp16; a bf16 cache's V converts to fp16 exactly up
 * to |V| = 65504.  A larger value becomes +-inf there, which makes the rows
 * of the work item (32 rows of one KV head) that take it non-finite: such an
 * item is flagged in the workspace and recomputed by a second launch of the
 * same call with bf16 V and P carried as bf16(p) plus its bf16 remainder
 * (as is an item whose inputs are not finite; its result is the same).
 * Workspace: flint_attn_prefill_workspace_size bytes, 16 + 4 per work item
 * (items: ceil(max_q_len / 32) x num_kv_heads x num_seqs): a work-item
 * counter, a count of flagged items and one flag per item; 8-byte aligned.
 * It must hold zeros
 * when the call runs, and every call leaves it zero again, so one zero-fill
 * when it is allocated serves every later call; calls that overlap in time
 * must not share it.  A call that fails its host-side checks does not touch
 * it.  Too small or NULL: FLINT_ERR_WORKSPACE_TOO_SMALL.
 */
size_t flint_attn_prefill_workspace_size(const flint_attn_layer* L, int32_t num_seqs,
                                         int32_t max_q_len, int32_t max_seq_len);
flint_status flint_attn_prefill(const flint_attn_layer* L, int32_t num_seqs, const uint16_t* q,
                                const int32_t* cu_q_lens, int32_t total_q, int32_t max_q_len,
                                const void* k_cache, const void* v_cache,
                                int32_t num_blocks, const int32_t* block_tables,
                                int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                                const float* sinks, float* out, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * MoE sublayer at small-batch decode (1..8 tokens): router, sigmoid top-k,
 * routed and shared SwiGLU experts ("Day-0 Support for Flint on vLLM",
 * hnkhoi.com, "Model architecture": hidden size 2048, 256 experts, sigmoid
 * top-6, a shared expert; newruntime.com, "What happened": small-batch MoE and
 * dense GEMV kernels).  Readings where the pages are silent: router logits
 * z_e = <x, w_router[e]> with no bias; the top_k experts by z, ties to the
 * lower index (the kernels rank their fp32 logits: the same experts as the
 * exact ranking unless two logits at the top-k boundary lie within fp32
 * rounding of each other); weights sigmoid(z_id) normalised over the selection; each
 * expert E(x) = W_down (silu(W_gate x) * (W_up x)) with silu(g) = g/(1+e^-g);
 * shared experts join with weight 1:
 *   out[t] = sum_k weight[t][k] E_{id[t][k]}(x[t]) + sum_s E_{experts+s}(x[t])
 * Weights are bf16 bit patterns, row-major, shared experts after the routed:
 *   w_router  [num_experts][hidden]
 *   w_gate_up [num_experts + num_shared][2][inter][hidden]  (gate, then up)
 *   w_down    [num_experts + num_shared][hidden][inter]
 *   x [T][hidden] fp32 in; out [T][hidden] fp32; topk_ids [T][top_k] int32 and
 *   topk_weights [T][top_k] fp32 out.  All 16-byte aligned.
 * Supported: hidden a multiple of 512 up to 4096, inter 512, 1..256 routed
 * experts, top_k 1..8, num_shared 0..2, num_tokens 0..8.  workspace: at least
 * flint_moe_workspace_size bytes, 256-byte aligned, contents irrelevant.
 * A NaN logit is never selected; NaN inputs give NaN outputs.
 */
typedef struct {
  int32_t hidden;       /* 2048                               */
  int32_t num_experts;  /* routed experts: 256                */
  int32_t top_k;        /* experts selected per token: 6      */
  int32_t inter;        /* FFN width of every expert: 512     */
  int32_t num_shared;   /* always-active experts: 1           */
} flint_moe_layer;

size_t flint_moe_workspace_size(const flint_moe_layer* M, int32_t num_tokens);
flint_status flint_moe_forward(const flint_moe_layer* M, int32_t num_tokens, const float* x,
                               const uint16_t* w_router, const uint16_t* w_gate_up,
                               const uint16_t* w_down, int32_t* topk_ids, float* topk_weights,
                               float* out, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Status text, thread-local detail of the last non-OK status on this thread,
 * and the ABI version (FLINT_ABI_VERSION). */
const char* flint_status_string(flint_status s);
const char* flint_last_error(void);
int32_t flint_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
