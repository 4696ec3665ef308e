// launch.h -- internal launchers behind the C ABI (host side).  Arguments are
// already validated by api.hip when these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flint {

struct AppendArgs {
  const float* q_in;
  const float* k_in;
  const float* v_in;
  const float* q_w;
  const float* k_w;
  const int32_t* positions;
  const int32_t* slots;
  float* q_out_f32;
  uint16_t* q_out_bf16;
  void* k_cache;             // bf16 bits, or fp8 E4M3 codes when kv_fp8
  void* v_cache;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t use_rope;
  float rope_theta;
  float rms_eps;
  int32_t kv_fp8;            // caches hold fp8(x / scale)
  float k_scale;
  float v_scale;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t s);

struct DecodeArgs {
  const float* q;            // [B][Hq][128] fp32 (normalised; unfused path)
  void* k_cache;             // [pages][Hkv][16][128] (written only by the fused path)
  void* v_cache;             // [pages][Hkv][128][16]; elements bf16 or fp8 (kv_fp8)
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const float* sinks;        // [Hq]
  float* out;                // [B][Hq][128]
  float* part_o;             // [B][S][Hq][128] (multi-split only)
  float* part_lse;           // [B][S][Hq], log2 units (multi-split only)
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t bt_stride;
  int32_t window;            // 0 = full
  int32_t max_seq_len;
  int32_t pages_per_split;
  int32_t num_splits;        // splits in the grid (per request)
  int32_t partials_only;     // write every split's partial (no merge, no sink)
  float qscale;              // softmax_scale * log2(e) (* k_scale for an fp8 cache)
  int32_t kv_fp8;            // 1: fp8 E4M3 codes of K / k_scale, V / v_scale
  float k_scale;             // fp8: divides the new token's K before encoding
  float v_scale;             // fp8: multiplies every output (1 for bf16)
  // fused append of the new token (flint_attn_decode_step); q_in == nullptr
  // selects the unfused path
  const float* q_in;         // [B][Hq][128] raw
  const float* k_in;         // [B][Hkv][128] raw
  const float* v_in;         // [B][Hkv][128] raw
  const float* q_w;
  const float* k_w;
  const int32_t* slots;      // [B]
  float* q_out;              // optional [B][Hq][128]
  int32_t use_rope;
  float rope_theta;
  float rms_eps;
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
// K3 alone: out from part_o / part_lse / sinks (num_seqs, num_kv_heads, num_splits)
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s);

struct PrefillArgs {
  const uint16_t* q;         // [total_q][Hq][128] bf16
  const int32_t* cu_q_lens;  // [B+1]
  int32_t total_q;           // rows of q and out
  const void* k_cache;       // bf16 bits, or fp8 codes in the fp8 tile order (kv_fp8)
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const float* sinks;
  float* out;                // [total_q][Hq][128] fp32
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t num_blocks;
  int32_t bt_stride;
  int32_t window;
  int32_t max_q_len;
  int32_t max_seq_len;
  float qscale;              // softmax_scale * log2(e) (* k_scale for an fp8 cache)
  int32_t kv_fp8;
  float v_scale;             // multiplies the output (1 for bf16)
  unsigned long long* claims;  // item counter (prefill_workspace_bytes > 0), else null
};
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s);
// Workspace of a prefill launch: one item counter when the items outnumber
// the persistent grid, else none.
size_t prefill_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t max_q_len);

// Waves per decode workgroup: kDecodeWaves when the key range is split (two
// workgroups per CU), kDecodeWavesSingle when one workgroup covers a short
// range by itself.  kSinglePages: ranges of at most this many pages run in
// one split with every page load in flight at once (kSinglePages /
// waves pages of registers per wave) and no merge launch -- at small batch
// in kVSlices slice workgroups per (request, KV head) (below), otherwise in
// one workgroup per (request, KV head).
constexpr int kDecodeWaves = 8;
constexpr int kDecodeWavesSingle = 8;
constexpr int kSinglePages = 40;
// kShortMinPages: least pages per split the plan gives a short range it
// splits (batches past the slice grid, or a caller's explicit split size).
// The 513-key window then takes 7 splits: at 8 splits or fewer the merge
// runs the one-pass small-merge kernel.  Measured per fused sliding step at
// batch 1 in a graph: 8.4 us at 7 splits, 9.0 us at 17 (2 pages each), 9.4
// at 4; the slice kernel (one launch) 8.1 us.
constexpr int kShortMinPages = 5;
// Short ranges (at most kSinglePages pages) at small batch: kVSlices
// workgroups per (request, KV head), each owning 16 of the 128 output dims,
// reading every K page of the range and its slice of V, with the sink folded
// in -- one launch and no merge.  Used while the grid (requests x KV heads x
// kVSlices) fits one round of kVSliceGrid workgroups.
constexpr int kVSlices = 8;
constexpr int kVSliceWaves = 8;
constexpr int kVSliceGrid = 256;

}  // namespace flint
