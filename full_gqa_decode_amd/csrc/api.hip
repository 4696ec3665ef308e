// api.hip -- the C ABI of libflint (declared in include/flint.h).
//
// Host-visible arguments are validated before any HIP call, so every
// invalid-argument path returns a status without touching the GPU.  The
// library allocates nothing: multi-split decode writes its partials into the
// caller's workspace.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/flint.h"
#include "launch.h"
#include "status.h"

namespace {
thread_local char g_err[512] = "";
}  // namespace

namespace flint::abi {

flint_status fail(flint_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

flint_status ok() {
  g_err[0] = '\0';
  return FLINT_OK;
}

flint_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(FLINT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

}  // namespace flint::abi

using namespace flint::abi;

namespace {

// The split plan is a pure function of its arguments (no device query), so the
// workspace size and the launch always agree.  kTargetWorkgroups sizes the
// grid for MI355X's 256 compute units at one long-running workgroup each.
constexpr int kMaxContext = 1 << 24;
constexpr int kTargetWorkgroups = 256;
// Longest split of a batch plan (a ragged batch of 64 requests up to 131072
// tokens streams at ~5.6 TB/s with 192-page splits, ~4 TB/s with whole requests).
constexpr int kMaxSplitPages = 192;

flint_status check_layer(const flint_attn_layer* L) {
  if (!L) return fail(FLINT_ERR_INVALID_ARGUMENT, "layer descriptor is NULL");
  if (L->head_dim != 128) return fail(FLINT_ERR_UNSUPPORTED, "head_dim %d (only 128)", L->head_dim);
  if (L->block_size != 16)
    return fail(FLINT_ERR_UNSUPPORTED, "block_size %d (only 16)", L->block_size);
  if (L->num_kv_heads < 1 || L->num_kv_heads > 8)
    return fail(FLINT_ERR_UNSUPPORTED, "num_kv_heads %d (1..8)", L->num_kv_heads);
  if (L->num_q_heads != 8 * L->num_kv_heads)
    return fail(FLINT_ERR_UNSUPPORTED, "num_q_heads %d must be 8 * num_kv_heads", L->num_q_heads);
  if (L->window < 0) return fail(FLINT_ERR_INVALID_ARGUMENT, "window %d < 0", L->window);
  if (L->use_rope != 0 && L->use_rope != 1)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "use_rope must be 0 or 1");
  if (!std::isfinite(L->softmax_scale))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "softmax_scale is not finite");
  if (L->use_rope && !(L->rope_theta > 0.f && std::isfinite(L->rope_theta)))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "rope_theta must be finite and > 0");
  if (!(L->rms_eps >= 0.f) || !std::isfinite(L->rms_eps))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "rms_eps must be finite and >= 0");
  if (L->kv_dtype != FLINT_KV_BF16 && L->kv_dtype != FLINT_KV_FP8_E4M3)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "kv_dtype %d (0 bf16, 1 fp8 e4m3)", L->kv_dtype);
  if (L->kv_dtype == FLINT_KV_FP8_E4M3 &&
      !(L->k_scale > 0.f && std::isfinite(L->k_scale) && L->v_scale > 0.f &&
        std::isfinite(L->v_scale)))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "fp8 k_scale / v_scale must be finite and > 0");
  return FLINT_OK;
}

// Most pages one query's key range can touch.
int64_t max_key_pages(const flint_attn_layer* L, int32_t max_seq_len) {
  const int64_t all = (max_seq_len + 15) / 16;
  if (L->window <= 0) return all;
  const int64_t win = (L->window + 14) / 16 + 1;
  return win < all ? win : all;
}

struct Plan {
  int32_t pages_per_split;
  int32_t num_splits;
};

// About kTargetWorkgroups workgroups of (split, KV head, request): a short
// range (the 513-key window) becomes small splits so its bytes spread over many
// CUs; a long one at batch 1 is cut into one split per CU; a batch of long
// requests keeps splits of at most kMaxSplitPages pages (so that its longest
// requests are spread too) in a grid of whole rounds of kTargetWorkgroups.
Plan make_plan(const flint_attn_layer* L, int32_t num_seqs, int32_t max_seq_len, int32_t pps) {
  const int64_t pages = max_key_pages(L, max_seq_len);
  int64_t p = pps;
  if (p <= 0) {
    const int64_t units = (int64_t)(num_seqs > 0 ? num_seqs : 1) * L->num_kv_heads;
    if (pages <= flint::kSinglePages && units * flint::kVSlices <= flint::kVSliceGrid) {
      // a short range at small batch: one split, run by the slice kernel
      Plan pl;
      pl.pages_per_split = (int32_t)pages;
      pl.num_splits = 1;
      return pl;
    }
    int64_t splits = (kTargetWorkgroups + units - 1) / units;
    p = (pages + splits - 1) / splits;
    if (p > kMaxSplitPages) {
      // a whole multiple of the base split count, so that the grid stays a
      // whole number of rounds of kTargetWorkgroups (a few workgroups past a
      // round would cost a whole extra round)
      splits *= (p + kMaxSplitPages - 1) / kMaxSplitPages;
      p = (pages + splits - 1) / splits;
    }
    if (p < flint::kShortMinPages) p = flint::kShortMinPages;
  }
  if (p > pages) p = pages;
  if (p < 1) p = 1;
  Plan pl;
  pl.pages_per_split = (int32_t)p;
  pl.num_splits = (int32_t)((pages + p - 1) / p);
  return pl;
}

// Workspace of a multi-split plan: [partial outputs | partial log-sum-exps],
// each part 256-byte aligned.
struct WsLayout {
  size_t part_o, part_lse, total;
};

WsLayout ws_layout(const flint_attn_layer* L, int32_t num_seqs, const Plan& pl) {
  WsLayout w{0, 0, 0};
  if (pl.num_splits <= 1 || num_seqs <= 0) return w;
  const size_t rows = (size_t)num_seqs * pl.num_splits * L->num_q_heads;
  w.part_o = 0;
  w.part_lse = align_up(rows * 128 * sizeof(float));
  w.total = w.part_lse + align_up(rows * sizeof(float));
  return w;
}

size_t decode_ws_bytes(const flint_attn_layer* L, int32_t num_seqs, const Plan& pl) {
  return ws_layout(L, num_seqs, pl).total;
}

// Library-owned scratch for flint_attn_decode_step_noalloc: the split
// partials of one call.  Every GPU the library runs on holds its own copy of
// this array for the life of the process.  In host code `scratch` only names
// the variable: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever handed to a kernel.
constexpr size_t kScratchBytes = FLINT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (looked up on its first use on that
// device, with the device current).
flint_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(FLINT_ERR_UNSUPPORTED, "device %d beyond the %d the library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(FLINT_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FLINT_OK;
}

}  // namespace

extern "C" {

const char* flint_status_string(flint_status s) {
  switch (s) {
    case FLINT_OK: return "FLINT_OK";
    case FLINT_ERR_INVALID_ARGUMENT: return "FLINT_ERR_INVALID_ARGUMENT";
    case FLINT_ERR_UNSUPPORTED: return "FLINT_ERR_UNSUPPORTED";
    case FLINT_ERR_WORKSPACE_TOO_SMALL: return "FLINT_ERR_WORKSPACE_TOO_SMALL";
    case FLINT_ERR_HIP: return "FLINT_ERR_HIP";
  }
  return "FLINT_STATUS_UNKNOWN";
}

const char* flint_last_error(void) { return g_err; }

int32_t flint_abi_version(void) { return FLINT_ABI_VERSION; }

flint_status flint_qk_norm_rope_append(const flint_attn_layer* L, int32_t num_tokens,
                                       const float* q_in, const float* k_in, const float* v_in,
                                       const float* q_norm_w, const float* k_norm_w,
                                       const int32_t* positions, const int32_t* slot_mapping,
                                       float* q_out_f32, uint16_t* q_out_bf16,
                                       void* k_cache, void* v_cache, int32_t num_blocks,
                                       void* stream) {
  flint_status st = check_layer(L);
  if (st != FLINT_OK) return st;
  if (num_tokens < 0) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return ok();
  if (!q_in || !k_in || !v_in || !q_norm_w || !k_norm_w || !positions || !slot_mapping ||
      !k_cache || !v_cache)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if ((q_out_f32 == nullptr) == (q_out_bf16 == nullptr))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "exactly one of q_out_f32 / q_out_bf16 must be set");
  if (num_blocks < 1) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_blocks %d < 1", num_blocks);
  if (!aligned(q_in, 4) || !aligned(k_in, 4) || !aligned(v_in, 4) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || (q_out_f32 && !aligned(q_out_f32, 4)) ||
      (q_out_bf16 && !aligned(q_out_bf16, 2)))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "misaligned pointer");
  if (q_out_f32 && q_out_f32 != q_in &&
      overlap(q_out_f32, (size_t)num_tokens * L->num_q_heads * 128 * 4, q_in,
              (size_t)num_tokens * L->num_q_heads * 128 * 4))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "q_out_f32 partially overlaps q_in");
  flint::AppendArgs a;
  a.q_in = q_in;
  a.k_in = k_in;
  a.v_in = v_in;
  a.q_w = q_norm_w;
  a.k_w = k_norm_w;
  a.positions = positions;
  a.slots = slot_mapping;
  a.q_out_f32 = q_out_f32;
  a.q_out_bf16 = q_out_bf16;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.num_tokens = num_tokens;
  a.num_q_heads = L->num_q_heads;
  a.num_kv_heads = L->num_kv_heads;
  a.num_blocks = num_blocks;
  a.use_rope = L->use_rope;
  a.rope_theta = L->rope_theta;
  a.rms_eps = L->rms_eps;
  a.kv_fp8 = L->kv_dtype == FLINT_KV_FP8_E4M3;
  a.k_scale = a.kv_fp8 ? L->k_scale : 1.f;
  a.v_scale = a.kv_fp8 ? L->v_scale : 1.f;
  return hip_status(flint::launch_append(a, (hipStream_t)stream), "append launch");
}

flint_status flint_attn_decode_plan(const flint_attn_layer* L, int32_t num_seqs,
                                    int32_t max_seq_len, int32_t pages_per_split,
                                    int32_t* out_pps, int32_t* out_splits) {
  flint_status st = check_layer(L);
  if (st != FLINT_OK) return st;
  if (num_seqs < 0 || max_seq_len < 1 || max_seq_len > kMaxContext || pages_per_split < 0)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "bad num_seqs / max_seq_len / pages_per_split");
  Plan pl = make_plan(L, num_seqs, max_seq_len, pages_per_split);
  if (out_pps) *out_pps = pl.pages_per_split;
  if (out_splits) *out_splits = pl.num_splits;
  return ok();
}

size_t flint_attn_decode_workspace_size_ex(const flint_attn_layer* L, int32_t num_seqs,
                                           int32_t max_seq_len, int32_t pages_per_split) {
  if (check_layer(L) != FLINT_OK || num_seqs < 0 || max_seq_len < 1 ||
      max_seq_len > kMaxContext || pages_per_split < 0)
    return 0;
  return decode_ws_bytes(L, num_seqs, make_plan(L, num_seqs, max_seq_len, pages_per_split));
}

size_t flint_attn_decode_workspace_size(const flint_attn_layer* L, int32_t num_seqs,
                                        int32_t max_seq_len) {
  return flint_attn_decode_workspace_size_ex(L, num_seqs, max_seq_len, 0);
}

}  // extern "C"

namespace {

// KV element format, the score scale in log2 units (an fp8 cache's k_scale
// folded in) and the output scale.
void set_kv_format(const flint_attn_layer* L, flint::DecodeArgs* a) {
  a->kv_fp8 = L->kv_dtype == FLINT_KV_FP8_E4M3;
  a->k_scale = a->kv_fp8 ? L->k_scale : 1.f;
  a->v_scale = a->kv_fp8 ? L->v_scale : 1.f;
  a->qscale = L->softmax_scale * 1.4426950408889634f * a->k_scale;
}

// Validation shared by the decode entry points; fills the launch arguments.
flint_status prepare_decode(const flint_attn_layer* L, int32_t num_seqs, const void* k_cache,
                            const void* v_cache, int32_t num_blocks,
                            const int32_t* block_tables, int32_t bt_stride,
                            const int32_t* seq_lens, int32_t max_seq_len, const float* sinks,
                            float* out, void* workspace, size_t workspace_bytes,
                            int32_t pages_per_split, flint::DecodeArgs* a) {
  flint_status st = check_layer(L);
  if (st != FLINT_OK) return st;
  if (num_seqs < 0) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", num_seqs);
  if (pages_per_split < 0)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "pages_per_split %d < 0", pages_per_split);
  if (max_seq_len < 1 || max_seq_len > kMaxContext)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "max_seq_len %d outside [1, %d]", max_seq_len,
                kMaxContext);
  if (num_seqs == 0) return FLINT_OK;
  if (!k_cache || !v_cache || !block_tables || !seq_lens || !sinks || !out)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (num_blocks < 1) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_blocks %d < 1", num_blocks);
  if (bt_stride < 1) return fail(FLINT_ERR_INVALID_ARGUMENT, "bt_stride %d < 1", bt_stride);
  if ((int64_t)max_seq_len > (int64_t)bt_stride * 16)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "max_seq_len %d exceeds bt_stride*16 = %lld",
                max_seq_len, (long long)bt_stride * 16);
  if (!aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(sinks, 4))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "misaligned pointer (out, caches need 16 B)");
  const Plan pl = make_plan(L, num_seqs, max_seq_len, pages_per_split);
  const size_t need = decode_ws_bytes(L, num_seqs, pl);
  if (need > 0) {
    if (workspace_bytes < need || !workspace)
      return fail(FLINT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu",
                  workspace_bytes, need);
    if (!aligned(workspace, kWsAlign))
      return fail(FLINT_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kWsAlign);
  }
  *a = flint::DecodeArgs{};
  a->k_cache = const_cast<void*>(k_cache);
  a->v_cache = const_cast<void*>(v_cache);
  a->block_tables = block_tables;
  a->seq_lens = seq_lens;
  a->sinks = sinks;
  a->out = out;
  const WsLayout wl = ws_layout(L, num_seqs, pl);
  a->part_o = need ? (float*)((char*)workspace + wl.part_o) : nullptr;
  a->part_lse = need ? (float*)((char*)workspace + wl.part_lse) : nullptr;
  a->num_seqs = num_seqs;
  a->num_kv_heads = L->num_kv_heads;
  a->num_blocks = num_blocks;
  a->bt_stride = bt_stride;
  a->window = L->window;
  a->max_seq_len = max_seq_len;
  a->pages_per_split = pl.pages_per_split;
  a->num_splits = pl.num_splits;
  set_kv_format(L, a);
  a->use_rope = L->use_rope;
  a->rope_theta = L->rope_theta;
  a->rms_eps = L->rms_eps;
  return FLINT_OK;
}

}  // namespace

extern "C" {

flint_status flint_attn_decode_ex(const flint_attn_layer* L, int32_t num_seqs, const float* q,
                                  const void* k_cache, const void* v_cache,
                                  int32_t num_blocks, const int32_t* block_tables,
                                  int32_t bt_stride, const int32_t* seq_lens,
                                  int32_t max_seq_len, const float* sinks, float* out,
                                  void* workspace, size_t workspace_bytes,
                                  int32_t pages_per_split, void* stream) {
  flint::DecodeArgs a;
  flint_status st = prepare_decode(L, num_seqs, k_cache, v_cache, num_blocks, block_tables,
                                   bt_stride, seq_lens, max_seq_len, sinks, out, workspace,
                                   workspace_bytes, pages_per_split, &a);
  if (st != FLINT_OK || num_seqs == 0) return st == FLINT_OK ? ok() : st;
  if (!q) return fail(FLINT_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(q, 16)) return fail(FLINT_ERR_INVALID_ARGUMENT, "misaligned pointer (q needs 16 B)");
  const size_t qbytes = (size_t)num_seqs * L->num_q_heads * 128 * sizeof(float);
  if (overlap(q, qbytes, out, qbytes))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "out must not alias q");
  a.q = q;
  return hip_status(flint::launch_decode(a, (hipStream_t)stream), "decode launch");
}

flint_status flint_attn_decode_step(const flint_attn_layer* L, int32_t num_seqs,
                                    const float* q_in, const float* k_in, const float* v_in,
                                    const float* q_norm_w, const float* k_norm_w,
                                    const int32_t* slot_mapping, float* q_out,
                                    void* k_cache, void* v_cache, int32_t num_blocks,
                                    const int32_t* block_tables, int32_t bt_stride,
                                    const int32_t* seq_lens, int32_t max_seq_len,
                                    const float* sinks, float* out, void* workspace,
                                    size_t workspace_bytes, int32_t pages_per_split,
                                    void* stream) {
  flint::DecodeArgs a;
  flint_status st = prepare_decode(L, num_seqs, k_cache, v_cache, num_blocks, block_tables,
                                   bt_stride, seq_lens, max_seq_len, sinks, out, workspace,
                                   workspace_bytes, pages_per_split, &a);
  if (st != FLINT_OK || num_seqs == 0) return st == FLINT_OK ? ok() : st;
  if (!q_in || !k_in || !v_in || !q_norm_w || !k_norm_w || !slot_mapping)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(q_in, 4) || !aligned(k_in, 4) || !aligned(v_in, 4) || !aligned(q_norm_w, 4) ||
      !aligned(k_norm_w, 4) || !aligned(slot_mapping, 4) || (q_out && !aligned(q_out, 4)))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "misaligned pointer");
  const size_t qbytes = (size_t)num_seqs * L->num_q_heads * 128 * sizeof(float);
  if (overlap(q_in, qbytes, out, qbytes) || (q_out && overlap(q_out, qbytes, out, qbytes)))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "out must not alias q_in or q_out");
  // every split workgroup reads the raw q_in while split 0 writes q_out, so a
  // shared buffer would let later splits normalise an already normalised q
  if (q_out && overlap(q_out, qbytes, q_in, qbytes))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "q_out must not alias q_in in the fused step");
  a.q_in = q_in;
  a.k_in = k_in;
  a.v_in = v_in;
  a.q_w = q_norm_w;
  a.k_w = k_norm_w;
  a.slots = slot_mapping;
  a.q_out = q_out;
  return hip_status(flint::launch_decode(a, (hipStream_t)stream), "decode step launch");
}

flint_status flint_attn_decode_step_noalloc(
    const flint_attn_layer* L, int32_t num_seqs, const float* q_in, const float* k_in,
    const float* v_in, const float* q_norm_w, const float* k_norm_w,
    const int32_t* slot_mapping, float* q_out, void* k_cache, void* v_cache, int32_t num_blocks,
    const int32_t* block_tables, int32_t bt_stride, const int32_t* seq_lens,
    int32_t max_seq_len, const float* sinks, float* out, int32_t pages_per_split, void* stream) {
  flint_status st = check_layer(L);
  if (st != FLINT_OK) return st;
  if (num_seqs < 0) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", num_seqs);
  if (pages_per_split < 0)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "pages_per_split %d < 0", pages_per_split);
  if (max_seq_len < 1 || max_seq_len > kMaxContext)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "max_seq_len %d outside [1, %d]", max_seq_len,
                kMaxContext);
  if (num_seqs == 0) return ok();
  const size_t need = decode_ws_bytes(L, num_seqs, make_plan(L, num_seqs, max_seq_len,
                                                             pages_per_split));
  if (need > kScratchBytes)
    return fail(FLINT_ERR_WORKSPACE_TOO_SMALL,
                "this batch needs %zu bytes of split partials, above the %zu-byte static "
                "scratch of the allocation-free step (use flint_attn_decode_step with a "
                "workspace)", need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_for_current_device(&ws);
    if (st != FLINT_OK) return st;
  }
  return flint_attn_decode_step(L, num_seqs, q_in, k_in, v_in, q_norm_w, k_norm_w, slot_mapping,
                                q_out, k_cache, v_cache, num_blocks, block_tables, bt_stride,
                                seq_lens, max_seq_len, sinks, out, ws, need, pages_per_split,
                                stream);
}

flint_status flint_attn_decode(const flint_attn_layer* L, int32_t num_seqs, const float* q,
                               const void* k_cache, const void* v_cache,
                               int32_t num_blocks, const int32_t* block_tables,
                               int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                               const float* sinks, float* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return flint_attn_decode_ex(L, num_seqs, q, k_cache, v_cache, num_blocks, block_tables,
                              bt_stride, seq_lens, max_seq_len, sinks, out, workspace,
                              workspace_bytes, 0, stream);
}

flint_status flint_attn_decode_partials(const flint_attn_layer* L, int32_t num_seqs,
                                        const float* q, const void* k_cache,
                                        const void* v_cache, int32_t num_blocks,
                                        const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* seq_lens, int32_t max_seq_len,
                                        int32_t pages_per_split, int32_t num_splits,
                                        float* part_o, float* part_lse, void* stream) {
  flint_status st = check_layer(L);
  if (st != FLINT_OK) return st;
  if (pages_per_split < 1)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "pages_per_split %d < 1", pages_per_split);
  if (num_seqs < 0) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", num_seqs);
  if (max_seq_len < 1 || max_seq_len > kMaxContext)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "max_seq_len %d outside [1, %d]", max_seq_len,
                kMaxContext);
  const Plan pl = make_plan(L, num_seqs, max_seq_len, pages_per_split);
  if (num_splits != pl.num_splits)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "num_splits %d, the plan has %d", num_splits,
                pl.num_splits);
  if (num_seqs == 0) return ok();
  if (!q || !k_cache || !v_cache || !block_tables || !seq_lens || !part_o || !part_lse)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (num_blocks < 1) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_blocks %d < 1", num_blocks);
  if (bt_stride < 1) return fail(FLINT_ERR_INVALID_ARGUMENT, "bt_stride %d < 1", bt_stride);
  if ((int64_t)max_seq_len > (int64_t)bt_stride * 16)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "max_seq_len %d exceeds bt_stride*16 = %lld",
                max_seq_len, (long long)bt_stride * 16);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(part_o, 16) || !aligned(part_lse, 4) || !aligned(block_tables, 4) ||
      !aligned(seq_lens, 4))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "misaligned pointer (q, caches, part_o need 16 B)");
  flint::DecodeArgs a{};
  a.q = q;
  a.k_cache = const_cast<void*>(k_cache);
  a.v_cache = const_cast<void*>(v_cache);
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.num_seqs = num_seqs;
  a.num_kv_heads = L->num_kv_heads;
  a.num_blocks = num_blocks;
  a.bt_stride = bt_stride;
  a.window = L->window;
  a.max_seq_len = max_seq_len;
  a.pages_per_split = pl.pages_per_split;
  a.num_splits = pl.num_splits;
  a.partials_only = 1;
  set_kv_format(L, &a);
  return hip_status(flint::launch_decode(a, (hipStream_t)stream), "partials launch");
}

flint_status flint_attn_merge(const flint_attn_layer* L, int32_t num_seqs, int32_t num_splits,
                              const float* part_o, const float* part_lse, const float* sinks,
                              float* out, void* stream) {
  flint_status st = check_layer(L);
  if (st != FLINT_OK) return st;
  if (num_seqs < 0) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", num_seqs);
  if (num_splits < 1) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_splits %d < 1", num_splits);
  if (num_seqs == 0) return ok();
  if (!part_o || !part_lse || !sinks || !out)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(part_o, 4) || !aligned(part_lse, 4) || !aligned(sinks, 4) || !aligned(out, 4))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "misaligned pointer");
  flint::DecodeArgs a{};
  a.part_o = const_cast<float*>(part_o);
  a.part_lse = const_cast<float*>(part_lse);
  a.sinks = sinks;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_kv_heads = L->num_kv_heads;
  a.num_splits = num_splits;
  return hip_status(flint::launch_merge(a, (hipStream_t)stream), "merge launch");
}

size_t flint_attn_prefill_workspace_size(const flint_attn_layer* L, int32_t num_seqs,
                                         int32_t max_q_len, int32_t max_seq_len) {
  (void)max_seq_len;
  if (!L) return 0;
  return flint::prefill_workspace_bytes(num_seqs, L->num_kv_heads, max_q_len);
}

flint_status flint_attn_prefill(const flint_attn_layer* L, int32_t num_seqs, const uint16_t* q,
                                const int32_t* cu_q_lens, int32_t total_q, int32_t max_q_len,
                                const void* k_cache, const void* v_cache,
                                int32_t num_blocks, const int32_t* block_tables,
                                int32_t bt_stride, const int32_t* seq_lens, int32_t max_seq_len,
                                const float* sinks, float* out, void* workspace,
                                size_t workspace_bytes, void* stream) {
  flint_status st = check_layer(L);
  if (st != FLINT_OK) return st;
  if (num_seqs < 0) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_seqs %d < 0", num_seqs);
  if (max_seq_len < 1 || max_seq_len > kMaxContext)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "max_seq_len %d outside [1, %d]", max_seq_len,
                kMaxContext);
  if (max_q_len < 0 || max_q_len > max_seq_len)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "max_q_len %d outside [0, max_seq_len]", max_q_len);
  if (total_q < 0) return fail(FLINT_ERR_INVALID_ARGUMENT, "total_q %d < 0", total_q);
  if (num_seqs == 0 || max_q_len == 0 || total_q == 0) return ok();
  if (!q || !cu_q_lens || !k_cache || !v_cache || !block_tables || !seq_lens || !sinks || !out)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (num_blocks < 1) return fail(FLINT_ERR_INVALID_ARGUMENT, "num_blocks %d < 1", num_blocks);
  if (bt_stride < 1) return fail(FLINT_ERR_INVALID_ARGUMENT, "bt_stride %d < 1", bt_stride);
  if ((int64_t)max_seq_len > (int64_t)bt_stride * 16)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "max_seq_len %d exceeds bt_stride*16", max_seq_len);
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(sinks, 4) ||
      !aligned(cu_q_lens, 4))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "misaligned pointer (q, out, caches need 16 B)");
  flint::PrefillArgs a;
  a.q = q;
  a.cu_q_lens = cu_q_lens;
  a.total_q = total_q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.sinks = sinks;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_kv_heads = L->num_kv_heads;
  a.num_blocks = num_blocks;
  a.bt_stride = bt_stride;
  a.window = L->window;
  a.max_q_len = max_q_len;
  a.max_seq_len = max_seq_len;
  a.kv_fp8 = L->kv_dtype == FLINT_KV_FP8_E4M3;
  a.qscale = L->softmax_scale * 1.4426950408889634f * (a.kv_fp8 ? L->k_scale : 1.f);
  a.v_scale = a.kv_fp8 ? L->v_scale : 1.f;
  const size_t need = flint::prefill_workspace_bytes(num_seqs, L->num_kv_heads, max_q_len);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(FLINT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                need);
  if (need > 0 && !aligned(workspace, 8))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "workspace must be 8-byte aligned");
  a.claims = need > 0 ? (unsigned long long*)workspace : nullptr;
  return hip_status(flint::launch_prefill(a, (hipStream_t)stream), "prefill launch");
}

}  // extern "C"
