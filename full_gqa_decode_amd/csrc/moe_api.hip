// moe_api.hip -- the C ABI of the MoE sublayer (declared in include/flint.h):
// argument checks, the workspace layout and the launch.  Like the attention
// entry points, every invalid argument returns a status before any HIP call.
#include <hip/hip_runtime.h>

#include "../../include/flint.h"
#include "moe.h"
#include "status.h"

using namespace flint::abi;

namespace {

flint_status check_moe(const flint_moe_layer* M, int32_t num_tokens) {
  if (!M) return fail(FLINT_ERR_INVALID_ARGUMENT, "MoE descriptor is NULL");
  if (M->hidden < 512 || M->hidden % 512 || M->hidden > flint::kMoeMaxChunks * 512)
    return fail(FLINT_ERR_UNSUPPORTED, "hidden %d (a multiple of 512 up to %d)", M->hidden,
                flint::kMoeMaxChunks * 512);
  if (M->inter != flint::kMoeMaxInter)
    return fail(FLINT_ERR_UNSUPPORTED, "inter %d (only %d)", M->inter, flint::kMoeMaxInter);
  if (M->num_experts < 1 || M->num_experts > flint::kMoeMaxExperts)
    return fail(FLINT_ERR_UNSUPPORTED, "num_experts %d (1..%d)", M->num_experts,
                flint::kMoeMaxExperts);
  if (M->top_k < 1 || M->top_k > flint::kMoeMaxTopK || M->top_k > M->num_experts)
    return fail(FLINT_ERR_UNSUPPORTED, "top_k %d (1..%d, at most num_experts)", M->top_k,
                flint::kMoeMaxTopK);
  if (M->num_shared < 0 || M->num_shared > flint::kMoeMaxShared)
    return fail(FLINT_ERR_UNSUPPORTED, "num_shared %d (0..%d)", M->num_shared,
                flint::kMoeMaxShared);
  if (num_tokens < 0 || num_tokens > flint::kMoeMaxTokens)
    return fail(FLINT_ERR_UNSUPPORTED, "num_tokens %d (0..%d)", num_tokens,
                flint::kMoeMaxTokens);
  return FLINT_OK;
}

// Workspace: [logits T x experts | h T x (top_k + shared) x inter], fp32.
struct MoeWs {
  size_t h, total;
};
MoeWs moe_ws(const flint_moe_layer* M, int32_t num_tokens) {
  MoeWs w;
  w.h = align_up((size_t)num_tokens * M->num_experts * sizeof(float));
  w.total = w.h + align_up((size_t)num_tokens * (M->top_k + M->num_shared) * M->inter *
                           sizeof(float));
  return w;
}

}  // namespace

extern "C" {

size_t flint_moe_workspace_size(const flint_moe_layer* M, int32_t num_tokens) {
  if (check_moe(M, num_tokens) != FLINT_OK) return 0;
  return moe_ws(M, num_tokens).total;
}

flint_status flint_moe_forward(const flint_moe_layer* M, int32_t num_tokens, const float* x,
                               const uint16_t* w_router, const uint16_t* w_gate_up,
                               const uint16_t* w_down, int32_t* topk_ids, float* topk_weights,
                               float* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  flint_status st = check_moe(M, num_tokens);
  if (st != FLINT_OK) return st;
  if (num_tokens == 0) return ok();
  if (!x || !w_router || !w_gate_up || !w_down || !topk_ids || !topk_weights || !out)
    return fail(FLINT_ERR_INVALID_ARGUMENT, "a required pointer is NULL");
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(w_gate_up, 16) ||
      !aligned(w_down, 16) || !aligned(topk_ids, 4) || !aligned(topk_weights, 4) ||
      !aligned(out, 4))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "misaligned pointer (x and weights need 16 B)");
  const size_t xbytes = (size_t)num_tokens * M->hidden * sizeof(float);
  if (overlap(x, xbytes, out, xbytes)) return fail(FLINT_ERR_INVALID_ARGUMENT, "out aliases x");
  const MoeWs wl = moe_ws(M, num_tokens);
  if (!workspace || workspace_bytes < wl.total)
    return fail(FLINT_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes, need %zu", workspace_bytes,
                wl.total);
  if (!aligned(workspace, kWsAlign))
    return fail(FLINT_ERR_INVALID_ARGUMENT, "workspace must be %zu-byte aligned", kWsAlign);
  flint::MoeArgs a;
  a.x = x;
  a.w_router = w_router;
  a.w_gate_up = w_gate_up;
  a.w_down = w_down;
  a.logits = (float*)workspace;
  a.h = (float*)((char*)workspace + wl.h);
  a.topk_ids = topk_ids;
  a.topk_weights = topk_weights;
  a.out = out;
  a.num_tokens = num_tokens;
  a.hidden = M->hidden;
  a.num_experts = M->num_experts;
  a.top_k = M->top_k;
  a.inter = M->inter;
  a.num_shared = M->num_shared;
  return hip_status(flint::launch_moe(a, (hipStream_t)stream), "moe launch");
}

}  // extern "C"
