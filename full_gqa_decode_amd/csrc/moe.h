// moe.h -- arguments and launcher of the MoE sublayer kernels (moe.hip).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace flint {

// MoE sublayer at small-batch decode (moe.hip).
struct MoeArgs {
  const float* x;            // [T][hidden] fp32
  const uint16_t* w_router;  // [experts][hidden] bf16
  const uint16_t* w_gate_up; // [experts + shared][2][inter][hidden] bf16
  const uint16_t* w_down;    // [experts + shared][hidden][inter] bf16
  float* logits;             // workspace [T][experts]
  float* h;                  // workspace [T][top_k + shared][inter]
  int32_t* topk_ids;         // [T][top_k]
  float* topk_weights;       // [T][top_k]
  float* out;                // [T][hidden]
  int32_t num_tokens;
  int32_t hidden;
  int32_t num_experts;
  int32_t top_k;
  int32_t inter;
  int32_t num_shared;
};
hipError_t launch_moe(const MoeArgs& a, hipStream_t s);
// Shapes the MoE kernels support (checked by the API): hidden a multiple of
// 512 up to kMoeMaxChunks * 512, inter == kMoeMaxInter, top_k, shared and
// tokens up to the bounds below, at most 256 routed experts.
constexpr int kMoeMaxChunks = 8;
constexpr int kMoeMaxTopK = 8;
constexpr int kMoeMaxShared = 2;
constexpr int kMoeMaxInter = 512;
constexpr int kMoeMaxTokens = 8;
constexpr int kMoeMaxExperts = 256;

}  // namespace flint
