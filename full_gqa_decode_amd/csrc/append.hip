// append.hip -- K1: fused per-head Q/K RMSNorm, RoPE and paged KV append.
//
// "Day-0 Support for Flint on vLLM" (newruntime.com), "What happened": the
// optimised path fuses normalisation, rotary-position and cache operations.
// "Day-0 Support for Flint on vLLM" (hnkhoi.com), "Model architecture":
// per-head Q/K RMSNorm; RoPE on the 35 sliding layers, none on the 14 full
// layers.  Order: norm, then rotation, then the cache write (bf16, or fp8
// E4M3 of the value over the layer's scale).
//
// One wave64 handles one head of one token: lane l holds dims l and l+64,
// which is exactly a rotate-half RoPE pair, so the rotation needs no lane
// exchange and the only cross-lane step is the sum of squares.  A workgroup of
// four waves covers four of the token's (num_q_heads + 2*num_kv_heads) heads.
// The arithmetic is fp64 (full rate on gfx950, and this kernel is tiny): the
// fp32 q output is the correctly rounded normalised/rotated value, and the
// bf16 K is rounded once from the fp64 value (round-to-odd to fp32, then
// round-to-nearest-even to bf16), so it matches an exact computation except
// on ties closer than ~1e-15 relative; fp8 codes are rounded once from the
// fp64 quotient.
// Launch-latency bound at decode (one token per request); bandwidth bound for
// long prefill chunks (~4.5 KB read and written per token for 32/4 heads).
#include "device.h"
#include "launch.h"

namespace flint {

namespace {

__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int tasks = hq + 2 * hkv;
  const int groups = (tasks + 3) >> 2;
  const int t = blockIdx.x / groups;
  const int task = (blockIdx.x % groups) * 4 + (threadIdx.x >> 6);
  if (t >= a.num_tokens || task >= tasks) return;

  const int pos = a.positions[t];
  const int slot = a.slots[t];
  const bool bad = pos < 0 || (int64_t)slot >= (int64_t)a.num_blocks * kPage;
  const bool write_cache = slot >= 0 && !bad;

  if (task >= hq + hkv) {  // V: round to bf16 (or fp8) and store dim-major
    if (!write_cache) return;
    const int g = task - hq - hkv;
    const float* x = a.v_in + ((int64_t)t * hkv + g) * kHeadDim;
    const float v0 = x[lane], v1 = x[lane + 64];
    const int64_t page = slot / kPage, row = slot % kPage;
    const int64_t tile = (page * hkv + g) * (int64_t)(kHeadDim * kPage);
    if (a.kv_fp8) {
      uint8_t* dst = (uint8_t*)a.v_cache + tile;
      dst[fp8_v_off(row, lane)] = (uint8_t)fp8_e4m3_rne_f64((double)v0 / (double)a.v_scale);
      dst[fp8_v_off(row, lane + 64)] =
          (uint8_t)fp8_e4m3_rne_f64((double)v1 / (double)a.v_scale);
    } else {
      uint16_t* dst = (uint16_t*)a.v_cache + tile + row;
      dst[lane * kPage] = bf16_bits_rne(v0);
      dst[(lane + 64) * kPage] = bf16_bits_rne(v1);
    }
    return;
  }

  const bool is_q = task < hq;
  if (!is_q && !write_cache) return;
  const float* x = is_q ? a.q_in + ((int64_t)t * hq + task) * kHeadDim
                        : a.k_in + ((int64_t)t * hkv + (task - hq)) * kHeadDim;
  // RMSNorm over the head's 128 values, then the rotate-half RoPE pair
  // (lane, lane+64) turned by pos * theta^(-2*lane/128).
  double cs = 1.0, sn = 0.0;
  if (a.use_rope) rope_cos_sin(pos < 0 ? 0 : pos, lane, a.rope_theta, &cs, &sn);
  double y0, y1;
  const float* wp = is_q ? a.q_w : a.k_w;
  norm_rope_head(x[lane], x[lane + 64], wp[lane], wp[lane + 64], a.rms_eps, a.use_rope, cs, sn,
                 &y0, &y1);

  if (is_q) {
    if (bad) y0 = y1 = __builtin_nan("");
    const int64_t o = ((int64_t)t * hq + task) * kHeadDim;
    if (a.q_out_f32) {
      a.q_out_f32[o + lane] = (float)y0;
      a.q_out_f32[o + lane + 64] = (float)y1;
    } else {
      a.q_out_bf16[o + lane] = bf16_bits_rne_f64(y0);
      a.q_out_bf16[o + lane + 64] = bf16_bits_rne_f64(y1);
    }
    return;
  }

  const int g = task - hq;
  const int64_t page = slot / kPage, row = slot % kPage;
  const int64_t tile = (page * hkv + g) * (int64_t)(kHeadDim * kPage);
  if (a.kv_fp8) {
    uint8_t* dst = (uint8_t*)a.k_cache + tile;
    dst[fp8_k_off(row, lane)] = (uint8_t)fp8_e4m3_rne_f64(y0 / (double)a.k_scale);
    dst[fp8_k_off(row, lane + 64)] = (uint8_t)fp8_e4m3_rne_f64(y1 / (double)a.k_scale);
  } else {
    uint16_t* dst = (uint16_t*)a.k_cache + tile;
    dst[bf16_k_off(row, lane)] = bf16_bits_rne_f64(y0);
    dst[bf16_k_off(row, lane + 64)] = bf16_bits_rne_f64(y1);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  const int tasks = a.num_q_heads + 2 * a.num_kv_heads;
  const int groups = (tasks + 3) / 4;
  const int64_t blocks = (int64_t)a.num_tokens * groups;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace flint
