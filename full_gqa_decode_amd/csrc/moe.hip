// moe.hip -- Flint's MoE sublayer at small-batch decode (1..8 tokens):
// router GEMV, sigmoid top-k, routed and shared SwiGLU expert GEMVs.
//
// What is computed ("Day-0 Support for Flint on vLLM", hnkhoi.com, "Model
// architecture": hidden size 2048, 256 experts, sigmoid top-6, a shared
// expert; newruntime.com, "What happened": small-batch MoE and dense GEMV
// kernels), with the readings the oracle states (no router bias; top-k on the
// fp32 logits, ties to the lower index; weights = selected sigmoid scores
// normalised to sum 1; SwiGLU experts; the shared expert with weight 1):
//   z_e = <x, Wr_e>,  w_k = s_{id_k} / sum_j s_{id_j},  s = sigmoid(z)
//   y = sum_k w_k Wd_{id_k} (silu(Wg_{id_k} x) * (Wu_{id_k} x)) + shared terms
//
// Design for gfx950.  At 1..8 tokens every weight row feeds at most a few dot
// products, so the sublayer is a stream of bf16 weight rows from HBM (45 MB
// per token at Flint's shape) and the work goes on the vector ALU, not the
// matrix cores.  Each wave owns whole weight rows and reads a row with
// 16-byte lane loads -- one 1 KiB contiguous load per instruction --, widens
// bf16 to fp32 exactly (a shift) and accumulates fp32 FMAs against x; a
// DPP/permlane reduction gives the dot product.  Three launches:
//   K5a router logits (one workgroup per expert row, one wave per 512-element
//       chunk of it, every token);
//   K5b top-k -- recomputed by one wave of every workgroup from the token's
//       logits, so no launch is spent on it -- then the gate and up rows and
//       SwiGLU (each wave two FFN rows of one (slot, token));
//   K5c down rows and the weighted combine (one wave per (output row, token)).
// Every wave issues all of its row loads before it waits for any, so each
// launch costs one dependent memory round trip after its inputs arrive.
#include <climits>

#include "device.h"
#include "moe.h"

namespace flint {

namespace {

constexpr int kMoeWaves = 4;  // waves per workgroup

// 8 bf16 (one 16-byte load) -> 8 fp32, exactly.
__device__ __forceinline__ void widen8(const u32x4& w, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ float dot8(const u32x4& w, const f32x4& x0, const f32x4& x1,
                                      float acc) {
  float f[8];
  widen8(w, f);
  acc = fmaf(f[0], x0[0], acc);
  acc = fmaf(f[1], x0[1], acc);
  acc = fmaf(f[2], x0[2], acc);
  acc = fmaf(f[3], x0[3], acc);
  acc = fmaf(f[4], x1[0], acc);
  acc = fmaf(f[5], x1[1], acc);
  acc = fmaf(f[6], x1[2], acc);
  return fmaf(f[7], x1[3], acc);
}

__device__ __forceinline__ int wave_min_i32(int x) {
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x124, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x122, 0xF, 0xF, false));
  x = min(x, __builtin_amdgcn_update_dpp(0, x, 0x121, 0xF, 0xF, false));
  return min(min(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             min(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// K5a: z[t][e] = <x_t, Wr_e> for every token.  One workgroup per expert row
// (the 1 MB of router rows spreads over every CU) and one wave per 512-element
// chunk of it (hidden / 512 waves).  A wave requests its 1 KiB of the row and
// the same chunk of every token's x at once -- unconditionally, with the token
// index clamped, since a load under a branch is waited for at the join -- so
// the launch costs one memory round trip; the chunks' partial dots meet in
// LDS.  NT: token slots, 1, 2, 4 or 8 >= num_tokens.
static_assert(kMoeMaxTokens == 8, "router token slots are 1, 2, 4 or 8");

template <int NT>
__global__ __launch_bounds__(kMoeMaxChunks * 64) void moe_router_kernel(MoeArgs a) {
  const int lane = threadIdx.x & 63;
  const int c = threadIdx.x >> 6;
  const int nch = blockDim.x >> 6;
  const int e = blockIdx.x;
  const int H = a.hidden;
  __shared__ float sm_z[kMoeMaxChunks][NT];
  const u32x4 wv =
      __builtin_nontemporal_load((const u32x4*)(a.w_router + (int64_t)e * H + c * 512 + lane * 8));
  f32x4 x0[NT], x1[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int tt = min(t, a.num_tokens - 1);
    const float* xp = a.x + (int64_t)tt * H + c * 512 + lane * 8;
    x0[t] = *(const f32x4*)xp;
    x1[t] = *(const f32x4*)(xp + 4);
  }
  // every load above is in flight before the first dot product waits
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float z = wave_sum_f32(dot8(wv, x0[t], x1[t], 0.f));
    if (lane == 0) sm_z[c][t] = z;
  }
  __syncthreads();
  const int t = threadIdx.x;
  if (t < NT && t < a.num_tokens) {
    float z = 0.f;
    for (int i = 0; i < nch; ++i) z += sm_z[i][t];
    a.logits[(int64_t)t * a.num_experts + e] = z;
  }
}

// The top_k experts of token t (largest logit first, lower index on ties) and
// their normalised sigmoid weights; every lane gets the same.  Lane l holds
// experts l, l+64, l+128, l+192 (at most 256 experts).
struct TopK {
  int ids[kMoeMaxTopK];
  float weights[kMoeMaxTopK];
};

__device__ __forceinline__ TopK select_topk(const MoeArgs& a, int t, int lane) {
  const int E = a.num_experts;
  float z[4], zs[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    // unconditional (a clamped index), so the four loads are in flight at once
    const float zl = a.logits[(int64_t)t * E + min(e, E - 1)];
    z[i] = e < E ? zl : -INFINITY;
    if (z[i] != z[i]) z[i] = -INFINITY;  // a NaN logit ranks last
    zs[i] = z[i];
  }
  TopK r;
  float ssum = 0.f;
#pragma unroll
  for (int k = 0; k < kMoeMaxTopK; ++k) {
    if (k >= a.top_k) break;
    float v = z[0];
    int idx = lane;
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (z[i] > v) {  // strict: the lower index wins among equals
        v = z[i];
        idx = lane + 64 * i;
      }
    const float m = wave_max_f32(v);
    int win = wave_min_i32(v == m ? idx : INT_MAX);
    win = win < E ? win : 0;  // unreachable for finite logits; keeps the index valid
    float zw = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (lane + 64 * i == win) {
        zw = zs[i];
        z[i] = -INFINITY;  // taken
      }
    }
    zw = wave_sum_f32(zw);  // the winner's logit, from its lane
    r.ids[k] = win;
    r.weights[k] = 1.f / (1.f + __expf(-zw));
    ssum += r.weights[k];
  }
#pragma unroll
  for (int k = 0; k < kMoeMaxTopK; ++k)
    if (k < a.top_k) r.weights[k] /= ssum;
  return r;
}

// K5b: h[t][slot][j] = silu(<x_t, Wg_j>) * <x_t, Wu_j> for the expert of the
// slot (slots top_k.. are the shared experts).  Grid (FFN rows / (4 * kJW),
// slots, tokens); each wave takes kJW FFN rows j.  Wave 0 selects the token's
// experts and passes the slot's expert to the others through LDS; the first
// workgroup of each token also writes the token's top-k ids and weights.
constexpr int kJW = 2;  // FFN rows per wave
static_assert(kMoeMaxInter % (kMoeWaves * kJW) == 0, "whole FFN rows per wave");

template <int CH>
__global__ __launch_bounds__(kMoeWaves * 64) void moe_gate_up_kernel(MoeArgs a) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int slot = blockIdx.y, t = blockIdx.z;
  const int j0 = (blockIdx.x * kMoeWaves + w) * kJW;
  const int H = a.hidden, I = a.inter;
  const int nslots = a.top_k + a.num_shared;
  __shared__ int sm_expert;
  // x does not wait for the selection
  f32x4 x0[CH], x1[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const float* xp = a.x + (int64_t)t * H + c * 512 + lane * 8;
    x0[c] = *(const f32x4*)xp;
    x1[c] = *(const f32x4*)(xp + 4);
  }
  int expert = a.num_experts + (slot - a.top_k);
  if (slot < a.top_k) {
    if (w == 0) {
      const TopK tk = select_topk(a, t, lane);
#pragma unroll
      for (int k = 0; k < kMoeMaxTopK; ++k)
        if (k == slot) expert = tk.ids[k];
      if (lane == 0) sm_expert = expert;
      if (blockIdx.x == 0 && slot == 0) {
        int id = 0;
        float wt = 0.f;
#pragma unroll
        for (int k = 0; k < kMoeMaxTopK; ++k)
          if (k == lane) {
            id = tk.ids[k];
            wt = tk.weights[k];
          }
        if (lane < a.top_k) {
          a.topk_ids[t * a.top_k + lane] = id;
          a.topk_weights[t * a.top_k + lane] = wt;
        }
      }
    }
    __syncthreads();
    expert = sm_expert;
  }
  // every row of the wave requested before any is used (I is a multiple of
  // 4 * kJW, so all kJW rows exist)
  u32x4 gv[kJW][CH], uv[kJW][CH];
#pragma unroll
  for (int jj = 0; jj < kJW; ++jj) {
    const uint16_t* wg = a.w_gate_up + ((int64_t)expert * 2 * I + j0 + jj) * H + lane * 8;
    const uint16_t* wu = wg + (int64_t)I * H;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      gv[jj][c] = __builtin_nontemporal_load((const u32x4*)(wg + c * 512));
      uv[jj][c] = __builtin_nontemporal_load((const u32x4*)(wu + c * 512));
    }
  }
#pragma unroll
  for (int jj = 0; jj < kJW; ++jj) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      g = dot8(gv[jj][c], x0[c], x1[c], g);
      u = dot8(uv[jj][c], x0[c], x1[c], u);
    }
    g = wave_sum_f32(g);
    u = wave_sum_f32(u);
    if (lane == 0)
      a.h[((int64_t)t * nslots + slot) * I + j0 + jj] = g / (1.f + __expf(-g)) * u;
  }
}

// K5c: out[t][r] = sum_k w_k <Wd_{id_k}[r], h[t][k]> + sum_s <Wd_s[r], h[t][s]>.
// One wave per (output row r, token t), every slot's row loaded up front.
// NS = top_k + num_shared, a template argument so that the slot loop has no
// branch: at a branch's join the compiler waits for the loads issued inside
// it, which would cost one memory round trip per slot.  The token's h (NS x
// 2 KiB) is staged once per workgroup in LDS: read by every wave from memory
// it would be twice the bytes of the wave's own rows (NS x 1 KiB), all
// through the CU's one load path.
template <int NS>
__global__ __launch_bounds__(kMoeWaves * 64) void moe_down_kernel(MoeArgs a) {
  static_assert(kMoeMaxInter == 512, "one 16-byte lane load per row");
  constexpr int kThreads = kMoeWaves * 64;
  constexpr int kChunks = NS * kMoeMaxInter / 4;  // 16-byte chunks of h
  constexpr int kPasses = (kChunks + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) float sm_h[NS * kMoeMaxInter];
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.y;
  const int H = a.hidden, I = a.inter;
  const int r_w = blockIdx.x * kMoeWaves + (threadIdx.x >> 6);
  const int r = min(r_w, H - 1);  // every wave meets the barrier; past H none stores
  // the token's expert ids and weights in one vector load (lane k holds slot
  // k's, the index clamped), so one wait precedes every row address
  const int kl = t * a.top_k + min(lane, a.top_k - 1);
  const int id_l = a.topk_ids[kl];
  const float wt_l = a.topk_weights[kl];
  // h: unconditional loads (index clamped), so no wait lands on a branch
  const f32x4* hg = (const f32x4*)(a.h + (int64_t)t * NS * I);
  f32x4 hs[kPasses];
#pragma unroll
  for (int i = 0; i < kPasses; ++i) hs[i] = hg[min((int)threadIdx.x + i * kThreads, kChunks - 1)];
  u32x4 wv[NS];
  float wk[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const bool routed = k < a.top_k;
    const int kr = min(k, kMoeMaxTopK - 1);
    const int e = routed ? __builtin_amdgcn_readlane(id_l, kr) : a.num_experts + (k - a.top_k);
    wk[k] = routed ? readlane_f32(wt_l, kr) : 1.f;
    const uint16_t* wd = a.w_down + ((int64_t)e * H + r) * I + lane * 8;
    wv[k] = __builtin_nontemporal_load((const u32x4*)wd);
  }
#pragma unroll
  for (int i = 0; i < kPasses; ++i) {
    const int c = threadIdx.x + i * kThreads;
    if (c < kChunks) ((f32x4*)sm_h)[c] = hs[i];
  }
  __syncthreads();
  float y = 0.f;
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const f32x4 h0 = *(const f32x4*)&sm_h[k * kMoeMaxInter + lane * 8];
    const f32x4 h1 = *(const f32x4*)&sm_h[k * kMoeMaxInter + lane * 8 + 4];
    y = fmaf(wk[k], wave_sum_f32(dot8(wv[k], h0, h1, 0.f)), y);
  }
  if (lane == 0 && r_w < H) a.out[(int64_t)t * H + r] = y;
}

template <int CH>
hipError_t launch_moe_ch(const MoeArgs& a, hipStream_t s) {
  const dim3 block(kMoeWaves * 64);
  const int rows_per_wg = kMoeWaves * kJW;
  const dim3 g2(a.inter / rows_per_wg, a.top_k + a.num_shared, a.num_tokens);
  hipLaunchKernelGGL((moe_gate_up_kernel<CH>), g2, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moe(const MoeArgs& a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  const dim3 block(kMoeWaves * 64);
  const dim3 rblock(a.hidden / 512 * 64);
  const dim3 rgrid(a.num_experts);
  if (a.num_tokens <= 1)
    hipLaunchKernelGGL((moe_router_kernel<1>), rgrid, rblock, 0, s, a);
  else if (a.num_tokens <= 2)
    hipLaunchKernelGGL((moe_router_kernel<2>), rgrid, rblock, 0, s, a);
  else if (a.num_tokens <= 4)
    hipLaunchKernelGGL((moe_router_kernel<4>), rgrid, rblock, 0, s, a);
  else
    hipLaunchKernelGGL((moe_router_kernel<8>), rgrid, rblock, 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.hidden / 512) {  // the API admits multiples of 512 up to kMoeMaxChunks * 512
    case 1: e = launch_moe_ch<1>(a, s); break;
    case 2: e = launch_moe_ch<2>(a, s); break;
    case 3: e = launch_moe_ch<3>(a, s); break;
    case 4: e = launch_moe_ch<4>(a, s); break;
    case 5: e = launch_moe_ch<5>(a, s); break;
    case 6: e = launch_moe_ch<6>(a, s); break;
    case 7: e = launch_moe_ch<7>(a, s); break;
    default: e = launch_moe_ch<8>(a, s); break;
  }
  if (e != hipSuccess) return e;
  const dim3 dgrid((a.hidden + kMoeWaves - 1) / kMoeWaves, a.num_tokens);
  static_assert(kMoeMaxTopK + kMoeMaxShared == 10, "one case per slot count");
  switch (a.top_k + a.num_shared) {  // the API admits 1..kMoeMaxTopK + kMoeMaxShared
    case 1: hipLaunchKernelGGL((moe_down_kernel<1>), dgrid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((moe_down_kernel<2>), dgrid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((moe_down_kernel<3>), dgrid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((moe_down_kernel<4>), dgrid, block, 0, s, a); break;
    case 5: hipLaunchKernelGGL((moe_down_kernel<5>), dgrid, block, 0, s, a); break;
    case 6: hipLaunchKernelGGL((moe_down_kernel<6>), dgrid, block, 0, s, a); break;
    case 7: hipLaunchKernelGGL((moe_down_kernel<7>), dgrid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((moe_down_kernel<8>), dgrid, block, 0, s, a); break;
    case 9: hipLaunchKernelGGL((moe_down_kernel<9>), dgrid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((moe_down_kernel<10>), dgrid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace flint
