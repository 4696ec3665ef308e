// prefill.hip -- K4: causal (optionally windowed) prefill attention with
// sinks on the gfx950 matrix cores.
//
// Same per-row result as decode ("Day-0 Support for Flint on vLLM",
// hnkhoi.com, "Model architecture"; newruntime.com, "What happened", which
// also reports the 8,192-token prefill the optimised path serves), for every
// query row of a chunk at its own position.
//
// Design.  A query vector is one (row, head) pair; the eight heads of a KV
// group share every key, so a 16-wide MFMA tile holds 2 rows x 8 heads.  A
// wave owns kTiles such tiles (kTiles*2 consecutive rows); a workgroup of
// four waves owns kRows rows of one KV group, and its waves walk the same
// key pages in step so the K/V lines fetched by one wave are L1/L2 hits for
// the others.  Per pair of 16-key pages:
//   S^T[32 keys x 16 qv] = K . Q^T     2 x 4 v_mfma_f32_16x16x32_bf16 per tile
//   O[16 qv x 128]      += P . V        8 x 2 v_mfma_f32_16x16x32_bf16 per tile
// The PV contraction runs over 32 keys: MFMA k index gq*8+j takes key gq*4+j
// of the first page for j < 4 and key gq*4+j-4 of the second page for j >= 4,
// which is exactly where the score MFMAs left P, and exactly 2 x 8 contiguous
// bytes of each dim-major V page row.  P is split into bf16(p) and its bf16
// remainder (two MFMAs) so the value product is fp32-accurate.  Online
// softmax in log2 units; the sink joins the denominator in the epilogue.
// Bound: the matrix cores for full layers (4*D flops per (query, key) pair).
#include "device.h"
#include "launch.h"

namespace flint {

namespace {

constexpr int kTiles = 2;               // 16-vector MFMA tiles per wave
constexpr int kWaveRows = kTiles * 2;   // query rows per wave
constexpr int kPWaves = 4;
constexpr int kRows = kWaveRows * kPWaves;  // query rows per workgroup

struct PairRegs {
  bf16x8 ka[4], kb[4];  // K of the two pages (MFMA A operand)
  u32x4 v[8];           // V: keys gq*4..+3 of page a and of page b, one dim
};

__device__ __forceinline__ void load_pair(const PrefillArgs& a, int pga, int pgb, bool has_b,
                                          int g, int n, int gq, PairRegs& r) {
  const int hkv = a.num_kv_heads;
  const uint16_t* ka = a.k_cache + (((int64_t)pga * hkv + g) * kPage + n) * kHeadDim + gq * 8;
  const uint16_t* kb = a.k_cache + (((int64_t)pgb * hkv + g) * kPage + n) * kHeadDim + gq * 8;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    r.ka[c] = *(const bf16x8*)(ka + c * 32);
    r.kb[c] = has_b ? *(const bf16x8*)(kb + c * 32) : bf16x8{};
  }
  const uint16_t* va = a.v_cache + (((int64_t)pga * hkv + g) * kHeadDim + n) * kPage + gq * 4;
  const uint16_t* vb = a.v_cache + (((int64_t)pgb * hkv + g) * kHeadDim + n) * kPage + gq * 4;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    const u32x2 x = *(const u32x2*)(va + nb * 16 * kPage);
    const u32x2 y = has_b ? *(const u32x2*)(vb + nb * 16 * kPage) : u32x2{0u, 0u};
    r.v[nb] = u32x4{x[0], x[1], y[0], y[1]};
  }
}

template <bool WINDOWED>
__global__ __launch_bounds__(kPWaves * 64) void prefill_kernel(PrefillArgs a) {
  const int ntile = gridDim.x;
  const int tile = ntile - 1 - blockIdx.x;  // longest key ranges first
  const int g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, gq = lane >> 4;
  const int hkv = a.num_kv_heads, hq = hkv * kGroup;

  const int q0 = a.cu_q_lens[b];
  const int q_len = a.cu_q_lens[b + 1] - q0;
  const int seq_len = a.seq_lens[b];
  const int row0 = tile * kRows + w * kWaveRows;  // first row of this wave
  if (q_len <= 0 || row0 >= q_len) return;         // no rows here
  const bool req_bad = q_len > a.max_q_len || seq_len > a.max_seq_len || q_len > seq_len;
  const int rows_here = min(kWaveRows, q_len - row0);
  const int pos0 = seq_len - q_len + row0;           // position of the wave's first row
  const int pos_last = pos0 + rows_here - 1;

  // Q operands: tile mt, column n -> row row0 + 2*mt + (n>>3), head g*8 + (n&7)
  bf16x8 qop[kTiles][4];
  int qpos[kTiles];
#pragma unroll
  for (int mt = 0; mt < kTiles; ++mt) {
    const int r = min(row0 + 2 * mt + (n >> 3), q_len - 1);
    qpos[mt] = seq_len - q_len + row0 + 2 * mt + (n >> 3);
    const uint16_t* qp = a.q + (((int64_t)(q0 + r) * hq) + g * kGroup + (n & 7)) * kHeadDim + gq * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c) qop[mt][c] = req_bad ? bf16x8{} : *(const bf16x8*)(qp + c * 32);
  }

  const int lo_first = WINDOWED ? max(0, pos0 - a.window + 1) : 0;
  const int lo_last = WINDOWED ? max(0, pos_last - a.window + 1) : 0;
  const int p_first = lo_first / kPage, p_last = pos_last / kPage;

  f32x4 acc[kTiles][8];
  float m_run[kTiles], l_part[kTiles];
#pragma unroll
  for (int mt = 0; mt < kTiles; ++mt) {
    m_run[mt] = -INFINITY;
    l_part[mt] = 0.f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int bad = req_bad;

  for (int p = req_bad ? p_last + 1 : p_first; p <= p_last; p += 2) {
    const bool has_b = p + 1 <= p_last;
    int pga = a.block_tables[(int64_t)b * a.bt_stride + p];
    int pgb = has_b ? a.block_tables[(int64_t)b * a.bt_stride + p + 1] : pga;
    if (pga < 0 || pga >= a.num_blocks) { bad = 1; pga = 0; }
    if (pgb < 0 || pgb >= a.num_blocks) { bad = 1; pgb = 0; }
    PairRegs pr;
    load_pair(a, pga, pgb, has_b, g, n, gq, pr);

    // keys of this pair that some row of the wave may not see
    const int key_lo = p * kPage, key_hi = p * kPage + 2 * kPage - 1;
    const bool edge = key_lo < lo_last || key_hi > pos0 || !has_b;
    if (edge) {  // zero V of keys no row of the wave may see (unwritten slots)
      uint32_t keep[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = p * kPage + (j >= 4 ? kPage : 0) + gq * 4 + (j & 3);
        const bool ok = key >= lo_first && key <= pos_last && (j < 4 || has_b);
        keep[j] = ok ? 0xffffu : 0u;
      }
      const u32x4 mk = {keep[0] | (keep[1] << 16), keep[2] | (keep[3] << 16),
                        keep[4] | (keep[5] << 16), keep[6] | (keep[7] << 16)};
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) pr.v[nb] &= mk;
    }

#pragma unroll
    for (int mt = 0; mt < kTiles; ++mt) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pr.ka[c], qop[mt][c], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pr.kb[c], qop[mt][c], sb, 0, 0, 0);
      }
      float sv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = sa[i] * a.qscale;
        sv[4 + i] = sb[i] * a.qscale;
      }
      if (edge) {
        const int qp = min(qpos[mt], pos_last);  // rows past the chunk end: any finite cut
        const int qlo = WINDOWED ? qp - a.window + 1 : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = p * kPage + (j >= 4 ? kPage : 0) + gq * 4 + (j & 3);
          if (key < qlo || key > qp || (j >= 4 && !has_b)) sv[j] = -INFINITY;
        }
      }
      float pmax = sv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) pmax = fmaxf(pmax, sv[j]);
      pmax = fmaxf(pmax, __shfl_xor(pmax, 16));
      pmax = fmaxf(pmax, __shfl_xor(pmax, 32));
      // rows past the chunk end see no key at all; keep them finite
      const float m_new = fmaxf(m_run[mt], pmax);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      if (__any(m_new > m_run[mt])) {
        const float alpha = exp2_fast(m_run[mt] - m_use);
        l_part[mt] *= alpha;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, gq * 4 + i);
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mt][nb][i] *= al[i];
      }
      m_run[mt] = m_new;
      float pv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) pv[j] = exp2_fast(sv[j] - m_use);
      l_part[mt] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
      bf16x8 ph, pl;
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const f32x2 pp = {pv[j], pv[j + 1]};
        const bf16x2 h = __builtin_convertvector(pp, bf16x2);
        const bf16x2 l = __builtin_convertvector(pp - __builtin_convertvector(h, f32x2), bf16x2);
        ph[j] = h[0];
        ph[j + 1] = h[1];
        pl[j] = l[0];
        pl[j + 1] = l[1];
      }
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const bf16x8 vv = __builtin_bit_cast(bf16x8, pr.v[nb]);
        acc[mt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vv, acc[mt][nb], 0, 0, 0);
        acc[mt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vv, acc[mt][nb], 0, 0, 0);
      }
    }
  }

  bad = __any(bad);
  // epilogue: acc rows gq*4+i are query vectors; their m and l live in lane gq*4+i
#pragma unroll
  for (int mt = 0; mt < kTiles; ++mt) {
    float l_c = l_part[mt] + __shfl_xor(l_part[mt], 16);
    l_c += __shfl_xor(l_c, 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = gq * 4 + i;  // query vector of acc row
      const float m = __shfl(m_run[mt], v);
      const float l = __shfl(l_c, v);
      const int r = row0 + 2 * mt + (v >> 3);
      if (r >= q_len) continue;
      const int h = g * kGroup + (v & 7);
      const float sink = a.sinks[h] * kLog2e;
      const float M2 = fmaxf(m, sink);
      const float so = exp2_fast(m - M2);
      const float inv = 1.f / (l * so + exp2_fast(sink - M2));
      float* dst = a.out + ((int64_t)(q0 + r) * hq + h) * kHeadDim + n;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        dst[nb * 16] = bad ? __builtin_nanf("") : acc[mt][nb][i] * so * inv;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.num_seqs == 0 || a.max_q_len == 0) return hipSuccess;
  const dim3 grid((a.max_q_len + kRows - 1) / kRows, a.num_kv_heads, a.num_seqs);
  if (a.window > 0) hipLaunchKernelGGL((prefill_kernel<true>), grid, dim3(kPWaves * 64), 0, st, a);
  else hipLaunchKernelGGL((prefill_kernel<false>), grid, dim3(kPWaves * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace flint
