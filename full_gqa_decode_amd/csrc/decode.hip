// decode.hip -- K2 split-K flash-decode and K3 log-sum-exp merge with sinks.
//
// What is computed ("Day-0 Support for Flint on vLLM", hnkhoi.com, "Model
// architecture": GQA with 32 query / 4 KV heads, learned attention sinks;
// newruntime.com, "What happened": 35 layers over a 513-token window, 14 over
// the full context):
//   out_h = sum_j e^{s_j} V_j / (e^{sink_h} + sum_j e^{s_j}),
//   s_j = scale * <q_h, K_j>, keys lo..t of the request.
//
// Design for gfx950.  One workgroup = kDecodeWaves wave64s on one
// (split, KV head, request); its waves take the split's 16-token pages
// round-robin.  The eight query heads of a KV group share every K and V row,
// so per page the work is two small dense contractions, done on the matrix
// cores:
//   scores  S[16 tok x 16]  = K_page[16 x 128] . Qhl^T[128 x 16]
//           (4 x v_mfma_f32_16x16x32_bf16; columns 0-7 carry bf16(q*c), columns
//           8-15 the bf16 remainder q*c - bf16(q*c) of the same heads, so the
//           sum of the two column halves is the fp32-accurate score)
//   values  O[16 x 128]    += Phl[16 x 16 tok] . V_page[16 tok x 128]
//           (8 x v_mfma_f32_16x16x16_bf16; rows 0-7 bf16(p), rows 8-15 the
//           bf16 remainder of p, summed at the end)
// K is token-major and V dim-major in the cache, so lane l loads its operand
// straight from HBM: 16 contiguous bytes of K row l%16 and 8 contiguous bytes
// (4 tokens) of V dim-row per MFMA, with no LDS staging and no transposes.
// The score tile lands in exactly the lanes that need it as the P operand of
// the value MFMA, so the online softmax (DPP row_ror:8 for the hi+lo sum,
// wavefront shuffles for the page max) never moves P between lanes.  The next
// page's loads are issued before the current page is processed.  Waves merge
// through LDS at the end; splits are merged by K3, which folds in the sink.
// Bound: HBM (8 KiB of K+V per page and KV head against ~20 VALU and 12 MFMA
// instructions per wave).
#include "device.h"
#include "launch.h"

namespace flint {

namespace {

constexpr int kWaves = kDecodeWaves;
constexpr int kThreads = kWaves * 64;

struct PageRegs {
  bf16x8 k[4];  // K rows: MFMA A operand, 32 dims each
  u32x2 v[8];   // V: 4 tokens x 1 dim per 16-dim block (MFMA B operand)
};

__device__ __forceinline__ void load_page(const DecodeArgs& a, int pg, int g, int n, int gq,
                                          PageRegs& r) {
  const int hkv = a.num_kv_heads;
  const uint16_t* kp =
      a.k_cache + (((int64_t)pg * hkv + g) * kPage + n) * kHeadDim + gq * 8;
#pragma unroll
  for (int c = 0; c < 4; ++c) r.k[c] = *(const bf16x8*)(kp + c * 32);
  const uint16_t* vp =
      a.v_cache + (((int64_t)pg * hkv + g) * kHeadDim + n) * kPage + gq * 4;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) r.v[nb] = *(const u32x2*)(vp + nb * 16 * kPage);
}

// Page id of logical page p of request b, or -1 when outside [0, num_blocks).
__device__ __forceinline__ int page_id(const DecodeArgs& a, int b, int p) {
  const int pg = a.block_tables[(int64_t)b * a.bt_stride + p];
  return (pg >= 0 && pg < a.num_blocks) ? pg : -1;
}

template <bool SINGLE, bool WINDOWED>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, gq = lane >> 4;
  const int hq = a.num_kv_heads * kGroup;

  __shared__ float sm_o[kWaves][kGroup][kHeadDim];
  __shared__ float sm_m[kWaves][kGroup];
  __shared__ float sm_l[kWaves][kGroup];
  __shared__ int sm_bad[kWaves];

  const int seq_len = a.seq_lens[b];
  if (seq_len < 1 || seq_len > a.max_seq_len) {
    if (s == 0) {  // poison this request's result
      for (int i = tid; i < kGroup * kHeadDim; i += kThreads) {
        const int h = g * kGroup + (i >> 7);
        if (SINGLE) a.out[((int64_t)b * hq + h) * kHeadDim + (i & 127)] = __builtin_nanf("");
        else if ((i & 127) == 0) a.part_lse[(int64_t)b * a.num_splits * hq + h] = __builtin_nanf("");
      }
    }
    return;
  }
  const int t = seq_len - 1;
  const int lo = WINDOWED ? max(0, t - a.window + 1) : 0;
  const int first_page = lo / kPage, last_page = t / kPage;
  const int p_begin = first_page + s * a.pages_per_split;
  if (p_begin > last_page) return;  // empty split; K3 never reads it
  const int p_end = min(p_begin + a.pages_per_split, last_page + 1);

  // q operand: column n holds head n&7; n < 8 the bf16 part of q*c, n >= 8 the
  // bf16 remainder.  Lane group gq holds dims c*32 + gq*8 .. +7 of block c.
  bf16x8 qop[4];
  {
    const float* qh = a.q + ((int64_t)b * hq + g * kGroup + (n & 7)) * kHeadDim + gq * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 x0 = *(const f32x4*)(qh + c * 32);
      const f32x4 x1 = *(const f32x4*)(qh + c * 32 + 4);
      const float xs[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const f32x2 v = {xs[j] * a.qscale, xs[j + 1] * a.qscale};
        const bf16x2 hi = __builtin_convertvector(v, bf16x2);
        const bf16x2 lo2 = __builtin_convertvector(v - __builtin_convertvector(hi, f32x2), bf16x2);
        const bf16x2 sel = (n < 8) ? hi : lo2;
        qop[c][j] = sel[0];
        qop[c][j + 1] = sel[1];
      }
    }
  }

  f32x4 acc[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  int bad = 0;

  PageRegs nxt;
  int p = p_begin + w;
  if (p < p_end) {
    int pg = page_id(a, b, p);
    bad |= pg < 0;
    load_page(a, pg < 0 ? 0 : pg, g, n, gq, nxt);
  }
  for (; p < p_end; p += kWaves) {
    PageRegs cur = nxt;
    const int pn = p + kWaves;
    if (pn < p_end) {
      int pg = page_id(a, b, pn);
      bad |= pg < 0;
      load_page(a, pg < 0 ? 0 : pg, g, n, gq, nxt);
    }

    // scores for tokens p*16 + gq*4 + i, head n&7 (hi + lo column halves)
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[c], qop[c], sc, 0, 0, 0);
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = sc[i] + lane_xor8(sc[i]);

    // ragged ends of the key range: mask scores, zero V so unwritten slots
    // (which may hold any bits) cannot reach the accumulator
    const int tok0 = p * kPage;
    if (tok0 < lo || tok0 + kPage - 1 > t) {
      uint32_t keep[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tok0 + gq * 4 + i;
        const bool ok = tok >= lo && tok <= t;
        if (!ok) sv[i] = -INFINITY;
        keep[i] = ok ? 0xffffu : 0u;
      }
      const uint32_t mx = keep[0] | (keep[1] << 16), my = keep[2] | (keep[3] << 16);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        cur.v[nb][0] &= mx;
        cur.v[nb][1] &= my;
      }
    }

    // online softmax in log2 units (q carries scale*log2(e))
    float pmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    pmax = fmaxf(pmax, __shfl_xor(pmax, 16));
    pmax = fmaxf(pmax, __shfl_xor(pmax, 32));
    const float m_new = fmaxf(m_run, pmax);
    if (__any(m_new > m_run)) {
      const float alpha = exp2_fast(m_run - m_new);
      l_part *= alpha;
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, (gq * 4 + i) & 7);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[nb][i] *= al[i];
    }
    m_run = m_new;
    float pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = exp2_fast(sv[i] - m_new);
    l_part += (pv[0] + pv[1]) + (pv[2] + pv[3]);

    // P operand: row n = head n&7; n < 8 bf16(p), n >= 8 its bf16 remainder
    const f32x2 p01 = {pv[0], pv[1]}, p23 = {pv[2], pv[3]};
    const bf16x2 h01 = __builtin_convertvector(p01, bf16x2);
    const bf16x2 h23 = __builtin_convertvector(p23, bf16x2);
    const bf16x2 r01 = __builtin_convertvector(p01 - __builtin_convertvector(h01, f32x2), bf16x2);
    const bf16x2 r23 = __builtin_convertvector(p23 - __builtin_convertvector(h23, f32x2), bf16x2);
    const bf16x2 s01 = (n < 8) ? h01 : r01;
    const bf16x2 s23 = (n < 8) ? h23 : r23;
    const bf16x4 pop = {s01[0], s01[1], s23[0], s23[1]};
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          pop, __builtin_bit_cast(bf16x4, cur.v[nb]), acc[nb], 0, 0, 0);
  }

  // per-wave state -> LDS.  l: sum over the four lane groups of head n&7.
  // acc rows gq*4+i: gq 0,1 the bf16 parts of heads 0-7, gq 2,3 the remainders.
  float l_h = l_part + __shfl_xor(l_part, 16);
  l_h += __shfl_xor(l_h, 32);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nb][i] += __shfl_xor(acc[nb][i], 32);
  if (gq < 2) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[w][gq * 4 + i][nb * 16 + n] = acc[nb][i];
  }
  if (lane < kGroup) {
    sm_m[w][lane] = m_run;
    sm_l[w][lane] = l_h;
  }
  bad = __any(bad);
  if (lane == 0) sm_bad[w] = bad;
  __syncthreads();

  int any_bad = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) any_bad |= sm_bad[v];

  for (int i = tid; i < kGroup * kHeadDim; i += kThreads) {
    const int h = i >> 7, d = i & 127;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sm_m[v][h]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float e = exp2_fast(sm_m[v][h] - M);
      L += e * sm_l[v][h];
      o += e * sm_o[v][h][d];
    }
    const int hg = g * kGroup + h;
    if (SINGLE) {
      const float sink = a.sinks[hg] * kLog2e;
      const float M2 = fmaxf(M, sink);
      const float scale_o = exp2_fast(M - M2);
      const float den = exp2_fast(sink - M2) + L * scale_o;
      float r = o * scale_o / den;
      if (any_bad) r = __builtin_nanf("");
      a.out[((int64_t)b * hq + hg) * kHeadDim + d] = r;
    } else {
      const int64_t row = ((int64_t)b * a.num_splits + s) * hq + hg;
      a.part_o[row * kHeadDim + d] = o / L;
      if (d == 0) a.part_lse[row] = any_bad ? __builtin_nanf("") : M + log2_fast(L);
    }
  }
}

// K3: out_h = sum_s w_s o_s / (e^{sink_h} + sum_s w_s), w_s = 2^{lse_s - M},
// in log2 units.  One workgroup per (query head, request), one lane per dim.
template <bool WINDOWED>
__global__ __launch_bounds__(kHeadDim) void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int hq = a.num_kv_heads * kGroup;
  float* dst = a.out + ((int64_t)b * hq + h) * kHeadDim + d;
  const int seq_len = a.seq_lens[b];
  if (seq_len < 1 || seq_len > a.max_seq_len) {
    *dst = __builtin_nanf("");
    return;
  }
  const int t = seq_len - 1;
  const int lo = WINDOWED ? max(0, t - a.window + 1) : 0;
  const int pages = t / kPage - lo / kPage + 1;
  const int ns = (pages + a.pages_per_split - 1) / a.pages_per_split;
  const int64_t base = (int64_t)b * a.num_splits * hq + h;
  const float sink = a.sinks[h] * kLog2e;
  float M = sink;
  bool nan = false;
  for (int s = 0; s < ns; ++s) {
    const float l = a.part_lse[base + (int64_t)s * hq];
    nan |= l != l;
    M = fmaxf(M, l);
  }
  float den = exp2_fast(sink - M), o = 0.f;
  for (int s = 0; s < ns; ++s) {
    const int64_t row = base + (int64_t)s * hq;
    const float wgt = exp2_fast(a.part_lse[row] - M);
    den += wgt;
    o += wgt * a.part_o[row * kHeadDim + d];
  }
  *dst = nan ? __builtin_nanf("") : o / den;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.num_seqs == 0) return hipSuccess;
  const dim3 grid(a.num_splits, a.num_kv_heads, a.num_seqs);
  const bool win = a.window > 0;
  if (a.num_splits == 1) {
    if (win) hipLaunchKernelGGL((decode_split_kernel<true, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((decode_split_kernel<true, false>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
  }
  const dim3 mgrid(a.num_kv_heads * kGroup, a.num_seqs);
  if (win) {
    hipLaunchKernelGGL((decode_split_kernel<false, true>), grid, dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL((decode_merge_kernel<true>), mgrid, dim3(kHeadDim), 0, st, a);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<false, false>), grid, dim3(kThreads), 0, st, a);
    hipLaunchKernelGGL((decode_merge_kernel<false>), mgrid, dim3(kHeadDim), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace flint
