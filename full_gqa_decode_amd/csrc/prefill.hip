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
// wave owns kTiles such tiles (kWaveRows consecutive rows); a workgroup of
// kPWaves waves owns kRows rows of one KV group.  The workgroup walks the key
// pages of its rows in pairs (32 keys): every thread fetches 16 bytes of K and
// 16 bytes of V of the pair two ahead while the waves compute on the current
// one, and each pair is staged once in LDS (double-buffered, one barrier per
// pair) for all waves -- HBM/L2 traffic per flop falls by the number of waves.
// Per pair and tile:
//   S^T[32 keys x 16 qv] = K . Q^T     2 x 4 v_mfma_f32_16x16x32_bf16
//   O[16 qv x 128]      += P . V        8 x 2 v_mfma_f32_16x16x32_bf16
// The PV contraction runs over 32 keys: MFMA k index gq*8+j takes key gq*4+j
// of the first page for j < 4 and key gq*4+j-4 of the second page for j >= 4,
// which is exactly where the score MFMAs left P; the LDS copy of V interleaves
// the two pages per dim row so that this operand is one 16-byte LDS read.  P
// is split into bf16(p) and its bf16 remainder (two MFMAs) so the value
// product is fp32-accurate.  Online softmax in log2 units with a lazy
// reference max (moved only when a probability would exceed 2^8), the sink joining
// the denominator in the epilogue.  An fp8 E4M3 cache is widened to bf16
// (exactly) as its pages are staged, with k_scale in the score scale and
// v_scale applied to the output.
// Bound: the matrix cores for full layers (4*D flops per (query, key) pair).
#include "device.h"
#include "launch.h"

namespace flint {

namespace {

constexpr int kTiles = 2;                    // 16-vector MFMA tiles per wave
constexpr int kWaveRows = kTiles * 2;        // query rows per wave
constexpr int kPWaves = 8;                   // waves per workgroup
constexpr int kPThreads = kPWaves * 64;
constexpr int kRows = kWaveRows * kPWaves;   // query rows per workgroup
// LDS copy of one page pair, unpadded, with 16-byte slots permuted so that
// every MFMA operand read is conflict-free.  gfx950's LDS serves a 16-byte
// read 32 lanes at a time from 128 four-byte banks, so the 32 slots those
// lanes read must fall in distinct 512-byte bank positions (measured: 4.8
// cycles per read per CU this way, 8.4 with rows padded to 272 or 80 bytes).
//   K: 32 key rows of 256 bytes (keys of page a, then page b); the chunk of
//      dims 8ch..8ch+7 of row r sits in slot ch ^ (r & 15).
//   V: 128 dim rows of 64 bytes; slot k holds keys 4k..4k+3 of page a, then
//      of page b (one MFMA operand), and sits at k ^ (2 * bit 3 of the dim).
constexpr int kKStride = kHeadDim * 2;
constexpr int kVStride = 2 * kPage * 2;
constexpr int kKBytes = 2 * kPage * kKStride;
constexpr int kBufBytes = kKBytes + kHeadDim * kVStride;
static_assert(kPThreads == 2 * 256, "staging: one K and one V 16-byte chunk per thread");

__device__ __forceinline__ int k_slot(int r, int ch) { return r * kKStride + ((ch ^ (r & 15)) << 4); }
__device__ __forceinline__ int v_slot(int d, int k) {
  return kKBytes + d * kVStride + ((k ^ (((d >> 3) & 1) << 1)) << 4);
}

struct PairRegs {
  bf16x8 ka[4], kb[4];  // K of the two pages (MFMA A operand)
  u32x4 v[8];           // V: keys gq*4..+3 of page a and of page b, one dim
};

// This thread's chunks of the pair (pga, pgb): K row c>>4, dims
// (c&15)*8 .. +7 and V dim c>>1, keys (c&1)*8 .. +7 of page sel.  bf16: one
// 16-byte load each.  fp8 (KV8): the same elements as codes, 8 bytes of K and
// two 4-byte runs of V in the fp8 tile order, held in the low dwords and
// widened to bf16 when staged.
template <bool KV8>
__device__ __forceinline__ void fetch_pair(const PrefillArgs& a, int pga, int pgb, int g, int tid,
                                           u32x4& kr, u32x4& vr) {
  const int sel = tid >> 8, c = tid & 255;
  const int64_t pg = sel ? pgb : pga;
  const int64_t tile = (pg * a.num_kv_heads + g) * (kPage * kHeadDim);
  if constexpr (KV8) {
    const uint8_t* kt = (const uint8_t*)a.k_cache + tile;
    const uint8_t* vt = (const uint8_t*)a.v_cache + tile;
    const u32x2 k8 = *(const u32x2*)(kt + fp8_k_off(c >> 4, (c & 15) * 8));
    const int d = c >> 1, key = (c & 1) * 8;
    kr = u32x4{k8[0], k8[1], 0u, 0u};
    vr = u32x4{*(const uint32_t*)(vt + fp8_v_off(key, d)),
               *(const uint32_t*)(vt + fp8_v_off(key + 4, d)), 0u, 0u};
  } else {
    const uint16_t* kt = (const uint16_t*)a.k_cache + tile;
    const uint16_t* vt = (const uint16_t*)a.v_cache + tile;
    kr = *(const u32x4*)(kt + bf16_k_off(c >> 4, (c & 15) * 8));
    vr = *(const u32x4*)(vt + (c >> 1) * kPage + (c & 1) * 8);
  }
}

template <bool KV8>
__device__ __forceinline__ void stage_pair(unsigned char* buf, int tid, u32x4 kr, u32x4 vr) {
  const int sel = tid >> 8, c = tid & 255;
  if constexpr (KV8) {  // codes -> bf16 (exact), same elements in the same order
    const u32x2 k0 = __builtin_bit_cast(u32x2, fp8x4_to_bf16x4(kr[0]));
    const u32x2 k1 = __builtin_bit_cast(u32x2, fp8x4_to_bf16x4(kr[1]));
    const u32x2 v0 = __builtin_bit_cast(u32x2, fp8x4_to_bf16x4(vr[0]));
    const u32x2 v1 = __builtin_bit_cast(u32x2, fp8x4_to_bf16x4(vr[1]));
    kr = u32x4{k0[0], k0[1], k1[0], k1[1]};
    vr = u32x4{v0[0], v0[1], v1[0], v1[1]};
  }
  *(u32x4*)(buf + k_slot(sel * kPage + (c >> 4), c & 15)) = kr;
  // V chunk: dim c>>1, keys h*8..h*8+7 = key groups 2h and 2h+1 of page sel
  const int d = c >> 1, h = c & 1;
  *(u32x2*)(buf + v_slot(d, 2 * h) + sel * 8) = u32x2{vr[0], vr[1]};
  *(u32x2*)(buf + v_slot(d, 2 * h + 1) + sel * 8) = u32x2{vr[2], vr[3]};
}

__device__ __forceinline__ void read_pair(const unsigned char* buf, int n, int gq, PairRegs& r) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    r.ka[c] = *(const bf16x8*)(buf + k_slot(n, 4 * c + gq));
    r.kb[c] = *(const bf16x8*)(buf + k_slot(kPage + n, 4 * c + gq));
  }
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
    r.v[nb] = *(const u32x4*)(buf + v_slot(nb * 16 + n, gq));
}

template <bool WINDOWED, bool KV8>
__global__ __launch_bounds__(kPThreads, 1) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char sm[2][kBufBytes];
  const int ntile = gridDim.x;
  const int tile = ntile - 1 - blockIdx.x;  // longest key ranges first
  const int g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, gq = lane >> 4;
  const int hkv = a.num_kv_heads, hq = hkv * kGroup;

  const int q0 = a.cu_q_lens[b];
  const int q_len = a.cu_q_lens[b + 1] - q0;
  const int seq_len = a.seq_lens[b];
  const int wg_row0 = tile * kRows;
  if (q_len <= 0 || wg_row0 >= q_len) return;  // no rows in this workgroup
  const bool req_bad = q_len > a.max_q_len || seq_len > a.max_seq_len || q_len > seq_len;
  const int base = seq_len - q_len;  // position of row 0

  // this wave's rows (possibly none: it still stages pages and meets barriers)
  const int row0 = wg_row0 + w * kWaveRows;
  const bool active = row0 < q_len;
  const int rows_here = active ? min(kWaveRows, q_len - row0) : 1;
  const int pos0 = base + row0;
  const int pos_last = pos0 + rows_here - 1;
  const int lo_first = WINDOWED ? max(0, pos0 - a.window + 1) : 0;
  const int lo_last = WINDOWED ? max(0, pos_last - a.window + 1) : 0;

  // the workgroup's page range: the union of its rows' key ranges
  const int wg_pos_last = base + min(wg_row0 + kRows, q_len) - 1;
  const int wg_lo = WINDOWED ? max(0, base + wg_row0 - a.window + 1) : 0;
  const int p_first = wg_lo / kPage, p_last = wg_pos_last / kPage;
  const int npairs = req_bad ? 0 : (p_last - p_first) / 2 + 1;

  // Q operands: tile mt, column n -> row row0 + 2*mt + (n>>3), head g*8 + (n&7)
  bf16x8 qop[kTiles][4];
  int qpos[kTiles];
#pragma unroll
  for (int mt = 0; mt < kTiles; ++mt) {
    const int r = min(row0 + 2 * mt + (n >> 3), q_len - 1);
    qpos[mt] = base + row0 + 2 * mt + (n >> 3);
    const uint16_t* qp = a.q + (((int64_t)(q0 + r) * hq) + g * kGroup + (n & 7)) * kHeadDim + gq * 8;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      qop[mt][c] = (req_bad || !active) ? bf16x8{} : *(const bf16x8*)(qp + c * 32);
  }

  // wait for the Q operands here, once: inside the loop the compiler cannot
  // tell them apart from the page loads in flight and would wait for all of
  // those before every pair's first MFMA
#pragma unroll
  for (int mt = 0; mt < kTiles; ++mt)
#pragma unroll
    for (int c = 0; c < 4; ++c) asm volatile("" ::"v"(qop[mt][c]));

  // m_run: the lazy reference max (log2 units).  It starts at the lowest
  // finite float rather than -inf, so that a row's first visible key always
  // moves it and a masked key (-inf) always gives exp2(-inf) = 0, never NaN.
  f32x4 acc[kTiles][8];
  float m_run[kTiles], l_part[kTiles];
#pragma unroll
  for (int mt = 0; mt < kTiles; ++mt) {
    m_run[mt] = -__FLT_MAX__;
    l_part[mt] = 0.f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[mt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int bad = req_bad;

  // Physical pages of pair j.  The page-table reads are vector loads, which
  // complete in issue order with the page loads, so each id is requested two
  // iterations before its pair's page loads need it: waiting for it then
  // never waits for a page load that is not already needed.  Loads are
  // unconditional (index clamped to the range) so no wait lands on a branch
  // join.  An id outside [0, num_blocks) marks the request bad and reads
  // page 0 instead; past the range end page b repeats page a.
  const int* bt_row = a.block_tables + (int64_t)b * a.bt_stride;
  auto load_ids = [&](int j, int& ia, int& ib) {
    const int p = min(p_first + 2 * j, p_last);
    ia = bt_row[p];
    ib = bt_row[min(p + 1, p_last)];
  };
  auto check_ids = [&](int j, int ia, int ib, int& pga, int& pgb) {
    const int p = p_first + 2 * j;
    pga = __builtin_amdgcn_readfirstlane(ia);
    pgb = p + 1 <= p_last ? __builtin_amdgcn_readfirstlane(ib) : pga;
    if (pga < 0 || pga >= a.num_blocks) { bad = 1; pga = 0; }
    if (pgb < 0 || pgb >= a.num_blocks) { bad = 1; pgb = 0; }
  };
  // page loads of pair j (ids ia, ib), if it exists
  auto fetch = [&](int j, int ia, int ib, u32x4& kr, u32x4& vr) {
    if (j < npairs) {
      int pga, pgb;
      check_ids(j, ia, ib, pga, pgb);
      fetch_pair<KV8>(a, pga, pgb, g, tid, kr, vr);
    }
  };

  auto compute = [&](int i) {
    const int p = p_first + 2 * i;
    const bool has_b = p + 1 <= p_last;
    const int key_lo = p * kPage, key_hi = p * kPage + 2 * kPage - 1;
    if (active && key_hi >= lo_first && key_lo <= pos_last) {
      PairRegs pr;
      read_pair(sm[i & 1], n, gq, pr);
      // keys of this pair that some row of the wave may not see
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

      // scores of every tile first, one branch for masking and one for the
      // (rare) rescale, then the value products: large basic blocks, so the
      // softmax arithmetic of one tile can overlap the other tile's MFMAs
      float sv[kTiles][8];
#pragma unroll
      for (int mt = 0; mt < kTiles; ++mt) {
        f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pr.ka[c], qop[mt][c], sa, 0, 0, 0);
          sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pr.kb[c], qop[mt][c], sb, 0, 0, 0);
        }
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
          sv[mt][i2] = sa[i2];
          sv[mt][4 + i2] = sb[i2];
        }
      }
      if (edge) {
#pragma unroll
        for (int mt = 0; mt < kTiles; ++mt) {
          const int qp = min(qpos[mt], pos_last);  // rows past the chunk end: any finite cut
          const int qlo = WINDOWED ? qp - a.window + 1 : 0;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int key = p * kPage + (j >= 4 ? kPage : 0) + gq * 4 + (j & 3);
            if (key < qlo || key > qp || (j >= 4 && !has_b)) sv[mt][j] = -INFINITY;
          }
        }
      }
      // exponent arguments x = s * qscale - m_run (log2 units).  Lazy
      // rescale: the reference max moves only when some x exceeds 8, so
      // p = 2^x < 2^8 and the accumulators are rescaled a few times per row
      // rather than every pair.  The exact row max is taken only then.
      float xv[kTiles][8];
      bool grow = false;
#pragma unroll
      for (int mt = 0; mt < kTiles; ++mt)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xv[mt][j] = fmaf(sv[mt][j], a.qscale, -m_run[mt]);
          grow |= xv[mt][j] > 8.f;
        }
      if (__any(grow)) {
#pragma unroll
        for (int mt = 0; mt < kTiles; ++mt) {
          float x = sv[mt][0];
#pragma unroll
          for (int j = 1; j < 8; ++j) x = fmaxf(x, sv[mt][j]);
          const float pmax = max_xor32(max_xor16(x)) * a.qscale;
          const float m_new = fmaxf(m_run[mt], pmax);
          // 0 for a row that had seen no key (its accumulators are zero)
          const float alpha = exp2_fast(m_run[mt] - m_new);
          l_part[mt] *= alpha;
          float al[4];
#pragma unroll
          for (int i2 = 0; i2 < 4; ++i2) al[i2] = __shfl(alpha, gq * 4 + i2);
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) acc[mt][nb][i2] *= al[i2];
          m_run[mt] = m_new;
#pragma unroll
          for (int j = 0; j < 8; ++j) xv[mt][j] = fmaf(sv[mt][j], a.qscale, -m_new);
        }
      }
#pragma unroll
      for (int mt = 0; mt < kTiles; ++mt) {
        float pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) pv[j] = exp2_fast(xv[mt][j]);
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
  };
  // In flight at the top of iteration i: pair i in LDS buffer i&1, the page
  // loads of pairs i+1 and i+2 in register sets (i+1)&1 and (i+2)&1, the ids
  // of pairs i+3 and i+4 in id sets (i+3)&1 and (i+4)&1 (loop unrolled by two
  // so every set is static).
  u32x4 kr0, vr0, kr1, vr1;
  int ia0, ib0, ia1, ib1, ia2, ib2;
  if (npairs > 0) {
    load_ids(0, ia0, ib0);
    load_ids(1, ia1, ib1);
    load_ids(2, ia2, ib2);
    fetch(0, ia0, ib0, kr0, vr0);
    stage_pair<KV8>(sm[0], tid, kr0, vr0);
    fetch(1, ia1, ib1, kr1, vr1);
    fetch(2, ia2, ib2, kr0, vr0);
    load_ids(3, ia1, ib1);
    load_ids(4, ia0, ib0);
  }
  __syncthreads();
  for (int i = 0; i < npairs; i += 2) {
    compute(i);
    if (i + 1 < npairs) stage_pair<KV8>(sm[1], tid, kr1, vr1);
    fetch(i + 3, ia1, ib1, kr1, vr1);
    load_ids(i + 5, ia1, ib1);
    __syncthreads();
    if (i + 1 >= npairs) break;
    compute(i + 1);
    if (i + 2 < npairs) stage_pair<KV8>(sm[0], tid, kr0, vr0);
    fetch(i + 4, ia0, ib0, kr0, vr0);
    load_ids(i + 6, ia0, ib0);
    __syncthreads();
  }
  if (!active) return;

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
      const float vs = KV8 ? a.v_scale : 1.f;
      float* dst = a.out + ((int64_t)(q0 + r) * hq + h) * kHeadDim + n;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        dst[nb * 16] = bad ? __builtin_nanf("") : acc[mt][nb][i] * so * inv * vs;
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.num_seqs == 0 || a.max_q_len == 0) return hipSuccess;
  const dim3 grid((a.max_q_len + kRows - 1) / kRows, a.num_kv_heads, a.num_seqs);
  if (a.kv_fp8) {
    if (a.window > 0)
      hipLaunchKernelGGL((prefill_kernel<true, true>), grid, dim3(kPThreads), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_kernel<false, true>), grid, dim3(kPThreads), 0, st, a);
  } else if (a.window > 0) {
    hipLaunchKernelGGL((prefill_kernel<true, false>), grid, dim3(kPThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((prefill_kernel<false, false>), grid, dim3(kPThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace flint
