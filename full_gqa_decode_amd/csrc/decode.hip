// decode.hip -- K2 split-K flash-decode (optionally fused with the append of
// the new token) and K3 log-sum-exp merge with sinks.
//
// What is computed ("Day-0 Support for Flint on vLLM", hnkhoi.com, "Model
// architecture": GQA with 32 query / 4 KV heads, learned attention sinks,
// per-head Q/K RMSNorm, RoPE on the sliding layers; newruntime.com, "What
// happened": 35 layers over a 513-token window, 14 over the full context,
// fused normalisation / rotary / cache operations):
//   out_h = sum_j e^{s_j} V_j / (e^{sink_h} + sum_j e^{s_j}),
//   s_j = scale * <q_h, K_j>, keys lo..t of the request.
//
// Design for gfx950.  One workgroup = WAVES wave64s on one (split, KV head,
// request); its waves take the split's 16-token pages round-robin.  The eight
// query heads of a KV group share every K and V row, so per page the work is
// two small dense contractions, done on the matrix cores:
//   scores  S[16 tok x 16]  = K_page[16 x 128] . Qhl^T[128 x 16]
//           (4 x v_mfma_f32_16x16x32_bf16; columns 0-7 carry bf16(q*c), columns
//           8-15 the bf16 remainder q*c - bf16(q*c) of the same heads, so the
//           sum of the two column halves is the fp32-accurate score)
//   values  O[16 x 128]    += Phl[16 x 16 tok] . V_page[16 tok x 128]
//           (8 x v_mfma_f32_16x16x16_bf16; rows 0-7 bf16(p), rows 8-15 the
//           bf16 remainder of p, summed at the end)
// K is stored in the order of the score MFMA's operands (bf16_k_off) and V
// dim-major, so lane l loads its operand straight from HBM: 16 contiguous
// bytes of K row l%16 and 8 contiguous bytes (4 tokens) of V dim-row per MFMA,
// with no LDS staging and no transposes.
// The score tile lands in exactly the lanes that need it as the P operand of
// the value MFMA, so the online softmax (DPP row_ror:8 for the hi+lo sum,
// wavefront shuffles for the page max) never moves P between lanes.
//
// Latency: page ids are fetched one page ahead of the K/V loads; in a split
// the next page's K is requested right after the score MFMAs consume this
// page's K, and its V right after the value MFMAs.  A short key range (the
// 513-key window) at small batch runs in decode_vsplit_kernel: 8 workgroups
// per (request, KV head), each reading every K page and a 16-dim slice of V,
// issuing every page load up front and folding the sink in directly, so no
// merge launch runs.  At larger batch one workgroup per (request, KV head)
// does the same over all 128 dims.
// Fused step: the workgroup normalises/rotates its own 8 query heads (one wave
// per head, into LDS) and the split holding the new token writes its K/V row
// into the cache and substitutes it in registers, so append and attention are
// one launch.  Bound: HBM (8 KiB of K+V per page and KV head against ~20 VALU
// and 12 MFMA instructions per wave).
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace flint {

namespace {

constexpr int kMergeThreads = 512;

// K and V tiles are read once per step, so their loads are nontemporal: on
// MI355X that streams a 204.8 MB layer ~9% faster than ordinary loads.
struct PageRegs {
  bf16x8 k[4];  // K rows: MFMA A operand, 32 dims each
  u32x2 v[8];   // V: 4 tokens x 1 dim per 16-dim block (MFMA B operand)
};

__device__ __forceinline__ void load_k(const DecodeArgs& a, int pg, int g, int n, int gq,
                                       PageRegs& r) {
  // the bf16 tile order (bf16_k_off): block c of row n is 16 bytes at
  // c * 1024 + lane * 16, so each load reads 1 KiB of contiguous bytes
  const uint16_t* kp = (const uint16_t*)a.k_cache +
                       ((int64_t)pg * a.num_kv_heads + g) * (kPage * kHeadDim) + (gq * 16 + n) * 8;
#pragma unroll
  for (int c = 0; c < 4; ++c) r.k[c] = __builtin_nontemporal_load((const bf16x8*)(kp + c * 512));
}

__device__ __forceinline__ void load_v(const DecodeArgs& a, int pg, int g, int n, int gq,
                                       PageRegs& r) {
  const uint16_t* vp =
      (const uint16_t*)a.v_cache + (((int64_t)pg * a.num_kv_heads + g) * kHeadDim + n) * kPage + gq * 4;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
    r.v[nb] = __builtin_nontemporal_load((const u32x2*)(vp + nb * 16 * kPage));
}

// fp8 cache, in its MFMA-native tile order (fp8_k_off / fp8_v_off): lane
// (n, gq) gets dims gq*32 .. gq*32+31 of K row n, and 4 tokens x 1 dim of V
// per 16-dim block (one dword each), from two 16-byte loads per tile, each
// load instruction reading 1 KiB of contiguous bytes.  The contraction's dim
// order is permuted to match: element j of MFMA block c is dim gq*32 + c*8 +
// j, and the q operand and the new token's K row follow it (kdim below).
struct PageRaw8 {
  u32x4 k[2];
  uint32_t v[8];
};

__device__ __forceinline__ void load_k(const DecodeArgs& a, int pg, int g, int n, int gq,
                                       PageRaw8& r) {
  const uint8_t* kp = (const uint8_t*)a.k_cache +
                      ((int64_t)pg * a.num_kv_heads + g) * (kPage * kHeadDim) + (gq * 16 + n) * 16;
  r.k[0] = __builtin_nontemporal_load((const u32x4*)kp);
  r.k[1] = __builtin_nontemporal_load((const u32x4*)(kp + 1024));
}

__device__ __forceinline__ void load_v(const DecodeArgs& a, int pg, int g, int n, int gq,
                                       PageRaw8& r) {
  const uint8_t* vp = (const uint8_t*)a.v_cache +
                      ((int64_t)pg * a.num_kv_heads + g) * (kPage * kHeadDim) + (gq * 16 + n) * 16;
  const u32x4 lo = __builtin_nontemporal_load((const u32x4*)vp);
  const u32x4 hi = __builtin_nontemporal_load((const u32x4*)(vp + 1024));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r.v[i] = lo[i];
    r.v[4 + i] = hi[i];
  }
}

// MFMA operands of a page: bf16 registers as loaded, or fp8 codes widened
// to bf16 (exact) right before their MFMA, so only the 4 KiB of raw codes
// stay live between pages.
__device__ __forceinline__ bf16x8 k_operand(const PageRegs& r, int c) { return r.k[c]; }
__device__ __forceinline__ bf16x8 k_operand(const PageRaw8& r, int c) {
  const bf16x4 x0 = fp8x4_to_bf16x4(r.k[c >> 1][(c & 1) * 2]);
  const bf16x4 x1 = fp8x4_to_bf16x4(r.k[c >> 1][(c & 1) * 2 + 1]);
  return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 v_operand(const PageRegs& r, int nb) {
  return __builtin_bit_cast(bf16x4, r.v[nb]);
}
__device__ __forceinline__ bf16x4 v_operand(const PageRaw8& r, int nb) {
  return fp8x4_to_bf16x4(r.v[nb]);
}

// Zero the V elements of tokens gq*4+i with keep[i] false.
__device__ __forceinline__ void mask_v(PageRegs& r, const bool (&keep)[4]) {
  const uint32_t mx = (keep[0] ? 0xffffu : 0u) | (keep[1] ? 0xffff0000u : 0u);
  const uint32_t my = (keep[2] ? 0xffffu : 0u) | (keep[3] ? 0xffff0000u : 0u);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) {
    r.v[nb][0] &= mx;
    r.v[nb][1] &= my;
  }
}
__device__ __forceinline__ void mask_v(PageRaw8& r, const bool (&keep)[4]) {
  const uint32_t m = (keep[0] ? 0xffu : 0u) | (keep[1] ? 0xff00u : 0u) |
                     (keep[2] ? 0xff0000u : 0u) | (keep[3] ? 0xff000000u : 0u);
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) r.v[nb] &= m;
}

// Dim held by element j of the q/K operand block c in lane group gq.
template <bool KV8>
__device__ __forceinline__ constexpr int kdim(int c, int gq, int j) {
  return KV8 ? gq * 32 + c * 8 + j : c * 32 + gq * 8 + j;
}

// Page id of logical page p of request b (wave-uniform scalar load), or -1
// when outside [0, num_blocks).
__device__ __forceinline__ int page_id(const DecodeArgs& a, int b, int p) {
  const int pg = a.block_tables[(int64_t)b * a.bt_stride + p];
  return (pg >= 0 && pg < a.num_blocks) ? pg : -1;
}

// Online-softmax state of one wave: PV accumulator (rows gq*4+i are the bf16
// parts (gq < 2) and remainders (gq >= 2) of heads, columns dims nb*16+n),
// running max of head n&7 (log2 units) and this lane's share of the sum.
struct WaveState {
  f32x4 acc[8];
  float m_run;
  float l_part;
};

// One page: scores, mask of the ragged ends, online softmax, value MFMAs.
// The K registers are dead after the score MFMAs and may be reloaded by the
// caller from that point (done through the `after_scores` callback).
template <typename Regs, typename AfterScores>
__device__ __forceinline__ void consume_page(Regs& r, const bf16x8 (&qop)[4], int p, int lo,
                                             int t, int n, int gq, WaveState& st,
                                             AfterScores after_scores) {
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(r, c), qop[c], sc, 0, 0, 0);
  after_scores();
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = sc[i] + lane_xor8(sc[i]);

  // ragged ends of the key range: mask scores, zero V so unwritten slots
  // (which may hold any bits) cannot reach the accumulator
  const int tok0 = p * kPage;
  if (tok0 < lo || tok0 + kPage - 1 > t) {
    bool keep[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tok0 + gq * 4 + i;
      keep[i] = tok >= lo && tok <= t;
      if (!keep[i]) sv[i] = -INFINITY;
    }
    mask_v(r, keep);
  }

  // online softmax in log2 units (q carries scale*log2(e))
  float pmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  pmax = max_xor32(max_xor16(pmax));
  const float m_new = fmaxf(st.m_run, pmax);
  if (__any(m_new > st.m_run)) {
    const float alpha = exp2_fast(st.m_run - m_new);
    st.l_part *= alpha;
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, (gq * 4 + i) & 7);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.acc[nb][i] *= al[i];
  }
  st.m_run = m_new;
  float pv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pv[i] = exp2_fast(sv[i] - m_new);
  st.l_part += (pv[0] + pv[1]) + (pv[2] + pv[3]);

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
    st.acc[nb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pop, v_operand(r, nb), st.acc[nb], 0,
                                                            0, 0);
}

// The new token's K row / V column, computed by this workgroup (as bf16
// bits of the cached values), replace what the page loads returned for row
// tr of the last page.
__device__ __forceinline__ void substitute_new_token(PageRegs& r, const uint16_t* knew,
                                                     const uint16_t* vnew, int tr, int n,
                                                     int gq) {
  if (n == tr) {
#pragma unroll
    for (int c = 0; c < 4; ++c) r.k[c] = *(const bf16x8*)(knew + kdim<false>(c, gq, 0));
  }
  if (gq == (tr >> 2)) {
    const int e = tr & 3;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const uint32_t bits = vnew[nb * 16 + n];
      uint32_t wv = r.v[nb][e >> 1];
      wv = (e & 1) ? ((wv & 0xffffu) | (bits << 16)) : ((wv & 0xffff0000u) | bits);
      r.v[nb][e >> 1] = wv;
    }
  }
}

// The same for an fp8 cache: knew / vnew hold the new token's fp8 codes.
__device__ __forceinline__ void substitute_new_token(PageRaw8& r, const uint8_t* knew,
                                                     const uint8_t* vnew, int tr, int n, int gq) {
  if (n == tr) {
    r.k[0] = *(const u32x4*)(knew + gq * 32);
    r.k[1] = *(const u32x4*)(knew + gq * 32 + 16);
  }
  if (gq == (tr >> 2)) {
    const int sh = (tr & 3) * 8;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      r.v[nb] = (r.v[nb] & ~(0xffu << sh)) | ((uint32_t)vnew[nb * 16 + n] << sh);
  }
}

// K2.  WAVES waves per workgroup.  MAXP > 1: the split has at most
// WAVES * MAXP pages and every wave issues all its page loads up front;
// MAXP == 1: the pipelined loop.  SINGLE: the split covers the whole key
// range, so the sink is folded in here and the output written directly.
// FUSED: also the norm/RoPE of q and the append of the new token.  KV8: the
// cache holds fp8 codes, widened to bf16 operand by operand (exact); k_scale
// rides in qscale and v_scale multiplies the result.  In the pipelined loop a
// wave keeps kAhead pages of loads in flight at one workgroup per CU, so that
// its compute between a page's arrival and the next request does not leave
// the load path idle.
//
// Start-up latency: the first loads (q, the first page ids and their K/V) are
// issued before seq_lens[b] has arrived, for the key range of a request of
// the host-side bound max_seq_len (the common batch-1 case); once seq_len is
// known they are kept if it equals that bound and reissued otherwise.  Every
// speculative page id is read inside the caller's block-table row and
// validated before it addresses the cache.
constexpr int kAhead = 2;
constexpr int kAhead8 = 2;  // the same for an fp8 cache
// MI355X's compute units: a grid of at most this many workgroups runs as one
// round at one workgroup per CU.
constexpr int kComputeUnits = 256;

// Launch bounds: MINW, the least waves per SIMD (fp8 kernels are held to 4,
// 128 VGPRs, so that two workgroups share a CU).  RING: pages in flight per
// wave in the pipelined loop.  A launch of at most one workgroup per CU whose
// waves walk at least 4 pages each takes MINW = 2 and RING = kAhead: the
// loads alone stream at ~6.4 TB/s in this shape, and one page per wave left
// the split kernel short of that, since the wave's math between a page's
// arrival and its next request leaves the load path idle.  Grids of several
// rounds keep RING = 1, whose smaller register file lets workgroups share a
// CU, and so do short splits, where a ring has nothing to fill.
template <int WAVES, int MAXP, bool SINGLE, bool WINDOWED, bool FUSED, bool KV8,
          int MINW = (MAXP > 1 ? 1 : (KV8 ? 4 : 2)), int RING = 1>
__global__ __launch_bounds__(WAVES * 64, MINW) void decode_split_kernel(DecodeArgs a) {
  constexpr int kThreads = WAVES * 64;
  // page buffers per wave
  constexpr int NR = MAXP > 1 ? MAXP : RING;
  using Raw = typename std::conditional<KV8, PageRaw8, PageRegs>::type;
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, gq = lane >> 4;
  const int hq = a.num_kv_heads * kGroup;

  __shared__ float sm_o[WAVES][kGroup][kHeadDim];
  __shared__ float sm_m[WAVES][kGroup];
  __shared__ float sm_l[WAVES][kGroup];
  __shared__ int sm_bad[WAVES];
  __shared__ float sm_q[FUSED ? kGroup : 1][kHeadDim];
  // the new token's K row / V column as cached (bf16 bits or fp8 codes)
  using Elem = typename std::conditional<KV8, uint8_t, uint16_t>::type;
  __shared__ __attribute__((aligned(16))) Elem sm_knew[FUSED ? kHeadDim : 16];
  __shared__ __attribute__((aligned(16))) Elem sm_vnew[FUSED ? kHeadDim : 16];
  __shared__ int sm_fused_bad;

  // ---- loads that do not wait for seq_len -------------------------------
  constexpr int QPW = (kGroup + WAVES - 1) / WAVES;  // fused: q heads per wave
  // fused: raw q of heads w, w+WAVES, ..., kept in fp32 until the norm
  // widens them, so that nothing waits for these loads before the page
  // loads below are issued.  With them, everything else the prologue reads:
  // the norm weights and, for the split that will hold the new token, its
  // raw K and V rows, its slot and the id of its page (for the speculated
  // length).  Requested before the pages, these never wait for a page.
  float x0[QPW], x1[QPW];
  float qw0 = 0.f, qw1 = 0.f, kw0 = 0.f, kw1 = 0.f, xk0 = 0.f, xk1 = 0.f, xv0 = 0.f, xv1 = 0.f;
  int slot_pre = 0, pg_last_pre = -1;
  f32x4 qraw[8];              // unfused: fp32 q of column n, dims c*32+gq*8..+7
  if (FUSED) {
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      // unconditional (a clamped head; only heads < kGroup are used): a load
      // under a branch would be waited for at the branch's join
      const int hh = min(w + j * WAVES, kGroup - 1);
      const float* x = a.q_in + ((int64_t)b * hq + g * kGroup + hh) * kHeadDim;
      x0[j] = x[lane];
      x1[j] = x[lane + 64];
    }
    qw0 = a.q_w[lane];
    qw1 = a.q_w[lane + 64];
    const float* xk = a.k_in + ((int64_t)b * a.num_kv_heads + g) * kHeadDim;
    const float* xv = a.v_in + ((int64_t)b * a.num_kv_heads + g) * kHeadDim;
    kw0 = a.k_w[lane];
    kw1 = a.k_w[lane + 64];
    xk0 = xk[lane];
    xk1 = xk[lane + 64];
    xv0 = xv[lane];
    xv1 = xv[lane + 64];
    slot_pre = a.slots[b];
    pg_last_pre = page_id(a, b, (a.max_seq_len - 1) / kPage);
  } else {
    const float* qh = a.q + ((int64_t)b * hq + g * kGroup + (n & 7)) * kHeadDim;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qraw[2 * c] = *(const f32x4*)(qh + kdim<KV8>(c, gq, 0));
      qraw[2 * c + 1] = *(const f32x4*)(qh + kdim<KV8>(c, gq, 4));
    }
  }
  // page range of this split for a request whose query sits at position tt
  auto range = [&](int tt, int& lo_, int& pb, int& pe) {
    lo_ = WINDOWED ? max(0, tt - a.window + 1) : 0;
    pb = lo_ / kPage + s * a.pages_per_split;
    pe = min(pb + a.pages_per_split, tt / kPage + 1);
  };
  int lo, p_begin, p_end;
  range(a.max_seq_len - 1, lo, p_begin, p_end);
  Raw r[NR];
  int bad = 0;
  auto issue = [&](int k) {  // page id and loads of this wave's k-th page
    const int p = p_begin + w + k * WAVES;
    if (p < p_end) {
      int pg = page_id(a, b, p);
      bad |= pg < 0;
      pg = max(pg, 0);
      load_k(a, pg, g, n, gq, r[k]);
      load_v(a, pg, g, n, gq, r[k]);
    }
  };
#pragma unroll
  for (int k = 0; k < NR; ++k) issue(k);
  // fused, rotating layers: this lane's RoPE angle for the speculated
  // position (fp64), computed while the loads above are in flight.  q_in was
  // requested before the pages, and loads complete in issue order, so
  // waiting for q later never waits for a page.
  double cs = 1.0, sn = 0.0;
  if (FUSED && a.use_rope) rope_cos_sin(a.max_seq_len - 1, lane, a.rope_theta, &cs, &sn);

  // ---- the request's real length ------------------------------------------
  const int seq_len = a.seq_lens[b];
  const bool len_bad = seq_len < 1 || seq_len > a.max_seq_len;
  const int t = seq_len - 1;
  if (!len_bad && seq_len != a.max_seq_len) {  // shorter request: redo the guesses
    range(t, lo, p_begin, p_end);
    bad = 0;
#pragma unroll
    for (int k = 0; k < NR; ++k) issue(k);
  }
  const int last_page = t / kPage;
  if (len_bad || p_begin > last_page) {
    // bad request: NaN output; empty split: lse -inf so the merge skips it
    const float fill = len_bad ? __builtin_nanf("") : -INFINITY;
    if (SINGLE) {
      for (int i = tid; i < kGroup * kHeadDim; i += kThreads)
        a.out[((int64_t)b * hq + g * kGroup + (i >> 7)) * kHeadDim + (i & 127)] = fill;
    } else if (tid < kGroup) {
      a.part_lse[((int64_t)b * a.num_splits + s) * hq + g * kGroup + tid] = fill;
    }
    return;
  }
  const bool has_new = FUSED && p_end == last_page + 1;  // this split holds token t

  // fused, fp8: the new token's K or V codes of this lane and where they go,
  // written after the page loop (below)
  uint8_t* st8_dst = nullptr;
  int st8_o0 = 0, st8_o1 = 0;
  uint32_t st8_c0 = 0, st8_c1 = 0;

  // ---- q operand ----------------------------------------------------------
  // column n holds head n&7; n < 8 the bf16 part of q*c, n >= 8 the bf16
  // remainder.  Lane group gq holds dims c*32 + gq*8 .. +7 of block c.
  bf16x8 qop[4];
  if (FUSED) {
    // wave w: q heads g*8 + w, w+WAVES, ...; has_new: wave 0 also the K row,
    // wave 1 the V row
    if (a.use_rope && t != a.max_seq_len - 1) rope_cos_sin(t, lane, a.rope_theta, &cs, &sn);
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      const int hh = w + j * WAVES;
      if (hh < kGroup) {
        double y0, y1;
        norm_rope_head(x0[j], x1[j], qw0, qw1, a.rms_eps, a.use_rope, cs, sn, &y0, &y1);
        sm_q[hh][lane] = (float)y0;
        sm_q[hh][lane + 64] = (float)y1;
        if (s == 0 && a.q_out) {
          float* qo = a.q_out + ((int64_t)b * hq + g * kGroup + hh) * kHeadDim;
          qo[lane] = (float)y0;
          qo[lane + 64] = (float)y1;
        }
      }
    }
    if (has_new && w < 2) {
      // the slot must be where the page table puts position t
      const int pg = t == a.max_seq_len - 1 ? pg_last_pre : page_id(a, b, last_page);
      const bool ok = pg >= 0 && slot_pre == pg * kPage + t % kPage;
      if (w == 0) {
        double y0, y1;
        norm_rope_head(xk0, xk1, kw0, kw1, a.rms_eps, a.use_rope, cs, sn, &y0, &y1);
        const int64_t o = ((int64_t)pg * a.num_kv_heads + g) * (kPage * kHeadDim);
        if (KV8) {
          const uint32_t c0 = fp8_e4m3_rne_f64(y0 / (double)a.k_scale);
          const uint32_t c1 = fp8_e4m3_rne_f64(y1 / (double)a.k_scale);
          sm_knew[lane] = (Elem)c0;
          sm_knew[lane + 64] = (Elem)c1;
          if (ok) {
            st8_dst = (uint8_t*)a.k_cache + o;
            st8_o0 = fp8_k_off(t % kPage, lane);
            st8_o1 = fp8_k_off(t % kPage, lane + 64);
            st8_c0 = c0;
            st8_c1 = c1;
          }
        } else {
          const uint16_t k0 = bf16_bits_rne_f64(y0), k1 = bf16_bits_rne_f64(y1);
          sm_knew[lane] = (Elem)k0;
          sm_knew[lane + 64] = (Elem)k1;
          if (ok) {
            uint16_t* dst = (uint16_t*)a.k_cache + o;
            dst[bf16_k_off(t % kPage, lane)] = k0;
            dst[bf16_k_off(t % kPage, lane + 64)] = k1;
          }
        }
        if (lane == 0) sm_fused_bad = !ok;
      } else {
        const int64_t o = ((int64_t)pg * a.num_kv_heads + g) * (kHeadDim * kPage) + t % kPage;
        if (KV8) {
          const uint32_t c0 = fp8_e4m3_rne_f64((double)xv0 / (double)a.v_scale);
          const uint32_t c1 = fp8_e4m3_rne_f64((double)xv1 / (double)a.v_scale);
          sm_vnew[lane] = (Elem)c0;
          sm_vnew[lane + 64] = (Elem)c1;
          if (ok) {
            st8_dst = (uint8_t*)a.v_cache + ((int64_t)pg * a.num_kv_heads + g) * (kHeadDim * kPage);
            st8_o0 = fp8_v_off(t % kPage, lane);
            st8_o1 = fp8_v_off(t % kPage, lane + 64);
            st8_c0 = c0;
            st8_c1 = c1;
          }
        } else {
          const uint16_t v0 = bf16_bits_rne(xv0), v1 = bf16_bits_rne(xv1);
          sm_vnew[lane] = (Elem)v0;
          sm_vnew[lane + 64] = (Elem)v1;
          if (ok) {
            uint16_t* dst = (uint16_t*)a.v_cache + o;
            dst[lane * kPage] = v0;
            dst[(lane + 64) * kPage] = v1;
          }
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float* qh = &sm_q[n & 7][kdim<KV8>(c, gq, 0)];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const f32x2 v = {qh[j] * a.qscale, qh[j + 1] * a.qscale};
        const bf16x2 hi = __builtin_convertvector(v, bf16x2);
        const bf16x2 lo2 = __builtin_convertvector(v - __builtin_convertvector(hi, f32x2), bf16x2);
        const bf16x2 sel = (n < 8) ? hi : lo2;
        qop[c][j] = sel[0];
        qop[c][j + 1] = sel[1];
      }
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 q0 = qraw[2 * c], q1 = qraw[2 * c + 1];
      const float xs[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
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

  // ---- pages ---------------------------------------------------------------
  WaveState st;
#pragma unroll
  for (int nb = 0; nb < 8; ++nb) st.acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_part = 0.f;
  const int tr = t % kPage;

  auto nothing = [] {};
  if (MAXP > 1) {
#pragma unroll
    for (int k = 0; k < NR; ++k) {
      const int p = p_begin + w + k * WAVES;
      if (p < p_end) {
        if (FUSED && p == last_page) substitute_new_token(r[k], sm_knew, sm_vnew, tr, n, gq);
        consume_page(r[k], qop, p, lo, t, n, gq, st, nothing);
      }
    }
  } else {
    // The pipelined loop.  A ring of NR page buffers per wave: buffer k is
    // consumed and refilled with the page NR rounds later, K as soon as the
    // score MFMAs have read it, V after the value MFMAs.
    // Raw page ids are read one more round ahead, at an index clamped into
    // the split, and checked when their loads are issued.
    //
    // Inside the main loop every load is unconditional: the pages that have
    // no page NR rounds later are peeled off into the tail below.  A load
    // under a branch would make the compiler's wait at the loop head count
    // the path that skipped it, and so wait for the current page's V before
    // its score MFMAs; the same holds for a page-id read that is checked
    // right away.
    const int64_t row = (int64_t)b * a.bt_stride;
    const int last_in_split = p_end - 1;
    int p = p_begin + w;
    const int n_mine = p < p_end ? (p_end - 1 - p) / WAVES + 1 : 0;
    int ids[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k)
      ids[k] = a.block_tables[row + min(p + (NR + k) * WAVES, last_in_split)];
    auto step = [&](int k, int pp, bool load_next) {
      const int raw = ids[k];
      const bool ok = raw >= 0 && raw < a.num_blocks;
      const int pg_next = ok ? raw : 0;
      if (load_next) {
        bad |= !ok;
        ids[k] = a.block_tables[row + min(pp + 2 * NR * WAVES, last_in_split)];
      }
      if (FUSED && pp == last_page) substitute_new_token(r[k], sm_knew, sm_vnew, tr, n, gq);
      consume_page(r[k], qop, pp, lo, t, n, gq, st, [&] {
        if (load_next) load_k(a, pg_next, g, n, gq, r[k]);
      });
      if (load_next) load_v(a, pg_next, g, n, gq, r[k]);
    };
    if constexpr (NR == 1) {
      for (int i = 1; i < n_mine; ++i, p += WAVES) step(0, p, true);
      if (n_mine > 0) step(0, p, false);
    } else {
      int i = 0;
      for (; i + 2 * NR <= n_mine; i += NR) {
#pragma unroll
        for (int k = 0; k < NR; ++k) step(k, p + k * WAVES, true);
        p += NR * WAVES;
      }
      // tail: the last n_mine - i (< 2 NR) pages
#pragma unroll
      for (int k = 0; k < NR; ++k)
        if (i + k < n_mine) step(k, p + k * WAVES, i + k + NR < n_mine);
#pragma unroll
      for (int k = 0; k < NR; ++k)
        if (i + NR + k < n_mine) step(k, p + (NR + k) * WAVES, false);
    }
  }

  // fused, fp8: the cache row of the new token, written only now.  A byte
  // store may alias any memory, so one issued before the loop would make the
  // compiler read the page table through vector loads, each waited for with
  // every page load in flight.  No workgroup reads this row from the cache
  // in this launch: the split that holds it substitutes it in registers.
  if (KV8 && FUSED && st8_dst) {
    st8_dst[st8_o0] = (uint8_t)st8_c0;
    st8_dst[st8_o1] = (uint8_t)st8_c1;
  }

  // ---- per-wave state -> LDS -> this split's result -----------------------
  // l: sum over the four lane groups of head n&7.  acc rows gq*4+i: gq 0,1 the
  // bf16 parts of heads 0-7, gq 2,3 the remainders.
  const float l_h = sum_xor32(sum_xor16(st.l_part));
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) st.acc[nb][i] = sum_xor32(st.acc[nb][i]);
  if (gq < 2) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[w][gq * 4 + i][nb * 16 + n] = st.acc[nb][i];
  }
  if (lane < kGroup) {
    sm_m[w][lane] = st.m_run;
    sm_l[w][lane] = l_h;
  }
  bad = __any(bad);
  if (lane == 0) sm_bad[w] = bad;
  __syncthreads();

  int any_bad = (FUSED && has_new) ? sm_fused_bad : 0;
#pragma unroll
  for (int v = 0; v < WAVES; ++v) any_bad |= sm_bad[v];

  for (int i = tid; i < kGroup * kHeadDim; i += kThreads) {
    const int h = i >> 7, d = i & 127;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) M = fmaxf(M, sm_m[v][h]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
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
      float res = o * scale_o / den;
      if (KV8) res *= a.v_scale;
      if (any_bad) res = __builtin_nanf("");
      a.out[((int64_t)b * hq + hg) * kHeadDim + d] = res;
    } else {
      const int64_t row = ((int64_t)b * a.num_splits + s) * hq + hg;
      a.part_o[row * kHeadDim + d] = KV8 ? o / L * a.v_scale : o / L;
      if (d == 0) a.part_lse[row] = any_bad ? __builtin_nanf("") : M + log2_fast(L);
    }
  }
}

// ---------------------------------------------------------------------------
// Short key ranges at small batch -- the 513-key window, or any range of at
// most kSinglePages pages -- in one launch with no merge.  kVSlices
// workgroups per (request, KV head); workgroup js owns output dims
// js*16 .. js*16+15 of the group's 8 query heads.  Each reads every K page of
// the range, so it forms the complete softmax of its heads (sink included)
// by itself, and only its 16-dim slice of V: one value MFMA per page instead
// of eight.  The kVSlices workgroups of one (request, KV head) are given
// workgroup ids that MI355X's round-robin dispatch sends to the same XCD
// (vsplit_item), so the repeated K reads are served from that XCD's L2 after
// the first.  Cutting the keys over workgroups instead needs a merge of their
// partials: a second launch or a hand-off through memory, each a further
// memory round trip on this latency-bound path.
static_assert(kVSlices * 16 == kHeadDim, "16-dim slices cover the head");

struct SliceRegs {
  bf16x8 k[4];  // K rows: MFMA A operand, 32 dims per block
  u32x2 v;      // V: 4 tokens of one dim of this workgroup's 16-dim slice
};
struct SliceRaw8 {
  u32x4 k[2];   // fp8 K codes, dims gq*32 .. gq*32+31 of row n
  uint32_t v;   // fp8 V codes: 4 tokens of one dim of the slice
};

// K of a page with ordinary loads (the other slices of this (request, KV
// head) read the same lines and should find them in L2); the V slice is read
// by this workgroup alone, so nontemporal.
__device__ __forceinline__ void load_slice(const DecodeArgs& a, int pg, int g, int n, int gq,
                                           int js, SliceRegs& r) {
  const int64_t tile = ((int64_t)pg * a.num_kv_heads + g) * (kPage * kHeadDim);
  const uint16_t* kp = (const uint16_t*)a.k_cache + tile + (gq * 16 + n) * 8;
#pragma unroll
  for (int c = 0; c < 4; ++c) r.k[c] = *(const bf16x8*)(kp + c * 512);
  const uint16_t* vp = (const uint16_t*)a.v_cache + tile + (js * 16 + n) * kPage + gq * 4;
  r.v = __builtin_nontemporal_load((const u32x2*)vp);
}

__device__ __forceinline__ void load_slice(const DecodeArgs& a, int pg, int g, int n, int gq,
                                           int js, SliceRaw8& r) {
  const int64_t tile = ((int64_t)pg * a.num_kv_heads + g) * (kPage * kHeadDim);
  const uint8_t* kp = (const uint8_t*)a.k_cache + tile + (gq * 16 + n) * 16;
  r.k[0] = *(const u32x4*)kp;
  r.k[1] = *(const u32x4*)(kp + 1024);
  // fp8_v_off(gq*4 + i, js*16 + n) for i = 0..3: one dword
  const uint8_t* vp =
      (const uint8_t*)a.v_cache + tile + (js >> 2) * 1024 + (gq * 16 + n) * 16 + (js & 3) * 4;
  r.v = __builtin_nontemporal_load((const uint32_t*)vp);
}

__device__ __forceinline__ bf16x8 k_operand(const SliceRegs& r, int c) { return r.k[c]; }
__device__ __forceinline__ bf16x8 k_operand(const SliceRaw8& r, int c) {
  const bf16x4 x0 = fp8x4_to_bf16x4(r.k[c >> 1][(c & 1) * 2]);
  const bf16x4 x1 = fp8x4_to_bf16x4(r.k[c >> 1][(c & 1) * 2 + 1]);
  return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x4 v_operand(const SliceRegs& r) {
  return __builtin_bit_cast(bf16x4, r.v);
}
__device__ __forceinline__ bf16x4 v_operand(const SliceRaw8& r) { return fp8x4_to_bf16x4(r.v); }

__device__ __forceinline__ void mask_v(SliceRegs& r, const bool (&keep)[4]) {
  r.v[0] &= (keep[0] ? 0xffffu : 0u) | (keep[1] ? 0xffff0000u : 0u);
  r.v[1] &= (keep[2] ? 0xffffu : 0u) | (keep[3] ? 0xffff0000u : 0u);
}
__device__ __forceinline__ void mask_v(SliceRaw8& r, const bool (&keep)[4]) {
  r.v &= (keep[0] ? 0xffu : 0u) | (keep[1] ? 0xff00u : 0u) | (keep[2] ? 0xff0000u : 0u) |
         (keep[3] ? 0xff000000u : 0u);
}

// The new token's K row (all dims) and this slice's 16 V values (bf16 bits
// or fp8 codes, as cached) replace what the loads returned for row tr.
__device__ __forceinline__ void substitute_new_token(SliceRegs& r, const uint16_t* knew,
                                                     const uint16_t* vslice, int tr, int n,
                                                     int gq) {
  if (n == tr) {
#pragma unroll
    for (int c = 0; c < 4; ++c) r.k[c] = *(const bf16x8*)(knew + kdim<false>(c, gq, 0));
  }
  if (gq == (tr >> 2)) {
    const int e = tr & 3;
    const uint32_t bits = vslice[n];
    uint32_t wv = r.v[e >> 1];
    wv = (e & 1) ? ((wv & 0xffffu) | (bits << 16)) : ((wv & 0xffff0000u) | bits);
    r.v[e >> 1] = wv;
  }
}
__device__ __forceinline__ void substitute_new_token(SliceRaw8& r, const uint8_t* knew,
                                                     const uint8_t* vslice, int tr, int n,
                                                     int gq) {
  if (n == tr) {
    r.k[0] = *(const u32x4*)(knew + gq * 32);
    r.k[1] = *(const u32x4*)(knew + gq * 32 + 16);
  }
  if (gq == (tr >> 2)) {
    const int sh = (tr & 3) * 8;
    r.v = (r.v & ~(0xffu << sh)) | ((uint32_t)vslice[n] << sh);
  }
}

// One page of a slice workgroup: the score MFMAs over the whole head, mask of
// the ragged ends, online softmax, one value MFMA for the 16-dim slice.
template <typename Regs>
__device__ __forceinline__ void consume_slice(Regs& r, const bf16x8 (&qop)[4], int p, int lo,
                                              int t, int n, int gq, f32x4& acc, float& m_run,
                                              float& l_part) {
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c)
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k_operand(r, c), qop[c], sc, 0, 0, 0);
  float sv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sv[i] = sc[i] + lane_xor8(sc[i]);
  const int tok0 = p * kPage;
  if (tok0 < lo || tok0 + kPage - 1 > t) {
    bool keep[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tok0 + gq * 4 + i;
      keep[i] = tok >= lo && tok <= t;
      if (!keep[i]) sv[i] = -INFINITY;
    }
    mask_v(r, keep);
  }
  float pmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  pmax = max_xor32(max_xor16(pmax));
  const float m_new = fmaxf(m_run, pmax);
  if (__any(m_new > m_run)) {
    const float alpha = exp2_fast(m_run - m_new);
    l_part *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= __shfl(alpha, (gq * 4 + i) & 7);
  }
  m_run = m_new;
  float pv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pv[i] = exp2_fast(sv[i] - m_new);
  l_part += (pv[0] + pv[1]) + (pv[2] + pv[3]);
  const f32x2 p01 = {pv[0], pv[1]}, p23 = {pv[2], pv[3]};
  const bf16x2 h01 = __builtin_convertvector(p01, bf16x2);
  const bf16x2 h23 = __builtin_convertvector(p23, bf16x2);
  const bf16x2 r01 = __builtin_convertvector(p01 - __builtin_convertvector(h01, f32x2), bf16x2);
  const bf16x2 r23 = __builtin_convertvector(p23 - __builtin_convertvector(h23, f32x2), bf16x2);
  const bf16x2 s01 = (n < 8) ? h01 : r01;
  const bf16x2 s23 = (n < 8) ? h23 : r23;
  const bf16x4 pop = {s01[0], s01[1], s23[0], s23[1]};
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pop, v_operand(r), acc, 0, 0, 0);
}

// An opaque zero that depends on three kernel arguments: adding it to the
// address of the first table read makes the compiler read those arguments
// before that load is issued, and not at their first use, where the wait for
// them would also wait for every table load issued in between.  (Not
// volatile: a volatile asm counts as a possible memory write and would turn
// the table reads after it into vector loads.)
__device__ __forceinline__ int zero_after(int x, float y, float z) {
  int r;
  asm("; zero_after %1 %2 %3" : "=s"(r) : "0"(0), "s"(x), "s"(y), "s"(z));
  return r;
}

// Work item of slice workgroup L of a grid of units * kVSlices, units =
// requests x KV heads.  Workgroups are dispatched to MI355X's 8 XCDs
// round-robin (L to XCD L % 8), so XCD x runs L = x, x+8, x+16, ...: giving
// it the items x*units .. x*units + units-1 of the unit-major order keeps the
// slices of a unit together on one XCD (or two, when units < 8).
__device__ __forceinline__ void vsplit_item(int L, int units, int& unit, int& js) {
  const int i = (L & 7) * units + (L >> 3);
  unit = i / kVSlices;
  js = i % kVSlices;
}

// WAVES waves; each takes the pages w, w+WAVES, ... of the range and issues
// all of its (at most MAXP) page loads up front.
//
// Start-up order.  Every scalar load is issued first (this wave's page ids
// for a request of the host-side bound max_seq_len, the request's length,
// the slot) together with the vector loads of the small inputs.  Everything
// that consumes those inputs -- the fp64 RoPE angle of the real position, the
// norm of the wave's q head or of the new K row, the new V row, the q operand
// -- runs before the wave issues its page loads: a wait for an input issued
// before a variable number of page loads (pages are issued under per-page
// conditions) would be compiled as a wait for every load, pages included.
// Waves with no start-up work (kKw+2 and up) issue their pages at once.
// Phase stamps of the slice kernel (the instrumented build only,
// -DFLINT_STAMPS, which bench.py --stamps loads): per workgroup and wave,
// s_memrealtime at entry (0), once the scalar inputs are in (1), before the
// page loads are issued (2), after the pages are consumed (3) and after the
// output is written (4); slot 6 holds the CU (__smid).  The product build
// compiles every stamp to nothing.
#ifdef FLINT_STAMPS
constexpr int kStampWorkgroups = 1024;
__device__ unsigned long long g_slice_stamps[kStampWorkgroups * 16 * 8];
#define SL_STAMP(k)                                                                       \
  do {                                                                                    \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    const unsigned long long t_ = __builtin_amdgcn_s_memrealtime();                       \
    if (lane == 0 && blockIdx.x < kStampWorkgroups && w < 16)                             \
      g_slice_stamps[(blockIdx.x * 16 + w) * 8 + (k)] = t_;                               \
    __builtin_amdgcn_sched_barrier(0);                                                    \
  } while (0)
#define SL_STAMP_VALUE(k, v)                                                              \
  do {                                                                                    \
    if (lane == 0 && blockIdx.x < kStampWorkgroups && w < 16)                             \
      g_slice_stamps[(blockIdx.x * 16 + w) * 8 + (k)] = (v);                              \
  } while (0)
#else
#define SL_STAMP(k) \
  do {              \
  } while (0)
#define SL_STAMP_VALUE(k, v) \
  do {                       \
  } while (0)
#endif

template <int WAVES, int MAXP, bool WINDOWED, bool FUSED, bool KV8>
__global__ __launch_bounds__(WAVES * 64, 1) void decode_vsplit_kernel(DecodeArgs a) {
  static_assert(WAVES >= kGroup, "one wave per query head of the group");
  using Raw = typename std::conditional<KV8, SliceRaw8, SliceRegs>::type;
  using Elem = typename std::conditional<KV8, uint8_t, uint16_t>::type;
  int unit, js;
  vsplit_item(blockIdx.x, a.num_seqs * a.num_kv_heads, unit, js);
  const int b = unit / a.num_kv_heads, g = unit % a.num_kv_heads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, gq = lane >> 4;
  const int hq = a.num_kv_heads * kGroup;
  SL_STAMP(0);
  SL_STAMP_VALUE(6, __smid());
  // fused: the new K row is normalised by wave kKw, the V row by wave kVw
  constexpr int kKw = WAVES > kGroup ? kGroup : 0;
  constexpr int kVw = WAVES > kGroup + 1 ? kGroup + 1 : 1;
  // waves that rotate: the q heads and the K row
  constexpr int kRotWaves = kKw + 1 > kGroup ? kKw + 1 : kGroup;

  __shared__ float sm_o[WAVES][kGroup][16];
  __shared__ float sm_m[WAVES][kGroup];
  __shared__ float sm_l[WAVES][kGroup];
  __shared__ int sm_bad[WAVES];
  __shared__ float sm_q[FUSED ? kGroup : 1][kHeadDim];
  __shared__ __attribute__((aligned(16))) Elem sm_knew[FUSED ? kHeadDim : 16];
  __shared__ __attribute__((aligned(16))) Elem sm_vnew[16];
  __shared__ int sm_fused_bad;

  const int use_rope = a.use_rope;
  const float theta = a.rope_theta;
  const float eps = a.rms_eps;
  // ---- scalar loads: page ids, the length, the slot ----------------------
  auto range = [&](int tt, int& lo_, int& pb, int& pe) {
    lo_ = WINDOWED ? max(0, tt - a.window + 1) : 0;
    pb = lo_ / kPage;
    pe = tt / kPage + 1;
  };
  int lo, p_begin, p_end;
  range(a.max_seq_len - 1, lo, p_begin, p_end);
  const int* bt_row =
      a.block_tables + (int64_t)b * a.bt_stride + zero_after(use_rope, theta, eps);
  int ids[MAXP];
  auto read_ids = [&] {  // unconditional reads, clamped into the range
#pragma unroll
    for (int k = 0; k < MAXP; ++k) ids[k] = bt_row[min(p_begin + w + k * WAVES, p_end - 1)];
  };
  read_ids();
  const int seq_len = a.seq_lens[b];
  int slot = 0, pg_last_raw = -1;
  if (FUSED) {
    slot = a.slots[b];
    pg_last_raw = bt_row[(a.max_seq_len - 1) / kPage];
  }
  // ---- vector loads of the small inputs (unconditional, clamped head) -----
  float x0 = 0.f, x1 = 0.f, qw0 = 0.f, qw1 = 0.f;
  float xk0 = 0.f, xk1 = 0.f, kw0 = 0.f, kw1 = 0.f, xv0 = 0.f, xv1 = 0.f;
  f32x4 qraw[8];
  if (FUSED) {
    const int hh = min(w, kGroup - 1);
    const float* x = a.q_in + ((int64_t)b * hq + g * kGroup + hh) * kHeadDim;
    x0 = x[lane];
    x1 = x[lane + 64];
    qw0 = a.q_w[lane];
    qw1 = a.q_w[lane + 64];
    const float* xk = a.k_in + ((int64_t)b * a.num_kv_heads + g) * kHeadDim;
    const float* xv = a.v_in + ((int64_t)b * a.num_kv_heads + g) * kHeadDim;
    xk0 = xk[lane];
    xk1 = xk[lane + 64];
    kw0 = a.k_w[lane];
    kw1 = a.k_w[lane + 64];
    xv0 = xv[lane];
    xv1 = xv[lane + 64];
  } else {
    const float* qh = a.q + ((int64_t)b * hq + g * kGroup + (n & 7)) * kHeadDim;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      qraw[2 * c] = *(const f32x4*)(qh + kdim<KV8>(c, gq, 0));
      qraw[2 * c + 1] = *(const f32x4*)(qh + kdim<KV8>(c, gq, 4));
    }
  }

  // fused, rotating layers: the angle of the speculated position, while the
  // loads above are in flight (waves that rotate: the q heads and the K row)
  double cs = 1.0, sn = 0.0;
  __builtin_amdgcn_sched_barrier(0);
  if (FUSED && use_rope && w < kRotWaves) rope_cos_sin(a.max_seq_len - 1, lane, theta, &cs, &sn);
  __builtin_amdgcn_sched_barrier(0);
  // one wait for every scalar value, before any branch on them (loads only
  // one side of a branch needs would otherwise be moved past it and issued
  // one round trip later)
  asm volatile("" ::"s"(seq_len), "s"(slot), "s"(pg_last_raw));
#pragma unroll
  for (int k = 0; k < MAXP; ++k) asm volatile("" ::"s"(ids[k]));
  SL_STAMP(1);

  // ---- the request's length ------------------------------------------------
  // A length outside [1, max_seq_len] runs the speculated range and writes
  // NaN outputs and no cache row (no early exit: see above).
  const bool len_bad = seq_len < 1 || seq_len > a.max_seq_len;
  const int t = len_bad ? a.max_seq_len - 1 : seq_len - 1;
  if (t != a.max_seq_len - 1) {  // shorter request: the real pages and angle
    range(t, lo, p_begin, p_end);
    read_ids();
    if (FUSED) pg_last_raw = bt_row[t / kPage];
    if (FUSED && use_rope && w < kRotWaves) rope_cos_sin(t, lane, theta, &cs, &sn);
  }
  const int last_page = t / kPage;
  const int tr = t % kPage;

  // ---- start-up work: q operand and, fused, the new token ------------------
  bf16x8 qop[4];
  if (FUSED) {
    const int pg = (pg_last_raw >= 0 && pg_last_raw < a.num_blocks) ? pg_last_raw : -1;
    // the slot must be where the page table puts position t; only slice 0
    // writes the cache, every slice substitutes the new row in registers
    const bool ok = pg >= 0 && slot == pg * kPage + tr && !len_bad;
    const bool write = ok && js == 0;
    if (w < kRotWaves) {
      if (w < kGroup) {
        double y0, y1;
        norm_rope_head(x0, x1, qw0, qw1, eps, use_rope, cs, sn, &y0, &y1);
        sm_q[w][lane] = (float)y0;
        sm_q[w][lane + 64] = (float)y1;
        if (js == 0 && a.q_out) {
          float* qo = a.q_out + ((int64_t)b * hq + g * kGroup + w) * kHeadDim;
          qo[lane] = (float)y0;
          qo[lane + 64] = (float)y1;
        }
      }
      if (w == kKw) {
        double y0, y1;
        norm_rope_head(xk0, xk1, kw0, kw1, eps, use_rope, cs, sn, &y0, &y1);
        const int64_t o = ((int64_t)max(pg, 0) * a.num_kv_heads + g) * (kPage * kHeadDim);
        if (KV8) {
          const uint32_t c0 = fp8_e4m3_rne_f64(y0 / (double)a.k_scale);
          const uint32_t c1 = fp8_e4m3_rne_f64(y1 / (double)a.k_scale);
          sm_knew[lane] = (Elem)c0;
          sm_knew[lane + 64] = (Elem)c1;
          if (write) {
            uint8_t* dst = (uint8_t*)a.k_cache + o;
            dst[fp8_k_off(tr, lane)] = (uint8_t)c0;
            dst[fp8_k_off(tr, lane + 64)] = (uint8_t)c1;
          }
        } else {
          const uint16_t k0 = bf16_bits_rne_f64(y0), k1 = bf16_bits_rne_f64(y1);
          sm_knew[lane] = (Elem)k0;
          sm_knew[lane + 64] = (Elem)k1;
          if (write) {
            uint16_t* dst = (uint16_t*)a.k_cache + o;
            dst[bf16_k_off(tr, lane)] = k0;
            dst[bf16_k_off(tr, lane + 64)] = k1;
          }
        }
        if (lane == 0) sm_fused_bad = !ok;
      }
    }
    if (w == kVw) {
      const int64_t o = ((int64_t)max(pg, 0) * a.num_kv_heads + g) * (kHeadDim * kPage);
      uint32_t c0, c1;
      if (KV8) {
        c0 = fp8_e4m3_rne_f64((double)xv0 / (double)a.v_scale);
        c1 = fp8_e4m3_rne_f64((double)xv1 / (double)a.v_scale);
        if (write) {
          uint8_t* dst = (uint8_t*)a.v_cache + o;
          dst[fp8_v_off(tr, lane)] = (uint8_t)c0;
          dst[fp8_v_off(tr, lane + 64)] = (uint8_t)c1;
        }
      } else {
        c0 = bf16_bits_rne(xv0);
        c1 = bf16_bits_rne(xv1);
        if (write) {
          uint16_t* dst = (uint16_t*)a.v_cache + o + tr;
          dst[lane * kPage] = (uint16_t)c0;
          dst[(lane + 64) * kPage] = (uint16_t)c1;
        }
      }
      // this slice's dims js*16 .. js*16+15 sit in lanes (js&3)*16 .. +15 of
      // the half (js >> 2)
      const int d = lane - (js & 3) * 16;
      if (d >= 0 && d < 16) sm_vnew[d] = (Elem)((js >> 2) ? c1 : c0);
    }
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 q0 = qraw[2 * c], q1 = qraw[2 * c + 1];
      const float xs[8] = {q0[0], q0[1], q0[2], q0[3], q1[0], q1[1], q1[2], q1[3]};
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

  // ---- page loads ------------------------------------------------------------
  SL_STAMP(2);
  Raw r[MAXP];
  int bad = len_bad;
#pragma unroll
  for (int k = 0; k < MAXP; ++k) {
    if (p_begin + w + k * WAVES < p_end) {
      const bool ok = ids[k] >= 0 && ids[k] < a.num_blocks;
      bad |= !ok;
      load_slice(a, ok ? ids[k] : 0, g, n, gq, js, r[k]);
    }
  }
  if (FUSED) {
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float* qh = &sm_q[n & 7][kdim<KV8>(c, gq, 0)];
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const f32x2 v = {qh[j] * a.qscale, qh[j + 1] * a.qscale};
        const bf16x2 hi = __builtin_convertvector(v, bf16x2);
        const bf16x2 lo2 = __builtin_convertvector(v - __builtin_convertvector(hi, f32x2), bf16x2);
        const bf16x2 sel = (n < 8) ? hi : lo2;
        qop[c][j] = sel[0];
        qop[c][j + 1] = sel[1];
      }
    }
  }

  // ---- pages ---------------------------------------------------------------
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
#pragma unroll
  for (int k = 0; k < MAXP; ++k) {
    const int p = p_begin + w + k * WAVES;
    if (p < p_end) {
      if (FUSED && p == last_page) substitute_new_token(r[k], sm_knew, sm_vnew, tr, n, gq);
      consume_slice(r[k], qop, p, lo, t, n, gq, acc, m_run, l_part);
    }
  }

  SL_STAMP(3);
  // ---- waves -> LDS -> this slice of the output ----------------------------
  const float l_h = sum_xor32(sum_xor16(l_part));
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = sum_xor32(acc[i]);
  if (gq < 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sm_o[w][gq * 4 + i][n] = acc[i];
  }
  if (lane < kGroup) {
    sm_m[w][lane] = m_run;
    sm_l[w][lane] = l_h;
  }
  bad = __any(bad);
  if (lane == 0) sm_bad[w] = bad;
  __syncthreads();
  if (tid < kGroup * 16) {
    int any_bad = FUSED ? sm_fused_bad : 0;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) any_bad |= sm_bad[v];
    const int h = tid >> 4, d = tid & 15;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) M = fmaxf(M, sm_m[v][h]);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
      const float e = exp2_fast(sm_m[v][h] - M);
      L += e * sm_l[v][h];
      o += e * sm_o[v][h][d];
    }
    const int hg = g * kGroup + h;
    const float sink = a.sinks[hg] * kLog2e;
    const float M2 = fmaxf(M, sink);
    const float scale_o = exp2_fast(M - M2);
    const float den = exp2_fast(sink - M2) + L * scale_o;
    float res = o * scale_o / den;
    if (KV8) res *= a.v_scale;
    if (any_bad) res = __builtin_nanf("");
    a.out[((int64_t)b * hq + hg) * kHeadDim + js * 16 + d] = res;
  }
  SL_STAMP(4);
}

// K3: out_h = sum_s w_s o_s / (e^{sink_h} + sum_s w_s), w_s = 2^{lse_s - M},
// in log2 units.  Every split of the grid left an lse (-inf when it held no
// key, NaN for a bad request or page), so no load here waits on seq_lens.
// One workgroup per (query head, request, quarter of the dims): 512 threads =
// 16 split groups x 32 dims, each group summing every 16th split, the first
// kMergeChunk of them loaded into registers before the block-wide max is
// known -- one memory round trip for plans of up to 256 splits.
constexpr int kMergeDims = 32;
constexpr int kMergeGroups = kMergeThreads / kMergeDims;
constexpr int kMergeChunk = 16;

__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int d = blockIdx.z * kMergeDims + (tid % kMergeDims), grp = tid / kMergeDims;
  const int hq = a.num_kv_heads * kGroup;
  const int ns = a.num_splits;
  __shared__ float red_m[kMergeThreads / 64];
  __shared__ int red_nan[kMergeThreads / 64];
  __shared__ float red_o[kMergeGroups][kMergeDims];
  __shared__ float red_den[kMergeGroups];

  const int64_t base = (int64_t)b * ns * hq + h;
  float lv[kMergeChunk], ov[kMergeChunk];
#pragma unroll
  for (int j = 0; j < kMergeChunk; ++j) {
    const int sp = grp + j * kMergeGroups;
    const int64_t row = base + (int64_t)min(sp, ns - 1) * hq;
    lv[j] = a.part_lse[row];
    ov[j] = a.part_o[row * kHeadDim + d];
    if (sp >= ns) lv[j] = -INFINITY;
  }
  const float sink = a.sinks[h] * kLog2e;
  float m = sink;
  int nan = 0;
#pragma unroll
  for (int j = 0; j < kMergeChunk; ++j) {
    nan |= lv[j] != lv[j];
    m = fmaxf(m, lv[j]);
  }
  for (int sp = grp + kMergeChunk * kMergeGroups; sp < ns; sp += kMergeGroups) {
    const float l = a.part_lse[base + (int64_t)sp * hq];
    nan |= l != l;
    m = fmaxf(m, l);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  nan = __any(nan);
  if ((tid & 63) == 0) {
    red_m[tid >> 6] = m;
    red_nan[tid >> 6] = nan;
  }
  __syncthreads();
  float M = red_m[0];
  nan = red_nan[0];
#pragma unroll
  for (int v = 1; v < kMergeThreads / 64; ++v) {
    M = fmaxf(M, red_m[v]);
    nan |= red_nan[v];
  }

  // an empty split (lse -inf, output never written) contributes 0
  float o = 0.f, den = 0.f;
#pragma unroll
  for (int j = 0; j < kMergeChunk; ++j) {
    const bool live = lv[j] > -INFINITY;
    const float wgt = live ? exp2_fast(lv[j] - M) : 0.f;
    den += wgt;
    o += live ? wgt * ov[j] : 0.f;
  }
#pragma unroll 8
  for (int sp = grp + kMergeChunk * kMergeGroups; sp < ns; sp += kMergeGroups) {
    const int64_t row = base + (int64_t)sp * hq;
    const float l = a.part_lse[row];
    const float x = a.part_o[row * kHeadDim + d];
    const bool live = l > -INFINITY;
    const float wgt = live ? exp2_fast(l - M) : 0.f;
    den += wgt;
    o += live ? wgt * x : 0.f;
  }
  red_o[grp][tid % kMergeDims] = o;
  if (tid % kMergeDims == 0) red_den[grp] = den;
  __syncthreads();
  if (grp == 0) {
    float os = 0.f, ds = exp2_fast(sink - M);
#pragma unroll
    for (int v = 0; v < kMergeGroups; ++v) {
      os += red_o[v][tid];
      ds += red_den[v];
    }
    a.out[((int64_t)b * hq + h) * kHeadDim + d] = nan ? __builtin_nanf("") : os / ds;
  }
}

// K3 for plans of at most kSmallMergeSplits splits (a batch of requests cut
// into a few splits each): one thread per output element, all of its
// partials loaded in one round trip.  The wide kernel above would leave most
// of its split groups idle and launch a workgroup per (head, request, quarter).
constexpr int kSmallMergeSplits = 8;
constexpr int kSmallMergeThreads = 256;

__global__ __launch_bounds__(kSmallMergeThreads) void decode_merge_small_kernel(DecodeArgs a) {
  const int hq = a.num_kv_heads * kGroup;
  const int ns = a.num_splits;
  const int64_t idx = (int64_t)blockIdx.x * kSmallMergeThreads + threadIdx.x;
  if (idx >= (int64_t)a.num_seqs * hq * kHeadDim) return;
  const int d = (int)(idx & (kHeadDim - 1));
  const int64_t bh = idx >> 7;
  const int h = (int)(bh % hq);
  const int64_t b = bh / hq;
  const int64_t base = b * ns * hq + h;
  float lv[kSmallMergeSplits], ov[kSmallMergeSplits];
#pragma unroll
  for (int s = 0; s < kSmallMergeSplits; ++s) {
    const int64_t row = base + (int64_t)min(s, ns - 1) * hq;
    lv[s] = a.part_lse[row];
    ov[s] = a.part_o[row * kHeadDim + d];
    if (s >= ns) lv[s] = -INFINITY;
  }
  const float sink = a.sinks[h] * kLog2e;
  float M = sink;
  int nan = 0;
#pragma unroll
  for (int s = 0; s < kSmallMergeSplits; ++s) {
    nan |= lv[s] != lv[s];
    M = fmaxf(M, lv[s]);
  }
  float o = 0.f, den = exp2_fast(sink - M);
#pragma unroll
  for (int s = 0; s < kSmallMergeSplits; ++s) {
    const bool live = lv[s] > -INFINITY;
    const float w = live ? exp2_fast(lv[s] - M) : 0.f;
    den += w;
    o += live ? w * ov[s] : 0.f;
  }
  a.out[bh * kHeadDim + d] = nan ? __builtin_nanf("") : o / den;
}

// K3 for plans of kSmallMergeSplits+1 .. kMidMergeSplits splits (batch 1:
// the 100K full layer's 64 splits).
constexpr int kMidMergeSplits = 64;

// K3 for plans of kSmallMergeSplits+1 .. kMidMergeSplits splits, spread
// over (request, query head, 16-dim slice): one wave each, so that a batch-1
// layer's 1 MB of partials is read by 256 workgroups at 4 KiB apiece rather
// than by 32 at 32 KiB.  Lane l holds split l's lse and its 16 values of the
// slice (four 16-byte loads), all requested before any is used; the max and
// the weights come from wave reductions, and the 16 output dims from one
// reduce-scatter over the lanes.
__global__ __launch_bounds__(64) void decode_merge_slice_kernel(DecodeArgs a) {
  const int hq = a.num_kv_heads * kGroup;
  const int ns = a.num_splits;
  const int js = blockIdx.x % kVSlices;
  const int bh = blockIdx.x / kVSlices;  // b * hq + h
  const int h = bh % hq, b = bh / hq;
  const int l = threadIdx.x;
  const int64_t row = (int64_t)b * ns * hq + h + (int64_t)min(l, ns - 1) * hq;
  // lanes past the last split re-read it (no branch between the loads);
  // their weights are 0
  float lse = a.part_lse[row];
  const float* po = a.part_o + row * kHeadDim + js * 16;
  f32x4 ov[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ov[i] = *(const f32x4*)(po + 4 * i);
  __builtin_amdgcn_sched_barrier(0);  // keep every load ahead of the reductions
  if (l >= ns) lse = -INFINITY;
  const bool nan = __any(lse != lse);
  const float sink = a.sinks[h] * kLog2e;
  const float M = fmaxf(sink, wave_max_f32(lse));
  // an empty split (lse -inf, output never written) contributes 0
  const float w = lse > -INFINITY ? exp2_fast(lse - M) : 0.f;
  const float inv = 1.f / (exp2_fast(sink - M) + wave_sum_f32(w));
  // The 16 sums over the 64 lanes, reduced and scattered at once: one
  // lane-32 exchange of the pair (x[i], x[i+8]) leaves lanes 0-31 the sums
  // of dims i and lanes 32-63 those of dims i+8 over their lane pair (8
  // exchanges for 16 dims); one lane-16 exchange of (y[i], y[i+4]) halves
  // them again; a row reduction finishes the 4 dims each row of 16 lanes
  // holds: dims 8h + 4p .. +3, h = l >> 5, p = (l >> 4) & 1.
  float x[16];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) x[4 * i + j] = w > 0.f ? w * ov[i][j] : 0.f;
  float y[8], z[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x[i]),
                                                    __builtin_bit_cast(unsigned, x[i + 8]),
                                                    false, false);
    const unsigned r0 = r[0], r1 = r[1];
    y[i] = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, y[i]),
                                                    __builtin_bit_cast(unsigned, y[i + 4]),
                                                    false, false);
    const unsigned r0 = r[0], r1 = r[1];
    float t = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
    t += row_ror<8>(t);
    t += row_ror<4>(t);
    t += row_ror<2>(t);
    t += row_ror<1>(t);
    z[i] = nan ? __builtin_nanf("") : t * inv;
  }
  if ((l & 15) == 0)
    *(f32x4*)(a.out + (int64_t)bh * kHeadDim + js * 16 + 8 * (l >> 5) + 4 * ((l >> 4) & 1)) =
        f32x4{z[0], z[1], z[2], z[3]};
}

hipError_t launch_merge_k(const DecodeArgs& a, hipStream_t st) {
  const bool al16 = ((uintptr_t)a.part_o % 16 == 0) && ((uintptr_t)a.out % 16 == 0);
  if (a.num_splits <= kSmallMergeSplits) {
    const int64_t n = (int64_t)a.num_seqs * a.num_kv_heads * kGroup * kHeadDim;
    const dim3 grid((unsigned)((n + kSmallMergeThreads - 1) / kSmallMergeThreads));
    hipLaunchKernelGGL(decode_merge_small_kernel, grid, dim3(kSmallMergeThreads), 0, st, a);
  } else if (a.num_splits <= kMidMergeSplits && al16) {
    const dim3 grid((unsigned)(a.num_seqs * a.num_kv_heads * kGroup * kVSlices));
    hipLaunchKernelGGL(decode_merge_slice_kernel, grid, dim3(64), 0, st, a);
  } else {
    const dim3 mgrid(a.num_kv_heads * kGroup, a.num_seqs, kHeadDim / kMergeDims);
    hipLaunchKernelGGL(decode_merge_kernel, mgrid, dim3(kMergeThreads), 0, st, a);
  }
  return hipGetLastError();
}

template <bool FUSED, bool KV8>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.num_splits, a.num_kv_heads, a.num_seqs);
  const bool win = a.window > 0;
  // one round of workgroups, each wave with at least 4 pages: the page ring
  const bool one_round = (int64_t)grid.x * grid.y * grid.z <= kComputeUnits &&
                         a.pages_per_split >= 4 * kDecodeWaves;
  constexpr int RG = KV8 ? kAhead8 : kAhead;  // page ring of one-round launches
  if (!FUSED && a.partials_only) {  // every split's partial, whatever the count
    constexpr int W = kDecodeWaves;
    if (one_round) {  // at most one workgroup per CU: the page ring
      if (win)
        hipLaunchKernelGGL((decode_split_kernel<W, 1, false, true, false, KV8, 2, RG>), grid,
                           dim3(W * 64), 0, st, a);
      else
        hipLaunchKernelGGL((decode_split_kernel<W, 1, false, false, false, KV8, 2, RG>), grid,
                           dim3(W * 64), 0, st, a);
    } else if (win)
      hipLaunchKernelGGL((decode_split_kernel<W, 1, false, true, false, KV8>), grid, dim3(W * 64),
                         0, st, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<W, 1, false, false, false, KV8>), grid, dim3(W * 64),
                         0, st, a);
    return hipGetLastError();
  }
  if (a.num_splits == 1 && a.pages_per_split <= kSinglePages &&
      (int64_t)a.num_seqs * a.num_kv_heads * kVSlices <= kVSliceGrid) {
    // one round of slice workgroups: one launch, no merge
    constexpr int W = kVSliceWaves;
    constexpr int P = (kSinglePages + W - 1) / W;
    const dim3 vgrid((unsigned)(a.num_seqs * a.num_kv_heads * kVSlices));
    if (win)
      hipLaunchKernelGGL((decode_vsplit_kernel<W, P, true, FUSED, KV8>), vgrid, dim3(W * 64), 0,
                         st, a);
    else
      hipLaunchKernelGGL((decode_vsplit_kernel<W, P, false, FUSED, KV8>), vgrid, dim3(W * 64), 0,
                         st, a);
    return hipGetLastError();
  }
  if (a.num_splits == 1 && a.pages_per_split <= kSinglePages) {
    constexpr int W = kDecodeWavesSingle;
    constexpr int P = (kSinglePages + W - 1) / W;
    if (win)
      hipLaunchKernelGGL((decode_split_kernel<W, P, true, true, FUSED, KV8>), grid, dim3(W * 64), 0,
                         st, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<W, P, true, false, FUSED, KV8>), grid, dim3(W * 64),
                         0, st, a);
    return hipGetLastError();
  }
  constexpr int W = kDecodeWaves;
  // at most one workgroup per CU: the looser register bound
  constexpr int MW = 2;
  const bool loose = one_round;
  if (a.num_splits == 1) {  // one long split: pipelined loop, sink folded in
    if (loose) {
      if (win)
        hipLaunchKernelGGL((decode_split_kernel<W, 1, true, true, FUSED, KV8, MW, RG>), grid,
                           dim3(W * 64), 0, st, a);
      else
        hipLaunchKernelGGL((decode_split_kernel<W, 1, true, false, FUSED, KV8, MW, RG>), grid,
                           dim3(W * 64), 0, st, a);
    } else if (win) {
      hipLaunchKernelGGL((decode_split_kernel<W, 1, true, true, FUSED, KV8>), grid, dim3(W * 64), 0,
                         st, a);
    } else {
      hipLaunchKernelGGL((decode_split_kernel<W, 1, true, false, FUSED, KV8>), grid, dim3(W * 64),
                         0, st, a);
    }
    return hipGetLastError();
  }
  if (loose) {
    if (win)
      hipLaunchKernelGGL((decode_split_kernel<W, 1, false, true, FUSED, KV8, MW, RG>), grid,
                         dim3(W * 64), 0, st, a);
    else
      hipLaunchKernelGGL((decode_split_kernel<W, 1, false, false, FUSED, KV8, MW, RG>), grid,
                         dim3(W * 64), 0, st, a);
  } else if (win) {
    hipLaunchKernelGGL((decode_split_kernel<W, 1, false, true, FUSED, KV8>), grid, dim3(W * 64), 0,
                       st, a);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<W, 1, false, false, FUSED, KV8>), grid, dim3(W * 64), 0,
                       st, a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge_k(a, st);
}

}  // namespace

#ifdef FLINT_STAMPS
// The last slice-kernel launch's stamps (instrumented build only): copies
// min(bytes, their size) bytes to host memory at dst.
extern "C" int flint_stamps_slice(void* dst, size_t bytes) {
  const size_t n = bytes < sizeof(g_slice_stamps) ? bytes : sizeof(g_slice_stamps);
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_slice_stamps), n, 0, hipMemcpyDeviceToHost) ==
                 hipSuccess
             ? 0
             : -1;
}
#endif

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  if (a.num_seqs == 0) return hipSuccess;
  if (a.kv_fp8)
    return a.q_in ? launch_decode_t<true, true>(a, st) : launch_decode_t<false, true>(a, st);
  return a.q_in ? launch_decode_t<true, false>(a, st) : launch_decode_t<false, false>(a, st);
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t st) {
  if (a.num_seqs == 0) return hipSuccess;
  return launch_merge_k(a, st);
}

}  // namespace flint
