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
// wave owns kTiles such tiles (kWaveRows consecutive rows); a work item is
// kRows rows of one KV group, run by a workgroup of kPWaves waves (a
// persistent grid of one workgroup per CU loops over the items).  The
// workgroup walks the key pages of the item's rows in pairs (32 keys): every
// thread fetches 16 bytes of K and 16 bytes of V of the pair two ahead while
// the waves compute on the current one, and each pair is staged once in LDS
// (double-buffered, one barrier per pair) for all waves -- HBM/L2 traffic per
// flop falls by the number of waves.
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
// sched_group_barrier classes (vector ALU, matrix, transcendental) and the
// issue order of the value products (see compute() below): the fp16 form's
// vector and transcendental work first, the bf16 form's softmax interleaved
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedTrans = 0x400;
constexpr int kSoftmaxValuFirst = 40, kValuPerMfma = 2;
constexpr int kFastValuFirst = 40;
constexpr int kWaveRows = kTiles * 2;        // query rows per wave
constexpr int kPWaves = 8;                   // waves per workgroup
constexpr int kPThreads = kPWaves * 64;
constexpr int kRows = kWaveRows * kPWaves;   // query rows per work item
constexpr int kPrefillWorkgroups = 256;      // persistent grid: one workgroup per CU
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
// V is staged as fp16, the value MFMA's operand.
constexpr int kBufBytes = kKBytes + kHeadDim * kVStride;
// P enters the value MFMA as fp16(p * kPScale): p < 2^8 (the lazy max), so
// p * 2^7 < 2^15 stays inside fp16's range and small p stay normal down to
// 2^-21; the output is scaled back by 1/kPScale.
constexpr float kPScale = 128.f, kPScaleLog2 = 7.f;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
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

// Two fp8 codes (byte pair HI of w) or two bf16 values (a word) as fp16,
// exactly (every E4M3 value is an fp16 number; a bf16 value is one when its
// magnitude is at most 65504, and a larger one becomes +-inf).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const float lo = __builtin_bit_cast(float, w << 16);
  const float hi = __builtin_bit_cast(float, w & 0xffff0000u);
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
}

// Stages this thread's chunk of a pair: K as bf16 (fp8 codes widened
// exactly); V as fp16 (F16) or bf16.
template <bool KV8, bool F16>
__device__ __forceinline__ void stage_pair(unsigned char* buf, int tid, u32x4 kr, u32x4 vr) {
  const int sel = tid >> 8, c = tid & 255;
  u32x4 vh;
  if constexpr (KV8) {  // codes -> bf16 / fp16 (exact), same elements in the same order
    const u32x2 k0 = __builtin_bit_cast(u32x2, fp8x4_to_bf16x4(kr[0]));
    const u32x2 k1 = __builtin_bit_cast(u32x2, fp8x4_to_bf16x4(kr[1]));
    kr = u32x4{k0[0], k0[1], k1[0], k1[1]};
    if constexpr (F16) {
      vh = u32x4{fp8x2_to_f16x2<false>(vr[0]), fp8x2_to_f16x2<true>(vr[0]),
                 fp8x2_to_f16x2<false>(vr[1]), fp8x2_to_f16x2<true>(vr[1])};
    } else {
      const u32x2 v0 = __builtin_bit_cast(u32x2, fp8x4_to_bf16x4(vr[0]));
      const u32x2 v1 = __builtin_bit_cast(u32x2, fp8x4_to_bf16x4(vr[1]));
      vh = u32x4{v0[0], v0[1], v1[0], v1[1]};
    }
  } else if constexpr (F16) {
    vh = u32x4{bf16x2_to_f16x2(vr[0]), bf16x2_to_f16x2(vr[1]), bf16x2_to_f16x2(vr[2]),
               bf16x2_to_f16x2(vr[3])};
  } else {
    vh = vr;
  }
  *(u32x4*)(buf + k_slot(sel * kPage + (c >> 4), c & 15)) = kr;
  // V chunk: dim c>>1, keys h*8..h*8+7 = key groups 2h and 2h+1 of page sel
  const int d = c >> 1, h = c & 1;
  *(u32x2*)(buf + v_slot(d, 2 * h) + sel * 8) = u32x2{vh[0], vh[1]};
  *(u32x2*)(buf + v_slot(d, 2 * h + 1) + sel * 8) = u32x2{vh[2], vh[3]};
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

// Phase stamps (the instrumented build only, -DFLINT_STAMPS, which
// bench.py --stamps loads): per work item (its slot in the item order) and
// wave, s_memrealtime at item entry (0), once the request's lengths are in
// (1), once pair 0 is staged (2), after the barrier before the loop (3), at
// the loop's end (4) and after the output stores (5); slot 6 holds the
// workgroup (bits 16 up) and the CU (__smid, the low 16 bits) and slot 7 the
// item's page pairs.  The product build compiles
// every stamp to nothing.
#ifdef FLINT_STAMPS
constexpr int kStampItems = 8192;
__device__ unsigned long long g_prefill_stamps[kStampItems * kPWaves * 8];
#define PF_STAMP(k)                                                                    \
  do {                                                                                 \
    __builtin_amdgcn_sched_barrier(0);                                                 \
    const unsigned long long t_ = __builtin_amdgcn_s_memrealtime();                    \
    if (lane == 0 && item < kStampItems) g_prefill_stamps[(item * kPWaves + w) * 8 + (k)] = t_; \
    __builtin_amdgcn_sched_barrier(0);                                                 \
  } while (0)
#define PF_STAMP_VALUE(k, v)                                                           \
  do {                                                                                 \
    if (lane == 0 && item < kStampItems) g_prefill_stamps[(item * kPWaves + w) * 8 + (k)] = (v); \
  } while (0)
#else
#define PF_STAMP(k) \
  do {              \
  } while (0)
#define PF_STAMP_VALUE(k, v) \
  do {                       \
  } while (0)
#endif

// A request's lengths as the kernel last read them (items of one request
// reuse them), and the page range of one of its row blocks.
struct ReqLens {
  int b, q0, q_len, seq_len;
};

// The page range [pf, pl] of row block `tile` of a request with lengths rl;
// false when the block has no page pairs to walk (no rows, a request outside
// q/out or an invalid one).  The same range prefill_item walks.
template <bool WINDOWED>
__device__ __forceinline__ bool item_pages(const PrefillArgs& a, int tile, const ReqLens& rl,
                                           int& pf, int& pl) {
  const int wg_row0 = tile * kRows;
  if (rl.q_len <= 0 || wg_row0 >= rl.q_len || rl.q0 < 0 ||
      (int64_t)rl.q0 + rl.q_len > a.total_q)
    return false;
  if (rl.q_len > a.max_q_len || rl.seq_len > a.max_seq_len || rl.q_len > rl.seq_len) return false;
  const int base = rl.seq_len - rl.q_len;
  const int wg_pos_last = base + min(wg_row0 + kRows, rl.q_len) - 1;
  const int wg_lo = WINDOWED ? max(0, base + wg_row0 - a.window + 1) : 0;
  pf = wg_lo / kPage;
  pl = wg_pos_last / kPage;
  return true;
}

// Page ids handed from one item to the next of the same request: pairs 0..2
// of the next item, requested after the current item's last pair (ids[2j],
// ids[2j+1] = the table entries of pair j's two pages).
struct IdCarry {
  int ids[6];
  bool valid;
};

// The item order: row blocks from the last down (longest key range first),
// then KV group, then request.  The first nfixed items are dealt out in
// rounds of gridDim.x, every other round in reverse; the rest are claimed one
// at a time from a counter in the workspace by whichever workgroup frees up
// first, so CUs that run faster take more of them.  With more items than
// workgroups the last third of the rounds, rounded up, is claimed (of 16
// rounds 6: 14% of one causal request's work, 37.5% of equal items'); with
// no more, every workgroup runs one item and nothing is claimed.
// a value every lane holds alike, in scalar registers
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// The workspace: the claim counter (8 bytes), the count of flagged items (4
// bytes, then 4 of padding) and one flag per item: set when a bf16 cache's
// page pairs of the item hold a V value beyond fp16's range, cleared by the
// fix-up launch once it has recomputed the item.
__device__ __forceinline__ unsigned* fix_count(const PrefillArgs& a) {
  return (unsigned*)(a.claims + 1);
}
__device__ __forceinline__ unsigned* fix_flags(const PrefillArgs& a) {
  return (unsigned*)(a.claims + 2);
}

struct ItemOrder {
  int ntile;                 // row blocks of the longest request
  int64_t per_tile, nitems;  // items per row block (groups x requests), all items
  int64_t nfixed;            // items dealt out in fixed rounds
  unsigned long long last_claim;  // value of the launch's last claim
};

__device__ __forceinline__ ItemOrder item_order(const PrefillArgs& a, int G) {
  ItemOrder o;
  o.ntile = (a.max_q_len + kRows - 1) / kRows;
  o.per_tile = (int64_t)a.num_kv_heads * a.num_seqs;
  o.nitems = o.per_tile * o.ntile;
  const int64_t rounds = (o.nitems + G - 1) / G;
  o.nfixed = o.nitems <= G ? o.nitems : (rounds - (rounds + 2) / 3) * G;
  // every workgroup claims until a claim fails: nitems - nfixed claims that
  // succeed and one per workgroup that does not
  o.last_claim = (unsigned long long)(o.nitems - o.nfixed + G - 1);
  return o;
}

// One work item: the kRows query rows of row block `tile` of request rl.b,
// for KV group g, at slot `item` of the item order.  Every wave of the
// workgroup runs it (waves without rows still stage pages and meet the
// barriers); items with no rows return at once.  Returns the slot of the
// workgroup's next item: next_fixed, or when `claim` the one claimed during
// this item.  Wave 0's lane 0 takes the claim (early, so that it has returned
// by the time pair 0 has been staged) and writes it to sm_claim[par] before
// a barrier; every wave reads it after that barrier.  par alternates between
// a workgroup's items: a wave may still read one item's claim while wave 0
// writes the next one's.  carry: in, the ids of this item's first three pairs
// if valid; out, those of the next item when it belongs to the same request.
template <bool WINDOWED, bool KV8, bool F16>
__device__ __forceinline__ int64_t prefill_item(const PrefillArgs& a, const ItemOrder& o,
                                                int tile, int g, const ReqLens& rl, int64_t item,
                                                unsigned char (&sm)[2][kBufBytes],
                                                float (&sm_sink)[kGroup], int64_t (&sm_claim)[2],
                                                int par, IdCarry& carry, bool claim,
                                                int64_t next_fixed) {
  const int b = rl.b;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, gq = lane >> 4;
  const int hkv = a.num_kv_heads, hq = hkv * kGroup;
  PF_STAMP(0);
  PF_STAMP_VALUE(6, ((unsigned long long)blockIdx.x << 16) | __smid());

  const int q0 = rl.q0, q_len = rl.q_len, seq_len = rl.seq_len;
  const bool carried = carry.valid;
  carry.valid = false;
  const int wg_row0 = tile * kRows;
  // the claim's value as wave 0 publishes it; the last claim of the launch
  // leaves the counter at zero for the next one
  auto publish = [&](unsigned long long c) {
    sm_claim[par] = (int64_t)c;
    if (c == o.last_claim) atomicExch(a.claims, 0ull);
  };
  // no rows in this workgroup, or rows outside q / out: a request whose
  // cu_q_lens range leaves [0, total_q) is not touched at all (no row of it
  // can be located safely)
  if (q_len <= 0 || wg_row0 >= q_len || q0 < 0 || (int64_t)q0 + q_len > a.total_q) {
    if (!claim) return next_fixed;
    if (tid == 0) publish(atomicAdd(a.claims, 1ull));
    __syncthreads();
    return o.nfixed + uniform64(sm_claim[par]);
  }
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
#ifdef FLINT_STAMPS
  asm volatile("" ::"s"(npairs));  // stamp 1 after the lengths have arrived
#endif
  PF_STAMP(1);
  PF_STAMP_VALUE(7, npairs);

  // Q operands (tile mt, column n -> row row0 + 2*mt + (n>>3), head
  // g*8 + (n&7)), loaded at start-up, below
  bf16x8 qop[kTiles][4] = {};
  int qpos[kTiles];
#pragma unroll
  for (int mt = 0; mt < kTiles; ++mt) qpos[mt] = base + row0 + 2 * mt + (n >> 3);

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
      // exponent arguments x = s * qscale - m_run (log2 units), carried as
      // x + 7 so that 2^(x+7) = kPScale * p.  Lazy rescale: the reference max
      // moves only when some x exceeds 8, so p = 2^x < 2^8 and the
      // accumulators are rescaled a few times per row rather than every
      // pair.  The exact row max is taken only then.
      float xv[kTiles][8];
      bool grow = false;
#pragma unroll
      for (int mt = 0; mt < kTiles; ++mt)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xv[mt][j] = fmaf(sv[mt][j], a.qscale, kPScaleLog2 - m_run[mt]);
          grow |= xv[mt][j] > 8.f + kPScaleLog2;
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
          for (int j = 0; j < 8; ++j) xv[mt][j] = fmaf(sv[mt][j], a.qscale, kPScaleLog2 - m_new);
        }
      }
      // p (scaled by kPScale) into the value product.  Common path: fp16 P
      // against the fp16 copy of V, one MFMA per 16 dims: fp16 carries p to
      // 2^-12 relative.  A pair with a V value beyond fp16's range (bf16
      // cache only) takes bf16 V, with P split into bf16(p) and its bf16
      // remainder (two MFMAs).
      if constexpr (F16) {
#pragma unroll
        for (int mt = 0; mt < kTiles; ++mt) {
          float pv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) pv[j] = exp2_fast(xv[mt][j]);
          l_part[mt] += ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
          f16x8 ph;
#pragma unroll
          for (int j = 0; j < 8; j += 2) {
            const f32x2 pp = {pv[j], pv[j + 1]};
            const f16x2 h = __builtin_convertvector(pp, f16x2);
            ph[j] = h[0];
            ph[j + 1] = h[1];
          }
#pragma unroll
          for (int nb = 0; nb < 8; ++nb)
            acc[mt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                ph, __builtin_bit_cast(f16x8, pr.v[nb]), acc[mt][nb], 0, 0, 0);
        }
        // Issue order: both tiles' exponentials, sums and conversions, then
        // the 16 value MFMAs back to back.  With two waves per SIMD one
        // wave's MFMA run then overlaps the other's vector run; spreading
        // tile 1's softmax between tile 0's MFMAs, or no order at all,
        // measured 1.5-3.5% slower.
        __builtin_amdgcn_sched_group_barrier(kSchedValu | kSchedTrans, kFastValuFirst, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 16, 0);
      } else {
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
        // Issue order of the block above: tile 0's exponentials and splits
        // first, then tile 0's 16 value MFMAs each followed by two vector
        // instructions of tile 1's softmax, then tile 1's value MFMAs.  Left to
        // itself the scheduler puts both tiles' softmax ahead of every value
        // MFMA, so a wave's vector work never runs under its own MFMAs
        // (measured: the 32K full layer 11.5 -> 11.1-11.2 ms).
        __builtin_amdgcn_sched_group_barrier(kSchedValu, kSoftmaxValuFirst, 0);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedValu, kValuPerMfma, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 16, 0);
      }
    }
  };
  // In flight at the top of iteration i: pair i in LDS buffer i&1, the page
  // loads of pairs i+1 and i+2 in register sets (i+1)&1 and (i+2)&1, the ids
  // of pairs i+3 and i+4 in id sets (i+3)&1 and (i+4)&1 (loop unrolled by two
  // so every set is static).
  //
  // Start-up: the group's sinks and the first page ids, then the Q operands,
  // then the first pair's pages once its ids are in.  Vector loads complete
  // in issue order, so the wait for the ids does not wait for Q, and Q
  // arrives under the id round trip instead of after it.  Every load here is
  // unconditional (a row index clamped into the chunk: waves without rows
  // load and ignore), so the compiler's counts of loads in flight are exact.
  // The sinks go to LDS (read in the epilogue) rather than holding registers
  // through the loop.
  u32x4 kr0, vr0, kr1, vr1;
  int ia0, ib0, ia1, ib1, ia2, ib2;
  float sink_l2 = 0.f;
  unsigned long long cval = 0;
  if (npairs > 0) {
    const float sink = a.sinks[g * kGroup + (lane & 7)];
    if (carried) {  // requested by the previous item, after its last pair
      ia0 = carry.ids[0], ib0 = carry.ids[1];
      ia1 = carry.ids[2], ib1 = carry.ids[3];
      ia2 = carry.ids[4], ib2 = carry.ids[5];
    } else {
      load_ids(0, ia0, ib0);
      load_ids(1, ia1, ib1);
      load_ids(2, ia2, ib2);
    }
#pragma unroll
    for (int mt = 0; mt < kTiles; ++mt) {
      const int r = min(row0 + 2 * mt + (n >> 3), q_len - 1);
      const uint16_t* qp =
          a.q + (((int64_t)(q0 + r) * hq) + g * kGroup + (n & 7)) * kHeadDim + gq * 8;
#pragma unroll
      for (int c = 0; c < 4; ++c) qop[mt][c] = *(const bf16x8*)(qp + c * 32);
    }
    // after the ids (the wait for them does not wait for the claim), before
    // pair 0's pages (the wait for them does)
    if (claim && tid == 0) cval = atomicAdd(a.claims, 1ull);
    fetch(0, ia0, ib0, kr0, vr0);  // waits for the ids, hence for the sinks
    sink_l2 = sink * kLog2e;
    stage_pair<KV8, F16>(sm[0], tid, kr0, vr0);
    if (claim && tid == 0) publish(cval);
    // Q and the sinks were issued before pair 0, so they are in; pinning
    // them here keeps the compiler from waiting for them inside the loop,
    // where it could not tell them from the page loads in flight
#pragma unroll
    for (int mt = 0; mt < kTiles; ++mt)
#pragma unroll
      for (int c = 0; c < 4; ++c) asm volatile("" ::"v"(qop[mt][c]));
    PF_STAMP(2);
    fetch(1, ia1, ib1, kr1, vr1);
    fetch(2, ia2, ib2, kr0, vr0);
    load_ids(3, ia1, ib1);
    load_ids(4, ia0, ib0);
  } else if (claim && tid == 0) {
    publish(atomicAdd(a.claims, 1ull));
  }
  __syncthreads();
  PF_STAMP(3);
  // every wave has left the previous item's epilogue (the last reader of
  // sm_sink) by the barrier above; the loop's first barrier publishes this
  if (npairs > 0 && tid < kGroup) sm_sink[tid] = sink_l2;
  // the next item, and its page range if it belongs to this request
  const int64_t next = claim ? o.nfixed + uniform64(sm_claim[par]) : next_fixed;
  bool next_ok = false;
  int next_pf = 0, next_pl = 0;
  if (next < o.nitems && (int)(next % o.per_tile) / hkv == b)
    next_ok = item_pages<WINDOWED>(a, o.ntile - 1 - (int)(next / o.per_tile), rl, next_pf, next_pl);
  for (int i = 0; i < npairs; i += 2) {
    compute(i);
    if (i + 1 < npairs) stage_pair<KV8, F16>(sm[1], tid, kr1, vr1);
    fetch(i + 3, ia1, ib1, kr1, vr1);
    load_ids(i + 5, ia1, ib1);
    __syncthreads();
    if (i + 1 >= npairs) break;
    compute(i + 1);
    if (i + 2 < npairs) stage_pair<KV8, F16>(sm[0], tid, kr0, vr0);
    fetch(i + 4, ia0, ib0, kr0, vr0);
    load_ids(i + 6, ia0, ib0);
    __syncthreads();
  }
  PF_STAMP(4);
  // the next item's first page ids, before this item's output stores (the
  // id registers are free: the last pair has been fetched)
  if (next_ok) {
    const int* nrow = a.block_tables + (int64_t)b * a.bt_stride;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int p = min(next_pf + 2 * j, next_pl);
      carry.ids[2 * j] = nrow[p];
      carry.ids[2 * j + 1] = nrow[min(p + 1, next_pl)];
    }
    carry.valid = true;
  }
  if (!active) return next;

  bad = __any(bad);
  // epilogue: acc rows gq*4+i are query vectors; their m and l live in lane gq*4+i
  bool nonfinite = false;
#pragma unroll
  for (int mt = 0; mt < kTiles; ++mt) {
    float l_c = l_part[mt] + __shfl_xor(l_part[mt], 16);
    l_c += __shfl_xor(l_c, 32);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = gq * 4 + i;  // query vector of acc row
      const float m = __shfl(m_run[mt], v);
      const float l = __shfl(l_c, v) * (1.f / kPScale);  // l_part sums kPScale * p
      const int r = row0 + 2 * mt + (v >> 3);
      if (r >= q_len) continue;
      const int h = g * kGroup + (v & 7);
      const float sink = sm_sink[v & 7];
      const float M2 = fmaxf(m, sink);
      const float so = exp2_fast(m - M2);
      const float inv = 1.f / (l * so + exp2_fast(sink - M2));
      const float vs = (KV8 ? a.v_scale : 1.f) * (1.f / kPScale);  // acc holds kPScale * P.V
      float* dst = a.out + ((int64_t)(q0 + r) * hq + h) * kHeadDim + n;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const float x = acc[mt][nb][i] * so * inv * vs;
        nonfinite |= !__builtin_isfinite(x);
        dst[nb * 16] = bad ? __builtin_nanf("") : x;
      }
    }
  }
  // A bf16 V value beyond fp16's range was staged as +-inf, and every row of
  // a wave whose MFMAs took it reads inf or NaN (0 * inf for the rows that
  // do not see that key): the item is flagged, and the fix-up launch
  // recomputes it with bf16 V.  (Non-finite inputs flag it too; the
  // recomputation then gives the same non-finite rows.)
  if (F16 && !KV8 && !bad && __any(nonfinite) && lane == 0) {
    if (atomicCAS(&fix_flags(a)[item], 0u, 1u) == 0u) atomicAdd(fix_count(a), 1u);
  }
  PF_STAMP(5);
  return next;
}

// Persistent grid: at most kPrefillWorkgroups workgroups (one per CU), each
// looping over items in the order of ItemOrder: fixed rounds first, balanced
// by the longest-first zig-zag deal, then claimed items, which even out the
// CUs' differing speeds.  Handing items to workgroups here rather than
// launching one workgroup per item leaves no dispatch gaps: MI355X deals
// workgroups to its 8 XCDs in turn, so with items of unequal length a CU that
// frees up waits until the XCD whose turn it is has a free CU too.
template <bool WINDOWED, bool KV8>
__global__ __launch_bounds__(kPThreads, 1) void prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char sm[2][kBufBytes];
  __shared__ float sm_sink[kGroup];  // log2-scaled sinks of the current item's heads
  __shared__ int64_t sm_claim[2];    // claimed item offsets, alternating between items
  const int G = gridDim.x;
  const ItemOrder o = item_order(a, G);
  auto slot_of = [&](int64_t r) {
    return r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
  };
  ReqLens rl = {-1, 0, 0, 0};
  IdCarry carry;
  carry.valid = false;
  int64_t slot = slot_of(0);
  for (int64_t r = 0; slot < o.nitems; ++r) {
    const int tile = o.ntile - 1 - (int)(slot / o.per_tile);
    const int rest = (int)(slot % o.per_tile);
    const int b = rest / a.num_kv_heads;
    if (b != rl.b) {
      rl.b = b;
      rl.q0 = a.cu_q_lens[b];
      rl.q_len = a.cu_q_lens[b + 1] - rl.q0;
      rl.seq_len = a.seq_lens[b];
    }
    // the next item is claimed from its last fixed one on
    const bool claim = o.nfixed < o.nitems && (r + 1) * G >= o.nfixed;
    slot = prefill_item<WINDOWED, KV8, true>(a, o, tile, rest % a.num_kv_heads, rl, slot, sm,
                                             sm_sink, sm_claim, (int)(r & 1), carry, claim,
                                             claim ? o.nitems : slot_of(r + 1));
  }
}

// Fix-up launch after a bf16-cache prefill: recomputes, with bf16 V and P
// split into bf16(p) and its bf16 remainder, every item the main launch
// flagged (a V value beyond fp16's range in its pages), and clears the flags.
// With no item flagged every workgroup returns after one load.
template <bool WINDOWED>
__global__ __launch_bounds__(kPThreads, 1) void prefill_fix_kernel(PrefillArgs a) {
  if (__hip_atomic_load(fix_count(a), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) return;
  __shared__ __attribute__((aligned(16))) unsigned char sm[2][kBufBytes];
  __shared__ float sm_sink[kGroup];
  __shared__ int64_t sm_claim[2];
  const int G = gridDim.x;
  ItemOrder o = item_order(a, G);
  o.nfixed = o.nitems;  // every item in fixed rounds: nothing is claimed
  unsigned* flags = fix_flags(a);
  for (int64_t r = 0;; ++r) {
    const int64_t slot = r * G + ((r & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
    if (slot >= o.nitems) break;
    if (__hip_atomic_load(&flags[slot], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) continue;
    const int tile = o.ntile - 1 - (int)(slot / o.per_tile);
    const int rest = (int)(slot % o.per_tile);
    const int b = rest / a.num_kv_heads;
    ReqLens rl;
    rl.b = b;
    rl.q0 = a.cu_q_lens[b];
    rl.q_len = a.cu_q_lens[b + 1] - rl.q0;
    rl.seq_len = a.seq_lens[b];
    IdCarry carry;
    carry.valid = false;
    prefill_item<WINDOWED, false, false>(a, o, tile, rest % a.num_kv_heads, rl, slot, sm, sm_sink,
                                         sm_claim, (int)(r & 1), carry, false, o.nitems);
    __syncthreads();
    if (threadIdx.x == 0) {
      flags[slot] = 0u;
      atomicSub(fix_count(a), 1u);
    }
  }
}

}  // namespace

#ifdef FLINT_STAMPS
// The last launch's prefill stamps (instrumented build only): copies
// min(bytes, their size) bytes to host memory at dst.
extern "C" int flint_stamps_prefill(void* dst, size_t bytes) {
  const size_t n = bytes < sizeof(g_prefill_stamps) ? bytes : sizeof(g_prefill_stamps);
  return hipMemcpyFromSymbol(dst, HIP_SYMBOL(g_prefill_stamps), n, 0, hipMemcpyDeviceToHost) ==
                 hipSuccess
             ? 0
             : -1;
}
#endif

static int64_t prefill_items(int32_t num_seqs, int32_t num_kv_heads, int32_t max_q_len) {
  return (int64_t)((max_q_len + kRows - 1) / kRows) * num_kv_heads * num_seqs;
}

// The claim counter, the flagged-item count and one flag per item (see
// fix_flags); the caller zero-fills it once and every call leaves it zero.
size_t prefill_workspace_bytes(int32_t num_seqs, int32_t num_kv_heads, int32_t max_q_len) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_q_len <= 0) return 0;
  return 16 + 4 * (size_t)prefill_items(num_seqs, num_kv_heads, max_q_len);
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  if (a.num_seqs == 0 || a.max_q_len == 0) return hipSuccess;
  if (!a.claims) return hipErrorInvalidValue;
  const int64_t items = prefill_items(a.num_seqs, a.num_kv_heads, a.max_q_len);
  const dim3 grid((unsigned)(items < kPrefillWorkgroups ? items : kPrefillWorkgroups));
  if (a.kv_fp8) {
    if (a.window > 0)
      hipLaunchKernelGGL((prefill_kernel<true, true>), grid, dim3(kPThreads), 0, st, a);
    else
      hipLaunchKernelGGL((prefill_kernel<false, true>), grid, dim3(kPThreads), 0, st, a);
    return hipGetLastError();
  }
  if (a.window > 0) {
    hipLaunchKernelGGL((prefill_kernel<true, false>), grid, dim3(kPThreads), 0, st, a);
    hipLaunchKernelGGL((prefill_fix_kernel<true>), grid, dim3(kPThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((prefill_kernel<false, false>), grid, dim3(kPThreads), 0, st, a);
    hipLaunchKernelGGL((prefill_fix_kernel<false>), grid, dim3(kPThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace flint
