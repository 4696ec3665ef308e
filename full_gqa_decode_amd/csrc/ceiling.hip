// ceiling.hip -- measurement kernels for the machine ceilings the decode
// kernels are compared against (libflint_ceiling.so, loaded by the bench
// only; nothing in libflint calls it).
//
//   flint_ceiling_stream_read  every byte of a buffer, in chunks of chunk_kb
//                              KiB placed at pseudo-random offsets (a fixed
//                              odd-multiplier permutation), 256 workgroups of
//                              8 waves, each wave keeping two steps of 8 KiB
//                              in flight; nontemporal or ordinary loads.
//   flint_ceiling_page_walk    the loads of the split-K decode kernel alone,
//                              in its shape: a workgroup per (split, KV head),
//                              8 waves, wave w walks pages w, w+8, ... of its
//                              split through a page table, one page of loads
//                              ahead; per page and head 4 KiB of K (4 x
//                              16-byte loads per lane) and 4 KiB of V (8 x
//                              8-byte loads) for a bf16 cache, or 2 KiB of
//                              each (2 x 16-byte loads) for an fp8 cache,
//                              nontemporal.  Every loaded dword is folded into
//                              one value per lane, so no load is dropped.
//   flint_ceiling_empty        a kernel that does nothing (launch cost).
//   flint_ceiling_atomics      count agent-scope atomic adds on one counter
//                              (throughput of a hot counter; no thread ever
//                              waits on another).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kWgs = 256;
constexpr int kLinesPerWave = 96;  // 1 KiB lines per wave
constexpr int kLinesPerStep = 8;
constexpr uint64_t kMul = 40505;   // odd and prime to 3: a permutation of C chunks

template <int T_KB, bool NT>
__global__ __launch_bounds__(kWaves * 64, 1) void stream_read_kernel(const char* base,
                                                                     uint32_t* out) {
  constexpr int S = kLinesPerWave / kLinesPerStep;
  constexpr int CPW = kLinesPerWave / T_KB;  // chunks per wave
  constexpr uint64_t C = (uint64_t)kWgs * kWaves * CPW;
  static_assert(kLinesPerWave % T_KB == 0 && S % 2 == 0, "whole chunks, whole step pairs");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint64_t first = (uint64_t)blockIdx.x * kWaves * CPW + w;
  u32x4 ra[kLinesPerStep], rb[kLinesPerStep];
  uint32_t acc = 0;
  auto issue = [&](u32x4 (&r)[kLinesPerStep], int s) {
#pragma unroll
    for (int i = 0; i < kLinesPerStep; ++i) {
      const int l = s * kLinesPerStep + i;
      const uint64_t chunk = first + (uint64_t)kWaves * (l / T_KB);
      const uint64_t pos = (chunk * kMul + 17) % C;  // < C: inside the buffer
      const u32x4* p =
          (const u32x4*)(base + pos * (T_KB * 1024) + (l % T_KB) * 1024 + lane * 16);
      r[i] = NT ? __builtin_nontemporal_load(p) : *p;
    }
  };
  auto fold = [&](const u32x4 (&r)[kLinesPerStep]) {
#pragma unroll
    for (int i = 0; i < kLinesPerStep; ++i) acc ^= r[i][0] ^ r[i][1] ^ r[i][2] ^ r[i][3];
  };
  issue(ra, 0);
#pragma unroll
  for (int s = 0; s < S; s += 2) {
    issue(rb, s + 1);
    fold(ra);
    if (s + 2 < S) issue(ra, s + 2);
    fold(rb);
  }
  out[blockIdx.x * (kWaves * 64) + threadIdx.x] = acc;
}

struct WalkArgs {
  const char* k;
  const char* v;
  const int* table;
  int pages_per_split;
  int pages;
  int heads;
  uint32_t* out;
};

template <bool FP8>
__global__ __launch_bounds__(kWaves * 64, 2) void page_walk_kernel(WalkArgs a) {
  constexpr int kTile = FP8 ? 2048 : 4096;
  const int s = blockIdx.x, g = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pb = s * a.pages_per_split;
  const int last = min(pb + a.pages_per_split, a.pages) - 1;
  int p = pb + w;
  const int n = p <= last ? (last - p) / kWaves + 1 : 0;
  constexpr int KL = FP8 ? 2 : 4;  // 16-byte K loads per lane and page
  constexpr int VL = FP8 ? 2 : 8;  // V loads per lane: 16 bytes (fp8) or 8 (bf16)
  u32x4 k[KL];
  u32x4 v4[FP8 ? VL : 1];
  u32x2 v2[FP8 ? 1 : VL];
  uint32_t acc = 0;
  auto load = [&](int id) {
    const int64_t tile = ((int64_t)id * a.heads + g) * kTile;
    const u32x4* kp = (const u32x4*)(a.k + tile + lane * 16);
#pragma unroll
    for (int c = 0; c < KL; ++c) k[c] = __builtin_nontemporal_load(kp + c * 64);
    if constexpr (FP8) {
      const u32x4* vp = (const u32x4*)(a.v + tile + lane * 16);
#pragma unroll
      for (int c = 0; c < VL; ++c) v4[c] = __builtin_nontemporal_load(vp + c * 64);
    } else {
      const u32x2* vp = (const u32x2*)(a.v + tile + lane * 8);
#pragma unroll
      for (int c = 0; c < VL; ++c) v2[c] = __builtin_nontemporal_load(vp + c * 64);
    }
  };
  auto fold = [&] {
#pragma unroll
    for (int c = 0; c < KL; ++c) acc ^= k[c][0] ^ k[c][1] ^ k[c][2] ^ k[c][3];
    if constexpr (FP8) {
#pragma unroll
      for (int c = 0; c < VL; ++c) acc ^= v4[c][0] ^ v4[c][1] ^ v4[c][2] ^ v4[c][3];
    } else {
#pragma unroll
      for (int c = 0; c < VL; ++c) acc ^= v2[c][0] ^ v2[c][1];
    }
  };
  if (n > 0) {
    // ids are table entries inside [pb, last]; the host checks the table
    load(a.table[p]);
    int next = a.table[min(p + kWaves, last)];
    for (int i = 1; i < n; ++i, p += kWaves) {
      const int after = a.table[min(p + 2 * kWaves, last)];
      fold();
      load(next);
      next = after;
    }
    fold();
  }
  a.out[((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * (kWaves * 64) + threadIdx.x] = acc;
}

__global__ void empty_kernel() {}

__global__ void atomics_kernel(unsigned int* counter, int per_wave) {
  if ((threadIdx.x & 63) == 0)
    for (int i = 0; i < per_wave; ++i)
      __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int T>
int stream_read_t(bool nt, const void* base, uint32_t* out, hipStream_t s) {
  if (nt)
    hipLaunchKernelGGL((stream_read_kernel<T, true>), dim3(kWgs), dim3(kWaves * 64), 0, s,
                       (const char*)base, out);
  else
    hipLaunchKernelGGL((stream_read_kernel<T, false>), dim3(kWgs), dim3(kWaves * 64), 0, s,
                       (const char*)base, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

extern "C" {

// Bytes one flint_ceiling_stream_read call reads (the buffer it needs).
long flint_ceiling_stream_bytes(void) { return (long)kWgs * kWaves * kLinesPerWave * 1024; }

// out: kWgs * 512 uint32 of device memory.  Returns 0, or -1 for a chunk
// size other than 1, 2, 4, 8, 16 or 32 KiB or a failed launch.
int flint_ceiling_stream_read(int chunk_kb, int nontemporal, const void* base, uint32_t* out,
                              void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const bool nt = nontemporal != 0;
  switch (chunk_kb) {
    case 1: return stream_read_t<1>(nt, base, out, s);
    case 2: return stream_read_t<2>(nt, base, out, s);
    case 4: return stream_read_t<4>(nt, base, out, s);
    case 8: return stream_read_t<8>(nt, base, out, s);
    case 16: return stream_read_t<16>(nt, base, out, s);
    case 32: return stream_read_t<32>(nt, base, out, s);
    default: return -1;
  }
}

// k, v: pages * heads * tile bytes each (4096 for a bf16 cache, 2048 for an
// fp8 one: fp8 != 0); table: pages entries, each in [0, pages) (checked by
// the caller); out: splits * heads * 512 uint32.
int flint_ceiling_page_walk(const void* k, const void* v, const int* table, int pages,
                            int heads, int pages_per_split, int fp8, uint32_t* out,
                            void* stream) {
  if (pages < 1 || heads < 1 || pages_per_split < 1) return -1;
  const WalkArgs a{(const char*)k, (const char*)v, table, pages_per_split, pages, heads, out};
  const dim3 grid((pages + pages_per_split - 1) / pages_per_split, heads);
  if (fp8)
    hipLaunchKernelGGL(page_walk_kernel<true>, grid, dim3(kWaves * 64), 0, (hipStream_t)stream,
                       a);
  else
    hipLaunchKernelGGL(page_walk_kernel<false>, grid, dim3(kWaves * 64), 0, (hipStream_t)stream,
                       a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int flint_ceiling_empty(void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// workgroups x 4 waves, each wave's first lane adding 1 per_wave times.
int flint_ceiling_atomics(unsigned int* counter, int workgroups, int per_wave, void* stream) {
  if (workgroups < 1 || per_wave < 0) return -1;
  hipLaunchKernelGGL(atomics_kernel, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, counter,
                     per_wave);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
