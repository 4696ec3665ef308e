/* A plain C11 client of libflint: one fused decode step through the C ABI,
 * with device memory and copies done by the HIP runtime API alone (no Python,
 * no PyTorch).  Used by tests/test_gpu_c_client.py, which writes the inputs
 * and reads the outputs.
 *
 * usage: c_client_decode_step DIR B NUM_BLOCKS BT_STRIDE MAX_SEQ_LEN WINDOW USE_ROPE
 *                             RMS_EPS SOFTMAX_SCALE
 * reads  DIR/{q_in,k_in,v_in,q_w,k_w,slots,k_cache,v_cache,block_tables,
 *             seq_lens,sinks}.bin
 * writes DIR/{out,k_cache_out,v_cache_out}.bin and prints the status. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "flint.h"

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s.bin", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes);
  const size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s.bin", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  const size_t put = fwrite(p, 1, bytes, f);
  return fclose(f) != 0 || put != bytes;
}

#define HIP_OK(x)                                                          \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));              \
      return 1;                                                            \
    }                                                                      \
  } while (0)

enum { IN_Q, IN_K, IN_V, IN_QW, IN_KW, IN_SLOTS, IN_KC, IN_VC, IN_BT, IN_SL, IN_SINKS, N_IN };

int main(int argc, char** argv) {
  if (argc != 10) {
    fprintf(stderr, "usage: %s DIR B NUM_BLOCKS BT_STRIDE MAX_SEQ_LEN WINDOW USE_ROPE "
                    "RMS_EPS SOFTMAX_SCALE\n", argv[0]);
    return 2;
  }
  const char* dir = argv[1];
  const int32_t B = atoi(argv[2]), nb = atoi(argv[3]), bt_stride = atoi(argv[4]);
  const int32_t max_seq_len = atoi(argv[5]);
  const flint_attn_layer L = {32, 4, 128, 16, atoi(argv[6]), atoi(argv[7]), 10000.0f,
                              strtof(argv[8], NULL), strtof(argv[9], NULL), FLINT_KV_BF16,
                              1.0f, 1.0f};
  const size_t cache = (size_t)nb * 4 * 16 * 128 * sizeof(uint16_t);
  const char* names[N_IN] = {"q_in", "k_in", "v_in", "q_w", "k_w", "slots", "k_cache",
                             "v_cache", "block_tables", "seq_lens", "sinks"};
  const size_t bytes[N_IN] = {
      (size_t)B * 32 * 128 * sizeof(float), (size_t)B * 4 * 128 * sizeof(float),
      (size_t)B * 4 * 128 * sizeof(float), 128 * sizeof(float), 128 * sizeof(float),
      (size_t)B * sizeof(int32_t), cache, cache, (size_t)B * bt_stride * sizeof(int32_t),
      (size_t)B * sizeof(int32_t), 32 * sizeof(float)};
  void* dev[N_IN];
  for (int i = 0; i < N_IN; ++i) {
    void* host = read_file(dir, names[i], bytes[i]);
    if (!host) {
      fprintf(stderr, "cannot read %s/%s.bin (%zu bytes)\n", dir, names[i], bytes[i]);
      return 1;
    }
    HIP_OK(hipMalloc(&dev[i], bytes[i]));
    HIP_OK(hipMemcpy(dev[i], host, bytes[i], hipMemcpyHostToDevice));
    free(host);
  }
  const size_t out_bytes = (size_t)B * 32 * 128 * sizeof(float);
  void* out = NULL;
  HIP_OK(hipMalloc(&out, out_bytes));
  const size_t ws_bytes = flint_attn_decode_workspace_size(&L, B, max_seq_len);
  void* ws = NULL;
  if (ws_bytes) HIP_OK(hipMalloc(&ws, ws_bytes));

  const flint_status st = flint_attn_decode_step(
      &L, B, (const float*)dev[IN_Q], (const float*)dev[IN_K], (const float*)dev[IN_V],
      (const float*)dev[IN_QW], (const float*)dev[IN_KW], (const int32_t*)dev[IN_SLOTS], NULL,
      dev[IN_KC], dev[IN_VC], nb, (const int32_t*)dev[IN_BT], bt_stride,
      (const int32_t*)dev[IN_SL], max_seq_len, (const float*)dev[IN_SINKS], (float*)out, ws,
      ws_bytes, 0, NULL);
  printf("status %d\n", (int)st);
  if (st != FLINT_OK) return 3;
  HIP_OK(hipDeviceSynchronize());

  void* host_out = malloc(out_bytes);
  void* host_k = malloc(cache);
  void* host_v = malloc(cache);
  if (!host_out || !host_k || !host_v) return 1;
  HIP_OK(hipMemcpy(host_out, out, out_bytes, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(host_k, dev[IN_KC], cache, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(host_v, dev[IN_VC], cache, hipMemcpyDeviceToHost));
  if (write_file(dir, "out", host_out, out_bytes) ||
      write_file(dir, "k_cache_out", host_k, cache) ||
      write_file(dir, "v_cache_out", host_v, cache))
    return 1;
  free(host_out);
  free(host_k);
  free(host_v);
  for (int i = 0; i < N_IN; ++i) HIP_OK(hipFree(dev[i]));
  HIP_OK(hipFree(out));
  if (ws) HIP_OK(hipFree(ws));
  return 0;
}
