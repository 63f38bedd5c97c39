/* A plain C99 program that runs both decode entry points on the GPU through
 * the C ABI: it reads a batch written by tests/test_gpu_c_abi.py (host arrays
 * in the device layouts), allocates device memory with hipMalloc, launches
 * lazy_attn_decode and lazy_attn_decode_shared on the null stream with
 * check_tables set, and writes both outputs back for the test to compare with
 * the oracle.  Every file's size is checked against the shapes before any
 * allocation, so a mismatch stops here and never reaches a kernel. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lazy_attn.h"

static const char* g_dir;

static void* read_exact(const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) {
    printf("cannot open %s\n", path);
    exit(2);
  }
  fseek(f, 0, SEEK_END);
  const long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  if (n < 0 || (size_t)n != bytes) {
    printf("%s holds %ld bytes, expected %zu\n", name, n, bytes);
    exit(2);
  }
  void* p = malloc(bytes ? bytes : 1);
  if (bytes && fread(p, 1, bytes, f) != bytes) {
    printf("short read of %s\n", name);
    exit(2);
  }
  fclose(f);
  return p;
}

static void write_all(const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", g_dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) {
    printf("cannot write %s\n", path);
    exit(2);
  }
  fclose(f);
}

/* Device buffer of `bytes`, filled from h (NULL: left uninitialised). */
static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 16) != hipSuccess) {
    printf("hipMalloc failed\n");
    exit(3);
  }
  if (h && bytes && hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) {
    printf("hipMemcpy failed\n");
    exit(3);
  }
  return d;
}

#define CALL(x)                                                                 \
  do {                                                                          \
    la_status s_ = (x);                                                         \
    if (s_ != LA_OK) {                                                          \
      printf("%s: %s: %s\n", #x, lazy_attn_status_string(s_), lazy_attn_last_error()); \
      return 4;                                                                 \
    }                                                                           \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) return 1;
  g_dir = argv[1];
  long long m[16];
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/meta.txt", g_dir);
    FILE* f = fopen(path, "r");
    if (!f) return 2;
    for (int i = 0; i < 16; ++i)
      if (fscanf(f, "%lld", &m[i]) != 1) return 2;
    fclose(f);
  }
  la_params p;
  memset(&p, 0, sizeof p);
  p.num_q_heads = (int32_t)m[0];
  p.num_kv_heads = (int32_t)m[1];
  p.head_dim = (int32_t)m[2];
  p.block_size = (int32_t)m[3];
  p.num_blocks = m[4];
  p.max_pos = (int32_t)m[5];
  const int32_t batch = (int32_t)m[6];
  const int32_t maxb = (int32_t)m[7];
  const size_t n_words = (size_t)m[8];
  uint32_t scale_bits = (uint32_t)m[9];
  memcpy(&p.scale, &scale_bits, sizeof p.scale);
  p.dtype = LA_BF16;
  p.check_tables = 1;
  la_shared_plan_info info;
  info.batch = batch;
  info.n_items = (int32_t)m[10];
  info.n_members = (int32_t)m[11];
  info.n_words = (int32_t)m[12];
  info.members_per_item = (int32_t)m[13];
  info.max_item_blocks = (int32_t)m[14];
  info.plan_bytes = m[15];
  info.workspace_bytes = 0;

  const size_t D = (size_t)p.head_dim, Hq = (size_t)p.num_q_heads, Hkv = (size_t)p.num_kv_heads;
  const size_t nb = (size_t)p.num_blocks, BS = (size_t)p.block_size;
  const size_t q_bytes = (size_t)batch * Hq * D * 2, pool_bytes = nb * Hkv * BS * D * 2;
  void* q = read_exact("q.bin", q_bytes);
  void* k = read_exact("k.bin", pool_bytes);
  void* v = read_exact("v.bin", pool_bytes);
  void* words = read_exact("words.bin", n_words * 8);
  void* rbs = read_exact("rbs.bin", (size_t)(batch + 1) * 4);
  void* qpos = read_exact("qpos.bin", (size_t)batch * 4);
  void* cs = read_exact("cs.bin", (size_t)p.max_pos * D * 4);
  void* plan = read_exact("plan.bin", (size_t)info.plan_bytes);

  void* dq = to_device(q, q_bytes);
  void* dk = to_device(k, pool_bytes);
  void* dv = to_device(v, pool_bytes);
  void* dwords = to_device(words, n_words * 8);
  void* drbs = to_device(rbs, (size_t)(batch + 1) * 4);
  void* dqpos = to_device(qpos, (size_t)batch * 4);
  void* dcs = to_device(cs, (size_t)p.max_pos * D * 4);
  void* dplan = to_device(plan, (size_t)info.plan_bytes);
  void* dout = to_device(NULL, q_bytes);
  void* host_out = malloc(q_bytes);

  size_t ws_bytes = 0;
  CALL(lazy_attn_decode_workspace_size(&p, batch, maxb, &ws_bytes));
  void* dws = ws_bytes ? to_device(NULL, ws_bytes) : NULL;
  CALL(lazy_attn_decode(&p, dq, dk, dv, (const uint64_t*)dwords, (const int32_t*)drbs,
                        (const int32_t*)dqpos, (const float*)dcs, batch, maxb, dout, NULL, dws,
                        ws_bytes, NULL));
  if (hipDeviceSynchronize() != hipSuccess) return 5;
  if (hipMemcpy(host_out, dout, q_bytes, hipMemcpyDeviceToHost) != hipSuccess) return 5;
  write_all("out_per_request.bin", host_out, q_bytes);

  /* the workspace the planner asked for: n_members x Hq x (D + 2) floats */
  const size_t sws = (size_t)info.n_members * Hq * (D + 2) * 4;
  void* dsws = to_device(NULL, sws);
  CALL(lazy_attn_decode_shared(&p, &info, dplan, dq, dk, dv, (const int32_t*)dqpos,
                               (const float*)dcs, batch, dout, NULL, dsws, sws, NULL));
  if (hipDeviceSynchronize() != hipSuccess) return 5;
  if (hipMemcpy(host_out, dout, q_bytes, hipMemcpyDeviceToHost) != hipSuccess) return 5;
  write_all("out_shared.bin", host_out, q_bytes);
  printf("OK\n");
  return 0;
}
