/*
 * One fused decode step through the C ABI from C, on the GPU, with the HIP
 * runtime and no Python: the pool's storage is hipMalloc'ed here, the prefix
 * K/V are placed with the strides pgqa_pool_layout reports, then
 * pgqa_decode_step runs (norm + rotary + cache write + decode) and the outputs
 * and the whole pool storage are written back to files.
 * tests/test_gpu_c_decode.py writes the inputs, runs this program and checks
 * the files against the fp64 oracle.
 *
 * usage: c_decode_step DIR num_blocks block_size num_kv_heads num_q_heads batch bt_stride max_ctx eps theta scale
 * DIR holds q.bin k.bin v.bin wq.bin wk.bin (bf16 bits), ctx.bin bt.bin (int32),
 * prefix_k.bin prefix_v.bin (bf16 bits, logical [num_blocks][block_size][num_kv_heads][128]);
 * it receives out.bin q_out.bin pool.bin layout.txt.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pgqa.h"

static char dir[4096];

static void* read_file(const char* name, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) { fprintf(stderr, "cannot open %s\n", path); exit(10); }
  void* p = malloc(bytes ? bytes : 1);
  if (fread(p, 1, bytes, f) != bytes) { fprintf(stderr, "short read %s\n", path); exit(11); }
  fclose(f);
  return p;
}

static void write_file(const char* name, const void* p, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(p, 1, bytes, f) != bytes) { fprintf(stderr, "cannot write %s\n", path); exit(12); }
  fclose(f);
}

#define HIP(x) do { hipError_t e_ = (x); if (e_ != hipSuccess) { \
  fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_)); exit(20); } } while (0)
#define PGQA(x) do { pgqa_status s_ = (x); if (s_ != PGQA_OK) { \
  fprintf(stderr, "%s: %s (%s)\n", #x, pgqa_status_string(s_), pgqa_last_error()); exit(30); } } while (0)

static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (h != NULL && bytes) HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
  else if (bytes) HIP(hipMemset(d, 0, bytes));
  return d;
}

int main(int argc, char** argv) {
  if (argc != 12) { fprintf(stderr, "usage: see the header comment\n"); return 2; }
  snprintf(dir, sizeof dir, "%s", argv[1]);
  const int32_t nb = atoi(argv[2]), bs = atoi(argv[3]), hkv = atoi(argv[4]), hq = atoi(argv[5]);
  const int32_t B = atoi(argv[6]), bt_stride = atoi(argv[7]), max_ctx = atoi(argv[8]);
  const float eps = (float)atof(argv[9]), scale = (float)atof(argv[11]);
  const double theta = atof(argv[10]);
  const size_t D = 128, qrow = (size_t)hq * D, kvrow = (size_t)hkv * D;

  HIP(hipSetDevice(0));
  pgqa_pool_config cfg = {nb, bs, hkv, 128, 0};
  const size_t pool_bytes = pgqa_pool_bytes(&cfg);
  if (pool_bytes == 0) { fprintf(stderr, "bad pool config\n"); return 3; }
  void* storage = NULL;
  HIP(hipMalloc(&storage, pool_bytes));
  pgqa_pool* pool = NULL;
  PGQA(pgqa_pool_create(&cfg, storage, &pool));

  /* the prefix, placed element by element through the reported strides */
  int64_t ks[4], vs[5], ko, vo;
  PGQA(pgqa_pool_layout(pool, ks, &ko, vs, &vo));
  const size_t cache_elems = (size_t)nb * bs * hkv * D;
  uint16_t* pk = read_file("prefix_k.bin", cache_elems * 2);
  uint16_t* pv = read_file("prefix_v.bin", cache_elems * 2);
  uint16_t* host_pool = calloc(pool_bytes / 2, 2);
  for (int32_t b = 0; b < nb; ++b)
    for (int32_t s = 0; s < bs; ++s)
      for (int32_t h = 0; h < hkv; ++h)
        for (size_t d = 0; d < D; ++d) {
          const size_t i = (((size_t)b * bs + s) * hkv + h) * D + d;
          host_pool[ko + b * ks[0] + s * ks[1] + h * ks[2] + d * ks[3]] = pk[i];
          host_pool[vo + b * vs[0] + (s / 16) * vs[1] + (s % 16) * vs[2] + h * vs[3] + d * vs[4]] = pv[i];
        }
  HIP(hipMemcpy(storage, host_pool, pool_bytes, hipMemcpyHostToDevice));

  void* q = read_file("q.bin", B * qrow * 2);
  void* k = read_file("k.bin", B * kvrow * 2);
  void* v = read_file("v.bin", B * kvrow * 2);
  void* wq = read_file("wq.bin", D * 2);
  void* wk = read_file("wk.bin", D * 2);
  void* ctx = read_file("ctx.bin", (size_t)B * 4);
  void* bt = read_file("bt.bin", (size_t)B * bt_stride * 4);
  void *dq = to_device(q, B * qrow * 2), *dk = to_device(k, B * kvrow * 2), *dv = to_device(v, B * kvrow * 2);
  void *dwq = to_device(wq, D * 2), *dwk = to_device(wk, D * 2);
  void *dctx = to_device(ctx, (size_t)B * 4), *dbt = to_device(bt, (size_t)B * bt_stride * 4);
  void *dout = to_device(NULL, B * qrow * 2), *dqo = to_device(NULL, B * qrow * 2);

  int cus = 0;
  HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  pgqa_decode_plan plan;
  PGQA(pgqa_plan_decode(cus, bs, B, hkv, hq, max_ctx, &plan));
  const size_t ws_bytes = pgqa_decode_workspace_bytes(pool, B, hq, max_ctx, &plan);
  void* ws = ws_bytes ? to_device(NULL, ws_bytes) : NULL;
  PGQA(pgqa_decode_step(pool, dq, (int64_t)qrow, dk, (int64_t)kvrow, dv, (int64_t)kvrow, dwq, dwk, eps, theta,
                        (const int32_t*)dctx, (const int32_t*)dbt, bt_stride, B, hq, max_ctx, scale, &plan, ws,
                        ws_bytes, dqo, dout, NULL));
  uint32_t flags = 0;
  PGQA(pgqa_pool_check_errors(pool, NULL, &flags));

  void* out = malloc(B * qrow * 2);
  void* q_out = malloc(B * qrow * 2);
  HIP(hipMemcpy(out, dout, B * qrow * 2, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(q_out, dqo, B * qrow * 2, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(host_pool, storage, pool_bytes, hipMemcpyDeviceToHost));
  write_file("out.bin", out, B * qrow * 2);
  write_file("q_out.bin", q_out, B * qrow * 2);
  write_file("pool.bin", host_pool, pool_bytes);
  char layout[512];
  const int n = snprintf(layout, sizeof layout, "%lld %lld %lld %lld %lld\n%lld %lld %lld %lld %lld %lld\n",
                         (long long)ks[0], (long long)ks[1], (long long)ks[2], (long long)ks[3], (long long)ko,
                         (long long)vs[0], (long long)vs[1], (long long)vs[2], (long long)vs[3], (long long)vs[4],
                         (long long)vo);
  write_file("layout.txt", layout, (size_t)n);

  PGQA(pgqa_pool_destroy(pool));
  HIP(hipFree(storage));
  printf("c_decode_step: batch %d, plan %d x %d, flags %u\n", B, plan.split_tokens, plan.max_splits, flags);
  return 0;
}
