// C ABI of libpgqa: argument validation, pointer-kind checks, the decode split
// planner and kernel launches.  No call here synchronises the device or copies
// device data to the host, except pgqa_pool_check_errors and pool set-up.
//
// Page "[2026春季][T2-1-3]" (InfiniLM issue 498), Review notes: the host checks
// that a buffer it is about to read really is host memory; here every pointer
// is checked to be device memory of the pool's device before anything is
// enqueued.  Page "perf: Qwen3 offline inference - ...", Summary item 3:
// routing decisions are made on the host with no device synchronisation; the
// split plan below uses host-known sizes and the CU count only.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "../../include/pgqa.h"
#include "errors.hpp"
#include "launch.hpp"

using namespace pgqa;

static_assert(kNoAllocScratchBytes == PGQA_NOALLOC_SCRATCH_BYTES, "fixed decode scratch size");
static_assert(kMixedItemInts == PGQA_MIXED_ITEM_INTS, "mixed work item size");

struct pgqa_pool {
  pgqa_pool_config cfg;
  PoolGeom geom;
  int device;
  int num_cus;
  // Rotary turn frequencies of the last rope_theta seen (host, fp64).
  std::mutex rope_mu;
  double rope_theta = 0.0;
  double rev_freq[64];
};

namespace {

pgqa_status hip_fail(hipError_t e, const char* what) {
  return fail(PGQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool valid_block_size(int32_t bs) { return bs == 16 || bs == 32 || bs == 64 || bs == 128 || bs == 256; }

// Device memory of `device`?  hipPointerGetAttributes is a host-side lookup (no sync).
pgqa_status check_device_ptr(const void* p, int device, const char* name, size_t align = 2) {
  if (p == nullptr) return fail(PGQA_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    return fail(PGQA_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  hipPointerAttribute_t at;
  hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PGQA_ERR_POINTER_KIND, "%s is not HIP device memory (%s)", name, hipGetErrorString(e));
  }
  if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged)
    return fail(PGQA_ERR_POINTER_KIND, "%s is host memory, device memory is required", name);
  if (at.device != device)
    return fail(PGQA_ERR_POINTER_KIND, "%s lives on device %d, the pool on device %d", name, at.device, device);
  return PGQA_OK;
}

#define PGQA_TRY(expr)                 \
  do {                                 \
    pgqa_status s_ = (expr);           \
    if (s_ != PGQA_OK) return s_;      \
  } while (0)

pgqa_status check_pool(const pgqa_pool* pool) {
  if (pool == nullptr) return fail(PGQA_ERR_INVALID_ARG, "pool is NULL");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != pool->device)
    return fail(PGQA_ERR_INVALID_ARG, "current device %d is not the pool's device %d", dev, pool->device);
  return PGQA_OK;
}

pgqa_status check_group(const pgqa_pool* pool, int32_t num_q_heads) {
  const int32_t hkv = pool->cfg.num_kv_heads;
  if (num_q_heads <= 0 || num_q_heads % hkv != 0)
    return fail(PGQA_ERR_INVALID_ARG, "num_q_heads=%d is not a positive multiple of num_kv_heads=%d", num_q_heads,
                hkv);
  const int32_t r = num_q_heads / hkv;
  if (r != 1 && r != 2 && r != 4 && r != 8)
    return fail(PGQA_ERR_UNSUPPORTED, "query heads per kv head = %d (supported: 1, 2, 4, 8)", r);
  return PGQA_OK;
}

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

constexpr int32_t kMaxSplitTokens = 4096;
constexpr int32_t kChunkStep = 32;  // chunk splits are whole 32-key steps
// Decode K/V loads are non-temporal (streaming) by default: K/V bytes are read
// once per launch, and V^T is stored in 16-slot pieces, so every 16-key tile
// load covers whole 128-byte lines at every block size.

pgqa_status validate_plan(const pgqa_decode_plan& p, int32_t block_size, int32_t max_context_len) {
  const int32_t gran = block_size > 64 ? block_size : 64;
  if (p.split_tokens <= 0 || p.split_tokens % gran != 0 || p.split_tokens > kMaxSplitTokens)
    return fail(PGQA_ERR_INVALID_ARG, "plan.split_tokens=%d must be a positive multiple of %d, at most %d",
                p.split_tokens, gran, kMaxSplitTokens);
  if (p.waves_per_split != 1 && p.waves_per_split != 2 && p.waves_per_split != 4 && p.waves_per_split != 8)
    return fail(PGQA_ERR_INVALID_ARG, "plan.waves_per_split=%d (1, 2, 4 or 8)", p.waves_per_split);
  if (p.split_tokens > 1024 * p.waves_per_split)
    return fail(PGQA_ERR_INVALID_ARG, "plan.split_tokens=%d exceeds 1024 keys per wave (%d waves)", p.split_tokens,
                p.waves_per_split);
  if (p.load_hint < 0 || p.load_hint > 2) return fail(PGQA_ERR_INVALID_ARG, "plan.load_hint=%d", p.load_hint);
  if (p.kernel < 0 || p.kernel > 2) return fail(PGQA_ERR_INVALID_ARG, "plan.kernel=%d (0, 1 or 2)", p.kernel);
  const int64_t need = (int64_t(max_context_len) + p.split_tokens - 1) / p.split_tokens;
  if (p.max_splits < need || p.max_splits > 65535)
    return fail(PGQA_ERR_INVALID_ARG, "plan.max_splits=%d does not cover max_context_len=%d", p.max_splits,
                max_context_len);
  return PGQA_OK;
}

// Split kernel of a decode plan with kernel = 0, by query heads per kv head.
// The dot-product kernel's VALU work per key grows with r while its bytes per
// key do not.  Measured on MI355X at r = 8 the matrix-core kernel is 24-32%
// faster (Qwen3-30B-A3B batch-64 step 29.8 -> 22.9 us; batch 1 at 32k keys
// 35.8 -> 24.4; batch 8 at up to 4k keys 20.9 -> 16.0); at r <= 4 the two are
// within a few percent and the dot-product kernel is ahead on the large
// batches, which stream at close to the memory system's rate.
int32_t default_decode_kernel(int32_t r) { return r >= 8 ? 2 : 1; }

// Keys per split of the decode planner (see pgqa_plan_decode) for `units`
// (sequence, kv head) pairs of at most ctx keys: one split when that gives at
// least half a workgroup per CU, else about one workgroup per CU with a floor
// on the split length (below 16k keys: 384, or 512 for the matrix-core
// kernel; from 16k keys: 1536, or 768 for the matrix-core kernel); a multiple
// of max(block_size, 64), at most 1024 keys per wave.  Measured on MI355X:
// batch 1 at 8k keys (r = 2) 13.2 us at 384-key splits, 16 us and more at
// 1024; batch 1 at 32k keys 27.0 us at 1536 (r = 2), 22.3 us at 768 (r = 8).
int64_t decode_split(int32_t num_cus, int32_t block_size, int64_t units, int64_t ctx, bool mfma, int32_t waves) {
  const int64_t gran = block_size > 64 ? block_size : 64;
  const int64_t max_split = std::min<int64_t>(1024ll * waves, kMaxSplitTokens);
  int64_t split;
  if (2 * units >= num_cus) {
    split = round_up(ctx, gran);
  } else {
    const int64_t want = (num_cus + units - 1) / units;
    split = round_up((ctx + want - 1) / want, gran);
    const int64_t floor_split = round_up(ctx >= 16384 ? (mfma ? 768 : 1536) : (mfma ? 512 : 384), gran);
    if (split < floor_split) split = floor_split;
    if (split > round_up(ctx, gran)) split = round_up(ctx, gran);
  }
  if (split > max_split) {
    const int64_t parts = (ctx + max_split - 1) / max_split;
    split = std::min(round_up((ctx + parts - 1) / parts, gran), max_split / gran * gran);
  }
  return split;
}

// Rotary turn frequencies of rope_theta (host fp64), cached in the pool.
void rope_table(pgqa_pool* pool, double rope_theta, double (&out)[64]) {
  std::lock_guard<std::mutex> lock(pool->rope_mu);
  if (pool->rope_theta != rope_theta) {
    for (int i = 0; i < 64; ++i) pool->rev_freq[i] = std::pow(rope_theta, -2.0 * i / 128.0) / (2.0 * M_PI);
    pool->rope_theta = rope_theta;
  }
  std::memcpy(out, pool->rev_freq, sizeof(out));
}

}  // namespace

extern "C" {

const char* pgqa_version(void) { return "0.1.0"; }

pgqa_status pgqa_stream_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, int32_t grid,
                             void* stream) {
  clear_error();
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PGQA_ERR_HIP, "no current HIP device");
  if (bytes == 0 || bytes % 16 != 0) return fail(PGQA_ERR_INVALID_ARG, "bytes=%zu (a positive multiple of 16)", bytes);
  if (grid == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return fail(PGQA_ERR_HIP, "cannot read the CU count");
    grid = 3 * cus;
  }
  if (grid < 1 || grid > 65535) return fail(PGQA_ERR_INVALID_ARG, "grid=%d", grid);
  if (sink_bytes < size_t(grid) * 256 * 4)
    return fail(PGQA_ERR_INVALID_ARG, "sink of %zu bytes, %zu needed", sink_bytes, size_t(grid) * 256 * 4);
  PGQA_TRY(check_device_ptr(src, dev, "src", 16));
  PGQA_TRY(check_device_ptr(sink, dev, "sink", 4));
  const hipError_t e = pgqa::launch_stream_read(src, int64_t(bytes / 16), sink, grid, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PGQA_ERR_HIP, "stream read launch: %s", hipGetErrorString(e));
  return PGQA_OK;
}

const char* pgqa_last_error(void) { return pgqa::last_error(); }

const char* pgqa_status_string(pgqa_status s) {
  switch (s) {
    case PGQA_OK: return "ok";
    case PGQA_ERR_INVALID_ARG: return "invalid argument";
    case PGQA_ERR_UNSUPPORTED: return "unsupported shape";
    case PGQA_ERR_POINTER_KIND: return "pointer is not device memory of the pool's device";
    case PGQA_ERR_WORKSPACE: return "workspace missing or too small";
    case PGQA_ERR_HIP: return "HIP runtime error";
    case PGQA_ERR_DEVICE: return "kernel-detected metadata error";
  }
  return "unknown status";
}

size_t pgqa_pool_bytes(const pgqa_pool_config* cfg) {
  if (cfg == nullptr || cfg->num_blocks <= 0 || cfg->num_kv_heads <= 0 || !valid_block_size(cfg->block_size) ||
      cfg->head_dim != 128)
    return 0;
  return size_t(cfg->num_blocks) * cfg->num_kv_heads * 2 * cfg->block_size * cfg->head_dim * sizeof(uint16_t);
}

pgqa_status pgqa_pool_create(const pgqa_pool_config* cfg, void* kv_storage, pgqa_pool** out) {
  clear_error();
  if (out == nullptr) return fail(PGQA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (cfg == nullptr) return fail(PGQA_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->num_blocks <= 0) return fail(PGQA_ERR_INVALID_ARG, "num_blocks=%d", cfg->num_blocks);
  if (cfg->num_kv_heads <= 0) return fail(PGQA_ERR_INVALID_ARG, "num_kv_heads=%d", cfg->num_kv_heads);
  if (cfg->max_batch_size < 0) return fail(PGQA_ERR_INVALID_ARG, "max_batch_size=%d", cfg->max_batch_size);
  if (cfg->head_dim != 128) return fail(PGQA_ERR_UNSUPPORTED, "head_dim=%d (only 128)", cfg->head_dim);
  if (!valid_block_size(cfg->block_size))
    return fail(PGQA_ERR_UNSUPPORTED, "block_size=%d (16, 32, 64, 128 or 256)", cfg->block_size);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  PGQA_TRY(check_device_ptr(kv_storage, dev, "kv_storage", 256));
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
  uint32_t* err = nullptr;
  e = hipMalloc(reinterpret_cast<void**>(&err), 256);
  if (e != hipSuccess) return hip_fail(e, "hipMalloc(error word)");
  e = hipMemset(err, 0, 256);
  if (e != hipSuccess) {
    (void)hipFree(err);
    return hip_fail(e, "hipMemset(error word)");
  }
  pgqa_pool* p = new (std::nothrow) pgqa_pool;
  if (p == nullptr) {
    (void)hipFree(err);
    return fail(PGQA_ERR_INVALID_ARG, "out of host memory");
  }
  p->cfg = *cfg;
  p->geom.kv = static_cast<uint16_t*>(kv_storage);
  p->geom.num_blocks = cfg->num_blocks;
  p->geom.block_size = cfg->block_size;
  p->geom.num_kv_heads = cfg->num_kv_heads;
  p->geom.err = err;
  p->device = dev;
  p->num_cus = cus;
  *out = p;
  return PGQA_OK;
}

pgqa_status pgqa_pool_destroy(pgqa_pool* pool) {
  if (pool == nullptr) return PGQA_OK;
  int prev = -1;
  (void)hipGetDevice(&prev);
  (void)hipSetDevice(pool->device);
  hipError_t e = hipFree(pool->geom.err);
  if (prev >= 0) (void)hipSetDevice(prev);
  delete pool;
  if (e != hipSuccess) return hip_fail(e, "hipFree(error word)");
  return PGQA_OK;
}

pgqa_status pgqa_pool_layout(const pgqa_pool* pool, int64_t k_strides[4], int64_t* k_offset, int64_t v_strides[5],
                             int64_t* v_offset) {
  if (pool == nullptr || k_strides == nullptr || k_offset == nullptr || v_strides == nullptr || v_offset == nullptr)
    return fail(PGQA_ERR_INVALID_ARG, "NULL argument");
  const int64_t bs = pool->cfg.block_size, D = 128, hkv = pool->cfg.num_kv_heads;
  const int64_t tile = 2 * bs * D;
  // order (block, slot, head, dim)
  k_strides[0] = tile * hkv;
  k_strides[1] = D;
  k_strides[2] = tile;
  k_strides[3] = 1;
  *k_offset = 0;
  // order (block, slot / 16, slot % 16, head, dim): V^T in 16-slot pieces
  v_strides[0] = tile * hkv;
  v_strides[1] = 16 * D;
  v_strides[2] = 1;
  v_strides[3] = tile;
  v_strides[4] = 16;
  *v_offset = bs * D;
  return PGQA_OK;
}

pgqa_status pgqa_pool_check_errors(pgqa_pool* pool, void* stream, uint32_t* flags) {
  PGQA_TRY(check_pool(pool));
  if (flags == nullptr) return fail(PGQA_ERR_INVALID_ARG, "flags is NULL");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
  uint32_t v = 0;
  e = hipMemcpy(&v, pool->geom.err, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "hipMemcpy(error word)");
  e = hipMemset(pool->geom.err, 0, sizeof(v));
  if (e != hipSuccess) return hip_fail(e, "hipMemset(error word)");
  *flags = v;
  if (v != 0) return fail(PGQA_ERR_DEVICE, "device metadata errors 0x%x", v);
  return PGQA_OK;
}

pgqa_status pgqa_rms_norm_rope_cache_write(pgqa_pool* pool, const void* q, int64_t q_row_stride, const void* k,
                                           int64_t k_row_stride, const void* v, int64_t v_row_stride,
                                           const void* q_norm_weight, const void* k_norm_weight,
                                           const int32_t* positions, const int32_t* seq_ids,
                                           const int32_t* block_tables, int32_t bt_stride, int32_t num_seqs,
                                           int32_t num_tokens, int32_t num_q_heads, float eps, double rope_theta,
                                           void* q_out, void* stream) {
  clear_error();
  PGQA_TRY(check_pool(pool));
  PGQA_TRY(check_group(pool, num_q_heads));
  const int64_t hkv = pool->cfg.num_kv_heads;
  if (num_tokens < 0) return fail(PGQA_ERR_INVALID_ARG, "num_tokens=%d", num_tokens);
  if (bt_stride <= 0 || num_seqs <= 0)
    return fail(PGQA_ERR_INVALID_ARG, "bt_stride=%d num_seqs=%d", bt_stride, num_seqs);
  if (pool->cfg.max_batch_size > 0 && num_seqs > pool->cfg.max_batch_size)
    return fail(PGQA_ERR_INVALID_ARG, "num_seqs=%d exceeds max_batch_size=%d", num_seqs, pool->cfg.max_batch_size);
  if (q_row_stride < int64_t(num_q_heads) * 128 || k_row_stride < hkv * 128 || v_row_stride < hkv * 128)
    return fail(PGQA_ERR_INVALID_ARG, "row strides (%lld, %lld, %lld) below the dense row length",
                (long long)q_row_stride, (long long)k_row_stride, (long long)v_row_stride);
  if (q_row_stride % 8 || k_row_stride % 8 || v_row_stride % 8)
    return fail(PGQA_ERR_INVALID_ARG, "row strides must be multiples of 8 elements");
  if (num_q_heads + 2 * hkv > 128)
    return fail(PGQA_ERR_UNSUPPORTED, "num_q_heads + 2 * num_kv_heads = %lld (at most 128)",
                (long long)(num_q_heads + 2 * hkv));
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(PGQA_ERR_INVALID_ARG, "eps=%g", double(eps));
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
    return fail(PGQA_ERR_INVALID_ARG, "rope_theta=%g", rope_theta);
  if (num_tokens == 0) return PGQA_OK;
  const int dev = pool->device;
  PGQA_TRY(check_device_ptr(q, dev, "q", 16));
  PGQA_TRY(check_device_ptr(k, dev, "k", 16));
  PGQA_TRY(check_device_ptr(v, dev, "v", 16));
  PGQA_TRY(check_device_ptr(q_norm_weight, dev, "q_norm_weight", 16));
  PGQA_TRY(check_device_ptr(k_norm_weight, dev, "k_norm_weight", 16));
  PGQA_TRY(check_device_ptr(positions, dev, "positions", 4));
  PGQA_TRY(check_device_ptr(seq_ids, dev, "seq_ids", 4));
  PGQA_TRY(check_device_ptr(block_tables, dev, "block_tables", 4));
  PGQA_TRY(check_device_ptr(q_out, dev, "q_out", 16));
  WriteArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.q_stride = q_row_stride;
  a.k = static_cast<const uint16_t*>(k);
  a.k_stride = k_row_stride;
  a.v = static_cast<const uint16_t*>(v);
  a.v_stride = v_row_stride;
  a.wq = static_cast<const uint16_t*>(q_norm_weight);
  a.wk = static_cast<const uint16_t*>(k_norm_weight);
  a.pos = positions;
  a.seq = seq_ids;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.eps = eps;
  rope_table(pool, rope_theta, a.rev_freq);
  a.q_out = static_cast<uint16_t*>(q_out);
  hipError_t e = launch_cache_write(pool->geom, a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cache write launch");
  return PGQA_OK;
}

pgqa_status pgqa_plan_decode(int32_t num_cus, int32_t block_size, int32_t batch, int32_t num_kv_heads,
                             int32_t num_q_heads, int32_t max_context_len, pgqa_decode_plan* out) {
  if (out == nullptr) return fail(PGQA_ERR_INVALID_ARG, "out is NULL");
  if (num_cus <= 0 || !valid_block_size(block_size) || batch < 0 || num_kv_heads <= 0 || num_q_heads <= 0 ||
      max_context_len < 0)
    return fail(PGQA_ERR_INVALID_ARG, "invalid planner input");
  // Measured on MI355X (decode sweeps over the five Qwen3 workloads): each
  // workgroup pays a few microseconds of dependent-load latency before its
  // first K/V tile arrives, so long splits win over many short ones.
  //  * one split per (sequence, kv head) when that already gives at least half
  //    a workgroup per CU (no partials, no combine launch);
  //  * otherwise about one workgroup per CU, with a floor on the split
  //    length (decode_split: 384 keys, 1536 from 16k keys; the batch-1
  //    32k-key step is fastest at 1536-key splits, 176 workgroups, 6% ahead
  //    of 2048);
  //  * 4 waves per workgroup;
  //  * the matrix-core kernel (8 query heads per kv head) was fastest with
  //    512-key splits below 16k keys and 768 from 16k keys.
  const int32_t r = num_q_heads / num_kv_heads;
  const int32_t kernel = default_decode_kernel(r);
  const int32_t waves = 4;
  const int64_t ctx = max_context_len > 0 ? max_context_len : 1;
  const int64_t split = decode_split(num_cus, block_size, int64_t(batch > 0 ? batch : 1) * num_kv_heads, ctx,
                                     kernel == 2, waves);
  out->split_tokens = int32_t(split);
  out->max_splits = int32_t((ctx + split - 1) / split);
  out->waves_per_split = waves;
  out->load_hint = 0;
  out->kernel = kernel;
  out->host_context_lens = nullptr;
  return PGQA_OK;
}

size_t pgqa_decode_workspace_bytes(const pgqa_pool* pool, int32_t batch, int32_t num_q_heads,
                                   int32_t max_context_len, const pgqa_decode_plan* plan) {
  if (pool == nullptr || batch < 0 || num_q_heads <= 0 || num_q_heads % pool->cfg.num_kv_heads != 0) return 0;
  pgqa_decode_plan p;
  if (plan != nullptr) {
    p = *plan;
  } else if (pgqa_plan_decode(pool->num_cus, pool->cfg.block_size, batch, pool->cfg.num_kv_heads, num_q_heads,
                              max_context_len, &p) != PGQA_OK) {
    return 0;
  }
  return decode_workspace_layout(batch, pool->cfg.num_kv_heads, num_q_heads / pool->cfg.num_kv_heads, p.max_splits)
      .total;
}

namespace {

// Shared by the plain decode call and the fused decode step (st != nullptr).
pgqa_status decode_common(pgqa_pool* pool, const void* q, int64_t q_row_stride, const int32_t* context_lens,
                          const int32_t* block_tables, int32_t bt_stride, int32_t batch, int32_t num_q_heads,
                          int32_t max_context_len, float scale, const pgqa_decode_plan* plan, void* workspace,
                          size_t workspace_bytes, void* out, void* stream, const StepArgs* st,
                          bool static_scratch = false) {
  PGQA_TRY(check_pool(pool));
  PGQA_TRY(check_group(pool, num_q_heads));
  if (batch < 0 || batch > 65535) return fail(PGQA_ERR_INVALID_ARG, "batch=%d", batch);
  if (pool->cfg.max_batch_size > 0 && batch > pool->cfg.max_batch_size)
    return fail(PGQA_ERR_INVALID_ARG, "batch=%d exceeds max_batch_size=%d", batch, pool->cfg.max_batch_size);
  if (bt_stride <= 0) return fail(PGQA_ERR_INVALID_ARG, "bt_stride=%d", bt_stride);
  if (max_context_len < 0) return fail(PGQA_ERR_INVALID_ARG, "max_context_len=%d", max_context_len);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PGQA_ERR_INVALID_ARG, "scale=%g", double(scale));
  if (q_row_stride < int64_t(num_q_heads) * 128 || q_row_stride % 8)
    return fail(PGQA_ERR_INVALID_ARG, "q row stride %lld (at least num_q_heads * 128, a multiple of 8)",
                (long long)q_row_stride);
  if (batch == 0) return PGQA_OK;
  pgqa_decode_plan p;
  if (plan != nullptr) {
    p = *plan;
  } else {
    PGQA_TRY(pgqa_plan_decode(pool->num_cus, pool->cfg.block_size, batch, pool->cfg.num_kv_heads, num_q_heads,
                              max_context_len, &p));
  }
  PGQA_TRY(validate_plan(p, pool->cfg.block_size, max_context_len));
  const int32_t r = num_q_heads / pool->cfg.num_kv_heads;
  const DecodeWorkspace wl = decode_workspace_layout(batch, pool->cfg.num_kv_heads, r, p.max_splits);
  const int dev = pool->device;
  PGQA_TRY(check_device_ptr(q, dev, "q", 16));
  PGQA_TRY(check_device_ptr(context_lens, dev, "context_lens", 4));
  PGQA_TRY(check_device_ptr(block_tables, dev, "block_tables", 4));
  PGQA_TRY(check_device_ptr(out, dev, "out"));
  if (static_scratch) {
    if (wl.total > workspace_bytes)
      return fail(PGQA_ERR_WORKSPACE,
                  "the split partials of this plan need %zu bytes, more than the %zu-byte fixed scratch of the "
                  "allocation-free decode step (use a plan with fewer splits or pgqa_decode_step with a workspace)",
                  wl.total, workspace_bytes);
  } else if (wl.total > 0) {
    if (workspace == nullptr || workspace_bytes < wl.total)
      return fail(PGQA_ERR_WORKSPACE, "decode workspace of %zu bytes needed, %zu given", wl.total,
                  workspace == nullptr ? size_t(0) : workspace_bytes);
    PGQA_TRY(check_device_ptr(workspace, dev, "workspace", 256));
  }
  DecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.q_stride = q_row_stride;
  a.ctx = context_lens;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.max_ctx = max_context_len;
  a.qk_scale_log2 = float(double(scale) * 1.4426950408889634);
  a.split_tokens = p.split_tokens;
  a.max_splits = p.max_splits;
  a.waves = p.waves_per_split;
  a.mfma = (p.kernel == 0 ? default_decode_kernel(r) : p.kernel) == 2;
  // load_hint 0: streaming loads in the dot-product kernel (whole lines, read
  // once), cached loads in the matrix-core kernel (each K line is read by two
  // load instructions; measured faster cached at every workload).
  a.stream_loads = p.load_hint == 2 || (p.load_hint == 0 && !a.mfma);
  char* ws = wl.total > 0 ? static_cast<char*>(workspace) : nullptr;
  a.part_o = ws ? reinterpret_cast<float*>(ws + wl.part_o_off) : nullptr;
  a.part_lse = ws ? reinterpret_cast<float*>(ws + wl.part_lse_off) : nullptr;
  a.out = static_cast<uint16_t*>(out);
  // Host-side lengths: order the units so that the workgroups sharing a CU
  // carry long and short units together.  Workgroups are dealt to the CUs in
  // linear order, those num_cus apart landing on the same CU, so the units go
  // longest first in a snake: rank k to position (k / C) C + j, j = k % C on
  // even rounds and C - 1 - (k % C) on odd ones (C = CUs).
  UnitOrder ord;
  ord.count = 0;
  const int64_t units = int64_t(batch) * pool->cfg.num_kv_heads;
  if (p.host_context_lens != nullptr && units <= kMaxOrderedUnits) {
    const int32_t* hl = p.host_context_lens;
    const int32_t hkv = pool->cfg.num_kv_heads;
    int32_t rank[kMaxOrderedUnits];
    for (int32_t u = 0; u < int32_t(units); ++u) rank[u] = u;
    std::stable_sort(rank, rank + units, [&](int32_t x, int32_t y) { return hl[x / hkv] > hl[y / hkv]; });
    const int64_t C = std::max<int64_t>(1, pool->num_cus);
    for (int64_t k = 0; k < units; ++k) {
      const int64_t round = k / C, j = k % C, rem = std::min<int64_t>(C, units - round * C);
      ord.unit[round * C + ((round & 1) ? rem - 1 - j : j)] = uint16_t(rank[k]);
    }
    ord.count = int32_t(units);
  }
  hipError_t e = launch_decode(pool->geom, a, st, ord.count > 0 ? &ord : nullptr, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return PGQA_OK;
}

}  // namespace

pgqa_status pgqa_paged_decode_attention(pgqa_pool* pool, const void* q, const int32_t* context_lens,
                                        const int32_t* block_tables, int32_t bt_stride, int32_t batch,
                                        int32_t num_q_heads, int32_t max_context_len, float scale,
                                        const pgqa_decode_plan* plan, void* workspace, size_t workspace_bytes,
                                        void* out, void* stream) {
  clear_error();
  PGQA_TRY(check_pool(pool));
  return decode_common(pool, q, int64_t(num_q_heads) * 128, context_lens, block_tables, bt_stride, batch,
                       num_q_heads, max_context_len, scale, plan, workspace, workspace_bytes, out, stream, nullptr);
}

namespace {

pgqa_status decode_step_common(pgqa_pool* pool, const void* q, int64_t q_row_stride, const void* k,
                               int64_t k_row_stride, const void* v, int64_t v_row_stride, const void* q_norm_weight,
                               const void* k_norm_weight, float eps, double rope_theta, const int32_t* context_lens,
                               const int32_t* block_tables, int32_t bt_stride, int32_t batch, int32_t num_q_heads,
                               int32_t max_context_len, float scale, const pgqa_decode_plan* plan, void* workspace,
                               size_t workspace_bytes, void* q_out, void* out, void* stream, bool static_scratch) {
  PGQA_TRY(check_pool(pool));
  PGQA_TRY(check_group(pool, num_q_heads));
  const int64_t hkv = pool->cfg.num_kv_heads;
  if (k_row_stride < hkv * 128 || v_row_stride < hkv * 128 || k_row_stride % 8 || v_row_stride % 8)
    return fail(PGQA_ERR_INVALID_ARG, "k/v row strides (%lld, %lld): at least num_kv_heads * 128, multiples of 8",
                (long long)k_row_stride, (long long)v_row_stride);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(PGQA_ERR_INVALID_ARG, "eps=%g", double(eps));
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
    return fail(PGQA_ERR_INVALID_ARG, "rope_theta=%g", rope_theta);
  if (batch > 0) {
    const int dev = pool->device;
    PGQA_TRY(check_device_ptr(k, dev, "k", 16));
    PGQA_TRY(check_device_ptr(v, dev, "v", 16));
    PGQA_TRY(check_device_ptr(q_norm_weight, dev, "q_norm_weight", 16));
    PGQA_TRY(check_device_ptr(k_norm_weight, dev, "k_norm_weight", 16));
    if (q_out != nullptr) PGQA_TRY(check_device_ptr(q_out, dev, "q_out", 16));
  }
  StepArgs st;
  st.k = static_cast<const uint16_t*>(k);
  st.k_stride = k_row_stride;
  st.v = static_cast<const uint16_t*>(v);
  st.v_stride = v_row_stride;
  st.wq = static_cast<const uint16_t*>(q_norm_weight);
  st.wk = static_cast<const uint16_t*>(k_norm_weight);
  st.eps = eps;
  st.q_out = static_cast<uint16_t*>(q_out);
  rope_table(pool, rope_theta, st.rev_freq);
  return decode_common(pool, q, q_row_stride, context_lens, block_tables, bt_stride, batch, num_q_heads,
                       max_context_len, scale, plan, workspace, workspace_bytes, out, stream, &st, static_scratch);
}

}  // namespace

pgqa_status pgqa_decode_step(pgqa_pool* pool, const void* q, int64_t q_row_stride, const void* k,
                             int64_t k_row_stride, const void* v, int64_t v_row_stride, const void* q_norm_weight,
                             const void* k_norm_weight, float eps, double rope_theta, const int32_t* context_lens,
                             const int32_t* block_tables, int32_t bt_stride, int32_t batch, int32_t num_q_heads,
                             int32_t max_context_len, float scale, const pgqa_decode_plan* plan, void* workspace,
                             size_t workspace_bytes, void* q_out, void* out, void* stream) {
  clear_error();
  return decode_step_common(pool, q, q_row_stride, k, k_row_stride, v, v_row_stride, q_norm_weight, k_norm_weight,
                            eps, rope_theta, context_lens, block_tables, bt_stride, batch, num_q_heads,
                            max_context_len, scale, plan, workspace, workspace_bytes, q_out, out, stream, false);
}

pgqa_status pgqa_decode_step_noalloc(pgqa_pool* pool, const void* q, int64_t q_row_stride, const void* k,
                                     int64_t k_row_stride, const void* v, int64_t v_row_stride,
                                     const void* q_norm_weight, const void* k_norm_weight, float eps,
                                     double rope_theta, const int32_t* context_lens, const int32_t* block_tables,
                                     int32_t bt_stride, int32_t batch, int32_t num_q_heads, int32_t max_context_len,
                                     float scale, const pgqa_decode_plan* plan, void* q_out, void* out,
                                     void* stream) {
  clear_error();
  PGQA_TRY(check_pool(pool));
  // The fixed scratch of this device (its address is looked up once per device).
  void* scratch = nullptr;
  const hipError_t e = noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "address of the fixed decode scratch");
  return decode_step_common(pool, q, q_row_stride, k, k_row_stride, v, v_row_stride, q_norm_weight, k_norm_weight,
                            eps, rope_theta, context_lens, block_tables, bt_stride, batch, num_q_heads,
                            max_context_len, scale, plan, scratch, kNoAllocScratchBytes, q_out, out, stream, true);
}

pgqa_status pgqa_plan_chunk(int32_t num_cus, int32_t block_size, int32_t num_segments, int32_t total_q,
                            int32_t num_kv_heads, int32_t num_q_heads, int32_t max_q_len,
                            int32_t max_context_len, pgqa_chunk_plan* out) {
  if (out == nullptr) return fail(PGQA_ERR_INVALID_ARG, "out is NULL");
  if (num_cus <= 0 || !valid_block_size(block_size) || num_segments < 0 || total_q < 0 || num_kv_heads <= 0 ||
      num_q_heads <= 0 || max_q_len < 0 || max_context_len < 0)
    return fail(PGQA_ERR_INVALID_ARG, "invalid planner input");
  // Wide items (segments of more than 32 rows per kv head) are 128 query rows
  // (4 waves) of one kv head over one key split: aim at two per CU over the
  // (row group, kv head) units the hints allow, splits of 256 .. 4096 keys.
  // Short items are one wave over one key split of a short segment.
  const int64_t r = num_q_heads / num_kv_heads;
  const int64_t ctx = max_context_len > 0 ? max_context_len : 1;
  const int64_t cap = std::min<int64_t>(round_up(ctx, kChunkStep), kMaxSplitTokens);
  auto pick = [&](int64_t units, int64_t per_cu, int64_t floor_keys) {
    const int64_t want = (per_cu * num_cus + units - 1) / units;
    int64_t split = round_up((ctx + want - 1) / want, kChunkStep);
    split = std::max(split, floor_keys);
    return std::min(split, cap);
  };
  if (int64_t(max_q_len) * r <= 16) {
    // every segment fits the 16 columns of the matrix-core decode kernel
    // (verify rows, single tokens): one workgroup per (kv head, segment,
    // split), splits as the decode planner makes them for that kernel
    const int64_t split = decode_split(num_cus, block_size, int64_t(std::max(num_segments, 1)) * num_kv_heads, ctx,
                                       true, 4);
    out->split_tokens = out->short_split_tokens = int32_t(split);
    out->max_splits = int32_t((ctx + split - 1) / split);
    out->kernel = 2;
    return PGQA_OK;
  }
  const ChunkLists lists = chunk_lists(num_segments, total_q, int32_t(r), max_q_len);
  const int64_t wide_groups = (int64_t(total_q) * r + 127) / 128;
  const int64_t wide = pick(std::max<int64_t>(wide_groups, 1) * num_kv_heads, 2, 256);
  // Short splits: 256 keys (8 steps) unless that would list more than 16 items
  // per CU, then as many keys as keep it at 16.
  const int64_t units_s = std::max<int64_t>(num_segments, 1) * num_kv_heads;
  const int64_t narrow =
      lists.narrow ? std::min(cap, std::max<int64_t>(256, round_up(ctx * units_s / (16ll * num_cus) + 1, kChunkStep)))
                   : wide;
  const int64_t smallest = lists.wide ? std::min(wide, narrow) : narrow;
  out->split_tokens = int32_t(wide);
  out->short_split_tokens = int32_t(narrow);
  out->max_splits = int32_t((ctx + smallest - 1) / smallest);
  out->kernel = 1;
  return PGQA_OK;
}

namespace {
struct ChunkSizing {
  bool columns;  // the call runs on the matrix-core decode kernel (plan kernel 2)
  int32_t split_wide, split_short, max_splits;
  ChunkGrids grids;
  ChunkWorkspace ws;
  DecodeWorkspace cws;  // columns: split partials, 16 columns per (segment, kv head)
  size_t total() const { return columns ? cws.total : ws.total; }
};

pgqa_status chunk_sizing(const pgqa_chunk_plan& p, int32_t block_size, int32_t num_segments, int32_t total_q,
                         int32_t hkv, int32_t hq, int32_t max_q_len, int32_t max_context_len, ChunkSizing* out) {
  if (p.kernel < 0 || p.kernel > 2) return fail(PGQA_ERR_INVALID_ARG, "chunk plan kernel=%d (0, 1 or 2)", p.kernel);
  out->columns = p.kernel == 2;
  if (out->columns) {
    const int32_t gran = block_size > 64 ? block_size : 64;
    if (int64_t(max_q_len) * (hq / hkv) > 16)
      return fail(PGQA_ERR_INVALID_ARG, "chunk plan kernel=2 needs max_q_len x group <= 16 (%d x %d)", max_q_len,
                  hq / hkv);
    if (p.split_tokens <= 0 || p.split_tokens % gran != 0 || p.split_tokens > 4096)
      return fail(PGQA_ERR_INVALID_ARG, "chunk plan kernel=2: split of %d keys must be a positive multiple of %d, "
                  "at most 4096", p.split_tokens, gran);
    if (p.max_splits < (int64_t(max_context_len) + p.split_tokens - 1) / p.split_tokens || p.max_splits > 65535)
      return fail(PGQA_ERR_INVALID_ARG, "plan.max_splits=%d does not cover max_context_len=%d", p.max_splits,
                  max_context_len);
    out->split_wide = out->split_short = p.split_tokens;
    out->max_splits = p.max_splits;
    out->cws = decode_workspace_layout(num_segments, hkv, 16, p.max_splits);
    return PGQA_OK;
  }
  const int32_t short_split = p.short_split_tokens == 0 ? p.split_tokens : p.short_split_tokens;
  for (const int32_t sp : {p.split_tokens, short_split})
    if (sp <= 0 || sp % kChunkStep != 0 || sp > kMaxSplitTokens)
      return fail(PGQA_ERR_INVALID_ARG, "chunk plan split of %d keys must be a positive multiple of %d, at most %d",
                  sp, kChunkStep, kMaxSplitTokens);
  const ChunkLists lists = chunk_lists(num_segments, total_q, hq / hkv, max_q_len);
  const int32_t smallest = !lists.narrow ? p.split_tokens : !lists.wide ? short_split
                                                                         : std::min(p.split_tokens, short_split);
  if (p.max_splits < (int64_t(max_context_len) + smallest - 1) / smallest || p.max_splits > 65535)
    return fail(PGQA_ERR_INVALID_ARG, "plan.max_splits=%d does not cover max_context_len=%d", p.max_splits,
                max_context_len);
  out->split_wide = p.split_tokens;
  out->split_short = short_split;
  out->max_splits = p.max_splits;
  out->grids = chunk_grids(num_segments, total_q, hkv, hq / hkv, max_q_len, max_context_len, p.split_tokens,
                           short_split, p.max_splits);
  if (out->grids.wide > 0x7fffffff || out->grids.narrow > 0x7fffffff || out->grids.combine > 0x7fffffff)
    return fail(PGQA_ERR_INVALID_ARG, "too many chunk work items");
  out->ws = chunk_workspace_layout(total_q, hq, p.max_splits);
  return PGQA_OK;
}
}  // namespace

size_t pgqa_chunk_workspace_bytes(const pgqa_pool* pool, int32_t num_segments, int32_t total_q, int32_t num_q_heads,
                                  int32_t max_q_len, int32_t max_context_len, const pgqa_chunk_plan* plan) {
  if (pool == nullptr || num_segments < 0 || total_q < 0 || num_q_heads <= 0 ||
      num_q_heads % pool->cfg.num_kv_heads != 0 || max_q_len < 0 || max_context_len < 0)
    return 0;
  pgqa_chunk_plan p;
  if (plan != nullptr) {
    p = *plan;
  } else if (pgqa_plan_chunk(pool->num_cus, pool->cfg.block_size, num_segments, total_q, pool->cfg.num_kv_heads,
                             num_q_heads, max_q_len, max_context_len, &p) != PGQA_OK) {
    return 0;
  }
  ChunkSizing z;
  if (chunk_sizing(p, pool->cfg.block_size, num_segments, total_q, pool->cfg.num_kv_heads, num_q_heads, max_q_len,
                   max_context_len, &z) != PGQA_OK)
    return 0;
  return z.total();
}

pgqa_status pgqa_paged_chunk_attention(pgqa_pool* pool, const void* q, const int32_t* query_start_loc,
                                       const int32_t* context_lens, const int32_t* block_tables, int32_t bt_stride,
                                       int32_t num_segments, int32_t total_q, int32_t num_q_heads, int32_t max_q_len,
                                       int32_t max_context_len, float scale, const pgqa_chunk_plan* plan,
                                       void* workspace, size_t workspace_bytes, void* out, void* stream) {
  clear_error();
  PGQA_TRY(check_pool(pool));
  PGQA_TRY(check_group(pool, num_q_heads));
  const int32_t hkv = pool->cfg.num_kv_heads;
  if (num_segments < 0 || num_segments > 4096)
    return fail(PGQA_ERR_INVALID_ARG, "num_segments=%d (at most 4096 per call)", num_segments);
  if (pool->cfg.max_batch_size > 0 && num_segments > pool->cfg.max_batch_size)
    return fail(PGQA_ERR_INVALID_ARG, "num_segments=%d exceeds max_batch_size=%d", num_segments,
                pool->cfg.max_batch_size);
  if (total_q < 0 || total_q > 65535 * 256)
    return fail(PGQA_ERR_INVALID_ARG, "total_q=%d", total_q);
  if (bt_stride <= 0) return fail(PGQA_ERR_INVALID_ARG, "bt_stride=%d", bt_stride);
  if (max_q_len < 0 || max_context_len < max_q_len)
    return fail(PGQA_ERR_INVALID_ARG, "max_q_len=%d max_context_len=%d", max_q_len, max_context_len);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PGQA_ERR_INVALID_ARG, "scale=%g", double(scale));
  if (num_segments == 0 || total_q == 0) return PGQA_OK;
  pgqa_chunk_plan p;
  if (plan != nullptr) {
    p = *plan;
  } else {
    PGQA_TRY(pgqa_plan_chunk(pool->num_cus, pool->cfg.block_size, num_segments, total_q, hkv, num_q_heads,
                             max_q_len, max_context_len, &p));
  }
  ChunkSizing z;
  PGQA_TRY(chunk_sizing(p, pool->cfg.block_size, num_segments, total_q, hkv, num_q_heads, max_q_len, max_context_len,
                        &z));
  const int dev = pool->device;
  PGQA_TRY(check_device_ptr(q, dev, "q", 16));
  PGQA_TRY(check_device_ptr(query_start_loc, dev, "query_start_loc", 4));
  PGQA_TRY(check_device_ptr(context_lens, dev, "context_lens", 4));
  PGQA_TRY(check_device_ptr(block_tables, dev, "block_tables", 4));
  PGQA_TRY(check_device_ptr(out, dev, "out", 8));
  if (z.total() > 0) {
    if (workspace == nullptr || workspace_bytes < z.total())
      return fail(PGQA_ERR_WORKSPACE, "chunk workspace of %zu bytes needed, %zu given", z.total(),
                  workspace == nullptr ? size_t(0) : workspace_bytes);
    PGQA_TRY(check_device_ptr(workspace, dev, "workspace", 256));
  }
  if (z.columns) {
    DecodeArgs d{};
    d.q = static_cast<const uint16_t*>(q);
    d.q_stride = int64_t(num_q_heads) * 128;
    d.ctx = context_lens;
    d.bt = block_tables;
    d.bt_stride = bt_stride;
    d.batch = num_segments;
    d.num_q_heads = num_q_heads;
    d.max_ctx = max_context_len;
    d.qk_scale_log2 = float(double(scale) * 1.4426950408889634);
    d.split_tokens = z.split_wide;
    d.max_splits = z.max_splits;
    d.waves = 4;
    d.mfma = 1;
    d.stream_loads = 0;
    char* ws = static_cast<char*>(workspace);
    d.part_o = z.cws.total > 0 ? reinterpret_cast<float*>(ws + z.cws.part_o_off) : nullptr;
    d.part_lse = z.cws.total > 0 ? reinterpret_cast<float*>(ws + z.cws.part_lse_off) : nullptr;
    d.out = static_cast<uint16_t*>(out);
    d.qsl = query_start_loc;
    d.total_q = total_q;
    d.max_q_len = max_q_len;
    hipError_t e = launch_decode_columns(pool->geom, d, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "chunk launch");
    return PGQA_OK;
  }
  ChunkArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.qsl = query_start_loc;
  a.ctx = context_lens;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_segments = num_segments;
  a.total_q = total_q;
  a.num_q_heads = num_q_heads;
  a.max_q_len = max_q_len;
  a.max_ctx = max_context_len;
  a.qk_scale_log2 = float(double(scale) * 1.4426950408889634);
  a.split_wide = z.split_wide;
  a.split_short = z.split_short;
  a.max_splits = z.max_splits;
  char* ws = static_cast<char*>(workspace);
  a.part_o = z.ws.total > 0 ? reinterpret_cast<float*>(ws + z.ws.part_o_off) : nullptr;
  a.part_lse = z.ws.total > 0 ? reinterpret_cast<float*>(ws + z.ws.part_lse_off) : nullptr;
  a.out = static_cast<uint16_t*>(out);
  hipError_t e = launch_chunk(pool->geom, a, z.grids, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "chunk launch");
  return PGQA_OK;
}

// ---------------------------------------------------------------- mixed step
namespace {

struct MixedSeg {
  int32_t s, q0, qlen, n;
};

// Keys a wide row group grp attends (up to its last query token's position).
int64_t mixed_wide_kend(int64_t qlen, int64_t n, int64_t r, int64_t grp) {
  const int64_t tiles = (qlen * r + 31) / 32;
  const int64_t t_last = std::min((grp + 1) * 4, tiles) - 1;
  const int64_t tok_last = std::min(qlen, (t_last * 32 + 32) / r) - 1;
  return n - qlen + tok_last + 1;
}

}  // namespace

pgqa_status pgqa_plan_mixed(int32_t num_cus, int32_t block_size, int32_t num_kv_heads, int32_t num_q_heads,
                            int32_t num_segments, const int32_t* query_start_loc, const int32_t* context_lens,
                            int32_t split_wide, int32_t split_columns, int32_t* items, int64_t item_capacity,
                            pgqa_mixed_plan* out) {
  clear_error();
  if (out == nullptr) return fail(PGQA_ERR_INVALID_ARG, "out is NULL");
  if (num_cus <= 0 || !valid_block_size(block_size) || num_kv_heads <= 0 || num_q_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || num_segments < 0)
    return fail(PGQA_ERR_INVALID_ARG, "invalid planner input");
  const int64_t hkv = num_kv_heads, r = num_q_heads / num_kv_heads;
  if (r != 1 && r != 2 && r != 4 && r != 8)
    return fail(PGQA_ERR_UNSUPPORTED, "query heads per kv head = %lld (supported: 1, 2, 4, 8)", (long long)r);
  if (num_segments > 0 && (query_start_loc == nullptr || context_lens == nullptr))
    return fail(PGQA_ERR_INVALID_ARG, "host query_start_loc / context_lens are NULL");
  const int64_t gran = block_size > 64 ? block_size : 64;
  if (split_wide < 0 || split_wide % kChunkStep || split_wide > kMaxSplitTokens)
    return fail(PGQA_ERR_INVALID_ARG, "split_wide=%d (0, or a multiple of 32 up to 4096)", split_wide);
  if (split_columns < 0 || split_columns % gran || split_columns > kMaxSplitTokens)
    return fail(PGQA_ERR_INVALID_ARG, "split_columns=%d (0, or a multiple of %lld up to 4096)", split_columns,
                (long long)gran);
  // Segments by kind: more than 16 query rows per kv head -> wide items.
  std::vector<MixedSeg> wide, cols;
  int64_t units_w = 0, keys_c = 0, kend_w = 0, n_c = 0;
  if (num_segments > 0 && query_start_loc[0] != 0) return fail(PGQA_ERR_INVALID_ARG, "query_start_loc[0] != 0");
  for (int32_t s = 0; s < num_segments; ++s) {
    const int32_t q0 = query_start_loc[s], qlen = query_start_loc[s + 1] - q0, n = context_lens[s];
    if (qlen < 0 || n < qlen)
      return fail(PGQA_ERR_INVALID_ARG, "segment %d: q_len %d, context %d (need 0 <= q_len <= context)", s, qlen, n);
    if (qlen == 0) continue;
    if (int64_t(qlen) * r > 16) {
      wide.push_back(MixedSeg{s, q0, qlen, n});
      units_w += (int64_t(qlen) * r + 127) / 128 * hkv;
      kend_w = std::max<int64_t>(kend_w, n);
    } else {
      cols.push_back(MixedSeg{s, q0, qlen, n});
      keys_c += int64_t(n) * hkv;
      n_c = std::max<int64_t>(n_c, n);
    }
  }
  // Split lengths.  Wide items (matrix-core bound) and column items (HBM bound)
  // share the CUs' two workgroup slots.  tw: the wide work's time with every
  // slot busy, from its 32-key steps over 128-row units (kWideStepUs per step
  // and slot, two wide items sharing a CU); tc: the columns' K/V bytes at
  // kColumnBytesPerUs.  Wide items get the share phi = tw / (tw + tc) of the
  // 2 num_cus slots, which sets their splits per unit (256 .. 4096 keys);
  // column items number about 4 num_cus (1 - phi)^2 (many per slot when they
  // are the critical path, about one per free slot when they only fill gaps
  // beside the wide items), at least 1024 keys per split (shorter splits only
  // add start-up latency and combine work when the column work is small).
  // Both rates were measured on MI355X; split_wide / split_columns override
  // the choice.
  constexpr double kWideStepUs = 1.45;
  constexpr double kColumnBytesPerUs = 5.5e6;
  int64_t steps_w = 0;
  for (const MixedSeg& m : wide) {
    const int64_t groups = ((int64_t(m.qlen) * r + 31) / 32 + 3) / 4;
    for (int64_t grp = 0; grp < groups; ++grp)
      steps_w += (mixed_wide_kend(m.qlen, m.n, r, grp) + kChunkStep - 1) / kChunkStep * hkv;
  }
  const double tw = double(steps_w) * kWideStepUs / (2.0 * num_cus);
  const double tc = double(keys_c) * 512.0 / kColumnBytesPerUs;  // K and V: 128 bf16 each per key and kv head
  const double phi = tw + tc > 0 ? tw / (tw + tc) : 0.0;
  int64_t sw = split_wide, sc = split_columns;
  if (sw == 0) {
    sw = 256;
    if (units_w > 0) {
      const double target = 2.0 * num_cus * phi;
      const int64_t want = std::max<int64_t>(1, std::llround(target / double(units_w)));
      sw = std::max<int64_t>(256, round_up((kend_w + want - 1) / want, kChunkStep));
      sw = std::min<int64_t>({sw, round_up(kend_w, kChunkStep), kMaxSplitTokens});
    }
  }
  if (sc == 0) {
    sc = round_up(1024, gran);
    if (keys_c > 0) {
      const double target = std::max(1.0, 4.0 * num_cus * (1.0 - phi) * (1.0 - phi));
      sc = std::max<int64_t>(round_up(1024, gran), round_up(int64_t(std::ceil(double(keys_c) / target)), gran));
      sc = std::min<int64_t>({sc, std::max<int64_t>(round_up(n_c, gran), gran), kMaxSplitTokens / gran * gran});
    }
  }
  // Item counts and the partial slots per row (a size query stops here).
  int64_t n_wide = 0, n_cols = 0, n_comb = 0, max_splits = 1, max_ns_w = 0;
  for (const MixedSeg& m : wide) {
    const int64_t rows = int64_t(m.qlen) * r, groups = ((rows + 31) / 32 + 3) / 4;
    max_ns_w = std::max<int64_t>(max_ns_w, (int64_t(m.n) + sw - 1) / sw);
    for (int64_t grp = 0; grp < groups; ++grp) {
      const int64_t ns = (mixed_wide_kend(m.qlen, m.n, r, grp) + sw - 1) / sw;
      n_wide += ns * hkv;
      max_splits = std::max(max_splits, ns);
      if (ns >= 2) n_comb += hkv * ((std::min<int64_t>(rows, (grp + 1) * 128) - grp * 128 + 7) / 8);
    }
  }
  for (const MixedSeg& m : cols) {
    const int64_t ns = (int64_t(m.n) + sc - 1) / sc;
    n_cols += ns * hkv;
    max_splits = std::max(max_splits, ns);
    if (ns >= 2) n_comb += hkv * ((int64_t(m.qlen) * r + 7) / 8);
  }
  if (n_wide + n_cols + n_comb > int64_t(0x7fffffff) || max_splits > 65535)
    return fail(PGQA_ERR_INVALID_ARG, "too many mixed work items");
  out->split_wide = int32_t(sw);
  out->split_columns = int32_t(sc);
  out->max_splits = int32_t(max_splits);
  out->num_items = int32_t(n_wide + n_cols);
  out->num_combine = int32_t(n_comb);
  if (items == nullptr) return PGQA_OK;
  if (item_capacity < n_wide + n_cols + n_comb)
    return fail(PGQA_ERR_INVALID_ARG, "item buffer holds %lld items, the plan has %lld", (long long)item_capacity,
                (long long)(n_wide + n_cols + n_comb));

  // Items.  Wide items with the kv head fastest, column items most keys
  // first; the two kinds alternate in runs of num_cus, so that a CU's two
  // slots start on one item of each kind.  Workgroups are dealt to the 8 XCDs
  // round-robin, and a run of num_cus (a multiple of 8) keeps wide item j on
  // XCD j % 8: one kv head's items share an L2.  Then the combine items.
  // Each item goes straight to its place in that order: wide item i after
  // i / run earlier wide runs and the column runs between them, column item j
  // after (j / run) + 1 wide runs and j / run column runs.
  const int64_t run = num_cus;
  auto put = [&](int64_t pos, int32_t s0, int32_t kind, int32_t g, int32_t grp, int32_t sp, const MixedSeg& m) {
    int32_t* d = items + pos * kMixedItemInts;
    d[0] = s0; d[1] = kind; d[2] = g; d[3] = grp; d[4] = sp; d[5] = m.q0; d[6] = m.qlen; d[7] = m.n;
  };
  int64_t wk = 0, wj = 0;  // wide item wk * run + wj
  for (int64_t sp = 0; sp < max_ns_w; ++sp)
    for (const MixedSeg& m : wide) {
      const int64_t groups = ((int64_t(m.qlen) * r + 31) / 32 + 3) / 4;
      for (int64_t grp = 0; grp < groups; ++grp) {
        const int64_t ns = (mixed_wide_kend(m.qlen, m.n, r, grp) + sw - 1) / sw;
        if (sp >= ns) continue;
        for (int64_t g = 0; g < hkv; ++g) {
          put(wk * run + std::min(wk * run, n_cols) + wj, m.s, 0, int32_t(g), int32_t(grp), int32_t(sp), m);
          if (++wj == run) wj = 0, ++wk;
        }
      }
    }
  // Column items, most keys first: every split but a segment's last holds
  // exactly sc keys, so the full splits go first in (segment, split, kv head)
  // order, then the shorter last splits by length, longest first (segment
  // order among equals).
  struct Tail {
    int32_t keys, sp;
    const MixedSeg* m;
  };
  std::vector<Tail> tails;
  tails.reserve(cols.size());
  int64_t ck = 0, cj = 0;  // column item ck * run + cj
  auto put_col = [&](const MixedSeg& m, int32_t sp) {
    for (int64_t g = 0; g < hkv; ++g) {
      put(std::min((ck + 1) * run, n_wide) + ck * run + cj, m.s, 1, int32_t(g), 0, sp, m);
      if (++cj == run) cj = 0, ++ck;
    }
  };
  for (const MixedSeg& m : cols) {
    const int32_t full = int32_t(int64_t(m.n) / sc), rest = int32_t(int64_t(m.n) - int64_t(full) * sc);
    for (int32_t sp = 0; sp < full; ++sp) put_col(m, sp);
    if (rest != 0) tails.push_back(Tail{rest, full, &m});
  }
  std::stable_sort(tails.begin(), tails.end(), [](const Tail& x, const Tail& y) { return x.keys > y.keys; });
  for (const Tail& t : tails) put_col(*t.m, t.sp);
  int32_t* dst = items + (n_wide + n_cols) * kMixedItemInts;
  auto add_combine = [&](const MixedSeg& m, int64_t rho0, int64_t rho1, int64_t ns) {
    if (ns < 2) return;
    for (int64_t g = 0; g < hkv; ++g)
      for (int64_t rho = rho0; rho < rho1; rho += 8) {
        dst[0] = m.s; dst[1] = 2; dst[2] = int32_t(g); dst[3] = int32_t(rho);
        dst[4] = int32_t(ns); dst[5] = m.q0; dst[6] = m.qlen; dst[7] = m.n;
        dst += kMixedItemInts;
      }
  };
  for (const MixedSeg& m : wide) {
    const int64_t rows = int64_t(m.qlen) * r, groups = ((rows + 31) / 32 + 3) / 4;
    for (int64_t grp = 0; grp < groups; ++grp)
      add_combine(m, grp * 128, std::min<int64_t>(rows, (grp + 1) * 128),
                  (mixed_wide_kend(m.qlen, m.n, r, grp) + sw - 1) / sw);
  }
  for (const MixedSeg& m : cols) add_combine(m, 0, int64_t(m.qlen) * r, (int64_t(m.n) + sc - 1) / sc);
  return PGQA_OK;
}

size_t pgqa_mixed_workspace_bytes(const pgqa_mixed_plan* plan, int32_t total_q, int32_t num_q_heads) {
  if (plan == nullptr || total_q < 0 || num_q_heads <= 0 || plan->max_splits < 1) return 0;
  return chunk_workspace_layout(total_q, num_q_heads, plan->max_splits).total;
}

pgqa_status pgqa_paged_mixed_attention(pgqa_pool* pool, const void* q, const int32_t* query_start_loc,
                                       const int32_t* context_lens, const int32_t* block_tables, int32_t bt_stride,
                                       int32_t num_segments, int32_t total_q, int32_t num_q_heads, int32_t max_q_len,
                                       int32_t max_context_len, float scale, const pgqa_mixed_plan* plan,
                                       const int32_t* items, void* workspace, size_t workspace_bytes, void* out,
                                       void* stream) {
  clear_error();
  PGQA_TRY(check_pool(pool));
  PGQA_TRY(check_group(pool, num_q_heads));
  if (plan == nullptr) return fail(PGQA_ERR_INVALID_ARG, "plan is NULL (pgqa_plan_mixed builds it)");
  if (num_segments < 0) return fail(PGQA_ERR_INVALID_ARG, "num_segments=%d", num_segments);
  if (pool->cfg.max_batch_size > 0 && num_segments > pool->cfg.max_batch_size)
    return fail(PGQA_ERR_INVALID_ARG, "num_segments=%d exceeds max_batch_size=%d", num_segments,
                pool->cfg.max_batch_size);
  if (total_q < 0) return fail(PGQA_ERR_INVALID_ARG, "total_q=%d", total_q);
  if (bt_stride <= 0) return fail(PGQA_ERR_INVALID_ARG, "bt_stride=%d", bt_stride);
  if (max_q_len < 0 || max_context_len < max_q_len)
    return fail(PGQA_ERR_INVALID_ARG, "max_q_len=%d max_context_len=%d", max_q_len, max_context_len);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PGQA_ERR_INVALID_ARG, "scale=%g", double(scale));
  const int32_t gran = pool->cfg.block_size > 64 ? pool->cfg.block_size : 64;
  if (plan->split_wide <= 0 || plan->split_wide % kChunkStep || plan->split_wide > kMaxSplitTokens ||
      plan->split_columns <= 0 || plan->split_columns % gran || plan->split_columns > kMaxSplitTokens ||
      plan->max_splits < 1 || plan->max_splits > 65535 || plan->num_items < 0 || plan->num_combine < 0)
    return fail(PGQA_ERR_INVALID_ARG, "plan (splits %d / %d, max_splits %d, items %d + %d) is not one of "
                "pgqa_plan_mixed's for this pool", plan->split_wide, plan->split_columns, plan->max_splits,
                plan->num_items, plan->num_combine);
  if (num_segments == 0 || total_q == 0 || plan->num_items == 0) return PGQA_OK;
  const size_t need = pgqa_mixed_workspace_bytes(plan, total_q, num_q_heads);
  const int dev = pool->device;
  PGQA_TRY(check_device_ptr(q, dev, "q", 16));
  PGQA_TRY(check_device_ptr(query_start_loc, dev, "query_start_loc", 4));
  PGQA_TRY(check_device_ptr(context_lens, dev, "context_lens", 4));
  PGQA_TRY(check_device_ptr(block_tables, dev, "block_tables", 4));
  PGQA_TRY(check_device_ptr(items, dev, "items", 16));
  PGQA_TRY(check_device_ptr(out, dev, "out", 8));
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(PGQA_ERR_WORKSPACE, "mixed workspace of %zu bytes needed, %zu given", need,
                  workspace == nullptr ? size_t(0) : workspace_bytes);
    PGQA_TRY(check_device_ptr(workspace, dev, "workspace", 256));
  }
  ChunkArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.qsl = query_start_loc;
  a.ctx = context_lens;
  a.bt = block_tables;
  a.bt_stride = bt_stride;
  a.num_segments = num_segments;
  a.total_q = total_q;
  a.num_q_heads = num_q_heads;
  a.max_q_len = max_q_len;
  a.max_ctx = max_context_len;
  a.qk_scale_log2 = float(double(scale) * 1.4426950408889634);
  a.split_wide = plan->split_wide;
  a.split_short = plan->split_columns;
  a.max_splits = plan->max_splits;
  const ChunkWorkspace wl = chunk_workspace_layout(total_q, num_q_heads, plan->max_splits);
  char* ws = static_cast<char*>(workspace);
  a.part_o = need > 0 ? reinterpret_cast<float*>(ws + wl.part_o_off) : nullptr;
  a.part_lse = need > 0 ? reinterpret_cast<float*>(ws + wl.part_lse_off) : nullptr;
  a.out = static_cast<uint16_t*>(out);
  a.items = items;
  a.num_items = plan->num_items;
  hipError_t e = launch_mixed(pool->geom, a, plan->num_combine, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mixed attention launch");
  return PGQA_OK;
}

}  // extern "C"
