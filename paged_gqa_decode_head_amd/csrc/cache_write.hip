// Fused per-head RMSNorm + neox rotary of q and k, and the paged K/V cache write.
//
// Page "perf: Qwen3 offline inference - hybrid attention backend, fused
// rms_norm_rope, chunked prefill + prompt-lookup spec decoding", Summary item 2:
// q and k of Qwen3 get a per-head RMSNorm and then full rotary embedding in one
// fused op; item 1: keys and values live in a block-table paged cache.  Here the
// cache write is folded into the same launch, so a decode step's q/k/v are read
// once and the normed/rotated k is never stored anywhere but its cache slot.
//
// One workgroup of four waves per token.  Each wave takes whole 128-element
// head rows; lane l holds dims l and l + 64, which are exactly the two members
// of rotary pair l, so the rotation is lane-local and only the sum of squares
// needs a cross-lane reduction.  The launch moves about 1 MB for a 64-token
// decode step, so it is bound by launch latency rather than bandwidth.
#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {
namespace {

constexpr int kWaves = 4;

__global__ __launch_bounds__(64 * kWaves) void cache_write_kernel(PoolGeom pool, WriteArgs a) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hq = a.num_q_heads, hkv = pool.num_kv_heads, bs = pool.block_size;

  const int pos = a.pos[t];
  const int seq = a.seq[t];
  uint32_t bad = 0;
  int32_t blk = 0;
  if (seq < 0 || seq >= a.num_seqs) {
    bad = kErrSeqId;
  } else if (pos < 0 || pos / bs >= a.bt_stride) {
    bad = kErrPosition;
  } else {
    blk = a.bt[int64_t(seq) * a.bt_stride + pos / bs];
    if (blk < 0 || blk >= pool.num_blocks) bad = kErrBlockId;
  }
  if (bad && threadIdx.x == 0) raise_error(pool.err, bad);
  const int off = pos & (bs - 1);

  // Rotation of pair `lane` at this token's position, from an fp64 angle: at
  // positions near 32768 an fp32 product p * f_i would already be off by
  // ~2e-3 rad.  sincos of the fp64 angle, then rounded to fp32.
  const double inv_freq = pow(a.theta, -2.0 * lane / double(kHeadDim));
  double sd, cd;
  sincos(double(pos) * inv_freq, &sd, &cd);
  const float sn = float(sd), cs = float(cd);

  const int rows = hq + 2 * hkv;
  for (int row = wave; row < rows; row += kWaves) {
    if (row < hq + hkv) {
      const bool is_q = row < hq;
      const int h = is_q ? row : row - hq;
      const uint16_t* src = is_q ? a.q + int64_t(t) * a.q_stride + h * kHeadDim
                                 : a.k + int64_t(t) * a.k_stride + h * kHeadDim;
      const uint16_t* w = is_q ? a.wq : a.wk;
      const float x0 = bf16_to_f32(src[lane]);
      const float x1 = bf16_to_f32(src[lane + 64]);
      const float ms = wave_sum(x0 * x0 + x1 * x1) * (1.0f / kHeadDim);
      const float inv = 1.0f / sqrtf(ms + a.eps);
      const float y0 = x0 * inv * bf16_to_f32(w[lane]);
      const float y1 = x1 * inv * bf16_to_f32(w[lane + 64]);
      const uint16_t o0 = f32_to_bf16(y0 * cs - y1 * sn);
      const uint16_t o1 = f32_to_bf16(y1 * cs + y0 * sn);
      if (is_q) {
        uint16_t* dst = a.q_out + (int64_t(t) * hq + h) * kHeadDim;
        dst[lane] = o0;
        dst[lane + 64] = o1;
      } else if (!bad) {
        uint16_t* dst = pool.kv + (int64_t(blk) * hkv + h) * tile_elems(pool) + int64_t(off) * kHeadDim;
        dst[lane] = o0;
        dst[lane + 64] = o1;
      }
    } else if (!bad) {
      // v is stored as it came, transposed: V^T[dim][slot].
      const int h = row - hq - hkv;
      const uint16_t* src = a.v + int64_t(t) * a.v_stride + h * kHeadDim;
      uint16_t* dst = pool.kv + (int64_t(blk) * hkv + h) * tile_elems(pool) + int64_t(bs) * kHeadDim + off;
      dst[int64_t(lane) * bs] = src[lane];
      dst[int64_t(lane + 64) * bs] = src[lane + 64];
    }
  }
}

}  // namespace

hipError_t launch_cache_write(const PoolGeom& pool, const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(cache_write_kernel, dim3(a.num_tokens), dim3(64 * kWaves), 0, stream, pool, a);
  return hipGetLastError();
}

}  // namespace pgqa
