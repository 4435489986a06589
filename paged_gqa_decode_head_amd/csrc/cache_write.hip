// Fused per-head RMSNorm + neox rotary of q and k, and the paged K/V cache write.
//
// Page "perf: Qwen3 offline inference - hybrid attention backend, fused
// rms_norm_rope, chunked prefill + prompt-lookup spec decoding", Summary item 2:
// q and k of Qwen3 get a per-head RMSNorm and then full rotary embedding in one
// fused op; item 1: keys and values live in a block-table paged cache.  Here the
// cache write is folded into the same launch, so a decode step's q/k/v are read
// once and the normed/rotated k is never stored anywhere but its cache slot.
//
// One workgroup per token; 8 lanes per 128-element head row (q rows, then k
// rows, then v rows).  Lane s of a row holds dims 8s..8s+7 and 64+8s..64+8s+7:
// the two members of each of its 8 rotary pairs, so the rotation is lane-local
// and the sum of squares needs three DPP steps.  All loads are issued before
// any dependent work.  A decode step moves about 1 MB here, so the launch is
// bound by latency, not bandwidth.
//
// Rotation angles: pair i of a token at position p turns by p * theta^(-2i/128)
// radians.  At p near 32768 an fp32 product is already off by ~2e-3 rad, so the
// angle is reduced in fp64 as a fraction of a turn, frac(p * f_i / 2pi), and
// only that fraction (exact to ~1e-12) goes to an fp32 sincos.  The 64 values
// f_i / 2pi come from the host in fp64.
#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {
namespace {

__global__ __launch_bounds__(1024) void cache_write_kernel(PoolGeom pool, WriteArgs a) {
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int row = tid >> 3, s = tid & 7;
  const int hq = a.num_q_heads, hkv = pool.num_kv_heads, bs = pool.block_size;
  const int rows = hq + 2 * hkv;

  __shared__ float s_cos[64], s_sin[64];

  const int pos = a.pos[t];
  const int seq = a.seq[t];
  // Issue this lane's row loads first.
  const bool active = row < rows;
  const bool is_q = row < hq, is_k = !is_q && row < hq + hkv;
  const int h = is_q ? row : is_k ? row - hq : row - hq - hkv;
  uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0, w0 = x0, w1 = x0;
  if (active) {
    const uint16_t* src = is_q ? a.q + int64_t(t) * a.q_stride + h * kHeadDim
                               : is_k ? a.k + int64_t(t) * a.k_stride + h * kHeadDim
                                      : a.v + int64_t(t) * a.v_stride + h * kHeadDim;
    x0 = *reinterpret_cast<const uint4*>(src + 8 * s);
    x1 = *reinterpret_cast<const uint4*>(src + 64 + 8 * s);
    if (is_q || is_k) {
      const uint16_t* wt = is_q ? a.wq : a.wk;
      w0 = *reinterpret_cast<const uint4*>(wt + 8 * s);
      w1 = *reinterpret_cast<const uint4*>(wt + 64 + 8 * s);
    }
  }
  if (tid < 64) {
    const double turns = double(pos) * a.rev_freq[tid];
    const float ang = float((turns - floor(turns)) * 6.283185307179586);
    float sn, cs;
    sincosf(ang, &sn, &cs);
    s_cos[tid] = cs;
    s_sin[tid] = sn;
  }

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
  if (bad && tid == 0) raise_error(pool.err, bad);
  const int off = pos & (bs - 1);
  __syncthreads();
  if (!active) return;

  uint16_t* kv_tile = pool.kv + (int64_t(blk) * hkv + h) * tile_elems(pool);
  if (!is_q && !is_k) {
    if (bad) return;
    // v goes into the cache as it came, transposed: V^T[dim][slot].
    uint16_t* dst = kv_tile + int64_t(bs) * kHeadDim + off;
    const uint32_t lo[4] = {x0.x, x0.y, x0.z, x0.w}, hi[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[int64_t(8 * s + 2 * e) * bs] = uint16_t(lo[e]);
      dst[int64_t(8 * s + 2 * e + 1) * bs] = uint16_t(lo[e] >> 16);
      dst[int64_t(64 + 8 * s + 2 * e) * bs] = uint16_t(hi[e]);
      dst[int64_t(64 + 8 * s + 2 * e + 1) * bs] = uint16_t(hi[e] >> 16);
    }
    return;
  }

  float y0[8], y1[8];
  const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w}, a1[4] = {x1.x, x1.y, x1.z, x1.w};
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y0[2 * e] = bf16_lo(a0[e]);
    y0[2 * e + 1] = bf16_hi(a0[e]);
    y1[2 * e] = bf16_lo(a1[e]);
    y1[2 * e + 1] = bf16_hi(a1[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) ss += y0[e] * y0[e] + y1[e] * y1[e];
  const float ms = sum8(ss) * (1.0f / kHeadDim);
  const float inv = 1.0f / sqrtf(ms + a.eps);
  const uint32_t g0[4] = {w0.x, w0.y, w0.z, w0.w}, g1[4] = {w1.x, w1.y, w1.z, w1.w};
  uint32_t o0[4], o1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float r0[2], r1[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = 8 * s + 2 * e + u;  // rotary pair (i, i + 64)
      const float wa = u ? bf16_hi(g0[e]) : bf16_lo(g0[e]);
      const float wb = u ? bf16_hi(g1[e]) : bf16_lo(g1[e]);
      const float ya = y0[2 * e + u] * inv * wa;
      const float yb = y1[2 * e + u] * inv * wb;
      const float cs = s_cos[i], sn = s_sin[i];
      r0[u] = ya * cs - yb * sn;
      r1[u] = yb * cs + ya * sn;
    }
    o0[e] = pack_bf16x2(r0[0], r0[1]);
    o1[e] = pack_bf16x2(r1[0], r1[1]);
  }
  const uint4 out0 = make_uint4(o0[0], o0[1], o0[2], o0[3]);
  const uint4 out1 = make_uint4(o1[0], o1[1], o1[2], o1[3]);
  if (is_q) {
    uint16_t* dst = a.q_out + (int64_t(t) * hq + h) * kHeadDim;
    *reinterpret_cast<uint4*>(dst + 8 * s) = out0;
    *reinterpret_cast<uint4*>(dst + 64 + 8 * s) = out1;
  } else if (!bad) {
    uint16_t* dst = kv_tile + int64_t(off) * kHeadDim;
    *reinterpret_cast<uint4*>(dst + 8 * s) = out0;
    *reinterpret_cast<uint4*>(dst + 64 + 8 * s) = out1;
  }
}

}  // namespace

hipError_t launch_cache_write(const PoolGeom& pool, const WriteArgs& a, hipStream_t stream) {
  if (a.num_tokens == 0) return hipSuccess;
  const int rows = a.num_q_heads + 2 * pool.num_kv_heads;
  const int threads = (rows * 8 + 63) / 64 * 64;
  if (threads > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(cache_write_kernel, dim3(a.num_tokens), dim3(threads), 0, stream, pool, a);
  return hipGetLastError();
}

}  // namespace pgqa
