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
// radians, reduced in fp64 as a fraction of a turn (norm_rope.hpp); the 64
// values f_i / 2pi come from the host in fp64.  The norm and rotation are the
// same device code the fused decode step uses, so both give identical bits.
#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"
#include "norm_rope.hpp"

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
    float cs, sn;
    rope_angle(pos, a.rev_freq[tid], cs, sn);
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
    // v goes into the cache as it came, transposed: V^T piece [dim][slot % 16].
    uint16_t* dst = kv_tile + v_elem(bs, off, 0);
    const uint32_t lo[4] = {x0.x, x0.y, x0.z, x0.w}, hi[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[(8 * s + 2 * e) * kVSub] = uint16_t(lo[e]);
      dst[(8 * s + 2 * e + 1) * kVSub] = uint16_t(lo[e] >> 16);
      dst[(64 + 8 * s + 2 * e) * kVSub] = uint16_t(hi[e]);
      dst[(64 + 8 * s + 2 * e + 1) * kVSub] = uint16_t(hi[e] >> 16);
    }
    return;
  }

  float cs[8], sn[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    cs[j] = s_cos[8 * s + j];
    sn[j] = s_sin[8 * s + j];
  }
  uint4 out0, out1;
  norm_rope_lane(x0, x1, w0, w1, cs, sn, a.eps, out0, out1);
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
