// Paged split-KV GQA decode attention with a log-sum-exp combine (gfx950).
//
// Page "perf: Qwen3 offline inference - hybrid attention backend, fused
// rms_norm_rope, chunked prefill + prompt-lookup spec decoding", Summary item 1:
// pure decode batches run a self-written paged split-KV kernel over the
// block-table cache.  That design targeted NVIDIA consumer parts; this one is
// laid out for CDNA4.
//
// Work decomposition.  One workgroup per (sequence b, kv head g, split sp); a
// split is split_tokens consecutive keys.  All r = Hq / Hkv query heads of the
// group are processed by the same workgroup, so each K/V byte is read from HBM
// once.  The W waves of the workgroup take the split's 16-key tiles in turn
// (wave w: tiles w, w+W, ...), each wave keeping its own online softmax state.
//
// Inside a wave, for one 16-key tile of one (block, kv head):
//   * keys: the 8-lane group G = lane/8 owns keys 2G and 2G+1, lane % 8 owns
//     16 of the 128 dims.  Each lane loads 2 x 32 contiguous bytes of K, takes
//     bf16 pair dot products with q (v_dot2_f32_bf16, no unpacking), and three
//     DPP steps finish the 128-dim sums inside the 8-lane group.
//   * softmax: scores are in log2 units (q.k * scale * log2 e).  The running
//     maximum is only raised when a score exceeds it by more than kTau, which a
//     wave-wide ballot detects; otherwise no max reduction and no rescale is
//     done.  The weights exp2(s - m) (at most 2^kTau) are packed to bf16 pairs
//     and broadcast through LDS.
//   * values: the cache stores each V tile transposed, [dim][slot], so lane l
//     loads dims 2l and 2l+1 for all 16 keys (64 contiguous bytes) and the
//     weighted sum over key pairs is again v_dot2_f32_bf16.  No lane needs
//     another lane's accumulator until the end of the split.
//   * the next tile's 128 bytes per lane are loaded while the current one is
//     computed (register double buffer, DEPTH tiles in flight per wave).
//
// Combine.  With one split the workgroup writes bf16 directly.  Otherwise it
// writes its normalised partial o_k and lse_k, and the last workgroup of the
// (b, g) pair to arrive (an atomic ticket, used for ordering only) merges all
// partials in split order: o = sum_k 2^(lse_k - lse) o_k.  The combine order is
// fixed, so results do not depend on which workgroup arrives last.
#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {
namespace {

constexpr float kTau = 8.0f;              // log2 headroom before the running max is raised
constexpr int kMaxSplitTokens = 4096;     // bounds the per-split block-id stage in LDS

struct Tile {
  uint4 k[4];  // k[0..1]: key 2G, dims 16*(lane%8) .. +16;  k[2..3]: key 2G+1
  uint4 v[4];  // v[0..1]: V^T row 2*lane (16 keys); v[2..3]: row 2*lane+1
  int ok;
};

__device__ __forceinline__ uint32_t comp(const uint4& x, int i) {
  return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
}

template <int R, int W, int DEPTH>
__global__ __launch_bounds__(64 * W) void decode_kernel(PoolGeom pool, DecodeArgs a) {
  const int sp = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 3, sub = lane & 7;
  const int hq = a.num_q_heads, hkv = pool.num_kv_heads, bs = pool.block_size;

  __shared__ int32_t s_blk[kMaxSplitTokens / 16];
  __shared__ __align__(16) uint32_t s_p[W][R][8];
  __shared__ float s_m[W][R], s_l[W][R];
  __shared__ __align__(16) float s_acc[W][R][kHeadDim];
  __shared__ int s_last;

  const int n = a.ctx[b];
  const bool bad_ctx = n < 0 || n > a.max_ctx || int64_t(n) > int64_t(a.bt_stride) * bs;
  uint16_t* out_bg = a.out + (int64_t(b) * hq + g * R) * kHeadDim;
  if (bad_ctx || n == 0) {
    if (sp == 0) {
      if (bad_ctx && tid == 0) raise_error(pool.err, kErrContext);
      for (int i = tid; i < R * kHeadDim; i += 64 * W) out_bg[i] = 0;
    }
    return;
  }
  const int ns = (n + a.split_tokens - 1) / a.split_tokens;
  if (sp >= ns) return;
  const int k0 = sp * a.split_tokens;
  const int k1 = min(n, k0 + a.split_tokens);
  const int nblk = (k1 - k0 + bs - 1) / bs;
  {
    const int32_t* row = a.bt + int64_t(b) * a.bt_stride + k0 / bs;
    for (int i = tid; i < nblk; i += 64 * W) s_blk[i] = row[i];
  }

  // q rows of the group: lane holds dims 16*sub .. 16*sub+15 of each head, as bf16 pairs.
  uint32_t qv[R][8];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q + (int64_t(b) * hq + g * R + h) * kHeadDim + sub * 16);
    const uint4 x = qp[0], y = qp[1];
    qv[h][0] = x.x; qv[h][1] = x.y; qv[h][2] = x.z; qv[h][3] = x.w;
    qv[h][4] = y.x; qv[h][5] = y.y; qv[h][6] = y.z; qv[h][7] = y.w;
  }
  __syncthreads();

  const int64_t tstride = tile_elems(pool);
  const int64_t bstride = tstride * hkv;
  const uint16_t* pool_g = pool.kv + int64_t(g) * tstride;
  const int ntiles = (k1 - k0 + 15) >> 4;

  float m[R], l[R], acc[R][2];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
    acc[h][0] = acc[h][1] = 0.f;
  }

  auto load = [&](Tile& tb, int tt) {
    const int rel = tt * 16;
    int32_t blk = s_blk[rel / bs];
    const int sub16 = (rel & (bs - 1)) >> 4;
    tb.ok = unsigned(blk) < unsigned(pool.num_blocks);
    if (!tb.ok) {
      if (lane == 0) raise_error(pool.err, kErrBlockId);
      blk = 0;
    }
    const uint16_t* base = pool_g + int64_t(blk) * bstride;
    const uint4* kp = reinterpret_cast<const uint4*>(base + (sub16 * 16 + 2 * grp) * kHeadDim + sub * 16);
    tb.k[0] = kp[0];
    tb.k[1] = kp[1];
    tb.k[2] = kp[kHeadDim / 8];
    tb.k[3] = kp[kHeadDim / 8 + 1];
    const uint16_t* vrow = base + int64_t(bs) * kHeadDim + int64_t(2 * lane) * bs + sub16 * 16;
    const uint4* vp0 = reinterpret_cast<const uint4*>(vrow);
    const uint4* vp1 = reinterpret_cast<const uint4*>(vrow + bs);
    tb.v[0] = vp0[0];
    tb.v[1] = vp0[1];
    tb.v[2] = vp1[0];
    tb.v[3] = vp1[1];
  };

  // Zero the V entries of keys that are not attended (past the split end, or
  // the whole tile when its block id was invalid): their weight is 0, but the
  // slots may hold any bits, and 0 * NaN would poison the accumulator.
  auto mask_v = [&](Tile& tb, int tt) {
    const int nv = tb.ok ? k1 - (k0 + tt * 16) : 0;  // valid keys in this tile
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t keep = 2 * c + 1 < nv ? 0xffffffffu : 2 * c < nv ? 0x0000ffffu : 0u;
      uint4& a0 = tb.v[c >> 2];
      uint4& a1 = tb.v[2 + (c >> 2)];
      switch (c & 3) {
        case 0: a0.x &= keep; a1.x &= keep; break;
        case 1: a0.y &= keep; a1.y &= keep; break;
        case 2: a0.z &= keep; a1.z &= keep; break;
        default: a0.w &= keep; a1.w &= keep; break;
      }
    }
  };

  auto compute = [&](Tile& tb, int tt) {
    if (!tb.ok || k0 + tt * 16 + 16 > k1) mask_v(tb, tt);
    const int key = k0 + tt * 16 + 2 * grp;
    const bool ok0 = tb.ok && key < k1;
    const bool ok1 = tb.ok && key + 1 < k1;
    float s0[R], s1[R];
    bool need = false;
#pragma unroll
    for (int h = 0; h < R; ++h) {
      float x = 0.f, y = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x = dot2_bf16(qv[h][i], comp(tb.k[0], i), x);
        y = dot2_bf16(qv[h][i], comp(tb.k[2], i), y);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x = dot2_bf16(qv[h][4 + i], comp(tb.k[1], i), x);
        y = dot2_bf16(qv[h][4 + i], comp(tb.k[3], i), y);
      }
      x = sum8(x) * a.qk_scale_log2;
      y = sum8(y) * a.qk_scale_log2;
      s0[h] = ok0 ? x : -INFINITY;
      s1[h] = ok1 ? y : -INFINITY;
      need |= fmaxf(s0[h], s1[h]) > m[h] + kTau;
    }
    if (__ballot(need)) {
#pragma unroll
      for (int h = 0; h < R; ++h) {
        float tm = fmaxf(s0[h], s1[h]);
        tm = fmaxf(tm, dpp<kDppRowMirror>(tm));
        tm = fmaxf(tm, __shfl_xor(tm, 16));
        tm = fmaxf(tm, __shfl_xor(tm, 32));
        if (tm > m[h]) {
          const float corr = fast_exp2(m[h] - tm);
          acc[h][0] *= corr;
          acc[h][1] *= corr;
          l[h] *= corr;
          m[h] = tm;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const float mh = m[h] == -INFINITY ? 0.f : m[h];
      const float p0 = fast_exp2(s0[h] - mh);
      const float p1 = fast_exp2(s1[h] - mh);
      l[h] += p0 + p1;
      if (sub == 0) s_p[wave][h][grp] = pack_bf16x2(p0, p1);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const uint4 pa = *reinterpret_cast<const uint4*>(&s_p[wave][h][0]);
      const uint4 pb = *reinterpret_cast<const uint4*>(&s_p[wave][h][4]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[h][0] = dot2_bf16(comp(pa, i), comp(tb.v[0], i), acc[h][0]);
        acc[h][1] = dot2_bf16(comp(pa, i), comp(tb.v[2], i), acc[h][1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[h][0] = dot2_bf16(comp(pb, i), comp(tb.v[1], i), acc[h][0]);
        acc[h][1] = dot2_bf16(comp(pb, i), comp(tb.v[3], i), acc[h][1]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  Tile buf[DEPTH];
#pragma unroll
  for (int j = 0; j < DEPTH - 1; ++j) {
    const int tt = wave + j * W;
    if (tt < ntiles) load(buf[j], tt);
  }
  for (int base = 0; wave + base * W < ntiles; base += DEPTH) {
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const int tt = wave + (base + j) * W;
      if (tt < ntiles) {
        const int tn = tt + (DEPTH - 1) * W;
        if (tn < ntiles) load(buf[(j + DEPTH - 1) % DEPTH], tn);
        compute(buf[j], tt);
      }
    }
  }

  // Wave totals: each 8-lane group summed the weights of its own keys.
#pragma unroll
  for (int h = 0; h < R; ++h) {
    l[h] += __shfl_xor(l[h], 8);
    l[h] += __shfl_xor(l[h], 16);
    l[h] += __shfl_xor(l[h], 32);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      s_m[wave][h] = m[h];
      s_l[wave][h] = l[h];
    }
  }
#pragma unroll
  for (int h = 0; h < R; ++h)
    *reinterpret_cast<float2*>(&s_acc[wave][h][2 * lane]) = make_float2(acc[h][0], acc[h][1]);
  __syncthreads();

  // Merge the W waves: thread handles (head, dim) pairs.
  constexpr int kPairs = R * kHeadDim;
  const bool single = ns == 1;
  float* po = a.part_o + ((int64_t(b) * hkv + g) * a.max_splits + sp) * kPairs;
  float* plse = a.part_lse + ((int64_t(b) * hkv + g) * a.max_splits + sp) * R;
  for (int idx = tid; idx < kPairs; idx += 64 * W) {
    const int h = idx >> 7, d = idx & (kHeadDim - 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float e = s_m[w][h] == -INFINITY ? 0.f : fast_exp2(s_m[w][h] - M);
        L += e * s_l[w][h];
        A += e * s_acc[w][h][d];
      }
    }
    const float o = L > 0.f ? A / L : 0.f;
    if (single) {
      out_bg[idx] = f32_to_bf16(o);
    } else {
      po[idx] = o;
      if (d == 0) plse[h] = L > 0.f ? M + __log2f(L) : -INFINITY;
    }
  }
  if (single) return;

  // Last workgroup of (b, g) combines the ns partials in split order.
  __threadfence();
  __syncthreads();
  uint32_t* ctr = a.counters + int64_t(b) * hkv + g;
  if (tid == 0) {
    const uint32_t ticket = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = ticket == uint32_t(ns - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const float* po0 = a.part_o + (int64_t(b) * hkv + g) * a.max_splits * kPairs;
  const float* pl0 = a.part_lse + (int64_t(b) * hkv + g) * a.max_splits * R;
  for (int idx = tid; idx < kPairs; idx += 64 * W) {
    const int h = idx >> 7;
    float M = -INFINITY;
    for (int k = 0; k < ns; ++k) M = fmaxf(M, pl0[k * R + h]);
    float o = 0.f;
    if (M != -INFINITY) {
      float L = 0.f;
      for (int k = 0; k < ns; ++k) {
        const float lk = pl0[k * R + h];
        const float e = lk == -INFINITY ? 0.f : fast_exp2(lk - M);
        L += e;
        o += e * po0[int64_t(k) * kPairs + idx];
      }
      o /= L;
    }
    out_bg[idx] = f32_to_bf16(o);
  }
  if (tid == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int R, int W>
hipError_t launch_rw(const PoolGeom& pool, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(a.max_splits, pool.num_kv_heads, a.batch);
  hipLaunchKernelGGL((decode_kernel<R, W, 2>), grid, dim3(64 * W), 0, stream, pool, a);
  return hipGetLastError();
}

template <int R>
hipError_t launch_r(const PoolGeom& pool, const DecodeArgs& a, hipStream_t stream) {
  switch (a.waves) {
    case 1: return launch_rw<R, 1>(pool, a, stream);
    case 2: return launch_rw<R, 2>(pool, a, stream);
    case 4: return launch_rw<R, 4>(pool, a, stream);
    case 8: return launch_rw<R, 8>(pool, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

DecodeWorkspace decode_workspace_layout(int32_t batch, int32_t num_kv_heads, int32_t group, int32_t max_splits) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  DecodeWorkspace w;
  const size_t units = size_t(batch) * num_kv_heads;
  w.counters_off = 0;
  w.part_o_off = up(units * sizeof(uint32_t));
  w.part_lse_off = w.part_o_off + up(units * max_splits * group * kHeadDim * sizeof(float));
  w.total = w.part_lse_off + up(units * max_splits * group * sizeof(float));
  return w;
}

hipError_t launch_decode(const PoolGeom& pool, const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (a.split_tokens > kMaxSplitTokens) return hipErrorInvalidValue;
  switch (a.num_q_heads / pool.num_kv_heads) {
    case 1: return launch_r<1>(pool, a, stream);
    case 2: return launch_r<2>(pool, a, stream);
    case 4: return launch_r<4>(pool, a, stream);
    case 8: return launch_r<8>(pool, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pgqa
