// Causal chunk attention over the paged cache: chunked-prefill slices and
// b x (k+1) speculative-verify rows (gfx950, MFMA).
//
// Page "perf: Qwen3 offline inference - hybrid attention backend, fused
// rms_norm_rope, chunked prefill + prompt-lookup spec decoding", Summary items 1
// and 4: prefill and mixed batches run a varlen attention kernel over the same
// paged cache that decode reads, a long prompt is fed in chunks, and
// speculative verification runs a fixed b x (k+1) query shape.  Segment s
// holds q_len query tokens at the end of its n keys; query i sits at position
// n - q_len + i and sees keys 0 .. that position (bottom-right causal).
//
// Unlike decode, QK^T and PV here are dense contractions: a 32-row query tile
// against a 32-key step is a 32x32x128 and a 128x32x32 product, so both run on
// v_mfma_f32_32x32x16_bf16.
//
// Work decomposition.  One workgroup per (segment, kv head g, row tile, key
// split).  The 32 rows of a tile are (token, head-in-group) pairs, row
// rho = token * r + hh, so the r query heads that share kv head g share every
// K/V operand.  The W waves of the workgroup take the split's 32-key steps in
// turn (wave w: steps w, w+W, ...) and merge their softmax states at the end.
//
// Operand layouts (verified on the hardware): lane l supplies A[m][k] with
// m = l%32, k = 8(l/32)+j and B[k][n] with n = l%32; D[i] of lane l is
// row 8(i/4)+4(l/32)+i%4, column l%32.
//   * S^T = K Q^T (M = keys, N = query rows, K = dims).  MFMA row m holds key
//     pi(m) of the step, pi swapping bits 2 and 3 of m; then D[i] of lane l is
//     key 16(i/8) + 8(l/32) + i%8, so the 8 weights a lane needs as its PV
//     operand for keys 16s + 8(l/32) .. +7 are its own D[8s .. 8s+7].
//   * O^T += V^T P^T (M = dims, N = query rows, K = keys): the cache keeps V
//     transposed per block, so a lane's 8 keys of one dim are 16 contiguous
//     bytes.  Nothing is transposed at run time.
//   * dims of the S product are split between the lane halves as
//     (l/32)*64 + 8*kstep + j, so a lane reads 128 contiguous bytes of its K
//     row and of its q row.
#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {
namespace {

constexpr float kTau = 8.0f;            // log2 headroom before the running max is raised
constexpr int kRows = 32;               // query rows per tile
constexpr int kStep = 32;               // keys per step

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

struct Step {
  uint4 k[8];     // K row pi(l%32), dims (l/32)*64 + 8ks .. +8 for ks = 0..7
  uint4 v[2][4];  // v[s16][dt]: V^T row 32dt + l%32, keys 16 s16 + 8(l/32) .. +7
  int ok_a, ok_b; // block ids of the step's two 16-key groups were in range
};

// Zero the bf16 elements of `x` (8 consecutive keys starting at `key`) at or past `end`.
__device__ __forceinline__ void zero_from(uint4& x, int key, int end) {
  auto keep = [&](int t) -> uint32_t {
    const int k = key + 2 * t;
    return k + 1 < end ? 0xffffffffu : k < end ? 0x0000ffffu : 0u;
  };
  x.x &= keep(0);
  x.y &= keep(1);
  x.z &= keep(2);
  x.w &= keep(3);
}

template <int R, int W>
__global__ __launch_bounds__(64 * W) void chunk_kernel(PoolGeom pool, ChunkArgs a) {
  const int sp = blockIdx.x, rt = blockIdx.y;
  const int hkv = pool.num_kv_heads, bs = pool.block_size, hq = a.num_q_heads;
  const int s = blockIdx.z / hkv, g = blockIdx.z - s * hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  __shared__ float s_m[W][kRows];
  __shared__ float s_l[kRows];
  __shared__ float s_acc[kRows][kHeadDim + 1];

  const int q0 = a.qsl[s], q1 = a.qsl[s + 1];
  const int n = a.ctx[s];
  const int qlen = q1 - q0;
  const bool rows_ok = q0 >= 0 && q1 >= q0 && q1 <= a.total_q;
  const bool bad = !rows_ok || qlen > a.max_q_len || n < qlen || n > a.max_ctx ||
                   int64_t(n) > int64_t(a.bt_stride) * bs;
  if (bad) {
    if (sp == 0 && rt == 0) {
      if (tid == 0) raise_error(pool.err, !rows_ok || qlen > a.max_q_len || n < qlen ? kErrQuery : kErrContext);
      if (rows_ok)
        for (int64_t i = tid; i < int64_t(qlen) * R * kHeadDim; i += 64 * W) {
          const int64_t tok = i / (R * kHeadDim), rem = i - tok * (R * kHeadDim);
          a.out[((q0 + tok) * hq + g * R) * kHeadDim + rem] = 0;
        }
    }
    return;
  }
  const int rows = qlen * R;
  if (rt * kRows >= rows) return;
  const int tok_last = min(qlen, (rt * kRows + kRows) / R) - 1;
  const int prefix = n - qlen;
  const int kend = prefix + tok_last + 1;      // keys this tile may attend
  const int ns = (kend + a.split_tokens - 1) / a.split_tokens;
  if (sp >= ns) return;
  const int k0 = sp * a.split_tokens;
  const int k1 = min(kend, k0 + a.split_tokens);

  // Block ids of this wave's 16-key groups, one per lane: lane j holds group
  // 2*(wave + (j/2)*W) + j%2 of the split (the two halves of step wave+(j/2)*W).
  int32_t lane_blk = -1;
  {
    const int step = wave + (lane >> 1) * W;
    const int key_off = step * kStep + 16 * (lane & 1);
    const int64_t entry = (int64_t(k0) + key_off) / bs;
    if (key_off < a.split_tokens && entry < a.bt_stride) lane_blk = a.bt[int64_t(s) * a.bt_stride + entry];
  }

  // This lane's query row: rho = rt*32 + col -> (token, head in group).
  const int rho = rt * kRows + col;
  const bool row_ok = rho < rows;
  const int tok = rho / R, hh = rho - tok * R;
  const int qpos = prefix + tok;                // absolute position of the row's token
  uint4 qv[8];
  {
    const uint16_t* qp = a.q + ((int64_t(q0) + tok) * hq + g * R + hh) * kHeadDim + half * 64;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qv[ks] = row_ok ? *reinterpret_cast<const uint4*>(qp + 8 * ks) : make_uint4(0, 0, 0, 0);
  }

  const int64_t tstride = tile_elems(pool);
  const int64_t bstride = tstride * hkv;
  const uint16_t* pool_g = pool.kv + int64_t(g) * tstride;
  const int nsteps = (k1 - k0 + kStep - 1) / kStep;
  const int my_steps = nsteps > wave ? (nsteps - wave + W - 1) / W : 0;
  const int mrow = col;                         // MFMA row of this lane's K operand
  const int kperm = (mrow & ~12) | ((mrow & 4) << 1) | ((mrow & 8) >> 1);   // pi(m): swap bits 2, 3

  auto load = [&](Step& st, int i) {
    const int stp = wave + i * W;
    const int key0 = k0 + stp * kStep;
    const int32_t ra = __builtin_amdgcn_readlane(lane_blk, 2 * i);
    const int32_t rb = __builtin_amdgcn_readlane(lane_blk, 2 * i + 1);
    st.ok_a = unsigned(ra) < unsigned(pool.num_blocks);
    st.ok_b = unsigned(rb) < unsigned(pool.num_blocks);
    const int32_t ba = st.ok_a ? ra : 0, bb = st.ok_b ? rb : 0;
    // K: this lane's row pi(mrow) of the step
    const int kk = key0 + kperm;
    const uint16_t* kp = pool_g + int64_t(kperm >= 16 ? bb : ba) * bstride + (kk & (bs - 1)) * kHeadDim + half * 64;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) st.k[ks] = *reinterpret_cast<const uint4*>(kp + 8 * ks);
    // V^T: rows 32dt + col, 8 keys per half
#pragma unroll
    for (int s16 = 0; s16 < 2; ++s16) {
      const int kv0 = key0 + 16 * s16 + 8 * half;
      const uint16_t* vp = pool_g + int64_t(s16 ? bb : ba) * bstride + int64_t(bs) * kHeadDim +
                           int64_t(col) * bs + (kv0 & (bs - 1));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) st.v[s16][dt] = *reinterpret_cast<const uint4*>(vp + int64_t(32 * dt) * bs);
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16_t{};
  float m = -INFINITY, l = 0.f;
  bool bad_blk = false;

  auto compute = [&](Step& st, int stp) {
    const int key0 = k0 + stp * kStep;
    // a group only counts as a bad block id if it holds keys this split reads
    bad_blk |= (!st.ok_a && key0 < k1) || (!st.ok_b && key0 + 16 < k1);
    // V entries past the split end, or of a bad block: weight 0, but the bits
    // may be anything (0 * NaN would poison O), so zero them.
    if (key0 + kStep > k1 || !st.ok_a || !st.ok_b) {
#pragma unroll
      for (int s16 = 0; s16 < 2; ++s16) {
        const bool okb = s16 ? st.ok_b : st.ok_a;
        const int kv0 = key0 + 16 * s16 + 8 * half;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) zero_from(st.v[s16][dt], kv0, okb ? k1 : kv0);
      }
    }
    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) sacc = mfma32(st.k[ks], qv[ks], sacc);
    float sv[16];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + 16 * (i >> 3) + 8 * half + (i & 7);
      const bool okk = (i < 8 ? st.ok_a : st.ok_b) && row_ok && key < k1 && key <= qpos;
      sv[i] = okk ? sacc[i] * a.qk_scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__ballot(mx > m + kTau)) {
      const float mn = fmaxf(m, mx);
      const float corr = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= corr;
      l *= corr;
      m = mn;
    }
    const float msafe = m == -INFINITY ? 0.f : m;
    uint4 pb[2];
#pragma unroll
    for (int s16 = 0; s16 < 2; ++s16) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = fast_exp2(sv[8 * s16 + j] - msafe);
        l += p[j];
      }
      pb[s16] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                           pack_bf16x2(p[6], p[7]));
    }
#pragma unroll
    for (int s16 = 0; s16 < 2; ++s16) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] = mfma32(st.v[s16][dt], pb[s16], o[dt]);
    }
  };

  if (my_steps > 0) {
    auto at = [&](int i) { return min(i, my_steps - 1); };
    Step sa, sb;
    load(sa, 0);
    for (int i = 0; i < my_steps; i += 2) {
      load(sb, at(i + 1));
      compute(sa, wave + i * W);
      load(sa, at(i + 2));
      if (i + 1 < my_steps) compute(sb, wave + (i + 1) * W);
    }
  }
  if (bad_blk && lane == 0) raise_error(pool.err, kErrBlockId);

  // Merge the W waves' states per query row, in wave order (deterministic).
  l += __shfl_xor(l, 32);
  if (half == 0) s_m[wave][col] = m;
  __syncthreads();
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, s_m[w][col]);
  const float sc = (m == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2(m - M);
  for (int w = 0; w < W; ++w) {
    if (wave == w) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = 32 * dt + 8 * (i >> 2) + 4 * half + (i & 3);
          const float v = o[dt][i] * sc;
          s_acc[col][d] = w == 0 ? v : s_acc[col][d] + v;
        }
      }
      if (half == 0) s_l[col] = w == 0 ? l * sc : s_l[col] + l * sc;
    }
    __syncthreads();
  }

  // Normalise and store: thread handles (row, dim) pairs of the tile.
  const bool single = ns == 1;
  for (int idx = tid; idx < kRows * kHeadDim; idx += 64 * W) {
    const int r = idx >> 7, d = idx & (kHeadDim - 1);
    const int rr = rt * kRows + r;
    if (rr >= rows) continue;
    const int t = rr / R, h2 = rr - t * R;
    const float L = s_l[r];
    const float ov = L > 0.f ? s_acc[r][d] / L : 0.f;
    const int64_t qrow = int64_t(q0) + t;
    if (single) {
      a.out[(qrow * hq + g * R + h2) * kHeadDim + d] = f32_to_bf16(ov);
    } else {
      float mr = -INFINITY;
#pragma unroll
      for (int w = 0; w < W; ++w) mr = fmaxf(mr, s_m[w][r]);
      const int64_t prow = ((int64_t(g) * a.max_splits + sp) * a.total_q + qrow) * R + h2;
      a.part_o[prow * kHeadDim + d] = ov;
      if (d == 0) a.part_lse[prow] = L > 0.f ? mr + __log2f(L) : -INFINITY;
    }
  }
}

// Log-sum-exp combine of chunk partials: one workgroup per (query token,
// query head), one thread per dim; splits merged in order.
__global__ __launch_bounds__(kHeadDim) void chunk_combine_kernel(PoolGeom pool, ChunkArgs a) {
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int hkv = pool.num_kv_heads, r = a.num_q_heads / hkv;
  const int g = h / r, hh = h - g * r;
  // segment of token t: last s with qsl[s] <= t (qsl ascending)
  int lo = 0, hi = a.num_segments;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.qsl[mid] <= t) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int q0 = a.qsl[s], q1 = a.qsl[s + 1], n = a.ctx[s];
  const int qlen = q1 - q0;
  if (t < q0 || t >= q1 || q0 < 0 || q1 > a.total_q || qlen > a.max_q_len || n < qlen || n > a.max_ctx ||
      int64_t(n) > int64_t(a.bt_stride) * pool.block_size)
    return;
  const int rho = (t - q0) * r + hh;
  const int rt = rho / kRows;
  const int tok_last = min(qlen, (rt * kRows + kRows) / r) - 1;
  const int kend = n - qlen + tok_last + 1;
  const int ns = (kend + a.split_tokens - 1) / a.split_tokens;
  if (ns <= 1) return;
  const int64_t stride = int64_t(a.total_q) * r;     // partial rows per split
  const int64_t base = (int64_t(g) * a.max_splits) * stride + int64_t(t) * r + hh;
  float M = -INFINITY;
  for (int k = 0; k < ns; ++k) M = fmaxf(M, a.part_lse[base + k * stride]);
  float o = 0.f;
  if (M != -INFINITY) {
    float L = 0.f;
    for (int k = 0; k < ns; ++k) {
      const float lk = a.part_lse[base + k * stride];
      const float e = lk == -INFINITY ? 0.f : fast_exp2(lk - M);
      L += e;
      o += e * a.part_o[(base + k * stride) * kHeadDim + d];
    }
    o /= L;
  }
  a.out[(int64_t(t) * a.num_q_heads + h) * kHeadDim + d] = f32_to_bf16(o);
}

template <int R, int W>
hipError_t launch_rw(const PoolGeom& pool, const ChunkArgs& a, hipStream_t stream) {
  const dim3 grid(a.max_splits, a.q_tiles, a.num_segments * pool.num_kv_heads);
  hipLaunchKernelGGL((chunk_kernel<R, W>), grid, dim3(64 * W), 0, stream, pool, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL(chunk_combine_kernel, dim3(a.total_q, a.num_q_heads), dim3(kHeadDim), 0, stream, pool, a);
  return hipGetLastError();
}

}  // namespace

ChunkWorkspace chunk_workspace_layout(int32_t total_q, int32_t num_q_heads, int32_t max_splits) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  ChunkWorkspace w;
  if (max_splits <= 1) {
    w.part_o_off = w.part_lse_off = w.total = 0;
    return w;
  }
  const size_t rows = size_t(max_splits) * total_q * num_q_heads;  // Hkv * r == Hq
  w.part_o_off = 0;
  w.part_lse_off = up(rows * kHeadDim * sizeof(float));
  w.total = w.part_lse_off + up(rows * sizeof(float));
  return w;
}

hipError_t launch_chunk(const PoolGeom& pool, const ChunkArgs& a, hipStream_t stream) {
  if (a.num_segments == 0 || a.total_q == 0) return hipSuccess;
  if (a.split_tokens > 64 * 16 * 4) return hipErrorInvalidValue;
  switch (a.num_q_heads / pool.num_kv_heads) {
    case 1: return launch_rw<1, 4>(pool, a, stream);
    case 2: return launch_rw<2, 4>(pool, a, stream);
    case 4: return launch_rw<4, 4>(pool, a, stream);
    case 8: return launch_rw<8, 4>(pool, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pgqa
