// One attention launch for a whole mixed serving step: decode rows, chunked-
// prefill slices and b x (k+1) speculative-verify rows together, from a work
// list built on the host (gfx950).
//
// Page "perf: Qwen3 offline inference - hybrid attention backend, fused
// rms_norm_rope, chunked prefill + prompt-lookup spec decoding", Summary items 1
// (decode and prefill routed by the host over one paged cache), 3 (routing
// decided on the host, no device synchronisation) and 4 (chunked prefill fused
// with the b x (k+1) verify shape in one forward).
//
// The host planner (pgqa_plan_mixed) turns the segments' host-side lengths into
// a list of work items, 8 int32 each (MixedItem), that the caller uploads with
// its other per-step metadata.  Workgroup i of the attention launch takes item i:
//   * wide    (a segment with more than 16 query rows per kv head: a prefill
//             slice): 128 query rows of one kv head over one key split, the
//             chunk kernels' wide body (chunk_common.hpp), MFMA-bound;
//   * column  (at most 16 rows per kv head: decode rows, verify rows): the
//             segment's (token, head) rows of one kv head as the 16 columns of
//             v_mfma_f32_16x16x32_bf16 products over one key split, 4 waves
//             taking 32-key steps in turn, K/V loaded straight into operand
//             registers; HBM-bound.
// Wide items are listed with the kv head fastest, so that workgroups dealt
// round-robin to the 8 XCDs keep one kv head's K/V of a slice in one L2, and
// column items longest first; the two kinds alternate in runs of num_cus, so
// that the two workgroups sharing a CU start on one item of each kind.  Split
// partials go to one [split][token][head] layout, merged by one combine launch
// whose items (8 rows each) follow the attention items in the same list.
//
// Every item carries the host's copy of its segment's offset, length and key
// count; the device compares them with query_start_loc and context_lens, and a
// mismatch (or any other bad metadata) flags the pool's error word and zeroes
// the item's rows instead of computing them.
#include "chunk_common.hpp"

namespace pgqa {
namespace {

constexpr int kKindWide = 0, kKindColumn = 1, kKindCombine = 2;
constexpr int kColW = 4;        // waves of a column item
constexpr int kColumns = 16;    // MFMA columns: (token, head) rows of a column segment
constexpr float kColTau = 8.0f; // log2 headroom before a column's running max is raised

struct MixedItem {
  int s, kind, g, grp, sp, q0, qlen, n;  // grp: wide row group / first combine row; sp: split / combine split count
};

__device__ __forceinline__ MixedItem load_item(const int32_t* items, int64_t idx) {
  const int4* p = reinterpret_cast<const int4*>(items + idx * kMixedItemInts);
  const int4 x = p[0], y = p[1];
  auto u = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  return MixedItem{u(x.x), u(x.y), u(x.z), u(x.w), u(y.x), u(y.y), u(y.z), u(y.w)};
}

// The segment as the device sees it, and whether the host item agrees with it.
__device__ __forceinline__ bool item_matches(const ChunkArgs& a, const PoolGeom& pool, const MixedItem& it, int r,
                                             SegInfo& si) {
  if (it.s < 0 || it.s >= a.num_segments || it.g < 0 || it.g >= pool.num_kv_heads) return false;
  si = seg_info(a, it.s, r, pool.block_size);
  return !si.bad && si.q0 == it.q0 && si.qlen == it.qlen && si.n == it.n && it.qlen > 0;
}

// Zero rows [rho0, rho1) of kv head g of the item's segment (host offsets, used
// only when they lie inside the call's query rows).
template <int R>
__device__ __forceinline__ void zero_item_rows(const ChunkArgs& a, const MixedItem& it, int rho0, int rho1) {
  if (it.q0 < 0 || it.qlen < 0 || int64_t(it.q0) + it.qlen > a.total_q || it.g < 0 || it.g * R >= a.num_q_heads)
    return;
  rho1 = min(rho1, it.qlen * R);
  for (int64_t i = int64_t(rho0) * kHeadDim + threadIdx.x; i < int64_t(rho1) * kHeadDim; i += blockDim.x) {
    const int rho = int(i >> 7), d = int(i & (kHeadDim - 1));
    a.out[((int64_t(it.q0) + rho / R) * a.num_q_heads + it.g * R + rho % R) * kHeadDim + d] = 0;
  }
}

// ---------------------------------------------------------------- column body
struct ColumnStep {
  uint4 k[2][4];  // score product u, dim slice s: key row of the lane, dims 32s + 8c .. +7
  uint4 v[8];     // PV product t: dim 16t + col, keys 8c .. 8c+7
  int ok;         // bit h: block id of the step's 16-key half h is valid
};

// LDS of a column item: each wave's unnormalised accumulators [16][128] and
// its per-column max and weight sum, for the final merge of the waves.
struct ColumnLds {
  float* acc01;  // waves 0, 1: [2][16][128]
  float* acc23;  // waves 2, 3
  float* m;      // [kColW][16]
  float* l;      // [kColW][16]
  // wave w's accumulators (no runtime-indexed pointer array: that would live in LDS)
  __device__ __forceinline__ float* acc(int w) const { return (w < 2 ? acc01 : acc23) + (w & 1) * kColumns * kHeadDim; }
};

// One column item: rows (token col / R, head g R + col % R) of segment s,
// col < qlen R <= 16, over keys [k0, k1) of its n keys, k0 = sp * split; each
// column sees the keys up to its token's position n - qlen + col / R.
// Operand layouts of v_mfma_f32_16x16x32_bf16 (c = lane / 16, col = lane % 16):
//   * S^T = K Q^T, two products per 32-key step (u = 0, 1), four 32-dim slices
//     each.  Row m of product u is key 8(m/4) + 4u + m%4 of the step, so D[j]
//     of product u in lane l is key 8c + 4u + j: the lane's 8 weights are keys
//     8c .. 8c+7 in order.
//   * O^T += V^T P^T, eight products (dims 16t .. 16t+15): the weights above
//     are the lane's B operand, and its A operand (dim 16t + col, keys
//     8c .. 8c+7) is 16 contiguous bytes of a 16-slot V^T piece of the cache.
// Scores are in log2 units; the running max rises only when a score exceeds it
// by more than kColTau.
template <int R>
__device__ __forceinline__ void column_body(PoolGeom& pool, const ChunkArgs& a, int s, int g, int sp, int split,
                                            int q0, int qlen, int n, const ColumnLds& lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, c = lane >> 4;
  const int hq = a.num_q_heads, hkv = pool.num_kv_heads, bs = pool.block_size;
  const int k0 = sp * split;
  const int ns = cdiv(n, split);
  const int k1 = min(n, k0 + split);
  // Block ids and q issued together.  Lane i fetches the block id of half
  // (i & 1) of the wave's step i / 2 (step wave + (i / 2) kColW of the split);
  // a split has at most 32 steps per wave.
  int32_t lane_blk = -1;
  {
    const int off = (wave + (lane >> 1) * kColW) * 32 + (lane & 1) * 16;
    const int64_t entry = (int64_t(k0) + off) / bs;
    if (off < split && entry < a.bt_stride) lane_blk = a.bt[int64_t(s) * a.bt_stride + entry];
  }
  const int tcol = col / R;
  const bool cvalid = tcol < qlen;
  // q through a buffer descriptor of the segment's rows: an unused column
  // reads past the end and gets zeros, so the loads are unconditional and no
  // select follows them (a select after plain loads let the compiler sink them
  // into per-dword loads under branches, which the wait before the first step
  // could not skip).
  uint4 qb[4];
  {
    const auto qrsrc = buffer_rsrc(a.q + int64_t(q0) * hq * kHeadDim,
                                   __builtin_amdgcn_readfirstlane(uint32_t(qlen) * uint32_t(hq) * (2u * kHeadDim)));
    const uint32_t qoff = cvalid ? uint32_t(((tcol * hq + g * R + col % R) * kHeadDim + 8 * c) * 2) : 0x80000000u;
#pragma unroll
    for (int t = 0; t < 4; ++t) qb[t] = load_buf<false>(qrsrc, qoff + 64 * t);
  }
  const int klim = cvalid ? min(k1, n - qlen + tcol + 1) : k0;  // keys the lane's column attends

  const int64_t tstride = tile_elems(pool);
  const int64_t bstride = tstride * hkv;
  const uint16_t* pool_g = pool.kv + int64_t(g) * tstride;
  const int nsteps = (k1 - k0 + 31) >> 5;
  // Lane offsets inside a 16-key half: K row of product 0 (product 1 is 4 rows
  // on) in half col / 8; V^T keys 8(c & 1) .. of dim col in half c / 2.
  const int khalf = col >> 3, vhalf = c >> 1;
  const int k_off = (8 * ((col >> 2) & 1) + (col & 3)) * kHeadDim + 8 * c;
  const int v_off = bs * kHeadDim + col * kVSub + 8 * (c & 1);

  auto load = [&](ColumnStep& ms, int i) {
    const int key = k0 + (wave + i * kColW) * 32;
    const int32_t r0 = __builtin_amdgcn_readlane(lane_blk, 2 * i);
    const int32_t r1 = __builtin_amdgcn_readlane(lane_blk, 2 * i + 1);
    const bool ok0 = unsigned(r0) < unsigned(pool.num_blocks), ok1 = unsigned(r1) < unsigned(pool.num_blocks);
    ms.ok = (ok0 ? 1 : 0) | (ok1 ? 2 : 0);
    const uint16_t* base0 = pool_g + int64_t(ok0 ? r0 : 0) * bstride + ((key & (bs - 1)) >> 4) * (16 * kHeadDim);
    const uint16_t* base1 =
        pool_g + int64_t(ok1 ? r1 : 0) * bstride + (((key + 16) & (bs - 1)) >> 4) * (16 * kHeadDim);
    const uint16_t* kp = (khalf ? base1 : base0) + k_off;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int t = 0; t < 4; ++t) ms.k[u][t] = *reinterpret_cast<const uint4*>(kp + 4 * u * kHeadDim + 32 * t);
    }
    const uint16_t* vp = (vhalf ? base1 : base0) + v_off;
#pragma unroll
    for (int t = 0; t < 8; ++t) ms.v[t] = *reinterpret_cast<const uint4*>(vp + 16 * t * kVSub);
  };

  f32x4_t acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // of column col; the four lane groups agree on m
  bool bad_blk = false;
  const float cs = a.qk_scale_log2;

  auto compute = [&](ColumnStep& ms, int i) {
    const int key = k0 + (wave + i * kColW) * 32;
    // a half past the split end is never attended: its block id is not checked
    bad_blk |= !(ms.ok & 1) || (key + 16 < k1 && !(ms.ok & 2));
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int t = 0; t < 4; ++t) s0 = mfma16(ms.k[0][t], qb[t], s0);
#pragma unroll
    for (int t = 0; t < 4; ++t) s1 = mfma16(ms.k[1][t], qb[t], s1);
    // the lane's keys key + 8c .. +7: how many hold data (nv) and how many its
    // column attends (na)
    const bool okc = (ms.ok >> vhalf) & 1;
    const int nv = okc ? min(max(k1 - (key + 8 * c), 0), 8) : 0;
    const int na = okc ? min(max(klim - (key + 8 * c), 0), 8) : 0;
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = j < na ? s0[j] * cs : -INFINITY;
      x[4 + j] = 4 + j < na ? s1[j] * cs : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
    if (__ballot(mx > m + kColTau)) {
      float tm = fmaxf(mx, __shfl_xor(mx, 16));
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      if (tm > m + kColTau) {  // only a column whose own scores left the headroom re-bases
        const float corr = fast_exp2(m - tm);
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[t] *= corr;
        l *= corr;
        m = tm;
      }
    }
    const float mh = m == -INFINITY ? 0.f : m;
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = fast_exp2(x[j] - mh);
      l += p[j];
    }
    const uint4 pb = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                pack_bf16x2(p[6], p[7]));
    // V of keys past the split end (or of a bad block) is zeroed: their weight
    // is 0, but the slots may hold any bits, and 0 * NaN would poison O.
    if (key + 32 > k1 || ms.ok != 3) {
      const uint32_t m0 = nv > 1 ? 0xffffffffu : nv > 0 ? 0x0000ffffu : 0u;
      const uint32_t m1 = nv > 3 ? 0xffffffffu : nv > 2 ? 0x0000ffffu : 0u;
      const uint32_t m2 = nv > 5 ? 0xffffffffu : nv > 4 ? 0x0000ffffu : 0u;
      const uint32_t m3 = nv > 7 ? 0xffffffffu : nv > 6 ? 0x0000ffffu : 0u;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        ms.v[t].x &= m0;
        ms.v[t].y &= m1;
        ms.v[t].z &= m2;
        ms.v[t].w &= m3;
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = mfma16(ms.v[t], pb, acc[t]);
  };

  const int my_steps = nsteps > wave ? (nsteps - wave + kColW - 1) / kColW : 0;
  if (my_steps > 0) {
    auto at = [&](int i) { return min(i, my_steps - 1); };
    ColumnStep ta, tb;
    load(ta, 0);
    for (int i = 0; i < my_steps; i += 2) {
      load(tb, at(i + 1));
      compute(ta, i);
      load(ta, at(i + 2));
      if (i + 1 < my_steps) compute(tb, i + 1);
    }
  }
  if (bad_blk && lane == 0) raise_error(pool.err, kErrBlockId);

  // Column totals (each lane group summed the weights of its own keys), then
  // the merge of the 4 waves' states: bf16 rows when the segment has one
  // split, else normalised partials and their lse (log2 units).
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const int ncols = qlen * R;
  if (col < ncols) {
    if (c == 0) {
      lds.m[wave * kColumns + col] = m;
      lds.l[wave * kColumns + col] = l;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
      *reinterpret_cast<float4*>(lds.acc(wave) + col * kHeadDim + 16 * t + 4 * c) =
          make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  }
  __syncthreads();
  for (int idx = tid; idx < ncols * kHeadDim; idx += 64 * kColW) {
    const int h = idx >> 7, d = idx & (kHeadDim - 1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kColW; ++w) M = fmaxf(M, lds.m[w * kColumns + h]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kColW; ++w) {
        const float mw = lds.m[w * kColumns + h];
        const float e = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
        L += e * lds.l[w * kColumns + h];
        A += e * lds.acc(w)[h * kHeadDim + d];
      }
    }
    const float o = L > 0.f ? A / L : 0.f;
    const int64_t row = (int64_t(q0) + h / R) * hq + g * R + h % R;  // output row (token, head)
    if (ns == 1) {
      a.out[row * kHeadDim + d] = f32_to_bf16(o);
    } else {
      const int64_t prow = int64_t(sp) * a.total_q * hq + row;
      a.part_o[prow * kHeadDim + d] = o;
      if (d == 0) a.part_lse[prow] = L > 0.f ? M + __log2f(L) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------- kernels
template <int R>
__global__ __launch_bounds__(kWideThreads, 2) void mixed_kernel(PoolGeom pool, ChunkArgs a) {
  const MixedItem it = load_item(a.items, blockIdx.x);
  __shared__ __align__(1024) uint8_t s_st0[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st1[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st2[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st3[kStageBytes];
  SegInfo si{};
  si.err = kErrQuery;
  const bool wide = it.kind == kKindWide;
  const int split = wide ? a.split_wide : a.split_short;
  bool ok = (wide || it.kind == kKindColumn) && item_matches(a, pool, it, R, si) && it.sp >= 0 &&
            it.sp < a.max_splits;
  if (ok) {
    // the item's rows and keys exist on the device too
    const int kend = wide ? wide_kend(si, it.grp, R) : si.n;
    ok = it.sp < cdiv(kend, split) && (wide ? it.grp >= 0 && it.grp < wide_groups(si) && si.tiles > 0
                                            : si.qlen * R <= kColumns);
  }
  if (!ok) {
    if (threadIdx.x == 0) raise_error(pool.err, si.bad ? si.err : kErrQuery);
    if (it.sp == 0 && it.kind != kKindCombine)
      zero_item_rows<R>(a, it, wide ? it.grp * kRows * kWideTiles : 0,
                        wide ? (it.grp + 1) * kRows * kWideTiles : kColumns);
    return;
  }
  if (wide) {
    wide_body<R>(pool, a, si, it.s, it.g, it.grp, it.sp, split, WideLds{s_st0, s_st1, s_st2, s_st3});
  } else {
    // the 4 waves' [16][128] accumulators fill two stages; the maxima and sums a third
    ColumnLds cl;
    cl.acc01 = reinterpret_cast<float*>(s_st0);
    cl.acc23 = reinterpret_cast<float*>(s_st1);
    cl.m = reinterpret_cast<float*>(s_st2);
    cl.l = cl.m + kColW * kColumns;
    column_body<R>(pool, a, it.s, it.g, it.sp, split, si.q0, si.qlen, si.n, cl);
  }
}

// Combine items: rows grp .. grp + 7 of segment s and kv head g, each merged
// over its sp split partials (32 lanes per row).  Items whose segment does not
// match the device metadata are skipped (the attention items zeroed the rows).
//
// Items of at most kCombineFast splits issue their partial loads before the
// segment metadata arrives, addressed from the item's own copy of the segment
// offset, so the merge waits one round trip after the item instead of two.
// The loads go through buffer descriptors over the partials: an address
// outside them reads zeros.  The rows are merged only once the item matches the
// metadata, and then those addresses are the ones combine_row would read.
template <int R>
__global__ __launch_bounds__(256) void mixed_combine_kernel(PoolGeom pool, ChunkArgs a) {
  const MixedItem it = load_item(a.items, int64_t(a.num_items) + blockIdx.x);
  __shared__ float s_w[kCombineRows][kCombineChunk];
  const int row = threadIdx.x >> 5, j = threadIdx.x & 31;
  const int ns = it.sp;
  const int64_t stride = int64_t(a.total_q) * a.num_q_heads;  // partial rows per split
  const int64_t lse_bytes = stride * a.max_splits * 4;
  const bool early = it.kind == kKindCombine && ns >= 2 && ns <= kCombineFast && ns <= a.max_splits &&
                     lse_bytes * kHeadDim < 0x7fffffff;
  float4 v[kCombineFast];
  float lk = -INFINITY;
  if (early) {
    const int rho_h = it.grp + row;
    const int64_t orow_h = (int64_t(it.q0) + rho_h / R) * a.num_q_heads + it.g * R + rho_h % R;
    const bool in = rho_h >= 0 && orow_h >= 0 && orow_h < stride;
    const auto ro = buffer_rsrc(a.part_o, uint32_t(lse_bytes * kHeadDim));
    const auto rl = buffer_rsrc(a.part_lse, uint32_t(lse_bytes));
    const uint32_t o0 = in ? uint32_t((orow_h * kHeadDim + 4 * j) * 4) : 0x80000000u;
    const uint32_t sstep = uint32_t(stride * kHeadDim * 4);
#pragma unroll
    for (int k = 0; k < kCombineFast; ++k) {
      const u32x4 x = k < ns ? __builtin_amdgcn_raw_buffer_load_b128(ro, o0 + k * sstep, 0, 0) : u32x4{0, 0, 0, 0};
      v[k] = make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
    }
    if (j < ns && in)
      lk = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rl, uint32_t((orow_h + j * stride) * 4), 0, 0));
  }
  SegInfo si{};
  if (it.kind != kKindCombine || !item_matches(a, pool, it, R, si) || ns < 2 || ns > a.max_splits) {
    if (threadIdx.x == 0 && it.kind != kKindCombine) raise_error(pool.err, kErrQuery);
    return;
  }
  const int rho = it.grp + row;
  const bool row_ok = rho >= 0 && rho < si.rows;
  const int64_t orow = (int64_t(si.q0) + rho / R) * a.num_q_heads + it.g * R + rho % R;
  if (early) {
    merge_row_fast(v, row_ok ? lk : -INFINITY, ns, row_ok, a.out + orow * kHeadDim + 4 * j);
    return;
  }
  combine_row(a, orow, ns, row_ok, j, s_w[row], a.out + orow * kHeadDim + 4 * j);
}

template <int R>
hipError_t launch_mixed_r(const PoolGeom& pool, const ChunkArgs& a, int num_combine, hipStream_t stream) {
  if (a.num_items > 0) {
    hipLaunchKernelGGL((mixed_kernel<R>), dim3(a.num_items), dim3(kWideThreads), 0, stream, pool, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (num_combine > 0) {
    hipLaunchKernelGGL((mixed_combine_kernel<R>), dim3(num_combine), dim3(256), 0, stream, pool, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_mixed(const PoolGeom& pool, const ChunkArgs& a, int32_t num_combine, hipStream_t stream) {
  if (a.num_segments == 0 || a.total_q == 0) return hipSuccess;
  if (a.split_wide > 4096 || a.split_wide % kStep || a.split_short > 4096 || a.split_short % 64)
    return hipErrorInvalidValue;
  switch (a.num_q_heads / pool.num_kv_heads) {
    case 1: return launch_mixed_r<1>(pool, a, num_combine, stream);
    case 2: return launch_mixed_r<2>(pool, a, num_combine, stream);
    case 4: return launch_mixed_r<4>(pool, a, num_combine, stream);
    case 8: return launch_mixed_r<8>(pool, a, num_combine, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pgqa
