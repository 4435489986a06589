// Shared by the chunk kernels (chunk.hip) and the mixed-step kernel
// (mixed.hip): v_mfma_f32_32x32x16_bf16 helpers, the device-side segment
// checks, the per-wave online softmax of a 32-row tile, the split partials,
// and the body of a wide work item (128 query rows of a prefill slice over one
// key split, K/V staged once in LDS for 4 waves).  Operand layouts and the LDS
// stage format are described in chunk.hip.
#pragma once

#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {
namespace {


constexpr float kTau = 8.0f;             // log2 headroom before the running max is raised
constexpr int kRows = 32;                // query rows per tile (one wave)
constexpr int kWideTiles = 4;            // row tiles (waves) of a wide item
constexpr int kWideThreads = 64 * kWideTiles;
constexpr int kStep = 32;                // keys per step
constexpr int kMaxBlockIds = 4096 / 16 + 1;  // block ids one split can touch
constexpr int kCombineRows = 8;          // rows per combine workgroup (32 lanes each)
constexpr int kCombineParts = kRows / kCombineRows;
constexpr int kCombineChunk = 256;       // splits whose weights are staged in LDS at a time
constexpr int kCombineFast = 16;         // rows with at most this many splits: all partial loads up front

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Maxima of scores straight out of the matrix cores.  These are never
// signalling NaNs, so the max needs no canonicalisation of its inputs (which
// the compiler adds to fmaxf in IEEE mode: one extra VALU instruction per score).
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// x of lane l combined with x of lane l ^ 32 (v_permlane32_swap: no LDS round
// trip).  Each lane receives the pair {x_l, x_(l^32)}, so both halves compute
// the same value.
__device__ __forceinline__ float halves_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_raw(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Segment metadata as read on the device; bad metadata makes the segment
// "bad": its rows are zeroed and a sticky flag raised.
struct SegInfo {
  int q0, qlen, n, rows, tiles;
  int claimed_tiles;  // tiles of the q_len the offsets claim (bad segments too)
  bool bad;
  uint32_t err;
};

__device__ __forceinline__ SegInfo seg_info_of(const ChunkArgs& a, int s, int q0, int q1, int n, int r, int bs) {
  SegInfo si;
  si.q0 = q0;
  si.n = n;
  si.qlen = q1 - si.q0;
  const bool rows_ok = si.q0 >= 0 && q1 >= si.q0 && q1 <= a.total_q;
  // the last segment must end at total_q: the host sized the call's work lists from total_q
  const bool end_ok = s + 1 < a.num_segments || q1 == a.total_q;
  const bool q_ok = rows_ok && end_ok && si.qlen <= a.max_q_len && si.n >= si.qlen;
  const bool c_ok = si.n <= a.max_ctx && int64_t(si.n) <= int64_t(a.bt_stride) * bs;
  si.bad = !(q_ok && c_ok);
  si.err = !q_ok ? kErrQuery : !c_ok ? kErrContext : 0u;
  if (!rows_ok) si.qlen = 0;
  si.claimed_tiles = (si.qlen * r + kRows - 1) / kRows;
  si.rows = si.bad ? 0 : si.qlen * r;
  si.tiles = si.bad ? 0 : si.claimed_tiles;
  return si;
}

__device__ __forceinline__ SegInfo seg_info(const ChunkArgs& a, int s, int r, int bs) {
  return seg_info_of(a, s, a.qsl[s], a.qsl[s + 1], a.ctx[s], r, bs);
}

__device__ __forceinline__ int wide_groups(const SegInfo& si) { return cdiv(si.tiles, kWideTiles); }

// Keys a wide tile group attends: up to the position of the group's last query token.
__device__ __forceinline__ int wide_kend(const SegInfo& si, int grp, int r) {
  const int t_last = min((grp + 1) * kWideTiles, si.tiles) - 1;
  const int tok_last = min(si.qlen, (t_last * kRows + kRows) / r) - 1;
  return si.n - si.qlen + tok_last + 1;
}

// Zero the output rows of kv head g of a bad segment.
template <int R>
__device__ __forceinline__ void zero_rows(const ChunkArgs& a, const SegInfo& si, int g, int tid, int nthreads) {
  for (int64_t i = tid; i < int64_t(si.qlen) * R * kHeadDim; i += nthreads) {
    const int64_t t = i / (R * kHeadDim), rem = i - t * (R * kHeadDim);
    a.out[((si.q0 + t) * a.num_q_heads + g * R) * kHeadDim + rem] = 0;
  }
}

// Block-table entries [b0, b0 + nblk) of segment s as (block, kv head g) tile
// indices; an id outside the pool reads tile (0, g) and raises the flag.
__device__ __forceinline__ void load_tiles(int32_t* s_blk, const ChunkArgs& a, const PoolGeom& pool, int s, int g,
                                           int b0, int nblk, int tid, int nthreads) {
  bool bad = false;
  for (int i = tid; i < nblk; i += nthreads) {
    const int32_t b = a.bt[int64_t(s) * a.bt_stride + b0 + i];
    const bool ok = unsigned(b) < unsigned(pool.num_blocks);
    bad |= !ok;
    s_blk[i] = (ok ? b : 0) * pool.num_kv_heads + g;
  }
  if (bad) raise_error(pool.err, kErrBlockId);
}

// ---------------------------------------------------------------- shared per-wave math
// Online softmax of one 32-key step for a wave's 32-row tile, then O^T += V^T P^T.
// Scores stay in raw units (q.k); c = softmax scale * log2 e is folded into the
// exponent, p = exp2(c s - c m).  The running max m is raised only when a score
// exceeds it by more than kTau / c (log2 headroom kTau), so most steps skip the
// rescale of the 64 accumulators.  l sums the same bf16-rounded weights PV uses.
struct RowState {
  f32x16_t o[4];
  float m, l;
};

// Phase 1 of one step's online softmax: the masked scores sv and the row max;
// the running max is raised (and o, l rescaled) only when a score exceeds it
// by more than the headroom.
__device__ __forceinline__ void softmax_max(RowState& st, const f32x16_t& sacc, bool full, int key0, int klim,
                                            int qpos, int half, float c, float tau_raw, float (&sv)[16]) {
  if (full) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
  } else {
    // key0 + 16(i/8) + 8 half + i%8 is visible iff it is < klim and <= qpos
    const int lim = min(qpos, klim - 1) - key0 - 8 * half;
#pragma unroll
    for (int i = 0; i < 16; ++i) sv[i] = 16 * (i >> 3) + (i & 7) <= lim ? sacc[i] : -INFINITY;
  }
  const float m0 = max3_raw(sv[0], sv[1], sv[2]), m1 = max3_raw(sv[3], sv[4], sv[5]);
  const float m2 = max3_raw(sv[6], sv[7], sv[8]), m3 = max3_raw(sv[9], sv[10], sv[11]);
  const float m4 = max3_raw(sv[12], sv[13], sv[14]);
  float mx = max_raw(max3_raw(m0, m1, m2), max3_raw(m3, m4, sv[15]));
  mx = halves_max(mx);
  const bool raise = mx > st.m + tau_raw;
  if (__builtin_amdgcn_ballot_w64(raise)) {
    // only rows whose own scores left the headroom re-base, so a row's result
    // depends on its own scores alone (not on the other rows of the tile)
    if (raise) {
      const float corr = st.m == -INFINITY ? 1.f : fast_exp2((st.m - mx) * c);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) st.o[dt] *= corr;
      st.l *= corr;
      st.m = mx;
    }
  }
}

// Phase 2: the bf16 weights as the PV operand, pb[s16] holding keys
// 16 s16 + 8 half .. +7 of the lane's row, and their sum into l (the same
// rounded weights PV uses).
__device__ __forceinline__ void softmax_exp(RowState& st, const float (&sv)[16], float c, uint4 (&pb)[2]) {
  const float neg_mc = st.m == -INFINITY ? 0.f : -st.m * c;
  constexpr uint32_t kOnes = 0x3f803f80u;  // bf16 pair (1, 1)
#pragma unroll
  for (int s16 = 0; s16 < 2; ++s16) {
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0 = fast_exp2(fmaf(sv[8 * s16 + 2 * e], c, neg_mc));
      const float p1 = fast_exp2(fmaf(sv[8 * s16 + 2 * e + 1], c, neg_mc));
      pk[e] = pack_bf16x2(p0, p1);
      st.l = dot2_bf16(pk[e], kOnes, st.l);
    }
    pb[s16] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  }
}

template <typename VOp>
__device__ __forceinline__ void softmax_pv(RowState& st, const f32x16_t& sacc, bool full, int key0, int klim,
                                           int qpos, int half, float c, float tau_raw, VOp&& vop) {
  float sv[16];
  softmax_max(st, sacc, full, key0, klim, qpos, half, c, tau_raw, sv);
  uint4 pb[2];
  softmax_exp(st, sv, c, pb);
#pragma unroll
  for (int s16 = 0; s16 < 2; ++s16) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.o[dt] = mfma32(vop(dt, s16), pb[s16], st.o[dt]);
  }
}

// Normalised rows of one tile: bf16 output when the row has a single split,
// else fp32 partials and the split's log2-sum-exp for the combine kernel.
template <int R>
__device__ __forceinline__ void write_rows(const ChunkArgs& a, const RowState& st, int half, bool row_ok,
                                           int64_t qrow, int g, int hh, int sp, int ns, float c) {
  const float L = halves_sum(st.l);
  if (!row_ok) return;
  const int hq = a.num_q_heads;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (ns == 1) {
    uint16_t* dst = a.out + (qrow * hq + g * R + hh) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * half;
        const uint2 pk = make_uint2(pack_bf16x2(st.o[dt][4 * q4] * inv, st.o[dt][4 * q4 + 1] * inv),
                                    pack_bf16x2(st.o[dt][4 * q4 + 2] * inv, st.o[dt][4 * q4 + 3] * inv));
        *reinterpret_cast<uint2*>(dst + d) = pk;
      }
    }
  } else {
    const int64_t prow = (int64_t(sp) * a.total_q + qrow) * hq + g * R + hh;  // [split][token][head]
    float* dst = a.part_o + prow * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * half;
        *reinterpret_cast<float4*>(dst + d) = make_float4(st.o[dt][4 * q4] * inv, st.o[dt][4 * q4 + 1] * inv,
                                                          st.o[dt][4 * q4 + 2] * inv, st.o[dt][4 * q4 + 3] * inv);
      }
    }
    if (half == 0) a.part_lse[prow] = L > 0.f ? st.m * c + __log2f(L) : -INFINITY;
  }
}

// The 8 q operands of one row (zero for rows past the segment).
__device__ __forceinline__ void load_q(uint4 (&qv)[8], const ChunkArgs& a, bool row_ok, int64_t qrow, int head,
                                       int half) {
  const uint16_t* qp = a.q + (qrow * a.num_q_heads + head) * kHeadDim + half * 64;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) qv[ks] = row_ok ? ld16(qp + 8 * ks) : make_uint4(0, 0, 0, 0);
}

// Keep-mask of a bf16 pair (keys key, key+1) against the split end.
__device__ __forceinline__ uint32_t keep2(int key, int klim) {
  return key + 1 < klim ? 0xffffffffu : key < klim ? 0x0000ffffu : 0u;
}

// The merge of one row from at most kCombineFast split partials already in
// registers: v[k] = lane j's 4 dims of split k (k < ns), lk = the lse of split j
// on lane j (-inf for j >= ns).  The weights travel between the row's 32 lanes
// by shuffle and the partials are summed in split order.
__device__ __forceinline__ void merge_row_fast(const float4 (&v)[kCombineFast], float lk, int ns, bool row_ok,
                                               uint16_t* dst) {
  float M = lk;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float e = lk == -INFINITY ? 0.f : fast_exp2(lk - M);
  float L = e;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int k = 0; k < kCombineFast; ++k) {
    const float w = __shfl(e, k, 32) * inv;  // lane k of this row's 32
    if (k < ns) {
      acc.x += w * v[k].x; acc.y += w * v[k].y; acc.z += w * v[k].z; acc.w += w * v[k].w;
    }
  }
  if (!row_ok) return;
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
}

// Log-sum-exp combine of the ns split partials of one output row: 32 lanes per
// row (lane j owns dims 4j .. 4j + 3); partial row base of split k is
// base + k * total_q * Hq ([split][token][head] layout), dst the row's bf16
// output at dim 4j.  Rows with at most kCombineFast splits load every partial
// at once and exchange the split weights by shuffle.  Longer rows first reduce
// the row's split lse values (lane j takes splits j, j+32, ...), then the split
// weights go through s_w (LDS, kCombineChunk floats per row) and every lane
// sums its 4 dims over the splits in order.  Called by every thread of the
// workgroup (the long path synchronises it).
__device__ __forceinline__ void combine_row(const ChunkArgs& a, int64_t base, int ns, bool row_ok, int j,
                                            float* s_w, uint16_t* dst) {
  const int64_t stride = int64_t(a.total_q) * a.num_q_heads;  // partial rows per split
  const float* src = a.part_o + base * kHeadDim + 4 * j;

  if (ns <= kCombineFast) {
    // Up to 16 splits: every partial load is issued first, beside the one lse
    // value lane j (< ns) reads.
    float4 v[kCombineFast];
#pragma unroll
    for (int k = 0; k < kCombineFast; ++k)
      v[k] = row_ok && k < ns ? *reinterpret_cast<const float4*>(src + k * stride * kHeadDim)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    const float lk = row_ok && j < ns ? a.part_lse[base + j * stride] : -INFINITY;
    merge_row_fast(v, lk, ns, row_ok, dst);
    return;
  }

  // Row max and weight sum in one pass over the split lse values (lanes of a
  // row are 32 consecutive threads): each lane keeps a running (max, sum) of
  // its splits, then the 32 pairs are merged.
  float M = -INFINITY, L = 0.f;
  if (row_ok)
    for (int k = j; k < ns; k += 32) {
      const float lk = a.part_lse[base + k * stride];
      if (lk > M) {
        L = L * fast_exp2(M - lk) + 1.f;
        M = lk;
      } else if (lk != -INFINITY) {
        L += fast_exp2(lk - M);
      }
    }
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) {
    const float Mo = __shfl_xor(M, o), Lo = __shfl_xor(L, o);
    const float Mn = fmaxf(M, Mo);
    L = (M == -INFINITY ? 0.f : L * fast_exp2(M - Mn)) + (Mo == -INFINITY ? 0.f : Lo * fast_exp2(Mo - Mn));
    M = Mn;
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;

  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < ns; c0 += kCombineChunk) {
    const int cn = min(kCombineChunk, ns - c0);
    __syncthreads();
    for (int k = j; k < cn; k += 32) {
      const float lk = row_ok ? a.part_lse[base + (c0 + k) * stride] : -INFINITY;
      s_w[k] = lk == -INFINITY || M == -INFINITY ? 0.f : fast_exp2(lk - M) * inv;
    }
    __syncthreads();
    if (row_ok) {
#pragma unroll 8
      for (int k = 0; k < cn; ++k) {
        const float w = s_w[k];
        const float4 v = *reinterpret_cast<const float4*>(src + (c0 + k) * stride * kHeadDim);
        acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
      }
    }
  }
  if (!row_ok) return;
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
}

// ---------------------------------------------------------------- wide kernel
// LDS stage of one 32-key step (16 KB, filled by direct global->LDS loads, so
// rows cannot be padded; an XOR swizzle keeps the operand reads free of bank
// conflicts instead):
//   K    bytes [0, 8192): key row kk (256 bytes) with its 16-byte chunk c at
//        position c ^ (kk % 16);
//   V^T  bytes 8192 + 4096 p: 16-key piece p as [dim][32 bytes], the 8-key half
//        h of dim d at position h ^ ((d / 8) % 2).
// Every 16-lane phase of a 16-byte operand read then touches 16 different
// 16-byte bank groups.
constexpr int kStageBytes = 16384;
constexpr int kVBytes0 = 8192;
constexpr int kWideRing = 4;  // stages: step i (V read), i+1 (K read), i+2 landing, i+3 issued
constexpr int kWideWindow = 1024;  // keys whose block ids the 64 lanes hold at a time (16 keys each)

typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte direct global->LDS load per lane: lane l writes LDS bytes
// [dst + 16 l, dst + 16 l + 16); dst must be the same in every lane.
__device__ __forceinline__ void dma16(const uint16_t* src, uint8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitVm4 = 0x0F74;      // vmcnt(4)
constexpr int kWaitVm16 = 0x4F70;     // vmcnt(16)
constexpr int kWaitVm0 = 0x0F70;      // vmcnt(0)
constexpr int kWaitLgkm0 = 0xC07F;    // lgkmcnt(0)

// A workgroup barrier that also orders the compiler's memory accesses, without
// the release fence of __syncthreads (which would wait for every direct load
// still in flight, prefetches included).
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// LDS of a wide item: the four stages of the ring are four separate arrays,
// not one indexed ring, so that the compiler tells them apart and does not make
// a read of one stage wait for the direct loads still landing in another.
struct WideLds {
  uint8_t* st0;
  uint8_t* st1;
  uint8_t* st2;
  uint8_t* st3;
};

// One wide item: the 128 query rows of row group grp of segment s and kv head
// g (si: the segment as checked on the device) over keys
// [sp * split, min(kend, (sp + 1) * split)), kend the position after the
// group's last query token.  256 threads (4 waves, one 32-row tile each).
template <int R>
__device__ __forceinline__ void wide_body(PoolGeom& pool, const ChunkArgs& a, const SegInfo& si, int s, int g,
                                          int grp, int sp, int split, const WideLds& lds) {
  uint8_t* const s_st0 = lds.st0;
  uint8_t* const s_st1 = lds.st1;
  uint8_t* const s_st2 = lds.st2;
  uint8_t* const s_st3 = lds.st3;
  const int bs = pool.block_size, lbs = __ffs(bs) - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  const int prefix = si.n - si.qlen;
  const int kend = wide_kend(si, grp, R);
  const int ns = cdiv(kend, split);
  const int k0 = sp * split;
  const int k1 = min(kend, k0 + split);
  // The split's keys stream through the pipeline below in windows of at most
  // kWideWindow keys (one window for splits up to that size).  For the current
  // window, lane h holds the (block, kv head) tile index of its 16-key half h,
  // read into scalar registers by v_readlane.  A block id outside the pool
  // reads tile (0, g) and raises the flag.
  int wk0 = k0, wk1 = min(k1, k0 + kWideWindow), nsteps = cdiv(wk1 - wk0, kStep);
  int32_t lblk = g;
  auto load_window = [&]() {
    const int key = wk0 + 16 * lane;
    lblk = g;
    if (key < wk1) {
      const int32_t b = a.bt[int64_t(s) * a.bt_stride + (key >> lbs)];
      const bool ok = unsigned(b) < unsigned(pool.num_blocks);
      if (!ok && wave == 0) raise_error(pool.err, kErrBlockId);
      lblk = (ok ? b : 0) * pool.num_kv_heads + g;
    }
  };
  load_window();

  // This wave's row tile.
  const int tile = grp * kWideTiles + wave;
  const bool tile_ok = tile < si.tiles;
  const int rho = tile * kRows + col;
  const bool row_ok = tile_ok && rho < si.rows;
  const int tok = rho / R, hh = rho - tok * R;
  const int qpos = prefix + tok;
  const int64_t qrow = int64_t(si.q0) + tok;
  uint4 qv[8];
  load_q(qv, a, row_ok, qrow, g * R + hh, half);
  __syncthreads();

  // Direct loads of a step (4 per lane, each wave instruction 1 KB of the stage):
  //   K u = 0, 1:  key row kr = 4 (2 wave + u) + lane / 16, its chunk
  //                (lane % 16) ^ (kr % 16), to stage bytes 1024 (2 wave + u) + 16 lane;
  //   V u = 0, 1:  dim vd = 32 wave + lane / 2, the 8 keys of half
  //                (lane % 2) ^ ((vd / 8) % 2) of piece u, to stage bytes
  //                8192 + 4096 u + 1024 wave + 16 lane.
  // Splits start at multiples of 32 keys, so each 16-key half of a step lies in
  // one block: a step needs two tile addresses, the same in every lane, and each
  // load adds a fixed per-lane offset.  A half past the split end re-reads the
  // half that holds the split's last key; keys past the end inside a half read
  // their own (unused) slots of the same block.  Their scores are masked and
  // their V is zeroed by fix_tail.  A (block, head) tile holds bs << 8 bf16: K
  // rows [bs][128], then V^T.
  const int tshift = lbs + 8;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int vd = 32 * wave + (lane >> 1);
  const int vhalf = (lane & 1) ^ ((vd >> 3) & 1);
  uint32_t koff[2];  // bytes from the K row of the half's first key
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int kr = 4 * (2 * wave + u) + (lane >> 4);
    koff[u] = uint32_t(((kr & 15) * kHeadDim + ((lane & 15) ^ (kr & 15)) * 8) * 2);
  }
  const uint32_t voff = uint32_t((bs * kHeadDim + vd * kVSub + 8 * vhalf) * 2);  // V^T follows the K rows
  const uint8_t* kv_bytes = reinterpret_cast<const uint8_t*>(pool.kv);
  // The two half tiles of a step (their tile indices read from the lanes that
  // hold them, into scalar registers), then the step's 4 loads.
  struct HalfBases {
    const uint8_t* h[2];
  };
  auto half_bases = [&](int step) {
    const int key0 = wk0 + step * kStep;
    HalfBases hb;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int hk = min(key0 + 16 * h, wk1 - 1) & ~15;
      const int blk = __builtin_amdgcn_readlane(lblk, (hk - wk0) >> 4);  // the half's lane (wave-uniform)
      hb.h[h] = kv_bytes + ((int64_t(blk) << tshift) + (hk & (bs - 1)) * kHeadDim) * 2;
    }
    return hb;
  };
  auto dma_step = [&](uint8_t* st, const HalfBases& hb) {
    const uint8_t* kb = (wv >> 1) ? hb.h[1] : hb.h[0];  // K rows of this wave: half wave / 2
    dma16(reinterpret_cast<const uint16_t*>(kb + koff[0]), st + 1024 * (2 * wv));
    dma16(reinterpret_cast<const uint16_t*>(kb + koff[1]), st + 1024 * (2 * wv + 1));
    dma16(reinterpret_cast<const uint16_t*>(hb.h[0] + voff), st + kVBytes0 + 1024 * wv);
    dma16(reinterpret_cast<const uint16_t*>(hb.h[1] + voff), st + kVBytes0 + 4096 + 1024 * wv);
  };
  // V of keys past the split end must be 0 (0 * NaN would poison O): each lane
  // clears its own chunks of the split's last step once they have landed.
  auto fix_tail = [&](uint8_t* st, int step) {
    const int key0 = wk0 + step * kStep;
    if (key0 + kStep <= k1) return;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kv = key0 + 16 * u + 8 * vhalf;
      if (kv + 8 > k1) {
        uint4* p = reinterpret_cast<uint4*>(st + kVBytes0 + 4096 * u + 1024 * wave + 16 * lane);
        uint4 v = *p;
        v.x &= keep2(kv + 0, k1); v.y &= keep2(kv + 2, k1);
        v.z &= keep2(kv + 4, k1); v.w &= keep2(kv + 6, k1);
        *p = v;
      }
    }
  };

  RowState rs;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) rs.o[dt] = f32x16_t{};
  rs.m = -INFINITY;
  rs.l = 0.f;
  const float c = a.qk_scale_log2;
  const float tau_raw = kTau / c;
  const int qpos_first = prefix + (tile * kRows) / R;  // position of the tile's first token
  const int kperm = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);  // pi(m): swap bits 2, 3
  // Operand read offsets in a stage: K chunk half*8 + ks of row kperm is at
  // k_off ^ (ks << 4); V^T of dim 32 dt + col, keys 16 s16 + 8 half at
  // v_off + 1024 dt + 4096 s16.
  const int k_off = kperm * 256 + ((half ^ ((kperm >> 3) & 1)) << 7) + ((kperm & 7) << 4);
  const int v_off = kVBytes0 + col * 32 + ((half ^ ((col >> 3) & 1)) << 4);

  auto read_k = [&](const uint8_t* st, uint4 (&kop)[8]) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kop[ks] = *reinterpret_cast<const uint4*>(st + (k_off ^ (ks << 4)));
  };
  auto qk = [&](const uint4 (&kop)[8]) -> f32x16_t {
    f32x16_t acc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) acc = mfma32(kop[ks], qv[ks], acc);
    return acc;
  };

  // Pipeline: iteration i issues the loads of step i+3 into the stage step i-1
  // used and looks up the tiles of step i+4, computes step i (its scores came
  // one iteration earlier) beside the scores of step i+1, then waits for its
  // own loads of step i+2 and meets the others at the barrier, after which
  // step i+2 is readable.  Loads are clamped to the last step, never skipped,
  // so every lane has exactly 4 loads per step in flight and vmcnt(4) means
  // "all but the latest step".
  HalfBases next_hb;
  f32x16_t s_cur;
  auto prologue = [&]() {
    dma_step(s_st0, half_bases(0));
    dma_step(s_st1, half_bases(min(1, nsteps - 1)));
    dma_step(s_st2, half_bases(min(2, nsteps - 1)));
    next_hb = half_bases(min(3, nsteps - 1));
    __builtin_amdgcn_s_waitcnt(kWaitVm4);
    fix_tail(s_st0, 0);
    if (nsteps > 1) fix_tail(s_st1, 1);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    stage_barrier();
    s_cur = f32x16_t{};
    if (tile_ok) {
      uint4 kop[8];
      read_k(s_st0, kop);
      s_cur = qk(kop);
    }
  };
  // st: step i (V), nst: step i+1 (K), fst: step i+2 (landing), lst: step i+3 (issued now)
  auto iter = [&](int i, const uint8_t* st, const uint8_t* nst, uint8_t* fst, uint8_t* lst) {
    dma_step(lst, next_hb);
    if (tile_ok && i < nsteps) {
      const int key0 = wk0 + i * kStep;
      const bool full = key0 + kStep <= k1 && key0 + kStep - 1 <= qpos_first;
      // All 16 operand reads of the iteration first (K of step i+1, V of step
      // i), each into registers of its own: reading every V operand just
      // before its MFMA into one reused register quad exposed the LDS latency
      // eight times per step.
      uint4 kop[8], vop[8];
      read_k(nst, kop);
#pragma unroll
      for (int s16 = 0; s16 < 2; ++s16) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          vop[4 * s16 + dt] = *reinterpret_cast<const uint4*>(st + v_off + 1024 * dt + 4096 * s16);
      }
      float sv[16];
      softmax_max(rs, s_cur, full, key0, k1, qpos, half, c, tau_raw, sv);
      const f32x16_t s_next = qk(kop);
      uint4 pb[2];
      softmax_exp(rs, sv, c, pb);
#pragma unroll
      for (int s16 = 0; s16 < 2; ++s16) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) rs.o[dt] = mfma32(vop[4 * s16 + dt], pb[s16], rs.o[dt]);
      }
      // Issue order of this block: one MFMA, then three VALU instructions, 16
      // times.  The score MFMAs of step i+1 (a dependent chain) are ready first
      // and fill the early MFMA slots, so their latency hides behind the
      // exponentials instead of stalling the wave after them.
#pragma unroll
      for (int gidx = 0; gidx < 16; ++gidx) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
      }
      s_cur = s_next;
    }
    next_hb = half_bases(min(i + 4, nsteps - 1));
    __builtin_amdgcn_s_waitcnt(kWaitVm4);
    if (i + 2 < nsteps) fix_tail(fst, i + 2);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    stage_barrier();
  };
  for (;;) {
    prologue();
    for (int base = 0; base < nsteps; base += kWideRing) {
      iter(base, s_st0, s_st1, s_st2, s_st3);
      iter(base + 1, s_st1, s_st2, s_st3, s_st0);
      iter(base + 2, s_st2, s_st3, s_st0, s_st1);
      iter(base + 3, s_st3, s_st0, s_st1, s_st2);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no direct load outlives the window (or the workgroup's LDS)
    if (wk1 >= k1) break;
    // next window: every wave is done with the stages before they are refilled
    stage_barrier();
    wk0 = wk1;
    wk1 = min(k1, wk0 + kWideWindow);
    nsteps = cdiv(wk1 - wk0, kStep);
    load_window();
  }
  if (!tile_ok) return;
  write_rows<R>(a, rs, half, row_ok, qrow, g, hh, sp, ns, c);
}

}  // namespace
}  // namespace pgqa
