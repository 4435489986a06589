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
// Unlike decode, QK^T and PV here are dense contractions, so both run on
// v_mfma_f32_32x32x16_bf16.
//
// Work decomposition.  Query rows of a segment and kv head g are the pairs
// (token, head in group), row rho = token * r + hh, cut into 32-row tiles; 8
// tiles form a group.  A work item is (segment, g, tile group, key split).  A
// one-workgroup schedule kernel lists exactly the items the device metadata
// calls for (no idle workgroups in the grid), and the main kernel runs one
// workgroup of 8 waves per item:
//   * every 32-key step of the split is staged once in LDS by all 512 threads
//     (K rows and V^T rows of the step, loads issued four steps ahead), and
//   * each of the 8 waves computes one row tile from it; the waves never merge
//     state (each owns its rows).
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
//     bytes, in the cache and in LDS.  Nothing is transposed at run time.
//   * dims of the S product are split between the lane halves as
//     (l/32)*64 + 8*kstep + j: a lane reads 128 contiguous bytes of its q row.
//   * LDS rows are padded (K: 272 bytes, V^T: 80 bytes) so that the 16 lanes
//     of each LDS read phase hit 16 different 4-bank groups.
#include <math.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace pgqa {
namespace {

constexpr float kTau = 8.0f;            // log2 headroom before the running max is raised
constexpr int kRows = 32;               // query rows per tile
constexpr int kTilesPerGroup = 8;       // row tiles per work item (one per wave)
constexpr int kStep = 32;               // keys per step
constexpr int kThreads = 64 * kTilesPerGroup;
constexpr int kSchedThreads = 256;
constexpr int kKRow = 136;              // LDS K row stride in bf16 (128 + 8 padding)
constexpr int kVRow = 40;               // LDS V^T row stride in bf16 (32 + 8 padding)
constexpr int kKStage = kStep * kKRow;  // bf16 elements per stage
constexpr int kVStage = kHeadDim * kVRow;
constexpr int kMaxBlockIds = 4096 / 16; // block ids of one split (split <= 4096 keys)
constexpr int kStages = 4;              // steps whose global loads are in flight

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Keys a tile group may attend: up to the position of the group's last query token.
struct SegInfo {
  int q0, qlen, n, tiles, groups;
  bool bad;
  uint32_t err;
};

__device__ __forceinline__ SegInfo seg_info(const ChunkArgs& a, int s, int r, int bs) {
  SegInfo si;
  si.q0 = a.qsl[s];
  const int q1 = a.qsl[s + 1];
  si.n = a.ctx[s];
  si.qlen = q1 - si.q0;
  const bool rows_ok = si.q0 >= 0 && q1 >= si.q0 && q1 <= a.total_q;
  const bool q_ok = rows_ok && si.qlen <= a.max_q_len && si.n >= si.qlen;
  const bool c_ok = si.n <= a.max_ctx && int64_t(si.n) <= int64_t(a.bt_stride) * bs;
  si.bad = !(q_ok && c_ok);
  si.err = !q_ok ? kErrQuery : !c_ok ? kErrContext : 0u;
  si.tiles = si.bad ? 0 : (si.qlen * r + kRows - 1) / kRows;
  si.groups = (si.tiles + kTilesPerGroup - 1) / kTilesPerGroup;
  if (!rows_ok) si.qlen = 0;
  return si;
}

__device__ __forceinline__ int group_kend(const SegInfo& si, int grp, int r) {
  const int t_last = min((grp + 1) * kTilesPerGroup, si.tiles) - 1;
  const int tok_last = min(si.qlen, (t_last * kRows + kRows) / r) - 1;
  return si.n - si.qlen + tok_last + 1;
}

// ---------------------------------------------------------------- schedule
// One workgroup: per-segment item counts, a workgroup-wide exclusive scan, then
// every thread writes the items of its own contiguous range of segments.
// Items: {segment, kv head, tile group, split}; a segment with bad metadata
// gets one item per kv head with tile group -1 (zero its rows, raise the flag).
__device__ __forceinline__ int seg_items(const ChunkArgs& a, const SegInfo& si, int r, int hkv) {
  if (si.bad) return hkv;
  int cnt = 0;
  for (int grp = 0; grp < si.groups; ++grp) cnt += hkv * ((group_kend(si, grp, r) + a.split_tokens - 1) / a.split_tokens);
  return cnt;
}

__global__ __launch_bounds__(kSchedThreads) void chunk_schedule_kernel(PoolGeom pool, ChunkArgs a) {
  const int tid = threadIdx.x;
  const int hkv = pool.num_kv_heads, r = a.num_q_heads / hkv;
  const int N = a.num_segments;
  const int per = (N + kSchedThreads - 1) / kSchedThreads;
  const int s_begin = min(N, tid * per), s_end = min(N, s_begin + per);
  __shared__ int s_scan[kSchedThreads];

  // 1. item count of each segment; workgroup-wide exclusive scan -> seg_off[]
  int mine = 0;
  for (int s = s_begin; s < s_end; ++s) mine += seg_items(a, seg_info(a, s, r, pool.block_size), r, hkv);
  s_scan[tid] = mine;
  __syncthreads();
  for (int off = 1; off < kSchedThreads; off <<= 1) {
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  int pos = s_scan[tid] - mine;
  for (int s = s_begin; s < s_end; ++s) {
    a.seg_off[s] = pos;
    pos += seg_items(a, seg_info(a, s, r, pool.block_size), r, hkv);
  }
  const int total = s_scan[kSchedThreads - 1];
  if (tid == 0) {
    a.seg_off[N] = total;
    *a.item_count = min(total, a.max_items);
    if (total > a.max_items) raise_error(pool.err, kErrQuery);
  }
  __threadfence_block();
  __syncthreads();

  // 2. every thread writes items tid, tid + 256, ...: find the segment by
  // binary search over seg_off, then (tile group, split, kv head) inside it.
  const int limit = min(total, a.max_items);
  for (int i = tid; i < limit; i += kSchedThreads) {
    int lo = 0, hi = N;  // seg_off[lo] <= i < seg_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.seg_off[mid] <= i) lo = mid; else hi = mid;
    }
    const SegInfo si = seg_info(a, lo, r, pool.block_size);
    int li = i - a.seg_off[lo];
    if (si.bad) {
      a.items[i] = make_int4(lo, li, -1, 0);
      continue;
    }
    for (int grp = 0; grp < si.groups; ++grp) {
      const int cnt = hkv * ((group_kend(si, grp, r) + a.split_tokens - 1) / a.split_tokens);
      if (li < cnt) {
        a.items[i] = make_int4(lo, li % hkv, grp, li / hkv);
        break;
      }
      li -= cnt;
    }
  }
}

// ---------------------------------------------------------------- main kernel
template <int R>
__global__ __launch_bounds__(kThreads) void chunk_kernel(PoolGeom pool, ChunkArgs a) {
  if (int(blockIdx.x) >= *a.item_count) return;
  const int4 item = a.items[blockIdx.x];
  const int s = item.x, g = item.y, grp = item.z, sp = item.w;
  const int hkv = pool.num_kv_heads, bs = pool.block_size, hq = a.num_q_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;

  __shared__ __align__(16) uint16_t s_k[2][kKStage];
  __shared__ __align__(16) uint16_t s_v[2][kVStage];
  __shared__ uint32_t s_valid[2];              // per stage: bit j = key j of the step is attendable
  __shared__ int32_t s_blk[kMaxBlockIds];

  const SegInfo si = seg_info(a, s, R, bs);
  if (grp < 0 || si.bad) {
    if (tid == 0) raise_error(pool.err, si.err ? si.err : kErrQuery);
    for (int64_t i = tid; i < int64_t(si.qlen) * R * kHeadDim; i += kThreads) {
      const int64_t tok = i / (R * kHeadDim), rem = i - tok * (R * kHeadDim);
      a.out[((si.q0 + tok) * hq + g * R) * kHeadDim + rem] = 0;
    }
    return;
  }
  const int prefix = si.n - si.qlen;
  const int kend = group_kend(si, grp, R);
  const int ns = (kend + a.split_tokens - 1) / a.split_tokens;
  const int k0 = sp * a.split_tokens;
  const int k1 = min(kend, k0 + a.split_tokens);
  const int nsteps = (k1 - k0 + kStep - 1) / kStep;

  // Block ids of the split (entries past the table row are never read).
  const int nblk = (k1 - k0 + bs - 1) / bs;
  for (int i = tid; i < nblk; i += kThreads) s_blk[i] = a.bt[int64_t(s) * a.bt_stride + k0 / bs + i];

  // This wave's row tile and its q operands (zero for rows past the segment).
  const int rows = si.qlen * R;
  const int tile = grp * kTilesPerGroup + wave;
  const bool tile_ok = tile < si.tiles;
  const int rho = tile * kRows + col;
  const bool row_ok = tile_ok && rho < rows;
  const int tok = rho / R, hh = rho - tok * R;
  const int qpos = prefix + tok;
  uint4 qv[8];
  {
    const uint16_t* qp = a.q + ((int64_t(si.q0) + tok) * hq + g * R + hh) * kHeadDim + half * 64;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qv[ks] = row_ok ? *reinterpret_cast<const uint4*>(qp + 8 * ks) : make_uint4(0, 0, 0, 0);
  }
  __syncthreads();

  // Staging: thread t moves 16 B of K (key t/16, 16-byte chunk t%16) and 16 B of
  // V^T (dim t/4, keys 8*(t%4) .. +7) per step.
  const int64_t tstride = tile_elems(pool);
  const int64_t bstride = tstride * hkv;
  const uint16_t* pool_g = pool.kv + int64_t(g) * tstride;
  const int kkey = tid >> 4, kchunk = tid & 15;
  const int vdim = tid >> 2, vq = tid & 3;
  struct Stage {
    uint4 k, v;
    bool kok, vok;
  };
  // Loads are unconditional (an invalid key reads block 0, slot 0) and their
  // validity is applied when the data is stored to LDS, so the compiler can
  // count outstanding loads exactly and keep the prefetch in flight.
  bool bad_blk = false;
  auto fetch = [&](Stage& st, int step) {
    const int key0 = k0 + step * kStep;
    const int kk = key0 + kkey;
    const int32_t bk = s_blk[min((kk - k0) / bs, nblk - 1)];
    st.kok = kk < k1 && unsigned(bk) < unsigned(pool.num_blocks);
    const uint16_t* kp =
        pool_g + int64_t(st.kok ? bk : 0) * bstride + ((st.kok ? kk : 0) & (bs - 1)) * kHeadDim + kchunk * 8;
    st.k = *reinterpret_cast<const uint4*>(kp);
    const int kv = key0 + 8 * vq;
    const int32_t bv = s_blk[min((kv - k0) / bs, nblk - 1)];
    st.vok = kv < k1 && unsigned(bv) < unsigned(pool.num_blocks);
    const uint16_t* vp = pool_g + int64_t(st.vok ? bv : 0) * bstride + int64_t(bs) * kHeadDim + int64_t(vdim) * bs +
                         ((st.vok ? kv : 0) & (bs - 1));
    st.v = *reinterpret_cast<const uint4*>(vp);
    bad_blk |= (kk < k1 && unsigned(bk) >= unsigned(pool.num_blocks)) ||
               (kv < k1 && unsigned(bv) >= unsigned(pool.num_blocks));
  };
  auto store = [&](const Stage& st, int step, int buf) {
    // V entries of keys past the split end are zeroed (0 * NaN would poison O).
    const int kv = k0 + step * kStep + 8 * vq;
    uint4 v = st.vok ? st.v : make_uint4(0, 0, 0, 0);
    if (kv + 8 > k1) {
      auto keep = [&](int key) -> uint32_t {
        return key + 1 < k1 ? 0xffffffffu : key < k1 ? 0x0000ffffu : 0u;
      };
      v.x &= keep(kv + 0); v.y &= keep(kv + 2); v.z &= keep(kv + 4); v.w &= keep(kv + 6);
    }
    *reinterpret_cast<uint4*>(&s_k[buf][kkey * kKRow + kchunk * 8]) = st.kok ? st.k : make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(&s_v[buf][vdim * kVRow + 8 * vq]) = v;
    if (tid < kStep) {
      const int key = k0 + step * kStep + tid;
      const int32_t b = s_blk[min((key - k0) / bs, nblk - 1)];
      const bool ok = key < k1 && unsigned(b) < unsigned(pool.num_blocks);
      const uint64_t msk = __ballot(ok);
      if (tid == 0) s_valid[buf] = uint32_t(msk);
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16_t{};
  float m = -INFINITY, l = 0.f;                 // running max (raw score units) and weight sum
  const float c = a.qk_scale_log2;
  const float tau_raw = kTau / c;
  const int qpos_first = prefix + (tile * kRows) / R;  // position of the tile's first token
  const int mrow = col;
  const int kperm = (mrow & ~12) | ((mrow & 4) << 1) | ((mrow & 8) >> 1);   // pi(m): swap bits 2, 3

  auto compute = [&](int step, int buf) {
    if (!tile_ok) return;
    const int key0 = k0 + step * kStep;
    const uint32_t valid = s_valid[buf];
    const uint16_t* kr = &s_k[buf][kperm * kKRow + half * 64];
    // two independent accumulation chains (even / odd dim steps) halve the
    // dependent-MFMA latency of the score product
    f32x16_t sacc = f32x16_t{}, sacc2 = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ks += 2) {
      sacc = mfma32(*reinterpret_cast<const uint4*>(kr + 8 * ks), qv[ks], sacc);
      sacc2 = mfma32(*reinterpret_cast<const uint4*>(kr + 8 * ks + 8), qv[ks + 1], sacc2);
    }
    sacc += sacc2;
    // Scores stay in raw units (q.k); the scale c = softmax scale * log2 e is
    // folded into the exponent: p = exp2(c * s - c * m).  Steps entirely below
    // the tile's first query position, with all keys present, need no mask.
    float sv[16];
    if (valid == 0xffffffffu && key0 + kStep - 1 <= qpos_first) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sv[i] = sacc[i];
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int koff = 16 * (i >> 3) + 8 * half + (i & 7);
        const bool okk = ((valid >> koff) & 1u) && key0 + koff <= qpos;
        sv[i] = okk ? sacc[i] : -INFINITY;
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__ballot(mx > m + tau_raw)) {
      const float mn = fmaxf(m, mx);
      const float corr = mn == -INFINITY ? 1.f : fast_exp2((m - mn) * c);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= corr;
      l *= corr;
      m = mn;
    }
    const float neg_mc = m == -INFINITY ? 0.f : -m * c;
    constexpr uint32_t kOnes = 0x3f803f80u;  // bf16 pair (1, 1)
#pragma unroll
    for (int s16 = 0; s16 < 2; ++s16) {
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(fmaf(sv[8 * s16 + 2 * e], c, neg_mc));
        const float p1 = fast_exp2(fmaf(sv[8 * s16 + 2 * e + 1], c, neg_mc));
        pk[e] = pack_bf16x2(p0, p1);
        l = dot2_bf16(pk[e], kOnes, l);  // l sums the same rounded weights PV uses
      }
      const uint4 pb = make_uint4(pk[0], pk[1], pk[2], pk[3]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const uint4 vop = *reinterpret_cast<const uint4*>(&s_v[buf][(32 * dt + col) * kVRow + 16 * s16 + 8 * half]);
        o[dt] = mfma32(vop, pb, o[dt]);
      }
    }
  };

  // Pipeline: a ring of kStages register stages keeps the global loads of the
  // next kStages steps in flight; two LDS stages alternate between the step
  // being computed and the next one being stored.  Loads are unconditional
  // (clamped to the last step) so the compiler can count them exactly; the
  // barriers are uniform across the workgroup.
  if (nsteps > 0) {
    Stage st[kStages];
#pragma unroll
    for (int j = 0; j < kStages; ++j) fetch(st[j], min(j, nsteps - 1));
    store(st[0], 0, 0);
    fetch(st[0], min(kStages, nsteps - 1));
    for (int base = 0; base < nsteps; base += kStages) {
#pragma unroll
      for (int j = 0; j < kStages; ++j) {
        const int i = base + j;
        __syncthreads();
        if (i < nsteps) compute(i, j & 1);
        if (i + 1 < nsteps) store(st[(j + 1) % kStages], i + 1, (j + 1) & 1);
        fetch(st[(j + 1) % kStages], min(i + 1 + kStages, nsteps - 1));
      }
    }
  }
  if (bad_blk) raise_error(pool.err, kErrBlockId);

  // Each wave finishes its own rows.
  if (!tile_ok) return;
  const float L = l + __shfl_xor(l, 32);
  if (!row_ok) return;
  const int64_t qrow = int64_t(si.q0) + tok;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (ns == 1) {
    uint16_t* dst = a.out + (qrow * hq + g * R + hh) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * half;
        const uint2 pk = make_uint2(pack_bf16x2(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv),
                                    pack_bf16x2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv));
        *reinterpret_cast<uint2*>(dst + d) = pk;
      }
    }
  } else {
    const int64_t prow = ((int64_t(g) * a.max_splits + sp) * a.total_q + qrow) * R + hh;
    float* dst = a.part_o + prow * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = 32 * dt + 8 * q4 + 4 * half;
        *reinterpret_cast<float4*>(dst + d) = make_float4(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv,
                                                          o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
      }
    }
    if (half == 0) a.part_lse[prow] = L > 0.f ? m * c + __log2f(L) : -INFINITY;
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
  const SegInfo si = seg_info(a, lo, r, pool.block_size);
  if (si.bad || t < si.q0 || t >= si.q0 + si.qlen) return;
  const int tile = ((t - si.q0) * r + hh) / kRows;
  const int kend = group_kend(si, tile / kTilesPerGroup, r);
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

template <int R>
hipError_t launch_r(const PoolGeom& pool, const ChunkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, pool, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_kernel<R>), dim3(a.max_items), dim3(kThreads), 0, stream, pool, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL(chunk_combine_kernel, dim3(a.total_q, a.num_q_heads), dim3(kHeadDim), 0, stream, pool, a);
  return hipGetLastError();
}

}  // namespace

int64_t chunk_max_items(int32_t num_segments, int32_t total_q, int32_t num_kv_heads, int32_t group,
                        int32_t max_splits) {
  const int64_t rows_per_group = int64_t(kRows) * kTilesPerGroup;
  const int64_t groups = (int64_t(total_q) * group + rows_per_group - 1) / rows_per_group + num_segments;
  return groups * max_splits * num_kv_heads + int64_t(num_segments) * num_kv_heads;
}

ChunkWorkspace chunk_workspace_layout(int32_t num_segments, int32_t total_q, int32_t num_kv_heads,
                                      int32_t num_q_heads, int32_t max_splits) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  ChunkWorkspace w;
  const int64_t items = chunk_max_items(num_segments, total_q, num_kv_heads, num_q_heads / num_kv_heads, max_splits);
  w.count_off = 0;
  w.seg_off_off = 256;
  w.items_off = w.seg_off_off + up((size_t(num_segments) + 1) * sizeof(int32_t));
  size_t end = w.items_off + up(size_t(items) * 4 * sizeof(int32_t));
  w.part_o_off = w.part_lse_off = end;
  if (max_splits > 1) {
    const size_t rows = size_t(max_splits) * total_q * num_q_heads;  // Hkv * r == Hq
    w.part_o_off = end;
    w.part_lse_off = w.part_o_off + up(rows * kHeadDim * sizeof(float));
    end = w.part_lse_off + up(rows * sizeof(float));
  }
  w.total = end;
  return w;
}

hipError_t launch_chunk(const PoolGeom& pool, const ChunkArgs& a, hipStream_t stream) {
  if (a.num_segments == 0 || a.total_q == 0) return hipSuccess;
  if (a.split_tokens > 4096 || a.max_items <= 0) return hipErrorInvalidValue;
  switch (a.num_q_heads / pool.num_kv_heads) {
    case 1: return launch_r<1>(pool, a, stream);
    case 2: return launch_r<2>(pool, a, stream);
    case 4: return launch_r<4>(pool, a, stream);
    case 8: return launch_r<8>(pool, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pgqa
