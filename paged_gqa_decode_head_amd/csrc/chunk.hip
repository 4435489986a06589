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
// QK^T and PV are dense contractions here, so both run on
// v_mfma_f32_32x32x16_bf16.
//
// Rows.  The query rows of a segment and kv head g are the pairs (token, head
// in group), row rho = token * r + hh, cut into 32-row tiles (one wave each).
// Two kinds of work item; every workgroup derives its own item from the
// device metadata (see the work lists below):
//   * wide (segments of more than 32 rows per kv head: prefill slices).  Item =
//     (segment, g, group of 4 tiles, key split); 4 waves share every 32-key step,
//     staged once in LDS by all 256 threads with direct global->LDS loads into a
//     4-stage ring (three steps in flight).  Each wave computes the scores of
//     step i+1 beside the softmax of step i, so the matrix core works while the
//     VALU does the softmax.  MFMA-bound.
//   * narrow (at most 32 rows per kv head: verify rows, decode-like rows).  Item =
//     (segment, g, key split), one wave, many short splits.  V^T is loaded from
//     the cache straight into the MFMA operand registers (whole 128-byte lines per
//     load); K goes through a per-wave LDS ring (direct loads) to reach the operand
//     layout.  HBM-bound.
// Splits are merged by a log-sum-exp combine kernel when a row has several.
//
// Operand layouts (verified on the hardware): lane l supplies A[m][k] with
// m = l%32, k = 8(l/32)+j and B[k][n] with n = l%32; D[i] of lane l is
// row 8(i/4)+4(l/32)+i%4, column l%32.
//   * S^T = K Q^T (M = keys, N = query rows, K = dims).  MFMA row m holds key
//     pi(m) of the step, pi swapping bits 2 and 3 of m; then D[i] of lane l is
//     key 16(i/8) + 8(l/32) + i%8, so the 8 weights a lane needs as its PV
//     operand for keys 16s + 8(l/32) .. +7 are its own D[8s .. 8s+7].
//   * O^T += V^T P^T (M = dims, N = query rows, K = keys): the cache keeps V
//     transposed in 16-slot pieces, so a lane's 8 keys of one dim are 16
//     contiguous bytes, in the cache and in LDS.  Nothing is transposed at run
//     time.
//   * dims of the S product are split between the lane halves as
//     (l/32)*64 + 8*kstep + j: a lane reads 128 contiguous bytes of its q row.
//   * LDS operand reads are conflict-free: the 16 lanes of each read phase hit
//     16 different 4-bank groups of the XOR-swizzled stages, which direct
//     global->LDS loads can fill.
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// x of lane l combined with x of lane l ^ 32 (v_permlane32_swap: no LDS round
// trip).  Each lane receives the pair {x_l, x_(l^32)}, so both halves compute
// the same value.
__device__ __forceinline__ float halves_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
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

__device__ __forceinline__ SegInfo seg_info(const ChunkArgs& a, int s, int r, int bs) {
  SegInfo si;
  si.q0 = a.qsl[s];
  const int q1 = a.qsl[s + 1];
  si.n = a.ctx[s];
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

__device__ __forceinline__ int wide_groups(const SegInfo& si) { return cdiv(si.tiles, kWideTiles); }

// Keys a wide tile group attends: up to the position of the group's last query token.
__device__ __forceinline__ int wide_kend(const SegInfo& si, int grp, int r) {
  const int t_last = min((grp + 1) * kWideTiles, si.tiles) - 1;
  const int tok_last = min(si.qlen, (t_last * kRows + kRows) / r) - 1;
  return si.n - si.qlen + tok_last + 1;
}

// ---------------------------------------------------------------- work lists
// Three lists, each in segment order:
//   wide    {segment, kv head, tile group, split} of segments with more than one
//           row tile per kv head; {segment, kv head, -1, 0} zeroes the rows of a
//           bad segment that claims more than one tile;
//   short   {segment, kv head, 0, split} of one-tile segments; {.., -1, 0} for bad
//           one-tile segments;
//   combine {segment, kv head, tile, part} for every row tile with several splits,
//           in kCombineParts parts of 8 rows.
// No list is stored: every workgroup derives its own item from the segment
// metadata (a wave-wide scan of per-segment counts, then a search), so no
// schedule kernel and no dependent read of a stored list sits in front of the
// K/V stream.
enum ListKind { kWideList, kShortList, kCombineList };

// Whether the host launched the short-item kernel: not for a call whose lone
// segment is wide by its host-side size (chunk_lists).  A bad segment whose
// claimed rows fit one tile is then zeroed by a wide-list item instead.
__device__ __forceinline__ bool short_launched(const ChunkArgs& a, int r) {
  return !(a.num_segments == 1 && int64_t(a.total_q) * r > kRows);
}

template <ListKind K>
__device__ __forceinline__ int list_count(const ChunkArgs& a, const SegInfo& si, int r, int hkv) {
  if (K == kWideList) {
    if (si.bad) return si.claimed_tiles > 1 || !short_launched(a, r) ? hkv : 0;
    if (si.tiles <= 1) return 0;
    int cnt = 0;
    for (int grp = 0; grp < wide_groups(si); ++grp) cnt += cdiv(wide_kend(si, grp, r), a.split_wide);
    return cnt * hkv;
  } else if (K == kShortList) {
    if (si.bad) return si.claimed_tiles == 1 && short_launched(a, r) ? hkv : 0;
    return si.tiles == 1 ? hkv * cdiv(si.n, a.split_short) : 0;
  } else {
    if (si.tiles == 0) return 0;
    if (si.tiles == 1) return cdiv(si.n, a.split_short) > 1 ? hkv * kCombineParts : 0;
    int cnt = 0;
    for (int grp = 0; grp < wide_groups(si); ++grp)
      if (cdiv(wide_kend(si, grp, r), a.split_wide) > 1) cnt += min(kWideTiles, si.tiles - grp * kWideTiles);
    return cnt * hkv * kCombineParts;
  }
}

template <ListKind K>
__device__ __forceinline__ int4 list_item(const ChunkArgs& a, const SegInfo& si, int s, int li, int r, int hkv) {
  if (K != kCombineList && si.bad) return make_int4(s, li, -1, 0);
  if (K == kShortList) return make_int4(s, li % hkv, 0, li / hkv);
  if (K == kCombineList && si.tiles == 1) return make_int4(s, li % hkv, 0, li / hkv);
  const int parts = K == kCombineList ? kCombineParts : 1;
  for (int grp = 0;; ++grp) {
    const int ns = cdiv(wide_kend(si, grp, r), a.split_wide);
    const int per_head = K == kWideList ? ns : ns > 1 ? min(kWideTiles, si.tiles - grp * kWideTiles) * parts : 0;
    if (li < per_head * hkv) {
      const int g = li % hkv, j = li / hkv;
      return K == kWideList ? make_int4(s, g, grp, j) : make_int4(s, g, grp * kWideTiles + j / parts, j % parts);
    }
    li -= per_head * hkv;
  }
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

struct Located {
  int4 item;  // item.x < 0: past the end of the list
  SegInfo si;
};

// The same Located in scalar registers: every lane of a wave holds the same
// values, and saying so lets the compiler do the per-step key and address
// arithmetic on the scalar unit.
__device__ __forceinline__ Located wave_uniform(const Located& l) {
  auto u = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
  Located r;
  r.item = make_int4(u(l.item.x), u(l.item.y), u(l.item.z), u(l.item.w));
  r.si.q0 = u(l.si.q0);
  r.si.qlen = u(l.si.qlen);
  r.si.n = u(l.si.n);
  r.si.rows = u(l.si.rows);
  r.si.tiles = u(l.si.tiles);
  r.si.claimed_tiles = u(l.si.claimed_tiles);
  r.si.bad = u(int(l.si.bad)) != 0;
  r.si.err = uint32_t(u(int(l.si.err)));
  return r;
}

// Item idx of list K, computed by one whole wave (every lane gets the result).
// Lane i counts segments [i*per, i*per + per); a second pass over the chosen
// lane's segments finds the segment (num_segments <= 4096, so per <= 64).
// Workgroup 0 also raises the flags of bad segments and of a list longer than
// the grid.
template <ListKind K>
__device__ Located locate(const ChunkArgs& a, PoolGeom& pool, int idx, int r) {
  const int lane = threadIdx.x & 63;
  const int hkv = pool.num_kv_heads, bs = pool.block_size, N = a.num_segments;
  const int per = (N + 63) >> 6;
  int c = 0;
  for (int k = 0; k < per; ++k) {
    const int s = lane * per + k;
    if (s < N) {
      const SegInfo si = seg_info(a, s, r, bs);
      c += list_count<K>(a, si, r, hkv);
      if (blockIdx.x == 0 && si.bad) raise_error(pool.err, si.err);
    }
  }
  const int incl = wave_incl_scan(c, lane);
  const int total = __shfl(incl, 63);
  if (blockIdx.x == 0 && lane == 0 && total > int(gridDim.x)) raise_error(pool.err, kErrQuery);
  Located out;
  out.item = make_int4(-1, 0, 0, 0);
  if (idx >= total) return out;
  const int L = __ffsll((unsigned long long)__ballot(incl > idx)) - 1;
  int li = idx - (__shfl(incl, L) - __shfl(c, L));
  int seg = L;
  if (per > 1) {
    const int s2 = L * per + lane;
    const int c2 = lane < per && s2 < N ? list_count<K>(a, seg_info(a, s2, r, bs), r, hkv) : 0;
    const int incl2 = wave_incl_scan(c2, lane);
    const int L2 = __ffsll((unsigned long long)__ballot(incl2 > li)) - 1;
    li -= __shfl(incl2, L2) - __shfl(c2, L2);
    seg = L * per + L2;
  }
  out.si = seg_info(a, seg, r, bs);
  out.item = list_item<K>(a, out.si, seg, li, r, hkv);
  return out;
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
  float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
  mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(sv[8], sv[9]), fmaxf(sv[10], sv[11])),
                       fmaxf(fmaxf(sv[12], sv[13]), fmaxf(sv[14], sv[15]))));
  mx = halves_max(mx);
  if (__builtin_amdgcn_ballot_w64(mx > st.m + tau_raw)) {
    const float mn = fmaxf(st.m, mx);
    const float corr = mn == -INFINITY ? 1.f : fast_exp2((st.m - mn) * c);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) st.o[dt] *= corr;
    st.l *= corr;
    st.m = mn;
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
    const int64_t prow = ((int64_t(g) * a.max_splits + sp) * a.total_q + qrow) * R + hh;
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

template <int R>
__global__ __launch_bounds__(kWideThreads, 2) void chunk_wide_kernel(PoolGeom pool, ChunkArgs a) {
  const Located loc = wave_uniform(locate<kWideList>(a, pool, blockIdx.x, R));
  if (loc.item.x < 0) return;
  const SegInfo& si = loc.si;
  const int s = loc.item.x, g = loc.item.y, grp = loc.item.z, sp = loc.item.w;
  const int bs = pool.block_size, lbs = __ffs(bs) - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  if (grp < 0) {
    zero_rows<R>(a, si, g, tid, kWideThreads);
    return;
  }

  // Four separate arrays, not one indexed ring: the compiler then tells the
  // stages apart and does not make a read of one stage wait for the direct
  // loads still landing in another.
  __shared__ __align__(1024) uint8_t s_st0[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st1[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st2[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st3[kStageBytes];
  __shared__ int32_t s_blk[kMaxBlockIds];

  const int prefix = si.n - si.qlen;
  const int kend = wide_kend(si, grp, R);
  const int ns = cdiv(kend, a.split_wide);
  const int k0 = sp * a.split_wide;
  const int k1 = min(kend, k0 + a.split_wide);
  const int nsteps = cdiv(k1 - k0, kStep);
  const int b0 = k0 >> lbs;
  load_tiles(s_blk, a, pool, s, g, b0, ((k1 - 1) >> lbs) - b0 + 1, tid, kWideThreads);

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
  // The two half tiles of a step (read from s_blk one iteration before their
  // loads are issued, so the LDS latency is hidden), then the step's 4 loads.
  struct HalfBases {
    const uint8_t* h[2];
  };
  auto half_bases = [&](int step) {
    const int key0 = k0 + step * kStep;
    HalfBases hb;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int hk = min(key0 + 16 * h, k1 - 1) & ~15;
      const int blk = __builtin_amdgcn_readfirstlane(s_blk[(hk >> lbs) - b0]);
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
    const int key0 = k0 + step * kStep;
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
  dma_step(s_st0, half_bases(0));
  dma_step(s_st1, half_bases(min(1, nsteps - 1)));
  dma_step(s_st2, half_bases(min(2, nsteps - 1)));
  HalfBases next_hb = half_bases(min(3, nsteps - 1));
  __builtin_amdgcn_s_waitcnt(kWaitVm4);
  fix_tail(s_st0, 0);
  if (nsteps > 1) fix_tail(s_st1, 1);
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  stage_barrier();
  f32x16_t s_cur = f32x16_t{};
  if (tile_ok) {
    uint4 kop[8];
    read_k(s_st0, kop);
    s_cur = qk(kop);
  }
  // st: step i (V), nst: step i+1 (K), fst: step i+2 (landing), lst: step i+3 (issued now)
  auto iter = [&](int i, const uint8_t* st, const uint8_t* nst, uint8_t* fst, uint8_t* lst) {
    dma_step(lst, next_hb);
    if (tile_ok && i < nsteps) {
      const int key0 = k0 + i * kStep;
      const bool full = key0 + kStep <= k1 && key0 + kStep - 1 <= qpos_first;
      uint4 kop[8];
      read_k(nst, kop);
      float sv[16];
      softmax_max(rs, s_cur, full, key0, k1, qpos, half, c, tau_raw, sv);
      const f32x16_t s_next = qk(kop);
      uint4 pb[2];
      softmax_exp(rs, sv, c, pb);
#pragma unroll
      for (int s16 = 0; s16 < 2; ++s16) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
          rs.o[dt] = mfma32(*reinterpret_cast<const uint4*>(st + v_off + 1024 * dt + 4096 * s16), pb[s16], rs.o[dt]);
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
  for (int base = 0; base < nsteps; base += kWideRing) {
    iter(base, s_st0, s_st1, s_st2, s_st3);
    iter(base + 1, s_st1, s_st2, s_st3, s_st0);
    iter(base + 2, s_st2, s_st3, s_st0, s_st1);
    iter(base + 3, s_st3, s_st0, s_st1, s_st2);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no direct load outlives the workgroup's LDS
  if (!tile_ok) return;
  write_rows<R>(a, rs, half, row_ok, qrow, g, hh, sp, ns, c);
}

// ---------------------------------------------------------------- narrow kernel
// One wave per (segment, kv head, split) of a segment with at most 32 rows per
// kv head.  Each 32-key step arrives by 16 direct global->LDS loads (K: 8 loads
// of 4 whole rows; V^T: 8 loads of 32 dims of one 16-key piece) into a 2-stage
// per-wave ring with the wide kernel's layout and swizzle, and is read back in
// operand order.  Two steps of loads are in flight.  A workgroup is one wave, so
// the wave's own waits are the only synchronisation.
//
// The 33 KB ring allows 4 such workgroups per CU (one wave per SIMD).  This file
// is compiled with the MFMA VGPR form (build option), which keeps the
// accumulators in ordinary VGPRs (178 in all), so the softmax rescale and the
// epilogue touch them without copies between the two register files.
template <int R>
__global__ __launch_bounds__(64) void chunk_narrow_kernel(PoolGeom pool, ChunkArgs a) {
  const Located loc = wave_uniform(locate<kShortList>(a, pool, blockIdx.x, R));
  if (loc.item.x < 0) return;
  const SegInfo& si = loc.si;
  const int s = loc.item.x, g = loc.item.y, sp = loc.item.w;
  const int bs = pool.block_size, lbs = __ffs(bs) - 1;
  const int lane = threadIdx.x, col = lane & 31, half = lane >> 5;
  if (loc.item.z < 0) {
    zero_rows<R>(a, si, g, lane, 64);
    return;
  }

  // Two separate arrays so the compiler tells the stages apart (see the wide kernel).
  __shared__ __align__(1024) uint8_t s_n0[kStageBytes];
  __shared__ __align__(1024) uint8_t s_n1[kStageBytes];
  __shared__ int32_t s_blk[kMaxBlockIds];

  const int prefix = si.n - si.qlen;
  const int kend = si.n;
  const int ns = cdiv(kend, a.split_short);
  const int k0 = sp * a.split_short;
  const int k1 = min(kend, k0 + a.split_short);
  const int nsteps = cdiv(k1 - k0, kStep);
  const int b0 = k0 >> lbs;
  load_tiles(s_blk, a, pool, s, g, b0, ((k1 - 1) >> lbs) - b0 + 1, lane, 64);

  const int rho = col;
  const bool row_ok = rho < si.rows;
  const int tok = rho / R, hh = rho - tok * R;
  const int qpos = prefix + tok;
  const int64_t qrow = int64_t(si.q0) + tok;
  uint4 qv[8];
  load_q(qv, a, row_ok, qrow, g * R + hh, half);
  __syncthreads();

  // Splits start at multiples of 32 keys: each 16-key half of a step lies in one
  // block (see the wide kernel).  K load u (rows 4u + lane/16, stage bytes 1024 u)
  // reads half u / 4; V load u (dims 32 (u % 4) + lane/2 of piece u / 4, stage
  // bytes 8192 + 1024 u) reads half u / 4.
  const int tshift = lbs + 8;
  uint32_t koff[4];  // bytes from the K row of the half's first key, for u % 4
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int kr = 4 * u + (lane >> 4);
    koff[u] = uint32_t((kr * kHeadDim + ((lane & 15) ^ kr) * 8) * 2);
  }
  const int vdim = lane >> 1;                     // + 32 (u % 4)
  const int vhalf = (lane & 1) ^ ((vdim >> 3) & 1);  // the lane's 8-key half of the piece
  const uint32_t voff = uint32_t((bs * kHeadDim + vdim * kVSub + 8 * vhalf) * 2);
  const uint8_t* kv_bytes = reinterpret_cast<const uint8_t*>(pool.kv);
  auto fetch = [&](uint8_t* st, int step) {
    const int key0 = k0 + step * kStep;
    const uint8_t* hb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int hk = min(key0 + 16 * h, k1 - 1) & ~15;
      const int blk = __builtin_amdgcn_readfirstlane(s_blk[(hk >> lbs) - b0]);
      hb[h] = kv_bytes + ((int64_t(blk) << tshift) + (hk & (bs - 1)) * kHeadDim) * 2;
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // this stage's operand reads are complete
#pragma unroll
    for (int u = 0; u < 8; ++u) dma16(reinterpret_cast<const uint16_t*>(hb[u >> 2] + koff[u & 3]), st + 1024 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      dma16(reinterpret_cast<const uint16_t*>(hb[u >> 2] + voff + 32 * kVSub * 2 * (u & 3)), st + kVBytes0 + 1024 * u);
  };

  RowState rs;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) rs.o[dt] = f32x16_t{};
  rs.m = -INFINITY;
  rs.l = 0.f;
  const float c = a.qk_scale_log2;
  const float tau_raw = kTau / c;
  const int kperm = (col & ~12) | ((col & 4) << 1) | ((col & 8) >> 1);
  const int k_off = kperm * 256 + ((half ^ ((kperm >> 3) & 1)) << 7) + ((kperm & 7) << 4);
  const int v_off = kVBytes0 + col * 32 + ((half ^ ((col >> 3) & 1)) << 4);

  // Step i: wait for its loads (the 16 of step i+1 may stay in flight), scores,
  // softmax and PV.  Loads are clamped to the last step.
  auto step = [&](const uint8_t* st, int i) {
    const int key0 = k0 + i * kStep;
    __builtin_amdgcn_s_waitcnt(kWaitVm16);
    if (key0 + kStep > k1) {
      // V of keys past the split end must be 0 (0 * NaN would poison O): each
      // lane clears its own chunks of the split's last step in the stage.
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kv = key0 + 16 * (u >> 2) + 8 * vhalf;
        if (kv + 8 > k1) {
          uint4* p = reinterpret_cast<uint4*>(const_cast<uint8_t*>(st) + kVBytes0 + 1024 * u + 16 * lane);
          uint4 v = *p;
          v.x &= keep2(kv + 0, k1); v.y &= keep2(kv + 2, k1);
          v.z &= keep2(kv + 4, k1); v.w &= keep2(kv + 6, k1);
          *p = v;
        }
      }
    }
    uint4 kop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kop[ks] = *reinterpret_cast<const uint4*>(st + (k_off ^ (ks << 4)));
    f32x16_t sacc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) sacc = mfma32(kop[ks], qv[ks], sacc);
    const bool full = key0 + kStep <= k1 && key0 + kStep - 1 <= prefix;
    softmax_pv(rs, sacc, full, key0, k1, qpos, half, c, tau_raw, [&](int dt, int s16) {
      return *reinterpret_cast<const uint4*>(st + v_off + 1024 * dt + 4096 * s16);
    });
  };

  fetch(s_n0, 0);
  fetch(s_n1, min(1, nsteps - 1));
  for (int base = 0; base < nsteps; base += 2) {
    step(s_n0, base);
    fetch(s_n0, min(base + 2, nsteps - 1));
    if (base + 1 < nsteps) step(s_n1, base + 1);
    fetch(s_n1, min(base + 3, nsteps - 1));
  }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no direct load outlives the workgroup's LDS
  write_rows<R>(a, rs, half, row_ok, qrow, g, hh, sp, ns, c);
}

// ---------------------------------------------------------------- combine
// Log-sum-exp combine of the split partials of 8 rows of one tile: 32 lanes
// per row, each owning 4 dims.  Rows with at most 16 splits load every partial
// at once and exchange the split weights by shuffle.  Longer rows first reduce
// the row's split lse values (lane j takes splits j, j+32, ...), then the split
// weights go through LDS and every lane sums its 4 dims over the splits in
// order.
template <int R>
__global__ __launch_bounds__(256) void chunk_combine_kernel(PoolGeom pool, ChunkArgs a) {
  const Located loc = locate<kCombineList>(a, pool, blockIdx.x, R);
  if (loc.item.x < 0) return;
  const SegInfo& si = loc.si;
  const int g = loc.item.y, tile = loc.item.z, part = loc.item.w;
  const int tid = threadIdx.x, row = tid >> 5, j = tid & 31;
  const int rho = tile * kRows + part * kCombineRows + row;
  const int ns = si.tiles == 1 ? cdiv(si.n, a.split_short) : cdiv(wide_kend(si, tile / kWideTiles, R), a.split_wide);
  const bool row_ok = rho < si.rows;
  const int tok = rho / R, hh = rho - tok * R;
  const int64_t qrow = int64_t(si.q0) + tok;
  const int64_t stride = int64_t(a.total_q) * R;  // partial rows per split
  const int64_t base = int64_t(g) * a.max_splits * stride + qrow * R + hh;
  __shared__ float s_w[kCombineRows][kCombineChunk];
  const float* src = a.part_o + base * kHeadDim + 4 * j;

  if (ns <= kCombineFast) {
    // Up to 16 splits: every partial load is issued first, beside the one lse
    // value lane j (< ns) reads; the weights then travel between the row's 32
    // lanes by shuffle, and the partials are summed in split order.
    float4 v[kCombineFast];
#pragma unroll
    for (int k = 0; k < kCombineFast; ++k)
      v[k] = row_ok && k < ns ? *reinterpret_cast<const float4*>(src + k * stride * kHeadDim)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
    const float lk = row_ok && j < ns ? a.part_lse[base + j * stride] : -INFINITY;
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
    uint16_t* dst = a.out + (qrow * a.num_q_heads + g * R + hh) * kHeadDim + 4 * j;
    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
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
      s_w[row][k] = lk == -INFINITY || M == -INFINITY ? 0.f : fast_exp2(lk - M) * inv;
    }
    __syncthreads();
    if (row_ok) {
#pragma unroll 8
      for (int k = 0; k < cn; ++k) {
        const float w = s_w[row][k];
        const float4 v = *reinterpret_cast<const float4*>(src + (c0 + k) * stride * kHeadDim);
        acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
      }
    }
  }
  if (!row_ok) return;
  uint16_t* dst = a.out + (qrow * a.num_q_heads + g * R + hh) * kHeadDim + 4 * j;
  *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
}

template <int R>
hipError_t launch_r(const PoolGeom& pool, const ChunkArgs& a, const ChunkGrids& grids, hipStream_t stream) {
  if (grids.wide > 0) {
    hipLaunchKernelGGL((chunk_wide_kernel<R>), dim3(grids.wide), dim3(kWideThreads), 0, stream, pool, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (grids.narrow > 0) {
    hipLaunchKernelGGL((chunk_narrow_kernel<R>), dim3(grids.narrow), dim3(64), 0, stream, pool, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (grids.combine > 0) {
    hipLaunchKernelGGL((chunk_combine_kernel<R>), dim3(grids.combine), dim3(256), 0, stream, pool, a);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

ChunkGrids chunk_grids(int32_t num_segments, int32_t total_q, int32_t num_kv_heads, int32_t group, int32_t max_q_len,
                       int32_t max_ctx, int32_t split_wide, int32_t split_short, int32_t max_splits) {
  ChunkGrids b;
  const int64_t ctx = max_ctx > 0 ? max_ctx : 1;
  const int64_t N = num_segments, hkv = num_kv_heads;
  const ChunkLists lists = chunk_lists(num_segments, total_q, group, max_q_len);
  const bool wide = lists.wide, narrow = lists.narrow;
  const int64_t rows_per_group = int64_t(kRows) * kWideTiles;
  const int64_t groups = (int64_t(total_q) * group + rows_per_group - 1) / rows_per_group + N;
  b.wide = wide ? (groups * ((ctx + split_wide - 1) / split_wide) + N) * hkv : 0;
  b.narrow = narrow ? N * hkv * ((ctx + split_short - 1) / split_short) : 0;
  const int64_t tiles = (int64_t(total_q) * group + kRows - 1) / kRows + N;
  b.combine = max_splits > 1 ? tiles * hkv * kCombineParts : 0;
  return b;
}

ChunkWorkspace chunk_workspace_layout(int32_t total_q, int32_t num_q_heads, int32_t max_splits) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  ChunkWorkspace w;
  w.part_o_off = w.part_lse_off = w.total = 0;
  if (max_splits > 1) {
    const size_t rows = size_t(max_splits) * total_q * num_q_heads;  // Hkv * r == Hq
    w.part_lse_off = up(rows * kHeadDim * sizeof(float));
    w.total = w.part_lse_off + up(rows * sizeof(float));
  }
  return w;
}

hipError_t launch_chunk(const PoolGeom& pool, const ChunkArgs& a, const ChunkGrids& grids, hipStream_t stream) {
  if (a.num_segments == 0 || a.total_q == 0) return hipSuccess;
  if (a.split_wide > 4096 || a.split_short > 4096 || a.split_wide % kStep || a.split_short % kStep ||
      a.num_segments > 4096)
    return hipErrorInvalidValue;
  switch (a.num_q_heads / pool.num_kv_heads) {
    case 1: return launch_r<1>(pool, a, grids, stream);
    case 2: return launch_r<2>(pool, a, grids, stream);
    case 4: return launch_r<4>(pool, a, grids, stream);
    case 8: return launch_r<8>(pool, a, grids, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pgqa
