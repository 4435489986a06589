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
// Splits are merged by a log-sum-exp combine kernel when a row has several:
// the row combine (one workgroup per 8 query rows, no item list) for calls of
// at most 64 segments, else the item combine over the combine list below.
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
#include <limits.h>

#include "chunk_common.hpp"

namespace pgqa {
namespace {

// ---------------------------------------------------------------- work lists
// Three lists, each in segment order:
//   wide    {segment, kv head, tile group, split} of segments with more than one
//           row tile per kv head; {segment, kv head, -1, 0} zeroes the rows of a
//           bad segment that claims more than one tile;
//   short   {segment, kv head, 0, split} of one-tile segments; {.., -1, 0} for bad
//           one-tile segments;
//   combine {segment, kv head, tile, part} for every row tile with several splits
//           (calls of more than 64 segments),
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
      // wide items: the kv head fastest (one head's items on one XCD); combine
      // items: the rows fastest within a head (consecutive workgroups read
      // neighbouring partial rows; 2% faster on a 512-token slice)
      const int g = K == kWideList ? li % hkv : li / per_head, j = K == kWideList ? li / hkv : li % per_head;
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

// ---------------------------------------------------------------- wide kernel
template <int R>
__global__ __launch_bounds__(kWideThreads, 2) void chunk_wide_kernel(PoolGeom pool, ChunkArgs a) {
  const Located loc = wave_uniform(locate<kWideList>(a, pool, blockIdx.x, R));
  if (loc.item.x < 0) return;
  if (loc.item.z < 0) {
    zero_rows<R>(a, loc.si, loc.item.y, threadIdx.x, kWideThreads);
    return;
  }
  __shared__ __align__(1024) uint8_t s_st0[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st1[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st2[kStageBytes];
  __shared__ __align__(1024) uint8_t s_st3[kStageBytes];
  wide_body<R>(pool, a, loc.si, loc.item.x, loc.item.y, loc.item.z, loc.item.w, a.split_wide,
               WideLds{s_st0, s_st1, s_st2, s_st3});
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
  const int64_t stride = int64_t(a.total_q) * a.num_q_heads;  // partial rows per split: [split][token][head]
  const int64_t base = qrow * a.num_q_heads + g * R + hh;
  __shared__ float s_w[kCombineRows][kCombineChunk];
  combine_row(a, base, ns, row_ok, j, s_w[row],
              a.out + (qrow * a.num_q_heads + g * R + hh) * kHeadDim + 4 * j);
}

// Row combine, for calls of at most 64 segments: one workgroup per kv head g
// and 8 consecutive query rows (token t, head in group) of the call, in token
// order.  A row's partials are addressed by (t, head) alone, so the loads of
// its first splits go out at once, beside the segment offsets and context
// lengths (one segment per lane): as many splits as a wide row can have, at
// most kCombineFast.  The row's segment is then the number of segments that
// end at or before t (a ballot), and its split count follows from the segment.
// Rows of bad segments, rows that no segment holds and rows with one split
// (written directly by the attention kernels) are skipped; a row with more
// splits than were loaded early loads them now.  The merges are combine_row's
// (same bits), the long one without LDS, since the rows of a workgroup may
// take different paths.  No item list is derived, so the common merge waits one
// round trip instead of the list scan and two.
constexpr int kRowCombineSegs = 64;

template <int R>
__global__ __launch_bounds__(256) void chunk_combine_rows_kernel(PoolGeom pool, ChunkArgs a) {
  const int hkv = pool.num_kv_heads, N = a.num_segments;
  const int g = blockIdx.x % hkv;
  const int64_t G = int64_t(blockIdx.x / hkv) * kCombineRows + (threadIdx.x >> 5);  // row of kv head g
  const int lane = threadIdx.x & 63, j = threadIdx.x & 31;
  const bool in = G < int64_t(a.total_q) * R;
  const int t = in ? int(G / R) : 0, hh = int(G % R);
  const int64_t stride = int64_t(a.total_q) * a.num_q_heads;  // partial rows per split
  const int64_t base = int64_t(t) * a.num_q_heads + g * R + hh;
  const float* src = a.part_o + base * kHeadDim + 4 * j;
  const float* lse = a.part_lse + base;
  // splits loaded early: a wide row's at most (its keys end by max_ctx)
  const int early = min(min(a.max_splits, cdiv(max(a.max_ctx, 1), a.split_wide)), kCombineFast);
  float4 v[kCombineFast];
#pragma unroll
  for (int k = 0; k < kCombineFast; ++k)
    v[k] = in && k < early ? *reinterpret_cast<const float4*>(src + k * stride * kHeadDim)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
  float lk = in && j < early ? lse[j * stride] : -INFINITY;
  const int e0 = lane < N ? a.qsl[lane] : 0;
  const int e1 = lane < N ? a.qsl[lane + 1] : INT_MAX;
  const int nn = lane < N ? a.ctx[lane] : 0;
  // the wave's two rows: lanes 0-31 and 32-63
  const int t_lo = __shfl(t, 0), t_hi = __shfl(t, 32);
  const int s_lo = __popcll(__ballot(e1 <= t_lo)), s_hi = __popcll(__ballot(e1 <= t_hi));
  const int s = lane < 32 ? s_lo : s_hi;
  const int q0 = __shfl(e0, s & 63), q1 = __shfl(e1, s & 63), n = __shfl(nn, s & 63);
  if (!in || s >= N) return;
  const SegInfo si = seg_info_of(a, s, q0, q1, n, R, pool.block_size);
  const int rho = (t - si.q0) * R + hh;
  if (si.bad || rho < 0 || rho >= si.rows) return;
  const int ns = si.tiles == 1 ? cdiv(si.n, a.split_short)
                               : cdiv(wide_kend(si, rho / (kRows * kWideTiles), R), a.split_wide);
  if (ns <= 1) return;
  uint16_t* dst = a.out + base * kHeadDim + 4 * j;
  if (ns <= kCombineFast) {
    if (ns > early) {
#pragma unroll
      for (int k = 0; k < kCombineFast; ++k)
        if (k >= early && k < ns) v[k] = *reinterpret_cast<const float4*>(src + k * stride * kHeadDim);
      lk = j < ns ? lse[j * stride] : -INFINITY;
    }
    merge_row_fast(v, j < ns ? lk : -INFINITY, ns, true, dst);
    return;
  }
  // Long rows: the row max and weight sum in one pass over the split lse values
  // (lane j takes splits j, j + 32, ...), then the weights of 32 splits at a
  // time travel by shuffle and every lane sums its 4 dims in split order.
  float M = -INFINITY, L = 0.f;
  for (int k = j; k < ns; k += 32) {
    const float l = lse[k * stride];
    if (l > M) {
      L = L * fast_exp2(M - l) + 1.f;
      M = l;
    } else if (l != -INFINITY) {
      L += fast_exp2(l - M);
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
  for (int c0 = 0; c0 < ns; c0 += 32) {
    const float l = c0 + j < ns ? lse[(c0 + j) * stride] : -INFINITY;
    const float wj = l == -INFINITY || M == -INFINITY ? 0.f : fast_exp2(l - M) * inv;
    const int cn = min(32, ns - c0);
    for (int k = 0; k < cn; ++k) {
      const float w = __shfl(wj, k, 32);
      const float4 x = *reinterpret_cast<const float4*>(src + int64_t(c0 + k) * stride * kHeadDim);
      acc.x += w * x.x; acc.y += w * x.y; acc.z += w * x.z; acc.w += w * x.w;
    }
  }
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
    if (a.num_segments <= kRowCombineSegs) {
      const int64_t rows = (int64_t(a.total_q) * R + kCombineRows - 1) / kCombineRows;
      hipLaunchKernelGGL((chunk_combine_rows_kernel<R>), dim3(rows * pool.num_kv_heads), dim3(256), 0, stream, pool,
                         a);
    } else {
      hipLaunchKernelGGL((chunk_combine_kernel<R>), dim3(grids.combine), dim3(256), 0, stream, pool, a);
    }
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
