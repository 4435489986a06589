// Paged split-KV GQA decode attention with a log-sum-exp combine (gfx950).
//
// Page "perf: Qwen3 offline inference - hybrid attention backend, fused
// rms_norm_rope, chunked prefill + prompt-lookup spec decoding", Summary item 1:
// pure decode batches run a self-written paged split-KV kernel over the
// block-table cache.  That design targeted NVIDIA consumer parts; this one is
// laid out for CDNA4.
//
// Work decomposition.  One workgroup per (sequence b, kv head g, split sp); a
// split is split_tokens consecutive keys.  The grid is ordered (g, b, sp), the
// split slowest, so that each split level spreads over all XCDs.  All r = Hq / Hkv query heads of the
// group are processed by the same workgroup, so each K/V byte is read from HBM
// once.  The W waves of the workgroup take the split's 16-key tiles in turn
// (wave w: tiles w, w+W, ...), each wave keeping its own online softmax state.
//
// Inside a wave, for one 16-key tile of one (block, kv head):
//   * keys: the 8-lane group G = lane/8 owns keys 2G and 2G+1; lane s = lane%8
//     owns dims 8s..8s+7 and 64+8s..64+8s+7.  With that split every 16-byte
//     load instruction reads whole 128-byte lines across its lanes.  Scores are
//     bf16 pair dot products (v_dot2_f32_bf16, no unpacking) finished by three
//     DPP steps inside the 8-lane group.
//   * softmax: scores are in log2 units (q.k * scale * log2 e).  The running
//     maximum is only raised when a score exceeds it by more than kTau, which a
//     wave-wide ballot detects; otherwise no max reduction and no rescale is
//     done.  The weights exp2(s - m) (at most 2^kTau) are packed to bf16 pairs
//     and broadcast through LDS.
//   * values: the cache stores V transposed in 16-slot pieces, [dim][slot % 16],
//     so lane l reads dims 32j + l/2 (j = 0..3) for keys 8(l&1)..8(l&1)+7:
//     consecutive lanes read consecutive 16-byte pieces of the tile's 4 KiB
//     piece, at every block size.
//     The weighted sum over key pairs is again v_dot2_f32_bf16; the two key
//     halves of a dim meet once, at the end of the split.
//   * the next tile is loaded while the current one is computed (two register
//     buffers per wave); K/V loads may carry the non-temporal hint.
//
// Combine.  With one split the workgroup writes bf16 directly.  Otherwise it
// writes its normalised partial o_k and lse_k (log2 units), and a second small
// kernel merges the partials of each (sequence, query head) in split order:
// o = sum_k 2^(lse_k - lse) o_k.  (Merging inside the split kernel, by the last
// workgroup to finish, needs device-scope release/acquire fences per
// workgroup; on this chip those write back and invalidate the XCD's L2 and cost
// far more than the extra launch.)
#include <math.h>

#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"
#include "norm_rope.hpp"

namespace pgqa {
namespace {

constexpr float kTau = 8.0f;              // log2 headroom before the running max is raised
constexpr int kMaxTilesPerWave = 64;      // block ids of a wave's tiles live one per lane
constexpr int kCombineFast = 32;          // plans with at most this many splits: one-shot combine

struct Tile {
  uint4 k[4];  // key 2G: k[0] dims 8s.., k[1] dims 64+8s..;  key 2G+1: k[2], k[3]
  uint4 v[4];  // v[j]: V^T row 32j + lane/2, keys 8(lane&1) .. +7 (four bf16 pairs)
  int ok;
};

__device__ __forceinline__ uint32_t comp(const uint4& x, int i) {
  return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
}

template <bool kStream>
__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  if constexpr (kStream) return load_stream(p);
  return *reinterpret_cast<const uint4*>(p);
}

// Merge the W waves' online-softmax states of one (sequence b, kv head g,
// split sp), left in LDS by each wave (max m, weight sum l and unnormalised
// accumulator per column: query head, or (token, head) row of a chunk
// segment), and store the result: bf16 rows (out_row(h): the output row of
// column h) when the sequence has one split, else the
// normalised partials and their lse (log2 units) for the combine.  Only the
// first ncols columns are merged and stored.  Thread i handles (column, dim)
// pairs i, i + 64 W, ...
template <int C, int W, typename OutRow>
__device__ __forceinline__ void merge_waves(const float (&s_m)[W][C], const float (&s_l)[W][C],
                                            const float (&s_acc)[W][C][kHeadDim], const DecodeArgs& a, int b, int g,
                                            int sp, bool single, int hkv, int ncols, OutRow out_row) {
  constexpr int kPairs = C * kHeadDim;
  float* po = a.part_o + ((int64_t(b) * hkv + g) * a.max_splits + sp) * kPairs;
  float* plse = a.part_lse + ((int64_t(b) * hkv + g) * a.max_splits + sp) * C;
  for (int idx = threadIdx.x; idx < ncols * kHeadDim; idx += 64 * W) {
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
      out_row(h)[d] = f32_to_bf16(o);
    } else {
      po[idx] = o;
      if (d == 0) plse[h] = L > 0.f ? M + __log2f(L) : -INFINITY;
    }
  }
}

// Fused step: the cache write of the new token of kv head g (position n - 1)
// into block blk, from LDS rows holding its normed, rotated k and its raw v.
// Called by lanes sub = 0..7 of one wave; lane sub stores dims 8 sub .. +7 and
// 64 + 8 sub .. +7.  A block id outside the pool is flagged, nothing written.
__device__ __forceinline__ void store_new_token(const PoolGeom& pool, int g, int32_t blk, int n, int sub,
                                                const uint16_t* s_newk, const uint16_t* s_newv) {
  if (unsigned(blk) < unsigned(pool.num_blocks)) {
    const int bs = pool.block_size;
    const int off = (n - 1) & (bs - 1);
    uint16_t* tile = pool.kv + (int64_t(blk) * pool.num_kv_heads + g) * tile_elems(pool);
    *reinterpret_cast<uint4*>(tile + int64_t(off) * kHeadDim + sub * 8) =
        *reinterpret_cast<const uint4*>(&s_newk[8 * sub]);
    *reinterpret_cast<uint4*>(tile + int64_t(off) * kHeadDim + 64 + sub * 8) =
        *reinterpret_cast<const uint4*>(&s_newk[64 + 8 * sub]);
    uint16_t* vt = tile + v_elem(bs, off, 0);  // V^T piece [dim][slot % 16]
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      vt[(8 * sub + e) * kVSub] = s_newv[8 * sub + e];
      vt[(64 + 8 * sub + e) * kVSub] = s_newv[64 + 8 * sub + e];
    }
  } else if (sub == 0) {
    raise_error(pool.err, kErrBlockId);
  }
}

template <int R, int W, bool kStream, bool kFused>
__global__ __launch_bounds__(64 * W) void decode_kernel(PoolGeom pool, DecodeArgs a, StepArgs st, UnitOrder ord) {
  // grid (kv head, sequence, split): the split index varies slowest, so every
  // split level is dealt over all 8 XCDs (workgroups go to XCDs round-robin by
  // linear id; with the split fastest, 2 or 4 splits would pin each split level,
  // and the always-present first splits, to a quarter or half of the XCDs)
  const int hq = a.num_q_heads, hkv = pool.num_kv_heads, bs = pool.block_size;
  int g = blockIdx.x, b = blockIdx.y;
  if (ord.count > 0) {  // the host's unit order (read from the kernel arguments)
    const int u = ord.unit[blockIdx.y * hkv + blockIdx.x];
    b = u / hkv;
    g = u - b * hkv;
  }
  const int sp = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 3, sub = lane & 7, khalf = lane & 1;

  __shared__ __align__(16) uint32_t s_p[W][R][8];
  __shared__ float s_m[W][R], s_l[W][R];
  __shared__ __align__(16) float s_acc[W][R][kHeadDim];
  __shared__ __align__(16) uint16_t s_newk[kFused ? kHeadDim : 1];  // fused step: the new token's k and v
  __shared__ __align__(16) uint16_t s_newv[kFused ? kHeadDim : 1];
  // fused step: each wave's normed, rotated q rows and the cos / sin of the 64
  // rotary pairs at the new token's position
  __shared__ __align__(16) uint16_t s_q[kFused ? W : 1][R][kHeadDim];
  __shared__ __align__(16) float s_cs[kFused ? W : 1][64], s_sn[kFused ? W : 1][64];

  // Issue the context length, this wave's block ids and q together: lane i
  // fetches the block id of the wave's i-th tile (tile wave + i*W of the
  // split), read back per tile with readlane.  Entries are fetched only inside
  // the table row, before the context length is known.
  const int n = a.ctx[b];
  const int k0 = sp * a.split_tokens;
  int32_t lane_blk = -1;
  {
    const int tile = wave + lane * W;
    const int64_t entry = (int64_t(k0) + tile * 16) / bs;
    if (tile * 16 < a.split_tokens && entry < a.bt_stride) lane_blk = a.bt[int64_t(b) * a.bt_stride + entry];
  }
  // q of the group, as bf16 pairs, for the lane's dims 8s.. and 64+8s..
  // (fused step: filled after the norm and rotary, below)
  uint32_t qv[R][8];
  if constexpr (!kFused) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const uint16_t* qrow = a.q + int64_t(b) * a.q_stride + (g * R + h) * kHeadDim + sub * 8;
      const uint4 x = *reinterpret_cast<const uint4*>(qrow);
      const uint4 y = *reinterpret_cast<const uint4*>(qrow + 64);
      qv[h][0] = x.x; qv[h][1] = x.y; qv[h][2] = x.z; qv[h][3] = x.w;
      qv[h][4] = y.x; qv[h][5] = y.y; qv[h][6] = y.z; qv[h][7] = y.w;
    }
  }

  // Fused step: lane i fetches the rotary frequency of pair i; lanes 8h + s
  // the raw q row of head g R + h % R and the q norm weight, dims 8s.. and
  // 64+8s.. (groups h < R use them); every lane the new token's raw k, v and
  // the k norm weight of its dims (lanes 0..7 of the wave that writes the token
  // use them; see below).  All are issued now, before the context length is
  // known, and without branches, so that the first tile's loads wait for the
  // block ids alone (the wait counts only loads issued on every path).
  uint4 qx, qy, nk0, nk1, nv0, nv1, nw0, nw1, qw0, qw1;
  double rf = 0.0;
  if constexpr (kFused) {
    static_assert(!kFused || (R <= 8 && (R & (R - 1)) == 0), "fused step: one q row per 8-lane group");
    rf = st.rev_freq[lane];
    const uint16_t* qrow = a.q + int64_t(b) * a.q_stride + (g * R + (grp & (R - 1))) * kHeadDim + sub * 8;
    qx = *reinterpret_cast<const uint4*>(qrow);
    qy = *reinterpret_cast<const uint4*>(qrow + 64);
    qw0 = *reinterpret_cast<const uint4*>(st.wq + 8 * sub);
    qw1 = *reinterpret_cast<const uint4*>(st.wq + 64 + 8 * sub);
    const uint16_t* kr = st.k + int64_t(b) * st.k_stride + g * kHeadDim + sub * 8;
    const uint16_t* vr = st.v + int64_t(b) * st.v_stride + g * kHeadDim + sub * 8;
    nk0 = *reinterpret_cast<const uint4*>(kr);
    nk1 = *reinterpret_cast<const uint4*>(kr + 64);
    nv0 = *reinterpret_cast<const uint4*>(vr);
    nv1 = *reinterpret_cast<const uint4*>(vr + 64);
    nw0 = *reinterpret_cast<const uint4*>(st.wk + 8 * sub);
    nw1 = *reinterpret_cast<const uint4*>(st.wk + 64 + 8 * sub);
  }

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
  const int k1 = min(n, k0 + a.split_tokens);

  // Fused step: the new token sits at position n - 1.  Every workgroup norms and
  // rotates its own q rows (the same device code as the cache-write kernel, so
  // identical bits).  In the workgroup whose split holds key n - 1, the wave
  // that computes the last tile norms and rotates the token's k and keeps it
  // and v in LDS for its own use when it reaches that tile; it stores them into
  // the cache slot only after its tile loop, so the stores hold up no tile
  // load (the slot is read again only after this kernel).  Each wave computes
  // every rotary angle once (lane i: pair i) and every q row once (the 8 lanes
  // of group h: row h), and shares them through its own LDS rows.
  const int patch_tile = kFused && sp == ns - 1 ? (n - 1 - k0) >> 4 : -1;
  const bool writer = kFused && patch_tile >= 0 && wave == patch_tile % W;
  auto wave_lds_order = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };
  auto fused_prologue = [&]() {
    if constexpr (kFused) {
      {
        float c1, s1;
        rope_angle(n - 1, rf, c1, s1);
        s_cs[wave][lane] = c1;
        s_sn[wave][lane] = s1;
      }
      wave_lds_order();
      if (grp < R || (writer && lane < 8)) {
        float cs[8], sn[8];
        const float4 c0 = *reinterpret_cast<const float4*>(&s_cs[wave][8 * sub]);
        const float4 c4 = *reinterpret_cast<const float4*>(&s_cs[wave][8 * sub + 4]);
        const float4 s0 = *reinterpret_cast<const float4*>(&s_sn[wave][8 * sub]);
        const float4 s4 = *reinterpret_cast<const float4*>(&s_sn[wave][8 * sub + 4]);
        cs[0] = c0.x; cs[1] = c0.y; cs[2] = c0.z; cs[3] = c0.w; cs[4] = c4.x; cs[5] = c4.y; cs[6] = c4.z; cs[7] = c4.w;
        sn[0] = s0.x; sn[1] = s0.y; sn[2] = s0.z; sn[3] = s0.w; sn[4] = s4.x; sn[5] = s4.y; sn[6] = s4.z; sn[7] = s4.w;
        if (grp < R) {
          uint4 o0, o1;
          norm_rope_lane(qx, qy, qw0, qw1, cs, sn, st.eps, o0, o1);
          *reinterpret_cast<uint4*>(&s_q[wave][grp][8 * sub]) = o0;
          *reinterpret_cast<uint4*>(&s_q[wave][grp][64 + 8 * sub]) = o1;
          if (st.q_out != nullptr && sp == 0 && wave == 0) {
            uint16_t* dst = st.q_out + (int64_t(b) * hq + g * R + grp) * kHeadDim + sub * 8;
            *reinterpret_cast<uint4*>(dst) = o0;
            *reinterpret_cast<uint4*>(dst + 64) = o1;
          }
        }
        if (writer && lane < 8) {
          uint4 o0, o1;
          norm_rope_lane(nk0, nk1, nw0, nw1, cs, sn, st.eps, o0, o1);
          *reinterpret_cast<uint4*>(&s_newk[8 * sub]) = o0;
          *reinterpret_cast<uint4*>(&s_newk[64 + 8 * sub]) = o1;
          *reinterpret_cast<uint4*>(&s_newv[8 * sub]) = nv0;
          *reinterpret_cast<uint4*>(&s_newv[64 + 8 * sub]) = nv1;
        }
      }
      // the q rows are read back now, the new token's rows in compute()
      wave_lds_order();
#pragma unroll
      for (int h = 0; h < R; ++h) {
        const uint4 x = *reinterpret_cast<const uint4*>(&s_q[wave][h][8 * sub]);
        const uint4 y = *reinterpret_cast<const uint4*>(&s_q[wave][h][64 + 8 * sub]);
        qv[h][0] = x.x; qv[h][1] = x.y; qv[h][2] = x.z; qv[h][3] = x.w;
        qv[h][4] = y.x; qv[h][5] = y.y; qv[h][6] = y.z; qv[h][7] = y.w;
      }
    }
  };
  // The slot write of the new token, from the LDS rows, after the tile loop.
  auto fused_epilogue = [&]() {
    if constexpr (kFused) {
      if (writer && lane < 8) {
        // block id of the token's slot: this wave's tile patch_tile / W
        store_new_token(pool, g, __builtin_amdgcn_readlane(lane_blk, patch_tile / W), n, sub, s_newk, s_newv);
      }
    }
  };

  const int64_t tstride = tile_elems(pool);
  const int64_t bstride = tstride * hkv;
  const uint16_t* pool_g = pool.kv + int64_t(g) * tstride;
  const int ntiles = (k1 - k0 + 15) >> 4;

  float m[R], l[R], acc[R][4];
#pragma unroll
  for (int h = 0; h < R; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
    acc[h][0] = acc[h][1] = acc[h][2] = acc[h][3] = 0.f;
  }

  // Branch-free tile load (no atomics, no divergent paths), so that the
  // compiler counts outstanding loads exactly and waits only for the tile
  // about to be used.  i is the wave-local tile number.  The loads go through
  // a buffer descriptor of the (block, kv head) tile: a prefetch past the
  // wave's last tile (live false) and a tile whose block id is invalid get a
  // descriptor of size 0, so their loads return zeros and read no memory.
  const uint32_t tile_bytes = uint32_t(tstride) * 2u;
  auto load = [&](Tile& tb, int i, bool live) {
    const int tt = wave + i * W;
    const int32_t raw = __builtin_amdgcn_readlane(lane_blk, i);
    const int sub16 = ((k0 + tt * 16) & (bs - 1)) >> 4;
    tb.ok = unsigned(raw) < unsigned(pool.num_blocks);
    const int32_t blk = tb.ok ? raw : 0;
    // (live depends on the wave index, which the compiler takes as varying per
    // lane: readfirstlane keeps the descriptor in scalar registers)
    const uint32_t nbytes = __builtin_amdgcn_readfirstlane(tb.ok && live ? tile_bytes : 0u);
    const auto rsrc = buffer_rsrc(pool_g + int64_t(blk) * bstride, nbytes);
    const uint32_t koff = uint32_t((sub16 * 16 + 2 * grp) * kHeadDim + sub * 8) * 2u;
    tb.k[0] = load_buf<kStream>(rsrc, koff);
    tb.k[1] = load_buf<kStream>(rsrc, koff + 128);
    tb.k[2] = load_buf<kStream>(rsrc, koff + 2 * kHeadDim);
    tb.k[3] = load_buf<kStream>(rsrc, koff + 2 * kHeadDim + 128);
    const uint32_t voff = uint32_t(v_elem(bs, sub16 * 16 + khalf * 8, lane >> 1)) * 2u;
#pragma unroll
    for (int j = 0; j < 4; ++j) tb.v[j] = load_buf<kStream>(rsrc, voff + 64 * j * kVSub);
  };

  // Zero the V entries of keys that are not attended (past the split end, or
  // the whole tile when its block id was invalid): their weight is 0, but the
  // slots may hold any bits, and 0 * NaN would poison the accumulator.
  auto mask_v = [&](Tile& tb, int tt) {
    const int nv = tb.ok ? k1 - (k0 + tt * 16) : 0;  // valid keys in this tile
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int key = 8 * khalf + 2 * t;  // first key of the lane's pair t
      const uint32_t keep = key + 1 < nv ? 0xffffffffu : key < nv ? 0x0000ffffu : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        switch (t) {
          case 0: tb.v[j].x &= keep; break;
          case 1: tb.v[j].y &= keep; break;
          case 2: tb.v[j].z &= keep; break;
          default: tb.v[j].w &= keep; break;
        }
      }
    }
  };

  // Fused step: the new key (tile offset o of the last tile) taken from LDS.
  // K: the 8-lane group o/2 holds it (k[0..1] for even o, k[2..3] for odd).
  // V: lanes with (lane & 1) == o/8 hold keys 8(lane&1).. of dims 32j + lane/2;
  // key o is the low or high half of pair (o%8)/2.
  auto patch = [&](Tile& tb) {
    const int o = (n - 1 - k0) & 15;
    {
      const uint4 x0 = *reinterpret_cast<const uint4*>(&s_newk[8 * sub]);
      const uint4 x1 = *reinterpret_cast<const uint4*>(&s_newk[64 + 8 * sub]);
      const bool ke = grp == (o >> 1) && !(o & 1), ko = grp == (o >> 1) && (o & 1);
      auto sel = [](bool c, const uint4& a, const uint4& b) {
        return make_uint4(c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w);
      };
      tb.k[0] = sel(ke, x0, tb.k[0]);
      tb.k[1] = sel(ke, x1, tb.k[1]);
      tb.k[2] = sel(ko, x0, tb.k[2]);
      tb.k[3] = sel(ko, x1, tb.k[3]);
    }
    // Selects only, no runtime component index (that would put the tile in scratch).
    const bool mine = khalf == (o >> 3);
    const int t = (o & 7) >> 1;
    const uint32_t keep = (o & 1) ? 0x0000ffffu : 0xffff0000u;
    const int shift = (o & 1) ? 16 : 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t nv = uint32_t(s_newv[32 * j + (lane >> 1)]) << shift;
      tb.v[j].x = mine && t == 0 ? (tb.v[j].x & keep) | nv : tb.v[j].x;
      tb.v[j].y = mine && t == 1 ? (tb.v[j].y & keep) | nv : tb.v[j].y;
      tb.v[j].z = mine && t == 2 ? (tb.v[j].z & keep) | nv : tb.v[j].z;
      tb.v[j].w = mine && t == 3 ? (tb.v[j].w & keep) | nv : tb.v[j].w;
    }
  };

  bool bad_blk = false;
  auto compute = [&](Tile& tb, int tt) {
    if constexpr (kFused) {
      if (tt == patch_tile) {
        // an opaque statement keeps this a branch: the patch must not be
        // turned into selects executed on every tile
        asm volatile("");
        patch(tb);
      }
    }
    bad_blk |= !tb.ok;
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
        // only a head whose own scores left the headroom re-bases (whatever the
        // other heads did), so each head's result depends on its scores alone
        if (tm > m[h] + kTau) {
          const float corr = fast_exp2(m[h] - tm);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[h][j] *= corr;
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
      const uint4 pp = *reinterpret_cast<const uint4*>(&s_p[wave][h][4 * khalf]);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[h][j] = dot2_bf16(comp(pp, t), comp(tb.v[j], t), acc[h][j]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Two register buffers; every iteration prefetches unconditionally (past
  // the wave's last tile the load is a no-op: descriptor of size 0).
  const int my_tiles = ntiles > wave ? (ntiles - wave + W - 1) / W : 0;
  if (my_tiles > 0) {
    auto at = [&](int i) { return min(i, my_tiles - 1); };
    Tile ta, tb;
    load(ta, 0, true);
    // fused step: the norm and rotary run while the first tile is in flight;
    // the barrier keeps the scheduler from moving them (and the reuse of the
    // tile's registers) ahead of its loads
    if constexpr (kFused) __builtin_amdgcn_sched_barrier(0);
    fused_prologue();
    for (int i = 0; i < my_tiles; i += 2) {
      load(tb, at(i + 1), i + 1 < my_tiles);
      compute(ta, wave + i * W);
      load(ta, at(i + 2), i + 2 < my_tiles);
      if (i + 1 < my_tiles) compute(tb, wave + (i + 1) * W);
    }
  }
  fused_epilogue();
  if (bad_blk && lane == 0) raise_error(pool.err, kErrBlockId);

  // Wave totals: each 8-lane group summed the weights of its own keys; each
  // lane pair (l, l^1) holds the two key halves of the same four dims.
#pragma unroll
  for (int h = 0; h < R; ++h) {
    l[h] += __shfl_xor(l[h], 8);
    l[h] += __shfl_xor(l[h], 16);
    l[h] += __shfl_xor(l[h], 32);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[h][j] += dpp<kDppXor1>(acc[h][j]);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      s_m[wave][h] = m[h];
      s_l[wave][h] = l[h];
    }
  }
  if (khalf == 0) {
#pragma unroll
    for (int h = 0; h < R; ++h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) s_acc[wave][h][32 * j + (lane >> 1)] = acc[h][j];
    }
  }
  __syncthreads();
  merge_waves<R, W>(s_m, s_l, s_acc, a, b, g, sp, ns == 1, hkv, R, [&](int h) { return out_bg + h * kHeadDim; });
}

// ---------------------------------------------------------------------------
// Matrix-core split kernel.  When several query heads share a kv head, the
// per-key dot products of the kernel above grow with the group size r while
// the bytes per key stay fixed; here both products of a 32-key step run on
// v_mfma_f32_16x16x32_bf16 instead, with the r query heads as MFMA columns
// (columns r..15 hold zero q and are discarded).  Same work unit, split plan,
// partial layout and combine as the kernel above.
//
// Operand layouts: lane l supplies A[m][k] with m = l%16, k = 8(l/16) + j and
// B[k][n] with n = l%16; D[j] of lane l is row 4(l/16) + j, column l%16.
// With c = l/16 and col = l%16:
//   * S^T = K Q^T, two products per step (u = 0, 1), four 32-dim slices each
//     (k of slice s is dim 32s + k).  Row m of product u is key
//     8(m/4) + 4u + m%4 of the step, so D[j] of product u in lane l is key
//     8c + 4u + j: the lane's 8 weights are keys 8c .. 8c+7 in order.
//   * O^T += V^T P^T, eight products (dims 16t .. 16t+15), k = key of the step:
//     the weights above are exactly the lane's B operand, and its A operand
//     (dim 16t + col, keys 8c .. 8c+7) is 16 contiguous bytes of a 16-slot V^T
//     piece.  No operand is transposed or moved between lanes; the only
//     cross-lane work is the row maximum (when it must rise) and the sums.
// Each wave takes every W-th 32-key step of the split and keeps the next
// step's 16 loads in flight while it computes the current one.  At most 256
// registers per lane, so that two waves share each SIMD at every W.

struct MStep {
  uint4 k[2][4];  // score product u, dim slice s: key row of the lane, dims 32s + 8c .. +7
  uint4 v[8];     // PV product t: dim 16t + col, keys 8c .. 8c+7
  int ok;         // bit h: block id of the step's 16-key half h is valid
};

// kStream: K/V loads carry the non-temporal hint.  A K load instruction covers
// 64 bytes of each of 16 key rows, so the other half of each 128-byte line
// comes with the next instruction; with cached loads (the default for this
// kernel) it hits in L2.
//
// kChunk: the same kernel over short causal chunk segments (speculative-verify
// rows, single tokens) instead of one query token per sequence.  Unit b is
// segment b of a chunk call: query tokens query_start_loc[b] .. +q_len - 1 at
// positions n - q_len .. n - 1 of its n keys.  Column col is the (token
// col / R, head col % R) row, so a segment fits when q_len R <= 16; each
// column sees the keys up to its token's position (bottom-right causal).
template <int R, int W, bool kStream, bool kFused, bool kChunk = false>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void decode_mfma_kernel(PoolGeom pool,
                                                                                                  DecodeArgs a,
                                                                                                  StepArgs st,
                                                                                                  UnitOrder ord) {
  static_assert(R <= 16, "query heads per kv head exceed the MFMA columns");
  static_assert(!(kFused && kChunk), "the fused step has one query token per sequence");
  constexpr int C = kChunk ? 16 : R;  // columns in use
  const int hq = a.num_q_heads, hkv = pool.num_kv_heads, bs = pool.block_size;
  int g = blockIdx.x, b = blockIdx.y;
  if (ord.count > 0) {  // the host's unit order (read from the kernel arguments)
    const int u = ord.unit[blockIdx.y * hkv + blockIdx.x];
    b = u / hkv;
    g = u - b * hkv;
  }
  const int sp = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, c = lane >> 4;

  __shared__ float s_m[W][C], s_l[W][C];
  __shared__ __align__(16) float s_acc[W][C][kHeadDim];
  // fused step: each wave's normed, rotated q rows, the cos / sin of the 64
  // rotary pairs at the new token's position, and the new token's k and v
  __shared__ __align__(16) uint16_t s_q[kFused ? W : 1][kFused ? R : 1][kHeadDim];
  __shared__ __align__(16) float s_cs[kFused ? W : 1][64], s_sn[kFused ? W : 1][64];
  __shared__ __align__(16) uint16_t s_newk[kFused ? kHeadDim : 1];
  __shared__ __align__(16) uint16_t s_newv[kFused ? kHeadDim : 1];

  // Context length, block ids and q issued together.  Lane i fetches the block
  // id of half (i & 1) of the wave's step i / 2 (step wave + (i / 2) W of the
  // split); the plan bounds a wave's steps by 32.
  const int n = a.ctx[b];
  const int k0 = sp * a.split_tokens;
  int32_t lane_blk = -1;
  {
    const int off = (wave + (lane >> 1) * W) * 32 + (lane & 1) * 16;
    const int64_t entry = (int64_t(k0) + off) / bs;
    if (off < a.split_tokens && entry < a.bt_stride) lane_blk = a.bt[int64_t(b) * a.bt_stride + entry];
  }
  // Chunk segment: its query rows and the checks of the chunk kernels.
  int q0 = 0, qlen = 1;
  bool rows_ok = true, q_ok = true;
  if constexpr (kChunk) {
    q0 = a.qsl[b];
    const int q1 = a.qsl[b + 1];
    qlen = q1 - q0;
    rows_ok = q0 >= 0 && q1 >= q0 && q1 <= a.total_q;
    q_ok = rows_ok && (b + 1 < a.batch || q1 == a.total_q) && qlen <= a.max_q_len && qlen * R <= 16 && n >= qlen;
  }
  const int tcol = col / R;  // chunk: the column's token in the segment
  const bool cvalid = kChunk ? q_ok && tcol < qlen : col < R;
  // Plain decode: q^T as the B operand of the score products, column col =
  // head g R + col (zero past R), dims 32s + 8c .. +7; chunk segments: head
  // g R + col % R of query token q0 + col / R.  Fused step: lanes
  // 8h + sub (h < R) hold dims 8 sub .. and 64 + 8 sub .. of the raw q row of
  // head g R + h (the layout of the shared norm + rotary code) and the q norm
  // weight of those dims (lanes past 8 R fetch row (h mod R) and leave it
  // unused); lane i fetches the rotary frequency of pair i; every lane fetches
  // the new token's raw k, v and the k norm weight of its dims (lanes 0..7 of
  // the writer use them).  All are issued here, without branches, so that the
  // first step's loads wait for the block ids alone (the wait counts only
  // loads issued on every path).
  uint4 qb[4];
  uint4 qx, qy, nk0, nk1, nv0, nv1, nw0, nw1, qw0, qw1;
  double rf = 0.0;
  const int sub = lane & 7;
  if constexpr (kFused) {
    static_assert(!kFused || (R <= 8 && (R & (R - 1)) == 0), "fused step: one q row per 8-lane group");
    rf = st.rev_freq[lane];
    const uint16_t* qrow = a.q + int64_t(b) * a.q_stride + (g * R + ((lane >> 3) & (R - 1))) * kHeadDim + 8 * sub;
    qx = *reinterpret_cast<const uint4*>(qrow);
    qy = *reinterpret_cast<const uint4*>(qrow + 64);
    qw0 = *reinterpret_cast<const uint4*>(st.wq + 8 * sub);
    qw1 = *reinterpret_cast<const uint4*>(st.wq + 64 + 8 * sub);
    const uint16_t* kr = st.k + int64_t(b) * st.k_stride + g * kHeadDim + sub * 8;
    const uint16_t* vr = st.v + int64_t(b) * st.v_stride + g * kHeadDim + sub * 8;
    nk0 = *reinterpret_cast<const uint4*>(kr);
    nk1 = *reinterpret_cast<const uint4*>(kr + 64);
    nv0 = *reinterpret_cast<const uint4*>(vr);
    nv1 = *reinterpret_cast<const uint4*>(vr + 64);
    nw0 = *reinterpret_cast<const uint4*>(st.wk + 8 * sub);
    nw1 = *reinterpret_cast<const uint4*>(st.wk + 64 + 8 * sub);
  } else {
    // q through a buffer descriptor of the rows this workgroup may read
    // (decode: the q heads of sequence b; chunk: the segment's rows, none when
    // its offsets are bad).  An unused column reads past the end and gets
    // zeros, so the loads are unconditional and no select follows them.  (With
    // a select after plain loads the compiler sank them into per-dword loads
    // under branches; the wait before the first step could then not skip them
    // and held that step's loads back until q had landed.)
    const int64_t row0 = kChunk ? (q_ok ? q0 : 0) : b;
    const int64_t span = kChunk ? (q_ok ? int64_t(qlen) * a.q_stride : 0) : int64_t(hq) * kHeadDim;
    const uint32_t qbytes =
        __builtin_amdgcn_readfirstlane(uint32_t(span * 2 < 0x7fffffff ? span * 2 : 0x7fffffff));
    const auto qrsrc = buffer_rsrc(a.q + row0 * a.q_stride, qbytes);
    const int64_t qe = (kChunk ? int64_t(tcol) * a.q_stride : 0) + (g * R + col % R) * kHeadDim + 8 * c;
    const uint32_t qoff = cvalid ? uint32_t(qe * 2) : 0x80000000u;
#pragma unroll
    for (int s = 0; s < 4; ++s) qb[s] = load_buf<false>(qrsrc, qoff + 64 * s);
  }

  const bool bad_ctx = n < 0 || n > a.max_ctx || int64_t(n) > int64_t(a.bt_stride) * bs;
  uint16_t* out_bg = a.out + (int64_t(b) * hq + g * R) * kHeadDim;
  if constexpr (kChunk) {
    if (!q_ok || bad_ctx) {
      // bad segment metadata: flagged, and its rows (when the offsets are
      // usable) zeroed, as in the chunk kernels
      if (sp == 0) {
        if (tid == 0) raise_error(pool.err, !q_ok ? kErrQuery : kErrContext);
        if (rows_ok) {
          for (int i = tid; i < qlen * R * kHeadDim; i += 64 * W) {
            const int row = i / (R * kHeadDim), e = i - row * (R * kHeadDim);
            a.out[(int64_t(q0) + row) * a.q_stride + g * R * kHeadDim + e] = 0;
          }
        }
      }
      return;
    }
    if (qlen == 0) return;
  } else if (bad_ctx || n == 0) {
    if (sp == 0) {
      if (bad_ctx && tid == 0) raise_error(pool.err, kErrContext);
      for (int i = tid; i < R * kHeadDim; i += 64 * W) out_bg[i] = 0;
    }
    return;
  }
  const int ns = (n + a.split_tokens - 1) / a.split_tokens;
  if (sp >= ns) return;
  const int k1 = min(n, k0 + a.split_tokens);
  // keys the lane's column attends in this split: all of them in decode, up
  // to its token's position in a chunk segment, none for an unused column
  const int klim = kChunk ? (cvalid ? min(k1, n - qlen + tcol + 1) : k0) : k1;

  // Fused step: the new token sits at position n - 1, key o of step
  // patch_step of the last split.  The wave that computes that step norms and
  // rotates its k into LDS beside the raw v, substitutes both into the step's
  // operands, and stores them into the cache slot after its step loop.
  const int patch_step = kFused && sp == ns - 1 ? (n - 1 - k0) >> 5 : -1;
  const int o = (n - 1 - k0) & 31;
  const bool writer = kFused && patch_step >= 0 && wave == patch_step % W;
  auto fused_prologue = [&]() {
    if constexpr (kFused) {
      {
        // each rotary angle once: lane i computes pair i
        float c1, s1;
        rope_angle(n - 1, rf, c1, s1);
        s_cs[wave][lane] = c1;
        s_sn[wave][lane] = s1;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane < 8 * R) {
        float cs[8], sn[8];
        const float4 c0 = *reinterpret_cast<const float4*>(&s_cs[wave][8 * sub]);
        const float4 c4 = *reinterpret_cast<const float4*>(&s_cs[wave][8 * sub + 4]);
        const float4 s0 = *reinterpret_cast<const float4*>(&s_sn[wave][8 * sub]);
        const float4 s4 = *reinterpret_cast<const float4*>(&s_sn[wave][8 * sub + 4]);
        cs[0] = c0.x; cs[1] = c0.y; cs[2] = c0.z; cs[3] = c0.w; cs[4] = c4.x; cs[5] = c4.y; cs[6] = c4.z; cs[7] = c4.w;
        sn[0] = s0.x; sn[1] = s0.y; sn[2] = s0.z; sn[3] = s0.w; sn[4] = s4.x; sn[5] = s4.y; sn[6] = s4.z; sn[7] = s4.w;
        const int h = lane >> 3;
        uint4 o0, o1;
        norm_rope_lane(qx, qy, qw0, qw1, cs, sn, st.eps, o0, o1);
        *reinterpret_cast<uint4*>(&s_q[wave][h][8 * sub]) = o0;
        *reinterpret_cast<uint4*>(&s_q[wave][h][64 + 8 * sub]) = o1;
        if (st.q_out != nullptr && sp == 0 && wave == 0) {
          uint16_t* dst = st.q_out + (int64_t(b) * hq + g * R + h) * kHeadDim + sub * 8;
          *reinterpret_cast<uint4*>(dst) = o0;
          *reinterpret_cast<uint4*>(dst + 64) = o1;
        }
        if (writer && lane < 8) {
          norm_rope_lane(nk0, nk1, nw0, nw1, cs, sn, st.eps, o0, o1);
          *reinterpret_cast<uint4*>(&s_newk[8 * sub]) = o0;
          *reinterpret_cast<uint4*>(&s_newk[64 + 8 * sub]) = o1;
          *reinterpret_cast<uint4*>(&s_newv[8 * sub]) = nv0;
          *reinterpret_cast<uint4*>(&s_newv[64 + 8 * sub]) = nv1;
        }
      }
      // the wave's own LDS rows are read back below
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 x = *reinterpret_cast<const uint4*>(&s_q[wave][col < R ? col : 0][32 * s + 8 * c]);
        qb[s] = sel4(col < R, x, make_uint4(0u, 0u, 0u, 0u));
      }
    }
  };

  const int64_t tstride = tile_elems(pool);
  const int64_t bstride = tstride * hkv;
  const uint16_t* pool_g = pool.kv + int64_t(g) * tstride;
  const int nsteps = (k1 - k0 + 31) >> 5;

  // Lane offsets inside a 16-key half: K row of product 0 (product 1 is 4 rows
  // on) in half col / 8; V^T keys 8(c & 1) .. of dim col in half c / 2.
  const int khalf = col >> 3, vhalf = c >> 1;
  const int k_off = (8 * ((col >> 2) & 1) + (col & 3)) * kHeadDim + 8 * c;
  const int v_off = bs * kHeadDim + col * kVSub + 8 * (c & 1);

  auto load = [&](MStep& ms, int i) {
    const int key = k0 + (wave + i * W) * 32;
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
      for (int s = 0; s < 4; ++s) ms.k[u][s] = ld16<kStream>(kp + 4 * u * kHeadDim + 32 * s);
    }
    const uint16_t* vp = (vhalf ? base1 : base0) + v_off;
#pragma unroll
    for (int t = 0; t < 8; ++t) ms.v[t] = ld16<kStream>(vp + 16 * t * kVSub);
  };

  // Fused step: key o of the step is the new token.  K: the lanes whose row of
  // product u is key o take their four dim slices from LDS.  V: lanes of group
  // c = o / 8 replace element o % 8 of their 8 keys in each product's operand
  // (selects only: a runtime component index would put the step in scratch).
  auto patch = [&](MStep& ms) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint4 x = *reinterpret_cast<const uint4*>(&s_newk[32 * s + 8 * c]);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // bit masks rather than selects: with selects the compiler kept both
        // versions of the step's K operands and spilled them
        const uint32_t nm = 8 * (col >> 2) + 4 * u + (col & 3) == o ? 0xffffffffu : 0u;
        ms.k[u][s].x = (ms.k[u][s].x & ~nm) | (x.x & nm);
        ms.k[u][s].y = (ms.k[u][s].y & ~nm) | (x.y & nm);
        ms.k[u][s].z = (ms.k[u][s].z & ~nm) | (x.z & nm);
        ms.k[u][s].w = (ms.k[u][s].w & ~nm) | (x.w & nm);
      }
    }
    const bool mine = c == (o >> 3);
    const int w = (o & 7) >> 1;
    const uint32_t keep = (o & 1) ? 0x0000ffffu : 0xffff0000u;
    const int shift = (o & 1) ? 16 : 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t nv = uint32_t(s_newv[16 * t + col]) << shift;
      ms.v[t].x = mine && w == 0 ? (ms.v[t].x & keep) | nv : ms.v[t].x;
      ms.v[t].y = mine && w == 1 ? (ms.v[t].y & keep) | nv : ms.v[t].y;
      ms.v[t].z = mine && w == 2 ? (ms.v[t].z & keep) | nv : ms.v[t].z;
      ms.v[t].w = mine && w == 3 ? (ms.v[t].w & keep) | nv : ms.v[t].w;
    }
  };

  f32x4_t acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // of column col; the four lane groups agree on m
  bool bad_blk = false;

  auto compute = [&](MStep& ms, int i) {
    const int step = wave + i * W;
    if constexpr (kFused) {
      if (step == patch_step) {
        // an opaque statement keeps this a branch, and its memory clobber keeps
        // the patch's LDS reads inside it (hoisted out of the step loop they
        // would hold ~24 registers for the whole loop)
        asm volatile("" ::: "memory");
        patch(ms);
      }
    }
    const int key = k0 + step * 32;
    // a half past the split end is never attended: its block id is not checked
    bad_blk |= !(ms.ok & 1) || (key + 16 < k1 && !(ms.ok & 2));
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int s = 0; s < 4; ++s) s0 = mfma16(ms.k[0][s], qb[s], s0);
#pragma unroll
    for (int s = 0; s < 4; ++s) s1 = mfma16(ms.k[1][s], qb[s], s1);
    // the lane's keys key + 8c .. +7: how many hold data (nv) and how many its
    // column attends (na)
    const bool okc = (ms.ok >> vhalf) & 1;
    const int nv = okc ? min(max(k1 - (key + 8 * c), 0), 8) : 0;
    const int na = kChunk ? (okc ? min(max(klim - (key + 8 * c), 0), 8) : 0) : nv;
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = j < na ? s0[j] * a.qk_scale_log2 : -INFINITY;
      x[4 + j] = 4 + j < na ? s1[j] * a.qk_scale_log2 : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
    if (__ballot(mx > m + kTau)) {
      float tm = fmaxf(mx, __shfl_xor(mx, 16));
      tm = fmaxf(tm, __shfl_xor(tm, 32));
      if (tm > m + kTau) {  // only a column whose own scores left the headroom re-bases
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
    // V of keys that are not attended is zeroed: their weight is 0, but the
    // slots may hold any bits, and 0 * NaN would poison the accumulator.
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

  const int my_steps = nsteps > wave ? (nsteps - wave + W - 1) / W : 0;
  if (my_steps > 0) {
    auto at = [&](int i) { return min(i, my_steps - 1); };
    MStep ta, tb;
    load(ta, 0);
    // fused step: the norm and rotary run while the first step is in flight
    // (the barrier keeps them behind its loads)
    if constexpr (kFused) __builtin_amdgcn_sched_barrier(0);
    fused_prologue();
    for (int i = 0; i < my_steps; i += 2) {
      load(tb, at(i + 1));
      compute(ta, i);
      load(ta, at(i + 2));
      if (i + 1 < my_steps) compute(tb, i + 1);
    }
  }
  // (wave 0 of split 0 and the writer wave always have steps: q_out and the
  // new token's slot are written whenever the context is not empty)
  if constexpr (kFused) {
    if (writer && lane < 8) {
      // block id of the token's slot: half o / 16 of this wave's step patch_step / W
      store_new_token(pool, g, __builtin_amdgcn_readlane(lane_blk, 2 * (patch_step / W) + (o >> 4)), n, sub, s_newk,
                      s_newv);
    }
  }
  if (bad_blk && lane == 0) raise_error(pool.err, kErrBlockId);

  // Column totals: each lane group summed the weights of its own keys.
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (col < (kChunk ? qlen * R : R)) {  // the columns the merge reads
    if (c == 0) {
      s_m[wave][col] = m;
      s_l[wave][col] = l;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
      *reinterpret_cast<float4*>(&s_acc[wave][col][16 * t + 4 * c]) =
          make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
  }
  __syncthreads();
  merge_waves<C, W>(s_m, s_l, s_acc, a, b, g, sp, ns == 1, hkv, kChunk ? qlen * R : R, [&](int h) -> uint16_t* {
    if constexpr (kChunk) {
      return a.out + (int64_t(q0) + h / R) * a.q_stride + (g * R + h % R) * kHeadDim;
    } else {
      return out_bg + h * kHeadDim;
    }
  });
}

// Log-sum-exp merge of ns split partials of one output element, in split
// order, for any ns: kCombineFast splits at a time, each group's loads issued
// at once (one lse per lane, weights exchanged by shuffle), groups merged with
// a running maximum and sum.  pl / po point at split 0's lse and partial;
// consecutive splits are lse_stride / o_stride floats apart.  Called by whole
// waves.
__device__ __forceinline__ float merge_splits(const float* pl, int64_t lse_stride, const float* po, int64_t o_stride,
                                              int ns) {
  const int lane = threadIdx.x & 63;
  float M = -INFINITY, L = 0.f, acc = 0.f;
  for (int k0 = 0; k0 < ns; k0 += kCombineFast) {
    float v[kCombineFast];
#pragma unroll
    for (int k = 0; k < kCombineFast; ++k) v[k] = k0 + k < ns ? po[(k0 + k) * o_stride] : 0.f;
    const float lk = lane < kCombineFast && k0 + lane < ns ? pl[(k0 + lane) * lse_stride] : -INFINITY;
    float mg = lk;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mg = fmaxf(mg, __shfl_xor(mg, o));
    const float mn = fmaxf(M, mg);
    if (mn == -INFINITY) continue;  // wave-uniform: no weight yet
    const float e = lk == -INFINITY ? 0.f : fast_exp2(lk - mn);
    float lg = e;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lg += __shfl_xor(lg, o);
    float ag = 0.f;
#pragma unroll
    for (int k = 0; k < kCombineFast; ++k) {
      const float ek = __shfl(e, k);
      if (k0 + k < ns) ag += ek * v[k];
    }
    const float corr = M == -INFINITY ? 0.f : fast_exp2(M - mn);
    L = L * corr + lg;
    acc = acc * corr + ag;
    M = mn;
  }
  return L > 0.f ? acc / L : 0.f;
}

// Log-sum-exp combine of the split partials: one workgroup per (sequence,
// query head), one thread per dim.  Partials are merged in split order, so
// the result does not depend on the order in which split workgroups ran.
// Plans of up to 32 splits issue every load at once, before the context
// length is known (one round trip); longer plans merge 32 splits at a time.
// A separate launch: the kernel boundary makes the partials visible without
// per-workgroup cache write-back fences.
__global__ __launch_bounds__(kHeadDim) void combine_kernel(PoolGeom pool, DecodeArgs a) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int hkv = pool.num_kv_heads, r = a.num_q_heads / hkv;
  const int g = h / r, hh = h - g * r;
  const int64_t unit = int64_t(b) * hkv + g;
  const float* pl = a.part_lse + unit * a.max_splits * r + hh;
  const float* po = a.part_o + (unit * a.max_splits * r + hh) * kHeadDim + d;

  if (a.max_splits <= kCombineFast) {
    // Every load at once: the context length, the partials of all the plan's
    // split slots (slots past this sequence's splits are read but unused) and
    // one lse per lane; the weights then go between lanes by shuffle.
    const int n = a.ctx[b];
    float v[kCombineFast];
#pragma unroll
    for (int k = 0; k < kCombineFast; ++k) v[k] = k < a.max_splits ? po[int64_t(k) * r * kHeadDim] : 0.f;
    const int lane = d & 63;
    const float lraw = lane < a.max_splits ? pl[lane * r] : -INFINITY;
    if (n <= 0 || n > a.max_ctx || int64_t(n) > int64_t(a.bt_stride) * pool.block_size) return;
    const int ns = (n + a.split_tokens - 1) / a.split_tokens;
    if (ns <= 1) return;  // written directly by the split kernel
    const float lk = lane < ns ? lraw : -INFINITY;
    float M = lk;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float e = lk == -INFINITY ? 0.f : fast_exp2(lk - M);
    float L = e;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < kCombineFast; ++k) {
      const float ek = __shfl(e, k);
      if (k < ns) acc += ek * v[k];
    }
    a.out[(int64_t(b) * a.num_q_heads + h) * kHeadDim + d] = f32_to_bf16(L > 0.f ? acc / L : 0.f);
    return;
  }

  const int n = a.ctx[b];
  if (n <= 0 || n > a.max_ctx || int64_t(n) > int64_t(a.bt_stride) * pool.block_size) return;
  const int ns = (n + a.split_tokens - 1) / a.split_tokens;
  if (ns <= 1) return;  // written directly by the split kernel
  a.out[(int64_t(b) * a.num_q_heads + h) * kHeadDim + d] = f32_to_bf16(merge_splits(pl, r, po, int64_t(r) * kHeadDim, ns));
}

// Columns a query-column call can use: max_q_len x group, between 1 and 16.
__host__ __device__ inline int columns_of(const DecodeArgs& a, int r) {
  const int64_t c = int64_t(a.max_q_len) * r;
  return c < 1 ? 1 : c < 16 ? int(c) : 16;
}

// Log-sum-exp combine of the query-column kernel's split partials: one
// workgroup per (kv head, column, segment), one thread per dim, splits merged
// in split order (merge_splits).
// Segments that the split kernel rejected, unused columns and rows with one
// split (written directly) are skipped.
__global__ __launch_bounds__(kHeadDim) void combine_columns_kernel(PoolGeom pool, DecodeArgs a) {
  const int hkv = pool.num_kv_heads, r = a.num_q_heads / hkv;
  const int cols = columns_of(a, r);
  const int g = blockIdx.x / cols, col = blockIdx.x - g * cols, s = blockIdx.y, d = threadIdx.x;
  const int64_t unit = int64_t(s) * hkv + g;
  const float* pl = a.part_lse + unit * a.max_splits * 16 + col;
  const float* po = a.part_o + (unit * a.max_splits * 16 + col) * kHeadDim + d;
  // Plans of up to kCombineFast splits load every partial slot of the column
  // (slots past the segment's splits are read but unused) together with the
  // segment's metadata, so the merge waits one round trip instead of two; the
  // arithmetic is merge_splits' for one group of splits (same bits).
  const bool fast = a.max_splits <= kCombineFast;
  float v[kCombineFast];
  float lraw = -INFINITY;
  const int lane = d & 63;
  if (fast) {
#pragma unroll
    for (int k = 0; k < kCombineFast; ++k) v[k] = k < a.max_splits ? po[int64_t(k) * 16 * kHeadDim] : 0.f;
    lraw = lane < a.max_splits ? pl[lane * 16] : -INFINITY;
  }
  const int q0 = a.qsl[s], q1 = a.qsl[s + 1], n = a.ctx[s];
  const int qlen = q1 - q0;
  const bool ok = q0 >= 0 && q1 >= q0 && q1 <= a.total_q && (s + 1 < a.batch || q1 == a.total_q) &&
                  qlen <= a.max_q_len && qlen * r <= 16 && n >= qlen &&
                  n <= a.max_ctx && int64_t(n) <= int64_t(a.bt_stride) * pool.block_size;
  if (!ok || col >= qlen * r) return;
  const int ns = (n + a.split_tokens - 1) / a.split_tokens;
  if (ns <= 1) return;
  uint16_t* dst = a.out + (int64_t(q0) + col / r) * a.q_stride + (g * r + col % r) * kHeadDim + d;
  if (!fast) {
    *dst = f32_to_bf16(merge_splits(pl, 16, po, 16 * kHeadDim, ns));
    return;
  }
  const float lk = lane < ns ? lraw : -INFINITY;
  float M = lk;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float e = lk == -INFINITY ? 0.f : fast_exp2(lk - M);
  float L = e;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o);
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kCombineFast; ++k) {
    const float ek = __shfl(e, k);
    if (k < ns) acc += ek * v[k];
  }
  *dst = f32_to_bf16(L > 0.f ? acc / L : 0.f);
}

// The combine launch that follows the split kernel when the plan has splits.
hipError_t launch_combine_if_split(const PoolGeom& pool, const DecodeArgs& a, hipStream_t stream) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL(combine_kernel, dim3(a.num_q_heads, a.batch), dim3(kHeadDim), 0, stream, pool, a);
  return hipGetLastError();
}

template <int R, int W, bool kStream>
hipError_t launch_dot(const PoolGeom& pool, const DecodeArgs& a, const StepArgs* st, const UnitOrder& ord,
                      hipStream_t stream) {
  const dim3 grid(pool.num_kv_heads, a.batch, a.max_splits);
  if (st != nullptr) {
    hipLaunchKernelGGL((decode_kernel<R, W, kStream, true>), grid, dim3(64 * W), 0, stream, pool, a, *st, ord);
  } else {
    hipLaunchKernelGGL((decode_kernel<R, W, kStream, false>), grid, dim3(64 * W), 0, stream, pool, a, StepArgs{},
                       ord);
  }
  return launch_combine_if_split(pool, a, stream);
}

template <int R, int W, bool kStream>
hipError_t launch_mfma(const PoolGeom& pool, const DecodeArgs& a, const StepArgs* st, const UnitOrder& ord,
                       hipStream_t stream) {
  const dim3 grid(pool.num_kv_heads, a.batch, a.max_splits);
  if (st != nullptr) {
    hipLaunchKernelGGL((decode_mfma_kernel<R, W, kStream, true>), grid, dim3(64 * W), 0, stream, pool, a, *st, ord);
  } else {
    hipLaunchKernelGGL((decode_mfma_kernel<R, W, kStream, false>), grid, dim3(64 * W), 0, stream, pool, a,
                       StepArgs{}, ord);
  }
  return launch_combine_if_split(pool, a, stream);
}

template <int R, int W>
hipError_t launch_rw(const PoolGeom& pool, const DecodeArgs& a, const StepArgs* st, const UnitOrder& ord,
                     hipStream_t stream) {
  if (a.mfma) {
    if (a.stream_loads) return launch_mfma<R, W, true>(pool, a, st, ord, stream);
    return launch_mfma<R, W, false>(pool, a, st, ord, stream);
  }
  if (a.stream_loads) return launch_dot<R, W, true>(pool, a, st, ord, stream);
  return launch_dot<R, W, false>(pool, a, st, ord, stream);
}

template <int R>
hipError_t launch_r(const PoolGeom& pool, const DecodeArgs& a, const StepArgs* st, const UnitOrder& ord,
                    hipStream_t stream) {
  switch (a.waves) {
    case 1: return launch_rw<R, 1>(pool, a, st, ord, stream);
    case 2: return launch_rw<R, 2>(pool, a, st, ord, stream);
    case 4: return launch_rw<R, 4>(pool, a, st, ord, stream);
    case 8: return launch_rw<R, 8>(pool, a, st, ord, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

DecodeWorkspace decode_workspace_layout(int32_t batch, int32_t num_kv_heads, int32_t group, int32_t max_splits) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  DecodeWorkspace w;
  const size_t units = size_t(batch) * num_kv_heads;
  if (max_splits <= 1) {
    w.part_o_off = w.part_lse_off = w.total = 0;
    return w;
  }
  w.part_o_off = 0;
  w.part_lse_off = w.part_o_off + up(units * max_splits * group * kHeadDim * sizeof(float));
  w.total = w.part_lse_off + up(units * max_splits * group * sizeof(float));
  return w;
}

// Chunk segments of at most 16 query rows per kv head on the matrix-core
// kernel (4 waves, cached loads), then the column combine when split.
template <int R>
hipError_t launch_columns_r(const PoolGeom& pool, const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid(pool.num_kv_heads, a.batch, a.max_splits);
  UnitOrder none;
  none.count = 0;
  hipLaunchKernelGGL((decode_mfma_kernel<R, 4, false, false, true>), grid, dim3(256), 0, stream, pool, a,
                     StepArgs{}, none);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.max_splits == 1) return e;
  hipLaunchKernelGGL(combine_columns_kernel, dim3(pool.num_kv_heads * columns_of(a, R), a.batch), dim3(kHeadDim), 0,
                     stream, pool, a);
  return hipGetLastError();
}

hipError_t launch_decode_columns(const PoolGeom& pool, const DecodeArgs& a, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (a.split_tokens > kMaxTilesPerWave * 16 * 4) return hipErrorInvalidValue;
  switch (a.num_q_heads / pool.num_kv_heads) {
    case 1: return launch_columns_r<1>(pool, a, stream);
    case 2: return launch_columns_r<2>(pool, a, stream);
    case 4: return launch_columns_r<4>(pool, a, stream);
    case 8: return launch_columns_r<8>(pool, a, stream);
    default: return hipErrorInvalidValue;
  }
}

// Split partials of the allocation-free decode step (pgqa_decode_step_noalloc):
// a fixed array in the code object, so each GPU that loads the library holds
// one copy until the process ends.  Host code never passes the array's name to
// a kernel (on the host it is only a stand-in for the symbol); it passes the
// device address that hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const PoolGeom& pool, const DecodeArgs& a, const StepArgs* st, const UnitOrder* ord,
                         hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  if (a.split_tokens > kMaxTilesPerWave * 16 * a.waves) return hipErrorInvalidValue;
  UnitOrder none;
  none.count = 0;
  const UnitOrder& o = ord != nullptr ? *ord : none;
  if (o.count != 0 && o.count != a.batch * pool.num_kv_heads) return hipErrorInvalidValue;
  switch (a.num_q_heads / pool.num_kv_heads) {
    case 1: return launch_r<1>(pool, a, st, o, stream);
    case 2: return launch_r<2>(pool, a, st, o, stream);
    case 4: return launch_r<4>(pool, a, st, o, stream);
    case 8: return launch_r<8>(pool, a, st, o, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pgqa
