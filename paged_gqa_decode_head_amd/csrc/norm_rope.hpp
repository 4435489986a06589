// Per-head RMSNorm + neox rotary of one 128-element row held by 8 lanes
// (gfx950), shared by the cache-write kernel and the fused decode step so both
// produce bit-identical q and k.
//
// Page "perf: Qwen3 offline inference - hybrid attention backend, fused
// rms_norm_rope, chunked prefill + prompt-lookup spec decoding", Summary item 2:
// q and k get a per-head RMSNorm, then full rotary embedding.  Lane s (0..7) of
// an aligned 8-lane group holds dims 8s..8s+7 and 64+8s..64+8s+7: both members
// of its 8 rotary pairs (i, i+64), so the rotation is lane-local and the sum of
// squares takes three DPP steps.  Every product is written out (explicit fmaf
// where a fused multiply-add is meant), so the result does not depend on how
// the compiler contracts the surrounding code.
#pragma once

#include <math.h>

#include "device_common.hpp"

namespace pgqa {

// cos and sin of the rotation of pair i at position pos: the angle pos * f_i
// is reduced in fp64 as a fraction of a turn (rev_freq_i = f_i / 2 pi), exact
// to ~1e-12; an fp32 product pos * f_i at pos ~ 32768 would already be off by
// ~2e-3 rad.  The fraction, centred on 0, goes to v_sin_f32 / v_cos_f32, which
// take their argument in turns: no range reduction left, no branches.
__device__ __forceinline__ void rope_angle(int pos, double rev_freq_i, float& cs, float& sn) {
  const double turns = double(pos) * rev_freq_i;
  const float t = float(turns - rint(turns));  // in [-1/2, 1/2]
  sn = __builtin_amdgcn_sinf(t);
  cs = __builtin_amdgcn_cosf(t);
}

// RMSNorm (weight w) and rotation of the lane's 16 elements x0 (dims 8s..) and
// x1 (dims 64+8s..); cs[j], sn[j] belong to pair 8s+j.  All 8 lanes of the
// group must take part (the sum of squares is a DPP reduction).
__device__ __forceinline__ void norm_rope_lane(const uint4& x0, const uint4& x1, const uint4& w0, const uint4& w1,
                                               const float (&cs)[8], const float (&sn)[8], float eps, uint4& out0,
                                               uint4& out1) {
  const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w}, a1[4] = {x1.x, x1.y, x1.z, x1.w};
  const uint32_t g0[4] = {w0.x, w0.y, w0.z, w0.w}, g1[4] = {w1.x, w1.y, w1.z, w1.w};
  float y0[8], y1[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y0[2 * e] = bf16_lo(a0[e]);
    y0[2 * e + 1] = bf16_hi(a0[e]);
    y1[2 * e] = bf16_lo(a1[e]);
    y1[2 * e + 1] = bf16_hi(a1[e]);
  }
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) ss = fmaf(y1[e], y1[e], fmaf(y0[e], y0[e], ss));
  const float ms = sum8(ss) * (1.0f / kHeadDim);
  const float inv = 1.0f / sqrtf(ms + eps);
  uint32_t o0[4], o1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float r0[2], r1[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 2 * e + u;
      const float wa = u ? bf16_hi(g0[e]) : bf16_lo(g0[e]);
      const float wb = u ? bf16_hi(g1[e]) : bf16_lo(g1[e]);
      const float ya = (y0[j] * inv) * wa;
      const float yb = (y1[j] * inv) * wb;
      r0[u] = fmaf(ya, cs[j], -(yb * sn[j]));
      r1[u] = fmaf(yb, cs[j], ya * sn[j]);
    }
    o0[e] = pack_bf16x2(r0[0], r0[1]);
    o1[e] = pack_bf16x2(r1[0], r1[1]);
  }
  out0 = make_uint4(o0[0], o0[1], o0[2], o0[3]);
  out1 = make_uint4(o1[0], o1[1], o1[2], o1[3]);
}

}  // namespace pgqa
