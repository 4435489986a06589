// Device helpers shared by the gfx950 kernels of libpgqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pgqa {

constexpr int kHeadDim = 128;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load that is not kept in the caches (global_load ... nt):
// K/V bytes are read once per launch.
__device__ __forceinline__ uint4 load_stream(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Raw buffer descriptor (stride 0; dword 3 as the gfx9 family expects) of
// `bytes` bytes at base.  A load past `bytes` returns zeros and makes no
// memory access, so a descriptor of size 0 turns a wave's loads into no-ops
// without a branch (the compiler's wait counts stay exact).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

// 16-byte load at byte offset off through a buffer descriptor; kStream adds
// the non-temporal hint (buffer_load ... nt).
template <bool kStream>
__device__ __forceinline__ uint4 load_buf(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream ? 2 : 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Sticky error bits, mirrored from include/pgqa.h.
constexpr uint32_t kErrSeqId = 0x1u;
constexpr uint32_t kErrPosition = 0x2u;
constexpr uint32_t kErrBlockId = 0x4u;
constexpr uint32_t kErrContext = 0x8u;
constexpr uint32_t kErrQuery = 0x10u;

__device__ __forceinline__ void raise_error(uint32_t* err, uint32_t bit) {
  __hip_atomic_fetch_or(err, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// bf16 halves of a 32-bit word widened to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t p = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, p);
}

// acc + a.lo*b.lo + a.hi*b.hi with bf16 pairs a, b and an fp32 accumulator.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b),
                                         acc, false);
}

// DPP lane exchanges within 16-lane rows.
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF,
                                                                false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes
constexpr int kDppRowMirror = 0x140;  // lane i <-> 15-i within each 16 lanes

// Sum over each aligned group of 8 lanes; every lane of the group gets the sum.
__device__ __forceinline__ float sum8(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16: lane l supplies A[m][k] with m = l%16, k = 8(l/16)+j
// and B[k][n] with n = l%16; D[i] of lane l is row 4(l/16)+i, column l%16.
__device__ __forceinline__ f32x4_t mfma16(const uint4& a, const uint4& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Component-wise select.  (A ternary on uint4 values can become a select
// between their addresses, which keeps the operands out of registers.)
__device__ __forceinline__ uint4 sel4(bool p, const uint4& x, const uint4& y) {
  return make_uint4(p ? x.x : y.x, p ? x.y : y.y, p ? x.z : y.z, p ? x.w : y.w);
}

}  // namespace pgqa
