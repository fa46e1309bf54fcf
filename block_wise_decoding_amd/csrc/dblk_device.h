// Device-side helpers shared by the libdblock kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dblk {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWave = 64;

// 16x16x32 bf16 MFMA (gfx950): D[16][16] += A[16][32] * B[32][16].
// Lane l supplies A row (l % 16) and B column (l % 16), each as 8 consecutive
// k values of the k-group (l / 16); it receives D rows 4*(l/16) + 0..3 of
// column (l % 16).  A and B use the same k grouping, so any consistent
// assignment of k indices to (lane group, slot) gives the same product.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32x32x16 bf16 MFMA (gfx950): D[32][32] += A[32][16] * B[16][32].  Lane l
// supplies A row (l % 32) and B column (l % 32) as 8 consecutive k of k-group
// (l / 32); accumulator register r of lane l holds D[8 (r / 4) + 4 (l / 32) +
// (r % 4)][l % 32].
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte load of data that one call streams through exactly once, issued so
// that each wave instruction covers whole 128-byte lines.  With the
// nontemporal hint such loads stream at ~6.9 TB/s on gfx950 against ~6.1 TB/s
// for plain loads (read probe over a 644 MB buffer); on half-line footprints
// the hint loses instead, so callers use it only for whole-line patterns.
__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Running (max, sum of exp(x - max), argmax) triple of a softmax over a
// vocabulary range.  Combination keeps the lowest index among equal maxima
// and is exact in the max / index; the sum is rescaled in fp32.
struct SoftmaxPart {
  float m;    // max logit (natural units); -inf when empty
  float s;    // sum of exp(logit - m)
  int32_t i;  // lowest index attaining m; INT32_MAX when empty
};

__device__ __forceinline__ SoftmaxPart combine(SoftmaxPart a, SoftmaxPart b) {
  SoftmaxPart r;
  if (b.m > a.m) {
    r.m = b.m;
    r.i = b.i;
    r.s = b.s + a.s * fast_exp2((a.m - b.m) * kLog2e);
  } else if (b.m < a.m) {
    r.m = a.m;
    r.i = a.i;
    r.s = a.s + b.s * fast_exp2((b.m - a.m) * kLog2e);
  } else {  // equal maxima (both -inf included): sums add, lowest index wins
    r.m = a.m;
    r.i = a.i < b.i ? a.i : b.i;
    r.s = a.s + b.s;
  }
  return r;
}

__device__ __forceinline__ SoftmaxPart shfl_xor(SoftmaxPart p, int mask) {
  SoftmaxPart r;
  r.m = __shfl_xor(p.m, mask, kWave);
  r.s = __shfl_xor(p.s, mask, kWave);
  r.i = __shfl_xor(p.i, mask, kWave);
  return r;
}

}  // namespace dblk
