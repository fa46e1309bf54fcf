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


// ---- LDS DMA (buffer loads that write LDS directly: lane i of an instruction
// fills bytes [16 i, 16 i + 16) of the 1 KiB block whose address is the
// instruction's LDS operand).
typedef __attribute__((address_space(3))) void* lds_ptr_t;
// Nontemporal (streaming) cache policy bit of a DMA load.
constexpr int kDmaStream = 2;

// Workgroup barrier after this wave's LDS reads have landed.  Written as asm
// with a memory clobber: LDS DMA writes still in flight must not be waited for
// here (a fence would add vmcnt(0)), and no LDS access may move across it.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// Wait until at most N of this wave's vector memory instructions (DMA loads
// among them) are outstanding; they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// 16-byte load of data that one call streams through exactly once, issued so
// that each wave instruction covers whole 128-byte lines.  With the
// nontemporal hint such loads stream at ~6.9 TB/s on gfx950 against ~6.1 TB/s
// for plain loads (read probe over a 644 MB buffer); on half-line footprints
// the hint loses instead, so callers use it only for whole-line patterns.
__device__ __forceinline__ u32x4 load_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Two floats -> packed bf16 (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two floats <-> packed IEEE half (lo in bits 0..15), round to nearest even.
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
__device__ __forceinline__ f32x2 unpack_f16x2(uint32_t v) {
  return __builtin_convertvector(__builtin_bit_cast(f16x2, v), f32x2);
}

// Running (max, sum of exp(x - max), argmax) triple of a softmax over a
// vocabulary range.  Combination keeps the lowest index among equal maxima
// and is exact in the max / index; the sum is rescaled in fp32.
struct SoftmaxPart {
  float m;    // max logit (natural units); -inf when empty
  float s;    // sum of exp(logit - m)
  int32_t i;  // lowest index attaining m; INT32_MAX when empty
};

// Branch-free (no divergence inside a wave): both sums are rescaled to the
// larger maximum; exp2(0) = 1 exactly, and with both maxima -inf the sums
// simply add.
__device__ __forceinline__ SoftmaxPart combine(SoftmaxPart a, SoftmaxPart b) {
  SoftmaxPart r;
  r.m = fmaxf(a.m, b.m);
  const bool empty = r.m == -__builtin_inff();
  const float ea = empty ? 1.f : fast_exp2((a.m - r.m) * kLog2e);
  const float eb = empty ? 1.f : fast_exp2((b.m - r.m) * kLog2e);
  r.s = a.s * ea + b.s * eb;
  r.i = a.m > b.m ? a.i : (b.m > a.m ? b.i : (a.i < b.i ? a.i : b.i));
  return r;
}

// Combine n partials held in registers as a fixed binary tree (depth
// log2 n instead of a chain of n): the result is deterministic, with the
// max and argmax exact and the sum rescaled in this fixed order.
template <int N>
__device__ __forceinline__ SoftmaxPart combine_tree(SoftmaxPart (&v)[N]) {
#pragma unroll
  for (int stride = 1; stride < N; stride *= 2)
#pragma unroll
    for (int u = 0; u + stride < N; u += 2 * stride) v[u] = combine(v[u], v[u + stride]);
  return v[0];
}

__device__ __forceinline__ SoftmaxPart shfl_xor(SoftmaxPart p, int mask) {
  SoftmaxPart r;
  r.m = __shfl_xor(p.m, mask, kWave);
  r.s = __shfl_xor(p.s, mask, kWave);
  r.i = __shfl_xor(p.i, mask, kWave);
  return r;
}

// ---- Cross-workgroup hand-off without fences.  On this multi-XCD part an
// agent-scope fence writes back and invalidates the whole L2 of the XCD,
// stalling every workgroup still streaming.  Instead partial results travel
// through agent-scope relaxed atomic stores and loads (write-through /
// coherent accesses to just those lines), the writer drains its own stores
// with s_waitcnt before an agent-scope arrival counter is incremented, and
// only that counter decides which workgroup reads them back.
__device__ __forceinline__ void store_coherent(f32x4* p, f32x4 v) {
  uint64_t* d = reinterpret_cast<uint64_t*>(p);
  __hip_atomic_store(d, __builtin_bit_cast(uint64_t, f32x2{v[0], v[1]}), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, __builtin_bit_cast(uint64_t, f32x2{v[2], v[3]}), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 load_coherent(const f32x4* p) {
  const uint64_t* d = reinterpret_cast<const uint64_t*>(p);
  const f32x2 a = __builtin_bit_cast(f32x2, __hip_atomic_load(d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const f32x2 b = __builtin_bit_cast(f32x2, __hip_atomic_load(d + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return f32x4{a[0], a[1], b[0], b[1]};
}

__device__ __forceinline__ void store_coherent(f32x2* p, f32x2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x2 load_coherent(const f32x2* p) {
  return __builtin_bit_cast(f32x2, __hip_atomic_load(reinterpret_cast<const uint64_t*>(p),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Count this workgroup's arrival on *ctr (after all of its coherent stores
// have completed) and tell every thread whether it is the last of `expected`.
__device__ __forceinline__ bool arrive_last(uint32_t* ctr, int expected, int tid, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's write-through stores are complete
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = (prev == (uint32_t)(expected - 1)) ? 1 : 0;
  }
  __syncthreads();
  return *s_flag != 0;
}

// Cache policy bits of a buffer instruction for agent-scope coherent
// accesses (sc1: what the compiler emits for agent-scope atomic loads and
// stores on gfx950), and the last descriptor word of a raw 32-bit buffer.
constexpr int kCachePolicySc1 = 16;
constexpr int kBufferDword3 = 0x00020000;

__device__ __forceinline__ void rearm_counter(uint32_t* ctr) {
  __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace dblk
