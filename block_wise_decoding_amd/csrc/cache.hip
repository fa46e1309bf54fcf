// Dual KV cache upkeep at block completion.
//
// With the dual cache (the README's dual KV-cache factory, usage section) a block's queries
// attend over a cached prefix, the block itself and a cached suffix.  When a
// block is complete its keys/values become part of the prefix of the next
// block: the L block rows of every (sequence, head) are appended after that
// sequence's prefix_len[b] valid prefix rows, and prefix_len[b] grows by L.
// Sequences have their own prefix lengths (ragged batches), so each (b, h)
// copies its L*D contiguous elements to its own offset.  The suffix needs no
// copy: the next block's suffix is the old one without its first L rows, a
// different base pointer over the same rows (attention takes the suffix row
// stride separately from its length).
//
// Pure data movement, HBM-bound: 2 * B*H*L*D*2 bytes read and written.
// Two launches: the copy reads prefix_len, a second one-thread-per-sequence
// kernel then advances it (so prefix_len can be updated in place).
#include "dblk_device.h"
#include "dblk_launch.h"

namespace dblk {

namespace {

constexpr int kCopyThreads = 256;
constexpr int kCopyPer = 4;      // 16-byte chunks per thread, all loads before any store

__device__ __forceinline__ int clamp_prefix(const int32_t* prefix_len, int b, int P_cap) {
  int P_b = prefix_len[b];
  return P_b < 0 ? 0 : (P_b > P_cap ? P_cap : P_b);
}

// grid (chunk groups, H, B)
__global__ void __launch_bounds__(kCopyThreads)
cache_append_kernel(uint16_t* __restrict__ kp, uint16_t* __restrict__ vp,
                    const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                    const int32_t* __restrict__ prefix_len, int H, int L, int D, int P_cap) {
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int P_b = clamp_prefix(prefix_len, b, P_cap);
  if (P_b + L > P_cap) return;                       // does not fit: sequence left as is
  const size_t bh = (size_t)b * H + h;
  const int nchunk = L * D / 8;
  const u32x4* src_k = reinterpret_cast<const u32x4*>(kb + bh * (size_t)L * D);
  const u32x4* src_v = reinterpret_cast<const u32x4*>(vb + bh * (size_t)L * D);
  u32x4* dst_k = reinterpret_cast<u32x4*>(kp + (bh * (size_t)P_cap + P_b) * D);
  u32x4* dst_v = reinterpret_cast<u32x4*>(vp + (bh * (size_t)P_cap + P_b) * D);
  const int c0 = blockIdx.x * (kCopyThreads * kCopyPer) + threadIdx.x;
  u32x4 rk[kCopyPer], rv[kCopyPer];
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int c = c0 + u * kCopyThreads;
    if (c < nchunk) {
      rk[u] = src_k[c];
      rv[u] = src_v[c];
    }
  }
#pragma unroll
  for (int u = 0; u < kCopyPer; ++u) {
    const int c = c0 + u * kCopyThreads;
    if (c < nchunk) {
      dst_k[c] = rk[u];
      dst_v[c] = rv[u];
    }
  }
}

__global__ void __launch_bounds__(256)
cache_advance_kernel(int32_t* __restrict__ prefix_len, int B, int L, int P_cap,
                     int32_t* __restrict__ appended) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  const int P_b = clamp_prefix(prefix_len, b, P_cap);
  const bool fits = P_b + L <= P_cap;
  prefix_len[b] = fits ? P_b + L : P_b;
  if (appended != nullptr) appended[b] = fits ? L : 0;
}

}  // namespace

hipError_t launch_cache_append(void* kp, void* vp, const void* kb, const void* vb,
                               int32_t* prefix_len, int B, int H, int L, int D, int P_cap,
                               int32_t* appended, hipStream_t stream) {
  const int nchunk = L * D / 8;
  const int gx = (nchunk + kCopyThreads * kCopyPer - 1) / (kCopyThreads * kCopyPer);
  hipError_t e = launch_kernel(cache_append_kernel, dim3(gx, H, B), dim3(kCopyThreads), 0, stream,
                               static_cast<uint16_t*>(kp), static_cast<uint16_t*>(vp),
                               static_cast<const uint16_t*>(kb), static_cast<const uint16_t*>(vb),
                               static_cast<const int32_t*>(prefix_len), H, L, D, P_cap);
  if (e != hipSuccess) return e;
  return launch_kernel(cache_advance_kernel, dim3((B + 255) / 256), dim3(256), 0, stream,
                       prefix_len, B, L, P_cap, appended);
}

}  // namespace dblk
