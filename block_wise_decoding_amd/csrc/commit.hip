// Threshold parallel decoder: one commit step per sequence.
//
// The dInfer README's usage section decodes with ThresholdParallelDecoder(0,
// threshold=0.9, ...): in one iteration every still-masked position whose
// confidence meets the threshold takes its argmax token, and when none does
// the single most confident masked position is committed so that every
// iteration makes progress.
//
// One 256-thread workgroup per sequence.  Each thread loads confidence, mask
// and argmax of its positions in one batch (a single memory round trip),
// the workgroup counts threshold hits and finds the most confident masked
// position (largest conf, lowest index on a tie; NaN ranks below every
// number), then the committing threads write tokens and mask.  The work is
// latency-bound (a few hundred bytes per sequence).
#include "dblk_device.h"
#include "dblk_launch.h"

namespace dblk {

namespace {

constexpr int kCommitThreads = 256;

struct Best {
  float v;
  int32_t i;
};

__device__ __forceinline__ Best better(Best a, Best b) {
  if (b.v > a.v) return b;
  if (b.v < a.v) return a;
  return a.i <= b.i ? a : b;
}

constexpr int kMaxPer = 4096 / kCommitThreads;   // positions per thread at L = 4096

__global__ void __launch_bounds__(kCommitThreads)
threshold_commit_kernel(const float* __restrict__ conf, const int32_t* __restrict__ amax,
                        int32_t* __restrict__ tokens, uint8_t* __restrict__ mask, int L,
                        float tau, int32_t* __restrict__ n_out) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t row = (size_t)b * (size_t)L;
  const int per = (L + kCommitThreads - 1) / kCommitThreads;

  // one batch of loads: this thread's positions tid, tid + 256, ...
  float c[kMaxPer];
  int32_t a[kMaxPer];
  uint8_t m[kMaxPer];
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = tid + k * kCommitThreads;
    const bool ok = k < per && i < L;
    m[k] = ok ? mask[row + i] : 0;
    c[k] = ok ? conf[row + i] : 0.f;
    a[k] = ok ? amax[row + i] : 0;
  }
  int hits = 0;
  Best best = {-__builtin_inff(), INT32_MAX};
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    if (m[k]) {
      const float x = c[k];
      hits += (x >= tau) ? 1 : 0;
      const float key = (x == x) ? x : -__builtin_inff();  // NaN ranks lowest
      best = better(best, Best{key, tid + k * kCommitThreads});
    }
  }
  // wave reduction, then across the workgroup's waves
  for (int off = 32; off > 0; off >>= 1) {
    hits += __shfl_xor(hits, off, kWave);
    Best o{__shfl_xor(best.v, off, kWave), __shfl_xor(best.i, off, kWave)};
    best = better(best, o);
  }
  __shared__ int s_hits[kCommitThreads / kWave];
  __shared__ Best s_best[kCommitThreads / kWave];
  const int w = tid / kWave;
  if ((tid % kWave) == 0) {
    s_hits[w] = hits;
    s_best[w] = best;
  }
  __syncthreads();
  int total = 0;
  Best fb = {-__builtin_inff(), INT32_MAX};
#pragma unroll
  for (int k = 0; k < kCommitThreads / kWave; ++k) {
    total += s_hits[k];
    fb = better(fb, s_best[k]);
  }

#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = tid + k * kCommitThreads;
    const bool commit = (total > 0) ? (m[k] && c[k] >= tau) : (i == fb.i);
    if (commit) {
      tokens[row + i] = a[k];
      mask[row + i] = 0;
    }
  }
  if (tid == 0 && n_out != nullptr) n_out[b] = total > 0 ? total : (fb.i != INT32_MAX ? 1 : 0);
}

}  // namespace

hipError_t launch_threshold_commit(const float* conf, const int32_t* amax, int32_t* tokens,
                                   uint8_t* mask, int B, int L, float tau, int32_t* n_out,
                                   hipStream_t stream) {
  return launch_kernel(threshold_commit_kernel, dim3(B), dim3(kCommitThreads), 0, stream, conf,
                       amax, tokens, mask, L, tau, n_out);
}

}  // namespace dblk
