// Threshold parallel decoder: one commit step per sequence.
//
// The dInfer README's usage section builds its decoder as a threshold-based
// parallel decoder (threshold 0.9, given the mask and end-of-text ids): in one iteration every
// still-masked position whose confidence meets the threshold takes its argmax
// token, and when none does the single most confident masked position is
// committed so that every iteration makes progress.
//
// One 256-thread workgroup per sequence.  Each thread loads confidence, mask
// and argmax of its positions in one batch (a single memory round trip),
// the workgroup counts threshold hits and finds the most confident masked
// position (largest conf, lowest index on a tie; NaN ranks below every
// number), then the committing threads write tokens and mask.  The work is
// latency-bound (a few hundred bytes per sequence).
//
// Optional parts (CommitOpts):
//  * EOS: after the threshold step, the first position of the row that holds
//    a committed eos_id ends the text; still-masked positions after it are
//    committed as eos_id and the row is flagged finished.
//  * Block loop: the step's iteration index is recorded per committed
//    position, and the number of still-masked positions per sequence is
//    written for the next iteration's kernels to skip complete sequences.
#include "dblk_device.h"
#include "dblk_launch.h"

namespace dblk {

namespace {

constexpr int kCommitThreads = 256;
constexpr int kCommitWaves = kCommitThreads / kWave;

struct Best {
  float v;
  int32_t i;
};

__device__ __forceinline__ Best better(Best a, Best b) {
  if (b.v > a.v) return b;
  if (b.v < a.v) return a;
  return a.i <= b.i ? a : b;
}

// Workgroup-wide sum / min of one int per thread (every thread gets the result).
__device__ __forceinline__ int wg_sum(int v, int* lds) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  __syncthreads();                       // lds may still be read from a previous use
  if ((threadIdx.x % kWave) == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int k = 0; k < kCommitWaves; ++k) t += lds[k];
  return t;
}

__device__ __forceinline__ int wg_min(int v, int* lds) {
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, kWave));
  __syncthreads();
  if ((threadIdx.x % kWave) == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  int t = INT32_MAX;
#pragma unroll
  for (int k = 0; k < kCommitWaves; ++k) t = min(t, lds[k]);
  return t;
}

constexpr int kMaxPer = 4096 / kCommitThreads;   // positions per thread at L = 4096

__global__ void __launch_bounds__(kCommitThreads)
threshold_commit_kernel(const float* __restrict__ conf, const int32_t* __restrict__ amax,
                        int32_t* __restrict__ tokens, uint8_t* __restrict__ mask, int L,
                        float tau, int32_t* __restrict__ n_out, CommitOpts opt) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t row = (size_t)b * (size_t)L;
  const int per = (L + kCommitThreads - 1) / kCommitThreads;
  const bool eos = opt.eos_id >= 0;

  // one batch of loads: this thread's positions tid, tid + 256, ...
  float c[kMaxPer];
  int32_t a[kMaxPer];
  int32_t t[kMaxPer];
  uint8_t m[kMaxPer];
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = tid + k * kCommitThreads;
    const bool ok = k < per && i < L;
    m[k] = ok ? mask[row + i] : 0;
    c[k] = ok ? conf[row + i] : 0.f;
    a[k] = ok ? amax[row + i] : 0;
    t[k] = (ok && eos) ? tokens[row + i] : 0;
  }
  int hits = 0, masked = 0;
  Best best = {-__builtin_inff(), INT32_MAX};
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    if (m[k]) {
      const float x = c[k];
      hits += (x >= tau) ? 1 : 0;
      masked += 1;
      const float key = (x == x) ? x : -__builtin_inff();  // NaN ranks lowest
      best = better(best, Best{key, tid + k * kCommitThreads});
    }
  }
  // wave reduction, then across the workgroup's waves
  for (int off = 32; off > 0; off >>= 1) {
    hits += __shfl_xor(hits, off, kWave);
    masked += __shfl_xor(masked, off, kWave);
    Best o{__shfl_xor(best.v, off, kWave), __shfl_xor(best.i, off, kWave)};
    best = better(best, o);
  }
  __shared__ int s_hits[kCommitWaves];
  __shared__ int s_masked[kCommitWaves];
  __shared__ Best s_best[kCommitWaves];
  __shared__ int s_red[kCommitWaves];
  const int w = tid / kWave;
  if ((tid % kWave) == 0) {
    s_hits[w] = hits;
    s_masked[w] = masked;
    s_best[w] = best;
  }
  __syncthreads();
  int total = 0, n_masked = 0;
  Best fb = {-__builtin_inff(), INT32_MAX};
#pragma unroll
  for (int k = 0; k < kCommitWaves; ++k) {
    total += s_hits[k];
    n_masked += s_masked[k];
    fb = better(fb, s_best[k]);
  }

  // commit decisions; v[k] = the token written when committed
  bool cm[kMaxPer];
  int32_t v[kMaxPer];
#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    const int i = tid + k * kCommitThreads;
    cm[k] = (total > 0) ? (m[k] && c[k] >= tau) : (m[k] && i == fb.i);
    v[k] = a[k];
  }
  int n = total > 0 ? total : (fb.i != INT32_MAX ? 1 : 0);

  if (eos) {
    // first position holding a committed EOS once this step's commits are in
    int first = INT32_MAX;
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      const int i = tid + k * kCommitThreads;
      const bool unmasked = (k < per && i < L) && (!m[k] || cm[k]);
      const int32_t tok = cm[k] ? a[k] : t[k];
      if (unmasked && tok == opt.eos_id && i < first) first = i;
    }
    first = wg_min(first, s_red);
    int fills = 0;
#pragma unroll
    for (int k = 0; k < kMaxPer; ++k) {
      const int i = tid + k * kCommitThreads;
      if (m[k] && !cm[k] && i > first) {   // first == INT32_MAX: never
        cm[k] = true;
        v[k] = opt.eos_id;
        ++fills;
      }
    }
    n += wg_sum(fills, s_red);
    if (tid == 0 && opt.finished != nullptr) opt.finished[b] = first != INT32_MAX ? 1 : 0;
  }

#pragma unroll
  for (int k = 0; k < kMaxPer; ++k) {
    if (cm[k]) {
      const int i = tid + k * kCommitThreads;
      tokens[row + i] = v[k];
      mask[row + i] = 0;
      if (opt.commit_iter != nullptr) opt.commit_iter[row + i] = opt.iter;
    }
  }
  if (tid == 0) {
    if (n_out != nullptr) n_out[b] = n;
    if (opt.remaining != nullptr) opt.remaining[b] = n_masked - n;
    if (opt.n_iters != nullptr && n > 0) opt.n_iters[b] = opt.iter + 1;
  }
}

// Start of a block loop, one workgroup per sequence.
__global__ void __launch_bounds__(kCommitThreads)
block_loop_init_kernel(const uint8_t* __restrict__ mask, int L, int32_t* __restrict__ remaining,
                       int32_t* __restrict__ commit_iter, int32_t* __restrict__ n_iters) {
  const int b = blockIdx.x;
  const size_t row = (size_t)b * (size_t)L;
  __shared__ int s_red[kCommitWaves];
  int cnt = 0;
  for (int i = threadIdx.x; i < L; i += kCommitThreads) {
    cnt += mask[row + i] ? 1 : 0;
    if (commit_iter != nullptr) commit_iter[row + i] = -1;
  }
  cnt = wg_sum(cnt, s_red);
  if (threadIdx.x == 0) {
    remaining[b] = cnt;
    if (n_iters != nullptr) n_iters[b] = 0;
  }
}

// Number of sequences that still have masked positions (block-loop progress).
__global__ void __launch_bounds__(kCommitThreads)
block_loop_count_kernel(const int32_t* __restrict__ remaining, int B, int32_t* __restrict__ out) {
  __shared__ int s_red[kCommitWaves];
  int cnt = 0;
  for (int b = threadIdx.x; b < B; b += kCommitThreads) cnt += remaining[b] > 0 ? 1 : 0;
  cnt = wg_sum(cnt, s_red);
  if (threadIdx.x == 0) out[0] = cnt;
}

}  // namespace

hipError_t launch_block_loop_count(const int32_t* remaining, int B, int32_t* out,
                                   hipStream_t stream) {
  return launch_kernel(block_loop_count_kernel, dim3(1), dim3(kCommitThreads), 0, stream,
                       remaining, B, out);
}

hipError_t launch_threshold_commit(const float* conf, const int32_t* amax, int32_t* tokens,
                                   uint8_t* mask, int B, int L, float tau, int32_t* n_out,
                                   const CommitOpts& opt, hipStream_t stream) {
  return launch_kernel(threshold_commit_kernel, dim3(B), dim3(kCommitThreads), 0, stream, conf,
                       amax, tokens, mask, L, tau, n_out, opt);
}

hipError_t launch_block_loop_init(const uint8_t* mask, int B, int L, int32_t* remaining,
                                  int32_t* commit_iter, int32_t* n_iters, hipStream_t stream) {
  return launch_kernel(block_loop_init_kernel, dim3(B), dim3(kCommitThreads), 0, stream, mask, L,
                       remaining, commit_iter, n_iters);
}

}  // namespace dblk
