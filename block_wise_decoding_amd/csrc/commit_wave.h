// The threshold decoder step (as threshold_commit_kernel in commit.hip) for
// the whole sequences held by one 64-row chunk, run by a single wave: lane r
// holds row m0 + r with its confidence and argmax; a sequence is a group of
// L consecutive lanes (L a power of two dividing 64), so every reduction is a
// segmented butterfly over xor offsets below L.  Decisions, tie-breaks, NaN
// handling, EOS fill and the block-loop records match the standalone kernel
// exactly (same fp32 values and comparisons).
#pragma once

#include "dblk_device.h"
#include "dblk_launch.h"

namespace dblk {

// The decoder-state inputs of row m0 + lane (mask, and tokens under EOS),
// loaded at kernel start by every workgroup so that the one that finishes
// the chunk does not wait for them.  Nothing writes them before that point.
struct CommitIn {
  uint8_t m;
  int32_t t;
};

__device__ __forceinline__ CommitIn commit_prefetch(const FusedCommit& fc, int m0, int M, int lane) {
  const int row = m0 + lane;
  CommitIn in{0, 0};
  if (fc.tokens != nullptr && row < M) {
    in.m = fc.mask[row];
    if (fc.opt.eos_id >= 0) in.t = fc.tokens[row];
  }
  return in;
}

__device__ __forceinline__ void commit_chunk_wave(const FusedCommit& fc, int m0, int M, int lane,
                                                  float c, int32_t a, CommitIn in) {
  const int L = fc.L;
  const int row = m0 + lane;
  const bool valid = row < M;
  const int pos = row & (L - 1);
  const int seq = row / L;
  const bool eos = fc.opt.eos_id >= 0;
  const bool m = valid && in.m != 0;
  const int32_t t = in.t;

  int hits = (m && c >= fc.tau) ? 1 : 0;
  int masked = m ? 1 : 0;
  float bv = m ? ((c == c) ? c : -__builtin_inff()) : -__builtin_inff();  // NaN ranks lowest
  int bi = m ? pos : INT32_MAX;
  for (int off = L >> 1; off > 0; off >>= 1) {
    hits += __shfl_xor(hits, off, kWave);
    masked += __shfl_xor(masked, off, kWave);
    const float ov = __shfl_xor(bv, off, kWave);
    const int oi = __shfl_xor(bi, off, kWave);
    if (ov > bv || (ov == bv && oi < bi)) {   // larger conf, then lower position
      bv = ov;
      bi = oi;
    }
  }
  const bool step = hits > 0 ? (m && c >= fc.tau) : (m && pos == bi);
  int n = hits > 0 ? hits : (bi != INT32_MAX ? 1 : 0);
  bool cm = step;
  int32_t v = a;
  if (eos) {
    int first = (valid && (!m || step) && (step ? a : t) == fc.opt.eos_id) ? pos : INT32_MAX;
    for (int off = L >> 1; off > 0; off >>= 1) first = min(first, __shfl_xor(first, off, kWave));
    const bool fill = m && !step && pos > first;
    int fills = fill ? 1 : 0;
    for (int off = L >> 1; off > 0; off >>= 1) fills += __shfl_xor(fills, off, kWave);
    if (fill) {
      cm = true;
      v = fc.opt.eos_id;
    }
    n += fills;
    if (valid && pos == 0 && fc.opt.finished != nullptr)
      fc.opt.finished[seq] = first != INT32_MAX ? 1 : 0;
  }
  if (cm) {
    fc.tokens[row] = v;
    fc.mask[row] = 0;
    if (fc.opt.commit_iter != nullptr) fc.opt.commit_iter[row] = fc.opt.iter;
  }
  if (valid && pos == 0) {
    if (fc.n_out != nullptr) fc.n_out[seq] = n;
    if (fc.opt.remaining != nullptr) fc.opt.remaining[seq] = masked - n;
    if (fc.opt.n_iters != nullptr && n > 0) fc.opt.n_iters[seq] = fc.opt.iter + 1;
  }
}

}  // namespace dblk
