// The threshold decoder step (as threshold_commit_kernel in commit.hip) for
// the whole sequences held by one 64-row chunk, run by a single wave: lane r
// holds row m0 + r with its confidence and argmax; a sequence is a group of
// L consecutive lanes (L a power of two dividing 64), i.e. L consecutive bits
// of a wave ballot, so counts and first positions are popcounts and
// trailing-zero counts of masked ballots, and only the fallback's maximum
// needs a (segmented, xor offsets below L) butterfly.  All 64 lanes must be
// active.  Decisions, tie-breaks, NaN handling, EOS fill and the block-loop
// records match the standalone kernel exactly (same fp32 values and
// comparisons).
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
  const int sbase = lane - pos;                          // first lane of this sequence
  const uint64_t smask = (L == kWave) ? ~0ull : (((1ull << L) - 1ull) << sbase);
  const bool eos = fc.opt.eos_id >= 0;
  const bool m = valid && in.m != 0;
  const int32_t t = in.t;

  // Counts are popcounts of the sequence's bits of a wave ballot.
  const bool hit = m && c >= fc.tau;
  const int hits = __popcll(__ballot(hit) & smask);
  const int masked = __popcll(__ballot(m) & smask);
  // Fallback position: the most confident masked position (NaN ranks lowest),
  // lowest position on a tie.  Only computed when some sequence needs it.
  int bi = INT32_MAX;
  if (__ballot(masked > 0 && hits == 0) != 0ull) {
    const float key = m ? ((c == c) ? c : -__builtin_inff()) : -__builtin_inff();
    float best = key;
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
      if (off < L) best = fmaxf(best, __shfl_xor(best, off, kWave));
    const uint64_t at = __ballot(m && key == best) & smask;
    if (at != 0ull) bi = __builtin_ctzll(at) - sbase;
  }
  const bool step = hits > 0 ? hit : (m && pos == bi);
  int n = hits > 0 ? hits : (masked > 0 ? 1 : 0);
  bool cm = step;
  int32_t v = a;
  if (eos) {
    // first position of the sequence holding a committed EOS after this step
    const uint64_t eb = __ballot(valid && (!m || step) && (step ? a : t) == fc.opt.eos_id) & smask;
    const int first = eb != 0ull ? __builtin_ctzll(eb) - sbase : INT32_MAX;
    const bool fill = m && !step && pos > first;
    n += __popcll(__ballot(fill) & smask);
    if (fill) {
      cm = true;
      v = fc.opt.eos_id;
    }
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
