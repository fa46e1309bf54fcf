// Host-side launch helpers and the internal launcher entry points of each
// kernel translation unit.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace dblk {

// Per-sequence guard of the device-side block loop.  `active[b]` holds the
// number of still-masked positions of sequence b after the previous commit
// step; a kernel of the loop skips the work of sequences whose count is 0.
// active == nullptr: no guard (every plain entry point).  Rows of the block
// matrix are sequence-major, rows_per_seq = L rows per sequence.
struct Guard {
  const int32_t* active;
  int rows_per_seq;
};

// True when any sequence owning a row in [r0, r1] is still active.  The same
// answer for every thread and workgroup that asks about the same rows, so a
// launch that skips does so uniformly.
__device__ __forceinline__ bool guard_any(const Guard& g, int r0, int r1) {
  if (g.active == nullptr) return true;
  for (int b = r0 / g.rows_per_seq; b <= r1 / g.rows_per_seq; ++b)
    if (g.active[b] > 0) return true;
  return false;
}

// Launch `kernel` and return the status of this launch itself (not a stale
// error left by earlier runtime calls).  Arguments are converted to the
// kernel's parameter types before their addresses are taken.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                         hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count mismatch");
  std::tuple<KArgs...> typed(static_cast<KArgs>(args)...);
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
  std::apply(
      [&](auto&... e) {
        int k = 0;
        ((ptrs[k++] = static_cast<void*>(&e)), ...);
      },
      typed);
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, shmem, stream);
}

// ---- commit.hip
// Optional parts of a commit step.  Zero-initialised = the plain decoder step.
struct CommitOpts {
  int32_t eos_id = -1;            // >= 0: masked positions after the first EOS are filled
  uint8_t* finished = nullptr;    // [B]: 1 when the row holds a committed EOS
  int32_t iter = 0;               // iteration index recorded below
  int32_t* commit_iter = nullptr; // [B][L]: iteration at which each position was committed
  int32_t* n_iters = nullptr;     // [B]: iter + 1 whenever this step commits something
  int32_t* remaining = nullptr;   // [B]: masked positions left after this step
};
hipError_t launch_threshold_commit(const float* conf, const int32_t* amax, int32_t* tokens,
                                   uint8_t* mask, int B, int L, float tau, int32_t* n_out,
                                   const CommitOpts& opt, hipStream_t stream);

// A decoder step fused into the LM head's final merge (tokens == nullptr:
// none).  Rows are sequence-major with L rows per sequence.
struct FusedCommit {
  int32_t* tokens = nullptr;
  uint8_t* mask = nullptr;
  int L = 1;
  float tau = 0.f;
  int32_t* n_out = nullptr;
  CommitOpts opt;
};
// Start of a block loop: remaining[b] = masked count, commit_iter = -1, n_iters = 0.
hipError_t launch_block_loop_init(const uint8_t* mask, int B, int L, int32_t* remaining,
                                  int32_t* commit_iter, int32_t* n_iters, hipStream_t stream);
// Block-loop progress: out[0] = number of b with remaining[b] > 0.
hipError_t launch_block_loop_count(const int32_t* remaining, int B, int32_t* out,
                                   hipStream_t stream);
// Dual-cache advance: append the block's K/V rows at each sequence's prefix end.
hipError_t launch_cache_append(void* kp, void* vp, const void* kb, const void* vb,
                               int32_t* prefix_len, int B, int H, int L, int D, int P_cap,
                               int32_t* appended, hipStream_t stream);

// ---- lmhead_gemm.hip (M >= 256)
struct GemmPlan {
  int nvt, nmt;      // 256-row vocabulary / h tiles
  int grid;          // persistent workgroups (one per CU)
  size_t partials_bytes;
  size_t rows_offset, rows_bytes;   // masked-row list (rows[M], count) in the workspace
};
// Rows the GEMM takes: all (rows == nullptr) or rows[0 .. *count).
struct RowList {
  const int32_t* rows = nullptr;
  const int32_t* count = nullptr;
};
GemmPlan gemm_plan(int M, int d, int V);
// masked_only != nullptr: only rows r with masked_only[r] != 0 go through the
// LM head (conf / argmax of the other rows are not written).
hipError_t launch_lmhead_gemm(const void* h, const void* W, int M, int d, int V, float* conf,
                              int32_t* amax, void* ws, const GemmPlan& g, const Guard& gd,
                              const uint8_t* masked_only, hipStream_t stream);

// ---- lmhead.hip
struct LmheadPlan {
  bool gemm;         // M >= 256: MFMA-bound GEMM path (lmhead_gemm.hip)
  GemmPlan g;
  bool rows_outer;   // K split over 8 waves, rows-outer walk (d <= 2048)
  int ntile;         // 16-row vocabulary tiles
  int nt;            // K-outer kernel: passes per workgroup
  int tiles_per_wg;  // vocabulary tiles per workgroup (rows-outer: about, see the kernel)
  int grid;          // workgroups per M-chunk
  int mchunks;   // 64-row chunks of M
  size_t counters_bytes;
  size_t partials_bytes;
};
LmheadPlan lmhead_plan(int M, int d, int V);
// True when the plan's final merge can also run the decoder step: the row
// paths finish 64 rows in one workgroup, which then holds whole sequences
// when L is a power of two dividing 64.
bool lmhead_can_fuse_commit(const LmheadPlan& plan, int L);
// fc.tokens != nullptr requires lmhead_can_fuse_commit(plan, fc.L).
// masked_only != nullptr: only rows masked there need conf / argmax.  The
// GEMM (see launch_lmhead_gemm) and the rows-outer kernel then compute only
// those rows and leave the others' conf / argmax unchanged; the K-outer
// kernel computes every row.
hipError_t launch_lmhead(const void* h, const void* W, int M, int d, int V, float* conf,
                         int32_t* amax, void* ws, const LmheadPlan& plan, const Guard& gd,
                         const FusedCommit& fc, const uint8_t* masked_only, hipStream_t stream);

// ---- attend.hip
// One cache segment as the kernel sees it: K and V share element strides
// (the head dimension is contiguous); rows [0, rows_b) of sequence b are
// attended, rows_b = clamp(len_b[b], 0, len) or len when len_b is null.
struct KVSeg {
  const uint16_t* k;
  const uint16_t* v;
  int64_t sb, sh, st;       // element strides: sequence, head, row
  int32_t len;              // rows per (b, h) available
  const int32_t* len_b;     // [B] rows used per sequence, or nullptr
};
// Everything dblk_attend / dblk_attend_segments describe, validated.
struct AttendArgs {
  int B, H, L, D;
  const uint16_t* q;
  int64_t q_sb, q_sl, q_sh;   // element strides of q [B][L][H][D]
  KVSeg seg[3];               // prefix, block, suffix
  float scale;                // > 0
  uint16_t* out;
  int64_t o_sb, o_sl, o_sh;
};
struct AttendPlan {
  int T_cap;     // summed segment capacities
  int kps;       // keys per split (multiple of the key tile)
  int nsplit;    // splits per (b, h)
  // workspace (nsplit > 1 only): fp16 partial outputs, then one
  // {max, sum, scale, 0} record per row
  size_t ml_offset, ws_bytes;
};
AttendPlan attend_plan(int B, int H, int L, int D, int T_cap);
hipError_t launch_attend(const AttendArgs& a, void* ws, const AttendPlan& plan, const Guard& gd,
                         hipStream_t stream);
// The dense layout of dblk_attend as segment arguments.
AttendArgs dense_attend_args(const void* q, const void* kp, const void* vp, const void* kb,
                             const void* vb, const void* ks, const void* vs,
                             const int32_t* prefix_len, int B, int H, int L, int D, int P_cap,
                             int S, int S_cap, float scale, void* out);

}  // namespace dblk
