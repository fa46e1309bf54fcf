// Host-side launch helpers and the internal launcher entry points of each
// kernel translation unit.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace dblk {

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
hipError_t launch_threshold_commit(const float* conf, const int32_t* amax, int32_t* tokens,
                                   uint8_t* mask, int B, int L, float tau, int32_t* n_out,
                                   hipStream_t stream);

// ---- lmhead_gemm.hip (M >= 256)
struct GemmPlan {
  int nvt, nmt;      // 256-row vocabulary / h tiles
  int SM, SV;        // h / vocabulary tiles per XCD super-tile
  int n_sv, NS;      // vocabulary super-tile columns, super-tiles
  int grid;          // workgroups (idle ones exit at once)
  size_t partials_bytes;
};
GemmPlan gemm_plan(int M, int d, int V);
hipError_t launch_lmhead_gemm(const void* h, const void* W, int M, int d, int V, float* conf,
                              int32_t* amax, void* ws, const GemmPlan& g, hipStream_t stream);

// ---- lmhead.hip
struct LmheadPlan {
  bool gemm;         // M >= 256: MFMA-bound GEMM path (lmhead_gemm.hip)
  GemmPlan g;
  bool rows_outer;   // K split over 8 waves, rows-outer walk (d <= 2048)
  int ntile;         // 16-row vocabulary tiles
  int nt;            // K-outer kernel: tiles per wave
  int tiles_per_wg;  // vocabulary tiles per workgroup
  int grid;          // workgroups per M-chunk
  int mchunks;   // 64-row chunks of M
  size_t counters_bytes;
  size_t partials_bytes;
};
LmheadPlan lmhead_plan(int M, int d, int V);
hipError_t launch_lmhead(const void* h, const void* W, int M, int d, int V, float* conf,
                         int32_t* amax, void* ws, const LmheadPlan& plan, hipStream_t stream);

// ---- attend.hip
struct AttendPlan {
  int T_cap;     // P_cap + L + S
  int kps;       // keys per split (multiple of the key tile)
  int nsplit;    // splits per (b, h)
  size_t partials_bytes;
};
AttendPlan attend_plan(int B, int H, int L, int D, int P_cap, int S);
hipError_t launch_attend(const void* q, const void* kp, const void* vp, const void* kb,
                         const void* vb, const void* ks, const void* vs,
                         const int32_t* prefix_len, int B, int H, int L, int D, int P_cap,
                         int S, float scale, void* out, void* ws, const AttendPlan& plan,
                         hipStream_t stream);

}  // namespace dblk
