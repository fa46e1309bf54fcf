// HBM read-ceiling probe (a measurement aid; contract in include/dblock_probe.h).
//
// 256-thread workgroups read 32 KiB per trip: 8 loads of 16 bytes per thread,
// load u of wave w covering bytes [1 KiB (8 w + u), +1 KiB) of the trip, so
// every wave instruction reads eight whole 128-byte lines.  All 8 loads of a
// trip are issued before any is used.
#include "dblock.h"
#include "dblock_probe.h"
#include "dblk_device.h"
#include "dblk_launch.h"

namespace dblk {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;
constexpr size_t kProbeTrip = (size_t)kProbeThreads * kProbeUnroll * 16;   // bytes per trip

template <bool NT>
__global__ void __launch_bounds__(kProbeThreads)
read_probe_kernel(const u32x4* __restrict__ p, size_t ntrips, uint32_t* __restrict__ sink) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t trip = blockIdx.x; trip < ntrips; trip += gridDim.x) {
    const u32x4* base = p + trip * (kProbeTrip / 16) + (size_t)wave * kProbeUnroll * kWave + lane;
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u)
      v[u] = NT ? __builtin_nontemporal_load(base + u * kWave) : base[u * kWave];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u];
  }
  sink[(size_t)blockIdx.x * kProbeThreads + tid] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace
}  // namespace dblk

extern "C" int32_t dblk_probe_read(const void* buf, size_t bytes, int32_t nontemporal,
                                   int32_t grid, uint32_t* sink, void* stream) {
  using namespace dblk;
  if (bytes == 0 || bytes % kProbeTrip != 0 || grid < 1 || grid > 65535) return DBLK_ERR_SHAPE;
  if (!buf || !sink) return DBLK_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) || (reinterpret_cast<uintptr_t>(sink) & 3u))
    return DBLK_ERR_ALIGN;
  const size_t ntrips = bytes / kProbeTrip;
  const u32x4* p = static_cast<const u32x4*>(buf);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e =
      nontemporal ? launch_kernel(read_probe_kernel<true>, dim3(grid), dim3(kProbeThreads), 0, s, p,
                                  ntrips, sink)
                  : launch_kernel(read_probe_kernel<false>, dim3(grid), dim3(kProbeThreads), 0, s,
                                  p, ntrips, sink);
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}
