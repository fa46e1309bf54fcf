// LM head + full-vocabulary softmax confidence + argmax, logits never stored.
//
// For the block's hidden states h [M][d] and the LM-head weight W [V][d]
// (row t = token t), every row m gets conf[m] = max_t softmax(h_m W^T)_t and
// argmax[m] = lowest t attaining the largest logit.  The threshold decoder of
// the dInfer README (usage section) consumes exactly these two numbers.
//
// Design (gfx950, wave64, 16x16x32 bf16 MFMA):
//  * The work is a skinny GEMM: M = B*L is 64 for one block, V is ~10^5, so
//    each W element is used M times and the kernel is bound by streaming W
//    from HBM (64 flop per byte at M = 64, far below the MFMA/HBM ridge).
//  * Workgroups are persistent over contiguous vocabulary ranges: workgroup g
//    owns 4 waves x NT tiles of 16 vocabulary rows.  The grid is sized so all
//    workgroups are resident at once (<= 3 per CU), so there is no tail wave.
//  * W goes straight from HBM into the MFMA A operand: lane l loads 16 bytes
//    of row (l % 16) at k-group (l / 16); no LDS round trip.  Two register
//    stages of 32 k each keep the next stage's loads in flight while the
//    current one is multiplied.
//  * h (64 rows per pass) is staged through LDS in MFMA fragment order, one
//    32-k stage at a time and double-buffered, so every wave reads its B
//    operands with conflict-free 16-byte LDS reads and h leaves L2 once per
//    workgroup instead of once per wave.
//  * Epilogue on the accumulators: per row, lane-local max/argmax and sum of
//    exp over the lane's logits, then xor-shuffles across the 4 lane groups,
//    then the 4 waves through LDS, giving one (max, sum, argmax) partial per
//    (row, workgroup) in the workspace.
//  * The last workgroup to arrive (device-scope counter) merges the partials
//    of every workgroup in a fixed order and writes conf = 1 / sum and argmax,
//    then re-arms the counter.  One launch per call; no logits in HBM.
#include "dblk_device.h"
#include "dblk_launch.h"

namespace dblk {

namespace {

constexpr int kLmWaves = 4;
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kMChunk = 64;              // rows of h per pass
constexpr int kMT = kMChunk / 16;        // 16-row MFMA tiles of h
constexpr int kTargetGrid = 768;         // resident workgroups aimed for (3 per CU)
constexpr int kMaxNT = 5;               // <= 168 VGPRs: 3 workgroups per CU

template <int NT>
__global__ void __launch_bounds__(kLmThreads, 3)
lmhead_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int M, int d,
              int V, float* __restrict__ conf, int32_t* __restrict__ amax,
              uint32_t* __restrict__ counters, f32x4* __restrict__ partials, int G) {
  const int g = blockIdx.x;
  const int mc = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int m0 = mc * kMChunk;
  static_assert(kMT == kLmWaves, "wave w stages h tile w");

  __shared__ u32x4 hs[2][kMT][kWave];
  __shared__ SoftmaxPart red[kLmWaves][kMChunk];
  __shared__ int s_last;

  // ---- this wave's vocabulary tiles; rows past V are clamped for loading
  // and excluded in the epilogue
  const int tile0 = (g * kLmWaves + wave) * NT;
  const uint16_t* wp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    int row = (tile0 + t) * 16 + l16;
    row = row < V ? row : V - 1;
    wp[t] = W + (size_t)row * (size_t)d + grp * 8;
  }

  // ---- h staging: thread loads fragment slot (ks = j, mt = wave, lane)
  const int hrow = m0 + wave * 16 + l16;
  const bool hvalid = hrow < M;
  const uint16_t* hp = h + (size_t)(hvalid ? hrow : 0) * (size_t)d + grp * 8;

  f32x4 acc[NT][kMT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) acc[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 wa[NT], wb[NT];
  u32x4 hr;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // A 32-wide k stage: one 16-byte load per tile for W, one for h.
  auto load_w = [&](u32x4 (&dst)[NT], int stage) {
#pragma unroll
    for (int t = 0; t < NT; ++t) dst[t] = *reinterpret_cast<const u32x4*>(wp[t] + stage * 32);
  };
  auto load_h = [&](int stage) {
    hr = hvalid ? *reinterpret_cast<const u32x4*>(hp + stage * 32) : zero4;
  };
  auto store_h = [&](int buf) { hs[buf][wave][lane] = hr; };
  auto compute = [&](const u32x4 (&src)[NT], int buf) {
    bf16x8 hf[kMT];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) hf[mt] = as_bf16x8(hs[buf][mt][lane]);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const bf16x8 a = as_bf16x8(src[t]);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) acc[t][mt] = mfma16x16x32(a, hf[mt], acc[t][mt]);
    }
  };

  // d is a multiple of 64, so the number of 32-wide stages is even and the
  // loop below runs two stages per trip with no early exit.  Loads are issued
  // unconditionally (the stage index is clamped at the end), which keeps the
  // wait counts the compiler inserts exact: waiting for stage s never waits
  // for the prefetch of stage s + 1.
  const int nk = d / 32;
  load_h(0);
  load_w(wa, 0);
  store_h(0);
  __syncthreads();
  load_h(1);
  load_w(wb, 1);
  for (int s = 0; s < nk; s += 2) {
    const int s2 = s + 2 < nk ? s + 2 : nk - 1;
    const int s3 = s + 3 < nk ? s + 3 : nk - 1;
    compute(wa, 0);                  // stage s     (in flight: h, W of s + 1)
    store_h(1);
    __syncthreads();
    load_h(s2);
    load_w(wa, s2);
    compute(wb, 1);                  // stage s + 1 (in flight: h, W of s + 2)
    store_h(0);
    __syncthreads();
    load_h(s3);
    load_w(wb, s3);
  }

  // ---- epilogue: (max, sum exp, argmax) per row over this wave's rows
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    float mx = -__builtin_inff();
    int ix = INT32_MAX;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = (tile0 + t) * 16 + grp * 4 + r;
        const float x = acc[t][mt][r];
        if (row < V && x > mx) {
          mx = x;
          ix = row;
        }
      }
    float sm = 0.f;
    if (ix != INT32_MAX) {
      const float mxs = mx * kLog2e;
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = (tile0 + t) * 16 + grp * 4 + r;
          if (row < V) sm += fast_exp2(acc[t][mt][r] * kLog2e - mxs);
        }
    }
    SoftmaxPart p{mx, sm, ix};
    p = combine(p, shfl_xor(p, 16));
    p = combine(p, shfl_xor(p, 32));
    if (grp == 0) red[wave][mt * 16 + l16] = p;
  }
  __syncthreads();
  if (tid < kMChunk) {
    SoftmaxPart q = red[0][tid];
#pragma unroll
    for (int w = 1; w < kLmWaves; ++w) q = combine(q, red[w][tid]);
    partials[((size_t)mc * G + g) * kMChunk + tid] = f32x4{q.m, q.s, __int_as_float(q.i), 0.f};
    __threadfence();
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(&counters[mc], 1u);
    s_last = (prev == (uint32_t)(G - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- last workgroup of this M chunk: merge the G partials of each row
  const int r = tid >> 2;       // row within the chunk (64 rows x 4 threads)
  const int part = tid & 3;
  SoftmaxPart q{-__builtin_inff(), 0.f, INT32_MAX};
  const f32x4* pp = partials + (size_t)mc * G * kMChunk + r;
  for (int s = part; s < G; s += 4) {
    const f32x4 v = __builtin_nontemporal_load(pp + (size_t)s * kMChunk);
    q = combine(q, SoftmaxPart{v[0], v[1], __float_as_int(v[2])});
  }
  q = combine(q, shfl_xor(q, 1));
  q = combine(q, shfl_xor(q, 2));
  if (part == 0 && m0 + r < M) {
    conf[m0 + r] = 1.0f / q.s;
    amax[m0 + r] = q.i;
  }
  if (tid == 0) counters[mc] = 0u;
}

template <int NT>
hipError_t launch_nt(const void* h, const void* W, int M, int d, int V, float* conf,
                     int32_t* amax, uint32_t* counters, f32x4* partials,
                     const LmheadPlan& p, hipStream_t stream) {
  return launch_kernel(lmhead_kernel<NT>, dim3(p.grid, p.mchunks), dim3(kLmThreads), 0, stream,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W), M, d,
                       V, conf, amax, counters, partials, p.grid);
}

}  // namespace

LmheadPlan lmhead_plan(int M, int d, int V) {
  (void)d;
  LmheadPlan p;
  p.ntile = (V + 15) / 16;
  int nt = (p.ntile + kLmWaves * kTargetGrid - 1) / (kLmWaves * kTargetGrid);
  p.nt = nt < 1 ? 1 : (nt > kMaxNT ? kMaxNT : nt);
  p.grid = (p.ntile + kLmWaves * p.nt - 1) / (kLmWaves * p.nt);
  p.mchunks = (M + kMChunk - 1) / kMChunk;
  p.counters_bytes = (((size_t)p.mchunks * sizeof(uint32_t)) + 255) / 256 * 256;
  p.partials_bytes = (size_t)p.mchunks * p.grid * kMChunk * sizeof(f32x4);
  return p;
}

hipError_t launch_lmhead(const void* h, const void* W, int M, int d, int V, float* conf,
                         int32_t* amax, void* ws, const LmheadPlan& p, hipStream_t stream) {
  uint32_t* counters = static_cast<uint32_t*>(ws);
  f32x4* partials = reinterpret_cast<f32x4*>(static_cast<char*>(ws) + p.counters_bytes);
  switch (p.nt) {
    case 1: return launch_nt<1>(h, W, M, d, V, conf, amax, counters, partials, p, stream);
    case 2: return launch_nt<2>(h, W, M, d, V, conf, amax, counters, partials, p, stream);
    case 3: return launch_nt<3>(h, W, M, d, V, conf, amax, counters, partials, p, stream);
    case 4: return launch_nt<4>(h, W, M, d, V, conf, amax, counters, partials, p, stream);
    default: return launch_nt<5>(h, W, M, d, V, conf, amax, counters, partials, p, stream);
  }
}

}  // namespace dblk
