// LM head + softmax confidence for many block rows (M >= 256): MFMA-bound GEMM.
//
// With a batch of sequences the block has M = B*L rows (512 and 4096 in the
// long-context and throughput workloads), each W element is used M times, and
// the LM head becomes a dense bf16 GEMM well above the MFMA/HBM ridge.
//
// Design (gfx950, 32x32x16 bf16 MFMA, fp32 accumulation):
//  * Workgroup tile: 256 vocabulary rows x 256 h rows, 8 waves arranged 4
//    (vocabulary) x 2 (h); each wave owns a 64 x 128 block = 2 x 4 MFMA tiles.
//  * K advances 64 at a time: both operand tiles are staged through
//    double-buffered LDS (row stride padded to 144 bytes, so the 16-byte
//    fragment reads of 16 consecutive rows hit distinct banks).  Two register
//    stages hold the next two stages' global loads, which stay in flight
//    across the LDS-only barriers (a full __syncthreads would drain them).
//    Measured: LDS fragment traffic + MFMA alone reach ~51% of the MFMA peak
//    on this tile shape; the kernel runs at ~40%.
//  * Persistent, XCD-aware: 256 workgroups (one per CU); workgroup i runs on
//    XCD i % 8 and walks that XCD's tiles (vocabulary tiles x, x + 8, ...
//    times the h tiles in use, h tile fastest) with stride 32, so the
//    workgroups resident on an XCD work on neighbouring tiles and share their
//    W and h in its L2.  Only the h tiles holding taken rows are walked: with
//    masked-row compaction their number is known on the device alone, and a
//    grid sized for all M rows left most workgroups exiting at once and every
//    other one paying a start-up chain of dependent loads (row count, row
//    list, operands): c3 530 -> 336 us, c4 1261 -> 906 us per call.
//  * Epilogue on the accumulators: per h row, (max, sum of exp, lowest
//    argmax) over the tile's 256 vocabulary rows -> one 16-byte partial per
//    (h row, vocabulary tile); logits never reach memory.  A second kernel
//    (one wave per h row) merges the partials in a fixed order.
#include <type_traits>

#include "dblk_device.h"
#include "dblk_launch.h"

namespace dblk {

namespace {

constexpr int kGV = 256;          // vocabulary rows per workgroup tile
constexpr int kGM = 256;          // h rows per workgroup tile
constexpr int kGK = 64;           // k per stage
constexpr int kGThreads = 512;    // 8 waves: 4 (vocabulary) x 2 (h)
constexpr int kGRow = kGK + 8;    // LDS row stride (elements) = 144 bytes
constexpr int kPerXcd = 32;       // persistent workgroups per XCD (one per CU)
constexpr int kXcd = 8;           // XCDs; workgroup i is dispatched to XCD i % 8
constexpr int kChunks = kGV * kGK / 8 / kGThreads;   // 16-byte chunks per thread per operand

// Workgroup barrier that orders LDS only: LDS stores before it are visible to
// LDS loads after it, while global loads stay in flight across it (a full
// __syncthreads would also wait for every outstanding global load).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

static_assert(kChunks == 4, "staging layout");

__global__ void __launch_bounds__(kGThreads, 1)
lmhead_gemm_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int M, int d,
                   int V, int nvt, f32x4* __restrict__ partials, Guard gd, RowList rl) {
  // rows taken: all M, or (masked-row compaction) the first *rl.count of rl.rows
  const int Me = rl.rows != nullptr ? *rl.count : M;
  const int nmt = (Me + kGM - 1) / kGM;
  // ---- persistent walk of XCD x's tiles (see the header)
  const int x = blockIdx.x % kXcd;
  const int j = blockIdx.x / kXcd;
  const int nj = gridDim.x / kXcd;
  const int nvx = nvt > x ? (nvt - x + kXcd - 1) / kXcd : 0;
  const int nu = nvx * nmt;

  __shared__ __attribute__((aligned(16))) uint16_t As[2][kGV * kGRow];   // W tile
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kGM * kGRow];   // h tile
  __shared__ SoftmaxPart red[4][kGM];
  for (int u = j; u < nu; u += nj) {
    const int vt = x + kXcd * (u / nmt);
    const int mt = u % nmt;
    const int v0 = vt * kGV;
    const int m0 = mt * kGM;
    if (rl.rows == nullptr && !guard_any(gd, m0, min(M, m0 + kGM) - 1)) continue;   // rows all complete

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int wv = wave & 3;          // 64-row vocabulary group
    const int wh = wave >> 2;         // 128-row h group
    const int l32 = lane & 31;
    const int kg = lane >> 5;

    // staging: chunk c of this thread is row (tid + 512 c) / 8, k chunk (tid % 8)
    const int kc = tid & 7;
    const uint16_t* wrow[kChunks];
    const uint16_t* hrow[kChunks];
  #pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int row = (tid + kGThreads * c) >> 3;
      int vr = v0 + row;
      vr = vr < V ? vr : V - 1;                 // rows past V: loaded, never reported
      wrow[c] = W + (size_t)vr * d + kc * 8;
      const int hr = m0 + row;
      // rows past the taken ones load a valid row (their output columns are
      // never written; every column depends only on its own h row)
      const int src = hr < Me ? (rl.rows != nullptr ? rl.rows[hr] : hr) : 0;
      hrow[c] = h + (size_t)src * d + kc * 8;
    }
    u32x4 ra[2][kChunks], rb[2][kChunks];
    auto gload = [&](int r, int stage) {
  #pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        ra[r][c] = *reinterpret_cast<const u32x4*>(wrow[c] + stage * kGK);
        rb[r][c] = *reinterpret_cast<const u32x4*>(hrow[c] + stage * kGK);
      }
    };
    auto lstore = [&](int r, int buf) {
  #pragma unroll
      for (int c = 0; c < kChunks; ++c) {
        const int row = (tid + kGThreads * c) >> 3;
        *reinterpret_cast<u32x4*>(&As[buf][row * kGRow + kc * 8]) = ra[r][c];
        *reinterpret_cast<u32x4*>(&Bs[buf][row * kGRow + kc * 8]) = rb[r][c];
      }
    };

    f32x16 acc[2][4];
  #pragma unroll
    for (int a = 0; a < 2; ++a)
  #pragma unroll
      for (int b = 0; b < 4; ++b)
  #pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    auto compute = [&](int buf) {
  #pragma unroll
      for (int kk = 0; kk < kGK / 16; ++kk) {
        bf16x8 af[2], bfr[4];
  #pragma unroll
        for (int a = 0; a < 2; ++a)
          af[a] = *reinterpret_cast<const bf16x8*>(&As[buf][(64 * wv + 32 * a + l32) * kGRow + 16 * kk + 8 * kg]);
  #pragma unroll
        for (int b = 0; b < 4; ++b)
          bfr[b] = *reinterpret_cast<const bf16x8*>(&Bs[buf][(128 * wh + 32 * b + l32) * kGRow + 16 * kk + 8 * kg]);
  #pragma unroll
        for (int a = 0; a < 2; ++a)
  #pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] = mfma32x32x16(af[a], bfr[b], acc[a][b]);
      }
    };

    // K loop.  Stage s is multiplied from buffer s % 2 while stage s + 1's loads
    // are in flight; they are then written to the other buffer, which every
    // wave finished reading before the previous barrier.  Loads are issued
    // unconditionally (clamped at the end) to keep the wait counts exact.
    const int nk = d / kGK;
    auto clampk = [&](int k) { return k < nk ? k : nk - 1; };
    gload(0, 0);
    gload(1, clampk(1));
    lstore(0, 0);
    lds_barrier();
    for (int s = 0; s < nk; s += 2) {
      gload(0, clampk(s + 2));
      __builtin_amdgcn_sched_barrier(0);   // keep the prefetch ahead of the multiply
      compute(0);
      lstore(1, 1);
      lds_barrier();
      gload(1, clampk(s + 3));
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < nk) compute(1);          // odd stage count: the last pair has one stage
      lstore(0, 0);
      lds_barrier();
    }

    // ---- epilogue: per h column, (max, sum exp, argmax) over this wave's 64
    // vocabulary rows, then over the 4 vocabulary waves through LDS.  Only
    // the last vocabulary tile has rows past V: every other tile takes the
    // path without the per-row bound (uniform branch).
    auto epilogue = [&](auto check_c) __attribute__((always_inline)) {
      constexpr bool CHECK = decltype(check_c)::value;
  #pragma unroll
      for (int b = 0; b < 4; ++b) {
        float mx = -__builtin_inff();
        int ix = INT32_MAX;
  #pragma unroll
        for (int a = 0; a < 2; ++a)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = v0 + 64 * wv + 32 * a + 8 * (r >> 2) + 4 * kg + (r & 3);
            const float xv = acc[a][b][r];
            if ((!CHECK || row < V) && xv > mx) {
              mx = xv;
              ix = row;
            }
          }
        float sm = 0.f;
        if (!CHECK || ix != INT32_MAX) {
          const float mxs = mx * kLog2e;
  #pragma unroll
          for (int a = 0; a < 2; ++a)
  #pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = v0 + 64 * wv + 32 * a + 8 * (r >> 2) + 4 * kg + (r & 3);
              if (!CHECK || row < V) sm += fast_exp2(acc[a][b][r] * kLog2e - mxs);
            }
        }
        SoftmaxPart p{mx, sm, ix};
        p = combine(p, shfl_xor(p, 32));
        if (kg == 0) red[wv][128 * wh + 32 * b + l32] = p;
      }
    };
    if (v0 + kGV <= V)
      epilogue(std::false_type{});
    else
      epilogue(std::true_type{});
    __syncthreads();
    if (tid < kGM) {
      SoftmaxPart q = red[0][tid];
  #pragma unroll
      for (int w = 1; w < 4; ++w) q = combine(q, red[w][tid]);
      const int hr = m0 + tid;   // partials are indexed by taken-row number
      if (hr < Me) partials[(size_t)hr * nvt + vt] = f32x4{q.m, q.s, __int_as_float(q.i), 0.f};
    }
    __syncthreads();   // red and the tile buffers are reused by the next tile
  }
}

// One wave per h row: merge its nvt partials in a fixed order.
__global__ void __launch_bounds__(256)
lmhead_gemm_merge(const f32x4* __restrict__ partials, int M, int nvt, float* __restrict__ conf,
                  int32_t* __restrict__ amax, Guard gd, RowList rl) {
  const int row = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int Me = rl.rows != nullptr ? *rl.count : M;
  if (row >= Me) return;
  // rows of complete sequences: their tile was skipped, keep conf / argmax
  if (rl.rows == nullptr && !guard_any(gd, row, row)) return;
  const int out_row = rl.rows != nullptr ? rl.rows[row] : row;
  const f32x4* p = partials + (size_t)row * nvt;
  SoftmaxPart q{-__builtin_inff(), 0.f, INT32_MAX};
  for (int t0 = 0; t0 < nvt; t0 += 4 * kWave) {
    f32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u * kWave + lane;
      v[u] = t < nvt ? p[t] : f32x4{-__builtin_inff(), 0.f, __int_as_float(INT32_MAX), 0.f};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) q = combine(q, SoftmaxPart{v[u][0], v[u][1], __float_as_int(v[u][2])});
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) q = combine(q, shfl_xor(q, off));
  if (lane == 0) {
    conf[out_row] = 1.0f / q.s;
    amax[out_row] = q.i;
  }
}

// Masked-row compaction (one workgroup): rows[0..count) = the positions r < M
// with mask[r] != 0, in increasing order.  Thread t scans a contiguous span;
// an exclusive scan of the span counts gives each thread its first slot.
constexpr int kCompactThreads = 1024;
__global__ void __launch_bounds__(kCompactThreads)
compact_masked_rows(const uint8_t* __restrict__ mask, int M, int32_t* __restrict__ rows,
                    int32_t* __restrict__ count) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int per = (M + kCompactThreads - 1) / kCompactThreads;
  const int begin = tid * per;
  const int end = begin + per < M ? begin + per : M;
  int n = 0;
  for (int r = begin; r < end; ++r) n += mask[r] != 0 ? 1 : 0;
  // inclusive scan within the wave, then over the wave totals
  int x = n;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  __shared__ int s_wave[kCompactThreads / kWave];
  if (lane == kWave - 1) s_wave[wave] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kCompactThreads / kWave; ++w) {
    before += w < wave ? s_wave[w] : 0;
    total += s_wave[w];
  }
  int slot = before + x - n;
  for (int r = begin; r < end; ++r)
    if (mask[r] != 0) rows[slot++] = r;
  if (tid == 0) count[0] = total;
}

}  // namespace

GemmPlan gemm_plan(int M, int d, int V) {
  (void)d;
  GemmPlan g;
  g.nvt = (V + kGV - 1) / kGV;
  g.nmt = (M + kGM - 1) / kGM;
  g.grid = kXcd * kPerXcd;   // persistent: one workgroup per CU
  g.partials_bytes = (size_t)M * g.nvt * sizeof(f32x4);
  g.rows_offset = (g.partials_bytes + 255) / 256 * 256;
  g.rows_bytes = ((size_t)(M + 1) * sizeof(int32_t) + 255) / 256 * 256;   // rows[M], count
  return g;
}

hipError_t launch_lmhead_gemm(const void* h, const void* W, int M, int d, int V, float* conf,
                              int32_t* amax, void* ws, const GemmPlan& g, const Guard& gd,
                              const uint8_t* masked_only, hipStream_t stream) {
  f32x4* partials = static_cast<f32x4*>(ws);
  RowList rl;
  hipError_t e = hipSuccess;
  if (masked_only != nullptr) {
    int32_t* rows = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + g.rows_offset);
    rl.rows = rows;
    rl.count = rows + M;
    e = launch_kernel(compact_masked_rows, dim3(1), dim3(kCompactThreads), 0, stream, masked_only,
                      M, rows, rows + M);
    if (e != hipSuccess) return e;
  }
  e = launch_kernel(lmhead_gemm_kernel, dim3(g.grid), dim3(kGThreads), 0, stream,
                    static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W), M, d, V,
                    g.nvt, partials, gd, rl);
  if (e != hipSuccess) return e;
  return launch_kernel(lmhead_gemm_merge, dim3((M + 3) / 4), dim3(256), 0, stream,
                       static_cast<const f32x4*>(partials), M, g.nvt, conf, amax, gd, rl);
}

}  // namespace dblk
