// LM head + softmax confidence for many block rows (M >= 256): MFMA-bound GEMM.
//
// With a batch of sequences the block has M = B*L rows (512 and 4096 in the
// long-context and throughput workloads), each W element is used M times, and
// the LM head becomes a dense bf16 GEMM well above the MFMA/HBM ridge.
//
// Design (gfx950, 32x32x16 bf16 MFMA, fp32 accumulation):
//  * Workgroup tile: 256 vocabulary rows x 256 h rows, 8 waves in two groups
//    of four (one wave of each group per SIMD); wave (g, i) owns vocabulary
//    rows [64 i, 64 i + 64) x h rows [128 g, 128 g + 128) = 2 x 4 MFMA tiles.
//  * Operands reach LDS by DMA (buffer loads with the LDS bit), 64 k per
//    stage: three W stages and two h stages resident, 160 KiB.  Rows are 128
//    bytes with the 16-byte chunks XOR-swizzled, so each DMA instruction
//    fills 8 whole rows from 8 whole 128-byte lines and the fragment reads of
//    32 consecutive rows are free of bank conflicts.
//  * Ping-pong: the two groups run one barrier apart, so on each SIMD one
//    wave issues its stage's 32 MFMAs while the other reads its next stage's
//    fragments from LDS; group 0 issues the h DMA one stage ahead, group 1 the
//    W DMA two stages ahead (schedule in the kernel).  Barriers are s_barrier
//    with only an lgkmcnt wait in front, so DMA stays in flight across them.
//  * In the last h tile of a batch only the 32-row h tiles holding taken rows
//    are read and multiplied.
//  * Persistent, XCD-aware: 256 workgroups (one per CU); workgroup i runs on
//    XCD i % 8.  The tiles (h tile fastest) are cut into 8 contiguous ranges
//    of equal size, one per XCD, walked with stride 32 by its workgroups, so
//    no workgroup has more than one tile more than another and the tiles in
//    flight on an XCD share W and h in its L2.  Only the h tiles holding
//    taken rows are walked: with masked-row compaction their number is known
//    on the device alone.
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
constexpr int kGThreads = 512;    // 8 waves: two groups of 4, one wave of each group per SIMD
constexpr int kSlot = 256 * kGK * 2;   // bytes of one operand stage: 256 rows x 64 k bf16 = 32 KiB
constexpr int kWSlots = 3;        // W stages resident (two in flight while one is read)
constexpr int kHSlots = 2;        // h stages resident
constexpr int kPerXcd = 32;       // persistent workgroups per XCD (one per CU)
constexpr int kXcd = 8;           // XCDs; workgroup i is dispatched to XCD i % 8
constexpr int kRsrcFlags = 0x00020000;   // buffer descriptor word 3: raw dword access
// W's DMA takes the nontemporal (streaming) policy, kDmaStream, when a W tile
// is read by one h tile only (at most 256 rows taken).  Measured on the
// 256-row, 4096-wide, 126464-token head: 249 against 254-259 us per call.
// With several h tiles the W tile is re-read through L2 and the hint costs
// (4096 rows: 690 against 646 us), so it is used only for the single-tile
// walk.

// LDS layout of a stage: tile row r occupies bytes [128 r, 128 r + 128); its
// 16-byte k chunk c sits in position c ^ swz(r).  Fragment reads (rows l..l+31
// of one chunk per half wave) then spread over all banks, and an LDS DMA
// instruction (lane i -> byte 16 i of a 1 KiB block) still fills 8 whole rows,
// each from one 128-byte line of the source.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void wait_dma_all() { wait_vm<0>(); }
__device__ __forceinline__ void wait_dma_but8() { wait_vm<8>(); }

// One wave's share of a stage: 8 DMA instructions, 64 tile rows x 128 bytes,
// into the 8 consecutive 1 KiB blocks at dst.  off[j] = byte offset of the
// lane's source chunk for block j; soff = byte offset of the stage's k range.
// AUX is the load's cache policy (0, or kDmaStream).
template <int AUX = 0>
__device__ __forceinline__ void dma_stage(__amdgpu_buffer_rsrc_t rs, const uint32_t (&off)[8], uint8_t* dst,
                                          uint32_t soff) {
#pragma unroll
  for (int j = 0; j < 8; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + j * 1024), 16, off[j], soff, 0, AUX);
}

struct Frags {
  bf16x8 a[4][2];   // W: 4 k16 steps x 2 row tiles of 32
  bf16x8 b[4][4];   // h: 4 k16 steps x 4 row tiles of 32
};

// Fragments of one stage for a wave owning 64 W rows at ws and 128 h rows at
// hs; roff[kk] = lane offset of k16 step kk.  PART: only the first nb 32-row
// h tiles hold taken rows (the last h tile of the batch), the rest are skipped.
template <bool PART>
__device__ __forceinline__ void read_frags(const uint8_t* ws, const uint8_t* hs, const uint32_t (&roff)[4],
                                           Frags& F, int nb) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
      if (!PART || nb > 0) F.a[kk][a] = *reinterpret_cast<const bf16x8*>(ws + a * 32 * 128 + roff[kk]);
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (!PART || b < nb) F.b[kk][b] = *reinterpret_cast<const bf16x8*>(hs + b * 32 * 128 + roff[kk]);
  }
}

template <bool PART>
__device__ __forceinline__ void multiply(const Frags& F, f32x16 (&acc)[2][4], int nb) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (!PART || b < nb) acc[a][b] = mfma32x32x16(F.a[kk][a], F.b[kk][b], acc[a][b]);
}

// The K loop of one wave group (see the schedule in the kernel).  Group 0
// loads h one stage ahead; group 1 loads W two stages ahead.
template <bool PART>
__device__ __forceinline__ void k_loop_g0(const uint8_t* wsrc, const uint8_t* hsrc, uint8_t* mydma,
                                          __amdgpu_buffer_rsrc_t hrs, const uint32_t (&off)[8],
                                          const uint32_t (&roff)[4], f32x16 (&acc)[2][4], int nk, int nb) {
  dma_stage(hrs, off, mydma + 3 * kSlot, 0);
  wait_dma_all();
  stage_barrier();
  for (int s = 0; s < nk; ++s) {
    if (s + 1 < nk) dma_stage(hrs, off, mydma + (3 + ((s + 1) & 1)) * kSlot, (uint32_t)(s + 1) * 128u);
    Frags F;
    read_frags<PART>(wsrc + (s % 3) * kSlot, hsrc + (s & 1) * kSlot, roff, F, nb);
    stage_barrier();
    multiply<PART>(F, acc, nb);
    wait_dma_all();
    stage_barrier();
  }
}

template <bool PART, int WAUX>
__device__ __forceinline__ void k_loop_g1(const uint8_t* wsrc, const uint8_t* hsrc, uint8_t* mydma,
                                          __amdgpu_buffer_rsrc_t wrs, const uint32_t (&off)[8],
                                          const uint32_t (&roff)[4], f32x16 (&acc)[2][4], int nk, int nb) {
  dma_stage<WAUX>(wrs, off, mydma, 0);
  if (nk > 1) {
    dma_stage<WAUX>(wrs, off, mydma + kSlot, 128u);
    wait_dma_but8();
  } else {
    wait_dma_all();
  }
  stage_barrier();
  stage_barrier();
  for (int s = 0; s < nk; ++s) {
    if (s + 2 < nk) dma_stage<WAUX>(wrs, off, mydma + ((s + 2) % 3) * kSlot, (uint32_t)(s + 2) * 128u);
    Frags F;
    read_frags<PART>(wsrc + (s % 3) * kSlot, hsrc + (s & 1) * kSlot, roff, F, nb);
    if (s + 2 < nk)
      wait_dma_but8();
    else
      wait_dma_all();
    stage_barrier();
    multiply<PART>(F, acc, nb);
    if (s + 1 < nk) stage_barrier();
  }
}

__global__ void __launch_bounds__(kGThreads, 1)
lmhead_gemm_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int M, int d,
                   int V, int nvt, f32x4* __restrict__ partials, Guard gd, RowList rl) {
  // rows taken: all M, or (masked-row compaction) the first *rl.count of rl.rows
  const int Me = rl.rows != nullptr ? *rl.count : M;
  const int nmt = (Me + kGM - 1) / kGM;
  // ---- persistent walk of XCD x's tiles (see the header)
  const int x = blockIdx.x % kXcd;
  const int jw = blockIdx.x / kXcd;
  const int nj = gridDim.x / kXcd;
  const int total = nvt * nmt;
  const int per_x = (total + gridDim.x - 1) / gridDim.x * nj;
  const int ubeg = min(total, x * per_x);
  const int uend = min(total, ubeg + per_x);

  // W stages in slots 0..2, h stages in slots 3..4; the epilogue's reduction
  // records reuse slot 4 (free once the K loop is done).
  __shared__ __attribute__((aligned(1024))) uint8_t lds[(kWSlots + kHSlots) * kSlot];
  SoftmaxPart(*red)[kGM] = reinterpret_cast<SoftmaxPart(*)[kGM]>(lds + 4 * kSlot);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int grp = wave >> 2;        // 0: h rows [0, 128) and the h DMA; 1: h rows [128, 256) and the W DMA
  const int wi = wave & 3;          // 64-row W group; also this wave's 64-row share of the DMA
  const int l32 = lane & 31;
  const int kg = lane >> 5;
  uint32_t roff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) roff[kk] = l32 * 128 + ((((2 * kk + kg) ^ swz(l32))) << 4);
  const int nk = d / kGK;
  const uint32_t row_bytes = (uint32_t)d * 2u;
  const __amdgpu_buffer_rsrc_t hrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)h, (short)0, (int)((int64_t)M * d * 2), kRsrcFlags);

  for (int u = ubeg + jw; u < uend; u += nj) {
    const int vt = u / nmt;
    const int mt = u % nmt;
    const int v0 = vt * kGV;
    const int m0 = mt * kGM;
    if (rl.rows == nullptr && !guard_any(gd, m0, min(M, m0 + kGM) - 1)) continue;   // rows all complete

    f32x16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // Ping-pong K loop.  Barriers are workgroup-wide; group 1 runs one barrier
    // behind group 0, so on every SIMD one wave multiplies while the other
    // reads its next stage's fragments from LDS and issues DMA:
    //   group 0: stage s read after barrier 2s, multiplied after 2s+1
    //   group 1: stage s read after barrier 2s+1, multiplied after 2s+2
    // Group 0 loads h stage s+1 while reading stage s and waits for it before
    // barrier 2s+2; group 1 loads W stage s+2 while reading stage s and waits
    // for stage s+1 before barrier 2s+2.  A slot is refilled only after the
    // barrier that follows its last reader (every wave drains its LDS reads
    // before each barrier), and both groups pass 2 nk + 1 barriers.
    const uint8_t* wsrc = lds + 64 * wi * 128;                 // + slot * kSlot: this wave's W rows
    uint8_t* mydma = lds + 64 * wi * 128;                      // + slot * kSlot: this wave's DMA rows
    // 32-row h tiles of this group holding taken rows (4 except in the last h tile)
    const int nb = min(4, max(0, (Me - m0 - 128 * grp + 31) / 32));
    if (grp == 0) {
      uint32_t off[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 64 * wi + 8 * j + (lane >> 3);
        const int hr = m0 + r;
        // rows past the taken ones load a valid row (their output columns are
        // never written; every column depends only on its own h row)
        const int src = hr < Me ? (rl.rows != nullptr ? rl.rows[hr] : hr) : 0;
        off[j] = (uint32_t)src * row_bytes + (uint32_t)((((lane & 7) ^ swz(r))) << 4);
      }
      const uint8_t* hsrc = lds + 3 * kSlot;                 // h rows [0, 128)
      if (nb == 4)
        k_loop_g0<false>(wsrc, hsrc, mydma, hrs, off, roff, acc, nk, nb);
      else
        k_loop_g0<true>(wsrc, hsrc, mydma, hrs, off, roff, acc, nk, nb);
    } else {
      const int nv = min(kGV, V - v0);   // W rows of this tile; rows past them load row nv - 1
      uint32_t off[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 64 * wi + 8 * j + (lane >> 3);
        const int rr = r < nv ? r : nv - 1;
        off[j] = (uint32_t)rr * row_bytes + (uint32_t)((((lane & 7) ^ swz(r))) << 4);
      }
      const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(W + (size_t)v0 * d), (short)0, (int)((uint32_t)nv * row_bytes), kRsrcFlags);
      const uint8_t* hsrc = lds + 3 * kSlot + 128 * 128;     // h rows [128, 256)
      if (nmt > 1) {
        if (nb == 4)
          k_loop_g1<false, 0>(wsrc, hsrc, mydma, wrs, off, roff, acc, nk, nb);
        else
          k_loop_g1<true, 0>(wsrc, hsrc, mydma, wrs, off, roff, acc, nk, nb);
      } else {
        if (nb == 4)
          k_loop_g1<false, kDmaStream>(wsrc, hsrc, mydma, wrs, off, roff, acc, nk, nb);
        else
          k_loop_g1<true, kDmaStream>(wsrc, hsrc, mydma, wrs, off, roff, acc, nk, nb);
      }
    }

    // ---- epilogue: per h column, (max, sum exp, argmax) over this wave's 64
    // vocabulary rows, then over the 4 vocabulary waves through LDS.  Only
    // the last vocabulary tile has rows past V: every other tile takes the
    // path without the per-row bound (uniform branch).
    auto epilogue = [&](auto check_c) __attribute__((always_inline)) {
      constexpr bool CHECK = decltype(check_c)::value;
  #pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (b >= nb) break;   // no taken rows in this 32-row h tile (uniform)
        float mx = -__builtin_inff();
        int ix = INT32_MAX;
  #pragma unroll
        for (int a = 0; a < 2; ++a)
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = v0 + 64 * wi + 32 * a + 8 * (r >> 2) + 4 * kg + (r & 3);
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
              const int row = v0 + 64 * wi + 32 * a + 8 * (r >> 2) + 4 * kg + (r & 3);
              if (!CHECK || row < V) sm += fast_exp2(acc[a][b][r] * kLog2e - mxs);
            }
        }
        SoftmaxPart p{mx, sm, ix};
        p = combine(p, shfl_xor(p, 32));
        if (kg == 0) red[wi][128 * grp + 32 * b + l32] = p;
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
    __syncthreads();   // red and the stage slots are reused by the next tile
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
