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
//  * One 8-wave workgroup per CU, persistent over a balanced contiguous range
//    of 16-row vocabulary tiles.
//    Two 4-wave workgroups per CU were measured to finish far apart: the
//    workgroup placed second on a CU streamed about a third slower than the
//    first (its waves lose the CU's arbitration to the older ones), so
//    per-workgroup times spread from 84 to 189 us on the 4096-wide head and
//    the launch waited for the slowest.  With one workgroup per CU, all
//    waves of a CU advance together (one barrier per stage).  The range is
//    walked in passes of 256 rows (2 tiles per wave).
//  * W and h stream in 64-k stages by LDS DMA (buffer loads that write LDS
//    directly) into a 3-slot ring, two stages in flight: every instruction
//    brings whole 128-byte lines of 8 rows, W with the nontemporal policy,
//    placed so that the MFMA fragment reads hit distinct bank groups.  No
//    register staging: the kernel needs ~120 VGPRs.  Each workgroup starts
//    its k walk on its own stage, so the CUs do not all read the same lines
//    of h at once.
//  * Epilogue on the accumulators of each pass (folded one h tile per step
//    over the following steps): per row, lane-local max/argmax and sum of exp
//    over the lane's logits, then xor-shuffles across the 4 lane groups, a
//    running partial per wave in pass order, then the 8 waves through LDS,
//    giving one (max, sum, argmax) partial per (row, workgroup).
//  * Partials are merged in two levels by the last workgroup to arrive
//    (device-scope counters): per group of workgroups, then across groups;
//    the final merger writes conf = 1 / sum and argmax (and, when asked, runs
//    the decoder step) and re-arms the counters.  Every merge combines its
//    partials in a fixed order (a fixed tree), so results are deterministic.
//    One launch per call; no logits in HBM.
//  This file holds that K-outer kernel (any d) and, below, the rows-outer
//  kernel used when d / 256 is 1, 2, 4 or 8.
#include "dblk_device.h"
#include "dblk_launch.h"
#include "commit_wave.h"

namespace dblk {

namespace {

constexpr int kLmWaves = 8;
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kMChunk = 64;              // rows of h per pass
constexpr int kMT = kMChunk / 16;        // 16-row MFMA tiles of h
constexpr int kTargetGrid = 256;         // workgroups aimed for (one per CU)
// K-outer kernel: 2 tiles of 16 vocabulary rows per wave per pass (256 rows
// per workgroup pass), 64-k stages in a 3-slot LDS ring (two stages in flight)
constexpr int kKoTiles = 2;
constexpr int kKoPassTiles = kLmWaves * kKoTiles;
constexpr int kKoSlots = 3;
constexpr int kKoWStage = kKoPassTiles * 16 * 128;   // 32 KiB of W per stage
constexpr int kKoHStage = kMChunk * 128;             // 8 KiB of h per stage
constexpr int kKoDmaPerStep = 2 * kKoTiles + 1;      // DMA instructions per wave per stage

constexpr int kGroup = 16;               // workgroups per first-level merge group
constexpr int kTopPer = 2;               // second-level blocks per thread per pass

// Softmax partials cross workgroups through the fence-free coherent
// hand-off of dblk_device.h (coherent stores / arrive_last / coherent loads).
// A partial is one 16-byte record {max, sum, argmax, 0}; it moves as one
// buffer instruction with the sc1 cache policy -- what the compiler emits for
// agent-scope atomic loads and stores on gfx950 -- rather than as two 8-byte
// atomics, which halves the instructions of every merge (each CU's memory
// pipeline, not the bytes, limits how fast one workgroup pulls the records).
// Offsets are bytes from the partials base, which every record lies above.
// (kCachePolicySc1 and kBufferDword3: dblk_device.h)
struct PartIO {
  __amdgpu_buffer_rsrc_t rsrc;
  const char* base;
  __device__ explicit PartIO(const f32x4* partials)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(const_cast<f32x4*>(partials), (short)0, 0x7fffffff,
                                               kBufferDword3)),
        base(reinterpret_cast<const char*>(partials)) {}
  __device__ int offset(const f32x4* p) const {
    return (int)(reinterpret_cast<const char*>(p) - base);
  }
  __device__ void store(f32x4* p, const SoftmaxPart& q) const {
    const u32x4 v = {__float_as_uint(q.m), __float_as_uint(q.s), (uint32_t)q.i, 0u};
    __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, offset(p), 0, kCachePolicySc1);
  }
  __device__ SoftmaxPart load(const f32x4* p) const {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, offset(p), 0, kCachePolicySc1);
    return SoftmaxPart{__uint_as_float(v[0]), __uint_as_float(v[1]), (int32_t)v[2]};
  }
};

// Merge `count` <= 8 * PER partial blocks of 64 rows (block j of row r at
// src[j * stride + r]) in a fixed order, in an 8-wave workgroup: wave w loads
// blocks [w PER, (w + 1) PER) for row (lane), all loads issued before any is
// used, and the eight wave results are merged in wave order through LDS.  The
// returned value is valid in threads 0..63 (thread r holds row r).
template <int PER>
__device__ __forceinline__ SoftmaxPart merge_blocks8(const PartIO& io, const f32x4* src, size_t stride,
                                                     int count, int tid, SoftmaxPart (*lds)[kMChunk]) {
  const int row = tid & (kMChunk - 1);
  const int w = tid / kMChunk;
  // Loads are unconditional (index clamped into range, the neutral element
  // selected afterwards): a branch per block would make the compiler wait out
  // each load before issuing the next.
  SoftmaxPart v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int blk = w * PER + u;
    v[u] = io.load(src + (size_t)(blk < count ? blk : count - 1) * stride + row);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (w * PER + u >= count) v[u] = SoftmaxPart{-__builtin_inff(), 0.f, INT32_MAX};
  SoftmaxPart q = combine_tree(v);
  __syncthreads();
  lds[w][row] = q;
  __syncthreads();
  if (tid < kMChunk) {
    SoftmaxPart r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) r[k] = lds[k][tid];
    q = combine_tree(r);
  }
  return q;
}

__global__ void __launch_bounds__(kLmThreads, 1)
lmhead_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int M, int d,
              int V, float* __restrict__ conf, int32_t* __restrict__ amax,
              uint32_t* __restrict__ counters, f32x4* __restrict__ partials, int G, Guard gd,
              FusedCommit fc) {
  const int g = blockIdx.x;
  const int mc = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int m0 = mc * kMChunk;
  // block loop: every sequence of this row chunk is complete.  All workgroups
  // of the chunk decide alike, so its arrival counter stays consistent.
  if (!guard_any(gd, m0, min(M, m0 + kMChunk) - 1)) return;
  const CommitIn cin = commit_prefetch(fc, m0, M, tid & (kMChunk - 1));
  static_assert(kMChunk == 8 * kLmWaves, "wave w loads h rows 8 w .. 8 w + 7 of each stage");

  // One LDS object holds the stage ring, the reduction records and the
  // arrival flag.  (With several LDS objects the compiler can tell the ring's
  // DMA targets and fragment reads apart only as the same object, and then
  // waits for every DMA in flight before each fragment read.)
  constexpr int kRingBytes = kKoSlots * (kKoWStage + kKoHStage);
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kRingBytes + kLmWaves * kMChunk * sizeof(SoftmaxPart) + 16];
  auto ring = [&](int i) { return lds + i * (kKoWStage + kKoHStage); };
  SoftmaxPart(*red)[kMChunk] = reinterpret_cast<SoftmaxPart(*)[kMChunk]>(lds + kRingBytes);
  int& s_last = *reinterpret_cast<int*>(lds + kRingBytes + kLmWaves * kMChunk * sizeof(SoftmaxPart));

  // Workgroup g owns the contiguous tiles [ntile g / G, ntile (g + 1) / G)
  // (at least one), walked in passes of kKoPassTiles tiles: in pass p, wave w
  // holds tiles tile_beg + 16 p + 2 w + {0, 1}.  Rows from row_end on (the
  // range's end, or V) read as zeros and are never reported.
  const int ntile_all = (V + 15) / 16;
  const int tile_beg = (int)((long long)ntile_all * g / G);
  const int tile_end = (int)((long long)ntile_all * (g + 1) / G);
  const int row_end = min(V, tile_end * 16);
  const int npass = (tile_end - tile_beg + kKoPassTiles - 1) / kKoPassTiles;
  const int nk = d / 64;                   // 64-wide k stages per pass
  // Every workgroup walks the k stages from its own starting stage: h is
  // read by all CUs, and in lockstep they all hit the same few L2 lines at
  // once (measured on the 4096-wide head: 182 us per call; every workgroup
  // of an XCD on its own starting stage: 162 us).  Under round-robin
  // dispatch g % 8 is the XCD and g / 8 the workgroup's place in it.
  const int k_rot = ((g >> 3) * max(1, nk / 32) + (g & 7)) % nk;
  const int nsteps = npass * nk;
  const uint32_t row_bytes = (uint32_t)d * 2u;

  // ---- DMA of one step (pass t / nk, k stage (t % nk + k_rot) % nk) into
  // ring slot t % 3.
  // W: per tile, 2 instructions of 8 rows x 128 bytes (whole lines, lane i:
  // row 8 j + i / 8, chunk (i % 8) ^ swz(row)) -- the tile image is 16 rows
  // x 128 bytes with chunk c of row r at position c ^ swz(r), so that the
  // A-fragment reads below hit distinct bank groups.  The W descriptor starts
  // at the pass's first row (byte offsets < 2^23).  h: one instruction per
  // wave, rows 8 w .. 8 w + 7 of the chunk as whole lines, laid out like a W
  // tile (rows past M load row 0; their columns are never reported).  W takes
  // the nontemporal policy (it streams through once; 7.0 against 6.2 TB/s in
  // a probe of this access pattern), h the default one (every CU re-reads it).
  auto swz = [](int r) { return (r >> 1) & 7; };
  const int hr_in = 8 * wave + (lane >> 3);                          // h row of the chunk this lane brings
  const int hrow = m0 + hr_in;
  const uint32_t h_off = (uint32_t)(hrow < M ? hrow : 0) * row_bytes + (uint32_t)(((lane & 7) ^ swz(hr_in)) << 4);
  const __amdgpu_buffer_rsrc_t hrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(h), (short)0, (int)((uint32_t)M * row_bytes), kBufferDword3);
  // Lane offsets within a pass are fixed (computed once); the pass enters
  // through the descriptor, which starts at the pass's first row and ends
  // after its last valid row, so rows past row_end read as zeros (and are
  // never reported).
  uint32_t woff[kKoTiles][2];
#pragma unroll
  for (int tt = 0; tt < kKoTiles; ++tt)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 8 * j + (lane >> 3);                           // row within the tile
      woff[tt][j] = (uint32_t)((2 * wave + tt) * 16 + r) * row_bytes + (uint32_t)(((lane & 7) ^ swz(r)) << 4);
    }
  auto issue = [&](int t) {
    const int pass = t / nk;
    const int ks = (t - pass * nk + k_rot) % nk;
    const int prow0 = (tile_beg + pass * kKoPassTiles) * 16;       // first row of the pass
    const int prows = min(row_end - prow0, kKoPassTiles * 16);     // rows this pass may read
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(W + (size_t)prow0 * (size_t)d), (short)0, (int)((uint32_t)prows * row_bytes),
        kBufferDword3);
    uint8_t* slot = ring(t % kKoSlots);
#pragma unroll
    for (int tt = 0; tt < kKoTiles; ++tt)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_ptr_t)(slot + ((2 * wave + tt) * 16 + 8 * j) * 128), 16,
                                                 woff[tt][j], (uint32_t)ks * 128u, 0, kDmaStream);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(hrs, (lds_ptr_t)(slot + kKoWStage + wave * 1024), 16, h_off,
                                             (uint32_t)ks * 128u, 0, 0);
  };

  f32x4 acc[kKoTiles][kMT];
#pragma unroll
  for (int tt = 0; tt < kKoTiles; ++tt)
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) acc[tt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  SoftmaxPart run[kMT];   // this wave's running partial per h row (mt * 16 + l16)
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) run[mt] = SoftmaxPart{-__builtin_inff(), 0.f, INT32_MAX};
  f32x4 prev[kKoTiles][kMT];   // the last finished pass's logits, folded over the next steps
  int prev_tile0 = 0;          // its first tile for this wave
  int pend = 0;                // h tiles of prev still to fold (kMT - pend is next)
  // ---- pass epilogue of h tile `sel` of prev: (max, sum exp, argmax) per h
  // row over this wave's 32 vocabulary rows, folded into the running partial
  // in pass order (so the result does not depend on timing)
  auto fold_prev = [&](int sel) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt) {
      if (mt != sel) continue;
      float mx = -__builtin_inff();
      int ix = INT32_MAX;
#pragma unroll
      for (int tt = 0; tt < kKoTiles; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = (prev_tile0 + tt) * 16 + grp * 4 + r;
          const float x = prev[tt][mt][r];
          if (row < row_end && x > mx) {
            mx = x;
            ix = row;
          }
        }
      float sm = 0.f;
      if (ix != INT32_MAX) {
        const float mxs = mx * kLog2e;
#pragma unroll
        for (int tt = 0; tt < kKoTiles; ++tt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = (prev_tile0 + tt) * 16 + grp * 4 + r;
            if (row < row_end) sm += fast_exp2(prev[tt][mt][r] * kLog2e - mxs);
          }
      }
      SoftmaxPart p{mx, sm, ix};
      p = combine(p, shfl_xor(p, 16));
      p = combine(p, shfl_xor(p, 32));
      run[mt] = combine(run[mt], p);
    }
  };

  issue(0);
  if (nsteps > 1) issue(1);
  for (int t = 0; t < nsteps; ++t) {
    // step t's DMA (this wave's share) has landed once only step t + 1's
    // kKoDmaPerStep instructions may still be outstanding; the barrier makes
    // every wave's share visible and frees slot (t + 2) % 3 (read at t - 1)
    if (t + 1 < nsteps)
      wait_vm<kKoDmaPerStep>();
    else
      wait_vm<0>();
    stage_barrier();
    if (t + 2 < nsteps) issue(t + 2);
    const uint8_t* slot = ring(t % kKoSlots);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 hf[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
        hf[mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(
            slot + kKoWStage + (mt * 16 + l16) * 128 + (((grp + 4 * kk) ^ swz(l16)) << 4)));
#pragma unroll
      for (int tt = 0; tt < kKoTiles; ++tt) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
            slot + ((2 * wave + tt) * 16 + l16) * 128 + (((grp + 4 * kk) ^ swz(l16)) << 4)));
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) acc[tt][mt] = mfma16x16x32(a, hf[mt], acc[tt][mt]);
      }
    }
    // A finished pass's logits move to prev and are folded one h tile per
    // step over the next steps, while the wave would otherwise wait for its
    // DMA; folding all four at once stalls every wave at the next barrier.
    if (pend > 0) {
      fold_prev(kMT - pend);
      --pend;
    }
    if (t % nk == nk - 1) {
      while (pend > 0) {   // passes shorter than four steps
        fold_prev(kMT - pend);
        --pend;
      }
#pragma unroll
      for (int tt = 0; tt < kKoTiles; ++tt)
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) {
          prev[tt][mt] = acc[tt][mt];
          acc[tt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      prev_tile0 = tile_beg + (t / nk) * kKoPassTiles + 2 * wave;
      pend = kMT;
    }
  }
  while (pend > 0) {
    fold_prev(kMT - pend);
    --pend;
  }
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
    if (grp == 0) red[wave][mt * 16 + l16] = run[mt];
  __syncthreads();
  if (tid < kMChunk) {
    SoftmaxPart q = red[0][tid];
#pragma unroll
    for (int w = 1; w < kLmWaves; ++w) q = combine(q, red[w][tid]);
    PartIO(partials).store(&partials[((size_t)mc * G + g) * kMChunk + tid], q);
  }

  // ---- two-level merge of the per-workgroup partials of this M chunk.
  // Level 1: the last workgroup of each group of kGroup merges the group's
  // partials.  Level 2: the last of those merges the group results and writes
  // conf / argmax.  Merges run in a fixed order; each level issues all of
  // its loads before the first wait, so it costs about one memory round trip.
  const int ngroups = (G + kGroup - 1) / kGroup;
  const int grp_id = g / kGroup;
  uint32_t* ctr = counters + (size_t)mc * (ngroups + 1);
  f32x4* gpart = partials + (size_t)mc * G * kMChunk;                       // [G][64]
  f32x4* tpart = partials + (size_t)gridDim.y * G * kMChunk + (size_t)mc * ngroups * kMChunk;
  if (!arrive_last(&ctr[grp_id], min(kGroup, G - grp_id * kGroup), tid, &s_last)) return;
  const PartIO io(partials);
  SoftmaxPart q = merge_blocks8<kGroup / kLmWaves>(io, gpart + (size_t)grp_id * kGroup * kMChunk, kMChunk,
                                                   min(kGroup, G - grp_id * kGroup), tid, red);
  if (tid < kMChunk) io.store(&tpart[(size_t)grp_id * kMChunk + tid], q);
  if (!arrive_last(&ctr[ngroups], ngroups, tid, &s_last)) return;
  q = SoftmaxPart{-__builtin_inff(), 0.f, INT32_MAX};
  for (int b0 = 0; b0 < ngroups; b0 += kLmWaves * kTopPer) {
    const SoftmaxPart r = merge_blocks8<kTopPer>(io, tpart + (size_t)b0 * kMChunk, kMChunk,
                                                 min(kLmWaves * kTopPer, ngroups - b0), tid, red);
    q = combine(q, r);
  }
  if (tid < kMChunk && m0 + tid < M) {
    conf[m0 + tid] = 1.0f / q.s;
    amax[m0 + tid] = q.i;
  }
  if (fc.tokens != nullptr && tid < kMChunk) commit_chunk_wave(fc, m0, M, tid, 1.0f / q.s, q.i, cin);
  if (tid == 0) {
    for (int k = 0; k <= ngroups; ++k)   // re-arm for the next call
      __hip_atomic_store(&ctr[k], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}


// Merge count <= N partial blocks in one wave (lane = row; block j of the row
// at src[j * stride + row]) as the fixed tree of combine_tree: the same result
// as merge_blocks8<1> with one block per wave.
template <int N>
__device__ __forceinline__ SoftmaxPart merge_wave(const PartIO& io, const f32x4* src, size_t stride,
                                                  int count, int lane) {
  SoftmaxPart v[N];
#pragma unroll
  for (int u = 0; u < N; ++u) v[u] = io.load(src + (size_t)(u < count ? u : count - 1) * stride + lane);
#pragma unroll
  for (int u = 0; u < N; ++u)
    if (u >= count) v[u] = SoftmaxPart{-__builtin_inff(), 0.f, INT32_MAX};
  return combine_tree(v);
}

// Position of the n-th (from 0) set bit of x; n < popcount(x).  Binary
// search over halves with popcounts.
__device__ __forceinline__ int nth_set_bit(uint64_t x, int n) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const uint64_t lo = x & ((1ull << w) - 1ull);
    const int c = __popcll(lo);
    if (n >= c) {
      n -= c;
      x >>= w;
      pos += w;
    } else {
      x = lo;
    }
  }
  return pos;
}

// ---------------------------------------------------------------------------
// Rows-outer variant for d <= 2048 (d a multiple of 256): K is split over the
// 8 waves of a workgroup and each wave keeps its 16 x (d/8) slice of every
// 16-row h tile resident in registers (B operands, loaded once).  The
// workgroup then walks its contiguous range of 16-row vocabulary tiles; the
// 8 waves together read each tile as 16 whole W rows (every row one
// contiguous d*2-byte run), so each workgroup streams one contiguous region
// of W -- the access pattern HBM serves best.  Per tile every wave multiplies
// its K slice (partial logits 16 rows x 64 columns), the partials are summed
// across the waves through a double-buffered LDS tile in fixed wave order,
// and each thread folds two logits of one column into an online
// (max, sum of exp, argmax).  The next tiles' W slices are in flight while
// the current one is multiplied and reduced.
constexpr int kRowWaves = 8;
constexpr int kRowThreads = kRowWaves * kWave;
constexpr int kRowGrid = 256;            // one workgroup per CU
constexpr int kRowRing = 2;              // W slices in registers (tiles in flight + 1)
constexpr int kRowGroups = 8;            // first-level merge groups (g mod 8: one per XCD)
// Vocabulary share of a workgroup with even / odd g.  Under round-robin
// dispatch g mod 8 is the XCD, and on MI355X the odd-numbered XCDs were
// measured to stream W about 5% slower than the even ones (every box tried,
// 2048-wide head); weighting the static split 20 : 19 evens out their finish
// times (about 2 us off a 108 us launch).
constexpr int kRowWeightEven = 20;
constexpr int kRowWeightOdd = 19;
constexpr int kRowMergePer = 4;          // group members per wave in a first-level merge
constexpr int kGemmMinRows = 256;        // from this many block rows on, the MFMA-bound GEMM path

template <int KS, int RR>   // 32-wide k steps per wave slice (d = 8*32*KS); W ring slots
__global__ void __launch_bounds__(kRowThreads, 1)
lmhead_rows_kernel(const uint16_t* __restrict__ h, const uint16_t* __restrict__ W, int M, int V,
                   float* __restrict__ conf, int32_t* __restrict__ amax,
                   uint32_t* __restrict__ counters, f32x4* __restrict__ partials, int G, Guard gd,
                   FusedCommit fc, const uint8_t* __restrict__ cmask) {
  constexpr int d = kRowWaves * 32 * KS;
  const int g = blockIdx.x;
  const int mc = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  const int m0 = mc * kMChunk;
  if (!guard_any(gd, m0, min(M, m0 + kMChunk) - 1)) return;   // as in lmhead_kernel
  const CommitIn cin = commit_prefetch(fc, m0, M, tid & (kMChunk - 1));
  const int kbase = wave * 32 * KS + grp * 8;   // this lane's k offset within a row
  // Rows of the chunk that go through the head: all, or (masked-row
  // compaction, cmask given) those masked on entry.  Column c of the chunk's
  // logits is row m0 + nth_set_bit(rows, c), c < nused; the other columns
  // are computed on duplicate data and never reported.
  const int nrows = min(M - m0, kMChunk);
  const uint8_t mk = (cmask != nullptr && lane < nrows) ? cmask[m0 + lane] : 1;

  __shared__ f32x4 red_tile[2][kRowWaves][kMT][kWave];   // 2 x 32 KB
  __shared__ SoftmaxPart fin[kRowWaves][kMChunk];
  __shared__ int s_last;

  // Workgroup g owns the contiguous tiles [start(g), start(g + 1)), with
  // start(g) = ntile * W(g) / W(G) and W(g) the summed weights of workgroups
  // 0..g-1 (exact integer arithmetic: the ranges tile [0, ntile) in order).
  // A workgroup may own no tile when ntile < G; it then contributes the
  // neutral partial.
  const int ntile_all = (V + 15) / 16;
  auto range_start = [&](int gg) -> int {
    const long long w = (long long)((gg + 1) / 2) * kRowWeightEven + (long long)(gg / 2) * kRowWeightOdd;
    const long long wt = (long long)((G + 1) / 2) * kRowWeightEven + (long long)(G / 2) * kRowWeightOdd;
    return (int)((long long)ntile_all * w / wt);
  };
  const int tile_begin = range_start(g);
  const int ntiles = range_start(g + 1) - tile_begin;

  u32x4 hreg[KS][kMT];   // this wave's K slice of the 64 h rows (B operands)
  u32x4 wr[RR][KS];
  // W loads.  Staged (KS >= 4, d >= 1024): instruction j of a tile covers RPI
  // whole rows of this wave's K slice (CPR 16-byte chunks = 64*KS >= 256 bytes
  // per row: whole 128-byte lines, so the streaming hint pays), and the chunks
  // pass through a wave-private LDS tile [16 rows][CPR slots] into the MFMA
  // A-fragment layout (lane: row l % 16, chunk l / 16 + 4 ks).  Slot =
  // chunk ^ swz(row) puts the 16 lanes of every store pass and of every
  // fragment-read pass on distinct 16-byte bank groups.  No barrier: only this
  // wave touches its tile, and its LDS operations stay in program order.
  // Measured on the 2048-wide head: 128 -> 111-119 us.  With shorter slices
  // (d <= 512) the staging costs more than it gains, and each lane loads its
  // fragment directly (16 rows x 64 bytes per instruction, plain loads).
  constexpr bool STAGED = KS >= 4;
  constexpr int CPR = 4 * KS;
  constexpr int RPI = 64 / CPR;                       // rows per load instruction
  constexpr int RPWIN = CPR >= 16 ? 1 : 16 / CPR;     // rows per 256-byte bank window
  constexpr int SWM = (CPR >= 16 ? 16 : CPR) - 1;
  __shared__ u32x4 stage[STAGED ? kRowWaves : 1][STAGED ? 16 * CPR : 1];
  const int ld_row = STAGED ? lane / CPR : l16;
  const int ld_chunk = STAGED ? lane % CPR : grp;
  auto slot_of = [](int row, int chunk) { return row * CPR + (chunk ^ ((row / RPWIN) & SWM)); };
  // Past the workgroup's last tile the ring still issues its loads (a fixed
  // load count keeps the wait counts exact) but aims them at row 0 of h, which
  // every workgroup has just read and L2 holds: a streamed W line would not be.
  // The address stays W + offset (one base pointer keeps these global loads).
  const int64_t h_rel = (int64_t)(reinterpret_cast<uintptr_t>(h) - reinterpret_cast<uintptr_t>(W)) / 2;
  auto issue = [&](int slot, int i) {
    const bool past = i >= ntiles;
    const int tile = tile_begin + (past ? 0 : i);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      // staged: rows ld_row + RPI j, chunk ld_chunk; direct: row l16, chunk grp + 4 j
      int row = tile * 16 + ld_row + (STAGED ? RPI * j : 0);
      row = row < V ? row : V - 1;
      const int64_t base = past ? h_rel : (int64_t)row * d;
      const uint16_t* wp = W + base + wave * 32 * KS + (ld_chunk + (STAGED ? 0 : 4 * j)) * 8;
      wr[slot][j] = STAGED ? load_stream(wp) : *reinterpret_cast<const u32x4*>(wp);
    }
  };

  // reduction-phase role of this thread: column m = 16 mt + (ln % 16) and
  // rows 4 (ln / 16) + 2 rh + {0, 1} of each tile
  const int r_mt = tid / 128;
  const int r_ln = (tid / 2) % kWave;
  const int r_rh = tid & 1;
  const int r_row = 4 * (r_ln >> 4) + 2 * r_rh;
  float run_m = -__builtin_inff(), run_s = 0.f;
  int run_i = INT32_MAX;

  auto step = [&](int i, int slot) {
    issue((slot + RR - 1) % RR, i + RR - 1);   // RR - 1 tiles' slices in flight
    __builtin_amdgcn_sched_barrier(0);   // keep those loads ahead of this tile's work
    if (i < ntiles) {
      u32x4* st = stage[STAGED ? wave : 0];
      if (STAGED) {
#pragma unroll
        for (int j = 0; j < KS; ++j) st[slot_of(ld_row + RPI * j, ld_chunk)] = wr[slot][j];
      }
      f32x4 acc[kMT];
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 a = as_bf16x8(STAGED ? st[slot_of(l16, grp + 4 * ks)] : wr[slot][ks]);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt) acc[mt] = mfma16x16x32(a, as_bf16x8(hreg[ks][mt]), acc[mt]);
      }
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt) red_tile[i & 1][wave][mt][lane] = acc[mt];
    }
    __syncthreads();
    if (i < ntiles) {
      // sum the 8 K-slice partials of two logits, in wave order
      const float* base = reinterpret_cast<const float*>(&red_tile[i & 1][0][r_mt][r_ln]) + 2 * r_rh;
      float x0 = 0.f, x1 = 0.f;
#pragma unroll
      for (int w = 0; w < kRowWaves; ++w) {
        const float* p = base + (size_t)w * kMT * kWave * 4;
        x0 += p[0];
        x1 += p[1];
      }
      const int row0 = (tile_begin + i) * 16 + r_row;
      const bool v0 = row0 < V, v1 = row0 + 1 < V;
      float mx = run_m;
      int ix = run_i;
      if (v0 && x0 > mx) { mx = x0; ix = row0; }
      if (v1 && x1 > mx) { mx = x1; ix = row0 + 1; }
      if (ix != INT32_MAX) {
        const float mxs = mx * kLog2e;
        float sm = run_s * fast_exp2(run_m * kLog2e - mxs);
        if (run_m == -__builtin_inff()) sm = 0.f;
        if (v0) sm += fast_exp2(x0 * kLog2e - mxs);
        if (v1) sm += fast_exp2(x1 * kLog2e - mxs);
        run_s = sm;
      }
      run_m = mx;
      run_i = ix;
    }
  };

#pragma unroll
  for (int r = 0; r < RR - 1; ++r) issue(r, r);   // W first: its round trip overlaps h's
  __builtin_amdgcn_sched_barrier(0);   // the W loads go out before the mask is awaited
  const uint64_t rows = __ballot(lane < nrows && mk != 0);
  const int nused = __popcll(rows);
  const int ntl = (nused + 15) / 16;    // h tiles holding a used column
  // h slice (loaded once): B operand of k step ks, h tile mt.  Only tiles
  // holding a used column are loaded (a uniform branch; the others are zero),
  // and within the last such tile only the used columns (the rest are zero):
  // this start-up load is bound by each CU's memory pipeline -- the first
  // tile of a 2048-wide launch lands 3 us earlier when half of the rows are
  // compacted away.
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const int c = mt * 16 + l16;
    const bool used = c < nused;
    const int row = m0 + (used ? nth_set_bit(rows, c) : 0);
    const uint16_t* hp = h + (size_t)row * d + kbase;
    if (mt < ntl) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        hreg[ks][mt] = used ? *reinterpret_cast<const u32x4*>(hp + ks * 32) : u32x4{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) hreg[ks][mt] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  for (int i = 0; i < ntiles; i += RR) {
#pragma unroll
    for (int r = 0; r < RR; ++r) step(i + r, r);
  }

  // ---- fold the 8 threads that share a column (in row-group order)
  fin[(r_ln >> 4) * 2 + r_rh][r_mt * 16 + (r_ln & 15)] = SoftmaxPart{run_m, run_s, run_i};
  __syncthreads();
  if (tid < kMChunk) {
    SoftmaxPart r[kRowWaves];
#pragma unroll
    for (int k = 0; k < kRowWaves; ++k) r[k] = fin[k][tid];
    const SoftmaxPart q = combine_tree(r);
    PartIO(partials).store(&partials[((size_t)mc * G + g) * kMChunk + tid], q);
  }

  // ---- two-level merge.  One CU pulls only a few tens of GB/s, so no single
  // workgroup reads all G partials.  Level 1: the workgroups with equal
  // g mod 8 -- the same XCD under round-robin dispatch, so a group finishes
  // with its XCD and the early XCDs' merges overlap the late XCDs' streaming
  // -- are merged by the group's last arrival.  Level 2: the last group merges
  // the group results, writes conf / argmax and runs the fused decoder step.
  // Any placement is correct: every hand-off is coherent.
  const int ngrp = G < kRowGroups ? G : kRowGroups;
  const int mgrp = g % ngrp;
  const int members = (G - mgrp + ngrp - 1) / ngrp;       // g' = mgrp, mgrp + ngrp, ... < G
  uint32_t* ctr = counters + (size_t)mc * (kRowGroups + 1);
  const f32x4* gpart = partials + (size_t)mc * G * kMChunk;
  f32x4* tpart = partials + (size_t)gridDim.y * G * kMChunk + (size_t)mc * kRowGroups * kMChunk;
  if (!arrive_last(&ctr[mgrp], members, tid, &s_last)) return;
  if (tid == 0) rearm_counter(&ctr[mgrp]);                 // every member has arrived
  const PartIO io(partials);
  SoftmaxPart q = merge_blocks8<kRowMergePer>(io, gpart + (size_t)mgrp * kMChunk,
                                              (size_t)ngrp * kMChunk, members, tid, fin);
  if (tid < kMChunk) io.store(&tpart[(size_t)mgrp * kMChunk + tid], q);
  if (!arrive_last(&ctr[kRowGroups], ngrp, tid, &s_last)) return;
  if (tid >= kMChunk) return;
  // wave 0 alone: the (at most 8) group results of its column, one tree
  q = merge_wave<kRowGroups>(io, tpart, kMChunk, ngrp, tid);
  const float cf = 1.0f / q.s;
  if (tid < nused) {
    const int row = m0 + nth_set_bit(rows, tid);
    conf[row] = cf;
    amax[row] = q.i;
  }
  if (fc.tokens != nullptr) {   // lane r takes row m0 + r's column (used rows only matter)
    const int col = __popcll(rows & ((1ull << tid) - 1ull));
    commit_chunk_wave(fc, m0, M, tid, __shfl(cf, col, kWave), __shfl(q.i, col, kWave), cin);
  }
  if (tid == 0) rearm_counter(&ctr[kRowGroups]);
}

hipError_t launch_kouter(const void* h, const void* W, int M, int d, int V, float* conf,
                         int32_t* amax, uint32_t* counters, f32x4* partials,
                         const LmheadPlan& p, const Guard& gd, const FusedCommit& fc,
                         hipStream_t stream) {
  return launch_kernel(lmhead_kernel, dim3(p.grid, p.mchunks), dim3(kLmThreads), 0, stream,
                       static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W), M, d,
                       V, conf, amax, counters, partials, p.grid, gd, fc);
}

template <int KS>
hipError_t launch_rows(const void* h, const void* W, int M, int V, float* conf, int32_t* amax,
                       uint32_t* counters, f32x4* partials, const LmheadPlan& p,
                       const Guard& gd, const FusedCommit& fc, const uint8_t* cmask,
                       hipStream_t stream) {
  return launch_kernel(lmhead_rows_kernel<KS, kRowRing>, dim3(p.grid, p.mchunks), dim3(kRowThreads), 0,
                       stream, static_cast<const uint16_t*>(h), static_cast<const uint16_t*>(W),
                       M, V, conf, amax, counters, partials, p.grid, gd, fc, cmask);
}

}  // namespace

bool lmhead_can_fuse_commit(const LmheadPlan& p, int L) {
  return !p.gemm && L >= 1 && L <= kMChunk && (L & (L - 1)) == 0;
}

LmheadPlan lmhead_plan(int M, int d, int V) {
  LmheadPlan p;
  p.gemm = M >= kGemmMinRows;
  if (p.gemm) {
    p.g = gemm_plan(M, d, V);
    p.rows_outer = false;
    p.ntile = p.nt = p.tiles_per_wg = p.grid = p.mchunks = 0;
    p.counters_bytes = 0;
    p.partials_bytes = p.g.rows_offset + p.g.rows_bytes;
    return p;
  }
  p.ntile = (V + 15) / 16;
  p.mchunks = (M + kMChunk - 1) / kMChunk;
  const int ks = d / (kRowWaves * 32);
  p.rows_outer = (d % (kRowWaves * 32) == 0) && (ks == 1 || ks == 2 || ks == 4 || ks == 8);
  if (p.rows_outer) {
    p.nt = 0;
    p.grid = p.ntile < kRowGrid ? p.ntile : kRowGrid;          // one workgroup per CU
    p.tiles_per_wg = (p.ntile + p.grid - 1) / p.grid;           // about; the kernel weights the split
  } else {
    // one workgroup per CU (fewer for a small vocabulary), each with a
    // balanced contiguous tile range walked in passes of kKoPassTiles tiles
    p.grid = p.ntile < kTargetGrid ? p.ntile : kTargetGrid;
    p.tiles_per_wg = (p.ntile + p.grid - 1) / p.grid;
    p.nt = (p.tiles_per_wg + kKoPassTiles - 1) / kKoPassTiles;   // passes
  }
  const int ngroups = p.rows_outer ? kRowGroups : (p.grid + kGroup - 1) / kGroup;
  p.counters_bytes = (((size_t)p.mchunks * (ngroups + 1) * sizeof(uint32_t)) + 255) / 256 * 256;
  p.partials_bytes = (size_t)p.mchunks * (p.grid + ngroups) * kMChunk * sizeof(f32x4);
  return p;
}

hipError_t launch_lmhead(const void* h, const void* W, int M, int d, int V, float* conf,
                         int32_t* amax, void* ws, const LmheadPlan& p, const Guard& gd,
                         const FusedCommit& fc, const uint8_t* masked_only, hipStream_t stream) {
  if (fc.tokens != nullptr && !lmhead_can_fuse_commit(p, fc.L)) return hipErrorInvalidValue;
  if (p.gemm)
    return launch_lmhead_gemm(h, W, M, d, V, conf, amax, ws, p.g, gd, masked_only, stream);
  uint32_t* counters = static_cast<uint32_t*>(ws);
  f32x4* partials = reinterpret_cast<f32x4*>(static_cast<char*>(ws) + p.counters_bytes);
  if (p.rows_outer) {
    switch (d / (kRowWaves * 32)) {
      case 1: return launch_rows<1>(h, W, M, V, conf, amax, counters, partials, p, gd, fc, masked_only, stream);
      case 2: return launch_rows<2>(h, W, M, V, conf, amax, counters, partials, p, gd, fc, masked_only, stream);
      case 4: return launch_rows<4>(h, W, M, V, conf, amax, counters, partials, p, gd, fc, masked_only, stream);
      default: return launch_rows<8>(h, W, M, V, conf, amax, counters, partials, p, gd, fc, masked_only, stream);
    }
  }
  return launch_kouter(h, W, M, d, V, conf, amax, counters, partials, p, gd, fc, stream);
}

}  // namespace dblk
