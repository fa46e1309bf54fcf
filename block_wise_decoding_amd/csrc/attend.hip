// Non-causal attention of the active block over the dual KV cache.
//
// dInfer's decoder runs with the dual KV-cache factory (README, usage section):
// keys/values of the prefix before the block and of the suffix after it are
// cached, only the block's own are fresh, and -- diffusion LMs attend
// bidirectionally (topic page, variable-size-block and Streaming-dLLM
// abstracts) -- every block query attends to all keys of the three segments.
//
// Design (gfx950, wave64, 16x16x32 bf16 MFMA, fp32 accumulation):
//  * Grid (split, head, batch); one 4-wave workgroup walks 64-key tiles of
//    its key range with an online (running max / running sum) softmax in
//    base 2.  Each wave owns one or two 16-query tiles of the block.
//  * Scores are computed transposed, S^T = K Q^T (A = K rows straight from
//    LDS, B = Q held in registers for the whole walk).  The S^T accumulator
//    then already has the layout of the B operand of O^T = V^T P^T, so the
//    probabilities are packed to bf16 in place, with no shuffle.
//  * K and V go straight from HBM into an LDS ring by DMA (global_load_lds,
//    whole key rows per instruction, nontemporal): the next tile(s) are in
//    flight while the current one is multiplied, one barrier per tile.  Both
//    tiles row-major, rows unpadded with their 16-byte chunks XOR-swizzled
//    by row (conflict-free fragment reads); V's A-fragments of the P.V
//    product (8 keys of one dimension per lane) come from gfx950's
//    transposed LDS read.  Against the earlier register staging: the
//    long-context batch's attention 123 -> 98 us per call, the LLaDA-8B and
//    LLaDA-MoE blocks' 15.9 -> 15.0 and 12.2 -> 11.8 us.
//  * Keys are numbered 0..T_b-1 over prefix ++ block ++ suffix; each loaded
//    key resolves its segment and row (every segment has its own element
//    strides and, optionally, per-sequence length), so ragged lengths, tiles
//    that straddle a segment boundary and head-interleaved caches need no
//    special case.  Keys past the range score -inf.
//  * With one split the kernel normalises and writes bf16 output; otherwise it
//    writes each row's unnormalised O as fp16 scaled by a power of two, plus
//    one {max, sum, scale} record per row, and a second kernel merges the
//    splits, spread over the whole chip.  (Merging in the same launch -- the
//    last workgroup of each (b, h) to arrive reads every split's partial --
//    was measured slower: on the LLaDA-MoE-shaped block one CU then pulls ten
//    33 KB fp32 partials, 26.7 us for the launch against 8.9 + 4.5 us for the
//    two kernels.)
#include "dblk_device.h"
#include "dblk_launch.h"

namespace dblk {

namespace {

constexpr int kAttThreads = 256;                // 4 waves
constexpr int kAttWaves = kAttThreads / kWave;
constexpr int kKT = 64;                          // keys per tile
constexpr int kTargetWGs = 256;                  // workgroups aimed for when choosing splits
constexpr int kLongRange = 8 * kKT;              // keys per split from which two waves share a tile
// Split merge: 128-thread workgroups, so that a 16-head block (32768 threads)
// spreads its partials over all 256 CUs; each CU pulls only a few tens of
// GB/s, so the bytes per CU set the merge time.
constexpr int kCombineThreads = 128;
constexpr float kRescaleSlack = 8.f;             // log2 units a score may pass the reference by
template <int N> struct SlotC { static constexpr int value = N; };

// As tr16_read4, with per-lane base addresses a[q] and the immediate byte
// offsets OFF (lo reads) and OFF + HI (hi reads): no address arithmetic per
// read (0 <= OFF, OFF + HI < 65536).
template <int OFF, int HI>
__device__ __forceinline__ void tr16_read4_imm(u32x2 (&lo)[4], u32x2 (&hi)[4], const uint32_t (&a)[4]) {
  static_assert(OFF >= 0 && OFF + HI < 65536, "16-bit DS offset");
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %1, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %2, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %3, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %10 offset:%13\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]),
        "=&v"(hi[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF), "i"(OFF + HI)
      : "memory");
}

// The 16 K fragments of one 64-key tile for head dimension 128: fragment
// 4u + k from lane address a[k] + OFF + u RS (u, k < 4), complete on return.
// One asm block, one wait: the compiler batched these reads four at a time,
// each batch behind a wait of its own.
template <int OFF, int RS>
__device__ __forceinline__ void k_read16(u32x4 (&f)[16], const uint32_t (&a)[4]) {
  static_assert(OFF >= 0 && OFF + 3 * RS < 65536, "16-bit DS offset");
  asm volatile(
      "ds_read_b128 %0, %16 offset:%20\n\t"
      "ds_read_b128 %1, %17 offset:%20\n\t"
      "ds_read_b128 %2, %18 offset:%20\n\t"
      "ds_read_b128 %3, %19 offset:%20\n\t"
      "ds_read_b128 %4, %16 offset:%21\n\t"
      "ds_read_b128 %5, %17 offset:%21\n\t"
      "ds_read_b128 %6, %18 offset:%21\n\t"
      "ds_read_b128 %7, %19 offset:%21\n\t"
      "ds_read_b128 %8, %16 offset:%22\n\t"
      "ds_read_b128 %9, %17 offset:%22\n\t"
      "ds_read_b128 %10, %18 offset:%22\n\t"
      "ds_read_b128 %11, %19 offset:%22\n\t"
      "ds_read_b128 %12, %16 offset:%23\n\t"
      "ds_read_b128 %13, %17 offset:%23\n\t"
      "ds_read_b128 %14, %18 offset:%23\n\t"
      "ds_read_b128 %15, %19 offset:%23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]), "=&v"(f[6]), "=&v"(f[7]),
        "=&v"(f[8]), "=&v"(f[9]), "=&v"(f[10]), "=&v"(f[11]), "=&v"(f[12]), "=&v"(f[13]), "=&v"(f[14]),
        "=&v"(f[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF), "i"(OFF + RS), "i"(OFF + 2 * RS), "i"(OFF + 3 * RS)
      : "memory");
}

// Four pairs of transposed LDS reads of 16-bit data (gfx950
// ds_read_b64_tr_b16) at 32-bit, 8-byte aligned LDS byte addresses, complete
// on return.  Within each group of 16 lanes the lanes' 4-element (8-byte)
// rows form a 16 x 4 matrix R; lane j receives R[j/4 + 4k][j % 4], k = 0..3
// (measured layout).  Written
// as one asm block that waits for its own reads: with LDS DMA in flight the
// compiler, which cannot tell where the intrinsic reads, would otherwise wait
// for every DMA outstanding before each such read.
__device__ __forceinline__ void tr16_read4(u32x2 (&lo)[4], u32x2 (&hi)[4], const uint32_t (&alo)[4],
                                           const uint32_t (&ahi)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %12\n\t"
      "ds_read_b64_tr_b16 %5, %13\n\t"
      "ds_read_b64_tr_b16 %6, %14\n\t"
      "ds_read_b64_tr_b16 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(lo[0]), "=&v"(lo[1]), "=&v"(lo[2]), "=&v"(lo[3]), "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(hi[2]),
        "=&v"(hi[3])
      : "v"(alo[0]), "v"(alo[1]), "v"(alo[2]), "v"(alo[3]), "v"(ahi[0]), "v"(ahi[1]), "v"(ahi[2]), "v"(ahi[3])
      : "memory");
}
typedef SlotC<0> Slot0;
typedef SlotC<1> Slot1;

template <int N> struct TilePtrs { const uint16_t* k[N]; const uint16_t* v[N]; };

// Maximum over the four 16-lane groups of a wave, every lane getting its
// group position's result (lanes l, l ^ 16, l ^ 32, l ^ 48).  The row-swap
// permutes of the VALU (swap of 16-lane rows 0 <-> 1 and 2 <-> 3, then of the
// 32-lane halves) replace two LDS permute round trips per score tile.
// Every lane of the wave must be active.
__device__ __forceinline__ float max_over_groups(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// Addresses of one thread's N keys, my_key + KSTEP c (c < N), in the 64-key
// tile starting at key tb of the range [.., k_end): prefix rows [0, P_b),
// block rows [P_b, P_b + L_b), suffix rows after.  Every argument is a
// value, so the selects below stay selects between registers.  Past the last
// tile (live false) and for keys past k_end, the loads read `dummy` (q row 0
// of (b, h): cached, finite).  Every pointer includes the lane's 16-byte
// chunk `chunk` (< D elements, so a dummy read stays inside that q row).
template <int N, int KSTEP>
__device__ __forceinline__ TilePtrs<N> tile_ptrs(bool live, int tb, int k_end, int my_key, int P_b,
                                                 int L_b, const uint16_t* pk, const uint16_t* pv,
                                                 const uint16_t* bk, const uint16_t* bv,
                                                 const uint16_t* sk, const uint16_t* sv,
                                                 int64_t st0, int64_t st1, int64_t st2,
                                                 const uint16_t* dummy, int chunk) {
  TilePtrs<N> r;
  const int last = tb + kKT - 1;
  const int s_lo = tb < P_b ? 0 : (tb < P_b + L_b ? 1 : 2);
  const int s_hi = last < P_b ? 0 : (last < P_b + L_b ? 1 : 2);
  if (!live) {
#pragma unroll
    for (int c = 0; c < N; ++c) r.k[c] = r.v[c] = dummy + chunk;
    return r;
  }
  if (s_lo == s_hi && last < k_end) {
    // the whole tile lies in one segment (every tile but at most three of a
    // walk): segment, base row and stride are wave-uniform, and each lane
    // adds its own key's row
    const uint16_t* kseg = s_lo == 0 ? pk : (s_lo == 1 ? bk : sk);
    const uint16_t* vseg = s_lo == 0 ? pv : (s_lo == 1 ? bv : sv);
    const int64_t st = s_lo == 0 ? st0 : (s_lo == 1 ? st1 : st2);
    const int row0 = tb - (s_lo == 0 ? 0 : (s_lo == 1 ? P_b : P_b + L_b));
    // row strides are below 2^24 elements (checked on the host), so the
    // lane's part fits 32 bits; the rest stays wave-uniform
    const uint32_t lane_off = (uint32_t)my_key * (uint32_t)st + (uint32_t)chunk;
#pragma unroll
    for (int c = 0; c < N; ++c) {
      const int64_t base = (int64_t)(row0 + KSTEP * c) * st;
      r.k[c] = kseg + base + lane_off;
      r.v[c] = vseg + base + lane_off;
    }
    return r;
  }
#pragma unroll
  for (int c = 0; c < N; ++c) {
    const int t = tb + my_key + KSTEP * c;
    const bool in_p = t < P_b, in_b = t < P_b + L_b;
    const uint16_t* kseg = in_p ? pk : (in_b ? bk : sk);
    const uint16_t* vseg = in_p ? pv : (in_b ? bv : sv);
    const int64_t st = in_p ? st0 : (in_b ? st1 : st2);
    const int row = in_p ? t : (in_b ? t - P_b : t - P_b - L_b);
    const bool real = t < k_end;
    r.k[c] = (real ? kseg + row * st : dummy) + chunk;
    r.v[c] = (real ? vseg + row * st : dummy) + chunk;
  }
  return r;
}

// Element offset of row 0 of segment s for (b, h).
__device__ __forceinline__ int64_t seg_off(const KVSeg& s, int b, int h) {
  return (int64_t)b * s.sb + (int64_t)h * s.sh;
}
// Rows of segment s attended by sequence b.
__device__ __forceinline__ int seg_rows(const KVSeg& s, int b) {
  int n = s.len;
  if (s.len_b != nullptr) {
    const int r = s.len_b[b];
    n = r < 0 ? 0 : (r > s.len ? s.len : r);
  }
  return n;
}

// Each wave owns QPW 16-query tiles of the block.  KH = 2 (one query tile
// per wave, long key ranges): eight waves, waves w and w + 4 take the same
// queries and the first / second 32 keys of every staged tile, and merge once
// through LDS at the end.  At one wave per SIMD every step of the per-tile
// chain (fragment reads, score MFMAs, the softmax, the P.V MFMAs) is exposed;
// two independent waves per SIMD hide each other's latencies.  Short ranges
// (a few tiles per workgroup) are bound by each CU's loads instead, and there
// the extra merge only costs: they keep KH = 1.
template <int D, int QPW, int KH>
__global__ void __launch_bounds__(kAttThreads * KH, 2 / KH)
attend_kernel(AttendArgs a, float scale_log2, int kps, int nsplit, float* __restrict__ ws_o,
              float* __restrict__ ws_ml, Guard gd) {
  // K and V tile rows: D elements, unpadded; chunk c of row r at kv_pos(r, c)
  // (the register-staged version padded rows to D + 16 instead: a DMA
  // instruction writes 1 KiB contiguously, so padding is not available).
  constexpr int KST = D;
  constexpr int VST = D;
  constexpr int NKK = D / 32;      // k steps of the score product
  constexpr int NDT = D / 16;      // 16-wide output tiles
  constexpr int NT = kAttThreads * KH;
  constexpr int NCH = kKT * D / 8; // 16-byte chunks per K (or V) tile
  constexpr int CPT = NCH / NT;
  constexpr int KTW = 4 / KH;      // 16-key score blocks per wave and tile
  // LDS slots of K + V tiles (NSLOT - 1 tiles in flight while one is
  // multiplied): three for eight waves, two for four (2 x 32 KB keeps two
  // four-wave workgroups on a CU)
  constexpr int NSLOT = KH == 2 ? 3 : 2;
  // lazy reference moves for the long-range kernels (see compute_tile)
  constexpr bool LAZY = QPW > 1 || KH > 1;
  static_assert(CPT * NT == NCH, "tile chunks must divide evenly");
  static_assert(KH == 1 || QPW == 1, "key halves only with one query tile per wave");
  // NSLOT x (K tile, V tile); after the walk (KH = 2) the same bytes hold the
  // second-half waves' (O, max, sum) for the merge.
  constexpr int TILE_BYTES = (kKT * KST + kKT * VST) * 2 * NSLOT;
  constexpr int MERGE_BYTES = kAttWaves * NDT * kWave * 16 + kAttWaves * 16 * 8;
  static_assert(KH == 1 || MERGE_BYTES <= TILE_BYTES, "merge buffer must fit in the tiles");
  // One LDS object (ring, then the KH = 2 merge): with several, the compiler
  // would wait for every DMA in flight before each read of the ring.
  __shared__ __attribute__((aligned(1024))) uint16_t lds[TILE_BYTES / 2];
  constexpr int SLOT_ELEMS = kKT * KST + kKT * VST;   // one slot's K + V (elements)
  // chunk position of 16-byte chunk c of tile row r
  auto kv_pos = [](int r, int c) __attribute__((always_inline)) { return r * (D / 8) + (c ^ (r & (D / 8 - 1))); };

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int L = a.L;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wq = wave % kAttWaves;   // query tiles wq, wq + 4, ...
  const int kh = wave / kAttWaves;   // key half of every tile (KH = 2)
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  if (!guard_any(gd, b * L, b * L)) return;     // block loop: sequence b is complete

  const int P_b = seg_rows(a.seg[0], b);
  const int L_b = seg_rows(a.seg[1], b);
  const int S_b = seg_rows(a.seg[2], b);
  const int T_b = P_b + L_b + S_b;
  const int k_begin = split * kps;
  int k_end = k_begin + kps;
  k_end = k_end < T_b ? k_end : T_b;
  const int ntiles = k_end > k_begin ? (k_end - k_begin + kKT - 1) / kKT : 0;

  // segment bases for (b, h); a segment with no rows is never dereferenced
  const int64_t off0 = seg_off(a.seg[0], b, h), off1 = seg_off(a.seg[1], b, h),
                off2 = seg_off(a.seg[2], b, h);
  const uint16_t* const pk = a.seg[0].k + off0;
  const uint16_t* const pv = a.seg[0].v + off0;
  const uint16_t* const bk = a.seg[1].k + off1;
  const uint16_t* const bv = a.seg[1].v + off1;
  const uint16_t* const sk = a.seg[2].k + off2;
  const uint16_t* const sv = a.seg[2].v + off2;
  const int64_t st0 = a.seg[0].st, st1 = a.seg[1].st, st2 = a.seg[2].st;
  const float sl2 = scale_log2;
  // q row 0 of (b, h): finite input data that every dead load reads instead
  const uint16_t* q_bh = a.q + (int64_t)b * a.q_sb + (int64_t)h * a.q_sh;

  const int nqt = L / 16;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // ---- Q fragments (B operand of S^T = K Q^T): query l16 of tile qt, d group grp
  u32x4 qf[QPW][NKK];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int qt = wq + kAttWaves * j;
    const bool ok = qt < nqt;
    const uint16_t* qrow = q_bh + (int64_t)(ok ? qt * 16 + l16 : 0) * a.q_sl + grp * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qf[j][kk] = ok ? *reinterpret_cast<const u32x4*>(qrow + kk * 32) : zero4;
  }

  f32x4 o[QPW][NDT];
  float m_run[QPW], l_run[QPW];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    m_run[j] = -__builtin_inff();
    l_run[j] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[j][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- K/V tile loads: thread t brings 16-byte chunk t % CPR of keys
  // t / CPR + KPR c (c < CPT), so one wave instruction covers 64 / CPR whole
  // key rows (whole 128-byte lines).  (With register staging, whole-row loads
  // took the 128-query throughput batch from 163.7 to 159.5 us.)
  constexpr int CPR = D / 8;                    // 16-byte chunks per key row
  constexpr int KPR = NT / CPR;                 // key step between a thread's chunks
  static_assert(KPR % CPR == 0, "a thread's keys share one swizzle");
  const int my_key = tid / CPR;
  const int my_seg = tid % CPR;

  // Four-wave kernels: the lane's part of each transposed V read address
  // (row 4 grp + l16 / 4 of a 32-key step, chunk 2 dt + ((l16 & 3) >> 1)
  // swizzled by that row, half l16 & 1), LDS byte address of slot 0, step 0.
  uint32_t v_lane[NDT];
  {
    const int rp = 4 * grp + (l16 >> 2);
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      v_lane[dt] = lds_base + (uint32_t)(rp * D * 2) +
                   (uint32_t)(((2 * dt + ((l16 & 3) >> 1)) ^ (rp & (D / 8 - 1))) * 16) + (uint32_t)((l16 & 1) * 8);
  }
  // Four-wave kernels with one query tile per wave, head dimension 128: the
  // lane's part of the K fragment read addresses (row l16 of a 16-key block,
  // chunk 4 kk + grp swizzled by the row), LDS byte address of slot 0, key
  // block 0.  (Split kernels of the 64-query blocks: 14.76 -> 14.58 us per
  // call on the LLaDA-8B shape; with two query tiles per wave the compiler's
  // batches measured 0.8 us faster on the throughput batch.)
  constexpr bool KASM = KH == 1 && D == 128 && QPW == 1;
  uint32_t k_lane[4];
  {
    const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      k_lane[kk] = lds_base + (uint32_t)((l16 * (D / 8) + ((kk * 4 + grp) ^ (l16 & (D / 8 - 1)))) * 16);
  }
  auto compute_tile = [&](int tile, auto slot_c) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    const uint16_t* kl = lds + slot * SLOT_ELEMS;
    const uint16_t* vl = kl + kKT * KST;
    const int nvalid = k_end - (k_begin + tile * kKT);
    // query tile j of this wave exists (act[1] implies act[0]).  The
    // products run for every j (wave-uniform, no exec masking between the
    // MFMAs): a missing tile has zero Q fragments, finite scores and
    // probabilities, and is never stored; only its softmax is skipped.
    bool act[QPW];
#pragma unroll
    for (int j = 0; j < QPW; ++j) act[j] = wq + kAttWaves * j < nqt;
    if (!act[0]) return;
    // S^T tiles: keys 16*kt + 4*grp + r (rows), query l16 (column), for this
    // wave's score blocks kt = KTW kh + u, u < KTW.  Each K fragment is read
    // once and multiplied into every query tile of the wave.
    f32x4 st[QPW][KTW];
#pragma unroll
    for (int j = 0; j < QPW; ++j)
#pragma unroll
      for (int u = 0; u < KTW; ++u) st[j][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 kf[KASM ? 16 : 1];
    if constexpr (KASM) k_read16<slot * SLOT_ELEMS * 2, 16 * D * 2>(kf, k_lane);
#pragma unroll
    for (int u = 0; u < KTW; ++u) {
      const int kt = KTW * kh + u;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        u32x4 av;
        if constexpr (KASM)
          av = kf[4 * u + kk];
        else
          av = *reinterpret_cast<const u32x4*>(&kl[kv_pos(kt * 16 + l16, kk * 4 + grp) * 8]);
#pragma unroll
        for (int j = 0; j < QPW; ++j)
          st[j][u] = mfma16x16x32(as_bf16x8(av), as_bf16x8(qf[j][kk]), st[j][u]);
      }
    }
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      if (!act[j]) continue;
      // raw scores; the scale (> 0) is applied once, inside the exponent's fma
      if (nvalid < kKT) {   // the range's last, partial tile: keys past it score -inf
#pragma unroll
        for (int u = 0; u < KTW; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((KTW * kh + u) * 16 + grp * 4 + r >= nvalid) st[j][u][r] = -__builtin_inff();
      }
      float tmax = -__builtin_inff();
#pragma unroll
      for (int u = 0; u < KTW; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, st[j][u][r]);
      tmax = max_over_groups(tmax);
      // The exponents' reference m_run (base-2 scaled domain).  LAZY: it
      // moves only when a score passes it by more than kRescaleSlack; below
      // that every p = 2^(s - m_run) <= 2^kRescaleSlack is exact in fp32 and
      // bf16, and O and l share the reference, so O / l is unchanged, and
      // when no query of the wave moves the rescale of O and l is skipped
      // (after the first tiles it almost never runs).  Measured: throughput
      // batch 160.6 -> 155.3 us, long-context batch 128.0 -> 125.2 us; on
      // the two-tile splits of the 64-query blocks the test costs more than
      // it saves (+0.2 us), so there the reference follows the max.
      // A key half can lie wholly past the range (KH = 2, the last tile);
      // while the reference is still -inf, exponents are taken against 0 so
      // every p and alpha is 0 rather than NaN.
      float m_use;
      if constexpr (LAZY) {
        const float m_cand = fmaxf(m_run[j], tmax * sl2);
        const bool move = m_cand > m_run[j] + kRescaleSlack;
        const float m_new = move ? m_cand : m_run[j];
        m_use = (KH > 1 && m_new == -__builtin_inff()) ? 0.f : m_new;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
          const float alpha = fast_exp2(m_run[j] - m_use);   // 1 where the reference stays
          l_run[j] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[j][dt] *= alpha;
        }
        m_run[j] = m_new;
      }
      float alpha_now = 1.f;
      if constexpr (!LAZY) {
        const float m_new = fmaxf(m_run[j], tmax * sl2);
        m_use = (KH > 1 && m_new == -__builtin_inff()) ? 0.f : m_new;
        alpha_now = fast_exp2(m_run[j] - m_use);
        m_run[j] = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < KTW; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(__builtin_fmaf(st[j][u][r], sl2, -m_use));
          st[j][u][r] = p;
          psum += p;
        }
      if constexpr (LAZY) {
        l_run[j] += psum;
      } else {
        l_run[j] = l_run[j] * alpha_now + psum;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[j][dt] *= alpha_now;
      }
    }
    // O^T += V^T P^T over this wave's 32-key steps c; the step's lane group
    // grp holds keys {32c + 4grp + 0..3} and {32c + 16 + 4grp + 0..3} in both
    // operands.  Each V fragment is read once for every query tile.
#pragma unroll
    for (int cc = 0; cc < 2 / KH; ++cc) {
      const int c = (2 / KH) * kh + cc;
      bf16x8 pf[QPW];
#pragma unroll
      for (int j = 0; j < QPW; ++j) {
        const u32x4 pw = {pack_bf16x2(st[j][2 * cc][0], st[j][2 * cc][1]),
                          pack_bf16x2(st[j][2 * cc][2], st[j][2 * cc][3]),
                          pack_bf16x2(st[j][2 * cc + 1][0], st[j][2 * cc + 1][1]),
                          pack_bf16x2(st[j][2 * cc + 1][2], st[j][2 * cc + 1][3])};
        pf[j] = as_bf16x8(pw);
      }
      // A operand V^T: lane (dim 16 dt + l16, grp) needs keys 32c + 4grp +
      // 0..3 and 32c + 16 + 4grp + 0..3 of its dimension.  In each 16-lane
      // group a transposed read hands lane j element j % 4 of the 4-element
      // rows that lanes j / 4 + 4k point at, k = 0..3, so lane s points at
      // key 32c + 4grp + s / 4 (+ 16), dims 16 dt + 4 (s % 4) ...
      // This lane reads row vr0 (and vr0 + 16), chunk 2 dt + ((l16 & 3) >> 1),
      // half (l16 & 1) of it.  Four waves: every part of the address but the
      // lane's (v_lane, computed once) is a compile-time offset.
      static_assert(NDT % 4 == 0, "transposed reads go four dims tiles at a time");
#pragma unroll
      for (int d4 = 0; d4 < NDT; d4 += 4) {
        u32x2 lo4[4], hi4[4];
        if constexpr (KH == 1) {
          constexpr int VOFF = (slot * SLOT_ELEMS + kKT * KST) * 2;   // V of the slot, step 0
          const uint32_t a4[4] = {v_lane[d4], v_lane[d4 + 1], v_lane[d4 + 2], v_lane[d4 + 3]};
          if (cc == 0)
            tr16_read4_imm<VOFF, 16 * D * 2>(lo4, hi4, a4);
          else
            tr16_read4_imm<VOFF + 32 * D * 2, 16 * D * 2>(lo4, hi4, a4);
        } else {
          const int vr0 = 32 * c + 4 * grp + (l16 >> 2);
          const uint32_t vl_addr = (uint32_t)(uintptr_t)(lds_ptr_t)vl;
          const int within = (l16 & 1) * 4;
          uint32_t alo[4], ahi[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ch = 2 * (d4 + q) + ((l16 & 3) >> 1);
            alo[q] = vl_addr + (uint32_t)(kv_pos(vr0, ch) * 8 + within) * 2u;
            ahi[q] = vl_addr + (uint32_t)(kv_pos(vr0 + 16, ch) * 8 + within) * 2u;
          }
          tr16_read4(lo4, hi4, alo, ahi);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 va = {lo4[q][0], lo4[q][1], hi4[q][0], hi4[q][1]};
#pragma unroll
          for (int j = 0; j < QPW; ++j)
            o[j][d4 + q] = mfma16x16x32(as_bf16x8(va), pf[j], o[j][d4 + q]);
        }
      }
    }
  };
  // Thread t's chunk c lands at LDS chunk (64 w + NT c) + lane of the slot's
  // K (or V) image -- key my_key + KPR c, position my_seg -- so it fetches
  // chunk my_seg ^ (key % CPR) of its key (KPR is a multiple of CPR: the
  // key's swizzle is my_key % CPR for every c).  The addresses come from
  // tile_ptrs, computed outside the lambdas (from a lambda, a select between
  // two captured values becomes a load from a selected address, and every
  // captured variable of the kernel then lives in scratch memory).
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int dma_chunk = (my_seg ^ (my_key & (CPR - 1))) * 8;
  auto dma_tile = [&](auto slot_c, const TilePtrs<CPT>& tp) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    uint16_t* ks = lds + slot * SLOT_ELEMS;
    uint16_t* vs = ks + kKT * KST;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int blk = (wave_u * kWave + c * NT) * 8;   // elements
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(tp.k[c]), (lds_ptr_t)(ks + blk), 16, 0,
                                       kDmaStream);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(tp.v[c]), (lds_ptr_t)(vs + blk), 16, 0,
                                       kDmaStream);
    }
  };
  // One tile: wait for its loads (NSLOT - 2 later tiles may still be in
  // flight), one barrier (the tile is visible; the slot read at tile - 1 is
  // free), refill that slot with tile + NSLOT - 1, multiply.  Barriers are
  // uniform over the workgroup: every thread runs the same number of trips.
  auto tile_step = [&](int tile, auto slot_c, const TilePtrs<CPT>& next) __attribute__((always_inline)) {
    constexpr int slot = decltype(slot_c)::value;
    wait_vm<(NSLOT - 2) * 2 * CPT>();
    stage_barrier();
    dma_tile(SlotC<(slot + NSLOT - 1) % NSLOT>{}, next);
    if (tile < ntiles) compute_tile(tile, slot_c);
  };
  auto ptrs = [&](int tile) __attribute__((always_inline)) {
    return tile_ptrs<CPT, KPR>(tile < ntiles, k_begin + tile * kKT, k_end, my_key, P_b, L_b,
                                pk, pv, bk, bv, sk, sv, st0, st1, st2, q_bh, dma_chunk);
  };

  if (ntiles > 0) {
    dma_tile(Slot0{}, ptrs(0));
    if constexpr (NSLOT == 3) dma_tile(Slot1{}, ptrs(1));
    for (int tile = 0; tile < ntiles; tile += NSLOT) {
      tile_step(tile, Slot0{}, ptrs(tile + NSLOT - 1));
      tile_step(tile + 1, Slot1{}, ptrs(tile + NSLOT));
      if constexpr (NSLOT == 3) tile_step(tile + 2, SlotC<2>{}, ptrs(tile + NSLOT + 1));
    }
    wait_vm<0>();   // no DMA may land in LDS after the walk (merge, exit)
  }

  // running sums over the lane groups (each lane summed its own keys)
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    l_run[j] += __shfl_xor(l_run[j], 16, kWave);
    l_run[j] += __shfl_xor(l_run[j], 32, kWave);
  }
  // ---- KH = 2: the second-half waves hand (O, max, sum) to their partner
  // through LDS (lane-major, so both sides are conflict-free); the partner
  // rescales both to the larger max and adds.
  if (KH > 1) {
    __syncthreads();   // every wave is done reading the tiles
    f32x4* mo = reinterpret_cast<f32x4*>(lds);                             // [wq][dt][lane]
    f32x2* mml = reinterpret_cast<f32x2*>(mo + kAttWaves * NDT * kWave);   // [wq][query]
    const bool active = wq < nqt;
    if (kh == 1 && active) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) mo[(wq * NDT + dt) * kWave + lane] = o[0][dt];
      if (grp == 0) mml[wq * 16 + l16] = f32x2{m_run[0], l_run[0]};
    }
    __syncthreads();
    if (kh == 0 && active) {
      const f32x2 ml = mml[wq * 16 + l16];
      const float M = fmaxf(m_run[0], ml[0]);
      const float Mu = M == -__builtin_inff() ? 0.f : M;
      const float a0 = fast_exp2(m_run[0] - Mu), a1 = fast_exp2(ml[0] - Mu);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[0][dt] = o[0][dt] * a0 + mo[(wq * NDT + dt) * kWave + lane] * a1;
      m_run[0] = M;
      l_run[0] = l_run[0] * a0 + ml[1] * a1;
    }
  }

  // ---- output: O^T accumulator lane holds d = 16dt + 4grp + r of query l16
  // (the lambdas below capture locals only: a captured kernel argument would
  // have its address taken and live in scratch memory)
  uint16_t* const o_bh = a.out + (int64_t)b * a.o_sb + (int64_t)h * a.o_sh + grp * 4;
  const int64_t o_sl = a.o_sl;
  auto write_out = [&](int query, const f32x4 (&acc)[NDT], float lsum) __attribute__((always_inline)) {
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;   // a row with no key: zeros
    uint16_t* orow = o_bh + (int64_t)query * o_sl;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x2 v = {pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv),
                       pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + dt * 16) = v;
    }
  };
  if (kh != 0) return;
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int qt = wq + kAttWaves * j;
    if (qt >= nqt) continue;
    const int query = qt * 16 + l16;
    if (nsplit == 1) {
      write_out(query, o[j], l_run[j]);
    } else {
      // split partials, rows (b, h, split, query), streaming stores (the
      // merge kernel reads them once from HBM).  O goes out as fp16 scaled by
      // 2^-e, e the exponent of the row's largest |O| (frexp: the largest
      // scaled value lies in [0.5, 1)), so nothing can overflow and every
      // element keeps 11 significant bits relative to its row's maximum;
      // the record {max, sum, 2^e, 0} carries the scale back.
      const size_t prow = (((size_t)b * a.H + h) * nsplit + split) * (size_t)L + query;
      float amax = 0.f;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) amax = fmaxf(amax, fabsf(o[j][dt][r]));
      amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
      amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
      const int e = __builtin_amdgcn_frexp_expf(amax);     // 0 for amax = 0
      const float sc = __builtin_ldexpf(1.f, -e);
      uint16_t* po = reinterpret_cast<uint16_t*>(ws_o) + prow * D + grp * 4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const u32x2 hv = {pack_f16x2(o[j][dt][0] * sc, o[j][dt][1] * sc),
                          pack_f16x2(o[j][dt][2] * sc, o[j][dt][3] * sc)};
        __builtin_nontemporal_store(hv, reinterpret_cast<u32x2*>(po + dt * 16));
      }
      if (grp == 0)
        __builtin_nontemporal_store(f32x4{m_run[j], l_run[j], __builtin_ldexpf(1.f, e), 0.f},
                                    reinterpret_cast<f32x4*>(ws_ml + 4 * prow));
    }
  }
}

// Merge the splits of one (b, h): O = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M)
// (O_s from its fp16 copy times its record's scale).
// One thread per 4 output dims.  Splits are taken NS at a time; within a
// batch every load is issued before any is used (one memory round trip per
// batch), and batches are merged online in split order.  A row with no key
// in any split (every m_s = -inf) is written as zeros.
template <int D, int NS>
__global__ void __launch_bounds__(kCombineThreads)
attend_combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml, int H,
                      int L, int nsplit, uint16_t* __restrict__ out, int64_t o_sb, int64_t o_sl,
                      int64_t o_sh, int total, Guard gd) {
  const int idx = blockIdx.x * kCombineThreads + threadIdx.x;
  if (idx >= total) return;
  constexpr int G4 = D / 4;
  const int d4 = idx % G4;
  const int rest = idx / G4;
  const int query = rest % L;
  const int bhi = rest / L;
  const int b = bhi / H;
  const int h = bhi % H;
  if (!guard_any(gd, b * L, b * L)) return;
  const size_t base = (size_t)bhi * nsplit * L + query;
  float M = -__builtin_inff();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lsum = 0.f;
  for (int s0 = 0; s0 < nsplit; s0 += NS) {
    float ms[NS], ls[NS], sc[NS];
    u32x2 hs[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const bool ok = s0 + u < nsplit;
      const size_t prow = base + (size_t)(ok ? s0 + u : 0) * L;
      const f32x4 rec = *reinterpret_cast<const f32x4*>(ws_ml + 4 * prow);
      ms[u] = ok ? rec[0] : -__builtin_inff();
      ls[u] = rec[1];
      sc[u] = rec[2];
      hs[u] = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(ws_o) + prow * D + d4 * 4);
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < NS; ++u) Mb = fmaxf(Mb, ms[u]);
    // 0 while M is -inf; 1 while no split so far had a key of this row,
    // where exp2(-inf - -inf) would be NaN
    const float al = Mb == -__builtin_inff() ? 1.f : fast_exp2(M - Mb);
    acc *= al;
    lsum *= al;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (ms[u] == -__builtin_inff()) continue;  // split with no key of this row
      const float w = fast_exp2(ms[u] - Mb);
      const f32x2 lo = unpack_f16x2(hs[u][0]), hi = unpack_f16x2(hs[u][1]);
      acc += f32x4{lo[0], lo[1], hi[0], hi[1]} * (w * sc[u]);
      lsum += ls[u] * w;
    }
    M = Mb;
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  const u32x2 v = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<u32x2*>(out + (int64_t)b * o_sb + (int64_t)query * o_sl + (int64_t)h * o_sh +
                            d4 * 4) = v;
}

template <int D, int QPW>
hipError_t launch_dq(const AttendArgs& a, float scale_log2, float* ws_o, float* ws_ml,
                     const AttendPlan& p, const Guard& gd, hipStream_t stream) {
  constexpr int KH2 = QPW == 1 ? 2 : 1;
  const dim3 grid(p.nsplit, a.H, a.B);
  hipError_t e;
  if (KH2 == 2 && p.kps >= kLongRange)
    e = launch_kernel(attend_kernel<D, QPW, KH2>, grid, dim3(2 * kAttThreads), 0, stream, a,
                      scale_log2, p.kps, p.nsplit, ws_o, ws_ml, gd);
  else
    e = launch_kernel(attend_kernel<D, QPW, 1>, grid, dim3(kAttThreads), 0, stream, a,
                      scale_log2, p.kps, p.nsplit, ws_o, ws_ml, gd);
  if (e != hipSuccess || p.nsplit == 1) return e;
  const int total = a.B * a.H * a.L * (D / 4);
  const dim3 cgrid((total + kCombineThreads - 1) / kCombineThreads), block(kCombineThreads);
  if (p.nsplit <= 8)
    return launch_kernel(attend_combine_kernel<D, 8>, cgrid, block, 0, stream, (const float*)ws_o,
                         (const float*)ws_ml, a.H, a.L, p.nsplit, a.out, a.o_sb, a.o_sl, a.o_sh,
                         total, gd);
  return launch_kernel(attend_combine_kernel<D, 16>, cgrid, block, 0, stream, (const float*)ws_o,
                       (const float*)ws_ml, a.H, a.L, p.nsplit, a.out, a.o_sb, a.o_sl, a.o_sh,
                       total, gd);
}

inline size_t round256(size_t n) { return (n + 255) / 256 * 256; }

}  // namespace

AttendPlan attend_plan(int B, int H, int L, int D, int T_cap) {
  AttendPlan p;
  p.T_cap = T_cap;
  const int ntile = (T_cap + kKT - 1) / kKT;
  const long bhn = (long)B * H;
  int want = bhn > 0 ? (int)((kTargetWGs + bhn - 1) / bhn) : 1;
  if (want < 1) want = 1;
  int tps = ntile > 0 ? (ntile + want - 1) / want : 1;  // tiles per split
  p.kps = tps * kKT;
  p.nsplit = T_cap > 0 ? (T_cap + p.kps - 1) / p.kps : 1;
  if (p.nsplit > 1) {
    // fp16 partial outputs, then one 16-byte {max, sum, scale, 0} record per row
    const size_t rows = (size_t)bhn * p.nsplit * L;
    p.ml_offset = round256(rows * D * sizeof(uint16_t));
    p.ws_bytes = p.ml_offset + rows * 4 * sizeof(float);
  } else {
    p.ml_offset = p.ws_bytes = 0;
  }
  return p;
}

AttendArgs dense_attend_args(const void* q, const void* kp, const void* vp, const void* kb,
                             const void* vb, const void* ks, const void* vs,
                             const int32_t* prefix_len, int B, int H, int L, int D, int P_cap,
                             int S, int S_cap, float scale, void* out) {
  typedef const uint16_t* cp;
  AttendArgs a;
  a.B = B; a.H = H; a.L = L; a.D = D;
  a.q = (cp)q;
  a.q_sh = D; a.q_sl = (int64_t)H * D; a.q_sb = (int64_t)L * H * D;
  a.out = static_cast<uint16_t*>(out);
  a.o_sh = D; a.o_sl = (int64_t)H * D; a.o_sb = (int64_t)L * H * D;
  a.seg[0] = KVSeg{P_cap > 0 ? (cp)kp : nullptr, P_cap > 0 ? (cp)vp : nullptr,
                   (int64_t)H * P_cap * D, (int64_t)P_cap * D, D, P_cap, prefix_len};
  a.seg[1] = KVSeg{(cp)kb, (cp)vb, (int64_t)H * L * D, (int64_t)L * D, D, L, nullptr};
  a.seg[2] = KVSeg{S > 0 ? (cp)ks : nullptr, S > 0 ? (cp)vs : nullptr,
                   (int64_t)H * S_cap * D, (int64_t)S_cap * D, D, S, nullptr};
  a.scale = scale;
  return a;
}

hipError_t launch_attend(const AttendArgs& a, void* ws, const AttendPlan& p, const Guard& gd,
                         hipStream_t stream) {
  const float scale = a.scale == 0.f ? 1.0f / sqrtf((float)a.D) : a.scale;
  const float scale_log2 = scale * kLog2e;
  float* ws_o = static_cast<float*>(ws);
  float* ws_ml = p.nsplit > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.ml_offset)
                              : nullptr;
  const bool two = a.L > 16 * kAttWaves;
  if (a.D == 64)
    return two ? launch_dq<64, 2>(a, scale_log2, ws_o, ws_ml, p, gd, stream)
               : launch_dq<64, 1>(a, scale_log2, ws_o, ws_ml, p, gd, stream);
  return two ? launch_dq<128, 2>(a, scale_log2, ws_o, ws_ml, p, gd, stream)
             : launch_dq<128, 1>(a, scale_log2, ws_o, ws_ml, p, gd, stream);
}

}  // namespace dblk
