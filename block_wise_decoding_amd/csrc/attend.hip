// Non-causal attention of the active block over the dual KV cache.
//
// dInfer's decoder runs with KVCacheFactory('dual') (README, usage section):
// keys/values of the prefix before the block and of the suffix after it are
// cached, only the block's own are fresh, and -- diffusion LMs attend
// bidirectionally (topic page, variable-size-block and Streaming-dLLM
// abstracts) -- every block query attends to all prefix[0:P_b] + L + S keys.
//
// Design (gfx950, wave64, 16x16x32 bf16 MFMA, fp32 accumulation):
//  * Grid (split, head, batch); one 4-wave workgroup walks 64-key tiles of
//    its key range with an online (running max / running sum) softmax in
//    base 2.  Each wave owns one or two 16-query tiles of the block.
//  * Scores are computed transposed, S^T = K Q^T (A = K rows straight from
//    LDS, B = Q held in registers for the whole walk).  The S^T accumulator
//    then already has the layout of the B operand of O^T = V^T P^T, so the
//    probabilities are packed to bf16 in place, with no shuffle.
//  * K and V tiles are loaded from HBM with 16-byte loads (16 keys x 64
//    contiguous bytes per wave instruction) into two register slots, so the
//    next tile is in flight while the current one is staged and multiplied,
//    then written to LDS: K row-major
//    (padded rows, conflict-free 16-byte reads), V transposed to [D][keys]
//    so each lane's 8 keys of one dimension are two 8-byte LDS reads.
//  * Keys are numbered 0..T_b-1 over prefix ++ block ++ suffix; each loaded
//    key resolves its segment, so ragged prefixes and tiles that straddle a
//    segment boundary need no special case.  Keys past the range score -inf.
//  * With one split the kernel normalises and writes bf16 output; otherwise it
//    writes fp32 (unnormalised O, running max, running sum) partials and a
//    second kernel merges the splits.
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
attend_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp,
              const uint16_t* __restrict__ vp, const uint16_t* __restrict__ kb,
              const uint16_t* __restrict__ vb, const uint16_t* __restrict__ ks,
              const uint16_t* __restrict__ vs, const int32_t* __restrict__ prefix_len, int H,
              int L, int P_cap, int S, int S_cap, float scale_log2, int kps, int nsplit,
              uint16_t* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
              Guard gd) {
  // K tile row stride (elements): rows 32 bytes apart in bank space.  A
  // 16-byte pad (D + 8) lost ~3% of the throughput batch's attention time to
  // LDS bank conflicts against this one; wider pads (D + 24, D + 40) gain
  // nothing more.
  constexpr int KST = D + 16;
  constexpr int VST = kKT + 4;     // V^T tile row stride (elements)
  constexpr int NKK = D / 32;      // k steps of the score product
  constexpr int NDT = D / 16;      // 16-wide output tiles
  constexpr int NT = kAttThreads * KH;
  constexpr int NCH = kKT * D / 8; // 16-byte chunks per K (or V) tile
  constexpr int CPT = NCH / NT;
  constexpr int KTW = 4 / KH;      // 16-key score blocks per wave and tile
  static_assert(CPT * NT == NCH, "tile chunks must divide evenly");
  static_assert(KH == 1 || QPW == 1, "key halves only with one query tile per wave");
  // K tile, then V^T tile; after the walk (KH = 2) the same bytes hold the
  // second-half waves' (O, max, sum) for the merge.
  constexpr int TILE_BYTES = (kKT * KST + D * VST) * 2;
  constexpr int MERGE_BYTES = kAttWaves * NDT * kWave * 16 + kAttWaves * 16 * 8;
  static_assert(KH == 1 || MERGE_BYTES <= TILE_BYTES, "merge buffer must fit in the tiles");
  __shared__ __attribute__((aligned(16))) uint16_t lds[TILE_BYTES / 2];
  uint16_t* k_lds = lds;
  uint16_t* vt_lds = lds + kKT * KST;

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wq = wave % kAttWaves;   // query tiles wq, wq + 4, ...
  const int kh = wave / kAttWaves;   // key half of every tile (KH = 2)
  const int l16 = lane & 15;
  const int grp = lane >> 4;
  if (!guard_any(gd, b * L, b * L)) return;     // block loop: sequence b is complete

  int P_b = P_cap;
  if (prefix_len != nullptr) {
    P_b = prefix_len[b];
    P_b = P_b < 0 ? 0 : (P_b > P_cap ? P_cap : P_b);
  }
  const int T_b = P_b + L + S;
  const int k_begin = split * kps;
  int k_end = k_begin + kps;
  k_end = k_end < T_b ? k_end : T_b;
  const int ntiles = k_end > k_begin ? (k_end - k_begin + kKT - 1) / kKT : 0;

  const size_t bh = (size_t)b * H + h;
  const uint16_t* kp_bh = kp ? kp + bh * (size_t)P_cap * D : nullptr;
  const uint16_t* vp_bh = vp ? vp + bh * (size_t)P_cap * D : nullptr;
  const uint16_t* kb_bh = kb + bh * (size_t)L * D;
  const uint16_t* vb_bh = vb + bh * (size_t)L * D;
  const uint16_t* ks_bh = ks ? ks + bh * (size_t)S_cap * D : nullptr;
  const uint16_t* vs_bh = vs ? vs + bh * (size_t)S_cap * D : nullptr;

  const int nqt = L / 16;
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // ---- Q fragments (B operand of S^T = K Q^T): query l16 of tile qt, d group grp
  u32x4 qf[QPW][NKK];
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int qt = wq + kAttWaves * j;
    const bool ok = qt < nqt;
    const uint16_t* qrow = q + (((size_t)b * L + (ok ? qt * 16 + l16 : 0)) * H + h) * D + grp * 8;
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

  // ---- K/V tile staging.  Thread t loads key (t & 15) | (((t >> 6) & 3) << 4)
  // of the tile and dims 8 * (s + 4 KH c), c < CPT, with s = ((t >> 4) & 3) +
  // 4 (t >> 8): one wave instruction reads 16 keys x 64 contiguous bytes, and
  // all of a thread's chunks belong to one key, so its segment is resolved
  // once per tile.
  const int my_key = (tid & 15) | (((tid >> 6) & 3) << 4);
  const int my_seg = ((tid >> 4) & 3) + 4 * (tid >> 8);
  u32x4 kr[2][CPT], vr[2][CPT];

  auto load_tile = [&](int slot, int tile) {
    // Past the last tile the loads still issue (so every trip has the same
    // load count and the compiler's wait counts stay exact) but all read one
    // fixed 16-byte chunk of the block segment, which stays cached.  A key
    // past the range end in the last, partial tile reads the block's first
    // row: finite input data whose score is then set to -inf, so its p is
    // exactly 0 and 0 * v adds nothing.
    const bool live = tile < ntiles;
    const int t = k_begin + tile * kKT + my_key;
    const uint16_t* kptr = kb_bh;
    const uint16_t* vptr = vb_bh;
    if (live && t < k_end) {
      if (t < P_b) {
        kptr = kp_bh + (size_t)t * D;
        vptr = vp_bh + (size_t)t * D;
      } else if (t < P_b + L) {
        kptr = kb_bh + (size_t)(t - P_b) * D;
        vptr = vb_bh + (size_t)(t - P_b) * D;
      } else {
        kptr = ks_bh + (size_t)(t - P_b - L) * D;
        vptr = vs_bh + (size_t)(t - P_b - L) * D;
      }
    }
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int off = live ? (my_seg + 4 * KH * c) * 8 : 0;
      kr[slot][c] = *reinterpret_cast<const u32x4*>(kptr + off);
      vr[slot][c] = *reinterpret_cast<const u32x4*>(vptr + off);
    }
  };
  // V^T is written as 32-bit words holding one dimension of two adjacent keys:
  // the lanes of keys 2p and 2p+1 (lane ^ 1) swap half of their 8 dimensions,
  // then the even-key lane writes dims d0..d0+3 and the odd-key lane dims
  // d0+4..d0+7, each word (key 2p, key 2p+1).  The 64 lanes of every store
  // instruction hit 64 distinct banks.
  const bool key_even = (my_key & 1) == 0;
  auto store_tile = [&](int slot) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int d0 = (my_seg + 4 * KH * c) * 8;
      *reinterpret_cast<u32x4*>(&k_lds[my_key * KST + d0]) = kr[slot][c];
      const u32x4 v = vr[slot][c];
      const uint32_t r0 = __shfl_xor(key_even ? v[2] : v[0], 1, kWave);
      const uint32_t r1 = __shfl_xor(key_even ? v[3] : v[1], 1, kWave);
      const uint32_t a0 = key_even ? v[0] : r0, a1 = key_even ? v[1] : r1;   // even key
      const uint32_t b0 = key_even ? r0 : v[2], b1 = key_even ? r1 : v[3];   // odd key
      uint32_t* col = reinterpret_cast<uint32_t*>(&vt_lds[(d0 + (key_even ? 0 : 4)) * VST + (my_key & ~1)]);
      col[0 * VST / 2] = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
      col[1 * VST / 2] = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
      col[2 * VST / 2] = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
      col[3 * VST / 2] = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
    }
  };

  auto compute_tile = [&](int tile) {
    const int nvalid = k_end - (k_begin + tile * kKT);
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      if (wq + kAttWaves * j >= nqt) continue;
      // S^T tile: keys 16*kt + 4*grp + r (rows), query l16 (column), for this
      // wave's score blocks kt = KTW kh + u, u < KTW
      f32x4 st[KTW];
#pragma unroll
      for (int u = 0; u < KTW; ++u) {
        const int kt = KTW * kh + u;
        st[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&k_lds[(kt * 16 + l16) * KST + kk * 32 + grp * 8]);
          st[u] = mfma16x16x32(as_bf16x8(a), as_bf16x8(qf[j][kk]), st[u]);
        }
      }
      // raw scores; the scale (> 0) is applied once, inside the exponent's fma
      if (nvalid < kKT) {   // the range's last, partial tile: keys past it score -inf
#pragma unroll
        for (int u = 0; u < KTW; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((KTW * kh + u) * 16 + grp * 4 + r >= nvalid) st[u][r] = -__builtin_inff();
      }
      float tmax = -__builtin_inff();
#pragma unroll
      for (int u = 0; u < KTW; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, st[u][r]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      const float m_new = fmaxf(m_run[j], tmax * scale_log2);   // base-2 scaled domain
      // A key half can lie wholly past the range (KH = 2, the last tile);
      // while the running max is still -inf, exponents are taken against 0 so
      // every p and alpha is 0 rather than NaN.
      const float m_use = (KH > 1 && m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[j] - m_use);
      m_run[j] = m_new;
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < KTW; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float p = fast_exp2(__builtin_fmaf(st[u][r], scale_log2, -m_use));
          st[u][r] = p;
          psum += p;
        }
      l_run[j] = l_run[j] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[j][dt] *= alpha;
      // O^T += V^T P^T over this wave's 32-key steps c; the step's lane group
      // grp holds keys {32c + 4grp + 0..3} and {32c + 16 + 4grp + 0..3} in
      // both operands
#pragma unroll
      for (int cc = 0; cc < 2 / KH; ++cc) {
        const int c = (2 / KH) * kh + cc;
        const u32x4 pw = {pack_bf16x2(st[2 * cc][0], st[2 * cc][1]),
                          pack_bf16x2(st[2 * cc][2], st[2 * cc][3]),
                          pack_bf16x2(st[2 * cc + 1][0], st[2 * cc + 1][1]),
                          pack_bf16x2(st[2 * cc + 1][2], st[2 * cc + 1][3])};
        const bf16x8 pf = as_bf16x8(pw);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint16_t* vrow = &vt_lds[(dt * 16 + l16) * VST + 32 * c + 4 * grp];
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
          const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
          o[j][dt] = mfma16x16x32(as_bf16x8(va), pf, o[j][dt]);
        }
      }
    }
  };
  // One tile: stage slot `slot` (waits only for this tile's loads), refill
  // the slot with tile + 2, multiply.  Barriers are uniform over the
  // workgroup: every thread runs the same number of trips.
  auto tile_step = [&](int tile, int slot) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile(slot);
    __syncthreads();
    load_tile(slot, tile + 2);
    if (tile < ntiles) compute_tile(tile);
  };

  if (ntiles > 0) {
    load_tile(0, 0);
    load_tile(1, 1);
    for (int tile = 0; tile < ntiles; tile += 2) {
      tile_step(tile, 0);
      tile_step(tile + 1, 1);
    }
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
    if (kh == 1) return;
    if (active) {
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

  // ---- write: O^T accumulator lane holds d = 16dt + 4grp + r of query l16
#pragma unroll
  for (int j = 0; j < QPW; ++j) {
    const int qt = wq + kAttWaves * j;
    if (qt >= nqt) continue;
    const float lt = l_run[j];
    const int query = qt * 16 + l16;
    if (nsplit == 1) {
      const float inv = 1.0f / lt;
      uint16_t* orow = out + (((size_t)b * L + query) * H + h) * D + grp * 4;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const u32x2 v = {pack_bf16x2(o[j][dt][0] * inv, o[j][dt][1] * inv),
                         pack_bf16x2(o[j][dt][2] * inv, o[j][dt][3] * inv)};
        *reinterpret_cast<u32x2*>(orow + dt * 16) = v;
      }
    } else {
      const size_t prow = (bh * nsplit + split) * (size_t)L + query;
      float* po = ws_o + prow * D + grp * 4;
      // streaming stores: the merge kernel reads these once, from HBM
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        __builtin_nontemporal_store(o[j][dt], reinterpret_cast<f32x4*>(po + dt * 16));
      if (grp == 0)
        __builtin_nontemporal_store(f32x2{m_run[j], lt}, reinterpret_cast<f32x2*>(ws_ml + 2 * prow));
    }
  }
}

// Merge the splits of one (b, h): O = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M).
// One thread per 4 output dims.  Splits are taken NS at a time; within a
// batch every load is issued before any is used (one memory round trip per
// batch), and batches are merged online in split order.
template <int D, int NS>
__global__ void __launch_bounds__(kCombineThreads)
attend_combine_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml, int H,
                      int L, int nsplit, uint16_t* __restrict__ out, int total, Guard gd) {
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
    float ms[NS], ls[NS];
    f32x4 os[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const bool ok = s0 + u < nsplit;
      const size_t prow = base + (size_t)(ok ? s0 + u : 0) * L;
      const float2 ml = *reinterpret_cast<const float2*>(ws_ml + 2 * prow);
      ms[u] = ok ? ml.x : -__builtin_inff();
      ls[u] = ml.y;
      os[u] = *reinterpret_cast<const f32x4*>(ws_o + prow * D + d4 * 4);
    }
    float Mb = M;
#pragma unroll
    for (int u = 0; u < NS; ++u) Mb = fmaxf(Mb, ms[u]);
    const float a = fast_exp2(M - Mb);       // 0 while M is -inf
    acc *= a;
    lsum *= a;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      if (ms[u] == -__builtin_inff()) continue;  // split with no key of this row
      const float w = fast_exp2(ms[u] - Mb);
      acc += os[u] * w;
      lsum += ls[u] * w;
    }
    M = Mb;
  }
  const float inv = 1.0f / lsum;
  const u32x2 v = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<u32x2*>(out + (((size_t)b * L + query) * H + h) * D + d4 * 4) = v;
}

template <int D, int QPW>
hipError_t launch_dq(const void* q, const void* kp, const void* vp, const void* kb,
                     const void* vb, const void* ks, const void* vs, const int32_t* prefix_len,
                     int B, int H, int L, int P_cap, int S, int S_cap, float scale_log2,
                     void* out, float* ws_o, float* ws_ml, const AttendPlan& p, const Guard& gd,
                     hipStream_t stream) {
  typedef const uint16_t* cp;
  hipError_t e;
  constexpr int KH2 = QPW == 1 ? 2 : 1;
  if (KH2 == 2 && p.kps >= kLongRange) {
    e = launch_kernel(attend_kernel<D, QPW, KH2>, dim3(p.nsplit, H, B), dim3(2 * kAttThreads), 0,
                      stream, (cp)q, (cp)kp, (cp)vp, (cp)kb, (cp)vb, (cp)ks, (cp)vs, prefix_len, H,
                      L, P_cap, S, S_cap, scale_log2, p.kps, p.nsplit, (uint16_t*)out, ws_o, ws_ml,
                      gd);
  } else {
    e = launch_kernel(attend_kernel<D, QPW, 1>, dim3(p.nsplit, H, B), dim3(kAttThreads), 0,
                      stream, (cp)q, (cp)kp, (cp)vp, (cp)kb, (cp)vb, (cp)ks, (cp)vs, prefix_len, H,
                      L, P_cap, S, S_cap, scale_log2, p.kps, p.nsplit, (uint16_t*)out, ws_o, ws_ml,
                      gd);
  }
  if (e != hipSuccess || p.nsplit == 1) return e;
  const int total = B * H * L * (D / 4);
  const dim3 grid((total + kCombineThreads - 1) / kCombineThreads), block(kCombineThreads);
  if (p.nsplit <= 8)
    return launch_kernel(attend_combine_kernel<D, 8>, grid, block, 0, stream, (const float*)ws_o,
                         (const float*)ws_ml, H, L, p.nsplit, (uint16_t*)out, total, gd);
  return launch_kernel(attend_combine_kernel<D, 16>, grid, block, 0, stream, (const float*)ws_o,
                       (const float*)ws_ml, H, L, p.nsplit, (uint16_t*)out, total, gd);
}

}  // namespace

AttendPlan attend_plan(int B, int H, int L, int D, int P_cap, int S) {
  AttendPlan p;
  p.T_cap = P_cap + L + S;
  const int ntile = (p.T_cap + kKT - 1) / kKT;
  const long bhn = (long)B * H;
  int want = bhn > 0 ? (int)((kTargetWGs + bhn - 1) / bhn) : 1;
  if (want < 1) want = 1;
  const int tps = (ntile + want - 1) / want;  // tiles per split
  p.kps = tps * kKT;
  p.nsplit = (p.T_cap + p.kps - 1) / p.kps;
  if (p.nsplit > 1) {
    const size_t rows = (size_t)bhn * p.nsplit * L;
    const size_t o_bytes = (rows * D * sizeof(float) + 255) / 256 * 256;
    p.partials_bytes = o_bytes + rows * 2 * sizeof(float);
  } else {
    p.partials_bytes = 0;
  }
  return p;
}

hipError_t launch_attend(const void* q, const void* kp, const void* vp, const void* kb,
                         const void* vb, const void* ks, const void* vs,
                         const int32_t* prefix_len, int B, int H, int L, int D, int P_cap,
                         int S, int S_cap, float scale, void* out, void* ws,
                         const AttendPlan& p, const Guard& gd, hipStream_t stream) {
  if (scale == 0.f) scale = 1.0f / sqrtf((float)D);
  const float scale_log2 = scale * kLog2e;
  float* ws_o = static_cast<float*>(ws);
  float* ws_ml = nullptr;
  if (p.nsplit > 1) {
    const size_t rows = (size_t)B * H * p.nsplit * L;
    ws_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                     (rows * D * sizeof(float) + 255) / 256 * 256);
  }
  const bool two = L > 16 * kAttWaves;
  if (D == 64) {
    return two ? launch_dq<64, 2>(q, kp, vp, kb, vb, ks, vs, prefix_len, B, H, L, P_cap, S, S_cap,
                                  scale_log2, out, ws_o, ws_ml, p, gd, stream)
               : launch_dq<64, 1>(q, kp, vp, kb, vb, ks, vs, prefix_len, B, H, L, P_cap, S, S_cap,
                                  scale_log2, out, ws_o, ws_ml, p, gd, stream);
  }
  return two ? launch_dq<128, 2>(q, kp, vp, kb, vb, ks, vs, prefix_len, B, H, L, P_cap, S, S_cap,
                                 scale_log2, out, ws_o, ws_ml, p, gd, stream)
             : launch_dq<128, 1>(q, kp, vp, kb, vb, ks, vs, prefix_len, B, H, L, P_cap, S, S_cap,
                                 scale_log2, out, ws_o, ws_ml, p, gd, stream);
}

}  // namespace dblk
