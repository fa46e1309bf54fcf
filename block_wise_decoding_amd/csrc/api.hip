// libdblock C ABI: argument validation and launch of the iteration's kernels.
// The contract of every entry point is documented in include/dblock.h.
#include "dblock.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "dblk_launch.h"

// Scratch of dblk_lmhead_confidence_commit_noalloc: the LM head's arrival
// counters and softmax partials, for callers that cannot allocate.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code
// never uses this name as an address: its device address on each GPU comes
// from hipGetSymbolAddress (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[DBLK_NOALLOC_SCRATCH_BYTES];


namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

constexpr int kMaxT = 65536;
constexpr int64_t kMaxRowStride = int64_t(1) << 24;   // cache row stride limit (elements)

int32_t validate_attend(const void* q, const void* kp, const void* vp, const void* kb,
                        const void* vb, const void* ks, const void* vs, int32_t B, int32_t H,
                        int32_t L, int32_t D, int32_t P_cap, int32_t S, int32_t S_cap,
                        const void* out) {
  if (B < 0 || H < 1 || P_cap < 0 || S < 0 || B > 65535 || H > 65535) return DBLK_ERR_SHAPE;
  if (S_cap < S) return DBLK_ERR_SHAPE;
  if (D != 64 && D != 128) return DBLK_ERR_SHAPE;
  if (L < 16 || L > 128 || (L % 16) != 0) return DBLK_ERR_SHAPE;
  if ((int64_t)P_cap + L + S > kMaxT) return DBLK_ERR_SHAPE;
  if ((int64_t)B * H * ((int64_t)P_cap + L + S_cap) * D > ((int64_t)1 << 40)) return DBLK_ERR_SHAPE;
  if (B == 0) return DBLK_OK;
  if (!q || !kb || !vb || !out) return DBLK_ERR_NULL;
  if (P_cap > 0 && (!kp || !vp)) return DBLK_ERR_NULL;
  if (S > 0 && (!ks || !vs)) return DBLK_ERR_NULL;
  const void* ptrs[] = {q, kp, vp, kb, vb, ks, vs, out};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return DBLK_ERR_ALIGN;
  return DBLK_OK;
}

int32_t validate_lmhead(const void* h, const void* W, int32_t M, int32_t d, int32_t V,
                        const float* conf, const int32_t* argmax) {
  if (M < 0 || V < 1 || V > (1 << 30) || d < 64 || d > 16384 || (d % 64) != 0)
    return DBLK_ERR_SHAPE;
  if (M == 0) return DBLK_OK;
  if (M > (1 << 24)) return DBLK_ERR_SHAPE;
  if (!h || !W || !conf || !argmax) return DBLK_ERR_NULL;
  if (!aligned16(h) || !aligned16(W)) return DBLK_ERR_ALIGN;
  if (((uintptr_t)conf & 3u) || ((uintptr_t)argmax & 3u)) return DBLK_ERR_ALIGN;
  const dblk::LmheadPlan plan = dblk::lmhead_plan(M, d, V);
  if (!plan.gemm && plan.mchunks > 65535) return DBLK_ERR_SHAPE;
  // the row paths address their softmax partials by 32-bit byte offsets
  if (!plan.gemm && plan.partials_bytes >= ((size_t)1 << 31)) return DBLK_ERR_SHAPE;
  if (plan.gemm && plan.g.grid <= 0) return DBLK_ERR_SHAPE;
  // the GEMM path addresses h through a buffer descriptor: byte offsets < 2^31
  if (plan.gemm && (int64_t)M * d > ((int64_t)1 << 30)) return DBLK_ERR_SHAPE;
  return DBLK_OK;
}

int32_t validate_commit(const float* conf, const int32_t* argmax, const int32_t* tokens,
                        const uint8_t* mask, int32_t B, int32_t L, const int32_t* n_committed) {
  if (B < 0 || L < 1 || L > 4096) return DBLK_ERR_SHAPE;
  if (B == 0) return DBLK_OK;
  if (!conf || !argmax || !tokens || !mask) return DBLK_ERR_NULL;
  if (((uintptr_t)conf & 3u) || ((uintptr_t)argmax & 3u) || ((uintptr_t)tokens & 3u) ||
      ((uintptr_t)n_committed & 3u))
    return DBLK_ERR_ALIGN;
  return DBLK_OK;
}

inline size_t round256(size_t n) { return (n + 255) / 256 * 256; }

// ---- the allocation-free entry point's scratch: one device address per
// GPU, taken once with that GPU current and kept for the process.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int32_t noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DBLK_ERR_LAUNCH;
  if (dev >= kMaxDevices) return DBLK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return DBLK_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DBLK_OK;
}

// Clears n 32-bit words (a fill kernel rather than hipMemsetAsync, so that a
// captured graph holds only kernel nodes).
__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// The LM head + decoder step of dblk_lmhead_confidence_commit on a validated
// plan and workspace.
hipError_t lmhead_commit_launch(const void* h, const void* W, int32_t d, int32_t V, float* conf,
                                int32_t* argmax, int32_t* tokens, uint8_t* mask, int32_t B,
                                int32_t L, float threshold, int32_t* n_committed, void* workspace,
                                const dblk::LmheadPlan& plan, hipStream_t s) {
  const int32_t M = B * L;
  const dblk::Guard none{nullptr, 1};
  if (dblk::lmhead_can_fuse_commit(plan, L)) {
    dblk::FusedCommit fc;
    fc.tokens = tokens;
    fc.mask = mask;
    fc.L = L;
    fc.tau = threshold;
    fc.n_out = n_committed;
    return dblk::launch_lmhead(h, W, M, d, V, conf, argmax, workspace, plan, none, fc, mask, s);
  }
  // only the masked rows go through the LM head where the path allows
  hipError_t e = dblk::launch_lmhead(h, W, M, d, V, conf, argmax, workspace, plan, none,
                                     dblk::FusedCommit{}, mask, s);
  if (e == hipSuccess)
    e = dblk::launch_threshold_commit(conf, argmax, tokens, mask, B, L, threshold, n_committed,
                                      dblk::CommitOpts{}, s);
  return e;
}

// dblk_attend_segments: every check of dblk_attend, for arbitrary element
// strides and optional per-sequence segment lengths.
inline bool stride_ok(int64_t s) { return s >= 0 && (s % 8) == 0; }
// Largest element offset + D of a [B][H or L][rows][D] view, or -1 when it
// passes 2^40 elements (nothing this large is plausible: a sign of garbage).
int64_t view_extent(int64_t n0, int64_t s0, int64_t n1, int64_t s1, int64_t n2, int64_t s2,
                    int64_t D) {
  const int64_t lim = (int64_t)1 << 40;
  if (n0 <= 0 || n1 <= 0 || n2 <= 0) return 0;
  if (s0 > lim || s1 > lim || s2 > lim) return -1;
  const double e = (double)(n0 - 1) * s0 + (double)(n1 - 1) * s1 + (double)(n2 - 1) * s2 + D;
  return e > (double)lim ? -1 : (int64_t)e;
}

int32_t validate_segments(const dblk_attend_args* a) {
  if (!a) return DBLK_ERR_NULL;
  if (a->B < 0 || a->B > 65535 || a->H < 1 || a->H > 65535) return DBLK_ERR_SHAPE;
  if (a->D != 64 && a->D != 128) return DBLK_ERR_SHAPE;
  if (a->L < 16 || a->L > 128 || (a->L % 16) != 0) return DBLK_ERR_SHAPE;
  if (!(a->scale >= 0.f && a->scale < 3.0e38f)) return DBLK_ERR_SHAPE;
  const dblk_kv_segment* segs[3] = {&a->prefix, &a->block, &a->suffix};
  int64_t T_cap = 0;
  for (const dblk_kv_segment* s : segs) {
    if (s->len < 0) return DBLK_ERR_SHAPE;
    T_cap += s->len;
    if (s->len == 0) continue;
    if (!stride_ok(s->stride_b) || !stride_ok(s->stride_h) || !stride_ok(s->stride_t))
      return DBLK_ERR_ALIGN;
    if (s->stride_t >= kMaxRowStride) return DBLK_ERR_SHAPE;   // lane offsets are 32-bit
    if (view_extent(a->B, s->stride_b, a->H, s->stride_h, s->len, s->stride_t, a->D) < 0)
      return DBLK_ERR_SHAPE;
  }
  if (T_cap > kMaxT) return DBLK_ERR_SHAPE;
  if (!stride_ok(a->q_stride_b) || !stride_ok(a->q_stride_l) || !stride_ok(a->q_stride_h) ||
      !stride_ok(a->o_stride_b) || !stride_ok(a->o_stride_l) || !stride_ok(a->o_stride_h))
    return DBLK_ERR_ALIGN;
  if (view_extent(a->B, a->q_stride_b, a->L, a->q_stride_l, a->H, a->q_stride_h, a->D) < 0 ||
      view_extent(a->B, a->o_stride_b, a->L, a->o_stride_l, a->H, a->o_stride_h, a->D) < 0)
    return DBLK_ERR_SHAPE;
  if (a->B == 0) return DBLK_OK;
  if (!a->q || !a->out) return DBLK_ERR_NULL;
  if (!aligned16(a->q) || !aligned16(a->out)) return DBLK_ERR_ALIGN;
  for (const dblk_kv_segment* s : segs) {
    if (s->len == 0) continue;
    if (!s->k || !s->v) return DBLK_ERR_NULL;
    if (!aligned16(s->k) || !aligned16(s->v)) return DBLK_ERR_ALIGN;
    if ((uintptr_t)s->len_per_b & 3u) return DBLK_ERR_ALIGN;
  }
  return DBLK_OK;
}

dblk::AttendArgs segment_args(const dblk_attend_args* a) {
  typedef const uint16_t* cp;
  dblk::AttendArgs r;
  r.B = a->B; r.H = a->H; r.L = a->L; r.D = a->D;
  r.q = (cp)a->q;
  r.q_sb = a->q_stride_b; r.q_sl = a->q_stride_l; r.q_sh = a->q_stride_h;
  r.out = static_cast<uint16_t*>(a->out);
  r.o_sb = a->o_stride_b; r.o_sl = a->o_stride_l; r.o_sh = a->o_stride_h;
  const dblk_kv_segment* segs[3] = {&a->prefix, &a->block, &a->suffix};
  for (int i = 0; i < 3; ++i) {
    const dblk_kv_segment* s = segs[i];
    const bool any = s->len > 0;
    r.seg[i] = dblk::KVSeg{any ? (cp)s->k : nullptr, any ? (cp)s->v : nullptr, s->stride_b,
                           s->stride_h, s->stride_t, s->len, any ? s->len_per_b : nullptr};
  }
  r.scale = a->scale;
  return r;
}

// dblk_decode_block workspace:
// [LM-head workspace | attention partials | masked counts [B] | active-sequence count]
struct DecodeLayout {
  size_t lm_bytes, att_off, att_bytes, rem_off, cnt_off, total;
};

DecodeLayout decode_layout(const dblk_decode_args* a) {
  DecodeLayout l;
  const int M = a->B * a->L;
  const dblk::LmheadPlan lp = dblk::lmhead_plan(M, a->d, a->V);
  l.lm_bytes = round256(lp.counters_bytes + lp.partials_bytes);
  l.att_off = l.lm_bytes;
  l.att_bytes = round256(dblk::attend_plan(a->B, a->H, a->L, a->D, a->P_cap + a->L + a->S).ws_bytes);
  l.rem_off = l.att_off + l.att_bytes;
  l.cnt_off = l.rem_off + round256((size_t)a->B * sizeof(int32_t));
  l.total = l.cnt_off + 256;
  return l;
}

int32_t validate_decode(const dblk_decode_args* a) {
  if (!a) return DBLK_ERR_NULL;
  int32_t st = validate_attend(a->q, a->k_prefix, a->v_prefix, a->k_block, a->v_block,
                               a->k_suffix, a->v_suffix, a->B, a->H, a->L, a->D, a->P_cap, a->S,
                               a->S_cap, a->attn_out);
  if (st != DBLK_OK || a->B == 0) return st;
  if (!(a->scale >= 0.f && a->scale < 3.0e38f)) return DBLK_ERR_SHAPE;
  st = validate_lmhead(a->h, a->W, a->B * a->L, a->d, a->V, a->conf, a->argmax);
  if (st != DBLK_OK) return st;
  st = validate_commit(a->conf, a->argmax, a->tokens, a->mask, a->B, a->L, nullptr);
  if (st != DBLK_OK) return st;
  if (((uintptr_t)a->commit_iter & 3u) || ((uintptr_t)a->n_iters & 3u)) return DBLK_ERR_ALIGN;
  return DBLK_OK;
}

// Enqueues iterations t0 .. t0+n-1 of a block loop (and, for t0 == 0, the
// initialisation of the per-sequence counts and records).  No host sync.
hipError_t enqueue_iterations(const dblk_decode_args* a, const DecodeLayout& lay, char* ws,
                              int t0, int n, hipStream_t s) {
  const int32_t M = a->B * a->L;
  int32_t* remaining = reinterpret_cast<int32_t*>(ws + lay.rem_off);
  const dblk::Guard gd{remaining, a->L};
  const dblk::LmheadPlan lp = dblk::lmhead_plan(M, a->d, a->V);
  const bool fuse = dblk::lmhead_can_fuse_commit(lp, a->L);
  const dblk::AttendPlan ap = dblk::attend_plan(a->B, a->H, a->L, a->D, a->P_cap + a->L + a->S);
  const dblk::AttendArgs aa = dblk::dense_attend_args(
      a->q, a->k_prefix, a->v_prefix, a->k_block, a->v_block, a->k_suffix, a->v_suffix,
      a->prefix_len, a->B, a->H, a->L, a->D, a->P_cap, a->S, a->S_cap, a->scale, a->attn_out);
  hipError_t e = hipSuccess;
  if (t0 == 0)
    e = dblk::launch_block_loop_init(a->mask, a->B, a->L, remaining, a->commit_iter, a->n_iters, s);
  for (int t = t0; t < t0 + n && e == hipSuccess; ++t) {
    e = dblk::launch_attend(aa, ws + lay.att_off, ap, gd, s);
    if (e != hipSuccess) break;
    dblk::CommitOpts opt;
    opt.eos_id = a->eos_id >= 0 ? a->eos_id : -1;
    opt.finished = a->eos_id >= 0 ? a->finished : nullptr;
    opt.iter = t;
    opt.commit_iter = a->commit_iter;
    opt.n_iters = a->n_iters;
    opt.remaining = remaining;
    if (fuse) {   // the decoder step runs in the LM head's final merge
      dblk::FusedCommit fc;
      fc.tokens = a->tokens;
      fc.mask = a->mask;
      fc.L = a->L;
      fc.tau = a->threshold;
      fc.opt = opt;
      e = dblk::launch_lmhead(a->h, a->W, M, a->d, a->V, a->conf, a->argmax, ws, lp, gd, fc,
                              a->mask, s);
    } else {
      // only the still-masked rows go through the LM head where the path allows
      e = dblk::launch_lmhead(a->h, a->W, M, a->d, a->V, a->conf, a->argmax, ws, lp, gd,
                              dblk::FusedCommit{}, a->mask, s);
      if (e == hipSuccess)
        e = dblk::launch_threshold_commit(a->conf, a->argmax, a->tokens, a->mask, a->B, a->L,
                                          a->threshold, nullptr, opt, s);
    }
  }
  return e;
}

}  // namespace

extern "C" {

const char* dblk_status_string(int32_t status) {
  switch (status) {
    case DBLK_OK: return "DBLK_OK";
    case DBLK_ERR_NULL: return "DBLK_ERR_NULL: a required pointer is NULL";
    case DBLK_ERR_SHAPE: return "DBLK_ERR_SHAPE: a size is out of the supported range";
    case DBLK_ERR_ALIGN: return "DBLK_ERR_ALIGN: a bf16 tensor is not 16-byte aligned";
    case DBLK_ERR_WORKSPACE: return "DBLK_ERR_WORKSPACE: workspace missing or too small";
    case DBLK_ERR_UNSUPPORTED: return "DBLK_ERR_UNSUPPORTED: not implemented by this build";
    case DBLK_ERR_LAUNCH: return "DBLK_ERR_LAUNCH: the HIP runtime rejected a launch";
    default: return "DBLK_ERR_?: unknown status code";
  }
}

int32_t dblk_abi_version(void) { return 3; }

size_t dblk_attend_workspace_size(int32_t B, int32_t H, int32_t L, int32_t D, int32_t P_cap,
                                  int32_t S) {
  if (B <= 0 || H <= 0 || L <= 0 || D <= 0 || P_cap < 0 || S < 0) return 0;
  return dblk::attend_plan(B, H, L, D, P_cap + L + S).ws_bytes;
}

size_t dblk_attend_segments_workspace_size(const dblk_attend_args* a) {
  if (!a || a->B <= 0 || a->H <= 0 || a->L <= 0 || a->D <= 0 || a->prefix.len < 0 ||
      a->block.len < 0 || a->suffix.len < 0)
    return 0;
  return dblk::attend_plan(a->B, a->H, a->L, a->D,
                           a->prefix.len + a->block.len + a->suffix.len).ws_bytes;
}

int32_t dblk_attend_segments(const dblk_attend_args* a, void* workspace, size_t workspace_bytes,
                             void* stream) {
  int32_t st = validate_segments(a);
  if (st != DBLK_OK || a->B == 0) return st;
  const dblk::AttendPlan plan = dblk::attend_plan(a->B, a->H, a->L, a->D,
                                                  a->prefix.len + a->block.len + a->suffix.len);
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return DBLK_ERR_WORKSPACE;
    if (!aligned256(workspace)) return DBLK_ERR_ALIGN;
  }
  hipError_t e = dblk::launch_attend(segment_args(a), workspace, plan, dblk::Guard{nullptr, a->L},
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

int32_t dblk_attend(const void* q, const void* k_prefix, const void* v_prefix,
                    const void* k_block, const void* v_block, const void* k_suffix,
                    const void* v_suffix, const int32_t* prefix_len, int32_t B, int32_t H,
                    int32_t L, int32_t D, int32_t P_cap, int32_t S, int32_t S_cap, float scale,
                    void* out, void* workspace, size_t workspace_bytes, void* stream) {
  int32_t st = validate_attend(q, k_prefix, v_prefix, k_block, v_block, k_suffix, v_suffix, B, H,
                               L, D, P_cap, S, S_cap, out);
  if (st != DBLK_OK || B == 0) return st;
  if (!(scale >= 0.f && scale < 3.0e38f)) return DBLK_ERR_SHAPE;  // NaN, negative or inf
  const dblk::AttendPlan plan = dblk::attend_plan(B, H, L, D, P_cap + L + S);
  if (plan.ws_bytes > 0) {
    if (!workspace) return DBLK_ERR_WORKSPACE;
    if (workspace_bytes < plan.ws_bytes) return DBLK_ERR_WORKSPACE;
    if (!aligned256(workspace)) return DBLK_ERR_ALIGN;
  }
  const dblk::AttendArgs aa = dblk::dense_attend_args(q, k_prefix, v_prefix, k_block, v_block,
                                                      k_suffix, v_suffix, prefix_len, B, H, L, D,
                                                      P_cap, S, S_cap, scale, out);
  hipError_t e = dblk::launch_attend(aa, workspace, plan, dblk::Guard{nullptr, L},
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

size_t dblk_lmhead_workspace_size(int32_t M, int32_t d, int32_t V) {
  if (M <= 0 || d <= 0 || V <= 0) return 0;
  const dblk::LmheadPlan p = dblk::lmhead_plan(M, d, V);
  return p.counters_bytes + p.partials_bytes;
}

int32_t dblk_lmhead_confidence(const void* h, const void* W, int32_t M, int32_t d, int32_t V,
                               float* conf, int32_t* argmax, void* workspace,
                               size_t workspace_bytes, void* stream) {
  int32_t st = validate_lmhead(h, W, M, d, V, conf, argmax);
  if (st != DBLK_OK || M == 0) return st;
  const dblk::LmheadPlan plan = dblk::lmhead_plan(M, d, V);
  if (!workspace || workspace_bytes < plan.counters_bytes + plan.partials_bytes)
    return DBLK_ERR_WORKSPACE;
  if (!aligned256(workspace)) return DBLK_ERR_ALIGN;
  hipError_t e = dblk::launch_lmhead(h, W, M, d, V, conf, argmax, workspace, plan,
                                     dblk::Guard{nullptr, 1}, dblk::FusedCommit{}, nullptr,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

int32_t dblk_lmhead_confidence_commit(const void* h, const void* W, int32_t d, int32_t V,
                                      float* conf, int32_t* argmax, int32_t* tokens,
                                      uint8_t* mask, int32_t B, int32_t L, float threshold,
                                      int32_t* n_committed, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  int32_t st = validate_commit(conf, argmax, tokens, mask, B, L, n_committed);
  if (st != DBLK_OK) return st;
  if ((int64_t)B * L > (1 << 24)) return DBLK_ERR_SHAPE;
  const int32_t M = B * L;
  st = validate_lmhead(h, W, M, d, V, conf, argmax);
  if (st != DBLK_OK || M == 0) return st;
  const dblk::LmheadPlan plan = dblk::lmhead_plan(M, d, V);
  if (!workspace || workspace_bytes < plan.counters_bytes + plan.partials_bytes)
    return DBLK_ERR_WORKSPACE;
  if (!aligned256(workspace)) return DBLK_ERR_ALIGN;
  const hipError_t e = lmhead_commit_launch(h, W, d, V, conf, argmax, tokens, mask, B, L,
                                            threshold, n_committed, workspace, plan,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

int32_t dblk_lmhead_confidence_commit_noalloc(const void* h, const void* W, int32_t d, int32_t V,
                                              float* conf, int32_t* argmax, int32_t* tokens,
                                              uint8_t* mask, int32_t B, int32_t L,
                                              float threshold, int32_t* n_committed,
                                              void* stream) {
  int32_t st = validate_commit(conf, argmax, tokens, mask, B, L, n_committed);
  if (st != DBLK_OK) return st;
  if ((int64_t)B * L > (1 << 24)) return DBLK_ERR_SHAPE;
  const int32_t M = B * L;
  st = validate_lmhead(h, W, M, d, V, conf, argmax);
  if (st != DBLK_OK || M == 0) return st;
  const dblk::LmheadPlan plan = dblk::lmhead_plan(M, d, V);
  if (plan.counters_bytes + plan.partials_bytes > (size_t)DBLK_NOALLOC_SCRATCH_BYTES)
    return DBLK_ERR_WORKSPACE;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != DBLK_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  // The scratch keeps whatever the last call on this GPU left there, and that
  // call may have had another plan: the arrival counters start from zero.
  if (!plan.gemm && plan.counters_bytes > 0) {
    const int n = (int)(plan.counters_bytes / sizeof(uint32_t));
    e = dblk::launch_kernel(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, s,
                            static_cast<uint32_t*>(ws), n);
  }
  if (e == hipSuccess)
    e = lmhead_commit_launch(h, W, d, V, conf, argmax, tokens, mask, B, L, threshold,
                             n_committed, ws, plan, s);
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

int32_t dblk_threshold_commit(const float* conf, const int32_t* argmax, int32_t* tokens,
                              uint8_t* mask, int32_t B, int32_t L, float threshold,
                              int32_t* n_committed, void* stream) {
  int32_t st = validate_commit(conf, argmax, tokens, mask, B, L, n_committed);
  if (st != DBLK_OK || B == 0) return st;
  hipError_t e = dblk::launch_threshold_commit(conf, argmax, tokens, mask, B, L, threshold,
                                               n_committed, dblk::CommitOpts{},
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

int32_t dblk_threshold_commit_eos(const float* conf, const int32_t* argmax, int32_t* tokens,
                                  uint8_t* mask, int32_t B, int32_t L, float threshold,
                                  int32_t eos_id, int32_t* n_committed, uint8_t* finished,
                                  void* stream) {
  int32_t st = validate_commit(conf, argmax, tokens, mask, B, L, n_committed);
  if (st != DBLK_OK) return st;
  if (eos_id < 0) return DBLK_ERR_SHAPE;
  if (B == 0) return DBLK_OK;
  dblk::CommitOpts opt;
  opt.eos_id = eos_id;
  opt.finished = finished;
  hipError_t e = dblk::launch_threshold_commit(conf, argmax, tokens, mask, B, L, threshold,
                                               n_committed, opt, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

size_t dblk_decode_block_workspace_size(const dblk_decode_args* a) {
  if (!a || a->B <= 0 || a->H <= 0 || a->L <= 0 || a->D <= 0 || a->P_cap < 0 || a->S < 0 ||
      a->d <= 0 || a->V <= 0)
    return 0;
  return decode_layout(a).total;
}

int32_t dblk_decode_block(const dblk_decode_args* a, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int32_t st = validate_decode(a);
  if (st != DBLK_OK || a->B == 0) return st;
  const DecodeLayout lay = decode_layout(a);
  if (!workspace || workspace_bytes < lay.total) return DBLK_ERR_WORKSPACE;
  if (!aligned256(workspace)) return DBLK_ERR_ALIGN;
  const int iters = a->max_iters > 0 ? a->max_iters : a->L;
  hipError_t e = enqueue_iterations(a, lay, static_cast<char*>(workspace), 0, iters,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

int32_t dblk_decode_block_run(const dblk_decode_args* a, int32_t chunk, int32_t* host_active,
                              void* workspace, size_t workspace_bytes, void* stream,
                              int32_t* iters_enqueued) {
  int32_t st = validate_decode(a);
  if (st != DBLK_OK) return st;
  if (chunk < 1) return DBLK_ERR_SHAPE;
  if (iters_enqueued) *iters_enqueued = 0;
  if (a->B == 0) return DBLK_OK;
  if (!host_active) return DBLK_ERR_NULL;
  if ((uintptr_t)host_active & 3u) return DBLK_ERR_ALIGN;
  const DecodeLayout lay = decode_layout(a);
  if (!workspace || workspace_bytes < lay.total) return DBLK_ERR_WORKSPACE;
  if (!aligned256(workspace)) return DBLK_ERR_ALIGN;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* remaining = reinterpret_cast<int32_t*>(ws + lay.rem_off);
  int32_t* dev_count = reinterpret_cast<int32_t*>(ws + lay.cnt_off);
  const int cap = a->max_iters > 0 ? a->max_iters : a->L;
  hipEvent_t ev[2] = {nullptr, nullptr};
  for (int k = 0; k < 2; ++k)
    if (hipEventCreateWithFlags(&ev[k], hipEventDisableTiming) != hipSuccess) {
      if (ev[0]) (void)hipEventDestroy(ev[0]);   // already failing: report the create error
      return DBLK_ERR_LAUNCH;
    }
  // chunk c: its iterations, then the count of active sequences copied into
  // host_active[c % 2] and event ev[c % 2].  Chunk c + 1 is queued before the
  // host waits for chunk c, so the device always has work while it waits.
  int t = 0, queued = 0, checked = 0;
  hipError_t e = hipSuccess;
  auto enqueue = [&]() {
    const int n = chunk < cap - t ? chunk : cap - t;
    const int slot = queued & 1;
    e = enqueue_iterations(a, lay, ws, t, n, s);
    if (e == hipSuccess) e = dblk::launch_block_loop_count(remaining, a->B, dev_count, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(host_active + slot, dev_count, sizeof(int32_t), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipEventRecord(ev[slot], s);
    t += n;
    ++queued;
  };
  enqueue();
  if (e == hipSuccess && t < cap) enqueue();
  while (e == hipSuccess && checked < queued) {
    e = hipEventSynchronize(ev[checked & 1]);
    if (e != hipSuccess) break;
    const int32_t active = host_active[checked & 1];
    ++checked;
    if (active == 0) break;                         // the block is complete
    if (t < cap) enqueue();
  }
  const hipError_t d0 = hipEventDestroy(ev[0]);
  const hipError_t d1 = hipEventDestroy(ev[1]);
  if (e == hipSuccess) e = d0 != hipSuccess ? d0 : d1;
  if (iters_enqueued) *iters_enqueued = t;
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

int32_t dblk_cache_append(void* k_prefix, void* v_prefix, const void* k_block,
                          const void* v_block, int32_t* prefix_len, int32_t B, int32_t H,
                          int32_t L, int32_t D, int32_t P_cap, int32_t* appended, void* stream) {
  if (B < 0 || H < 1 || B > 65535 || H > 65535 || L < 1 || L > 4096 || P_cap < L)
    return DBLK_ERR_SHAPE;
  if (D != 64 && D != 128) return DBLK_ERR_SHAPE;
  if ((int64_t)B * H * P_cap * D > ((int64_t)1 << 40)) return DBLK_ERR_SHAPE;
  if (B == 0) return DBLK_OK;
  if (!k_prefix || !v_prefix || !k_block || !v_block || !prefix_len) return DBLK_ERR_NULL;
  const void* ptrs[] = {k_prefix, v_prefix, k_block, v_block};
  for (const void* p : ptrs)
    if (!aligned16(p)) return DBLK_ERR_ALIGN;
  if (((uintptr_t)prefix_len & 3u) || ((uintptr_t)appended & 3u)) return DBLK_ERR_ALIGN;
  hipError_t e = dblk::launch_cache_append(k_prefix, v_prefix, k_block, v_block, prefix_len, B, H,
                                           L, D, P_cap, appended,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? DBLK_OK : DBLK_ERR_LAUNCH;
}

}  // extern "C"
