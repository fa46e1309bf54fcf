/*
 * libdblock -- one denoising iteration of block-wise diffusion-LLM decoding
 * on AMD Instinct MI355X (gfx950).
 *
 * An iteration, as the dInfer framework composes it (its README's usage
 * section builds a BlockWiseDiffusionLLM from a ThresholdParallelDecoder and a
 * 'dual' KV-cache factory, decoding 1024 tokens in blocks of 64):
 *
 *   1. dblk_attend             -- the active block's queries attend, with no
 *                                  causal mask, over the dual KV cache:
 *                                  cached prefix, the block itself, cached suffix.
 *   2. dblk_lmhead_confidence  -- LM-head logits of the block's hidden states,
 *                                  softmax over the whole vocabulary, per
 *                                  position the largest probability
 *                                  ("confidence") and its token (argmax).
 *   3. dblk_threshold_commit   -- the threshold parallel decoder: commit every
 *                                  still-masked position whose confidence meets
 *                                  the threshold, and at least the single most
 *                                  confident masked one.
 *   (2+3 dblk_lmhead_confidence_commit -- both in one call, fused where the
 *                                  shapes allow.)
 *
 * Around the iteration:
 *   dblk_threshold_commit_eos  -- the decoder step with end-of-text handling.
 *   dblk_decode_block          -- the iteration repeated on the device until
 *                                  the block has no masked position left, with
 *                                  no host round trip between iterations.
 *   dblk_decode_block_run      -- the same, enqueued a few iterations ahead of
 *                                  a host-side completion check.
 *   dblk_cache_append          -- at block completion, the block's keys and
 *                                  values join the cached prefix.
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or copies to the host, and keeps no global state.
 *   - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16),
 *     stored as 2-byte little-endian words.  All bf16 tensors are dense,
 *     row-major, with the innermost dimension contiguous -- except in
 *     dblk_attend_segments, which takes element strides for every tensor.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise with the host, except
 *     dblk_decode_block_run, which waits for device progress by design.
 *   - Arguments are validated on the host BEFORE anything is launched; a
 *     failed validation returns a status code and has no side effects.  A
 *     launch failure returns DBLK_ERR_LAUNCH.  No exception crosses the ABI.
 *   - Outputs are bitwise deterministic for given inputs and device (no
 *     floating-point atomics; all reductions run in a fixed order).
 *   - Workspace: scratch device memory the caller provides, sized by the
 *     matching *_workspace_size() query (a pure host function).  It must be
 *     zero-filled before its FIRST use; every call leaves its counters at zero
 *     again on completion, so it can be reused without clearing.  Two calls
 *     that may run concurrently must not share a workspace.
 */
#ifndef DBLOCK_H_
#define DBLOCK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DBLK_OK = 0,
  DBLK_ERR_NULL = 1,        /* a required pointer is NULL                        */
  DBLK_ERR_SHAPE = 2,       /* a size is out of the supported range              */
  DBLK_ERR_ALIGN = 3,       /* a bf16 tensor is not 16-byte aligned              */
  DBLK_ERR_WORKSPACE = 4,   /* workspace pointer NULL or smaller than required   */
  DBLK_ERR_UNSUPPORTED = 5, /* valid request this build does not implement       */
  DBLK_ERR_LAUNCH = 6,      /* the HIP runtime rejected a launch / device query  */
} dblk_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *dblk_status_string(int32_t status);

/* ABI version of this header: 3. */
int32_t dblk_abi_version(void);

/* ------------------------------------------------------------------------
 * dblk_attend -- non-causal attention of the block over the dual KV cache.
 *
 * For every sequence b and head h, with P_b = prefix_len[b] (clamped to
 * [0, P_cap]) the keys/values seen by row (b, h) are, in order,
 *   prefix[b][h][0:P_b]  ++  block[b][h][0:L]  ++  suffix[b][h][0:S]
 * (T_b = P_b + L + S rows), and for each block query l
 *   out[b][l][h][:] = softmax_t( q[b][l][h]·k_t * scale ) · V
 * with no causal or other mask: every query sees every key, its own included.
 * (Dual cache: the README's dual KV-cache factory, usage section; bidirectional attention of
 * diffusion LMs: the topic page's variable-size-block and Streaming-dLLM
 * abstracts.)
 *
 *   q            bf16 [B][L][H][D]        block queries (RoPE already applied)
 *   k_prefix,
 *   v_prefix     bf16 [B][H][P_cap][D]    cached prefix; rows >= P_b never read.
 *                                         May be NULL when P_cap == 0.
 *   k_block,
 *   v_block      bf16 [B][H][L][D]        the block's own keys/values
 *   k_suffix,
 *   v_suffix     bf16 [B][H][S_cap][D]    cached suffix; rows >= S never read.
 *                                         May be NULL when S == 0.  S_cap is the
 *                                         row stride, so a window of the first
 *                                         S rows, or the suffix advanced by a
 *                                         block (base + L*D elements), needs no copy.
 *   prefix_len   int32 [B] device, or NULL (then P_b = P_cap for every b);
 *                values outside [0, P_cap] are clamped into it by the kernel
 *   0 <= B <= 65535, 1 <= H <= 65535, D in {64, 128}, L in {16, 32, ..., 128}, P_cap >= 0,
 *   0 <= S <= S_cap, P_cap + L + S <= 65536
 *   scale        score scale, finite and >= 0; 0 selects 1/sqrt(D)
 *   out          bf16 [B][L][H][D]; must not alias any input
 *   workspace    >= dblk_attend_workspace_size(...) bytes (split
 *                partials; 0 bytes when the key range is not split),
 *                256-byte aligned
 * B == 0 is a valid no-op.  A row with no key at all (P_b = L = S = 0 cannot
 * happen here; see dblk_attend_segments) is written as zeros.
 * ---------------------------------------------------------------------- */
size_t dblk_attend_workspace_size(int32_t B, int32_t H, int32_t L, int32_t D,
                                  int32_t P_cap, int32_t S);

int32_t dblk_attend(const void *q,
                    const void *k_prefix, const void *v_prefix,
                    const void *k_block, const void *v_block,
                    const void *k_suffix, const void *v_suffix,
                    const int32_t *prefix_len,
                    int32_t B, int32_t H, int32_t L, int32_t D,
                    int32_t P_cap, int32_t S, int32_t S_cap, float scale,
                    void *out, void *workspace, size_t workspace_bytes,
                    void *stream);

/* ------------------------------------------------------------------------
 * dblk_attend_segments -- dblk_attend with every tensor described by element
 * strides and each cache segment by its own (optionally per-sequence)
 * length: q taken straight from a fused QKV projection, caches stored
 * head-interleaved ([B][T][H][D]) or in any other layout whose head dimension
 * is contiguous, and ragged block or suffix lengths, all without a copy.
 * (Same operation: the README's 'dual' KV cache, the topic page's
 * bidirectional attention and Streaming-dLLM suffix pruning.)
 *
 * For sequence b the keys/values seen by row (b, h) are, in order,
 *   prefix rows [0, P_b)  ++  block rows [0, Lk_b)  ++  suffix rows [0, S_b)
 * where each segment's rows_b = clamp(len_per_b[b], 0, len), or len when
 * len_per_b is NULL; row t of a segment for (b, h) starts at element
 *   k + b*stride_b + h*stride_h + t*stride_t     (v likewise, same strides)
 * and out[b][l][h] = softmax_t(q[b][l][h] . k_t * scale) . V, no mask.  A
 * row whose three lengths are all 0 is written as zeros.
 *
 *   dblk_kv_segment  k, v: bf16 device pointers, 16-byte aligned (may be
 *                    NULL when len == 0); stride_b, stride_h, stride_t:
 *                    element strides, >= 0 and multiples of 8 (16-byte rows),
 *                    stride_t < 2^24 (else DBLK_ERR_SHAPE);
 *                    len >= 0 rows available per (b, h); len_per_b: device
 *                    int32 [B] or NULL
 *   dblk_attend_args B, H, L, D as for dblk_attend; q / out: bf16 device
 *                    pointers, 16-byte aligned, element (b, l, h, 0) at
 *                    b*q_stride_b + l*q_stride_l + h*q_stride_h (out likewise;
 *                    strides >= 0, multiples of 8; out's elements must be
 *                    distinct and alias no input); scale as for dblk_attend;
 *                    prefix.len + block.len + suffix.len <= 65536; every view
 *                    spans at most 2^40 elements
 *   workspace        >= dblk_attend_segments_workspace_size(args) bytes,
 *                    256-byte aligned
 * B == 0 is a valid no-op.  dblk_attend(...) is this call with the dense
 * strides of its layout, prefix.len_per_b = prefix_len, block.len = L and
 * suffix.len = S; both give bit-identical outputs on the same data.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void *k, *v;
  int64_t stride_b, stride_h, stride_t;
  int32_t len;
  const int32_t *len_per_b;
} dblk_kv_segment;

typedef struct {
  int32_t B, H, L, D;
  const void *q;
  int64_t q_stride_b, q_stride_l, q_stride_h;
  dblk_kv_segment prefix, block, suffix;
  float scale;
  void *out;
  int64_t o_stride_b, o_stride_l, o_stride_h;
} dblk_attend_args;

size_t dblk_attend_segments_workspace_size(const dblk_attend_args *args);

int32_t dblk_attend_segments(const dblk_attend_args *args, void *workspace,
                             size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * dblk_lmhead_confidence -- LM head, full-vocabulary softmax confidence and
 * argmax for M = B*L block rows.
 *
 *   logits[m][t] = sum_k h[m][k] * W[t][k]     (fp32 accumulation of bf16)
 *   conf[m]      = max_t softmax(logits[m])_t  = 1 / sum_t exp(logits[m][t] - max)
 *   argmax[m]    = lowest t attaining max_t logits[m][t]
 * The logits are never written to memory.  (Confidence-driven parallel
 * decoding: the README's ThresholdParallelDecoder and the DepCap abstract on
 * the topic page; softmax at temperature 1 over every vocabulary id.)
 *
 *   h       bf16 [M][d]   block hidden states, row m = b*L + l
 *   W       bf16 [V][d]   LM-head weight, row t = token t
 *   M >= 0, d multiple of 64 with 64 <= d <= 16384, 1 <= V <= 2^30; with
 *           M < 256 the per-workgroup softmax partials in the workspace must
 *           stay under 2 GiB (reached only past V ~ 6e8 / ceil(M/64) when d
 *           is not 256, 512, 1024 or 2048); with M >= 256, M*d <= 2^30
 *           (h under 2 GiB); else DBLK_ERR_SHAPE
 *   conf    fp32 [M]  out;  argmax  int32 [M]  out
 *   workspace >= dblk_lmhead_workspace_size(M, d, V) bytes, 256-byte aligned,
 *           zero-filled before first use (holds arrival counters)
 * M == 0 is a valid no-op.  Non-finite logits give unspecified results.
 * ---------------------------------------------------------------------- */
size_t dblk_lmhead_workspace_size(int32_t M, int32_t d, int32_t V);

int32_t dblk_lmhead_confidence(const void *h, const void *W,
                               int32_t M, int32_t d, int32_t V,
                               float *conf, int32_t *argmax,
                               void *workspace, size_t workspace_bytes,
                               void *stream);

/* ------------------------------------------------------------------------
 * dblk_threshold_commit -- one step of the threshold parallel decoder
 * (the README's threshold-based parallel decoder, threshold 0.9; usage section).
 *
 * Per sequence b, with masked set Mb = { i : mask[b][i] != 0 }:
 *   C = { i in Mb : conf[b][i] >= threshold }     (fp32 comparison)
 *   if C is empty and Mb is not: C = { the i in Mb with the largest conf,
 *                                      lowest i on an exact tie }
 *   for i in C: tokens[b][i] = argmax[b][i]; mask[b][i] = 0
 *   n_committed[b] = |C|
 * Positions outside C, and rows with no masked position, are left unchanged.
 * NaN confidences never meet the threshold and never win the fallback
 * (a row whose masked confidences are all NaN commits its first masked one).
 *
 *   conf         fp32  [B][L]   in
 *   argmax       int32 [B][L]   in
 *   tokens       int32 [B][L]   in/out
 *   mask         uint8 [B][L]   in/out (nonzero = still masked); committed
 *                               positions are set to 0, others are not written
 *   B >= 0, 1 <= L <= 4096; threshold any fp32 value
 *   n_committed  int32 [B] out, or NULL
 * ---------------------------------------------------------------------- */
int32_t dblk_threshold_commit(const float *conf, const int32_t *argmax,
                              int32_t *tokens, uint8_t *mask,
                              int32_t B, int32_t L, float threshold,
                              int32_t *n_committed, void *stream);

/* ------------------------------------------------------------------------
 * dblk_lmhead_confidence_commit -- the LM head's confidence and argmax for
 * the block rows, then dblk_threshold_commit: tokens, mask and n_committed
 * are identical bit for bit to dblk_lmhead_confidence + dblk_threshold_commit,
 * and so are conf/argmax of every row that is masked on entry.  The decoder
 * reads nothing else, so only those rows are guaranteed: where the path
 * allows, only the masked rows go through the LM head (masked-row compaction:
 * with M >= 256 a device scan lists them and the GEMM reads h through the
 * list; with M < 256 and d a multiple of 256 up to 2048 each 64-row chunk
 * takes its masked rows from a wave ballot) and conf/argmax of the other rows
 * are left unchanged; otherwise (M < 256, other d) every row is computed.
 * When M < 256 and L is a power of two <= 64, the decoder step runs inside
 * the LM head's final merge (one launch: the workgroup that finishes 64 rows
 * holds whole sequences).
 *   Arguments as for the two calls; workspace as for
 *   dblk_lmhead_confidence(h, W, B*L, d, V, ...).
 * ---------------------------------------------------------------------- */
int32_t dblk_lmhead_confidence_commit(const void *h, const void *W,
                                      int32_t d, int32_t V,
                                      float *conf, int32_t *argmax,
                                      int32_t *tokens, uint8_t *mask,
                                      int32_t B, int32_t L, float threshold,
                                      int32_t *n_committed,
                                      void *workspace, size_t workspace_bytes,
                                      void *stream);

/* ------------------------------------------------------------------------
 * dblk_lmhead_confidence_commit_noalloc -- dblk_lmhead_confidence_commit for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument, and the call allocates nothing.  Its scratch (arrival counters
 * and softmax partials) is a file-scope device array of
 * DBLK_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends; the calling thread's current device must be the
 * stream's.  Results are bit-identical to dblk_lmhead_confidence_commit.
 *   Arguments as for dblk_lmhead_confidence_commit, without the workspace.
 *   Returns DBLK_ERR_WORKSPACE when the call would need more scratch than
 *   DBLK_NOALLOC_SCRATCH_BYTES (dblk_lmhead_workspace_size(B*L, d, V) above
 *   it; e.g. 4096 block rows at vocabulary 157184), before anything runs.
 * Every call on a GPU shares that GPU's array: calls that may overlap on one
 * GPU (other streams, other threads) race and must not be issued.  Each call
 * clears the counters it uses first, so a call after one with other shapes,
 * or after a call that did not complete, starts clean.
 * ---------------------------------------------------------------------- */
#define DBLK_NOALLOC_SCRATCH_BYTES (16u << 20)

int32_t dblk_lmhead_confidence_commit_noalloc(const void *h, const void *W,
                                              int32_t d, int32_t V,
                                              float *conf, int32_t *argmax,
                                              int32_t *tokens, uint8_t *mask,
                                              int32_t B, int32_t L, float threshold,
                                              int32_t *n_committed, void *stream);

/* ------------------------------------------------------------------------
 * dblk_threshold_commit_eos -- the decoder step of dblk_threshold_commit,
 * then end-of-text handling (the README's decoder takes an eos_id; what it
 * does with it is not described there, the reading here is the common one
 * that nothing but EOS follows an EOS):
 *   e = the lowest position of row b that is unmasked after the step and
 *       holds eos_id (committed now or earlier);
 *   every position i > e still masked after the step is committed with
 *       tokens[b][i] = eos_id, mask[b][i] = 0;
 *   finished[b] = 1 if e exists, else 0.
 * n_committed[b] counts both kinds of commits.  Unmasked tokens after e are
 * never rewritten.  Arguments as for dblk_threshold_commit, plus
 *   eos_id    >= 0
 *   finished  uint8 [B] out, or NULL
 * ---------------------------------------------------------------------- */
int32_t dblk_threshold_commit_eos(const float *conf, const int32_t *argmax,
                                  int32_t *tokens, uint8_t *mask,
                                  int32_t B, int32_t L, float threshold,
                                  int32_t eos_id, int32_t *n_committed,
                                  uint8_t *finished, void *stream);

/* ------------------------------------------------------------------------
 * dblk_decode_block -- the denoising iterations of one block, enqueued on
 * the device with no host synchronisation between them (dInfer's loop
 * unrolling across diffusion iterations, the framework overview on its
 * page; the stop condition is the block's mask running empty).
 *
 * Enqueues an initialisation kernel and then max_iters iterations; iteration
 * t is dblk_attend, dblk_lmhead_confidence on the M = B*L rows and the
 * decoder step (with EOS handling when eos_id >= 0), each skipping every
 * sequence whose block has no masked position left.  Because every
 * iteration commits at least one position of every sequence that has one,
 * max_iters = L (the default) always empties every block.  The layers that
 * would turn the attention output into new hidden states are outside this
 * library: h, the cache and the queries stay as given, so every iteration
 * sees the same logits.
 *
 * Fields of dblk_decode_args: the attention arguments exactly as for
 * dblk_attend (attn_out is written every iteration), then
 *   h, W, d, V        as for dblk_lmhead_confidence with M = B*L
 *   conf, argmax      fp32 / int32 [B][L] out: for each position masked at
 *                     the start of the call, the values of the last
 *                     iteration in which it was still masked (the same in
 *                     every iteration); other positions may be left
 *                     unchanged (with B*L >= 256 only masked rows go
 *                     through the LM head)
 *   tokens, mask      int32 / uint8 [B][L] in/out, as for dblk_threshold_commit
 *   threshold         fp32
 *   eos_id            < 0: no EOS handling; >= 0: as dblk_threshold_commit_eos
 *   max_iters         iterations enqueued; <= 0 selects L
 *   commit_iter       int32 [B][L] out or NULL: iteration index (0-based) at
 *                     which each position was committed, -1 if it was not
 *                     committed by this call
 *   n_iters           int32 [B] out or NULL: iterations in which the sequence
 *                     still had masked positions (= 1 + its last commit's index)
 *   finished          uint8 [B] out or NULL (EOS handling only)
 * workspace >= dblk_decode_block_workspace_size(args) bytes, 256-byte
 * aligned, zero-filled before first use; it holds the attention and LM-head
 * workspaces and the per-sequence masked counts that the skipping reads.
 * The call enqueues a fixed sequence of kernels and allocates nothing, so it
 * can be captured into a HIP graph and replayed.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void *q, *k_prefix, *v_prefix, *k_block, *v_block, *k_suffix, *v_suffix;
  const int32_t *prefix_len;
  int32_t B, H, L, D, P_cap, S, S_cap;
  float scale;
  void *attn_out;
  const void *h, *W;
  int32_t d, V;
  float *conf;
  int32_t *argmax;
  int32_t *tokens;
  uint8_t *mask;
  float threshold;
  int32_t eos_id;
  int32_t max_iters;
  int32_t *commit_iter;
  int32_t *n_iters;
  uint8_t *finished;
} dblk_decode_args;

size_t dblk_decode_block_workspace_size(const dblk_decode_args *args);

int32_t dblk_decode_block(const dblk_decode_args *args, void *workspace,
                          size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * dblk_decode_block_run -- one block decoded to completion with iterations
 * enqueued `chunk` at a time, one chunk ahead of the host's completion check
 * (dInfer's loop unrolling, the framework overview on its page: no stream
 * bubble between iterations, and only the iterations of about two chunks
 * skipped after the block is complete, instead of all the remaining ones).
 *
 * Chunk c enqueues iterations [c*chunk, (c+1)*chunk) exactly as
 * dblk_decode_block does (the first chunk also the initialisation), then
 * copies the number of sequences that still have a masked position into
 * host_active[c % 2].  Chunk c + 1 is queued before the host waits for chunk
 * c; once a chunk reports 0, or max_iters iterations (<= 0: L) are enqueued,
 * no further chunk is queued.
 *
 * Unlike every other call this one WAITS on the host for device progress.
 * It returns when the block is complete (or the iteration cap is reached);
 * the one chunk queued behind the last checked one may still be running (all
 * of its kernels skip), so synchronise the stream before reading results.
 * Not capturable into a graph.
 *
 *   args, workspace, workspace_bytes   as for dblk_decode_block
 *   chunk            iterations per chunk, >= 1
 *   host_active      int32 [2], pinned host memory (hipHostMalloc), written
 *                    by the stream, read by this call; it must stay allocated
 *                    until the stream has finished the call's work (the last
 *                    queued chunk still copies into it after the return)
 *   iters_enqueued   host int32 out, or NULL: iterations enqueued in total
 * ---------------------------------------------------------------------- */
int32_t dblk_decode_block_run(const dblk_decode_args *args, int32_t chunk,
                              int32_t *host_active, void *workspace,
                              size_t workspace_bytes, void *stream,
                              int32_t *iters_enqueued);

/* ------------------------------------------------------------------------
 * dblk_cache_append -- dual-cache upkeep when a block is complete: its keys
 * and values become prefix rows of the next block.
 *
 * For every b with P_b = prefix_len[b] (clamped to [0, P_cap]) and
 * P_b + L <= P_cap, and every head h:
 *   k_prefix[b][h][P_b + j] = k_block[b][h][j],  v likewise,  j < L
 *   prefix_len[b] = P_b + L,  appended[b] = L
 * A sequence whose prefix would exceed P_cap is left unchanged
 * (prefix_len[b] = P_b, appended[b] = 0).  The suffix of the next block is
 * the old suffix advanced by L rows: pass k_suffix + L*D with the same
 * S_cap to dblk_attend, no copy.
 *
 *   k_prefix, v_prefix  bf16 [B][H][P_cap][D] in/out
 *   k_block,  v_block   bf16 [B][H][L][D] in; must not overlap the prefix
 *   prefix_len          int32 [B] in/out (device)
 *   0 <= B <= 65535, 1 <= H <= 65535, D in {64, 128}, 1 <= L <= 4096, P_cap >= L
 *   appended            int32 [B] out, or NULL
 * ---------------------------------------------------------------------- */
int32_t dblk_cache_append(void *k_prefix, void *v_prefix,
                          const void *k_block, const void *v_block,
                          int32_t *prefix_len, int32_t B, int32_t H, int32_t L,
                          int32_t D, int32_t P_cap, int32_t *appended, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DBLOCK_H_ */
