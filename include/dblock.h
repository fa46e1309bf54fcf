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
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *     never allocates, frees or copies to the host, and keeps no global state.
 *   - bf16 means IEEE-754 binary32 truncated to its upper 16 bits (bfloat16),
 *     stored as 2-byte little-endian words.  All bf16 tensors are dense,
 *     row-major, with the innermost dimension contiguous.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise with the host.
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

/* ABI version of this header: 1. */
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
 * (Dual cache: the README's KVCacheFactory('dual'); bidirectional attention of
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
 *   v_suffix     bf16 [B][H][S][D]        cached suffix; may be NULL when S == 0
 *   prefix_len   int32 [B] device, or NULL (then P_b = P_cap for every b);
 *                values outside [0, P_cap] are clamped into it by the kernel
 *   0 <= B <= 65535, 1 <= H <= 65535, D in {64, 128}, L in {16, 32, ..., 128}, P_cap >= 0,
 *   S >= 0, P_cap + L + S <= 65536
 *   scale        score scale, finite and >= 0; 0 selects 1/sqrt(D)
 *   out          bf16 [B][L][H][D]; must not alias any input
 *   workspace    >= dblk_attend_workspace_size(...) bytes (fp32 split
 *                partials), 256-byte aligned
 * B == 0 is a valid no-op.
 * ---------------------------------------------------------------------- */
size_t dblk_attend_workspace_size(int32_t B, int32_t H, int32_t L, int32_t D,
                                  int32_t P_cap, int32_t S);

int32_t dblk_attend(const void *q,
                    const void *k_prefix, const void *v_prefix,
                    const void *k_block, const void *v_block,
                    const void *k_suffix, const void *v_suffix,
                    const int32_t *prefix_len,
                    int32_t B, int32_t H, int32_t L, int32_t D,
                    int32_t P_cap, int32_t S, float scale,
                    void *out, void *workspace, size_t workspace_bytes,
                    void *stream);

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
 *   M >= 0, d multiple of 64 with 64 <= d <= 16384, 1 <= V <= 2^30
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
 * (the README's ThresholdParallelDecoder(0, threshold=0.9, ...)).
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

#ifdef __cplusplus
}
#endif

#endif /* DBLOCK_H_ */
