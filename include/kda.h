/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention operator.
 *
 * Pages cited (by title and section):
 *   [XT] xutianle.me, "Kimi Linear：用 KDA 重写长上下文注意力"
 *   [XD] xiudou.site, "Kimi Delta Attention：把遗忘门做到每个通道"
 *   [DS] docsaid.org, "Kimi Linear" (逐通道的遺忘)
 *   [RM] remio.ai, "Kimi Linear 以自己的方式击败了全注意力"
 *
 * The operator, per (sequence, head), token t = 1..L:
 *   S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_(t-1) + beta_t k_t v_t^T
 *   o_t = scale * S_t^T q_t
 * with S a d_k x d_v matrix whose ROWS are key channels, alpha_t = exp(g_t) a
 * per-channel gate in (0,1] held in log space (g <= 0), beta_t a scalar per
 * token and head, and q, k L2-normalised per head when qk_l2norm is set
 * (q / sqrt(sum q^2 + 1e-6)).  [XT §3 boxed KDA update and its decay-then-
 * correct split; XT §1 read-out o_t = S_t^T q_t; XT §6.2 L2 normalisation;
 * DS §"KDA：把衰減拆到每個通道" state orientation and its two-channel table]
 *
 * Conventions common to every entry point:
 *  - Tensor pointers are DEVICE pointers to dense row-major arrays (last
 *    index fastest).  Alignment: kda_chunk_fwd needs q, k, v, g, o and the
 *    workspace 16-byte aligned and every other pointer 4-byte aligned;
 *    kda_decode_step needs the state 16-byte aligned and every other pointer
 *    aligned to its element size.  The caller owns every buffer; the
 *    library keeps no pointer after a call returns and never allocates device
 *    memory (scratch comes in through `workspace`, or, for
 *    kda_chunk_fwd_noalloc, is a fixed device array the library holds).
 *  - Calls are asynchronous on `stream`; outputs are valid once the stream
 *    has reached the point of the call.  Host-side validation never
 *    synchronises the device; on any error nothing is launched, the status is
 *    returned and kda_last_error() holds a message.  Launch failures return
 *    KDA_ERR_HIP with the HIP error string.
 *  - Results are bitwise deterministic for fixed inputs and descriptor.
 *  - NaN or Inf in inputs propagate to outputs; no kernel waits on data, so
 *    none can hang on them.
 *  - g > 0 (alpha > 1) is outside the operator's domain; it is not checked on
 *    the device and its results are unspecified (no fault, no hang).
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 7

typedef enum {
  KDA_OK = 0,
  KDA_ERR_INVALID_ARGUMENT = 1,   /* null/misaligned pointer, bad shape or value */
  KDA_ERR_UNSUPPORTED = 2,        /* valid but not implemented (e.g. dk = 96)   */
  KDA_ERR_WORKSPACE_TOO_SMALL = 3,
  KDA_ERR_HIP = 4                 /* a HIP runtime call or launch failed         */
} kda_status_t;

/* Element type of q, k, v and o.  g, beta and every state are always fp32. */
typedef enum { KDA_DTYPE_F32 = 0, KDA_DTYPE_BF16 = 1 } kda_dtype_t;

/* Problem descriptor (plain old data, passed by pointer).
 *   batch      B.  Dense layout: inputs are [B, T, H, d].  Must be 1 when
 *              cu_seqlens is given (varlen packing).
 *   seqlen     T: tokens per sequence (dense) or total packed tokens (varlen).
 *              T = 0 is legal (nothing to compute; final = init).
 *   num_seqs   N: = B (dense) or len(cu_seqlens) - 1 (varlen).  For decode,
 *              the number of independent sequences.
 *   heads      H >= 1.
 *   dk, dv     key / value head dims; supported: dk = dv, 64 or 128.
 *   dtype      element type of q, k, v, o.
 *   chunk      must be 64 (the chunk size the pages' FLOP model uses,
 *              [XT §5]).
 *   qk_l2norm  1: normalise q and k inside the operator; 0: use as given.
 *   scale      o = scale * S^T q (the pages use no query scale: 1.0).
 *   ckpt_every 0 = no checkpoints; else a positive multiple of `chunk` that
 *              divides T; dense layout only.
 *   gate_per_head  0 (KDA): g holds one log-gate per key channel, [.., dk].
 *              1 (Gated DeltaNet): g holds one log-gate per (token, head),
 *              broadcast over the key channels, [..] without the dk axis.
 *              [XT §3: GDN's scalar forget gate is the special case of KDA's
 *              per-channel gate with all channels equal.]
 */
typedef struct {
  int32_t batch;
  int32_t num_seqs;
  int64_t seqlen;
  int32_t heads;
  int32_t dk;
  int32_t dv;
  int32_t dtype;      /* kda_dtype_t */
  int32_t chunk;
  int32_t qk_l2norm;
  float scale;
  int32_t gate_per_head;  /* 0: per-channel gates; 1: one gate per (token, head) */
  int64_t ckpt_every;
} kda_desc_t;

/* Bytes of device workspace kda_chunk_fwd needs for this descriptor (an upper
 * bound that does not read cu_seqlens).  Returns 0 for an invalid or
 * unsupported descriptor (kda_last_error() then says why).  The workspace is
 * scratch: its contents on entry do not matter and are undefined on exit. */
size_t kda_chunk_fwd_workspace_bytes(const kda_desc_t* desc);

/* Chunkwise prefill.  [XT §5: chunk-parallel within a chunk, recurrent across
 * chunks; the UT transform turns a chunk of rank-1 transitions into dense
 * products; the output adds an inter-chunk read of the entering state to an
 * intra-chunk read of earlier in-chunk pseudo-values.  XT §4: the shared-key
 * DPLR structure this relies on.]
 *   q, k       [B, T, H, dk]  dtype          (raw; normalised inside if qk_l2norm)
 *   v          [B, T, H, dv]  dtype
 *   g          [B, T, H, dk]  fp32, log of the per-channel forget gate, <= 0
 *              ([B, T, H] when desc->gate_per_head = 1)
 *   beta       [B, T, H]      fp32
 *   init_state [N, H, dk, dv] fp32, or NULL for zeros
 *   cu_seqlens [N + 1] int32 device array, cu[0] = 0, non-decreasing,
 *              cu[N] = T; NULL for the dense layout.  Sequences are
 *              independent; chunks restart at every sequence start and never
 *              straddle two sequences.  Zero-length sequences are allowed
 *              (their final state equals their initial state).  The values
 *              are not checked on the host (that would need a sync).
 *   o          [B, T, H, dv]  dtype, output; must not alias an input.
 *   final_state [N, H, dk, dv] fp32 output or NULL; may equal init_state
 *              (each (sequence, head) state is read before it is written).
 *   state_ckpt [B, T / ckpt_every, H, dk, dv] fp32 output or NULL; slot j is
 *              the state after (j + 1) * ckpt_every tokens of sequence b.
 *   workspace  device scratch of at least kda_chunk_fwd_workspace_bytes().
 */
kda_status_t kda_chunk_fwd(const kda_desc_t* desc, const void* q, const void* k,
                           const void* v, const float* g, const float* beta,
                           const float* init_state, const int32_t* cu_seqlens, void* o,
                           float* final_state, float* state_ckpt, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Scratch (bytes, per device) that kda_chunk_fwd_noalloc holds. */
#define KDA_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* Largest token row of kda_short_conv_swish, in bytes (channels x element
 * size): 8,388,608 fp32 or 16,777,216 bf16 channels. */
#define KDA_CONV_MAX_ROW_BYTES (1 << 25)

/* kda_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace and allocates nothing: its scratch (chunk records,
 * carried states, varlen map) is a fixed array of KDA_NOALLOC_SCRATCH_BYTES
 * (64 MiB) that the library holds on every device it runs on until the
 * process ends, and the chunk records are processed in segments small enough
 * to fit it.  Arguments, layouts, alignment and results are those of
 * kda_chunk_fwd, and the outputs are bitwise identical to it.  A descriptor
 * whose scratch need exceeds the array (the carried states of many
 * sequences x heads, or records of one 8-chunk segment that do not fit)
 * returns KDA_ERR_WORKSPACE_TOO_SMALL and launches nothing.  Every call on a
 * device shares that device's array and leaves its contents behind (nothing
 * in it needs to start at zero): calls that overlap on one device -- other
 * streams, other threads -- race and must be serialised by the caller. */
kda_status_t kda_chunk_fwd_noalloc(const kda_desc_t* desc, const void* q, const void* k,
                                   const void* v, const float* g, const float* beta,
                                   const float* init_state, const int32_t* cu_seqlens, void* o,
                                   float* final_state, float* state_ckpt, hipStream_t stream);

/* Prefill with the ShortConv + Swish prologue fused into the operator's
 * loads.  [XT §6 layer diagram: the q, k, v projections pass ShortConv ->
 * Swish before the operator; XT §6.1; XD preprocessing list.]  The results
 * (o, final_state, state_ckpt, conv_state_out) are bitwise those of
 * kda_short_conv_swish at width 4 on each of xq, xk, xv followed by
 * kda_chunk_fwd on its three outputs; the prologue's outputs never go
 * through memory.  The filter width is 4 (every workload's); for another
 * width call the two steps.
 *   desc, g, beta, init_state, cu_seqlens, o, final_state, state_ckpt,
 *   workspace, workspace_bytes: as for kda_chunk_fwd (the same workspace
 *              size, kda_chunk_fwd_workspace_bytes)
 *   xq, xk, xv the prologue's inputs, each laid out as q / k / v of
 *              kda_chunk_fwd ([B, T, H, dk], dtype, 16-byte aligned), so a
 *              token row is the prologue's C = H * dk channels
 *   conv_w     3 pointers (q, k, v), each [C, 4] fp32, 16-byte aligned: the
 *              filters of kda_short_conv_swish
 *   conv_bias  NULL, or 3 pointers, each [C] fp32 or NULL (no bias)
 *   conv_state_in   NULL, or 3 pointers, each [N, C, 3] fp32 (the inputs
 *              before each sequence, oldest first) or NULL (zeros)
 *   conv_state_out  NULL, or 3 pointers, each [N, C, 3] fp32 or NULL: the
 *              last 3 inputs of each sequence, preceded by its carried-in
 *              ones (what decode continues from); each may equal the
 *              matching conv_state_in (only that overlap is checked) and must
 *              not otherwise overlap it or any other argument.
 * o must not alias xq, xk or xv.  Asynchronous on `stream`; on a validation
 * error nothing is launched.  Not for the backward: kda_chunk_bwd takes the
 * prologue's outputs q, k, v. */
kda_status_t kda_chunk_fwd_conv(const kda_desc_t* desc, const void* xq, const void* xk,
                                const void* xv, const float* const* conv_w,
                                const float* const* conv_bias,
                                const float* const* conv_state_in, float* const* conv_state_out,
                                const float* g, const float* beta, const float* init_state,
                                const int32_t* cu_seqlens, void* o, float* final_state,
                                float* state_ckpt, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Bytes of device workspace kda_chunk_bwd needs for this descriptor (an upper
 * bound that does not read cu_seqlens); 0 for an invalid or unsupported
 * descriptor.  It holds a forward workspace plus, per chunk slot and head,
 * the entering state and its gradient (2 x dk x dv elements of dtype: they
 * serve only as operands of products in that type, and in one fp32 row sum
 * of the gate gradient) and the reverse pass's operands ((dk + 64) x dk
 * elements of dtype), plus the exact path's fp32 scratch (at most 124 MB at
 * dk = 128). */
size_t kda_chunk_bwd_workspace_bytes(const kda_desc_t* desc);

/* Gradients of kda_chunk_fwd (training).  [XT §5: training runs the
 * chunkwise form; the pages give no gradient algorithm.  What is computed is
 * the exact vector-Jacobian product of the operator's map
 * (q, k, v, g, beta, init_state) -> (o, final_state) with the upstream
 * gradients (d_o, d_final_state), formed chunkwise: a forward pass that keeps
 * every chunk's entering state, a reverse pass over the chunks for the state
 * gradients, then every chunk's input gradients in parallel.]
 *   q, k, v, g, beta, init_state, cu_seqlens   as kda_chunk_fwd (the same
 *              values the forward ran on; desc->ckpt_every is ignored)
 *   d_o        [B, T, H, dv]  dtype, gradient of o
 *   d_final_state [N, H, dk, dv] fp32 or NULL (zero)
 *   dq, dk     [B, T, H, dk]  dtype, outputs (gradients of the raw q, k:
 *              through the L2 norm when qk_l2norm is set)
 *   dv         [B, T, H, dv]  dtype, output
 *   dg         fp32, output shaped like g ([B, T, H] when gate_per_head = 1:
 *              the sum over the key channels)
 *   dbeta      [B, T, H]      fp32, output
 *   d_init_state [N, H, dk, dv] fp32 output or NULL
 *   range_flag NULL, or one device uint32 (4-byte aligned): the call stores 1
 *              into it when some chunk lies beyond the fast exponent range
 *              below (its gradients then came from the slow exact kernel)
 *              and leaves it untouched otherwise; the caller clears it and
 *              reads it after the call (no host synchronisation inside the
 *              call)
 *   workspace  device scratch of at least kda_chunk_bwd_workspace_bytes().
 * Supported: bf16 with dk = dv = 64 or 128, fp32 with dk = dv = 64
 * (KDA_ERR_UNSUPPORTED otherwise).  Alignment as kda_chunk_fwd (d_o, dq, dk,
 * dv 16-byte; dg, dbeta 4-byte).  Outputs must not alias inputs.  Any
 * finite log-gates g <= 0 are supported ([XT §4] names the precision of the
 * chunk form's e^(-G) division as its concern).  Fast exponent range: within
 * each 64-token chunk, each half (32 tokens) decays by at most 80 per channel
 * (the sum of its log-gates >= -80; chunk decays down to about -160).  A
 * chunk beyond that takes an exact path (every gate factor from its own
 * exponent difference, fp32 arithmetic without matrix cores: much slower per
 * chunk) and range_flag is set. */
kda_status_t kda_chunk_bwd(const kda_desc_t* desc, const void* q, const void* k,
                           const void* v, const float* g, const float* beta,
                           const float* init_state, const int32_t* cu_seqlens, const void* d_o,
                           const float* d_final_state, void* dq, void* dk, void* dv, float* dg,
                           float* dbeta, float* d_init_state, uint32_t* range_flag,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* One decode step for N independent sequences, state updated in place.
 * [XT §3 decay-then-correct split; XT §5 recurrent form "S_(t-1) + current
 * token -> S_t + output"; XD §"从推理成本看它省在哪": a fixed-size state read
 * and written per step, independent of context length.]
 *   q, k, g    [N, H, dk]   (q, k dtype; g fp32; g is [N, H] when
 *              desc->gate_per_head = 1)
 *   v          [N, H, dv]   dtype
 *   beta       [N, H]       fp32
 *   state      [N, H, dk, dv] fp32, read and overwritten with S_t
 *   o          [N, H, dv]   dtype, output; must not alias an input.
 * desc->seqlen, batch and ckpt_every are ignored; num_seqs = N.
 * No workspace is needed. */
kda_status_t kda_decode_step(const kda_desc_t* desc, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, float* state,
                             void* o, hipStream_t stream);

/* ShortConv + Swish prologue, the step before q, k and v enter the
 * operator.  [XT §6 layer diagram: the q, k, v projections pass ShortConv ->
 * Swish (q, k then the L2 norm, which kda_chunk_fwd / kda_decode_step apply);
 * XT §6.1; XD preprocessing list: a small-window causal convolution mixing
 * each position with the few tokens just before it, then Swish.]  One filter
 * of `width` taps per channel; per sequence n, channel c, token t:
 *   y[t, c] = swish(bias[c] + sum_{i<width} w[c, i] * x~[t - (width-1) + i, c])
 * where x~ is the sequence's input preceded by state_in[n, c, :] (its previous
 * width-1 inputs, oldest first) or by zeros when state_in is NULL, and
 * swish(a) = a * sigmoid(a).  state_out[n, c, :] receives the last width-1
 * entries of x~.  For decode, call it with seqlen = 1 and batch = N.
 *   batch, seqlen, num_seqs  as in kda_desc_t: x, y are [B, T, C]; varlen
 *              (cu_seqlens != NULL) needs batch == 1, dense needs
 *              num_seqs == batch
 *   channels   C >= 1, a multiple of 8 (bf16) or 4 (fp32), and at most
 *              KDA_CONV_MAX_ROW_BYTES / element size (a token row's bytes fit
 *              the kernel's 32-bit offsets); for q/k/v of H heads, C = H * d
 *   width      1 ... 4 (the pages give none; 4 in every workload)
 *   dtype      element type of x and y
 *   x, y       device, 16-byte aligned; y must not overlap x
 *   w          [C, width] fp32 (16-byte aligned when width = 4); bias [C]
 *              fp32 or NULL
 *   state_in, state_out  [N, C, width-1] fp32 or NULL; state_out may equal
 *              state_in only in the dense layout with seqlen <= 32 (then one
 *              thread covers each sequence, e.g. decode steps); otherwise
 *              they must not overlap
 *   cu_seqlens as in kda_chunk_fwd (int32 [N+1], not checked on the host)
 * Asynchronous on `stream`; on a validation error nothing is launched. */
kda_status_t kda_short_conv_swish(int32_t batch, int64_t seqlen, int32_t num_seqs,
                                  int32_t channels, int32_t width, int32_t dtype, const void* x,
                                  const float* w, const float* bias, const float* state_in,
                                  const int32_t* cu_seqlens, void* y, float* state_out,
                                  hipStream_t stream);

/* Output epilogue: head-wise RMSNorm times a sigmoid output gate, the two
 * steps that follow the operator in the layer.  [XT §6 layer diagram: KDA ->
 * RMSNorm -> sigmoid output gate -> output projection; XT §6.3: the output is
 * normalised per head, then multiplied by a sigmoid gate computed from the
 * input.]  Per row r (one (token, head) pair) and channel j:
 *   y[r, j] = o[r, j] / sqrt(mean_i o[r, i]^2 + eps) * w[j] * sigmoid(z[r, j])
 *   rows     number of rows: B*T*H after kda_chunk_fwd, N*H after
 *            kda_decode_step (0 is a no-op)
 *   dv       64 or 128
 *   dtype    KDA_DTYPE_F32 or KDA_DTYPE_BF16, the element type of o, z and y
 *   o, z, y  [rows, dv] row-major, device, 16-byte aligned; y may equal o
 *            (in place) but must not otherwise overlap o or z
 *   w        [dv] fp32 device, one weight per channel shared by all heads,
 *            or NULL for weight 1
 *   eps      finite and >= 0 (the pages give none; 1e-6 in the workloads)
 * Asynchronous on `stream`; on a validation error nothing is launched. */
kda_status_t kda_output_gate_norm(int64_t rows, int32_t dv, int32_t dtype, const void* o,
                                  const void* z, const float* w, float eps, void* y,
                                  hipStream_t stream);

/* Static description of a status code. */
const char* kda_status_string(kda_status_t status);

/* Detail message for the last non-OK status returned on this thread ("" if
 * none).  The pointer stays valid until the next call on this thread. */
const char* kda_last_error(void);

/* KDA_ABI_VERSION of the built library. */
int kda_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
