// kda_internal.h -- declarations shared by the host layer (kda_api.cpp) and the
// HIP kernel translation units of the KDA library.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "kda.h"

namespace kda {

// Runs `set` (kernel attribute calls, idempotent) the first time a call site
// reaches it on each device; `done` holds one bit per device id.  Two threads
// may both run `set` for the same device, which is harmless.
template <typename F>
hipError_t once_per_device(std::atomic<uint64_t>& done, F&& set) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  const hipError_t e = set();
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Launch the single-token decode kernel.  Shapes are validated by the caller.
hipError_t launch_decode(const kda_desc_t& d, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float* state, void* o,
                         hipStream_t stream);

// Chunkwise prefill.  Workspace size and launch plan live in kda_chunk.hip.
// chunk_states (or nullptr): the state entering every chunk slot, [slot][H]
// of D x D in the element type of q/k/v (bf16 or fp32), slice-blocked as sblk
// (kda_chunk_common.h) lays it out, for the backward; only with o == nullptr
// (the pass that writes states produces no output; both set is an invalid
// value).
size_t chunk_workspace_bytes(const kda_desc_t& d);
hipError_t launch_chunk_fwd(const kda_desc_t& d, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* init_state,
                            const int32_t* cu_seqlens, void* o, float* final_state,
                            float* state_ckpt, void* chunk_states, void* workspace,
                            hipStream_t stream);
// States-only chunkwise pass whose chunk records come from the caller: for
// each segment of chunk slots [s0, s1), stage(ctx, s0, s1, recs, stream)
// launches, on `stream`, kernels that write the records of those slots (the
// blocks a state pass without output reads: K~, -Wk, U, e^gamma) at `recs`,
// head h and slot s at recs + (h (s1 - s0) + s - s0) record bytes; the state
// pass then runs over them.  chunk_states and the workspace are as for
// launch_chunk_fwd without o.
typedef hipError_t (*chunk_record_stage_fn)(void* ctx, int64_t s0, int64_t s1, char* recs,
                                            hipStream_t stream);
hipError_t launch_chunk_states(const kda_desc_t& d, const float* init_state,
                               const int32_t* cu_seqlens, void* chunk_states, void* workspace,
                               chunk_record_stage_fn stage, void* stage_ctx, hipStream_t stream);
// Chunk slots of a batch (dense: B * ceil(T/64); varlen: an upper bound that
// does not read cu_seqlens, T/64 + N).
int64_t chunk_slot_bound(const kda_desc_t& d, bool varlen);

// Prefill without a caller workspace (kda_chunk_fwd_noalloc): scratch in a
// fixed device array of kNoAllocScratchBytes per device.  noalloc_seg_slots
// is the segment length (chunk slots) that fits the array, 0 if even the
// smallest segment does not (then noalloc_min_bytes says what it would need).
constexpr size_t kNoAllocScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
int64_t noalloc_seg_slots(const kda_desc_t& d);
int64_t noalloc_min_bytes(const kda_desc_t& d);
hipError_t launch_chunk_fwd_noalloc(const kda_desc_t& d, const void* q, const void* k,
                                    const void* v, const float* g, const float* beta,
                                    const float* init_state, const int32_t* cu_seqlens, void* o,
                                    float* final_state, float* state_ckpt, hipStream_t stream);

// Prefill with the ShortConv + Swish prologue (width 4) fused into the
// intra-chunk kernel's loads: x[t] are the prologue inputs of q, k, v
// ([B, T, H, d] as q, k, v are for launch_chunk_fwd); w, bias, state_in,
// state_out per tensor as for launch_short_conv at width 4 (C = H d).  The
// workspace is launch_chunk_fwd's.  Shapes are validated by the caller.
hipError_t launch_chunk_fwd_conv(const kda_desc_t& d, const void* const x[3],
                                 const float* const w[3], const float* const bias[3],
                                 const float* const state_in[3], float* const state_out[3],
                                 const float* g, const float* beta, const float* init_state,
                                 const int32_t* cu_seqlens, void* o, float* final_state,
                                 float* state_ckpt, void* workspace, hipStream_t stream);
// The carried-out prologue inputs of width 4 (kda_conv.hip), for each of
// three tensors whose state_out is not null: state_out[n, c, :] = the last 3
// entries of sequence n's input preceded by state_in[n, c, :] (or zeros); x
// is [B, T, C] (dense, B = num_seqs) or packed (cu != null).  One launch.
hipError_t launch_conv_state_out(int64_t seqlen, int32_t num_seqs, int32_t channels,
                                 int32_t dtype, const void* const x[3],
                                 const float* const state_in[3], float* const state_out[3],
                                 const int32_t* cu, hipStream_t stream);

// Chunkwise backward (kda_chunk_bwd.hip).
size_t chunk_bwd_workspace_bytes(const kda_desc_t& d);
hipError_t launch_chunk_bwd(const kda_desc_t& d, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* init_state,
                            const int32_t* cu_seqlens, const void* d_o, const float* d_final,
                            void* dq, void* dk, void* dv, float* dg, float* dbeta,
                            float* d_init, uint32_t* range_flag, void* workspace,
                            hipStream_t stream);

// ShortConv + Swish prologue.  Shapes are validated by the caller.
struct kda_conv_args {
  int32_t batch;
  int64_t seqlen;
  int32_t num_seqs;
  int32_t channels;
  int32_t width;
  int32_t dtype;
  const void* x;
  const float* w;
  const float* bias;
  const float* state_in;
  const int32_t* cu;
  void* y;
  float* state_out;
};
hipError_t launch_short_conv(const kda_conv_args& a, hipStream_t stream);
// Largest seqlen for which one thread covers a whole sequence (the carried
// state may then be updated in place).
constexpr int64_t kConvInPlaceMaxTokens = 32;

// Output epilogue: head-wise RMSNorm x sigmoid gate over [rows, dv].
hipError_t launch_gate_norm(int64_t rows, int dv, int dtype, const void* o, const void* z,
                            const float* w, float eps, void* y, hipStream_t stream);

}  // namespace kda
