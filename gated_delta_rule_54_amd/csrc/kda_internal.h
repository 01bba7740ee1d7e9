// kda_internal.h -- declarations shared by the host layer (kda_api.cpp) and the
// HIP kernel translation units of the KDA library.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda.h"

namespace kda {

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
// Chunk slots of a batch (dense: B * ceil(T/64); varlen: an upper bound that
// does not read cu_seqlens, T/64 + N).
int64_t chunk_slot_bound(const kda_desc_t& d, bool varlen);

// Chunkwise backward (kda_chunk_bwd.hip).
size_t chunk_bwd_workspace_bytes(const kda_desc_t& d);
hipError_t launch_chunk_bwd(const kda_desc_t& d, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* init_state,
                            const int32_t* cu_seqlens, const void* d_o, const float* d_final,
                            void* dq, void* dk, void* dv, float* dg, float* dbeta,
                            float* d_init, void* workspace, hipStream_t stream);

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
