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
size_t chunk_workspace_bytes(const kda_desc_t& d);
hipError_t launch_chunk_fwd(const kda_desc_t& d, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, const float* init_state,
                            const int32_t* cu_seqlens, void* o, float* final_state,
                            float* state_ckpt, void* workspace, hipStream_t stream);

// Output epilogue: head-wise RMSNorm x sigmoid gate over [rows, dv].
hipError_t launch_gate_norm(int64_t rows, int dv, int dtype, const void* o, const void* z,
                            const float* w, float eps, void* y, hipStream_t stream);

}  // namespace kda
