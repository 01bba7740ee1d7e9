// kda_chunk.hip -- chunkwise prefill (placeholder until the kernels land).
#include "kda_internal.h"

namespace kda {

size_t chunk_workspace_bytes(const kda_desc_t& d) { (void)d; return 0; }

hipError_t launch_chunk_fwd(const kda_desc_t&, const void*, const void*, const void*,
                            const float*, const float*, const float*, const int32_t*, void*,
                            float*, float*, void*, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace kda
