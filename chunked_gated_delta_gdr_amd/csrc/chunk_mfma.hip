// bf16 matrix-core chunk kernel (placeholder until the MFMA path lands).
#include "common.h"

namespace gdr {

bool chunk_mfma_supports(const gdr_desc_t &, const gdr_inputs_t &, const float *, const void *,
                         const float *) {
  return false;
}

hipError_t launch_chunk_mfma(const ChunkArgs &, hipStream_t) { return hipErrorInvalidConfiguration; }

}  // namespace gdr
