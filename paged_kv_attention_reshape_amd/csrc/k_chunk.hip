// Prefill-chunk attention on the matrix cores (bf16 MFMA) -- see below.
#include "pa_internal.h"

namespace pa {

bool chunk_kernel_supports(bool /*bf16*/, int32_t /*D*/, int32_t /*G*/) { return false; }

hipError_t launch_chunk(const AttnArgs& a, hipStream_t /*s*/) {
  return a.ps.n_ck == 0 ? hipSuccess : hipErrorInvalidValue;
}

}  // namespace pa
