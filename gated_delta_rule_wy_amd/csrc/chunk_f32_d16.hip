// Prefill kernels for fp32 inputs and d_k = 16.
#include "chunk_impl.hpp"

namespace gdn2 {
template hipError_t dispatch_dv<float, float, 16>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
}
