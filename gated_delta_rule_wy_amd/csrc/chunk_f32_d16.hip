// Prefill kernels for fp32 inputs and d_k = 16.
#include "chunk_bwd_impl.hpp"

namespace gdn2 {
template hipError_t dispatch_dv<float, float, 16>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
template hipError_t dispatch_bwd<float, float, 16>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);
}
