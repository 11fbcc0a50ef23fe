// Prefill kernels for fp32 inputs and d_k = 128.
#include "chunk_bwd_impl.hpp"

namespace gdn2 {
template hipError_t dispatch_dv<float, float, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
template hipError_t dispatch_bwd<float, float, 128>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);
}
