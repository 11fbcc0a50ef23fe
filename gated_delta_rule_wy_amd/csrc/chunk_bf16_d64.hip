// Prefill kernels for bf16 inputs and d_k = 64.
#include "chunk_bwd_impl.hpp"

namespace gdn2 {
template hipError_t dispatch_dv<uint16_t, _Float16, 64>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
template hipError_t dispatch_bwd<uint16_t, _Float16, 64>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);
}
