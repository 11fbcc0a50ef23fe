// Chunk-size variants (32- and 128-token chunks) of the prefill for bf16 inputs, d_k = 32.
#include "chunk_cs_impl.hpp"

namespace gdn2 {
template hipError_t dispatch_dv_cs<uint16_t, _Float16, 32, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
template hipError_t dispatch_dv_cs<uint16_t, _Float16, 32, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
} // namespace gdn2
