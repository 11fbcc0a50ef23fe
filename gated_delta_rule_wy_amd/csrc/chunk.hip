// Chunkwise prefill: workspace planning, the packed-batch chunk table and
// the dispatch over input type and head sizes. The kernels are in
// chunk_impl.hpp; each (input type, d_k) is instantiated in a translation
// unit of its own (chunk_<type>_d<d_k>.hip) so they compile in parallel.
#include "chunk_impl.hpp"

namespace gdn2 {

extern template hipError_t dispatch_dv<uint16_t, _Float16, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<uint16_t, _Float16, 64>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<uint16_t, _Float16, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<float, float, 16>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<float, float, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<float, float, 64>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<float, float, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);

// chunk offsets for packed batches: co[i] = sum_{i'<i} ceil(len_i'/64), capped
__global__ __launch_bounds__(1024) void chunk_plan_kernel(const int32_t *__restrict__ cu, int N, int T,
                                                          int max_chunks, int32_t *__restrict__ co)
{
    __shared__ int part[1024];
    const int t = threadIdx.x;
    const int per = (N + 1023) / 1024;
    const int i0 = t * per, i1 = min(N, i0 + per);
    int sum = 0;
    for (int i = i0; i < i1; ++i) {
        const int a = clampi(cu[i], 0, T), b = clampi(cu[i + 1], a, T);
        sum += (b - a + 63) >> 6;
    }
    part[t] = sum;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int x = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += x;
        __syncthreads();
    }
    int run = part[t] - sum;   // exclusive prefix
    for (int i = i0; i < i1; ++i) {
        co[i] = min(run, max_chunks);
        const int a = clampi(cu[i], 0, T), b = clampi(cu[i + 1], a, T);
        run += (b - a + 63) >> 6;
    }
    if (t == 1023) co[N] = min(part[1023], max_chunks);
}

// ---------------------------------------------------------------------------
static size_t blk_bytes(int dk, bool bf16)
{
    switch (dk) {
    case 16: return bf16 ? 0 : Blk<float, 16>::bytes;
    case 32: return bf16 ? Blk<_Float16, 32>::bytes : Blk<float, 32>::bytes;
    case 64: return bf16 ? Blk<_Float16, 64>::bytes : Blk<float, 64>::bytes;
    case 128: return bf16 ? Blk<_Float16, 128>::bytes : Blk<float, 128>::bytes;
    }
    return 0;
}

bool chunk_plan(int B, int T, int N, int H, int dk, int dv, bool bf16, bool varlen, ChunkPlan *p)
{
    if (dv != 16 && dv != 32 && dv != 64 && dv != 128) return false;
    const size_t bb = blk_bytes(dk, bf16);
    if (!bb) return false;
    const long long per = ((long long)T + 63) / 64;
    const long long mc = varlen ? per + N : per * B;
    if (mc * H > 0x7fffffffLL) return false;
    const long long chains = (long long)(varlen ? N : B) * H;
    p->max_chunks = (int)mc;
    p->plan_bytes = varlen ? ((size_t)(N + 1) * 4 + 255) / 256 * 256 : 0;
    p->prog_bytes = ((size_t)chains * 4 + 255) / 256 * 256;
    p->block_bytes = bb;
    p->total_bytes = p->plan_bytes + p->prog_bytes + (size_t)mc * H * bb;
    return true;
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st)
{
    if (a.cu_seqlens) {
        prof_before("gdn2_chunk_plan", st);
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.N, a.T,
                           p.max_chunks, (int32_t *)a.workspace);
        prof_after(st);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (a.bf16) {
        switch (a.dk) {
        case 32: return dispatch_dv<uint16_t, _Float16, 32>(a, p, st);
        case 64: return dispatch_dv<uint16_t, _Float16, 64>(a, p, st);
        case 128: return dispatch_dv<uint16_t, _Float16, 128>(a, p, st);
        }
    } else {
        switch (a.dk) {
        case 16: return dispatch_dv<float, float, 16>(a, p, st);
        case 32: return dispatch_dv<float, float, 32>(a, p, st);
        case 64: return dispatch_dv<float, float, 64>(a, p, st);
        case 128: return dispatch_dv<float, float, 128>(a, p, st);
        }
    }
    return hipErrorInvalidValue;
}

} // namespace gdn2
