// Chunkwise prefill: workspace planning, the packed-batch chunk table and
// the dispatch over input type and head sizes. The kernels are in
// chunk_impl.hpp; each (input type, d_k) is instantiated in a translation
// unit of its own (chunk_<type>_d<d_k>.hip) so they compile in parallel.
#include "chunk_bwd_impl.hpp"
#include "chunk_cs_impl.hpp"

namespace gdn2 {

extern template hipError_t dispatch_dv<uint16_t, _Float16, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<uint16_t, _Float16, 64>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<uint16_t, _Float16, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<float, float, 16>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<float, float, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<float, float, 64>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv<float, float, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);

extern template hipError_t dispatch_dv_cs<uint16_t, _Float16, 32, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<uint16_t, _Float16, 32, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<uint16_t, _Float16, 64, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<uint16_t, _Float16, 64, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<uint16_t, _Float16, 128, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<uint16_t, _Float16, 128, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<float, float, 16, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<float, float, 16, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<float, float, 32, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<float, float, 32, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<float, float, 64, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<float, float, 64, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<float, float, 128, 32>(const ChunkArgs &, const ChunkPlan &, hipStream_t);
extern template hipError_t dispatch_dv_cs<float, float, 128, 128>(const ChunkArgs &, const ChunkPlan &, hipStream_t);

// chunk offsets for packed batches: co[i] = sum_{i'<i} ceil(len_i' / 2^lc), capped
__global__ __launch_bounds__(1024) void chunk_plan_kernel(const int32_t *__restrict__ cu, int N, int T,
                                                          int max_chunks, int lc, int32_t *__restrict__ co)
{
    __shared__ int part[1024];
    const int t = threadIdx.x;
    const int per = (N + 1023) / 1024;
    const int i0 = t * per, i1 = min(N, i0 + per);
    int sum = 0;
    for (int i = i0; i < i1; ++i) {
        const int a = clampi(cu[i], 0, T), b = clampi(cu[i + 1], a, T);
        sum += (b - a + (1 << lc) - 1) >> lc;
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
        run += (b - a + (1 << lc) - 1) >> lc;
    }
    if (t == 1023) co[N] = min(part[1023], max_chunks);
}

// ---------------------------------------------------------------------------
// operand block bytes per (chunk, head); 0 where the prep does not support the chunk size
template <typename Op, int DK> static size_t blk_bytes_t(int chunk)
{
    switch (chunk) {
    case 32: return PrepCS<Op, DK, 32>::fits ? Blk<Op, DK, 32>::bytes : 0;
    case 64: return Blk<Op, DK, 64>::bytes;
    case 128: return PrepCS<Op, DK, 128>::fits ? Blk<Op, DK, 128>::bytes : 0;
    }
    return 0;
}

static size_t blk_bytes(int dk, bool bf16, int chunk)
{
    switch (dk) {
    case 16: return bf16 ? 0 : blk_bytes_t<float, 16>(chunk);
    case 32: return bf16 ? blk_bytes_t<_Float16, 32>(chunk) : blk_bytes_t<float, 32>(chunk);
    case 64: return bf16 ? blk_bytes_t<_Float16, 64>(chunk) : blk_bytes_t<float, 64>(chunk);
    case 128: return bf16 ? blk_bytes_t<_Float16, 128>(chunk) : blk_bytes_t<float, 128>(chunk);
    }
    return 0;
}

static size_t bblk_bytes(int dk, bool bf16)
{
    switch (dk) {
    case 16: return bf16 ? 0 : BBlk<float, 16>::bytes;
    case 32: return bf16 ? BBlk<_Float16, 32>::bytes : BBlk<float, 32>::bytes;
    case 64: return bf16 ? BBlk<_Float16, 64>::bytes : BBlk<float, 64>::bytes;
    case 128: return bf16 ? BBlk<_Float16, 128>::bytes : BBlk<float, 128>::bytes;
    }
    return 0;
}

bool chunk_bwd_plan(int B, int T, int N, int H, int dk, int dv, bool bf16, bool varlen, BwdPlan *p)
{
    if (!chunk_plan(B, T, N, H, dk, dv, bf16, varlen, &p->fwd)) return false;
    const size_t ops = bf16 ? 2 : 4;
    const auto r256 = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t slots = (size_t)p->fwd.max_chunks * H;
    p->bblock_bytes = bblk_bytes(dk, bf16);
    p->state_bytes = (size_t)dk * dv * ops;
    p->delta_bytes = (size_t)64 * dv * ops;
    p->off_bblocks = r256(p->fwd.total_bytes);
    p->off_states = p->off_bblocks + r256(slots * p->bblock_bytes);
    p->off_delta = p->off_states + r256(slots * p->state_bytes);
    p->off_grads = p->off_delta + r256(slots * p->delta_bytes);
    p->total_bytes = p->off_grads + r256(slots * p->state_bytes);
    return p->bblock_bytes != 0;
}

hipError_t launch_chunk_bwd(const ChunkBwdArgs &a, const BwdPlan &p, hipStream_t st)
{
    if (a.cu_seqlens) {
        prof_before("gdn2_chunk_plan", st);
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.N, a.T,
                           p.fwd.max_chunks, 6, (int32_t *)a.workspace);
        prof_after(st);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (a.bf16) {
        switch (a.dk) {
        case 32: return dispatch_bwd<uint16_t, _Float16, 32>(a, p, st);
        case 64: return dispatch_bwd<uint16_t, _Float16, 64>(a, p, st);
        case 128: return dispatch_bwd<uint16_t, _Float16, 128>(a, p, st);
        }
    } else {
        switch (a.dk) {
        case 16: return dispatch_bwd<float, float, 16>(a, p, st);
        case 32: return dispatch_bwd<float, float, 32>(a, p, st);
        case 64: return dispatch_bwd<float, float, 64>(a, p, st);
        case 128: return dispatch_bwd<float, float, 128>(a, p, st);
        }
    }
    return hipErrorInvalidValue;
}

bool chunk_plan(int B, int T, int N, int H, int dk, int dv, bool bf16, bool varlen, ChunkPlan *p, int chunk)
{
    if (dv != 16 && dv != 32 && dv != 64 && dv != 128) return false;
    const size_t bb = blk_bytes(dk, bf16, chunk);
    if (!bb) return false;
    const long long per = ((long long)T + chunk - 1) / chunk;
    const long long mc = varlen ? per + N : per * B;
    if (mc * H > 0x7fffffffLL) return false;
    const long long chains = (long long)(varlen ? N : B) * H;
    p->chunk = chunk;
    p->max_chunks = (int)mc;
    p->plan_bytes = varlen ? ((size_t)(N + 1) * 4 + 255) / 256 * 256 : 0;
    p->prog_bytes = ((size_t)chains * 4 + 255) / 256 * 256;
    p->block_bytes = bb;
    p->total_bytes = p->plan_bytes + p->prog_bytes + (size_t)mc * H * bb;
    return true;
}

static hipError_t launch_chunk_fwd_kernels(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st);
extern template hipError_t dispatch_bwd<uint16_t, _Float16, 32>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);
extern template hipError_t dispatch_bwd<uint16_t, _Float16, 64>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);
extern template hipError_t dispatch_bwd<uint16_t, _Float16, 128>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);
extern template hipError_t dispatch_bwd<float, float, 16>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);
extern template hipError_t dispatch_bwd<float, float, 32>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);
extern template hipError_t dispatch_bwd<float, float, 64>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);
extern template hipError_t dispatch_bwd<float, float, 128>(const ChunkBwdArgs &, const BwdPlan &, hipStream_t);

// Convolution history after a prefill (fused prologue): for each sequence
// and head, the last three raw inputs of q, k and v, reaching back into the
// history given at the start when the sequence is shorter than three tokens.
// One workgroup per (sequence, head) reads every value it writes before
// writing any, so the history out may alias the history in.
struct HistOut {
    const void *x[3];         // raw q, k, v [tokens][H][d]
    const void *in[3];        // history in [N][H][3][d] or null (zeros)
    void *out[3];             // history out
    int d[3];
};

template <typename In>
__global__ __launch_bounds__(256) void conv_hist_kernel(HistOut hp, Seqs sq, int H)
{
    constexpr int NT = 256, MAXE = 3 * 3 * 128 / NT + 1;
    const int nh = blockIdx.x, i = nh / H, h = nh % H, t = threadIdx.x;
    const int tb = sq.t0(i), L = sq.t1(i) - tb;
    const int e0 = 3 * hp.d[0], e1 = e0 + 3 * hp.d[1], e2 = e1 + 3 * hp.d[2];
    In val[MAXE];
#pragma unroll
    for (int m = 0; m < MAXE; ++m) {
        const int e = t + m * NT;
        if (e >= e2) break;
        const int x = e < e0 ? 0 : (e < e1 ? 1 : 2);
        const int le = e - (x == 0 ? 0 : (x == 1 ? e0 : e1)), d = hp.d[x];
        const int j = le / d, c = le % d, p = L - 3 + j;   // token p of the sequence
        const In *hin = (const In *)hp.in[x];
        if (p >= 0) val[m] = ((const In *)hp.x[x])[((size_t)(tb + p) * H + h) * d + c];
        else val[m] = hin ? hin[((size_t)nh * 3 + 3 + p) * d + c] : (In)0;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MAXE; ++m) {
        const int e = t + m * NT;
        if (e >= e2) break;
        const int x = e < e0 ? 0 : (e < e1 ? 1 : 2);
        const int le = e - (x == 0 ? 0 : (x == 1 ? e0 : e1)), d = hp.d[x];
        ((In *)hp.out[x])[(size_t)nh * 3 * d + le] = val[m];
    }
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st)
{
    hipError_t err = launch_chunk_fwd_kernels(a, p, st);
    if (err != hipSuccess || !a.pro.on || !a.pro.q.hist_out) return err;
    Seqs sq;
    sq.m.cu = a.cu_seqlens;
    sq.m.co = nullptr;
    sq.m.N = a.N;
    sq.m.T = a.T;
    sq.Ttot = a.cu_seqlens ? a.T : a.B * a.T;
    sq.max_chunks = p.max_chunks;
    sq.gates = 0;
    HistOut hp;
    const ConvTensor *ct[3] = {&a.pro.q, &a.pro.k, &a.pro.v};
    const void *xs[3] = {a.q, a.k, a.v};
    const int ds[3] = {a.dk, a.dk, a.dv};
    for (int x = 0; x < 3; ++x) {
        hp.x[x] = xs[x];
        hp.in[x] = ct[x]->hist_in;
        hp.out[x] = ct[x]->hist_out;
        hp.d[x] = ds[x];
    }
    prof_before("gdn2_conv_state", st);
    if (a.bf16) hipLaunchKernelGGL(conv_hist_kernel<uint16_t>, dim3(a.N * a.H), dim3(256), 0, st, hp, sq, a.H);
    else hipLaunchKernelGGL(conv_hist_kernel<float>, dim3(a.N * a.H), dim3(256), 0, st, hp, sq, a.H);
    prof_after(st);
    return hipGetLastError();
}

static hipError_t launch_chunk_fwd_kernels(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st)
{
    if (a.cu_seqlens) {
        prof_before("gdn2_chunk_plan", st);
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.N, a.T,
                           p.max_chunks, __builtin_ctz((unsigned)p.chunk), (int32_t *)a.workspace);
        prof_after(st);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (p.chunk != 64) {
        // chunk-size variants: per-channel gates, no prologue (checked by the caller)
        const bool c32 = p.chunk == 32;
        if (a.bf16) {
            switch (a.dk) {
            case 32: return c32 ? dispatch_dv_cs<uint16_t, _Float16, 32, 32>(a, p, st) : dispatch_dv_cs<uint16_t, _Float16, 32, 128>(a, p, st);
            case 64: return c32 ? dispatch_dv_cs<uint16_t, _Float16, 64, 32>(a, p, st) : dispatch_dv_cs<uint16_t, _Float16, 64, 128>(a, p, st);
            case 128: return c32 ? dispatch_dv_cs<uint16_t, _Float16, 128, 32>(a, p, st) : dispatch_dv_cs<uint16_t, _Float16, 128, 128>(a, p, st);
            }
        } else {
            switch (a.dk) {
            case 16: return c32 ? dispatch_dv_cs<float, float, 16, 32>(a, p, st) : dispatch_dv_cs<float, float, 16, 128>(a, p, st);
            case 32: return c32 ? dispatch_dv_cs<float, float, 32, 32>(a, p, st) : dispatch_dv_cs<float, float, 32, 128>(a, p, st);
            case 64: return c32 ? dispatch_dv_cs<float, float, 64, 32>(a, p, st) : dispatch_dv_cs<float, float, 64, 128>(a, p, st);
            case 128: return c32 ? dispatch_dv_cs<float, float, 128, 32>(a, p, st) : dispatch_dv_cs<float, float, 128, 128>(a, p, st);
            }
        }
        return hipErrorInvalidValue;
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
