// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn2 {

// Gate layouts (bit set = one value per token and head instead of one per channel)
enum : int { kGateB = 1, kGateW = 2, kGateAlpha = 4 };

// Short convolution of one raw tensor (fused prologue): taps [H*d][4] with
// tap 3 on the current token, optional bias [H*d], optional history in and
// out [N][H][3][d] (input dtype, oldest first). Device pointers.
struct ConvTensor {
    const float *w = nullptr;
    const float *bias = nullptr;
    const void *hist_in = nullptr;
    void *hist_out = nullptr;
};

// The fused prologue: q, k, v through their short convolutions, q and k to
// unit norm, b and w through the sigmoid. Off: the inputs are used as given.
struct Prologue {
    bool on = false;
    ConvTensor q, k, v;
};

struct DecodeArgs {
    const void *q, *k, *v, *b, *w;
    const float *log_alpha;
    float *S;
    void *o;
    int N, H, dk, dv;
    int gates;
    bool bf16;
    Prologue pro;
};

struct ChunkArgs {
    const void *q, *k, *v, *b, *w;
    const float *log_alpha;
    const float *S0;
    void *o;
    float *ST;
    const int32_t *cu_seqlens;   // device, or null for uniform batches
    int B, T, N, H, dk, dv;
    int gates;
    bool bf16;
    void *workspace;
    size_t workspace_bytes;
    Prologue pro;
};

// Workspace layout for one call (all offsets 256-byte aligned):
//   [0, plan_bytes)                      int32 chunk offsets co[N+1] (varlen only)
//   [plan_bytes, +prog_bytes)            int32 per-chain progress of the pass
//   [plan_bytes + prog_bytes, ...)       operand blocks, head-major:
//                                        block (h, j) at (h * max_chunks + j)
struct ChunkPlan {
    int chunk;                   // tokens per chunk: 64, or 32 / 128 (per-channel gates, no prologue)
    int max_chunks;              // grid bound on chunk ids
    size_t plan_bytes;           // bytes reserved for co[]
    size_t prog_bytes;           // bytes reserved for the progress counters
    size_t block_bytes;          // bytes per (chunk, head) operand block
    size_t total_bytes;
};

// Returns false when the sizes (or the chunk size) are not supported.
bool chunk_plan(int B, int T, int N, int H, int dk, int dv, bool bf16, bool varlen, ChunkPlan *p, int chunk = 64);

// Backward of the prefill (gradients of a loss through o and S_T).
struct ChunkBwdArgs {
    const void *q, *k, *v, *b, *w;
    const float *log_alpha;
    const float *S0;             // or null (zeros)
    const float *dO;             // [tokens][H][dv]
    const float *dST;            // [N][H][dk][dv] or null (zero)
    const int32_t *cu_seqlens;
    int B, T, N, H, dk, dv;
    bool bf16;
    float *dq, *dk_, *dv_, *dlog_alpha, *db, *dw;   // gradients, layouts of their inputs
    float *dS0;                  // or null
    void *workspace;
    size_t workspace_bytes;
    // which part runs: the whole backward (its own forward first), only the
    // training forward (o and S_T, keeping the operand blocks, S_c and Delta
    // in the workspace), or only the backward over what a training forward
    // kept there
    int part;                    // kBwdAll, kBwdForward, kBwdFromKept
    void *o;                     // kBwdForward: [tokens][H][dv] float
    float *ST;                   // kBwdForward: [N][H][dk][dv] float, or null
};
enum { kBwdAll = 0, kBwdForward = 1, kBwdFromKept = 2 };

// Backward workspace: the forward plan's regions, then (256-byte aligned)
//   backward operand blocks   [H * max_chunks] x bblock_bytes
//   chunk start states S_c    [H * max_chunks][dk][dv]  operand type, 16x16 accumulator-tile order
//   chunk Delta               [H * max_chunks][64][dv]  operand type, same order
//   chunk end gradients G     [H * max_chunks][dk][dv]  operand type, same order
struct BwdPlan {
    ChunkPlan fwd;
    size_t bblock_bytes, state_bytes, delta_bytes;   // per (chunk, head)
    size_t off_bblocks, off_states, off_delta, off_grads;
    size_t total_bytes;
};

bool chunk_bwd_plan(int B, int T, int N, int H, int dk, int dv, bool bf16, bool varlen, BwdPlan *p);
hipError_t launch_chunk_bwd(const ChunkBwdArgs &a, const BwdPlan &p, hipStream_t st);

// Optional per-kernel event timing (see gdn2_profile_begin): the launchers
// bracket every kernel launch with these; they do nothing unless enabled.
void prof_before(const char *kernel, hipStream_t st);
void prof_after(hipStream_t st);

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st);
hipError_t launch_chunk_fwd(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st);

} // namespace gdn2
