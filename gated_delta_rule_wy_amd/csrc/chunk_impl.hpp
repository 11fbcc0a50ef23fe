// Chunkwise (C = 64) WY-form prefill of the Gated Delta Rule-2 on gfx950.
//
// Per head and chunk of n <= 64 tokens starting from state S0 (dk x dv), with
// g_r = sum_{s<=r} log alpha_s per key channel and u_r = w_r * v_r, the
// token recurrence (snilld.dk, "Hvad Gated DeltaNet-2 ændrer", update
// equation) unrolls to the chunk form ("Hvad betyder det for træning og
// inferens": chunkwise WY form with the cumulative channel-wise decay folded
// into the rank-one erase factors):
//   A_rs  = sum_c b_rc k_rc k_sc e^{g_rc - g_sc}   (s < r)      Gram / erase
//   T     = (I + A)^{-1}                                         unit lower
//   W     = T E,   E_r = b_r * k_r * e^{g_r}                    WY factor
//   Delta = T U - W S0                                           corrected writes
//   P_rs  = sum_c q_rc k_sc e^{g_rc - g_sc}        (s <= r)
//   O     = Q+ S0 + P Delta,   Q+_r = q_r * e^{g_r}
//   S_n   = Diag(e^{g_n}) S0 + Khat^T Delta,   Khat_s = k_s * e^{g_n - g_s}
//
// Two kernels:
//  * chunk_prep: one workgroup per (chunk, head), all chunks in parallel.
//    Builds A and P on the matrix cores, inverts I + A in LDS, forms W, and
//    writes -W, Q+, Khat^T, P, T (as ready-to-use MFMA A-fragments) and
//    gamma = e^{g_n} to the workspace.
//  * chunk_pass: one workgroup per (sequence, head, 16-column slice of dv);
//    walks the sequence's chunks in order with its slice of the state in
//    registers (fp32). Value columns of S evolve independently because the
//    transition acts on the key axis only, which is what allows the slicing.
//
// Decay factoring. Exponent differences g_r - g_s (s <= r) are <= 0, but
// the products above are formed as (row factor) x (column factor).
//  * When the chunk's decay spread is moderate (half spread <= Lim::chunk,
//    every chunk of ordinary gating), all factors are taken around one
//    per-channel midpoint and stay within e^{+-Lim::chunk}.
//  * Otherwise row block R (rows 16R..16R+15) uses ref_R = g_{16R-1}
//    (0 for R = 0): off-diagonal blocks S < R use
//    e^{g_r - ref_R} * e^{ref_R - ref_{S+1}} * e^{ref_{S+1} - g_s}, every
//    factor <= 1, so nothing overflows whatever the decay; diagonal blocks
//    take factors around the block's middle row, bounded by e^{Lim::v}, and
//    a block whose decay spread exceeds that is computed exactly (pairwise
//    exponents) on the vector ALUs instead.
#pragma once

#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"

#include <algorithm>
#include <atomic>

#include <type_traits>

namespace gdn2 {

// Operand block written by the prep for one (chunk, head) of CS tokens;
// every fragment is 64 lanes x 16 bytes in the lane order the consumer loads it.
template <typename Op, int DK, int CS = 64> struct Blk {
    using M = Mma<Op>;
    static constexpr int KB = M::KB, NE = M::NE;
    static constexpr int NRB = CS / 16;   // 16-row tiles over chunk rows
    static constexpr int NKB = DK / KB;   // k-blocks over key channels
    static constexpr int NSB = CS / KB;   // k-blocks over chunk rows
    static constexpr int NCT = DK / 16;   // 16-row tiles over key channels
    static constexpr size_t FRAG = 64 * 16;
    static constexpr size_t oW = 0;                            // -W   [NRB][NKB] frags
    static constexpr size_t oQ = oW + NRB * NKB * FRAG;        // Q+   [NRB][NKB]
    static constexpr size_t oK = oQ + NRB * NKB * FRAG;        // Khat^T [NCT][NSB]
    // P and T are lower triangular: only the k-blocks sb <= sbmax(mt) of row
    // tile mt are stored, in row-tile order (tpos)
    static constexpr __host__ __device__ int sbmax(int mt) { return (16 * mt + 15) / KB; }
    // closed form (a loop over a runtime mt would stay a loop in the pass):
    // row tile m holds m / 2 + 1 stored k-blocks of 32 rows, m + 1 of 16
    static_assert(KB == 32 || KB == 16, "k-block of 16 or 32 rows");
    static_assert(CS == 32 || CS == 64 || CS == 128, "chunk of 32, 64 or 128 tokens");
    static constexpr __host__ __device__ int tpos(int mt, int sb) {
        if (CS == 64) return (KB == 32 ? (mt < 2 ? mt : 2 * mt - 2) : mt * (mt + 1) / 2) + sb;
        return (KB == 32 ? mt + (mt - 1) * (mt - 1) / 4 : mt * (mt + 1) / 2) + sb;
    }
    static constexpr int NTRI = tpos(NRB - 1, sbmax(NRB - 1)) + 1;   // stored fragments of P (and of T)
    static constexpr size_t oP = oK + NCT * NSB * FRAG;        // P    [NTRI]
    static constexpr size_t oT = oP + NTRI * FRAG;             // T    [NTRI]
    static constexpr size_t oG = oT + NTRI * FRAG;             // gamma float[DK]
    static constexpr size_t bytes = (oG + DK * 4 + 255) / 256 * 256;
};

// Bounds on decay-factor exponents: `v` for the diagonal blocks of the
// per-block factoring, `chunk` for the half spread of the chunk-wide one.
template <typename Op> struct Lim;
template <> struct Lim<_Float16> { static constexpr float v = 8.0f, chunk = 6.0f; };
template <> struct Lim<float> { static constexpr float v = 60.0f, chunk = 40.0f; };

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Column l = lane & 15 of the inverse of a 16x16 unit lower-triangular block
// I + A (A strictly lower, fp32, row stride lda, in LDS), by forward
// substitution on the whole wave: row x_r = [r == l] - sum_{s<r} A_rs x_s,
// lane l + 16 g summing the terms with s = g (mod 4), and the four 16-lane
// rows adding their partial sums with gfx950's lane swaps (permlane16_swap
// pairs rows 0-1 and 2-3, permlane32_swap the halves; each lane gets its own
// and its partner's value, and both orders of a two-term float sum agree, so
// every lane of a column holds the same x_r). Returns rows g + 4 j in x[j].
__device__ __forceinline__ void unit_lower_inverse16(const float *A, int lda, int lane, float x[4])
{
    const int l = lane & 15, g = lane >> 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float part = 0.f;
#pragma unroll
        for (int j = 0; j < r / 4 + 1; ++j) {
            const int s = g + 4 * j;
            if (s < r) part += A[r * lda + s] * x[j];
        }
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        part = __uint_as_float(a[0]) + __uint_as_float(a[1]);
        const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false, false);
        part = __uint_as_float(b[0]) + __uint_as_float(b[1]);
        const float xr = (r == l ? 1.f : 0.f) - part;
        if ((r & 3) == g) x[r >> 2] = xr;
    }
}

// ---------------------------------------------------------------------------

// Short convolution of one raw input (fused prologue), device pointers:
// taps [H*d][4] (tap 3 on the current token), bias [H*d] or null, history
// [N][H][3][d] in the input type (oldest first) or null for zeros.
struct ConvIn {
    const float *w;
    const float *bias;
    const void *hist;
};

// Token range and chunk ids with the host-unchecked preconditions made safe:
// offsets are clamped into [0, Ttot] and chunk ids capped at max_chunks.
struct Seqs {
    SeqMap m;
    int Ttot, max_chunks;
    int gates;   // kGateB / kGateW / kGateAlpha: per token-head instead of per channel
    __device__ __forceinline__ int t0(int i) const { return clampi(m.tok0(i), 0, Ttot); }
    __device__ __forceinline__ int t1(int i) const { return clampi(m.tok1(i), t0(i), Ttot); }
};

// Operand-block stores (whole fragments: each wave writes whole lines). The
// blocks are read only by later kernels, so they are written non-temporally:
// left dirty in the L2s, about a gigabyte of them would be written back
// while the next kernel's loads evict them (measured at T = 64K, H = 16: the
// pass 0.852 -> 0.823 ms, the backward's saving pass 1.05 -> 0.72 ms).
template <typename T> __device__ __forceinline__ void block_store(uint8_t *p, const T &x)
{
    __builtin_nontemporal_store(x, reinterpret_cast<T *>(p));
}

// ---------------------------------------------------------------------------
// Chunk preparation, one workgroup (4 waves) per (chunk, head).
//
// Fast path (the chunk's decay spread is moderate): every exponent is taken
// around one per-channel midpoint m = (g_first + g_last) / 2, so
//   E^m_r = b_r k_r e^{g_r - m},  Q^m_r = q_r e^{g_r - m},  K^m_s = k_s e^{m - g_s}
// are bounded by e^{LIMC} and A = E^m K^mT, P = Q^m K^mT need no per-tile
// scaling. Otherwise the per-block factoring described at the top of the file
// is used, with the exact pairwise path for diagonal blocks that need it.
// All global loads are issued up front and unconditionally (rows past the
// chunk's end are clamped and zeroed), so the wave waits once.
//
// PRO (fused prologue): q, k and b arrive raw. Each thread also loads the
// three rows before its first one (the previous chunk's, or the history
// before a sequence's start), applies the short convolution, scales q and k
// to unit norm (a sum over the row's lanes) and takes the sigmoid of b, all
// where the values are used.
template <typename In, typename Op, int DK, int G, bool PRO>
__global__ __launch_bounds__(256) void chunk_prep_kernel(
    const In *__restrict__ q, const In *__restrict__ k, const float *__restrict__ la,
    const In *__restrict__ b, Seqs sq, int H, uint8_t *__restrict__ ops, int *__restrict__ prog, int nprog,
    ConvIn cq, ConvIn ck)
{
    static_assert(!PRO || G == 0, "the prologue takes per-channel gates");
    using M = Mma<Op>;
    using L = Blk<Op, DK>;
    using frag = typename M::frag;
    using raw2 = typename Ld<In>::raw2;
    constexpr int KB = M::KB, NE = M::NE, NKB = L::NKB, NSB = L::NSB, NCT = L::NCT;
    constexpr int LDE = DK + 4;                 // row stride of the [64][DK] tiles
    constexpr int LDT = 64 + 4;                 // row stride of the [64][64] tiles
    constexpr int REG = 64 * (LDE > LDT ? LDE : LDT);
    constexpr int LDA = 65;
    constexpr int CP = DK / 2, NRG = 256 / CP, RPG = 64 / NRG;
    constexpr float LIM = Lim<Op>::v;
    constexpr float LIMC = Lim<Op>::chunk;

    __shared__ __attribute__((aligned(16))) Op sE[REG];   // E-side operand; later -W staging
    __shared__ __attribute__((aligned(16))) Op sQ[REG];   // Q-side operand; later P
    __shared__ __attribute__((aligned(16))) Op sK[REG];   // K-side operand; later T
    __shared__ float sA[64 * LDA];                        // A (fp32); early: cumsum scratch
    __shared__ float sTab[19 * DK];
    __shared__ int sFlag[5];                              // [0,4): exact diagonal blocks; [4]: slow chunk

    // Chunks are dealt last to first, all heads of a chunk together, so the
    // blocks the pass reads first are the ones written last (the most likely
    // to still sit in the last-level cache).
    const int t = threadIdx.x;
    const int h = (int)(blockIdx.x % (unsigned)H), j = sq.max_chunks - 1 - (int)(blockIdx.x / (unsigned)H);
    const int lane = t & 63, wv = wave_id(), m16 = lane & 15, g4 = lane >> 4;
    if (blockIdx.x == 0)
        for (int x = t; x < nprog; x += 256) prog[x] = 0;
    if (j >= min(sq.m.nchunks(), sq.max_chunks)) return;
    const int i = sq.m.seq_of(j);
    const int t0 = sq.t0(i) + 64 * (j - sq.m.chunk0(i));
    const int n = min(64, sq.t1(i) - t0);
    uint8_t *blk = ops + ((size_t)h * sq.max_chunks + j) * L::bytes;

    // tables (rows of DK floats): [0,4) Q+/E scale per row block; [4,8) Khat
    // scale per row block; [8,11) e^{ref_R - ref_{S+1}} for (R,S) = (2,0),
    // (3,0), (3,1); [11,15) e^{ref_R - mid_R}; [15,19) e^{mid_R - ref_{R+1}}.
    // The fast path uses rows 0 and 4 for every block.
    float *tExpRef = sTab, *tExpKh = sTab + 4 * DK, *tDec = sTab + 8 * DK;
    float *tDiagE = sTab + 11 * DK, *tDiagK = sTab + 15 * DK;

    // ---- stage 1: all loads, cumulative log-decay g, references ----
    const int cp = t % CP, rg = t / CP, c0 = 2 * cp, r0 = rg * RPG;
    float *sPart = sA;                  // [NRG][DK]
    float *sRef = sA + NRG * DK;        // [5][DK]: ref_0..ref_4 (ref_4 = g_n)
    float *sMid = sRef + 5 * DK;        // [4][DK]
    float *sG0 = sMid + 4 * DK;         // [DK]: g at the chunk's first row
    f2 gg[RPG];
    // raw k, b, q of the thread's rows; rows past the chunk's end are zeroed
    // where the values are used (rowf), not here, so no load waits early
    constexpr bool BSC = (G & kGateB) != 0;   // b: one value per token-head
    constexpr int XO = PRO ? 3 : 0;             // raw rows before the first (convolution)
    raw2 kr[RPG + XO], qr[RPG + XO];            // row r0 + x - XO in slot x
    typename std::conditional<BSC, In, raw2>::type br[RPG];
    auto bf2 = [&](int u) {
        if constexpr (BSC) { const float x = in2f<In>(br[u]); f2 r = {x, x}; return r; }
        else return Ld<In>::cvt2(br[u]);
    };
    auto rowf = [&](int u) { return r0 + u < n ? 1.f : 0.f; };
    float hz[XO > 0 ? XO : 1];      // PRO: 0 for a row before the start with no history
    f4 cwq[2], cwk[2];              // PRO: taps of columns c0, c0 + 1
    f2 cbq, cbk;                    // PRO: biases
    {
        f2 lv[RPG];
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const int r = r0 + u;
            const bool ok = r < n;
            const size_t th = (size_t)(t0 + min(r, n - 1)) * H + h, off = th * DK + c0;
            // G (compile time): which gates hold one value per token-head
            f2 x;
            if constexpr ((G & kGateAlpha) != 0) { const float a1 = la[th]; x[0] = a1; x[1] = a1; }
            else x = *reinterpret_cast<const f2 *>(la + off);
            if constexpr (BSC) br[u] = b[th];
            else br[u] = Ld<In>::ldraw2(b + off);
            if constexpr (!PRO) {
                kr[u] = Ld<In>::ldraw2(k + off);
                qr[u] = Ld<In>::ldraw2(q + off);
            }
            const f2 z = {0.f, 0.f};
            lv[u] = ok ? x : z;
        }
        if constexpr (PRO) {
            // rows r0-3 .. r0+RPG-1; a row before the sequence's start reads
            // the history (zeroed at use when there is none)
            const int tb = sq.t0(i);
            const In *hq = (const In *)cq.hist, *hk = (const In *)ck.hist;
#pragma unroll
            for (int x = 0; x < RPG + XO; ++x) {
                const int rr = r0 + x - XO, rc = min(rr, n - 1);
                const bool before = t0 + rr < tb;
                const In *sq_ = q, *sk_ = k;
                size_t off = ((size_t)(t0 + max(rc, tb - t0)) * H + h) * DK + c0;
                if (before && hq) {
                    sq_ = hq;
                    sk_ = hk;
                    off = ((size_t)(i * H + h) * 3 + 3 + rr) * DK + c0;
                }
                qr[x] = Ld<In>::ldraw2(sq_ + off);
                kr[x] = Ld<In>::ldraw2(sk_ + off);
                if (x < XO) hz[x] = (before && !hq) ? 0.f : 1.f;
            }
            const size_t wo = (size_t)h * DK + c0;
            cwq[0] = *reinterpret_cast<const f4 *>(cq.w + 4 * wo);
            cwq[1] = *reinterpret_cast<const f4 *>(cq.w + 4 * wo + 4);
            cwk[0] = *reinterpret_cast<const f4 *>(ck.w + 4 * wo);
            cwk[1] = *reinterpret_cast<const f4 *>(ck.w + 4 * wo + 4);
            // without a bias, read the taps (any valid address) and zero at use
            cbq = *reinterpret_cast<const f2 *>(cq.bias ? cq.bias + wo : cq.w + 4 * wo);
            cbk = *reinterpret_cast<const f2 *>(ck.bias ? ck.bias + wo : ck.w + 4 * wo);
        }
        f2 run = {0.f, 0.f};
#pragma unroll
        for (int u = 0; u < RPG; ++u) { run += lv[u]; gg[u] = run; }
        *reinterpret_cast<f2 *>(sPart + rg * DK + c0) = run;
    }
    if (t < 5) sFlag[t] = 0;
    __syncthreads();
    {
        f2 pre = {0.f, 0.f};
        for (int q2 = 0; q2 < rg; ++q2) pre += *reinterpret_cast<const f2 *>(sPart + q2 * DK + c0);
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            gg[u] += pre;
            const int r = r0 + u;
            if ((r & 15) == 15) *reinterpret_cast<f2 *>(sRef + ((r + 1) >> 4) * DK + c0) = gg[u];
            if ((r & 15) == 7) *reinterpret_cast<f2 *>(sMid + (r >> 4) * DK + c0) = gg[u];
            if (r == 0) *reinterpret_cast<f2 *>(sG0 + c0) = gg[u];
        }
        if (rg == 0) { sRef[c0] = 0.f; sRef[c0 + 1] = 0.f; }
    }
    __syncthreads();
    for (int c = t; c < DK; c += 256)
        if (0.5f * (sG0[c] - sRef[4 * DK + c]) > LIMC) atomicOr(&sFlag[4], 1);
    __syncthreads();
    const bool fast = sFlag[4] == 0;

    // the thread's q, k (rows past the chunk's end zeroed) and b values
    f2 qp[PRO ? RPG : 1], kp[PRO ? RPG : 1];
    if constexpr (PRO) {
        const float bfq = cq.bias ? 1.f : 0.f, bfk = ck.bias ? 1.f : 0.f;
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            f2 yq = cbq * bfq, yk = cbk * bfk;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) {
                const int x = u + jt;   // slot of row r0 + u - 3 + jt
                f2 xq = Ld<In>::cvt2(qr[x]), xk = Ld<In>::cvt2(kr[x]);
                if (x < XO) { xq *= hz[x < XO ? x : 0]; xk *= hz[x < XO ? x : 0]; }
                yq[0] += cwq[0][jt] * xq[0]; yq[1] += cwq[1][jt] * xq[1];
                yk[0] += cwk[0][jt] * xk[0]; yk[1] += cwk[1][jt] * xk[1];
            }
            const float nq = lane_group_sum<CP>(yq[0] * yq[0] + yq[1] * yq[1]);
            const float nk = lane_group_sum<CP>(yk[0] * yk[0] + yk[1] * yk[1]);
            // 1 / max(norm, 1e-12)
            const float rf = rowf(u);
            qp[u] = yq * (rsqrtf(fmaxf(nq, 1e-24f)) * rf);
            kp[u] = yk * (rsqrtf(fmaxf(nk, 1e-24f)) * rf);
        }
    }
    auto qval = [&](int u) {
        if constexpr (PRO) return qp[u];
        else return Ld<In>::cvt2(qr[u]) * rowf(u);
    };
    auto kval = [&](int u) {
        if constexpr (PRO) return kp[u];
        else return Ld<In>::cvt2(kr[u]) * rowf(u);
    };
    auto bval = [&](int u) {
        if constexpr (PRO) {
            const f2 x = bf2(u);
            f2 r;
            r[0] = __builtin_amdgcn_rcpf(1.f + __expf(-x[0]));
            r[1] = __builtin_amdgcn_rcpf(1.f + __expf(-x[1]));
            return r;
        } else return bf2(u);
    };

    // ---- stage 2: decay factors, gamma, scaled operands in LDS ----
    if (t < DK) reinterpret_cast<float *>(blk + L::oG)[t] = __expf(sRef[4 * DK + t]);
    if (fast) {
        for (int c = t; c < DK; c += 256) {
            const float gn = sRef[4 * DK + c], mid = 0.5f * (sG0[c] + gn);
            tExpRef[c] = __expf(mid);
            tExpKh[c] = __expf(gn - mid);
        }
        const f2 mid = 0.5f * (*reinterpret_cast<const f2 *>(sG0 + c0) + *reinterpret_cast<const f2 *>(sRef + 4 * DK + c0));
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const int r = r0 + u;
            f2 e1, e2;
            e1[0] = __expf(gg[u][0] - mid[0]); e1[1] = __expf(gg[u][1] - mid[1]);
            e2[0] = __expf(mid[0] - gg[u][0]); e2[1] = __expf(mid[1] - gg[u][1]);
            const f2 kv = kval(u), bv = bval(u), qv = qval(u);
            const f2 eh = bv * kv * e1, qh = qv * e1, kb_ = kv * e2;
            sE[r * LDE + c0] = (Op)eh[0]; sE[r * LDE + c0 + 1] = (Op)eh[1];
            sQ[r * LDE + c0] = (Op)qh[0]; sQ[r * LDE + c0 + 1] = (Op)qh[1];
            sK[r * LDE + c0] = (Op)kb_[0]; sK[r * LDE + c0 + 1] = (Op)kb_[1];
        }
    } else {
        for (int idx = t; idx < 4 * DK; idx += 256) {
            const int R = idx / DK, c = idx % DK;
            const float rR = sRef[R * DK + c], rR1 = sRef[(R + 1) * DK + c];
            const float mid = sMid[R * DK + c], gn = sRef[4 * DK + c];
            tExpRef[R * DK + c] = __expf(rR);
            tExpKh[R * DK + c] = __expf(gn - rR1);
            const float de = rR - mid, dq = mid - rR1;
            tDiagE[R * DK + c] = __expf(de);
            tDiagK[R * DK + c] = __expf(dq);
            if (fmaxf(de, dq) > LIM) atomicOr(&sFlag[R], 1);
            if (R < 3) {
                const int Rr = R == 0 ? 2 : 3, Ss = R == 2 ? 1 : 0;
                tDec[R * DK + c] = __expf(sRef[Rr * DK + c] - sRef[(Ss + 1) * DK + c]);
            }
        }
        // e1_r = e^{g_r - ref_R} forward, e2_r = e^{ref_{R+1} - g_r} backward,
        // as running products of alpha within the 16-row block
        f2 al[RPG], e1[RPG], e2[RPG];
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const f2 gprev = u ? gg[u - 1] : gg[0];
            al[u][0] = __expf(u ? gg[u][0] - gprev[0] : 0.f);
            al[u][1] = __expf(u ? gg[u][1] - gprev[1] : 0.f);
        }
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const int r = r0 + u;
            if (u == 0 || (r & 15) == 0) {
                const float *ref = sRef + (r >> 4) * DK + c0;
                e1[u][0] = __expf(gg[u][0] - ref[0]);
                e1[u][1] = __expf(gg[u][1] - ref[1]);
            } else e1[u] = e1[u - 1] * al[u];
        }
#pragma unroll
        for (int u = RPG - 1; u >= 0; --u) {
            const int r = r0 + u;
            if ((r & 15) == 15) { e2[u][0] = 1.f; e2[u][1] = 1.f; }
            else if (u == RPG - 1) {
                const float *ref = sRef + ((r >> 4) + 1) * DK + c0;
                e2[u][0] = __expf(ref[0] - gg[u][0]);
                e2[u][1] = __expf(ref[1] - gg[u][1]);
            } else e2[u] = e2[u + 1] * al[u + 1];
        }
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const int r = r0 + u;
            const f2 kv = kval(u), bv = bval(u), qv = qval(u);
            const f2 eh = bv * kv * e1[u], qh = qv * e1[u], kb_ = kv * e2[u];
            sE[r * LDE + c0] = (Op)eh[0]; sE[r * LDE + c0 + 1] = (Op)eh[1];
            sQ[r * LDE + c0] = (Op)qh[0]; sQ[r * LDE + c0 + 1] = (Op)qh[1];
            sK[r * LDE + c0] = (Op)kb_[0]; sK[r * LDE + c0 + 1] = (Op)kb_[1];
        }
    }
    __syncthreads();
    // Q+ / E scale of row block R, Khat scale of row block S
    const int tabR = fast ? 0 : 1;   // table row step per block

    // ---- stage 3: A and P blocks on the matrix cores; pack Q+ and Khat^T ----
    for (int idx = t; idx < 6 * 256; idx += 256) {   // strictly-upper blocks of A
        const int bi = idx >> 8, e = idx & 255;
        const int R = bi < 3 ? 0 : (bi < 5 ? 1 : 2);
        const int S = bi < 3 ? bi + 1 : (bi < 5 ? bi - 1 : 3);
        sA[(16 * R + (e >> 4)) * LDA + 16 * S + (e & 15)] = 0.f;
    }
    const bool any_slow = !fast && (sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3]);
    f4 pacc[5];
    int ptile[5];
    if (fast) {
        // waves 0,1 build A, waves 2,3 build P; wave parity picks the row
        // blocks {0,3} or {1,2}, five 16x16 blocks each
        const int kind = wv >> 1, par = wv & 1;
        const Op *src = kind ? sQ : sE;
#pragma unroll
        for (int qq = 0; qq < 5; ++qq) {
            const int R = par ? (qq < 2 ? 1 : 2) : (qq == 0 ? 0 : 3);
            const int S = par ? (qq < 2 ? qq : qq - 2) : (qq == 0 ? 0 : qq - 1);
            f4 acc = f4zero();
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                acc = M::mma(lds_row_frag<Op>(src + (16 * R + m16) * LDE, kb * KB, g4),
                             lds_row_frag<Op>(sK + (16 * S + m16) * LDE, kb * KB, g4), acc);
            if (kind == 0) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int rr = 4 * g4 + ii;
                    sA[(16 * R + rr) * LDA + 16 * S + m16] = (R > S || rr > m16) ? acc[ii] : 0.f;
                }
                ptile[qq] = -1;
            } else {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int rr = 4 * g4 + ii;
                    acc[ii] = (R > S || rr >= m16) ? acc[ii] : 0.f;
                }
                ptile[qq] = (R * (R + 1)) / 2 + S;
            }
            pacc[qq] = acc;
        }
    } else {
        // wave wv takes jobs wv + 4*qq: ids 0..9 are the A blocks, 10..19 the P blocks
#pragma unroll
        for (int qq = 0; qq < 5; ++qq) {
            const int jb = wv + 4 * qq;
            const int kind = jb / 10, tile = jb % 10;
            const int R = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int S = tile - (R * (R + 1)) / 2;
            ptile[qq] = -1;
            pacc[qq] = f4zero();
            if (R == S && sFlag[R]) continue;   // exact path below
            const Op *src = kind ? sQ : sE;
            f4 acc = f4zero();
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                frag a, bb;
#pragma unroll
                for (int i4 = 0; i4 < NE; ++i4) {
                    const int ch = kb * KB + kofs(g4, i4);
                    float av = (float)src[(16 * R + m16) * LDE + ch];
                    float bvv = (float)sK[(16 * S + m16) * LDE + ch];
                    if (R == S) { av *= tDiagE[R * DK + ch]; bvv *= tDiagK[R * DK + ch]; }
                    else if (R > S + 1) bvv *= tDec[(R == 2 ? 0 : (S == 0 ? 1 : 2)) * DK + ch];
                    a[i4] = (Op)av;
                    bb[i4] = (Op)bvv;
                }
                acc = M::mma(a, bb, acc);
            }
            if (kind == 0) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int rr = 4 * g4 + ii;
                    sA[(16 * R + rr) * LDA + 16 * S + m16] = (R > S || rr > m16) ? acc[ii] : 0.f;
                }
            } else {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int rr = 4 * g4 + ii;
                    acc[ii] = (R > S || rr >= m16) ? acc[ii] : 0.f;
                }
                pacc[qq] = acc;
                ptile[qq] = tile;
            }
        }
    }
    // Q+ fragments: rows 16 mt + m, channels kb*KB + kofs, scaled to e^{g_r}
    for (int f = wv; f < 4 * NKB; f += 4) {
        const int mt = f / NKB, kb = f % NKB;
        const frag x = lds_row_frag<Op>(sQ + (16 * mt + m16) * LDE, kb * KB, g4);
        const float *sc = tExpRef + mt * tabR * DK + kb * KB;
        frag a;
#pragma unroll
        for (int i4 = 0; i4 < NE; ++i4) a[i4] = (Op)((float)x[i4] * sc[kofs(g4, i4)]);
        block_store(blk + L::oQ + ((size_t)f * 64 + lane) * 16, a);
    }
    // Khat^T fragments: rows = channel 16 ct + m, contraction = chunk rows
    for (int f = wv; f < NCT * NSB; f += 4) {
        const int ct = f / NSB, sb = f % NSB;
        const int c = 16 * ct + m16;
        frag a;
#pragma unroll
        for (int i4 = 0; i4 < NE; ++i4) {
            const int s = sb * KB + kofs(g4, i4);
            a[i4] = (Op)((float)sK[s * LDE + c] * tExpKh[(s >> 4) * tabR * DK + c]);
        }
        block_store(blk + L::oK + ((size_t)f * 64 + lane) * 16, a);
    }
    __syncthreads();

    // ---- stage 4: P into LDS (over Q^), exact diagonal blocks if needed ----
    Op *sP = sQ, *sT = sK, *sW = sE;
    for (int idx = t; idx < 6 * 256; idx += 256) {
        const int bi = idx >> 8, e = idx & 255;
        const int R = bi < 3 ? 0 : (bi < 5 ? 1 : 2);
        const int S = bi < 3 ? bi + 1 : (bi < 5 ? bi - 1 : 3);
        sP[(16 * R + (e >> 4)) * LDT + 16 * S + (e & 15)] = (Op)0.f;
        sT[(16 * R + (e >> 4)) * LDT + 16 * S + (e & 15)] = (Op)0.f;
    }
#pragma unroll
    for (int s3 = 0; s3 < 5; ++s3) {
        if (ptile[s3] < 0) continue;
        const int tile = ptile[s3];
        const int R = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
        const int S = tile - (R * (R + 1)) / 2;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            sP[(16 * R + 4 * g4 + ii) * LDT + 16 * S + m16] = (Op)pacc[s3][ii];
    }
    if (any_slow) {
        // exact pairwise exponents for flagged diagonal blocks (strong decay)
        for (int R = 0; R < 4; ++R) {
            if (!sFlag[R]) continue;
            const int rl = t >> 4, sl = t & 15;
            const int r = 16 * R + rl, s = 16 * R + sl;
            float aA = 0.f, aP = 0.f;
            if (sl <= rl && r < n) {
                const size_t br_ = ((size_t)(t0 + r) * H + h) * DK, bs = ((size_t)(t0 + s) * H + h) * DK;
                constexpr bool asc = (G & kGateAlpha) != 0, bsc = (G & kGateB) != 0;
                for (int c = 0; c < DK; ++c) {
                    float d = 0.f;
                    for (int x = s + 1; x <= r; ++x) {
                        const size_t th = (size_t)(t0 + x) * H + h;
                        d += la[asc ? th : th * DK + c];
                    }
                    const float e = __expf(d) * Ld<In>::one(k + bs + c);
                    const float bv = Ld<In>::one(b + (bsc ? (size_t)(t0 + r) * H + h : br_ + c));
                    aA += bv * Ld<In>::one(k + br_ + c) * e;
                    aP += Ld<In>::one(q + br_ + c) * e;
                }
            }
            sA[r * LDA + s] = sl < rl ? aA : 0.f;
            sP[r * LDT + s] = (Op)aP;
        }
    }
    __syncthreads();

    // ---- stage 5: T = (I + A)^{-1}, block forward substitution ----
    {
        // diagonal blocks, one per wave, all 64 lanes (see unit_lower_inverse16)
        const int R = wv;
        float x[4];
        unit_lower_inverse16(sA + (16 * R) * LDA + 16 * R, LDA, lane, x);
#pragma unroll
        for (int j = 0; j < 4; ++j) sT[(16 * R + g4 + 4 * j) * LDT + 16 * R + m16] = (Op)x[j];
    }
    __syncthreads();
    for (int d = 1; d < 4; ++d) {
        if (wv < 4 - d) {
            const int S = wv, R = S + d;
            f4 y = f4zero();
            for (int J = S; J < R; ++J) {
                f4 a, bb;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    a[ii] = sA[(16 * R + m16) * LDA + 16 * J + 4 * g4 + ii];
                    bb[ii] = (float)sT[(16 * J + 4 * g4 + ii) * LDT + 16 * S + m16];
                }
                y = M::mma16(a, bb, y);
            }
            f4 a;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) a[ii] = (float)sT[(16 * R + m16) * LDT + 16 * R + 4 * g4 + ii];
            const f4 z = M::mma16(a, y, f4zero());
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sT[(16 * R + 4 * g4 + ii) * LDT + 16 * S + m16] = (Op)(-z[ii]);
        }
        __syncthreads();
    }

    // ---- stage 6: W = T E (E = stored E-side operand x e^{ref}); pack -W, P, T ----
    // wave wv takes output column tiles nt = wv, wv+4, ...; T fragments are
    // shared across them, E column fragments across the row tiles
    constexpr int NWT = (NCT + 3) / 4;
    frag tf[4][NSB];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
            if (sb <= (16 * mt + 15) / KB) tf[mt][sb] = lds_row_frag<Op>(sT + (16 * mt + m16) * LDT, sb * KB, g4);
    f4 wacc[NWT][4];
#pragma unroll
    for (int qq = 0; qq < NWT; ++qq) {
        const int nt = wv + 4 * qq;
        if (nt >= NCT) continue;
        const int c = 16 * nt + m16;
        frag eb[NSB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int i4 = 0; i4 < NE; ++i4) {
                const int s = sb * KB + kofs(g4, i4);
                eb[sb][i4] = (Op)((float)sE[s * LDE + c] * tExpRef[(s >> 4) * tabR * DK + c]);
            }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f4 acc = f4zero();
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
                if (sb <= (16 * mt + 15) / KB) acc = M::mma(tf[mt][sb], eb[sb], acc);
            wacc[qq][mt] = acc;
        }
    }
    // P and T fragments (the nonzero k-blocks only)
    for (int f = wv; f < 4 * NSB; f += 4) {
        const int mt = f / NSB, sb = f % NSB;
        if (sb > L::sbmax(mt)) continue;
        const int pos = L::tpos(mt, sb);
        block_store(blk + L::oP + ((size_t)pos * 64 + lane) * 16,
                    lds_row_frag<Op>(sP + (16 * mt + m16) * LDT, sb * KB, g4));
        block_store(blk + L::oT + ((size_t)pos * 64 + lane) * 16,
                    lds_row_frag<Op>(sT + (16 * mt + m16) * LDT, sb * KB, g4));
    }
    __syncthreads();   // every read of the E-side operand done
#pragma unroll
    for (int qq = 0; qq < NWT; ++qq) {
        const int nt = wv + 4 * qq;
        if (nt >= NCT) continue;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                sW[(16 * mt + 4 * g4 + ii) * LDE + 16 * nt + m16] = (Op)(-wacc[qq][mt][ii]);
    }
    __syncthreads();
    for (int f = wv; f < 4 * NKB; f += 4) {
        const int mt = f / NKB, kb = f % NKB;
        block_store(blk + L::oW + ((size_t)f * 64 + lane) * 16,
                    lds_row_frag<Op>(sW + (16 * mt + m16) * LDE, kb * KB, g4));
    }
}

// ---------------------------------------------------------------------------
// Sequential state pass.
//
// Workgroup = (chain = sequence*H + head, 16-column slice of dv), 8 waves in
// two roles:
//  * state waves 0..3 carry the recurrence. Wave w owns rows 16w..16w+15 of
//    each chunk's Delta and state tiles [w*TPW, (w+1)*TPW) (16 key channels
//    each), fp32 in registers:
//        Delta_w = T_w U - W_w S;   S_tile <- gamma * S_tile + Khat^T_tile Delta
//  * output waves 4..7 stage U = w*v (hi + lo f16) into LDS and compute
//        O_w = Q+_w S + P_w Delta
//    off the serial path.
// Per chunk, two barriers: (1) state tiles and U in LDS, (2) Delta in LDS.
// Each role loads its operand fragments two chunks ahead into a ring of
// three register sets; the loads are unconditional (clamped chunk index) so
// the compiler waits only for the chunk at hand. A compute unit streams
// operand bytes at ~60 B/cycle, so the loads are placed where each role would
// otherwise wait at a barrier: the state waves issue half after writing
// Delta and half after the state update, the output waves right after
// barrier (1). The output tile goes through LDS and leaves as one 16-byte
// store per thread.
//
// Workgroups are numbered so that the slices of one chain land on the same
// XCD (the dispatcher deals workgroups to the 8 XCDs round-robin), where they
// share that XCD's L2 for the chain's operand blocks.
// Row tiles of a chunk handled by wave w (0..3) of either role: one (w) for
// 64-token chunks, two ({w, 7 - w}, which evens out the triangular T and P
// fragments between waves) for 128, and for 32 (two row tiles) waves 0 and 1
// take one each while waves 2 and 3 have none.
template <int CS> struct RowTiles {
    static constexpr int NRB = CS / 16;
    static constexpr int RPW = NRB >= 4 ? NRB / 4 : 1;
    static_assert(RPW <= 2, "at most two row tiles per wave");
    static __device__ __forceinline__ int rt(int w, int j) { return RPW == 1 ? w : ((j & 1) ? 4 * j + 3 - w : 4 * j + w); }
    static constexpr bool ALL = NRB >= 4;   // every wave has row tiles
    static __device__ __forceinline__ bool active(int w) { return ALL || w < NRB; }
};

template <typename Op, int DK, int CS = 64> struct StateFrags {
    using M = Mma<Op>;
    using L = Blk<Op, DK, CS>;
    using RT = RowTiles<CS>;
    using frag = typename M::frag;
    static constexpr int TPW = (L::NCT + 3) / 4, RPW = RT::RPW;
    frag nW[RPW][L::NKB], Ti[RPW][L::NSB], Kh[TPW][L::NSB];
    f4 gam[TPW];
    // T k-blocks past a row tile's diagonal are never loaded, and the
    // products that skip them sit under a runtime condition, which the
    // compiler may leave without a branch around it (a matrix instruction
    // then runs whatever the execution mask): they must read as zero. (The
    // 64-token kernel keeps its loads inside the skipped region, which keeps
    // the branch.)
    __device__ __forceinline__ void zero_tri() {
#pragma unroll
        for (int j = 0; j < RPW; ++j)
#pragma unroll
            for (int sb = 0; sb < L::NSB; ++sb)
#pragma unroll
                for (int e = 0; e < M::NE; ++e) Ti[j][sb][e] = (Op)0;
    }
    // first half: what the Delta step needs (T fragments above the diagonal are zero and skipped)
    __device__ __forceinline__ void load_a(const uint8_t *blk, int wv, int lane) {
        if (!RT::ALL && !RT::active(wv)) return;
        // (a one-trip loop over row tiles changes the 64-token kernel's schedule)
        load_rows(blk, 0, RT::rt(wv, 0), lane);
        if constexpr (RPW > 1) load_rows(blk, 1, RT::rt(wv, 1), lane);
    }
    __device__ __forceinline__ void load_rows(const uint8_t *blk, int j, int rt, int lane) {
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb)
            nW[j][kb] = *reinterpret_cast<const frag *>(blk + L::oW + ((size_t)(rt * L::NKB + kb) * 64 + lane) * 16);
        const int sbmax = (16 * rt + 15) / M::KB;
#pragma unroll
        for (int sb = 0; sb < L::NSB; ++sb)
            if (sb <= sbmax)
                Ti[j][sb] = *reinterpret_cast<const frag *>(blk + L::oT + ((size_t)L::tpos(rt, sb) * 64 + lane) * 16);
    }
    // second half: what the state update needs
    __device__ __forceinline__ void load_b(const uint8_t *blk, int wv, int lane) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int ct = wv * TPW + u;
            if (L::NCT % 4 == 0 || ct < L::NCT) {   // static when all waves own tiles
                gam[u] = *reinterpret_cast<const f4 *>(blk + L::oG + (size_t)(16 * ct + 4 * (lane >> 4)) * 4);
#pragma unroll
                for (int sb = 0; sb < L::NSB; ++sb)
                    Kh[u][sb] = *reinterpret_cast<const frag *>(blk + L::oK + ((size_t)(ct * L::NSB + sb) * 64 + lane) * 16);
            }
        }
    }
};

template <typename Op, int DK, int CS = 64> struct OutFrags {
    using M = Mma<Op>;
    using L = Blk<Op, DK, CS>;
    using RT = RowTiles<CS>;
    using frag = typename M::frag;
    static constexpr int RPW = RT::RPW;
    frag Qp[RPW][L::NKB], Pm[RPW][L::NSB];
    // as StateFrags::zero_tri, for P
    __device__ __forceinline__ void zero_tri() {
#pragma unroll
        for (int j = 0; j < RPW; ++j)
#pragma unroll
            for (int sb = 0; sb < L::NSB; ++sb)
#pragma unroll
                for (int e = 0; e < M::NE; ++e) Pm[j][sb][e] = (Op)0;
    }
    __device__ __forceinline__ void load(const uint8_t *blk, int wo, int lane) {
        if (!RT::ALL && !RT::active(wo)) return;
        load_rows(blk, 0, RT::rt(wo, 0), lane);
        if constexpr (RPW > 1) load_rows(blk, 1, RT::rt(wo, 1), lane);
    }
    __device__ __forceinline__ void load_rows(const uint8_t *blk, int j, int rt, int lane) {
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb)
            Qp[j][kb] = *reinterpret_cast<const frag *>(blk + L::oQ + ((size_t)(rt * L::NKB + kb) * 64 + lane) * 16);
        const int sbmax = (16 * rt + 15) / M::KB;   // P is lower triangular
#pragma unroll
        for (int sb = 0; sb < L::NSB; ++sb)
            if (sb <= sbmax)
                Pm[j][sb] = *reinterpret_cast<const frag *>(blk + L::oP + ((size_t)L::tpos(rt, sb) * 64 + lane) * 16);
    }
};

// v and w for one chunk and column slice: output-wave thread t (0..255)
// holds row t/4, columns 4*(t%4)..+3 of both.
template <typename In> struct UVTile {
    In v[4], w[4];
    bool ok;
    // `off` always addresses a valid row; `ok` false stands for a row past
    // the end and zeroes the product where it is used, not here: a select on
    // the loaded values would make the wave wait for this load (and every
    // load issued before it) at once.
    // `woff` addresses w when it holds one gate per token-head (WSC)
    template <bool WSC>
    __device__ __forceinline__ void load(const In *vp, const In *wp, size_t off, size_t woff, bool ok_) {
        ok = ok_;
        if constexpr (sizeof(In) == 2) {
            uint2 a = *reinterpret_cast<const uint2 *>(vp + off);
            v[0] = (In)(a.x & 0xFFFF); v[1] = (In)(a.x >> 16); v[2] = (In)(a.y & 0xFFFF); v[3] = (In)(a.y >> 16);
            if constexpr (WSC) {
                const In x = wp[woff];
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = x;
            } else {
                uint2 b = *reinterpret_cast<const uint2 *>(wp + off);
                w[0] = (In)(b.x & 0xFFFF); w[1] = (In)(b.x >> 16); w[2] = (In)(b.y & 0xFFFF); w[3] = (In)(b.y >> 16);
            }
        } else {
            const f4 a = *reinterpret_cast<const f4 *>(vp + off);
            f4 b;
            if constexpr (WSC) { const float x = wp[woff]; b[0] = x; b[1] = x; b[2] = x; b[3] = x; }
            else b = *reinterpret_cast<const f4 *>(wp + off);
#pragma unroll
            for (int e = 0; e < 4; ++e) { v[e] = a[e]; w[e] = b[e]; }
        }
    }
};


template <typename Op> __device__ __forceinline__ typename Mma<Op>::frag lds_bfrag(const Op *base, int lane)
{
    // B fragment of a KB-deep block from KB/16 consecutive accumulator-layout tiles
    typedef Op op4 __attribute__((ext_vector_type(4)));
    typename Mma<Op>::frag f;
#pragma unroll
    for (int p = 0; p < Mma<Op>::KB / 16; ++p) {
        const op4 x = *reinterpret_cast<const op4 *>(base + (p * 64 + lane) * 4);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) f[4 * p + ii] = x[ii];
    }
    return f;
}

template <typename Op> __device__ __forceinline__ void lds_tile_store(Op *dst, int lane, const f4 &x)
{
    typedef Op op4 __attribute__((ext_vector_type(4)));
    op4 y;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) y[ii] = (Op)x[ii];
    *reinterpret_cast<op4 *>(dst + lane * 4) = y;
}

// ---- tile scales of the f16 operands ---------------------------------------
// The pass rounds the state S, the writes U = w * v and the corrected writes
// Delta to f16 for the matrix cores. Value columns of the state evolve
// independently (the transition acts on the key axis only), so the columns
// of a 16-column tile may be carried divided by a power of two 2^e of their
// own: every product is then an exact multiple of the unscaled one. One
// exponent per chunk and tile serves S_c, U_c and Delta_c = T U_c - W S_c
// alike, so the products need no rescaling between them, and the state
// registers hold S_c / 2^e too. The exponent maps a bound B on the three
// into [2^9, 2^10): far from f16's overflow at 2^16 and from its subnormals
// below 2^-14 (unscaled, a state near 1e-6 kept ~4 significant bits and one
// past 65504 became inf). For chunk c + 1 (keys of at most unit norm, every
// decay factor <= 1):
//   |S_{c+1}| <= max|S_c| + CS max|Delta_c| <= 2 max(max|S_c|, CS max|Delta_c|),
//   B = max(that, max|U_{c+1}|),
// each wave's maxima put in LDS slots during step c (U's at the start of
// the step, the state's and Delta's once Delta is formed) and read by all
// after the second barrier. A tile far below the largest of the three keeps
// its relative precision down to 2^-14 of 2^9.

// exponent e of the scale for a bound B >= 0 given as its bits: B / 2^e in
// [2^9, 2^10), clamped to [-100, 100] (B = 0 and subnormal B give -100)
__device__ __forceinline__ int scale_exp(uint32_t Bbits)
{
    return min(max((int)(Bbits >> 23) - 127 - 9, -100), 100);
}
// 2^e for e in [-126, 127] (exact)
__device__ __forceinline__ float exp2i(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// Maxima of magnitudes as bit patterns: for non-negative floats the
// unsigned order is the float order, so the lane exchanges below take them
// as integers.
// max over each 16-lane row, in every lane of the row (quad swaps, then the
// row's half mirror and mirror)
__device__ __forceinline__ uint32_t rowmax16(uint32_t m)
{
    auto dpp = [](uint32_t y, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)y, decltype(ctrl)::value, 0xF, 0xF, true);
    };
    m = max(m, dpp(m, std::integral_constant<int, 0xB1>{}));    // quad_perm [1,0,3,2]
    m = max(m, dpp(m, std::integral_constant<int, 0x4E>{}));    // quad_perm [2,3,0,1]
    m = max(m, dpp(m, std::integral_constant<int, 0x141>{}));   // row_half_mirror
    return max(m, dpp(m, std::integral_constant<int, 0x140>{}));   // row_mirror
}
// max over the whole wave, in every lane: the rows, then across them with
// gfx950's lane swaps (permlane16_swap pairs each odd 16-lane row with the
// even row below it and permlane32_swap the two halves; of the two results
// one is the lane's own value and the other its partner's)
__device__ __forceinline__ uint32_t wave_umax(uint32_t x)
{
    x = rowmax16(x);
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max(a[0], a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max(b[0], b[1]);
}

// L2 prefetch workgroups. A pass workgroup holds a bounded number of
// cache-line requests in flight, so its step time grows with the latency of
// the level its operands come from. When the chip has workgroup slots to
// spare, each chain gets `npf` extra workgroups on the same XCD that read
// the chain's upcoming operand blocks and v / w rows a few chunks ahead of
// the pass, so that the pass finds them in that XCD's L2. Wave k of such a
// workgroup takes chunks k, k + 8, ...: it reads the chain's progress
// counter (chunks finished by the pass's first slice), waits while it is
// more than 3 + kPfWindow chunks ahead, skips chunks closer than 3, and
// reads one dword per line of its share of the chunk straight into an LDS
// scratch area that nothing reads (so no register waits for a line; the
// counter read waits only for this wave's reads of 8 chunks before). Every
// loop and wait is bounded, and the pass never waits for these workgroups.
static constexpr int kPfWindow = 8;
static constexpr int kPfMaxSleeps = 64;

typedef const __attribute__((address_space(1))) void *gptr_t;
typedef __attribute__((address_space(3))) void *lptr_t;

// Byte ranges [X0, X1) and [Y0, Y1) of the block (line-aligned, Y0 >= X1)
// are left out: the saving pass of the backward reads no Q+ and no P.
template <typename In, int DV, size_t BYTES, int CS = 64, size_t X0 = 0, size_t X1 = 0, size_t Y0 = 0,
          size_t Y1 = 0>
__device__ __forceinline__ void pass_prefetch(const uint8_t *blk0, const In *v, const In *w, const int *prog,
                                              int chain, int h, int H, int pf, int npf, int nch, int tb, int te,
                                              int gates)
{
    static_assert(X0 % 128 == 0 && X1 % 128 == 0 && Y0 % 128 == 0 && Y1 % 128 == 0 && X0 <= X1 &&
                  (Y0 == Y1 || Y0 >= X1) && Y0 <= Y1, "line-aligned, ordered ranges");
    constexpr int XL0 = (int)(X0 / 128), XN = (int)((X1 - X0) / 128), YL0 = (int)(Y0 / 128) - XN,
                  YN = (int)((Y1 - Y0) / 128);
    constexpr int NL = (int)(BYTES / 128) - XN - YN;              // block lines fetched
    constexpr int RB = DV * (int)sizeof(In);                      // bytes per v / w row
    constexpr int RL = (RB + 127) / 128;                          // lines per row
    // lines per chunk: the block, then the v rows and (per-channel gates) the w rows
    const int PL = NL + ((gates & kGateW) ? 1 : 2) * CS * RL;
    constexpr int NW = 8;                                         // waves
    __shared__ uint32_t sSink[NW * 64];
    const int t = threadIdx.x, wv = wave_id(), lane = t & 63;
    lptr_t scratch = (lptr_t)(sSink + wv * 64);
    auto done = [&]() {
        return __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(prog + chain, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    };
    for (int c = wv; c < nch; c += NW) {
        int d = done();
        for (int s = 0; c > d + 3 + kPfWindow && s < kPfMaxSleeps; ++s) {
            __builtin_amdgcn_s_sleep(4);
            d = done();
        }
        while (c < d + 3) c += NW;
        if (c >= nch) break;
        for (int l = pf + npf * lane; l < PL; l += npf * 64) {
            const uint8_t *a;
            if (l < NL) {
                const int lb = l + (l >= XL0 ? XN : 0);          // line of the block
                a = blk0 + (size_t)c * BYTES + (size_t)(lb + (lb - XN >= YL0 && l >= XL0 ? YN : 0)) * 128;
            } else {
                const int k = l - NL, which = k / (CS * RL), row = (k / RL) % CS, part = k % RL;
                const int tok = min(tb + CS * c + row, te - 1);
                a = reinterpret_cast<const uint8_t *>(which ? w : v) + ((size_t)tok * H + h) * RB +
                    min(part * 128, RB - 4);
            }
            __builtin_amdgcn_global_load_lds((gptr_t)a, scratch, 4, 0, 0);
        }
    }
    __syncthreads();   // drains the line reads before the workgroup ends
}

//
// PRO (fused prologue): v and w arrive raw. The output waves keep the raw v
// rows of four chunks in LDS (slot c % 4): each step stages the next
// chunk's rows, and forms this chunk's U = sigmoid(w) * ShortConv(v) from
// its own row (registers) and the three before it (LDS, reaching into the
// previous chunk's slot, or the history rows placed in slot 3 before the
// first chunk).
//
// SAVE (for the backward): no output; the state waves store each chunk's
// start state S_c [dk][dv] and Delta [64][dv] (operand type, the values the
// step used) at (head, chunk) slots of two buffers, head-major like the
// operand blocks, in accumulator-tile order: tile (row tile rt, column tile
// ct) at (rt * dv/16 + ct) * 256, lane l = n + 16g holding rows 4g..4g+3 of
// column n (one 8- or 16-byte store per lane and tile).
//
// KEEP (the training forward): the state waves store S_c and Delta as under
// SAVE while the output waves form o as in the plain forward, so one pass
// gives o, S_T and what the backward keeps.
struct SaveOut {
    void *S;          // [H * max_chunks][dk/16][dv/16][64][4]
    void *D;          // [H * max_chunks][4][dv/16][64][4]
    bool with_out;    // KEEP: also o and S_T
};

// (a whole 16x16 tile per wave: non-temporal, like the operand blocks)
template <typename Op>
__device__ __forceinline__ void tile_store(Op *dst, int lane, const f4 &x)
{
    typedef Op op4 __attribute__((ext_vector_type(4)));
    op4 y;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) y[ii] = (Op)x[ii];
    __builtin_nontemporal_store(y, reinterpret_cast<op4 *>(dst + lane * 4));
}

template <typename In, typename Op, int DK, int DV, int NC, bool WSC, bool PRO, bool SAVE = false, int CS = 64,
          bool KEEP = false>
__global__ __launch_bounds__(512) void chunk_pass_kernel(
    const In *__restrict__ v, const In *__restrict__ w, const float *__restrict__ S0,
    float *__restrict__ o, float *__restrict__ ST, Seqs sq, int H,
    const uint8_t *__restrict__ ops, int *__restrict__ prog, int npf, ConvIn cv, SaveOut so)
{
    static_assert(!PRO || !WSC, "the prologue takes per-channel gates");
    static_assert(CS == 64 || (!PRO && !SAVE && !KEEP), "the prologue and the backward use 64-token chunks");
    static_assert(!(SAVE && KEEP) && !(KEEP && (PRO || WSC)), "KEEP: the training forward, per-channel gates");
    constexpr bool STORE_SD = SAVE || KEEP;   // the state waves keep S_c and Delta
    using M = Mma<Op>;
    using L = Blk<Op, DK, CS>;
    using RT = RowTiles<CS>;
    using frag = typename M::frag;
    using SF = StateFrags<Op, DK, CS>;
    using OF = OutFrags<Op, DK, CS>;
    constexpr int KB = M::KB, NE = M::NE, NKB = L::NKB, NSB = L::NSB, NCT = L::NCT, NRB = L::NRB;
    constexpr int TPW = SF::TPW, RPW = RT::RPW;
    constexpr int TPK = KB / 16;              // accumulator tiles per k-block
    constexpr int NSL = DV / (16 * NC);       // column slices (workgroups per chain)
    // register ring of operand fragments: three chunks (prefetch distance 2),
    // two for 128-token chunks (their fragment sets are twice the size)
    constexpr int RING = CS >= 128 ? 2 : 3;
    constexpr int PD = RING - 1;
    // the output waves load one chunk further ahead (a ring of four; three
    // with the fused prologue on two column tiles, whose registers would not
    // hold a fourth): v and w arrive from memory with a long latency
    constexpr int ORING = CS >= 128 ? 2 : (PRO && NC == 2 ? 3 : 4);
    constexpr int OPD = ORING - 1;
    constexpr int UR = CS >= 64 ? CS / 64 : 1;   // v / w rows per output-wave thread
    constexpr int LCS = __builtin_ctz(CS);
    static_assert(NSL >= 1 && NSL * 16 * NC == DV, "slice width must divide dv");

    // per 16-column tile q of the slice
    __shared__ __attribute__((aligned(16))) Op sS[NC][NCT * 64 * 4];        // state operand tiles
    __shared__ __attribute__((aligned(16))) Op sD[NC][NRB * 64 * 4];        // Delta tiles
    // U as B-fragments: f16 hi / lo pairs (U = hi + lo to ~22 bits), or one
    // f16 part when kUSplit is off
    constexpr bool kUSplit = false;
    constexpr int NUP = std::is_same<Op, _Float16>::value && kUSplit ? 2 : 1;
    __shared__ __attribute__((aligned(16))) Op sU[NC][NUP * NSB * 64 * NE];
    constexpr int LDO = 16 * NC + 4;                                         // o staging row stride (floats)
    __shared__ __attribute__((aligned(16))) float sO[2][CS * LDO];          // o tiles
    constexpr int LDV = 16 * NC;                                             // raw-v row stride (floats)
    __shared__ __attribute__((aligned(16))) float sVr[PRO ? ORING : 1][PRO ? 64 * LDV : 4];   // PRO: raw v rows
    // f16 tiles carry a power-of-two scale per chunk and 16-column tile
    // (scale_exp above); fp32 operands need none
    constexpr bool SCL = std::is_same<Op, _Float16>::value;
    // each wave's part of the bound for the next chunk's scale, [parity of
    // the step that forms it][tile][wave] (plain stores: every slot is
    // rewritten each step)
    __shared__ __attribute__((aligned(16))) float sM[2][NC][8];
    // the first chunk's maxima, [wave][tile]
    __shared__ __attribute__((aligned(16))) float sM0[8][NC];
    auto first_exp = [&](int q) {
        uint32_t m = 0u;
#pragma unroll
        for (int x = 0; x < 8; ++x) m = max(m, __float_as_uint(sM0[x][q]));
        return scale_exp(__builtin_amdgcn_readfirstlane(m));
    };
    auto next_exp = [&](int c, int q) {
        const uint4 a = *reinterpret_cast<const uint4 *>(&sM[c & 1][q][0]);
        const uint4 b = *reinterpret_cast<const uint4 *>(&sM[c & 1][q][4]);
        const uint32_t m = max(max(max(a.x, a.y), max(a.z, a.w)), max(max(b.x, b.y), max(b.z, b.w)));
        return scale_exp(__builtin_amdgcn_readfirstlane(m));
    };

    // XCD-aware numbering: the slices (and prefetch workgroups) of chain c
    // sit on XCD c % 8
    const int Lid = blockIdx.x;
    const int kq = Lid >> 3, role = kq % (NSL + npf), js = role;
    const int chain = (kq / (NSL + npf)) * 8 + (Lid & 7);
    const int chains = sq.m.N * H;
    if (chain >= chains) return;
    const int i = chain / H, h = chain % H;

    const int t = threadIdx.x;
    const int lane = t & 63, wv = wave_id(), m16 = lane & 15, g4 = lane >> 4;
    const int col0 = 16 * NC * js;            // first value column of the slice
    const size_t sbase = ((size_t)i * H + h) * DK * DV;
    const int tb = sq.t0(i), te = sq.t1(i);
    const int cbeg = sq.m.template chunk0<CS>(i);
    const int nch = min((te - tb + CS - 1) >> LCS, max(0, sq.max_chunks - cbeg));
    auto blk_of = [&](int c) { return ops + ((size_t)h * sq.max_chunks + cbeg + min(c, nch - 1)) * L::bytes; };
    if (role >= NSL) {
        constexpr size_t X0 = SAVE ? L::oQ : 0, X1 = SAVE ? L::oK : 0, Y0 = SAVE ? L::oP : 0, Y1 = SAVE ? L::oT : 0;
        pass_prefetch<In, DV, L::bytes, CS, X0, X1, Y0, Y1>(ops + ((size_t)h * sq.max_chunks + cbeg) * L::bytes, v,
                                                            w, prog, chain, h, H, role - NSL, npf, nch, tb, te,
                                                            sq.gates);
        return;
    }
    const bool report = npf > 0 && js == 0 && t == 0;   // progress for the prefetch workgroups

    if (wv < 4) {
        // ------------------------------------------------ state waves
        // the serial chain runs here: these waves win issue ties on their SIMD
        __builtin_amdgcn_s_setprio(3);
        f4 Sr[NC][TPW];
#pragma unroll
        for (int q = 0; q < NC; ++q)
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int ct = wv * TPW + u;
                Sr[q][u] = f4zero();
                if (ct < NCT) {
                    if (S0) {
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii)
                            Sr[q][u][ii] = S0[sbase + (size_t)(16 * ct + 4 * g4 + ii) * DV + col0 + 16 * q + m16];
                    }
                    if constexpr (!SCL) lds_tile_store<Op>(sS[q] + ct * 256, lane, Sr[q][u]);
                }
            }
        // exponent of the current chunk's scale, per column tile (uniform)
        int esc[NC];
#pragma unroll
        for (int q = 0; q < NC; ++q) esc[q] = 0;
        // max of |S| (of the registers as they stand) over this lane's values in tile q
        auto state_lmax = [&](int q) {
            float m = 0.f;   // (|x| is a free source modifier of the float max)
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                if (NCT % 4 != 0 && wv * TPW + u >= NCT) continue;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) m = fmaxf(m, fabsf(Sr[q][u][ii]));
            }
            return m;
        };
        if constexpr (SCL) {
            // this wave's part of the first chunk's maxima (S_0; the output
            // waves put U_0's)
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                const uint32_t m = wave_umax(__float_as_uint(state_lmax(q)));
                if (lane == 0) sM0[wv][q] = __uint_as_float(m);
            }
        }
        const bool rows = RT::active(wv);
        // last stored k-block of T / P for the wave's row tile j (RPW <= 2)
        const int sbm0 = (16 * RT::rt(wv, 0) + 15) / KB;
        const int sbm1 = RPW > 1 ? (16 * RT::rt(wv, 1) + 15) / KB : 0;
        auto sbmax = [&](int j) { return j == 0 ? sbm0 : sbm1; };
        SF f0, f1, f2;
        if constexpr (CS != 64) { f0.zero_tri(); f1.zero_tri(); f2.zero_tri(); }
        if (nch > 0) {
            f0.load_a(blk_of(0), wv, lane);
            f0.load_b(blk_of(0), wv, lane);
            if constexpr (RING == 3) {
                f1.load_a(blk_of(1), wv, lane);
                f1.load_b(blk_of(1), wv, lane);
            }
        }
        if constexpr (PRO) __syncthreads();   // pairs with the output waves' staging of chunk 0
        if constexpr (SCL) {
            __syncthreads();   // the first chunk's maxima
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                esc[q] = first_exp(q);
                const float r = exp2i(-esc[q]);
#pragma unroll
                for (int u = 0; u < TPW; ++u) {
                    const int ct = wv * TPW + u;
                    if (ct >= NCT) continue;
                    Sr[q][u] = Sr[q][u] * r;
                    lds_tile_store<Op>(sS[q] + ct * 256, lane, Sr[q][u]);
                }
            }
        }
        // The prefetch of chunk c+PD is split over the two windows in which
        // the state waves would otherwise wait for the output waves.
        const size_t slot0 = (size_t)h * sq.max_chunks + cbeg;
        auto step = [&](int c, SF &cur, SF &pre) {
            f4 dkeep[NC];      // STORE_SD: this wave's Delta tile, stored after barrier (2)
            __syncthreads();   // (1) state tiles and U ready
            // this lane's max |S_c| and max |Delta_c| per tile (in units of the scale)
            float mS[NC], mD[NC];
#pragma unroll
            for (int q = 0; q < NC; ++q) { mS[q] = 0.f; mD[q] = 0.f; }
            if (RT::ALL || rows) {
                // T U, then -W S (both divided by the chunk's scale; the -W S
                // k-blocks in two accumulators by parity, two dependent chains
                // of half the length: pass at T = 64K 0.838 -> 0.829 ms)
                f4 acc[RPW][NC], accw[RPW][NC], accw2[RPW][NC];
#pragma unroll
                for (int j = 0; j < RPW; ++j)
#pragma unroll
                    for (int q = 0; q < NC; ++q) { acc[j][q] = f4zero(); accw[j][q] = f4zero(); accw2[j][q] = f4zero(); }
                // every B fragment is read from LDS before the products, so
                // that the reads overlap rather than each wait on its own
                frag sfr[NC][NKB];
#pragma unroll
                for (int q = 0; q < NC; ++q)
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) sfr[q][kb] = lds_bfrag<Op>(sS[q] + kb * TPK * 256, lane);
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    if (RPW == 1 && sb > sbmax(0)) break;
#pragma unroll
                    for (int q = 0; q < NC; ++q) {
                        const frag uh = *reinterpret_cast<const frag *>(&sU[q][((0 * NSB + sb) * 64 + lane) * NE]);
                        const frag ul = *reinterpret_cast<const frag *>(&sU[q][(((NUP - 1) * NSB + sb) * 64 + lane) * NE]);
#pragma unroll
                        for (int j = 0; j < RPW; ++j) {
                            if (RPW > 1 && sb > sbmax(j)) continue;
                            acc[j][q] = M::mma(cur.Ti[j][sb], uh, acc[j][q]);
                            if constexpr (NUP == 2) acc[j][q] = M::mma(cur.Ti[j][sb], ul, acc[j][q]);
                        }
                    }
                }
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int q = 0; q < NC; ++q)
#pragma unroll
                        for (int j = 0; j < RPW; ++j) {
                            if (kb & 1) accw2[j][q] = M::mma(cur.nW[j][kb], sfr[q][kb], accw2[j][q]);
                            else accw[j][q] = M::mma(cur.nW[j][kb], sfr[q][kb], accw[j][q]);
                        }
                // the state maxima, while the products run
                if constexpr (SCL) {
#pragma unroll
                    for (int q = 0; q < NC; ++q) mS[q] = state_lmax(q);
                }
#pragma unroll
                for (int j = 0; j < RPW; ++j)
#pragma unroll
                    for (int q = 0; q < NC; ++q) {
                        const f4 d = acc[j][q] + (accw[j][q] + accw2[j][q]);
                        if constexpr (SCL) {
#pragma unroll
                            for (int ii = 0; ii < 4; ++ii) mD[q] = fmaxf(mD[q], fabsf(d[ii]));
                        }
                        lds_tile_store<Op>(sD[q] + RT::rt(wv, j) * 256, lane, d);
                        if constexpr (STORE_SD) {
                            if (j == 0) dkeep[q] = d;
                        }
                    }
            } else if constexpr (SCL) {
#pragma unroll
                for (int q = 0; q < NC; ++q) mS[q] = state_lmax(q);
            }
            // the prefetch goes out ahead of the maxima below: the compiler
            // does not move global loads across their LDS atomics
            pre.load_a(blk_of(c + PD), wv, lane);
            if constexpr (SCL) {
                // this wave's part of the bound on S_{c+1}: 2 max(|S_c|, CS |Delta_c|),
                // unscaled
                uint32_t mr[NC];
#pragma unroll
                for (int q = 0; q < NC; ++q)
                    mr[q] = wave_umax(__float_as_uint(fmaxf(mS[q], (float)CS * mD[q]) * exp2i(esc[q] + 1)));
                if (lane == 0) {
#pragma unroll
                    for (int q = 0; q < NC; ++q) sM[c & 1][q][wv] = __uint_as_float(mr[q]);
                }
            }
            __syncthreads();   // (2) Delta tiles ready
            frag Db[NC][NSB];
#pragma unroll
            for (int q = 0; q < NC; ++q)
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) Db[q][sb] = lds_bfrag<Op>(sD[q] + sb * TPK * 256, lane);
            // the second half of the prefetch, ahead of the products (2% on
            // the pass at T = 64K)
            pre.load_b(blk_of(c + PD), wv, lane);
            // S_c and Delta leave here, after the barrier, rather than on the
            // way to barriers (1) and (2) (keeping pass at T = 64K 0.955 ->
            // 0.875 ms); S_c is still in the registers and the exponent is
            // still this chunk's
            if constexpr (STORE_SD) {
                Op *sp = (Op *)so.S + (slot0 + c) * DK * DV;
#pragma unroll
                for (int q = 0; q < NC; ++q)
#pragma unroll
                    for (int u = 0; u < TPW; ++u) {
                        const int ct = wv * TPW + u;
                        if (NCT % 4 != 0 && ct >= NCT) continue;
                        tile_store<Op>(sp + ((size_t)ct * (DV / 16) + NC * js + q) * 256, lane,
                                       SCL ? Sr[q][u] * exp2i(esc[q]) : Sr[q][u]);
                    }
                if (RT::ALL || rows) {
                    Op *dp = (Op *)so.D + (slot0 + c) * 64 * DV;
#pragma unroll
                    for (int q = 0; q < NC; ++q)
                        tile_store<Op>(dp + ((size_t)wv * (DV / 16) + NC * js + q) * 256, lane,
                                       SCL ? dkeep[q] * exp2i(esc[q]) : dkeep[q]);
                }
            }
            // the next chunk's exponents, read after the Delta fragments so
            // that those reads do not wait behind these, and the factors that
            // take the state into their units (powers of two: exact)
            float rs[NC];
            if constexpr (SCL) {
#pragma unroll
                for (int q = 0; q < NC; ++q) {
                    const int en = next_exp(c, q);
                    rs[q] = exp2i(min(max(esc[q] - en, -126), 127));
                    esc[q] = en;
                }
            }
            // S_{c+1} = gamma S_c + Khat^T Delta_c: the products accumulate
            // onto the decayed state (in the chunk's units), and each tile
            // leaves for LDS in the next chunk's units as soon as it is done.
            // (Every tile is multiplied: a branch that skipped the multiply
            // where the exponent stays gave wrong, run-to-run varying states,
            // its untaken path reusing the product registers a few
            // instructions after the matrix instruction that writes them.)
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int ct = wv * TPW + u;
                if (NCT % 4 != 0 && ct >= NCT) continue;
#pragma unroll
                for (int q = 0; q < NC; ++q) {
                    f4 s = Sr[q][u] * cur.gam[u];
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) s = M::mma(cur.Kh[u][sb], Db[q][sb], s);
                    if constexpr (SCL) s = s * rs[q];
                    Sr[q][u] = s;
                    lds_tile_store<Op>(sS[q] + ct * 256, lane, s);
                }
            }
            // A device-scope store is written through to memory and, since
            // stores and loads retire in order, would hold up this wave's
            // later operand waits; the prefetch workgroups sit on the same
            // XCD and read the counter from the shared L2.
            if (report) __hip_atomic_store(prog + chain, c + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        };
        // Full rounds of RING steps carry no branches, so the register ring
        // needs no merge copies (a copy of a register with a load in flight
        // waits for that load and every load issued before it).
        int c = 0;
        if constexpr (RING == 3) {
            for (; c + 3 <= nch; c += 3) {
                step(c, f0, f2);
                step(c + 1, f1, f0);
                step(c + 2, f2, f1);
            }
            if (c < nch) step(c, f0, f2);
            if (c + 1 < nch) step(c + 1, f1, f0);
        } else {
            for (; c + 2 <= nch; c += 2) {
                step(c, f0, f1);
                step(c + 1, f1, f0);
            }
            if (c < nch) step(c, f0, f1);
        }
        __syncthreads();   // final: pairs with the output waves' last o tile
        if (ST) {
#pragma unroll
            for (int q = 0; q < NC; ++q)
#pragma unroll
                for (int u = 0; u < TPW; ++u) {
                    const int ct = wv * TPW + u;
                    if (ct >= NCT) continue;
                    const f4 x = SCL ? Sr[q][u] * exp2i(esc[q]) : Sr[q][u];
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        ST[sbase + (size_t)(16 * ct + 4 * g4 + ii) * DV + col0 + 16 * q + m16] = x[ii];
                }
        }
    } else {
        // ------------------------------------------------ output waves
        const int wo = wv - 4, to = t - 256;
        const bool rows = RT::active(wo);
        // last stored k-block of T / P for the wave's row tile j (RPW <= 2)
        const int sbm0 = (16 * RT::rt(wo, 0) + 15) / KB;
        const int sbm1 = RPW > 1 ? (16 * RT::rt(wo, 1) + 15) / KB : 0;
        auto sbmax = [&](int j) { return j == 0 ? sbm0 : sbm1; };
        // v / w tile coordinates of this thread (rows ur + 64 x, per column
        // tile) and where its U values go: four lanes per row, so that one
        // load instruction takes 16 rows of 32 bytes (rows of 16 bytes from
        // twice the rows made the pass 30% slower). A 32-row block of U (the
        // depth of one product step) is staged by waves 2b and 2b + 1.
        const int ur = to >> 2, uc = 4 * (to & 3);
        const bool urow = CS >= 64 || ur < CS;
        const size_t uoff0 = (size_t)h * DV + col0 + uc;
        const int usb = ur / KB, usl = ur % KB;
        const int ug = (usl & 15) >> 2, ui = 4 * (usl >> 4) + (usl & 3);
        auto uv_ok = [&](int c, int x) { return c < nch && urow && tb + CS * c + ur + 64 * x < te; };
        auto uv_off = [&](int c, int x) { return (size_t)min(tb + CS * c + ur + 64 * x, te - 1) * H * DV + uoff0; };
        auto w_off = [&](int c, int x) { return (size_t)min(tb + CS * c + ur + 64 * x, te - 1) * H + h; };
        struct UV { UVTile<In> q[NC * UR]; };   // tile q of row ur + 64 x at q + NC x
        auto uv_load = [&](UV &u, int c) {
#pragma unroll
            for (int x = 0; x < UR; ++x)
#pragma unroll
                for (int q = 0; q < NC; ++q)
                    u.q[q + NC * x].template load<WSC>(v, w, uv_off(c, x) + 16 * q, w_off(c, x), uv_ok(c, x));
        };
        OF g0, g1, g2, g3;
        UV u0, u1, u2, u3;
        if constexpr (CS != 64) { g0.zero_tri(); g1.zero_tri(); g2.zero_tri(); g3.zero_tri(); }
        if (nch > 0) {
            // v and w first: the loop reads the next chunk's rows at each step
            // start, and the wait the compiler places at the loop's head also
            // covers the first entry, which then finds them old enough
            uv_load(u0, 0);
            if constexpr (ORING >= 3) uv_load(u1, 1);
            if constexpr (ORING == 4) uv_load(u2, 2);
            if constexpr (!SAVE) {
                g0.load(blk_of(0), wo, lane);
                if constexpr (ORING >= 3) g1.load(blk_of(1), wo, lane);
                if constexpr (ORING == 4) g2.load(blk_of(2), wo, lane);
            }
        }
        // PRO: taps and bias of the thread's columns (per column tile)
        f4 ctap[PRO ? NC : 1][4], cbias[PRO ? NC : 1];
        auto stage_v = [&](const UV &u, int slot) {   // raw v row ur of a chunk into LDS
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                f4 x;
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = in2f<In>(u.q[q].v[e]);
                *reinterpret_cast<f4 *>(&sVr[slot][ur * LDV + 16 * q + uc]) = x;
            }
        };
        // PRO: U = sigmoid(w) * ShortConv(v) of row ur of one chunk, from its
        // raw rows in LDS slot `slot` (and rows 61..63 of slot `pslot` for the
        // rows before it), its own row and w in registers; zero past the end
        f4 ucarry[PRO ? NC : 1];
#pragma unroll
        for (int q = 0; q < (PRO ? NC : 1); ++q) ucarry[q] = f4zero();
        auto conv_u = [&](const UV &u, int slot, int pslot) {
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                f4 acc = cbias[q];
#pragma unroll
                for (int jt = 0; jt < 3; ++jt) {
                    const int row = ur - 3 + jt;
                    const float *src = row >= 0 ? &sVr[slot][row * LDV] : &sVr[pslot][(row + 64) * LDV];
                    const f4 xr = *reinterpret_cast<const f4 *>(src + 16 * q + uc);
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[e] += ctap[q][e][jt] * xr[e];
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = acc[e] + ctap[q][e][3] * in2f<In>(u.q[q].v[e]);
                    const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-in2f<In>(u.q[q].w[e])));
                    ucarry[q][e] = u.q[q].ok ? y * sg : 0.f;
                }
            }
        };
        if constexpr (PRO) {
            const float bflag = cv.bias ? 1.f : 0.f;
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                const size_t cofs = (size_t)h * DV + col0 + 16 * q + uc;
#pragma unroll
                for (int e = 0; e < 4; ++e) ctap[q][e] = *reinterpret_cast<const f4 *>(cv.w + 4 * (cofs + e));
                // without a bias, read the taps (any valid address) and zero them
                cbias[q] = *reinterpret_cast<const f4 *>(cv.bias ? cv.bias + cofs : cv.w + 4 * cofs) * bflag;
            }
            if (nch > 0) {
                stage_v(u0, 0);
                // rows 61..63 of the last slot stand for the three tokens before the
                // sequence: the history, or zeros
                if (ur >= 61) {
                    const In *hv = (const In *)cv.hist;
#pragma unroll
                    for (int q = 0; q < NC; ++q) {
                        f4 x = f4zero();
                        if (hv) {
                            const In *hp = hv + ((size_t)(i * H + h) * 3 + (ur - 61)) * DV + col0 + 16 * q + uc;
#pragma unroll
                            for (int e = 0; e < 4; ++e) x[e] = in2f<In>(hp[e]);
                        }
                        *reinterpret_cast<f4 *>(&sVr[ORING - 1][ur * LDV + 16 * q + uc]) = x;
                    }
                }
            }
            __syncthreads();   // pairs with the state waves' barrier before their loop
            if (nch > 0) conv_u(u0, 0, ORING - 1);
        }
        // U = w * v of one chunk (the prologue form keeps it in ucarry), to be
        // multiplied by u_ok: 1, or 0 for a row past the end (a factor per
        // lane and tile rather than a select per value, which the compiler
        // turns into branches)
        auto u_val = [&](const UV &u, int q, int x, int e) {
            if constexpr (PRO) return ucarry[q][e];
            else {
                const UVTile<In> &uq = u.q[q + NC * x];
                return in2f<In>(uq.w[e]) * in2f<In>(uq.v[e]);
            }
        };
        auto u_ok = [&](const UV &u, int q, int x) {
            if constexpr (PRO) return 1.f;
            else return u.q[q + NC * x].ok ? 1.f : 0.f;
        };
        // max |U| over this lane's values of tile q (rows ur + 64 x)
        // With scales (and no prologue, whose ucarry already holds U) the
        // products U of the next chunk are formed once, for its maximum a
        // step ahead, and kept for its write, in slot (chunk parity) of two
        // (the ring without the prologue has an even length, so the slot of
        // each step's chunk is sl & 1)
        constexpr bool UC = SCL && !PRO;
        static_assert(!UC || ORING % 2 == 0, "cache slots by ring position");
        float ucache[UC ? 2 : 1][UC ? NC * UR : 1][4];
        auto u_form = [&](const UV &u, int slot) {
            if constexpr (UC) {
#pragma unroll
                for (int x = 0; x < UR; ++x)
#pragma unroll
                    for (int q = 0; q < NC; ++q)
#pragma unroll
                        for (int e = 0; e < 4; ++e) ucache[slot & 1][q + NC * x][e] = u_val(u, q, x, e);
            }
        };
        // max |U| over this lane's values of tile q (rows ur + 64 x): of the
        // cached products, or of ucarry with the prologue
        auto u_lmax = [&](const UV &u, int q, int slot) {
            float mf = 0.f;
            if (urow) {
#pragma unroll
                for (int x = 0; x < UR; ++x) {
                    float mx = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        mx = fmaxf(mx, fabsf(UC ? ucache[slot & 1][(q + NC * x) % (UC ? NC * UR : 1)][e] : u_val(u, q, x, e)));
                    mf = fmaxf(mf, mx * u_ok(u, q, x));
                }
            }
            return __float_as_uint(mf);
        };
        // exponent of the current chunk's scale per column tile, as the state
        // waves hold it (both read the same maxima)
        int eo[NC];
#pragma unroll
        for (int q = 0; q < NC; ++q) eo[q] = 0;
        if constexpr (SCL) {
            // this wave's part of the first chunk's maxima (U_0; ucarry with the prologue)
#pragma unroll
            for (int q = 0; q < NC; ++q) {
                if (q == 0) u_form(u0, 0);
                const uint32_t m = nch > 0 ? wave_umax(u_lmax(u0, q, 0)) : 0u;
                if (lane == 0) sM0[4 + wo][q] = __uint_as_float(m);
            }
            __syncthreads();   // pairs with the state waves' barrier for the first chunk's maxima
#pragma unroll
            for (int q = 0; q < NC; ++q) eo[q] = first_exp(q);
        }
        // o tiles go through LDS (double-buffered) and leave as 16-byte
        // stores (CS * NC / 64 per thread) after the next barrier
        auto store_o = [&](int c) {
            const int tok = tb + CS * c, n = min(CS, te - tok);
            constexpr int NPC = CS * 4 * NC;   // 16-byte pieces per chunk
#pragma unroll
            for (int pq = 0; pq < (NPC + 255) / 256; ++pq) {
                const int x = to + 256 * pq, row = x / (4 * NC), q4 = x % (4 * NC);
                if ((NPC % 256 == 0 || x < NPC) && row < n)
                    *reinterpret_cast<f4 *>(o + ((size_t)(tok + row) * H + h) * DV + col0 + 4 * q4) =
                        *reinterpret_cast<const f4 *>(&sO[c & 1][row * LDO + 4 * q4]);
            }
        };
        // `sl` = c % ORING (a constant at every call site). Under PRO, U of chunk
        // c was formed during the previous step (ucarry); this step stages
        // the raw v rows of chunk c + 1 in slot (c + 1) % ORING before the first
        // barrier and forms its U after it, where these waves would wait.
        auto step = [&](int c, OF &cur, OF &pre, UV &ucur, UV &unext, UV &upre, int sl) {
            const int sln = sl == ORING - 1 ? 0 : sl + 1;
            if constexpr (PRO) stage_v(unext, sln);
            // this wave's part of the bound for the next chunk's scale: max |U|
            // of the next chunk. With a ring of three or four its rows were
            // loaded steps ago and it is formed right after barrier (1), while
            // the state fragments' LDS reads are in flight (at the start of the
            // step it sat on the path to barrier (1): pass at T = 64K 0.823 ->
            // 0.783 ms); with a ring of two it is the load issued after barrier
            // (1), and with the prologue it is formed there, both before (2).
            auto next_umax = [&]() {
                if constexpr (SCL) {
                    uint32_t mr[NC];
                    u_form(ORING >= 3 ? unext : upre, sln);
#pragma unroll
                    for (int q = 0; q < NC; ++q) mr[q] = wave_umax(u_lmax(ORING >= 3 ? unext : upre, q, sln));
                    if (lane == 0) {
#pragma unroll
                        for (int q = 0; q < NC; ++q) sM[c & 1][q][4 + wo] = __uint_as_float(mr[q]);
                    }
                }
            };
            constexpr bool kEarlyU = ORING >= 3 && !PRO;
            if (urow) {
#pragma unroll
                for (int x = 0; x < UR; ++x)
#pragma unroll
                    for (int q = 0; q < NC; ++q) {
                        // u_ok over the chunk's scale (a power of two: exact)
                        const float f = (SCL ? exp2i(-eo[q]) : 1.f) * u_ok(ucur, q, x);
                        const int sbx = usb + 64 * x / KB;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float uu = (UC ? ucache[sl & 1][(q + NC * x) % (UC ? NC * UR : 1)][e] : u_val(ucur, q, x, e)) * f;
                            const Op hi = (Op)uu;
                            const int ln = (uc + e) + 16 * ug;
                            sU[q][((0 * NSB + sbx) * 64 + ln) * NE + ui] = hi;
                            if constexpr (NUP == 2) sU[q][((1 * NSB + sbx) * 64 + ln) * NE + ui] = (Op)(uu - (float)hi);
                        }
                    }
            }
            __syncthreads();   // (1)
            // the state fragments of Q+ S, read first so that the reads
            // overlap one another and the o tile's store (each waiting on
            // its own: pass at T = 64K 0.865 -> 0.840 ms)
            frag sfo[NC][NKB];
            if (!SAVE && (RT::ALL || rows)) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int q = 0; q < NC; ++q) sfo[q][kb] = lds_bfrag<Op>(sS[q] + kb * TPK * 256, lane);
            }
            if constexpr (kEarlyU) next_umax();   // (see next_umax)
            // The previous chunk's o tile goes out here, ahead of this
            // step's loads, with per-channel gates given as they are; with one
            // w per token and head (fewer loads) or with the fused prologue
            // (raw v staged and convolved here) after them instead. Each order
            // is the faster one for its form (pass at T = 64K, H = 16: 0.802 ->
            // 0.777 ms; 0.790 against 0.823 ms; 0.892 against 0.922 ms).
            if (!SAVE && !WSC && !PRO && c > 0) store_o(c - 1);
            if constexpr (!SAVE) pre.load(blk_of(c + OPD), wo, lane);
            uv_load(upre, c + OPD);
            if constexpr (PRO) conv_u(unext, sln, sl);
            if constexpr (SAVE) {
                if constexpr (!kEarlyU) next_umax();
                __syncthreads();   // (2)
                if constexpr (SCL) {
#pragma unroll
                    for (int q = 0; q < NC; ++q) eo[q] = next_exp(c, q);
                }
                return;
            }
            if ((WSC || PRO) && c > 0) store_o(c - 1);
            // O = 2^e (Q+ (S / 2^e) + P (Delta / 2^e))
            f4 oacc[RPW][NC];
            if (RT::ALL || rows) {
#pragma unroll
                for (int j = 0; j < RPW; ++j)
#pragma unroll
                    for (int q = 0; q < NC; ++q) oacc[j][q] = f4zero();
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int q = 0; q < NC; ++q) {
                        const frag sf = sfo[q][kb];
#pragma unroll
                        for (int j = 0; j < RPW; ++j) oacc[j][q] = M::mma(cur.Qp[j][kb], sf, oacc[j][q]);
                    }
            }
            if constexpr (!kEarlyU) next_umax();
            __syncthreads();   // (2)
            if (RT::ALL || rows) {
                // likewise the Delta fragments (all k-blocks: a row tile's
                // unused ones are in bounds and cost one read)
                frag dfo[NC][NSB];
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                    for (int q = 0; q < NC; ++q) dfo[q][sb] = lds_bfrag<Op>(sD[q] + sb * TPK * 256, lane);
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb) {
                    if (RPW == 1 && sb > sbmax(0)) break;
#pragma unroll
                    for (int q = 0; q < NC; ++q) {
                        const frag df = dfo[q][sb];
#pragma unroll
                        for (int j = 0; j < RPW; ++j) {
                            if (RPW > 1 && sb > sbmax(j)) continue;
                            oacc[j][q] = M::mma(cur.Pm[j][sb], df, oacc[j][q]);
                        }
                    }
                }
            }
            int en[NC];
            if constexpr (SCL) {
#pragma unroll
                for (int q = 0; q < NC; ++q) en[q] = next_exp(c, q);
            }
            if (RT::ALL || rows) {
#pragma unroll
                for (int j = 0; j < RPW; ++j)
#pragma unroll
                    for (int q = 0; q < NC; ++q) {
                        const f4 ov = SCL ? oacc[j][q] * exp2i(eo[q]) : oacc[j][q];
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii)
                            sO[c & 1][(16 * RT::rt(wo, j) + 4 * g4 + ii) * LDO + 16 * q + m16] = ov[ii];
                    }
            }
            if constexpr (SCL) {
#pragma unroll
                for (int q = 0; q < NC; ++q) eo[q] = en[q];
            }
        };
        int c = 0;
        if constexpr (ORING == 4) {
            for (; c + 4 <= nch; c += 4) {
                step(c, g0, g3, u0, u1, u3, 0);
                step(c + 1, g1, g0, u1, u2, u0, 1);
                step(c + 2, g2, g1, u2, u3, u1, 2);
                step(c + 3, g3, g2, u3, u0, u2, 3);
            }
            if (c < nch) step(c, g0, g3, u0, u1, u3, 0);
            if (c + 1 < nch) step(c + 1, g1, g0, u1, u2, u0, 1);
            if (c + 2 < nch) step(c + 2, g2, g1, u2, u3, u1, 2);
        } else if constexpr (ORING == 3) {
            for (; c + 3 <= nch; c += 3) {
                step(c, g0, g2, u0, u1, u2, 0);
                step(c + 1, g1, g0, u1, u2, u0, 1);
                step(c + 2, g2, g1, u2, u0, u1, 2);
            }
            if (c < nch) step(c, g0, g2, u0, u1, u2, 0);
            if (c + 1 < nch) step(c + 1, g1, g0, u1, u2, u0, 1);
        } else {
            for (; c + 2 <= nch; c += 2) {
                step(c, g0, g1, u0, u0, u1, 0);
                step(c + 1, g1, g0, u1, u1, u0, 1);
            }
            if (c < nch) step(c, g0, g1, u0, u0, u1, 0);
        }
        __syncthreads();   // final
        if (!SAVE && nch > 0) store_o(nch - 1);
    }
}


static constexpr int kMaxPrefetchWgs = 8;   // (4 -> 8: saving pass 0.63 -> 0.56 ms, forward pass no change)

// compute units of the current device, queried once per device
static hipError_t device_cus(int *cus)
{
    constexpr int kMaxDev = 64;
    static std::atomic<int> cached[kMaxDev];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if ((e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    *cus = n;
    return hipSuccess;
}

// The chunk bookkeeping of one call as the kernels see it.
static inline Seqs make_seqs(const ChunkArgs &a, const ChunkPlan &p)
{
    Seqs sq;
    sq.m.cu = a.cu_seqlens;
    sq.m.co = a.cu_seqlens ? (const int32_t *)a.workspace : nullptr;
    sq.m.N = a.N;
    sq.m.T = a.T;
    sq.Ttot = a.cu_seqlens ? a.T : a.B * a.T;
    sq.max_chunks = p.max_chunks;
    sq.gates = a.gates;
    return sq;
}

// Shape of the pass grid. One 16-column tile per workgroup with L2 prefetch
// workgroups where the grid stays resident at one workgroup per compute
// unit; two tiles per workgroup where one tile would oversubscribe the chip
// (half the workgroups, each streaming the same operand blocks once for
// twice the columns), with prefetch workgroups if the halved grid leaves room.
struct PassShape {
    bool two;          // two 16-column tiles per workgroup
    int npf;           // prefetch workgroups per chain
    long long grid;    // workgroups
};

template <int DV> static hipError_t pass_shape(long long chains, const ChunkPlan &p, PassShape *ps)
{
    int cus = 0;
    const hipError_t err = device_cus(&cus);
    if (err != hipSuccess) return err;
    const long long groups = (chains + 7) / 8;
    constexpr int NSL1 = DV / 16;
    ps->two = (DV / 16) % 2 == 0 && 8LL * NSL1 * groups > cus;
    const int nsl = ps->two ? NSL1 / 2 : NSL1;
    const int n = (int)std::min<long long>(kMaxPrefetchWgs, cus / (8 * groups) - nsl);
    ps->npf = (n < 2 || p.max_chunks == 0) ? 0 : n;
    ps->grid = 8LL * (nsl + ps->npf) * groups;
    return ps->grid > 0x7fffffffLL ? hipErrorInvalidValue : hipSuccess;
}

template <typename In, typename Op, int DK, int DV>
static hipError_t launch_t(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st,
                           SaveOut so = {nullptr, nullptr, false})
{
    uint8_t *ws = (uint8_t *)a.workspace;
    const Seqs sq = make_seqs(a, p);
    hipError_t err = hipSuccess;
    int *prog = (int *)(ws + p.plan_bytes);
    uint8_t *ops = ws + p.plan_bytes + p.prog_bytes;
    const long long chains = (long long)a.N * a.H;
    if (p.max_chunks > 0) {
        prof_before("gdn2_chunk_prep", st);
        const dim3 pg((unsigned)((long long)p.max_chunks * a.H));
        const ConvIn cq = {a.pro.q.w, a.pro.q.bias, a.pro.q.hist_in}, ck = {a.pro.k.w, a.pro.k.bias, a.pro.k.hist_in};
        auto prep = [&](auto kern) {
            hipLaunchKernelGGL(kern, pg, dim3(256), 0, st, (const In *)a.q, (const In *)a.k, a.log_alpha,
                               (const In *)a.b, sq, a.H, ops, prog, (int)chains, cq, ck);
        };
        if (a.pro.on) prep(chunk_prep_kernel<In, Op, DK, 0, true>);
        else switch (a.gates & (kGateB | kGateAlpha)) {
        case 0: prep(chunk_prep_kernel<In, Op, DK, 0, false>); break;
        case kGateB: prep(chunk_prep_kernel<In, Op, DK, kGateB, false>); break;
        case kGateAlpha: prep(chunk_prep_kernel<In, Op, DK, kGateAlpha, false>); break;
        default: prep(chunk_prep_kernel<In, Op, DK, kGateB | kGateAlpha, false>); break;
        }
        prof_after(st);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    PassShape ps;
    if ((err = pass_shape<DV>(chains, p, &ps)) != hipSuccess) return err;
    const bool two = ps.two;
    const int npf = ps.npf;
    prof_before(so.S && so.with_out ? "gdn2_chunk_pass_keep" : "gdn2_chunk_pass", st);
    const ConvIn cv = {a.pro.v.w, a.pro.v.bias, a.pro.v.hist_in};
    auto pass = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)ps.grid), dim3(512), 0, st, (const In *)a.v, (const In *)a.w, a.S0,
                           (float *)a.o, a.ST, sq, a.H, (const uint8_t *)ops, prog, npf, cv, so);
    };
    const bool wsc = a.gates & kGateW;
    if (so.S && so.with_out) {
        // the training forward: o and S_T, and S_c, Delta kept for the backward
        if constexpr ((DV / 16) % 2 == 0) {
            if (two) pass(chunk_pass_kernel<In, Op, DK, DV, 2, false, false, false, 64, true>);
            else pass(chunk_pass_kernel<In, Op, DK, DV, 1, false, false, false, 64, true>);
        } else pass(chunk_pass_kernel<In, Op, DK, DV, 1, false, false, false, 64, true>);
    } else if (so.S) {
        // the forward part of the backward: per-channel gates, raw inputs
        if constexpr ((DV / 16) % 2 == 0) {
            if (two) pass(chunk_pass_kernel<In, Op, DK, DV, 2, false, false, true>);
            else pass(chunk_pass_kernel<In, Op, DK, DV, 1, false, false, true>);
        } else pass(chunk_pass_kernel<In, Op, DK, DV, 1, false, false, true>);
    } else if (two) {
        if constexpr ((DV / 16) % 2 == 0) {
            if (a.pro.on) pass(chunk_pass_kernel<In, Op, DK, DV, 2, false, true>);
            else if (wsc) pass(chunk_pass_kernel<In, Op, DK, DV, 2, true, false>);
            else pass(chunk_pass_kernel<In, Op, DK, DV, 2, false, false>);
        }
    } else {
        if (a.pro.on) pass(chunk_pass_kernel<In, Op, DK, DV, 1, false, true>);
        else if (wsc) pass(chunk_pass_kernel<In, Op, DK, DV, 1, true, false>);
        else pass(chunk_pass_kernel<In, Op, DK, DV, 1, false, false>);
    }
    prof_after(st);
    return hipGetLastError();
}

template <typename In, typename Op, int DK>
hipError_t dispatch_dv(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st)
{
    switch (a.dv) {
    case 16: return launch_t<In, Op, DK, 16>(a, p, st);
    case 32: return launch_t<In, Op, DK, 32>(a, p, st);
    case 64: return launch_t<In, Op, DK, 64>(a, p, st);
    case 128: return launch_t<In, Op, DK, 128>(a, p, st);
    }
    return hipErrorInvalidValue;
}

} // namespace gdn2
