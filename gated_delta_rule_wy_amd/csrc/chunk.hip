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
// the products above are formed as (row factor) x (column factor). Row block
// R (rows 16R..16R+15) uses ref_R = g_{16R-1} (0 for R = 0):
//   off-diagonal blocks S < R: e^{g_r - ref_R} * e^{ref_R - ref_{S+1}} * e^{ref_{S+1} - g_s},
//   every factor <= 1, so nothing overflows whatever the decay;
//   diagonal blocks: factors around the block's middle row, which are bounded
//   by e^{LIM}; a block whose decay spread exceeds LIM is computed exactly
//   (pairwise exponents) on the vector ALUs instead.
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"

#include <type_traits>

namespace gdn2 {

// Operand block written by chunk_prep for one (chunk, head); every fragment
// is 64 lanes x 16 bytes in the lane order the consumer loads it.
template <typename Op, int DK> struct Blk {
    using M = Mma<Op>;
    static constexpr int KB = M::KB, NE = M::NE;
    static constexpr int NKB = DK / KB;   // k-blocks over key channels
    static constexpr int NSB = 64 / KB;   // k-blocks over chunk rows
    static constexpr int NCT = DK / 16;   // 16-row tiles over key channels
    static constexpr size_t FRAG = 64 * 16;
    static constexpr size_t oW = 0;                          // -W   [4][NKB] frags
    static constexpr size_t oQ = oW + 4 * NKB * FRAG;        // Q+   [4][NKB]
    static constexpr size_t oK = oQ + 4 * NKB * FRAG;        // Khat^T [NCT][NSB]
    static constexpr size_t oP = oK + NCT * NSB * FRAG;      // P    [4][NSB]
    static constexpr size_t oT = oP + 4 * NSB * FRAG;        // T    [4][NSB]
    static constexpr size_t oG = oT + 4 * NSB * FRAG;        // gamma float[DK]
    static constexpr size_t bytes = (oG + DK * 4 + 255) / 256 * 256;
};

template <typename Op> struct Lim;
template <> struct Lim<_Float16> { static constexpr float v = 8.0f; };
template <> struct Lim<float> { static constexpr float v = 60.0f; };

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// ---------------------------------------------------------------------------
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

// Token range and chunk ids with the host-unchecked preconditions made safe:
// offsets are clamped into [0, Ttot] and chunk ids capped at max_chunks.
struct Seqs {
    SeqMap m;
    int Ttot, max_chunks;
    __device__ __forceinline__ int t0(int i) const { return clampi(m.tok0(i), 0, Ttot); }
    __device__ __forceinline__ int t1(int i) const { return clampi(m.tok1(i), t0(i), Ttot); }
};

// ---------------------------------------------------------------------------
template <typename In, typename Op, int DK>
__global__ __launch_bounds__(256) void chunk_prep_kernel(
    const In *__restrict__ q, const In *__restrict__ k, const float *__restrict__ la,
    const In *__restrict__ b, Seqs sq, int H, uint8_t *__restrict__ ops)
{
    using M = Mma<Op>;
    using L = Blk<Op, DK>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NE = M::NE, NKB = L::NKB, NSB = L::NSB, NCT = L::NCT;
    constexpr int PAD = 16 / (int)sizeof(Op);
    constexpr int LDE = DK + PAD;               // row stride of the [64][DK] tiles
    constexpr int LDT = 64 + PAD;               // row stride of the [64][64] tiles
    constexpr int REG = 64 * (LDE > LDT ? LDE : LDT);
    constexpr int LDA = 65;
    constexpr int CP = DK / 2, NRG = 256 / CP, RPG = 64 / NRG;
    constexpr float LIM = Lim<Op>::v;

    __shared__ __attribute__((aligned(16))) Op sE[REG];   // E^ ; later -W staging
    __shared__ __attribute__((aligned(16))) Op sQ[REG];   // Q^ ; later P
    __shared__ __attribute__((aligned(16))) Op sK[REG];   // K- ; later T
    __shared__ float sA[64 * LDA];                        // A (fp32); early: cumsum scratch
    __shared__ float sTab[19 * DK];
    __shared__ int sFlag[4];

    const int j = blockIdx.x, h = blockIdx.y, t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6, m16 = lane & 15, g4 = lane >> 4;
    if (j >= min(sq.m.nchunks(), sq.max_chunks)) return;
    const int i = sq.m.seq_of(j);
    const int t0 = sq.t0(i) + 64 * (j - sq.m.chunk0(i));
    const int n = min(64, sq.t1(i) - t0);
    uint8_t *blk = ops + ((size_t)j * H + h) * L::bytes;

    // tables: [0,4) e^{ref_R}  [4,8) e^{g_n - ref_{R+1}}  [8,11) e^{ref_R - ref_{S+1}}
    //         for (R,S) = (2,0),(3,0),(3,1)   [11,15) e^{ref_R - mid_R}  [15,19) e^{mid_R - ref_{R+1}}
    float *tExpRef = sTab, *tExpKh = sTab + 4 * DK, *tDec = sTab + 8 * DK;
    float *tDiagE = sTab + 11 * DK, *tDiagK = sTab + 15 * DK;

    // ---- stage 1: cumulative log-decay g (registers), block references ----
    const int cp = t % CP, rg = t / CP, c0 = 2 * cp, r0 = rg * RPG;
    float *sPart = sA;                  // [NRG][DK]
    float *sRef = sA + NRG * DK;        // [5][DK]: ref_0..ref_4 (ref_4 = g_n)
    float *sMid = sRef + 5 * DK;        // [4][DK]
    f2 al[RPG], gg[RPG];
    {
        f2 run = {0.f, 0.f};
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const int r = r0 + u;
            f2 x = {0.f, 0.f};
            if (r < n) x = *reinterpret_cast<const f2 *>(la + ((size_t)(t0 + r) * H + h) * DK + c0);
            al[u][0] = __expf(x[0]);
            al[u][1] = __expf(x[1]);
            run += x;
            gg[u] = run;
        }
        *reinterpret_cast<f2 *>(sPart + rg * DK + c0) = run;
    }
    if (t < 4) sFlag[t] = 0;
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
        }
        if (rg == 0) { sRef[c0] = 0.f; sRef[c0 + 1] = 0.f; }
    }
    __syncthreads();

    // ---- stage 2: factor tables, gamma, decay-scaled operands in LDS ----
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
    if (t < DK) reinterpret_cast<float *>(blk + L::oG)[t] = __expf(sRef[4 * DK + t]);
    {
        // e1_r = e^{g_r - ref_R} forward, e2_r = e^{ref_{R+1} - g_r} backward,
        // both as running products of alpha within the 16-row block.
        f2 e1[RPG], e2[RPG];
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const int r = r0 + u;
            if ((r & 15) == 0) e1[u] = al[u];
            else if (u == 0) {
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
            f2 kv = {0.f, 0.f}, bv = {0.f, 0.f}, qv = {0.f, 0.f};
            if (r < n) {
                const size_t off = ((size_t)(t0 + r) * H + h) * DK + c0;
                kv = Ld<In>::two(k + off);
                bv = Ld<In>::two(b + off);
                qv = Ld<In>::two(q + off);
            }
            const f2 eh = bv * kv * e1[u], qh = qv * e1[u], kb_ = kv * e2[u];
            sE[r * LDE + c0] = (Op)eh[0]; sE[r * LDE + c0 + 1] = (Op)eh[1];
            sQ[r * LDE + c0] = (Op)qh[0]; sQ[r * LDE + c0 + 1] = (Op)qh[1];
            sK[r * LDE + c0] = (Op)kb_[0]; sK[r * LDE + c0 + 1] = (Op)kb_[1];
        }
    }
    __syncthreads();

    // ---- stage 3: A and P blocks on the matrix cores; pack Q+ and Khat^T ----
    // zero the strictly-upper 16x16 blocks of A
    for (int idx = t; idx < 6 * 256; idx += 256) {
        const int bi = idx >> 8, e = idx & 255;
        const int R = bi < 3 ? 0 : (bi < 5 ? 1 : 2);
        const int S = bi < 3 ? bi + 1 : (bi < 5 ? bi - 1 : 3);
        sA[(16 * R + (e >> 4)) * LDA + 16 * S + (e & 15)] = 0.f;
    }
    const bool any_slow = sFlag[0] | sFlag[1] | sFlag[2] | sFlag[3];
    // wave wv takes jobs wv + 4*qq: ids 0..9 are the A blocks, 10..19 the P blocks
    f4 pacc[5];
    int ptile[5];
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
    // Q+ fragments: rows 16 mt + m, channels kb*KB + kofs; scaled by e^{ref_R}
    for (int f = wv; f < 4 * NKB; f += 4) {
        const int mt = f / NKB, kb = f % NKB;
        frag a;
#pragma unroll
        for (int i4 = 0; i4 < NE; ++i4) {
            const int ch = kb * KB + kofs(g4, i4);
            a[i4] = (Op)((float)sQ[(16 * mt + m16) * LDE + ch] * tExpRef[mt * DK + ch]);
        }
        *reinterpret_cast<frag *>(blk + L::oQ + ((size_t)f * 64 + lane) * 16) = a;
    }
    // Khat^T fragments: rows = channel 16 ct + m, contraction = chunk rows
    for (int f = wv; f < NCT * NSB; f += 4) {
        const int ct = f / NSB, sb = f % NSB;
        const int c = 16 * ct + m16;
        frag a;
#pragma unroll
        for (int i4 = 0; i4 < NE; ++i4) {
            const int s = sb * KB + kofs(g4, i4);
            a[i4] = (Op)((float)sK[s * LDE + c] * tExpKh[(s >> 4) * DK + c]);
        }
        *reinterpret_cast<frag *>(blk + L::oK + ((size_t)f * 64 + lane) * 16) = a;
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
                const size_t br = ((size_t)(t0 + r) * H + h) * DK, bs = ((size_t)(t0 + s) * H + h) * DK;
                for (int c = 0; c < DK; ++c) {
                    float d = 0.f;
                    for (int x = s + 1; x <= r; ++x) d += la[((size_t)(t0 + x) * H + h) * DK + c];
                    const float e = __expf(d) * Ld<In>::one(k + bs + c);
                    aA += Ld<In>::one(b + br + c) * Ld<In>::one(k + br + c) * e;
                    aP += Ld<In>::one(q + br + c) * e;
                }
            }
            sA[r * LDA + s] = sl < rl ? aA : 0.f;
            sP[r * LDT + s] = (Op)aP;
        }
    }
    __syncthreads();

    // ---- stage 5: T = (I + A)^{-1}, block forward substitution ----
    {
        const int R = wv;
        if (lane < 16) {
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < r; ++s) acc -= sA[(16 * R + r) * LDA + 16 * R + s] * x[s];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sT[(16 * R + r) * LDT + 16 * R + lane] = (Op)x[r];
        }
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

    // ---- stage 6: W = T E (E_s = E^_s e^{ref_R(s)}); pack -W, P, T ----
    constexpr int NWT = (4 * NCT + 3) / 4;
    f4 wacc[NWT];
#pragma unroll
    for (int qq = 0; qq < NWT; ++qq) {
        const int f = wv + 4 * qq;
        wacc[qq] = f4zero();
        if (f >= 4 * NCT) continue;
        const int mt = f / NCT, nt = f % NCT;
        const int sbmax = (16 * mt + 15) / KB;
        for (int sb = 0; sb <= sbmax; ++sb) {
            frag a, bb;
#pragma unroll
            for (int i4 = 0; i4 < NE; ++i4) {
                const int s = sb * KB + kofs(g4, i4);
                a[i4] = sT[(16 * mt + m16) * LDT + s];
                const int c = 16 * nt + m16;
                bb[i4] = (Op)((float)sE[s * LDE + c] * tExpRef[(s >> 4) * DK + c]);
            }
            wacc[qq] = M::mma(a, bb, wacc[qq]);
        }
    }
    // P and T fragments
    for (int f = wv; f < 4 * NSB; f += 4) {
        const int mt = f / NSB, sb = f % NSB;
        frag a, c;
#pragma unroll
        for (int i4 = 0; i4 < NE; ++i4) {
            const int s = sb * KB + kofs(g4, i4);
            a[i4] = sP[(16 * mt + m16) * LDT + s];
            c[i4] = sT[(16 * mt + m16) * LDT + s];
        }
        *reinterpret_cast<frag *>(blk + L::oP + ((size_t)f * 64 + lane) * 16) = a;
        *reinterpret_cast<frag *>(blk + L::oT + ((size_t)f * 64 + lane) * 16) = c;
    }
    __syncthreads();   // every read of E^ done
#pragma unroll
    for (int qq = 0; qq < NWT; ++qq) {
        const int f = wv + 4 * qq;
        if (f >= 4 * NCT) continue;
        const int mt = f / NCT, nt = f % NCT;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            sW[(16 * mt + 4 * g4 + ii) * LDE + 16 * nt + m16] = (Op)(-wacc[qq][ii]);
    }
    __syncthreads();
    for (int f = wv; f < 4 * NKB; f += 4) {
        const int mt = f / NKB, kb = f % NKB;
        frag a;
#pragma unroll
        for (int i4 = 0; i4 < NE; ++i4) a[i4] = sW[(16 * mt + m16) * LDE + kb * KB + kofs(g4, i4)];
        *reinterpret_cast<frag *>(blk + L::oW + ((size_t)f * 64 + lane) * 16) = a;
    }
}

// ---------------------------------------------------------------------------
// Sequential state pass.
//
// Workgroup = (chain = sequence*H + head, 16-column slice of dv); wave w owns
// rows 16w..16w+15 of each chunk's Delta and O, and state tiles
// [w*TPW, (w+1)*TPW) (16 key channels each). Per chunk, two barriers:
//   1: state operand tiles and U = w*v (hi + lo f16) ready in LDS
//      Delta_w = T_w U - W_w S,  O_w = Q+_w S          (MFMA)
//   2: Delta tiles ready in LDS
//      O_w += P_w Delta,  S_tile = gamma * S_tile + Khat^T_tile Delta
// The next chunk's operand fragments and v/w tile are loaded into registers
// while the current chunk computes.
//
// Workgroups are numbered so that the slices of one chain land on the same
// XCD (the dispatcher deals workgroups to the 8 XCDs round-robin), where they
// share that XCD's L2 for the chain's operand blocks.
template <typename Op, int DK> struct PassFrags {
    using M = Mma<Op>;
    using L = Blk<Op, DK>;
    using frag = typename M::frag;
    static constexpr int TPW = (L::NCT + 3) / 4;
    frag nW[L::NKB], Qp[L::NKB], Ti[L::NSB], Pm[L::NSB], Kh[TPW][L::NSB];
    f4 gam[TPW];
    __device__ __forceinline__ void load(const uint8_t *blk, int wv, int lane) {
#pragma unroll
        for (int kb = 0; kb < L::NKB; ++kb) {
            nW[kb] = *reinterpret_cast<const frag *>(blk + L::oW + ((size_t)(wv * L::NKB + kb) * 64 + lane) * 16);
            Qp[kb] = *reinterpret_cast<const frag *>(blk + L::oQ + ((size_t)(wv * L::NKB + kb) * 64 + lane) * 16);
        }
#pragma unroll
        for (int sb = 0; sb < L::NSB; ++sb) {
            Ti[sb] = *reinterpret_cast<const frag *>(blk + L::oT + ((size_t)(wv * L::NSB + sb) * 64 + lane) * 16);
            Pm[sb] = *reinterpret_cast<const frag *>(blk + L::oP + ((size_t)(wv * L::NSB + sb) * 64 + lane) * 16);
        }
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

// v and w for one chunk and column slice: thread t holds row t/4, columns
// 4*(t%4)..+3 of both.
template <typename In> struct UVTile {
    In v[4], w[4];
    // `off` always addresses a valid row; `ok` false zeroes the values after
    // the load (no branch, so the load count per iteration stays fixed)
    __device__ __forceinline__ void load(const In *vp, const In *wp, size_t off, bool ok) {
        if constexpr (sizeof(In) == 2) {
            uint2 a = *reinterpret_cast<const uint2 *>(vp + off);
            uint2 b = *reinterpret_cast<const uint2 *>(wp + off);
            v[0] = (In)(a.x & 0xFFFF); v[1] = (In)(a.x >> 16); v[2] = (In)(a.y & 0xFFFF); v[3] = (In)(a.y >> 16);
            w[0] = (In)(b.x & 0xFFFF); w[1] = (In)(b.x >> 16); w[2] = (In)(b.y & 0xFFFF); w[3] = (In)(b.y >> 16);
        } else {
            const f4 a = *reinterpret_cast<const f4 *>(vp + off);
            const f4 b = *reinterpret_cast<const f4 *>(wp + off);
#pragma unroll
            for (int e = 0; e < 4; ++e) { v[e] = a[e]; w[e] = b[e]; }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) { v[e] = ok ? v[e] : (In)0; w[e] = ok ? w[e] : (In)0; }
    }
};

template <typename In> __device__ __forceinline__ float in2f(In x);
template <> __device__ __forceinline__ float in2f<uint16_t>(uint16_t x) { return bf16f(x); }
template <> __device__ __forceinline__ float in2f<float>(float x) { return x; }

template <typename In, typename Op, int DK, int DV>
__global__ __launch_bounds__(256) void chunk_pass_kernel(
    const In *__restrict__ v, const In *__restrict__ w, const float *__restrict__ S0,
    float *__restrict__ o, float *__restrict__ ST, Seqs sq, int H,
    const uint8_t *__restrict__ ops)
{
    using M = Mma<Op>;
    using L = Blk<Op, DK>;
    using frag = typename M::frag;
    using F = PassFrags<Op, DK>;
    constexpr int KB = M::KB, NE = M::NE, NKB = L::NKB, NSB = L::NSB, NCT = L::NCT;
    constexpr int TPW = F::TPW;
    constexpr int TPK = KB / 16;              // accumulator tiles per k-block
    constexpr int NSL = DV / 16;              // column slices

    __shared__ __attribute__((aligned(16))) Op sS[NCT * 64 * 4];        // state operand tiles
    __shared__ __attribute__((aligned(16))) Op sD[4 * 64 * 4];          // Delta tiles
    __shared__ __attribute__((aligned(16))) Op sU[2 * NSB * 64 * NE];   // U hi / lo B-fragments

    // XCD-aware numbering: slices of chain c sit on XCD c % 8
    const int Lid = blockIdx.x;
    const int kq = Lid >> 3, js = kq % NSL;
    const int chain = (kq / NSL) * 8 + (Lid & 7);
    const int chains = sq.m.N * H;
    if (chain >= chains) return;
    const int i = chain / H, h = chain % H;

    const int t = threadIdx.x;
    const int lane = t & 63, wv = t >> 6, m16 = lane & 15, g4 = lane >> 4;
    const int col = 16 * js + m16;
    const size_t sbase = ((size_t)i * H + h) * DK * DV;

    f4 Sr[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int ct = wv * TPW + u;
        Sr[u] = f4zero();
        if (ct < NCT) {
            if (S0) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) Sr[u][ii] = S0[sbase + (size_t)(16 * ct + 4 * g4 + ii) * DV + col];
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sS[(ct * 64 + lane) * 4 + ii] = (Op)Sr[u][ii];
        }
    }

    const int tb = sq.t0(i), te = sq.t1(i);
    const int cbeg = sq.m.chunk0(i);
    const int nch = min((te - tb + 63) >> 6, max(0, sq.max_chunks - cbeg));
    const int sbmax = (16 * wv + 15) / KB;
    // v / w tile coordinates of this thread
    const int ur = t >> 2, uc = 4 * (t & 3);
    const size_t uoff0 = (size_t)h * DV + 16 * js + uc;
    // where this thread's 4 U values go in the B-fragment layout
    const int usb = ur / KB, usl = ur % KB;
    const int ug = (usl & 15) >> 2, ui = 4 * (usl >> 4) + (usl & 3);

    auto blk_of = [&](int c) { return ops + ((size_t)(cbeg + c) * H + h) * L::bytes; };
    auto uv_ok = [&](int c) { return tb + 64 * c + ur < te; };
    auto uv_off = [&](int c) { return (size_t)min(tb + 64 * c + ur, te - 1) * H * DV + uoff0; };

    F fa, fb;
    UVTile<In> ua, ub;
    if (nch > 0) {
        fa.load(blk_of(0), wv, lane);
        ua.load(v, w, uv_off(0), uv_ok(0));
    }

    // One chunk. The next chunk's loads are issued unconditionally (the index
    // is clamped, re-reading the last chunk at the end) so that the compiler
    // can count them and only wait for the current chunk's data. LAST marks
    // the final, possibly partial, chunk: only there are o stores guarded.
    auto step = [&](auto last_tag, int c, F &cur, F &nxt, UVTile<In> &ucur, UVTile<In> &unxt) {
        constexpr bool LAST = decltype(last_tag)::value;
        const int tok = tb + 64 * c;
        const int n = min(64, te - tok);
        const int cn = min(c + 1, nch - 1);
        nxt.load(blk_of(cn), wv, lane);
        unxt.load(v, w, uv_off(cn), uv_ok(cn));
        // U = w * v as hi + lo operand-precision parts, into B-fragment order
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float uu = in2f<In>(ucur.w[e]) * in2f<In>(ucur.v[e]);
            const Op hi = (Op)uu;
            const int ln = (uc + e) + 16 * ug;
            sU[((0 * NSB + usb) * 64 + ln) * NE + ui] = hi;
            sU[((1 * NSB + usb) * 64 + ln) * NE + ui] = (Op)(uu - (float)hi);
        }
        __syncthreads();   // (1) state tiles and U ready

        f4 acc = f4zero(), oacc = f4zero();
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            if (sb > sbmax) break;
            const frag uh = *reinterpret_cast<const frag *>(&sU[((0 * NSB + sb) * 64 + lane) * NE]);
            const frag ul = *reinterpret_cast<const frag *>(&sU[((1 * NSB + sb) * 64 + lane) * NE]);
            acc = M::mma(cur.Ti[sb], uh, acc);
            acc = M::mma(cur.Ti[sb], ul, acc);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            frag sbf;
#pragma unroll
            for (int p = 0; p < TPK; ++p) {
                typedef Op op4 __attribute__((ext_vector_type(4)));
                const op4 x = *reinterpret_cast<const op4 *>(&sS[((kb * TPK + p) * 64 + lane) * 4]);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) sbf[4 * p + ii] = x[ii];
            }
            acc = M::mma(cur.nW[kb], sbf, acc);
            oacc = M::mma(cur.Qp[kb], sbf, oacc);
        }
        {
            typedef Op op4 __attribute__((ext_vector_type(4)));
            op4 x;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) x[ii] = (Op)acc[ii];
            *reinterpret_cast<op4 *>(&sD[(wv * 64 + lane) * 4]) = x;
        }
        __syncthreads();   // (2) Delta tiles ready

        frag Db[NSB];
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int p = 0; p < TPK; ++p) {
                typedef Op op4 __attribute__((ext_vector_type(4)));
                const op4 x = *reinterpret_cast<const op4 *>(&sD[((sb * TPK + p) * 64 + lane) * 4]);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) Db[sb][4 * p + ii] = x[ii];
            }
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            if (sb > sbmax) break;
            oacc = M::mma(cur.Pm[sb], Db[sb], oacc);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int r = 16 * wv + 4 * g4 + ii;
            if (!LAST || r < n) o[((size_t)(tok + r) * H + h) * DV + col] = oacc[ii];
        }
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int ct = wv * TPW + u;
            if (NCT % 4 != 0 && ct >= NCT) continue;
            f4 s = Sr[u] * cur.gam[u];
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) s = M::mma(cur.Kh[u][sb], Db[sb], s);
            Sr[u] = s;
            typedef Op op4 __attribute__((ext_vector_type(4)));
            op4 x;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) x[ii] = (Op)s[ii];
            *reinterpret_cast<op4 *>(&sS[(ct * 64 + lane) * 4]) = x;
        }
    };

    using NotLast = std::integral_constant<bool, false>;
    using Last = std::integral_constant<bool, true>;
    int c = 0;
    for (; c + 2 < nch; c += 2) {
        step(NotLast{}, c, fa, fb, ua, ub);
        step(NotLast{}, c + 1, fb, fa, ub, ua);
    }
    if (c + 1 < nch) {
        step(NotLast{}, c, fa, fb, ua, ub);
        step(Last{}, c + 1, fb, fa, ub, ua);
    } else if (c < nch) {
        step(Last{}, c, fa, fb, ua, ub);
    }

    if (ST) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int ct = wv * TPW + u;
            if (ct >= NCT) continue;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) ST[sbase + (size_t)(16 * ct + 4 * g4 + ii) * DV + col] = Sr[u][ii];
        }
    }
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
    if (mc > 0x7fffffffLL) return false;
    p->max_chunks = (int)mc;
    p->plan_bytes = varlen ? ((size_t)(N + 1) * 4 + 255) / 256 * 256 : 0;
    p->block_bytes = bb;
    p->total_bytes = p->plan_bytes + (size_t)mc * H * bb;
    return true;
}

template <typename In, typename Op, int DK, int DV>
static hipError_t launch_t(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st)
{
    uint8_t *ws = (uint8_t *)a.workspace;
    Seqs sq;
    sq.m.cu = a.cu_seqlens;
    sq.m.co = a.cu_seqlens ? (const int32_t *)ws : nullptr;
    sq.m.N = a.N;
    sq.m.T = a.T;
    sq.Ttot = a.cu_seqlens ? a.T : a.B * a.T;
    sq.max_chunks = p.max_chunks;
    hipError_t err = hipSuccess;
    if (a.cu_seqlens) {
        prof_before("gdn2_chunk_plan", st);
        hipLaunchKernelGGL(chunk_plan_kernel, dim3(1), dim3(1024), 0, st, a.cu_seqlens, a.N, a.T,
                           p.max_chunks, (int32_t *)ws);
        prof_after(st);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    uint8_t *ops = ws + p.plan_bytes;
    if (p.max_chunks > 0) {
        prof_before("gdn2_chunk_prep", st);
        hipLaunchKernelGGL((chunk_prep_kernel<In, Op, DK>), dim3(p.max_chunks, a.H), dim3(256), 0, st,
                           (const In *)a.q, (const In *)a.k, a.log_alpha, (const In *)a.b, sq, a.H, ops);
        prof_after(st);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    prof_before("gdn2_chunk_pass", st);
    const long long chains = (long long)a.N * a.H;
    const long long pass_grid = 8LL * (DV / 16) * ((chains + 7) / 8);
    if (pass_grid > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((chunk_pass_kernel<In, Op, DK, DV>), dim3((unsigned)pass_grid), dim3(256), 0, st,
                       (const In *)a.v, (const In *)a.w, a.S0, (float *)a.o, a.ST, sq, a.H,
                       (const uint8_t *)ops);
    prof_after(st);
    return hipGetLastError();
}

template <typename In, typename Op, int DK>
static hipError_t dispatch_dv(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st)
{
    switch (a.dv) {
    case 16: return launch_t<In, Op, DK, 16>(a, p, st);
    case 32: return launch_t<In, Op, DK, 32>(a, p, st);
    case 64: return launch_t<In, Op, DK, 64>(a, p, st);
    case 128: return launch_t<In, Op, DK, 128>(a, p, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st)
{
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
