// Chunk-size variants of the chunkwise prefill: chunks of 32 or 128 tokens
// instead of 64 (snilld.dk, section "POC-matrix der dækker de hårde
// hjørner": latency, throughput and peak memory are to be measured at C = 32
// and 128 besides the C = 64 of the implementation). A longer chunk halves
// the serial chain of the pass and doubles the triangular work per token; a
// shorter one does the opposite.
//
// The pass is the C = 64 pass kernel with the chunk size as a template
// parameter (RowTiles: two row tiles per wave at C = 128, waves 2 and 3 idle
// on rows at C = 32). The prep below is written for any C; it forms the same
// operand block (Blk<Op, DK, C>) as the C = 64 prep, with a layout that keeps
// 128-token chunks within one compute unit's LDS:
//  * A and P are computed transposed (K-side operand as the A fragment), so
//    an accumulator lane holds one row and four consecutive columns of the
//    block: exactly half (f16) or all (fp32) of a row-major A-fragment lane.
//    P goes from the accumulators straight to the operand block, A into LDS
//    as 16x16 blocks of its lower triangle only.
//  * T is kept the same way (lower blocks), and W = T E is formed transposed
//    too, so -W also goes from the accumulators to the operand block.
//  * A takes the space of the Q- and K-side operands once those are packed;
//    the cumulative-decay scratch sits where T goes later.
// Per-channel gates only, no fused prologue; the backward uses C = 64.
#pragma once

#include "chunk_impl.hpp"

namespace gdn2 {

constexpr size_t cmax_sz(size_t a, size_t b) { return a > b ? a : b; }

// threads of the prep workgroup: 4 waves, 8 for 128-token chunks
template <int CS> constexpr int prep_cs_threads() { return CS >= 128 ? 512 : 256; }

// LDS plan of the chunk-size-generic prep (byte offsets into one array).
template <typename Op, int DK, int CS> struct PrepCS {
    static constexpr int NRB = CS / 16;                  // 16-row tiles of the chunk
    static constexpr int NTB = NRB * (NRB + 1) / 2;      // lower 16x16 blocks, diagonal included
    static constexpr int NT = prep_cs_threads<CS>();
    static constexpr int NW = NT / 64;                   // waves
    static constexpr int LDE = DK + 4;                   // row stride of the [CS][DK] operand tiles
    static constexpr int BLD = 20;                       // row stride of a stored 16x16 block
    static constexpr int BSZ = 16 * BLD;                 // elements per stored block
    static constexpr int CP = DK / 2, NRG = NT / CP, RPG = CS / NRG;   // 2 channels x RPG rows per thread
    static_assert(RPG >= 1 && RPG * NRG == CS, "rows per thread");
    static constexpr size_t bE = (size_t)CS * LDE * sizeof(Op);
    static constexpr size_t bA = (size_t)NTB * BSZ * 4;
    static constexpr size_t bT = (size_t)NTB * BSZ * sizeof(Op);
    static constexpr int NDEC = (NRB - 1) * (NRB - 2) / 2;         // block pairs (R, S), R >= S + 2
    // scratch: partial sums, references, middles, g at row 0; then the slow
    // path's factor tables (diagonal E and K sides, off-diagonal pairs)
    static constexpr size_t bScr = (size_t)(NRG + 2 * NRB + 2 + 2 * NRB + NDEC) * DK * 4;
    static constexpr size_t bTab = (size_t)2 * NRB * DK * 4;
    static constexpr size_t oE = 0;                                  // E-side operand
    static constexpr size_t oQK = oE + bE;                           // Q-, K-side operands; then A
    static constexpr size_t oT = oQK + cmax_sz(2 * bE, bA);          // scratch; then T
    static constexpr size_t oTab = oT + cmax_sz(bT, bScr);           // decay tables
    static constexpr size_t oFlag = oTab + bTab;                     // flags
    static constexpr size_t bytes = oFlag + 16 * 4;
    static constexpr bool fits = bytes <= 160 * 1024;
    static __device__ __forceinline__ int bidx(int R, int S) { return R * (R + 1) / 2 + S; }
};

// Chunk preparation for CS-token chunks, one workgroup per (chunk, head).
// Same stages and decay factoring as chunk_prep_kernel (per-channel gates):
// the chunk-wide midpoint when the chunk's decay spread is moderate, else
// row-block references with exact pairwise exponents for diagonal blocks
// whose spread is too large.
template <typename In, typename Op, int DK, int CS>
__global__ __launch_bounds__(prep_cs_threads<CS>()) void chunk_prep_cs_kernel(
    const In *__restrict__ q, const In *__restrict__ k, const float *__restrict__ la,
    const In *__restrict__ b, Seqs sq, int H, uint8_t *__restrict__ ops, int *__restrict__ prog, int nprog)
{
    using M = Mma<Op>;
    using L = Blk<Op, DK, CS>;
    using PL = PrepCS<Op, DK, CS>;
    using frag = typename M::frag;
    using raw2 = typename Ld<In>::raw2;
    typedef Op op4 __attribute__((ext_vector_type(4)));
    constexpr int KB = M::KB, NE = M::NE, NKB = L::NKB, NSB = L::NSB, NCT = L::NCT, NRB = L::NRB;
    constexpr int NW = PL::NW, NT = PL::NT, LDE = PL::LDE, BLD = PL::BLD, BSZ = PL::BSZ;
    constexpr int CP = PL::CP, RPG = PL::RPG, NRG = PL::NRG, NTB = PL::NTB;
    constexpr int HPB = KB / 16;   // 16-column halves per k-block
    constexpr float LIM = Lim<Op>::v;
    constexpr float LIMC = Lim<Op>::chunk;
    static_assert(PL::fits, "LDS plan above 160 KB");

    __shared__ __attribute__((aligned(16))) uint8_t lds[PL::bytes];
    Op *sE = (Op *)(lds + PL::oE);
    Op *sQ = (Op *)(lds + PL::oQK), *sK = sQ + CS * LDE;
    float *sA = (float *)(lds + PL::oQK);
    Op *sT = (Op *)(lds + PL::oT);
    float *sPart = (float *)(lds + PL::oT);   // [NRG][DK]
    float *sRef = sPart + NRG * DK;           // [NRB + 1][DK]: ref_0..ref_NRB (ref_NRB = g at the last row)
    float *sMid = sRef + (NRB + 1) * DK;      // [NRB][DK]
    float *sG0 = sMid + NRB * DK;             // [DK]: g at the first row
    // slow path: e^{ref_R - mid_R} (E side) and e^{mid_R - ref_{R+1}} (K side)
    // of diagonal block R; e^{ref_R - ref_{S+1}} of block (R, S), R >= S + 2,
    // at row (R - 2)(R - 1)/2 + S
    float *tDiagE = sG0 + DK, *tDiagK = tDiagE + NRB * DK, *tDec = tDiagK + NRB * DK;
    // [0, NRB): Q+ / E scale per row block; [NRB, 2 NRB): Khat scale (the fast path uses rows 0 and NRB)
    float *tExpRef = (float *)(lds + PL::oTab), *tExpKh = tExpRef + NRB * DK;
    int *sFlag = (int *)(lds + PL::oFlag);    // [0, NRB): exact diagonal blocks; [NRB]: slow chunk

    // chunks dealt last to first, all heads of a chunk together (as chunk_prep_kernel)
    const int t = threadIdx.x;
    const int h = (int)(blockIdx.x % (unsigned)H), j = sq.max_chunks - 1 - (int)(blockIdx.x / (unsigned)H);
    const int lane = t & 63, wv = wave_id(), m16 = lane & 15, g4 = lane >> 4;
    if (blockIdx.x == 0)
        for (int x = t; x < nprog; x += NT) prog[x] = 0;
    if (j >= min(sq.m.template nchunks<CS>(), sq.max_chunks)) return;
    const int i = sq.m.template seq_of<CS>(j);
    const int t0 = sq.t0(i) + CS * (j - sq.m.template chunk0<CS>(i));
    const int n = min(CS, sq.t1(i) - t0);
    uint8_t *blk = ops + ((size_t)h * sq.max_chunks + j) * L::bytes;

    // ---- stage 1: all loads, cumulative log-decay g, references ----
    const int cp = t % CP, rg = t / CP, c0 = 2 * cp, r0 = rg * RPG;
    f2 gg[RPG];
    raw2 kr[RPG], qr[RPG], br[RPG];
    auto rowf = [&](int u) { return r0 + u < n ? 1.f : 0.f; };
    {
        f2 lv[RPG];
#pragma unroll
        for (int u = 0; u < RPG; ++u) {
            const int r = r0 + u;
            const size_t off = ((size_t)(t0 + min(r, n - 1)) * H + h) * DK + c0;
            const f2 x = *reinterpret_cast<const f2 *>(la + off);
            br[u] = Ld<In>::ldraw2(b + off);
            kr[u] = Ld<In>::ldraw2(k + off);
            qr[u] = Ld<In>::ldraw2(q + off);
            const f2 z = {0.f, 0.f};
            lv[u] = r < n ? x : z;
        }
        f2 run = {0.f, 0.f};
#pragma unroll
        for (int u = 0; u < RPG; ++u) { run += lv[u]; gg[u] = run; }
        *reinterpret_cast<f2 *>(sPart + rg * DK + c0) = run;
    }
    if (t <= NRB) sFlag[t] = 0;
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
    for (int c = t; c < DK; c += NT)
        if (0.5f * (sG0[c] - sRef[NRB * DK + c]) > LIMC) atomicOr(&sFlag[NRB], 1);
    __syncthreads();
    const bool fast = sFlag[NRB] == 0;
    auto kval = [&](int u) { return Ld<In>::cvt2(kr[u]) * rowf(u); };
    // fragment element i times tab[kbase + kofs(g4, i)] (tab null: zero)
    auto scale_frag = [](frag x, const float *tab, int kbase, int g) {
        frag y;
#pragma unroll
        for (int pq = 0; pq < NE / 4; ++pq) {
            f4 f = f4zero();
            if (tab) f = *reinterpret_cast<const f4 *>(tab + kbase + 16 * pq + 4 * g);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) y[4 * pq + ii] = (Op)((float)x[4 * pq + ii] * f[ii]);
        }
        return y;
    };
    auto qval = [&](int u) { return Ld<In>::cvt2(qr[u]) * rowf(u); };
    auto bval = [&](int u) { return Ld<In>::cvt2(br[u]); };

    // ---- stage 2: decay factors, gamma, scaled operands in LDS ----
    for (int c = t; c < DK; c += NT) reinterpret_cast<float *>(blk + L::oG)[c] = __expf(sRef[NRB * DK + c]);
    if (fast) {
        for (int c = t; c < DK; c += NT) {
            const float gn = sRef[NRB * DK + c], mid = 0.5f * (sG0[c] + gn);
            tExpRef[c] = __expf(mid);
            tExpKh[c] = __expf(gn - mid);
        }
        const f2 mid = 0.5f * (*reinterpret_cast<const f2 *>(sG0 + c0) + *reinterpret_cast<const f2 *>(sRef + NRB * DK + c0));
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
        for (int idx = t; idx < NRB * DK; idx += NT) {
            const int R = idx / DK, c = idx % DK;
            const float rR = sRef[R * DK + c], rR1 = sRef[(R + 1) * DK + c];
            const float mid = sMid[R * DK + c], gn = sRef[NRB * DK + c];
            tExpRef[R * DK + c] = __expf(rR);
            tExpKh[R * DK + c] = __expf(gn - rR1);
            tDiagE[R * DK + c] = __expf(rR - mid);
            tDiagK[R * DK + c] = __expf(mid - rR1);
            if (fmaxf(rR - mid, mid - rR1) > LIM) atomicOr(&sFlag[R], 1);
        }
        for (int idx = t; idx < PL::NDEC * DK; idx += NT) {
            const int pr = idx / DK, c = idx % DK;
            int R = 2;
            while ((R - 1) * R / 2 <= pr) ++R;   // pair row pr: R with (R-2)(R-1)/2 <= pr < (R-1)R/2
            const int S = pr - (R - 2) * (R - 1) / 2;
            tDec[pr * DK + c] = __expf(sRef[R * DK + c] - sRef[(S + 1) * DK + c]);
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
    const int tabR = fast ? 0 : 1;   // table row step per block
    bool any_slow = false;
#pragma unroll
    for (int R = 0; R < NRB; ++R) any_slow |= !fast && sFlag[R];

    // ---- stage 3: A and P blocks on the matrix cores; P and Q+, Khat^T packed ----
    // Job jb of NTB A blocks then NTB P blocks, wave wv taking jb = wv, wv + NW, ...;
    // lower block number x = R (R + 1) / 2 + S
    auto block_rs = [](int x, int &R, int &S) {
        int r = 0;
#pragma unroll
        for (int y = 1; y < NRB; ++y) r += x >= y * (y + 1) / 2 ? 1 : 0;
        R = r;
        S = x - r * (r + 1) / 2;
    };
    constexpr int NJ = (2 * NTB + NW - 1) / NW;
    f4 aacc[NJ];   // the wave's A blocks, transposed, until A has its LDS space
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq) {
        const int jb = wv + NW * qq;
        aacc[qq] = f4zero();
        if (2 * NTB % NW != 0 && jb >= 2 * NTB) continue;
        const int kind = jb >= NTB ? 1 : 0;   // 0: A (E side), 1: P (Q side)
        int R, S;
        block_rs(jb - kind * NTB, R, S);
        const bool exact = !fast && R == S && sFlag[R];
        const Op *src = kind ? sQ : sE;
        // The operands are formed under the (workgroup-uniform) path
        // conditions, the products are not: a matrix instruction under a
        // runtime condition can be issued with no branch around it and then
        // runs whatever the execution mask, on registers the skipped path
        // never loaded. Exact blocks get zero operands here.
        f4 acc = f4zero();
        // (not unrolled: nine jobs of unrolled slow-path operand code overflow the instruction cache)
#pragma unroll 1
        for (int kb = 0; kb < NKB; ++kb) {
            frag a = lds_row_frag<Op>(sK + (16 * S + m16) * LDE, kb * KB, g4);
            frag bb = lds_row_frag<Op>(src + (16 * R + m16) * LDE, kb * KB, g4);
            if (!fast) {
                // block factors (row-fragment reads, 4 channels per table read)
                if (exact) {
                    a = scale_frag(a, nullptr, 0, g4);
                    bb = scale_frag(bb, nullptr, 0, g4);
                } else if (R == S) {
                    bb = scale_frag(bb, tDiagE + R * DK, kb * KB, g4);
                    a = scale_frag(a, tDiagK + R * DK, kb * KB, g4);
                } else if (R > S + 1) {
                    a = scale_frag(a, tDec + ((R - 2) * (R - 1) / 2 + S) * DK, kb * KB, g4);
                }
            }
            acc = M::mma(a, bb, acc);
        }
        // lane m16 + 16 g4 holds row m16, columns 4 g4 .. 4 g4 + 3 of block (R, S):
        // A keeps column < row on the diagonal, P column <= row
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int col = 4 * g4 + ii;
            if (R == S && (kind ? col > m16 : col >= m16)) acc[ii] = 0.f;
        }
        if (kind == 0) {
            aacc[qq] = acc;
        } else {
            // half S % HPB of P fragment (R, S / HPB); the half above a diagonal block is zero
            uint8_t *dst = blk + L::oP + ((size_t)L::tpos(R, S / HPB) * 64 + lane) * 16 + (S % HPB) * 4 * sizeof(Op);
            op4 y;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) y[ii] = (Op)acc[ii];
            if (!exact) *reinterpret_cast<op4 *>(dst) = y;
            if (HPB == 2 && R == S && (R & 1) == 0) {
                op4 z;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) z[ii] = (Op)0.f;
                *reinterpret_cast<op4 *>(dst + 4 * sizeof(Op)) = z;
            }
        }
    }
    // Q+ fragments: rows 16 mt + m, channels kb*KB + kofs, scaled to e^{g_r}
    for (int f = wv; f < NRB * NKB; f += NW) {
        const int mt = f / NKB, kb = f % NKB;
        const frag x = lds_row_frag<Op>(sQ + (16 * mt + m16) * LDE, kb * KB, g4);
        const float *sc = tExpRef + mt * tabR * DK + kb * KB;
        frag a;
#pragma unroll
        for (int i4 = 0; i4 < NE; ++i4) a[i4] = (Op)((float)x[i4] * sc[kofs(g4, i4)]);
        *reinterpret_cast<frag *>(blk + L::oQ + ((size_t)f * 64 + lane) * 16) = a;
    }
    // Khat^T fragments: rows = channel 16 ct + m, contraction = chunk rows
    for (int f = wv; f < NCT * NSB; f += NW) {
        const int ct = f / NSB, sb = f % NSB;
        const int c = 16 * ct + m16;
        frag a;
#pragma unroll
        for (int i4 = 0; i4 < NE; ++i4) {
            const int s = sb * KB + kofs(g4, i4);
            a[i4] = (Op)((float)sK[s * LDE + c] * tExpKh[(s >> 4) * tabR * DK + c]);
        }
        *reinterpret_cast<frag *>(blk + L::oK + ((size_t)f * 64 + lane) * 16) = a;
    }
    __syncthreads();   // every read of the Q- and K-side operands done: A takes their space

    // ---- stage 4: A into LDS, exact diagonal blocks if needed ----
#pragma unroll
    for (int qq = 0; qq < NJ; ++qq) {
        const int jb = wv + NW * qq;
        if (jb >= NTB) continue;
        int R, S;
        block_rs(jb, R, S);
        if (!fast && R == S && sFlag[R]) continue;   // exact path below
        *reinterpret_cast<f4 *>(sA + PL::bidx(R, S) * BSZ + m16 * BLD + 4 * g4) = aacc[qq];
    }
    if (any_slow) {
        // exact pairwise exponents for flagged diagonal blocks (strong decay)
        for (int R = 0; R < NRB; ++R) {
            if (!sFlag[R]) continue;
            for (int e = t; e < 256; e += NT) {
                const int rl = e >> 4, sl = e & 15;
                const int r = 16 * R + rl, s = 16 * R + sl;
                float aA = 0.f, aP = 0.f;
                if (sl <= rl && r < n) {
                    const size_t br_ = ((size_t)(t0 + r) * H + h) * DK, bs = ((size_t)(t0 + s) * H + h) * DK;
                    for (int c = 0; c < DK; ++c) {
                        float d = 0.f;
                        for (int x = s + 1; x <= r; ++x) d += la[((size_t)(t0 + x) * H + h) * DK + c];
                        const float ex = __expf(d) * Ld<In>::one(k + bs + c);
                        aA += Ld<In>::one(b + br_ + c) * Ld<In>::one(k + br_ + c) * ex;
                        aP += Ld<In>::one(q + br_ + c) * ex;
                    }
                }
                sA[PL::bidx(R, R) * BSZ + rl * BLD + sl] = sl < rl ? aA : 0.f;
                // element (rl, 16 (R % HPB) + sl) of P fragment (R, R / HPB)
                const int ln = rl + 16 * (sl >> 2), el = 4 * (R % HPB) + (sl & 3);
                *reinterpret_cast<Op *>(blk + L::oP + ((size_t)L::tpos(R, R / HPB) * 64 + ln) * 16 + el * sizeof(Op)) =
                    (Op)aP;
            }
        }
    }
    __syncthreads();

    // ---- stage 5: T = (I + A)^{-1}, block forward substitution ----
    if (wv < NRB) {   // (whole waves: the solve uses all 64 lanes)
        float x[4];
        unit_lower_inverse16(sA + PL::bidx(wv, wv) * BSZ, BLD, lane, x);
        Op *Tb = sT + PL::bidx(wv, wv) * BSZ;
#pragma unroll
        for (int j = 0; j < 4; ++j) Tb[(g4 + 4 * j) * BLD + m16] = (Op)x[j];
    }
    __syncthreads();
    // T_RS = -T_RR sum_{J=S}^{R-1} A_RJ T_JS, by distance R - S
    for (int d = 1; d < NRB; ++d) {
        if (wv < NRB - d) {
            const int S = wv, R = S + d;
            f4 y = f4zero();
            for (int J = S; J < R; ++J) {
                const f4 a = *reinterpret_cast<const f4 *>(sA + PL::bidx(R, J) * BSZ + m16 * BLD + 4 * g4);
                f4 bb;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) bb[ii] = (float)sT[PL::bidx(J, S) * BSZ + (4 * g4 + ii) * BLD + m16];
                y = M::mma16(a, bb, y);
            }
            f4 a;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) a[ii] = (float)sT[PL::bidx(R, R) * BSZ + m16 * BLD + 4 * g4 + ii];
            const f4 z = M::mma16(a, y, f4zero());
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sT[PL::bidx(R, S) * BSZ + (4 * g4 + ii) * BLD + m16] = (Op)(-z[ii]);
        }
        __syncthreads();
    }

    // ---- stage 6: T fragments; W = T E formed transposed, into -W fragments ----
    // T fragment (mt, sb): halves S = HPB sb + hf, zero above the diagonal
    auto tfrag = [&](int mt, int sb) {
        frag f;
#pragma unroll
        for (int hf = 0; hf < HPB; ++hf) {
            const int S = HPB * sb + hf;
            op4 x;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) x[ii] = (Op)0.f;
            if (S <= mt) x = *reinterpret_cast<const op4 *>(sT + PL::bidx(mt, S) * BSZ + m16 * BLD + 4 * g4);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) f[4 * hf + ii] = x[ii];
        }
        return f;
    };
    for (int f = wv; f < NRB * NSB; f += NW) {
        const int mt = f / NSB, sb = f % NSB;
        if (sb > L::sbmax(mt)) continue;
        *reinterpret_cast<frag *>(blk + L::oT + ((size_t)L::tpos(mt, sb) * 64 + lane) * 16) = tfrag(mt, sb);
    }
    // wave wv: row tiles of group wv % RG, column tiles wv / RG, + NCG, ...
    constexpr int RG = NRB >= 8 ? 2 : 1, RTW = NRB / RG, NCG = NW / RG;
    const int rgrp = wv % RG, cgrp = wv / RG;
    // every k-block, zero above the diagonal (no product under a runtime condition)
    frag tf[RTW][NSB];
#pragma unroll
    for (int x = 0; x < RTW; ++x)
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) tf[x][sb] = tfrag(rgrp * RTW + x, sb);
    for (int nt = cgrp; nt < NCT; nt += NCG) {
        const int c = 16 * nt + m16;
        frag eb[NSB];   // E column fragments: lane c + 16 g holds E[sb KB + kofs(g, i)][c] x e^{ref}
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
            for (int i4 = 0; i4 < NE; ++i4) {
                const int s = sb * KB + kofs(g4, i4);
                eb[sb][i4] = (Op)((float)sE[s * LDE + c] * tExpRef[(s >> 4) * tabR * DK + c]);
            }
#pragma unroll
        for (int x = 0; x < RTW; ++x) {
            const int mt = rgrp * RTW + x;
            f4 acc = f4zero();
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) acc = M::mma(eb[sb], tf[x][sb], acc);
            // lane m16 + 16 g4: W row 16 mt + m16, channels 16 nt + 4 g4 .. + 3
            op4 y;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) y[ii] = (Op)(-acc[ii]);
            *reinterpret_cast<op4 *>(blk + L::oW + ((size_t)(mt * NKB + nt / HPB) * 64 + lane) * 16 +
                                     (nt % HPB) * 4 * sizeof(Op)) = y;
        }
    }
}

template <typename In, typename Op, int DK, int DV, int CS>
static hipError_t launch_cs(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st)
{
    using PL = PrepCS<Op, DK, CS>;
    uint8_t *ws = (uint8_t *)a.workspace;
    const Seqs sq = make_seqs(a, p);
    hipError_t err = hipSuccess;
    int *prog = (int *)(ws + p.plan_bytes);
    uint8_t *ops = ws + p.plan_bytes + p.prog_bytes;
    const long long chains = (long long)a.N * a.H;
    if (p.max_chunks > 0) {
        prof_before("gdn2_chunk_prep", st);
        hipLaunchKernelGGL((chunk_prep_cs_kernel<In, Op, DK, CS>), dim3((unsigned)((long long)p.max_chunks * a.H)),
                           dim3(PL::NT), 0, st, (const In *)a.q, (const In *)a.k, a.log_alpha, (const In *)a.b, sq,
                           a.H, ops, prog, (int)chains);
        prof_after(st);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    PassShape ps;
    if ((err = pass_shape<DV>(chains, p, &ps)) != hipSuccess) return err;
    prof_before("gdn2_chunk_pass", st);
    const ConvIn cv = {nullptr, nullptr, nullptr};
    const SaveOut so = {nullptr, nullptr, false};
    auto pass = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)ps.grid), dim3(512), 0, st, (const In *)a.v, (const In *)a.w, a.S0,
                           (float *)a.o, a.ST, sq, a.H, (const uint8_t *)ops, prog, ps.npf, cv, so);
    };
    if constexpr ((DV / 16) % 2 == 0) {
        if (ps.two) pass(chunk_pass_kernel<In, Op, DK, DV, 2, false, false, false, CS>);
        else pass(chunk_pass_kernel<In, Op, DK, DV, 1, false, false, false, CS>);
    } else pass(chunk_pass_kernel<In, Op, DK, DV, 1, false, false, false, CS>);
    prof_after(st);
    return hipGetLastError();
}

// Forward over CS-token chunks (CS = 32 or 128); per-channel gates, no
// prologue. Unsupported combinations (the prep's LDS plan above 160 KB)
// return hipErrorInvalidValue; chunk_plan rejects them first.
template <typename In, typename Op, int DK, int CS>
hipError_t dispatch_dv_cs(const ChunkArgs &a, const ChunkPlan &p, hipStream_t st)
{
    if constexpr (!PrepCS<Op, DK, CS>::fits) {
        return hipErrorInvalidValue;
    } else {
        switch (a.dv) {
        case 16: return launch_cs<In, Op, DK, 16, CS>(a, p, st);
        case 32: return launch_cs<In, Op, DK, 32, CS>(a, p, st);
        case 64: return launch_cs<In, Op, DK, 64, CS>(a, p, st);
        case 128: return launch_cs<In, Op, DK, 128, CS>(a, p, st);
        }
        return hipErrorInvalidValue;
    }
}

} // namespace gdn2
