// Chunkwise backward of the Gated Delta Rule-2 prefill on gfx950.
//
// A loss with gradients dO (outputs) and dS_T (final states) propagates
// backwards through each chunk's affine map of the state. With the forward
// chunk quantities (chunk_impl.hpp: W = T E, Q+, Khat, P, T, gamma = e^{g_n}):
//   S_n = M S_c + Khat^T T U,  M = Diag(gamma) - Khat^T W
//   O   = R S_c + P T U,       R = Q+ - P W
// so the gradient at a chunk's start state, from the gradient G at its end
// state, is
//   G_c = M^T G + R^T dO = gamma * G + N^T G + R^T dO,  N^T = -W^T Khat,
//   R^T = Q+^T - W^T P^T
// (the chunk form is the plainest reading of the pages' chunkwise WY form;
// snilld.dk, section "Hvad betyder det for træning og inferens").
//
// Kernels (all per head, chunk blocks head-major like the forward's):
//  * chunk_bprep: per (chunk, head), N^T and R^T from the forward operand
//    block, as MFMA A-fragments (gamma stays fp32, applied separately).
//  * chunk_rpass: per (sequence, head, column slice), the chain G_c in
//    registers from the last chunk to the first; stores each chunk's end
//    gradient G, returns dS0.
#pragma once

#include "chunk_impl.hpp"

namespace gdn2 {

// Backward operand block for one (chunk, head).
template <typename Op, int DK> struct BBlk {
    using M = Mma<Op>;
    static constexpr int KB = M::KB;
    static constexpr int NKB = DK / KB;   // k-blocks over key channels
    static constexpr int NSB = 64 / KB;   // k-blocks over chunk rows
    static constexpr int NCT = DK / 16;   // 16-row tiles over key channels
    static constexpr size_t FRAG = 64 * 16;
    static constexpr size_t oN = 0;                          // N^T [NCT][NKB]
    static constexpr size_t oR = oN + NCT * NKB * FRAG;      // R^T [NCT][NSB]
    static constexpr size_t oPT = oR + NCT * NSB * FRAG;     // P^T [4][NSB] (rows = chunk rows)
    static constexpr size_t oTT = oPT + 4 * NSB * FRAG;      // T^T [4][NSB]
    static constexpr size_t oKH = oTT + 4 * NSB * FRAG;      // Khat [4][NKB]
    static constexpr size_t oG = oKH + 4 * NKB * FRAG;       // gamma float[DK]
    static constexpr size_t bytes = (oG + DK * 4 + 255) / 256 * 256;
};

// ---------------------------------------------------------------------------
// N^T = (-W)^T Khat and R^T = Q+^T + (-W)^T P^T from one forward block.
// The forward fragments serve directly as B operands: a Khat^T A-fragment
// (rows = channels, contraction = chunk rows) is the B-fragment of Khat, and
// a P A-fragment the B-fragment of P^T. (-W)^T and Q+ go through LDS.
template <typename Op, int DK>
__global__ __launch_bounds__(256) void chunk_bprep_kernel(const uint8_t *__restrict__ ops, uint8_t *__restrict__ bops,
                                                          Seqs sq, int H, int *__restrict__ prog, int nprog)
{
    using M = Mma<Op>;
    using L = Blk<Op, DK>;
    using BL = BBlk<Op, DK>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NE = M::NE, NKB = L::NKB, NSB = L::NSB, NCT = L::NCT;
    constexpr int LDW = 64 + 8;          // (-W)^T rows (chunk rows along a row)
    constexpr int LDQ = DK + 8;          // Q+ rows
    constexpr int LDX = (DK > 64 ? DK : 64) + 8;   // output staging rows (N^T: DK wide; R^T: 64 wide)
    // two phases over one area: (-W)^T, Q+ and the output staging, then
    // P^T, T^T and Khat
    constexpr int LDP = 64 + 8, LDK = DK + 8;
    constexpr size_t PH1 = (size_t)DK * LDW + 64 * LDQ + (size_t)DK * LDX, PH2 = 2 * 64 * LDP + 64 * LDK;
    __shared__ __attribute__((aligned(16))) Op sArea[PH1 > PH2 ? PH1 : PH2];
    Op *sWt = sArea, *sQp = sArea + DK * LDW, *sX = sArea + DK * LDW + 64 * LDQ;

    const int t = threadIdx.x, lane = t & 63, wv = wave_id(), m16 = lane & 15, g4 = lane >> 4;
    const int h = (int)(blockIdx.x % (unsigned)H), j = (int)(blockIdx.x / (unsigned)H);
    if (blockIdx.x == 0)   // progress counters of the reverse pass's prefetch workgroups
        for (int x = t; x < nprog; x += 256) prog[x] = 0;
    if (j >= min(sq.m.nchunks(), sq.max_chunks)) return;
    const uint8_t *blk = ops + ((size_t)h * sq.max_chunks + j) * L::bytes;
    uint8_t *bb = bops + ((size_t)h * sq.max_chunks + j) * BL::bytes;

    // unpack -W transposed and Q+ as is
    constexpr int NU = (4 * NKB * 64) / 256;   // fragment lanes per thread (all loads first)
    frag wf[NU], qfs[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int x = t + 256 * u;
        wf[u] = *reinterpret_cast<const frag *>(blk + L::oW + (size_t)x * 16);
        qfs[u] = *reinterpret_cast<const frag *>(blk + L::oQ + (size_t)x * 16);
    }
    // (the P, T and Khat^T fragments for the transposed copies, loaded with the rest)
    constexpr int NPU = (L::NTRI * 64 + 255) / 256, NKU = NCT * NSB * 64 / 256;
    frag pfs[NPU], tfs[NPU], kfs[NKU];
#pragma unroll
    for (int u = 0; u < NPU; ++u) {
        const int x = min(t + 256 * u, L::NTRI * 64 - 1);
        pfs[u] = *reinterpret_cast<const frag *>(blk + L::oP + (size_t)x * 16);
        tfs[u] = *reinterpret_cast<const frag *>(blk + L::oT + (size_t)x * 16);
    }
#pragma unroll
    for (int u = 0; u < NKU; ++u) kfs[u] = *reinterpret_cast<const frag *>(blk + L::oK + (size_t)(t + 256 * u) * 16);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int x = t + 256 * u;
        const int f = x >> 6, ln = x & 63, mt = f / NKB, kb = f % NKB, m = ln & 15, g = ln >> 4;
        const frag w = wf[u], qf = qfs[u];
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            const int c = kb * KB + kofs(g, i), r = 16 * mt + m;
            sWt[c * LDW + r] = w[i];
            sQp[r * LDQ + c] = qf[i];
        }
    }
    if (t < DK) reinterpret_cast<float *>(bb + BL::oG)[t] = reinterpret_cast<const float *>(blk + L::oG)[t];
    __syncthreads();

    // N^T tiles (at, bt): contraction over the chunk rows (a fixed trip
    // count, so that the fragment loads of all the wave's tiles issue together)
#pragma unroll
    for (int kt = 0; kt < (NCT * NCT + 3) / 4; ++kt) {
        const int tile = wv + 4 * kt;
        if ((NCT * NCT) % 4 != 0 && tile >= NCT * NCT) break;   // (wave-uniform)
        const int at = tile / NCT, bt = tile % NCT;
        f4 acc = f4zero();
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            const frag a = lds_row_frag<Op>(sWt + (16 * at + m16) * LDW, sb * KB, g4);
            const frag b = *reinterpret_cast<const frag *>(blk + L::oK + ((size_t)(bt * NSB + sb) * 64 + lane) * 16);
            acc = M::mma(a, b, acc);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sX[(16 * at + 4 * g4 + ii) * LDX + 16 * bt + m16] = (Op)acc[ii];
    }
    __syncthreads();
    for (int f = wv; f < NCT * NKB; f += 4) {
        const int at = f / NKB, kb = f % NKB;
        *reinterpret_cast<frag *>(bb + BL::oN + ((size_t)f * 64 + lane) * 16) =
            lds_row_frag<Op>(sX + (16 * at + m16) * LDX, kb * KB, g4);
    }
    __syncthreads();

    // R^T tiles (at, rt): Q+^T plus (-W)^T P^T (P lower triangular)
#pragma unroll
    for (int at = 0; at < NCT; ++at) {
        const int rt = wv;
        f4 acc = f4zero();
#pragma unroll
        for (int sb = 0; sb < NSB; ++sb) {
            if (sb > L::sbmax(rt)) break;
            const frag a = lds_row_frag<Op>(sWt + (16 * at + m16) * LDW, sb * KB, g4);
            const frag b = *reinterpret_cast<const frag *>(blk + L::oP + ((size_t)L::tpos(rt, sb) * 64 + lane) * 16);
            acc = M::mma(a, b, acc);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int a_ = 16 * at + 4 * g4 + ii, r = 16 * rt + m16;
            sX[a_ * LDX + r] = (Op)(acc[ii] + (float)sQp[r * LDQ + a_]);
        }
    }
    __syncthreads();
    for (int f = wv; f < NCT * NSB; f += 4) {
        const int at = f / NSB, sb = f % NSB;
        *reinterpret_cast<frag *>(bb + BL::oR + ((size_t)f * 64 + lane) * 16) =
            lds_row_frag<Op>(sX + (16 * at + m16) * LDX, sb * KB, g4);
    }
    __syncthreads();

    // P^T, T^T and Khat as A-fragments (rows = chunk rows) for the gradient
    // kernel: unpack P and T transposed (over (-W)^T) and Khat^T transposed
    // (over the staging area), then pack
    Op *PT = sArea, *TT = sArea + 64 * LDP, *Kh = sArea + 2 * 64 * LDP;
    for (int x = t; x < 64 * LDP; x += 256) { PT[x] = (Op)0.f; TT[x] = (Op)0.f; }
    __syncthreads();
    {
#pragma unroll
        for (int u = 0; u < NPU; ++u) {
            const int x = t + 256 * u;
            if (x >= L::NTRI * 64) break;
            const int f = x >> 6, ln = x & 63, m = ln & 15, g = ln >> 4;
            int mt = 0;
            while (mt < 3 && L::tpos(mt + 1, 0) <= f) ++mt;
            const int sb = f - L::tpos(mt, 0);
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                const int cc = sb * KB + kofs(g, e), r = 16 * mt + m;
                PT[cc * LDP + r] = pfs[u][e];
                TT[cc * LDP + r] = tfs[u][e];
            }
        }
#pragma unroll
        for (int u = 0; u < NKU; ++u) {
            const int x = t + 256 * u;
            const int f = x >> 6, ln = x & 63, m = ln & 15, g = ln >> 4, ct = f / NSB, sb = f % NSB;
#pragma unroll
            for (int e = 0; e < NE; ++e) Kh[(sb * KB + kofs(g, e)) * LDK + 16 * ct + m] = kfs[u][e];
        }
    }
    __syncthreads();
    for (int f = wv; f < 4 * NSB; f += 4) {
        const int rt = f / NSB, sb = f % NSB;
        *reinterpret_cast<frag *>(bb + BL::oPT + ((size_t)f * 64 + lane) * 16) =
            lds_row_frag<Op>(PT + (16 * rt + m16) * LDP, sb * KB, g4);
        *reinterpret_cast<frag *>(bb + BL::oTT + ((size_t)f * 64 + lane) * 16) =
            lds_row_frag<Op>(TT + (16 * rt + m16) * LDP, sb * KB, g4);
    }
    for (int f = wv; f < 4 * NKB; f += 4) {
        const int rt = f / NKB, kb = f % NKB;
        *reinterpret_cast<frag *>(bb + BL::oKH + ((size_t)f * 64 + lane) * 16) =
            lds_row_frag<Op>(Kh + (16 * rt + m16) * LDK, kb * KB, g4);
    }
}

// ---------------------------------------------------------------------------
// L2 prefetch workgroups of the reverse pass, as for the forward pass (see
// pass_prefetch): wave k of a prefetch workgroup takes steps k, k + 8, ...
// (step s handles chunk nch - 1 - s), waits while it is more than
// 3 + kPfWindow steps ahead of the chain's progress counter, skips steps
// closer than 3, and reads one dword per line of its share of the step's
// N^T, R^T and gamma and of the chunk's dO rows into an LDS sink. Every loop
// and wait is bounded; the pass never waits for these workgroups.
template <typename Op, int DK, int DV>
__device__ __forceinline__ void rpass_prefetch(const uint8_t *bops0, const float *dO, const int *prog, int chain,
                                               int h, int H, int pf, int npf, int nch, int tb, int te)
{
    using BL = BBlk<Op, DK>;
    constexpr int NNR = (int)(BL::oPT / 128);         // lines of N^T and R^T
    constexpr int NGL = (DK * 4 + 127) / 128;         // lines of gamma
    constexpr int RL = (DV * 4 + 127) / 128;          // lines per dO row (or the one holding it)
    constexpr int PL = NNR + NGL + 64 * RL;
    constexpr int NW = 8;
    __shared__ uint32_t sSink[NW * 64];
    const int t = threadIdx.x, wv = wave_id(), lane = t & 63;
    lptr_t scratch = (lptr_t)(sSink + wv * 64);
    auto done = [&]() {
        return __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(prog + chain, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    };
    for (int k = wv; k < nch; k += NW) {
        int d = done();
        for (int s = 0; k > d + 3 + kPfWindow && s < kPfMaxSleeps; ++s) {
            __builtin_amdgcn_s_sleep(4);
            d = done();
        }
        while (k < d + 3) k += NW;
        if (k >= nch) break;
        const int c = nch - 1 - k;
        const uint8_t *blk = bops0 + (size_t)c * BL::bytes;
        for (int l = pf + npf * lane; l < PL; l += npf * 64) {
            const uint8_t *a;
            if (l < NNR) {
                a = blk + (size_t)l * 128;
            } else if (l < NNR + NGL) {
                a = blk + BL::oG + (size_t)(l - NNR) * 128;
            } else {
                const int x = l - NNR - NGL, row = x / RL, part = x % RL;
                const int tok = min(tb + 64 * c + row, te - 1);
                a = reinterpret_cast<const uint8_t *>(dO + ((size_t)tok * H + h) * DV) + part * 128;
            }
            __builtin_amdgcn_global_load_lds((gptr_t)a, scratch, 4, 0, 0);
        }
    }
    __syncthreads();   // drains the line reads before the workgroup ends
}

// ---------------------------------------------------------------------------
// Reverse state pass. Workgroup = (chain, slice of 16*NC value columns), 8
// waves: state waves 0..3 hold the gradient G of their key rows (fp32 in
// registers), loader waves 4..7 stage dO of the next chunk (hi + lo f16, the
// B operand) in LDS. One barrier per chunk: G and dO live in two LDS buffers
// by chunk parity. Each step stores the incoming G (the gradient at the
// chunk's end state) for the gradient kernel.
template <typename Op, int DK, int DV, int NC>
__global__ __launch_bounds__(512) void chunk_rpass_kernel(const float *__restrict__ dO, const float *__restrict__ dST,
                                                          float *__restrict__ dS0, Seqs sq, int H,
                                                          const uint8_t *__restrict__ bops, Op *__restrict__ gbuf,
                                                          int *__restrict__ prog, int npf)
{
    using M = Mma<Op>;
    using BL = BBlk<Op, DK>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NE = M::NE, NKB = BL::NKB, NSB = BL::NSB, NCT = BL::NCT;
    constexpr int TPW = (NCT + 3) / 4;
    constexpr int TPK = KB / 16;
    constexpr int NSL = DV / (16 * NC);
    __shared__ __attribute__((aligned(16))) Op sG[2][NC][NCT * 64 * 4];
    __shared__ __attribute__((aligned(16))) Op sD[2][NC][2 * NSB * 64 * NE];

    // XCD-aware numbering: the slices and prefetch workgroups of chain c sit
    // on XCD c % 8
    const int Lid = blockIdx.x;
    const int kq = Lid >> 3, role = kq % (NSL + npf), js = role;
    const int chain = (kq / (NSL + npf)) * 8 + (Lid & 7);
    if (chain >= sq.m.N * H) return;
    const int i = chain / H, h = chain % H;
    const int t = threadIdx.x, lane = t & 63, wv = wave_id(), m16 = lane & 15, g4 = lane >> 4;
    const int col0 = 16 * NC * js;
    const size_t sbase = ((size_t)i * H + h) * DK * DV;
    const int tb = sq.t0(i), te = sq.t1(i);
    const int cbeg = sq.m.chunk0(i);
    const int nch = min((te - tb + 63) >> 6, max(0, sq.max_chunks - cbeg));
    const size_t slot0 = (size_t)h * sq.max_chunks + cbeg;
    // step k handles chunk nch - 1 - k
    auto bblk = [&](int k) { return bops + (slot0 + max(nch - 1 - k, 0)) * BL::bytes; };
    if (role >= NSL) {
        rpass_prefetch<Op, DK, DV>(bops + slot0 * BL::bytes, dO, prog, chain, h, H, role - NSL, npf, nch, tb, te);
        return;
    }
    const bool report = npf > 0 && js == 0 && t == 0;   // progress for the prefetch workgroups

    if (wv < 4) {
        __builtin_amdgcn_s_setprio(3);
        struct F {
            frag Nt[TPW][NKB], Rt[TPW][NSB];
            f4 gam[TPW];
        };
        auto fload = [&](F &f, const uint8_t *b) {
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int ct = wv * TPW + u;
                if (NCT % 4 != 0 && ct >= NCT) continue;
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    f.Nt[u][kb] = *reinterpret_cast<const frag *>(b + BL::oN + ((size_t)(ct * NKB + kb) * 64 + lane) * 16);
#pragma unroll
                for (int sb = 0; sb < NSB; ++sb)
                    f.Rt[u][sb] = *reinterpret_cast<const frag *>(b + BL::oR + ((size_t)(ct * NSB + sb) * 64 + lane) * 16);
                f.gam[u] = *reinterpret_cast<const f4 *>(b + BL::oG + (size_t)(16 * ct + 4 * g4) * 4);
            }
        };
        f4 Gr[NC][TPW];
#pragma unroll
        for (int q = 0; q < NC; ++q)
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int ct = wv * TPW + u;
                Gr[q][u] = f4zero();
                if (ct < NCT) {
                    if (dST) {
#pragma unroll
                        for (int ii = 0; ii < 4; ++ii)
                            Gr[q][u][ii] = dST[sbase + (size_t)(16 * ct + 4 * g4 + ii) * DV + col0 + 16 * q + m16];
                    }
                    lds_tile_store<Op>(sG[0][q] + ct * 256, lane, Gr[q][u]);
                }
            }
        // fp32 operands (four times the fragments) load at the step itself;
        // f16 ones two steps ahead into a ring of three
        constexpr bool RING = sizeof(Op) == 2;
        F f0, f1, f2;
        if (RING && nch > 0) {
            fload(f0, bblk(0));
            fload(f1, bblk(1));
        }
        auto step = [&](int k, F &cur, F &pre, int par) {
            const int c = nch - 1 - k;
            if constexpr (!RING) fload(cur, bblk(k));
            Op *gp = gbuf + (slot0 + c) * DK * DV;   // accumulator-tile order, as the forward's S_c
#pragma unroll
            for (int q = 0; q < NC; ++q)
#pragma unroll
                for (int u = 0; u < TPW; ++u) {
                    const int ct = wv * TPW + u;
                    if (NCT % 4 != 0 && ct >= NCT) continue;
                    tile_store<Op>(gp + ((size_t)ct * (DV / 16) + NC * js + q) * 256, lane, Gr[q][u]);
                }
            __syncthreads();   // G and dO of this step in LDS buffer `par`
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int ct = wv * TPW + u;
                if (NCT % 4 != 0 && ct >= NCT) continue;
#pragma unroll
                for (int q = 0; q < NC; ++q) {
                    f4 s = Gr[q][u] * cur.gam[u];
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb)
                        s = M::mma(cur.Nt[u][kb], lds_bfrag<Op>(sG[par][q] + kb * TPK * 256, lane), s);
#pragma unroll
                    for (int sb = 0; sb < NSB; ++sb) {
                        const frag dh = *reinterpret_cast<const frag *>(&sD[par][q][((0 * NSB + sb) * 64 + lane) * NE]);
                        const frag dl = *reinterpret_cast<const frag *>(&sD[par][q][((1 * NSB + sb) * 64 + lane) * NE]);
                        s = M::mma(cur.Rt[u][sb], dh, s);
                        s = M::mma(cur.Rt[u][sb], dl, s);
                    }
                    Gr[q][u] = s;
                    lds_tile_store<Op>(sG[par ^ 1][q] + ct * 256, lane, s);
                }
            }
            if constexpr (RING) fload(pre, bblk(k + 2));
            if (report) __hip_atomic_store(prog + chain, k + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        };
        int k = 0;
        if constexpr (RING) {
            for (; k + 6 <= nch; k += 6) {
                step(k, f0, f2, 0);
                step(k + 1, f1, f0, 1);
                step(k + 2, f2, f1, 0);
                step(k + 3, f0, f2, 1);
                step(k + 4, f1, f0, 0);
                step(k + 5, f2, f1, 1);
            }
            // tail: up to five more steps, ring slot k % 3 and parity k % 2
            if (k < nch) step(k, f0, f2, 0);
            if (k + 1 < nch) step(k + 1, f1, f0, 1);
            if (k + 2 < nch) step(k + 2, f2, f1, 0);
            if (k + 3 < nch) step(k + 3, f0, f2, 1);
            if (k + 4 < nch) step(k + 4, f1, f0, 0);
        } else {
            for (; k + 2 <= nch; k += 2) {
                step(k, f0, f0, 0);
                step(k + 1, f0, f0, 1);
            }
            if (k < nch) step(k, f0, f0, 0);
        }
        if (dS0) {
#pragma unroll
            for (int q = 0; q < NC; ++q)
#pragma unroll
                for (int u = 0; u < TPW; ++u) {
                    const int ct = wv * TPW + u;
                    if (ct >= NCT) continue;
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii)
                        dS0[sbase + (size_t)(16 * ct + 4 * g4 + ii) * DV + col0 + 16 * q + m16] = Gr[q][u][ii];
                }
        }
    } else {
        // loader waves: thread `to` holds row ur, columns uc..uc+3 of each tile
        const int to = t - 256, ur = to >> 2, uc = 4 * (to & 3);
        const int usb = ur / KB, usl = ur % KB;
        const int ug = (usl & 15) >> 2, ui = 4 * (usl >> 4) + (usl & 3);
        struct D4 { f4 x[NC]; bool ok; };
        auto dload = [&](D4 &d, int k) {
            const int c = max(nch - 1 - k, 0);
            const int tok = tb + 64 * c + ur;
            d.ok = k < nch && tok < te;
            const size_t off = ((size_t)min(tok, te - 1) * H + h) * DV + col0 + uc;
#pragma unroll
            for (int q = 0; q < NC; ++q) d.x[q] = *reinterpret_cast<const f4 *>(dO + off + 16 * q);
        };
        auto dstage = [&](const D4 &d, int par) {
#pragma unroll
            for (int q = 0; q < NC; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = d.ok ? d.x[q][e] : 0.f;
                    const Op hi = (Op)x;
                    const int ln = (uc + e) + 16 * ug;
                    sD[par][q][((0 * NSB + usb) * 64 + ln) * NE + ui] = hi;
                    sD[par][q][((1 * NSB + usb) * 64 + ln) * NE + ui] = (Op)(x - (float)hi);
                }
        };
        D4 d0, d1, d2;
        if (nch > 0) {
            dload(d0, 0);
            dload(d1, 1);
            dstage(d0, 0);
        }
        auto step = [&](int k, D4 &nxt, D4 &pre, int par) {
            __syncthreads();
            dstage(nxt, par ^ 1);    // dO of step k + 1
            dload(pre, k + 2);
        };
        int k = 0;
        for (; k + 6 <= nch; k += 6) {
            step(k, d1, d2, 0);
            step(k + 1, d2, d0, 1);
            step(k + 2, d0, d1, 0);
            step(k + 3, d1, d2, 1);
            step(k + 4, d2, d0, 0);
            step(k + 5, d0, d1, 1);
        }
        if (k < nch) step(k, d1, d2, 0);
        if (k + 1 < nch) step(k + 1, d2, d0, 1);
        if (k + 2 < nch) step(k + 2, d0, d1, 0);
        if (k + 3 < nch) step(k + 3, d1, d2, 1);
        if (k + 4 < nch) step(k + 4, d2, d0, 0);
    }
}

// Inclusive running sums down (REV: up) the 64 rows of NCOL columns of an
// LDS tile with row stride ld, by all NT threads of the workgroup: thread t
// takes column t % NCOL and one segment of rows; segment totals pass through
// `part` (NT floats). Contains two barriers.
template <int NCOL, bool REV, int NT>
__device__ __forceinline__ void col_scan64(float *buf, int ld, float *part, int t)
{
    constexpr int SEGS = NT / NCOL, SL = 64 / SEGS;
    static_assert(SEGS * NCOL == NT && SEGS * SL == 64, "NT threads over 64 rows");
    const int c = t % NCOL, sg = t / NCOL;
    const int r0 = REV ? 64 - SL * (sg + 1) : SL * sg;
    float x[SL], tot = 0.f;
#pragma unroll
    for (int i = 0; i < SL; ++i) { x[i] = buf[(r0 + i) * ld + c]; tot += x[i]; }
    part[sg * NCOL + c] = tot;
    __syncthreads();
    float a = 0.f;
    for (int s = 0; s < sg; ++s) a += part[s * NCOL + c];
    if constexpr (!REV) {
#pragma unroll
        for (int i = 0; i < SL; ++i) { a += x[i]; buf[(r0 + i) * ld + c] = a; }
    } else {
#pragma unroll
        for (int i = SL - 1; i >= 0; --i) { a += x[i]; buf[(r0 + i) * ld + c] = a; }
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// Per-chunk gradients, one workgroup per (chunk, head) of one or two halves
// of 4 waves (wave w & 3 owns the 16-row block; with two halves each takes
// every other work unit of a step, so that two waves share a SIMD), from the
// forward's chunk start state S_c and Delta, the reverse pass's end gradient
// G, the forward block's P and T, dO and the raw inputs. With g the chunk's
// cumulative log decay (g_n its last row) and, per channel,
// e^{g_r - g_s} written Dec_rs:
//   dDelta = P^T dO + Khat G,   dX = T^T dDelta,   dv = dX * w,  dw = dX * v
//   dA = -strict_tril(dX Delta^T),   dP = tril(dO Delta^T)
//   dq  = (dO S_c^T) * e^g + (dP o Dec) k
//   dE~ = -(dX S_c^T) * e^g + (dA o Dec) k          (dE scaled by e^g)
//   dk  = (dP o Dec)^T q + (dA o Dec)^T (b k) + (Delta G^T) * e^{g_n - g} + dE~ * b
//   db  = dE~ * k
//   dlog_alpha = reverse cumulative sum over the chunk of
//     dq q - (dk through k e^{-g}) k - (dk through Khat) k + dE~ b k,
//     plus, at the last row, sum_r (dk through Khat) k + e^{g_n} diag(G S_c^T)
// where (M o Dec) x means sum_s M_rs x_s e^{g_r - g_s}.
// Phase A (value columns in slices through LDS, matrix cores on the operand
// type) forms dDelta, dX, dv, dw and accumulates dA, dP, dO S_c^T, dX S_c^T,
// Delta G^T in registers. Phase B (key channels in slices, fp32 matrix
// cores) forms the four decayed products blockwise over 16-row blocks:
// off-diagonal blocks S < R through the references ref_{S+1} (every factor
// <= 1), diagonal blocks around the block's middle row while the decay
// across a half block stays within kBwdDiagSpread (factors within e^40 of
// 1), else with exact pairwise exponents e^{g_r - g_s} <= 1 (any decay),
// then the elementwise gradients and the reverse cumulative sum.
// Largest log-decay between a diagonal block's middle row and its ends for
// the factored form; beyond it the block takes the exact pairwise form.
constexpr float kBwdDiagSpread = 40.f;

template <typename Op, int DK, int DV> struct GradShape {
    static constexpr int VS = (sizeof(Op) == 2 ? 32 : 16) < DV ? (sizeof(Op) == 2 ? 32 : 16) : DV;   // value cols per slice
    static constexpr int VT = VS / 16, CT = DK / 16;
    static constexpr int CW = DK < 32 ? DK : 32;          // key channels per phase-B slice
    static constexpr int CWT = CW / 16;
    // two halves of four waves when every step splits evenly between them
    static constexpr int NT = (VT % 2 == 0 && CT % 2 == 0 && CWT % 2 == 0) ? 512 : 256;
};

template <typename In, typename Op, int DK, int DV, int NT>
__global__ __launch_bounds__(NT) void chunk_grad_kernel(
    const In *__restrict__ q, const In *__restrict__ k, const In *__restrict__ v, const float *__restrict__ la,
    const In *__restrict__ b, const In *__restrict__ w, const float *__restrict__ dO, Seqs sq, int H,
    const uint8_t *__restrict__ bops, const Op *__restrict__ sbuf, const Op *__restrict__ dbuf,
    const Op *__restrict__ gbuf, float *__restrict__ dq, float *__restrict__ dk_, float *__restrict__ dv_,
    float *__restrict__ dla, float *__restrict__ db, float *__restrict__ dw)
{
    using M = Mma<Op>;
    using MF = Mma<float>;
    using BL = BBlk<Op, DK>;
    using frag = typename M::frag;
    constexpr int KB = M::KB, NE = M::NE, NKB = BL::NKB, NSB = BL::NSB;
    using GS = GradShape<Op, DK, DV>;
    constexpr int VS = GS::VS, NVS = DV / VS, VT = GS::VT, VKB = VS / KB > 0 ? VS / KB : 1;
    constexpr int CT = GS::CT, CW = GS::CW, NCS = DK / CW, CWT = GS::CWT;
    // work units of a step are dealt to the halves of the workgroup in turn:
    // value tiles vt = hv + HV i, dA/dP column blocks st = STH hv + i, key
    // channel tiles ct = hv + HV i (in phase B, of the slice)
    constexpr int HV = NT / 256, VTH = VT / HV, STH = 4 / HV, CTH = CT / HV, CWH = CWT / HV;
    static_assert(VT % HV == 0 && CT % HV == 0 && CWT % HV == 0, "whole units per half");
    static_assert(VS % KB == 0 || VS < KB, "slice width");
    // LDS: persistent tables, then phase A and phase B regions over the same bytes
    constexpr int VSP = VS < KB ? KB : VS;                // slice width padded to a k-block (zeros)
    constexpr int LDP = 64 + 8, LDK = DK + 8, LDV = VSP + 8;
    // f16 operands: dO (for dDelta), dDelta and dX also as low parts (value - f16(value))
    constexpr bool SPLIT = sizeof(Op) == 2;
    constexpr int LO = SPLIT ? 1 : 0;
    constexpr size_t A_GT = 0, A_GR = A_GT + VS * LDK, A_SJ = A_GR + DK * LDV, A_DJ = A_SJ + DK * LDV, A_OJ = A_DJ + 64 * LDV,
                     A_OT = A_OJ + 64 * LDV, A_XJ = A_OT + VS * LDP, A_DT = A_XJ + 64 * LDV,
                     A_OTL = A_DT + VS * LDP, A_XJL = A_OTL + LO * VS * LDP, A_DTL = A_XJL + LO * 64 * LDV,
                     A_END = A_DTL + LO * VS * LDP;                                // elements of Op
    constexpr int LDF = 64 + 4, LDC = CW;
    // phase B (floats, then the raw inputs of the slice in the input type)
    constexpr size_t B_DA = 0, B_DP = B_DA + 64 * LDF, B_XT = B_DP + 64 * LDF, B_XM = B_XT + CW * LDF,
                     B_BT = B_XM + CW * LDF, B_BM = B_BT + CW * LDF, B_QT = B_BM + CW * LDF, B_QM = B_QT + CW * LDF,
                     B_DG = B_QM + CW * LDF, B_GAM = B_DG + 64 * LDC, B_KHK = B_GAM + DK,
                     B_KHS = B_KHK + 16 * CW, B_END = B_KHS + CW;                   // floats
    constexpr int LDR = 64 + 4;                           // raw inputs of the slice, transposed
    constexpr size_t B_BYTES = B_END * 4 + 3 * CW * LDR * sizeof(In);
    constexpr size_t REGION = (A_END * sizeof(Op) > B_BYTES ? A_END * sizeof(Op) : B_BYTES);
    // g (the chunk's cumulative log decay, all channels) from phase 0 to the end
    constexpr int LDL = DK + 1;
    __shared__ float sRef[5 * DK], sMid[4 * DK], sPart[NT], sGc[64 * LDL];
    __shared__ int sExactB[4];   // diagonal blocks that take the exact pairwise form
    __shared__ __attribute__((aligned(16))) unsigned char smem[REGION];
    Op *GT = (Op *)smem + A_GT;
    Op *Gr = (Op *)smem + A_GR, *Sj = (Op *)smem + A_SJ, *Dj = (Op *)smem + A_DJ, *Oj = (Op *)smem + A_OJ;
    Op *OT = (Op *)smem + A_OT, *Xj = (Op *)smem + A_XJ, *DT = (Op *)smem + A_DT;
    Op *OTl = (Op *)smem + A_OTL, *Xjl = (Op *)smem + A_XJL, *DTl = (Op *)smem + A_DTL;
    float *fb = (float *)smem;
    float *sdA = fb + B_DA, *sdP = fb + B_DP, *XtT = fb + B_XT, *XmT = fb + B_XM, *BtT = fb + B_BT, *BmT = fb + B_BM;
    float *QtT = fb + B_QT, *QmT = fb + B_QM, *sdG = fb + B_DG;
    // sum over the chunk's rows of (dk through Khat) k, per channel of the
    // slice: the part of each (wave, 4-row group) in its own slot, then their
    // sum in a fixed order (deterministic, unlike float atomics)
    float *sGam = fb + B_GAM, *sKhK = fb + B_KHK, *sKhS = fb + B_KHS;
    In *sqT = (In *)(fb + B_END), *skT = sqT + CW * LDR, *sbT = skT + CW * LDR;

    const int t = threadIdx.x, lane = t & 63, wv = wave_id() & 3, hv = wave_id() >> 2, m16 = lane & 15, g4 = lane >> 4;
    const int h = (int)(blockIdx.x % (unsigned)H), j = (int)(blockIdx.x / (unsigned)H);
    if (j >= min(sq.m.nchunks(), sq.max_chunks)) return;
    const int i = sq.m.seq_of(j);
    const int t0 = sq.t0(i) + 64 * (j - sq.m.chunk0(i));
    const int n = min(64, sq.t1(i) - t0);
    const size_t slot = (size_t)h * sq.max_chunks + j;
    const uint8_t *bblk = bops + slot * BL::bytes;
    const Op *Sc = sbuf + slot * DK * DV, *Dl = dbuf + slot * 64 * DV, *Gp = gbuf + slot * DK * DV;
    auto tok_k = [&](int r) { return ((size_t)(t0 + r) * H + h) * DK; };
    auto tok_v = [&](int r) { return ((size_t)(t0 + r) * H + h) * DV; };

    // log alpha of the chunk for phase 0, then (arriving during phase 0)
    // this wave's fragments of the forward block and the first value
    // slice's inputs
    constexpr int NU = 64 * DK / NT;
    float lv[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int x = t + NT * u, r = x / DK, c = x % DK;
        lv[u] = la[tok_k(min(r, n - 1)) + c];
    }
    // A-fragments of this wave's 16 chunk rows of P^T, T^T and Khat
    frag PTf[NSB], TTf[NSB], KHf[NKB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
        PTf[sb] = *reinterpret_cast<const frag *>(bblk + BL::oPT + ((size_t)(wv * NSB + sb) * 64 + lane) * 16);
        TTf[sb] = *reinterpret_cast<const frag *>(bblk + BL::oTT + ((size_t)(wv * NSB + sb) * 64 + lane) * 16);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
        KHf[kb] = *reinterpret_cast<const frag *>(bblk + BL::oKH + ((size_t)(wv * NKB + kb) * 64 + lane) * 16);
    // value-column slices, software-pipelined: the next slice's loads (G,
    // S_c, Delta, dO, and v, w for dv and dw) are issued before this slice's
    // work, into a second set of registers
    // G, S_c and Delta arrive in accumulator-tile order (tile (rt, ct) at
    // (rt * DV/16 + ct) * 256; lane l = n + 16g holds rows 4g..4g+3 of
    // column n): one 4-element load per lane and tile
    typedef Op op4 __attribute__((ext_vector_type(4)));
    constexpr int NG = (DK * VS / 4 + NT - 1) / NT, ND = (64 * VS / 4 + NT - 1) / NT;
    static_assert((DK * VS / 4) % 64 == 0 && (64 * VS / 4) % 64 == 0, "whole tiles");
    // x = tile * 64 + lane over the slice's tiles (row tile major)
    auto tile_at = [&](int x, int &rt, int &ctl, int &ln) { ln = x & 63; rt = (x >> 6) / VT; ctl = (x >> 6) % VT; };
    struct SR {
        op4 g[NG], s[NG], d[ND];
        f4 o[ND];
        In vv[VTH][4], ww[VTH][4];
    };
    auto sload = [&](SR &R_, int vs) {
        const int j0 = vs * VS;
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            int rt, ctl, ln;
            tile_at(min(t + NT * u, DK * VS / 4 - 1), rt, ctl, ln);
            const size_t o = ((size_t)rt * (DV / 16) + j0 / 16 + ctl) * 256 + ln * 4;
            R_.g[u] = *reinterpret_cast<const op4 *>(Gp + o);
            R_.s[u] = *reinterpret_cast<const op4 *>(Sc + o);
        }
#pragma unroll
        for (int u = 0; u < ND; ++u) {
            int rt, ctl, ln;
            tile_at(min(t + NT * u, 64 * VS / 4 - 1), rt, ctl, ln);
            R_.d[u] = *reinterpret_cast<const op4 *>(Dl + ((size_t)rt * (DV / 16) + j0 / 16 + ctl) * 256 + ln * 4);
            const int x = min(t + NT * u, 64 * VS / 4 - 1), r = x / (VS / 4), jj = 4 * (x % (VS / 4));
            R_.o[u] = *reinterpret_cast<const f4 *>(dO + tok_v(min(r, n - 1)) + j0 + jj);
        }
#pragma unroll
        for (int i = 0; i < VTH; ++i)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const size_t o = tok_v(min(16 * wv + 4 * g4 + ii, n - 1)) + j0 + 16 * (hv + HV * i) + m16;
                R_.vv[i][ii] = v[o];
                R_.ww[i][ii] = w[o];
            }
    };
    SR ra, rb;
    sload(ra, 0);

    // ---- phase 0: g and the references of the 16-row blocks, per channel ----
    // (log alpha staged through LDS with coalesced loads and summed down the
    // rows in place; phase B reads g from there)
    {
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int x = t + NT * u, r = x / DK, c = x % DK;
            sGc[r * LDL + c] = r < n ? lv[u] : 0.f;
        }
        if (t < 4) sExactB[t] = 0;
        __syncthreads();
        col_scan64<DK, false, NT>(sGc, LDL, sPart, t);
        for (int c = t; c < DK; c += NT) {
            sRef[c] = 0.f;
            float ref = 0.f;
#pragma unroll
            for (int R = 0; R < 4; ++R) {
                const float md = sGc[(16 * R + 7) * LDL + c], ref1 = sGc[(16 * R + 15) * LDL + c];
                sRef[(R + 1) * DK + c] = ref1;
                sMid[R * DK + c] = md;
                if (fmaxf(ref - md, md - ref1) > kBwdDiagSpread) atomicOr(&sExactB[R], 1);
                ref = ref1;
            }
        }
        __syncthreads();
    }

    // ---- phase A ----
    if constexpr (VSP > VS) {   // padding columns of the slice tiles stay zero
        for (int x = t; x < DK * (VSP - VS); x += NT) {
            const int c = x / (VSP - VS), jj = VS + x % (VSP - VS);
            Gr[c * LDV + jj] = (Op)0.f;
            Sj[c * LDV + jj] = (Op)0.f;
        }
        for (int x = t; x < 64 * (VSP - VS); x += NT) {
            const int r = x / (VSP - VS), jj = VS + x % (VSP - VS);
            Dj[r * LDV + jj] = (Op)0.f;
            Oj[r * LDV + jj] = (Op)0.f;
            Xj[r * LDV + jj] = (Op)0.f;
            if constexpr (SPLIT) Xjl[r * LDV + jj] = (Op)0.f;
        }
    }
    f4 accA[STH], accP[STH], F1[CTH], F2[CTH], F3[CTH];
#pragma unroll
    for (int x = 0; x < STH; ++x) { accA[x] = f4zero(); accP[x] = f4zero(); }
#pragma unroll
    for (int x = 0; x < CTH; ++x) { F1[x] = f4zero(); F2[x] = f4zero(); F3[x] = f4zero(); }
    float gam = 0.f;
    auto sstore = [&](const SR &R_) {
#pragma unroll
        for (int u = 0; u < NG; ++u) {
            const int x = t + NT * u;
            if (x >= DK * VS / 4) break;
            int rt, ctl, ln;
            tile_at(x, rt, ctl, ln);
            const int jj = 16 * ctl + (ln & 15);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = 16 * rt + 4 * (ln >> 4) + e;
                Gr[c * LDV + jj] = R_.g[u][e];
                GT[jj * LDK + c] = R_.g[u][e];
                Sj[c * LDV + jj] = R_.s[u][e];
            }
        }
#pragma unroll
        for (int u = 0; u < ND; ++u) {
            const int x = t + NT * u;
            if (x >= 64 * VS / 4) break;
            int rt, ctl, ln;
            tile_at(x, rt, ctl, ln);
#pragma unroll
            for (int e = 0; e < 4; ++e) Dj[(16 * rt + 4 * (ln >> 4) + e) * LDV + 16 * ctl + (ln & 15)] = R_.d[u][e];
        }
#pragma unroll
        for (int u = 0; u < ND * 4; ++u) {
            const int x = t + NT * (u / 4), r = x / (VS / 4), jj = 4 * (x % (VS / 4)) + (u % 4);
            if (x >= 64 * VS / 4) break;
            const float of = r < n ? R_.o[u / 4][u % 4] : 0.f;
            const Op o = (Op)of;
            Oj[r * LDV + jj] = o;
            OT[jj * LDP + r] = o;
            if constexpr (SPLIT) OTl[jj * LDP + r] = (Op)(of - (float)o);
        }
    };
#pragma unroll
    for (int vs = 0; vs < NVS; ++vs) {
        const int j0 = vs * VS;
        SR &cur = (vs & 1) ? rb : ra;
        SR &nxt = (vs & 1) ? ra : rb;
        __syncthreads();   // previous slice's readers are done
        if (vs + 1 < NVS) sload(nxt, vs + 1);
        sstore(cur);
        __syncthreads();
        // dDelta row tile wv: P^T dO + Khat G
#pragma unroll
        for (int i = 0; i < VTH; ++i) {
            const int vt = hv + HV * i;
            f4 acc = f4zero();
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const frag ap = PTf[sb];
                acc = M::mma(ap, lds_row_frag<Op>(OT + (16 * vt + m16) * LDP, sb * KB, g4), acc);
                if constexpr (SPLIT) acc = M::mma(ap, lds_row_frag<Op>(OTl + (16 * vt + m16) * LDP, sb * KB, g4), acc);
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                acc = M::mma(KHf[kb], lds_row_frag<Op>(GT + (16 * vt + m16) * LDK, kb * KB, g4), acc);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const Op hi = (Op)acc[ii];
                DT[(16 * vt + m16) * LDP + 16 * wv + 4 * g4 + ii] = hi;
                if constexpr (SPLIT) DTl[(16 * vt + m16) * LDP + 16 * wv + 4 * g4 + ii] = (Op)(acc[ii] - (float)hi);
            }
        }
        __syncthreads();
        // dX row tile wv: T^T dDelta; dv, dw
#pragma unroll
        for (int i = 0; i < VTH; ++i) {
            const int vt = hv + HV * i;
            f4 acc = f4zero();
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const frag at_ = TTf[sb];
                acc = M::mma(at_, lds_row_frag<Op>(DT + (16 * vt + m16) * LDP, sb * KB, g4), acc);
                if constexpr (SPLIT) acc = M::mma(at_, lds_row_frag<Op>(DTl + (16 * vt + m16) * LDP, sb * KB, g4), acc);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int r = 16 * wv + 4 * g4 + ii, jj = 16 * vt + m16;
                const Op hi = (Op)acc[ii];
                Xj[r * LDV + jj] = hi;
                if constexpr (SPLIT) Xjl[r * LDV + jj] = (Op)(acc[ii] - (float)hi);
                if (r < n) {
                    const size_t o = tok_v(r) + j0 + jj;
                    dv_[o] = acc[ii] * in2f<In>(cur.ww[i][ii]);
                    dw[o] = acc[ii] * in2f<In>(cur.vv[i][ii]);
                }
            }
        }
        __syncthreads();
        // accumulate over this slice's columns
#pragma unroll
        for (int kb = 0; kb < VKB; ++kb) {
            const frag ax = lds_row_frag<Op>(Xj + (16 * wv + m16) * LDV, kb * KB, g4);
            const frag axl = SPLIT ? lds_row_frag<Op>(Xjl + (16 * wv + m16) * LDV, kb * KB, g4) : ax;
            const frag ao = lds_row_frag<Op>(Oj + (16 * wv + m16) * LDV, kb * KB, g4);
            const frag ad = lds_row_frag<Op>(Dj + (16 * wv + m16) * LDV, kb * KB, g4);
#pragma unroll
            for (int i = 0; i < STH; ++i) {
                const int st = STH * hv + i;
                const frag bd = lds_row_frag<Op>(Dj + (16 * st + m16) * LDV, kb * KB, g4);
                accA[i] = M::mma(ax, bd, accA[i]);
                if constexpr (SPLIT) accA[i] = M::mma(axl, bd, accA[i]);
                accP[i] = M::mma(ao, bd, accP[i]);
            }
#pragma unroll
            for (int i = 0; i < CTH; ++i) {
                const int ct = hv + HV * i;
                const frag bs = lds_row_frag<Op>(Sj + (16 * ct + m16) * LDV, kb * KB, g4);
                const frag bg = lds_row_frag<Op>(Gr + (16 * ct + m16) * LDV, kb * KB, g4);
                F1[i] = M::mma(ao, bs, F1[i]);
                F2[i] = M::mma(ax, bs, F2[i]);
                if constexpr (SPLIT) F2[i] = M::mma(axl, bs, F2[i]);
                F3[i] = M::mma(ad, bg, F3[i]);
            }
        }
        if (t < DK)
            for (int jj = 0; jj < VS; ++jj) gam += (float)Gr[t * LDV + jj] * (float)Sj[t * LDV + jj];
    }
    // the first phase-B slice's inputs load while phase A finishes
    constexpr int SL = 64 * CW / NT, NIT = SL / 4;
    static_assert(NT % CW == 0 && SL % 4 == 0, "whole four-row groups per thread");
    struct alignas(4 * sizeof(In)) In4 { In v[4]; };
    struct BR { In q[SL], k[SL], b[SL]; };
    const int bcl = t % CW, bs = t / CW, r0 = SL * bs;
    auto bload = [&](BR &R_, int cs) {
#pragma unroll
        for (int i = 0; i < SL; ++i) {
            const size_t o = tok_k(min(r0 + i, n - 1)) + cs * CW + bcl;
            R_.q[i] = q[o];
            R_.k[i] = k[o];
            R_.b[i] = b[o];
        }
    };
    BR ba, bb2;
    bload(ba, 0);
    __syncthreads();   // phase A's LDS is free from here
#pragma unroll
    for (int i = 0; i < STH; ++i)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int r = 16 * wv + 4 * g4 + ii, s_ = 16 * (STH * hv + i) + m16;
            sdA[r * LDF + s_] = r > s_ ? -accA[i][ii] : 0.f;
            sdP[r * LDF + s_] = r >= s_ ? accP[i][ii] : 0.f;
        }
    if (t < DK) sGam[t] = gam * __expf(sRef[4 * DK + t]);

    // ---- phase B, key channels in slices of CW ----
    // Thread t owns channel bcl = t % CW of the slice and the SL consecutive
    // rows from r0 = SL * (t / CW). q, k, b of the next slice load while this
    // one is worked on; g comes from phase 0; the decay-scaled operands and
    // the raw inputs are written transposed, four rows per store.
#pragma unroll
    for (int cs = 0; cs < NCS; ++cs) {
        const int c0 = cs * CW;
        BR &bc = (cs & 1) ? bb2 : ba;
        BR &bn = (cs & 1) ? ba : bb2;
        // (the previous slice's readers of the phase-B regions finished before
        // its reverse scan)
        if (cs + 1 < NCS) bload(bn, cs + 1);
        const In zero_ = (In)0;
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int rb = r0 + 4 * it, R = rb >> 4, c = c0 + bcl;
            const float rf1 = sRef[(R + 1) * DK + c], rf0 = sRef[R * DK + c], md = sMid[R * DK + c];
            f4 xt, xm, bt, bm, qt, qm;
            In4 q4, k4, b4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * it + e;
                const bool ok = rb + e < n;
                const In kr_ = ok ? bc.k[i] : zero_, qr_ = ok ? bc.q[i] : zero_, br_ = ok ? bc.b[i] : zero_;
                const float kv = in2f<In>(kr_), qv = in2f<In>(qr_), bv = in2f<In>(br_);
                const float gv = sGc[(rb + e) * LDL + c];
                // (the middle-row factors of a block that takes the exact
                // form go unused; capped so that they stay finite)
                const float e1 = __expf(rf1 - gv), em = __expf(fminf(md - gv, 80.f));
                const float e2 = __expf(gv - rf0), en = __expf(fminf(gv - md, 80.f));
                xt[e] = kv * e1;
                xm[e] = kv * em;
                bt[e] = bv * kv * e2;   // row side of (dA o Dec)^T (b k), like q
                bm[e] = bv * kv * en;
                qt[e] = qv * e2;
                qm[e] = qv * en;
                q4.v[e] = qr_;
                k4.v[e] = kr_;
                b4.v[e] = br_;
            }
            *reinterpret_cast<f4 *>(XtT + bcl * LDF + rb) = xt;
            *reinterpret_cast<f4 *>(XmT + bcl * LDF + rb) = xm;
            *reinterpret_cast<f4 *>(BtT + bcl * LDF + rb) = bt;
            *reinterpret_cast<f4 *>(BmT + bcl * LDF + rb) = bm;
            *reinterpret_cast<f4 *>(QtT + bcl * LDF + rb) = qt;
            *reinterpret_cast<f4 *>(QmT + bcl * LDF + rb) = qm;
            *reinterpret_cast<In4 *>(sqT + bcl * LDR + rb) = q4;
            *reinterpret_cast<In4 *>(skT + bcl * LDR + rb) = k4;
            *reinterpret_cast<In4 *>(sbT + bcl * LDR + rb) = b4;
        }
        __syncthreads();
        const int R = wv;   // this wave's 16-row block (rows for Y, rows s for Z)
        const bool exactR = __builtin_amdgcn_readfirstlane(sExactB[R]) != 0;   // (uniform per wave)
        // Y1 = (dP o Dec) x, Y2 = (dA o Dec) x for the rows of block R and
        // Z = (dP o Dec)^T q + (dA o Dec)^T (b k) for the rows s of block R,
        // for the half's channel tiles ct = hv + HV j of the slice at once:
        // the left operands (rows or columns of dP and dA) are shared by the
        // tiles, the decay factors by the paired products
        float gR[CWH][4], midR[CWH];
        f4 Y1[CWH], Y2[CWH], Z[CWH];
#pragma unroll
        for (int ct = 0; ct < CWH; ++ct) {
            const int cl = 16 * (hv + HV * ct) + m16;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) gR[ct][ii] = sGc[(16 * R + 4 * g4 + ii) * LDL + c0 + cl];
            midR[ct] = sMid[R * DK + c0 + cl];
            Y1[ct] = f4zero();
            Y2[ct] = f4zero();
            Z[ct] = f4zero();
        }
        // row side: off-diagonal blocks S < R through ref_{S+1}, then the
        // diagonal block around its middle row
        for (int S = 0; S <= (exactR ? R - 1 : R); ++S) {
            const bool dg = S == R;
            const f4 a1 = *reinterpret_cast<const f4 *>(sdP + (16 * R + m16) * LDF + 16 * S + 4 * g4);
            const f4 a2 = *reinterpret_cast<const f4 *>(sdA + (16 * R + m16) * LDF + 16 * S + 4 * g4);
            const float *X = dg ? XmT : XtT;
#pragma unroll
            for (int ct = 0; ct < CWH; ++ct) {
                const int cl = 16 * (hv + HV * ct) + m16;
                const f4 bx = *reinterpret_cast<const f4 *>(X + cl * LDF + 16 * S + 4 * g4);
                const f4 p1 = MF::mma(a1, bx, f4zero()), p2 = MF::mma(a2, bx, f4zero());
                const float ref = dg ? midR[ct] : sRef[(S + 1) * DK + c0 + cl];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const float f = __expf(gR[ct][ii] - ref);
                    Y1[ct][ii] += p1[ii] * f;
                    Y2[ct][ii] += p2[ii] * f;
                }
            }
        }
        // column side: the diagonal block around its middle row, then the
        // off-diagonal blocks Rb > R through ref_Rb
        for (int Rb = exactR ? R + 1 : R; Rb < 4; ++Rb) {
            const bool dg = Rb == R;
            f4 a1, a2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a1[e] = sdP[(16 * Rb + 4 * g4 + e) * LDF + 16 * R + m16];
                a2[e] = sdA[(16 * Rb + 4 * g4 + e) * LDF + 16 * R + m16];
            }
            const float *Q_ = dg ? QmT : QtT, *B_ = dg ? BmT : BtT;
#pragma unroll
            for (int ct = 0; ct < CWH; ++ct) {
                const int cl = 16 * (hv + HV * ct) + m16;
                const f4 b1 = *reinterpret_cast<const f4 *>(Q_ + cl * LDF + 16 * Rb + 4 * g4);
                const f4 b2 = *reinterpret_cast<const f4 *>(B_ + cl * LDF + 16 * Rb + 4 * g4);
                const f4 p1 = MF::mma(a1, b1, f4zero()), p2 = MF::mma(a2, b2, f4zero());
                const float ref = dg ? midR[ct] : sRef[Rb * DK + c0 + cl];
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const float f = __expf(ref - gR[ct][ii]);
                    Z[ct][ii] += p1[ii] * f + p2[ii] * f;
                }
            }
        }
        // the diagonal terms dP_rr k_r of Y1 and dP_rr q_r of Z, kept apart in
        // exact blocks: they cancel in dq q - dk k, and at strong decay the
        // decay gradient is the small remainder of that difference
        float dY1[CWH][4], dZ[CWH][4];
#pragma unroll
        for (int ct = 0; ct < CWH; ++ct)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) { dY1[ct][ii] = 0.f; dZ[ct][ii] = 0.f; }
        if (exactR) {
            // the diagonal block with exact pairwise decay: e^{g_r - g_s}
            // (s <= r) as the running product of alpha over (s, r], from log
            // alpha itself (a difference of the chunk's cumulative sums would
            // carry their rounding, ~1e-4 at a cumulative decay near -1000)
            //   Y1, Y2 += sum_{s < r} (dP_rs, dA_rs) k_s e^{g_r - g_s}   (row r = this lane's)
            //   Z      += sum_{r > s} (dP_rs q_r + dA_rs b_r k_r) e^{g_r - g_s}   (row s = this lane's)
            // (s = r apart; dA_rr = 0)
            // (loops kept rolled and alpha read where used: this rare path
            // must not add registers to the common one)
            auto alpha = [&](int o, int c) { return o < n ? __expf(la[tok_k(o) + c]) : 1.f; };
#pragma unroll
            for (int ct = 0; ct < CWH; ++ct) {
                const int cl = 16 * (hv + HV * ct) + m16, c = c0 + cl;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int xl = 4 * g4 + ii, x = 16 * R + xl;   // r for Y, s for Z
                    float y1 = 0.f, y2 = 0.f, z = 0.f, f = 1.f;
#pragma unroll 1
                    for (int l = xl - 1; l >= 0; --l) {   // o = s < x, nearest first
                        const int o = 16 * R + l;
                        f *= alpha(o + 1, c);
                        const float ko = in2f<In>(skT[cl * LDR + o]) * f;
                        y1 += sdP[x * LDF + o] * ko;
                        y2 += sdA[x * LDF + o] * ko;
                    }
                    f = 1.f;
#pragma unroll 1
                    for (int l = xl + 1; l < 16; ++l) {   // o = r > x, nearest first
                        const int o = 16 * R + l;
                        f *= alpha(o, c);
                        const float ko = in2f<In>(skT[cl * LDR + o]);
                        const float qo = in2f<In>(sqT[cl * LDR + o]), bo = in2f<In>(sbT[cl * LDR + o]);
                        z += (sdP[o * LDF + x] * qo + sdA[o * LDF + x] * bo * ko) * f;
                    }
                    const float dpx = sdP[x * LDF + x];
                    Y1[ct][ii] += y1;
                    Y2[ct][ii] += y2;
                    Z[ct][ii] += z;
                    dY1[ct][ii] = dpx * in2f<In>(skT[cl * LDR + x]);
                    dZ[ct][ii] = dpx * in2f<In>(sqT[cl * LDR + x]);
                }
            }
        }
#pragma unroll
        for (int ct = 0; ct < CWH; ++ct) {
            // (F1..F3 hold the half's key channel tiles hv + HV i; this one is
            // tile cs CWT + hv + HV ct of the head)
            const int cl = 16 * (hv + HV * ct) + m16, c = c0 + cl, ctg = cs * CWH + ct;
            const float gn = sRef[4 * DK + c];
            float khk = 0.f;
            const In4 q4 = *reinterpret_cast<const In4 *>(sqT + cl * LDR + 16 * R + 4 * g4);
            const In4 k4 = *reinterpret_cast<const In4 *>(skT + cl * LDR + 16 * R + 4 * g4);
            const In4 b4 = *reinterpret_cast<const In4 *>(sbT + cl * LDR + 16 * R + 4 * g4);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int r = 16 * R + 4 * g4 + ii;
                const float gv = gR[ct][ii], eg = __expf(gv), egn = __expf(gn - gv);
                const float qv = in2f<In>(q4.v[ii]), kv = in2f<In>(k4.v[ii]), bv = in2f<In>(b4.v[ii]);
                const float dqo = F1[ctg][ii] * eg + Y1[ct][ii], dqv = dqo + dY1[ct][ii];
                const float dEe = -F2[ctg][ii] * eg + Y2[ct][ii];
                const float dkm = Z[ct][ii] + dZ[ct][ii];
                const float dkh = F3[ctg][ii] * egn;
                const float dkv = dkm + dkh + dEe * bv;
                const float dbv = dEe * kv;
                // (the diagonal terms dY1 q - dZ k cancel exactly: left out)
                sdG[r * LDC + cl] = dqo * qv - Z[ct][ii] * kv - dkh * kv + dEe * bv * kv;
                khk += dkh * kv;
                if (r < n) {
                    const size_t o = tok_k(r) + c;
                    dq[o] = dqv;
                    dk_[o] = dkv;
                    db[o] = dbv;
                }
            }
            sKhK[(wv * 4 + g4) * CW + cl] = khk;   // rows 16 wv + 4 g4 .. + 3
        }
        __syncthreads();
        if (t < CW) {
            float x = 0.f;
#pragma unroll
            for (int sl = 0; sl < 16; ++sl) x += sKhK[sl * CW + t];
            sKhS[t] = x;   // (read after the scan's barriers)
        }
        col_scan64<CW, true, NT>(sdG, LDC, sPart, t);
#pragma unroll
        for (int u = 0; u < 64 * CW / NT; ++u) {
            const int x = t + NT * u, r = x / CW, cl = x % CW, c = c0 + cl;
            if (r < n) dla[tok_k(r) + c] = sdG[r * LDC + cl] + sKhS[cl] + sGam[c];
        }
    }
}

// ---------------------------------------------------------------------------
template <typename In, typename Op, int DK, int DV>
static hipError_t bwd_t(const ChunkBwdArgs &a, const BwdPlan &bp, hipStream_t st)
{
    uint8_t *ws = (uint8_t *)a.workspace;
    ChunkArgs fa;
    fa.q = a.q; fa.k = a.k; fa.v = a.v; fa.b = a.b; fa.w = a.w;
    fa.log_alpha = a.log_alpha;
    fa.S0 = a.S0;
    fa.o = a.part == kBwdForward ? a.o : nullptr;
    fa.ST = a.part == kBwdForward ? a.ST : nullptr;
    fa.cu_seqlens = a.cu_seqlens;
    fa.B = a.B; fa.T = a.T; fa.N = a.N; fa.H = a.H; fa.dk = a.dk; fa.dv = a.dv;
    fa.gates = 0;
    fa.bf16 = a.bf16;
    fa.workspace = a.workspace;
    fa.workspace_bytes = a.workspace_bytes;
    // forward: operand blocks, then the pass keeping S_c and Delta (the
    // training forward also forms o and S_T); a backward over what a training
    // forward kept starts after it
    hipError_t err = hipSuccess;
    if (a.part != kBwdFromKept) {
        const SaveOut so = {ws + bp.off_states, ws + bp.off_delta, a.part == kBwdForward};
        err = launch_t<In, Op, DK, DV>(fa, bp.fwd, st, so);
        if (err != hipSuccess || a.part == kBwdForward) return err;
    }

    Seqs sq;
    sq.m.cu = a.cu_seqlens;
    sq.m.co = a.cu_seqlens ? (const int32_t *)ws : nullptr;
    sq.m.N = a.N;
    sq.m.T = a.T;
    sq.Ttot = a.cu_seqlens ? a.T : a.B * a.T;
    sq.max_chunks = bp.fwd.max_chunks;
    sq.gates = 0;
    const uint8_t *ops = ws + bp.fwd.plan_bytes + bp.fwd.prog_bytes;
    uint8_t *bops = ws + bp.off_bblocks;
    int *prog = (int *)(ws + bp.fwd.plan_bytes);
    if (bp.fwd.max_chunks > 0) {
        prof_before("gdn2_chunk_bprep", st);
        hipLaunchKernelGGL((chunk_bprep_kernel<Op, DK>), dim3((unsigned)((long long)bp.fwd.max_chunks * a.H)),
                           dim3(256), 0, st, ops, bops, sq, a.H, prog, (int)((long long)a.N * a.H));
        prof_after(st);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    int cus = 0;
    if ((err = device_cus(&cus)) != hipSuccess) return err;
    const long long chains = (long long)a.N * a.H, groups = (chains + 7) / 8;
    constexpr int NSL1 = DV / 16;
    const bool two = NSL1 % 2 == 0 && 8LL * NSL1 * groups > cus;
    const int nsl = two ? NSL1 / 2 : NSL1;
    // prefetch workgroups per chain where the chip has slots to spare, as for the forward pass
    const int npfc = (int)std::min<long long>(kMaxPrefetchWgs, cus / (8 * groups) - nsl);
    const int npf = (npfc < 2 || bp.fwd.max_chunks == 0) ? 0 : npfc;
    const long long grid = 8LL * (nsl + npf) * groups;
    if (grid > 0x7fffffffLL) return hipErrorInvalidValue;
    Op *gbuf = (Op *)(ws + bp.off_grads);
    prof_before("gdn2_chunk_rpass", st);
    if constexpr (NSL1 % 2 == 0) {
        if (two)
            hipLaunchKernelGGL((chunk_rpass_kernel<Op, DK, DV, 2>), dim3((unsigned)grid), dim3(512), 0, st, a.dO,
                               a.dST, a.dS0, sq, a.H, (const uint8_t *)bops, gbuf, prog, npf);
        else
            hipLaunchKernelGGL((chunk_rpass_kernel<Op, DK, DV, 1>), dim3((unsigned)grid), dim3(512), 0, st, a.dO,
                               a.dST, a.dS0, sq, a.H, (const uint8_t *)bops, gbuf, prog, npf);
    } else {
        hipLaunchKernelGGL((chunk_rpass_kernel<Op, DK, DV, 1>), dim3((unsigned)grid), dim3(512), 0, st, a.dO, a.dST,
                           a.dS0, sq, a.H, (const uint8_t *)bops, gbuf, prog, npf);
    }
    prof_after(st);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (bp.fwd.max_chunks > 0) {
        prof_before("gdn2_chunk_grad", st);
        constexpr int NTG = GradShape<Op, DK, DV>::NT;
        hipLaunchKernelGGL((chunk_grad_kernel<In, Op, DK, DV, NTG>), dim3((unsigned)((long long)bp.fwd.max_chunks * a.H)),
                           dim3(NTG), 0, st, (const In *)a.q, (const In *)a.k, (const In *)a.v, a.log_alpha,
                           (const In *)a.b, (const In *)a.w, a.dO, sq, a.H, (const uint8_t *)bops,
                           (const Op *)(ws + bp.off_states),
                           (const Op *)(ws + bp.off_delta), (const Op *)gbuf, a.dq, a.dk_, a.dv_, a.dlog_alpha, a.db,
                           a.dw);
        prof_after(st);
    }
    return hipGetLastError();
}

template <typename In, typename Op, int DK>
hipError_t dispatch_bwd(const ChunkBwdArgs &a, const BwdPlan &p, hipStream_t st)
{
    switch (a.dv) {
    case 16: return bwd_t<In, Op, DK, 16>(a, p, st);
    case 32: return bwd_t<In, Op, DK, 32>(a, p, st);
    case 64: return bwd_t<In, Op, DK, 64>(a, p, st);
    case 128: return bwd_t<In, Op, DK, 128>(a, p, st);
    }
    return hipErrorInvalidValue;
}

} // namespace gdn2
