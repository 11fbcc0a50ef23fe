// Fused single-token decode step of the Gated Delta Rule-2.
//
// For each (sequence, head) with state S [dk][dv] fp32 (rows = key channels),
// one token (snilld.dk, "Hvad Gated DeltaNet-2 ændrer", update equation):
//   S~ = Diag(alpha) S,  e = S~^T (b*k),  r = S~^T q,
//   delta = w*v - e,     S_new = S~ + k delta^T,   o = S_new^T q = r + delta (k.q)
// The last identity lets the readout come from the same pass that reads S,
// so S is read from HBM once and written once (the step is bound by HBM
// bandwidth: about 0.86 flop per byte).
//
// One workgroup per (sequence, head). Thread t owns 4 consecutive columns and
// DK/ROWG rows of S, kept in registers between the reductions and the update.
//
// PRO (fused prologue): q, k, v arrive raw with their convolution history
// (three earlier raw inputs per channel) and b, w as logits. q, k and v are
// the short convolutions, b and w the sigmoids. The unit-norm scales of q and
// k are applied to the reduced quantities (e, r, k.q) and to the rank-one
// update rather than to every element: the sums of squares are reduced
// alongside k.q, before they are needed. The history moves up by one token
// (each thread rewrites the channels it read, so it may be updated in place).
#include "gdn2_device.hpp"
#include "gdn2_launch.hpp"

namespace gdn2 {

template <int DK, int DV> struct DecodeShape {
    static constexpr int COLG = DV / 4;                                  // column groups
    static constexpr int ROWG = (DK < 512 / COLG) ? DK : 512 / COLG;     // row groups (512 threads: 6.8 vs 6.6 TB/s at 256)
    static constexpr int RPT = DK / ROWG;                                // rows per thread
    static constexpr int NT = COLG * ROWG;                               // threads
};

struct DecConv {
    const float *w, *bias;   // taps [H*d][4] (tap 3 on the current token), bias [H*d] or null
    const void *hin;         // history [N*H][3][d] or null (zeros)
    void *hout;              // shifted history, or null; may equal hin
};

template <typename In, int D>
__device__ __forceinline__ float conv_token(const In *x, const DecConv &c, int nh, int h, int ch, In raw[4])
{
    // raw[0..2]: the history (oldest first), raw[3]: this token
    const In *hin = (const In *)c.hin;
#pragma unroll
    for (int j = 0; j < 3; ++j) raw[j] = hin ? hin[((size_t)nh * 3 + j) * D + ch] : (In)0;
    raw[3] = x[(size_t)nh * D + ch];
    const f4 tap = *reinterpret_cast<const f4 *>(c.w + 4 * ((size_t)h * D + ch));
    float y = c.bias ? c.bias[(size_t)h * D + ch] : 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) y += tap[j] * in2f<In>(raw[j]);
    return y;
}

template <typename In, int D>
__device__ __forceinline__ void shift_history(const DecConv &c, int nh, int ch, const In raw[4])
{
    if (!c.hout) return;
    In *ho = (In *)c.hout;
#pragma unroll
    for (int j = 0; j < 3; ++j) ho[((size_t)nh * 3 + j) * D + ch] = raw[j + 1];
}

__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

template <typename In, int DK, int DV, bool PRO>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) void decode_kernel(
    const In *__restrict__ q, const In *__restrict__ k, const In *__restrict__ v,
    const float *__restrict__ la, const In *__restrict__ b, const In *__restrict__ w,
    float *__restrict__ S, float *__restrict__ o, int gates, int H, int rev, DecConv cq, DecConv ck, DecConv cv)
{
    using Sh = DecodeShape<DK, DV>;
    constexpr int COLG = Sh::COLG, ROWG = Sh::ROWG, RPT = Sh::RPT, NT = Sh::NT;
    // sequence * H + head, in the order of this call (see decode_order)
    const int nh = rev ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
    const int t = threadIdx.x;
    const int cg = t % COLG, rg = t / COLG;

    __shared__ float s_a[DK], s_bk[DK], s_q[DK], s_k[DK], s_u[DV];
    __shared__ f4 s_e[ROWG][COLG], s_r[ROWG][COLG];
    constexpr int NW = NT / 64 > 0 ? NT / 64 : 1;
    __shared__ float s_kq[NW], s_qq[NW], s_kk[NW], s_kqp[PRO ? ROWG : 1];

    float *Sp = S + (size_t)nh * DK * DV;
    f4 sv[RPT];
    auto load_state = [&]() {
#pragma unroll
        for (int r = 0; r < RPT; ++r)
            sv[r] = *reinterpret_cast<const f4 *>(Sp + (size_t)(rg + r * ROWG) * DV + 4 * cg);
    };
    // (with the fused prologue the state rows load after the convolution's
    // few, latency-bound loads, which the first barrier waits for: 96 -> 91
    // us for 256 x 16 chains at d = 128)
    if constexpr (!PRO) load_state();

    // gates: one value per channel, or per (sequence, head) where the bit is set
    const bool asc = gates & kGateAlpha, bsc = gates & kGateB, wsc = gates & kGateW;
    float kq = 0.f, qq = 0.f, kk = 0.f;
    if constexpr (PRO) {
        // one job per thread: a q channel, a k channel, a v channel (with its
        // write gate), or an erase gate and decay; k.q waits for the first
        // barrier (its factors come from different threads)
        const int h = nh % H;
        for (int x = t; x < 3 * DK + DV; x += NT) {
            In raw[4];
            if (x < DK) {
                const float y = conv_token<In, DK>(q, cq, nh, h, x, raw);
                shift_history<In, DK>(cq, nh, x, raw);
                s_q[x] = y;
                qq += y * y;
            } else if (x < 2 * DK) {
                const int c = x - DK;
                const float y = conv_token<In, DK>(k, ck, nh, h, c, raw);
                shift_history<In, DK>(ck, nh, c, raw);
                s_k[c] = y;
                kk += y * y;
            } else if (x < 2 * DK + DV) {
                const int j = x - 2 * DK;
                const float y = conv_token<In, DV>(v, cv, nh, h, j, raw);
                shift_history<In, DV>(cv, nh, j, raw);
                s_u[j] = sigmoidf_(Ld<In>::one(w + (size_t)nh * DV + j)) * y;
            } else {
                const int c = x - 2 * DK - DV;
                const size_t i = (size_t)nh * DK + c;
                s_bk[c] = sigmoidf_(Ld<In>::one(b + i));   // the erase gate alone here
                s_a[c] = __expf(la[i]);
            }
        }
        load_state();
    } else {
        for (int c = t; c < DK; c += NT) {
            const size_t i = (size_t)nh * DK + c;
            const float kc = Ld<In>::one(k + i), qc = Ld<In>::one(q + i);
            s_a[c] = __expf(la[asc ? (size_t)nh : i]);
            s_k[c] = kc;
            s_q[c] = qc;
            s_bk[c] = Ld<In>::one(b + (bsc ? (size_t)nh : i)) * kc;
            kq += kc * qc;
        }
        for (int j = t; j < DV; j += NT) {
            const size_t i = (size_t)nh * DV + j;
            s_u[j] = Ld<In>::one(w + (wsc ? (size_t)nh : i)) * Ld<In>::one(v + i);
        }
    }
    // k.q (PRO: the squared norms of q and k): wave reduction, then across waves
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        if constexpr (PRO) {
            qq += __shfl_xor(qq, off);
            kk += __shfl_xor(kk, off);
        } else {
            kq += __shfl_xor(kq, off);
        }
    }
    if ((t & 63) == 0) {
        if constexpr (PRO) {
            s_qq[t >> 6] = qq;
            s_kk[t >> 6] = kk;
        } else {
            s_kq[t >> 6] = kq;
        }
    }
    __syncthreads();

    f4 e = f4zero(), rr = f4zero();
    float kqp = 0.f;   // PRO: this thread's rows of k.q (one column group adds them)
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int c = rg + r * ROWG;
        sv[r] = sv[r] * s_a[c];
        if constexpr (PRO) {
            const float kc = s_k[c], qc = s_q[c];
            e += sv[r] * (s_bk[c] * kc);
            kqp += kc * qc;
        } else {
            e += sv[r] * s_bk[c];
        }
        rr += sv[r] * s_q[c];
    }
    s_e[rg][cg] = e;
    s_r[rg][cg] = rr;
    if constexpr (PRO)
        if (cg == 0) s_kqp[rg] = kqp;
    __syncthreads();

    f4 E = f4zero(), R = f4zero();
#pragma unroll
    for (int g = 0; g < ROWG; ++g) { E += s_e[g][cg]; R += s_r[g][cg]; }
    float KQ = 0.f;
    if constexpr (PRO) {
#pragma unroll
        for (int g = 0; g < ROWG; ++g) KQ += s_kqp[g];
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) KQ += s_kq[i];
    }
    float kscale = 1.f;   // PRO: 1 / max(|k|, 1e-12), and likewise for q
    if constexpr (PRO) {
        float QQ = 0.f, KK = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) { QQ += s_qq[i]; KK += s_kk[i]; }
        const float qscale = rsqrtf(fmaxf(QQ, 1e-24f));
        kscale = rsqrtf(fmaxf(KK, 1e-24f));
        E *= kscale;
        R *= qscale;
        KQ *= qscale * kscale;
    }
    f4 u = *reinterpret_cast<const f4 *>(&s_u[4 * cg]);
    const f4 delta = u - E;
    if (rg == 0)
        *reinterpret_cast<f4 *>(o + (size_t)nh * DV + 4 * cg) = R + delta * KQ;
    // The new state is written with non-temporal stores (measured: 6.6 vs
    // 6.2 TB/s for the 256 x 16 x 128 x 128 state; non-temporal loads gain
    // as much alone, but the two together lose).
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int c = rg + r * ROWG;
        __builtin_nontemporal_store(sv[r] + delta * (s_k[c] * kscale),
                                    reinterpret_cast<f4 *>(Sp + (size_t)(rg + r * ROWG) * DV + 4 * cg));
    }
}

// Order of the chains for this call on state buffer S. Successive calls on
// one state visit the (sequence, head) chains in alternating directions, so
// the chains written last, which the last-level cache still holds, are read
// first: with a state of 1 GiB (four times that cache) the step takes 16%
// less time (431 -> 363 us at 1024 x 16 chains, d = 128). Each chain is read
// and written by one workgroup, so the results do not depend on the order.
// The parity is kept per thread in a small table keyed by the state's
// address; a state that loses its entry restarts at the forward order.
static int decode_order(const void *S)
{
    constexpr int kSlots = 64;
    struct Slot {
        const void *p = nullptr;
        unsigned n = 0;
    };
    thread_local Slot slots[kSlots];
    Slot &x = slots[((uintptr_t)S >> 8) % kSlots];
    if (x.p != S) {
        x.p = S;
        x.n = 0;
    }
    return (int)(x.n++ & 1u);
}

template <typename In, int DK, int DV>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t st)
{
    constexpr int NT = DecodeShape<DK, DV>::NT;
    const DecConv cq = {a.pro.q.w, a.pro.q.bias, a.pro.q.hist_in, a.pro.q.hist_out};
    const DecConv ck = {a.pro.k.w, a.pro.k.bias, a.pro.k.hist_in, a.pro.k.hist_out};
    const DecConv cv = {a.pro.v.w, a.pro.v.bias, a.pro.v.hist_in, a.pro.v.hist_out};
    const int rev = decode_order(a.S);
    prof_before("gdn2_decode", st);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(a.N * a.H), dim3(NT), 0, st, (const In *)a.q, (const In *)a.k,
                           (const In *)a.v, a.log_alpha, (const In *)a.b, (const In *)a.w, a.S, (float *)a.o,
                           a.gates, a.H, rev, cq, ck, cv);
    };
    if (a.pro.on) go(decode_kernel<In, DK, DV, true>);
    else go(decode_kernel<In, DK, DV, false>);
    prof_after(st);
    return hipGetLastError();
}

template <typename In, int DK>
static hipError_t dispatch_dv(const DecodeArgs &a, hipStream_t st)
{
    switch (a.dv) {
    case 16: return launch_decode_t<In, DK, 16>(a, st);
    case 32: return launch_decode_t<In, DK, 32>(a, st);
    case 64: return launch_decode_t<In, DK, 64>(a, st);
    case 128: return launch_decode_t<In, DK, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

template <typename In>
static hipError_t dispatch_dk(const DecodeArgs &a, hipStream_t st)
{
    switch (a.dk) {
    case 16: return dispatch_dv<In, 16>(a, st);
    case 32: return dispatch_dv<In, 32>(a, st);
    case 64: return dispatch_dv<In, 64>(a, st);
    case 128: return dispatch_dv<In, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st)
{
    return a.bf16 ? dispatch_dk<uint16_t>(a, st) : dispatch_dk<float>(a, st);
}

} // namespace gdn2
