// Device-side helpers shared by the gdn2 kernels (gfx950 / CDNA4).
//
// MFMA fragment conventions used throughout (one 64-wide wavefront, lane
// l = n + 16*g with n = l % 16 and g = l / 16):
//  * D / accumulator tile 16x16 fp32: lane l holds rows 4g..4g+3 of column n.
//  * A fragment of a 16 x KB block (rows m, contraction k): lane l = m + 16g
//    holds KB/4 values A[m][kofs(g, i)], i = 0..KB/4-1.
//  * B fragment of a KB x 16 block: lane l = n + 16g holds B[kofs(g, i)][n].
//  kofs(g, i) = 16*(i/4) + 4g + (i%4). Any bijection works as long as A and B
//  use the same one, because the hardware pairs A element i of lane m+16g
//  with B element i of lane n+16g. This one makes the B fragment of a
//  32-deep block equal to two stacked accumulator tiles, so a product can
//  feed the next product without a trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace gdn2 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int kofs(int g, int i) { return 16 * (i >> 2) + 4 * g + (i & 3); }

// ---- input element loads (bf16 bit patterns or fp32) -----------------------
__device__ __forceinline__ float bf16f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
// one input element (bf16 bit pattern or fp32) as float
template <typename In> __device__ __forceinline__ float in2f(In x);
template <> __device__ __forceinline__ float in2f<uint16_t>(uint16_t x) { return bf16f(x); }
template <> __device__ __forceinline__ float in2f<float>(float x) { return x; }

template <typename In> struct Ld;
template <> struct Ld<uint16_t> {
    // a pair of consecutive elements kept packed until use
    typedef uint32_t raw2;
    static __device__ __forceinline__ raw2 ldraw2(const uint16_t *p) { return *reinterpret_cast<const uint32_t *>(p); }
    static __device__ __forceinline__ f2 cvt2(raw2 u) {
        f2 r;
        r[0] = __uint_as_float(u << 16);
        r[1] = __uint_as_float(u & 0xFFFF0000u);
        return r;
    }
    static __device__ __forceinline__ raw2 zero2() { return 0u; }
    // one element, twice
    static __device__ __forceinline__ raw2 splat2(const uint16_t *p) { const uint32_t x = *p; return x | (x << 16); }
    // two consecutive elements
    static __device__ __forceinline__ f2 two(const uint16_t *p) {
        uint32_t u = *reinterpret_cast<const uint32_t *>(p);
        f2 r;
        r[0] = __uint_as_float(u << 16);
        r[1] = __uint_as_float(u & 0xFFFF0000u);
        return r;
    }
    static __device__ __forceinline__ float one(const uint16_t *p) { return bf16f(*p); }
};
template <> struct Ld<float> {
    typedef f2 raw2;
    static __device__ __forceinline__ raw2 ldraw2(const float *p) { return *reinterpret_cast<const f2 *>(p); }
    static __device__ __forceinline__ f2 cvt2(raw2 u) { return u; }
    static __device__ __forceinline__ raw2 zero2() { f2 z = {0.f, 0.f}; return z; }
    static __device__ __forceinline__ raw2 splat2(const float *p) { const float x = *p; f2 r = {x, x}; return r; }
    static __device__ __forceinline__ f2 two(const float *p) { return *reinterpret_cast<const f2 *>(p); }
    static __device__ __forceinline__ float one(const float *p) { return *p; }
};

// ---- matrix-core operand traits ---------------------------------------------
// Op = _Float16: v_mfma_f32_16x16x32_f16, k-blocks of 32, 8 halves per lane.
// Op = float:    four v_mfma_f32_16x16x4_f32, k-blocks of 16, 4 floats per lane.
template <typename Op> struct Mma;

template <> struct Mma<_Float16> {
    static constexpr int KB = 32;
    static constexpr int NE = 8;
    typedef h8 frag;
    static __device__ __forceinline__ f4 mma(const frag &a, const frag &b, f4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    // 16x16x16 product from fp32 values (lane holds A[m][4g+i], B[4g+i][n]).
    static __device__ __forceinline__ f4 mma16(const f4 &a, const f4 &b, f4 c) {
        h4 ah, bh;
        for (int i = 0; i < 4; ++i) { ah[i] = (_Float16)a[i]; bh[i] = (_Float16)b[i]; }
        return __builtin_amdgcn_mfma_f32_16x16x16f16(ah, bh, c, 0, 0, 0);
    }
};

template <> struct Mma<float> {
    static constexpr int KB = 16;
    static constexpr int NE = 4;
    typedef f4 frag;
    static __device__ __forceinline__ f4 mma(const frag &a, const frag &b, f4 c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
        return c;
    }
    static __device__ __forceinline__ f4 mma16(const f4 &a, const f4 &b, f4 c) { return mma(a, b, c); }
};

// Index of the calling wave within its workgroup as a scalar (wave-uniform)
// value. Conditions and loop bounds derived from it then compile to scalar
// branches, which really skip what they guard: a matrix instruction issued
// under an empty execution mask still runs, so skipping it by masking lanes
// alone is not enough.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6); }

// Sum over aligned groups of G lanes (G = 8, 16, 32 or 64), the result in
// every lane of the group; all 64 lanes must be active. Within rows of 16
// lanes: DPP swaps (xor 1, xor 2, then the half-row and row mirrors, which
// pair the halves once the smaller groups already hold their sums). Across
// rows: the row broadcasts add row 0 into row 1 and row 2 into row 3 (lanes
// 31 and 63 then hold the 32-lane sums) and lane 31 into rows 2 and 3 (lane
// 63 holds the total), read back with readlane.
template <int G> __device__ __forceinline__ float lane_group_sum(float x)
{
    static_assert(G == 8 || G == 16 || G == 32 || G == 64, "group of 8 to 64 lanes");
    auto dpp = [](float v, auto ctrl, auto rows) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), decltype(ctrl)::value,
                                                          decltype(rows)::value, 0xF, false));
    };
    using all = std::integral_constant<int, 0xF>;
    x += dpp(x, std::integral_constant<int, 0xB1>{}, all{});    // quad_perm [1,0,3,2]
    x += dpp(x, std::integral_constant<int, 0x4E>{}, all{});    // quad_perm [2,3,0,1]
    x += dpp(x, std::integral_constant<int, 0x141>{}, all{});   // row_half_mirror
    if constexpr (G >= 16) x += dpp(x, std::integral_constant<int, 0x140>{}, all{});   // row_mirror
    if constexpr (G >= 32) {
        x += dpp(x, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xA>{});   // row_bcast:15
        if constexpr (G == 64) {
            x += dpp(x, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xC>{});   // row_bcast:31
            x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
        } else {
            const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
            const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
            x = (__lane_id() < 32) ? lo : hi;
        }
    }
    return x;
}

__device__ __forceinline__ f4 f4zero() { f4 z = {0.f, 0.f, 0.f, 0.f}; return z; }

// Fragment whose contraction runs along a row of a row-major LDS tile:
// element i is rowp[kbase + kofs(g, i)], read as NE/4 runs of 4 elements
// (8-byte reads for f16, 16-byte for fp32; the caller keeps them aligned).
template <typename Op>
__device__ __forceinline__ typename Mma<Op>::frag lds_row_frag(const Op *rowp, int kbase, int g4)
{
    typedef Op op4 __attribute__((ext_vector_type(4)));
    typename Mma<Op>::frag f;
#pragma unroll
    for (int p = 0; p < Mma<Op>::NE / 4; ++p) {
        const op4 x = *reinterpret_cast<const op4 *>(rowp + kbase + 16 * p + 4 * g4);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) f[4 * p + ii] = x[ii];
    }
    return f;
}

// ---- chunk bookkeeping -------------------------------------------------------
// Sequences are token ranges [cu[i], cu[i+1]); each is cut into CS-token
// chunks (64 unless a chunk-size variant asks otherwise) starting at its first
// token; chunk ids are numbered sequence by sequence (co[i] = first chunk id
// of sequence i). Uniform batches (no cu_seqlens) use cu[i] = i*T and
// co[i] = i*ceil(T/CS) computed in place.
struct SeqMap {
    const int32_t *cu;   // device [N+1] or null (uniform)
    const int32_t *co;   // device [N+1] chunk offsets (varlen) or null
    int N, T;            // T: tokens per sequence when uniform
    __device__ __forceinline__ int tok0(int i) const { return cu ? cu[i] : i * T; }
    __device__ __forceinline__ int tok1(int i) const { return cu ? cu[i + 1] : (i + 1) * T; }
    template <int CS = 64> __device__ __forceinline__ int per_seq() const { return (T + CS - 1) >> __builtin_ctz(CS); }
    template <int CS = 64> __device__ __forceinline__ int chunk0(int i) const { return co ? co[i] : i * per_seq<CS>(); }
    template <int CS = 64> __device__ __forceinline__ int nchunks() const { return co ? co[N] : N * per_seq<CS>(); }
    // sequence owning chunk id j (j < nchunks()): largest i with chunk0(i) <= j
    template <int CS = 64> __device__ __forceinline__ int seq_of(int j) const {
        if (!co) return j / per_seq<CS>();
        int lo = 0, hi = N - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (co[mid] <= j) lo = mid; else hi = mid - 1;
        }
        return lo;
    }
};

} // namespace gdn2
