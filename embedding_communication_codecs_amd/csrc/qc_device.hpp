// qc_device.hpp -- device-side building blocks shared by the libqc kernels
// (gfx950, wave64).  Host code never includes this file.
//
// Numeric rule for every kernel: each fp32 operation of a codec formula
// rounds once, to nearest even, in the order written.  Multiply-add
// contraction is switched off twice over (the pragma below, which every
// kernel source includes first, and -ffp-contract=off on the command line);
// division and sqrtf keep HIP's correctly rounded defaults (the "_rn"
// intrinsics are avoided: without extra configuration __fsqrt_rn maps to
// the approximate native square root); fp32 denormals stay enabled.
#pragma once
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qc {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ---------------------------------------------------------------- memory
// Outputs are written once and not re-read by the same kernel, so they go
// out as non-temporal stores (they should not displace inputs in L2).

__device__ __forceinline__ f32x4 ld_f4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ u32x4 ld_u4(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Streaming loads, for inputs each kernel reads exactly once: the
// non-temporal hint keeps them from displacing reused lines.  Measured on
// MI355X: +10% on the QSGD encoder's read/write mix.
__device__ __forceinline__ f32x4 ld_stream_f4(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ u32x4 ld_stream_u4(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld_stream_u2(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ uint32_t ld_stream_u32(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint32_t ld_stream_u16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}
__device__ __forceinline__ void st_f4(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void st_u4(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_u32(void* p, uint32_t v) {
    __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}

// ----------------------------------------------------- cross-lane reduces
// Butterfly over aligned groups of G lanes (G a power of two <= 64): step
// `off` combines lane t with lane t^off, i.e. two adjacent, equally sized,
// contiguous blocks, so a sum built this way adds exactly the sibling
// subtrees of a contiguous pairwise tree (fp32 addition is commutative, so
// both partners obtain identical bits).
//
// The steps inside a 16-lane row are DPP moves, which read the partner's
// register directly (__shfl_xor goes through the LDS crossbar,
// ds_bpermute, whose latency the FP8 encoder paid 20 times per wave:
// measured 0.119 -> 0.113 ms at 1e6 x 128 on MI355X).  off = 1 and 2 are the
// quad permutations [1,0,3,2] and [2,3,0,1]; off = 4 and 8 are the half-row
// and row mirrors (lane i with 7-i, 15-i), which meet the same partner
// group as the xor does, and since the butterfly has made each of those
// groups uniform by then, deliver the same value.  Across rows, the four
// row results are read with v_readlane and combined in the same order:
// rows (0,1) and (2,3), then the two pairs.  Every lane of a group must be
// active; lanes of other groups may be inactive.

template <int OFF>
__device__ __forceinline__ uint32_t dpp_partner(uint32_t v) {
    static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8, "row step");
    constexpr int ctrl = OFF == 1 ? 0xB1 : (OFF == 2 ? 0x4E : (OFF == 4 ? 0x141 : 0x140));
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, true);
}

template <int G, class T, class Op>
__device__ __forceinline__ T group_reduce(T v, Op op) {
    static_assert(sizeof(T) == 4, "32-bit values");
    auto bits = [](T x) { return __builtin_bit_cast(uint32_t, x); };
    auto val = [](uint32_t x) { return __builtin_bit_cast(T, x); };
    if constexpr (G >= 2) v = op(v, val(dpp_partner<1>(bits(v))));
    if constexpr (G >= 4) v = op(v, val(dpp_partner<2>(bits(v))));
    if constexpr (G >= 8) v = op(v, val(dpp_partner<4>(bits(v))));
    if constexpr (G >= 16) v = op(v, val(dpp_partner<8>(bits(v))));
    if constexpr (G >= 32) {
        const T r0 = val((uint32_t)__builtin_amdgcn_readlane((int)bits(v), 0));
        const T r1 = val((uint32_t)__builtin_amdgcn_readlane((int)bits(v), 16));
        const T r2 = val((uint32_t)__builtin_amdgcn_readlane((int)bits(v), 32));
        const T r3 = val((uint32_t)__builtin_amdgcn_readlane((int)bits(v), 48));
        if constexpr (G == 32) v = lane_id() < 32 ? op(r0, r1) : op(r2, r3);
        else v = op(op(r0, r1), op(r2, r3));
    }
    return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
    return group_reduce<G>(v, [](float a, float b) { return a + b; });
}

template <int G>
__device__ __forceinline__ float group_min(float v) {
    return group_reduce<G>(v, [](float a, float b) { return fminf(a, b); });
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
    return group_reduce<G>(v, [](float a, float b) { return fmaxf(a, b); });
}

// Unsigned maximum over a group (a DPP move folds into v_max_u32).
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    return group_reduce<G>(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

template <int G>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
    return group_reduce<G>(v, [](uint32_t a, uint32_t b) { return a | b; });
}

// The value of lane t^1 (neighbouring lanes exchange).
__device__ __forceinline__ uint32_t lane_xor1(uint32_t v) { return dpp_partner<1>(v); }

// Contiguous pairwise tree over N (power of two) values held in registers.
template <int N>
__device__ __forceinline__ float tree_sum_regs(float (&s)[N]) {
#pragma unroll
    for (int w = 1; w < N; w <<= 1) {
#pragma unroll
        for (int i = 0; i < N; i += 2 * w) s[i] = s[i] + s[i + w];
    }
    return s[0];
}

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): each round takes the
// 32x32->64 products of counter words 0 and 2 with two fixed multipliers;
// new words are (hi(B*c2) ^ c1 ^ k0, lo(B*c2), hi(A*c0) ^ c3 ^ k1, lo(A*c0)),
// and the key is advanced by two Weyl increments after every round.

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
    constexpr uint32_t A = 0xD2511F53u, B = 0xCD9E8D57u;
    constexpr uint32_t KA = 0x9E3779B9u, KB = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t pa = (uint64_t)A * c0;
        const uint64_t pb = (uint64_t)B * c2;
        const uint32_t n0 = (uint32_t)(pb >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(pa >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)pb;
        c3 = (uint32_t)pa;
        c0 = n0;
        c2 = n2;
        k0 += KA;
        k1 += KB;
    }
    return u32x4{c0, c1, c2, c3};
}

// ------------------------------------------------------------ OCP E4M3FN
// Encode |y| <= 448 with round-to-nearest-even on the integer bit pattern.
// Normal results (|y| >= 2^-6): add half an e4m3 ulp minus one plus the
// kept lsb to the 20 discarded mantissa bits, shift, and rebias the
// exponent from 127 to 7 (a carry out of the mantissa bumps the exponent,
// which is the correct rounding).  Subnormal results: |y| * 2^9 is exact,
// rint gives the number of 2^-9 steps (8 steps is the smallest normal,
// whose code is also 8).  The sign bit is kept, so negative underflow
// gives 0x80.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    const uint32_t b = __float_as_uint(y);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7FFFFFFFu;
    const uint32_t rounded = a + 0x7FFFFu + ((a >> 20) & 1u);
    const uint32_t normal = (rounded >> 20) - (120u << 3);
    const uint32_t sub = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    return sign | (a >= 0x3C800000u ? normal : sub);
}

// e4m3_encode for |y| >= 2^-6 (the normal codes), where the subnormal
// branch above is never taken.
__device__ __forceinline__ uint32_t e4m3_encode_normal(float y) {
    const uint32_t b = __float_as_uint(y);
    const uint32_t sign = (b >> 24) & 0x80u;
    const uint32_t a = b & 0x7FFFFFFFu;
    const uint32_t rounded = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((rounded >> 20) - (120u << 3));
}

// Exact E4M3 -> fp32: normal codes rebias the exponent by +120 and place
// the 3 mantissa bits at the top of the fp32 mantissa; subnormal codes are
// m * 2^-9.
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
    const uint32_t em = c & 0x7Fu;
    const float mag = em >= 8u ? __uint_as_float((em << 20) + (120u << 23))
                               : (float)em * 0x1p-9f;
    return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// ------------------------------------------------- wave-span stores
// Orders a wave's LDS accesses before and after it (lanes exchange data
// through LDS within one wave; a wave's LDS instructions run in order).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane l holds elements [16l, 16l + 16) of a 1,024-element span at dst.
// Stored from registers, each instruction would cover every fourth
// 16-byte piece of the 4 KiB span and touch 32 cache lines (the compute
// units' limit on outstanding requests is what the streaming kernels run
// into); passed through the wave's 4 KiB LDS buffer xw, each of the four
// store instructions writes 1 KiB contiguously (8 lines), with streaming
// stores.  All 64 lanes must be active and the whole span inside dst.
// Piece q (elements 4q..4q+3) of this lane's 16 into the wave's buffer.
__device__ __forceinline__ void span16_put(float* xw, int q, f32x4 v) {
    *reinterpret_cast<f32x4*>(xw + 16 * lane_id() + 4 * q) = v;
}
// Every lane's 16 elements are in xw: store the span from it.
__device__ __forceinline__ void span16_store(float* __restrict__ dst, float* xw) {
    const int l = lane_id();
    wave_lds_sync();
#pragma unroll
    for (int q = 0; q < 4; ++q)
        st_f4(dst + 256 * q + 4 * l, *reinterpret_cast<const f32x4*>(xw + 256 * q + 4 * l));
    wave_lds_sync();  // xw may be rewritten right after
}
__device__ __forceinline__ void store_wave_span16(float* __restrict__ dst, const float (&v)[16], float* xw) {
#pragma unroll
    for (int q = 0; q < 4; ++q) span16_put(xw, q, f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]});
    span16_store(dst, xw);
}

// ------------------------------------------------------- division by d
// fl(x / d) without a division, for x >= +0 and a divisor shared by many
// x: with r = fl(1/d), q0 = fl(x r) is within an ulp of x/d, the
// remainder x - q0 d is exact (one fma), and fl(q0 + rem r) is the
// correctly rounded quotient (Markstein, IBM J. Res. Dev. 34(1), 1990), as
// long as nothing underflows or overflows: d and 1/d normal (the caller's
// `dok`), x finite and >= 2^-102 (so the remainder does not fall below the
// subnormal grid) and the quotient in [2^-100, 2^126].  x = +0 gives +0
// (and x = -0 gives +0 too, where x / d is -0).  Otherwise `fast` is false
// and the caller divides.
__device__ __forceinline__ float quot_fast(float x, float d, float r, bool dok, bool& fast) {
    const float q0 = x * r;
    const float rem = __builtin_fmaf(-q0, d, x);
    const float aq = fabsf(q0);
    fast = dok && (x == 0.0f || (x >= 0x1p-102f && x <= 0x1.fffffep127f && aq >= 0x1p-100f && aq <= 0x1p126f));
    return __builtin_fmaf(rem, r, q0);
}

// q[j] = fl(x[j] / d) for N values x >= +0 or NaN (a -0 gives +0), r = fl(1/d):
// quot_fast, and the division for the rare value outside its range, under
// a wave-uniform branch so the division stays off the common path.
template <int N>
__device__ __forceinline__ void quot_n(const float (&x)[N], float d, float r, bool dok, float (&q)[N]) {
    bool fast[N], all = true;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        q[j] = quot_fast(x[j], d, r, dok, fast[j]);
        all = all && fast[j];
    }
    if (!__all(all)) {
#pragma unroll
        for (int j = 0; j < N; ++j)
            if (!fast[j]) q[j] = x[j] / d;
    }
}

// d and 1/d both normal
__device__ __forceinline__ bool quot_divisor_ok(float d) {
    const float a = fabsf(d);
    return a >= 0x1p-126f && a <= 0x1p126f;
}

// --------------------------------------------------------------- misc
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

}  // namespace qc
