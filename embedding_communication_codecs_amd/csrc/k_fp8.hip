// k_fp8.hip -- rowwise FP8 (OCP E4M3FN) encoder for embedding-lookup rows.
//
// Per row: scale = amax/448; code = e4m3(clamp(x/scale, +-448)).  A row of
// dim = 4*LPR values (LPR a power of two <= 64) is held by LPR lanes, one
// 16-byte chunk each, so one wave covers 64/LPR rows per load instruction
// (for dim = 128: 2 rows, 1 KiB contiguous); RG such row groups are loaded
// before any is processed to keep enough bytes in flight.  Other dims
// (multiples of 4) take one wave per row and read the row twice (the second
// read hits L2).  The power-of-two dims compute the scale and codes without
// dividing (exact shortcuts, below) and divide only where a shortcut does
// not apply: the division was the encoder's main ALU cost.
#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"

namespace qc {
namespace {

// Exact forms: sc = fl(amax/448); code = e4m3(clamp(fl(x/sc), +-448)).
// Only the rare fallback below and odd dims use them, so the divisions run
// one at a time (unrolled, four division sequences in flight held the
// whole kernel at 82 registers and 5 waves per SIMD; rolled, 63 and 8).
__device__ __forceinline__ uint32_t fp8_pack4_exact(f32x4 v, float sc) {
    if (sc == 0.0f) return 0u;
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0;
#pragma unroll 1
    for (int j = 0; j < 4; ++j) word |= e4m3_encode(fminf(fmaxf(x[j] / sc, -448.0f), 448.0f)) << (8 * j);
    return word;
}

// The same results without a division, for all but rare inputs; `fix` is
// set where the shortcut does not apply, and the caller then redoes the
// row group with the exact forms.
//
// Row scale: q0 = fl(amax * fl(1/448)) and one correction with the exact
// remainder fma(-448, q0, amax).  For every amax from 2^-120 up to the
// largest float this equals the correctly rounded quotient (checked over
// all of them); other amax are fixed up.
__device__ __forceinline__ float fp8_row_scale_fast(float amax, bool& fix) {
    constexpr float r448 = 0x1.24924ap-9f;
    fix |= !(amax >= 0x1p-120f && amax <= 0x1.fffffep127f);
    const float q0 = amax * r448;
    return __builtin_fmaf(__builtin_fmaf(-448.0f, q0, amax), r448, q0);
}

// Codes: y = fl(x/sc) matters only through its E4M3 rounding.  r
// approximates 1/sc (hardware reciprocal, good to 1 ulp, and one Newton
// step: relative error about 2^-24, far below 2^-22), so q = fl(x*r) rounds
// a point within x/sc * 2^-22, i.e. less than 4 fp32 ulps, of x/sc;
// rounding is monotone, so q and y are at most 4 ulps apart (8 across a
// binade edge, where no E4M3 rounding point lies).  For |q| >= 2^-6 the
// E4M3 code steps only where the 20 discarded mantissa bits of |y| pass
// 0x80000, so when those bits of q differ from 0x80000 by more than 8 the
// codes of q and y are equal (clamping at 448 is monotone too).  Values
// below 2^-6, values near a rounding point and subnormal scales are fixed
// up.  A zero scale gives code 0 either way.
__device__ __forceinline__ uint32_t fp8_pack4_fast(f32x4 v, float sc, bool& fix) {
    const float r0 = __builtin_amdgcn_rcpf(sc);
    const float r = __builtin_fmaf(__builtin_fmaf(-sc, r0, 1.0f), r0, r0);
    const float x[4] = {v.x, v.y, v.z, v.w};
    float y[4];
    uint32_t near[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        y[j] = x[j] * r;
        // |D - 0x80000| <= 8 maps to [0, 16], D the discarded bits
        near[j] = (__float_as_uint(y[j]) - 0x7FFF8u) & 0xFFFFFu;
    }
    const uint32_t nmin = min(min(near[0], near[1]), min(near[2], near[3]));
    const float ymin = fminf(fminf(fabsf(y[0]), fabsf(y[1])), fminf(fabsf(y[2]), fabsf(y[3])));
    fix |= sc != 0.0f && (nmin <= 16u || ymin < 0x1p-6f || !(sc >= 0x1p-126f));
    // where the word is kept (no fix-up), every |y| >= 2^-6: normal codes only
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) word |= e4m3_encode_normal(fminf(fmaxf(y[j], -448.0f), 448.0f)) << (8 * j);
    return sc == 0.0f ? 0u : word;
}

__device__ __forceinline__ float amax4(f32x4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// The row maximum of |x| as the reference loop takes it (a running maximum
// from +0 that a NaN never replaces, so an all-NaN row gives +0), in
// unsigned integer form: key(x) = (bits(x) << 1) + 0x00FFFFFE drops the
// sign and maps |x| from +0 to +inf, in order, onto [0x00FFFFFE,
// 0xFFFFFFFE], while every NaN wraps below 0x00FFFFFE.  Integer maxima
// take one instruction per cross-lane step (the DPP move folds into
// v_max_u32); float maxima took four (each operand is quieted first).
constexpr uint32_t kKeyZero = 0x00FFFFFEu;
__device__ __forceinline__ uint32_t amax_key(float x) { return (__float_as_uint(x) << 1) + kKeyZero; }
__device__ __forceinline__ uint32_t amax4_key(f32x4 v) {
    const uint32_t a = amax_key(v.x), b = amax_key(v.y), c = amax_key(v.z), d = amax_key(v.w);
    const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
    return ab > cd ? ab : cd;
}
__device__ __forceinline__ float amax_of_key(uint32_t k) {
    return k < kKeyZero ? 0.0f : __uint_as_float((k - kKeyZero) >> 1);
}

// The payload is rows*dim bytes rounded up to 16; whoever owns the last row
// zeroes the (at most 12) padding bytes after it.
__device__ __forceinline__ void fp8_zero_tail(uint8_t* codes, int64_t used, int64_t pbytes) {
    for (int64_t b = used; b < pbytes; b += 4) st_u32(codes + b, 0u);
}

template <int LPR, int RG, bool FULL>
__device__ __forceinline__ void fp8_rows(const float* __restrict__ x, int64_t rows, uint8_t* __restrict__ codes,
                                         int64_t pbytes, float* __restrict__ scale, int64_t r0) {
    constexpr int DIM = LPR * 4;
    constexpr int RPG = WAVE / LPR;  // rows per load instruction
    const int l = lane_id() % LPR;
    const int rsub = lane_id() / LPR;
    f32x4 v[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int64_t row = r0 + g * RPG + rsub;
        v[g] = (FULL || row < rows) ? ld_stream_f4(x + row * DIM + l * 4) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // every row group through the division-free forms first, branch-free,
    // then one rarely taken branch redoes the lane's groups exactly if any
    // needed it: amax is kept (no cross-lane work inside the branch) and the
    // values are read again (an L2 hit) rather than kept in registers.
    // The fallback loop is not unrolled, so it adds nothing to the
    // registers the fast path holds.
    float amax[RG], sc[RG];
    uint32_t word[RG];
    bool fix = false;
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        amax[g] = amax_of_key(group_max_u32<LPR>(amax4_key(v[g])));
        sc[g] = fp8_row_scale_fast(amax[g], fix);
        word[g] = fp8_pack4_fast(v[g], sc[g], fix);
    }
    if (__builtin_expect(fix, 0)) {
#pragma unroll 1
        for (int g = 0; g < RG; ++g) {
            const int64_t row = r0 + g * RPG + rsub;
            const f32x4 vg = (FULL || row < rows) ? ld_f4(x + row * DIM + l * 4) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            sc[g] = amax[g] / 448.0f;
            word[g] = fp8_pack4_exact(vg, sc[g]);
        }
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int64_t row = r0 + g * RPG + rsub;
        if (FULL || row < rows) st_u32(codes + row * DIM + l * 4, word[g]);
    }
    if constexpr (FULL && LPR >= 16) {
        // With few rows per load (dim >= 64) the wave's RPG*RG row scales
        // are gathered with readlane (every lane of a row holds its row's
        // scale) and written as whole 16-byte pieces, lane p writing rows
        // 4p..4p+3 of the wave's consecutive rows.  (Written one 4-byte value
        // per row, each went to HBM as its own partial write: 1.10x the
        // algorithmic write bytes at dim 128.)  Smaller dims already store
        // RPG >= 8 consecutive scales per instruction.
        constexpr int RPW = RPG * RG;
        float s[RPW];
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int rs = 0; rs < RPG; ++rs)
                s[g * RPG + rs] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc[g]), rs * LPR));
        const int p = lane_id();
        if (p < RPW / 4) {
            f32x4 o = f32x4{s[0], s[1], s[2], s[3]};
#pragma unroll
            for (int q = 1; q < RPW / 4; ++q)
                if (p == q) o = f32x4{s[4 * q], s[4 * q + 1], s[4 * q + 2], s[4 * q + 3]};
            st_f4(scale + r0 + 4 * p, o);
        }
    } else {
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int64_t row = r0 + g * RPG + rsub;
            if ((FULL || row < rows) && l == 0) scale[row] = sc[g];
        }
    }
    // the owner of the last row zeroes the payload's padding
    if (lane_id() == 0 && r0 <= rows - 1 && rows - 1 < r0 + RPG * RG)
        fp8_zero_tail(codes, rows * DIM, pbytes);
}

// Wave w of the grid handles RPW = RG * 64/LPR consecutive rows per
// iteration; groups of rows wholly inside `rows` take the branch-free path.
// Two waves per block and one short-lived wave per RPW rows measured best
// on MI355X at 1e6 x 128: 4-wave blocks were 3% slower, 8-wave blocks 8%;
// RG = 6 or 8 and persistent waves that load their next rows before
// encoding the current ones were 5-25% slower; plain (not streaming) loads
// were 50% slower right after a write-heavy kernel.
template <int LPR, int RG>
__global__ void __launch_bounds__(128)
k_enc_fp8_pow2(const float* __restrict__ x, int64_t rows, uint8_t* __restrict__ codes,
               int64_t pbytes, float* __restrict__ scale) {
    constexpr int RPW = (WAVE / LPR) * RG;
    const int64_t wstride = (int64_t)gridDim.x * 2;
    for (int64_t r0 = ((int64_t)blockIdx.x * 2 + wave_id()) * RPW; r0 < rows; r0 += wstride * RPW) {
        if (r0 + RPW <= rows)
            fp8_rows<LPR, RG, true>(x, rows, codes, pbytes, scale, r0);
        else
            fp8_rows<LPR, RG, false>(x, rows, codes, pbytes, scale, r0);
    }
}

__global__ void __launch_bounds__(256)
k_enc_fp8_rowwave(const float* __restrict__ x, int64_t rows, int32_t dim, uint8_t* __restrict__ codes,
                  int64_t pbytes, float* __restrict__ scale) {
    const int chunks = dim / 4;
    const int64_t wstride = (int64_t)gridDim.x * 4;
    for (int64_t row = (int64_t)blockIdx.x * 4 + wave_id(); row < rows; row += wstride) {
        const float* xr = x + row * dim;
        float amax = 0.0f;
        for (int c = lane_id(); c < chunks; c += WAVE) amax = fmaxf(amax, amax4(ld_f4(xr + 4 * c)));
        amax = group_max<WAVE>(amax);
        const float sc = amax / 448.0f;
        for (int c = lane_id(); c < chunks; c += WAVE)
            st_u32(codes + row * dim + 4 * c, fp8_pack4_exact(ld_f4(xr + 4 * c), sc));
        if (lane_id() == 0) {
            scale[row] = sc;
            if (row == rows - 1) fp8_zero_tail(codes, rows * dim, pbytes);
        }
    }
}

template <int LPR>
hipError_t launch_pow2(const float* x, int64_t rows, uint8_t* codes, int64_t pbytes, float* scale,
                       hipStream_t stream) {
    constexpr int RG = 4;
    constexpr int RPW = (WAVE / LPR) * RG;
    const int64_t waves = (rows + RPW - 1) / RPW;
    const dim3 grid((unsigned)grid_for(waves, 2)), block(128);
    hipLaunchKernelGGL((k_enc_fp8_pow2<LPR, RG>), grid, block, 0, stream, x, rows, codes, pbytes, scale);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode_fp8(const float* x, int64_t rows, int32_t dim, uint8_t* codes,
                             int64_t payload_bytes, float* scale, hipStream_t stream) {
    switch (dim) {
        case 4: return launch_pow2<1>(x, rows, codes, payload_bytes, scale, stream);
        case 8: return launch_pow2<2>(x, rows, codes, payload_bytes, scale, stream);
        case 16: return launch_pow2<4>(x, rows, codes, payload_bytes, scale, stream);
        case 32: return launch_pow2<8>(x, rows, codes, payload_bytes, scale, stream);
        case 64: return launch_pow2<16>(x, rows, codes, payload_bytes, scale, stream);
        case 128: return launch_pow2<32>(x, rows, codes, payload_bytes, scale, stream);
        case 256: return launch_pow2<64>(x, rows, codes, payload_bytes, scale, stream);
        default: break;
    }
    const dim3 grid((unsigned)grid_for(rows, 4)), block(256);
    hipLaunchKernelGGL(k_enc_fp8_rowwave, grid, block, 0, stream, x, rows, dim, codes, payload_bytes,
                       scale);
    return hipGetLastError();
}

}  // namespace qc
