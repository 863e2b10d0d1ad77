// k_fp8.hip -- rowwise FP8 (OCP E4M3FN) encoder for embedding-lookup rows.
//
// Per row: scale = amax/448; code = e4m3(clamp(x/scale, +-448)).  A row of
// dim = 4*LPR values (LPR a power of two <= 64) is held by LPR lanes, one
// 16-byte chunk each, so one wave covers 64/LPR rows per load instruction
// (for dim = 128: 2 rows, 1 KiB contiguous); RG such row groups are loaded
// before any is processed to keep enough bytes in flight.  Other dims
// (multiples of 4) take one wave per row and read the row twice (the second
// read hits L2).
#include "qc_device.hpp"
#include "qc_bucket.hpp"
#include "qc_launch.hpp"

namespace qc {
namespace {

__device__ __forceinline__ uint32_t fp8_pack4(f32x4 v, float sc) {
    if (sc == 0.0f) return 0u;
    const float x[4] = {v.x, v.y, v.z, v.w};
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float y = fminf(fmaxf(x[j] / sc, -448.0f), 448.0f);
        word |= e4m3_encode(y) << (8 * j);
    }
    return word;
}

__device__ __forceinline__ float amax4(f32x4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
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
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int64_t row = r0 + g * RPG + rsub;
        const float amax = group_max<LPR>(amax4(v[g]));
        const float sc = amax / 448.0f;
        const uint32_t word = fp8_pack4(v[g], sc);
        if (FULL || row < rows) {
            st_u32(codes + row * DIM + l * 4, word);
            if (l == 0) {
                scale[row] = sc;
                if (row == rows - 1) fp8_zero_tail(codes, rows * DIM, pbytes);
            }
        }
    }
}

// Wave w of the grid handles RPW = RG * 64/LPR consecutive rows per
// iteration; groups of rows wholly inside `rows` take the branch-free path.
template <int LPR, int RG>
__global__ void __launch_bounds__(256)
k_enc_fp8_pow2(const float* __restrict__ x, int64_t rows, uint8_t* __restrict__ codes,
               int64_t pbytes, float* __restrict__ scale) {
    constexpr int RPW = (WAVE / LPR) * RG;
    const int64_t wstride = (int64_t)gridDim.x * 4;
    for (int64_t r0 = ((int64_t)blockIdx.x * 4 + wave_id()) * RPW; r0 < rows; r0 += wstride * RPW) {
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
            st_u32(codes + row * dim + 4 * c, fp8_pack4(ld_f4(xr + 4 * c), sc));
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
    const dim3 grid((unsigned)grid_for(waves, 4)), block(256);
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
